// Device helpers shared by the kernel translation units.
#pragma once

#include "tl_internal.h"

namespace tl {

template <typename T> struct DT;
template <> struct DT<float> { static constexpr int id = TL_DTYPE_F32; };
template <> struct DT<half_t> { static constexpr int id = TL_DTYPE_F16; };

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(half_t v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ half_t from_f<half_t>(float v) { return (half_t)v; }

__device__ __forceinline__ uint16_t h_bits(half_t v) { return __builtin_bit_cast(uint16_t, v); }
__device__ __forceinline__ half_t h_from_bits(uint16_t b) { return __builtin_bit_cast(half_t, b); }

// Warp (64-lane) reductions in a fixed butterfly order.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block reductions (blockDim.x a multiple of 64, at most 1024). Every thread
// gets the result. The partial of wave w is combined in order w = 0, 1, ...
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
  for (int i = 1; i < nw; ++i) s = fmaxf(s, red[i]);
  return s;
}

// Merge of one (row, head)'s ns >= 1 key-split partials p[s] = (max m_s, sum
// l_s, unnormalised o_s[DH]) by a block of NTH threads (blockDim.x == NTH):
// o = sum_s w_s o_s / sum_s w_s l_s with w_s = exp(m_s - M), M the largest
// m_s. Thread (dim, group g) sums the splits s = g, g + G, ... (G = NTH / DH)
// for its dimension and the G group sums are added in order g = 0, 1, ...,
// so the result depends only on ns, NTH and the partials. Each thread loads
// its (m, l, o[dim]) of max(32 / G, 1) splits at a time, the first batch
// together with the maxima. Scratch: osum [NTH], lsum [G], red [NTH / 64] in
// LDS. Every thread of the block must call it. COHERENT: read the partials
// with device-coherent loads (written in the same launch by workgroups on
// other XCDs with device-coherent stores).
template <typename T, int DH, bool COHERENT = false, int NTH = 256>
__device__ __forceinline__ void merge_splits(const float* p, int ns, T* out, float* osum,
                                             float* lsum, float* red) {
  constexpr int G = NTH / DH, U = 32 / G > 1 ? 32 / G : 1;
  static_assert(G * DH == NTH, "threads per merge");
  constexpr float kL2e = 1.4426950408889634f;
  const int t = threadIdx.x, dim = t % DH, g = t / DH;
  auto ld = [](const float* a) -> float {
    if constexpr (COHERENT) return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *a;
  };
  float mv[U], lv[U], ov[U];
  auto load = [&](int c) {   // splits c + g + G u (the last split stands in past ns)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* ps = p + (size_t)min(c + g + G * u, ns - 1) * (DH + 2);
      mv[u] = ld(ps);
      lv[u] = ld(ps + 1);
      ov[u] = ld(ps + 2 + dim);
    }
  };
  load(0);
  float M = -__builtin_inff();
  for (int s = t; s < ns; s += NTH) M = fmaxf(M, ld(p + (size_t)s * (DH + 2)));
  M = block_max(M, red);
  float acc = 0.f, lacc = 0.f;
  for (int c = 0; c < ns; c += G * U) {
    if (c) load(c);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c + g + G * u < ns) {
        const float w = exp2f((mv[u] - M) * kL2e);
        acc = fmaf(ov[u], w, acc);
        lacc = fmaf(lv[u], w, lacc);
      }
  }
  osum[g * DH + dim] = acc;
  if (dim == 0) lsum[g] = lacc;
  __syncthreads();
  if (g == 0) {
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      o += osum[k * DH + dim];
      L += lsum[k];
    }
    out[dim] = from_f<T>(__fdiv_rn(o, L));
  }
}

// ---------------------------------------------------------------------------
// h codec: symmetric absmax, fp16 scale (IEEE fp32 divide, round half to even)
// ---------------------------------------------------------------------------
// scale = fp16(absmax / qmax)
__device__ __forceinline__ half_t codec_scale(float absmax, float qmax) {
  return (half_t)__fdiv_rn(absmax, qmax);
}
// q = clamp(rint(h / s), qmin, qmax), 0 when s == 0
__device__ __forceinline__ int codec_code(float h, float s, float qmin, float qmax) {
  if (s == 0.f) return 0;
  float q = rintf(__fdiv_rn(h, s));
  q = fminf(fmaxf(q, qmin), qmax);
  return (int)q;
}

// Order of the codes inside one 64-element block row of an INT4 / INT8 cache
// entry: the row is split into two halves; half hb holds, for k-steps
// kk = 0..3, the 8 elements 16*kk + 8*hb .. 16*kk + 8*hb + 7. That is exactly
// the run of k values one half-wave feeds to a 32x32x16 MFMA, so a lane reads
// its four k-steps' codes as one contiguous 16-byte (INT4) or 32-byte (INT8)
// load. Returns the index of the 8-element group holding element w (0..63).
__host__ __device__ __forceinline__ int code_group(int w) { return ((w >> 3) & 1) * 4 + (w >> 4); }

// INT4 nibble placement inside a 32-bit word of 8 consecutive elements
// e0..e7: element j sits at bit 4*(j/2) for even j and 16 + 4*(j/2) for odd j,
// so (w >> 4i) & 0x000F000F yields the pair (e_2i, e_2i+1) in the two halves
// of a word. Codes are stored offset by 8 (0..15).
__device__ __forceinline__ int int4_shift(int j) { return (j & 1) ? 16 + 4 * (j >> 1) : 4 * (j >> 1); }

// Dequantise 8 INT4 codes (one word) with scale s into 8 fp16: fp16(q * s).
// (1024 + u) is exact in fp16; subtracting 1032 gives q exactly; the product
// with s is one correctly rounded fp16 multiply.
// (w >> 4i) & 0x000F000F | 0x64006400 is one three-input bitwise op (truth
// table 0xEA: (a & b) | c); the four pairs are formed, then offset, then
// scaled, so no packed op waits on the one right before it.
__device__ __forceinline__ half8 int4_dequant8(uint32_t w, half_t s) {
  const half2v bias = {(half_t)1032.f, (half_t)1032.f};
  const half2v sv = {s, s};
  half2v x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    x[i] = __builtin_bit_cast(half2v, __builtin_amdgcn_bitop3_b32(w >> (4 * i), 0x000F000Fu, 0x64006400u, 0xEA));
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = x[i] - bias;
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = x[i] * sv;
  return half8{x[0][0], x[0][1], x[1][0], x[1][1], x[2][0], x[2][1], x[3][0], x[3][1]};
}

// Dequantise 4 INT8 codes (one word, two's complement bytes) into fp16(q * s).
// (byte ^ 0x80) | 0x6400 = 1024 + (q + 128) exactly; minus 1152 gives q.
__device__ __forceinline__ half4 int8_dequant4(uint32_t w, half_t s) {
  const uint32_t f = w ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, f, 0x07010700u);  // bytes b1,b0 -> halves
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, f, 0x07030702u);
  const half2v bias = {(half_t)1152.f, (half_t)1152.f};
  const half2v sv = {s, s};
  half2v a = (__builtin_bit_cast(half2v, lo) - bias) * sv;
  half2v b = (__builtin_bit_cast(half2v, hi) - bias) * sv;
  half4 r = {a[0], a[1], b[0], b[1]};
  return r;
}

// EPT codes of one delta row (8- or 4-byte vector loads where EPT allows)
template <int EPT>
struct DeltaRow {
  int8_t q[EPT];
};
template <int EPT>
__device__ __forceinline__ DeltaRow<EPT> delta_load(const int8_t* p) {
  DeltaRow<EPT> r;
  if constexpr (EPT == 8) {
    typedef int8_t v8 __attribute__((ext_vector_type(8)));
    const v8 v = *(const v8*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.q[i] = v[i];
  } else if constexpr (EPT == 4) {
    typedef int8_t v4 __attribute__((ext_vector_type(4)));
    const v4 v = *(const v4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.q[i] = v[i];
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) r.q[i] = p[i];
  }
  return r;
}
// Delta mode: elements e0 .. e0+EPT-1 of the FP32 reconstruction of `layer`
// at (lane, pos): a unique layer's own h, or the prefix sum of the anchor
// (layer n_pre - 1) and scale * code of loop layers n_pre .. layer, added in
// that order (each product is exact in fp32; the addition rounds).
// EPT divides the head width, so one scale covers a thread's elements.
template <int EPT>
__device__ __forceinline__ void delta_prefix(const CacheView& c, int layer, int lane, int pos,
                                             int e0, float (&r)[EPT]) {
  const half_t* a = c.delta_anchor(layer < c.n_pre ? layer : c.n_pre - 1, lane, pos) + e0;
  if constexpr (EPT == 8) {
    const half8 v = *(const half8*)a;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (float)v[i];
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) r[i] = (float)a[i];
  }
  const int head = e0 / c.dh;
  int j = c.n_pre;
  // four layers' codes and scales in flight at a time
  for (; j + 3 <= layer; j += 4) {
    DeltaRow<EPT> q[4];
    half_t sc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      q[u] = delta_load<EPT>(c.delta_codes(j + u, lane, pos) + e0);
      sc[u] = h_from_bits(c.delta_scales(j + u, lane, pos)[head]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < EPT; ++i) r[i] = r[i] + (float)sc[u] * (float)q[u].q[i];
  }
  for (; j <= layer; ++j) {
    const DeltaRow<EPT> q = delta_load<EPT>(c.delta_codes(j, lane, pos) + e0);
    const float sf = (float)h_from_bits(c.delta_scales(j, lane, pos)[head]);
#pragma unroll
    for (int i = 0; i < EPT; ++i) r[i] = r[i] + sf * (float)q.q[i];
  }
}

// Store elements e0 .. e0+EPT-1 of h (already rounded to the model dtype) of
// one cache entry (layer, lane, pos) in the cache's h codec. The threads of a
// row hold consecutive runs of EPT elements, so an INT4 group is 32 / EPT
// consecutive lanes and an 8-code INT4 word 8 / EPT of them; rowmax(v) returns
// the maximum of v over all threads of the row (the INT8 per-token scale) and
// must be called by all of them. Delta mode: rec (the thread's EPT elements
// of the row's FP32 reconstruction of the previous layer) is updated to this
// layer's; a head of dh elements is dh / EPT consecutive lanes of one wave.
template <typename T, int EPT, typename RowMax>
__device__ __forceinline__ void cache_store_h(const CacheView& c, int layer, int lane, int pos,
                                              int e0, const float (&h)[EPT], RowMax&& rowmax,
                                              float* rec = nullptr) {
  if (c.mode == TL_CACHE_H_DELTA8) {
    if (layer < c.n_pre) {
      half_t* dst = c.delta_anchor(layer, lane, pos) + e0;
#pragma unroll
      for (int i = 0; i < EPT; ++i) dst[i] = (half_t)h[i];
#pragma unroll
      for (int i = 0; i < EPT; ++i) rec[i] = h[i];
      return;
    }
    float d[EPT], am = 0.f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      d[i] = h[i] - rec[i];
      am = fmaxf(am, fabsf(d[i]));
    }
    const int tph = c.dh / EPT;   // threads of one head
    for (int o = 1; o < tph; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    const half_t s = codec_scale(am, 127.f);
    const float sf = (float)s;
    int8_t* qp = c.delta_codes(layer, lane, pos) + e0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int q = codec_code(d[i], sf, -127.f, 127.f);
      qp[i] = (int8_t)q;
      rec[i] = rec[i] + sf * (float)q;
    }
    if (e0 % c.dh == 0) c.delta_scales(layer, lane, pos)[e0 / c.dh] = h_bits(s);
    return;
  }
  const int kb = e0 / kKBlock, w = e0 % kKBlock;
  char* row = c.code_row(layer, lane, kb, pos);
  if (c.mode == TL_CACHE_H_F32 || c.mode == TL_CACHE_H_F16) {
    T* dst = (T*)row + w;
#pragma unroll
    for (int i = 0; i < EPT; ++i) dst[i] = from_f<T>(h[i]);
    return;
  }
  if (c.mode == TL_CACHE_H_INT8) {
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) am = fmaxf(am, fabsf(h[i]));
    am = rowmax(am);
    const half_t s = codec_scale(am, 127.f);
    const float sf = (float)s;
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      ((int8_t*)row)[code_group(w + i) * 8 + ((w + i) & 7)] = (int8_t)codec_code(h[i], sf, -127.f, 127.f);
    if (e0 == 0) *c.int8_scale(layer, lane, pos) = h_bits(s);
    return;
  }
  // INT4: group of 32 elements = 32 / EPT consecutive threads
  constexpr int TPG = kInt4Group / EPT;
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) am = fmaxf(am, fabsf(h[i]));
#pragma unroll
  for (int o = 1; o < TPG; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  const half_t s = codec_scale(am, 7.f);
  const float sf = (float)s;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int q = codec_code(h[i], sf, -8.f, 7.f);
    word |= (uint32_t)(q + 8) << int4_shift((e0 + i) & 7);
  }
  static_assert(EPT <= 8, "one INT4 word per thread at most");
  if constexpr (EPT < 8) {
    constexpr int TPW = 8 / EPT;   // threads sharing one word
#pragma unroll
    for (int o = 1; o < TPW; o <<= 1) word |= __shfl_xor(word, o, 64);
    if ((e0 & 7) == 0) ((uint32_t*)row)[code_group(w)] = word;
  } else {
    ((uint32_t*)row)[code_group(w)] = word;
  }
  if ((e0 % kInt4Group) == 0) {
    const int g = e0 / kInt4Group;
    c.int4_scale(layer, lane, g / 2, pos)[g & 1] = h_bits(s);
  }
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) for synthetic inputs
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}
// Synthetic h element: centred sum of the eight 16-bit halves, one fp32 multiply.
__device__ __forceinline__ float synth_h(uint32_t seed, int layer, int lane, int pos, int k) {
  uint32_t c[4] = {(uint32_t)k, (uint32_t)pos, (uint32_t)lane, (uint32_t)layer};
  philox4x32_10(c, seed, 0x1F0E9D75u);
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += (int)(c[i] & 0xFFFFu) + (int)(c[i] >> 16);
  float v = (float)(s - 262140) * __builtin_bit_cast(float, 0x379CC471u);
  // keep the fp32 rounding of the product: without this the backend folds a
  // later fp16 conversion into one mixed-precision FMA that rounds only once
  __asm__ volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float gelu_f(float v) {
  return 0.5f * v * (1.f + erff(v * 0.70710678118654752f));
}

}  // namespace tl
