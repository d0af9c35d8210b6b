// Store-h attention: rebuild K = W_k h' and V = W_v h' for cached positions
// from the stored h (TinyLoop architecture-exclusive features page, "Store-h
// KV cache"; novel-contributions page, "Store-h KV Cache") on MFMA, and either
// fold them straight into online-softmax attention partials (decode) or store
// them for the causal prefill attention.
//
// One workgroup computes the product tile C[f, j] = sum_k W[f, k] h'[j, k] for
// BF features (the K and V rows of whole heads) and BJ cached positions of one
// lane, streaming d_model in BK-deep stages:
//   * W rows (fp16, from L2 / MALL) and the stored h entries (INT4 / INT8
//     codes + fp16 scales, or fp16 / fp32 h, from HBM) are loaded one stage
//     ahead into registers; h codes are dequantised to fp16(q * s) on the way
//     into LDS, so the MFMA operands are exactly the dequantised cache values;
//   * both tiles sit in LDS (double buffered, rows padded to 144 B so the
//     16-byte fragment reads of 16 lanes hit disjoint banks);
//   * four waves, 2 x 2, each own a 128 x 128 tile (fp16: 4 x 4
//     v_mfma_f32_32x32x16_f16 blocks, 256 accumulators per lane).
// The decode epilogue reads the scores q . K_j out of the MFMA accumulator
// layout (features in rows, positions in columns, so each lane holds one
// position), applies a wave-level online softmax and reduces p_j V_j across
// lanes, writing (max, sum, o) per (row, head, 128-position split).
#include "tl_device.h"

namespace tl {

namespace {

template <typename T> struct Cfg;
template <> struct Cfg<half_t> {
  static constexpr int BF = 256, BJ = 256, WF = 128, WJ = 128, BK = 64;
};
template <> struct Cfg<float> {
  static constexpr int BF = 128, BJ = 128, WF = 64, WJ = 64, BK = 64;
};

enum { EPI_ATTN = 0, EPI_KVSTORE = 1 };

template <typename T> struct Mma;
template <> struct Mma<half_t> {
  typedef half8 frag;
  static __device__ __forceinline__ float16v mma(half8 a, half8 b, float16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
typedef float float8v __attribute__((ext_vector_type(8)));
template <> struct Mma<float> {
  typedef float8v frag;
  static __device__ __forceinline__ float16v mma(float8v a, float8v b, float16v c) {
    // element j of lane l stands for k = 8*(l/32) + j in both operands
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
    return c;
  }
};

struct KArgs {
  CacheView cache;
  int layer;
  const void* w_qkv;
  int D, H;
  int n_hg, n_ptiles;
  // decode
  const int32_t* row_lane;
  const int32_t* row_pos;
  const int32_t* status;
  const float* q;
  float* part;
  int S;
  // prefill store
  int lane, T;
  void* kvbuf;
};

// chunks of 16 bytes per thread per stage for the h tile
template <int MODE> struct HLoad;
template <> struct HLoad<TL_CACHE_H_INT4> { static constexpr int NCH = 2, CPP = 2; };
template <> struct HLoad<TL_CACHE_H_INT8> { static constexpr int NCH = 4, CPP = 4; };
template <> struct HLoad<TL_CACHE_H_F16> { static constexpr int NCH = 8, CPP = 8; };
template <> struct HLoad<TL_CACHE_H_F32> { static constexpr int NCH = 8, CPP = 16; };

template <typename T, int MODE, int DH, int EPI>
__global__ __launch_bounds__(256, 1) void recon_kernel(KArgs a) {
  typedef Cfg<T> C;
  constexpr int BF = C::BF, BJ = C::BJ, WF = C::WF, WJ = C::WJ, BK = C::BK;
  constexpr int ES = sizeof(T);
  constexpr int ROWB = BK * ES + 16;          // padded LDS row bytes
  constexpr int RB = WF / 32, CB = WJ / 32;   // MFMA blocks per wave
  constexpr int A_CPR = BK * ES / 16;         // 16-byte chunks per W row per stage
  constexpr int A_NCH = BF * A_CPR / 256;     // per thread
  constexpr int B_NCH = HLoad<MODE>::NCH;
  constexpr int B_CPP = HLoad<MODE>::CPP;     // chunks per position
  static_assert(BJ * B_CPP == 256 * B_NCH, "h tile chunks");
  __shared__ __attribute__((aligned(16))) char smem[2 * (BF + BJ) * ROWB];

  const int tid = threadIdx.x, l = tid & 63, wave = tid >> 6;
  const int wf = wave >> 1, wj = wave & 1;
  const int D = a.D;

  int hg, ptile, r = 0, lane, Tn;
  if (EPI == EPI_ATTN) {
    hg = blockIdx.x % a.n_hg;
    const int rest = blockIdx.x / a.n_hg;
    ptile = rest % a.n_ptiles;
    r = rest / a.n_ptiles;
    lane = a.row_lane[r];
    if (a.status[lane] == TL_LANE_ABORTED) return;
    Tn = a.row_pos[r] + 1;
  } else {
    hg = blockIdx.x % a.n_hg;
    ptile = blockIdx.x / a.n_hg;
    lane = a.lane;
    if (a.status && a.status[lane] == TL_LANE_ABORTED) return;
    Tn = a.T;
  }
  const int j0 = ptile * BJ;
  if (j0 >= Tn) return;

  // ---- W rows of this workgroup's BF features ------------------------------
  const T* W = (const T*)a.w_qkv;
  const T* arow[A_NCH];
#pragma unroll
  for (int i = 0; i < A_NCH; ++i) {
    const int c = tid + 256 * i;
    const int f = c / A_CPR, part = c % A_CPR;
    int wrow;
    if (EPI == EPI_ATTN) {
      // head-interleaved: [K_t | V_t] per head, heads t0, t0 + 1, ...
      const int within = f % (2 * DH);
      const int head = hg * (BF / (2 * DH)) + f / (2 * DH);
      wrow = D * (within < DH ? 1 : 2) + head * DH + (within % DH);
    } else {
      wrow = D + hg * BF + f;   // natural K | V order
    }
    arow[i] = W + (size_t)wrow * D + part * (16 / ES);
  }
  // ---- h entries of this workgroup's BJ positions ----------------------------
  const CacheView& cv = a.cache;
  int bpos[B_NCH], bpart[B_NCH];
  bool bok[B_NCH];
#pragma unroll
  for (int i = 0; i < B_NCH; ++i) {
    const int c = tid + 256 * i;
    bpos[i] = c / B_CPP;
    bpart[i] = c % B_CPP;
    bok[i] = j0 + bpos[i] < Tn;
  }
  half_t s8[B_NCH];   // INT8: per-position scale, fixed over the k loop
  if (MODE == TL_CACHE_H_INT8) {
#pragma unroll
    for (int i = 0; i < B_NCH; ++i)
      s8[i] = bok[i] ? h_from_bits(*cv.int8_scale(a.layer, lane, j0 + bpos[i])) : (half_t)0.f;
  }

  u32x4 ra[A_NCH], rb[B_NCH];
  uint16_t rs[B_NCH];
  auto load_stage = [&](int st) {
    const int k0 = st * BK;
#pragma unroll
    for (int i = 0; i < A_NCH; ++i) ra[i] = *(const u32x4*)(arow[i] + k0);
    const int kb = k0 / kKBlock;
#pragma unroll
    for (int i = 0; i < B_NCH; ++i) {
      if (bok[i]) {
        const char* p = cv.code_row(a.layer, lane, kb, j0 + bpos[i]) + bpart[i] * 16;
        rb[i] = *(const u32x4*)p;
        if (MODE == TL_CACHE_H_INT4) rs[i] = cv.int4_scale(a.layer, lane, kb, j0 + bpos[i])[bpart[i]];
      } else {
        rb[i] = u32x4{0u, 0u, 0u, 0u};
        rs[i] = 0;
      }
    }
  };
  auto store_stage = [&](int buf) {
    char* As = smem + buf * (BF + BJ) * ROWB;
    char* Bs = As + BF * ROWB;
#pragma unroll
    for (int i = 0; i < A_NCH; ++i) {
      const int c = tid + 256 * i;
      *(u32x4*)(As + (c / A_CPR) * ROWB + (c % A_CPR) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_NCH; ++i) {
      char* dst = Bs + bpos[i] * ROWB;
      if (MODE == TL_CACHE_H_INT4) {
        const half_t s = h_from_bits(rs[i]);
#pragma unroll
        for (int w = 0; w < 4; ++w)
          *(half8*)(dst + bpart[i] * 64 + w * 16) = int4_dequant8(rb[i][w], s);
      } else if (MODE == TL_CACHE_H_INT8) {
#pragma unroll
        for (int w = 0; w < 4; w += 2) {
          const half4 lo = int8_dequant4(rb[i][w], s8[i]);
          const half4 hi = int8_dequant4(rb[i][w + 1], s8[i]);
          half8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          *(half8*)(dst + bpart[i] * 32 + w * 8) = v;
        }
      } else {
        *(u32x4*)(dst + bpart[i] * 16) = rb[i];
      }
    }
  };

  float16v acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = float16v{};

  // waves whose positions all lie past T have an all-zero tile and skip the epilogue
  const bool wave_live = j0 + wj * WJ < Tn;
  const int nst = D / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) load_stage(st + 1);
    {
      const char* As = smem + (st & 1) * (BF + BJ) * ROWB;
      const char* Bs = As + BF * ROWB;
      const int koff = 8 * (l >> 5) * ES;
#pragma unroll 1
      for (int kk = 0; kk < BK / 16; ++kk) {
        typename Mma<T>::frag fa[RB], fb[CB];
#pragma unroll
        for (int i = 0; i < RB; ++i)
          fa[i] = *(const typename Mma<T>::frag*)(As + (wf * WF + i * 32 + (l & 31)) * ROWB + kk * 16 * ES + koff);
#pragma unroll
        for (int j = 0; j < CB; ++j)
          fb[j] = *(const typename Mma<T>::frag*)(Bs + (wj * WJ + j * 32 + (l & 31)) * ROWB + kk * 16 * ES + koff);
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
          for (int j = 0; j < CB; ++j) acc[i][j] = Mma<T>::mma(fa[i], fb[j], acc[i][j]);
      }
    }
    if (st + 1 < nst) store_stage((st + 1) & 1);
    __syncthreads();
  }

  // ---- epilogues -------------------------------------------------------------
  // accumulator element i of block (rb, cb) in lane l:
  //   feature row = rb*32 + 8*(i/4) + 4*(l/32) + i%4, position col = cb*32 + l%32
  const int half_id = l >> 5;
  if (EPI == EPI_KVSTORE) {
    if (!wave_live) return;
    float* out = (float*)a.kvbuf;
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int pos = j0 + wj * WJ + j * 32 + (l & 31);
      if (pos >= Tn) continue;
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int f = hg * BF + wf * WF + i * 32 + 8 * g4 + 4 * half_id;
          float* dst = out + (size_t)pos * 2 * D + f;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = acc[i][j][4 * g4 + e];
        }
    }
    return;
  }

  constexpr float kLog2e = 1.4426950408889634f;
  const int split = ptile * (BJ / WJ) + wj;
  constexpr bool kCross = 2 * DH > WF;
  constexpr int HPW = kCross ? 1 : WF / (2 * DH);   // heads per wave
  constexpr int KB = DH / 32;                        // row blocks per K (or V) of a head

  auto scores = [&](int rb0, int head, float (&s)[CB]) {
    const float* qh = a.q + (size_t)r * D + head * DH;
#pragma unroll
    for (int j = 0; j < CB; ++j) s[j] = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float qv = qh[kb * 32 + 8 * (i >> 2) + 4 * half_id + (i & 3)];
#pragma unroll
        for (int j = 0; j < CB; ++j) s[j] = fmaf(qv, acc[rb0 + kb][j][i], s[j]);
      }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      s[j] += __shfl_xor(s[j], 32, 64);
      const int pos = j0 + wj * WJ + j * 32 + (l & 31);
      if (pos >= Tn) s[j] = -__builtin_inff();
    }
  };
  auto softmax = [&](float (&s)[CB], float& m, float& lsum) {
    m = s[0];
#pragma unroll
    for (int j = 1; j < CB; ++j) m = fmaxf(m, s[j]);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    lsum = 0.f;
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      s[j] = s[j] == -__builtin_inff() ? 0.f : exp2f((s[j] - m) * kLog2e);
      lsum += s[j];
    }
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o, 64);
  };
  // o over V blocks rb0 .. rb0+KB-1 with weights p, reduced over the 32 lanes
  // of each half and written to the partial of (r, head, split).
  auto values = [&](int rb0, int head, const float (&p)[CB], float m, float lsum) {
    constexpr int NV = KB * 16;
    float v[NV];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < CB; ++j) t = fmaf(p[j], acc[rb0 + kb][j][i], t);
        v[kb * 16 + i] = t;
      }
    // reduce-scatter across lane bits 4..0
    int len = NV;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) {
      if (len >= 2) {
        const int hl = len >> 1;
        const bool up = (l & o) != 0;
#pragma unroll
        for (int e = 0; e < NV / 2; ++e) {
          if (e < hl) {
            const float keep = up ? v[e + hl] : v[e];
            const float send = up ? v[e] : v[e + hl];
            v[e] = keep + __shfl_xor(send, o, 64);
          }
        }
        len = hl;
      } else {
        v[0] += __shfl_xor(v[0], o, 64);
      }
    }
    float* dst = a.part + (((size_t)r * a.H + head) * a.S + split) * (DH + 2);
    if (l == 0) { dst[0] = m; dst[1] = lsum; }
    constexpr int FL = NV >= 32 ? NV / 32 : 1;
    if (NV >= 32 || (l & 1) == 0) {
#pragma unroll
      for (int k = 0; k < FL; ++k) {
        const int idx = NV >= 32 ? (l & 31) * FL + k : (l & 31) >> 1;
        const int kb = idx >> 4, i = idx & 15;
        dst[2 + kb * 32 + 8 * (i >> 2) + 4 * half_id + (i & 3)] = v[k];
      }
    }
  };

  if constexpr (!kCross) {
    if (!wave_live) return;
#pragma unroll
    for (int g = 0; g < HPW; ++g) {
      const int head = hg * (BF / (2 * DH)) + wf * HPW + g;
      float s[CB], m, lsum;
      scores(g * 2 * KB, head, s);
      softmax(s, m, lsum);
      values(g * 2 * KB + KB, head, s, m, lsum);
    }
  } else {
    // K rows live in wave wf = 0, V rows in wf = 1 (same positions): pass the
    // weights p through LDS.
    float* ex = (float*)smem;               // [2][WJ] p, then [2][2] (m, l)
    const int head = hg;
    __syncthreads();
    if (wf == 0 && wave_live) {
      float s[CB], m, lsum;
      scores(0, head, s);
      softmax(s, m, lsum);
      if (l < 32)
#pragma unroll
        for (int j = 0; j < CB; ++j) ex[wj * WJ + j * 32 + l] = s[j];
      if (l == 0) { ex[2 * WJ + 2 * wj] = m; ex[2 * WJ + 2 * wj + 1] = lsum; }
    }
    __syncthreads();
    if (wf == 1 && wave_live) {
      float p[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) p[j] = ex[wj * WJ + j * 32 + (l & 31)];
      values(0, head, p, ex[2 * WJ + 2 * wj], ex[2 * WJ + 2 * wj + 1]);
    }
  }
}

template <typename T, int MODE, int DH>
hipError_t launch_mode(const KArgs& k, int grid, hipStream_t s, int epi) {
  if (epi == EPI_ATTN) recon_kernel<T, MODE, DH, EPI_ATTN><<<grid, 256, 0, s>>>(k);
  else recon_kernel<T, MODE, DH, EPI_KVSTORE><<<grid, 256, 0, s>>>(k);
  return hipGetLastError();
}

hipError_t dispatch(const ModelView& m, const KArgs& k, int grid, hipStream_t s, int epi) {
  if (m.dtype == TL_DTYPE_F32) {
    if (m.dh == 32 && k.cache.mode == TL_CACHE_H_F32)
      return launch_mode<float, TL_CACHE_H_F32, 32>(k, grid, s, epi);
    return hipErrorInvalidValue;
  }
  const int mode = k.cache.mode;
#define TL_RECON_CASE(MODE_, DH_) \
  if (mode == MODE_ && m.dh == DH_) return launch_mode<half_t, MODE_, DH_>(k, grid, s, epi);
  TL_RECON_CASE(TL_CACHE_H_INT4, 64)
  TL_RECON_CASE(TL_CACHE_H_INT4, 128)
  TL_RECON_CASE(TL_CACHE_H_INT8, 64)
  TL_RECON_CASE(TL_CACHE_H_INT8, 128)
  TL_RECON_CASE(TL_CACHE_H_F16, 64)
  TL_RECON_CASE(TL_CACHE_H_F16, 128)
#undef TL_RECON_CASE
  return hipErrorInvalidValue;
}

}  // namespace

int recon_split_len(const ModelView& m) {
  return m.dtype == TL_DTYPE_F32 ? Cfg<float>::WJ : Cfg<half_t>::WJ;
}

hipError_t launch_recon_attn(const ModelView& m, const ReconArgs& r, hipStream_t s) {
  const int BF = m.dtype == TL_DTYPE_F32 ? Cfg<float>::BF : Cfg<half_t>::BF;
  const int BJ = m.dtype == TL_DTYPE_F32 ? Cfg<float>::BJ : Cfg<half_t>::BJ;
  KArgs k{};
  k.cache = r.cache;
  k.layer = r.layer;
  k.w_qkv = r.w_qkv;
  k.D = m.D;
  k.H = m.H;
  k.n_hg = 2 * m.D / BF;
  k.n_ptiles = (r.t_ub + BJ - 1) / BJ;
  k.row_lane = r.row_lane;
  k.row_pos = r.row_pos;
  k.status = r.status;
  k.q = r.q;
  k.part = r.part;
  k.S = r.S;
  const long grid = (long)k.n_hg * k.n_ptiles * r.n_rows;
  if (grid <= 0 || grid > (1L << 30)) return hipErrorInvalidValue;
  return dispatch(m, k, (int)grid, s, EPI_ATTN);
}

hipError_t launch_recon_store(const ModelView& m, const CacheView& c, int layer, int lane, int T,
                              const void* w_qkv, void* kvbuf, const int32_t* status,
                              hipStream_t s) {
  const int BF = m.dtype == TL_DTYPE_F32 ? Cfg<float>::BF : Cfg<half_t>::BF;
  const int BJ = m.dtype == TL_DTYPE_F32 ? Cfg<float>::BJ : Cfg<half_t>::BJ;
  KArgs k{};
  k.cache = c;
  k.layer = layer;
  k.w_qkv = w_qkv;
  k.D = m.D;
  k.H = m.H;
  k.n_hg = 2 * m.D / BF;
  k.n_ptiles = (T + BJ - 1) / BJ;
  k.lane = lane;
  k.T = T;
  k.status = status;
  k.kvbuf = kvbuf;
  return dispatch(m, k, k.n_hg * k.n_ptiles, s, EPI_KVSTORE);
}

}  // namespace tl
