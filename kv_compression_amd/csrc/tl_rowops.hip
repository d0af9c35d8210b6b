// Row-wise kernels of the decode step: setup + embedding gather, RMSNorm +
// h encode + cache append, residual-norm safety check, argmax/finish, and the
// cache test hooks.
//
// The h codec follows the INT8-h / INT4-h store-h modes (TinyLoop
// architecture-exclusive features page, "Store-h KV cache"): symmetric absmax
// with an fp16 scale, one scale per token (INT8) or per 32 consecutive d_model
// elements (INT4), codes clamp(rint(h / s)) computed with an IEEE fp32 divide
// and round-half-to-even.
#include "tl_device.h"

namespace tl {

namespace {

constexpr int kRowThreads = 256;

template <typename T>
__global__ __launch_bounds__(kRowThreads) void step_setup_kernel(ModelView m, Workspace ws,
                                                                 StepMap map,
                                                                 const int32_t* tokens_in,
                                                                 int l_max) {
  const int r = blockIdx.x;
  const int lane = map.lane[r], slot = map.slot[r];
  const int st = ws.status[lane];
  if (threadIdx.x == 0) {
    ws.row_lane[r] = lane;
    ws.row_slot[r] = slot;
    ws.row_pos[r] = st == TL_LANE_ABORTED ? -1 : ws.len[lane];
    ws.row_dead[r] = st == TL_LANE_ABORTED ? 1 : 0;
  }
  if (st == TL_LANE_ABORTED) return;
  for (int i = threadIdx.x; i < l_max; i += blockDim.x) ws.norms[(size_t)lane * l_max + i] = __builtin_nanf("");
  // ids outside [0, vocab) are clamped so the gather stays inside the table
  const int tok = min(max(tokens_in[slot], 0), m.V - 1);
  const T* e = (const T*)m.embed + (size_t)tok * m.D;
  for (int i = threadIdx.x; i < m.D; i += blockDim.x) ws.x[(size_t)r * m.D + i] = to_f(e[i]);
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void prefill_setup_kernel(ModelView m, Workspace ws,
                                                                    int lane, const int32_t* tokens,
                                                                    int pos0) {
  const int r = blockIdx.x;
  if (threadIdx.x == 0) {
    ws.row_lane[r] = lane;
    ws.row_pos[r] = pos0 + r;
    ws.row_dead[r] = ws.status[lane] == TL_LANE_ABORTED ? 1 : 0;
  }
  if (!tokens) return;   // resuming: the caller's residuals are copied in instead
  const int tok = min(max(tokens[r], 0), m.V - 1);
  const T* e = (const T*)m.embed + (size_t)tok * m.D;
  for (int i = threadIdx.x; i < m.D; i += blockDim.x) ws.x[(size_t)r * m.D + i] = to_f(e[i]);
}

// One block per row; thread t owns elements [t*EPT, t*EPT + EPT).
template <typename T, int EPT>
__global__ __launch_bounds__(kRowThreads) void norm_append_kernel(ModelView m, CacheView c,
                                                                  AppendArgs a) {
  __shared__ float red[kRowThreads / 64];
  const int r = blockIdx.x;
  const int lane = a.row_lane ? a.row_lane[r] : a.fixed_lane;
  const int pos = a.row_pos ? a.row_pos[r] : a.pos0 + r;
  if (a.status && a.status[lane] == TL_LANE_ABORTED) return;
  const int D = m.D;
  const int e0 = threadIdx.x * EPT;
  float h[EPT];
  if (a.src == HS_NORM) {
    float xv[EPT];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      xv[i] = a.x[(size_t)r * D + e0 + i];
      ss += xv[i] * xv[i];
    }
    ss = block_sum(ss, red);
    if (a.check_iter >= 0) {
      // safety check of the previous loop iteration (every thread holds the
      // same sum, so the early exit is uniform)
      const float nrm = __fsqrt_rn(ss);
      if (threadIdx.x == 0) a.norms[(size_t)lane * a.l_max + a.check_iter] = nrm;
      if (a.check && !(nrm <= a.thr)) {
        if (threadIdx.x == 0) a.status_w[lane] = TL_LANE_ABORTED;
        return;
      }
    }
    const float inv = __fdiv_rn(1.f, __fsqrt_rn(__fdiv_rn(ss, (float)D) + m.eps));
    const T* g = (const T*)a.gain;
#pragma unroll
    for (int i = 0; i < EPT; ++i) h[i] = to_f(from_f<T>(xv[i] * inv * to_f(g[e0 + i])));
  } else if (a.src == HS_INPUT) {
    const T* hi = (const T*)a.h_in + (size_t)r * D;
#pragma unroll
    for (int i = 0; i < EPT; ++i) h[i] = to_f(hi[e0 + i]);
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      h[i] = to_f(from_f<T>(synth_h(a.seed, a.layer, lane, pos, e0 + i)));
  }
  if (a.h_out) {
    T* ho = (T*)a.h_out + (size_t)r * D;
#pragma unroll
    for (int i = 0; i < EPT; ++i) ho[e0 + i] = from_f<T>(h[i]);
  }
  if (c.mode == TL_CACHE_KV) return;
  float rl[EPT];
  float* rec = rl;
  if (c.mode == TL_CACHE_H_DELTA8) {
    if (a.rec) rec = a.rec + (size_t)r * D + e0;
    else if (a.layer >= c.n_pre) delta_prefix<EPT>(c, a.layer - 1, lane, pos, e0, rl);
  }
  cache_store_h<T, EPT>(c, a.layer, lane, pos, e0, h, [&](float v) { return block_max(v, red); }, rec);
}

// Delta mode: h' = fp16(FP32 prefix sum) of `layer` into layer 0 of the fp16
// tiled view `mat`. Block (x, r): positions x * ppb .. of row r's lane; a
// position's D elements are D / EPT consecutive threads (one contiguous read
// of each code row, 16-byte stores).
template <int EPT>
__global__ __launch_bounds__(256) void delta_mat_kernel(CacheView c, CacheView mat, int layer,
                                                        const int32_t* row_lane,
                                                        const int32_t* row_pos,
                                                        const int32_t* status, int fixed_T,
                                                        int ppb) {
  const int r = blockIdx.y;
  const int lane = row_lane[r];
  if (status && status[lane] == TL_LANE_ABORTED) return;
  const int T = fixed_T > 0 ? fixed_T : row_pos[r] + 1;
  const int tpp = c.D / EPT;
  const int pos = blockIdx.x * ppb + (int)threadIdx.x / tpp;
  if (pos >= T || (int)threadIdx.x >= ppb * tpp) return;
  const int e0 = ((int)threadIdx.x % tpp) * EPT;
  float acc[EPT];
  delta_prefix<EPT>(c, layer, lane, pos, e0, acc);
  half_t* dst = (half_t*)mat.code_row(0, lane, e0 / kKBlock, pos) + e0 % kKBlock;
#pragma unroll
  for (int i = 0; i < EPT; ++i) dst[i] = (half_t)acc[i];
}

template <int EPT>
__global__ __launch_bounds__(256) void delta_rec_kernel(CacheView c, int layer, int lane, int pos0,
                                                        int n, float* rec) {
  const int tpp = c.D / EPT, ppb = 256 / tpp;
  const int i = blockIdx.x * ppb + (int)threadIdx.x / tpp;
  if (i >= n || (int)threadIdx.x >= ppb * tpp) return;
  const int e0 = ((int)threadIdx.x % tpp) * EPT;
  float acc[EPT];
  delta_prefix<EPT>(c, layer, lane, pos0 + i, e0, acc);
#pragma unroll
  for (int k = 0; k < EPT; ++k) rec[(size_t)i * c.D + e0 + k] = acc[k];
}

template <typename T, int EPT>
__global__ __launch_bounds__(kRowThreads) void rmsnorm_kernel(ModelView m, const float* x,
                                                              const void* gain, void* out,
                                                              const int32_t* row_lane,
                                                              const int32_t* status) {
  __shared__ float red[kRowThreads / 64];
  const int r = blockIdx.x;
  if (status && status[row_lane[r]] == TL_LANE_ABORTED) return;
  const int D = m.D, e0 = threadIdx.x * EPT;
  float xv[EPT], ss = 0.f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    xv[i] = x[(size_t)r * D + e0 + i];
    ss += xv[i] * xv[i];
  }
  ss = block_sum(ss, red);
  const float inv = __fdiv_rn(1.f, __fsqrt_rn(__fdiv_rn(ss, (float)D) + m.eps));
  const T* g = (const T*)gain;
  T* o = (T*)out + (size_t)r * D;
#pragma unroll
  for (int i = 0; i < EPT; ++i) o[e0 + i] = from_f<T>(xv[i] * inv * to_f(g[e0 + i]));
}

// argmax with ties to the lowest index: (value, index) pairs, larger value
// wins, equal values keep the smaller index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
__device__ int block_argmax(const float* lg, int V) {
  __shared__ float sv[kRowThreads / 64];
  __shared__ int si[kRowThreads / 64];
  // eight independent (value, index) pairs so the loads of a thread are all in
  // flight together; the merge (larger value, then lower index) is
  // order-independent, so the result is the same as a sequential scan
  float bv[8];
  int bx[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) { bv[u] = -__builtin_inff(); bx[u] = 0x7fffffff; }
  const int step = blockDim.x;
  int j = threadIdx.x;
  for (; j + 7 * step < V; j += 8 * step) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = lg[j + u * step];
#pragma unroll
    for (int u = 0; u < 8; ++u) argmax_merge(bv[u], bx[u], v[u], j + u * step);
  }
  for (; j < V; j += step) argmax_merge(bv[0], bx[0], lg[j], j);
  float best = bv[0];
  int bi = bx[0];
#pragma unroll
  for (int u = 1; u < 8; ++u) argmax_merge(best, bi, bv[u], bx[u]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(best, o, 64);
    const int i2 = __shfl_xor(bi, o, 64);
    argmax_merge(best, bi, v2, i2);
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = best; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  float b = sv[0];
  int ib = si[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) argmax_merge(b, ib, sv[w], si[w]);
  return ib == 0x7fffffff ? 0 : ib;
}

// End of a decode step, one workgroup of kFinishThreads per row: the safety
// check of the row's last loop iteration on its final residual (the norm is
// recorded; a failure, NaN included, stops the lane, whose logits from the LM
// head are then replaced by NaN), the row's token (the argmax of its logits,
// ties to the lowest index), the residual kept for a later resume, the lane's
// new length and the step's outputs.
// Every thread issues its kFinishLoads logit loads of a batch together (one
// batch covers a 32768-entry vocabulary); each thread, then each wave, then
// the waves in order merge (value, index) pairs, and since that merge (larger
// value, then lower index) does not depend on the order, the token is the one
// a sequential scan finds.
constexpr int kFinishThreads = 1024, kFinishLoads = 32;
__global__ __launch_bounds__(kFinishThreads) void finish_kernel(ModelView m, Workspace ws,
                                                                const float* logits, int ld,
                                                                int by_slot, int32_t* tokens_out,
                                                                int32_t* lane_status,
                                                                float* user_logits, NormCheck chk) {
  __shared__ float sv[kFinishThreads / 64];
  __shared__ int si[kFinishThreads / 64];
  const int r = blockIdx.x;
  const int lane = ws.row_lane[r], slot = ws.row_slot[r];
  const bool started = ws.row_pos[r] >= 0;
  bool stopped = ws.status[lane] == TL_LANE_ABORTED;
  if (!stopped) {
    float ss = 0.f;
    for (int i = threadIdx.x; i < m.D; i += blockDim.x) {
      const float v = ws.x[(size_t)r * m.D + i];
      ss += v * v;
    }
    ss = block_sum(ss, sv);
    const float nrm = __fsqrt_rn(ss);
    if (threadIdx.x == 0) chk.norms[(size_t)lane * chk.l_max + chk.iter[r]] = nrm;
    if (chk.check && !(nrm <= chk.thr)) {
      stopped = true;
      if (threadIdx.x == 0) ws.status[lane] = TL_LANE_ABORTED;
    }
    __syncthreads();   // sv is reused below
  }
  if (stopped) {
    if (threadIdx.x == 0) { tokens_out[slot] = -1; lane_status[slot] = TL_LANE_ABORTED; }
    if (user_logits)
      for (int j = threadIdx.x; j < m.V; j += blockDim.x)
        user_logits[(size_t)slot * m.V + j] = __builtin_nanf("");
    if (started)
      for (int i = threadIdx.x; i < m.D; i += blockDim.x)
        ws.xres[(size_t)lane * m.D + i] = ws.x[(size_t)r * m.D + i];
    return;
  }
  const float* lg = logits + (size_t)(by_slot ? slot : r) * ld;
  float best = -__builtin_inff();
  int bi = 0x7fffffff;
  for (int base = 0; base < m.V; base += kFinishThreads * kFinishLoads) {
    float v[kFinishLoads];
#pragma unroll
    for (int u = 0; u < kFinishLoads; ++u) {
      const int j = base + u * kFinishThreads + (int)threadIdx.x;
      v[u] = j < m.V ? lg[j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kFinishLoads; ++u) {
      const int j = base + u * kFinishThreads + (int)threadIdx.x;
      if (j < m.V) argmax_merge(best, bi, v[u], j);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(best, o, 64);
    const int i2 = __shfl_xor(bi, o, 64);
    argmax_merge(best, bi, v2, i2);
  }
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = best; si[threadIdx.x >> 6] = bi; }
  for (int i = threadIdx.x; i < m.D; i += blockDim.x)
    ws.xres[(size_t)lane * m.D + i] = ws.x[(size_t)r * m.D + i];
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = sv[0];
    int ib = si[0];
    for (int w = 1; w < kFinishThreads / 64; ++w) argmax_merge(b, ib, sv[w], si[w]);
    tokens_out[slot] = ib == 0x7fffffff ? 0 : ib;
    lane_status[slot] = TL_LANE_OK;
    ws.len[lane] = ws.row_pos[r] + 1;
  }
}

__global__ __launch_bounds__(kRowThreads) void prefill_finish_kernel(ModelView m, Workspace ws,
                                                                     int lane, int new_len,
                                                                     const float* logits,
                                                                     int32_t* next_token) {
  if (ws.status[lane] == TL_LANE_ABORTED) {
    if (threadIdx.x == 0 && next_token) *next_token = -1;
    return;
  }
  const int tok = block_argmax(logits, m.V);
  if (threadIdx.x == 0) {
    if (next_token) *next_token = tok;
    ws.len[lane] = new_len;
  }
}

// One block per verification row: the verifier's greedy token after it.
__global__ __launch_bounds__(kRowThreads) void spec_argmax_kernel(ModelView m, Workspace ws,
                                                                  int lane, const float* logits) {
  if (ws.status[lane] == TL_LANE_ABORTED) return;
  const int r = blockIdx.x;
  const int tok = block_argmax(logits + (size_t)r * m.V, m.V);
  if (threadIdx.x == 0) ws.spec[kSpecRows + r] = tok;
}

__global__ void spec_accept_kernel(Workspace ws, int lane, int pos0, int k, int32_t* tokens_out) {
  const int32_t* drafted = ws.spec;               // [0] the round's input token, [1..k] drafts
  const int32_t* verified = ws.spec + kSpecRows;  // [j]: the verifier's token after row j
  int n = 0;
  if (ws.status[lane] != TL_LANE_ABORTED) {
    int acc = 0;
    while (acc < k && drafted[acc + 1] == verified[acc]) ++acc;
    n = acc + 1;
  }
  const int j = threadIdx.x;
  if (j <= k) tokens_out[j] = j < n ? verified[j] : -1;
  if (j == 0) {
    ws.spec[2 * kSpecRows] = n;
    if (n) ws.len[lane] = pos0 + n;
  }
}

__global__ void lane_reset_kernel(Workspace ws, int l0, int n, int l_max, int length) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    ws.len[l0 + i] = length;
    ws.status[l0 + i] = TL_LANE_OK;
  }
  for (int j = i; j < n * l_max; j += gridDim.x * blockDim.x)
    ws.norms[(size_t)l0 * l_max + j] = __builtin_nanf("");
}

__global__ void fill_i32_kernel(int32_t* p, int n, int v) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

// One block per (row); threads over d_model.
template <typename T>
__global__ void cache_read_kernel(ModelView m, CacheView c, int lane, int layer, int pos0,
                                  int8_t* codes, uint16_t* scales, void* hout) {
  const int r = blockIdx.x, pos = pos0 + r, D = m.D;
  if (c.mode == TL_CACHE_H_DELTA8) {
    for (int e = threadIdx.x; e < D; e += blockDim.x) {
      float acc[1];
      delta_prefix<1>(c, layer, lane, pos, e, acc);
      if (hout) ((T*)hout)[(size_t)r * D + e] = from_f<T>(acc[0]);
      if (layer < c.n_pre) continue;
      if (codes) codes[(size_t)r * D + e] = c.delta_codes(layer, lane, pos)[e];
      if (scales && e % c.dh == 0) scales[(size_t)r * c.H + e / c.dh] = c.delta_scales(layer, lane, pos)[e / c.dh];
    }
    return;
  }
  if (c.mode == TL_CACHE_KV) {
    if (!hout) return;
    const T* src = (const T*)c.kv_row(layer, lane, pos);
    for (int e = threadIdx.x; e < 2 * D; e += blockDim.x) ((T*)hout)[(size_t)r * 2 * D + e] = src[e];
    return;
  }
  for (int e = threadIdx.x; e < D; e += blockDim.x) {
    const int kb = e / kKBlock, w = e % kKBlock;
    const char* row = c.code_row(layer, lane, kb, pos);
    if (c.mode == TL_CACHE_H_F32 || c.mode == TL_CACHE_H_F16) {
      if (hout) ((T*)hout)[(size_t)r * D + e] = ((const T*)row)[w];
      continue;
    }
    int q;
    half_t s;
    if (c.mode == TL_CACHE_H_INT8) {
      q = ((const int8_t*)row)[code_group(w) * 8 + (w & 7)];
      s = h_from_bits(*c.int8_scale(layer, lane, pos));
      if (scales && e == 0) scales[r] = h_bits(s);
    } else {
      const uint32_t word = ((const uint32_t*)row)[code_group(w)];
      q = (int)((word >> int4_shift(w & 7)) & 0xF) - 8;
      const int g = e / kInt4Group;
      s = h_from_bits(c.int4_scale(layer, lane, kb, pos)[g & 1]);
      if (scales && (e % kInt4Group) == 0) scales[(size_t)r * (D / kInt4Group) + g] = h_bits(s);
    }
    if (codes) codes[(size_t)r * D + e] = (int8_t)q;
    if (hout) ((T*)hout)[(size_t)r * D + e] = (half_t)((float)q * (float)s);
  }
}

__global__ void copy_f32_kernel(const float* src, float* dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

int row_threads(int D) { return D < kRowThreads ? D : kRowThreads; }

}  // namespace

hipError_t launch_step_setup(const ModelView& m, const Workspace& ws, const StepMap& map,
                             const int32_t* tokens_in, int l_max, hipStream_t s) {
  if (m.dtype == TL_DTYPE_F32)
    step_setup_kernel<float><<<map.n, kRowThreads, 0, s>>>(m, ws, map, tokens_in, l_max);
  else
    step_setup_kernel<half_t><<<map.n, kRowThreads, 0, s>>>(m, ws, map, tokens_in, l_max);
  return hipGetLastError();
}

hipError_t launch_prefill_setup(const ModelView& m, const Workspace& ws, int lane, int n,
                                const int32_t* tokens, int pos0, hipStream_t s) {
  if (m.dtype == TL_DTYPE_F32)
    prefill_setup_kernel<float><<<n, kRowThreads, 0, s>>>(m, ws, lane, tokens, pos0);
  else
    prefill_setup_kernel<half_t><<<n, kRowThreads, 0, s>>>(m, ws, lane, tokens, pos0);
  return hipGetLastError();
}

hipError_t launch_norm_append(const ModelView& m, const CacheView& c, const AppendArgs& a,
                              hipStream_t s) {
  const int nt = row_threads(m.D);
  const int ept = m.D / nt;
  if (m.dtype == TL_DTYPE_F32) {
    if (ept != 1) return hipErrorInvalidValue;
    norm_append_kernel<float, 1><<<a.n, nt, 0, s>>>(m, c, a);
  } else if (ept == 1) {
    norm_append_kernel<half_t, 1><<<a.n, nt, 0, s>>>(m, c, a);
  } else if (ept == 4) {
    norm_append_kernel<half_t, 4><<<a.n, nt, 0, s>>>(m, c, a);
  } else if (ept == 8) {
    norm_append_kernel<half_t, 8><<<a.n, nt, 0, s>>>(m, c, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const ModelView& m, int n, const float* x, const void* gain, void* out,
                          const int32_t* row_lane, const int32_t* status, hipStream_t s) {
  const int nt = row_threads(m.D);
  const int ept = m.D / nt;
#define TL_RN(T_, E_) rmsnorm_kernel<T_, E_><<<n, nt, 0, s>>>(m, x, gain, out, row_lane, status)
  if (m.dtype == TL_DTYPE_F32 && ept == 1) TL_RN(float, 1);
  else if (m.dtype == TL_DTYPE_F16 && ept == 1) TL_RN(half_t, 1);
  else if (m.dtype == TL_DTYPE_F16 && ept == 4) TL_RN(half_t, 4);
  else if (m.dtype == TL_DTYPE_F16 && ept == 8) TL_RN(half_t, 8);
  else return hipErrorInvalidValue;
#undef TL_RN
  return hipGetLastError();
}

hipError_t launch_finish(const ModelView& m, const Workspace& ws, int n, const float* logits,
                         int ld_logits, int logits_by_slot, int32_t* tokens_out,
                         int32_t* lane_status, float* user_logits, const NormCheck& chk,
                         hipStream_t s) {
  finish_kernel<<<n, kFinishThreads, 0, s>>>(m, ws, logits, ld_logits, logits_by_slot, tokens_out,
                                             lane_status, user_logits, chk);
  return hipGetLastError();
}

hipError_t launch_prefill_finish(const ModelView& m, const Workspace& ws, int lane, int new_len,
                                 const float* logits, int32_t* next_token, hipStream_t s) {
  prefill_finish_kernel<<<1, kRowThreads, 0, s>>>(m, ws, lane, new_len, logits, next_token);
  return hipGetLastError();
}

hipError_t launch_spec_accept(const ModelView& m, const Workspace& ws, int lane, int pos0, int k,
                              const float* logits, int32_t* tokens_out, hipStream_t s) {
  if (k < 1 || k > kSpecMax) return hipErrorInvalidValue;
  spec_argmax_kernel<<<k + 1, kRowThreads, 0, s>>>(m, ws, lane, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  spec_accept_kernel<<<1, 64, 0, s>>>(ws, lane, pos0, k, tokens_out);
  return hipGetLastError();
}

// elements per thread of the delta kernels: 8 (16-byte fp16 stores) when a
// position's threads fit a block and 8 divides the head width
static int delta_ept(const CacheView& c) {
  return (c.D / 8 <= 256 && c.dh % 8 == 0) ? 8 : (c.D / 4 <= 256 && c.dh % 4 == 0) ? 4 : 0;
}

hipError_t launch_delta_mat(const CacheView& c, const CacheView& mat, int layer,
                            const int32_t* row_lane, const int32_t* row_pos,
                            const int32_t* status, int n_rows, int t_ub, int fixed_T,
                            hipStream_t s) {
  const int ept = delta_ept(c);
  if (!ept || n_rows < 1 || t_ub < 1 || layer < 0 || layer >= c.n_layers) return hipErrorInvalidValue;
  const int ppb = 256 / (c.D / ept);
  const dim3 grid((t_ub + ppb - 1) / ppb, n_rows);
  if (ept == 8)
    delta_mat_kernel<8><<<grid, 256, 0, s>>>(c, mat, layer, row_lane, row_pos, status, fixed_T, ppb);
  else
    delta_mat_kernel<4><<<grid, 256, 0, s>>>(c, mat, layer, row_lane, row_pos, status, fixed_T, ppb);
  return hipGetLastError();
}

hipError_t launch_delta_rec(const CacheView& c, int layer, int lane, int pos0, int n, float* rec,
                            hipStream_t s) {
  const int ept = delta_ept(c);
  if (!ept || n < 1 || layer < c.n_pre - 1 || layer >= c.n_layers) return hipErrorInvalidValue;
  const int ppb = 256 / (c.D / ept);
  const int grid = (n + ppb - 1) / ppb;
  if (ept == 8)
    delta_rec_kernel<8><<<grid, 256, 0, s>>>(c, layer, lane, pos0, n, rec);
  else
    delta_rec_kernel<4><<<grid, 256, 0, s>>>(c, layer, lane, pos0, n, rec);
  return hipGetLastError();
}

hipError_t launch_lane_reset(const Workspace& ws, int l0, int n, int l_max, int length,
                             hipStream_t s) {
  const int blocks = (n * l_max + 255) / 256 + 1;
  lane_reset_kernel<<<blocks < 1024 ? blocks : 1024, 256, 0, s>>>(ws, l0, n, l_max, length);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int n, int v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (n + 255) / 256;
  fill_i32_kernel<<<blocks < 1024 ? blocks : 1024, 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_cache_read(const ModelView& m, const CacheView& c, int lane, int layer, int pos0,
                             int n, int8_t* codes, uint16_t* scales, void* h, hipStream_t s) {
  if (m.dtype == TL_DTYPE_F32)
    cache_read_kernel<float><<<n, 256, 0, s>>>(m, c, lane, layer, pos0, codes, scales, h);
  else
    cache_read_kernel<half_t><<<n, 256, 0, s>>>(m, c, lane, layer, pos0, codes, scales, h);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t s) {
  const size_t blocks = (n + 255) / 256;
  copy_f32_kernel<<<blocks < 1024 ? (unsigned)blocks : 1024u, 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

}  // namespace tl
