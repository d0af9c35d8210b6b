// Attention pieces around the reconstruction kernel:
//  * kv_attn: decode attention over stored K|V rows, the stored-K/V baseline
//    the store-h cache is measured against (TinyLoop measured-benchmarks page,
//    section 3, "FP16 KV baseline"); HBM-bound streaming of K and V;
//  * attn_merge: combines the per-split (max, sum, o) partials of one row and
//    head (split-T / flash-decoding merge) in a fixed order;
//  * prefill_attn: causal attention of a prefill chunk over K|V rows (chunked
//    prefill; features page, closing list of supported techniques).
#include "tl_device.h"

namespace tl {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int EPT> struct Vec;
template <> struct Vec<half_t, 4> {
  static __device__ __forceinline__ void load(const half_t* p, float* v) {
    const half4 x = *(const half4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (float)x[i];
  }
};
template <> struct Vec<half_t, 8> {
  static __device__ __forceinline__ void load(const half_t* p, float* v) {
    const half8 x = *(const half8*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
  }
};
template <> struct Vec<float, 1> {
  static __device__ __forceinline__ void load(const float* p, float* v) { v[0] = *p; }
};

// One block per (row, split of kKvSplit positions); thread t owns d_model
// elements [t*EPT, t*EPT + EPT) of q, K and V.
template <typename T, int EPT, int DH>
__global__ __launch_bounds__(256) void kv_attn_kernel(ModelView m, ReconArgs a, int n_splits) {
  constexpr int TPH = DH / EPT;   // threads per head
  const int r = blockIdx.x / n_splits, split = blockIdx.x % n_splits;
  const int lane = a.row_lane[r];
  if (a.status[lane] == TL_LANE_ABORTED) return;
  const int Tn = a.row_pos[r] + 1;
  const int j0 = split * kKvSplit;
  if (j0 >= Tn) return;
  const int jn = min(kKvSplit, Tn - j0);
  const int D = m.D, t = threadIdx.x, e0 = t * EPT, head = e0 / DH;
  float q[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) q[i] = a.q[(size_t)r * D + e0 + i];
  const T* kv = (const T*)a.cache.kv_row(a.layer, lane, j0);
  float mx = -__builtin_inff(), lsum = 0.f, o[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) o[i] = 0.f;
  constexpr int U = 16;
  for (int jj = 0; jj < jn; jj += U) {
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d = 0.f;
      if (jj + u < jn) {
        float k[EPT];
        Vec<T, EPT>::load(kv + (size_t)(jj + u) * 2 * D + e0, k);
#pragma unroll
        for (int i = 0; i < EPT; ++i) d = fmaf(q[i], k[i], d);
      }
      sc[u] = d;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int off = 1; off < TPH; off <<= 1) sc[u] += __shfl_xor(sc[u], off, 64);
      if (jj + u >= jn) sc[u] = -__builtin_inff();
    }
    float cm = sc[0];
#pragma unroll
    for (int u = 1; u < U; ++u) cm = fmaxf(cm, sc[u]);
    const float mn = fmaxf(mx, cm);
    const float corr = mx == -__builtin_inff() ? 0.f : exp2f((mx - mn) * kLog2e);
    lsum *= corr;
#pragma unroll
    for (int i = 0; i < EPT; ++i) o[i] *= corr;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (jj + u < jn) {
        const float p = exp2f((sc[u] - mn) * kLog2e);
        lsum += p;
        float v[EPT];
        Vec<T, EPT>::load(kv + (size_t)(jj + u) * 2 * D + D + e0, v);
#pragma unroll
        for (int i = 0; i < EPT; ++i) o[i] = fmaf(p, v[i], o[i]);
      }
    }
    mx = mn;
  }
  float* dst = a.part + (((size_t)r * m.H + head) * a.S + split) * (DH + 2);
  if ((t % TPH) == 0) { dst[0] = mx; dst[1] = lsum; }
#pragma unroll
  for (int i = 0; i < EPT; ++i) dst[2 + (e0 % DH) + i] = o[i];
}

// One block of 256 threads per (row, head). The split weights exp(m_s - M)
// are computed once per split into LDS; thread (dim, group g) then sums the
// splits s = g, g + G, ... for its dimension, and the G group sums are added
// in order g = 0, 1, ... . The summation order depends only on T.
template <typename T, int DH>
__global__ __launch_bounds__(256) void merge_kernel(int D, int H, const int32_t* row_lane,
                                                    const int32_t* row_pos, const int32_t* status,
                                                    const float* part, int S, int split_len,
                                                    void* out) {
  constexpr int G = 256 / DH, CH = 1024;
  __shared__ float wgt[CH];
  __shared__ float red[4];
  __shared__ float osum[G][DH];
  __shared__ float lsum[G];
  const int r = blockIdx.x / H, head = blockIdx.x % H;
  if (status[row_lane[r]] == TL_LANE_ABORTED) return;
  const int Tn = row_pos[r] + 1;
  const int ns = (Tn + split_len - 1) / split_len;
  const float* p = part + ((size_t)r * H + head) * S * (DH + 2);
  const int t = threadIdx.x, dim = t % DH, g = t / DH;
  float M = -__builtin_inff();
  for (int s = t; s < ns; s += 256) M = fmaxf(M, p[(size_t)s * (DH + 2)]);
  M = block_max(M, red);
  float acc = 0.f, lacc = 0.f;
  for (int c0 = 0; c0 < ns; c0 += CH) {
    const int cend = min(ns, c0 + CH);
    __syncthreads();
    for (int s = c0 + t; s < cend; s += 256) wgt[s - c0] = exp2f((p[(size_t)s * (DH + 2)] - M) * kLog2e);
    __syncthreads();
    for (int s = c0 + g; s < cend; s += G) {
      const float* ps = p + (size_t)s * (DH + 2);
      const float w = wgt[s - c0];
      acc = fmaf(ps[2 + dim], w, acc);
      if (dim == 0) lacc = fmaf(ps[1], w, lacc);
    }
  }
  osum[g][dim] = acc;
  if (dim == 0) lsum[g] = lacc;
  __syncthreads();
  if (g != 0) return;
  float o = 0.f, L = 0.f;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    o += osum[k][dim];
    L += lsum[k];
  }
  ((T*)out)[(size_t)r * D + head * DH + dim] = from_f<T>(__fdiv_rn(o, L));
}

// One block per (head, 64 queries); four threads per query, each owning
// DH/4 dimensions. K|V rows are staged through LDS 32 keys at a time.
template <typename T, typename KT, int DH>
__global__ __launch_bounds__(256) void prefill_attn_kernel(ModelView m, int n, int pos0,
                                                           const float* q, const KT* kv, T* out,
                                                           int lane, const int32_t* status) {
  constexpr int QB = 64, KC = 32, DPT = DH / 4;
  __shared__ float Ks[KC][DH + 1];
  __shared__ float Vs[KC][DH + 1];
  if (status && status[lane] == TL_LANE_ABORTED) return;
  const int D = m.D;
  const int head = blockIdx.x % m.H, qb = blockIdx.x / m.H;
  const int t = threadIdx.x, qi = t >> 2, sub = t & 3;
  const int i = qb * QB + qi;
  const bool qv = i < n;
  const int qpos = pos0 + i;
  float qr[DPT], o[DPT];
#pragma unroll
  for (int d = 0; d < DPT; ++d) {
    qr[d] = qv ? q[(size_t)i * D + head * DH + sub * DPT + d] : 0.f;
    o[d] = 0.f;
  }
  float mx = -__builtin_inff(), lsum = 0.f;
  const int last_q = min(n, qb * QB + QB) - 1;
  const int kend = pos0 + last_q + 1;   // keys 0 .. kend-1
  for (int k0 = 0; k0 < kend; k0 += KC) {
    __syncthreads();
    for (int e = t; e < KC * DH; e += 256) {
      const int kk = e / DH, d = e % DH;
      const int kp = k0 + kk;
      float kvk = 0.f, kvv = 0.f;
      if (kp < kend) {
        kvk = to_f(kv[(size_t)kp * 2 * D + head * DH + d]);
        kvv = to_f(kv[(size_t)kp * 2 * D + D + head * DH + d]);
      }
      Ks[kk][d] = kvk;
      Vs[kk][d] = kvv;
    }
    __syncthreads();
    float sc[KC];
#pragma unroll
    for (int u = 0; u < KC; ++u) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < DPT; ++d) s = fmaf(qr[d], Ks[u][sub * DPT + d], s);
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      sc[u] = (k0 + u <= qpos && k0 + u < kend) ? s : -__builtin_inff();
    }
    float cm = sc[0];
#pragma unroll
    for (int u = 1; u < KC; ++u) cm = fmaxf(cm, sc[u]);
    if (cm == -__builtin_inff()) continue;
    const float mn = fmaxf(mx, cm);
    const float corr = mx == -__builtin_inff() ? 0.f : exp2f((mx - mn) * kLog2e);
    lsum *= corr;
#pragma unroll
    for (int d = 0; d < DPT; ++d) o[d] *= corr;
#pragma unroll
    for (int u = 0; u < KC; ++u) {
      const float p = sc[u] == -__builtin_inff() ? 0.f : exp2f((sc[u] - mn) * kLog2e);
      lsum += p;
#pragma unroll
      for (int d = 0; d < DPT; ++d) o[d] = fmaf(p, Vs[u][sub * DPT + d], o[d]);
    }
    mx = mn;
  }
  if (!qv) return;
#pragma unroll
  for (int d = 0; d < DPT; ++d)
    out[(size_t)i * D + head * DH + sub * DPT + d] = from_f<T>(__fdiv_rn(o[d], lsum));
}

}  // namespace

hipError_t launch_kv_attn(const ModelView& m, const ReconArgs& a, hipStream_t s) {
  const int n_splits = (a.t_ub + kKvSplit - 1) / kKvSplit;
  const int grid = n_splits * a.n_rows;
  if (m.dtype == TL_DTYPE_F32 && m.D == 128 && m.dh == 32)
    kv_attn_kernel<float, 1, 32><<<grid, 128, 0, s>>>(m, a, n_splits);
  else if (m.dtype == TL_DTYPE_F16 && m.D == 1024 && m.dh == 64)
    kv_attn_kernel<half_t, 4, 64><<<grid, 256, 0, s>>>(m, a, n_splits);
  else if (m.dtype == TL_DTYPE_F16 && m.D == 2048 && m.dh == 128)
    kv_attn_kernel<half_t, 8, 128><<<grid, 256, 0, s>>>(m, a, n_splits);
  else if (m.dtype == TL_DTYPE_F16 && m.D == 2048 && m.dh == 64)
    kv_attn_kernel<half_t, 8, 64><<<grid, 256, 0, s>>>(m, a, n_splits);
  else if (m.dtype == TL_DTYPE_F16 && m.D == 1024 && m.dh == 128)
    kv_attn_kernel<half_t, 4, 128><<<grid, 256, 0, s>>>(m, a, n_splits);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attn_merge(const ModelView& m, int n_rows, const int32_t* row_lane,
                             const int32_t* row_pos, const int32_t* status, const float* part,
                             int S, int split_len, void* o, hipStream_t s) {
  const int grid = n_rows * m.H;
#define TL_MG(T_, DH_)                                                                    \
  merge_kernel<T_, DH_><<<grid, 256, 0, s>>>(m.D, m.H, row_lane, row_pos, status, part, S, \
                                              split_len, o)
  if (m.dtype == TL_DTYPE_F32 && m.dh == 32) TL_MG(float, 32);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 64) TL_MG(half_t, 64);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 128) TL_MG(half_t, 128);
  else return hipErrorInvalidValue;
#undef TL_MG
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const ModelView& m, int n, int pos0, const float* q,
                               const void* kv, int kv_f32, void* o, int lane,
                               const int32_t* status, hipStream_t s) {
  const int grid = m.H * ((n + 63) / 64);
#define TL_PA(T_, KT_, DH_)                                                                  \
  prefill_attn_kernel<T_, KT_, DH_><<<grid, 256, 0, s>>>(m, n, pos0, q, (const KT_*)kv, (T_*)o, \
                                                          lane, status)
  if (m.dtype == TL_DTYPE_F32 && m.dh == 32) TL_PA(float, float, 32);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 64 && kv_f32) TL_PA(half_t, float, 64);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 64) TL_PA(half_t, half_t, 64);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 128 && kv_f32) TL_PA(half_t, float, 128);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 128) TL_PA(half_t, half_t, 128);
  else return hipErrorInvalidValue;
#undef TL_PA
  return hipGetLastError();
}

}  // namespace tl
