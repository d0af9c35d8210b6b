// Matrix products of the step: Y[row, f] = sum_k W[f, k] X[row, k] with the
// weights in their natural [out, in] layout, for the Q / QKV, W_o, MLP and LM
// head projections (TinyLoop architecture-exclusive features page,
// introduction: the loop block's W_q, W_k, W_v, W_o and MLP matrices).
//
// Decode runs them with a handful of rows (one per active lane), so the kernel
// is built for weight streaming: a workgroup owns 16 output features and up to
// 64 rows; its four waves split the reduction dimension into four contiguous
// quarters, each issuing 16-byte row loads of W straight into
// v_mfma_f32_16x16x32_f16 operands (fp32 models: eight v_mfma_f32_16x16x4_f32
// per 32-deep step), and the quarters are summed in LDS in a fixed order. The
// result of an output element therefore never depends on how many rows the
// call has or where the row sits in it.
#include "tl_device.h"

namespace tl {

namespace {

constexpr int kRowsPerBlock = 64;

template <typename T> struct Frag;
template <> struct Frag<half_t> {
  typedef half8 type;
  static __device__ __forceinline__ half8 load(const half_t* p) { return *(const half8*)p; }
  static __device__ __forceinline__ half8 zero() { return half8{}; }
  static __device__ __forceinline__ float4v mma(half8 a, half8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
typedef float float8v __attribute__((ext_vector_type(8)));
template <> struct Frag<float> {
  typedef float8v type;
  static __device__ __forceinline__ float8v load(const float* p) { return *(const float8v*)p; }
  static __device__ __forceinline__ float8v zero() { return float8v{}; }
  static __device__ __forceinline__ float4v mma(float8v a, float8v b, float4v c) {
    // lane l holds k = 8*(l/16) + j in element j of both operands; eight 4-deep
    // products cover the 32-deep step.
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
  }
};

template <typename T, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& g, int D, int row, int f, float v) {
  if (EPI == EPI_STORE_F32) {
    ((float*)g.out)[(size_t)row * g.ldo + f] = v * g.scale;
  } else if (EPI == EPI_STORE_T) {
    ((T*)g.out)[(size_t)row * g.ldo + f] = from_f<T>(v * g.scale);
  } else if (EPI == EPI_ADD_F32) {
    ((float*)g.out)[(size_t)row * g.ldo + f] += v;
  } else if (EPI == EPI_GELU_T) {
    ((T*)g.out)[(size_t)row * g.ldo + f] = from_f<T>(gelu_f(v));
  } else if (EPI == EPI_LOGITS) {
    const int o = g.row_slot ? g.row_slot[row] : row;
    ((float*)g.out)[(size_t)o * g.ldo + f] = v;
  } else {  // EPI_QKV
    const int fg = f + g.f_offset;
    if (fg < D) {
      if (g.q_is_t) ((T*)g.out)[(size_t)row * g.ldo + fg] = from_f<T>(v * g.scale);
      else ((float*)g.out)[(size_t)row * g.ldo + fg] = v * g.scale;
    } else {
      const int lane = g.row_lane ? g.row_lane[row] : g.fixed_lane;
      const int pos = g.row_pos ? g.row_pos[row] : g.pos0 + row;
      ((T*)g.cache.kv_row(g.layer, lane, pos))[fg - D] = from_f<T>(v);
    }
  }
}

template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(ModelView m, GemmArgs g) {
  __shared__ float4v red[4][4][64];
  typedef Frag<T> F;
  const int f0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * kRowsPerBlock;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int kq = g.K >> 2;
  const int kbeg = wave * kq;
  int ng = (g.M - m0 + 15) >> 4;
  ng = ng > 4 ? 4 : ng;
  const T* W = (const T*)g.W + (size_t)(f0 + (l & 15)) * g.ldw + 8 * (l >> 4) + kbeg;
  const T* X[4];
  bool ok[4];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    const int row = m0 + 16 * gi + (l & 15);
    ok[gi] = row < g.M;
    X[gi] = (const T*)g.X + (size_t)(ok[gi] ? row : 0) * g.ldx + 8 * (l >> 4) + kbeg;
  }
  float4v acc[4] = {};
  // U 32-deep steps per batch: all their loads are issued before the first
  // MFMA, so a wave keeps U weight loads in flight (decode is latency-bound).
  // The MFMAs still run in k order, so the sums do not depend on U.
  constexpr int U = 8;
  for (int k = 0; k < kq; k += 32 * U) {
    typename F::type a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = k + 32 * u < kq ? F::load(W + k + 32 * u) : F::zero();
    if (ng == 1) {
      typename F::type b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) b[u] = (ok[0] && k + 32 * u < kq) ? F::load(X[0] + k + 32 * u) : F::zero();
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (k + 32 * u < kq) acc[0] = F::mma(a[u], b[u], acc[0]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (k + 32 * u >= kq) break;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          if (gi < ng) {
            const typename F::type b = ok[gi] ? F::load(X[gi] + k + 32 * u) : F::zero();
            acc[gi] = F::mma(a[u], b, acc[gi]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) red[wave][gi][l] = acc[gi];
  __syncthreads();
  const int gi = threadIdx.x >> 6;
  if (gi >= ng) return;
  const int row = m0 + 16 * gi + (l & 15);
  if (row >= g.M) return;
  if (g.status && g.status[g.row_lane[row]] == TL_LANE_ABORTED) return;
  float4v v = red[0][gi][l];
  v += red[1][gi][l];
  v += red[2][gi][l];
  v += red[3][gi][l];
  const int fb = f0 + 4 * (l >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) epilogue<T, EPI>(g, m.D, row, fb + i, v[i]);
}

template <typename T>
hipError_t launch_t(const ModelView& m, const GemmArgs& g, hipStream_t s) {
  dim3 grid(g.N / 16, (g.M + kRowsPerBlock - 1) / kRowsPerBlock);
  switch (g.epi) {
    case EPI_STORE_F32: gemm_kernel<T, EPI_STORE_F32><<<grid, 256, 0, s>>>(m, g); break;
    case EPI_STORE_T: gemm_kernel<T, EPI_STORE_T><<<grid, 256, 0, s>>>(m, g); break;
    case EPI_ADD_F32: gemm_kernel<T, EPI_ADD_F32><<<grid, 256, 0, s>>>(m, g); break;
    case EPI_GELU_T: gemm_kernel<T, EPI_GELU_T><<<grid, 256, 0, s>>>(m, g); break;
    case EPI_LOGITS: gemm_kernel<T, EPI_LOGITS><<<grid, 256, 0, s>>>(m, g); break;
    case EPI_QKV: gemm_kernel<T, EPI_QKV><<<grid, 256, 0, s>>>(m, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const ModelView& m, const GemmArgs& g, hipStream_t s) {
  if (g.N % 16 || g.K % 128 || g.M <= 0) return hipErrorInvalidValue;
  return m.dtype == TL_DTYPE_F32 ? launch_t<float>(m, g, s) : launch_t<half_t>(m, g, s);
}

}  // namespace tl
