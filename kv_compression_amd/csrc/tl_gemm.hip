// Matrix products of the step: Y[row, f] = sum_k W[f, k] X[row, k] with the
// weights in their natural [out, in] layout, for the Q / QKV, W_o, MLP and LM
// head projections (TinyLoop architecture-exclusive features page,
// introduction: the loop block's W_q, W_k, W_v, W_o and MLP matrices).
//
// Decode runs them with a handful of rows (one per active lane), so the kernel
// is built for weight streaming: a workgroup owns fb output features (16, or 8
// or 4 when the output is too narrow to give every CU a workgroup; the MFMA
// rows past fb load nothing and are not written) and up to 64 rows; its KS waves split the reduction dimension into KS contiguous
// parts, each issuing 16-byte row loads of W straight into
// v_mfma_f32_16x16x32_f16 operands (fp32 models: eight v_mfma_f32_16x16x4_f32
// per 32-deep step), and the parts are summed in LDS in a fixed order. KS is 4,
// or 16 when there are too few 16-feature groups to give every CU a
// workgroup (the d_model-wide outputs), so that more weight loads are in
// flight. KS depends only on the matrix shape, so the result of an output
// element never depends on how many rows the call has or where the row sits.
//
// With XS_NORM the operand rows are RMSNorm(x) * gain of fp32 residual rows
// (the attention and MLP inputs), formed as x is loaded. The workgroup's waves
// together load every element of its rows, so each row's sum of squares is
// reduced from the operand loads themselves in a fixed order (a lane's own
// elements in k order, then the four lanes of the row, then the waves in
// order), the same in every workgroup and for any batch. For the
// attention input the same kernel does the row work that precedes the
// projection: the safety check of the previous loop iteration on the entering
// residual (every workgroup evaluates it from its own sums, so all agree on
// which rows stop) and the append of h to the cache, one row per workgroup.
#include "tl_device.h"

namespace tl {

namespace {

constexpr int kRowsPerBlock = 64;
// XS_ONE: plain operand rows, at most 16 of them (one row group), a wave's
// whole k range (NU <= 8 steps) in one batch with the operand rows, and the
// epilogue's inputs (row_dead, the residual it adds to) loaded up front
enum { XS_PLAIN = 0, XS_NORM = 1, XS_ONE = 2 };

// 32-deep steps per load batch: the weight loads a wave keeps in flight.
// With fp32 operand rows (XS_NORM) NU, the exact number of steps of a wave's
// k range, is a template argument and one batch covers it, so the row sums
// can be taken from the operand loads.
constexpr int gemm_batch(int KS, int XS, int NU) {
  return XS != XS_PLAIN ? NU : (KS >= 16 ? 4 : 8);
}

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

// Row work of the attention input for rows m0 .. m0+nrows-1, row m0+r done by
// workgroup r (r, r + gridDim.x, ...): the safety check of loop iteration
// check_iter (norm of the entering residual, written to norms; a failure
// stops the lane) and, in the h modes, h = RMSNorm(x) * gain appended to the
// cache at the row's position. Thread t holds elements t*EPT .. t*EPT+EPT-1.
// The first row's lane status, x and gain elements come prefetched.
template <typename T, int EPT>
struct TaskPre {
  int status;
  float x[EPT];
  T gn[EPT];
};
template <typename T, int EPT>
__device__ __forceinline__ void task_load(const ModelView& m, const GemmArgs& g, int row, TaskPre<T, EPT>& p) {
  const int e0 = threadIdx.x * EPT;
  const float* xr = (const float*)g.X + (size_t)row * g.ldx;
  const T* gn = (const T*)g.norm_gain;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    p.x[i] = e0 < m.D ? xr[e0 + i] : 0.f;
    p.gn[i] = e0 < m.D ? gn[e0 + i] : from_f<T>(0.f);
  }
}
template <typename T, int EPT>
__device__ void row_tasks_ept(const ModelView& m, const GemmArgs& g, int m0, int nrows,
                              const float* rss, const float* rinv, const int* rdead, float* rmax,
                              TaskPre<T, EPT> pre) {
  const int D = m.D, e0 = threadIdx.x * EPT;
  const bool holds = e0 < D;
  for (int rr = blockIdx.x; rr < nrows; rr += gridDim.x) {
    const int row = m0 + rr;
    if (rr != (int)blockIdx.x) {
      pre.status = g.status[g.row_lane[row]];
      task_load<T, EPT>(m, g, row, pre);
    }
    // rows that had stopped before this layer (at an earlier layer of this
    // step, or before the step) are left alone
    if (g.row_pos[row] < 0 || pre.status == TL_LANE_ABORTED) continue;
    const int lane = g.row_lane[row];
    if (g.check_iter >= 0) {
      const float nrm = __fsqrt_rn(rss[rr]);
      if (threadIdx.x == 0) g.norms[(size_t)lane * g.l_max + g.check_iter] = nrm;
      if (rdead[rr]) {
        if (threadIdx.x == 0) {
          g.status_w[lane] = TL_LANE_ABORTED;
          if (g.row_dead) g.row_dead[row] = 1;
        }
        continue;
      }
    }
    if (g.cache.mode == TL_CACHE_KV) continue;   // the K|V rows are the projection's own output
    float h[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) h[i] = holds ? to_f(from_f<T>(pre.x[i] * rinv[rr] * to_f(pre.gn[i]))) : 0.f;
    auto rowmax = [&](float v) { return block_max(v, rmax); };
    if (holds) {
      cache_store_h<T, EPT>(g.cache, g.layer, lane, g.row_pos[row], e0, h, rowmax,
                            g.rec ? g.rec + (size_t)row * D + e0 : nullptr);
    } else if (g.cache.mode == TL_CACHE_H_INT8) {
      rowmax(0.f);   // threads past the row still join the INT8 scale reduction
    }
  }
}

template <typename T, int EPI, int KS, int XS, int NU>
__global__ __launch_bounds__(64 * KS) void gemm_kernel(ModelView m, GemmArgs g) {
  __shared__ float4v red[KS][4][64];
  __shared__ float rinv[XS == XS_NORM ? kRowsPerBlock : 1];
  __shared__ float rss[XS == XS_NORM ? kRowsPerBlock : 1];
  __shared__ int rdead[XS == XS_NORM ? kRowsPerBlock : 1];
  __shared__ float rmax[XS == XS_NORM ? 16 : 1];
  __shared__ float rpart[XS == XS_NORM ? kRowsPerBlock * KS * 4 : 1];
  typedef Frag<T> F;
  const int fbk = g.fb, f0 = blockIdx.x * fbk;
  const int m0 = blockIdx.y * kRowsPerBlock;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const bool wrow = (l & 15) < fbk;       // this lane's A row is a feature of the block
  const bool wout = 4 * (l >> 4) < fbk;   // this lane's accumulator rows are features of it
  const int kq = g.K / KS;
  const int kbeg = wave * kq;
  int ng = (g.M - m0 + 15) >> 4;
  ng = ng > 4 ? 4 : ng;
  if constexpr (XS == XS_ONE) ng = 1;   // M <= 16
  const T* W = (const T*)g.W + (size_t)(f0 + (wrow ? (l & 15) : 0)) * g.ldw + 8 * (l >> 4) + kbeg;
  // operand rows of the four row groups (fp32 residual rows for XS_NORM)
  typedef typename std::conditional<XS == XS_NORM, float, T>::type XT;
  const XT* X[4];
  bool ok[4];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    const int row = m0 + 16 * gi + (l & 15);
    ok[gi] = row < g.M;
    X[gi] = (const XT*)g.X + (size_t)(ok[gi] ? row : 0) * g.ldx + 8 * (l >> 4) + kbeg;
  }
  const T* gain = XS == XS_NORM ? (const T*)g.norm_gain + 8 * (l >> 4) + kbeg : nullptr;
  // XS_NORM operand parts of row group gi at k (8 consecutive elements of the
  // row and of the gain), loaded apart from forming them so the loads can be
  // in flight while the row norms are reduced
  struct XRaw {
    float4v x0, x1;
    typename F::type gv;
  };
  auto xraw = [&](int gi, int k) -> XRaw {
    XRaw r;
    r.x0 = *(const float4v*)((const float*)X[gi] + k);
    r.x1 = *(const float4v*)((const float*)X[gi] + k + 4);
    r.gv = F::load(gain + k);
    return r;
  };
  auto xform = [&](int gi, const XRaw& r) -> typename F::type {
    const float inv = rinv[16 * gi + (l & 15)];
    typename F::type v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = from_f<T>(r.x0[e] * inv * to_f(r.gv[e]));
      v[e + 4] = from_f<T>(r.x1[e] * inv * to_f(r.gv[e + 4]));
    }
    return v;
  };
  // operand fragment of row group gi at k
  auto xfrag = [&](int gi, int k) -> typename F::type {
    if constexpr (XS == XS_NORM) return xform(gi, xraw(gi, k));
    else return F::load((const T*)X[gi] + k);
  };
  float4v acc[4] = {};
  // U 32-deep steps per batch: all their loads are issued before the first
  // MFMA, so a wave keeps U weight loads in flight (decode is latency-bound).
  // The MFMAs still run in k order, so the sums do not depend on U. With
  // XS_NORM one batch covers the wave's whole k range (the row sums need it).
  constexpr int U = gemm_batch(KS, XS, NU);
  typename F::type a[U];
  XRaw xr[XS == XS_NORM ? U : 1];
  typename F::type xb[XS == XS_ONE ? U : 1];
  auto load_a = [&](int k) {
    if constexpr (XS == XS_ONE) {
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = wrow ? F::load(W + 32 * u) : F::zero();
#pragma unroll
      for (int u = 0; u < U; ++u) xb[u] = F::load((const T*)X[0] + 32 * u);   // rows past M read row 0
    } else if constexpr (XS == XS_NORM) {
      // kq == 32 * U: the whole range in one batch, no guards
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = wrow ? F::load(W + 32 * u) : F::zero();
      if (ng == 1) {
#pragma unroll
        for (int u = 0; u < U; ++u) xr[u] = xraw(0, 32 * u);   // rows past M read row 0
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = (wrow && k + 32 * u < kq) ? F::load(W + k + 32 * u) : F::zero();
    }
  };
  const int nrows = min(kRowsPerBlock, g.M - m0);
  const bool task = XS == XS_NORM && g.row_tasks && (int)blockIdx.x < nrows;
  // row work: thread t holds elements 2t and 2t + 1 (threads past the row idle)
  TaskPre<T, 2> pre{};
  int task_lane = 0, rpos_l = 0;
  if constexpr (XS == XS_NORM) {
    // position of row l % 16 of the first row group (negative: stopped), and
    // the row-work inputs, which are only used after the products
    rpos_l = g.row_pos[m0 + min(l & 15, nrows - 1)];
    if (task) {
      task_lane = g.row_lane[m0 + blockIdx.x];
      task_load<T, 2>(m, g, m0 + blockIdx.x, pre);
    }
  }
  load_a(0);
  // XS_ONE: wave 0 finishes row l % 16; its status and (EPI_ADD_F32) the four
  // residual values it adds to are fetched before the weights
  // (row_dead when given: one load, no dependent status lookup)
  int one_dead = 0;
  float4v one_x = float4v{0.f, 0.f, 0.f, 0.f};
  if constexpr (XS == XS_ONE) {
    if (wave == 0 && ok[0] && wout) {
      const int row = m0 + (l & 15);
      if constexpr (EPI == EPI_ADD_F32) one_x = *(const float4v*)((float*)g.out + (size_t)row * g.ldo + f0 + 4 * (l >> 4));
      one_dead = g.row_dead[row];
    }
  }
  if constexpr (XS == XS_NORM) {
    // the rows' sums of squares, inverse RMS and dead flags; a row is dead
    // when its lane stopped before the step (negative position) or fails this
    // layer's safety check (a lane that stopped at an earlier layer of the
    // step kept its residual, so it fails again); products without row work
    // also skip the rows the step's checks have stopped so far (row_dead,
    // written by the attention input's row work, an earlier launch)
    auto finish_row = [&](int rr, float ss, int rpos) {
      rss[rr] = ss;
      rinv[rr] = __fdiv_rn(1.f, __fsqrt_rn(__fdiv_rn(ss, (float)g.K) + m.eps));
      rdead[rr] = rpos < 0 || (!g.row_tasks && g.row_dead && g.row_dead[m0 + rr]) ||
                  (g.row_tasks && g.check_iter >= 0 && g.check && !(__fsqrt_rn(ss) <= g.thr));
    };
    if (ng == 1) {
      // from the operand loads: lane l holds 8 elements of row l % 16 per step
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) ps += xr[u].x0[e] * xr[u].x0[e];
#pragma unroll
        for (int e = 0; e < 4; ++e) ps += xr[u].x1[e] * xr[u].x1[e];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      if (l < 16) rpart[wave * 16 + l] = ps;
      __syncthreads();
      if (wave == 0 && l < nrows) {
        float ss = 0.f;
#pragma unroll
        for (int w = 0; w < KS; ++w) ss += rpart[w * 16 + l];
        finish_row(l, ss, rpos_l);
      }
    } else {
      // more than 16 rows: the same partial sums (wave w, lane group q) formed
      // by threads from x, then combined in the same order
      const int ntask = nrows * KS * 4;
      for (int t = threadIdx.x; t < ntask; t += blockDim.x) {
        const int rr = t / (KS * 4), w = (t / 4) % KS, q = t % 4;
        const float* base = (const float*)g.X + (size_t)(m0 + rr) * g.ldx + w * kq + 8 * q;
        float p = 0.f;
        for (int u = 0; 32 * u < kq; ++u)
          for (int e = 0; e < 8; ++e) {
            const float v = base[32 * u + e];
            p += v * v;
          }
        rpart[t] = p;
      }
      __syncthreads();
      for (int rr = threadIdx.x; rr < nrows; rr += blockDim.x) {
        float ss = 0.f;
        for (int w = 0; w < KS; ++w) {
          const float* pp = rpart + (rr * KS + w) * 4;
          ss += (pp[0] + pp[1]) + (pp[2] + pp[3]);
        }
        finish_row(rr, ss, g.row_pos[m0 + rr]);
      }
    }
    __syncthreads();
    if (task) pre.status = g.status[task_lane];
  }
  if constexpr (XS == XS_ONE) {
    // one batch, loaded above (kq == 32 * U)
#pragma unroll
    for (int u = 0; u < U; ++u) acc[0] = F::mma(a[u], ok[0] ? xb[u] : F::zero(), acc[0]);
  } else if constexpr (XS == XS_NORM) {
    // one batch, loaded above (kq == 32 * U)
    if (ng == 1) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const typename F::type b = ok[0] ? xform(0, xr[u]) : F::zero();
        acc[0] = F::mma(a[u], b, acc[0]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
          if (gi < ng) {
            const typename F::type b = ok[gi] ? xfrag(gi, 32 * u) : F::zero();
            acc[gi] = F::mma(a[u], b, acc[gi]);
          }
    }
  } else {
  for (int k = 0; k < kq; k += 32 * U) {
    if (k > 0) load_a(k);
    if (ng == 1) {
      typename F::type b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) b[u] = (ok[0] && k + 32 * u < kq) ? xfrag(0, k + 32 * u) : F::zero();
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
            const typename F::type b = ok[gi] ? xfrag(gi, k + 32 * u) : F::zero();
            acc[gi] = F::mma(a[u], b, acc[gi]);
          }
        }
      }
    }
  }
  }
  if constexpr (XS == XS_NORM) {
    if (g.row_tasks) row_tasks_ept<T, 2>(m, g, m0, nrows, rss, rinv, rdead, rmax, pre);
  }
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) red[wave][gi][l] = acc[gi];
  __syncthreads();
  const int gi = threadIdx.x >> 6;
  if (gi >= 4 || gi >= ng || !wout) return;
  const int row = m0 + 16 * gi + (l & 15);
  if (row >= g.M) return;
  if constexpr (XS == XS_NORM) {
    if (rdead[row - m0]) return;
  } else if constexpr (XS == XS_ONE) {
    if (one_dead) return;
  } else {
    if (g.status && g.status[g.row_lane[row]] == TL_LANE_ABORTED) return;
  }
  float4v v = red[0][gi][l];
#pragma unroll
  for (int w = 1; w < KS; ++w) v += red[w][gi][l];
  const int fb = f0 + 4 * (l >> 4);
  if constexpr (XS == XS_ONE && EPI == EPI_ADD_F32) {
    *(float4v*)((float*)g.out + (size_t)row * g.ldo + fb) = one_x + v;
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) epilogue<T, EPI>(g, m.D, row, fb + i, v[i]);
}

// Products of a prefill chunk (fp16, up to 512 rows): BM x 64 output tiles
// (BM = 64, or 32 when 64-row tiles would leave CUs idle) and 64-deep k tiles
// staged through LDS (rows padded to 72 halves), on v_mfma_f32_16x16x32_f16.
// Wave w computes rows (BM/2) (w / 2) .. + BM/2 - 1 and features 32 (w % 2)
// .. +31 of the tile as (BM/32) x 2 blocks of 16 x 16; the next four k tiles
// are in flight in registers while the current one is multiplied (the
// products are latency-bound at these sizes). Every output is one fp32 sum
// over k in ascending order, then the epilogue, whatever BM is.
template <int EPI, int BM>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(ModelView m, GemmArgs g) {
  constexpr int BN = 64, BK = 64, LDT = BK + 8, RB = BM / 32, XP = BM / 32;
  static_assert(BM == 64 || BM == 32, "row tile");
  __shared__ __attribute__((aligned(16))) half_t xs[2][BM * LDT];
  __shared__ __attribute__((aligned(16))) half_t wsm[2][BN * LDT];
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, lr = l & 15, lk = l >> 4;
  // staging: thread t moves 16 halves (k offset 16 (t % 4)) of W tile row
  // t / 4, and 8 XP halves of X tile row t / (8 / XP) at k offset
  // 8 XP (t % (8 / XP))
  const int srow = t >> 2, sk = (t & 3) * 16;
  const int xrow = t / (8 / XP), xk = (t % (8 / XP)) * 8 * XP;
  const half_t* xsrc = (const half_t*)g.X + (size_t)min(m0 + xrow, g.M - 1) * g.ldx + xk;
  const half_t* wsrc = (const half_t*)g.W + (size_t)(n0 + srow) * g.ldw + sk;
  // the thread's parts of the next PF k tiles are in flight in registers
  constexpr int PF = 4;
  half8 ring[PF][2 + XP];
  const int nkt = g.K / BK;
#pragma unroll
  for (int u = 0; u < PF; ++u)
    if (u < nkt) {
#pragma unroll
      for (int x = 0; x < XP; ++x) ring[u][x] = *(const half8*)(xsrc + u * BK + 8 * x);
      ring[u][XP] = *(const half8*)(wsrc + u * BK);
      ring[u][XP + 1] = *(const half8*)(wsrc + u * BK + 8);
    }
  float4v acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = float4v{0.f, 0.f, 0.f, 0.f};
  for (int kt0 = 0; kt0 < nkt; kt0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int kt = kt0 + u;
      if (kt >= nkt) break;
      // LDS buffer b was last read two tiles ago, before the previous barrier
      const int b = kt & 1;
#pragma unroll
      for (int x = 0; x < XP; ++x) *(half8*)&xs[b][xrow * LDT + xk + 8 * x] = ring[u][x];
      *(half8*)&wsm[b][srow * LDT + sk] = ring[u][XP];
      *(half8*)&wsm[b][srow * LDT + sk + 8] = ring[u][XP + 1];
      __syncthreads();
      if (kt + PF < nkt) {
        const int k1 = (kt + PF) * BK;
#pragma unroll
        for (int x = 0; x < XP; ++x) ring[u][x] = *(const half8*)(xsrc + k1 + 8 * x);
        ring[u][XP] = *(const half8*)(wsrc + k1);
        ring[u][XP + 1] = *(const half8*)(wsrc + k1 + 8);
      }
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        half8 av[RB], bv[2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          av[rb] = *(const half8*)&xs[b][((BM / 2) * (w >> 1) + 16 * rb + lr) * LDT + 32 * ks + 8 * lk];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          bv[cb] = *(const half8*)&wsm[b][(32 * (w & 1) + 16 * cb + lr) * LDT + 32 * ks + 8 * lk];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[rb], bv[cb], acc[rb][cb], 0, 0, 0);
      }
    }
  }
  // lane l holds rows 4 (l / 16) + i of each block, feature l % 16
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + (BM / 2) * (w >> 1) + 16 * rb + 4 * lk + i;
      if (row >= g.M) continue;
      if (g.status && g.status[g.row_lane[row]] == TL_LANE_ABORTED) continue;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        epilogue<half_t, EPI>(g, m.D, row, n0 + 32 * (w & 1) + 16 * cb + lr, acc[rb][cb][i]);
    }
}

template <int BM>
hipError_t launch_tiled_bm(const ModelView& m, const GemmArgs& g, hipStream_t s) {
  const dim3 grid(g.N / 64, (g.M + BM - 1) / BM);
  switch (g.epi) {
    case EPI_STORE_F32: gemm_tiled_kernel<EPI_STORE_F32, BM><<<grid, 256, 0, s>>>(m, g); break;
    case EPI_STORE_T: gemm_tiled_kernel<EPI_STORE_T, BM><<<grid, 256, 0, s>>>(m, g); break;
    case EPI_ADD_F32: gemm_tiled_kernel<EPI_ADD_F32, BM><<<grid, 256, 0, s>>>(m, g); break;
    case EPI_GELU_T: gemm_tiled_kernel<EPI_GELU_T, BM><<<grid, 256, 0, s>>>(m, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_tiled(const ModelView& m, const GemmArgs& g, hipStream_t s) {
  // 32-row tiles when 64-row ones would leave CUs without a workgroup
  if ((g.N / 64) * ((g.M + 63) / 64) < kCUs) return launch_tiled_bm<32>(m, g, s);
  return launch_tiled_bm<64>(m, g, s);
}

template <typename T, int KS, int NU>
hipError_t launch_norm(const ModelView& m, const GemmArgs& g, dim3 grid, hipStream_t s) {
  switch (g.epi) {
    case EPI_GELU_T: gemm_kernel<T, EPI_GELU_T, KS, XS_NORM, NU><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_STORE_F32: gemm_kernel<T, EPI_STORE_F32, KS, XS_NORM, NU><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_QKV: gemm_kernel<T, EPI_QKV, KS, XS_NORM, NU><<<grid, 64 * KS, 0, s>>>(m, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int KS, int NU>
hipError_t launch_one(const ModelView& m, const GemmArgs& g, dim3 grid, hipStream_t s) {
  switch (g.epi) {
    case EPI_STORE_F32: gemm_kernel<T, EPI_STORE_F32, KS, XS_ONE, NU><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_STORE_T: gemm_kernel<T, EPI_STORE_T, KS, XS_ONE, NU><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_ADD_F32: gemm_kernel<T, EPI_ADD_F32, KS, XS_ONE, NU><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_GELU_T: gemm_kernel<T, EPI_GELU_T, KS, XS_ONE, NU><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_LOGITS: gemm_kernel<T, EPI_LOGITS, KS, XS_ONE, NU><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_QKV: gemm_kernel<T, EPI_QKV, KS, XS_ONE, NU><<<grid, 64 * KS, 0, s>>>(m, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int KS>
hipError_t launch_ks(const ModelView& m, const GemmArgs& g, hipStream_t s) {
  dim3 grid(g.N / g.fb, (g.M + kRowsPerBlock - 1) / kRowsPerBlock);
  if (g.norm_gain) {
    // RMSNorm-input products: the attention input projection (with its row
    // work) and the MLP up projection
    // the rows' positions (negative: stopped) are read by every workgroup
    if (g.K != m.D || m.D % 64 || g.K % (32 * KS) || !g.row_pos) return hipErrorInvalidValue;
    if (g.row_tasks && (64 * KS * 2 < m.D || !g.row_lane || !g.status ||
                        (g.check_iter >= 0 && (!g.norms || (g.check && !g.status_w)))))
      return hipErrorInvalidValue;
    // steps per wave: 1 (d_model 128), 2 / 4 (d_model 1024 / 2048 over 16
    // waves), 8 / 16 (over 4 waves)
    switch (g.K / KS / 32) {
      case 1: return launch_norm<T, KS, 1>(m, g, grid, s);
      case 2: return launch_norm<T, KS, 2>(m, g, grid, s);
      case 4: return launch_norm<T, KS, 4>(m, g, grid, s);
      case 8: return launch_norm<T, KS, 8>(m, g, grid, s);
      case 16: return launch_norm<T, KS, 16>(m, g, grid, s);
      default: return hipErrorInvalidValue;
    }
  }
  // at most 16 rows with row_dead flags: the one-batch variant (its steps
  // per wave, 1..8, as a template argument)
  const int steps = g.K % (32 * KS) ? 0 : g.K / KS / 32;
  if (g.M <= 16 && g.row_dead && (steps == 1 || steps == 2 || steps == 4 || steps == 8)) {
    switch (steps) {
      case 1: return launch_one<T, KS, 1>(m, g, grid, s);
      case 2: return launch_one<T, KS, 2>(m, g, grid, s);
      case 4: return launch_one<T, KS, 4>(m, g, grid, s);
      default: return launch_one<T, KS, 8>(m, g, grid, s);
    }
  }
  switch (g.epi) {
    case EPI_STORE_F32: gemm_kernel<T, EPI_STORE_F32, KS, XS_PLAIN, 0><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_STORE_T: gemm_kernel<T, EPI_STORE_T, KS, XS_PLAIN, 0><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_ADD_F32: gemm_kernel<T, EPI_ADD_F32, KS, XS_PLAIN, 0><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_GELU_T: gemm_kernel<T, EPI_GELU_T, KS, XS_PLAIN, 0><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_LOGITS: gemm_kernel<T, EPI_LOGITS, KS, XS_PLAIN, 0><<<grid, 64 * KS, 0, s>>>(m, g); break;
    case EPI_QKV: gemm_kernel<T, EPI_QKV, KS, XS_PLAIN, 0><<<grid, 64 * KS, 0, s>>>(m, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}


template <typename T>
hipError_t launch_t(const ModelView& m, const GemmArgs& g, hipStream_t s) {
  // 16 waves when the output has too few 16-feature groups for every CU, and
  // when the row work needs them: its threads cover a d_model row two
  // elements each (the stored-K/V projection of 3 d_model features at
  // d_model 2048 has groups enough for 4 waves, but not the threads)
  const bool row_threads = g.norm_gain && g.row_tasks && 64 * 4 * 2 < m.D;
  if ((g.N / 16 < kCUs || row_threads) && g.K % (32 * 16) == 0) return launch_ks<T, 16>(m, g, s);
  return launch_ks<T, 4>(m, g, s);
}

}  // namespace

hipError_t launch_gemm(const ModelView& m, const GemmArgs& g0, hipStream_t s) {
  if (g0.N % 16 || g0.K % 128 || g0.M <= 0) return hipErrorInvalidValue;
  // features per workgroup: enough workgroups (over all row blocks) for
  // every CU when possible
  GemmArgs g = g0;
  if (g.tiled && m.dtype == TL_DTYPE_F16 && !g.norm_gain && g.K % 64 == 0 && g.N % 64 == 0 &&
      g.ldx % 8 == 0 && g.ldw % 8 == 0 &&
      (g.epi == EPI_STORE_F32 || g.epi == EPI_STORE_T || g.epi == EPI_ADD_F32 || g.epi == EPI_GELU_T))
    return launch_tiled(m, g, s);
  const int by = (g.M + kRowsPerBlock - 1) / kRowsPerBlock;
  g.fb = (g.N / 16) * by >= kCUs ? 16 : (g.N / 8) * by >= kCUs ? 8 : 4;
  return m.dtype == TL_DTYPE_F32 ? launch_t<float>(m, g, s) : launch_t<half_t>(m, g, s);
}

}  // namespace tl
