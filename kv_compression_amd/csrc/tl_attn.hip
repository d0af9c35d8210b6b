// Attention pieces around the reconstruction kernel:
//  * kv_attn: decode attention over stored K|V rows, the stored-K/V baseline
//    the store-h cache is measured against (TinyLoop measured-benchmarks page,
//    section 3, "FP16 KV baseline"); HBM-bound streaming of K and V;
//  * attn_merge: combines the per-split (max, sum, o) partials of one row and
//    head (split-T / flash-decoding merge) in a fixed order;
//  * prefill_attn: causal attention of a prefill chunk over K|V rows (chunked
//    prefill; features page, closing list of supported techniques).
#include <algorithm>
#include <type_traits>

#include "tl_device.h"

namespace tl {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// keys per LDS tile of the fp16-MFMA prefill attention (key splits are
// multiples of it)
constexpr int kPrefillKeyTile16 = 64;
// threads per workgroup of that kernel: NT / 64 waves of 16 queries each
constexpr int kPrefillThreads16 = 512;

// All-reduce (sum) over aligned groups of N lanes (N = 8 or 16) with row-level
// data-parallel moves: partners l ^ 1, l ^ 2 (quad permutations), l ^ 7
// (row_half_mirror) and, for 16, l ^ 15 (row_mirror) together reach every lane
// of the group.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "8 or 16 lanes");
  x += dpp_mov<0xB1>(x);                         // l ^ 1
  x += dpp_mov<0x4E>(x);                         // l ^ 2
  x += dpp_mov<0x141>(x);                        // l ^ 7
  if constexpr (N == 16) x += dpp_mov<0x140>(x); // l ^ 15
  return x;
}

// Decode attention over stored K|V rows. One workgroup per (row, split of
// kKvSplit positions). Thread t reads 16 bytes (EPT elements) of a K row and
// of a V row: TPR = D / EPT threads cover one position, and the workgroup's
// PPS = NT / TPR position groups take positions j0 + PPS*i + g. Every K and V
// load of the split is issued before the first score, so the whole split is
// in flight at once; the scores of a head are summed over its TPH = DH / EPT
// threads, each thread keeps an online softmax over its STEPS positions, and
// the position groups are combined in LDS in group order into one
// (max, sum, o) partial per (row, head, split).
template <typename T, int D, int DH, int NT>
__global__ __launch_bounds__(NT) void kv_attn_kernel(ModelView m, ReconArgs a, int n_splits) {
  constexpr int EPT = 16 / (int)sizeof(T);
  constexpr int TPR = D / EPT, PPS = NT / TPR, STEPS = kKvSplit / PPS, TPH = DH / EPT;
  static_assert(NT % TPR == 0 && kKvSplit % PPS == 0 && DH % EPT == 0, "tiling");
  typedef T vec_t __attribute__((ext_vector_type(EPT)));
  __shared__ float comb[PPS][TPR][EPT + 2];
  const int r = blockIdx.x / n_splits, split = blockIdx.x % n_splits;
  // the row's lane and length load together; the lane's status is read once
  // the split's loads (into registers) are in flight
  const int lane = a.row_lane[r];
  const int Tn = a.row_pos[r] + 1;
  __asm__ volatile("" ::"s"(lane), "s"(Tn));
  const int j0 = split * kKvSplit;
  if (j0 >= Tn) return;
  const int t = threadIdx.x, g = t / TPR, c = t % TPR, e0 = c * EPT, head = e0 / DH;
  const T* kv = (const T*)a.cache.kv_row(a.layer, lane, 0);
  // all loads of the split first (positions past T read position T-1)
  vec_t kr[STEPS], vr[STEPS];
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    const int j = min(j0 + PPS * i + g, Tn - 1);
    const T* row = kv + (size_t)j * 2 * D + e0;
    kr[i] = *(const vec_t*)row;
    vr[i] = *(const vec_t*)(row + D);
  }
  __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the first use
  if (a.status[lane] == TL_LANE_ABORTED) return;
  float q[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) q[e] = a.q[(size_t)r * D + e0 + e];
  float s[STEPS];
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) d = fmaf(q[e], to_f(kr[i][e]), d);
    if constexpr (TPH == 1) s[i] = d;
    else s[i] = group_sum<TPH>(d);
    if (j0 + PPS * i + g >= Tn) s[i] = -__builtin_inff();
  }
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < STEPS; ++i) mx = fmaxf(mx, s[i]);
  float lsum = 0.f, o[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) o[e] = 0.f;
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    const float p = s[i] == -__builtin_inff() ? 0.f : exp2f((s[i] - mx) * kLog2e);
    lsum += p;
#pragma unroll
    for (int e = 0; e < EPT; ++e) o[e] = fmaf(p, to_f(vr[i][e]), o[e]);
  }
  comb[g][c][0] = mx;
  comb[g][c][1] = lsum;
#pragma unroll
  for (int e = 0; e < EPT; ++e) comb[g][c][2 + e] = o[e];
  __syncthreads();
  if (g != 0) return;
  float M = comb[0][c][0];
#pragma unroll
  for (int k = 1; k < PPS; ++k) M = fmaxf(M, comb[k][c][0]);
  float L = 0.f, O[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) O[e] = 0.f;
#pragma unroll
  for (int k = 0; k < PPS; ++k) {
    const float mk = comb[k][c][0];
    const float w = mk == -__builtin_inff() ? 0.f : exp2f((mk - M) * kLog2e);
    L = fmaf(comb[k][c][1], w, L);
#pragma unroll
    for (int e = 0; e < EPT; ++e) O[e] = fmaf(comb[k][c][2 + e], w, O[e]);
  }
  float* dst = a.part + (((size_t)r * m.H + head) * a.S + split) * (DH + 2);
  if ((c % TPH) == 0) { dst[0] = M; dst[1] = L; }
#pragma unroll
  for (int e = 0; e < EPT; ++e) dst[2 + (e0 % DH) + e] = O[e];
}

// One block of 256 threads per (row, head): merge_splits over the row's
// ceil(T / split_len) splits.
template <typename T, int DH>
__global__ __launch_bounds__(256) void merge_kernel(int D, int H, const int32_t* row_lane,
                                                    const int32_t* row_pos, const int32_t* status,
                                                    const float* part, int S, int split_len,
                                                    void* out) {
  __shared__ float osum[256];
  __shared__ float lsum[256 / DH];
  __shared__ float red[4];
  const int r = blockIdx.x / H, head = blockIdx.x % H;
  if (status[row_lane[r]] == TL_LANE_ABORTED) return;
  const int Tn = row_pos[r] + 1;
  const int ns = (Tn + split_len - 1) / split_len;   // >= 1, <= S
  merge_splits<T, DH>(part + ((size_t)r * H + head) * S * (DH + 2), ns,
                      (T*)out + (size_t)r * D + head * DH, osum, lsum, red);
}

// Causal attention of a prefill chunk on fp32 MFMA (v_mfma_f32_16x16x4_f32).
// One workgroup per (head, 64 queries); wave w owns queries 16w .. 16w+15 of
// the tile and computes, per tile of 32 keys staged in LDS,
//   S^T = K Q^T   (A: K rows from LDS, B: the wave's queries in registers),
// so lane l holds S^T[key 16kb + 4*(l/16) + i][query l%16] (kb = 0, 1;
// i = 0..3): all of a lane's scores belong to one query. The online softmax
// reduces each query over its 8 values and the 4 lane groups, and
//   O^T += V^T P^T   (A: V^T from LDS, B: P^T straight from the registers),
// pairs k-slot j of k-step (kb, i) with key 16kb + 4j + i, which is exactly
// the key lane group j holds, so P needs no transpose. K and V stay in fp32
// (the rebuilt K|V buffer; stored-K/V caches are widened on the way in), and
// the next tile's loads are in flight while the current tile is multiplied.
// With S > 1 the keys are split into ranges of split_len: workgroup
// (split, query block, head) covers one range and writes its (max, sum,
// unnormalised o) per query to part [n][H][S][DH + 2], which the split merge
// combines; blocks of one head and split sit 16 apart in the grid, on one XCD,
// so its query blocks share that XCD's L2 copy of the keys.
template <typename T, typename KT, int DH>
__global__ __launch_bounds__(256) void prefill_attn_kernel(ModelView m, int n, int pos0,
                                                           const float* q, const KT* kv, T* out,
                                                           int lane, const int32_t* status,
                                                           float* part, int S, int split_len,
                                                           int n_qb) {
  constexpr int QB = 64, KC = 32, KS = DH / 4, DB = DH / 16;
  constexpr int LD = DH + 1;                  // padded LDS rows (floats)
  constexpr int PER = KC * DH / 256;          // tile elements per thread (K, and V)
  __shared__ float Ks[KC * LD];
  __shared__ float Vs[KC * LD];
  if (status && status[lane] == TL_LANE_ABORTED) return;
  const int D = m.D;
  const int head = blockIdx.x % m.H, qb = (blockIdx.x / m.H) % n_qb, split = blockIdx.x / (m.H * n_qb);
  const int t = threadIdx.x, wave = t >> 6, l = t & 63, lq = l & 15, lg = l >> 4;
  const int qi = qb * QB + wave * 16 + lq;    // this lane's query (B operand / output column)
  const bool qv = qi < n;
  const int qpos = pos0 + qi;
  // Q^T as B operand: k-step s holds dim 4s + lg of query lq
  float qb_op[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qb_op[s] = qv ? q[(size_t)qi * D + head * DH + 4 * s + lg] : 0.f;
  float4v ot[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) ot[d] = float4v{0.f, 0.f, 0.f, 0.f};
  float mx = -__builtin_inff(), lsum = 0.f;
  const int last_q = min(n, qb * QB + QB) - 1;
  const int k_lo = split * split_len;
  const int kend = min(pos0 + last_q + 1, k_lo + split_len);   // keys k_lo .. kend-1
  if (k_lo >= kend) return;
  // tile loads: thread t takes elements e = t + 256 p of the KC x DH tile
  float kreg[PER], vreg[PER];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = t + 256 * p, kk = e / DH, d = e % DH;
      const int kp = min(k0 + kk, kend - 1);
      kreg[p] = to_f(kv[(size_t)kp * 2 * D + head * DH + d]);
      vreg[p] = to_f(kv[(size_t)kp * 2 * D + D + head * DH + d]);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = t + 256 * p, kk = e / DH, d = e % DH;
      Ks[kk * LD + d] = kreg[p];
      Vs[kk * LD + d] = vreg[p];
    }
  };
  load_tile(k_lo);
  for (int k0 = k_lo; k0 < kend; k0 += KC) {
    __syncthreads();   // the previous tile is no longer read
    store_tile();
    __syncthreads();
    if (k0 + KC < kend) load_tile(k0 + KC);   // next tile in flight under this one
    // S^T for key blocks kb = 0, 1
    float4v st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const float a = Ks[(16 * kb + lq) * LD + 4 * s + lg];
        st[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qb_op[s], st[kb], 0, 0, 0);
      }
    }
    // mask and online softmax of query lq (keys 16kb + 4lg + i)
    float cm = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kp = k0 + 16 * kb + 4 * lg + i;
        if (kp > qpos || kp >= kend) st[kb][i] = -__builtin_inff();
        cm = fmaxf(cm, st[kb][i]);
      }
    cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
    cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
    const float mn = fmaxf(mx, cm);
    const float corr = mx == -__builtin_inff() ? 0.f : exp2f((mx - mn) * kLog2e);
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = st[kb][i] == -__builtin_inff() ? 0.f : exp2f((st[kb][i] - mn) * kLog2e);
        st[kb][i] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    lsum = lsum * corr + ps;
    mx = mn;
#pragma unroll
    for (int d = 0; d < DB; ++d) ot[d] *= corr;
    // O^T += V^T P^T: k-step (kb, i), A = V[16kb + 4lg + i][16d + lq]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const float a = Vs[(16 * kb + 4 * lg + i) * LD + 16 * d + lq];
          ot[d] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, st[kb][i], ot[d], 0, 0, 0);
        }
  }
  if (!qv) return;
  // lane l holds O^T[dim 16d + 4lg + i][query lq]
  if (part) {
    float* pp = part + (((size_t)qi * m.H + head) * S + split) * (DH + 2);
    if (lg == 0) {
      pp[0] = mx;
      pp[1] = lsum;
    }
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[2 + 16 * d + 4 * lg + i] = ot[d][i];
    return;
  }
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[(size_t)qi * D + head * DH + 16 * d + 4 * lg + i] = from_f<T>(__fdiv_rn(ot[d][i], lsum));
}


// Merge of the prefill's key splits, one thread per output element (query
// row r, column head * DH + dim): o = sum_s w_s o_s / sum_s w_s l_s with
// w_s = exp(m_s - M) over the row's ceil(T / split_len) splits in split
// order, loaded 8 splits at a time. A prefill chunk has up to 512 query rows
// and few splits per row, so one thread per element keeps the launch wide.
template <typename T, int DH>
__global__ __launch_bounds__(256) void merge_rows_kernel(int n_rows, int D, int H, const int32_t* row_lane,
                                                         const int32_t* row_pos, const int32_t* status,
                                                         const float* part, int S, int split_len,
                                                         void* out) {
  constexpr int U = 8;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_rows * D) return;
  const int r = i / D, col = i % D, head = col / DH, dim = col % DH;
  if (status[row_lane[r]] == TL_LANE_ABORTED) return;
  const int ns = (row_pos[r] + split_len) / split_len;   // ceil((pos + 1) / split_len) >= 1
  const float* p = part + ((size_t)r * H + head) * S * (DH + 2);
  float M = -__builtin_inff();
  for (int c = 0; c < ns; c += U) {
    float mv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) mv[u] = p[(size_t)min(c + u, ns - 1) * (DH + 2)];
#pragma unroll
    for (int u = 0; u < U; ++u) M = fmaxf(M, mv[u]);
  }
  float o = 0.f, L = 0.f;
  for (int c = 0; c < ns; c += U) {
    float mv[U], lv[U], ov[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* ps = p + (size_t)min(c + u, ns - 1) * (DH + 2);
      mv[u] = ps[0];
      lv[u] = ps[1];
      ov[u] = ps[2 + dim];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c + u < ns) {
        const float w = exp2f((mv[u] - M) * kLog2e);
        o = fmaf(ov[u], w, o);
        L = fmaf(lv[u], w, L);
      }
  }
  ((T*)out)[(size_t)r * D + col] = from_f<T>(__fdiv_rn(o, L));
}

// x = hi + lo with hi = fp16(x) and lo = fp16(x - hi) (the difference is exact
// in fp32): the pair holds about 22 significant bits of x.
__device__ __forceinline__ void split_half(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

// Causal attention of a prefill chunk on fp16 MFMA (v_mfma_f32_16x16x32_f16).
// The fp32 queries, and the fp32 K|V rows rebuilt from h, enter as fp16
// (hi, lo) pairs and every product is formed as hi*hi + hi*lo + lo*hi in the
// fp32 accumulators (the lo*lo term lies below fp32 rounding), so the scores
// and the weighted values keep fp32 accuracy on the fp16 MFMA pipe. Stored
// fp16 K|V rows (the stored-K/V mode) have no lo half.
// Same masking, online softmax, key splits and outputs as
// prefill_attn_kernel, with 8 waves: one workgroup per (key split, 128
// queries, head), so each staged key tile serves twice the queries; wave w
// owns queries 16w .. 16w+15 and, per tile of 64 keys staged in LDS,
//   S^T = K Q^T   (A: K rows from LDS, B: the wave's queries in registers),
// so lane l holds S^T[key 16kb + 4*(l/16) + i][query l%16] (kb = 0 .. 3), and
//   O^T += V^T P^T   over two 32-key k-steps,
// where MFMA k-slot 8g + j of lane group g in k-step ks stands for key
// 32ks + 16 (j/4) + 4g + j%4: those are keys lane group g holds scores for,
// so P^T comes straight from the score registers. V is staged transposed
// (each thread loads four keys of one dimension, coalesced over the
// dimensions, and writes them as one 8-byte row piece), so each lane's A
// operand is two 8-byte LDS reads. |K|, |V| and |q| must stay within the
// fp16 range (below 65504); beyond it the attention is not finite.
template <typename T, typename KT, int DH>
__global__ __launch_bounds__(kPrefillThreads16) void prefill_attn16_kernel(ModelView m, int n, int pos0,
                                                             const float* q, const KT* kv, T* out,
                                                             int lane, const int32_t* status,
                                                             float* part, int S, int split_len,
                                                             int n_qb) {
  constexpr bool KV_LO = std::is_same<KT, float>::value;
  constexpr int NT = kPrefillThreads16, QB = NT / 4, KC = kPrefillKeyTile16, KB = KC / 16, NS = DH / 32, DB = DH / 16;
  constexpr int KLD = DH + 8;                 // K row stride (halfs), 16-byte aligned
  constexpr int VLD = KC + 8;                 // V^T row stride (halfs), 16-byte aligned
  constexpr int C4 = KC * DH / 4 / NT;        // 4-element chunks of K (and of V) per thread
  static_assert(KC % 32 == 0 && C4 >= 1, "key tile");
  __shared__ __attribute__((aligned(16))) _Float16 Kh[KC * KLD];
  __shared__ __attribute__((aligned(16))) _Float16 Kl[KV_LO ? KC * KLD : 8];
  __shared__ __attribute__((aligned(16))) _Float16 Vh[DH * VLD];
  __shared__ __attribute__((aligned(16))) _Float16 Vl[KV_LO ? DH * VLD : 8];
  if (status && status[lane] == TL_LANE_ABORTED) return;
  const int D = m.D;
  const int head = blockIdx.x % m.H, qb = (blockIdx.x / m.H) % n_qb, split = blockIdx.x / (m.H * n_qb);
  const int t = threadIdx.x, wave = t >> 6, l = t & 63, lq = l & 15, lg = l >> 4;
  const int qi = qb * QB + wave * 16 + lq;    // this lane's query (B operand / output column)
  const bool qv = qi < n;
  const int qpos = pos0 + qi;
  // Q^T as B operand: k-step s holds dims 32s + 8lg + j of query lq
  half8 qh[NS], ql[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float* qr = q + (size_t)(qv ? qi : 0) * D + head * DH + 32 * s + 8 * lg;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      _Float16 hi, lo;
      split_half(qv ? qr[j] : 0.f, hi, lo);
      qh[s][j] = hi;
      ql[s][j] = lo;
    }
  }
  float4v ot[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) ot[d] = float4v{0.f, 0.f, 0.f, 0.f};
  float mx = -__builtin_inff(), lsum = 0.f;
  const int last_q = min(n, qb * QB + QB) - 1;
  const int k_lo = split * split_len;
  const int kend = min(pos0 + last_q + 1, k_lo + split_len);   // keys k_lo .. kend-1
  if (k_lo >= kend) return;
  // Tile loads. K: chunk c = t + NT p is key c / (DH/4), dims 4 (c % (DH/4))
  // .. +3 (one 16- or 8-byte load). V: chunk c is dim c % DH, keys
  // 4 (c / DH) .. +3 (four loads, each coalesced over the lanes' dims).
  float4v kr[C4], vr[C4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int p = 0; p < C4; ++p) {
      const int c = t + NT * p;
      {
        const int kk = c / (DH / 4), d0 = 4 * (c % (DH / 4));
        const KT* row = kv + (size_t)min(k0 + kk, kend - 1) * 2 * D + head * DH + d0;
        if constexpr (KV_LO) {
          kr[p] = *(const float4v*)row;
        } else {
          const half4 a = *(const half4*)row;
          kr[p] = float4v{(float)a[0], (float)a[1], (float)a[2], (float)a[3]};
        }
      }
      const int d = c % DH, k4 = 4 * (c / DH);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vr[p][e] = (float)kv[(size_t)min(k0 + k4 + e, kend - 1) * 2 * D + D + head * DH + d];
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < C4; ++p) {
      const int c = t + NT * p;
      half4 xh, xl;
      {
        const int kk = c / (DH / 4), d0 = 4 * (c % (DH / 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          _Float16 hi, lo;
          split_half(kr[p][e], hi, lo);
          xh[e] = hi;
          xl[e] = lo;
        }
        *(half4*)&Kh[kk * KLD + d0] = xh;
        if constexpr (KV_LO) *(half4*)&Kl[kk * KLD + d0] = xl;
      }
      const int d = c % DH, k4 = 4 * (c / DH);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        _Float16 hi, lo;
        split_half(vr[p][e], hi, lo);
        xh[e] = hi;
        xl[e] = lo;
      }
      *(half4*)&Vh[d * VLD + k4] = xh;
      if constexpr (KV_LO) *(half4*)&Vl[d * VLD + k4] = xl;
    }
  };
  load_tile(k_lo);
  for (int k0 = k_lo; k0 < kend; k0 += KC) {
    __syncthreads();   // the previous tile is no longer read
    store_tile();
    __syncthreads();
    if (k0 + KC < kend) load_tile(k0 + KC);   // next tile in flight under this one
    // S^T for key blocks kb
    float4v st[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      st[kb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int off = (16 * kb + lq) * KLD + 32 * s + 8 * lg;
        const half8 ah = *(const half8*)&Kh[off];
        st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, ql[s], st[kb], 0, 0, 0);
        if constexpr (KV_LO) {
          const half8 al = *(const half8*)&Kl[off];
          st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, qh[s], st[kb], 0, 0, 0);
        }
        st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, qh[s], st[kb], 0, 0, 0);
      }
    }
    // mask and online softmax of query lq (keys k0 + 16kb + 4lg + i)
    float cm = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kp = k0 + 16 * kb + 4 * lg + i;
        if (kp > qpos || kp >= kend) st[kb][i] = -__builtin_inff();
        cm = fmaxf(cm, st[kb][i]);
      }
    cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
    cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
    const float mn = fmaxf(mx, cm);
    const float corr = mx == -__builtin_inff() ? 0.f : exp2f((mx - mn) * kLog2e);
    float ps = 0.f;
    half8 ph[KB / 2], pl[KB / 2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = st[kb][i] == -__builtin_inff() ? 0.f : exp2f((st[kb][i] - mn) * kLog2e);
        ps += p;
        _Float16 hi, lo;
        split_half(p, hi, lo);
        ph[kb / 2][4 * (kb & 1) + i] = hi;
        pl[kb / 2][4 * (kb & 1) + i] = lo;
      }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    lsum = lsum * corr + ps;
    mx = mn;
    // O^T += V^T P^T: k-step ks, A = V^T[dim 16d + lq][keys 32ks + 4lg .. +3,
    // 32ks + 16 + 4lg .. +3]
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      ot[d] *= corr;
#pragma unroll
      for (int ks = 0; ks < KB / 2; ++ks) {
        const int off = (16 * d + lq) * VLD + 32 * ks + 4 * lg;
        const half4 a0 = *(const half4*)&Vh[off], a1 = *(const half4*)&Vh[off + 16];
        const half8 ah = half8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        ot[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, pl[ks], ot[d], 0, 0, 0);
        if constexpr (KV_LO) {
          const half4 b0 = *(const half4*)&Vl[off], b1 = *(const half4*)&Vl[off + 16];
          const half8 al = half8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          ot[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, ph[ks], ot[d], 0, 0, 0);
        }
        ot[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, ph[ks], ot[d], 0, 0, 0);
      }
    }
  }
  if (!qv) return;
  // lane l holds O^T[dim 16d + 4lg + i][query lq]
  if (part) {
    float* pp = part + (((size_t)qi * m.H + head) * S + split) * (DH + 2);
    if (lg == 0) {
      pp[0] = mx;
      pp[1] = lsum;
    }
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[2 + 16 * d + 4 * lg + i] = ot[d][i];
    return;
  }
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[(size_t)qi * D + head * DH + 16 * d + 4 * lg + i] = from_f<T>(__fdiv_rn(ot[d][i], lsum));
}

}  // namespace

hipError_t launch_kv_attn(const ModelView& m, const ReconArgs& a, hipStream_t s) {
  const int n_splits = (a.t_ub + kKvSplit - 1) / kKvSplit;
  const int grid = n_splits * a.n_rows;
  if (n_splits > a.S) return hipErrorInvalidValue;
  if (m.dtype == TL_DTYPE_F32 && m.D == 128 && m.dh == 32)
    return launch_timed(kv_attn_kernel<float, 128, 32, 256>, grid, 256, s, a.ev, m, a, n_splits);
  else if (m.dtype == TL_DTYPE_F16 && m.D == 1024 && m.dh == 64)
    return launch_timed(kv_attn_kernel<half_t, 1024, 64, 256>, grid, 256, s, a.ev, m, a, n_splits);
  else if (m.dtype == TL_DTYPE_F16 && m.D == 2048 && m.dh == 128)
    return launch_timed(kv_attn_kernel<half_t, 2048, 128, 512>, grid, 512, s, a.ev, m, a, n_splits);
  else if (m.dtype == TL_DTYPE_F16 && m.D == 2048 && m.dh == 64)
    return launch_timed(kv_attn_kernel<half_t, 2048, 64, 512>, grid, 512, s, a.ev, m, a, n_splits);
  else if (m.dtype == TL_DTYPE_F16 && m.D == 1024 && m.dh == 128)
    return launch_timed(kv_attn_kernel<half_t, 1024, 128, 256>, grid, 256, s, a.ev, m, a, n_splits);
  return hipErrorInvalidValue;
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

// queries per workgroup of the prefill attention kernel the model uses
static int prefill_qb(const ModelView& m) { return m.dtype == TL_DTYPE_F32 ? 64 : kPrefillThreads16 / 4; }

int prefill_splits(const ModelView& m, int n, int pos0, int part_floats, int* split_len) {
  const int KC = m.dtype == TL_DTYPE_F32 ? 32 : kPrefillKeyTile16;   // the kernel's key tile
  const int n_qb = (n + prefill_qb(m) - 1) / prefill_qb(m);
  const int tiles = (pos0 + n + KC - 1) / KC;            // key tiles of the last query block
  // about four 4-wave (fp32) or two 8-wave (fp16) workgroups per CU, at
  // least four (fp32) or two (fp16) key tiles per split, and the partials
  // within their buffer
  const bool f32 = m.dtype == TL_DTYPE_F32;
  int S = ((f32 ? 1024 : 512) + m.H * n_qb - 1) / (m.H * n_qb);
  S = std::min(S, std::max(1, tiles / (f32 ? 4 : 2)));
  S = std::min(S, std::max(1, part_floats / (n * m.H * (m.dh + 2))));
  *split_len = (tiles + S - 1) / S * KC;
  return (pos0 + n + *split_len - 1) / *split_len;
}

hipError_t launch_prefill_attn(const ModelView& m, int n, int pos0, const float* q,
                               const void* kv, int kv_f32, void* o, int lane,
                               const int32_t* status, float* part, int part_floats,
                               const int32_t* row_lane, const int32_t* row_pos, hipStream_t s) {
  const int n_qb = (n + prefill_qb(m) - 1) / prefill_qb(m);
  int split_len = 0;
  const int S = part ? prefill_splits(m, n, pos0, part_floats, &split_len) : 1;
  if (S == 1) split_len = pos0 + n;
  float* pp = S > 1 ? part : nullptr;
  const int grid = m.H * n_qb * S;
#define TL_PA(T_, KT_, DH_)                                                                  \
  prefill_attn_kernel<T_, KT_, DH_><<<grid, 256, 0, s>>>(m, n, pos0, q, (const KT_*)kv, (T_*)o, \
                                                          lane, status, pp, S, split_len, n_qb)
#define TL_PA16(T_, KT_, DH_)                                                                  \
  prefill_attn16_kernel<T_, KT_, DH_><<<grid, kPrefillThreads16, 0, s>>>(m, n, pos0, q, (const KT_*)kv, (T_*)o, \
                                                            lane, status, pp, S, split_len, n_qb)
  if (m.dtype == TL_DTYPE_F32 && m.dh == 32) TL_PA(float, float, 32);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 64 && kv_f32) TL_PA16(half_t, float, 64);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 64) TL_PA16(half_t, half_t, 64);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 128 && kv_f32) TL_PA16(half_t, float, 128);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 128) TL_PA16(half_t, half_t, 128);
  else return hipErrorInvalidValue;
#undef TL_PA
#undef TL_PA16
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const int mgrid = (n * m.D + 255) / 256;
#define TL_MR(T_, DH_)                                                                            \
  merge_rows_kernel<T_, DH_><<<mgrid, 256, 0, s>>>(n, m.D, m.H, row_lane, row_pos, status, part, S, \
                                                   split_len, o)
  if (m.dtype == TL_DTYPE_F32 && m.dh == 32) TL_MR(float, 32);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 64) TL_MR(half_t, 64);
  else if (m.dtype == TL_DTYPE_F16 && m.dh == 128) TL_MR(half_t, 128);
  else return hipErrorInvalidValue;
#undef TL_MR
  return hipGetLastError();
}

}  // namespace tl
