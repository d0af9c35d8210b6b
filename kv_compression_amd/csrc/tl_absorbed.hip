// Absorbed evaluation order of store-h decode attention (novel-contributions
// page, "Novel Mechanism: Store-h KV Cache", which relates store-h to MLA).
//
// With K = W_k h' and V = W_v h', head h's score is q_h . (W_k,h h'_j) =
// (W_k,h^T q_h) . h'_j and its output is W_v,h (sum_j p_j h'_j). So every head
// attends over the same D-wide rows h'_j (multi-query attention with head
// width D) with the query qt_h = W_k,h^T q_h, and W_v,h is applied once to the
// weighted sum r_h. Per position that is 4 H D flops instead of the 4 D^2 of
// rebuilding K and V.
//
// Three kernels per layer:
//   absorb_q_kernel        qt[row][h][c] = sum_j q[row][h d + j] W_k[h d + j][c]  (fp32)
//   absorbed_attn_kernel   per (row, key split): the scores and the weighted sum
//                          of h' on MFMA, written as (max, sum, r[D]) per head
//   absorbed_merge_kernel  per (row, head, column quarter): merge the splits, r / l
//   absorbed_o_kernel      o = W_v,h r per row and head (fp32 sums, model dtype out)
#include <algorithm>

#include "tl_device.h"

#define TL_LDS __attribute__((address_space(3)))
typedef __fp16 fp16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));

namespace tl {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kAbsTP = 32;    // positions per tile of the attention kernel

// qt = W_k^T q per head. Grid (D / 64, H), 64 threads: thread c of column
// block cb holds W_k rows h d .. h d + d - 1 of column cb * 64 + c in
// registers (all loads in flight together) and sums them against each row's
// q, staged 64 rows at a time in LDS. The sum runs over j in order. The
// result is written in the attention kernel's operand order (16 heads): per
// row 4 waves x D / 128 k-steps x 64 lanes x (8 high, 8 low) halves, which
// is also the order of 8 waves x D / 256 k-steps (the k-steps of wave w of 8
// are k-steps 4 (w % 2) .. of wave w / 2 of 4).
template <int DH>
__global__ __launch_bounds__(64) void absorb_q_kernel(int D, int n_rows, const float* q,
                                                      const half_t* wk, float* qt) {
  __shared__ float qs[64][DH];
  const int c = blockIdx.x * 64 + threadIdx.x, h = blockIdx.y, H = gridDim.y;
  float wr[DH];
#pragma unroll
  for (int j = 0; j < DH; ++j) wr[j] = (float)wk[((size_t)h * DH + j) * D + c];
  for (int r0 = 0; r0 < n_rows; r0 += 64) {
    const int nr = min(64, n_rows - r0);
    __syncthreads();
    for (int e = threadIdx.x; e < nr * DH; e += 64)
      qs[e / DH][e % DH] = q[(size_t)(r0 + e / DH) * D + h * DH + e % DH];
    __syncthreads();
    for (int u = 0; u < nr; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < DH; ++j) acc = fmaf(qs[u][j], wr[j], acc);
      // stored as the attention kernel's B fragments: column c of head h is
      // element e = c % 8 of lane 16 ((c / 8) % 4) + h in k-step (c % 256) / 32 of
      // wave c / 256, as an fp16 high half and the fp16 rest
      const half_t hi = (half_t)acc, lo = (half_t)(acc - (float)hi);
      const int wc = D / 4, nks = wc / 32;
      const int wv = c / wc, ks = (c % wc) >> 5, ln = 16 * ((c >> 3) & 3) + h, e = c & 7;
      half_t* f = (half_t*)qt + ((((size_t)(r0 + u) * 4 + wv) * nks + ks) * 64 + ln) * 16;
      f[e] = hi;
      f[8 + e] = lo;
    }
  }
}

// The raw cache bytes of the 64-element block kb of one position, and their
// dequantisation into an LDS row (fp16 h' in natural element order; zeros
// for a position past the tile's end).
template <int MODE> struct BlockRaw;
template <> struct BlockRaw<TL_CACHE_H_F16> { u32x4 v[8]; };
template <> struct BlockRaw<TL_CACHE_H_INT8> { u32x4 v[4]; uint16_t s; };
template <> struct BlockRaw<TL_CACHE_H_INT4> { u32x4 v[2]; uint32_t s; };

template <int MODE>
__device__ __forceinline__ BlockRaw<MODE> load_block(const CacheView& c, int layer, int lane, int kb,
                                                     int pos) {
  BlockRaw<MODE> b;
  const u32x4* row = (const u32x4*)c.code_row(layer, lane, kb, pos);
  constexpr int NV = sizeof(b.v) / sizeof(u32x4);
#pragma unroll
  for (int i = 0; i < NV; ++i) b.v[i] = row[i];
  if constexpr (MODE == TL_CACHE_H_INT4) b.s = *(const uint32_t*)c.int4_scale(layer, lane, kb, pos);
  if constexpr (MODE == TL_CACHE_H_INT8) b.s = *c.int8_scale(layer, lane, pos);
  return b;
}

template <int MODE>
__device__ __forceinline__ void store_block(const BlockRaw<MODE>& b, bool valid, half_t* dst) {
  if (!valid) {
    half8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (half_t)0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(half8*)(dst + 8 * i) = z;
    return;
  }
  if constexpr (MODE == TL_CACHE_H_F16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4*)(dst + 8 * i) = b.v[i];
  } else if constexpr (MODE == TL_CACHE_H_INT4) {
    // word g holds elements 16 (g % 4) + 8 (g / 4) .. +7; elements 32.. use the second scale
    const half_t s0 = h_from_bits((uint16_t)(b.s & 0xFFFFu)), s1 = h_from_bits((uint16_t)(b.s >> 16));
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int base = 16 * (g & 3) + 8 * (g >> 2);
      *(half8*)(dst + base) = int4_dequant8(b.v[g >> 2][g & 3], (g & 3) >= 2 ? s1 : s0);
    }
  } else {  // INT8: group g of 8 bytes holds elements 16 (g % 4) + 8 (g / 4) .. +7
    const half_t s = h_from_bits(b.s);
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int g = 2 * v + k, base = 16 * (g & 3) + 8 * (g >> 2);
        const half4 lo = int8_dequant4(b.v[v][2 * k], s), hi = int8_dequant4(b.v[v][2 * k + 1], s);
        const half8 e = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        *(half8*)(dst + base) = e;
      }
  }
}

struct AbsArgs {
  CacheView cache;
  int layer;
  const int32_t* row_lane;
  const int32_t* row_pos;
  const int32_t* status;
  const float* qt;       // [rows, H, D]
  float* part;           // [rows, S, H, D + 2]
  int S, split_len;
};

// One workgroup per (row, key split) of NW waves (8 at D = 1024, two per
// SIMD, so one wave's LDS and memory waits run under the other's MFMAs; 4 at
// D = 2048, whose staged tile and sums leave room for no more); wave w owns
// d_model columns w D / NW .. (w + 1) D / NW - 1 of both products. Per tile of 32 positions:
//   S^T[pos][head] = h'[pos][:] . qt[head][:] on v_mfma_f32_16x16x32_f16, in
//     two blocks of 16 positions: row m of block b is position
//     8 (m / 4) + 4 b + m % 4, so that lane l's accumulators hold positions
//     8 (l / 16) + j (j = 4 b + i) of head l % 16. A = h' rows from LDS; B =
//     qt held in registers as fp16 high and low halves (fp32 accuracy). The
//     waves' partial sums over their columns are added in LDS in wave
//     order;
//   online softmax per head;
//   R[head][d] += P[head][pos] h'[pos][d]: the lane's eight weights are exactly
//     the A operand (row = head, k = 8 (l / 16) + j); B = h' from LDS through
//     two transpose reads (ds_read_b64_tr_b16) per product.
// LDS row of position p starts at p * LDR + 8 ((p / 8) % 4) halves and its
// 64-element blocks are 72 halves apart: the row shift keeps the weighted
// sum's strided B reads (rows 8 (l / 16) + j) on distinct banks, the block
// padding the staging writes (one block per lane), and every 8-element run
// stays 16-byte aligned.
template <int MODE, int D, int NW>
__global__ __launch_bounds__(NW * 64) void absorbed_attn_kernel(AbsArgs a) {
  constexpr int NT = NW * 64;
  constexpr int H = 16, TP = 32, BS = 72, LDR = D / 64 * BS + 32, WC = D / NW, KS = WC / 32, NB = WC / 16;
  static_assert((D == 1024 || D == 2048) && (NW == 4 || NW == 8), "d_model / NW columns per wave");
  __shared__ __attribute__((aligned(16))) half_t hs[TP * LDR];
  __shared__ float sp[NW][512];
  auto row_of = [](int p) { return p * LDR + 8 * ((p >> 3) & 3); };
  auto col_of = [](int k) { return (k >> 6) * BS + (k & 63); };
  // the kernel arguments the prologue uses, fetched in one batch at the start
  __asm__ volatile("" ::"s"(a.cache.base), "s"(a.cache.scales), "s"(a.cache.mode), "s"(a.cache.max_seq),
                   "s"(a.cache.n_lanes), "s"(a.layer), "s"(a.row_lane), "s"(a.row_pos), "s"(a.status),
                   "s"(a.qt), "s"(a.S), "s"(a.split_len));
  const int row = blockIdx.x / a.S, split = blockIdx.x % a.S;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, lq = l & 15, lg = l >> 4;
  const int c0 = w * WC;
  // qt as B operand: k-step s holds columns c0 + 32 s + 8 lg + j of head lq,
  // stored in this order by absorb_q_kernel (one contiguous 32 bytes per lane);
  // its loads (they depend on the row only) go out with the row's lookups,
  // and the lane's status is read once the first tiles' loads are in flight
  half8 qh[KS], ql[KS];
  {
    const half8* qp = (const half8*)a.qt + (((size_t)row * NW + w) * KS * 64 + l) * 2;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qh[s] = qp[s * 128];
      ql[s] = qp[s * 128 + 1];
    }
  }
  const int lane = a.row_lane[row];
  const int rpos = a.row_pos[row];
  __asm__ volatile("" ::"s"(lane), "s"(rpos));   // both lookups in flight together
  if (rpos < 0) return;
  const int T = rpos + 1;
  const int p_lo = split * a.split_len, p_hi = min(T, p_lo + a.split_len);
  if (p_lo >= p_hi) return;
  float4v R[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) R[n] = float4v{0.f, 0.f, 0.f, 0.f};
  float mx = -__builtin_inff(), lsum = 0.f;   // head lq
  // staging: thread t dequantises blocks t % 16 + 16 b (b < D / 1024) of
  // positions t / 16 + PPP i (i < NPP: PPP = NT / 16 positions per pass);
  // staged block s is position spos + PPP (s % NPP), block skb + 16 (s / NPP)
  constexpr int PPP = NT / 16, NPP = TP / PPP;
  constexpr int NS = NPP * (D / 1024);
  const int spos = t >> 4, skb = t & 15;
  auto s_pos = [&](int q) { return PPP * (q % NPP) + spos; };
  auto s_blk = [&](int q) { return skb + 16 * (q / NPP); };
  half_t* sdst[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) sdst[q] = hs + row_of(s_pos(q)) + s_blk(q) * BS;
  // the thread's blocks of the next PF tiles are loaded while the current
  // one is multiplied (positions past p_hi are clamped in and staged as zeros)
  // (at D = 2048 the INT8 and fp16 blocks are loaded right before they are
  // staged: the operands of both products leave no registers for a ring)
  constexpr bool DIRECT = D == 2048 && MODE != TL_CACHE_H_INT4;
  constexpr int PF = MODE == TL_CACHE_H_INT4 && D == 1024 ? 2 : 1;
  BlockRaw<MODE> ring[DIRECT ? 1 : PF][DIRECT ? 1 : NS];
  if constexpr (!DIRECT) {
#pragma unroll
    for (int u = 0; u < PF; ++u)
#pragma unroll
      for (int q = 0; q < NS; ++q)
        ring[u][q] = load_block<MODE>(a.cache, a.layer, lane, s_blk(q), min(p_lo + u * TP + s_pos(q), p_hi - 1));
  }
  if (a.status[lane] == TL_LANE_ABORTED) return;   // (loads into registers only so far)
  for (int pr = p_lo; pr < p_hi; pr += PF * TP) {
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    const int p0 = pr + u * TP;
    if (p0 >= p_hi) break;
    if constexpr (DIRECT) {
      __syncthreads();   // the previous tile is no longer read
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        const BlockRaw<MODE> b1 = load_block<MODE>(a.cache, a.layer, lane, s_blk(q), min(p0 + s_pos(q), p_hi - 1));
        store_block<MODE>(b1, p0 + s_pos(q) < p_hi, sdst[q]);
      }
    } else {
      BlockRaw<MODE> cur[NS];
#pragma unroll
      for (int q = 0; q < NS; ++q) cur[q] = ring[u][q];
      if (p0 + PF * TP < p_hi) {
#pragma unroll
        for (int q = 0; q < NS; ++q)
          ring[u][q] = load_block<MODE>(a.cache, a.layer, lane, s_blk(q), min(p0 + PF * TP + s_pos(q), p_hi - 1));
      }
      __syncthreads();   // the previous tile is no longer read
#pragma unroll
      for (int q = 0; q < NS; ++q) store_block<MODE>(cur[q], p0 + s_pos(q) < p_hi, sdst[q]);
    }
    __syncthreads();
    // partial scores over this wave's columns: block b in two chains
    // (even and odd k-steps), added chain 0 then chain 1
    float4v sa[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sa[b][0] = float4v{0.f, 0.f, 0.f, 0.f};
      sa[b][1] = float4v{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int prow = 8 * (lq >> 2) + 4 * b + (lq & 3);
        const half8 av = *(const half8*)(hs + row_of(prow) + col_of(c0 + 32 * s + 8 * lg));
        sa[b][s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qh[s], sa[b][s & 1], 0, 0, 0);
        sa[b][s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, ql[s], sa[b][s & 1], 0, 0, 0);
      }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float4v st = sa[b][0] + sa[b][1];
      *(float4v*)&sp[w][256 * b + 4 * l] = st;
    }
    __syncthreads();
    // lane l: positions 8 lg + j of head lq (j = 4 b + i)
    float sc[8];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      // the waves' column sums added in wave order
      float4v sv = *(const float4v*)&sp[0][256 * b + 4 * l];
#pragma unroll
      for (int u = 1; u < NW; ++u) sv += *(const float4v*)&sp[u][256 * b + 4 * l];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sv[i];
        if (p0 + 8 * lg + 4 * b + i >= p_hi) v = -__builtin_inff();
        sc[4 * b + i] = v;
      }
    }
    // online softmax of head lq over the tile's 32 positions
    float cm = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) cm = fmaxf(cm, sc[j]);
    cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
    cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
    const float mn = fmaxf(mx, cm);
    const float corr = mx == -__builtin_inff() ? 0.f : exp2f((mx - mn) * kLog2e);
    float pv[8], ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pv[j] = sc[j] == -__builtin_inff() ? 0.f : exp2f((sc[j] - mn) * kLog2e);
      ps += pv[j];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    lsum = lsum * corr + ps;
    mx = mn;
    // R rows are heads 4 lg + i: their correction factors sit in lanes 4 lg + i
    float ci[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ci[i] = __shfl(corr, 4 * lg + i, 64);
    half8 ph;
#pragma unroll
    for (int j = 0; j < 8; ++j) ph[j] = (half_t)pv[j];
    // B = h'[8 lg + j][c0 + 16 n + lq] (j = 0 .. 7) through two LDS transpose
    // reads: within each group of 16 lanes, output lane i gets element i % 4
    // of the 8 bytes read by lane 4 k + i / 4, as its element k. So lane lq
    // reads columns 4 (lq % 4) .. +3 of row 8 lg + lq / 4 (then of row
    // 8 lg + 4 + lq / 4), and lane lq receives column lq of rows 8 lg + k.
    const int trow0 = row_of(8 * lg + (lq >> 2)), trow1 = row_of(8 * lg + 4 + (lq >> 2));
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int tcol = col_of(c0 + 16 * n + 4 * (lq & 3));
      const half4 b0 = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((TL_LDS fp16x4*)(hs + trow0 + tcol)));
      const half4 b1 = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((TL_LDS fp16x4*)(hs + trow1 + tcol)));
      const half8 bv = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
      float4v r = R[n];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] *= ci[i];
      R[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bv, r, 0, 0, 0);
    }
  }
  }
  // partial of (row, split): per head [max, sum, r[0..D)]
  float* pp = a.part + ((size_t)row * a.S + split) * H * (D + 2);
  if (w == 0 && lg == 0) {
    pp[(size_t)lq * (D + 2)] = mx;
    pp[(size_t)lq * (D + 2) + 1] = lsum;
  }
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) pp[(size_t)(4 * lg + i) * (D + 2) + 2 + c0 + 16 * n + lq] = R[n][i];
}

// Merge of the key splits, one workgroup per (row, head, 256 columns): every workgroup forms the split weights exp(m_s - M) and the
// total L = sum_s l_s w_s in split order, then r[c] = (sum_s w_s r_s[c]) / L
// for its 256 columns, the splits added in order (their loads issued sixteen
// at a time). r goes to out [rows][H][D] (fp32).
__global__ __launch_bounds__(256) void absorbed_merge_kernel(int D, int H, const int32_t* row_lane,
                                                             const int32_t* row_pos,
                                                             const int32_t* status,
                                                             const float* part, int S,
                                                             int split_len, float* out) {
  constexpr int U = 64;   // splits whose column values a thread loads at once
  __shared__ float ms[1024];
  __shared__ float wgt[1024];
  __shared__ float red[4];
  __shared__ float lsh;
  const int parts = D / 256, q4 = blockIdx.x % parts, rh = blockIdx.x / parts;
  const int r = rh / H, h = rh % H;
  if (status[row_lane[r]] == TL_LANE_ABORTED || row_pos[r] < 0) return;
  const int T = row_pos[r] + 1;
  const int ns = (T + split_len - 1) / split_len;   // >= 1, <= S
  const size_t sstride = (size_t)H * (D + 2);
  const float* p = part + (size_t)r * S * sstride + (size_t)h * (D + 2);
  const int t = threadIdx.x;
  const int c = q4 * 256 + t;
  const float* pc = p + 2 + c;
  // the first U splits' values of this column go out with the maxima and sums
  float v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = pc[(size_t)min(u, ns - 1) * sstride];
  float mloc = -__builtin_inff();
  for (int s = t; s < ns; s += 256) {
    const float m = p[s * sstride];
    ms[s] = m;
    wgt[s] = p[s * sstride + 1];
    mloc = fmaxf(mloc, m);
  }
  const float M = block_max(mloc, red);   // (its barriers also publish ms, wgt)
  for (int s = t; s < ns; s += 256) ms[s] = exp2f((ms[s] - M) * kLog2e);
  __syncthreads();
  if (t == 0) {
    float L = 0.f;
    for (int s = 0; s < ns; ++s) L = fmaf(wgt[s], ms[s], L);
    lsh = L;
  }
  float acc = 0.f;
  for (int c0 = 0; c0 < ns; c0 += U) {
    if (c0) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = pc[(size_t)min(c0 + u, ns - 1) * sstride];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u < ns) acc = fmaf(v[u], ms[c0 + u], acc);
  }
  __syncthreads();
  out[((size_t)r * H + h) * D + c] = __fdiv_rn(acc, lsh);
}

// o[row][h d + j] = W_v[h d + j][:] . r[row][h][:] in fp32, rounded to the
// model dtype. One workgroup per (head, 4 outputs); wave w takes output
// j0 + w for every row, lane l columns CPL l .. CPL l + CPL - 1 (CPL = D / 64),
// the lanes added in a fixed butterfly order.
template <int D>
__global__ __launch_bounds__(256) void absorbed_o_kernel(int H, int dh, int n_rows,
                                                         const int32_t* row_lane,
                                                         const int32_t* row_pos,
                                                         const int32_t* status, const float* rbuf,
                                                         const half_t* wv, half_t* out) {
  constexpr int CPL = D / 64;
  const int h = blockIdx.x / (dh / 4), j = (blockIdx.x % (dh / 4)) * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  float wr[CPL];
  {
    const half_t* src = wv + ((size_t)h * dh + j) * D + CPL * l;
#pragma unroll
    for (int k = 0; k < CPL; k += 8) {
      const half8 a0 = *(const half8*)(src + k);
#pragma unroll
      for (int i = 0; i < 8; ++i) wr[k + i] = (float)a0[i];
    }
  }
  for (int r = 0; r < n_rows; ++r) {
    if (status[row_lane[r]] == TL_LANE_ABORTED || row_pos[r] < 0) continue;
    const float* rr = rbuf + ((size_t)r * H + h) * D + CPL * l;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; i += 4) {
      const float4v v = *(const float4v*)(rr + i);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc = fmaf(wr[i + k], v[k], acc);
    }
    acc = wave_sum(acc);
    if (l == 0) out[(size_t)r * D + h * dh + j] = (half_t)acc;
  }
}

}  // namespace

bool absorbed_supported(const ModelView& m, int view_mode) {
  const bool shape = m.dtype == TL_DTYPE_F16 && m.H == 16 &&
                     ((m.D == 1024 && m.dh == 64) || (m.D == 2048 && m.dh == 128));
  return shape && (view_mode == TL_CACHE_H_INT4 || view_mode == TL_CACHE_H_INT8 ||
                   view_mode == TL_CACHE_H_F16);
}

int absorbed_splits(int n_rows, int t_ub, int pair_cap, int* split_len) {
  // The staged tile takes more than half of a CU's LDS, so one workgroup runs
  // per CU: the splits of all rows are sized to fit one dispatch round of
  // kCUs workgroups, each covering a whole number of 32-position tiles, at
  // least two (a split pays a fixed cost: its qt operands and an H x D
  // partial). (A rule aiming at about 512 workgroups gave 528, three rounds,
  // for 48 rows of 2049 positions.)
  const int tiles = (t_ub + kAbsTP - 1) / kAbsTP;
  const int per_row = std::max(1, kCUs / n_rows);
  int tps = std::max(2, (tiles + per_row - 1) / per_row);
  int S = (tiles + tps - 1) / tps;
  const int cap = std::max(1, pair_cap / n_rows);
  if (S > cap) {
    tps = (tiles + cap - 1) / cap;
    S = (tiles + tps - 1) / tps;
  }
  *split_len = tps * kAbsTP;
  return std::max(1, (t_ub + *split_len - 1) / *split_len);
}

hipError_t launch_absorb_q(const ModelView& m, int n_rows, const float* q, const void* w_qkv,
                           float* qt, hipStream_t s) {
  if (m.D % 128 || n_rows < 1) return hipErrorInvalidValue;
  const half_t* wk = (const half_t*)w_qkv + (size_t)m.D * m.D;
  const dim3 grid(m.D / 64, m.H);
  if (m.dh == 64) absorb_q_kernel<64><<<grid, 64, 0, s>>>(m.D, n_rows, q, wk, qt);
  else if (m.dh == 128) absorb_q_kernel<128><<<grid, 64, 0, s>>>(m.D, n_rows, q, wk, qt);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_absorbed_attn(const ModelView& m, const CacheView& c, int layer, int n_rows,
                                const int32_t* row_lane, const int32_t* row_pos,
                                const int32_t* status, const float* qt, float* part, int S,
                                int split_len, hipStream_t s, const LaunchEvents& ev) {
  if (!absorbed_supported(m, c.mode) || n_rows < 1 || S < 1) return hipErrorInvalidValue;
  AbsArgs a{};
  a.cache = c; a.layer = layer; a.row_lane = row_lane; a.row_pos = row_pos; a.status = status;
  a.qt = qt; a.part = part; a.S = S; a.split_len = split_len;
  const int grid = n_rows * S;
#define TL_ABS(D_)                                                                              \
  do {                                                                                          \
    constexpr int NW_ = D_ == 1024 ? 8 : 4;                                                    \
    if (c.mode == TL_CACHE_H_INT4) return launch_timed(absorbed_attn_kernel<TL_CACHE_H_INT4, D_, NW_>, grid, NW_ * 64, s, ev, a); \
    if (c.mode == TL_CACHE_H_INT8) return launch_timed(absorbed_attn_kernel<TL_CACHE_H_INT8, D_, NW_>, grid, NW_ * 64, s, ev, a); \
    return launch_timed(absorbed_attn_kernel<TL_CACHE_H_F16, D_, NW_>, grid, NW_ * 64, s, ev, a);          \
  } while (0)
  if (m.D == 1024) TL_ABS(1024);
  else TL_ABS(2048);
#undef TL_ABS
}

hipError_t launch_absorbed_out(const ModelView& m, int n_rows, const int32_t* row_lane,
                               const int32_t* row_pos, const int32_t* status, const float* part,
                               int S, int split_len, const void* w_qkv, float* rbuf, void* o,
                               hipStream_t s) {
  if ((m.D != 1024 && m.D != 2048) || m.dh % 4 || S > 1024 || n_rows < 1) return hipErrorInvalidValue;
  absorbed_merge_kernel<<<n_rows * m.H * (m.D / 256), 256, 0, s>>>(m.D, m.H, row_lane, row_pos, status,
                                                                  part, S, split_len, rbuf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const half_t* wv = (const half_t*)w_qkv + (size_t)2 * m.D * m.D;
  const int grid = m.H * (m.dh / 4);
  if (m.D == 1024)
    absorbed_o_kernel<1024><<<grid, 256, 0, s>>>(m.H, m.dh, n_rows, row_lane, row_pos, status, rbuf, wv, (half_t*)o);
  else
    absorbed_o_kernel<2048><<<grid, 256, 0, s>>>(m.H, m.dh, n_rows, row_lane, row_pos, status, rbuf, wv, (half_t*)o);
  return hipGetLastError();
}

}  // namespace tl
