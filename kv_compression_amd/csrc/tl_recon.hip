// Store-h attention: rebuild K = W_k h' and V = W_v h' for cached positions
// from the stored h (TinyLoop architecture-exclusive features page, "Store-h
// KV cache"; novel-contributions page, "Store-h KV Cache") on MFMA, and either
// fold them straight into online-softmax attention partials (decode) or store
// them for the causal prefill attention.
//
// One workgroup computes the product tile C[f, j] = sum_k W[f, k] h'[j, k] for
// BF features (the K and V rows of whole heads, interleaved per head at
// decode) and BJ cached positions of one lane, streaming d_model in BK = 64
// deep stages on v_mfma_f32_32x32x16_f16 (fp32 accumulators). Features run
// down the MFMA rows and positions along its columns, so each lane ends up
// holding whole positions.
//   * INT4 / INT8 h: the W tile, the h codes and the INT4 scales of a stage
//     are copied by the memory unit straight into an LDS ring of two or
//     three stage buffers (buffer loads to LDS); each of four waves owns all
//     the tile's features for 64 positions and dequantises its codes in
//     registers into the B operand, fp16(q * s) exactly, one k-step ahead of
//     the MFMAs.
//   * fp16 h at 64-wide heads: the W and h tiles are copied into the ring
//     the same way and the h fragments are read from it as the B operand.
//   * other fp16 configurations and fp32 h: both operands go through
//     registers into a two-buffer LDS tile, one stage ahead; waves are laid
//     out over features and positions.
// The decode epilogue reads the scores q . K_j out of the accumulators,
// applies a wave-level online softmax and reduces p_j V_j across lanes into
// (max, sum, o) per (row, head, position tile); the last workgroup to finish
// a (row, head group) merges that row's tiles itself. The prefill epilogue
// stores the K | V rows for the causal attention kernel.
#include <type_traits>

#include "tl_device.h"

namespace tl {

namespace {

// Tile shapes (BF features x BJ positions per workgroup, WF x WJ per wave).
//   INT4 / INT8 h (operands copied to LDS, h dequantised in registers): 4
//   waves, one per SIMD, each owning all the tile's features for 64
//   positions: 256 features (two heads of 64 or one of 128; 256 accumulators
//   in AGPRs), or 128 (one head of 64, two workgroups per CU). Every
//   dequantised h operand feeds 8 (or 4) MFMAs, and the MFMAs of one k-step
//   cover the dequantisation and LDS reads of the next.
//   fp16 h (staged through LDS from registers): 8 waves, 2 per SIMD, 128 x 64.
//   fp32: 4 waves of 64 x 64.
// OCC: workgroups resident per CU (waves per SIMD), which sets the register
// budget of a wave (512 / OCC, accumulators included). NBUF: stage buffers of
// the LDS ring of the copied-operand path.
template <typename T, int MODE, int DH, int VAR = 0> struct Cfg {
  static constexpr int BF = 256, BJ = 256, WF = 128, WJ = 64, BK = 64, OCC = 1, NBUF = 3;
  static constexpr int NT = 64 * (BF / WF) * (BJ / WJ);
  static constexpr bool COPY16 = false;   // fp16 h through the copied-operand ring
};
// fp16 h at 64-wide heads: the W tile and the h tile (both 128-byte rows of
// one stage) are copied into a two-buffer ring and the h fragments are read
// from it as the MFMA B operand, 8 waves of one head x 64 positions
template <> struct Cfg<half_t, TL_CACHE_H_F16, 64> {
  static constexpr int BF = 256, BJ = 256, WF = 128, WJ = 64, BK = 64, OCC = 1, NBUF = 2;
  static constexpr int NT = 64 * (BF / WF) * (BJ / WJ);
  static constexpr bool COPY16 = true;
};
// fp16 h at 64-wide heads when a launch has too few rows and position tiles
// to give every CU a workgroup of the configuration above (one lane at a
// context of about a thousand: 40 workgroups): one head (its 64 K and 64 V
// rows) per workgroup, so twice the workgroups with half the work each.
template <> struct Cfg<half_t, TL_CACHE_H_F16, 64, 1> {
  static constexpr int BF = 128, BJ = 256, WF = 128, WJ = 64, BK = 64, OCC = 1, NBUF = 3;
  static constexpr int NT = 64 * (BF / WF) * (BJ / WJ);
  static constexpr bool COPY16 = false;
};
// ... and with 128-position tiles, four waves of 32 positions, when even that
// leaves CUs idle (all four SIMDs of a CU busy: 19.8 against 24.4 us for two
// waves of 64 at one lane and context 1030-1150)
template <> struct Cfg<half_t, TL_CACHE_H_F16, 64, 2> {
  static constexpr int BF = 128, BJ = 128, WF = 128, WJ = 32, BK = 64, OCC = 1, NBUF = 3;
  static constexpr int NT = 64 * (BF / WF) * (BJ / WJ);
  static constexpr bool COPY16 = false;
};
// integer codes: every wave covers all BF features of its positions
template <int MODE, int DH> struct CfgCodes {
  static constexpr int BF = 256, BJ = 256, WF = 256, WJ = 64, BK = 64, OCC = 1, NBUF = 3;
  static constexpr int NT = 64 * (BF / WF) * (BJ / WJ);
  static constexpr bool COPY16 = false;
};
template <int DH> struct Cfg<half_t, TL_CACHE_H_INT8, DH> : CfgCodes<TL_CACHE_H_INT8, DH> {};
template <int DH> struct Cfg<half_t, TL_CACHE_H_INT4, DH> : CfgCodes<TL_CACHE_H_INT4, DH> {};
// INT4 codes with 64-wide heads: one head (K and V rows) per workgroup and two
// workgroups per CU, so one workgroup's prologue and epilogue run under the
// other's MFMAs, and a dispatch round that is only partly filled still
// spreads over twice as many CUs. (Eight waves over 512 positions, one
// workgroup per CU, time the same at 4096 positions and lose a third
// dispatch round just past it.)
template <> struct Cfg<half_t, TL_CACHE_H_INT4, 64> {
  static constexpr int BF = 128, BJ = 256, WF = 128, WJ = 64, BK = 64, OCC = 2, NBUF = 3;
  static constexpr int NT = 64 * (BF / WF) * (BJ / WJ);
  static constexpr bool COPY16 = false;
};
// INT8 codes with 64-wide heads: the same shape, two workgroups per CU; a
// stage's h codes are twice INT4's, so the ring has two stage buffers (a
// stage's copies have one stage of MFMA work to land, which the other
// workgroup's MFMAs lengthen)
template <> struct Cfg<half_t, TL_CACHE_H_INT8, 64> {
  static constexpr int BF = 128, BJ = 256, WF = 128, WJ = 64, BK = 64, OCC = 2, NBUF = 2;
  static constexpr int NT = 64 * (BF / WF) * (BJ / WJ);
  static constexpr bool COPY16 = false;
};
template <int MODE, int DH> struct Cfg<float, MODE, DH> {
  static constexpr int BF = 128, BJ = 128, WF = 64, WJ = 64, BK = 64, OCC = 1, NBUF = 3;
  static constexpr int NT = 64 * (BF / WF) * (BJ / WJ);
  static constexpr bool COPY16 = false;
};
// the fp16 configurations other than INT4 at 64-wide heads share BJ and WJ
// (split length); the one-head fp16 ones run only with the tile merge in the
// launch, whose partials are per tile
static_assert(Cfg<half_t, TL_CACHE_H_INT4, 128>::BJ == Cfg<half_t, TL_CACHE_H_F16, 64>::BJ &&
              Cfg<half_t, TL_CACHE_H_F16, 64, 1>::BJ == Cfg<half_t, TL_CACHE_H_F16, 64>::BJ &&
              Cfg<half_t, TL_CACHE_H_INT8, 64>::BJ == Cfg<half_t, TL_CACHE_H_F16, 64>::BJ &&
              Cfg<half_t, TL_CACHE_H_INT4, 64>::WJ == Cfg<half_t, TL_CACHE_H_F16, 64>::WJ &&
              Cfg<half_t, TL_CACHE_H_INT8, 64>::WJ == Cfg<half_t, TL_CACHE_H_F16, 64>::WJ, "fp16 tiles");

enum { EPI_ATTN = 0, EPI_KVSTORE = 1 };
// position tiles a decode workgroup of the INT4 / INT8 configurations at
// 64-wide heads takes, one after the other
constexpr int kMaxTilesPerWorkgroup = 2;

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
  int n_hg, n_ptiles, n_rows, hpx;
  // decode
  const int32_t* row_lane;
  const int32_t* row_pos;
  const int32_t* status;
  const float* q;
  float* part;
  int S;
  void* o;                   // with tilecnt: merged output [rows, D]
  int32_t* tilecnt;          // [rows, n_hg] workgroups done, zero between launches
  int tpw;                   // decode, INT4 / INT8 tiles: position tiles per workgroup (1 or 2)
  // prefill store
  int lane, T;
  void* kvbuf;
};

// chunks of 16 bytes per thread per stage for an LDS-staged h tile
template <int MODE> struct HLoad { static constexpr int NCH = 1, CPP = 1; };
template <> struct HLoad<TL_CACHE_H_F16> { static constexpr int NCH = 4, CPP = 8; };   // (NCH of 512 threads)
template <> struct HLoad<TL_CACHE_H_F32> { static constexpr int NCH = 8, CPP = 16; };  // 256 threads

// Value of lane partner(l) for a data-parallel-primitive pattern within each
// row of 16 lanes: row_mirror (l ^ 15), row_half_mirror (l ^ 7) and the quad
// permutations l ^ 2 and l ^ 1. Lane bit 4 goes through the LDS crossbar.
constexpr int kDppRowMirror = 0x140, kDppHalfMirror = 0x141, kDppXor2 = 0x4E, kDppXor1 = 0xB1;
template <int CTRL>
__device__ __forceinline__ float lane_swap(float x) {
  if constexpr (CTRL == 16) return __shfl_xor(x, 16, 64);
  else return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Lane bits of a 32-lane half-wave in the order the reductions visit them,
// with the partner pattern of each: the partner differs in the visited bit and
// agrees in the bits visited before it, which is all a butterfly needs.
constexpr int kRsBit[5] = {3, 2, 1, 0, 4};
constexpr int kRsCtrl[5] = {kDppRowMirror, kDppHalfMirror, kDppXor2, kDppXor1, 16};

// One level of a reduce-scatter over lane bit kRsBit[LV]: the lanes with that
// bit set keep the upper half of v, the others the lower half, each adding its
// partner's copy. LEN is the current length (compile time, so v stays in
// registers); at LEN 1 the level is a plain all-reduce.
template <int LEN, int LV>
__device__ __forceinline__ void rs_level(float* v, int l) {
  constexpr int CTRL = kRsCtrl[LV];
  if constexpr (LEN >= 2) {
    const bool up = (l >> kRsBit[LV]) & 1;
#pragma unroll
    for (int e = 0; e < LEN / 2; ++e) {
      const float keep = up ? v[e + LEN / 2] : v[e];
      const float send = up ? v[e] : v[e + LEN / 2];
      v[e] = keep + lane_swap<CTRL>(send);
    }
  } else {
    v[0] += lane_swap<CTRL>(v[0]);
  }
}
// Sum v[0..NV) over the 32 lanes of each half-wave. Lane l ends with
// max(NV / 32, 1) values, v[k] holding index rs_index<NV>(l, k); for NV == 16
// lanes l and l ^ 16 hold the same value.
template <int NV>
__device__ __forceinline__ void reduce_scatter32(float* v, int l) {
  rs_level<NV, 0>(v, l);
  rs_level<(NV >> 1), 1>(v, l);
  rs_level<(NV >> 2), 2>(v, l);
  rs_level<(NV >> 3), 3>(v, l);
  rs_level<(NV >> 4), 4>(v, l);
}
template <int NV>
__device__ __forceinline__ int rs_index(int l, int k) {
  int idx = 0, len = NV;
#pragma unroll
  for (int lv = 0; lv < 5; ++lv)
    if (len >= 2) {
      len >>= 1;
      idx += ((l >> kRsBit[lv]) & 1) * len;
    }
  return idx + k;
}
// All-reduce (max or sum) over the 32 lanes of each half-wave.
template <bool MAX>
__device__ __forceinline__ float allreduce32(float x) {
#pragma unroll
  for (int lv = 0; lv < 5; ++lv) {
    float y;
    switch (lv) {
      case 0: y = lane_swap<kRsCtrl[0]>(x); break;
      case 1: y = lane_swap<kRsCtrl[1]>(x); break;
      case 2: y = lane_swap<kRsCtrl[2]>(x); break;
      case 3: y = lane_swap<kRsCtrl[3]>(x); break;
      default: y = lane_swap<kRsCtrl[4]>(x); break;
    }
    x = MAX ? fmaxf(x, y) : x + y;
  }
  return x;
}

// Call f(integral_constant<int, n>) for the run-time n in [0, CB].
template <int CB, typename F>
__device__ __forceinline__ void dispatch_nb(int n, F&& f) {
  if constexpr (CB == 4) {
    if (n >= 4) f(std::integral_constant<int, 4>{});
    else if (n == 3) f(std::integral_constant<int, 3>{});
    else if (n == 2) f(std::integral_constant<int, 2>{});
    else if (n == 1) f(std::integral_constant<int, 1>{});
    else f(std::integral_constant<int, 0>{});
  } else if constexpr (CB == 2) {
    if (n >= 2) f(std::integral_constant<int, 2>{});
    else if (n == 1) f(std::integral_constant<int, 1>{});
    else f(std::integral_constant<int, 0>{});
  } else {
    static_assert(CB == 1, "1, 2 or 4 position blocks per wave");
    if (n >= 1) f(std::integral_constant<int, 1>{});
    else f(std::integral_constant<int, 0>{});
  }
}

// Raw codes of one lane for one stage: per 32-position block, the lane's
// 16-byte (INT4) or 32-byte (INT8) k-run and, for INT4, the two group scales.
template <int MODE, int CB> struct Raw { u32x4 w[CB]; };
template <int CB> struct Raw<TL_CACHE_H_INT4, CB> {
  u32x4 w[CB];
  uint32_t s[CB];
};
template <int CB> struct Raw<TL_CACHE_H_INT8, CB> {
  u32x4 w[CB][2];
};
// fp16 h is read from the ring as the operand is needed: nothing to hold
template <int CB> struct Raw<TL_CACHE_H_F16, CB> {
};

#define TL_LDS __attribute__((address_space(3)))

// Word 3 of a raw buffer resource on this architecture: 32-bit data format,
// no swizzling, offsets checked against the byte extent.
constexpr int kRsrcWord3 = 0x00020000;

// One buffer of the LDS ring: a separate LDS array per index, so the compiler
// can tell that reads of one buffer do not depend on copies into another.
template <int B, int BYTES> struct Ring {
  static __device__ __forceinline__ char* p() {
    __shared__ __attribute__((aligned(16))) char buf[BYTES];
    return buf;
  }
};

// Wait until at most N of this wave's memory loads (LDS copies included) are
// outstanding and its LDS reads are done, then synchronise the workgroup. The
// empty asm statements keep the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void dma_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  // s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4] (7: no wait), lgkmcnt [11:8]
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Make this wave's LDS writes visible to the workgroup without waiting for its
// memory loads (LDS copies in flight stay in flight): wait for LDS only, then
// synchronise.
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  // vmcnt 63 (no wait), expcnt 7 (no wait), lgkmcnt 0
  __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Slot swizzle of the 128-byte W rows in the LDS ring: rows R..R+15 (R a
// multiple of 16) reading the same chunk land on 16 distinct 16-byte slots of
// a 256-byte bank window, and any 8 consecutive rows on 8 distinct slots.
__device__ __forceinline__ int w_swz(int R) { return ((R >> 1) ^ (R << 2)) & 7; }

template <typename T, int MODE, int DH, int EPI, int VAR = 0>
__global__ __launch_bounds__((Cfg<T, MODE, DH, VAR>::NT), (Cfg<T, MODE, DH, VAR>::OCC)) void recon_kernel(KArgs a) {
  typedef Cfg<T, MODE, DH, VAR> C;
  constexpr int BF = C::BF, BJ = C::BJ, WF = C::WF, WJ = C::WJ, BK = C::BK, NT = C::NT, NBUF = C::NBUF;
  static_assert(NBUF == 2 || NBUF == 3, "ring depth");
  constexpr int WJN = BJ / WJ;                // waves along positions
  constexpr int ES = sizeof(T);
  constexpr int ROWB = BK * ES + 16;          // padded LDS row bytes
  constexpr int RB = WF / 32, CB = WJ / 32;   // MFMA blocks per wave
  constexpr int A_CPR = BK * ES / 16;         // 16-byte chunks per W row per stage
  constexpr int A_NCH = BF * A_CPR / NT;      // per thread
  constexpr bool B_REG = MODE == TL_CACHE_H_INT4 || MODE == TL_CACHE_H_INT8;   // codes dequantised in registers
  constexpr bool H16C = C::COPY16;                    // fp16 h read from the ring
  constexpr bool COPY = B_REG || H16C;                // operands copied into an LDS ring
  static_assert(!H16C || (MODE == TL_CACHE_H_F16 && std::is_same<T, half_t>::value), "fp16 h");
  constexpr int B_NCH = B_REG ? HLoad<MODE>::NCH : BJ * HLoad<MODE>::CPP / NT;   // h chunks per thread
  constexpr int B_CPP = HLoad<MODE>::CPP;     // chunks per position
  static_assert(B_REG || BJ * B_CPP == NT * B_NCH, "h tile chunks");
  static_assert(!COPY || (std::is_same<T, half_t>::value && BK == kKBlock), "copied-operand path");
  constexpr int TILE_BYTES = (COPY ? BF : BF + BJ) * ROWB;   // one LDS buffer (LDS-staged h)
  __shared__ __attribute__((aligned(16))) char smem[COPY ? 16 : 2 * TILE_BYTES];
  constexpr int HRB = block_row_bytes(MODE);
  // one LDS ring buffer of the copied path: W tile, h codes, INT4 scales
  constexpr int RING = COPY ? BF * BK * ES + BJ * HRB + (MODE == TL_CACHE_H_INT4 ? BJ * 4 : 0) : 16;
  // per-wave attention partials of the copied-operand path, combined in LDS
  constexpr int NWV = NT / 64;
  constexpr int HPW_T = 2 * DH > WF ? 1 : WF / (2 * DH);   // heads per wave
  constexpr int HGT = 2 * DH > BF ? 1 : BF / (2 * DH);     // heads per workgroup
  __shared__ __attribute__((aligned(16))) float comb_lds[COPY && EPI == EPI_ATTN ? NWV * HPW_T * (DH + 2) : 1];
  // the queries of the workgroup's heads, staged at the start
  __shared__ __attribute__((aligned(16))) float q_lds[COPY && EPI == EPI_ATTN ? HGT * DH : 1];

  const int tid = threadIdx.x, l = tid & 63, wave = tid >> 6;
  const int wf = wave / WJN, wj = wave % WJN;
  const int D = a.D;

  // the kernel arguments the prologue uses, fetched in one batch at the start
  // (otherwise each is loaded where it is first needed, one scalar round trip
  // after another ahead of the first copy)
  __asm__ volatile("" ::"s"(a.cache.base), "s"(a.cache.scales), "s"(a.cache.mode), "s"(a.cache.max_seq),
                   "s"(a.cache.n_lanes),
                   "s"(a.layer), "s"(a.w_qkv), "s"(a.D), "s"(a.n_hg), "s"(a.hpx), "s"(a.n_rows),
                   "s"(a.n_ptiles), "s"(a.row_lane), "s"(a.row_pos), "s"(a.status), "s"(a.q));
  int hg, ptile, r = 0, lane, Tn;
  if (EPI == EPI_ATTN) {
    // head group fastest (consecutive workgroups land on different XCDs, each
    // XCD keeping its head group's W rows in L2), position tile slowest so the
    // partial last tiles of the lanes form the final dispatch round
    // Workgroup b runs on XCD b % 8. Each XCD takes a set of a.hpx head groups
    // (their W rows stay in its L2) and every (8 / sets)-th tile, and runs the
    // head groups of one tile back to back, so a tile's h codes are fetched
    // into that XCD's L2 once and reused by the set. Tiles are numbered
    // position-tile-major so the partial last tiles dispatch last.
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int sets = a.n_hg / a.hpx, parts = 8 / sets;
    hg = (xcd % sets) * a.hpx + idx % a.hpx;
    const int tile = (idx / a.hpx) * parts + xcd / sets;
    r = tile % a.n_rows;
    ptile = tile / a.n_rows;
    if (ptile >= a.n_ptiles) return;
    // the row's lane and length load together; with the copied operands the
    // lane's status is read after the first stages' copies have gone out (a
    // stopped lane's workgroup then waits for them and leaves), so the
    // prologue takes two dependent lookups instead of three
    lane = a.row_lane[r];
    Tn = a.row_pos[r] + 1;
    __asm__ volatile("" ::"s"(lane), "s"(Tn));   // both loads in flight together
    if constexpr (!COPY)
      if (a.status[lane] == TL_LANE_ABORTED) return;
  } else {
    hg = blockIdx.x % a.n_hg;
    ptile = blockIdx.x / a.n_hg;
    lane = a.lane;
    if (a.status && a.status[lane] == TL_LANE_ABORTED) return;
    Tn = a.T;
  }
  // A decode workgroup of the INT4 / INT8 configurations takes TPW
  // consecutive position tiles of its (row, head group), one after the other
  // (each writes its own partial, as a workgroup per tile would), and counts
  // itself once for the tile merge: one prologue's lookups and one handoff
  // per TPW tiles.
  // (INT4 / INT8 codes at 64-wide heads only: at 128 the loop leaves the
  // register allocation no room and spills)
  constexpr int TPW_MAX = EPI == EPI_ATTN && B_REG && DH == 64 ? kMaxTilesPerWorkgroup : 1;
  const int TPW = TPW_MAX > 1 ? min(max(a.tpw, 1), TPW_MAX) : 1;
  const int wtile = ptile;
#pragma nounroll
  for (int sub = 0; sub < TPW_MAX; ++sub) {
  if (sub >= TPW) break;
  // the row and head group are opaque to the compiler here, so what the tile
  // derives from them is recomputed per tile rather than held in registers
  // across the loop
  hg = __builtin_amdgcn_readfirstlane(hg);
  r = __builtin_amdgcn_readfirstlane(r);
  lane = __builtin_amdgcn_readfirstlane(lane);
  Tn = __builtin_amdgcn_readfirstlane(Tn);
  __asm__ volatile("" : "+s"(hg), "+s"(r), "+s"(lane), "+s"(Tn));
  ptile = wtile * TPW + sub;
  const int j0 = ptile * BJ;
  if (j0 >= Tn) {
    if (sub == 0) return;
    break;
  }
  // the workgroup's last tile (it then counts itself)
  const bool last_sub = sub + 1 == TPW || j0 + BJ >= Tn;

  // ---- W rows of this workgroup's BF features ------------------------------
  // Thread t loads 16-byte chunk `part` of A-tile rows f = f0 + F0STEP * i
  // (f0 = t / A_CPR). The W row of tile row f is f0 + C(i) with C(i) uniform:
  // decode tiles interleave heads as [K_t | V_t] per head, prefill tiles keep
  // the natural K | V order.
  constexpr int F0STEP = NT / A_CPR;
  static_assert(DH % F0STEP == 0, "head dim must be a multiple of the row step");
  const T* W = (const T*)a.w_qkv;
  const int f0 = tid / A_CPR, apart = tid % A_CPR;
  const T* wbase = W + (size_t)f0 * D + apart * (16 / ES);
  auto wrow_off = [&](int i) -> size_t {
    const int fi = F0STEP * i;
    int r0;
    if (EPI == EPI_ATTN) {
      const int within = fi % (2 * DH);
      const int head = hg * (BF / (2 * DH)) + fi / (2 * DH);
      r0 = D * (within < DH ? 1 : 2) + head * DH + (within % DH);
    } else {
      r0 = D + hg * BF + fi;
    }
    return (size_t)r0 * D;
  };

  // W row of tile row f
  auto wrow = [&](int f) -> int {
    if (EPI == EPI_ATTN) {
      const int within = f % (2 * DH);
      const int head = hg * (BF / (2 * DH)) + f / (2 * DH);
      return D * (within < DH ? 1 : 2) + head * DH + (within % DH);
    }
    return D + hg * BF + f;
  };

  const CacheView& cv = a.cache;
  const char* hbase = cv.code_row(a.layer, lane, 0, 0);
  const size_t kb_stride = (size_t)cv.max_seq * HRB;
  const int nst = D / BK;

  // Tile-local position of this lane in the wave's 32-position block j. The
  // copied-operand path deals the tile's blocks round-robin to the waves
  // (block j*WJN + wj), so a partial last tile spreads over all waves; the
  // LDS-staged path gives each wave WJ consecutive positions.
  auto pos_local = [&](int j) -> int {
    return COPY ? (j * WJN + wj) * 32 + (l & 31) : wj * WJ + j * 32 + (l & 31);
  };
  // blocks of this wave that hold positions < T (a prefix of j = 0, 1, ...);
  // the others are all zero, so their MFMAs are skipped while the wave keeps
  // loading and synchronising
  int ncb;
  if constexpr (COPY) {
    const int nbl = min(max((Tn - j0 + 31) / 32, 0), BJ / 32);
    ncb = 0;
#pragma unroll
    for (int j = 0; j < CB; ++j)
      if (j * WJN + wj < nbl) ncb = j + 1;
  } else {
    ncb = min(max((Tn - (j0 + wj * WJ) + 31) / 32, 0), CB);
  }
  const bool wave_live = ncb > 0;

  typedef typename Mma<T>::frag Frag;
  float16v acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = float16v{};

  u32x4 ra[A_NCH];
  auto load_w = [&](int st) {
    const T* wk = wbase + st * BK;
#pragma unroll
    for (int i = 0; i < A_NCH; ++i) ra[i] = *(const u32x4*)(wk + wrow_off(i));
  };
  auto store_w = [&](int buf) {
    char* As = smem + buf * TILE_BYTES;
#pragma unroll
    for (int i = 0; i < A_NCH; ++i) {
      const int c = tid + NT * i;
      *(u32x4*)(As + (c / A_CPR) * ROWB + (c % A_CPR) * 16) = ra[i];
    }
  };
  const int koff = 8 * (l >> 5) * ES;
  auto read_a = [&](int buf, int kk, Frag (&fa)[RB]) {
    const char* As = smem + buf * TILE_BYTES;
#pragma unroll
    for (int i = 0; i < RB; ++i)
      fa[i] = *(const Frag*)(As + (wf * WF + i * 32 + (l & 31)) * ROWB + kk * 16 * ES + koff);
  };

  if constexpr (COPY) {
    // ---- W rows and h copied by the memory unit straight into LDS -----------
    // A ring of NBUF stage buffers, each one separate LDS array: stage st
    // reads buffer st % NBUF while the copies of the next NBUF - 1 stages are
    // in flight, so every load has NBUF - 1 stages of MFMA work to land. Each
    // wave issues exactly DMA_PER_STAGE copies per stage; waiting until only
    // the copies after stage st+1 are outstanding (the counter drains in issue
    // order) and then synchronising the workgroup publishes the next stage's
    // buffer.
    //   W tile: BF rows x 128 bytes, 16-byte chunk c of row R at slot
    //     c ^ swz(R), so the fragment reads of 16 consecutive rows are spread
    //     over all banks without padding. One copy instruction fills 1 KB
    //     (64 lanes x 16 B in lane order); lane l of a wave's copy fetches
    //     whichever chunk belongs at its slot.
    //   h codes: per 16 positions, the 16-byte runs of run index hq (half hb,
    //     part q of that half's k-run) sit side by side, so lanes 0..15 of a
    //     fragment read touch 16 consecutive slots.
    //   fp16 h: BJ position rows of 128 bytes, laid out as the W tile (the
    //     B fragments are read from it like the A fragments).
    //   INT4 scales: one 32-bit word (two fp16 group scales) per position.
    // Positions past T copy the entry of position T-1 (always in bounds); the
    // codes are zeroed through their scale when the operand is built, and
    // fp16 rows are left as they are: their scores are masked, so their
    // finite K and V rows weigh nothing.
    constexpr int NW = NT / 64;
    constexpr int NQ = HRB / 32;                         // 16-byte runs per half row
    constexpr int W_BYTES = BF * BK * ES;
    constexpr int H_BYTES = BJ * HRB;
    constexpr int S_BYTES = MODE == TL_CACHE_H_INT4 ? BJ * 4 : 0;
    constexpr int W_IPW = W_BYTES / 1024 / NW, H_IPW = H_BYTES / 1024 / NW;
    constexpr int DMA_PER_STAGE = W_IPW + H_IPW + (S_BYTES ? 1 : 0);
    static_assert(W_IPW * NW * 1024 == W_BYTES && H_IPW * NW * 1024 == H_BYTES, "copy split");
    static_assert(S_BYTES == 0 || S_BYTES == NW * 256, "one 4-byte copy per lane and wave for the scales");
    static_assert(C::OCC * NBUF * (W_BYTES + H_BYTES + S_BYTES) <= 160 * 1024, "LDS ring");
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);

    uint32_t woff[W_IPW];     // byte offset of the lane's W chunk (stage 0)
#pragma unroll
    for (int i = 0; i < W_IPW; ++i) {
      const int u = (wave_u * W_IPW + i) * 64 + l;
      const int R = u >> 3;
      const int c = (u & 7) ^ w_swz(R);
      woff[i] = (uint32_t)(wrow(R) * (size_t)D * ES) + c * 16;
    }
    uint32_t hoff[H_IPW];     // byte offset of the lane's h run (stage 0)
#pragma unroll
    for (int i = 0; i < H_IPW; ++i) {
      const int S = (wave_u * H_IPW + i) * 64 + l;
      if constexpr (H16C) {
        const int R = S >> 3;
        const int c = (S & 7) ^ w_swz(R);
        hoff[i] = (uint32_t)min(j0 + R, Tn - 1) * HRB + c * 16;
      } else {
        const int pos = (S / (32 * NQ)) * 16 + S % 16;
        const int hq = (S / 16) % (2 * NQ);
        hoff[i] = (uint32_t)min(j0 + pos, Tn - 1) * HRB + hq * 16;
      }
    }
    const uint16_t* s4base = MODE == TL_CACHE_H_INT4 ? cv.int4_scale(a.layer, lane, 0, 0) : nullptr;
    // scale copy (LDS copies write one dword per lane): lane l of wave w
    // fetches the word of position 64 w + l
    const uint32_t soff = (uint32_t)min(j0 + wave_u * 64 + l, Tn - 1) * 2;

    // Copies go through buffer resources: the lane's offset stays in one VGPR,
    // the stage offset is a scalar, and the hardware drops any access past the
    // resource's extent instead of faulting.
    const __amdgpu_buffer_rsrc_t w_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.w_qkv, 0, 3 * D * D * ES, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t h_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)hbase, 0, (int)(nst * kb_stride), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)s4base, 0, S_BYTES ? nst * cv.max_seq * 4 : 0, kRsrcWord3);
    // The wave's copies of one stage, numbered 0 .. DMA_PER_STAGE-1 (W chunks,
    // then h runs, then the scale words); issue_ops<LO, HI> issues ops LO..HI-1.
    auto issue_ops = [&](auto buf_c, auto lo_c, auto hi_c, int st) {
      constexpr int LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
      char* rb = Ring<decltype(buf_c)::value, RING>::p();
#pragma unroll
      for (int i = 0; i < W_IPW; ++i)
        if (i >= LO && i < HI)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (TL_LDS void*)(rb + (wave_u * W_IPW + i) * 1024), 16,
                                                   (int)woff[i], st * BK * ES, 0, 0);
#pragma unroll
      for (int i = 0; i < H_IPW; ++i)
        if (W_IPW + i >= LO && W_IPW + i < HI)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(h_rsrc,
                                                   (TL_LDS void*)(rb + W_BYTES + (wave_u * H_IPW + i) * 1024), 16,
                                                   (int)hoff[i], (int)(st * kb_stride), 0, 0);
      if constexpr (S_BYTES > 0) {
        if (W_IPW + H_IPW >= LO && W_IPW + H_IPW < HI)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (TL_LDS void*)(rb + W_BYTES + H_BYTES + wave_u * 256), 4,
                                                   (int)(soff * 2), st * cv.max_seq * 4, 0, 0);
      }
    };
    // The copies of a stage go out in three parts, so that the four waves'
    // requests never queue up behind each other in the memory pipeline (a
    // wave stalls at issue while its request waits, MFMAs included): part A
    // right after the barrier that frees the buffer, parts B and C during the
    // first two k-steps of the following stage.
    constexpr int PA = (DMA_PER_STAGE + 2) / 3, PB = (DMA_PER_STAGE + 1) / 3;
    using IA0 = std::integral_constant<int, 0>;
    using IA1 = std::integral_constant<int, PA>;
    using IB1 = std::integral_constant<int, PA + PB>;
    using IC1 = std::integral_constant<int, DMA_PER_STAGE>;
    auto issue = [&](auto buf_c, int st) {
      issue_ops(buf_c, IA0{}, IC1{}, st);
    };

    // lane l serves positions p_j = j0 + wj*WJ + 32 j + l % 32 and, within each
    // 64-element block, the k-run of half-wave hb = l / 32
    const int hb = l >> 5;
    uint32_t vmask = 0;   // positions < T
#pragma unroll
    for (int j = 0; j < CB; ++j)
      if (j0 + pos_local(j) < Tn) vmask |= 1u << j;
    half_t s8[CB];
    if constexpr (MODE == TL_CACHE_H_INT8) {
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int pc = min(j0 + pos_local(j), Tn - 1);
        s8[j] = ((vmask >> j) & 1) ? h_from_bits(*cv.int8_scale(a.layer, lane, pc)) : (half_t)0.f;
      }
    }
    // fragment reads: W chunk kk*2 + hb of row wf*WF + i*32 + l%32 (the
    // swizzle depends on l % 32 only), and the lane's h runs
    const int arow = wf * WF + (l & 31);
    const int aswz = w_swz(arow);
    typedef Raw<MODE, CB> R;
    auto read_a3 = [&](const char* rb, int kk, Frag (&fa)[RB]) {
      const char* base = rb + arow * (BK * ES) + (((kk * 2 + hb) ^ aswz) * 16);
#pragma unroll
      for (int i = 0; i < RB; ++i) fa[i] = *(const Frag*)(base + i * 32 * (BK * ES));
    };
    auto read_raw = [&](auto nb_c, const char* rb, R& raw) {
      constexpr int NB = decltype(nb_c)::value;
      if constexpr (H16C) {
        (void)rb;
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int pos = pos_local(j);
          const char* hs = rb + W_BYTES + ((pos >> 4) * (32 * NQ) + hb * NQ * 16 + (pos & 15)) * 16;
          if constexpr (MODE == TL_CACHE_H_INT4) {
            raw.w[j] = *(const u32x4*)hs;
            raw.s[j] = *(const uint32_t*)(rb + W_BYTES + H_BYTES + pos * 4);
          } else {
            raw.w[j][0] = *(const u32x4*)hs;
            raw.w[j][1] = *(const u32x4*)(hs + 16 * 16);
          }
        }
      }
    };
    // MFMA operand of block j, k-step kk: 8 fp16 = fp16(q * s), or the fp16
    // h fragment (chunk kk*2 + hb of the block's position row) of ring
    // buffer rb.
    auto b_frag = [&](const R& raw, const char* rb, int j, int kk) -> half8 {
      if constexpr (H16C) {
        const uint32_t pos = (uint32_t)pos_local(j);
        uint32_t off = W_BYTES + pos * (BK * ES) + (((uint32_t)(kk * 2 + hb) ^ (uint32_t)w_swz(pos)) << 4);
        // The address is kept one offset away from the ring's LDS array (the
        // empty asm stops the offset being split into a chain of steps): the
        // compiler tells which copies in flight a read may depend on only by
        // tracing its address back to the array within a few steps, and
        // otherwise waits for all of them (here: the next stage's copies, at
        // every stage).
        __asm__("" : "+v"(off));
        return *(const half8*)(rb + off);
      } else if constexpr (MODE == TL_CACHE_H_INT4) {
        const uint32_t sv = ((vmask >> j) & 1) ? raw.s[j] : 0u;   // positions past T: scale 0
        const half_t sc = h_from_bits((uint16_t)(kk < 2 ? (sv & 0xFFFFu) : (sv >> 16)));
        return int4_dequant8(raw.w[j][kk], sc);
      } else {
        const u32x4& w = raw.w[j][kk >> 1];
        const half4 lo = int8_dequant4(w[(kk & 1) * 2], s8[j]);
        const half4 hi = int8_dequant4(w[(kk & 1) * 2 + 1], s8[j]);
        return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    };

    // One stage on ring buffer BUF, software-pipelined over its four k-steps.
    // On entry ca / fbc hold the A and B operands of k-step 0 and `raw` the
    // lane's codes of this stage. While the MFMAs of k-step kk run, the A
    // fragments of kk+1 are read and its B operands dequantised. Before the
    // last k-step the wave waits for the copies of stage st+1 and joins the
    // workgroup barrier: every wave is then done with buffer BUF, which takes
    // the copies of stage st+NBUF (three buffers: part A now, parts B and C
    // during k-steps 0 and 1 of stage st+1; two buffers: all of them now), and
    // the operands of the next stage's first k-step are read and dequantised
    // under the last k-step's MFMAs.
    // Every stage issues its copies and waits the same way, past the last
    // stage too (the copy index is clamped to the last stage), so all paths
    // through the loop leave the same copies in flight.
    auto stage = [&](auto buf_c, auto nb_c, int st, Frag (&ca)[RB], half8 (&fbc)[CB], R& raw) {
      constexpr int BUF = decltype(buf_c)::value;
      constexpr int NB = decltype(nb_c)::value;
      constexpr int NXT = (BUF + 1) % NBUF;
      const char* rb = Ring<BUF, RING>::p();
      Frag na[RB];
      half8 fbn[CB];
      auto mfmas = [&](Frag (&fa)[RB], half8 (&fb)[CB]) {
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = Mma<T>::mma(fa[i], fb[j], acc[i][j]);
      };
      auto copy_ops = [&](Frag (&dst)[RB], const Frag (&src)[RB], half8 (&fd)[CB], const half8 (&fs)[CB]) {
#pragma unroll
        for (int i = 0; i < RB; ++i) dst[i] = src[i];
#pragma unroll
        for (int j = 0; j < CB; ++j) fd[j] = fs[j];
      };
      constexpr int PREV = (BUF + NBUF - 1) % NBUF;   // three buffers: stage st+2's (freed by the last barrier)
      const int st2 = min(st + 2, nst - 1);
#pragma unroll
      for (int kk = 0; kk < BK / 16 - 1; ++kk) {
        if constexpr (NBUF == 3) {
          if (kk == 0) issue_ops(std::integral_constant<int, PREV>{}, IA1{}, IB1{}, st2);
          if (kk == 1) issue_ops(std::integral_constant<int, PREV>{}, IB1{}, IC1{}, st2);
        }
        if constexpr (NB > 0) {
          read_a3(rb, kk + 1, na);
#pragma unroll
          for (int j = 0; j < NB; ++j) fbn[j] = b_frag(raw, rb, j, kk + 1);
          mfmas(ca, fbc);
          if constexpr (H16C) {
            // RB * NB MFMAs and RB + NB fragment reads
#pragma unroll
            for (int g = 0; g < RB * NB; ++g) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
              if (g < RB + NB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            }
          } else {
            // 16 MFMAs, up to 4 copies, 8 fragment reads, ~40 dequantisation
#pragma unroll
            for (int g = 0; g < RB; ++g) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
              if (NBUF == 3 && g < 4) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // copy
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
              __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // VALU
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NB > 0) copy_ops(ca, na, fbc, fbn);
      }
      // copies of stage st+1 landed once only stage st+2's remain (three
      // buffers) or none (two); after the barrier no wave reads buffer BUF
      if constexpr (NBUF == 3) {
        dma_sync<DMA_PER_STAGE>();
        issue_ops(std::integral_constant<int, BUF>{}, IA0{}, IA1{}, min(st + 3, nst - 1));
      } else {
        dma_sync<0>();
        issue_ops(std::integral_constant<int, BUF>{}, IA0{}, IC1{}, min(st + 2, nst - 1));
      }
      if constexpr (NB > 0) {
        // operands of the next stage's k-step 0 (its buffer has landed; past
        // the last stage it holds a clamped copy and the values go unused)
        read_raw(nb_c, Ring<NXT, RING>::p(), raw);
        read_a3(Ring<NXT, RING>::p(), 0, na);
#pragma unroll
        for (int j = 0; j < NB; ++j) fbn[j] = b_frag(raw, Ring<NXT, RING>::p(), j, 0);
        mfmas(ca, fbc);
        // copies first (they follow no read of this wave), then the code and
        // fragment reads, then the dequantisation
        constexpr int CPG = NBUF == 3 ? 1 : (DMA_PER_STAGE + 3) / 4;   // copies per MFMA
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
          __builtin_amdgcn_sched_group_barrier(0x010, CPG, 0);     // copies
        }
        if constexpr (H16C) {
          // the A and B fragment reads of the next stage's k-step 0
#pragma unroll
          for (int g = 0; g < NB * RB - 4; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        } else {
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * NB, 0);   // code reads
#pragma unroll
          for (int g = 0; g < RB / 2; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // A fragment reads
          }
#pragma unroll
          for (int g = 0; g < NB * RB - 4 - RB / 2; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        copy_ops(ca, na, fbc, fbn);
      }
    };

    // the workgroup's queries ride along with the first copies
    float qpre = 0.f;
    if constexpr (EPI == EPI_ATTN)
      if (tid < HGT * DH) qpre = a.q[(size_t)r * D + hg * HGT * DH + tid];
    // stages 0 and 1 (and, with three buffers, part A of stage 2) are issued
    // back to back; the loop starts once stage 0 has landed, with the rest in
    // flight exactly as at the end of every stage (the counter drains in
    // issue order, so the queries, issued first, have arrived too)
    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, min(1, nst - 1));
    if constexpr (NBUF == 3)
      issue_ops(std::integral_constant<int, 2>{}, IA0{}, IA1{}, min(2, nst - 1));   // parts B, C: stage 0
    if constexpr (EPI == EPI_ATTN) {
      // (uniform over the workgroup: every wave leaves, after its copies have landed)
      if (sub == 0 && a.status[lane] == TL_LANE_ABORTED) {
        dma_sync<0>();
        return;
      }
    }
    if constexpr (NBUF == 3) {
      dma_sync<DMA_PER_STAGE + PA>();
    } else {
      dma_sync<DMA_PER_STAGE>();
    }
    if constexpr (EPI == EPI_ATTN)
      if (tid < HGT * DH) q_lds[tid] = qpre;   // read after the loop's barriers
    auto loop = [&](auto nb_c) {
      constexpr int NB = decltype(nb_c)::value;
      Frag ca[RB];
      half8 fbc[CB];
      R raw;
      if constexpr (NB > 0) {
        read_raw(nb_c, Ring<0, RING>::p(), raw);
        read_a3(Ring<0, RING>::p(), 0, ca);
#pragma unroll
        for (int j = 0; j < NB; ++j) fbc[j] = b_frag(raw, Ring<0, RING>::p(), j, 0);
      }
      int st = 0;
      if constexpr (NBUF == 3) {
        for (; st + 3 <= nst; st += 3) {
          stage(std::integral_constant<int, 0>{}, nb_c, st, ca, fbc, raw);
          stage(std::integral_constant<int, 1>{}, nb_c, st + 1, ca, fbc, raw);
          stage(std::integral_constant<int, 2>{}, nb_c, st + 2, ca, fbc, raw);
        }
        if (st < nst) stage(std::integral_constant<int, 0>{}, nb_c, st, ca, fbc, raw);
        if (st + 1 < nst) stage(std::integral_constant<int, 1>{}, nb_c, st + 1, ca, fbc, raw);
      } else {
        for (; st + 2 <= nst; st += 2) {
          stage(std::integral_constant<int, 0>{}, nb_c, st, ca, fbc, raw);
          stage(std::integral_constant<int, 1>{}, nb_c, st + 1, ca, fbc, raw);
        }
        if (st < nst) stage(std::integral_constant<int, 0>{}, nb_c, st, ca, fbc, raw);
      }
      dma_sync<0>();   // no copy may still be writing LDS past this point
    };
    // A tile with at most one live 32-position block (the tile just past a
    // multiple of BJ, or a context of a few positions) would leave its MFMAs
    // to one wave: instead every wave takes RB / NW of the block's row blocks
    // over the same stages, and the waves then hand their rows to wave 0,
    // which runs the epilogue as if it had computed the block alone.
    // With more waves than row blocks the waves past the row blocks only copy.
    // (tiles whose waves each hold all the tile's rows; the others run a
    // partial last tile through the ordinary loop)
    if constexpr (B_REG && WF == BF) {
      constexpr int RBT = RB >= NW ? RB / NW : 1;
      static_assert((RB >= NW ? RBT * NW == RB : NW % RB == 0) && RB * 16 * 64 * 4 <= RING, "tail split");
      const bool tail = Tn - j0 <= 32;
      if (tail) {
        const bool trows = wave_u * RBT < RB;
        const int trow = min(wave_u * RBT, RB - RBT) * 32 + (l & 31);
        const uint32_t tmask = j0 + (l & 31) < Tn ? 1u : 0u;
        auto read_at = [&](const char* rb, int kk, Frag (&fa)[RBT]) {
          const char* base = rb + trow * (BK * ES) + (((kk * 2 + hb) ^ aswz) * 16);
#pragma unroll
          for (int i = 0; i < RBT; ++i) fa[i] = *(const Frag*)(base + i * 32 * (BK * ES));
        };
        // block 0 of the tile: position l % 32, the same for every wave
        auto read_rawt = [&](const char* rb, R& raw) {
          const int pos = l & 31;
          const char* hs = rb + W_BYTES + ((pos >> 4) * (32 * NQ) + hb * NQ * 16 + (pos & 15)) * 16;
          if constexpr (MODE == TL_CACHE_H_INT4) {
            raw.w[0] = *(const u32x4*)hs;
            raw.s[0] = *(const uint32_t*)(rb + W_BYTES + H_BYTES + pos * 4);
          } else {
            raw.w[0][0] = *(const u32x4*)hs;
            raw.w[0][1] = *(const u32x4*)(hs + 16 * 16);
          }
        };
        half_t s8t = (half_t)0.f;
        if constexpr (MODE == TL_CACHE_H_INT8)
          s8t = tmask ? h_from_bits(*cv.int8_scale(a.layer, lane, j0 + (l & 31))) : (half_t)0.f;
        auto b_fragt = [&](const R& raw, int kk) -> half8 {
          if constexpr (MODE == TL_CACHE_H_INT4) {
            const uint32_t sv = tmask ? raw.s[0] : 0u;
            const half_t sc = h_from_bits((uint16_t)(kk < 2 ? (sv & 0xFFFFu) : (sv >> 16)));
            return int4_dequant8(raw.w[0][kk], sc);
          } else {
            const u32x4& w = raw.w[0][kk >> 1];
            const half4 lo = int8_dequant4(w[(kk & 1) * 2], s8t);
            const half4 hi = int8_dequant4(w[(kk & 1) * 2 + 1], s8t);
            return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        };
        // the copies go out and are waited for exactly as in `stage`
        auto stage_t = [&](auto buf_c, int st, Frag (&ca)[RBT], half8& fbc, R& raw) {
          constexpr int BUF = decltype(buf_c)::value;
          constexpr int NXT = (BUF + 1) % NBUF, PREV = (BUF + NBUF - 1) % NBUF;
          const char* rb = Ring<BUF, RING>::p();
          const int st2 = min(st + 2, nst - 1);
          Frag na[RBT];
          half8 fbn;
#pragma unroll
          for (int kk = 0; kk < BK / 16 - 1; ++kk) {
            if constexpr (NBUF == 3) {
              if (kk == 0) issue_ops(std::integral_constant<int, PREV>{}, IA1{}, IB1{}, st2);
              if (kk == 1) issue_ops(std::integral_constant<int, PREV>{}, IB1{}, IC1{}, st2);
            }
            read_at(rb, kk + 1, na);
            fbn = b_fragt(raw, kk + 1);
            if (trows)
#pragma unroll
              for (int i = 0; i < RBT; ++i) acc[i][0] = Mma<T>::mma(ca[i], fbc, acc[i][0]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < RBT; ++i) ca[i] = na[i];
            fbc = fbn;
          }
          if constexpr (NBUF == 3) {
            dma_sync<DMA_PER_STAGE>();
            issue_ops(std::integral_constant<int, BUF>{}, IA0{}, IA1{}, min(st + 3, nst - 1));
          } else {
            dma_sync<0>();
            issue_ops(std::integral_constant<int, BUF>{}, IA0{}, IC1{}, min(st + 2, nst - 1));
          }
          read_rawt(Ring<NXT, RING>::p(), raw);
          read_at(Ring<NXT, RING>::p(), 0, na);
          fbn = b_fragt(raw, 0);
          if (trows)
#pragma unroll
            for (int i = 0; i < RBT; ++i) acc[i][0] = Mma<T>::mma(ca[i], fbc, acc[i][0]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < RBT; ++i) ca[i] = na[i];
          fbc = fbn;
        };
        {
          Frag ca[RBT];
          half8 fbc;
          R raw;
          read_rawt(Ring<0, RING>::p(), raw);
          read_at(Ring<0, RING>::p(), 0, ca);
          fbc = b_fragt(raw, 0);
          int st = 0;
          if constexpr (NBUF == 3) {
            for (; st + 3 <= nst; st += 3) {
              stage_t(std::integral_constant<int, 0>{}, st, ca, fbc, raw);
              stage_t(std::integral_constant<int, 1>{}, st + 1, ca, fbc, raw);
              stage_t(std::integral_constant<int, 2>{}, st + 2, ca, fbc, raw);
            }
            if (st < nst) stage_t(std::integral_constant<int, 0>{}, st, ca, fbc, raw);
            if (st + 1 < nst) stage_t(std::integral_constant<int, 1>{}, st + 1, ca, fbc, raw);
          } else {
            for (; st + 2 <= nst; st += 2) {
              stage_t(std::integral_constant<int, 0>{}, st, ca, fbc, raw);
              stage_t(std::integral_constant<int, 1>{}, st + 1, ca, fbc, raw);
            }
            if (st < nst) stage_t(std::integral_constant<int, 0>{}, st, ca, fbc, raw);
          }
          dma_sync<0>();
        }
        // row blocks w*RBT .. w*RBT+RBT-1 of wave w -> wave 0, through ring
        // buffer 0 (no copy is in flight any more): [row block][element][lane]
        float* xch = (float*)Ring<0, RING>::p();
        if (wave_u > 0 && trows) {
#pragma unroll
          for (int i = 0; i < RBT; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) xch[((wave_u * RBT + i) * 16 + e) * 64 + l] = acc[i][0][e];
        }
        lds_sync();
        if (wave_u == 0) {
#pragma unroll
          for (int i = RBT; i < RB; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][0][e] = xch[(i * 16 + e) * 64 + l];
        }
        __syncthreads();   // the exchange is read before the epilogue reuses LDS
      } else {
        dispatch_nb<CB>(ncb, loop);
      }
    } else {
      dispatch_nb<CB>(ncb, loop);
    }
  } else {
    // ---- fp16 / fp32 h staged through LDS ----------------------------------
    // positions past T read the entry of position T-1 (always in bounds) and are
    // zeroed by a select when stored, so the loop has no data-dependent branches
    int bpos[B_NCH];
    uint32_t hoff[B_NCH];
    uint32_t bokmask = 0;
#pragma unroll
    for (int i = 0; i < B_NCH; ++i) {
      const int c = tid + NT * i;
      bpos[i] = c / B_CPP;
      if (j0 + bpos[i] < Tn) bokmask |= 1u << i;
      const int pos = min(j0 + bpos[i], Tn - 1);
      hoff[i] = (uint32_t)pos * HRB + (c % B_CPP) * 16;
    }
    u32x4 rh[B_NCH];
    auto load_h = [&](int st) {
      const char* hk = hbase + (size_t)st * kb_stride;
#pragma unroll
      for (int i = 0; i < B_NCH; ++i) rh[i] = *(const u32x4*)(hk + hoff[i]);
    };
    auto store_h = [&](int buf) {
      char* Bs = smem + buf * TILE_BYTES + BF * ROWB;
#pragma unroll
      for (int i = 0; i < B_NCH; ++i) {
        const int c = tid + NT * i;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        *(u32x4*)(Bs + bpos[i] * ROWB + (c % B_CPP) * 16) = ((bokmask >> i) & 1) ? rh[i] : zero;
      }
    };
    auto read_b = [&](auto nb_c, int buf, int kk, Frag (&fb)[CB]) {
      constexpr int NB = decltype(nb_c)::value;
      const char* Bs = smem + buf * TILE_BYTES + BF * ROWB;
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fb[j] = *(const Frag*)(Bs + (wj * WJ + j * 32 + (l & 31)) * ROWB + kk * 16 * ES + koff);
    };
    auto stage = [&](auto buf_c, auto nb_c, int st, Frag (&f0a)[RB], Frag (&f0b)[CB]) {
      constexpr int BUF = decltype(buf_c)::value;
      constexpr int NB = decltype(nb_c)::value;
      Frag f1a[RB], f1b[CB];
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        Frag (&ca)[RB] = (kk & 1) ? f1a : f0a;
        Frag (&cb)[CB] = (kk & 1) ? f1b : f0b;
        Frag (&na)[RB] = (kk & 1) ? f0a : f1a;
        Frag (&nb)[CB] = (kk & 1) ? f0b : f1b;
        if (kk + 1 < BK / 16 && NB > 0) {
          read_a(BUF, kk + 1, na);
          read_b(nb_c, BUF, kk + 1, nb);
        }
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = Mma<T>::mma(ca[i], cb[j], acc[i][j]);
        if (kk == BK / 16 - 2) {
          store_h(BUF ^ 1);
          load_h(min(st + 2, nst - 1));
        }
        if (kk == BK / 16 - 1) {
          store_w(BUF ^ 1);
          load_w(min(st + 2, nst - 1));
        }
      }
      __syncthreads();
      if (NB > 0) {
        read_a(BUF ^ 1, 0, f0a);
        read_b(nb_c, BUF ^ 1, 0, f0b);
      }
    };
    load_w(0);
    load_h(0);
    store_w(0);
    store_h(0);
    load_w(min(1, nst - 1));
    load_h(min(1, nst - 1));
    __syncthreads();
    Frag fa[RB], fb[CB];
    auto loop = [&](auto nb_c) {
      if (decltype(nb_c)::value > 0) {
        read_a(0, 0, fa);
        read_b(nb_c, 0, 0, fb);
      }
      for (int st = 0; st < nst; st += 2) {
        stage(std::integral_constant<int, 0>{}, nb_c, st, fa, fb);
        stage(std::integral_constant<int, 1>{}, nb_c, st + 1, fa, fb);
      }
    };
    dispatch_nb<CB>(ncb, loop);
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
      const int pos = j0 + pos_local(j);
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

  auto scores = [&](int rb0, const float* qh, float (&s)[CB]) {
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
      const int pos = j0 + pos_local(j);
      if (pos >= Tn) s[j] = -__builtin_inff();
    }
  };
  auto softmax = [&](float (&s)[CB], float& m, float& lsum) {
    m = s[0];
#pragma unroll
    for (int j = 1; j < CB; ++j) m = fmaxf(m, s[j]);
    m = allreduce32<true>(m);
    lsum = 0.f;
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      s[j] = s[j] == -__builtin_inff() ? 0.f : exp2f((s[j] - m) * kLog2e);
      lsum += s[j];
    }
    lsum = allreduce32<false>(lsum);
  };
  // o over V blocks rb0 .. rb0+KB-1 with weights p, reduced over the 32 lanes
  // of each half and written, with (m, lsum), to dst[0 .. DH+2).
  auto values = [&](int rb0, float* dst, const float (&p)[CB], float m, float lsum) {
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
    reduce_scatter32<NV>(v, l);
    if (l == 0) { dst[0] = m; dst[1] = lsum; }
    constexpr int FL = NV >= 32 ? NV / 32 : 1;
    if (NV >= 32 || (l & 16) == 0) {
#pragma unroll
      for (int k = 0; k < FL; ++k) {
        const int idx = rs_index<NV>(l, k);
        const int kb = idx >> 4, i = idx & 15;
        dst[2 + kb * 32 + 8 * (i >> 2) + 4 * half_id + (i & 3)] = v[k];
      }
    }
  };

  auto part_of = [&](int head, int sp) -> float* {
    return a.part + (((size_t)r * a.H + head) * a.S + sp) * (DH + 2);
  };
  constexpr int HG = BF / (2 * DH);   // heads of the workgroup
  // Partial of head g (0 .. HG-1) of the tile: M, L, O[dim] to the partial
  // buffer, with device-coherent stores when the launch merges its own tiles
  // (the merging workgroup may sit on another XCD).
  auto store_partial = [&](int g, int dim, float M, float L, float O) {
    float* dst = part_of(hg * HG + g, ptile);
    if (a.tilecnt) {
      if (dim == 0) {
        __hip_atomic_store(dst, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(dst + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __hip_atomic_store(dst + 2 + dim, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (dim == 0) { dst[0] = M; dst[1] = L; }
      dst[2 + dim] = O;
    }
  };
  // The workgroup that completes a (row, head group) merges the row's tiles
  // for those heads, exactly as the split merge would. The partials went out
  // with device-coherent stores, which have completed (vmcnt 0) before the
  // workgroup counts itself; the last one reads them with device-coherent
  // loads. No cache is written back or invalidated, so the W rows and h codes
  // other workgroups share in L2 stay there. It also zeroes the count for the
  // next launch. scratch: NT + NT / DH + NT / 64 floats of LDS.
  auto count_and_merge = [&](float* scratch) {
    __shared__ int last_tile;
    const int n_t = (Tn + BJ - 1) / BJ;      // the row's tiles (partials)
    const int n_w = (n_t + TPW - 1) / TPW;   // the workgroups that count
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      int* cnt = a.tilecnt + r * a.n_hg + hg;
      const int done = atomicAdd(cnt, 1) + 1;
      last_tile = done == n_w;
      if (done == n_w) atomicExch(cnt, 0);
    }
    __syncthreads();
    if (!last_tile) return;
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      const int head = hg * HG + g;
      merge_splits<T, DH, true, NT>(part_of(head, 0), n_t, (T*)a.o + (size_t)r * D + head * DH, scratch,
                                    scratch + NT, scratch + NT + NT / DH);
    }
  };
  if constexpr (COPY) {
    // Every wave holds whole heads (HPW of them, the workgroup's rows split
    // over BF / WF feature waves) for its positions: each writes its (max,
    // sum, o) per head to LDS (a wave with no position < T writes the neutral
    // partial), and one partial per (row, head, tile) is formed by combining,
    // in order, the WJN waves that hold the head (w = wf * WJN + 0, 1, ...).
    static_assert(!kCross, "copied-operand tiles hold whole heads");
    static_assert(HPW * (BF / WF) == HG && WJN * (BF / WF) == NWV, "waves cover the workgroup's heads");
    float* comb = (float*)comb_lds;   // [NWV][HPW][DH + 2]
#pragma unroll
    for (int g = 0; g < HPW; ++g) {
      float* dst = comb + (wave * HPW + g) * (DH + 2);
      if (wave_live) {
        float s[CB], m, lsum;
        scores(g * 2 * KB, q_lds + (wf * HPW + g) * DH, s);
        softmax(s, m, lsum);
        values(g * 2 * KB + KB, dst, s, m, lsum);
      } else {
        for (int e = l; e < DH + 2; e += 64) dst[e] = e == 0 ? -__builtin_inff() : 0.f;
      }
    }
    lds_sync();
    if (tid < HG * DH) {
      const int gg = tid / DH, dim = tid % DH, g = gg % HPW, w0 = (gg / HPW) * WJN;
      float M = comb[(w0 * HPW + g) * (DH + 2)];
#pragma unroll
      for (int w = 1; w < WJN; ++w) M = fmaxf(M, comb[((w0 + w) * HPW + g) * (DH + 2)]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < WJN; ++w) {
        const float* c = comb + ((w0 + w) * HPW + g) * (DH + 2);
        const float e = c[0] == -__builtin_inff() ? 0.f : exp2f((c[0] - M) * kLog2e);
        L = fmaf(c[1], e, L);
        O = fmaf(c[2 + dim], e, O);
      }
      store_partial(gg, dim, M, L, O);
    }
    if (a.tilecnt && last_sub) {
      static_assert(NWV * HPW_T * (DH + 2) >= NT + NT / DH + NT / 64, "merge scratch within comb_lds");
      count_and_merge(comb);
    }
  } else if (a.tilecnt) {
    // LDS-staged h with the tile merge in the launch: the position waves'
    // partials of each head go to LDS (the staging buffers are free once the
    // last stage has been multiplied), are combined in position order into
    // one partial per (row, head, tile), and the last tile of a (row, head
    // group) merges the row's tiles.
    float* ex = (float*)smem;                          // [WJN][WJ] p, then [WJN][2] (m, l)
    float* comb = ex + WJN * WJ + 2 * WJN;             // [HG][WJN][DH + 2]
    float* scratch = comb + HG * WJN * (DH + 2);       // merge scratch
    static_assert((WJN * WJ + 2 * WJN + HG * WJN * (DH + 2) + NT + NT / DH + NT / 64) * 4 <= 2 * TILE_BYTES,
                  "combine and merge scratch within the staging buffers");
    __syncthreads();
    if constexpr (!kCross) {
#pragma unroll
      for (int g = 0; g < HPW; ++g) {
        float* dst = comb + ((wf * HPW + g) * WJN + wj) * (DH + 2);
        if (wave_live) {
          const int head = hg * HG + wf * HPW + g;
          float s[CB], m, lsum;
          scores(g * 2 * KB, a.q + (size_t)r * D + head * DH, s);
          softmax(s, m, lsum);
          values(g * 2 * KB + KB, dst, s, m, lsum);
        } else {
          for (int e = l; e < DH + 2; e += 64) dst[e] = e == 0 ? -__builtin_inff() : 0.f;
        }
      }
    } else {
      // K rows live in wave wf = 0, V rows in wf = 1 (same positions): the
      // weights p pass through LDS
      if (wf == 0 && wave_live) {
        float s[CB], m, lsum;
        scores(0, a.q + (size_t)r * D + hg * DH, s);
        softmax(s, m, lsum);
        if (l < 32)
#pragma unroll
          for (int j = 0; j < CB; ++j) ex[wj * WJ + j * 32 + l] = s[j];
        if (l == 0) { ex[WJN * WJ + 2 * wj] = m; ex[WJN * WJ + 2 * wj + 1] = lsum; }
      }
      __syncthreads();
      if (wf == 1) {
        float* dst = comb + wj * (DH + 2);
        if (wave_live) {
          float p[CB];
#pragma unroll
          for (int j = 0; j < CB; ++j) p[j] = ex[wj * WJ + j * 32 + (l & 31)];
          values(0, dst, p, ex[WJN * WJ + 2 * wj], ex[WJN * WJ + 2 * wj + 1]);
        } else {
          for (int e = l; e < DH + 2; e += 64) dst[e] = e == 0 ? -__builtin_inff() : 0.f;
        }
      }
    }
    __syncthreads();
    if (tid < HG * DH) {
      const int g = tid / DH, dim = tid % DH;
      const float* cg = comb + g * WJN * (DH + 2);
      float M = cg[0];
#pragma unroll
      for (int w = 1; w < WJN; ++w) M = fmaxf(M, cg[w * (DH + 2)]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < WJN; ++w) {
        const float* c = cg + w * (DH + 2);
        const float e = c[0] == -__builtin_inff() ? 0.f : exp2f((c[0] - M) * kLog2e);
        L = fmaf(c[1], e, L);
        O = fmaf(c[2 + dim], e, O);
      }
      store_partial(g, dim, M, L, O);
    }
    count_and_merge(scratch);
  } else if constexpr (!kCross) {
    if (!wave_live) return;
#pragma unroll
    for (int g = 0; g < HPW; ++g) {
      const int head = hg * HG + wf * HPW + g;
      float s[CB], m, lsum;
      scores(g * 2 * KB, a.q + (size_t)r * D + head * DH, s);
      softmax(s, m, lsum);
      values(g * 2 * KB + KB, part_of(head, split), s, m, lsum);
    }
  } else {
    // K rows live in wave wf = 0, V rows in wf = 1 (same positions): pass the
    // weights p through LDS.
    char* ex_base;
    if constexpr (COPY) ex_base = Ring<0, RING>::p();
    else ex_base = smem;
    float* ex = (float*)ex_base;            // [WJN][WJ] p, then [WJN][2] (m, l)
    const int head = hg;
    __syncthreads();
    if (wf == 0 && wave_live) {
      float s[CB], m, lsum;
      scores(0, a.q + (size_t)r * D + head * DH, s);
      softmax(s, m, lsum);
      if (l < 32)
#pragma unroll
        for (int j = 0; j < CB; ++j) ex[wj * WJ + j * 32 + l] = s[j];
      if (l == 0) { ex[WJN * WJ + 2 * wj] = m; ex[WJN * WJ + 2 * wj + 1] = lsum; }
    }
    __syncthreads();
    if (wf == 1 && wave_live) {
      float p[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) p[j] = ex[wj * WJ + j * 32 + (l & 31)];
      values(0, part_of(head, split), p, ex[WJN * WJ + 2 * wj], ex[WJN * WJ + 2 * wj + 1]);
    }
  }
  }   // position tiles of the workgroup
}

template <typename T, int MODE, int DH, int VAR = 0>
hipError_t launch_mode(const KArgs& k, int grid, hipStream_t s, int epi, const LaunchEvents& ev) {
  constexpr int NT = Cfg<T, MODE, DH, VAR>::NT;
  if (epi == EPI_ATTN) return launch_timed(recon_kernel<T, MODE, DH, EPI_ATTN, VAR>, grid, NT, s, ev, k);
  recon_kernel<T, MODE, DH, EPI_KVSTORE, VAR><<<grid, NT, 0, s>>>(k);
  return hipGetLastError();
}

// var 1, 2: the one-head fp16-h configurations (decode attention only)
hipError_t dispatch(const ModelView& m, const KArgs& k, int grid, hipStream_t s, int epi, int var = 0,
                    const LaunchEvents& ev = {}) {
  if (var == 1 || var == 2) {
    if (!(m.dtype == TL_DTYPE_F16 && k.cache.mode == TL_CACHE_H_F16 && m.dh == 64 && epi == EPI_ATTN))
      return hipErrorInvalidValue;
    return var == 1 ? launch_mode<half_t, TL_CACHE_H_F16, 64, 1>(k, grid, s, epi, ev)
                    : launch_mode<half_t, TL_CACHE_H_F16, 64, 2>(k, grid, s, epi, ev);
  }
  if (m.dtype == TL_DTYPE_F32) {
    if (m.dh == 32 && k.cache.mode == TL_CACHE_H_F32)
      return launch_mode<float, TL_CACHE_H_F32, 32>(k, grid, s, epi, ev);
    return hipErrorInvalidValue;
  }
  const int mode = k.cache.mode;
#define TL_RECON_CASE(MODE_, DH_) \
  if (mode == MODE_ && m.dh == DH_) return launch_mode<half_t, MODE_, DH_>(k, grid, s, epi, ev);
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

bool combined_splits(const ModelView& m, int mode) {
  return m.dtype == TL_DTYPE_F16 &&
         (mode == TL_CACHE_H_INT4 || mode == TL_CACHE_H_INT8 || mode == TL_CACHE_H_F16);
}


// features (K and V rows) per workgroup and positions per tile of the
// configuration dispatch() picks
static int recon_bf(const ModelView& m, int mode, int var = 0) {
  if (var == 1) return Cfg<half_t, TL_CACHE_H_F16, 64, 1>::BF;
  if (var == 2) return Cfg<half_t, TL_CACHE_H_F16, 64, 2>::BF;
  if (m.dtype == TL_DTYPE_F32) return Cfg<float, TL_CACHE_H_F32, 32>::BF;
  if (mode == TL_CACHE_H_INT4 && m.dh == 64) return Cfg<half_t, TL_CACHE_H_INT4, 64>::BF;
  if (mode == TL_CACHE_H_INT8 && m.dh == 64) return Cfg<half_t, TL_CACHE_H_INT8, 64>::BF;
  static_assert(Cfg<half_t, TL_CACHE_H_INT4, 128>::BF == 256 &&
                    Cfg<half_t, TL_CACHE_H_INT8, 128>::BF == 256 && Cfg<half_t, TL_CACHE_H_F16, 64>::BF == 256 &&
                    Cfg<half_t, TL_CACHE_H_F16, 128>::BF == 256,
                "other fp16 configurations");
  return 256;
}
static int recon_bj(const ModelView& m, int mode, int var = 0) {
  if (var == 2) return Cfg<half_t, TL_CACHE_H_F16, 64, 2>::BJ;
  if (m.dtype == TL_DTYPE_F32) return Cfg<float, TL_CACHE_H_F32, 32>::BJ;
  if (mode == TL_CACHE_H_INT4 && m.dh == 64) return Cfg<half_t, TL_CACHE_H_INT4, 64>::BJ;
  return Cfg<half_t, TL_CACHE_H_F16, 64>::BJ;
}

int recon_split_len(const ModelView& m, int mode) {
  if (combined_splits(m, mode)) return recon_bj(m, mode);
  return m.dtype == TL_DTYPE_F32 ? Cfg<float, TL_CACHE_H_F32, 32>::WJ : Cfg<half_t, TL_CACHE_H_F16, 64>::WJ;
}

hipError_t launch_recon_attn(const ModelView& m, const ReconArgs& r, hipStream_t s) {
  if (r.tilecnt && (!r.o || !combined_splits(m, r.cache.mode))) return hipErrorInvalidValue;
  // fp16 h at 64-wide heads: the one-head configurations when the regular one
  // would leave CUs without a workgroup (128-position tiles when 256-position
  // ones still would)
  int var = 0;
  if (m.dtype == TL_DTYPE_F16 && r.cache.mode == TL_CACHE_H_F16 && m.dh == 64 && r.tilecnt) {
    auto wgs = [&](int v) {
      const int bj = recon_bj(m, r.cache.mode, v);
      return (long)((r.t_ub + bj - 1) / bj) * r.n_rows * (2 * m.D / recon_bf(m, r.cache.mode, v));
    };
    if (wgs(0) < kCUs) var = wgs(1) < kCUs ? 2 : 1;
  }
  const int BF = recon_bf(m, r.cache.mode, var);
  const int BJ = recon_bj(m, r.cache.mode, var);
  KArgs k{};
  k.cache = r.cache;
  k.layer = r.layer;
  k.w_qkv = r.w_qkv;
  k.D = m.D;
  k.H = m.H;
  k.n_hg = 2 * m.D / BF;
  // two position tiles per workgroup where the launch still has two
  // workgroups per CU with them: INT4 / INT8 h at 64-wide heads (measured on
  // one GPU: 64.9 -> 64.0 us per launch for INT4, 69.8 -> 67.5 us for INT8 at
  // 4 lanes and T = 4097..4121; the fp16-h copied ring, one workgroup per
  // CU, measured no gain and takes one)
  const int tiles = (r.t_ub + BJ - 1) / BJ;
  k.tpw = var == 0 && m.dh == 64 && combined_splits(m, r.cache.mode) &&
                  (r.cache.mode == TL_CACHE_H_INT4 || r.cache.mode == TL_CACHE_H_INT8) &&
                  (long)((tiles + 1) / 2) * r.n_rows * k.n_hg >= 2L * kCUs
              ? kMaxTilesPerWorkgroup
              : 1;
  k.n_ptiles = (tiles + k.tpw - 1) / k.tpw;
  k.n_rows = r.n_rows;
  k.row_lane = r.row_lane;
  k.row_pos = r.row_pos;
  k.status = r.status;
  k.q = r.q;
  k.part = r.part;
  k.S = r.S;
  k.o = r.o;
  k.tilecnt = r.tilecnt;
  // head groups per XCD: as many as keep their W rows within 2 MB of the
  // XCD's 4 MB L2 (the rest streams h), with the sets dividing the 8 XCDs
  const size_t hg_bytes = (size_t)BF * m.D * (m.dtype == TL_DTYPE_F32 ? 4 : 2);
  k.hpx = k.n_hg;
  for (int h = k.n_hg; h >= 1; h >>= 1) {
    if (k.n_hg % h || (k.n_hg / h) > 8 || 8 % (k.n_hg / h)) continue;
    k.hpx = h;
    if ((size_t)h * hg_bytes <= ((size_t)2 << 20)) break;
  }
  const int sets = k.n_hg / k.hpx, parts = 8 / sets;
  const long n_tiles = (long)k.n_ptiles * r.n_rows;
  const long grid = ((n_tiles + parts - 1) / parts) * parts * k.n_hg;
  if (grid <= 0 || grid > (1L << 30)) return hipErrorInvalidValue;
  return dispatch(m, k, (int)grid, s, EPI_ATTN, var, r.ev);
}

hipError_t launch_recon_store(const ModelView& m, const CacheView& c, int layer, int lane, int T,
                              const void* w_qkv, void* kvbuf, const int32_t* status,
                              hipStream_t s) {
  const int BF = recon_bf(m, c.mode);
  const int BJ = recon_bj(m, c.mode);
  KArgs k{};
  k.cache = c;
  k.layer = layer;
  k.w_qkv = w_qkv;
  k.D = m.D;
  k.H = m.H;
  k.n_hg = 2 * m.D / BF;
  k.n_ptiles = (T + BJ - 1) / BJ;
  k.n_rows = 1;
  k.lane = lane;
  k.T = T;
  k.status = status;
  k.kvbuf = kvbuf;
  return dispatch(m, k, k.n_hg * k.n_ptiles, s, EPI_KVSTORE);
}

}  // namespace tl
