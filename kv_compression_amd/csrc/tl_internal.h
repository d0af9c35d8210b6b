// Internal declarations shared by the host ABI (tl_api.hip) and the kernel
// translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tl.h"

namespace tl {

constexpr int kMaxBatch = 256;        // lanes per decode call
constexpr int kMaxChunk = 512;        // tokens per prefill call
constexpr int kKBlock = 64;           // d_model elements per tiled cache block
constexpr int kInt4Group = 32;        // INT4-h scale group along d_model
constexpr int kKvSplit = 32;          // positions per split in the stored-K/V attention
constexpr int kCUs = 256;             // compute units of the GPU (grid sizing heuristics)
constexpr int kSpecMax = 15;          // drafted tokens per speculative round
constexpr int kSpecRows = 16;         // verification rows of a round (kSpecMax + 1)

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Bytes of one tiled block row (kKBlock d_model elements of one position).
constexpr __host__ __device__ inline int block_row_bytes(int mode) {
  switch (mode) {
    case TL_CACHE_H_F32: return kKBlock * 4;
    case TL_CACHE_H_F16: return kKBlock * 2;
    case TL_CACHE_H_INT8: return kKBlock;
    case TL_CACHE_H_INT4: return kKBlock / 2;
    default: return 0;
  }
}

// Device view of a cache (H modes use the tiled layout, KV mode plain rows).
//
// H modes:  codes[layer][lane][kb][pos][block_row_bytes]   kb = k / 64
//           INT8 scales[layer][lane][pos]                  (fp16 bits)
//           INT4 scales[layer][lane][kb][pos][2]           (fp16 bits, groups 2kb, 2kb+1)
// KV mode:  kv[layer][lane][pos][2D]                       K | V, model dtype
// Delta mode (plain rows, read only by the delta kernels):
//           anchors[layer < n_pre][lane][pos][D]              fp16 h
//           codes[layer - n_pre][lane][pos][D]                int8 deltas
//           scales[layer - n_pre][lane][pos][H]               fp16 bits
struct CacheView {
  char* base;          // entries (codes, or K|V rows)
  uint16_t* scales;    // INT modes
  int mode, dtype;
  int D, n_lanes, max_seq, n_layers;
  int n_pre, H, dh;    // delta mode addressing and head groups

  __host__ __device__ half_t* delta_anchor(int layer, int lane, int pos) const {
    return (half_t*)base + (lane_block(layer, lane) * max_seq + pos) * D;
  }
  __host__ __device__ int8_t* delta_codes(int layer, int lane, int pos) const {
    return (int8_t*)(base + (size_t)n_pre * n_lanes * max_seq * D * 2) +
           (((size_t)(layer - n_pre) * n_lanes + lane) * max_seq + pos) * D;
  }
  __host__ __device__ uint16_t* delta_scales(int layer, int lane, int pos) const {
    return scales + (((size_t)(layer - n_pre) * n_lanes + lane) * max_seq + pos) * H;
  }

  __host__ __device__ size_t lane_block(int layer, int lane) const {
    return (size_t)layer * n_lanes + lane;
  }
  // H modes: byte address of position `pos`, block `kb`.
  __host__ __device__ char* code_row(int layer, int lane, int kb, int pos) const {
    const size_t rb = block_row_bytes(mode);
    return base + ((lane_block(layer, lane) * (D / kKBlock) + kb) * max_seq + pos) * rb;
  }
  __host__ __device__ uint16_t* int8_scale(int layer, int lane, int pos) const {
    return scales + lane_block(layer, lane) * max_seq + pos;
  }
  __host__ __device__ uint16_t* int4_scale(int layer, int lane, int kb, int pos) const {
    return scales + ((lane_block(layer, lane) * (D / kKBlock) + kb) * max_seq + pos) * 2;
  }
  // KV mode: element pointer of row `pos` (2D elements, model dtype).
  __host__ __device__ char* kv_row(int layer, int lane, int pos) const {
    const size_t es = dtype == TL_DTYPE_F32 ? 4 : 2;
    return base + (lane_block(layer, lane) * max_seq + pos) * (size_t)(2 * D) * es;
  }
};

// Per-lane device state and scratch inside the caller's workspace.
struct Workspace {
  int32_t* len;        // [n_lanes]
  int32_t* status;     // [n_lanes]
  float* norms;        // [n_lanes, l_max]
  float* xres;         // [n_lanes, D]
  int32_t* row_lane;   // [R]   decode: row -> lane id
  int32_t* row_slot;   // [R]   decode: row -> caller slot
  int32_t* row_pos;    // [R]   position the row writes / attends from
  int32_t* row_dead;   // [R]   1 once the row's lane has stopped (before or during the step)
  float* x;            // [R, D]   residual
  void* h;             // [R, D]   model dtype
  float* q;            // [R, D]   f32 queries (decode) / model dtype (prefill)
  void* o;             // [R, D]   model dtype
  void* u;             // [R, D]
  void* a;             // [R, F]
  void* z;             // [max(Bmax, kSpecRows), D]
  float* logits;       // [max(Bmax, kSpecRows), V]
  float* part;         // [Bmax, H, S, d + 2]
  void* kvbuf;         // [max_seq, 2D] f32 (prefill K/V rebuilt from h)
  float* hrec;         // [R, D]   delta mode: each row's FP32 reconstruction of the last layer written
  void* hmat;          // delta mode: one layer's h' of every lane, fp16 tiled (a one-layer H_F16 cache)
  float* qt;           // [Bmax, H, D] absorbed order: W_k,h^T q per row and head
  float* apart;        // [apair_cap, H, D + 2] absorbed order: per (row, split) partials
  int apair_cap;
  float* ppart;        // [kMaxChunk * H * 8 * (d + 2)] prefill key-split partials
  int ppart_floats;
  int32_t* tilecnt;    // [Bmax, 2 D / 128] decode attention: tiles done per (row, head group)
  int32_t* spec;       // speculative round: [0, kSpecRows) input token then drafts,
                       // [kSpecRows, 2 kSpecRows) verified tokens, [2 kSpecRows] count,
                       // [2 kSpecRows + 1] draft lane status
  int R, Bmax, S;      // rows, decode rows, splits per (row, head)
};

struct LayerW {
  const void *norm1, *w_qkv, *w_o, *norm2, *w_up, *w_down;
};

struct ModelView {
  int D, H, dh, F, n_pre, V, dtype;
  float eps;
  const void* embed;
  const void* final_norm;
  const void* lm_head;
};

// ---------------------------------------------------------------------------
// launchers (one per kernel family); all return hipGetLastError() of the launch
// ---------------------------------------------------------------------------
struct StepMap {
  int n;
  int32_t lane[kMaxBatch];
  int32_t slot[kMaxBatch];
};

// rows 0..n-1: row_lane/row_slot from the map, row_pos = len[lane], norms of the
// lane cleared to NaN, x[row] = embed[tokens_in[slot]] (skipped for aborted lanes).
hipError_t launch_step_setup(const ModelView& m, const Workspace& ws, const StepMap& map,
                             const int32_t* tokens_in, int l_max, hipStream_t s);
// prefill rows: row_lane = lane, row_pos = pos0 + i, x[i] = embed[tokens[i]].
hipError_t launch_prefill_setup(const ModelView& m, const Workspace& ws, int lane, int n,
                                const int32_t* tokens, int pos0, hipStream_t s);

enum HSource { HS_NORM = 0, HS_INPUT = 1, HS_SYNTH = 2 };
// For rows 0..n-1: h = dtype(RMSNorm(x) * g) (HS_NORM), or the given h rows
// (HS_INPUT), or synthetic Philox h (HS_SYNTH); h is written to h_out (model
// dtype, may be null for HS_INPUT) and, for H modes, encoded into the cache at
// (layer, row lane, row pos). Rows whose lane is aborted are skipped when
// `status` is non-null.
struct AppendArgs {
  int src;
  int n;
  int layer;
  const float* x;            // HS_NORM
  const void* gain;          // HS_NORM
  const void* h_in;          // HS_INPUT
  uint32_t seed;             // HS_SYNTH
  const int32_t* row_lane;   // or null: fixed_lane
  const int32_t* row_pos;    // or null: pos0 + row
  int fixed_lane, pos0;
  const int32_t* status;     // nullable
  void* h_out;               // nullable
  // delta mode: rows [n, D] holding each row's reconstruction of layer - 1,
  // updated to this layer's; null: rebuilt from the cache (layers in order)
  float* rec = nullptr;
  // HS_NORM, decode: the residual entering this layer is the one after loop
  // iteration check_iter (-1: none); its FP32 norm goes to norms[lane, iter]
  // and, if check and !(norm <= thr), the lane aborts before this layer
  int check_iter = -1;
  float* norms = nullptr;
  int32_t* status_w = nullptr;
  int l_max = 0, check = 0;
  float thr = 0.f;
};
hipError_t launch_norm_append(const ModelView& m, const CacheView& c, const AppendArgs& a,
                              hipStream_t s);

// The safety check of each decode row's last loop iteration (done by the
// step's end kernel): row r holds the residual after loop iteration iter[r];
// its FP32 norm goes to norms[lane, iter[r]] and, if check and
// !(norm <= thr), the lane aborts.
struct NormCheck {
  float* norms;
  int32_t* status;
  int l_max, check;
  float thr;
  int32_t iter[kMaxBatch];
};

// out[row] = dtype(RMSNorm(x[row]) * g) for rows 0..n-1 (skips aborted rows).
hipError_t launch_rmsnorm(const ModelView& m, int n, const float* x, const void* gain, void* out,
                          const int32_t* row_lane, const int32_t* status, hipStream_t s);



// Skinny / prefill GEMM: Y[row, f] = sum_k W[f, k] X[row, k] for rows < M,
// f < N, then the epilogue.
enum GemmEpi {
  EPI_STORE_F32 = 0,   // out_f32[row*ldo + f] = v * scale
  EPI_STORE_T = 1,     // out_t[row*ldo + f] = dtype(v * scale)
  EPI_ADD_F32 = 2,     // out_f32[row*ldo + f] += v
  EPI_GELU_T = 3,      // out_t[row*ldo + f] = dtype(gelu(v))
  EPI_LOGITS = 4,      // out_f32[slot(row)*ldo + f] = v   (slot via row_slot, or row)
  EPI_QKV = 5          // f < D: q (f32 or T by q_is_t) scaled; f >= D: K|V into the KV cache
};
struct GemmArgs {
  const void* W; int ldw;
  const void* X; int ldx;
  int M, N, K;
  int epi;
  void* out; int ldo;
  float scale;
  const int32_t* row_lane;   // nullable: skip aborted rows (with status)
  const int32_t* status;
  const int32_t* row_slot;   // EPI_LOGITS
  // EPI_QKV
  int q_is_t;
  CacheView cache;
  int layer;
  const int32_t* row_pos;
  int fixed_lane, pos0;
  int f_offset;              // EPI_QKV: global feature index = f + f_offset
  int fb;                    // output features per workgroup: 16, 8 or 4 (set by launch_gemm)
  int tiled;                 // a prefill chunk's product: LDS-tiled MFMA kernel where it applies
  // nullable: 1 when the row's lane has stopped (read instead of status by
  // the products of at most 16 rows; the attention input's safety check sets it)
  int32_t* row_dead;
  // nullable: X holds fp32 residual rows and the operand is fp16 / fp32
  // RMSNorm(X) * norm_gain, formed on the fly exactly as rmsnorm_kernel forms it
  const void* norm_gain;
  // with norm_gain, the pre-QKV row work of the attention input: the safety
  // check of loop iteration check_iter (>= 0) on the entering residual, then
  // (h modes) the append of h to the cache at (layer, row_lane, row_pos)
  int row_tasks;
  float* rec;                // delta mode: the rows' FP32 reconstructions (Workspace::hrec)
  int check_iter;
  float* norms;              // [lanes, l_max]
  int32_t* status_w;
  int l_max, check;
  float thr;
};
hipError_t launch_gemm(const ModelView& m, const GemmArgs& g, hipStream_t s);

// Timing of one kernel: events that take that launch's own start and end
// timestamps (hipExtLaunchKernel), so the time between them is the kernel's
// execution without the launch gaps around it. Null: not timed.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
template <typename F, typename... A>
hipError_t launch_timed(F kernel, dim3 grid, dim3 block, hipStream_t s, const LaunchEvents& ev, A... args) {
  if (ev.start) hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
  else kernel<<<grid, block, 0, s>>>(args...);
  return hipGetLastError();
}

// Decode attention over the store-h cache: rebuild K|V of every position with
// MFMA and fold them into per-split online-softmax partials.
struct ReconArgs {
  CacheView cache;
  int layer;
  const void* w_qkv;
  int n_rows;
  int t_ub;                  // upper bound of T over rows (grid sizing)
  const int32_t* row_lane;
  const int32_t* row_pos;
  const int32_t* status;
  const float* q;            // [rows, D] f32 (scaled)
  float* part;
  int S;                     // splits capacity per (row, head)
  // non-null (combined_splits configurations only): the last workgroup of
  // each (row, head group) merges the tiles into o, and no split merge follows
  void* o;
  int32_t* tilecnt;          // [rows, 2 D / 128] zero before the first launch
  LaunchEvents ev;           // timing of the attention kernel
};
hipError_t launch_recon_attn(const ModelView& m, const ReconArgs& a, hipStream_t s);
int recon_split_len(const ModelView& m, int mode);
// fp16 INT4 / INT8 h: one partial per (row, head, 256-position tile), and
// the attention kernel can merge them itself (ReconArgs::tilecnt)
bool combined_splits(const ModelView& m, int mode);

// Prefill: rebuild K|V (fp32 accumulators, kept in fp32) for positions 0..T-1
// into kvbuf [T, 2D].
hipError_t launch_recon_store(const ModelView& m, const CacheView& c, int layer, int lane, int T,
                              const void* w_qkv, void* kvbuf, const int32_t* status,
                              hipStream_t s);

// Decode attention over stored K|V rows (KV mode).
hipError_t launch_kv_attn(const ModelView& m, const ReconArgs& a, hipStream_t s);

// o[row] = dtype(merge of the row's split partials), split length `split_len`.
hipError_t launch_attn_merge(const ModelView& m, int n_rows, const int32_t* row_lane,
                             const int32_t* row_pos, const int32_t* status, const float* part,
                             int S, int split_len, void* o, hipStream_t s);

// Causal prefill attention: query i (position pos0+i) over K|V rows 0..pos0+i.
// q: [n, D] f32 (scaled); o: [n, D] model dtype; kv: rows of 2D elements
// (K | V), f32 when kv_f32 (rebuilt from h) else the model dtype (stored K/V).
// part (part_floats floats) takes the key-split partials; the split count
// adapts to the chunk (one split writes o directly). row_lane / row_pos: the
// chunk's rows, for the merge.
hipError_t launch_prefill_attn(const ModelView& m, int n, int pos0, const float* q,
                               const void* kv, int kv_f32, void* o, int lane,
                               const int32_t* status, float* part, int part_floats,
                               const int32_t* row_lane, const int32_t* row_pos, hipStream_t s);

// Per decode row: the safety check of the row's last loop iteration (norm of
// the final residual x[row] -> chk.norms; a failure stops the lane), then the
// argmax of logits (lowest index on ties) -> tokens_out[slot],
// lane_status[slot]; len[lane] += 1 unless stopped (stopped rows: token -1,
// user_logits NaN); xres[lane] = x[row].
hipError_t launch_finish(const ModelView& m, const Workspace& ws, int n, const float* logits,
                         int ld_logits, int logits_by_slot, int32_t* tokens_out,
                         int32_t* lane_status, float* user_logits, const NormCheck& chk,
                         hipStream_t s);
// Prefill: argmax of the last row's logits -> next_token; len[lane] = new_len.
hipError_t launch_prefill_finish(const ModelView& m, const Workspace& ws, int lane, int new_len,
                                 const float* logits, int32_t* next_token, hipStream_t s);

// Speculative round over the k + 1 verification rows (drafts d_1..d_k at
// spec[1..k]): every row's argmax -> spec[kSpecRows + j]; the leading drafts
// equal to the verified tokens are accepted; tokens_out[0..n) = the verified
// tokens through the first mismatch (n = accepted + 1, or 0 for an aborted
// lane), -1 after; spec[2 kSpecRows] = n; len[lane] = pos0 + n.
hipError_t launch_spec_accept(const ModelView& m, const Workspace& ws, int lane, int pos0, int k,
                              const float* logits, int32_t* tokens_out, hipStream_t s);

// Delta mode: h' of `layer` for the positions of each of the n_rows rows'
// lanes (0 .. row_pos[r], or 0 .. fixed_T - 1 when fixed_T > 0) into layer 0
// of the fp16 tiled view `mat`; t_ub bounds the positions for the grid.
hipError_t launch_delta_mat(const CacheView& c, const CacheView& mat, int layer,
                            const int32_t* row_lane, const int32_t* row_pos,
                            const int32_t* status, int n_rows, int t_ub, int fixed_T,
                            hipStream_t s);
// Delta mode: rec[i] = FP32 reconstruction of `layer` at position pos0 + i of
// `lane`, for i < n (the state a chunk resuming at layer + 1 continues from).
hipError_t launch_delta_rec(const CacheView& c, int layer, int lane, int pos0, int n, float* rec,
                            hipStream_t s);

// Absorbed evaluation order (decode). Covered: fp16 models with D 1024,
// 16 heads of 64, the h view in INT4, INT8 or fp16.
bool absorbed_supported(const ModelView& m, int view_mode);
// key splits and their length (a multiple of 16) for n_rows rows of up to
// t_ub positions, at most pair_cap (row, split) partials
int absorbed_splits(int n_rows, int t_ub, int pair_cap, int* split_len);
// qt[row][h][:] = W_k,h^T q[row][h d .. h d + d) in fp32
hipError_t launch_absorb_q(const ModelView& m, int n_rows, const float* q, const void* w_qkv,
                           float* qt, hipStream_t s);
// per (row, split): per head (max, sum, r[D]) into part [rows][S][H][D + 2]
hipError_t launch_absorbed_attn(const ModelView& m, const CacheView& c, int layer, int n_rows,
                                const int32_t* row_lane, const int32_t* row_pos,
                                const int32_t* status, const float* qt, float* part, int S,
                                int split_len, hipStream_t s, const LaunchEvents& ev = {});
// merge the splits into rbuf [rows][H][D] (r / l, fp32), then
// o[row][h d + j] = W_v,h r (model dtype)
hipError_t launch_absorbed_out(const ModelView& m, int n_rows, const int32_t* row_lane,
                               const int32_t* row_pos, const int32_t* status, const float* part,
                               int S, int split_len, const void* w_qkv, float* rbuf, void* o,
                               hipStream_t s);

// Fill lane state: len, status for lanes [l0, l0+n) and norms to NaN.
hipError_t launch_lane_reset(const Workspace& ws, int l0, int n, int l_max, int length,
                             hipStream_t s);
// p[0 .. n) = v (a kernel, so that it may sit in a captured graph)
hipError_t launch_fill_i32(int32_t* p, int n, int v, hipStream_t s);

// Cache read-back (test hook).
hipError_t launch_cache_read(const ModelView& m, const CacheView& c, int lane, int layer, int pos0,
                             int n, int8_t* codes, uint16_t* scales, void* h, hipStream_t s);

hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t s);

}  // namespace tl
