/*
 * tl.h — C ABI of the store-h looped-decoder library (libtl.so, gfx950).
 *
 * The library runs one decode step of a weight-shared looped transformer
 * (n_pre unique layers, then one loop block applied L times with the same
 * W_q, W_k, W_v, W_o, norms and MLP at every iteration; TinyLoop
 * architecture-exclusive features page, introduction) over a store-h KV
 * cache: the cache keeps the pre-QKV norm output h of every token and every
 * layer-iteration, and attention rebuilds K = W_k h and V = W_v h from it
 * with the layer's own weights (same page, "Store-h KV cache"; novel
 * contributions page, "Store-h KV Cache").
 *
 * Conventions shared by every call:
 *  - Device memory belongs to the caller. The library never allocates device
 *    memory; weights, the cache, the workspace and all inputs and outputs are
 *    caller buffers. Pointers documented as "device" must be device memory
 *    (hipMalloc / torch CUDA tensors); "host" pointers are ordinary memory.
 *  - Every call is asynchronous on the given HIP stream (hipStream_t passed as
 *    void*, NULL = the default stream) unless documented to synchronise.
 *  - Every call returns a tl_status. Arguments are validated before anything
 *    is enqueued; on an error nothing is enqueued, the cache is unchanged, and
 *    tl_last_error() returns a message (thread-local).
 *  - Calls on one cache must be serialised by the caller (one stream, or
 *    external synchronisation). Weights must outlive the model; the cache and
 *    workspace buffers must outlive the cache handle.
 *  - Matrices are row-major with y = W x (W is [out, in]).
 */
#ifndef TL_H
#define TL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TL_OK = 0,
  TL_E_ARG = 1,          /* an argument is out of range or inconsistent */
  TL_E_UNSUPPORTED = 2,  /* a shape / dtype / mode combination the kernels do not cover */
  TL_E_CAPACITY = 3,     /* appending would pass max_seq positions */
  TL_E_CACHE_GAP = 4,    /* a deeper L than the lane's upper layers were filled for */
  TL_E_HIP = 5           /* a HIP runtime error; the cache contents are undefined */
} tl_status;

/* What one cache entry (one token, one layer-iteration) holds.
 * KV:      K and V rows, model dtype (the stored-K/V baseline; measured-benchmarks
 *          page, section 3, "FP16 KV baseline"), 2*D elements.
 * H_F32:   h in fp32 (fp32 models only), 4*D bytes.
 * H_F16:   h in fp16 (fp16 models), 2*D bytes.
 * H_INT8:  h as int8 codes with one fp16 absmax scale per token, D + 2 bytes.
 * H_INT4:  h as 4-bit codes with one fp16 absmax scale per 32 consecutive
 *          d_model elements, D/2 + D/16 bytes.
 * (features page, "Store-h KV cache": FP16-h, INT8-h and INT4-h modes.)
 * H_DELTA8: the iteration-axis delta codec (features page, "4) Iteration-axis
 *          delta-KV"; fp16 models with n_pre >= 1). The n_pre unique layers
 *          keep fp16 h (2*D bytes); the last of them is the anchor h0. Loop
 *          layer n_pre + i keeps the INT8 delta of its h against the previous
 *          layer's reconstruction with one fp16 absmax scale per head
 *          (D + 2*n_heads bytes); its h' is fp16 of the FP32 prefix sum
 *          h0 + sum over loop layers 0..i of scale * code. The delta is taken
 *          against that same prefix sum (closed loop), so each layer's h'
 *          carries one quantisation error. Attention rebuilds a layer's h'
 *          for all positions into workspace before reconstructing K/V. */
typedef enum {
  TL_CACHE_KV = 0,
  TL_CACHE_H_F32 = 1,
  TL_CACHE_H_F16 = 2,
  TL_CACHE_H_INT8 = 3,
  TL_CACHE_H_INT4 = 4,
  TL_CACHE_H_DELTA8 = 5
} tl_cache_mode;

typedef enum { TL_LANE_OK = 0, TL_LANE_ABORTED = 1 } tl_lane_status;
typedef enum { TL_DTYPE_F32 = 0, TL_DTYPE_F16 = 1 } tl_dtype;

/* Model shape. Supported: d_model = n_heads * d_head; fp16 models with
 * d_head in {64, 128}, d_model a multiple of 256; fp32 models with d_head 32
 * and d_model 128. d_mlp a multiple of 128. */
typedef struct {
  int32_t d_model, n_heads, d_head, d_mlp, n_pre, vocab;
  float norm_eps;   /* RMSNorm epsilon */
  int32_t dtype;    /* tl_dtype: weights, h, and matrix-product operands */
} tl_config;

/* Device pointers (model dtype) of one unique layer. u = n_pre is the loop
 * block shared by every loop iteration. */
typedef struct {
  const void* norm1;   /* [D]      RMSNorm gain before QKV */
  const void* w_qkv;   /* [3D, D]  rows q | k | v, head-major inside each */
  const void* w_o;     /* [D, D]   */
  const void* norm2;   /* [D]      RMSNorm gain before the MLP */
  const void* w_up;    /* [F, D]   */
  const void* w_down;  /* [D, F]   */
} tl_layer_weights;

typedef struct {
  const void* embed;                 /* [V, D] */
  const void* final_norm;            /* [D]    */
  const void* lm_head;               /* [V, D] */
  const tl_layer_weights* layers;    /* host array of n_pre + 1 entries */
} tl_weights;

typedef struct tl_model tl_model;
typedef struct tl_cache tl_cache;

/* Library version (major * 100 + minor). */
int tl_version(void);

/* Message for the calling thread's last failed call ("" if none). */
const char* tl_last_error(void);

/* Create a model handle over caller-owned device weights (borrowed, not
 * copied). Host state only; enqueues nothing. */
tl_status tl_model_create(const tl_config* cfg, const tl_weights* w, tl_model** out);
void tl_model_destroy(tl_model* m);

/* Exact payload bytes of a cache of n_pre + l_max layers x n_lanes x max_seq
 * entries in `mode` (closed form; features page, "Variable-L KV cache": the
 * cache is sized by n_pre + L_max). 0 if the arguments are invalid, including
 * a max_seq whose code rows of one (layer, lane) would reach 2^31 bytes
 * (max_seq x row bytes without the INT scales; the delta mode counts its
 * 2 * d_model-byte anchor rows): the decode attention addresses one such slab
 * in 32 bits. At d_model
 * 2048 that caps max_seq below 1,048,576 in INT8-h, 2,097,152 in INT4-h and
 * 524,288 in fp16-h. */
size_t tl_cache_bytes(const tl_config* cfg, int mode, int n_lanes, int max_seq, int l_max);

/* Bytes of device workspace a cache needs: per-lane state (length, status,
 * residual norms, last residual) and step scratch for up to
 * min(n_lanes, 256) lanes per decode call and 512 tokens per prefill call. */
size_t tl_workspace_bytes(const tl_config* cfg, int mode, int n_lanes, int max_seq, int l_max);

/* Bind a cache to caller memory: d_cache (tl_cache_bytes) holds the entries,
 * d_workspace (tl_workspace_bytes) the per-lane state and scratch. Enqueues a
 * reset of every lane (length 0, status OK) on `stream`, and zeroes the
 * decode attention's per-(row, head group) tile counters, which every decode
 * step leaves at zero again: the workspace belongs to the library while the
 * cache handle lives and must not be written by the caller. A lane's cache layer
 * n_pre + i is written only by loop iteration i, so it stays valid for every
 * later call with loops >= i + 1. Errors: TL_E_UNSUPPORTED for a mode the
 * model cannot store or a max_seq past the per-slab limit of tl_cache_bytes;
 * TL_E_ARG for bad sizes and short or unaligned buffers. */
tl_status tl_cache_alloc(const tl_model* m, int mode, int n_lanes, int max_seq, int l_max,
                         void* d_cache, size_t cache_bytes, void* d_workspace, size_t ws_bytes,
                         void* stream, tl_cache** out);
/* Host state only; the caller frees the device buffers after the stream is idle. */
void tl_cache_free(tl_cache* c);

/* Prefill: append n_tokens (1..512) prompt tokens to `lane` at its current
 * length and run them through n_pre + loops layers (chunked prefill; features
 * page, closing list of supported techniques). Every layer first appends the
 * chunk's h rows, then rebuilds K/V for all of the lane's positions and runs
 * causal attention (query i at position len + i). Residual norms are not
 * checked during prefill. d_tokens: device int32 [n_tokens].
 * d_next_token (nullable): device int32 [1], greedy token after the chunk.
 * d_last_logits (nullable): device f32 [vocab], logits of the chunk's last token.
 * A lane left aborted by a decode step is skipped on the device (next token
 * -1) until tl_cache_reset_lane.
 * Errors: TL_E_ARG (loops not in 1..l_max, lane out of range, n_tokens out of
 * range), TL_E_CAPACITY, TL_E_CACHE_GAP (the lane already holds positions and
 * n_pre + loops exceeds the layers filled for them). */
tl_status tl_prefill_chunk(tl_cache* c, int lane, int loops, const int32_t* d_tokens,
                           int n_tokens, int32_t* d_next_token, float* d_last_logits,
                           void* stream);

/* tl_prefill_chunk that also returns the chunk's residuals after its last
 * layer: d_x_out (nullable) device f32 [n_tokens, d_model], row i for the
 * token at position len + i. Those rows are what tl_extend_depth resumes
 * from. Errors as tl_prefill_chunk, and TL_E_ARG while a depth extension of
 * the lane is in progress. */
tl_status tl_prefill_chunk_x(tl_cache* c, int lane, int loops, const int32_t* d_tokens,
                             int n_tokens, float* d_x_out, int32_t* d_next_token,
                             float* d_last_logits, void* stream);

/* Warm start mid-loop (features page, "Warm-start mid-loop"): a lane whose
 * positions were all run at old_loops (its cache holds n_pre + old_loops
 * layers) is deepened to new_loops without re-running the first old_loops
 * iterations. Chunk by chunk, in position order starting at 0, positions
 * pos0 .. pos0+n-1 (n in 1..512) run layers n_pre + old_loops ..
 * n_pre + new_loops - 1 from their residual after iteration old_loops - 1,
 * each layer appending h rows and attending causally over the positions
 * before them (already deepened by the earlier chunks). d_x: device f32
 * [n, d_model], in: those residuals (tl_prefill_chunk_x's d_x_out for the
 * same positions), out: the residuals after iteration new_loops - 1, from
 * which a later extension can resume. d_next_token / d_last_logits
 * (nullable): the greedy token and logits after position pos0+n-1. The lane's
 * length does not change; after the chunk that reaches it the lane holds
 * n_pre + new_loops layers and decodes at up to new_loops. Until then the
 * lane takes no prefill or decode call.
 * Errors: TL_E_ARG (lane, loops not 1 <= old < new <= l_max, empty lane, n,
 * a chunk out of order or of another extension), TL_E_CACHE_GAP (the lane
 * does not hold exactly n_pre + old_loops layers). */
tl_status tl_extend_depth(tl_cache* c, int lane, int pos0, int n, int old_loops, int new_loops,
                          float* d_x, int32_t* d_next_token, float* d_last_logits, void* stream);

/* One greedy decode step for n lanes (1..min(n_lanes, 256)), lane k running
 * loops[k] iterations of the loop block (features page, "L-aware batching";
 * lanes never interact, so a lane's result does not depend on its batch mates).
 * lanes, loops: host int32 [n] (distinct lane ids; 1 <= loops[k] <= l_max).
 * d_tokens_in: device int32 [n], the token at each lane's current position (ids
 * outside [0, vocab) are clamped into it).
 * safety_threshold: after every loop iteration the FP32 L2 norm of the lane's
 * residual is compared with it and the lane aborts iff !(norm <= threshold)
 * (novel-contributions page, "Per-Iteration Safety Check"); +INF turns the
 * check off. An abort is not an error: the lane's remaining iterations and its
 * token are skipped, d_lane_status[k] = TL_LANE_ABORTED, d_tokens_out[k] = -1,
 * its row of d_logits (if given) is NaN, its length does not advance, and
 * later calls skip it until tl_cache_reset_lane.
 * d_tokens_out: device int32 [n]. d_logits (nullable): device f32 [n, vocab].
 * d_lane_status: device int32 [n].
 * Errors: TL_E_ARG, TL_E_CAPACITY, TL_E_CACHE_GAP (as for prefill). */
tl_status tl_decode_step(tl_cache* c, int n, const int32_t* lanes, const int32_t* loops,
                         const int32_t* d_tokens_in, float safety_threshold,
                         int32_t* d_tokens_out, float* d_logits, int32_t* d_lane_status,
                         void* stream);

/* For callers that cannot allocate device memory or take a workspace per
 * call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): tl_decode_step with the same arguments, results and
 * errors, whose step scratch (the rows' activations, logits, attention
 * partials and tile counters) lives in a static array of the
 * library, 16 MiB per GPU, held until the process ends; the cache's per-lane
 * state stays in its workspace. It allocates nothing and enqueues the same
 * kernels plus one fill that zeroes the tile counters. The step must fit:
 * about n x (16 d_model + 2 d_mlp + 4 vocab) bytes for an fp16 model
 * (24 d_model + 4 d_mlp + 4 vocab for fp32) plus
 * n x n_heads x ceil(context / 64) x (d_head + 2) x 4 bytes of attention
 * partials (ceil(context / 32) splits for stored K/V), where context is the
 * longest lane's length + 1; a larger step returns TL_E_CAPACITY before
 * anything is enqueued (the 407M shape with 4 lanes at 4224 positions needs
 * about 2 MB). Explicit attention order only, and not
 * the delta-KV mode (TL_E_UNSUPPORTED). Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams, other threads, other
 * caches) race, and the caller must serialise them. The stream must belong to
 * the current device. */
tl_status tl_decode_step_static(tl_cache* c, int n, const int32_t* lanes, const int32_t* loops,
                                const int32_t* d_tokens_in, float safety_threshold,
                                int32_t* d_tokens_out, float* d_logits, int32_t* d_lane_status,
                                void* stream);

/* Self-speculative decoding, chain mode (features page, "Self-speculative
 * decoding"; the greedy-equality claim is in its "Tree speculative decoding"
 * section): one round for `lane`, whose cache holds positions 0 .. len-1 at
 * n_pre + verify_loops layers or more and whose token at position len is
 * *d_token_in. The same weights draft and verify:
 *  1. draft: draft_ahead greedy decode steps at draft_loops, each fed the
 *     previous one's token (d_1 .. d_k, k = draft_ahead);
 *  2. verify: the input token and d_1 .. d_k run as one chunk at
 *     verify_loops from position len, giving the verifier's greedy token
 *     v_j after each of the k + 1 positions;
 *  3. accept the longest prefix with d_j == v_j (a drafts); the round emits
 *     v_1 .. v_{a+1} and the lane's length becomes len + a + 1.
 * The emitted tokens are those plain greedy decoding at verify_loops would
 * produce; the last one is the token at the new length, the input of the
 * next round. Cache entries past the new length are left behind and are
 * overwritten by later calls. The safety check does not run (as in prefill).
 * d_token_in: device int32 [1]. d_tokens_out: device int32 [draft_ahead + 1],
 * the emitted tokens, then -1. n_out: host, the number emitted (1 ..
 * draft_ahead + 1; 0 if the lane was aborted, which leaves it unchanged).
 * Synchronises `stream` (the host needs the new length to place later
 * chunks). Residual norms and tl_lane_residual afterwards describe the last
 * draft step, not the verification.
 * Errors: TL_E_ARG (lane, draft_ahead not in 1..15, not 1 <= draft_loops <=
 * verify_loops <= l_max, null pointers, a depth extension in progress),
 * TL_E_CAPACITY (len + draft_ahead + 1 > max_seq), TL_E_CACHE_GAP. */
tl_status tl_spec_step(tl_cache* c, int lane, int draft_loops, int verify_loops, int draft_ahead,
                       const int32_t* d_token_in, int32_t* d_tokens_out, int* n_out, void* stream);

/* Evaluation order of the decode attention over a store-h cache.
 * EXPLICIT (default): K = W_k h' and V = W_v h' are rebuilt on MFMA for every
 * position, then attended (features page, "Store-h KV cache").
 * ABSORBED: the same attention with the products reassociated (the
 * novel-contributions page relates store-h to MLA): head h scores position j
 * as (W_k,h^T q_h) . h'_j and outputs W_v,h (sum_j p_j h'_j), so all heads
 * attend over the shared rows h' and no K or V is formed; 4*H*D instead of
 * 4*D^2 flops per position. Rounding differs from EXPLICIT (the sums are
 * taken in another order), within the same tolerance of the exact result.
 * Prefill and speculative verification keep the explicit order. */
typedef enum { TL_ATTN_EXPLICIT = 0, TL_ATTN_ABSORBED = 1 } tl_attn_order;

/* Choose the decode attention's evaluation order for later tl_decode_step
 * calls on `c`. Errors: TL_E_ARG (unknown order), TL_E_UNSUPPORTED (ABSORBED
 * covers fp16 models with 16 heads of 64 at d_model 1024 or of 128 at 2048,
 * and the h cache modes; stored-K/V caches have no h to absorb into). */
tl_status tl_cache_set_attention(tl_cache* c, int order);

/* Residual norms of `lane`'s last decode step, one per loop iteration
 * (NaN for iterations that did not run). h_out: host float [l_max].
 * Synchronises `stream`. */
tl_status tl_residual_norms(const tl_cache* c, int lane, float* h_out, void* stream);

/* Copy the lane's residual after its last decode step (f32 [d_model]) into
 * device memory d_out. */
tl_status tl_lane_residual(const tl_cache* c, int lane, float* d_out, void* stream);

/* Write n rows of h (device, model dtype, [n, d_model]) into cache layer
 * `layer` of `lane` at positions pos0 .. pos0+n-1 through the same encoder the
 * step uses (KV mode: K = W_k h and V = W_v h of that layer are stored).
 * Does not change the lane's length. */
tl_status tl_cache_write_h(tl_cache* c, int lane, int layer, int pos0, int n, const void* d_h,
                           void* stream);

/* Fill positions pos0 .. pos0+n-1 of cache layer `layer` of `lane` with
 * synthetic h drawn on the GPU: Philox4x32-10 (Salmon et al., SC'11) with
 * counter (k, pos, lane, layer) and key (seed, 0x1F0E9D75); the eight 16-bit
 * halves of the output are summed, centred (minus 262140) and multiplied in
 * fp32 by 1/(65536*sqrt(2/3)) (bits 0x379CC471), then rounded to the model
 * dtype and encoded like tl_cache_write_h. Does not change the lane's length. */
tl_status tl_cache_fill_synthetic(tl_cache* c, int lane, int layer, int pos0, int n,
                                  uint32_t seed, void* stream);

/* Declare that `lane` holds `length` valid positions in its first
 * `layers_valid` cache layers (after tl_cache_write_h / _fill_synthetic).
 * Resets the lane's status to OK. */
tl_status tl_cache_set_length(tl_cache* c, int lane, int length, int layers_valid, void* stream);

/* Read entries of positions pos0 .. pos0+n-1 of layer `layer`, lane `lane`.
 * d_codes (nullable, INT modes): device int8 [n, d_model], unpacked codes.
 * d_scales (nullable, INT modes): device uint16 (fp16 bits) [n, groups]
 *   (INT8: 1 group, INT4: d_model/32 groups).
 * d_h (nullable): device, model dtype: [n, d_model] the h the attention uses
 *   (dequantised fp16(q*s) for INT modes, fp16 of the prefix sum in delta
 *   mode), or [n, 2*d_model] K|V in KV mode.
 * Delta mode, loop layers: d_codes the INT8 deltas [n, d_model], d_scales the
 *   per-head scales [n, n_heads]. tl_cache_write_h and tl_cache_fill_synthetic
 *   code a loop layer against the cache's reconstruction of the layer below,
 *   so layers are written in order. */
tl_status tl_cache_read(const tl_cache* c, int lane, int layer, int pos0, int n, int8_t* d_codes,
                        uint16_t* d_scales, void* d_h, void* stream);

/* Forget a lane: length 0, status OK, no valid layers. */
tl_status tl_cache_reset_lane(tl_cache* c, int lane, void* stream);

/* Kernel timing for measurement: between tl_profile_start and tl_profile_stop
 * every launch of the decode attention kernel made by tl_decode_step (store-h
 * reconstruction + attention, the absorbed-order attention, or the stored-K/V
 * streaming attention) is timed by a pair of HIP events attached to that
 * launch, which take its own start and end timestamps (hipExtLaunchKernel);
 * the causal attention of tl_prefill_chunk (with its split merge, when the
 * keys are split) is bracketed by events recorded on the call's stream
 * before and after it. tl_profile_stop waits for the last event and returns
 * the summed time in milliseconds and the number of timed launches.
 * Host-side events only; no device memory. */
tl_status tl_profile_start(tl_cache* c);
tl_status tl_profile_stop(tl_cache* c, double* total_ms, int* n_launches);

#ifdef __cplusplus
}
#endif
#endif /* TL_H */
