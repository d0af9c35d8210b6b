// Host side of the C ABI declared in include/tl.h: argument validation, the
// cache / workspace layout, and the per-step schedule of kernel launches.
//
// Decode step (one call, a batch of lanes each with its own loop count;
// TinyLoop architecture-exclusive features page, "L-aware batching"):
//   rows are the call's lanes sorted by loop count (descending, stable), so the
//   lanes still running at layer-iteration l are always the first B_l rows;
//   for l = 0 .. n_pre + max(loops) - 1:
//     RMSNorm + h encode + append at the lane's position (cache layer l)
//     q = W_q h / sqrt(d)                (stored-K/V mode: W_qkv, K|V appended)
//     attention over the cache: K|V rebuilt from h on MFMA (store-h) or
//       streamed (stored-K/V), split over positions, then merged
//     x += W_o o; x += W_down gelu(W_up RMSNorm(x))
//     after loop iterations: residual norm + safety abort (novel-contributions
//       page, "Per-Iteration Safety Check")
//   final RMSNorm, LM head, argmax.
// Layer n_pre + i of the cache is written only by loop iteration i (features
// page, "Variable-L KV cache"), so any later call with loops >= i + 1 reads it.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "tl_internal.h"

using namespace tl;

struct tl_model {
  tl_config cfg;
  ModelView mv;
  std::vector<LayerW> layers;
};

struct tl_cache {
  const tl_model* m;
  int mode, n_lanes, max_seq, l_max, n_layers;
  CacheView cv;
  CacheView mat;                   // delta mode: the one-layer fp16 view of Workspace::hmat
  int order = TL_ATTN_EXPLICIT;    // decode attention's evaluation order
  Workspace ws;
  std::vector<int> host_len;       // upper bound of each lane's length
  std::vector<int> layers_valid;   // layers filled for every position < length
  // depth extension in progress: next position, loops from / to (-1: none)
  std::vector<int> ext_next, ext_from, ext_to;
  bool prof_on = false;
  std::vector<hipEvent_t> prof_ev; // pool of events, pairs (start, stop)
  size_t prof_used = 0;
  ~tl_cache() {
    for (hipEvent_t e : prof_ev) (void)hipEventDestroy(e);
  }
};

namespace {

thread_local std::string g_err;

tl_status fail(tl_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tl_status fail(tl_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

#define TL_HIP(expr)                                                              \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess)                                                         \
      return fail(TL_E_HIP, "%s: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, __LINE__); \
  } while (0)

size_t dtype_size(int dtype) { return dtype == TL_DTYPE_F32 ? 4 : 2; }

bool config_ok(const tl_config* c, std::string* why) {
  if (!c) { *why = "null config"; return false; }
  if (c->d_model <= 0 || c->n_heads <= 0 || c->d_head <= 0 || c->d_mlp <= 0 || c->n_pre < 0 ||
      c->vocab <= 0 || !(c->norm_eps >= 0.f)) { *why = "non-positive dimension"; return false; }
  if (c->n_heads * c->d_head != c->d_model) { *why = "d_model != n_heads * d_head"; return false; }
  if (c->d_mlp % 128 || c->vocab % 16) { *why = "d_mlp must be a multiple of 128, vocab of 16"; return false; }
  if (c->dtype == TL_DTYPE_F32) {
    if (c->d_model != 128 || c->d_head != 32) { *why = "fp32 models: d_model 128, d_head 32"; return false; }
  } else if (c->dtype == TL_DTYPE_F16) {
    if (c->d_model % 256 || c->d_model > 2048 || (c->d_head != 64 && c->d_head != 128)) {
      *why = "fp16 models: d_model a multiple of 256 up to 2048, d_head 64 or 128";
      return false;
    }
  } else {
    *why = "unknown dtype";
    return false;
  }
  return true;
}

bool mode_ok(const tl_config* c, int mode, std::string* why) {
  if (mode < TL_CACHE_KV || mode > TL_CACHE_H_DELTA8) { *why = "unknown cache mode"; return false; }
  if (mode == TL_CACHE_H_DELTA8 && (c->dtype != TL_DTYPE_F16 || c->n_pre < 1)) {
    *why = "the delta codec needs an fp16 model and a unique layer for its anchor";
    return false;
  }
  if (c->dtype == TL_DTYPE_F32 && !(mode == TL_CACHE_KV || mode == TL_CACHE_H_F32)) {
    *why = "fp32 models store fp32 h or K/V";
    return false;
  }
  if (c->dtype == TL_DTYPE_F16 && mode == TL_CACHE_H_F32) {
    *why = "fp16 models store fp16, INT8 or INT4 h, or fp16 K/V";
    return false;
  }
  if (mode == TL_CACHE_KV && c->dtype == TL_DTYPE_F16 && !(c->d_model == 1024 || c->d_model == 2048)) {
    *why = "stored-K/V attention covers d_model 1024 and 2048";
    return false;
  }
  return true;
}

bool dims_ok(int n_lanes, int max_seq, int l_max) {
  return n_lanes > 0 && max_seq > 0 && l_max > 0 && n_lanes <= (1 << 20) && max_seq <= (1 << 24) &&
         l_max <= 4096;
}

size_t entry_bytes(const tl_config* c, int mode) {
  const size_t D = c->d_model;
  switch (mode) {
    case TL_CACHE_KV: return 2 * D * dtype_size(c->dtype);
    case TL_CACHE_H_F32: return 4 * D;
    case TL_CACHE_H_F16: return 2 * D;
    case TL_CACHE_H_INT8: return D + 2;
    case TL_CACHE_H_INT4: return D / 2 + 2 * (D / kInt4Group);
  }
  return 0;
}

// bytes of one position of one lane over all n_pre + l_max layers
size_t position_bytes(const tl_config* c, int mode, int l_max) {
  if (mode == TL_CACHE_H_DELTA8)
    return (size_t)c->n_pre * 2 * c->d_model + (size_t)l_max * (c->d_model + 2 * c->n_heads);
  return (size_t)(c->n_pre + l_max) * entry_bytes(c, mode);
}

struct Layout {
  size_t off[25];
  size_t total;
  int R, Bmax, S, apair_cap;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The decode attention kernels address one (layer, lane) slab of codes
// through a buffer resource whose extent and offsets are 32-bit, so every
// slab (max_seq rows of one layer and lane, without the INT scales, which
// live in their own array; in the delta mode the fp16 anchor rows) stays
// below 2^31 bytes. A layout past that is refused.
constexpr size_t kMaxSlabBytes = (size_t)1 << 31;
bool slab_ok(const tl_config* c, int mode, int max_seq, std::string* why) {
  const size_t D = c->d_model;
  size_t row = 0;
  switch (mode) {
    case TL_CACHE_H_INT8: row = D; break;
    case TL_CACHE_H_INT4: row = D / 2; break;
    case TL_CACHE_H_DELTA8: row = 2 * D; break;
    default: row = entry_bytes(c, mode);
  }
  if ((size_t)max_seq * row >= kMaxSlabBytes) {
    *why = "one layer and lane of the cache would reach 2^31 bytes (max_seq x entry bytes)";
    return false;
  }
  return true;
}

Layout workspace_layout(const tl_config* c, int mode, int n_lanes, int max_seq, int l_max) {
  Layout L{};
  const size_t D = c->d_model, F = c->d_mlp, V = c->vocab, es = dtype_size(c->dtype);
  L.Bmax = std::min(n_lanes, kMaxBatch);
  L.R = std::max(L.Bmax, kMaxChunk);
  // splits per row: the shortest split is kKvSplit positions (stored K/V),
  // 64 in the h modes
  const int min_split = mode == TL_CACHE_KV ? kKvSplit : 64;
  L.S = (max_seq + min_split - 1) / min_split;
  const size_t head_rows = std::max(L.Bmax, kSpecRows);
  const size_t ppart = (size_t)kMaxChunk * c->n_heads * 8 * (c->d_head + 2);
  const bool delta = mode == TL_CACHE_H_DELTA8;
  // the absorbed order's buffers, for the shapes and modes it covers
  const bool absorbed = c->dtype == TL_DTYPE_F16 && c->n_heads == 16 && mode != TL_CACHE_KV &&
                        ((c->d_model == 1024 && c->d_head == 64) || (c->d_model == 2048 && c->d_head == 128));
  L.apair_cap = absorbed ? std::min(1024, L.Bmax * 64) : 0;
  const size_t sizes[25] = {
      (size_t)n_lanes * 4,                        // len
      (size_t)n_lanes * 4,                        // status
      (size_t)n_lanes * l_max * 4,                // norms
      (size_t)n_lanes * D * 4,                    // xres
      (size_t)L.R * 4, (size_t)L.R * 4, (size_t)L.R * 4,   // row_lane, row_slot, row_pos
      (size_t)L.R * D * 4,                        // x
      (size_t)L.R * D * es,                       // h
      (size_t)L.R * D * 4,                        // q
      (size_t)L.R * D * es,                       // o
      (size_t)L.R * D * es,                       // u
      (size_t)L.R * F * es,                       // a
      head_rows * D * es,                         // z
      head_rows * V * 4,                          // logits
      (size_t)L.Bmax * c->n_heads * L.S * (c->d_head + 2) * 4,   // part
      mode == TL_CACHE_KV ? 0 : (size_t)max_seq * 2 * D * 4,     // kvbuf (f32)
      (size_t)L.R * 4,                            // row_dead
      (size_t)(2 * kSpecRows + 2) * 4,            // spec
      ppart * 4,                                  // ppart
      delta ? (size_t)L.R * D * 4 : 0,            // hrec
      delta ? (size_t)n_lanes * max_seq * D * 2 : 0,   // hmat
      absorbed ? (size_t)L.Bmax * c->n_heads * D * 4 : 0,                    // qt
      (size_t)L.apair_cap * c->n_heads * (D + 2) * 4,                       // apart
      (size_t)L.Bmax * (2 * D / 128) * 4,         // tilecnt
  };
  size_t o = 0;
  for (int i = 0; i < 25; ++i) {
    L.off[i] = o;
    o = align256(o + sizes[i]);
  }
  L.total = o;
  return L;
}

tl_status check_lane(const tl_cache* c, int lane) {
  if (!c) return fail(TL_E_ARG, "null cache");
  if (lane < 0 || lane >= c->n_lanes) return fail(TL_E_ARG, "lane %d out of range [0, %d)", lane, c->n_lanes);
  return TL_OK;
}

const LayerW& layer_w(const tl_cache* c, int layer) {
  return c->m->layers[std::min(layer, c->m->cfg.n_pre)];
}

GemmArgs gemm_args(const void* W, int ldw, const void* X, int ldx, int M, int N, int K, int epi,
                   void* out, int ldo) {
  GemmArgs g{};
  g.W = W; g.ldw = ldw; g.X = X; g.ldx = ldx;
  g.M = M; g.N = N; g.K = K; g.epi = epi; g.out = out; g.ldo = ldo;
  g.scale = 1.f;
  return g;
}

}  // namespace

extern "C" {

int tl_version(void) { return 100; }

const char* tl_last_error(void) { return g_err.c_str(); }

tl_status tl_model_create(const tl_config* cfg, const tl_weights* w, tl_model** out) {
  std::string why;
  if (!out) return fail(TL_E_ARG, "null output handle");
  *out = nullptr;
  if (!config_ok(cfg, &why)) return fail(TL_E_UNSUPPORTED, "config: %s", why.c_str());
  if (!w || !w->embed || !w->final_norm || !w->lm_head || !w->layers)
    return fail(TL_E_ARG, "missing weight pointer");
  tl_model* m = new tl_model();
  m->cfg = *cfg;
  for (int u = 0; u <= cfg->n_pre; ++u) {
    const tl_layer_weights& lw = w->layers[u];
    if (!lw.norm1 || !lw.w_qkv || !lw.w_o || !lw.norm2 || !lw.w_up || !lw.w_down) {
      delete m;
      return fail(TL_E_ARG, "missing weight pointer in layer %d", u);
    }
    m->layers.push_back(LayerW{lw.norm1, lw.w_qkv, lw.w_o, lw.norm2, lw.w_up, lw.w_down});
  }
  ModelView& v = m->mv;
  v.D = cfg->d_model; v.H = cfg->n_heads; v.dh = cfg->d_head; v.F = cfg->d_mlp;
  v.n_pre = cfg->n_pre; v.V = cfg->vocab; v.dtype = cfg->dtype; v.eps = cfg->norm_eps;
  v.embed = w->embed; v.final_norm = w->final_norm; v.lm_head = w->lm_head;
  *out = m;
  return TL_OK;
}

void tl_model_destroy(tl_model* m) { delete m; }

size_t tl_cache_bytes(const tl_config* cfg, int mode, int n_lanes, int max_seq, int l_max) {
  std::string why;
  if (!config_ok(cfg, &why) || !mode_ok(cfg, mode, &why) || !dims_ok(n_lanes, max_seq, l_max) ||
      !slab_ok(cfg, mode, max_seq, &why))
    return 0;
  return (size_t)n_lanes * max_seq * position_bytes(cfg, mode, l_max);
}

size_t tl_workspace_bytes(const tl_config* cfg, int mode, int n_lanes, int max_seq, int l_max) {
  std::string why;
  if (!config_ok(cfg, &why) || !mode_ok(cfg, mode, &why) || !dims_ok(n_lanes, max_seq, l_max) ||
      !slab_ok(cfg, mode, max_seq, &why))
    return 0;
  return workspace_layout(cfg, mode, n_lanes, max_seq, l_max).total;
}

tl_status tl_cache_alloc(const tl_model* m, int mode, int n_lanes, int max_seq, int l_max,
                         void* d_cache, size_t cache_bytes, void* d_workspace, size_t ws_bytes,
                         void* stream, tl_cache** out) {
  std::string why;
  if (!out) return fail(TL_E_ARG, "null output handle");
  *out = nullptr;
  if (!m) return fail(TL_E_ARG, "null model");
  const tl_config* cfg = &m->cfg;
  if (!mode_ok(cfg, mode, &why)) return fail(TL_E_UNSUPPORTED, "mode: %s", why.c_str());
  if (!dims_ok(n_lanes, max_seq, l_max)) return fail(TL_E_ARG, "bad n_lanes / max_seq / l_max");
  if (!slab_ok(cfg, mode, max_seq, &why)) return fail(TL_E_UNSUPPORTED, "max_seq %d: %s", max_seq, why.c_str());
  const size_t need = tl_cache_bytes(cfg, mode, n_lanes, max_seq, l_max);
  const Layout L = workspace_layout(cfg, mode, n_lanes, max_seq, l_max);
  if (!d_cache || cache_bytes < need) return fail(TL_E_ARG, "cache buffer: need %zu bytes", need);
  if (!d_workspace || ws_bytes < L.total) return fail(TL_E_ARG, "workspace: need %zu bytes", L.total);
  if (((uintptr_t)d_cache | (uintptr_t)d_workspace) & 255) return fail(TL_E_ARG, "buffers must be 256-byte aligned");

  tl_cache* c = new tl_cache();
  c->m = m;
  c->mode = mode; c->n_lanes = n_lanes; c->max_seq = max_seq; c->l_max = l_max;
  c->n_layers = cfg->n_pre + l_max;
  CacheView& v = c->cv;
  v.base = (char*)d_cache;
  v.mode = mode; v.dtype = cfg->dtype; v.D = cfg->d_model;
  v.n_lanes = n_lanes; v.max_seq = max_seq; v.n_layers = c->n_layers;
  const size_t D = cfg->d_model;
  const size_t n_entries = (size_t)c->n_layers * n_lanes * max_seq;
  v.scales = nullptr;
  if (mode == TL_CACHE_H_INT8) v.scales = (uint16_t*)(v.base + n_entries * D);
  if (mode == TL_CACHE_H_INT4) v.scales = (uint16_t*)(v.base + n_entries * (D / 2));
  char* w = (char*)d_workspace;
  Workspace& s = c->ws;
  s.len = (int32_t*)(w + L.off[0]);
  s.status = (int32_t*)(w + L.off[1]);
  s.norms = (float*)(w + L.off[2]);
  s.xres = (float*)(w + L.off[3]);
  s.row_lane = (int32_t*)(w + L.off[4]);
  s.row_slot = (int32_t*)(w + L.off[5]);
  s.row_pos = (int32_t*)(w + L.off[6]);
  s.x = (float*)(w + L.off[7]);
  s.h = w + L.off[8];
  s.q = (float*)(w + L.off[9]);
  s.o = w + L.off[10];
  s.u = w + L.off[11];
  s.a = w + L.off[12];
  s.z = w + L.off[13];
  s.logits = (float*)(w + L.off[14]);
  s.part = (float*)(w + L.off[15]);
  s.kvbuf = mode == TL_CACHE_KV ? nullptr : w + L.off[16];
  s.row_dead = (int32_t*)(w + L.off[17]);
  s.spec = (int32_t*)(w + L.off[18]);
  s.ppart = (float*)(w + L.off[19]);
  s.ppart_floats = (int)((size_t)kMaxChunk * cfg->n_heads * 8 * (cfg->d_head + 2));
  s.hrec = mode == TL_CACHE_H_DELTA8 ? (float*)(w + L.off[20]) : nullptr;
  s.hmat = mode == TL_CACHE_H_DELTA8 ? (void*)(w + L.off[21]) : nullptr;
  s.qt = L.apair_cap ? (float*)(w + L.off[22]) : nullptr;
  s.apart = L.apair_cap ? (float*)(w + L.off[23]) : nullptr;
  s.apair_cap = L.apair_cap;
  s.tilecnt = (int32_t*)(w + L.off[24]);
  v.n_pre = cfg->n_pre; v.H = cfg->n_heads; v.dh = cfg->d_head;
  if (mode == TL_CACHE_H_DELTA8) {
    v.scales = (uint16_t*)(v.base + (size_t)n_lanes * max_seq *
                                        ((size_t)cfg->n_pre * 2 * D + (size_t)l_max * D));
    CacheView& mt = c->mat;
    mt = v;
    mt.base = (char*)s.hmat; mt.scales = nullptr; mt.mode = TL_CACHE_H_F16; mt.n_layers = 1;
  }
  s.R = L.R; s.Bmax = L.Bmax; s.S = L.S;
  c->host_len.assign(n_lanes, 0);
  c->layers_valid.assign(n_lanes, 0);
  c->ext_next.assign(n_lanes, -1);
  c->ext_from.assign(n_lanes, 0);
  c->ext_to.assign(n_lanes, 0);
  hipError_t e = launch_lane_reset(s, 0, n_lanes, l_max, 0, (hipStream_t)stream);
  if (e == hipSuccess) e = launch_fill_i32(s.tilecnt, L.Bmax * (int)(2 * D / 128), 0, (hipStream_t)stream);
  if (e != hipSuccess) {
    delete c;
    return fail(TL_E_HIP, "lane reset: %s", hipGetErrorString(e));
  }
  *out = c;
  return TL_OK;
}

void tl_cache_free(tl_cache* c) { delete c; }

tl_status tl_cache_reset_lane(tl_cache* c, int lane, void* stream) {
  tl_status st = check_lane(c, lane);
  if (st) return st;
  TL_HIP(launch_lane_reset(c->ws, lane, 1, c->l_max, 0, (hipStream_t)stream));
  c->host_len[lane] = 0;
  c->layers_valid[lane] = 0;
  c->ext_next[lane] = -1;
  return TL_OK;
}

tl_status tl_cache_set_length(tl_cache* c, int lane, int length, int layers_valid, void* stream) {
  tl_status st = check_lane(c, lane);
  if (st) return st;
  if (length < 0 || length > c->max_seq) return fail(TL_E_ARG, "length out of range");
  if (layers_valid < 0 || layers_valid > c->n_layers) return fail(TL_E_ARG, "layers_valid out of range");
  TL_HIP(launch_lane_reset(c->ws, lane, 1, c->l_max, length, (hipStream_t)stream));
  c->host_len[lane] = length;
  c->layers_valid[lane] = length ? layers_valid : 0;
  c->ext_next[lane] = -1;
  return TL_OK;
}

tl_status tl_cache_write_h(tl_cache* c, int lane, int layer, int pos0, int n, const void* d_h,
                           void* stream) {
  tl_status st = check_lane(c, lane);
  if (st) return st;
  if (layer < 0 || layer >= c->n_layers) return fail(TL_E_ARG, "layer out of range");
  if (n <= 0 || pos0 < 0 || pos0 + n > c->max_seq) return fail(TL_E_CAPACITY, "positions out of range");
  if (!d_h) return fail(TL_E_ARG, "null h");
  hipStream_t s = (hipStream_t)stream;
  const ModelView& mv = c->m->mv;
  if (c->mode == TL_CACHE_KV) {
    const LayerW& W = layer_w(c, layer);
    const size_t es = dtype_size(mv.dtype);
    GemmArgs g = gemm_args((const char*)W.w_qkv + (size_t)mv.D * mv.D * es, mv.D, d_h, mv.D, n,
                           2 * mv.D, mv.D, EPI_QKV, nullptr, mv.D);
    g.cache = c->cv; g.layer = layer; g.fixed_lane = lane; g.pos0 = pos0; g.f_offset = mv.D;
    TL_HIP(launch_gemm(mv, g, s));
    return TL_OK;
  }
  AppendArgs a{};
  a.src = HS_INPUT; a.n = n; a.layer = layer; a.h_in = d_h;
  a.fixed_lane = lane; a.pos0 = pos0;
  TL_HIP(launch_norm_append(mv, c->cv, a, s));
  return TL_OK;
}

tl_status tl_cache_fill_synthetic(tl_cache* c, int lane, int layer, int pos0, int n, uint32_t seed,
                                  void* stream) {
  tl_status st = check_lane(c, lane);
  if (st) return st;
  if (layer < 0 || layer >= c->n_layers) return fail(TL_E_ARG, "layer out of range");
  if (n <= 0 || pos0 < 0 || pos0 + n > c->max_seq) return fail(TL_E_CAPACITY, "positions out of range");
  hipStream_t s = (hipStream_t)stream;
  const ModelView& mv = c->m->mv;
  AppendArgs a{};
  a.src = HS_SYNTH; a.layer = layer; a.seed = seed; a.fixed_lane = lane;
  if (c->mode != TL_CACHE_KV) {
    a.n = n; a.pos0 = pos0;
    TL_HIP(launch_norm_append(mv, c->cv, a, s));
    return TL_OK;
  }
  // stored-K/V: draw h into scratch rows, then K|V = W_kv h
  const LayerW& W = layer_w(c, layer);
  const size_t es = dtype_size(mv.dtype);
  for (int p = 0; p < n; p += c->ws.R) {
    const int k = std::min(c->ws.R, n - p);
    a.n = k; a.pos0 = pos0 + p; a.h_out = c->ws.h;
    TL_HIP(launch_norm_append(mv, c->cv, a, s));
    GemmArgs g = gemm_args((const char*)W.w_qkv + (size_t)mv.D * mv.D * es, mv.D, c->ws.h, mv.D, k,
                           2 * mv.D, mv.D, EPI_QKV, nullptr, mv.D);
    g.cache = c->cv; g.layer = layer; g.fixed_lane = lane; g.pos0 = pos0 + p; g.f_offset = mv.D;
    TL_HIP(launch_gemm(mv, g, s));
  }
  return TL_OK;
}

tl_status tl_cache_read(const tl_cache* c, int lane, int layer, int pos0, int n, int8_t* d_codes,
                        uint16_t* d_scales, void* d_h, void* stream) {
  tl_status st = check_lane(c, lane);
  if (st) return st;
  if (layer < 0 || layer >= c->n_layers) return fail(TL_E_ARG, "layer out of range");
  if (n <= 0 || pos0 < 0 || pos0 + n > c->max_seq) return fail(TL_E_ARG, "positions out of range");
  const bool int_mode = c->mode == TL_CACHE_H_INT8 || c->mode == TL_CACHE_H_INT4 ||
                        (c->mode == TL_CACHE_H_DELTA8 && layer >= c->m->mv.n_pre);
  if ((d_codes || d_scales) && !int_mode)
    return fail(TL_E_ARG, "codes and scales exist in INT modes only (delta mode: loop layers)");
  TL_HIP(launch_cache_read(c->m->mv, c->cv, lane, layer, pos0, n, d_codes, d_scales, d_h,
                           (hipStream_t)stream));
  return TL_OK;
}

tl_status tl_residual_norms(const tl_cache* c, int lane, float* h_out, void* stream) {
  tl_status st = check_lane(c, lane);
  if (st) return st;
  if (!h_out) return fail(TL_E_ARG, "null output");
  hipStream_t s = (hipStream_t)stream;
  TL_HIP(hipMemcpyAsync(h_out, c->ws.norms + (size_t)lane * c->l_max, sizeof(float) * c->l_max,
                        hipMemcpyDeviceToHost, s));
  TL_HIP(hipStreamSynchronize(s));
  return TL_OK;
}

tl_status tl_lane_residual(const tl_cache* c, int lane, float* d_out, void* stream) {
  tl_status st = check_lane(c, lane);
  if (st) return st;
  if (!d_out) return fail(TL_E_ARG, "null output");
  TL_HIP(launch_copy_f32(c->ws.xres + (size_t)lane * c->m->mv.D, d_out, c->m->mv.D,
                         (hipStream_t)stream));
  return TL_OK;
}

static // One chunk of positions pos0 .. pos0+n-1 of `lane` through layers
// layer_begin .. layer_end-1 (every layer appends its h rows before the
// chunk's causal attention over positions 0 .. pos0+i reads them); then the
// last position's next token. d_x_in: the residuals entering layer_begin
// (resume) instead of the token embeddings; d_x_out: the residuals after
// layer_end-1. Arguments are checked by the callers.
tl_status run_chunk(tl_cache* c, int lane, int pos0, int n, int layer_begin, int layer_end,
                    const int32_t* d_tokens, const float* d_x_in, float* d_x_out, int new_len,
                    int32_t* d_next_token, float* d_last_logits, hipStream_t s,
                    int32_t* d_spec_out = nullptr) {
  const tl_model* m = c->m;
  const ModelView& mv = m->mv;
  const Workspace& ws = c->ws;
  const int T = pos0 + n, D = mv.D;
  const size_t es = dtype_size(mv.dtype);
  const float qscale = (float)(1.0 / sqrt((double)mv.dh));
  // rows of the chunk: positions pos0 .. pos0+n-1; x from the token
  // embeddings, or the caller's residuals when resuming mid-loop
  TL_HIP(launch_prefill_setup(mv, ws, lane, n, d_x_in ? nullptr : d_tokens, pos0, s));
  if (d_x_in) TL_HIP(launch_copy_f32(d_x_in, ws.x, (size_t)n * D, s));
  const bool delta = c->mode == TL_CACHE_H_DELTA8;
  // chunks of 64 tokens or more run their products on the LDS-tiled kernel
  const int tiled = n >= 64 ? 1 : 0;
  // delta mode, resuming mid-loop: the rows' reconstruction of the layer below
  if (delta && layer_begin > 0)
    TL_HIP(launch_delta_rec(c->cv, layer_begin - 1, lane, pos0, n, ws.hrec, s));
  for (int layer = layer_begin; layer < layer_end; ++layer) {
    const LayerW& W = layer_w(c, layer);
    AppendArgs a{};
    a.src = HS_NORM; a.n = n; a.layer = layer; a.x = ws.x; a.gain = W.norm1;
    a.row_lane = ws.row_lane; a.row_pos = ws.row_pos; a.status = ws.status; a.h_out = ws.h;
    a.rec = ws.hrec;
    TL_HIP(launch_norm_append(mv, c->cv, a, s));
    const void* kv;
    if (c->mode == TL_CACHE_KV) {
      GemmArgs g = gemm_args(W.w_qkv, D, ws.h, D, n, 3 * D, D, EPI_QKV, ws.q, D);
      g.scale = qscale; g.q_is_t = 0; g.cache = c->cv; g.layer = layer;
      g.row_lane = ws.row_lane; g.status = ws.status; g.row_dead = ws.row_dead; g.row_pos = ws.row_pos;
      TL_HIP(launch_gemm(mv, g, s));
      kv = c->cv.kv_row(layer, lane, 0);
    } else {
      GemmArgs g = gemm_args(W.w_qkv, D, ws.h, D, n, D, D, EPI_STORE_F32, ws.q, D);
      g.scale = qscale; g.row_lane = ws.row_lane; g.status = ws.status; g.row_dead = ws.row_dead;
      g.tiled = tiled;
      TL_HIP(launch_gemm(mv, g, s));
      if (delta) {
        // h' of this layer for positions 0 .. T-1, then the fp16-h reconstruction
        TL_HIP(launch_delta_mat(c->cv, c->mat, layer, ws.row_lane, ws.row_pos, ws.status, 1, T, T, s));
        TL_HIP(launch_recon_store(mv, c->mat, 0, lane, T, W.w_qkv, ws.kvbuf, ws.status, s));
      } else {
        TL_HIP(launch_recon_store(mv, c->cv, layer, lane, T, W.w_qkv, ws.kvbuf, ws.status, s));
      }
      kv = ws.kvbuf;
    }
    if (c->prof_on) {
      // profiling: events around the prefill attention kernel alone
      while (c->prof_ev.size() < c->prof_used + 2) {
        hipEvent_t e;
        TL_HIP(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
        c->prof_ev.push_back(e);
      }
      TL_HIP(hipEventRecord(c->prof_ev[c->prof_used], s));
    }
    TL_HIP(launch_prefill_attn(mv, n, pos0, ws.q, kv, c->mode != TL_CACHE_KV, ws.o, lane,
                               ws.status, ws.ppart, ws.ppart_floats, ws.row_lane, ws.row_pos, s));
    if (c->prof_on) {
      TL_HIP(hipEventRecord(c->prof_ev[c->prof_used + 1], s));
      c->prof_used += 2;
    }
    GemmArgs go = gemm_args(W.w_o, D, ws.o, D, n, D, D, EPI_ADD_F32, ws.x, D);
    go.row_lane = ws.row_lane; go.status = ws.status; go.row_dead = ws.row_dead; go.tiled = tiled;
    TL_HIP(launch_gemm(mv, go, s));
    TL_HIP(launch_rmsnorm(mv, n, ws.x, W.norm2, ws.u, ws.row_lane, ws.status, s));
    GemmArgs gu = gemm_args(W.w_up, D, ws.u, D, n, mv.F, D, EPI_GELU_T, ws.a, mv.F);
    gu.row_lane = ws.row_lane; gu.status = ws.status; gu.row_dead = ws.row_dead; gu.tiled = tiled;
    TL_HIP(launch_gemm(mv, gu, s));
    GemmArgs gd = gemm_args(W.w_down, mv.F, ws.a, mv.F, n, D, mv.F, EPI_ADD_F32, ws.x, D);
    gd.row_lane = ws.row_lane; gd.status = ws.status; gd.row_dead = ws.row_dead; gd.tiled = tiled;
    TL_HIP(launch_gemm(mv, gd, s));
  }
  if (d_x_out) TL_HIP(launch_copy_f32(ws.x, d_x_out, (size_t)n * D, s));
  if (d_spec_out) {
    // speculative verification: every row's token, then the acceptance
    TL_HIP(launch_rmsnorm(mv, n, ws.x, mv.final_norm, ws.z, ws.row_lane, ws.status, s));
    GemmArgs gh = gemm_args(mv.lm_head, D, ws.z, D, n, mv.V, D, EPI_STORE_F32, ws.logits, mv.V);
    gh.row_lane = ws.row_lane; gh.status = ws.status; gh.row_dead = ws.row_dead;
    TL_HIP(launch_gemm(mv, gh, s));
    TL_HIP(launch_spec_accept(mv, ws, lane, pos0, n - 1, ws.logits, d_spec_out, s));
    return TL_OK;
  }
  // the last position's token
  TL_HIP(launch_rmsnorm(mv, 1, ws.x + (size_t)(n - 1) * D, mv.final_norm, ws.z, ws.row_lane,
                        ws.status, s));
  float* lg = d_last_logits ? d_last_logits : ws.logits;
  GemmArgs gh = gemm_args(mv.lm_head, D, ws.z, D, 1, mv.V, D, EPI_STORE_F32, lg, mv.V);
  gh.row_lane = ws.row_lane; gh.status = ws.status; gh.row_dead = ws.row_dead;
  TL_HIP(launch_gemm(mv, gh, s));
  TL_HIP(launch_prefill_finish(mv, ws, lane, new_len, lg, d_next_token, s));
  (void)es;
  return TL_OK;
}

tl_status tl_prefill_chunk(tl_cache* c, int lane, int loops, const int32_t* d_tokens, int n_tokens,
                           int32_t* d_next_token, float* d_last_logits, void* stream) {
  return tl_prefill_chunk_x(c, lane, loops, d_tokens, n_tokens, nullptr, d_next_token, d_last_logits,
                            stream);
}

tl_status tl_prefill_chunk_x(tl_cache* c, int lane, int loops, const int32_t* d_tokens, int n_tokens,
                             float* d_x_out, int32_t* d_next_token, float* d_last_logits,
                             void* stream) {
  tl_status st = check_lane(c, lane);
  if (st) return st;
  if (loops < 1 || loops > c->l_max) return fail(TL_E_ARG, "loops %d not in [1, %d]", loops, c->l_max);
  if (n_tokens < 1 || n_tokens > kMaxChunk) return fail(TL_E_ARG, "n_tokens %d not in [1, %d]", n_tokens, kMaxChunk);
  if (!d_tokens) return fail(TL_E_ARG, "null tokens");
  if (c->ext_next[lane] >= 0) return fail(TL_E_ARG, "lane %d: a depth extension is in progress", lane);
  const int pos0 = c->host_len[lane];
  if (pos0 + n_tokens > c->max_seq) return fail(TL_E_CAPACITY, "lane %d: %d + %d positions exceed %d", lane, pos0, n_tokens, c->max_seq);
  const ModelView& mv = c->m->mv;
  const int n_layers = mv.n_pre + loops;
  if (pos0 > 0 && n_layers > c->layers_valid[lane])
    return fail(TL_E_CACHE_GAP, "lane %d: layers %d.. miss earlier positions", lane, c->layers_valid[lane]);
  const int T = pos0 + n_tokens;
  st = run_chunk(c, lane, pos0, n_tokens, 0, n_layers, d_tokens, nullptr, d_x_out, T, d_next_token,
                 d_last_logits, (hipStream_t)stream);
  if (st) return st;
  c->host_len[lane] = T;
  c->layers_valid[lane] = pos0 == 0 ? n_layers : std::min(c->layers_valid[lane], n_layers);
  return TL_OK;
}

tl_status tl_extend_depth(tl_cache* c, int lane, int pos0, int n, int old_loops, int new_loops,
                          float* d_x, int32_t* d_next_token, float* d_last_logits, void* stream) {
  tl_status st = check_lane(c, lane);
  if (st) return st;
  const ModelView& mv = c->m->mv;
  if (!(1 <= old_loops && old_loops < new_loops && new_loops <= c->l_max))
    return fail(TL_E_ARG, "loops %d -> %d not 1 <= old < new <= %d", old_loops, new_loops, c->l_max);
  if (!d_x) return fail(TL_E_ARG, "null residuals");
  const int len = c->host_len[lane];
  if (len < 1) return fail(TL_E_ARG, "lane %d is empty", lane);
  if (n < 1 || n > kMaxChunk) return fail(TL_E_ARG, "n %d not in [1, %d]", n, kMaxChunk);
  const int expect = c->ext_next[lane] >= 0 ? c->ext_next[lane] : 0;
  if (pos0 != expect || pos0 + n > len)
    return fail(TL_E_ARG, "lane %d: extension chunk at %d (+%d) but %d of %d positions done", lane, pos0, n, expect, len);
  if (c->ext_next[lane] >= 0 && (c->ext_from[lane] != old_loops || c->ext_to[lane] != new_loops))
    return fail(TL_E_ARG, "lane %d: extension %d -> %d in progress", lane, c->ext_from[lane], c->ext_to[lane]);
  if (c->ext_next[lane] < 0 && c->layers_valid[lane] != mv.n_pre + old_loops)
    return fail(TL_E_CACHE_GAP, "lane %d holds %d layers, not n_pre + %d", lane, c->layers_valid[lane], old_loops);
  st = run_chunk(c, lane, pos0, n, mv.n_pre + old_loops, mv.n_pre + new_loops, nullptr, d_x, d_x, len,
                 d_next_token, d_last_logits, (hipStream_t)stream);
  if (st) return st;
  if (pos0 + n == len) {
    c->ext_next[lane] = -1;
    c->layers_valid[lane] = mv.n_pre + new_loops;
  } else {
    c->ext_next[lane] = pos0 + n;
    c->ext_from[lane] = old_loops;
    c->ext_to[lane] = new_loops;
  }
  return TL_OK;
}

}  // extern "C"

namespace {

// Checks of a decode call, before anything is enqueued; returns the deepest
// loop count and the longest context of the call.
tl_status decode_validate(tl_cache* c, int n, const int32_t* lanes, const int32_t* loops,
                          const int32_t* d_tokens_in, float safety_threshold,
                          const int32_t* d_tokens_out, const int32_t* d_lane_status, int* lmax_out,
                          int* t_ub_out) {
  if (!c) return fail(TL_E_ARG, "null cache");
  if (n < 1 || n > c->ws.Bmax) return fail(TL_E_ARG, "n = %d not in [1, %d]", n, c->ws.Bmax);
  if (!lanes || !loops || !d_tokens_in || !d_tokens_out || !d_lane_status)
    return fail(TL_E_ARG, "null argument");
  if (isnan(safety_threshold)) return fail(TL_E_ARG, "NaN threshold");
  const ModelView& mv = c->m->mv;
  std::vector<char> seen(c->n_lanes, 0);
  int lmax_call = 0, t_ub = 0;
  for (int k = 0; k < n; ++k) {
    const int lane = lanes[k], L = loops[k];
    if (lane < 0 || lane >= c->n_lanes) return fail(TL_E_ARG, "lane %d out of range", lane);
    if (seen[lane]) return fail(TL_E_ARG, "lane %d appears twice", lane);
    seen[lane] = 1;
    if (c->ext_next[lane] >= 0) return fail(TL_E_ARG, "lane %d: a depth extension is in progress", lane);
    if (L < 1 || L > c->l_max) return fail(TL_E_ARG, "loops %d not in [1, %d]", L, c->l_max);
    if (c->host_len[lane] + 1 > c->max_seq) return fail(TL_E_CAPACITY, "lane %d is full", lane);
    if (c->host_len[lane] > 0 && mv.n_pre + L > c->layers_valid[lane])
      return fail(TL_E_CACHE_GAP, "lane %d: layers %d.. miss earlier positions", lane, c->layers_valid[lane]);
    lmax_call = std::max(lmax_call, L);
    t_ub = std::max(t_ub, c->host_len[lane] + 1);
  }
  *lmax_out = lmax_call;
  *t_ub_out = t_ub;
  return TL_OK;
}

// The launches of one validated decode step on the step scratch of `ws` (the
// cache's per-lane state, its other fields, is shared by every variant).
tl_status decode_enqueue(tl_cache* c, const Workspace& ws, int n, const int32_t* lanes,
                         const int32_t* loops, const int32_t* d_tokens_in, float safety_threshold,
                         int32_t* d_tokens_out, float* d_logits, int32_t* d_lane_status, void* stream,
                         int lmax_call, int t_ub) {
  const tl_model* m = c->m;
  const ModelView& mv = m->mv;
  // rows sorted by loop count, deepest first: the active rows of every layer form a prefix
  std::vector<int> order(n);
  for (int k = 0; k < n; ++k) order[k] = k;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return loops[a] > loops[b]; });
  StepMap map;
  map.n = n;
  for (int r = 0; r < n; ++r) {
    map.lane[r] = lanes[order[r]];
    map.slot[r] = order[r];
  }
  hipStream_t s = (hipStream_t)stream;
  const int D = mv.D;
  const float qscale = (float)(1.0 / sqrt((double)mv.dh));
  const bool check = !(safety_threshold == INFINITY);
  TL_HIP(launch_step_setup(mv, ws, map, d_tokens_in, c->l_max, s));
  const int n_layers = mv.n_pre + lmax_call;
  int rows = n;
  for (int layer = 0; layer < n_layers; ++layer) {
    while (rows > 0 && mv.n_pre + loops[order[rows - 1]] <= layer) --rows;
    const LayerW& W = layer_w(c, layer);
    // the attention input projection forms h = RMSNorm1(x) itself and does
    // the row work before it: the safety check of the residual entering this
    // layer (the one after loop iteration layer - 1 - n_pre) and the append
    // of h to the cache
    auto row_work = [&](GemmArgs& g) {
      g.norm_gain = W.norm1; g.row_tasks = 1; g.check_iter = -1; g.rec = ws.hrec;
      g.cache = c->cv; g.layer = layer; g.row_pos = ws.row_pos;
      g.row_lane = ws.row_lane; g.status = ws.status; g.row_dead = ws.row_dead;
      if (layer > mv.n_pre) {
        g.check_iter = layer - 1 - mv.n_pre;
        g.norms = ws.norms; g.status_w = ws.status; g.l_max = c->l_max;
        g.check = check ? 1 : 0; g.thr = safety_threshold;
      }
    };
    ReconArgs ra{};
    ra.cache = c->cv; ra.layer = layer; ra.w_qkv = W.w_qkv; ra.n_rows = rows; ra.t_ub = t_ub;
    ra.row_lane = ws.row_lane; ra.row_pos = ws.row_pos; ra.status = ws.status; ra.q = ws.q;
    ra.part = ws.part; ra.S = ws.S;
    int split_len;
    if (c->prof_on) {
      // profiling: a pair of events that take the attention kernel's own
      // start and end (the launch gaps around it, and any merge launch
      // after it, are not counted)
      while (c->prof_ev.size() < c->prof_used + 2) {
        hipEvent_t e;
        TL_HIP(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
        c->prof_ev.push_back(e);
      }
      ra.ev.start = c->prof_ev[c->prof_used];
      ra.ev.stop = c->prof_ev[c->prof_used + 1];
    }
    if (c->mode == TL_CACHE_KV) {
      GemmArgs g = gemm_args(W.w_qkv, D, ws.x, D, rows, 3 * D, D, EPI_QKV, ws.q, D);
      g.scale = qscale; g.q_is_t = 0;
      row_work(g);
      TL_HIP(launch_gemm(mv, g, s));
      TL_HIP(launch_kv_attn(mv, ra, s));
      split_len = kKvSplit;
    } else {
      GemmArgs g = gemm_args(W.w_qkv, D, ws.x, D, rows, D, D, EPI_STORE_F32, ws.q, D);
      g.scale = qscale;
      row_work(g);
      TL_HIP(launch_gemm(mv, g, s));
      if (c->mode == TL_CACHE_H_DELTA8) {
        // h' of this layer for every active row's positions, then the fp16-h kernel
        TL_HIP(launch_delta_mat(c->cv, c->mat, layer, ws.row_lane, ws.row_pos, ws.status, rows, t_ub, 0, s));
        ra.cache = c->mat;
        ra.layer = 0;
      }
      if (c->order == TL_ATTN_ABSORBED) {
        // absorbed order: qt = W_k^T q, attention over h' itself, o = W_v r
        TL_HIP(launch_absorb_q(mv, rows, ws.q, W.w_qkv, ws.qt, s));
        int sl = 0;
        const int S = absorbed_splits(rows, t_ub, ws.apair_cap, &sl);
        TL_HIP(launch_absorbed_attn(mv, ra.cache, ra.layer, rows, ws.row_lane, ws.row_pos, ws.status,
                                    ws.qt, ws.apart, S, sl, s, ra.ev));
        // (the merged r reuses the qt rows, which the attention kernel has consumed)
        TL_HIP(launch_absorbed_out(mv, rows, ws.row_lane, ws.row_pos, ws.status, ws.apart, S, sl,
                                   W.w_qkv, ws.qt, ws.o, s));
        split_len = 0;
      } else {
        // fp16 models: the attention kernel merges its own tiles into o
        const bool fused = combined_splits(mv, ra.cache.mode);
        if (fused) {
          ra.o = ws.o;
          ra.tilecnt = ws.tilecnt;
        }
        TL_HIP(launch_recon_attn(mv, ra, s));
        split_len = fused ? 0 : recon_split_len(mv, ra.cache.mode);
      }
    }
    if (c->prof_on) c->prof_used += 2;   // the pair was taken by a launch
    if (split_len) {
      TL_HIP(launch_attn_merge(mv, rows, ws.row_lane, ws.row_pos, ws.status, ws.part, ws.S, split_len,
                               ws.o, s));
    }
    GemmArgs go = gemm_args(W.w_o, D, ws.o, D, rows, D, D, EPI_ADD_F32, ws.x, D);
    go.row_lane = ws.row_lane; go.status = ws.status; go.row_dead = ws.row_dead;
    TL_HIP(launch_gemm(mv, go, s));
    // MLP: the up projection forms RMSNorm2(x) itself
    GemmArgs gu = gemm_args(W.w_up, D, ws.x, D, rows, mv.F, D, EPI_GELU_T, ws.a, mv.F);
    gu.row_lane = ws.row_lane; gu.status = ws.status; gu.row_dead = ws.row_dead; gu.row_pos = ws.row_pos; gu.norm_gain = W.norm2;
    TL_HIP(launch_gemm(mv, gu, s));
    GemmArgs gd = gemm_args(W.w_down, mv.F, ws.a, mv.F, rows, D, mv.F, EPI_ADD_F32, ws.x, D);
    gd.row_lane = ws.row_lane; gd.status = ws.status; gd.row_dead = ws.row_dead;
    TL_HIP(launch_gemm(mv, gd, s));
  }
  // the final RMSNorm, the LM head, then the step's end: every row's last
  // loop iteration is checked there on the final residual (the earlier ones
  // were checked on entry to the next layer), and a row stopped there has its
  // logits replaced. (The LM head forming the norm itself, as the Q and MLP-up
  // products do, was slower: its 2000 workgroups each repeat the norm.)
  NormCheck fc{};
  fc.norms = ws.norms; fc.status = ws.status; fc.l_max = c->l_max;
  fc.check = check ? 1 : 0; fc.thr = safety_threshold;
  for (int r = 0; r < n; ++r) fc.iter[r] = loops[order[r]] - 1;
  float* lg = d_logits ? d_logits : ws.logits;
  TL_HIP(launch_rmsnorm(mv, n, ws.x, mv.final_norm, ws.z, ws.row_lane, ws.status, s));
  GemmArgs gh = gemm_args(mv.lm_head, D, ws.z, D, n, mv.V, D, EPI_LOGITS, lg, mv.V);
  gh.row_lane = ws.row_lane; gh.status = ws.status; gh.row_dead = ws.row_dead;
  gh.row_slot = d_logits ? ws.row_slot : nullptr;
  TL_HIP(launch_gemm(mv, gh, s));
  TL_HIP(launch_finish(mv, ws, n, lg, mv.V, d_logits ? 1 : 0, d_tokens_out, d_lane_status,
                       d_logits, fc, s));
  for (int k = 0; k < n; ++k) {
    const int lane = lanes[k];
    const int nl = mv.n_pre + loops[k];
    c->layers_valid[lane] = c->host_len[lane] == 0 ? nl : std::min(c->layers_valid[lane], nl);
    c->host_len[lane] += 1;
  }
  return TL_OK;
}

// Step scratch of tl_decode_step_static, for callers that cannot allocate:
// one array per GPU, held until the process ends. Host code uses only its
// device address from hipGetSymbolAddress (taken once per device, on the
// first call with that device current), never the name itself.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

tl_status static_scratch(char** out) {
  int dev = -1;
  TL_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(TL_E_ARG, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(TL_E_HIP, "static scratch address: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = (char*)p;
  }
  *out = g_scratch_ptr[dev];
  return TL_OK;
}

}  // namespace

extern "C" {

tl_status tl_decode_step(tl_cache* c, int n, const int32_t* lanes, const int32_t* loops,
                         const int32_t* d_tokens_in, float safety_threshold,
                         int32_t* d_tokens_out, float* d_logits, int32_t* d_lane_status,
                         void* stream) {
  int lmax_call = 0, t_ub = 0;
  tl_status st = decode_validate(c, n, lanes, loops, d_tokens_in, safety_threshold, d_tokens_out,
                                 d_lane_status, &lmax_call, &t_ub);
  if (st != TL_OK) return st;
  return decode_enqueue(c, c->ws, n, lanes, loops, d_tokens_in, safety_threshold, d_tokens_out,
                        d_logits, d_lane_status, stream, lmax_call, t_ub);
}

tl_status tl_decode_step_static(tl_cache* c, int n, const int32_t* lanes, const int32_t* loops,
                                const int32_t* d_tokens_in, float safety_threshold,
                                int32_t* d_tokens_out, float* d_logits, int32_t* d_lane_status,
                                void* stream) {
  int lmax_call = 0, t_ub = 0;
  tl_status st = decode_validate(c, n, lanes, loops, d_tokens_in, safety_threshold, d_tokens_out,
                                 d_lane_status, &lmax_call, &t_ub);
  if (st != TL_OK) return st;
  if (c->mode == TL_CACHE_H_DELTA8 || c->order != TL_ATTN_EXPLICIT)
    return fail(TL_E_UNSUPPORTED, "the static-scratch step covers the explicit order of the K/V and h modes "
                                  "other than delta-KV");
  // the step scratch of this call: rows, activations, logits, attention
  // partials (splits of the longest context), tile counters
  const tl_config& cfg = c->m->cfg;
  const size_t D = cfg.d_model, F = cfg.d_mlp, V = cfg.vocab, es = dtype_size(cfg.dtype);
  const int min_split = c->mode == TL_CACHE_KV ? kKvSplit : 64;
  const int S = (t_ub + min_split - 1) / min_split;
  const size_t sizes[14] = {
      (size_t)n * 4, (size_t)n * 4, (size_t)n * 4, (size_t)n * 4,   // row_lane, row_slot, row_pos, row_dead
      (size_t)n * D * 4, (size_t)n * D * es, (size_t)n * D * 4,      // x, h, q
      (size_t)n * D * es, (size_t)n * D * es, (size_t)n * F * es,    // o, u, a
      (size_t)n * D * es, (size_t)n * V * 4,                         // z, logits
      (size_t)n * cfg.n_heads * S * (cfg.d_head + 2) * 4,            // part
      (size_t)n * (2 * D / 128) * 4,                                 // tilecnt
  };
  size_t off[14], total = 0;
  for (int i = 0; i < 14; ++i) {
    off[i] = total;
    total = align256(total + sizes[i]);
  }
  if (total > kStaticScratchBytes)
    return fail(TL_E_CAPACITY, "the step needs %zu bytes of static scratch (%d lanes, context %d); the limit is %zu",
                total, n, t_ub, kStaticScratchBytes);
  char* base = nullptr;
  st = static_scratch(&base);
  if (st != TL_OK) return st;
  Workspace w = c->ws;   // per-lane state stays in the cache's workspace
  w.row_lane = (int32_t*)(base + off[0]);
  w.row_slot = (int32_t*)(base + off[1]);
  w.row_pos = (int32_t*)(base + off[2]);
  w.row_dead = (int32_t*)(base + off[3]);
  w.x = (float*)(base + off[4]);
  w.h = base + off[5];
  w.q = (float*)(base + off[6]);
  w.o = base + off[7];
  w.u = base + off[8];
  w.a = base + off[9];
  w.z = base + off[10];
  w.logits = (float*)(base + off[11]);
  w.part = (float*)(base + off[12]);
  w.tilecnt = (int32_t*)(base + off[13]);
  w.S = S;
  w.R = n;
  w.Bmax = n;
  w.kvbuf = nullptr; w.ppart = nullptr; w.ppart_floats = 0; w.spec = nullptr;
  w.hrec = nullptr; w.hmat = nullptr; w.qt = nullptr; w.apart = nullptr; w.apair_cap = 0;
  // the array keeps the last call's contents: the attention's tile counters
  // must start at zero (a fill kernel, so the call can be captured in a graph)
  TL_HIP(launch_fill_i32(w.tilecnt, n * (int)(2 * D / 128), 0, (hipStream_t)stream));
  return decode_enqueue(c, w, n, lanes, loops, d_tokens_in, safety_threshold, d_tokens_out, d_logits,
                        d_lane_status, stream, lmax_call, t_ub);
}

tl_status tl_spec_step(tl_cache* c, int lane, int draft_loops, int verify_loops, int draft_ahead,
                       const int32_t* d_token_in, int32_t* d_tokens_out, int* n_out, void* stream) {
  tl_status st = check_lane(c, lane);
  if (st != TL_OK) return st;
  if (!d_token_in || !d_tokens_out || !n_out) return fail(TL_E_ARG, "null argument");
  *n_out = 0;
  if (c->ext_next[lane] >= 0) return fail(TL_E_ARG, "lane %d: a depth extension is in progress", lane);
  if (draft_ahead < 1 || draft_ahead > kSpecMax)
    return fail(TL_E_ARG, "draft_ahead %d not in [1, %d]", draft_ahead, kSpecMax);
  if (draft_loops < 1 || draft_loops > verify_loops || verify_loops > c->l_max)
    return fail(TL_E_ARG, "need 1 <= draft_loops (%d) <= verify_loops (%d) <= %d", draft_loops,
                verify_loops, c->l_max);
  const ModelView& mv = c->m->mv;
  const int pos0 = c->host_len[lane], valid = c->layers_valid[lane];
  const int n = draft_ahead + 1;
  if (pos0 + n > c->max_seq) return fail(TL_E_CAPACITY, "lane %d: %d + %d positions exceed %d", lane, pos0, n, c->max_seq);
  if (pos0 > 0 && mv.n_pre + verify_loops > valid)
    return fail(TL_E_CACHE_GAP, "lane %d: layers %d.. miss earlier positions", lane, valid);
  hipStream_t s = (hipStream_t)stream;
  const Workspace& ws = c->ws;
  int32_t* chunk = ws.spec;   // the round's input token, then the drafts
  TL_HIP(hipMemcpyAsync(chunk, d_token_in, sizeof(int32_t), hipMemcpyDeviceToDevice, s));
  // drafts: greedy decode steps at the shallow depth, each fed the previous
  // draft; they append positions pos0 .. pos0+k-1 in the first
  // n_pre + draft_loops layers, which the verification rewrites identically
  for (int j = 0; j < draft_ahead; ++j) {
    st = tl_decode_step(c, 1, &lane, &draft_loops, chunk + j, INFINITY, chunk + j + 1, nullptr,
                        ws.spec + 2 * kSpecRows + 1, stream);
    if (st != TL_OK) {
      c->host_len[lane] = pos0;
      c->layers_valid[lane] = valid;
      return st;
    }
  }
  // verification: the input token and the drafts as one chunk at the full
  // depth from pos0, every row's greedy token, the acceptance and the lane's
  // new length
  st = run_chunk(c, lane, pos0, n, 0, mv.n_pre + verify_loops, chunk, nullptr, nullptr, pos0 + n,
                 nullptr, nullptr, s, d_tokens_out);
  c->host_len[lane] = pos0;
  c->layers_valid[lane] = valid;
  if (st != TL_OK) return st;
  int32_t got = 0;
  TL_HIP(hipMemcpyAsync(&got, ws.spec + 2 * kSpecRows, sizeof(int32_t), hipMemcpyDeviceToHost, s));
  TL_HIP(hipStreamSynchronize(s));
  if (got > 0) {
    const int nl = mv.n_pre + verify_loops;
    c->layers_valid[lane] = pos0 == 0 ? nl : std::min(valid, nl);
    c->host_len[lane] = pos0 + got;
  }
  *n_out = got;
  return TL_OK;
}

tl_status tl_cache_set_attention(tl_cache* c, int order) {
  if (!c) return fail(TL_E_ARG, "null cache");
  if (order != TL_ATTN_EXPLICIT && order != TL_ATTN_ABSORBED) return fail(TL_E_ARG, "unknown order %d", order);
  if (order == TL_ATTN_ABSORBED) {
    const int view = c->mode == TL_CACHE_H_DELTA8 ? TL_CACHE_H_F16 : c->mode;
    if (!c->ws.apair_cap || !absorbed_supported(c->m->mv, view))
      return fail(TL_E_UNSUPPORTED, "absorbed order covers fp16 models with 16 heads of 64 (d_model 1024) or 128 (2048), h caches");
  }
  c->order = order;
  return TL_OK;
}

tl_status tl_profile_start(tl_cache* c) {
  if (!c) return fail(TL_E_ARG, "null cache");
  c->prof_on = true;
  c->prof_used = 0;
  return TL_OK;
}

tl_status tl_profile_stop(tl_cache* c, double* total_ms, int* n_launches) {
  if (!c) return fail(TL_E_ARG, "null cache");
  c->prof_on = false;
  double tot = 0.0;
  if (c->prof_used) TL_HIP(hipEventSynchronize(c->prof_ev[c->prof_used - 1]));
  for (size_t i = 0; i + 1 < c->prof_used; i += 2) {
    float ms = 0.f;
    TL_HIP(hipEventElapsedTime(&ms, c->prof_ev[i], c->prof_ev[i + 1]));
    tot += ms;
  }
  if (total_ms) *total_ms = tot;
  if (n_launches) *n_launches = (int)(c->prof_used / 2);
  c->prof_used = 0;
  return TL_OK;
}

}  // extern "C"
