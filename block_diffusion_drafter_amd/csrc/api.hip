// C ABI of the drafter library: argument validation, workspace and
// packed-weight layouts, and the launch sequence of each call. No device
// memory is allocated here: scratch comes from the caller's workspace, the
// tiled weight copy from the caller's packed buffer.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "internal.h"

// Offsets (bytes) of the tiled projection weights inside the packed buffer.
struct PackedLayout {
  size_t qkv[dflash::kMaxLayers], wo[dflash::kMaxLayers], gate[dflash::kMaxLayers];
  size_t up[dflash::kMaxLayers], down[dflash::kMaxLayers];
  size_t fc, kv, lm, total;
};

struct dflash_handle {
  dflash_config cfg;
  dflash_weights w;
  std::vector<dflash_layer_weights> layers;
  PackedLayout pl;
};

namespace dflash {

// ---------------------------------------------------------------------------
// Kernel timing: HIP events bracket every launch while enabled.
// ---------------------------------------------------------------------------
struct ProfRec {
  int kind;
  double bytes, flops;
  hipEvent_t e0, e1;
  bool closed;
};
static std::vector<ProfRec> g_rec;
static std::vector<hipEvent_t> g_pool;
static size_t g_pool_next = 0;
static bool g_prof_on = false;
static uint32_t g_prof_mask = 0xFFFFFFFFu;
static int g_open = -1;

void prof_begin(int kind, double bytes, double flops, hipStream_t st) {
  g_open = -1;
  if (!g_prof_on || !((g_prof_mask >> kind) & 1u) || g_pool_next + 2 > g_pool.size()) return;
  ProfRec r{kind, bytes, flops, g_pool[g_pool_next], g_pool[g_pool_next + 1], false};
  g_pool_next += 2;
  if (hipEventRecord(r.e0, st) != hipSuccess) return;
  g_rec.push_back(r);
  g_open = (int)g_rec.size() - 1;
}

void prof_end(hipStream_t st) {
  if (g_open < 0) return;
  if (hipEventRecord(g_rec[g_open].e1, st) == hipSuccess) g_rec[g_open].closed = true;
  g_open = -1;
}

}  // namespace dflash

using namespace dflash;

// A captured decoding round: the graph and its executable instance.
struct dflash_round_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {

inline int elem_size(int dtype) { return dtype == DFLASH_BF16 ? 2 : 4; }
inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

#define DF_HIP(expr)                         \
  do {                                       \
    if ((expr) != hipSuccess) return DFLASH_ERR_HIP; \
  } while (0)

// Tiled copies, in order: per layer [wq; wk; wv] (stacked rows), wo, w_gate,
// w_up, w_down; then fc; then every layer's [wk; wv] stacked (the context K/V
// projection of all layers in one GEMM); then the LM head.
PackedLayout packed_layout(const dflash_config& c) {
  PackedLayout p{};
  const int dt = c.dtype, d = c.hidden, hd = c.head_dim, I = c.intermediate;
  const int q_dim = c.n_heads * hd, kv_dim = c.n_kv_heads * hd;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  for (int l = 0; l < c.n_layers; ++l) {
    p.qkv[l] = take(tiled_bytes(dt, q_dim + 2 * kv_dim, d));
    p.wo[l] = take(tiled_bytes(dt, d, q_dim));
    p.gate[l] = take(tiled_bytes(dt, I, d));
    p.up[l] = take(tiled_bytes(dt, I, d));
    p.down[l] = take(tiled_bytes(dt, d, I));
  }
  p.fc = take(tiled_bytes(dt, d, c.n_target_feats * c.target_hidden));
  p.kv = take(tiled_bytes(dt, (int64_t)c.n_layers * 2 * kv_dim, d));
  p.lm = take(tiled_bytes(dt, c.vocab, d));
  p.total = off;
  return p;
}

// Whether caller rows (features, context rows) are first copied into the
// tiled layout: always for the MFMA kernel; on the weight-streaming kernel
// from two 16-row tiles up (bf16), where reading several row-major rows per
// wave costs as much as the weight stream itself (37 rows: 2.0 TB/s for the
// context K/V projection against 3.4 at 4 rows).
bool packs_rows(int dtype, int M, int K) {
  return gemm_uses_mfma(dtype, M, K, true) || (dtype == DFLASH_BF16 && M > 16);
}

struct Plan {
  size_t x, h, qkv, q, po, pml, attn, act, y, amax, arr, part, sq, fwd_end;
  size_t u, ua, upart, proj_end;  // ua: tiled copy of the fused features (MFMA path)
  size_t kv, ca, kvpart, lens, app_end;  // ca: tiled copy of the context rows (MFMA path);
                                         // lens: ctx_len snapshot [batch]
  int64_t part_elems, upart_elems, kvpart_elems;  // split-K partials (floats)
  int attn_wg, n_vtiles;  // attention workgroups per KV head; LM-head keys per row
  size_t total;
};

// Attention split: each KV head's keys (all sequences, end to end) are cut
// into equal ranges over up to 512 / Hkv workgroups, one round over the chip
// at 2 workgroups of a KV group per CU, each range at least 2 blocks of 32
// keys; the device sizes the split from ctx_len, the host only bounds it.
// (Per-sequence chunks left a ragged batch with a part-filled last round:
// batch 32 at 512-8192 keys ran 1.6 rounds of 1024-key chunks.)
constexpr int kAttnSlots = 512;
constexpr int kAttnMinBlocks = 2;
int attn_wg_per_head(int hkv) { return std::max(1, kAttnSlots / std::max(1, hkv)); }

// Floats of split-K partials a tiled-A projection needs on the MFMA path (0 if none).
int64_t splitk_elems(int dtype, int epi, int M, int N, int K) {
  if (!gemm_uses_mfma(dtype, M, K, true, epi)) return 0;
  const int ks = mfma_gemm_ksplit(epi, M, N, K);
  return ks > 1 ? (int64_t)ks * M * N : 0;
}

// The same for a call of any row count up to Mmax (the plan's split is not
// monotone in M): the bound every K split of the MFMA path stays within.
int64_t splitk_elems_upto(int dtype, int M, int N, int K) {
  if (!gemm_uses_mfma(dtype, M, K, true)) return 0;
  return kMfmaMaxSplit * std::min<int64_t>((int64_t)M * N, kMfmaSplitMaxElems);
}

Plan make_plan(const dflash_config& c, int batch, int cap, int max_tokens) {
  Plan p{};
  const size_t es = elem_size(c.dtype);
  const size_t B = c.block_size, M = (size_t)batch * B, d = c.hidden, hd = c.head_dim;
  const size_t Hq = c.n_heads, Hkv = c.n_kv_heads, G = Hq / Hkv, I = c.intermediate;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const int dt = c.dtype;
  p.x = take(M * d * 4);
  p.h = take(tiled_bytes(dt, (int64_t)M, (int)d));
  p.qkv = take(M * (Hq + 2 * Hkv) * hd * 4);
  p.q = take((size_t)batch * Hq * 16 * hd * es);
  p.attn_wg = attn_wg_per_head((int)Hkv);
  // one partial entry per (KV head, workgroup or sequence boundary)
  const size_t entries = Hkv * (size_t)(p.attn_wg + batch);
  p.po = take(entries * G * hd * 16 * 4);
  p.pml = take(entries * G * 16 * 2 * 4);
  p.attn = take(tiled_bytes(dt, (int64_t)M, (int)(Hq * hd)));
  p.act = take(tiled_bytes(dt, (int64_t)M, (int)I));
  const size_t R = (size_t)batch * (B - 1);
  p.y = take(tiled_bytes(dt, (int64_t)R, (int)d));
  // LM head: one (max, argmax) key per row and workgroup column.
  p.n_vtiles = R > 0 ? gemm_amax_cols(c.dtype, (int)R, c.vocab, c.hidden) : 1;
  p.amax = take(R * p.n_vtiles * 8);
  p.arr = take((size_t)batch * 4);
  {
    const int Mi = (int)M, Nqkv = (int)((Hq + 2 * Hkv) * hd), qd = (int)(Hq * hd);
    p.part_elems = std::max({splitk_elems(dt, EPI_STORE_F32, Mi, Nqkv, (int)d),
                             splitk_elems(dt, EPI_RESID, Mi, (int)d, qd),
                             splitk_elems(dt, EPI_RESID, Mi, (int)d, (int)I)});
    p.part = take((size_t)p.part_elems * 4);
  }
  // Per-tile row sums of squares of a deferred norm (weight-streaming path).
  p.sq = take((((d + 15) / 16 + 3) & ~(size_t)3) * M * 4);
  p.fwd_end = off;
  off = 0;
  p.u = take((size_t)max_tokens * d * 4);
  const int fk = c.n_target_feats * c.target_hidden;
  p.ua = packs_rows(dt, max_tokens, fk) ? take(tiled_bytes(dt, max_tokens, fk)) : 0;
  p.upart_elems = splitk_elems_upto(dt, max_tokens, (int)d, fk);
  p.upart = take((size_t)p.upart_elems * 4);
  p.proj_end = off;
  off = 0;
  p.kv = take((size_t)max_tokens * c.n_layers * 2 * Hkv * hd * 4);
  p.ca = packs_rows(dt, max_tokens, (int)d) ? take(tiled_bytes(dt, max_tokens, (int)d)) : 0;
  p.kvpart_elems = splitk_elems_upto(dt, max_tokens, (int)(c.n_layers * 2 * Hkv * hd), (int)d);
  p.kvpart = take((size_t)p.kvpart_elems * 4);
  p.lens = take((size_t)batch * 4);
  p.app_end = off;
  p.total = std::max(p.fwd_end, std::max(p.proj_end, p.app_end));
  return p;
}

int32_t check_config(const dflash_config& c) {
  if (c.dtype != DFLASH_BF16 && c.dtype != DFLASH_FP32) return DFLASH_ERR_DTYPE;
  const int mult = c.dtype == DFLASH_BF16 ? 32 : 16;
  if (c.hidden <= 0 || c.n_heads <= 0 || c.n_kv_heads <= 0 || c.intermediate <= 0 ||
      c.n_target_feats <= 0 || c.target_hidden <= 0 || c.vocab < 2 || c.n_layers <= 0)
    return DFLASH_ERR_SHAPE;
  if (c.n_heads % c.n_kv_heads) return DFLASH_ERR_SHAPE;
  const int G = c.n_heads / c.n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return DFLASH_ERR_UNSUPPORTED;
  if (c.head_dim != 64 && c.head_dim != 128) return DFLASH_ERR_UNSUPPORTED;
  if (c.block_size < 1 || c.block_size > 16) return DFLASH_ERR_UNSUPPORTED;
  if (c.n_layers > kMaxLayers) return DFLASH_ERR_UNSUPPORTED;
  if (c.sliding_layer_mask != 0u) {
    if (c.sliding_window < 1) return DFLASH_ERR_SHAPE;
    if (c.n_layers < 32 && (c.sliding_layer_mask >> c.n_layers) != 0u) return DFLASH_ERR_SHAPE;
  }
  if (c.n_target_feats > kMaxASeg) return DFLASH_ERR_UNSUPPORTED;
  if (c.hidden % mult || c.intermediate % mult || c.target_hidden % mult) return DFLASH_ERR_SHAPE;
  // Fused features are separate A segments; a 256-byte GEMM chunk must not straddle two.
  if (c.n_target_feats > 1 && c.target_hidden % (c.dtype == DFLASH_BF16 ? 128 : 64))
    return DFLASH_ERR_SHAPE;
  if (c.mask_token_id < 0 || c.mask_token_id >= c.vocab) return DFLASH_ERR_SHAPE;
  if (!(c.rms_eps >= 0.f) || !std::isfinite(c.rms_eps)) return DFLASH_ERR_SHAPE;
  if (!std::isfinite(c.rope_theta)) return DFLASH_ERR_SHAPE;
  return DFLASH_OK;
}

// A projection reading a tiled activation matrix a [M, K] from the workspace
// and the tiled weight w (w2: the up matrix of the SwiGLU pair).
GemmArgs gemm_tiled(const void* a, const void* w, int M, int N, int K, const void* w2 = nullptr) {
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.a[0] = a;
  g.a_nseg = 1;
  g.a_seg_k = K;
  g.a_tiled = 1;
  g.w = w;
  g.w2 = w2;
  g.M = M;
  g.N = N;
  g.K = K;
  return g;
}

// Asks a residual projection's K-slice reduce for the RMSNorm of its rows too.
void set_norm(GemmArgs& g, const void* gain, void* out, int nck, float eps) {
  g.norm_w = gain;
  g.norm_out = out;
  g.norm_nck = nck;
  g.norm_eps = eps;
}

// A projection whose tiled A rows hold x * gain of a deferred RMSNorm: it
// scales each output row by the norm's 1/rms (from the producer's per-tile
// sums of squares of the d-wide rows).
void take_norm(GemmArgs& g, const float* sq, int d, float eps) {
  g.sq_in = sq;
  g.sq_d = d;
  g.norm_eps = eps;
}

// Whether the norm between a residual projection of M rows (inner size K)
// and the next projection (inner size d) is deferred: both on the
// weight-streaming kernel with one 16-row tile (each consumer workgroup then
// reads only its 16 rows' d/16 partial sums, issued ahead of its weight
// stream); at more rows those reads cost more than the norm's own pass.
bool streams_both(int M, int K, int d) {
  return M <= 16 && !gemm_uses_mfma(DFLASH_BF16, M, K, true) &&
         !gemm_uses_mfma(DFLASH_BF16, M, d, true);
}

// A projection of caller-provided row-major rows (stride a_stride elements).
GemmArgs gemm_rows(const void* a, int64_t a_stride, const void* w, int M, int N, int K) {
  GemmArgs g = gemm_tiled(a, w, M, N, K);
  g.a_tiled = 0;
  g.a_stride = a_stride;
  return g;
}

int32_t run_gemm(int dtype, int epi, const GemmArgs& g, hipStream_t st) {
  const int kind = epi == EPI_STORE_F32 ? DFLASH_K_GEMM_F32OUT
                   : epi == EPI_RESID   ? DFLASH_K_GEMM_RESID
                   : epi == EPI_SWIGLU  ? DFLASH_K_GEMM_SWIGLU
                                        : DFLASH_K_LMHEAD;
  const double es = elem_size(dtype);
  const double nb = epi == EPI_SWIGLU ? 2.0 : 1.0;
  double out_bytes = 0;
  if (epi == EPI_STORE_F32) out_bytes = 4.0 * g.M * g.N;
  else if (epi == EPI_RESID) out_bytes = 8.0 * g.M * g.N;
  else if (epi == EPI_SWIGLU) out_bytes = es * g.M * g.N;
  else out_bytes = 8.0 * g.M * ((g.N + 15) / 16);
  const double bytes = nb * es * g.N * g.K + es * g.M * g.K + out_bytes;
  const double flops = 2.0 * nb * g.M * g.N * g.K;
  prof_begin(kind, bytes, flops, st);
  const hipError_t e = launch_gemm(dtype, epi, g, st);
  prof_end(st);
  return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

int32_t check_cache(const dflash_handle* h, const dflash_kv_cache* c) {
  if (!c || !c->k || !c->v || !c->ctx_len) return DFLASH_ERR_NULL;
  if (!al16(c->k) || !al16(c->v)) return DFLASH_ERR_ALIGN;
  if (c->batch <= 0 || c->capacity <= 0 || c->capacity % kKeyBlock) return DFLASH_ERR_SHAPE;
  if (c->capacity < h->cfg.block_size) return DFLASH_ERR_SHAPE;
  return DFLASH_OK;
}

}  // namespace

extern "C" {

const char* dflash_status_string(int32_t code) {
  switch (code) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_NULL: return "a required pointer is NULL";
    case DFLASH_ERR_SHAPE: return "a size is out of range or inconsistent";
    case DFLASH_ERR_DTYPE: return "unknown dtype";
    case DFLASH_ERR_ALIGN: return "a pointer or stride is not 16-byte aligned";
    case DFLASH_ERR_WORKSPACE: return "workspace or packed buffer is smaller than its size query";
    case DFLASH_ERR_UNSUPPORTED: return "configuration not covered by the kernels";
    case DFLASH_ERR_HIP: return "a HIP launch reported an error";
    case DFLASH_ERR_STATE: return "profiler misuse, or graph capture while the profiler records";
    case DFLASH_ERR_SCRATCH: return "request exceeds the library's static scratch";
    default: return "unknown status";
  }
}

int64_t dflash_packed_weight_bytes(const dflash_config* cfg) {
  if (!cfg) return DFLASH_ERR_NULL;
  const int32_t rc = check_config(*cfg);
  if (rc) return rc;
  return (int64_t)packed_layout(*cfg).total;
}

int32_t dflash_pack_weights(const dflash_config* cfg, const dflash_weights* w, void* packed,
                            int64_t packed_bytes, void* stream) {
  if (!cfg || !w) return DFLASH_ERR_NULL;
  int32_t rc = check_config(*cfg);
  if (rc) return rc;
  if (!w->lm_head || !w->fc || !w->layers || !packed) return DFLASH_ERR_NULL;
  if (!al16(w->lm_head) || !al16(w->fc) || !al16(packed)) return DFLASH_ERR_ALIGN;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dflash_layer_weights& lw = w->layers[l];
    const void* ps[] = {lw.wq, lw.wk, lw.wv, lw.wo, lw.w_gate, lw.w_up, lw.w_down};
    for (const void* q : ps) {
      if (!q) return DFLASH_ERR_NULL;
      if (!al16(q)) return DFLASH_ERR_ALIGN;
    }
  }
  const PackedLayout pl = packed_layout(*cfg);
  if (packed_bytes < (int64_t)pl.total) return DFLASH_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int dt = cfg->dtype, d = cfg->hidden, I = cfg->intermediate;
  const int q_dim = cfg->n_heads * cfg->head_dim, kv_dim = cfg->n_kv_heads * cfg->head_dim;
  char* base = (char*)packed;
  // Stacked matrices: each part starts on a 16-row tile boundary (q_dim and
  // kv_dim are multiples of 16), so a part is packed at its rows' byte offset.
  auto pack = [&](const void* src, int rows, int K, size_t off, int64_t row0) {
    return launch_pack_tiled(dt, pack_src(src, K), rows, K, base + off + tiled_bytes(dt, row0, K),
                             st) == hipSuccess;
  };
  bool ok = true;
  for (int l = 0; l < cfg->n_layers && ok; ++l) {
    const dflash_layer_weights& lw = w->layers[l];
    ok = pack(lw.wq, q_dim, d, pl.qkv[l], 0) && pack(lw.wk, kv_dim, d, pl.qkv[l], q_dim) &&
         pack(lw.wv, kv_dim, d, pl.qkv[l], q_dim + kv_dim) && pack(lw.wo, d, q_dim, pl.wo[l], 0) &&
         pack(lw.w_gate, I, d, pl.gate[l], 0) && pack(lw.w_up, I, d, pl.up[l], 0) &&
         pack(lw.w_down, d, I, pl.down[l], 0) &&
         pack(lw.wk, kv_dim, d, pl.kv, (int64_t)(2 * l) * kv_dim) &&
         pack(lw.wv, kv_dim, d, pl.kv, (int64_t)(2 * l + 1) * kv_dim);
  }
  ok = ok && pack(w->fc, d, cfg->n_target_feats * cfg->target_hidden, pl.fc, 0) &&
       pack(w->lm_head, cfg->vocab, d, pl.lm, 0);
  return ok ? DFLASH_OK : DFLASH_ERR_HIP;
}

int32_t dflash_create(const dflash_config* cfg, const dflash_weights* w, dflash_handle** out) {
  if (!out) return DFLASH_ERR_NULL;
  *out = nullptr;
  if (!cfg || !w) return DFLASH_ERR_NULL;
  int32_t rc = check_config(*cfg);
  if (rc) return rc;
  if (!w->embed || !w->fc_norm || !w->final_norm || !w->layers || !w->packed)
    return DFLASH_ERR_NULL;
  const void* top[] = {w->embed, w->fc_norm, w->final_norm, w->packed};
  for (const void* p : top)
    if (!al16(p)) return DFLASH_ERR_ALIGN;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dflash_layer_weights& lw = w->layers[l];
    const void* ps[] = {lw.in_norm, lw.q_norm, lw.k_norm, lw.post_norm};
    for (const void* p : ps) {
      if (!p) return DFLASH_ERR_NULL;
      if (!al16(p)) return DFLASH_ERR_ALIGN;
    }
  }
  const PackedLayout pl = packed_layout(*cfg);
  if (w->packed_bytes < (int64_t)pl.total) return DFLASH_ERR_WORKSPACE;
  dflash_handle* hd = new (std::nothrow) dflash_handle;
  if (!hd) return DFLASH_ERR_SHAPE;
  hd->cfg = *cfg;
  hd->w = *w;
  hd->layers.assign(w->layers, w->layers + cfg->n_layers);
  hd->w.layers = hd->layers.data();
  hd->pl = pl;
  *out = hd;
  return DFLASH_OK;
}

void dflash_destroy(dflash_handle* h) { delete h; }

int64_t dflash_workspace_bytes(const dflash_handle* h, int32_t max_batch, int32_t capacity,
                               int32_t max_tokens) {
  if (!h) return DFLASH_ERR_NULL;
  if (max_batch < 1 || capacity < 1 || max_tokens < 0) return DFLASH_ERR_SHAPE;
  size_t best = 0;
  for (int b = 1; b <= max_batch; ++b)
    best = std::max(best, make_plan(h->cfg, b, capacity, max_tokens).total);
  return (int64_t)best;
}

int32_t dflash_ctx_project(const dflash_handle* h, const void* const* feats,
                           int64_t feat_row_stride, int32_t n_tok, void* ctx_out, void* ws,
                           int64_t ws_bytes, void* stream) {
  if (!h) return DFLASH_ERR_NULL;
  const dflash_config& c = h->cfg;
  if (n_tok < 0) return DFLASH_ERR_SHAPE;
  if (n_tok == 0) return DFLASH_OK;
  if (!feats || !ctx_out || !ws) return DFLASH_ERR_NULL;
  if (feat_row_stride < c.target_hidden || feat_row_stride % 8) return DFLASH_ERR_SHAPE;
  for (int f = 0; f < c.n_target_feats; ++f) {
    if (!feats[f]) return DFLASH_ERR_NULL;
    if (!al16(feats[f])) return DFLASH_ERR_ALIGN;
  }
  if (!al16(ctx_out) || !al16(ws)) return DFLASH_ERR_ALIGN;
  const Plan P = make_plan(c, 1, kKeyBlock, n_tok);
  if (ws_bytes < (int64_t)P.proj_end) return DFLASH_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  float* u = reinterpret_cast<float*>((char*)ws + P.u);
  const char* pk = (const char*)h->w.packed;
  const int K = c.n_target_feats * c.target_hidden;
  GemmArgs g;
  if (packs_rows(c.dtype, n_tok, K)) {
    // Tile the features first (MFMA kernel, or several row tiles).
    PackSrc src{};
    for (int f = 0; f < c.n_target_feats; ++f) src.seg[f] = feats[f];
    src.nseg = c.n_target_feats;
    src.seg_k = c.target_hidden;
    src.row_stride = feat_row_stride;
    void* at = (char*)ws + P.ua;
    prof_begin(DFLASH_K_SMALL, 0, 0, st);
    const hipError_t pe = launch_pack_tiled(c.dtype, src, n_tok, K, at, st);
    prof_end(st);
    if (pe != hipSuccess) return DFLASH_ERR_HIP;
    g = gemm_tiled(at, pk + h->pl.fc, n_tok, c.hidden, K);
    g.part = reinterpret_cast<float*>((char*)ws + P.upart);
    g.part_elems = P.upart_elems;
  } else {
    g = gemm_rows(nullptr, feat_row_stride, pk + h->pl.fc, n_tok, c.hidden, K);
    for (int f = 0; f < c.n_target_feats; ++f) g.a[f] = feats[f];
    g.a_nseg = c.n_target_feats;
    g.a_seg_k = c.target_hidden;
  }
  g.out = u;
  g.out_stride = c.hidden;
  // Split over K on the MFMA path: the slice reduce writes the normalised
  // rows straight to ctx_out (no fp32 rows, no separate norm pass).
  const bool fused = gemm_fuses_norm(c.dtype, g, EPI_STORE_F32);
  if (fused) set_norm(g, h->w.fc_norm, ctx_out, 0, c.rms_eps);
  int32_t rc = run_gemm(c.dtype, EPI_STORE_F32, g, st);
  if (rc || fused) return rc;
  prof_begin(DFLASH_K_RMSNORM, 0, 0, st);
  hipError_t e = launch_rmsnorm(c.dtype, u, c.hidden, h->w.fc_norm, ctx_out, c.hidden, 0, n_tok,
                                c.hidden, c.rms_eps, n_tok, 0, 0, st);
  prof_end(st);
  return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

// Context K/V injection of n_tok rows; a row's sequence and position come from
// the prefix offsets cu_new, or, when accept_len is given, from the block
// layout (row s*B + i, kept for i <= accept_len[s]).
static int32_t append_rows(const dflash_handle* h, const dflash_kv_cache* cache, const void* ctx,
                           const int32_t* cu_new, const int32_t* accept_len, int32_t n_tok,
                           int32_t* dev_status, void* ws, int64_t ws_bytes, void* stream) {
  const dflash_config& c = h->cfg;
  int32_t rc = check_cache(h, cache);
  if (rc) return rc;
  if (n_tok < 0) return DFLASH_ERR_SHAPE;
  if (!cu_new && !accept_len) return DFLASH_ERR_NULL;
  if (n_tok > 0 && (!ctx || !ws)) return DFLASH_ERR_NULL;
  if ((ctx && !al16(ctx)) || (ws && !al16(ws))) return DFLASH_ERR_ALIGN;
  const Plan P = make_plan(c, cache->batch, cache->capacity, n_tok);
  if (n_tok > 0 && ws_bytes < (int64_t)P.app_end) return DFLASH_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int Hkv = c.n_kv_heads, hd = c.head_dim, L = c.n_layers;
  if (n_tok > 0) {
    float* kv = reinterpret_cast<float*>((char*)ws + P.kv);
    const int N = L * 2 * Hkv * hd;
    const char* wkv = (const char*)h->w.packed + h->pl.kv;
    GemmArgs g;
    if (packs_rows(c.dtype, n_tok, c.hidden)) {
      void* at = (char*)ws + P.ca;
      prof_begin(DFLASH_K_SMALL, 0, 0, st);
      const hipError_t pe = launch_pack_tiled(c.dtype, pack_src(ctx, c.hidden), n_tok, c.hidden, at, st);
      prof_end(st);
      if (pe != hipSuccess) return DFLASH_ERR_HIP;
      g = gemm_tiled(at, wkv, n_tok, N, c.hidden);
      g.part = reinterpret_cast<float*>((char*)ws + P.kvpart);
      g.part_elems = P.kvpart_elems;
    } else {
      g = gemm_rows(ctx, c.hidden, wkv, n_tok, N, c.hidden);
    }
    g.out = kv;
    g.out_stride = N;
    // The projection snapshots ctx_len; the scatter reads the rows' positions
    // from the snapshot and updates ctx_len itself (no third launch).
    int32_t* lens = reinterpret_cast<int32_t*>((char*)ws + P.lens);
    g.snap_src = cache->ctx_len;
    g.snap_dst = lens;
    g.snap_n = cache->batch;
    // Split over K: the append kernel sums the slices' partials itself.
    g.defer_reduce = 1;
    const int slices = gemm_store_slices(c.dtype, g);
    rc = run_gemm(c.dtype, EPI_STORE_F32, g, st);
    if (rc) return rc;
    NormRopeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.src = slices > 1 ? g.part : kv;
    a.src_stride = N;
    a.src_slices = slices;
    a.slice_stride = (int64_t)n_tok * N;
    a.k_cache = cache->k;
    a.v_cache = cache->v;
    for (int l = 0; l < L; ++l) a.k_norm[l] = h->layers[l].k_norm;
    a.ctx_len = lens;
    a.ctx_len_out = cache->ctx_len;
    a.cu_new = cu_new;
    a.accept_len = accept_len;
    a.dev_status = dev_status;
    a.batch = cache->batch;
    a.cache_batch = cache->batch;
    a.n_heads = c.n_heads;
    a.n_kv_heads = Hkv;
    a.head_dim = hd;
    a.block = c.block_size;
    a.cap = cache->capacity;
    a.n_layers = L;
    a.n_tok = n_tok;
    a.eps = c.rms_eps;
    a.rope_theta = c.rope_theta;
    prof_begin(DFLASH_K_NORM_ROPE, 0, 0, st);
    hipError_t e = launch_norm_rope_append(c.dtype, a, st);
    prof_end(st);
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
  }
  // No rows: only the length bookkeeping (and the offset checks).
  prof_begin(DFLASH_K_SMALL, 0, 0, st);
  hipError_t e = launch_ctx_len_add(cache->ctx_len, cu_new, accept_len, c.block_size,
                                    cache->batch, n_tok, cache->capacity, dev_status, st);
  prof_end(st);
  return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

int32_t dflash_ctx_kv_append(const dflash_handle* h, const dflash_kv_cache* cache, const void* ctx,
                             const int32_t* cu_new, int32_t n_tok, int32_t* dev_status, void* ws,
                             int64_t ws_bytes, void* stream) {
  if (!h) return DFLASH_ERR_NULL;
  if (!cu_new) return DFLASH_ERR_NULL;
  return append_rows(h, cache, ctx, cu_new, nullptr, n_tok, dev_status, ws, ws_bytes, stream);
}

int32_t dflash_ctx_kv_append_accepted(const dflash_handle* h, const dflash_kv_cache* cache,
                                      const void* ctx, const int32_t* accept_len,
                                      int32_t* dev_status, void* ws, int64_t ws_bytes,
                                      void* stream) {
  if (!h || !cache) return DFLASH_ERR_NULL;
  if (!accept_len) return DFLASH_ERR_NULL;
  if (!al16(accept_len)) return DFLASH_ERR_ALIGN;
  if (cache->batch < 0 || (int64_t)cache->batch * h->cfg.block_size > INT32_MAX)
    return DFLASH_ERR_SHAPE;
  return append_rows(h, cache, ctx, nullptr, accept_len, cache->batch * h->cfg.block_size,
                     dev_status, ws, ws_bytes, stream);
}

int32_t dflash_draft_forward(const dflash_handle* h, const dflash_kv_cache* cache,
                             const int32_t* anchor, int32_t batch, int32_t* draft_tokens,
                             float* logits, float* hidden_out, const int32_t* target_tokens,
                             int32_t* accept_len, int32_t* bonus, int32_t* dev_status, void* ws,
                             int64_t ws_bytes, void* stream) {
  if (!h) return DFLASH_ERR_NULL;
  const dflash_config& c = h->cfg;
  int32_t rc = check_cache(h, cache);
  if (rc) return rc;
  if (batch < 1 || batch > cache->batch) return DFLASH_ERR_SHAPE;
  const int B = c.block_size;
  if (!anchor || !ws) return DFLASH_ERR_NULL;
  if (B > 1 && !draft_tokens) return DFLASH_ERR_NULL;
  if (target_tokens && (!accept_len || !bonus)) return DFLASH_ERR_NULL;
  if (!al16(ws) || (logits && !al16(logits)) || (hidden_out && !al16(hidden_out)))
    return DFLASH_ERR_ALIGN;
  const int cap = cache->capacity;
  const Plan P = make_plan(c, batch, cap, 0);
  if (ws_bytes < (int64_t)P.fwd_end) return DFLASH_ERR_WORKSPACE;

  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;
  float* x = reinterpret_cast<float*>(w + P.x);
  void* hbuf = w + P.h;
  float* qkv = reinterpret_cast<float*>(w + P.qkv);
  void* qbuf = w + P.q;
  void* attn = w + P.attn;
  void* act = w + P.act;
  void* ybuf = w + P.y;
  unsigned long long* amax = reinterpret_cast<unsigned long long*>(w + P.amax);

  const int es = elem_size(c.dtype);
  const int d = c.hidden, hd = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads, I = c.intermediate;
  const int M = batch * B, L = c.n_layers;
  const size_t layer_elems = (size_t)cache->batch * Hkv * cap * hd;
  const int nck_d = tiled_nck(c.dtype, d);
  const char* pk = (const char*)h->w.packed;
  const PackedLayout& pl = h->pl;

  prof_begin(DFLASH_K_SMALL, 0, 0, st);
  int32_t* arrivals = reinterpret_cast<int32_t*>(w + P.arr);
  hipError_t e = launch_embed(c.dtype, h->w.embed, anchor, batch, B, d, c.vocab, c.mask_token_id,
                              x, h->layers[0].in_norm, c.rms_eps, hbuf, dev_status, arrivals, st);
  prof_end(st);
  if (e != hipSuccess) return DFLASH_ERR_HIP;

  // The pre-norm of layer 0 came with the embedding; a later layer's comes
  // with the previous down projection: written normalised when that one
  // reduces K slices (MFMA path), or deferred on the weight-streaming path
  // (the down projection writes x * gain and the rows' sums of squares, the
  // QKV projection scales its rows).
  float* sq = reinterpret_cast<float*>(w + P.sq);
  const bool bf = c.dtype == DFLASH_BF16;
  enum { kNormNone, kNormDone, kNormDeferred };
  int pre_norm = kNormDone;
  bool final_fused = false;  // the final norm written by the last slice reduce
  for (int l = 0; l < L; ++l) {
    const dflash_layer_weights& lw = h->layers[l];
    if (pre_norm == kNormNone) {
      prof_begin(DFLASH_K_RMSNORM, 0, 0, st);
      e = launch_rmsnorm(c.dtype, x, d, lw.in_norm, hbuf, 0, nck_d, M, d, c.rms_eps, M, 0, 0, st);
      prof_end(st);
      if (e != hipSuccess) return DFLASH_ERR_HIP;
    }

    const int Nqkv = (Hq + 2 * Hkv) * hd;
    float* part = reinterpret_cast<float*>(w + P.part);
    GemmArgs g = gemm_tiled(hbuf, pk + pl.qkv[l], M, Nqkv, d);
    g.part = part;
    g.part_elems = P.part_elems;
    g.out = qkv;
    g.out_stride = Nqkv;
    if (pre_norm == kNormDeferred) take_norm(g, sq, d, c.rms_eps);
    if ((rc = run_gemm(c.dtype, EPI_STORE_F32, g, st))) return rc;

    NormRopeArgs nr;
    std::memset(&nr, 0, sizeof(nr));
    nr.src = qkv;
    nr.src_stride = Nqkv;
    nr.q_out = qbuf;
    nr.k_cache = (char*)cache->k + layer_elems * es * l;
    nr.v_cache = (char*)cache->v + layer_elems * es * l;
    nr.q_norm[0] = lw.q_norm;
    nr.k_norm[0] = lw.k_norm;
    nr.ctx_len = cache->ctx_len;
    nr.dev_status = dev_status;
    nr.batch = batch;
    nr.cache_batch = cache->batch;
    nr.n_heads = Hq;
    nr.n_kv_heads = Hkv;
    nr.head_dim = hd;
    nr.block = B;
    nr.cap = cap;
    nr.n_layers = 1;
    nr.eps = c.rms_eps;
    nr.rope_theta = c.rope_theta;
    prof_begin(DFLASH_K_NORM_ROPE, 0, 0, st);
    e = launch_norm_rope_forward(c.dtype, nr, st);
    prof_end(st);
    if (e != hipSuccess) return DFLASH_ERR_HIP;

    AttnArgs at;
    std::memset(&at, 0, sizeof(at));
    at.q = qbuf;
    at.k = nr.k_cache;
    at.v = nr.v_cache;
    at.ctx_len = cache->ctx_len;
    at.batch = batch;
    at.n_heads = Hq;
    at.n_kv_heads = Hkv;
    at.head_dim = hd;
    at.block = B;
    at.cap = cap;
    at.window = ((c.sliding_layer_mask >> l) & 1u) ? c.sliding_window : 0;
    at.wg_per_head = P.attn_wg;
    at.min_blocks = kAttnMinBlocks;
    at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)hd));
    at.part_o = reinterpret_cast<float*>(w + P.po);
    at.part_ml = reinterpret_cast<float*>(w + P.pml);
    at.out = attn;
    at.out_nck = tiled_nck(c.dtype, Hq * hd);
    prof_begin(DFLASH_K_ATTN, 0, 0, st);
    e = launch_attention(c.dtype, at, st);
    prof_end(st);
    if (e != hipSuccess) return DFLASH_ERR_HIP;

    g = gemm_tiled(attn, pk + pl.wo[l], M, d, Hq * hd);
    g.part = part;
    g.part_elems = P.part_elems;
    g.resid = x;
    g.out_stride = d;
    const bool post_fused = gemm_fuses_norm(c.dtype, g);
    const bool post_deferred = !post_fused && bf && streams_both(M, Hq * hd, d);
    if (post_fused || post_deferred) set_norm(g, lw.post_norm, hbuf, nck_d, c.rms_eps);
    if (post_deferred) g.sq_out = sq;
    if ((rc = run_gemm(c.dtype, EPI_RESID, g, st))) return rc;

    if (!post_fused && !post_deferred) {
      prof_begin(DFLASH_K_RMSNORM, 0, 0, st);
      e = launch_rmsnorm(c.dtype, x, d, lw.post_norm, hbuf, 0, nck_d, M, d, c.rms_eps, M, 0, 0, st);
      prof_end(st);
      if (e != hipSuccess) return DFLASH_ERR_HIP;
    }

    g = gemm_tiled(hbuf, pk + pl.gate[l], M, I, d, pk + pl.up[l]);
    g.out = act;
    if (post_deferred) take_norm(g, sq, d, c.rms_eps);
    if ((rc = run_gemm(c.dtype, EPI_SWIGLU, g, st))) return rc;

    g = gemm_tiled(act, pk + pl.down[l], M, d, I);
    g.part = part;
    g.part_elems = P.part_elems;
    g.resid = x;
    g.out_stride = d;
    pre_norm = kNormNone;
    if (l + 1 < L) {
      if (gemm_fuses_norm(c.dtype, g)) pre_norm = kNormDone;
      else if (bf && streams_both(M, I, d)) pre_norm = kNormDeferred;
    }
    if (pre_norm != kNormNone) set_norm(g, h->layers[l + 1].in_norm, hbuf, nck_d, c.rms_eps);
    if (pre_norm == kNormDeferred) g.sq_out = sq;
    // The last layer's slice reduce also writes the final norm of the slots
    // after each anchor (the LM head's rows).
    if (l + 1 == L && B > 1 && gemm_fuses_norm(c.dtype, g)) {
      set_norm(g, h->w.final_norm, ybuf, nck_d, c.rms_eps);
      g.norm_block = B;
      final_fused = true;
    }
    if ((rc = run_gemm(c.dtype, EPI_RESID, g, st))) return rc;

    if (hidden_out) {
      DF_HIP(hipMemcpy2DAsync(hidden_out + (size_t)l * B * d, (size_t)L * B * d * 4, x,
                              (size_t)B * d * 4, (size_t)B * d * 4, batch,
                              hipMemcpyDeviceToDevice, st));
    }
  }

  const int R = batch * (B - 1);
  if (R > 0) {
    if (!final_fused) {
      prof_begin(DFLASH_K_RMSNORM, 0, 0, st);
      e = launch_rmsnorm(c.dtype, x, d, h->w.final_norm, ybuf, 0, nck_d, R, d, c.rms_eps, B - 1,
                         B, 1, st);
      prof_end(st);
      if (e != hipSuccess) return DFLASH_ERR_HIP;
    }
    GemmArgs g = gemm_tiled(ybuf, pk + pl.lm, R, c.vocab, d);
    g.amax = amax;
    g.amax_stride = P.n_vtiles;
    g.logits = logits;
    g.logits_stride = c.vocab;
    if ((rc = run_gemm(c.dtype, EPI_ARGMAX, g, st))) return rc;
    prof_begin(DFLASH_K_SMALL, 0, 0, st);
    e = launch_argmax_accept(amax, P.n_vtiles, P.n_vtiles, batch, B, draft_tokens, target_tokens,
                             accept_len, bonus, arrivals, st);
    prof_end(st);
    if (e != hipSuccess) return DFLASH_ERR_HIP;
  } else if (target_tokens) {  // B == 1: nothing drafted, the bonus is the first target
    prof_begin(DFLASH_K_SMALL, 0, 0, st);
    e = launch_accept(draft_tokens, target_tokens, batch, B, accept_len, bonus, nullptr, st);
    prof_end(st);
    if (e != hipSuccess) return DFLASH_ERR_HIP;
  }
  return DFLASH_OK;
}

int64_t dflash_sampling_workspace_bytes(int32_t batch, int32_t block_size, int32_t vocab) {
  if (batch < 0 || block_size < 2 || block_size > 17 || vocab < 2) return DFLASH_ERR_SHAPE;
  const int b = std::max(batch, 1);
  return std::max(sample_ws_bytes(b * (block_size - 1), vocab), verify_ws_bytes(b, block_size, vocab));
}

int32_t dflash_sample_drafts(const float* logits, int64_t row_stride, int32_t rows, int32_t vocab,
                             float temperature, uint64_t seed, int32_t round, int32_t* tokens,
                             float* logq, void* ws, int64_t ws_bytes, void* stream) {
  if (rows < 0 || vocab < 2 || row_stride < vocab || !(temperature > 0.f) ||
      !std::isfinite(temperature))
    return DFLASH_ERR_SHAPE;
  if (rows == 0) return DFLASH_OK;
  if (!logits || !tokens || !ws) return DFLASH_ERR_NULL;
  if (!al16(logits) || !al16(tokens) || !al16(ws) || (logq && !al16(logq))) return DFLASH_ERR_ALIGN;
  if (ws_bytes < sample_ws_bytes(rows, vocab)) return DFLASH_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  prof_begin(DFLASH_K_SAMPLING, (double)rows * vocab * 4, 0.0, st);
  const hipError_t e = launch_sample_drafts(logits, row_stride, rows, vocab, temperature, seed,
                                            round, tokens, logq, ws, st);
  prof_end(st);
  return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

int32_t dflash_sample_drafts_static(const float* logits, int64_t row_stride, int32_t rows,
                                    int32_t vocab, float temperature, uint64_t seed,
                                    int32_t round, int32_t* tokens, float* logq, void* stream) {
  if (rows < 0 || vocab < 2 || row_stride < vocab || !(temperature > 0.f) ||
      !std::isfinite(temperature))
    return DFLASH_ERR_SHAPE;
  if (rows == 0) return DFLASH_OK;
  if (!logits || !tokens) return DFLASH_ERR_NULL;
  if (!al16(logits) || !al16(tokens) || (logq && !al16(logq))) return DFLASH_ERR_ALIGN;
  // The size check comes first: an oversized request touches no device state.
  if (sample_ws_bytes(rows, vocab) > sample_static_scratch_bytes()) return DFLASH_ERR_SCRATCH;
  void* scratch = nullptr;
  if (sample_static_scratch(&scratch) != hipSuccess) return DFLASH_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  prof_begin(DFLASH_K_SAMPLING, (double)rows * vocab * 4, 0.0, st);
  const hipError_t e = launch_sample_drafts(logits, row_stride, rows, vocab, temperature, seed,
                                            round, tokens, logq, scratch, st);
  prof_end(st);
  return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

int32_t dflash_verify_sampled(const int32_t* drafts, const float* draft_logits,
                              const float* draft_logq, const float* target_logits,
                              int32_t batch, int32_t block_size,
                              int32_t vocab, float temperature, uint64_t seed, int32_t round,
                              int32_t* accept_len, int32_t* out_token, int32_t* anchor_out,
                              void* ws, int64_t ws_bytes, void* stream) {
  if (batch < 0 || block_size < 2 || block_size > 17 || vocab < 2 || !(temperature > 0.f) ||
      !std::isfinite(temperature))
    return DFLASH_ERR_SHAPE;
  if (batch == 0) return DFLASH_OK;
  if (!drafts || !draft_logits || !target_logits || !accept_len || !out_token || !ws)
    return DFLASH_ERR_NULL;
  const void* ps[] = {drafts, draft_logits, target_logits, accept_len, out_token, ws};
  for (const void* q : ps)
    if (!al16(q)) return DFLASH_ERR_ALIGN;
  if (anchor_out && !al16(anchor_out)) return DFLASH_ERR_ALIGN;
  if (draft_logq && !al16(draft_logq)) return DFLASH_ERR_ALIGN;
  if (ws_bytes < verify_ws_bytes(batch, block_size, vocab)) return DFLASH_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  // bytes: every target row (and without log q every draft row) is read once
  // for its normaliser, the emitted position's target and draft rows once more
  const double rows = (double)batch * block_size +
                      (draft_logq ? 0.0 : (double)batch * (block_size - 1)) + 2.0 * batch;
  prof_begin(DFLASH_K_SAMPLING, rows * vocab * 4, 0.0, st);
  const hipError_t e = launch_verify_sampled(drafts, draft_logits, draft_logq, target_logits,
                                             batch, block_size,
                                             vocab, temperature, seed, round, accept_len,
                                             out_token, anchor_out, ws, st);
  prof_end(st);
  return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

int32_t dflash_accept(const int32_t* draft_tokens, const int32_t* target_tokens, int32_t batch,
                      int32_t block_size, int32_t* accept_len, int32_t* bonus,
                      int32_t* anchor_out, void* stream) {
  if (batch < 0 || block_size < 1) return DFLASH_ERR_SHAPE;
  if (batch == 0) return DFLASH_OK;
  if (!target_tokens || !accept_len || !bonus) return DFLASH_ERR_NULL;
  if (block_size > 1 && !draft_tokens) return DFLASH_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  prof_begin(DFLASH_K_SMALL, 0, 0, st);
  hipError_t e = launch_accept(draft_tokens, target_tokens, batch, block_size, accept_len, bonus,
                               anchor_out, st);
  prof_end(st);
  return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

int32_t dflash_packed_block_attention(const dflash_handle* h, const dflash_kv_cache* cache,
                                      int32_t layer, int32_t n_seq, int32_t blocks_per_seq,
                                      const int32_t* anchors, const void* q, const void* k_blk,
                                      const void* v_blk, void* out, int32_t* dev_status,
                                      void* stream) {
  if (!h) return DFLASH_ERR_NULL;
  int32_t rc = check_cache(h, cache);
  if (rc != DFLASH_OK) return rc;
  const dflash_config& c = h->cfg;
  if (layer < 0 || layer >= c.n_layers || n_seq < 0 || blocks_per_seq < 0 || n_seq > cache->batch)
    return DFLASH_ERR_SHAPE;
  const int64_t n_blk = (int64_t)n_seq * blocks_per_seq;
  if (n_blk * c.block_size > INT32_MAX) return DFLASH_ERR_SHAPE;
  if (n_blk == 0) return DFLASH_OK;
  if (!anchors || !q || !k_blk || !v_blk || !out) return DFLASH_ERR_NULL;
  if (!al16(q) || !al16(k_blk) || !al16(v_blk) || !al16(out)) return DFLASH_ERR_ALIGN;
  const int hd = c.head_dim, Hkv = c.n_kv_heads;
  const size_t es = elem_size(c.dtype);
  const size_t layer_elems = (size_t)cache->batch * Hkv * cache->capacity * hd;
  PackedAttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.k = (const char*)cache->k + layer_elems * es * layer;
  a.v = (const char*)cache->v + layer_elems * es * layer;
  a.ctx_len = cache->ctx_len;
  a.anchors = anchors;
  a.out = out;
  a.dev_status = dev_status;
  a.n_blk = (int)n_blk;
  a.blocks_per_seq = blocks_per_seq;
  a.n_heads = c.n_heads;
  a.n_kv_heads = Hkv;
  a.head_dim = hd;
  a.block = c.block_size;
  a.cap = cache->capacity;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)hd));
  hipStream_t st = (hipStream_t)stream;
  prof_begin(DFLASH_K_ATTN_PACKED, 0.0, 0.0, st);
  const hipError_t e = launch_packed_attention(c.dtype, a, st);
  prof_end(st);
  return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

int32_t dflash_round_graph_create(const dflash_handle* h, const dflash_kv_cache* cache,
                                  const dflash_round_io* io, void* stream,
                                  dflash_round_graph** out) {
  if (!out) return DFLASH_ERR_NULL;
  *out = nullptr;
  if (!h || !cache || !io || !stream) return DFLASH_ERR_NULL;
  if (g_prof_on) return DFLASH_ERR_STATE;  // its event records would be baked into the graph
  if (io->batch <= 0 || io->batch != cache->batch) return DFLASH_ERR_SHAPE;
  const int B = h->cfg.block_size;
  if ((int64_t)io->batch * B > INT32_MAX) return DFLASH_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal) != hipSuccess)
    return DFLASH_ERR_HIP;
  // Each call validates its arguments before enqueuing anything; the first
  // error ends the capture and discards what it holds.
  int32_t rc = dflash_accept(io->draft_tokens, io->target_tokens, io->batch, B, io->accept_len,
                             io->anchor, nullptr, stream);
  if (!rc)
    rc = dflash_ctx_project(h, io->feats, io->feat_row_stride, io->batch * B, io->ctx, io->ws,
                            io->ws_bytes, stream);
  if (!rc)
    rc = dflash_ctx_kv_append_accepted(h, cache, io->ctx, io->accept_len, io->dev_status, io->ws,
                                       io->ws_bytes, stream);
  if (!rc)
    rc = dflash_draft_forward(h, cache, io->anchor, io->batch, io->draft_tokens, io->logits,
                              nullptr, nullptr, nullptr, nullptr, io->dev_status, io->ws,
                              io->ws_bytes, stream);
  hipGraph_t graph = nullptr;
  const hipError_t ec = hipStreamEndCapture(st, &graph);
  if (rc || ec != hipSuccess || !graph) {
    if (graph) (void)hipGraphDestroy(graph);
    return rc ? rc : DFLASH_ERR_HIP;
  }
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return DFLASH_ERR_HIP;
  }
  dflash_round_graph* g = new (std::nothrow) dflash_round_graph{graph, exec};
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return DFLASH_ERR_HIP;
  }
  *out = g;
  return DFLASH_OK;
}

int32_t dflash_round_graph_launch(dflash_round_graph* g, void* stream) {
  if (!g) return DFLASH_ERR_NULL;
  return hipGraphLaunch(g->exec, (hipStream_t)stream) == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

void dflash_round_graph_destroy(dflash_round_graph* g) {
  if (!g) return;
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
}

int32_t dflash_profiler_start(int32_t max_launches, uint32_t class_mask) {
  if (max_launches < 1) return DFLASH_ERR_SHAPE;
  if (g_prof_on) return DFLASH_ERR_STATE;
  g_prof_mask = class_mask ? class_mask : 0xFFFFFFFFu;
  const size_t need = 2 * (size_t)max_launches;
  while (g_pool.size() < need) {
    hipEvent_t ev;
    if (hipEventCreate(&ev) != hipSuccess) return DFLASH_ERR_HIP;
    g_pool.push_back(ev);
  }
  g_prof_on = true;
  return DFLASH_OK;
}

int32_t dflash_profiler_stop(void) {
  g_prof_on = false;
  g_open = -1;
  return DFLASH_OK;
}

int32_t dflash_profiler_read(int32_t kind, int64_t* launches, double* total_ms, double* total_bytes,
                             double* total_flops) {
  if (kind < 0 || kind >= DFLASH_K_NCLASSES) return DFLASH_ERR_SHAPE;
  if (!launches || !total_ms || !total_bytes || !total_flops) return DFLASH_ERR_NULL;
  int64_t n = 0;
  double ms = 0, by = 0, fl = 0;
  for (const ProfRec& r : g_rec) {
    if (r.kind != kind || !r.closed) continue;
    if (hipEventSynchronize(r.e1) != hipSuccess) return DFLASH_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.e0, r.e1) != hipSuccess) return DFLASH_ERR_HIP;
    ++n;
    ms += t;
    by += r.bytes;
    fl += r.flops;
  }
  *launches = n;
  *total_ms = ms;
  *total_bytes = by;
  *total_flops = fl;
  return DFLASH_OK;
}

int32_t dflash_profiler_reset(void) {
  if (g_prof_on) return DFLASH_ERR_STATE;
  g_rec.clear();
  g_pool_next = 0;
  for (hipEvent_t ev : g_pool) (void)hipEventDestroy(ev);
  g_pool.clear();
  return DFLASH_OK;
}

}  // extern "C"
