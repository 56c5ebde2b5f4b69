// C ABI of the DFlash draft-and-accept path: argument validation, workspace
// layout and the launch sequence of each entry point.  No allocation, no
// synchronisation: every launch goes to the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "internal.h"

using namespace dflash;

namespace {

thread_local std::string g_last_error;

dflash_status fail(dflash_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dflash_status fail(dflash_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

dflash_status hip_fail(hipError_t e, const char* what) {
  return fail(DFLASH_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int act_bytes(int dt) { return dt == DFLASH_BF16 ? 2 : 4; }

dflash_status check_config(const dflash_config* c) {
  if (c == nullptr) return fail(DFLASH_EINVAL, "config is NULL");
  if (c->n_layers < 1 || c->n_layers > DFLASH_MAX_LAYERS)
    return fail(DFLASH_EUNSUPPORTED, "n_layers %d outside 1..%d", c->n_layers, DFLASH_MAX_LAYERS);
  if (c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->inter <= 0 ||
      c->vocab <= 0 || c->feat_dim <= 0 || c->page_size <= 0)
    return fail(DFLASH_EINVAL, "non-positive model dimension");
  if (c->page_size % 16)
    return fail(DFLASH_EUNSUPPORTED, "page_size %d (must be a multiple of 16)", c->page_size);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(DFLASH_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", c->head_dim);
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(DFLASH_EUNSUPPORTED, "n_q_heads %d not a multiple of n_kv_heads %d",
                c->n_q_heads, c->n_kv_heads);
  if (c->block_size < 2 || c->block_size > 16)
    return fail(DFLASH_EUNSUPPORTED, "block_size %d outside 2..16", c->block_size);
  if ((c->n_q_heads / c->n_kv_heads) * c->block_size > 64)
    return fail(DFLASH_EUNSUPPORTED, "(n_q_heads / n_kv_heads) * block_size = %d > 64",
                (c->n_q_heads / c->n_kv_heads) * c->block_size);
  if (c->hidden % 32 || c->feat_dim % 32 || c->inter % 64)
    return fail(DFLASH_EUNSUPPORTED, "hidden and feat_dim must be multiples of 32, inter of 64");
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab)
    return fail(DFLASH_EINVAL, "mask_token_id %d outside the vocabulary", c->mask_token_id);
  if (c->act_dtype != DFLASH_F32 && c->act_dtype != DFLASH_BF16)
    return fail(DFLASH_EUNSUPPORTED, "act_dtype %d (supported: F32, BF16)", c->act_dtype);
  if (c->act_dtype == DFLASH_F32 && c->kv_dtype != DFLASH_F32)
    return fail(DFLASH_EUNSUPPORTED, "an F32 model needs an F32 cache");
  if (c->act_dtype == DFLASH_BF16 && c->kv_dtype != DFLASH_BF16 && c->kv_dtype != DFLASH_FP8_E4M3)
    return fail(DFLASH_EUNSUPPORTED, "a BF16 model needs a BF16 or FP8_E4M3 cache");
  if (!(c->rms_eps >= 0.f) || !isfinite(c->rms_eps))
    return fail(DFLASH_EINVAL, "rms_eps must be finite and >= 0");
  if (!(c->rope_theta > 0.f) || !isfinite(c->rope_theta))
    return fail(DFLASH_EINVAL, "rope_theta must be finite and > 0");
  for (int l = 0; l < c->n_layers; ++l)
    if (c->sliding_window[l] < 0) return fail(DFLASH_EINVAL, "negative sliding_window[%d]", l);
  if (c->context_window < 0) return fail(DFLASH_EINVAL, "negative context_window");
  return DFLASH_OK;
}

#define REQUIRE_PTR(p, name)                                                     \
  do {                                                                           \
    if ((p) == nullptr) return fail(DFLASH_EINVAL, "%s is NULL", name);          \
    if (!aligned16(p)) return fail(DFLASH_EINVAL, "%s is not 16-byte aligned", name); \
  } while (0)

dflash_status check_layer_weights(const dflash_config* c, const dflash_weights* w, bool draft) {
  if (w == nullptr) return fail(DFLASH_EINVAL, "weights is NULL");
  char nm[64];
  for (int l = 0; l < c->n_layers; ++l) {
    const dflash_layer_weights& L = w->layer[l];
    snprintf(nm, sizeof nm, "layer[%d].w_qkv", l);
    REQUIRE_PTR(L.w_qkv, nm);
    snprintf(nm, sizeof nm, "layer[%d].k_norm", l);
    REQUIRE_PTR(L.k_norm, nm);
    if (!draft) continue;
    const void* ps[] = {L.in_norm, L.q_norm, L.w_o, L.post_norm, L.w_gate, L.w_up, L.w_down};
    const char* ns[] = {"in_norm", "q_norm", "w_o", "post_norm", "w_gate", "w_up", "w_down"};
    for (int i = 0; i < 7; ++i) {
      snprintf(nm, sizeof nm, "layer[%d].%s", l, ns[i]);
      REQUIRE_PTR(ps[i], nm);
    }
  }
  return DFLASH_OK;
}

dflash_status check_cache(const dflash_config* c, const dflash_kv_cache* kv) {
  if (kv == nullptr) return fail(DFLASH_EINVAL, "cache is NULL");
  if (kv->num_pages <= 0) return fail(DFLASH_EINVAL, "cache.num_pages must be > 0");
  char nm[64];
  for (int l = 0; l < c->n_layers; ++l) {
    snprintf(nm, sizeof nm, "cache.k[%d]", l);
    REQUIRE_PTR(kv->k[l], nm);
    snprintf(nm, sizeof nm, "cache.v[%d]", l);
    REQUIRE_PTR(kv->v[l], nm);
  }
  return DFLASH_OK;
}

// Bump allocator over the caller's workspace (256-byte aligned regions).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

constexpr int kInjectChunk = 8192;  // context rows per injection pass

struct ContextWs {
  float2* cs; void* cg; float* ss; float* kv_raw; GemmScratch gs; size_t bytes;
};

int64_t inject_chunk_rows(int64_t rows) { return rows < kInjectChunk ? rows : kInjectChunk; }

ContextWs layout_context(const dflash_config* c, int64_t chunk, void* ws) {
  Carver cv(ws);
  ContextWs L;
  const int M = (int)chunk;
  L.cs = (float2*)cv.take(sizeof(float2) * M * (c->head_dim / 2));
  // (a last chunk of <= 64 rows keeps it in 16 x 32 blocks: at most 64 rows)
  L.cg = cv.take((size_t)act_bytes(c->act_dtype) * act_rows(M) * c->hidden);
  L.ss = (float*)cv.take(sizeof(float) * (size_t)M * ss_tiles(c->hidden));
  // the last chunk of a call can be any size up to `chunk`: take the worst
  // case over row counts.  A plan depends on the row count only through its
  // kernel and its number of row tiles, so one count per (kernel, tile count)
  // covers every case: the streaming kernel's 16 / 32 / 64-row tiles, the
  // 128- and 256-row tiles of the tiled kernels (bf16), 64-row tiles beyond
  // 64 rows (fp32).
  const bool bf = c->act_dtype == DFLASH_BF16;
  size_t pf = 0;
  auto probe = [&](int m) {
    if (m < 1 || m > M) return;
    const GemmPlan ps[2] = {plan_gemm(m, c->hidden, c->feat_dim, bf, 1),
                            plan_gemm(m, c->n_layers * 2 * c->n_kv_heads * c->head_dim,
                                      c->hidden, bf)};
    for (const GemmPlan& p : ps)
      if (gemm_partial_floats(p) > pf) pf = gemm_partial_floats(p);
  };
  for (int m : {16, 32, 64, 128, 192}) probe(m);
  for (int t = 1; (int64_t)(t - 1) * (bf ? 256 : 64) < M; ++t) probe(t * (bf ? 256 : 64));
  probe(M);
  L.gs.partial = (float*)cv.take(sizeof(float) * (pf ? pf : 1));
  L.gs.partial_floats = pf;
  // 1/rms per row for the tiled K/V GEMM (chunks of more than 64 rows)
  if (M > 64) {
    L.gs.rstd = (float*)cv.take(sizeof(float) * (size_t)M);
    L.gs.rstd_floats = (size_t)M;
  }
  // fp32 K/V partials of the narrow path (a call of <= 64 rows)
  const int nraw = kv_inject_raw_floats(M, c->n_layers, c->n_kv_heads, c->head_dim);
  L.kv_raw = nraw > 0 ? (float*)cv.take(sizeof(float) * (size_t)nraw) : nullptr;
  L.bytes = cv.off;
  return L;
}

struct DraftWs {
  float* x; float* ss; void* xg; void* act; void* q; void* kb; void* vb; void* o; float2* cs;
  float* o_part; float2* ml_part; int4* seg; float2* lm_part; float* qkv_raw; GemmScratch gs;
  size_t bytes;
  AttnPlan plans[DFLASH_MAX_LAYERS];
};

int layer_max_keys(const dflash_config* c, int l, int max_prefix) {
  const int W = c->sliding_window[l];
  int keys = max_prefix;
  if (W > 0 && W - 1 < keys) keys = W - 1;
  if (c->context_window > 0 && c->context_window < keys) keys = c->context_window;
  return keys;
}

DraftWs layout_draft(const dflash_config* c, int B, int max_prefix, void* ws) {
  Carver cv(ws);
  DraftWs L;
  const int S = c->block_size, M = B * S, M1 = B * (S - 1), H = c->hidden;
  const int nq = c->n_q_heads, nkv = c->n_kv_heads, D = c->head_dim, I = c->inter;
  const size_t ab = act_bytes(c->act_dtype);
  L.x = (float*)cv.take(sizeof(float) * (size_t)M * H);
  L.ss = (float*)cv.take(sizeof(float) * (size_t)M * ss_tiles(H));
  // the GEMMs' A operands, in 16 x 32 blocks (rows rounded up to 16) at <= 64 rows
  const size_t Ma = (size_t)act_rows(M);
  L.xg = cv.take(ab * Ma * H);
  L.act = cv.take(ab * Ma * I);
  L.q = cv.take(ab * (size_t)M * nq * D);
  L.kb = cv.take(ab * (size_t)B * nkv * 16 * D);
  L.vb = cv.take(ab * (size_t)B * nkv * 16 * D);
  L.o = cv.take(ab * Ma * nq * D);
  L.cs = (float2*)cv.take(sizeof(float2) * (size_t)M * (D / 2));
  // one (O, m, l) partial of 64 query rows per attention workgroup
  const bool dma = attn_uses_dma(c->act_dtype, c->kv_dtype, D);
  size_t max_launch = 1;
  for (int l = 0; l < c->n_layers; ++l) {
    L.plans[l] = plan_attention(layer_max_keys(c, l, max_prefix), B, nkv, dma);
    if ((size_t)L.plans[l].n_partials > max_launch) max_launch = (size_t)L.plans[l].n_partials;
  }
  L.o_part = (float*)cv.take(sizeof(float) * max_launch * 64 * D);
  L.ml_part = (float2*)cv.take(sizeof(float2) * max_launch * 64);
  L.seg = (int4*)cv.take(sizeof(int4) * (size_t)B);
  L.lm_part = (float2*)cv.take(sizeof(float2) * (size_t)M1 * logits_tiles(c->vocab));
  // fp32 q/k/v of the narrow QKV GEMM (up to 64 block rows)
  L.qkv_raw = M <= 64 ? (float*)cv.take(sizeof(float) * (size_t)qkv_k_splits((nq + 2 * nkv) * D) *
                                         M * (nq + 2 * nkv) * D)
                      : nullptr;
  const bool bf = c->act_dtype == DFLASH_BF16;
  const GemmPlan ps[] = {plan_gemm(M, (nq + 2 * nkv) * D, H, bf, M <= 64 ? qkv_slabs() : 0,
                                   qkv_k_splits((nq + 2 * nkv) * D)),
                         plan_gemm(M, H, nq * D, bf, 1),
                         plan_gemm(M, ((I + 63) / 64) * 128, H, bf, 2), plan_gemm(M, H, I, bf, 1),
                         plan_gemm(M1, c->vocab, H, bf, 8)};
  size_t pf = 0;
  for (const GemmPlan& p : ps)
    if (gemm_partial_floats(p) > pf) pf = gemm_partial_floats(p);
  L.gs.partial = (float*)cv.take(sizeof(float) * (pf ? pf : 1));
  L.gs.partial_floats = pf;
  // 1/rms per row for the tiled GEMMs (more than 64 block rows)
  if (M > 64) {
    L.gs.rstd = (float*)cv.take(sizeof(float) * (size_t)M);
    L.gs.rstd_floats = (size_t)M;
  }
  L.bytes = cv.off;
  return L;
}

struct LmHeadWs {
  float2* part; GemmScratch gs; size_t bytes;
};

LmHeadWs layout_lm_head(const dflash_config* c, int rows, void* ws) {
  Carver cv(ws);
  LmHeadWs L;
  L.part = (float2*)cv.take(sizeof(float2) * (size_t)rows * logits_tiles(c->vocab));
  const GemmPlan p = plan_gemm(rows, c->vocab, c->hidden, c->act_dtype == DFLASH_BF16, 8);
  const size_t pf = gemm_partial_floats(p);
  L.gs.partial = (float*)cv.take(sizeof(float) * (pf ? pf : 1));
  L.gs.partial_floats = pf;
  L.bytes = cv.off;
  return L;
}

}  // namespace

namespace dflash {
dflash_status set_error(dflash_status s, const char* msg) { return fail(s, "%s", msg); }
}  // namespace dflash

extern "C" {

const char* dflash_status_string(dflash_status s) {
  switch (s) {
    case DFLASH_OK: return "ok";
    case DFLASH_EINVAL: return "invalid argument";
    case DFLASH_EUNSUPPORTED: return "unsupported configuration";
    case DFLASH_EWORKSPACE: return "workspace too small";
    case DFLASH_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* dflash_last_error(void) { return g_last_error.c_str(); }

size_t dflash_packed_matrix_bytes(int32_t rows, int32_t cols, int32_t dtype) {
  if (rows <= 0 || cols <= 0 || cols % 32 || (dtype != DFLASH_F32 && dtype != DFLASH_BF16))
    return 0;
  return packed_matrix_elems(rows, cols) * act_bytes(dtype);
}

dflash_status dflash_pack_matrix(const void* src, void* dst, int32_t rows, int32_t cols,
                                 int32_t dtype, void* stream) {
  if (dtype != DFLASH_F32 && dtype != DFLASH_BF16)
    return fail(DFLASH_EUNSUPPORTED, "dtype %d (supported: F32, BF16)", dtype);
  if (rows <= 0 || cols <= 0) return fail(DFLASH_EINVAL, "non-positive matrix size");
  if (cols % 32) return fail(DFLASH_EUNSUPPORTED, "cols %d not a multiple of 32", cols);
  REQUIRE_PTR(src, "src");
  REQUIRE_PTR(dst, "dst");
  const uintptr_t s0 = (uintptr_t)src, s1 = s0 + (size_t)rows * cols * act_bytes(dtype);
  const uintptr_t d0 = (uintptr_t)dst, d1 = d0 + dflash_packed_matrix_bytes(rows, cols, dtype);
  if (s0 < d1 && d0 < s1) return fail(DFLASH_EINVAL, "src and dst overlap");
  const hipError_t e = pack_matrix(dtype, src, dst, rows, cols, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "pack");
}

size_t dflash_context_workspace_bytes(const dflash_config* cfg, int64_t rows) {
  if (check_config(cfg) != DFLASH_OK || rows < 0) return 0;
  return layout_context(cfg, inject_chunk_rows(rows > 0 ? rows : 1), nullptr).bytes;
}

size_t dflash_draft_workspace_bytes(const dflash_config* cfg, int32_t batch,
                                    int32_t max_prefix_len) {
  if (check_config(cfg) != DFLASH_OK || batch <= 0 || max_prefix_len < 0) return 0;
  return layout_draft(cfg, batch, max_prefix_len, nullptr).bytes;
}

dflash_status dflash_project_context(const dflash_config* cfg, const dflash_weights* w,
                                     const dflash_kv_cache* cache, const void* feats,
                                     int64_t feat_row_stride, const int32_t* positions,
                                     const int32_t* slots, const int32_t* valid_rows,
                                     int32_t n_req, int32_t rows_per_req, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  dflash_status s = check_config(cfg);
  if (s != DFLASH_OK) return s;
  if (n_req < 0 || rows_per_req < 0) return fail(DFLASH_EINVAL, "negative row counts");
  const int64_t T = (int64_t)n_req * rows_per_req;
  if (T == 0) return DFLASH_OK;
  if (T > (int64_t)1 << 30) return fail(DFLASH_EINVAL, "too many rows (%lld)", (long long)T);
  if ((s = check_layer_weights(cfg, w, false)) != DFLASH_OK) return s;
  REQUIRE_PTR(w->fc, "weights.fc");
  REQUIRE_PTR(w->hidden_norm, "weights.hidden_norm");
  if ((s = check_cache(cfg, cache)) != DFLASH_OK) return s;
  REQUIRE_PTR(feats, "feats");
  if (positions == nullptr || slots == nullptr)
    return fail(DFLASH_EINVAL, "positions and slots must not be NULL");
  if (feat_row_stride < cfg->feat_dim || feat_row_stride % 8)
    return fail(DFLASH_EINVAL, "feat_row_stride %lld must be >= feat_dim and a multiple of 8",
                (long long)feat_row_stride);
  // chunks of up to kInjectChunk rows: a chunk may start or end inside a
  // request (the K/V epilogue finds each row's request from its grid row)
  const int64_t chunk = inject_chunk_rows(T);
  const ContextWs L = layout_context(cfg, chunk, workspace);
  if (workspace == nullptr || workspace_bytes < L.bytes)
    return fail(DFLASH_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, L.bytes);
  if (!aligned16(workspace)) return fail(DFLASH_EINVAL, "workspace is not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  KVTargets tg;
  memset(&tg, 0, sizeof tg);
  for (int l = 0; l < cfg->n_layers; ++l) {
    tg.w_qkv[l] = w->layer[l].w_qkv;
    tg.k_norm[l] = w->layer[l].k_norm;
    tg.kc[l] = cache->k[l];
    tg.vc[l] = cache->v[l];
  }
  const int dt = cfg->act_dtype;
  hipError_t e;
  for (int64_t t0 = 0; t0 < T; t0 += chunk) {
    const int M = (int)((T - t0) < chunk ? (T - t0) : chunk);
    const void* f = static_cast<const char*>(feats) + (size_t)t0 * feat_row_stride * act_bytes(dt);
    // the tiled K/V path reads a RoPE table; the narrow one forms its own
    if (!kv_inject_is_narrow(M, cfg->n_layers, L.kv_raw) &&
        (e = launch_rope_table(positions + t0, M, cfg->head_dim, cfg->rope_theta, L.cs, st)) !=
            hipSuccess)
      return hip_fail(e, "rope table");
    // c = fc(f): the fc epilogue writes c * hidden_norm (act dtype) and the
    // row sums of squares of c; the K/V GEMM streams the former and scales
    // its rows by 1/rms(c) (RMSNorm by linearity)
    const int blk = act_blocked(M);
    if ((e = gemm_store_f32(dt, asrc_plain(f, feat_row_stride), M, cfg->feat_dim, w->fc,
                            cfg->hidden, nullptr, L.ss, L.cg, blk, w->hidden_norm, L.gs, st)) !=
        hipSuccess)
      return hip_fail(e, "fc gemm");
    const ASrc cin = asrc_normed(L.cg, cfg->hidden, L.ss, cfg->rms_eps, 0, blk);
    if ((e = gemm_kv_inject(dt, cfg->kv_dtype, cin, M, cfg->hidden, tg, cfg->n_layers,
                            cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim, cfg->rms_eps, L.cs,
                            positions + t0, cfg->rope_theta, slots + t0, valid_rows,
                            rows_per_req > 0 ? rows_per_req : 1, t0,
                            cfg->page_size, cache->num_pages, L.kv_raw, L.gs, st)) != hipSuccess)
      return hip_fail(e, "kv inject gemm");
  }
  return DFLASH_OK;
}

static dflash_status check_draft_args(const dflash_config* cfg, const dflash_weights* w,
                                 const dflash_kv_cache* cache, const int32_t* anchor,
                                 const int32_t* prefix_len, const int32_t* page_table,
                                 int32_t max_pages, int32_t batch, int32_t max_prefix_len,
                                 int32_t* block_ids, int32_t* positions, int32_t* slots,
                                 int32_t* candidates, void* logits, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  dflash_status s = check_config(cfg);
  if (s != DFLASH_OK) return s;
  if (batch < 0 || max_pages <= 0 || max_prefix_len < 0)
    return fail(DFLASH_EINVAL, "batch, max_pages or max_prefix_len out of range");
  if (batch == 0) return DFLASH_OK;
  if ((int64_t)batch * cfg->block_size > (1 << 24)) return fail(DFLASH_EINVAL, "batch too large");
  if ((s = check_layer_weights(cfg, w, true)) != DFLASH_OK) return s;
  REQUIRE_PTR(w->embed, "weights.embed");
  REQUIRE_PTR(w->lm_head, "weights.lm_head");
  REQUIRE_PTR(w->final_norm, "weights.final_norm");
  if ((s = check_cache(cfg, cache)) != DFLASH_OK) return s;
  if (!anchor || !prefix_len || !page_table || !positions || !slots || !candidates)
    return fail(DFLASH_EINVAL, "anchor, prefix_len, page_table, positions, slots and candidates "
                               "must not be NULL");
  if (logits != nullptr && !aligned16(logits)) return fail(DFLASH_EINVAL, "logits not aligned");
  return DFLASH_OK;
}

// The backbone pass, the lm_head and the argmax (candidates 1..S-1), on a
// workspace already carved by layout_draft.
static dflash_status draft_core(const dflash_config* cfg, const dflash_weights* w,
                                const dflash_kv_cache* cache, const int32_t* anchor,
                                const int32_t* prefix_len, const int32_t* page_table,
                                int32_t max_pages, int32_t batch, int32_t max_prefix_len,
                                int32_t* block_ids, int32_t* positions, int32_t* slots,
                                int32_t* candidates, void* logits, const DraftWs& L,
                                hipStream_t st) {
  const int dt = cfg->act_dtype, S = cfg->block_size, M = batch * S, M1 = batch * (S - 1);
  const int H = cfg->hidden, nq = cfg->n_q_heads, nkv = cfg->n_kv_heads, D = cfg->head_dim;
  const int I = cfg->inter;
  hipError_t e;
  const int n_ss = ss_tiles(H);
  const float eps = cfg->rms_eps;
  // Every RMSNorm is applied by linearity: the producer of the residual x writes
  // xg = x * g_next (act dtype) and the row sums of squares of x; the consumer
  // GEMM streams xg and scales its output rows by 1/rms(x).  The GEMMs' A
  // operands (xg, the attention output, the SwiGLU activations) sit in 16 x 32
  // blocks when the pass has at most 64 block rows.
  const int blk = act_blocked(M);
  if ((e = launch_block_prep(dt, *cfg, w->embed, anchor, prefix_len, page_table, max_pages, batch,
                             block_ids, positions, slots, candidates, L.x, L.ss, n_ss, L.xg, blk,
                             w->layer[0].in_norm, L.cs, st)) != hipSuccess)
    return hip_fail(e, "block prep");
  const ASrc xin = asrc_normed(L.xg, H, L.ss, eps, 0, blk);
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dflash_layer_weights& W = w->layer[l];
    const void* g_after = (l + 1 < cfg->n_layers) ? w->layer[l + 1].in_norm : w->final_norm;
    if ((e = gemm_qkv(dt, xin, M, H, W.w_qkv, W.q_norm, W.k_norm, nq, nkv, D, eps, L.cs, L.q, L.kb,
                      L.vb, S, L.qkv_raw, L.gs, st)) != hipSuccess)
      return hip_fail(e, "qkv gemm");
    if ((e = launch_attention(dt, cfg->kv_dtype, D, L.q, L.kb, L.vb, cache->k[l], cache->v[l],
                              page_table, max_pages, cache->num_pages, prefix_len, max_prefix_len,
                              batch, S, nq, nkv, cfg->page_size, cfg->sliding_window[l],
                              cfg->context_window, L.plans[l], L.o_part, L.ml_part, L.seg, L.o,
                              blk, st)) != hipSuccess)
      return hip_fail(e, "attention");
    if ((e = gemm_residual(dt, asrc_plain(L.o, nq * D, 0, blk), M, nq * D, W.w_o, H, L.x, L.ss,
                           L.xg, blk, W.post_norm, L.gs, st)) != hipSuccess)
      return hip_fail(e, "o-proj gemm");
    if ((e = gemm_silu_mul(dt, xin, M, H, W.w_gate, W.w_up, I, L.act, blk, L.gs, st)) !=
        hipSuccess)
      return hip_fail(e, "gate/up gemm");
    if ((e = gemm_residual(dt, asrc_plain(L.act, I, 0, blk), M, I, W.w_down, H, L.x, L.ss, L.xg,
                           blk, g_after, L.gs, st)) != hipSuccess)
      return hip_fail(e, "down gemm");
  }
  // final norm of rows 1..S-1 of every block, applied by the lm_head GEMM
  if ((e = gemm_logits(dt, asrc_normed(L.xg, H, L.ss, eps, S, blk), M1, H, w->lm_head, cfg->vocab,
                       logits, L.lm_part, L.gs, st)) != hipSuccess)
    return hip_fail(e, "lm_head gemm");
  if ((e = launch_argmax_reduce(L.lm_part, M1, logits_tiles(cfg->vocab), S, candidates, st)) !=
      hipSuccess)
    return hip_fail(e, "argmax");
  return DFLASH_OK;
}

dflash_status dflash_draft_block(const dflash_config* cfg, const dflash_weights* w,
                                 const dflash_kv_cache* cache, const int32_t* anchor,
                                 const int32_t* prefix_len, const int32_t* page_table,
                                 int32_t max_pages, int32_t batch, int32_t max_prefix_len,
                                 int32_t* block_ids, int32_t* positions, int32_t* slots,
                                 int32_t* candidates, void* logits, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  dflash_status s = check_draft_args(cfg, w, cache, anchor, prefix_len, page_table, max_pages,
                                     batch, max_prefix_len, block_ids, positions, slots,
                                     candidates, logits, workspace, workspace_bytes, stream);
  if (s != DFLASH_OK || batch == 0) return s;
  const DraftWs L = layout_draft(cfg, batch, max_prefix_len, workspace);
  if (workspace == nullptr || workspace_bytes < L.bytes)
    return fail(DFLASH_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, L.bytes);
  if (!aligned16(workspace)) return fail(DFLASH_EINVAL, "workspace is not 16-byte aligned");
  return draft_core(cfg, w, cache, anchor, prefix_len, page_table, max_pages, batch,
                    max_prefix_len, block_ids, positions, slots, candidates, logits, L,
                    static_cast<hipStream_t>(stream));
}

dflash_status dflash_accept_sampling_sparse(
    const int32_t* candidates, const void* target_logits, int32_t logits_dtype, int32_t vocab,
    float target_temperature, const int32_t* q_ids, const float* q_probs, int32_t q_k,
    const float* uniforms, const int32_t* prefix_len, int32_t batch, int32_t block_size,
    int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens, int32_t* next_anchor,
    int32_t* new_seq_len, void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0) return fail(DFLASH_EINVAL, "batch %d < 0", batch);
  if (block_size < 2 || block_size > 64)
    return fail(DFLASH_EUNSUPPORTED, "block_size %d outside 2..64", block_size);
  if (vocab <= 0) return fail(DFLASH_EINVAL, "vocab %d <= 0", vocab);
  if (vocab > 524288) return fail(DFLASH_EUNSUPPORTED, "vocab %d > 524288", vocab);
  if (q_k < 1 || q_k > 16) return fail(DFLASH_EUNSUPPORTED, "q_k %d outside 1..16", q_k);
  if (logits_dtype != DFLASH_F32 && logits_dtype != DFLASH_BF16)
    return fail(DFLASH_EUNSUPPORTED, "logits_dtype %d (supported: F32, BF16)", logits_dtype);
  if (!(target_temperature > 0.f) || !isfinite(target_temperature))
    return fail(DFLASH_EINVAL, "target_temperature must be finite and > 0");
  if ((int64_t)batch * (2 * block_size - 1) > (int64_t)1 << 30)
    return fail(DFLASH_EUNSUPPORTED, "batch %d too large", batch);
  if (batch == 0) return DFLASH_OK;
  if (!candidates || !target_logits || !q_ids || !q_probs || !uniforms || !prefix_len ||
      !accept_len || !commit_len || !out_tokens || !next_anchor || !new_seq_len)
    return fail(DFLASH_EINVAL, "NULL pointer argument");
  const SpecPlan pl = plan_spec(batch, block_size, vocab, false);
  if (workspace == nullptr || workspace_bytes < pl.bytes)
    return fail(DFLASH_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, pl.bytes);
  if (!aligned16(workspace)) return fail(DFLASH_EINVAL, "workspace is not 16-byte aligned");
  const int esz = logits_dtype == DFLASH_BF16 ? 2 : 4;
  int vec = 16 / esz;
  if (vocab % vec || !aligned16(target_logits)) vec = 1;
  const float ct = (float)(1.4426950408889634 / (double)target_temperature);
  hipError_t e = launch_accept_sampling(logits_dtype, vec, candidates, target_logits, nullptr,
                                        q_ids, q_probs, q_k, uniforms, prefix_len, batch,
                                        block_size, vocab, ct, 0.f, pl, workspace, accept_len,
                                        commit_len, out_tokens, next_anchor, new_seq_len,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "accept_sampling_sparse");
  return DFLASH_OK;
}

static dflash_status relay(bool stash, const dflash_request_pool* pool, const int32_t* req_slots,
                           int32_t batch, const int32_t* anchor, const int32_t* len,
                           const int32_t* pt, const int32_t* np, void* stream) {
  if (pool == nullptr) return fail(DFLASH_EINVAL, "pool is NULL");
  if (batch < 0 || pool->capacity < 0 || pool->max_pages < 0)
    return fail(DFLASH_EINVAL, "negative batch, capacity or max_pages");
  if ((int64_t)pool->capacity * pool->max_pages > ((int64_t)1 << 40))
    return fail(DFLASH_EINVAL, "pool too large");
  const void* pairs[4][2] = {{pool->anchor, anchor}, {pool->seq_len, len},
                             {pool->page_table, pt}, {pool->n_pages, np}};
  const char* names[4] = {"anchor", "seq_len", "page_table", "n_pages"};
  for (int i = 0; i < 4; ++i)
    if ((pairs[i][0] == nullptr) != (pairs[i][1] == nullptr))
      return fail(DFLASH_EINVAL, "%s: the pool and the batch array must both be given or both NULL",
                  names[i]);
  if (pt != nullptr && pool->max_pages == 0)
    return fail(DFLASH_EINVAL, "page_table given with max_pages 0");
  if (batch == 0) return DFLASH_OK;
  if (req_slots == nullptr) return fail(DFLASH_EINVAL, "req_slots is NULL");
  hipError_t e = launch_relay(stash, req_slots, batch, pool->capacity, pool->max_pages,
                              pool->anchor, pool->seq_len, pool->page_table, pool->n_pages,
                              const_cast<int32_t*>(anchor), const_cast<int32_t*>(len),
                              const_cast<int32_t*>(pt), const_cast<int32_t*>(np),
                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, stash ? "relay stash" : "relay resolve");
  return DFLASH_OK;
}

dflash_status dflash_relay_resolve(const dflash_request_pool* pool, const int32_t* req_slots,
                                   int32_t batch, int32_t* anchor, int32_t* prefix_len,
                                   int32_t* page_table, int32_t* n_pages, void* stream) {
  return relay(false, pool, req_slots, batch, anchor, prefix_len, page_table, n_pages, stream);
}

dflash_status dflash_relay_stash(const dflash_request_pool* pool, const int32_t* req_slots,
                                 int32_t batch, const int32_t* next_anchor,
                                 const int32_t* new_seq_len, const int32_t* page_table,
                                 const int32_t* n_pages, void* stream) {
  return relay(true, pool, req_slots, batch, next_anchor, new_seq_len, page_table, n_pages,
               stream);
}

dflash_status dflash_reserve_pages(const int32_t* seq_len, int32_t batch, int32_t block_size,
                                   int32_t page_size, int32_t* page_table, int32_t max_pages,
                                   int32_t* n_pages, const int32_t* free_pages,
                                   int32_t free_capacity, int32_t* free_count, int32_t* status,
                                   void* stream) {
  if (batch < 0 || block_size < 1 || page_size < 1 || max_pages < 1 || free_capacity < 0)
    return fail(DFLASH_EINVAL, "batch, block_size, page_size, max_pages or capacity out of range");
  if (!seq_len || !page_table || !n_pages || !free_pages || !free_count || !status)
    return fail(DFLASH_EINVAL, "NULL pointer argument");
  hipError_t e = launch_reserve(seq_len, batch, block_size, page_size, page_table, max_pages,
                                n_pages, free_pages, free_capacity, free_count, status,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "reserve");
  return DFLASH_OK;
}

dflash_status dflash_release_pages(const int32_t* mask, int32_t batch, const int32_t* page_table,
                                   int32_t max_pages, int32_t* n_pages, int32_t* free_pages,
                                   int32_t free_capacity, int32_t* free_count, void* stream) {
  if (batch < 0 || max_pages < 1 || free_capacity < 0)
    return fail(DFLASH_EINVAL, "batch, max_pages or capacity out of range");
  if (batch == 0) return DFLASH_OK;
  if (!mask || !page_table || !n_pages || !free_pages || !free_count)
    return fail(DFLASH_EINVAL, "NULL pointer argument");
  hipError_t e = launch_release(mask, batch, page_table, max_pages, n_pages, free_pages,
                                free_capacity, free_count, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "release");
  return DFLASH_OK;
}

dflash_status dflash_check_draft_inputs(const dflash_config* cfg, const dflash_kv_cache* cache,
                                        const int32_t* anchor, const int32_t* prefix_len,
                                        const int32_t* page_table, int32_t max_pages,
                                        int32_t batch, int32_t max_prefix_len, int32_t* report,
                                        void* stream) {
  if (!cfg || !cache || !report) return fail(DFLASH_EINVAL, "NULL pointer argument");
  if (batch < 0 || max_prefix_len < 0 || max_pages < 1)
    return fail(DFLASH_EINVAL, "batch, max_prefix_len or max_pages out of range");
  if ((int64_t)batch * max_pages > INT32_MAX)
    return fail(DFLASH_EINVAL, "batch * max_pages exceeds the int32 report index");
  if (batch > 0 && (!anchor || !prefix_len || !page_table))
    return fail(DFLASH_EINVAL, "NULL pointer argument");
  if (cfg->page_size < 1 || cfg->block_size < 1 || cfg->vocab < 1)
    return fail(DFLASH_EINVAL, "page_size, block_size or vocab out of range");
  hipError_t e = launch_check_draft(anchor, prefix_len, page_table, max_pages, batch,
                                    max_prefix_len, cfg->block_size, cfg->page_size, cfg->vocab,
                                    cache->num_pages, cfg->context_window > 0 ? cfg->context_window
                                                                              : 0,
                                    report, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "check draft inputs");
  return DFLASH_OK;
}

dflash_status dflash_check_context_inputs(const dflash_config* cfg, const dflash_kv_cache* cache,
                                          const int32_t* positions, const int32_t* slots,
                                          const int32_t* valid_rows, int32_t n_req,
                                          int32_t rows_per_req, int32_t* report, void* stream) {
  if (!cfg || !cache || !report) return fail(DFLASH_EINVAL, "NULL pointer argument");
  if (n_req < 0 || rows_per_req < 0) return fail(DFLASH_EINVAL, "negative row counts");
  if ((int64_t)n_req * rows_per_req > INT32_MAX)
    return fail(DFLASH_EINVAL, "more than 2^31 - 1 rows");
  if ((int64_t)n_req * rows_per_req > 0 && (!positions || !slots))
    return fail(DFLASH_EINVAL, "NULL pointer argument");
  if (cfg->page_size < 1) return fail(DFLASH_EINVAL, "page_size out of range");
  hipError_t e = launch_check_context(positions, slots, valid_rows, n_req, rows_per_req,
                                      cache->num_pages * cfg->page_size, report,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "check context inputs");
  return DFLASH_OK;
}

dflash_status dflash_check_accept_inputs(const int32_t* candidates, const int32_t* posterior,
                                         const int32_t* prefix_len, int32_t batch,
                                         int32_t block_size, int32_t vocab, int32_t* report,
                                         void* stream) {
  if (!report) return fail(DFLASH_EINVAL, "NULL pointer argument");
  if (batch < 0 || block_size < 1 || vocab < 1)
    return fail(DFLASH_EINVAL, "batch, block_size or vocab out of range");
  if ((int64_t)batch * block_size > INT32_MAX) return fail(DFLASH_EINVAL, "batch too large");
  if (batch > 0 && (!candidates || !posterior || !prefix_len))
    return fail(DFLASH_EINVAL, "NULL pointer argument");
  hipError_t e = launch_check_accept(candidates, posterior, prefix_len, batch, block_size, vocab,
                                     report, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "check accept inputs");
  return DFLASH_OK;
}

// Workspace of the selector stage, carved after the draft pass's.
struct SelectorWs {
  void* logits; float* unary; float* w; GemmScratch gs; size_t bytes;
};
static SelectorWs layout_selector(const dflash_config* c, const dflash_selector* sel, int B,
                                  bool own_logits, void* base) {
  Carver cv(base);
  SelectorWs L;
  const int M1 = B * (c->block_size - 1), K = sel->top_k, r = sel->rank;
  L.logits = own_logits ? cv.take((size_t)act_bytes(c->act_dtype) * M1 * c->vocab) : nullptr;
  L.unary = (float*)cv.take(sizeof(float) * (size_t)M1 * K);
  L.w = (float*)cv.take(sizeof(float) * (size_t)M1 * r);
  const GemmPlan gp = plan_gemm(M1, r, c->hidden, c->act_dtype == DFLASH_BF16, 1);
  L.gs.partial_floats = gemm_partial_floats(gp);
  L.gs.partial = (float*)cv.take(sizeof(float) * (L.gs.partial_floats > 0 ? L.gs.partial_floats : 1));
  L.bytes = cv.off;
  return L;
}

static dflash_status check_selector(const dflash_config* c, const dflash_selector* sel) {
  if (sel == nullptr) return fail(DFLASH_EINVAL, "selector is NULL");
  const int K = sel->top_k;
  if (K != 1 && K != 2 && K != 4 && K != 8 && K != 16)
    return fail(DFLASH_EUNSUPPORTED, "top_k %d (supported: 1, 2, 4, 8, 16)", K);
  if (K > c->vocab) return fail(DFLASH_EINVAL, "top_k %d > vocab %d", K, c->vocab);
  if (sel->rank != 16 && sel->rank != 32 && sel->rank != 64 && sel->rank != 128)
    return fail(DFLASH_EUNSUPPORTED, "rank %d (supported: 16, 32, 64, 128)", sel->rank);
  if (c->vocab > 524288) return fail(DFLASH_EUNSUPPORTED, "vocab %d > 524288", c->vocab);
  REQUIRE_PTR(sel->a, "selector.a");
  REQUIRE_PTR(sel->b, "selector.b");
  REQUIRE_PTR(sel->w_h, "selector.w_h");
  return DFLASH_OK;
}

size_t dflash_selector_workspace_bytes(const dflash_config* cfg, const dflash_selector* sel,
                                       int32_t batch, int32_t max_prefix_len) {
  if (check_config(cfg) != DFLASH_OK || sel == nullptr || batch <= 0 || max_prefix_len < 0 ||
      sel->top_k < 1 || sel->top_k > 16 || sel->rank < 1 || sel->rank > 128)
    return 0;
  const size_t d = layout_draft(cfg, batch, max_prefix_len, nullptr).bytes;
  return ((d + 255) & ~(size_t)255) + layout_selector(cfg, sel, batch, true, nullptr).bytes;
}

dflash_status dflash_draft_block_selector(
    const dflash_config* cfg, const dflash_weights* w, const dflash_kv_cache* cache,
    const dflash_selector* sel, const int32_t* anchor, const int32_t* prefix_len,
    const int32_t* page_table, int32_t max_pages, int32_t batch, int32_t max_prefix_len,
    int32_t* block_ids, int32_t* positions, int32_t* slots, int32_t* candidates,
    int32_t* cand_ids, float* q_rows, const float* uniforms, float temperature, void* logits,
    void* workspace, size_t workspace_bytes, void* stream) {
  dflash_status s = check_draft_args(cfg, w, cache, anchor, prefix_len, page_table, max_pages,
                                     batch, max_prefix_len, block_ids, positions, slots,
                                     candidates, logits, workspace, workspace_bytes, stream);
  if (s != DFLASH_OK || batch == 0) return s;
  if ((s = check_selector(cfg, sel)) != DFLASH_OK) return s;
  if (!cand_ids || !q_rows) return fail(DFLASH_EINVAL, "cand_ids and q_rows must not be NULL");
  if (uniforms && (!(temperature > 0.f) || !isfinite(temperature)))
    return fail(DFLASH_EINVAL, "temperature must be finite and > 0 when sampling");
  const DraftWs L = layout_draft(cfg, batch, max_prefix_len, workspace);
  const size_t d = (L.bytes + 255) & ~(size_t)255;
  const SelectorWs SL = layout_selector(cfg, sel, batch, logits == nullptr,
                                        workspace ? static_cast<char*>(workspace) + d : nullptr);
  if (workspace == nullptr || workspace_bytes < d + SL.bytes)
    return fail(DFLASH_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, d + SL.bytes);
  if (!aligned16(workspace)) return fail(DFLASH_EINVAL, "workspace is not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* lg = logits ? logits : SL.logits;
  if ((s = draft_core(cfg, w, cache, anchor, prefix_len, page_table, max_pages, batch,
                      max_prefix_len, block_ids, positions, slots, candidates, lg, L, st)) !=
      DFLASH_OK)
    return s;
  const int S = cfg->block_size, M1 = batch * (S - 1), K = sel->top_k;
  hipError_t e;
  // candidates and their unary logits from the logits just written and the
  // lm_head's per-tile argmax partials
  if ((e = launch_topk(cfg->act_dtype, lg, L.lm_part, M1, cfg->vocab, K, cand_ids, SL.unary,
                       st)) != hipSuccess)
    return hip_fail(e, "top-k");
  // w_j = W_h y_j for the final-normed rows 1..S-1 (the norm applied by linearity)
  if ((e = gemm_store_f32(cfg->act_dtype,
                          asrc_normed(L.xg, cfg->hidden, L.ss, cfg->rms_eps, S,
                                      act_blocked((int64_t)batch * S)),
                          M1, cfg->hidden, sel->w_h, sel->rank, SL.w, nullptr, nullptr, 0, nullptr,
                          SL.gs, st)) != hipSuccess)
    return hip_fail(e, "selector projection");
  if ((e = launch_lattice_walk(cfg->act_dtype, cand_ids, SL.unary, SL.w, sel->a, sel->b, anchor,
                               uniforms, uniforms ? temperature : 1.f, batch, S, K, sel->rank,
                               cfg->vocab, candidates, q_rows, st)) != hipSuccess)
    return hip_fail(e, "selector walk");
  return DFLASH_OK;
}

size_t dflash_lm_head_workspace_bytes(const dflash_config* cfg, int32_t rows) {
  if (check_config(cfg) != DFLASH_OK || rows <= 0) return 0;
  return layout_lm_head(cfg, rows, nullptr).bytes;
}

dflash_status dflash_lm_head_argmax(const dflash_config* cfg, const void* lm_head,
                                    const void* hidden, int32_t rows, void* logits, int32_t* ids,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  dflash_status s = check_config(cfg);
  if (s != DFLASH_OK) return s;
  if (rows < 0) return fail(DFLASH_EINVAL, "rows %d < 0", rows);
  if (rows == 0) return DFLASH_OK;
  REQUIRE_PTR(lm_head, "lm_head");
  REQUIRE_PTR(hidden, "hidden");
  if (ids == nullptr) return fail(DFLASH_EINVAL, "ids is NULL");
  if (logits != nullptr && !aligned16(logits)) return fail(DFLASH_EINVAL, "logits not aligned");
  const LmHeadWs L = layout_lm_head(cfg, rows, workspace);
  if (workspace == nullptr || workspace_bytes < L.bytes)
    return fail(DFLASH_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, L.bytes);
  if (!aligned16(workspace)) return fail(DFLASH_EINVAL, "workspace is not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = gemm_logits(cfg->act_dtype, asrc_plain(hidden, cfg->hidden), rows, cfg->hidden, lm_head,
                       cfg->vocab, logits, L.part, L.gs, st)) != hipSuccess)
    return hip_fail(e, "lm_head gemm");
  if ((e = launch_argmax_reduce(L.part, rows, logits_tiles(cfg->vocab), 0, ids, st)) != hipSuccess)
    return hip_fail(e, "argmax");
  return DFLASH_OK;
}

dflash_status dflash_accept(const int32_t* candidates, const int32_t* posterior,
                            const int32_t* prefix_len, int32_t batch, int32_t block_size,
                            int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                            int32_t* next_anchor, int32_t* new_seq_len, void* stream) {
  if (batch < 0) return fail(DFLASH_EINVAL, "batch %d < 0", batch);
  if (block_size < 1 || block_size > 4096)
    return fail(DFLASH_EINVAL, "block_size %d outside 1..4096", block_size);
  if (batch == 0) return DFLASH_OK;
  if (!candidates || !posterior || !prefix_len || !accept_len || !commit_len || !out_tokens ||
      !next_anchor || !new_seq_len)
    return fail(DFLASH_EINVAL, "NULL pointer argument");
  hipError_t e = launch_accept(candidates, posterior, prefix_len, batch, block_size, accept_len,
                               commit_len, out_tokens, next_anchor, new_seq_len,
                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "accept");
  return DFLASH_OK;
}

size_t dflash_accept_logits_workspace_bytes(int32_t batch, int32_t block_size, int32_t vocab) {
  if (batch <= 0 || block_size < 2 || block_size > 64 || vocab <= 0 || vocab > 524288) return 0;
  return sizeof(float2) * (size_t)batch * block_size * accept_logits_chunks(vocab);
}

dflash_status dflash_accept_logits(const int32_t* candidates, const void* target_logits,
                                   int32_t logits_dtype, int32_t vocab,
                                   const int32_t* prefix_len, int32_t batch, int32_t block_size,
                                   int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                                   int32_t* next_anchor, int32_t* new_seq_len, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (batch < 0) return fail(DFLASH_EINVAL, "batch %d < 0", batch);
  if (block_size < 2 || block_size > 64)
    return fail(DFLASH_EUNSUPPORTED, "block_size %d outside 2..64", block_size);
  if (vocab <= 0) return fail(DFLASH_EINVAL, "vocab %d <= 0", vocab);
  if (vocab > 524288) return fail(DFLASH_EUNSUPPORTED, "vocab %d > 524288", vocab);
  if (logits_dtype != DFLASH_F32 && logits_dtype != DFLASH_BF16)
    return fail(DFLASH_EUNSUPPORTED, "logits_dtype %d (supported: F32, BF16)", logits_dtype);
  if ((int64_t)batch * block_size > (int64_t)1 << 24)
    return fail(DFLASH_EUNSUPPORTED, "batch %d too large", batch);
  if (batch == 0) return DFLASH_OK;
  if (!candidates || !target_logits || !prefix_len || !accept_len || !commit_len || !out_tokens ||
      !next_anchor || !new_seq_len)
    return fail(DFLASH_EINVAL, "NULL pointer argument");
  const size_t need = dflash_accept_logits_workspace_bytes(batch, block_size, vocab);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DFLASH_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(DFLASH_EINVAL, "workspace is not 16-byte aligned");
  // 16-byte loads when every run of 8 columns starts on a 16-byte boundary
  const bool vec = vocab % 8 == 0 && aligned16(target_logits);
  hipError_t e = launch_accept_logits(logits_dtype, target_logits, vocab, vec, candidates,
                                      prefix_len, batch, block_size,
                                      static_cast<float2*>(workspace), accept_len, commit_len,
                                      out_tokens, next_anchor, new_seq_len,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "accept from logits");
  return DFLASH_OK;
}

size_t dflash_accept_sampling_workspace_bytes(int32_t batch, int32_t block_size, int32_t vocab,
                                              int32_t has_draft_logits) {
  if (batch <= 0 || block_size < 2 || block_size > 64 || vocab <= 0 || vocab > 524288) return 0;
  return plan_spec(batch, block_size, vocab, has_draft_logits != 0).bytes;
}

dflash_status dflash_accept_sampling(const int32_t* candidates, const void* target_logits,
                                     const void* draft_logits, int32_t logits_dtype,
                                     int32_t vocab, float target_temperature,
                                     float draft_temperature, const float* uniforms,
                                     const int32_t* prefix_len, int32_t batch,
                                     int32_t block_size, int32_t* accept_len,
                                     int32_t* commit_len, int32_t* out_tokens,
                                     int32_t* next_anchor, int32_t* new_seq_len, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (batch < 0) return fail(DFLASH_EINVAL, "batch %d < 0", batch);
  if (block_size < 2 || block_size > 64)
    return fail(DFLASH_EUNSUPPORTED, "block_size %d outside 2..64", block_size);
  if (vocab <= 0) return fail(DFLASH_EINVAL, "vocab %d <= 0", vocab);
  if (vocab > 524288) return fail(DFLASH_EUNSUPPORTED, "vocab %d > 524288", vocab);
  if (logits_dtype != DFLASH_F32 && logits_dtype != DFLASH_BF16)
    return fail(DFLASH_EUNSUPPORTED, "logits_dtype %d (supported: F32, BF16)", logits_dtype);
  if (!(target_temperature > 0.f) || !isfinite(target_temperature))
    return fail(DFLASH_EINVAL, "target_temperature must be finite and > 0");
  if (draft_logits && (!(draft_temperature > 0.f) || !isfinite(draft_temperature)))
    return fail(DFLASH_EINVAL, "draft_temperature must be finite and > 0");
  if ((int64_t)batch * (2 * block_size - 1) > (int64_t)1 << 30)
    return fail(DFLASH_EUNSUPPORTED, "batch %d too large", batch);
  if (batch == 0) return DFLASH_OK;
  if (!candidates || !target_logits || !uniforms || !prefix_len || !accept_len || !commit_len ||
      !out_tokens || !next_anchor || !new_seq_len)
    return fail(DFLASH_EINVAL, "NULL pointer argument");
  const SpecPlan pl = plan_spec(batch, block_size, vocab, draft_logits != nullptr);
  if (workspace == nullptr || workspace_bytes < pl.bytes)
    return fail(DFLASH_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, pl.bytes);
  if (!aligned16(workspace)) return fail(DFLASH_EINVAL, "workspace is not 16-byte aligned");
  // 16-byte loads when every row starts on a 16-byte boundary
  const int esz = logits_dtype == DFLASH_BF16 ? 2 : 4;
  int vec = 16 / esz;
  if (vocab % vec || !aligned16(target_logits) || (draft_logits && !aligned16(draft_logits)))
    vec = 1;
  const double log2e = 1.4426950408889634;
  const float ct = (float)(log2e / (double)target_temperature);
  const float cd = draft_logits ? (float)(log2e / (double)draft_temperature) : 0.f;
  hipError_t e = launch_accept_sampling(logits_dtype, vec, candidates, target_logits, draft_logits,
                                        nullptr, nullptr, 0, uniforms, prefix_len, batch,
                                        block_size, vocab, ct, cd, pl,
                                        workspace, accept_len, commit_len, out_tokens,
                                        next_anchor, new_seq_len,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "accept_sampling");
  return DFLASH_OK;
}

}  // extern "C"
