// C ABI of the HiLS-Attention forward pass (declared in include/hils.h):
// argument validation on the host, workspace layout, launch geometry and
// HIP error mapping.  Nothing here allocates memory or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/hils.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

hils_status fail(hils_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

hils_status hip_fail(hipError_t e, const char *what) {
  return fail(HILS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

float tau_of(const hils_config *c) {
  return c->scale > 0.f ? c->scale : 1.0f / std::sqrt(static_cast<float>(c->head_dim));
}

size_t elem_bytes(const hils_config *c) { return c->dtype == HILS_BF16 ? 2 : 4; }

int eligible(int i, int W, int S) {
  int w0 = i - W + 1;
  return w0 > 0 ? w0 / S : 0;
}

// Checks shared by every call.
hils_status check_config(const hils_config *c) {
  if (!c) return fail(HILS_ERR_INVALID_ARG, "config is NULL");
  if (c->batch < 1 || c->seq_len < 1) return fail(HILS_ERR_INVALID_ARG, "batch and seq_len must be >= 1");
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads != 0)
    return fail(HILS_ERR_INVALID_ARG, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                c->n_q_heads, c->n_kv_heads);
  if (c->n_q_heads / c->n_kv_heads > 16) return fail(HILS_ERR_UNSUPPORTED, "GQA group size above 16");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(HILS_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->chunk_size != 64) return fail(HILS_ERR_UNSUPPORTED, "chunk_size must be 64");
  if (c->top_k < 0) return fail(HILS_ERR_INVALID_ARG, "top_k must be >= 0");
  if (c->top_k > 32) return fail(HILS_ERR_UNSUPPORTED, "top_k above 32");
  if (c->window < 1) return fail(HILS_ERR_INVALID_ARG, "window must be >= 1");
  if (c->qcal_rank < 0) return fail(HILS_ERR_INVALID_ARG, "qcal_rank must be >= 0");
  if (c->qcal_rank > 64) return fail(HILS_ERR_UNSUPPORTED, "qcal_rank above 64");
  if (c->qcal_rank > 0 && c->hidden_dim < 1) return fail(HILS_ERR_INVALID_ARG, "hidden_dim must be >= 1 with Q-Cal");
  if (c->dtype != HILS_BF16 && c->dtype != HILS_F32) return fail(HILS_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
  if (!(c->scale >= 0.f) || std::isinf(c->scale)) return fail(HILS_ERR_INVALID_ARG, "scale must be finite and >= 0");
  return HILS_OK;
}

hils_status check_ptr(const void *p, const char *name) {
  if (!p) return fail(HILS_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(HILS_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return HILS_OK;
}

#define CHECK(expr)                      \
  do {                                   \
    hils_status s_ = (expr);             \
    if (s_ != HILS_OK) return s_;        \
  } while (0)

hils_status check_qcal_ptrs(const hils_config *c, const void *h, const void *wd, const void *wu) {
  if (c->qcal_rank == 0) {
    if (h || wd || wu) return fail(HILS_ERR_INVALID_ARG, "h, w_down and w_up must be NULL when qcal_rank == 0");
    return HILS_OK;
  }
  CHECK(check_ptr(h, "h"));
  CHECK(check_ptr(wd, "w_down"));
  CHECK(check_ptr(wu, "w_up"));
  return HILS_OK;
}

// ------------------------------------------------------------ decode geometry
struct DecodeGeom {
  int P, NW, nslots, nslot_blocks;
  size_t off_counts, off_qhat, off_sig, off_hsc, off_smax, off_parts, total;
};

constexpr int kDecodeCPB = 64;      // chunks per score slice
constexpr int kMaxSlotRows = 2040;  // partial records one combine step holds in LDS

hils_status decode_geom(const hils_config *c, DecodeGeom *g) {
  const int G = c->n_q_heads / c->n_kv_heads, K = c->top_k, S = c->chunk_size;
  const int nmax = eligible(c->seq_len - 1, c->window, S);
  g->P = nmax > 0 ? (nmax + kDecodeCPB - 1) / kDecodeCPB : 1;
  g->NW = (c->window + S - 1 + 63) / 64;
  g->nslots = K + g->NW;
  if (g->nslots * G > kMaxSlotRows)
    return fail(HILS_ERR_UNSUPPORTED, "decode: (top_k + window units) x group = %d exceeds %d", g->nslots * G,
                kMaxSlotRows);
  g->nslot_blocks = K > 0 ? K : 1;
  const size_t B = c->batch, Hkv = c->n_kv_heads, Hq = c->n_q_heads, D = c->head_dim;
  size_t off = 0;
  const size_t Cmax = static_cast<size_t>(c->seq_len / S);
  g->off_counts = off;
  off = align_up(off + sizeof(unsigned) * (B * Hkv + 1));
  g->off_qhat = off;
  if (c->qcal_rank > 0) off = align_up(off + sizeof(float) * B * Hq * D);
  g->off_sig = off;
  off = align_up(off + sizeof(float) * B * Hkv * Cmax);
  g->off_hsc = off;
  off = align_up(off + sizeof(float) * B * Hkv * Cmax * G);
  g->off_smax = off;
  off = align_up(off + sizeof(float) * B * Hkv * g->P);
  g->off_parts = off;
  off = align_up(off + sizeof(float) * B * Hkv * g->nslots * G * (D + 2));
  g->total = off;
  return HILS_OK;
}

struct DenseGeom {
  int P, L;
  size_t off_counts, off_parts, total;
};

void dense_geom(const hils_config *c, DenseGeom *g) {
  const long long T = c->seq_len;
  const long long units = (T + 63) / 64;
  const long long G = c->n_q_heads / c->n_kv_heads;
  long long per_seq_target = 4096 / (static_cast<long long>(c->batch) * c->n_kv_heads) + 1;
  if (per_seq_target > kMaxSlotRows / G) per_seq_target = kMaxSlotRows / G;
  long long upb = (units + per_seq_target - 1) / per_seq_target;  // units per block
  if (upb < 4) upb = 4;
  g->L = static_cast<int>(upb * 64);
  g->P = static_cast<int>((T + g->L - 1) / g->L);
  const size_t B = c->batch, Hkv = c->n_kv_heads, D = c->head_dim;
  g->off_counts = 0;
  g->off_parts = align_up(sizeof(unsigned) * (B * Hkv + 1));
  g->total = align_up(g->off_parts + sizeof(float) * B * Hkv * g->P * G * (D + 2));
}

size_t prefill_u_bytes(const hils_config *c) {
  return c->qcal_rank > 0 ? align_up(sizeof(float) * c->batch * static_cast<size_t>(c->seq_len) * c->qcal_rank) : 0;
}

hils_status finish(hipError_t e, const char *what) {
  if (e != hipSuccess) return hip_fail(e, what);
  return HILS_OK;
}

// Paged caches: pages of S keys of every KV head, [num_pages, H_kv, S, d];
// every position below seq_len (the per-sequence capacity) needs a slot of
// the block table.
hils_status check_pages(const hils_config *c, const int32_t *block_table, int32_t max_pages, int32_t num_pages) {
  if (!block_table) return fail(HILS_ERR_INVALID_ARG, "block_table is NULL");
  if (num_pages < 1) return fail(HILS_ERR_INVALID_ARG, "num_pages must be >= 1 (got %d)", num_pages);
  const long long need = (static_cast<long long>(c->seq_len) + c->chunk_size - 1) / c->chunk_size;
  if (max_pages < need)
    return fail(HILS_ERR_INVALID_ARG, "max_pages (%d) below the %lld pages of seq_len %d", max_pages, need,
                c->seq_len);
  return HILS_OK;
}

hils_status summary_impl(const hils_config *cfg, const void *k, const int32_t *block_table, int32_t max_pages,
                         int32_t num_pages, const void *q_lm, int32_t chunk_begin, int32_t chunk_end, void *k_sum,
                         float *b_sum, void *stream) {
  const int C = cfg->seq_len / cfg->chunk_size;
  if (chunk_begin < 0 || chunk_end < chunk_begin || chunk_end > C)
    return fail(HILS_ERR_INVALID_ARG, "chunk range [%d, %d) outside [0, %d]", chunk_begin, chunk_end, C);
  if (chunk_end == chunk_begin) return HILS_OK;
  CHECK(check_ptr(k, block_table ? "k_pages" : "k"));
  CHECK(check_ptr(q_lm, "q_lm"));
  CHECK(check_ptr(k_sum, "k_sum"));
  CHECK(check_ptr(b_sum, "b_sum"));
  hils::SummaryArgs a{k, q_lm, k_sum, b_sum, cfg->batch, cfg->seq_len, cfg->n_q_heads, cfg->n_kv_heads, C,
                      cfg->head_dim, chunk_begin, chunk_end, tau_of(cfg), cfg->dtype == HILS_BF16,
                      block_table, max_pages, num_pages};
  return finish(hils::launch_summary(a, static_cast<hipStream_t>(stream)), "landmark summary launch");
}

hils_status decode_impl(const hils_config *cfg, const void *q, const void *h, const void *w_down, const void *w_up,
                        const void *k_cache, const void *v_cache, const int32_t *block_table, int32_t max_pages,
                        int32_t num_pages, const void *k_sum, const float *b_sum, const int32_t *seq_lens, void *o,
                        int32_t *topk_idx, float *topk_score, void *workspace, size_t workspace_bytes,
                        void *stream);

}  // namespace

extern "C" {

const char *hils_status_string(hils_status s) {
  switch (s) {
    case HILS_OK: return "HILS_OK";
    case HILS_ERR_INVALID_ARG: return "HILS_ERR_INVALID_ARG";
    case HILS_ERR_UNSUPPORTED: return "HILS_ERR_UNSUPPORTED";
    case HILS_ERR_WORKSPACE: return "HILS_ERR_WORKSPACE";
    case HILS_ERR_HIP: return "HILS_ERR_HIP";
  }
  return "unknown hils_status";
}

const char *hils_last_error(void) { return g_last_error.c_str(); }

hils_status hils_landmark_summary(const hils_config *cfg, const void *k, const void *q_lm, int32_t chunk_begin,
                                  int32_t chunk_end, void *k_sum, float *b_sum, void *stream) {
  g_last_error.clear();
  CHECK(check_config(cfg));
  return summary_impl(cfg, k, nullptr, 0, 0, q_lm, chunk_begin, chunk_end, k_sum, b_sum, stream);
}

hils_status hils_landmark_summary_paged(const hils_config *cfg, const void *k_pages, const int32_t *block_table,
                                        int32_t max_pages, int32_t num_pages, const void *q_lm, int32_t chunk_begin,
                                        int32_t chunk_end, void *k_sum, float *b_sum, void *stream) {
  g_last_error.clear();
  CHECK(check_config(cfg));
  CHECK(check_pages(cfg, block_table, max_pages, num_pages));
  return summary_impl(cfg, k_pages, block_table, max_pages, num_pages, q_lm, chunk_begin, chunk_end, k_sum, b_sum,
                      stream);
}

size_t hils_prefill_workspace_bytes(const hils_config *cfg) {
  if (check_config(cfg) != HILS_OK) return 0;
  const int C = cfg->seq_len / cfg->chunk_size;
  // scoring uses the workspace first; the attention call then reuses it for
  // the K/V operand-order copy and row statistics of its MFMA path (bf16)
  const size_t score = prefill_u_bytes(cfg) +
                       align_up(hils::score_mfma_ws_bytes(cfg->batch, cfg->seq_len, cfg->n_q_heads, C, cfg->qcal_rank)) +
                       kAlign;
  const size_t attn = cfg->dtype == HILS_BF16
                          ? align_up(hils::attn_mfma_ws_bytes(cfg->batch, cfg->n_q_heads, cfg->n_kv_heads, cfg->seq_len,
                                              cfg->head_dim, cfg->top_k))
                          : 0;
  return score > attn ? score : attn;
}

hils_status hils_chunk_score_topk(const hils_config *cfg, const void *q, const void *h, const void *w_down,
                                  const void *w_up, const void *k_sum, const float *b_sum, int32_t *topk_idx,
                                  float *topk_score, void *workspace, size_t workspace_bytes, void *stream) {
  g_last_error.clear();
  CHECK(check_config(cfg));
  CHECK(check_ptr(q, "q"));
  CHECK(check_qcal_ptrs(cfg, h, w_down, w_up));
  const int C = cfg->seq_len / cfg->chunk_size;
  if (C > 0) {
    CHECK(check_ptr(k_sum, "k_sum"));
    CHECK(check_ptr(b_sum, "b_sum"));
  }
  if (cfg->top_k > 0) {
    CHECK(check_ptr(topk_idx, "topk_idx"));
    CHECK(check_ptr(topk_score, "topk_score"));
  }
  if (C > 8192) return fail(HILS_ERR_UNSUPPORTED, "prefill scoring supports at most 8192 chunks (got %d)", C);
  const size_t need = hils_prefill_workspace_bytes(cfg);
  if (!workspace || workspace_bytes < need)
    return fail(HILS_ERR_WORKSPACE, "prefill workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (cfg->top_k == 0) return HILS_OK;
  hils::ScoreArgs a{q, h, w_down, w_up, k_sum, b_sum, topk_idx, topk_score, static_cast<float *>(workspace),
                    static_cast<char *>(workspace) + prefill_u_bytes(cfg), cfg->batch, cfg->seq_len,
                    cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim, cfg->chunk_size, cfg->top_k, cfg->window,
                    cfg->qcal_rank, cfg->hidden_dim, C, tau_of(cfg), cfg->dtype == HILS_BF16};
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hils::score_mfma_supported(a)) return finish(hils::launch_score_mfma(a, st), "chunk score/top-k launch");
  return finish(hils::launch_score_valu(a, st), "chunk score/top-k launch");
}

hils_status hils_sparse_attn_prefill(const hils_config *cfg, const void *q, const void *k, const void *v,
                                     const int32_t *topk_idx, const float *topk_score, void *o, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  g_last_error.clear();
  CHECK(check_config(cfg));
  CHECK(check_ptr(q, "q"));
  CHECK(check_ptr(k, "k"));
  CHECK(check_ptr(v, "v"));
  CHECK(check_ptr(o, "o"));
  if (cfg->top_k > 0) {
    CHECK(check_ptr(topk_idx, "topk_idx"));
    CHECK(check_ptr(topk_score, "topk_score"));
  }
  const size_t need = hils_prefill_workspace_bytes(cfg);
  if (!workspace || workspace_bytes < need)
    return fail(HILS_ERR_WORKSPACE, "prefill workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  hils::AttnArgs a{q, k, v, topk_idx, topk_score, o, workspace, cfg->batch, cfg->seq_len, cfg->n_q_heads,
                   cfg->n_kv_heads, cfg->head_dim, cfg->chunk_size, cfg->top_k, cfg->window, tau_of(cfg),
                   cfg->dtype == HILS_BF16, nullptr};
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hils::attn_mfma_supported(a)) return finish(hils::launch_attn_mfma(a, st), "sparse attention launch");
  return finish(hils::launch_attn_valu(a, st), "sparse attention launch");
}

// ------------------------------------------------------------ backward
namespace {

struct BwdGeom {
  size_t off_u, off_du, off_qhat, off_dqhat, off_logz, off_delta, off_lw, off_doo, off_ds, off_z, off_zb, off_gpart;
  size_t off_cnt, off_qboff, off_choff, off_list, off_pos, total;
};

BwdGeom bwd_geom(const hils_config *c) {
  const size_t B = c->batch, T = c->seq_len, Hq = c->n_q_heads, Hkv = c->n_kv_heads, d = c->head_dim;
  const size_t K = c->top_k, r = c->qcal_rank, C = T / c->chunk_size, nqb = (T + 255) / 256;
  BwdGeom g{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  g.off_u = take(sizeof(float) * B * T * r);
  g.off_du = take(sizeof(float) * B * T * r);
  g.off_qhat = take(r ? sizeof(float) * B * Hq * T * d : 0);
  g.off_dqhat = take(r ? sizeof(float) * B * Hq * T * d : 0);
  g.off_logz = take(sizeof(float) * B * Hq * T);
  g.off_delta = take(sizeof(float) * B * Hq * T);
  g.off_lw = take(sizeof(float) * B * Hq * T * K);  // per list entry and head: B Hkv (T K) G
  g.off_doo = take(sizeof(float) * B * Hq * T * K);
  g.off_ds = take(sizeof(float) * B * Hq * T * K);
  g.off_z = take(sizeof(float) * B * Hq * C * r);
  g.off_zb = take(sizeof(float) * B * Hq * C);
  const size_t Dh = c->qcal_rank ? c->hidden_dim : 0;
  size_t gp = hils::kBwdSplitW * (Hq * d * r > r * Dh ? Hq * d * r : r * Dh);
  if (hils::kBwdSplitDu * B * T * r > gp) gp = hils::kBwdSplitDu * B * T * r;
  g.off_gpart = take(sizeof(float) * gp);
  g.off_cnt = take(sizeof(int32_t) * B * Hkv * nqb * C);
  g.off_qboff = take(sizeof(int32_t) * B * Hkv * nqb * C);
  g.off_choff = take(sizeof(int32_t) * B * Hkv * (C + 1));
  g.off_list = take(sizeof(int32_t) * B * Hkv * T * K);
  g.off_pos = take(sizeof(int32_t) * B * Hkv * T * K);
  g.total = o + kAlign;
  return g;
}

hils_status check_backward_shape(const hils_config *c) {
  const int C = c->seq_len / c->chunk_size;
  if (C > hils::kMaxBwdChunks)
    return fail(HILS_ERR_UNSUPPORTED, "backward supports at most %d chunks (T <= %d), got %d", hils::kMaxBwdChunks,
                hils::kMaxBwdChunks * c->chunk_size, C);
  return HILS_OK;
}

}  // namespace

size_t hils_backward_workspace_bytes(const hils_config *cfg) {
  if (check_config(cfg) != HILS_OK || check_backward_shape(cfg) != HILS_OK) return 0;
  return bwd_geom(cfg).total;
}

hils_status hils_sparse_attn_backward(const hils_config *cfg, const void *q, const void *k, const void *v,
                                      const void *q_lm, const void *h, const void *w_down, const void *w_up,
                                      const void *k_sum, const float *b_sum, const int32_t *topk_idx,
                                      const void *d_o, float *dq, float *dk, float *dv, float *dq_lm, float *dh,
                                      float *dw_down, float *dw_up, void *workspace, size_t workspace_bytes,
                                      void *stream) {
  g_last_error.clear();
  CHECK(check_config(cfg));
  CHECK(check_backward_shape(cfg));
  CHECK(check_ptr(q, "q"));
  CHECK(check_ptr(k, "k"));
  CHECK(check_ptr(v, "v"));
  CHECK(check_ptr(d_o, "d_o"));
  CHECK(check_ptr(dq, "dq"));
  CHECK(check_ptr(dk, "dk"));
  CHECK(check_ptr(dv, "dv"));
  CHECK(check_qcal_ptrs(cfg, h, w_down, w_up));
  if (cfg->qcal_rank == 0) {
    if (dh || dw_down || dw_up)
      return fail(HILS_ERR_INVALID_ARG, "dh, dw_down and dw_up must be NULL when qcal_rank == 0");
  } else {
    CHECK(check_ptr(dh, "dh"));
    CHECK(check_ptr(dw_down, "dw_down"));
    CHECK(check_ptr(dw_up, "dw_up"));
  }
  const int C = cfg->seq_len / cfg->chunk_size;
  if (C > 0) {
    CHECK(check_ptr(q_lm, "q_lm"));
    CHECK(check_ptr(dq_lm, "dq_lm"));
    if (cfg->top_k > 0) {
      CHECK(check_ptr(k_sum, "k_sum"));
      CHECK(check_ptr(b_sum, "b_sum"));
    }
  }
  if (cfg->top_k > 0) CHECK(check_ptr(topk_idx, "topk_idx"));
  const BwdGeom g = bwd_geom(cfg);
  if (!workspace || workspace_bytes < g.total)
    return fail(HILS_ERR_WORKSPACE, "backward workspace of %zu bytes given, %zu needed", workspace_bytes, g.total);
  if (!aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  char *ws = static_cast<char *>(workspace);
  auto f = [&](size_t off) { return reinterpret_cast<float *>(ws + off); };
  auto n = [&](size_t off) { return reinterpret_cast<int32_t *>(ws + off); };
  hils::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.q_lm = q_lm; a.h = h; a.w_down = w_down; a.w_up = w_up;
  a.k_sum = k_sum; a.d_o = d_o; a.b_sum = b_sum; a.topk_idx = topk_idx;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dq_lm = dq_lm; a.dh = dh; a.dw_down = dw_down; a.dw_up = dw_up;
  a.u = f(g.off_u); a.du = f(g.off_du); a.qhat = f(g.off_qhat); a.dqhat = f(g.off_dqhat);
  a.logz = f(g.off_logz); a.delta = f(g.off_delta);
  a.ent_lw = f(g.off_lw); a.ent_doo = f(g.off_doo); a.ent_ds = f(g.off_ds);
  a.zsum = f(g.off_z); a.zb = f(g.off_zb); a.gpart = f(g.off_gpart);
  a.inv_cnt = n(g.off_cnt); a.inv_qboff = n(g.off_qboff); a.inv_choff = n(g.off_choff); a.inv_list = n(g.off_list);
  a.inv_pos = n(g.off_pos);
  a.B = cfg->batch; a.T = cfg->seq_len; a.Hq = cfg->n_q_heads; a.Hkv = cfg->n_kv_heads; a.d = cfg->head_dim;
  a.K = cfg->top_k; a.W = cfg->window; a.r = cfg->qcal_rank; a.Dh = cfg->hidden_dim;
  a.tau = tau_of(cfg);
  a.bf16 = cfg->dtype == HILS_BF16;
  return finish(hils::launch_backward(a, static_cast<hipStream_t>(stream)), "backward launch");
}

size_t hils_decode_workspace_bytes(const hils_config *cfg) {
  if (check_config(cfg) != HILS_OK) return 0;
  DecodeGeom g;
  if (decode_geom(cfg, &g) != HILS_OK) return 0;
  return g.total;
}

size_t hils_decode_error_offset(const hils_config *cfg) {
  if (check_config(cfg) != HILS_OK) return 0;
  return sizeof(unsigned) * static_cast<size_t>(cfg->batch) * cfg->n_kv_heads;
}

hils_status hils_sparse_attn_decode(const hils_config *cfg, const void *q, const void *h, const void *w_down,
                                    const void *w_up, const void *k_cache, const void *v_cache, const void *k_sum,
                                    const float *b_sum, const int32_t *seq_lens, void *o, int32_t *topk_idx,
                                    float *topk_score, void *workspace, size_t workspace_bytes, void *stream) {
  g_last_error.clear();
  CHECK(check_config(cfg));
  return decode_impl(cfg, q, h, w_down, w_up, k_cache, v_cache, nullptr, 0, 0, k_sum, b_sum, seq_lens, o, topk_idx,
                     topk_score, workspace, workspace_bytes, stream);
}

hils_status hils_sparse_attn_decode_paged(const hils_config *cfg, const void *q, const void *h, const void *w_down,
                                          const void *w_up, const void *k_pages, const void *v_pages,
                                          const int32_t *block_table, int32_t max_pages, int32_t num_pages,
                                          const void *k_sum, const float *b_sum, const int32_t *seq_lens, void *o,
                                          int32_t *topk_idx, float *topk_score, void *workspace,
                                          size_t workspace_bytes, void *stream) {
  g_last_error.clear();
  CHECK(check_config(cfg));
  CHECK(check_pages(cfg, block_table, max_pages, num_pages));
  return decode_impl(cfg, q, h, w_down, w_up, k_pages, v_pages, block_table, max_pages, num_pages, k_sum, b_sum,
                     seq_lens, o, topk_idx, topk_score, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

hils_status decode_impl(const hils_config *cfg, const void *q, const void *h, const void *w_down, const void *w_up,
                        const void *k_cache, const void *v_cache, const int32_t *block_table, int32_t max_pages,
                        int32_t num_pages, const void *k_sum, const float *b_sum, const int32_t *seq_lens, void *o,
                        int32_t *topk_idx, float *topk_score, void *workspace, size_t workspace_bytes,
                        void *stream) {
  CHECK(check_ptr(q, "q"));
  CHECK(check_qcal_ptrs(cfg, h, w_down, w_up));
  CHECK(check_ptr(k_cache, block_table ? "k_pages" : "k_cache"));
  CHECK(check_ptr(v_cache, block_table ? "v_pages" : "v_cache"));
  const int Cmax = cfg->seq_len / cfg->chunk_size;
  if (Cmax > 0) {
    CHECK(check_ptr(k_sum, "k_sum"));
    CHECK(check_ptr(b_sum, "b_sum"));
  }
  if (!seq_lens) return fail(HILS_ERR_INVALID_ARG, "seq_lens is NULL");
  CHECK(check_ptr(o, "o"));
  if (cfg->top_k > 0) {
    CHECK(check_ptr(topk_idx, "topk_idx"));
    CHECK(check_ptr(topk_score, "topk_score"));
  }
  DecodeGeom g;
  CHECK(decode_geom(cfg, &g));
  if (!workspace || workspace_bytes < g.total)
    return fail(HILS_ERR_WORKSPACE, "decode workspace of %zu bytes given, %zu needed", workspace_bytes, g.total);
  if (!aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  char *ws = static_cast<char *>(workspace);
  const size_t BH = static_cast<size_t>(cfg->batch) * cfg->n_kv_heads;
  unsigned *counts = reinterpret_cast<unsigned *>(ws + g.off_counts);
  hils::DecodeArgs a{};
  a.q = q; a.h = h; a.w_down = w_down; a.w_up = w_up; a.k_cache = k_cache; a.v_cache = v_cache;
  a.k_sum = k_sum; a.b_sum = b_sum; a.seq_lens = seq_lens; a.o = o; a.topk_idx = topk_idx;
  a.topk_score = topk_score;
  a.qhat = reinterpret_cast<float *>(ws + g.off_qhat);
  a.sig = reinterpret_cast<float *>(ws + g.off_sig);
  a.hsc = reinterpret_cast<float *>(ws + g.off_hsc);
  a.smax = reinterpret_cast<float *>(ws + g.off_smax);
  a.parts = reinterpret_cast<float *>(ws + g.off_parts);
  a.count = counts; a.err = counts + BH;
  a.B = cfg->batch; a.Tmax = cfg->seq_len; a.Hq = cfg->n_q_heads; a.Hkv = cfg->n_kv_heads;
  a.d = cfg->head_dim; a.S = cfg->chunk_size; a.K = cfg->top_k; a.W = cfg->window;
  a.r = cfg->qcal_rank; a.Dh = cfg->hidden_dim; a.Cmax = Cmax;
  a.P = g.P; a.NW = g.NW; a.nslots = g.nslots; a.nslot_blocks = g.nslot_blocks;
  a.tau = tau_of(cfg); a.bf16 = cfg->dtype == HILS_BF16;
  a.block_table = block_table; a.max_pages = max_pages; a.num_pages = num_pages;
  return finish(hils::launch_decode(a, static_cast<hipStream_t>(stream)), "sparse decode launch");
}

}  // namespace

extern "C" {

size_t hils_dense_decode_workspace_bytes(const hils_config *cfg) {
  if (check_config(cfg) != HILS_OK) return 0;
  DenseGeom g;
  dense_geom(cfg, &g);
  return g.total;
}

hils_status hils_dense_attn_decode(const hils_config *cfg, const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *seq_lens, void *o, void *workspace, size_t workspace_bytes,
                                   void *stream) {
  g_last_error.clear();
  CHECK(check_config(cfg));
  CHECK(check_ptr(q, "q"));
  CHECK(check_ptr(k_cache, "k_cache"));
  CHECK(check_ptr(v_cache, "v_cache"));
  if (!seq_lens) return fail(HILS_ERR_INVALID_ARG, "seq_lens is NULL");
  CHECK(check_ptr(o, "o"));
  DenseGeom g;
  dense_geom(cfg, &g);
  if (!workspace || workspace_bytes < g.total)
    return fail(HILS_ERR_WORKSPACE, "dense decode workspace of %zu bytes given, %zu needed", workspace_bytes, g.total);
  if (!aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  char *ws = static_cast<char *>(workspace);
  unsigned *counts = reinterpret_cast<unsigned *>(ws + g.off_counts);
  const size_t BH = static_cast<size_t>(cfg->batch) * cfg->n_kv_heads;
  hils::DenseArgs a{q, k_cache, v_cache, seq_lens, o, reinterpret_cast<float *>(ws + g.off_parts), counts,
                    counts + BH, cfg->batch, cfg->seq_len, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim,
                    g.P, g.L, tau_of(cfg), cfg->dtype == HILS_BF16};
  return finish(hils::launch_dense_decode(a, static_cast<hipStream_t>(stream)), "dense decode launch");
}

}  // extern "C"

// ------------------------------------------------------------ allocation-free decode
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops): the decode step's scratch -- group scores,
// per-head scores, slice maxima, partial records, arrival tickets -- lives
// in one file-scope device array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy of the array until the process
// ends.  Its address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels; the
// array's name in host code is a host-side stand-in, not a device address.
namespace {

constexpr size_t kScratchBytes = size_t(48) << 20;  // 48 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hils_status scratch_for_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HILS_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(HILS_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HILS_OK;
}

// Zeroes the first n words of the scratch (the arrival tickets and the error
// word): a kernel rather than hipMemsetAsync, so the step stays correct when
// a caller captures it into a graph and replays it.
__global__ void zero_words_kernel(unsigned *p, int n) {
  for (int x = blockIdx.x * blockDim.x + threadIdx.x; x < n; x += gridDim.x * blockDim.x) p[x] = 0u;
}

}  // namespace

extern "C" {

size_t hils_noalloc_scratch_bytes(void) { return kScratchBytes; }

hils_status hils_sparse_attn_decode_noalloc(const hils_config *cfg, const void *q, const void *h, const void *w_down,
                                            const void *w_up, const void *k_cache, const void *v_cache,
                                            const void *k_sum, const float *b_sum, const int32_t *seq_lens, void *o,
                                            int32_t *topk_idx, float *topk_score, void *stream) {
  g_last_error.clear();
  CHECK(check_config(cfg));
  DecodeGeom g;
  CHECK(decode_geom(cfg, &g));
  if (g.total > kScratchBytes)
    return fail(HILS_ERR_UNSUPPORTED,
                "decode scratch of %zu bytes needed, the allocation-free call holds %zu (use "
                "hils_sparse_attn_decode with a workspace)",
                g.total, kScratchBytes);
  void *ws = nullptr;
  CHECK(scratch_for_current_device(&ws));
  // the previous call may have had another batch or head count, so its
  // tickets and error word need not sit where this call's do
  const int nwords = static_cast<int>(static_cast<size_t>(cfg->batch) * cfg->n_kv_heads + 1);
  hipStream_t st = static_cast<hipStream_t>(stream);
  zero_words_kernel<<<1, 256, 0, st>>>(static_cast<unsigned *>(ws), nwords);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "scratch clear launch");
  return decode_impl(cfg, q, h, w_down, w_up, k_cache, v_cache, nullptr, 0, 0, k_sum, b_sum, seq_lens, o, topk_idx,
                     topk_score, ws, g.total, stream);
}

}  // extern "C"
