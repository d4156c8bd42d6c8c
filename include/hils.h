/*
 * hils.h -- C ABI of the HiLS-Attention forward pass for AMD Instinct MI355X
 * (gfx950).
 *
 * HiLS-Attention ("Hierarchical Sparse Attention Done Right: Toward Infinite
 * Context Modeling", arXiv 2607.02980) splits the context into chunks of S
 * tokens, summarises each chunk with a landmark query, scores every chunk for
 * each query, keeps the top-K chunks per GQA group, attends inside each kept
 * chunk and fuses the chunk outputs with a sliding-window term under one
 * normaliser.  Section references below are to the pages on that paper:
 *   [p1] picx.dev summary, Methodology 1-3 (Eq. 7, 8, 10);
 *   [p3] rcap.io explainer, per-query pseudo-code and recipe.
 *
 * Conventions shared by every call
 *   Memory      Every tensor pointer is a DEVICE pointer (hipMalloc or a torch
 *               CUDA/HIP tensor), contiguous, in the layouts stated per call,
 *               16-byte aligned.  The caller owns every buffer.  The library
 *               allocates nothing and keeps no state between calls; the only
 *               persistent objects are the caller-owned decode workspace and
 *               the fixed scratch array of the allocation-free decode call.
 *   Streams     `stream` is a hipStream_t passed as void* (NULL = the default
 *               stream).  Calls only enqueue work; outputs are valid once the
 *               stream has been synchronised.  No call synchronises the host.
 *   Types       hils_config.dtype names the element type of q, k, v, q_lm, h,
 *               w_down, w_up, k_sum and o: HILS_BF16 (raw bf16) or HILS_F32.
 *               b_sum and topk_score are always float32, topk_idx int32.
 *   Shapes      B batch, T tokens (prefill) or cache capacity T_max (decode),
 *               H_q query heads, H_kv KV heads (H_q % H_kv == 0, G = H_q/H_kv),
 *               d head dim, S chunk size, C = floor(T/S) complete chunks,
 *               K top-k, W window, r Q-Cal rank, D_h hidden size.
 *               Query head h belongs to group g = h / G.
 *   Partition   For a query at position i: w0 = max(0, i-W+1); the n_i =
 *               floor(w0/S) complete chunks before the window are eligible
 *               for selection; the window is the token range [n_i*S, i].
 *               Chunks and window thus split [0, i] exactly.
 *   Errors      Arguments are checked on the host before anything is
 *               enqueued; a failed check returns a negative hils_status and
 *               launches nothing.  hils_last_error() gives a thread-local
 *               description of the last failure.  No C++ exception crosses
 *               the ABI.
 */
#ifndef HILS_H_
#define HILS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HILS_OK = 0,
  HILS_ERR_INVALID_ARG = -1, /* null pointer, bad shape, misaligned buffer   */
  HILS_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels support   */
  HILS_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
  HILS_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed    */
} hils_status;

typedef enum { HILS_BF16 = 0, HILS_F32 = 1 } hils_dtype;

typedef struct {
  int32_t batch;       /* B >= 1                                              */
  int32_t seq_len;     /* prefill: T >= 1; decode: cache capacity T_max >= 1  */
  int32_t n_q_heads;   /* H_q >= 1                                            */
  int32_t n_kv_heads;  /* H_kv >= 1, divides H_q; G = H_q / H_kv <= 16        */
  int32_t head_dim;    /* d: 64 or 128                                        */
  int32_t chunk_size;  /* S: 64                                               */
  int32_t top_k;       /* K: 0..32                                            */
  int32_t window;      /* W >= 1                                              */
  int32_t qcal_rank;   /* r: 0 (Q-Cal off) .. 64                              */
  int32_t hidden_dim;  /* D_h (Q-Cal input width); ignored when r == 0       */
  int32_t dtype;       /* hils_dtype                                          */
  float scale;         /* logit scale tau; 0 selects 1/sqrt(d)                */
} hils_config;

/*
 * Landmark chunk summary -- [p1] Methodology 1, Eq. 8.
 * For every batch b, query head h and chunk c in [chunk_begin, chunk_end):
 *   p_j     = softmax_j( tau * q_lm[b,h,c] . k[b,g(h),c*S+j] ),  j < S
 *   k_sum   = sum_j p_j k[b,g(h),c*S+j]       (stored in dtype, rounded RNE)
 *   b_sum   = -sum_j p_j log p_j              (float32)
 * so that tau*q.k_sum + b_sum is the first-order expansion of the chunk's
 * log-mass about q = q_lm (Eq. 7).
 *   k      [B, H_kv, T, d]   dtype   keys (post positional encoding)
 *   q_lm   [B, H_q,  C, d]   dtype   landmark queries, one per head and chunk
 *   k_sum  [B, H_q,  C, d]   dtype   out (only chunks in the range written)
 *   b_sum  [B, H_q,  C]      f32     out
 * 0 <= chunk_begin <= chunk_end <= C (an empty range enqueues nothing).
 * Decode callers run it for each chunk as it completes.
 */
hils_status hils_landmark_summary(const hils_config *cfg, const void *k, const void *q_lm,
                                  int32_t chunk_begin, int32_t chunk_end, void *k_sum,
                                  float *b_sum, void *stream);

/* Workspace bytes needed by hils_chunk_score_topk and hils_sparse_attn_prefill
 * for this configuration (one buffer may serve both, used in turn). */
size_t hils_prefill_workspace_bytes(const hils_config *cfg);

/*
 * Chunk scoring and GQA top-K selection for all T prefill queries --
 * [p1] Eq. 7 with Eq. 10's s-hat, Methodology 3 (Q-Cal, GQA adaptation);
 * [p3] pseudo-code (score every chunk, arg-top-K).
 *   q-hat_i = q_i + (w_up (w_down h_i))[h*d : h*d+d]          (when r > 0)
 *   s[b,h,i,c] = tau * q-hat . k_sum[b,h,c] + b_sum[b,h,c],   c < n_i
 *   sigma[c]   = max over the G heads of group g of s[b,h,i,c]
 *   keep min(K, n_i) chunks by (sigma descending, c ascending)
 *   q          [B, H_q, T, d]     dtype
 *   h          [B, T, D_h]        dtype  } all three NULL iff r == 0
 *   w_down     [r, D_h]           dtype  }
 *   w_up       [H_q*d, r]         dtype  }
 *   k_sum      [B, H_q, C, d]     dtype  (from hils_landmark_summary)
 *   b_sum      [B, H_q, C]        f32
 *   topk_idx   [B, H_kv, T, K]    int32  out: chunk ids in selection order, -1 pad
 *   topk_score [B, H_q, T, K]     f32    out: each head's own s of those
 *                                        chunks, -inf pad
 *   workspace  >= hils_prefill_workspace_bytes(cfg) bytes, device memory.
 * C = floor(T/S) may reach 8192 (T = 512K at S = 64; UNSUPPORTED above);
 * sequences of more than 256 chunks stream the summaries and keep a running
 * top-K per query (same result, same order).
 */
hils_status hils_chunk_score_topk(const hils_config *cfg, const void *q, const void *h,
                                  const void *w_down, const void *w_up, const void *k_sum,
                                  const float *b_sum, int32_t *topk_idx, float *topk_score,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Hierarchical sparse attention for all T prefill queries --
 * [p1] Methodology 2, Eq. 10; [p3] pseudo-code (per-chunk attention, fusion
 * by the chunk scores, sliding-window term).  For query i, head h:
 *   o_c   = softmax over chunk c's S keys of tau*q.k, applied to its values
 *   o_win = softmax over the window tokens, applied to their values
 *   o     = ( sum_c e^{s_c} o_c + Z_win o_win ) / ( sum_c e^{s_c} + Z_win )
 * with s_c = topk_score[b,h,i,k] for the selected chunk c = topk_idx[b,g,i,k]
 * and Z_win = sum over window tokens of e^{tau q.k}: one joint normaliser over
 * the selected chunks and the window.  Token logits use the raw q.
 *   q, o       [B, H_q, T, d]   dtype (o out)
 *   k, v       [B, H_kv, T, d]  dtype
 *   topk_idx   [B, H_kv, T, K]  int32 (as written by hils_chunk_score_topk;
 *                               entries must be -1 or eligible chunks < n_i,
 *                               no chunk twice in one list)
 *   topk_score [B, H_q, T, K]   f32
 *   workspace  >= hils_prefill_workspace_bytes(cfg) bytes, device memory
 *              (may be the one given to hils_chunk_score_topk: this call
 *              overwrites it, in stream order, with K and V in the matrix
 *              units' operand order, each 64-key block's largest |v| and each
 *              row's chunk log-mass).
 */
hils_status hils_sparse_attn_prefill(const hils_config *cfg, const void *q, const void *k,
                                     const void *v, const int32_t *topk_idx,
                                     const float *topk_score, void *o, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* Workspace bytes needed by hils_sparse_attn_backward (0 for an invalid or
 * unsupported configuration). */
size_t hils_backward_workspace_bytes(const hils_config *cfg);

/*
 * Backward pass of the prefill forward for a FIXED selection -- the chunk
 * score s-hat sits inside the joint softmax of [p1] Methodology 2 (Eq. 10),
 * so the loss reaches the landmark summary (Methodology 1, Eq. 8), the
 * landmark queries and, with Q-Cal, the calibration weights (Methodology 3);
 * the top-K choice itself is discrete and carries no gradient.  Given
 * d_o = dL/dO, returns the gradients of L = sum(d_o * O) where O is the
 * output of hils_sparse_attn_prefill with topk_score = each head's s-hat of
 * the selected chunks, recomputed here as tau * q-hat . k_sum + b_sum from the
 * STORED summaries (as hils_chunk_score_topk computes it).  The rounding of
 * k_sum to dtype is taken as the identity in the chain rule.
 *   q, d_o     [B, H_q, T, d]   dtype
 *   k, v       [B, H_kv, T, d]  dtype
 *   q_lm       [B, H_q, C, d]   dtype  (NULL allowed iff C == 0)
 *   h, w_down, w_up                    as for hils_chunk_score_topk (NULL iff r == 0)
 *   k_sum      [B, H_q, C, d]   dtype  } the summaries the forward scored;
 *   b_sum      [B, H_q, C]      f32    } NULL allowed iff C == 0 or K == 0
 *   topk_idx   [B, H_kv, T, K]  int32  the forward's selection (-1 pad; an id
 *                                      outside [0, n_i) counts as no chunk)
 * Outputs, all float32 and overwritten (no accumulation into them):
 *   dq [B, H_q, T, d], dk / dv [B, H_kv, T, d], dq_lm [B, H_q, C, d]
 *   (NULL allowed iff C == 0), and with r > 0: dh [B, T, D_h],
 *   dw_down [r, D_h], dw_up [H_q*d, r] (all three NULL iff r == 0).
 *   workspace  >= hils_backward_workspace_bytes(cfg) bytes, device memory.
 * Every sum runs in a fixed order: repeated calls give identical bits.
 * T is limited to 32768 (C <= 512; UNSUPPORTED above).
 */
hils_status hils_sparse_attn_backward(const hils_config *cfg, const void *q, const void *k,
                                      const void *v, const void *q_lm, const void *h,
                                      const void *w_down, const void *w_up, const void *k_sum,
                                      const float *b_sum, const int32_t *topk_idx, const void *d_o,
                                      float *dq, float *dk, float *dv, float *dq_lm, float *dh,
                                      float *dw_down, float *dw_up, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* Bytes of the decode workspace.  The caller zeroes it ONCE after allocating
 * it (hipMemset / torch.zeros); the library leaves its counters at zero after
 * every call.  A decode workspace must not be shared with another call kind
 * or used by two decode calls that may run concurrently. */
size_t hils_decode_workspace_bytes(const hils_config *cfg);

/*
 * One decode step for B sequences -- the same method for a single query per
 * sequence at position i = seq_lens[b] - 1, whose K/V are already in the
 * cache.  Scores every eligible chunk from the stored summaries, keeps the
 * top-K per group, and fuses their attention with the window term (Eq. 10).
 *   q          [B, H_q, d]        dtype
 *   h          [B, D_h]           dtype  } NULL iff r == 0
 *   w_down     [r, D_h], w_up [H_q*d, r] } dtype
 *   k_cache    [B, H_kv, T_max, d] dtype
 *   v_cache    [B, H_kv, T_max, d] dtype
 *   k_sum      [B, H_q, C_max, d] dtype  C_max = floor(T_max/S); chunks < n_i
 *   b_sum      [B, H_q, C_max]    f32    must hold summaries
 *   seq_lens   [B]                int32, device; 1 <= seq_lens[b] <= T_max.
 *              Out-of-range values are clamped to that range on the device
 *              (no out-of-bounds access) and counted in the workspace
 *              word at byte offset hils_decode_error_offset(cfg).
 *   o          [B, H_q, d]        dtype out
 *   topk_idx   [B, H_kv, K]       int32 out (-1 pad)
 *   topk_score [B, H_q, K]        f32 out (-inf pad)
 *   workspace  >= hils_decode_workspace_bytes(cfg), zeroed once.
 */
hils_status hils_sparse_attn_decode(const hils_config *cfg, const void *q, const void *h,
                                    const void *w_down, const void *w_up, const void *k_cache,
                                    const void *v_cache, const void *k_sum, const float *b_sum,
                                    const int32_t *seq_lens, void *o, int32_t *topk_idx,
                                    float *topk_score, void *workspace, size_t workspace_bytes,
                                    void *stream);

/* Byte offset, inside a decode workspace, of the uint32 that counts clamped
 * seq_lens entries and, for the paged call, page indices outside the pool
 * (cumulative; the caller may reset it to zero). */
size_t hils_decode_error_offset(const hils_config *cfg);

/*
 * Paged caches for serving.  A page holds one chunk (S = 64 consecutive
 * positions of one sequence) for every KV head:
 *   k_pages, v_pages  [num_pages, H_kv, S, d]  dtype
 *   block_table       [B, max_pages]           int32, device: page of chunk
 *                     (64-position block) c of sequence b
 * cfg->seq_len is the per-sequence capacity T_max; max_pages must be at least
 * ceil(T_max / S) (INVALID_ARG otherwise).  Only the table entries of blocks
 * a call reads must be valid; a page index outside [0, num_pages) is never
 * dereferenced (see each call).  The pool, the table and its pages stay owned
 * by the caller; the library does not allocate or free pages.
 *
 * hils_landmark_summary_paged: hils_landmark_summary on a paged key cache
 * (same math, same k_sum / b_sum layout, which stay per sequence).  A chunk
 * whose page index lies outside the pool gets NaN summaries for every head.
 */
hils_status hils_landmark_summary_paged(const hils_config *cfg, const void *k_pages,
                                        const int32_t *block_table, int32_t max_pages,
                                        int32_t num_pages, const void *q_lm,
                                        int32_t chunk_begin, int32_t chunk_end, void *k_sum,
                                        float *b_sum, void *stream);

/*
 * hils_sparse_attn_decode_paged: hils_sparse_attn_decode reading the window
 * and the selected chunks from paged caches; same arguments otherwise, same
 * workspace (hils_decode_workspace_bytes), bit-identical results for the
 * same cache contents.  A block the step reads whose page index lies outside
 * the pool contributes no keys and adds one to the error word at
 * hils_decode_error_offset(cfg).
 */
hils_status hils_sparse_attn_decode_paged(const hils_config *cfg, const void *q, const void *h,
                                          const void *w_down, const void *w_up,
                                          const void *k_pages, const void *v_pages,
                                          const int32_t *block_table, int32_t max_pages,
                                          int32_t num_pages, const void *k_sum,
                                          const float *b_sum, const int32_t *seq_lens, void *o,
                                          int32_t *topk_idx, float *topk_score, void *workspace,
                                          size_t workspace_bytes, void *stream);

/* Bytes of the workspace hils_dense_attn_decode needs (zero it once, as for
 * the sparse decode workspace). */
size_t hils_dense_decode_workspace_bytes(const hils_config *cfg);

/*
 * Full causal attention for one decode query per sequence -- the dense
 * comparator the pages measure HiLS against ([p1] Inference Efficiency).
 *   o[b,h] = sum_{j <= i} softmax_j(tau q.k_j) v_j,  i = seq_lens[b]-1.
 * Shapes and seq_lens handling as for hils_sparse_attn_decode.
 */
hils_status hils_dense_attn_decode(const hils_config *cfg, const void *q, const void *k_cache,
                                   const void *v_cache, const int32_t *seq_lens, void *o,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Allocation-free decode step, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments and results as
 * hils_sparse_attn_decode (contiguous caches), without the workspace: the
 * step's scratch lives in a device array inside the library, of
 * hils_noalloc_scratch_bytes() bytes per GPU (48 MiB), which each GPU the
 * library runs on holds until the process ends.  The first call on a device
 * looks the array up on that device (the current device); the call itself
 * allocates nothing and calls no allocating routine.
 *   A configuration whose decode workspace (hils_decode_workspace_bytes)
 *   exceeds the array returns HILS_ERR_UNSUPPORTED and enqueues nothing
 *   (128K x 8, 512K x 4 and 4M x 1 at 32/8 heads, d = 128, K = 16 fit).
 *   Every call on one GPU shares that GPU's array: calls that may overlap
 *   on one GPU (two streams, two threads) race and must be serialised by
 *   the caller.  Each call clears the array's tickets and error word on its
 *   stream first (a kernel, not a memset, so graph replays stay correct);
 *   out-of-range seq_lens are clamped as in hils_sparse_attn_decode, and
 *   their count is not reported.
 */
hils_status hils_sparse_attn_decode_noalloc(const hils_config *cfg, const void *q, const void *h,
                                            const void *w_down, const void *w_up,
                                            const void *k_cache, const void *v_cache,
                                            const void *k_sum, const float *b_sum,
                                            const int32_t *seq_lens, void *o, int32_t *topk_idx,
                                            float *topk_score, void *stream);
size_t hils_noalloc_scratch_bytes(void);

const char *hils_status_string(hils_status status);
const char *hils_last_error(void); /* thread-local, "" when none */

#ifdef __cplusplus
}
#endif

#endif /* HILS_H_ */
