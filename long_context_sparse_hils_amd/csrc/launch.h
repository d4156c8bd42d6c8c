// Internal interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hils {

struct SummaryArgs {
  const void *k, *q_lm;
  void *k_sum;
  float *b_sum;
  int B, T, Hq, Hkv, C, d, c0, c1;
  float tau;
  bool bf16;
  // paged K (null: contiguous [B, Hkv, T, d]): k holds pages
  // [num_pages, Hkv, S, d] and block_table [B, max_pages] maps chunk c of
  // sequence b to its page
  const int32_t *block_table;
  int max_pages, num_pages;
};

struct ScoreArgs {
  const void *q, *h, *w_down, *w_up, *k_sum;
  const float *b_sum;
  int32_t *topk_idx;
  float *topk_score;
  float *u_ws;  // [B*T, r] fp32 (Q-Cal down projection)
  void *ws;     // remaining prefill workspace
  int B, T, Hq, Hkv, d, S, K, W, r, Dh, C;
  float tau;
  bool bf16;
};

struct AttnArgs {
  const void *q, *k, *v;
  const int32_t *topk_idx;
  const float *topk_score;
  void *o;
  void *vt_ws;  // prefill workspace of the MFMA path: chunk log-mass, block |v| bounds, K/V in operand order
  int B, T, Hq, Hkv, d, S, K, W;
  float tau;
  bool bf16;
  // set by the MFMA path between its two passes: each row's chunk log-mass
  // [B, Hq, T] (o then holds the rows' normalised chunk parts)
  const float *lse_c;
};

struct DecodeArgs {
  const void *q, *h, *w_down, *w_up, *k_cache, *v_cache, *k_sum;
  const float *b_sum;
  const int32_t *seq_lens;
  void *o;
  int32_t *topk_idx;
  float *topk_score;
  float *qhat;                   // [B, Hq, d] (Q-Cal only)
  float *sig;                    // [B, Hkv, Cmax]: group score of each eligible chunk
  float *hsc;                    // [B, Hkv, Cmax, G]: each head's own score
  float *smax;                   // [B, Hkv, P]: the largest group score of each 64-chunk slice
  float *parts;                  // [B, Hkv, nslots, G, d+2]
  unsigned *count, *err;
  int B, Tmax, Hq, Hkv, d, S, K, W, r, Dh, Cmax;
  int P, NW, nslots, nslot_blocks;
  float tau;
  bool bf16;
  // paged caches (null: contiguous [B, Hkv, Tmax, d]): k_cache / v_cache hold
  // pages [num_pages, Hkv, S, d]; block_table [B, max_pages] maps the 64-key
  // block j / S of sequence b to its page
  const int32_t *block_table;
  int max_pages, num_pages;
};

struct DenseArgs {
  const void *q, *k_cache, *v_cache;
  const int32_t *seq_lens;
  void *o;
  float *parts;  // [B, Hkv, P, G, d+2]
  unsigned *count, *err;
  int B, Tmax, Hq, Hkv, d, P, L;
  float tau;
  bool bf16;
};

// Backward pass for a fixed selection (all gradients float32).
constexpr int kMaxBwdChunks = 512;  // C = T / S bound of the inverse selection lists
constexpr int kMaxBwdG = 16;
constexpr int kBwdSplitW = 16;  // k splits of the Q-Cal weight-gradient GEMMs (k = tokens)
constexpr int kBwdSplitDu = 4;  // k splits of u = h W_down^T and du = dq_hat W_up (k = D_h, H_q d)
struct BwdArgs {
  const void *q, *k, *v, *q_lm, *h, *w_down, *w_up, *k_sum, *d_o;
  const float *b_sum;
  const int32_t *topk_idx;
  // outputs: dq [B,Hq,T,d], dk / dv [B,Hkv,T,d], dq_lm [B,Hq,C,d],
  // dh [B*T,Dh], dw_down [r,Dh], dw_up [Hq*d,r]
  float *dq, *dk, *dv, *dq_lm, *dh, *dw_down, *dw_up;
  // workspace: u / du [B*T,r]; qhat [B,Hq,T,d]; dqhat [B,T,Hq,d] (token
  // major); logz / delta [B,Hq,T]; per selection-list entry and head
  // ent_lw / ent_doo / ent_ds [B,Hkv,T*K,G]; zsum [B,Hq,C,r], zb [B,Hq,C]
  float *u, *du, *qhat, *dqhat, *logz, *delta, *ent_lw, *ent_doo, *ent_ds, *zsum, *zb;
  float *gpart;  // split-k partial sums of the Q-Cal GEMMs

  // inverse selection lists: inv_cnt / inv_qboff [B,Hkv,nqb,C],
  // inv_choff [B,Hkv,C+1], inv_list [B,Hkv,T*K] (query << 5 | slot),
  // inv_pos [B,Hkv,T,K] (each slot's place in its list, -1: none)
  int32_t *inv_cnt, *inv_qboff, *inv_choff, *inv_list, *inv_pos;
  int B, T, Hq, Hkv, d, K, W, r, Dh;
  float tau;
  bool bf16;
};

hipError_t launch_summary(const SummaryArgs &a, hipStream_t st);
hipError_t launch_score_valu(const ScoreArgs &a, hipStream_t st);
hipError_t launch_backward(const BwdArgs &a, hipStream_t st);
bool bwd_keys_mfma_supported(const BwdArgs &a);
bool bwd_rows_mfma_supported(const BwdArgs &a);
hipError_t launch_bwd_rows_mfma(const BwdArgs &a, hipStream_t st);
hipError_t launch_bwd_keys_mfma(const BwdArgs &a, hipStream_t st);
bool score_mfma_supported(const ScoreArgs &a);
size_t score_mfma_ws_bytes(int B, int T, int Hq, int C, int r);
hipError_t launch_score_mfma(const ScoreArgs &a, hipStream_t st);
hipError_t launch_attn_valu(const AttnArgs &a, hipStream_t st);
bool attn_mfma_supported(const AttnArgs &a);
size_t attn_mfma_ws_bytes(int B, int Hq, int Hkv, int T, int d, int K);
hipError_t launch_attn_chunks(const AttnArgs &a, uint16_t *ops, float *lse, const float *vmax, int nblk,
                              hipStream_t st);
// every 64-key block's K and V^T in the MFMA passes' operand order: complete
// chunks into ops, a partial last block into ops_tail; each block's largest
// |v| into vmax (when given)
hipError_t launch_kv_operand_order(const AttnArgs &a, uint16_t *ops, uint16_t *ops_tail, float *vmax, hipStream_t st);
// The chunk terms of sequences longer than kLongMinChunks chunks run
// chunk-major over the whole sequence, in segments of queries whose
// per-(query, slot) partial results take at most kLongPartBytes.
constexpr int kLongMinChunks = 256;
constexpr size_t kLongPartBytes = size_t(8) << 30;
bool attn_long_used(int T, int K);
size_t attn_long_ws_bytes(int B, int Hq, int Hkv, int T, int d, int K);
hipError_t launch_attn_long(const AttnArgs &a, uint16_t *ops, float *lse, uint8_t *ws, hipStream_t st);
inline int eligible_chunks_host(int i, int W, int S) {
  const int w0 = i - W + 1;
  return w0 > 0 ? w0 / S : 0;
}
hipError_t launch_attn_mfma(const AttnArgs &a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t st);
hipError_t launch_dense_decode(const DenseArgs &a, hipStream_t st);

}  // namespace hils
