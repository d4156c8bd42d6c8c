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
  void *vt_ws;  // prefill workspace: transposed value tiles of the MFMA path, then its query grouping
  int B, T, Hq, Hkv, d, S, K, W;
  float tau;
  bool bf16;
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

hipError_t launch_summary(const SummaryArgs &a, hipStream_t st);
hipError_t launch_score_valu(const ScoreArgs &a, hipStream_t st);
bool score_mfma_supported(const ScoreArgs &a);
size_t score_mfma_ws_bytes(int B, int T, int Hq, int C, int r);
hipError_t launch_score_mfma(const ScoreArgs &a, hipStream_t st);
hipError_t launch_attn_valu(const AttnArgs &a, hipStream_t st);
bool attn_mfma_supported(const AttnArgs &a);
size_t attn_mfma_ws_bytes(int B, int Hkv, int T, int d);
hipError_t launch_attn_mfma(const AttnArgs &a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t st);
hipError_t launch_dense_decode(const DenseArgs &a, hipStream_t st);

}  // namespace hils
