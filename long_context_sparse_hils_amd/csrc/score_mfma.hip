// Prefill chunk scoring with Q-Cal and GQA top-K on the MFMA units --
// HiLS-Attention, picx.dev summary, Eq. 7 with Eq. 10's s-hat, Methodology 3
// (Q-Cal: q-hat = q + W_up W_down h; GQA: max over the group's heads), and
// the rcap.io pseudo-code's arg-top-K.
//
// The Q-Cal term is regrouped so that every product is a bf16 MFMA:
//   s = tau * (q . k' + u . m) + b',   u = W_down h (per token, r values),
//                                      m = W_up[h*d:(h+1)*d, :]^T k' (per head and chunk)
// q and k' are bf16 inputs (exact products); u and m are fp32 values carried
// as bf16 hi + lo pairs (u ~= u_hi + u_lo to ~2^-16 relative), multiplied as
// hi*hi + hi*lo + lo*hi.
//
// Kernels:
//   qcal_u_mfma      u[token, a]   MFMA GEMM over D_h  -> u_hi/u_lo [B*T, RP]
//   qcal_m           m[b, h, c, a] VALU (tiny)          -> m_hi/m_lo [B, Hq, C, RP]
//   score_topk_mfma  per (64 queries, KV head, batch): S^T tiles of 16
//                    chunks x 16 queries per head, max over the group's heads
//                    into LDS, then per query a ballot-driven radix select of
//                    the K-th largest group score and a rank pass that orders
//                    the winners by (score desc, chunk asc); a second MFMA
//                    pass (same arithmetic, bit-identical) writes each head's
//                    own score for the winners.
#include "hils_common.h"
#include "launch.h"

namespace hils {

typedef __bf16 bf16x8s __attribute__((ext_vector_type(8)));
typedef float f32x4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4s mfma_s(const uint4 &a, const uint4 &b, const f32x4s &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8s, a), __builtin_bit_cast(bf16x8s, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ void split_bf16(float x, uint16_t &hi, uint16_t &lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// ------------------------------------------------------------------ u = W_down h
// 64 tokens per workgroup (16 per wave), RP/16 output tiles; K-loop over D_h.
__global__ void __launch_bounds__(256)
qcal_u_mfma_kernel(const uint16_t *__restrict__ h, const uint16_t *__restrict__ w_down, uint16_t *__restrict__ u_hi,
                   uint16_t *__restrict__ u_lo, int Ntok, int r, int RP, int Dh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int tok0 = blockIdx.x * 64 + wave * 16;
  const int NT = RP / 16;
  const int tok = tok0 + ln;
  const bool tok_ok = tok < Ntok;
  const uint16_t *hrow = h + static_cast<size_t>(tok_ok ? tok : 0) * Dh + 8 * lg;
  f32x4s acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4s{0.f, 0.f, 0.f, 0.f};
  constexpr int UK = 8;  // k-steps whose loads are issued together
  int e0 = 0;
  for (; e0 + 32 * UK <= Dh; e0 += 32 * UK) {
    uint4 av[UK], bv[UK][2];
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      av[u] = tok_ok ? *reinterpret_cast<const uint4 *>(hrow + e0 + 32 * u) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int aa = 16 * nt + ln;
        bv[u][nt] = (nt < NT && aa < r)
                        ? *reinterpret_cast<const uint4 *>(w_down + static_cast<size_t>(aa) * Dh + e0 + 32 * u + 8 * lg)
                        : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < UK; ++u)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[nt] = mfma_s(av[u], bv[u][nt], acc[nt]);
    if (NT > 2) {
#pragma unroll
      for (int u = 0; u < UK; ++u)
#pragma unroll
        for (int nt = 2; nt < 4; ++nt) {
          const int aa = 16 * nt + ln;
          const uint4 b2 = (nt < NT && aa < r)
                               ? *reinterpret_cast<const uint4 *>(w_down + static_cast<size_t>(aa) * Dh + e0 + 32 * u + 8 * lg)
                               : make_uint4(0, 0, 0, 0);
          acc[nt] = mfma_s(av[u], b2, acc[nt]);
        }
    }
  }
  for (; e0 < Dh; e0 += 32) {
    const uint4 av = tok_ok ? *reinterpret_cast<const uint4 *>(hrow + e0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (nt < NT) {
        const int aa = 16 * nt + ln;
        const uint4 bv = aa < r ? *reinterpret_cast<const uint4 *>(w_down + static_cast<size_t>(aa) * Dh + e0 + 8 * lg)
                                : make_uint4(0, 0, 0, 0);
        acc[nt] = mfma_s(av, bv, acc[nt]);
      }
    }
  }
  // D[m = token 4 lg + i][n = a]
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if (nt < NT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tk = tok0 + 4 * lg + i, aa = 16 * nt + ln;
        if (tk < Ntok) {
          uint16_t hi, lo;
          split_bf16(acc[nt][i], hi, lo);
          u_hi[static_cast<size_t>(tk) * RP + aa] = hi;
          u_lo[static_cast<size_t>(tk) * RP + aa] = lo;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ m = W_up_h^T k'
// One workgroup per (32 chunks, query head, batch); W_up's head slice in LDS.
template <int D>
__global__ void __launch_bounds__(256)
qcal_m_kernel(const uint16_t *__restrict__ k_sum, const uint16_t *__restrict__ w_up, uint16_t *__restrict__ m_hi,
              uint16_t *__restrict__ m_lo, int Hq, int C, int r, int RP) {
  __shared__ float wu[D][65];
  __shared__ float kc[32][D + 1];
  const int c0 = blockIdx.x * 32, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  for (int x = t; x < D * r; x += 256) wu[x / r][x % r] = bf16_to_f32(w_up[(static_cast<size_t>(h) * D + x / r) * r + x % r]);
  for (int x = t; x < 32 * D; x += 256) {
    const int cc = x / D, e = x % D;
    kc[cc][e] = (c0 + cc < C) ? bf16_to_f32(k_sum[((static_cast<size_t>(b) * Hq + h) * C + c0 + cc) * D + e]) : 0.f;
  }
  __syncthreads();
  for (int x = t; x < 32 * RP; x += 256) {
    const int cc = x / RP, aa = x % RP;
    if (c0 + cc >= C) continue;
    float acc = 0.f;
    if (aa < r)
      for (int e = 0; e < D; ++e) acc += wu[e][aa] * kc[cc][e];
    uint16_t hi, lo;
    split_bf16(acc, hi, lo);
    const size_t o = ((static_cast<size_t>(b) * Hq + h) * C + c0 + cc) * RP + aa;
    m_hi[o] = hi;
    m_lo[o] = lo;
  }
}

// ------------------------------------------------------------------ scores + top-K
constexpr int kScoreMaxC = 256;

template <int NJ>
struct ScoreWaveSmem {
  float sig[16][64 * NJ];
  int8_t rank[16][64 * NJ];
};

// s for head h, chunk tile ct (16 chunks) and the wave's 16 queries.
// Lane holds chunks 16 ct + 4 lg + i (i < 4) for query ln.
template <int D>
__device__ __forceinline__ f32x4s score_tile(const ScoreArgs &a, const uint16_t *ks_h, const float *bs_h,
                                             const uint4 *qv, const uint16_t *mh_h, const uint16_t *ml_h,
                                             const uint4 *uh, const uint4 *ul, int ct, int ln, int lg, int RP,
                                             bool qcal) {
  constexpr int KS = D / 32;
  const int c_row = 16 * ct + ln;  // A-operand row (chunk)
  const bool c_ok = c_row < a.C;
  f32x4s acc = f32x4s{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const uint4 av = c_ok ? *reinterpret_cast<const uint4 *>(ks_h + static_cast<size_t>(c_row) * D + 32 * s + 8 * lg)
                          : make_uint4(0, 0, 0, 0);
    acc = mfma_s(av, qv[s], acc);
  }
  if (qcal) {
    for (int s = 0; s < RP / 32; ++s) {
      const size_t mo = static_cast<size_t>(c_row) * RP + 32 * s + 8 * lg;
      const uint4 mh = c_ok ? *reinterpret_cast<const uint4 *>(mh_h + mo) : make_uint4(0, 0, 0, 0);
      const uint4 ml = c_ok ? *reinterpret_cast<const uint4 *>(ml_h + mo) : make_uint4(0, 0, 0, 0);
      acc = mfma_s(mh, uh[s], acc);
      acc = mfma_s(mh, ul[s], acc);
      acc = mfma_s(ml, uh[s], acc);
    }
  }
  f32x4s sv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 16 * ct + 4 * lg + i;
    sv[i] = a.tau * acc[i] + (c < a.C ? bs_h[c] : 0.f);
  }
  return sv;
}

template <int D, int NJ>
__global__ void __launch_bounds__(256)
score_topk_mfma_kernel(ScoreArgs a, const uint16_t *__restrict__ u_hi, const uint16_t *__restrict__ u_lo,
                       const uint16_t *__restrict__ m_hi, const uint16_t *__restrict__ m_lo, int RP) {
  constexpr int KS = D / 32;
  __shared__ ScoreWaveSmem<NJ> wsm[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int T = a.T, C = a.C, K = a.K, Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  const int g = blockIdx.y, b = blockIdx.z;
  const int qw0 = blockIdx.x * 64 + wave * 16;  // the wave's first query
  if (qw0 >= T) return;                         // whole wave idle (no barriers below)
  ScoreWaveSmem<NJ> &sm = wsm[wave];
  const bool qcal = a.r > 0;
  const int i_me = qw0 + ln;                     // this lane's query (B column)
  const bool q_ok = i_me < T;
  const int n_me = q_ok ? min(eligible_chunks(i_me, a.W, a.S), C) : 0;
  const int i_last = min(qw0 + 15, T - 1);
  const int n_wave = min(eligible_chunks(i_last, a.W, a.S), C);
  const int nct = (n_wave + 15) / 16;

  uint4 uh[2], ul[2];
  if (qcal) {
    const size_t uo = (static_cast<size_t>(b) * T + (q_ok ? i_me : 0)) * RP + 8 * lg;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bool ok = q_ok && s < RP / 32;
      uh[s] = ok ? *reinterpret_cast<const uint4 *>(u_hi + uo + 32 * s) : make_uint4(0, 0, 0, 0);
      ul[s] = ok ? *reinterpret_cast<const uint4 *>(u_lo + uo + 32 * s) : make_uint4(0, 0, 0, 0);
    }
  }
  const uint16_t *qb = static_cast<const uint16_t *>(a.q);
  const uint16_t *ksb = static_cast<const uint16_t *>(a.k_sum);

  // ---- pass 1: group score sigma into LDS
  for (int x = lane; x < 16 * 64 * NJ; x += 64) (&sm.sig[0][0])[x] = -INFINITY;
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    uint4 qv[KS];
    const size_t qo = ((static_cast<size_t>(b) * Hq + h) * T + (q_ok ? i_me : 0)) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s) qv[s] = q_ok ? *reinterpret_cast<const uint4 *>(qb + qo + 32 * s) : make_uint4(0, 0, 0, 0);
    const uint16_t *ks_h = ksb + (static_cast<size_t>(b) * Hq + h) * C * D;
    const float *bs_h = a.b_sum + (static_cast<size_t>(b) * Hq + h) * C;
    const uint16_t *mh_h = qcal ? m_hi + (static_cast<size_t>(b) * Hq + h) * C * RP : nullptr;
    const uint16_t *ml_h = qcal ? m_lo + (static_cast<size_t>(b) * Hq + h) * C * RP : nullptr;
    for (int ct = 0; ct < nct; ct += 2) {
      // two chunk tiles per step so their operand loads overlap
      const f32x4s sv0 = score_tile<D>(a, ks_h, bs_h, qv, mh_h, ml_h, uh, ul, ct, ln, lg, RP, qcal);
      const f32x4s sv1 = score_tile<D>(a, ks_h, bs_h, qv, mh_h, ml_h, uh, ul, ct + 1, ln, lg, RP, qcal);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c0 = 16 * ct + 4 * lg + i, c1 = c0 + 16;
        if (c0 < n_me) sm.sig[ln][c0] = fmaxf(sm.sig[ln][c0], sv0[i]);
        if (c1 < n_me) sm.sig[ln][c1] = fmaxf(sm.sig[ln][c1], sv1[i]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();

  // ---- selection per query: radix select of the K-th largest key
  for (int q = 0; q < 16; ++q) {
    const int i = qw0 + q;
    if (i >= T) break;
    const int n = min(eligible_chunks(i, a.W, a.S), C);
    const int keep = min(K, n);
    uint32_t ord[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = lane + 64 * j;
      ord[j] = c < n ? orderable(sm.sig[q][c]) : 0u;  // 0 = below every real score
      sm.rank[q][c] = -1;
    }
    // theta = the largest value with #{ord >= theta} >= keep
    uint32_t theta = 0u;
    if (keep > 0) {
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = theta | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) cnt += __popcll(__ballot(ord[j] >= cand));
        if (cnt >= keep) theta = cand;
      }
    }
    // winners: ord > theta, then the lowest-index ord == theta to fill
    int cnt_gt = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) cnt_gt += __popcll(__ballot(keep > 0 && ord[j] > theta));
    int need_eq = keep - cnt_gt;
    bool win[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bool gt = keep > 0 && ord[j] > theta;
      const bool eq = keep > 0 && ord[j] == theta && (lane + 64 * j) < n;
      const unsigned long long eqm = __ballot(eq);
      const int before = __popcll(eqm & ((1ull << lane) - 1ull));
      win[j] = gt || (eq && before < need_eq);
      need_eq -= min(need_eq, __popcll(eqm));
    }
    // rank of each winner among the winners by (score desc, chunk asc)
    int rk[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) rk[j] = 0;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      unsigned long long wm = __ballot(win[jj]);
      while (wm) {
        const int src = __ffsll(static_cast<long long>(wm)) - 1;
        wm &= wm - 1ull;
        const uint32_t o2 = __shfl(ord[jj], src, 64);
        const int c2 = src + 64 * jj;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int c = lane + 64 * j;
          if (win[j] && (o2 > ord[j] || (o2 == ord[j] && c2 < c))) ++rk[j];
        }
      }
    }
    const size_t ibase = ((static_cast<size_t>(b) * Hkv + g) * T + i) * K;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = lane + 64 * j;
      if (win[j]) {
        sm.rank[q][c] = static_cast<int8_t>(rk[j]);
        a.topk_idx[ibase + rk[j]] = c;
      }
    }
    for (int k = keep + lane; k < K; k += 64) a.topk_idx[ibase + k] = -1;
    for (int x = lane; x < G * (K - keep); x += 64) {
      const int hh = x / (K - keep), k = keep + x % (K - keep);
      a.topk_score[((static_cast<size_t>(b) * Hq + g * G + hh) * T + i) * K + k] = -INFINITY;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();

  // ---- pass 2: each head's own score of the winners (same arithmetic as pass 1)
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    uint4 qv[KS];
    const size_t qo = ((static_cast<size_t>(b) * Hq + h) * T + (q_ok ? i_me : 0)) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s) qv[s] = q_ok ? *reinterpret_cast<const uint4 *>(qb + qo + 32 * s) : make_uint4(0, 0, 0, 0);
    const uint16_t *ks_h = ksb + (static_cast<size_t>(b) * Hq + h) * C * D;
    const float *bs_h = a.b_sum + (static_cast<size_t>(b) * Hq + h) * C;
    const uint16_t *mh_h = qcal ? m_hi + (static_cast<size_t>(b) * Hq + h) * C * RP : nullptr;
    const uint16_t *ml_h = qcal ? m_lo + (static_cast<size_t>(b) * Hq + h) * C * RP : nullptr;
    for (int ct = 0; ct < nct; ct += 2) {
      const f32x4s sv0 = score_tile<D>(a, ks_h, bs_h, qv, mh_h, ml_h, uh, ul, ct, ln, lg, RP, qcal);
      const f32x4s sv1 = score_tile<D>(a, ks_h, bs_h, qv, mh_h, ml_h, uh, ul, ct + 1, ln, lg, RP, qcal);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int c = 16 * (ct + hf) + 4 * lg + i;
          if (c < n_me) {
            const int rk = sm.rank[ln][c];
            if (rk >= 0) a.topk_score[((static_cast<size_t>(b) * Hq + h) * T + i_me) * K + rk] = hf ? sv1[i] : sv0[i];
          }
        }
      }
    }
  }
}

bool score_mfma_supported(const ScoreArgs &a) {
  return a.bf16 && (a.d == 64 || a.d == 128) && a.C <= kScoreMaxC && a.K <= 32 && a.K > 0 &&
         (a.r == 0 || (a.Dh % 32 == 0 && a.r <= 64));
}

size_t score_mfma_ws_bytes(int B, int T, int Hq, int C, int r) {
  if (r == 0) return 0;
  const int RP = r <= 32 ? 32 : 64;
  return 2 * sizeof(uint16_t) * (static_cast<size_t>(B) * T * RP + static_cast<size_t>(B) * Hq * C * RP) + 1024;
}

hipError_t launch_score_mfma(const ScoreArgs &a, hipStream_t st) {
  const int RP = a.r <= 32 ? 32 : 64;
  uint16_t *base = static_cast<uint16_t *>(a.ws);
  uint16_t *u_hi = base, *u_lo = u_hi + static_cast<size_t>(a.B) * a.T * RP;
  uint16_t *m_hi = u_lo + static_cast<size_t>(a.B) * a.T * RP;
  uint16_t *m_lo = m_hi + static_cast<size_t>(a.B) * a.Hq * a.C * RP;
  if (a.r > 0) {
    const int ntok = a.B * a.T;
    qcal_u_mfma_kernel<<<(ntok + 63) / 64, 256, 0, st>>>(static_cast<const uint16_t *>(a.h),
                                                      static_cast<const uint16_t *>(a.w_down), u_hi, u_lo, ntok,
                                                      a.r, RP, a.Dh);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 gm((a.C + 31) / 32, a.Hq, a.B);
    if (a.C == 0) {
      // no complete chunk: nothing to project
    } else if (a.d == 128)
      qcal_m_kernel<128><<<gm, 256, 0, st>>>(static_cast<const uint16_t *>(a.k_sum), static_cast<const uint16_t *>(a.w_up),
                                              m_hi, m_lo, a.Hq, a.C, a.r, RP);
    else
      qcal_m_kernel<64><<<gm, 256, 0, st>>>(static_cast<const uint16_t *>(a.k_sum), static_cast<const uint16_t *>(a.w_up),
                                             m_hi, m_lo, a.Hq, a.C, a.r, RP);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid((a.T + 63) / 64, a.Hkv, a.B);
  // candidates per lane in the selection: ceil(C / 64) rounded to 1, 2 or 4
  const int nj = a.C <= 64 ? 1 : (a.C <= 128 ? 2 : 4);
#define HILS_SCORE(DD, NN) \
  if (a.d == DD && nj == NN) score_topk_mfma_kernel<DD, NN><<<grid, 256, 0, st>>>(a, u_hi, u_lo, m_hi, m_lo, RP);
  HILS_SCORE(128, 1) HILS_SCORE(128, 2) HILS_SCORE(128, 4) HILS_SCORE(64, 1) HILS_SCORE(64, 2) HILS_SCORE(64, 4)
#undef HILS_SCORE
  return hipGetLastError();
}

}  // namespace hils
