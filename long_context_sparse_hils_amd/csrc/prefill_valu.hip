// Prefill path on the vector ALUs: Q-Cal down-projection, chunk scoring with
// GQA top-K, and hierarchical sparse attention, one query per workgroup.
// This is the fp32-mode path (and the path for shapes the MFMA kernels do not
// tile).  HiLS-Attention, picx.dev summary: Methodology 1-3 (Eq. 7, Eq. 10,
// Q-Cal, GQA adaptation); rcap.io pseudo-code.
#include "attn_unit.h"
#include "hils_common.h"
#include "launch.h"

namespace hils {

// ------------------------------------------------------------------ Q-Cal
// u[b, i, a] = sum_e W_down[a, e] h[b, i, e]   (fp32), 64 tokens per block.
constexpr int kQcalTok = 64;
constexpr int kQcalSlab = 64;

template <typename T>
__global__ void __launch_bounds__(256)
qcal_down_kernel(const T *__restrict__ h, const T *__restrict__ w_down, float *__restrict__ u,
                 int Ntok, int r, int Dh) {
  __shared__ float hs[kQcalTok][kQcalSlab + 1];
  __shared__ float ws[64][kQcalSlab + 1];
  const int t = threadIdx.x;
  const int tok0 = blockIdx.x * kQcalTok;
  const int tt = t >> 2, aq = t & 3;
  const int per = (r + 3) / 4;  // outputs per thread (<= 16)
  float acc[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = 0.f;
  for (int e0 = 0; e0 < Dh; e0 += kQcalSlab) {
    for (int x = t; x < kQcalTok * kQcalSlab; x += 256) {
      int row = x / kQcalSlab, col = x % kQcalSlab;
      int tok = tok0 + row;
      hs[row][col] = (tok < Ntok && e0 + col < Dh) ? Elem<T>::load(h, static_cast<size_t>(tok) * Dh + e0 + col) : 0.f;
    }
    for (int x = t; x < r * kQcalSlab; x += 256) {
      int row = x / kQcalSlab, col = x % kQcalSlab;
      ws[row][col] = (e0 + col < Dh) ? Elem<T>::load(w_down, static_cast<size_t>(row) * Dh + e0 + col) : 0.f;
    }
    __syncthreads();
    for (int e = 0; e < kQcalSlab; ++e) {
      const float hv = hs[tt][e];
#pragma unroll
      for (int x = 0; x < 16; ++x)
        if (x < per && aq * per + x < r) acc[x] += hv * ws[aq * per + x][e];
    }
    __syncthreads();
  }
  const int tok = tok0 + tt;
  if (tok < Ntok)
#pragma unroll
    for (int x = 0; x < 16; ++x)
      if (x < per && aq * per + x < r) u[static_cast<size_t>(tok) * r + aq * per + x] = acc[x];
}

// ------------------------------------------------------------------ scores + top-K
// One wave per (query i, KV head g, batch b).
//   q-hat_h = q_h + W_up[h*D:(h+1)*D, :] u_i
//   s_h(c)  = tau q-hat_h . k_sum[b,h,c] + b_sum[b,h,c]      c < n_i
//   sigma(c)= max_h s_h(c); top-K by (sigma desc, c asc)
template <typename T, int D>
__device__ __forceinline__ float chunk_score(const float *qh, const T *ks_row, float bs, float tau) {
  float acc = 0.f;
#pragma unroll 4
  for (int e8 = 0; e8 < D / 8; ++e8) {
    float kv[8];
    Elem<T>::load8(ks_row + e8 * 8, kv);
#pragma unroll
    for (int x = 0; x < 8; ++x) acc += qh[e8 * 8 + x] * kv[x];
  }
  return tau * acc + bs;
}

template <typename T, int D>
__global__ void __launch_bounds__(64)
score_topk_valu_kernel(const T *__restrict__ q, const float *__restrict__ u, const T *__restrict__ w_up,
                       const T *__restrict__ k_sum, const float *__restrict__ b_sum,
                       int32_t *__restrict__ topk_idx, float *__restrict__ topk_score, int T_len, int Hq,
                       int Hkv, int C, int S, int K, int W, int r, float tau) {
  extern __shared__ float smem[];
  const int G = Hq / Hkv;
  float *qh = smem;            // [G][D]
  float *ur = qh + G * D;      // [r]
  float *sig = ur + 64;        // [C]
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int n = min(eligible_chunks(i, W, S), C);
  for (int a = lane; a < r; a += 64) ur[a] = u[(static_cast<size_t>(b) * T_len + i) * r + a];
  __syncthreads();
  for (int x = lane; x < G * D; x += 64) {
    const int hh = x / D, e = x % D, h = g * G + hh;
    float val = Elem<T>::load(q, ((static_cast<size_t>(b) * Hq + h) * T_len + i) * D + e);
    float acc = 0.f;
    for (int a = 0; a < r; ++a) acc += Elem<T>::load(w_up, (static_cast<size_t>(h) * D + e) * r + a) * ur[a];
    qh[x] = val + acc;
  }
  __syncthreads();
  const size_t sbase = (static_cast<size_t>(b) * Hq + g * G) * C;
  for (int c = lane; c < n; c += 64) {
    float best = -INFINITY;
    for (int hh = 0; hh < G; ++hh) {
      const size_t so = sbase + static_cast<size_t>(hh) * C + c;
      best = fmaxf(best, chunk_score<T, D>(qh + hh * D, k_sum + so * D, b_sum[so], tau));
    }
    sig[c] = best;
  }
  __syncthreads();
  const int keep = min(K, n);
  unsigned long long prev = ~0ull;
  const size_t ibase = ((static_cast<size_t>(b) * Hkv + g) * T_len + i) * K;
  for (int k = 0; k < keep; ++k) {
    unsigned long long best = kNoKey;
    for (int c = lane; c < n; c += 64) {
      unsigned long long key = make_key(sig[c], c);
      if (key < prev && key > best) best = key;
    }
    best = wave_max_u64(best);
    prev = best;
    const int c = key_chunk(best);
    if (lane == 0) topk_idx[ibase + k] = c;
    for (int hh = lane; hh < G; hh += 64) {
      const int h = g * G + hh;
      const size_t so = sbase + static_cast<size_t>(hh) * C + c;
      topk_score[((static_cast<size_t>(b) * Hq + h) * T_len + i) * K + k] =
          chunk_score<T, D>(qh + hh * D, k_sum + so * D, b_sum[so], tau);
    }
  }
  for (int k = keep + lane; k < K; k += 64) topk_idx[ibase + k] = -1;
  for (int x = lane; x < G * (K - keep); x += 64) {
    const int hh = x / (K - keep), k = keep + x % (K - keep);
    topk_score[((static_cast<size_t>(b) * Hq + g * G + hh) * T_len + i) * K + k] = -INFINITY;
  }
}

// ------------------------------------------------------------------ attention
// One workgroup per (query i, KV head g, batch b); units of 64 keys.
template <typename T, int D>
__global__ void __launch_bounds__(kUnitThreads)
attn_valu_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                 const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_score,
                 T *__restrict__ o, int T_len, int Hq, int Hkv, int S, int K, int W, float tau) {
  __shared__ UnitSmem<T, D> sm;
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int G = Hq / Hkv;
  const size_t qstride = static_cast<size_t>(T_len) * D;  // between heads
  load_q_rows<T, D>(sm, q + ((static_cast<size_t>(b) * Hq + g * G) * T_len + i) * D, qstride, G);
  __syncthreads();
  const T *kb = k + (static_cast<size_t>(b) * Hkv + g) * T_len * D;
  const T *vb = v + (static_cast<size_t>(b) * Hkv + g) * T_len * D;
  constexpr int NP = pairs_per_thread<D>();
  PairAcc<D> chunks, win;
  chunks.init();
  win.init();
  float2 ou[NP];
  const size_t ibase = ((static_cast<size_t>(b) * Hkv + g) * T_len + i) * K;
  const int n = eligible_chunks(i, W, S);
  for (int kk = 0; kk < K; ++kk) {
    const int c = topk_idx[ibase + kk];
    // -1 pads; an id outside the eligible chunks [0, n_i) is no chunk (it
    // would overlap the window or lie past the sequence).  Uniform across
    // the block.
    if (c < 0 || c >= n) continue;
    attend_unit<T, D>(sm, kb + static_cast<size_t>(c) * S * D, vb + static_cast<size_t>(c) * S * D, S, G, tau, ou);
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int pr = t + r * kUnitThreads, hh = pr / (D / 2);
      if (hh < G) {
        const float alpha = topk_score[((static_cast<size_t>(b) * Hq + g * G + hh) * T_len + i) * K + kk];
        const float inv = 1.f / sm.l[hh];
        chunks.add(r, alpha, 1.f, make_float2(ou[r].x * inv, ou[r].y * inv));
      }
    }
    __syncthreads();
  }
  for (int j0 = n * S; j0 <= i; j0 += kUnitKeys) {
    const int nk = min(kUnitKeys, i - j0 + 1);
    attend_unit<T, D>(sm, kb + static_cast<size_t>(j0) * D, vb + static_cast<size_t>(j0) * D, nk, G, tau, ou);
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int pr = t + r * kUnitThreads, hh = pr / (D / 2);
      if (hh < G) win.add(r, sm.m[hh], sm.l[hh], ou[r]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < NP; ++r) {
    const int pr = t + r * kUnitThreads, hh = pr / (D / 2), e2 = pr % (D / 2);
    if (hh < G) {
      chunks.add(r, win.m[r], win.l[r], win.o[r]);
      const float inv = 1.f / chunks.l[r];
      T *dst = o + ((static_cast<size_t>(b) * Hq + g * G + hh) * T_len + i) * D + 2 * e2;
      Elem<T>::store2(dst, chunks.o[r].x * inv, chunks.o[r].y * inv);
    }
  }
}

// ------------------------------------------------------------------ launchers
template <typename T, int D>
static hipError_t score_valu_t(const ScoreArgs &a, hipStream_t st) {
  if (a.r > 0) {
    dim3 g1((a.B * a.T + kQcalTok - 1) / kQcalTok);
    qcal_down_kernel<T><<<g1, 256, 0, st>>>(static_cast<const T *>(a.h), static_cast<const T *>(a.w_down), a.u_ws,
                                          a.B * a.T, a.r, a.Dh);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int G = a.Hq / a.Hkv;
  size_t smem = sizeof(float) * (G * D + 64 + a.C);
  dim3 grid(a.T, a.Hkv, a.B);
  score_topk_valu_kernel<T, D><<<grid, 64, smem, st>>>(
      static_cast<const T *>(a.q), a.u_ws, static_cast<const T *>(a.w_up), static_cast<const T *>(a.k_sum),
      a.b_sum, a.topk_idx, a.topk_score, a.T, a.Hq, a.Hkv, a.C, a.S, a.K, a.W, a.r, a.tau);
  return hipGetLastError();
}

hipError_t launch_score_valu(const ScoreArgs &a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? score_valu_t<uint16_t, 128>(a, st) : score_valu_t<uint16_t, 64>(a, st);
  return a.d == 128 ? score_valu_t<float, 128>(a, st) : score_valu_t<float, 64>(a, st);
}

template <typename T, int D>
static hipError_t attn_valu_t(const AttnArgs &a, hipStream_t st) {
  dim3 grid(a.T, a.Hkv, a.B);
  attn_valu_kernel<T, D><<<grid, kUnitThreads, 0, st>>>(
      static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v), a.topk_idx,
      a.topk_score, static_cast<T *>(a.o), a.T, a.Hq, a.Hkv, a.S, a.K, a.W, a.tau);
  return hipGetLastError();
}

hipError_t launch_attn_valu(const AttnArgs &a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? attn_valu_t<uint16_t, 128>(a, st) : attn_valu_t<uint16_t, 64>(a, st);
  return a.d == 128 ? attn_valu_t<float, 128>(a, st) : attn_valu_t<float, 64>(a, st);
}

}  // namespace hils
