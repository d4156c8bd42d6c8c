// Landmark chunk summary (HiLS-Attention, picx.dev summary, Methodology 1,
// Eq. 8): for one chunk of S = 64 keys and each landmark query q'_c of the
// group, p = softmax(tau q'_c . k_j), k' = sum_j p_j k_j, b' = -sum_j p_j log p_j.
//
// One workgroup per (chunk, KV head, batch).  The chunk's keys are read from
// HBM once (coalesced 16-byte loads), widened to fp32 in LDS with a padded
// row stride so that one key per lane reads conflict-free, and shared by the
// G query heads of the group (one wave per head).  HBM-bound: 16 KB of keys
// per (b, g, c) against G*(d*2+4) bytes written.
#include "hils_common.h"
#include "launch.h"

namespace hils {

constexpr int kSumS = 64;      // chunk size handled here
constexpr int kSumThreads = 256;

template <typename T, int D>
__global__ void __launch_bounds__(kSumThreads)
landmark_summary_kernel(const T *__restrict__ k, const T *__restrict__ q_lm, T *__restrict__ k_sum,
                        float *__restrict__ b_sum, int T_len, int Hq, int Hkv, int C, int c0,
                        float tau, const int32_t *__restrict__ block_table, int max_pages, int num_pages) {
  constexpr int LD = D + 1;  // padded fp32 row stride (conflict-free column reads)
  __shared__ float keys[kSumS * LD];
  __shared__ float qrow[4][D];
  __shared__ float prob[4][kSumS];
  const int c = c0 + blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const T *kc;
  if (block_table) {
    // paged keys: the chunk is one page; a page index outside the pool
    // makes the chunk's summary NaN for every head of the group
    const int pg = block_table[static_cast<size_t>(b) * max_pages + c];
    if (pg < 0 || pg >= num_pages) {
      for (int x = tid; x < G * (D + 1); x += kSumThreads) {
        const size_t so = (static_cast<size_t>(b) * Hq + g * G + x / (D + 1)) * C + c;
        if (x % (D + 1) == D)
          b_sum[so] = NAN;
        else
          Elem<T>::store(k_sum, so * D + x % (D + 1), NAN);
      }
      return;
    }
    kc = k + (static_cast<size_t>(pg) * Hkv + g) * kSumS * D;
  } else {
    kc = k + ((static_cast<size_t>(b) * Hkv + g) * T_len + static_cast<size_t>(c) * kSumS) * D;
  }
  // The chunk's keys (64 x D, pieces of 8 elements) and the first four
  // heads' landmark rows (lane e and e + 64 of the wave's head): every load
  // issued before any is used, raw, so that they share one round trip.
  constexpr int KP = kSumS * D / 8 / kSumThreads;  // pieces per thread
  constexpr int RPP = static_cast<int>(sizeof(T)) / 2;  // 16-byte loads per piece
  static_assert(kSumS * D / 8 % kSumThreads == 0, "whole pieces per thread");
  uint4 raw[KP][RPP];
#pragma unroll
  for (int r = 0; r < KP; ++r)
#pragma unroll
    for (int u = 0; u < RPP; ++u) raw[r][u] = reinterpret_cast<const uint4 *>(kc + (tid + r * kSumThreads) * 8)[u];
  T qraw[D / 64];
  {
    const int hq = g * G + (wave < G ? wave : 0);  // (a wave past G reads head 0 of the group, unused)
    const size_t so = (static_cast<size_t>(b) * Hq + hq) * C + c;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) qraw[i] = q_lm[so * D + lane + 64 * i];
  }
#pragma unroll
  for (int r = 0; r < KP; ++r) {
    float v[8];
    Elem<T>::load8(reinterpret_cast<const T *>(&raw[r][0]), v);
    const int e8 = tid + r * kSumThreads, row = (e8 * 8) / D, col = (e8 * 8) % D;
#pragma unroll
    for (int t = 0; t < 8; ++t) keys[row * LD + col + t] = v[t];
  }
  // (parked by every wave, used or not: a use under a branch would let the
  // compiler move the loads there, a round trip later)
#pragma unroll
  for (int i = 0; i < D / 64; ++i) qrow[wave][lane + 64 * i] = Elem<T>::load(qraw, i);

  __shared__ float ent_s[4];
  for (int h0 = 0; h0 < G; h0 += 4) {
    const int h = g * G + h0 + wave;
    const bool active = (h0 + wave) < G;
    const size_t so = (static_cast<size_t>(b) * Hq + h) * C + c;
    if (active && h0 > 0)  // the first four heads' rows are in place already
      for (int e = lane; e < D; e += 64) qrow[wave][e] = Elem<T>::load(q_lm, so * D + e);
    __syncthreads();
    if (active) {
      // logit of key j = lane
      float acc = 0.f;
#pragma unroll 8
      for (int e = 0; e < D; ++e) acc += qrow[wave][e] * keys[lane * LD + e];
      const float l = tau * acc;
      const float m = wave_max(l);
      const float ex = expf(l - m);
      const float z = wave_sum(ex);
      const float p = ex / z;
      // entropy in the shifted form: -sum p log p = log z - sum p (l - m)
      const float ent = logf(z) - wave_sum(p * (l - m));
      prob[wave][lane] = p;
      if (lane == 0) ent_s[wave] = ent;
    }
    __syncthreads();
    if (active) {
      for (int e = lane; e < D; e += 64) {
        float s = 0.f;
#pragma unroll 8
        for (int j = 0; j < kSumS; ++j) s += prob[wave][j] * keys[j * LD + e];
        Elem<T>::store(k_sum, so * D + e, s);
      }
      if (lane == 0) b_sum[so] = fmaxf(ent_s[wave], 0.f);
    }
    __syncthreads();
  }
}

template <typename T, int D>
static hipError_t launch_summary_t(const SummaryArgs &a, hipStream_t st) {
  dim3 grid(a.c1 - a.c0, a.Hkv, a.B);
  landmark_summary_kernel<T, D><<<grid, kSumThreads, 0, st>>>(
      static_cast<const T *>(a.k), static_cast<const T *>(a.q_lm), static_cast<T *>(a.k_sum),
      a.b_sum, a.T, a.Hq, a.Hkv, a.C, a.c0, a.tau, a.block_table, a.max_pages, a.num_pages);
  return hipGetLastError();
}

hipError_t launch_summary(const SummaryArgs &a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_summary_t<uint16_t, 128>(a, st) : launch_summary_t<uint16_t, 64>(a, st);
  return a.d == 128 ? launch_summary_t<float, 128>(a, st) : launch_summary_t<float, 64>(a, st);
}

}  // namespace hils
