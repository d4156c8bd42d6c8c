// Landmark chunk summary (HiLS-Attention, picx.dev summary, Methodology 1,
// Eq. 8): for one chunk of S = 64 keys and each landmark query q'_c of the
// group, p = softmax(tau q'_c . k_j), k' = sum_j p_j k_j, b' = -sum_j p_j log p_j.
//
// One workgroup per (chunk, KV head, batch).  The chunk's keys are read from
// HBM once (coalesced 16-byte loads) and kept in LDS in their storage type
// (bf16: 16 KB, so that eight workgroups share a CU), rows padded by one
// 32-bit word so that one key per lane reads conflict-free; they are shared
// by the G query heads of the group (one wave per head) and widened to fp32
// as they are read, two bf16 per 32-bit read.  HBM-bound: 16 KB of keys per
// (b, g, c) against G*(d*2+4) bytes written.
#include "hils_common.h"
#include "launch.h"

namespace hils {

constexpr int kSumS = 64;      // chunk size handled here
constexpr int kSumThreads = 256;

template <typename T, int D>
__global__ void __launch_bounds__(kSumThreads, sizeof(T) == 2 ? 8 : 4)  // bf16: eight workgroups per CU (LDS)
landmark_summary_kernel(const T *__restrict__ k, const T *__restrict__ q_lm, T *__restrict__ k_sum,
                        float *__restrict__ b_sum, int T_len, int Hq, int Hkv, int C, int c0,
                        float tau, const int32_t *__restrict__ block_table, int max_pages, int num_pages) {
  constexpr int EPW = 4 / static_cast<int>(sizeof(T));  // elements per 32-bit word
  constexpr int LW = D / EPW + 1;                       // padded row stride in words
  __shared__ uint32_t keys[kSumS * LW];
  __shared__ __align__(16) float qrow[4][D];
  __shared__ __align__(16) float prob[4][kSumS];
  // word x of key row j as EPW floats
  auto key_word = [&](int j, int x, float (&o)[EPW]) {
    const uint32_t w = keys[j * LW + x];
    if constexpr (EPW == 2) {
      o[0] = __uint_as_float(w << 16);
      o[1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      o[0] = __uint_as_float(w);
    }
  };
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
    const int e8 = tid + r * kSumThreads, row = (e8 * 8) / D, col = (e8 * 8) % D;
    const uint32_t *w = reinterpret_cast<const uint32_t *>(&raw[r][0]);
#pragma unroll
    for (int t = 0; t < 8 / EPW; ++t) keys[row * LW + col / EPW + t] = w[t];
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
      // logit of key j = lane (products in order of e)
      float acc = 0.f;
#pragma unroll 8
      for (int e4 = 0; e4 < D; e4 += 4) {
        const float4 q4 = *reinterpret_cast<const float4 *>(&qrow[wave][e4]);
        const float qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int x = 0; x < 4 / EPW; ++x) {
          float kv[EPW];
          key_word(lane, e4 / EPW + x, kv);
#pragma unroll
          for (int u = 0; u < EPW; ++u) acc = fmaf(qv[x * EPW + u], kv[u], acc);
        }
      }
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
      // k' over the keys in order of j; lane x owns the EPW elements of
      // word x of a row
      for (int x = lane; x < D / EPW; x += 64) {
        float sacc[EPW];
#pragma unroll
        for (int u = 0; u < EPW; ++u) sacc[u] = 0.f;
#pragma unroll 4
        for (int j4 = 0; j4 < kSumS; j4 += 4) {
          const float4 p4 = *reinterpret_cast<const float4 *>(&prob[wave][j4]);
          const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float kv[EPW];
            key_word(j4 + jj, x, kv);
#pragma unroll
            for (int u = 0; u < EPW; ++u) sacc[u] = fmaf(pv[jj], kv[u], sacc[u]);
          }
        }
        if constexpr (EPW == 2) {
          reinterpret_cast<uint32_t *>(k_sum)[(so * D) / 2 + x] =
              static_cast<uint32_t>(f32_to_bf16(sacc[0])) | (static_cast<uint32_t>(f32_to_bf16(sacc[1])) << 16);
        } else {
          Elem<T>::store(k_sum, so * D + x, sacc[0]);
        }
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
