// Block-level attention over one "unit" of up to 64 consecutive keys of one
// KV head, for the G query heads of its group (VALU, fp32 accumulation).
//
// A unit is either one selected chunk (S = 64 keys) or a 64-key slice of the
// sliding window / of the whole causal prefix.  For each head h it yields the
// online-softmax partial
//     m_h = max_j lam_hj,  l_h = sum_j e^{lam_hj - m_h},  o_h = sum_j e^{lam_hj - m_h} v_j
// with lam_hj = tau * q_h . k_j.  Partials of different units combine by the
// usual log-sum-exp rescaling; a selected chunk enters the hierarchical
// fusion (Eq. 10 of the picx.dev summary) as the partial (s_hat, 1, o_h/l_h).
//
// Thread layout (256 threads):
//   logits  thread t -> key t/4, quarter t%4 of the head dim (dot product of
//           D/4 elements per head, reduced over the 4 quarter lanes);
//   softmax one wave per head (lane = key);
//   P.V     thread t -> output pairs (head, 2 dims) t, t+256, ...; each
//           thread walks the unit's value rows (coalesced row reads).
#pragma once

#include "hils_common.h"

namespace hils {

constexpr int kUnitThreads = 256;
constexpr int kMaxG = 16;
constexpr int kUnitKeys = 64;

template <typename T, int D>
struct UnitSmem {
  float q[kMaxG][D];          // query rows of the group (fp32)
  float p[kMaxG][kUnitKeys];  // logits, then probabilities
  float m[kMaxG], l[kMaxG];
  uint4 v[kUnitKeys * D * sizeof(T) / 16];  // the unit's value rows, raw
};

// Number of (head, dim-pair) outputs each thread owns.
template <int D>
constexpr int pairs_per_thread() { return (kMaxG * D / 2 + kUnitThreads - 1) / kUnitThreads; }

template <typename T, int D>
__device__ __forceinline__ void load_q_rows(UnitSmem<T, D> &sm, const T *q, size_t head_stride, int G) {
  for (int x = threadIdx.x; x < G * D; x += kUnitThreads)
    sm.q[x / D][x % D] = Elem<T>::load(q, static_cast<size_t>(x / D) * head_stride + (x % D));
}

// Attend the G rows in sm.q to keys [0, nk) of krow/vrow (row stride D).
// On return sm.m / sm.l hold the per-head statistics and o[] the caller's
// unnormalised output pairs (see pairs_per_thread).  Must be called by all
// threads of the block.
template <typename T, int D>
__device__ __forceinline__ void attend_unit(UnitSmem<T, D> &sm, const T *__restrict__ krow,
                                            const T *__restrict__ vrow, int nk, int G, float tau,
                                            float2 (&o)[pairs_per_thread<D>()]) {
  constexpr int QD = D / 4;  // elements per quarter
  constexpr int VPT = kUnitKeys * D * static_cast<int>(sizeof(T)) / 16 / kUnitThreads;  // 16-B pieces per thread
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // value rows: issue the loads first, park them in LDS after the logits.
  // No load sits under a lane-dependent branch (a lane past the unit reads
  // piece / row 0 again; those values are zeroed or masked afterwards), so
  // every load is in flight before the first is used.
  const int vpieces = nk * D * static_cast<int>(sizeof(T)) / 16;
  uint4 vreg[VPT];
#pragma unroll
  for (int r = 0; r < VPT; ++r) {
    const int pc = t + r * kUnitThreads;
    vreg[r] = reinterpret_cast<const uint4 *>(vrow)[pc < vpieces ? pc : 0];
  }
  {
    const int j = t >> 2, qq = t & 3;
    float kv[QD];
    const int jr = j < nk ? j : 0;
#pragma unroll
    for (int e8 = 0; e8 < QD / 8; ++e8) Elem<T>::load8(krow + static_cast<size_t>(jr) * D + qq * QD + e8 * 8, kv + e8 * 8);
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < QD; ++e) acc += sm.q[h][qq * QD + e] * kv[e];
      acc = group_sum<4>(acc);
      if (qq == 0) sm.p[h][j] = (j < nk) ? tau * acc : -INFINITY;
    }
  }
#pragma unroll
  for (int r = 0; r < VPT; ++r) {
    const int pc = t + r * kUnitThreads;
    sm.v[pc] = pc < vpieces ? vreg[r] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  for (int h = wave; h < G; h += kUnitThreads / 64) {
    const float lam = sm.p[h][lane];
    const float m = wave_reduce_f32<1>(lam);
    const float e = (lam == -INFINITY) ? 0.f : __expf(lam - m);
    const float l = wave_reduce_f32<2>(e);
    sm.p[h][lane] = e;
    if (lane == 0) { sm.m[h] = m; sm.l[h] = l; }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < pairs_per_thread<D>(); ++r) {
    const int pr = t + r * kUnitThreads;
    const int h = pr / (D / 2), e2 = pr % (D / 2);
    float2 acc = make_float2(0.f, 0.f);
    if (h < G) {
      // eight keys per step, their LDS reads issued together (keys past nk
      // have p = 0 and zero value rows)
      const T *vs = reinterpret_cast<const T *>(sm.v);
      for (int j0 = 0; j0 < nk; j0 += 8) {
        float v2[8][2], pj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          Elem<T>::load2(vs + (j0 + u) * D + 2 * e2, v2[u]);
          pj[u] = sm.p[h][j0 + u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          acc.x += pj[u] * v2[u][0];
          acc.y += pj[u] * v2[u][1];
        }
      }
    }
    o[r] = acc;
  }
  __syncthreads();
}

// Running log-sum-exp accumulator for the output pairs a thread owns.
template <int D>
struct PairAcc {
  float2 o[pairs_per_thread<D>()];
  float m[pairs_per_thread<D>()], l[pairs_per_thread<D>()];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int r = 0; r < pairs_per_thread<D>(); ++r) { o[r] = make_float2(0.f, 0.f); m[r] = -INFINITY; l[r] = 0.f; }
  }
  // add partial (m2, l2, o2) for the pair r
  __device__ __forceinline__ void add(int r, float m2, float l2, float2 o2) {
    if (m2 == -INFINITY) return;
    const float mn = fmaxf(m[r], m2);
    const float sa = (m[r] == -INFINITY) ? 0.f : __expf(m[r] - mn);
    const float sb = __expf(m2 - mn);
    o[r].x = o[r].x * sa + o2.x * sb;
    o[r].y = o[r].y * sa + o2.y * sb;
    l[r] = l[r] * sa + l2 * sb;
    m[r] = mn;
  }
};

}  // namespace hils
