// Pieces shared by the two key-major backward kernels (VALU and MFMA): the
// backward of the Eq. 8 landmark summary of one chunk (picx.dev summary,
// Methodology 1), run after the chunk's key and value gradients from the
// attention rows are complete.
#pragma once

#include "hils_common.h"
#include "launch.h"

namespace hils {
namespace bwd {

constexpr int kBT = 256;    // threads per workgroup
constexpr int kBK = 64;     // keys per block (= chunk size S)
constexpr int kQBlk = 256;  // queries per block of the inverse-list build

// Reduce over the 4 consecutive lanes 4m .. 4m+3.
__device__ __forceinline__ float sum4(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  return v;
}

template <int D>
struct SummaryScratch {
  float qlm[D], kp[D], pl[kBK], dlj[kBK];
  float red[4][2];
};

// The summary backward of chunk kb for every head of group g, by a 256-thread
// workgroup in which thread t owns key j = t >> 2 and the quarter qd = t & 3
// of the head dimension.  On entry:
//   kt        [64][D + 1]   the chunk's keys (fp32, LDS)
//   kr        the thread's QD = D/4 key elements (registers)
//   dk        the thread's key-gradient elements so far (updated in place)
//   dkp       [G][D] (LDS)  tau * sum over the chunk's selecting rows of ds q
//                           (the raw-q part of dk'); completed here with the
//                           Q-Cal part tau * W_up_h z_{c,h} when r > 0
// z [B,Hq,C,r] and zb [B,Hq,C] hold sum ds u and sum ds per (chunk, head)
// (not read when K = 0: both are zero then).
// With l_j = tau q'_c.k_j, p = softmax(l), k' = sum p_j k_j, E = sum p_j l_j:
//   dl_j = p_j (dk'.(k_j - k') - db' (l_j - E)),
//   dk_j += p_j dk' + tau dl_j q'_c,   dq'_c = tau sum_j dl_j k_j.
template <typename T, int D>
__device__ void summary_backward(const BwdArgs &a, int b, int g, int kb, const float (*kt)[D + 1], const float *kr,
                                 float *dk, float (*dkp)[D], SummaryScratch<D> &ss) {
  constexpr int QD = D / 4;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, j = t >> 2, qd = t & 3;
  const int Hq = a.Hq, G = a.Hq / a.Hkv, C = a.T / kBK, r = a.r;
  const float tau = a.tau;
  if (r > 0 && a.K > 0) {  // dk' += tau W_up_h z_{c,h} (z is zero without a selection)
    const T *wu = static_cast<const T *>(a.w_up);
    for (int x = t; x < G * D; x += kBT) {
      const int hh = x / D, e = x % D, h = g * G + hh;
      const float *zr = a.zsum + ((static_cast<size_t>(b) * Hq + h) * C + kb) * r;
      const T *wr = wu + (static_cast<size_t>(h) * D + e) * r;
      float acc = 0.f;
      for (int q = 0; q < r; ++q) acc += Elem<T>::load(wr, q) * zr[q];
      dkp[hh][e] += tau * acc;
    }
    __syncthreads();
  }
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    const size_t so = (static_cast<size_t>(b) * Hq + h) * C + kb;
    const float dbp = a.K > 0 ? a.zb[so] : 0.f;
    for (int x = t; x < D; x += kBT) ss.qlm[x] = Elem<T>::load(static_cast<const T *>(a.q_lm), so * D + x);
    __syncthreads();
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < QD; ++u) l += ss.qlm[qd * QD + u] * kr[u];
    l = tau * sum4(l);
    // softmax over the 64 keys (4 lanes per key): block maximum, then sums
    float m = wave_max(l);
    if (lane == 0) ss.red[wv][0] = m;
    __syncthreads();
    m = fmaxf(fmaxf(ss.red[0][0], ss.red[1][0]), fmaxf(ss.red[2][0], ss.red[3][0]));
    __syncthreads();
    const float ex = __expf(l - m);
    const float s = wave_sum(ex) * 0.25f;  // each key counted by its 4 lanes
    const float sl = wave_sum(ex * l) * 0.25f;
    if (lane == 0) {
      ss.red[wv][0] = s;
      ss.red[wv][1] = sl;
    }
    __syncthreads();
    const float z = ss.red[0][0] + ss.red[1][0] + ss.red[2][0] + ss.red[3][0];
    const float El = (ss.red[0][1] + ss.red[1][1] + ss.red[2][1] + ss.red[3][1]) / z;
    const float p = ex / z;
    if (qd == 0) ss.pl[j] = p;
    __syncthreads();
    // k' (unrounded) = sum_j p_j k_j, a fixed key order per element
    for (int e = t; e < D; e += kBT) {
      float acc = 0.f;
      for (int jk = 0; jk < kBK; ++jk) acc += ss.pl[jk] * kt[jk][e];
      ss.kp[e] = acc;
    }
    __syncthreads();
    float proj = 0.f;
#pragma unroll
    for (int u = 0; u < QD; ++u) proj += dkp[hh][qd * QD + u] * (kr[u] - ss.kp[qd * QD + u]);
    proj = sum4(proj);
    const float dl = p * (proj - dbp * (l - El));
#pragma unroll
    for (int u = 0; u < QD; ++u) dk[u] += p * dkp[hh][qd * QD + u] + tau * dl * ss.qlm[qd * QD + u];
    if (qd == 0) ss.dlj[j] = dl;
    __syncthreads();
    for (int e = t; e < D; e += kBT) {
      float acc = 0.f;
      for (int jk = 0; jk < kBK; ++jk) acc += ss.dlj[jk] * kt[jk][e];
      a.dq_lm[so * D + e] = tau * acc;
    }
    __syncthreads();
  }
}

}  // namespace bwd
}  // namespace hils
