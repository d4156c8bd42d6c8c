// Backward pass of the HiLS-Attention prefill forward, for a fixed top-K
// selection (fp32 accumulation).
//
// The pages train chunk selection through the forward weights: each selected
// chunk's score s_hat sits in the joint softmax of Eq. 10 (picx.dev
// summary, Methodology 2), so the loss reaches s_hat, hence k'_c, b'_c and,
// through Eq. 8 (Methodology 1), the landmark queries and the chunk keys;
// Q-Cal (Methodology 3) passes the score gradient on to W_up, W_down and h.
// The top-K choice itself is discrete and carries no gradient.
//
// For a row (b, h, i) with selected chunks c (score s_c), window tokens j and
// logZ = log( sum_c e^{s_c} + sum_j e^{l_j} ), l_j = tau q.k_j:
//   w_c = e^{s_c - logZ}, P_cj = chunk softmax, o_c = sum_j P_cj v_j,
//   u_j = e^{l_j - logZ}, Delta = dO.o = sum_c w_c dO.o_c + sum_j u_j dO.v_j
//   ds_c = w_c (dO.o_c - Delta)
//   dl_j = w_c P_cj (dO.v_j - dO.o_c)   (chunk)   or   u_j (dO.v_j - Delta)   (window)
//   dq += tau sum_j dl_j k_j + tau sum_c ds_c k'_c (through q_hat),
//   dk_j += tau sum_rows dl_j q,   dv_j += sum_rows (w_c P_cj or u_j) dO
//   dk'_c += tau ds_c q_hat,  db'_c += ds_c
// and per (b, h, c), with l_j = tau q'_c.k_j, p = softmax(l), k' = sum p_j k_j,
// E = sum p_j l_j:
//   dl_j = p_j ( dk'.(k_j - k') - db' (l_j - E) ),
//   dq'_c = tau sum_j dl_j k_j,   dk_j += p_j dk' + tau dl_j q'_c.
// Q-Cal: q_hat = q + W_up u, u = W_down h, so dk'_c = tau sum ds q +
// tau W_up_h z_c with z_c = sum ds u over the rows that selected chunk c.
//
// Kernels (all on the caller's stream):
//   [qcal]  u = h W_down^T, q_hat = q + u W_up^T           (tiled fp32 GEMM)
//   lists   the inverse of the selection: for every (b, g, chunk) the
//           (query, slot) entries that selected it, ordered by query
//           (counted per 256-query block, no atomics on the order), and
//           each slot's place in its list.
//   rows    one workgroup per (i, g, b), one wave per head (4 at a time), one
//           pass over the row's selected chunks and window blocks (staged in
//           LDS): logZ and Delta, and dq and dq_hat from running sums that
//           the normaliser scales at the end.  Writes dq, dq_hat, logZ and
//           Delta, and each list entry's log-weight, dO.o_c and ds_c.
//   z       per (b, g, chunk): z = sum ds u and sum ds over the chunk's list.
//   keys    per 64-key block (b, g): every row whose window covers the block,
//           then (complete chunks) every entry of the chunk's list with its
//           G heads; accumulates dk, dv (bf16 MFMA kernel where the shape
//           allows, else the VALU kernel below), then the chunk's summary
//           backward.
//   [qcal]  du = dq_hat W_up, dW_up = dq_hat^T u, dW_down = du^T h,
//           dh = du W_down                                  (tiled fp32 GEMM)
// Every sum runs in a fixed order: the results are the same on every run.
#include "bwd_common.h"

namespace hils {

using bwd::kBK;
using bwd::kBT;
using bwd::kQBlk;
using bwd::sum4;

namespace {

constexpr int kRowsPerBatch = 8;

// A 64-row key or value tile of the row kernel in LDS, in the storage type:
// bf16 rows D + 4 elements apart (8-byte aligned groups of 4), fp32 rows
// D + 2 apart (8-byte aligned pairs); lane j of a wave reading row j meets
// bank 2 j + const.  Rows past T are zero.
template <typename T, int D>
struct RowTile;

template <int D>
struct RowTile<uint16_t, D> {
  uint16_t x[kBK][D + 4];
  __device__ __forceinline__ void stage(const uint16_t *src, int j0, int T_len) {
    for (int p = threadIdx.x; p < kBK * D / 8; p += kBT) {
      const int r = p / (D / 8), s = p % (D / 8);
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (j0 + r < T_len) u = *reinterpret_cast<const uint4 *>(src + static_cast<size_t>(j0 + r) * D + s * 8);
      *reinterpret_cast<uint2 *>(&x[r][s * 8]) = make_uint2(u.x, u.y);
      *reinterpret_cast<uint2 *>(&x[r][s * 8 + 4]) = make_uint2(u.z, u.w);
    }
  }
  // elements e .. e + 3 of row j (e a multiple of 4)
  __device__ __forceinline__ void load4(int j, int e, float *o) const {
    const uint2 w = *reinterpret_cast<const uint2 *>(&x[j][e]);
    o[0] = __uint_as_float(w.x << 16);
    o[1] = __uint_as_float(w.x & 0xFFFF0000u);
    o[2] = __uint_as_float(w.y << 16);
    o[3] = __uint_as_float(w.y & 0xFFFF0000u);
  }
  // elements e .. e + N - 1 of row j (N = 1 or 2, e a multiple of N)
  template <int N>
  __device__ __forceinline__ void loadn(int j, int e, float *o) const {
    if (N == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t *>(&x[j][e]);
      o[0] = __uint_as_float(w << 16);
      o[N - 1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      o[0] = bf16_to_f32(x[j][e]);
    }
  }
};

template <int D>
struct RowTile<float, D> {
  float x[kBK][D + 2];
  __device__ __forceinline__ void stage(const float *src, int j0, int T_len) {
    for (int p = threadIdx.x; p < kBK * D / 4; p += kBT) {
      const int r = p / (D / 4), s = p % (D / 4);
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j0 + r < T_len) u = *reinterpret_cast<const float4 *>(src + static_cast<size_t>(j0 + r) * D + s * 4);
      *reinterpret_cast<float2 *>(&x[r][s * 4]) = make_float2(u.x, u.y);
      *reinterpret_cast<float2 *>(&x[r][s * 4 + 2]) = make_float2(u.z, u.w);
    }
  }
  __device__ __forceinline__ void load4(int j, int e, float *o) const {
    const float2 a = *reinterpret_cast<const float2 *>(&x[j][e]);
    const float2 b = *reinterpret_cast<const float2 *>(&x[j][e + 2]);
    o[0] = a.x; o[1] = a.y; o[2] = b.x; o[3] = b.y;
  }
  template <int N>
  __device__ __forceinline__ void loadn(int j, int e, float *o) const {
    if (N == 2) {
      const float2 a = *reinterpret_cast<const float2 *>(&x[j][e]);
      o[0] = a.x;
      o[N - 1] = a.y;
    } else {
      o[0] = x[j][e];
    }
  }
};

}  // namespace

// ------------------------------------------------------------------ fp32 GEMM
// C[m, n] = sum_k A(m, k) B(k, n) with A(m, k) = A[m lam + k lak] and
// B(k, n) = B[k lbk + n lbn] (any strides), fp32 accumulation in a fixed k
// order.  64 x 64 output tiles per 256-thread workgroup (4 x 4 per thread),
// k in slabs of 16 staged in LDS.  MODE 0 stores C[m lcm + n lcn]; MODE 1 is
// the Q-Cal q_hat: m = token b T + i, n = h D + e, and the tile adds
// q[b, h, i, e] and stores q_hat in the same [B, Hq, T, D] layout.  With
// gridDim.z > 1 workgroup z takes the k range [z kc, z kc + kc) and stores
// its partial sums at Cm + z M N, row-major (MODE 0); gemm_reduce_kernel
// then adds the partials in z order.
template <typename TA, typename TB, int MODE>
__global__ void __launch_bounds__(256)
bwd_gemm_kernel(const TA *__restrict__ A, long lam, long lak, const TB *__restrict__ Bm, long lbk, long lbn,
                float *__restrict__ Cm, long lcm, long lcn, int M, int N, int Kd, int kc, const TB *__restrict__ qadd,
                int Hq, int T_len, int D) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int t = threadIdx.x, tm = t >> 4, tn = t & 15;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int kbeg = blockIdx.z * kc, kend = min(Kd, kbeg + kc);
  if (gridDim.z > 1) {
    Cm += static_cast<size_t>(blockIdx.z) * M * N;
    lcm = N;
    lcn = 1;
  }
  const bool a_kfast = lak == 1, b_nfast = lbn == 1;
  float acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.f;
  for (int k0 = kbeg; k0 < kend; k0 += 16) {
    float av[4], bv[4];
    int am[4], ak[4], bk[4], bn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = t + 256 * j;  // 1024 elements of each slab
      am[j] = a_kfast ? x / 16 : x % 64;
      ak[j] = a_kfast ? x % 16 : x / 64;
      bk[j] = b_nfast ? x / 64 : x % 16;
      bn[j] = b_nfast ? x % 64 : x / 16;
      const int gm = m0 + am[j], gk = k0 + ak[j];
      av[j] = (gm < M && gk < kend) ? Elem<TA>::load(A, gm * lam + gk * lak) : 0.f;
      const int gk2 = k0 + bk[j], gn = n0 + bn[j];
      bv[j] = (gk2 < kend && gn < N) ? Elem<TB>::load(Bm, gk2 * lbk + gn * lbn) : 0.f;
    }
    __syncthreads();  // the previous slab is no longer read
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      As[ak[j]][am[j]] = av[j];
      Bs[bk[j]][bn[j]] = bv[j];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const float4 a4 = *reinterpret_cast<const float4 *>(&As[kk][tm * 4]);
      const float4 b4 = *reinterpret_cast<const float4 *>(&Bs[kk][tn * 4]);
      const float a_[4] = {a4.x, a4.y, a4.z, a4.w}, b_[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] += a_[x] * b_[y];
    }
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int m = m0 + tm * 4 + x;
    if (m >= M) continue;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int n = n0 + tn * 4 + y;
      if (n >= N) continue;
      if (MODE == 0) {
        Cm[m * lcm + n * lcn] = acc[x][y];
      } else {
        const int b = m / T_len, i = m % T_len, h = n / D, e = n % D;
        const size_t o = ((static_cast<size_t>(b) * Hq + h) * T_len + i) * D + e;
        Cm[o] = Elem<TB>::load(qadd, o) + acc[x][y];
      }
    }
  }
}

__global__ void __launch_bounds__(256)
gemm_reduce_kernel(const float *__restrict__ part, int nsplit, float *__restrict__ Cm, long lcm, long lcn, int M, int N) {
  const size_t x = blockIdx.x * static_cast<size_t>(256) + threadIdx.x, MN = static_cast<size_t>(M) * N;
  if (x >= MN) return;
  float acc = 0.f;
  for (int z = 0; z < nsplit; ++z) acc += part[z * MN + x];
  const int m = static_cast<int>(x / N), n = static_cast<int>(x % N);
  Cm[m * lcm + n * lcn] = acc;
}

// nsplit > 1 splits k over nsplit workgroups per tile, through part
// (nsplit M N floats), then sums the partials in a fixed order.
template <typename TA, typename TB, int MODE = 0>
static hipError_t gemm(const TA *A, long lam, long lak, const TB *Bm, long lbk, long lbn, float *Cm, long lcm, long lcn,
                       int M, int N, int Kd, hipStream_t st, int nsplit = 1, float *part = nullptr,
                       const TB *qadd = nullptr, int Hq = 0, int T_len = 1, int D = 1) {
  const int kc = ((Kd + nsplit - 1) / nsplit + 15) / 16 * 16;
  nsplit = kc > 0 ? (Kd + kc - 1) / kc : 1;
  const dim3 grid((N + 63) / 64, (M + 63) / 64, nsplit);
  bwd_gemm_kernel<TA, TB, MODE><<<grid, 256, 0, st>>>(A, lam, lak, Bm, lbk, lbn, nsplit > 1 ? part : Cm, lcm, lcn,
                                                      M, N, Kd, kc, qadd, Hq, T_len, D);
  if (nsplit > 1) {
    const size_t MN = static_cast<size_t>(M) * N;
    gemm_reduce_kernel<<<static_cast<unsigned>((MN + 255) / 256), 256, 0, st>>>(part, nsplit, Cm, lcm, lcn, M, N);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ inverse lists
// For each (b, g) and chunk c, the entries (i, slot) with topk_idx[b,g,i,slot]
// == c (and c < n_i), ordered by i.  cnt [B, Hkv, nqb, C]: entries per
// 256-query block; qboff: their offset inside the chunk's list; choff
// [B, Hkv, C + 1]: each chunk's first entry; list [B, Hkv, T K]: i * 32 + slot;
// pos [B, Hkv, T, K]: the entry's place in the list (-1 for no chunk).
struct InvSmem {
  uint32_t mask[kMaxBwdChunks][kQBlk / 32];
};

__device__ __forceinline__ void inv_masks(InvSmem &sm, const BwdArgs &a, int qb, int g, int b, int C) {
  const int t = threadIdx.x, i = qb * kQBlk + t;
  for (int x = t; x < C * (kQBlk / 32); x += kBT) (&sm.mask[0][0])[x] = 0u;
  __syncthreads();
  if (i < a.T) {
    const int n = eligible_chunks(i, a.W, kBK);
    const int32_t *ir = a.topk_idx + ((static_cast<size_t>(b) * a.Hkv + g) * a.T + i) * a.K;
    for (int k = 0; k < a.K; ++k) {
      const int c = ir[k];
      if (c >= 0 && c < n) atomicOr(&sm.mask[c][t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(kBT) bwd_inv_count_kernel(BwdArgs a) {
  __shared__ InvSmem sm;
  const int qb = blockIdx.x, g = blockIdx.y, b = blockIdx.z, C = a.T / kBK, nqb = gridDim.x;
  inv_masks(sm, a, qb, g, b, C);
  int *cnt = a.inv_cnt + ((static_cast<size_t>(b) * a.Hkv + g) * nqb + qb) * C;
  for (int c = threadIdx.x; c < C; c += kBT) {
    int s = 0;
#pragma unroll
    for (int x = 0; x < kQBlk / 32; ++x) s += __popc(sm.mask[c][x]);
    cnt[c] = s;
  }
}

__global__ void __launch_bounds__(kBT) bwd_inv_scan_kernel(BwdArgs a, int nqb) {
  __shared__ int tot[kMaxBwdChunks + 1];
  const int g = blockIdx.x, b = blockIdx.y, C = a.T / kBK;
  const size_t pg = static_cast<size_t>(b) * a.Hkv + g;
  for (int c = threadIdx.x; c < C; c += kBT) {
    int run = 0;
    for (int qb = 0; qb < nqb; ++qb) {
      const size_t o = (pg * nqb + qb) * C + c;
      a.inv_qboff[o] = run;
      run += a.inv_cnt[o];
    }
    tot[c] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // C <= 512: a short serial prefix
    int run = 0;
    for (int c = 0; c < C; ++c) {
      a.inv_choff[pg * (C + 1) + c] = run;
      run += tot[c];
    }
    a.inv_choff[pg * (C + 1) + C] = run;
  }
}

__global__ void __launch_bounds__(kBT) bwd_inv_fill_kernel(BwdArgs a) {
  __shared__ InvSmem sm;
  const int qb = blockIdx.x, g = blockIdx.y, b = blockIdx.z, C = a.T / kBK, nqb = gridDim.x;
  inv_masks(sm, a, qb, g, b, C);
  const int t = threadIdx.x, i = qb * kQBlk + t;
  if (i >= a.T) return;
  const size_t pg = static_cast<size_t>(b) * a.Hkv + g;
  const int n = eligible_chunks(i, a.W, kBK);
  const int32_t *ir = a.topk_idx + (pg * a.T + i) * a.K;
  int32_t *pr = a.inv_pos + (pg * a.T + i) * a.K;
  for (int k = 0; k < a.K; ++k) {
    const int c = ir[k];
    if (c < 0 || c >= n) {
      pr[k] = -1;
      continue;
    }
    int rank = 0;
    for (int x = 0; x < (t >> 5); ++x) rank += __popc(sm.mask[c][x]);
    rank += __popc(sm.mask[c][t >> 5] & ((1u << (t & 31)) - 1u));
    const int pos = a.inv_choff[pg * (C + 1) + c] + a.inv_qboff[(pg * nqb + qb) * C + c] + rank;
    a.inv_list[pg * static_cast<size_t>(a.T) * a.K + pos] = i * 32 + k;
    pr[k] = pos;
  }
}

// ------------------------------------------------------------------ rows
template <typename T, int D>
struct RowSmem {
  RowTile<T, D> kt, vt;
  float qs[4][D], qhs[4][D], dos[4][D];
  float ew[4][kBK], dvw[4][kBK];      // per head: the block's weights and dO.v_j
  float sl_m[4][32], sl_l[4][32];     // per selected chunk: max and sum of e^{l - max}
  float sl_doo[4][32], sl_s[4][32];   // dO.o_c and s_hat
  int sel[32];                        // the row's chunks (list order; -1: none)
};

// One pass over the row's blocks.  The chunk scores are computed first (from
// the stored summaries), so their maximum Mc is known before any chunk is
// read; the window keeps an online maximum mw.  Running sums, per lane's
// elements e of d:
//   window  A1 = sum e^{l_j - mw} dO.v_j k_j,  A2 = sum e^{l_j - mw} k_j
//   chunks  Bq = sum_c e^{s_c - Mc} sum_j P_cj (dO.v_j - dO.o_c) k_j,
//           B1 = sum_c e^{s_c - Mc} dO.o_c k'_c,  B2 = sum_c e^{s_c - Mc} k'_c
// and at the end, with logZ and Delta:
//   dq_hat = tau e^{Mc - logZ} (B1 - Delta B2)
//   dq     = tau (e^{Mc - logZ} Bq + e^{mw - logZ} (A1 - Delta A2)) + dq_hat.
template <typename T, int D, bool QCAL>
__global__ void __launch_bounds__(kBT)
bwd_rows_kernel(BwdArgs a) {
  __shared__ RowSmem<T, D> sm;
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int T_len = a.T, K = a.K, Hq = a.Hq, Hkv = a.Hkv, C = T_len / kBK;
  const int G = Hq / Hkv;
  const float tau = a.tau;
  const int n = eligible_chunks(i, a.W, kBK), w_lo = n * kBK;
  const int nwb = (i - w_lo) / kBK + 1;
  const size_t pg = static_cast<size_t>(b) * Hkv + g;
  const T *kb = static_cast<const T *>(a.k) + pg * T_len * D;
  const T *vb = static_cast<const T *>(a.v) + pg * T_len * D;
  const T *ksum = static_cast<const T *>(a.k_sum);
  // the row's selection (an id outside [0, n_i) is no chunk)
  if (t < 32) {
    int c = -1;
    if (t < K) c = a.topk_idx[(pg * T_len + i) * K + t];
    sm.sel[t] = (c >= 0 && c < n) ? c : -1;
  }
  __syncthreads();
  constexpr int EPL = D / 64;  // elements of d per lane
  for (int h0 = 0; h0 < G; h0 += 4) {
    const int hh = h0 + w, h = g * G + hh;
    const bool act = hh < G;
    const size_t ro = (static_cast<size_t>(b) * Hq + (act ? h : g * G)) * T_len + i;  // row (b, h, i)
    for (int x = lane; x < D; x += 64) {
      sm.qs[w][x] = Elem<T>::load(static_cast<const T *>(a.q), ro * D + x);
      sm.qhs[w][x] = QCAL ? a.qhat[ro * D + x] : sm.qs[w][x];
      sm.dos[w][x] = Elem<T>::load(static_cast<const T *>(a.d_o), ro * D + x);
    }
    // the chunk scores s_hat = tau q_hat . k'_c + b'_c and their maximum
    float Mc = -INFINITY;
    if (act) {
      for (int x = 0; x < K; ++x) {
        if (sm.sel[x] < 0) continue;
        const size_t so = (static_cast<size_t>(b) * Hq + h) * C + sm.sel[x];
        float sp = 0.f;
#pragma unroll
        for (int u = 0; u < EPL; ++u) sp += sm.qhs[w][lane * EPL + u] * Elem<T>::load(ksum, so * D + lane * EPL + u);
        const float s = tau * wave_sum(sp) + a.b_sum[so];
        if (lane == 0) sm.sl_s[w][x] = s;
        Mc = fmaxf(Mc, s);
      }
    }
    float mw = -INFINITY, zw = 0.f, dw = 0.f;  // window: max, sum e^{l - mw}, sum e^{l - mw} dO.v
    float A1[EPL], A2[EPL], Bq[EPL], B1[EPL], B2[EPL];
#pragma unroll
    for (int u = 0; u < EPL; ++u) A1[u] = A2[u] = Bq[u] = B1[u] = B2[u] = 0.f;
    for (int x = 0; x < K + nwb; ++x) {
      const bool chunk = x < K;
      if (chunk && sm.sel[x] < 0) continue;  // uniform across the workgroup
      const int j0 = chunk ? sm.sel[x] * kBK : w_lo + (x - K) * kBK;
      __syncthreads();  // the previous block's tiles are no longer read
      sm.kt.stage(kb, j0, T_len);
      sm.vt.stage(vb, j0, T_len);
      __syncthreads();
      if (!act) continue;
      // lane = key j of the block: l_j and dO.v_j
      float l = 0.f, dov = 0.f;
#pragma unroll 4
      for (int e = 0; e < D; e += 4) {
        const float4 q4 = *reinterpret_cast<const float4 *>(&sm.qs[w][e]);
        const float4 o4 = *reinterpret_cast<const float4 *>(&sm.dos[w][e]);
        float k4[4], v4[4];
        sm.kt.load4(lane, e, k4);
        sm.vt.load4(lane, e, v4);
        l += q4.x * k4[0] + q4.y * k4[1] + q4.z * k4[2] + q4.w * k4[3];
        dov += o4.x * v4[0] + o4.y * v4[1] + o4.z * v4[2] + o4.w * v4[3];
      }
      l *= tau;
      float wj, cj;  // the key's weight and the value it is compared against
      if (chunk) {
        const float m = wave_max(l);
        const float p = __expf(l - m);
        const float lsum = wave_sum(p);
        const float doo = wave_sum(p * dov) / lsum;
        if (lane == 0) {
          sm.sl_m[w][x] = m;
          sm.sl_l[w][x] = lsum;
          sm.sl_doo[w][x] = doo;
        }
        wj = p / lsum;
        cj = doo;
        // dq_hat terms: e^{s - Mc} dO.o_c k'_c and e^{s - Mc} k'_c
        const float sw = __expf(sm.sl_s[w][x] - Mc);
        const size_t so = (static_cast<size_t>(b) * Hq + h) * C + sm.sel[x];
#pragma unroll
        for (int u = 0; u < EPL; ++u) {
          const float kp = Elem<T>::load(ksum, so * D + lane * EPL + u);
          B1[u] += sw * doo * kp;
          B2[u] += sw * kp;
        }
        sm.ew[w][lane] = wj * (dov - cj);
      } else {
        const int jj = j0 + lane;
        const float lm = jj <= i ? l : -INFINITY;
        const float mn = fmaxf(mw, wave_max(lm));
        const float sc = mw == -INFINITY ? 0.f : __expf(mw - mn);
        const float e = jj <= i ? __expf(lm - mn) : 0.f;
        zw = zw * sc + wave_sum(e);
        dw = dw * sc + wave_sum(e * dov);
        mw = mn;
#pragma unroll
        for (int u = 0; u < EPL; ++u) {
          A1[u] *= sc;
          A2[u] *= sc;
        }
        sm.ew[w][lane] = e;
        sm.dvw[w][lane] = dov;
      }
      // the wave's own LDS rows, written and read by its lanes (LDS
      // operations of one wave complete in order: no wait needed)
      __builtin_amdgcn_wave_barrier();
      if (chunk) {
        const float sw = __expf(sm.sl_s[w][x] - Mc);
        float acc[EPL];
#pragma unroll
        for (int u = 0; u < EPL; ++u) acc[u] = 0.f;
        for (int j = 0; j < kBK; ++j) {
          const float c = sm.ew[w][j];
          float kv[EPL];
          sm.kt.template loadn<EPL>(j, lane * EPL, kv);
#pragma unroll
          for (int u = 0; u < EPL; ++u) acc[u] += c * kv[u];
        }
#pragma unroll
        for (int u = 0; u < EPL; ++u) Bq[u] += sw * acc[u];
      } else {
        for (int j = 0; j < kBK; ++j) {
          const float e = sm.ew[w][j], ed = e * sm.dvw[w][j];
          float kv[EPL];
          sm.kt.template loadn<EPL>(j, lane * EPL, kv);
#pragma unroll
          for (int u = 0; u < EPL; ++u) {
            A1[u] += ed * kv[u];
            A2[u] += e * kv[u];
          }
        }
      }
    }
    __syncthreads();
    if (act) {
      // ---- the joint normaliser, Delta, the list entries' values, dq
      const float M = fmaxf(Mc, mw);
      float z = zw * __expf(mw - M);
      for (int x = 0; x < K; ++x)
        if (sm.sel[x] >= 0) z += __expf(sm.sl_s[w][x] - M);
      const float logZ = M + __logf(z);
      float Delta = dw * __expf(mw - logZ);
      for (int x = 0; x < K; ++x)
        if (sm.sel[x] >= 0) Delta += __expf(sm.sl_s[w][x] - logZ) * sm.sl_doo[w][x];
      if (lane == 0) {
        a.logz[ro] = logZ;
        a.delta[ro] = Delta;
      }
      for (int x = lane; x < K; x += 64) {
        if (sm.sel[x] < 0) continue;
        const int pos = a.inv_pos[(pg * T_len + i) * K + x];
        const size_t eo = (pg * T_len * K + pos) * G + hh;
        // w_c P_cj = e^{l_j + lw}: lw = s_hat - logZ - max - log(sum)
        a.ent_lw[eo] = sm.sl_s[w][x] - logZ - sm.sl_m[w][x] - __logf(sm.sl_l[w][x]);
        a.ent_doo[eo] = sm.sl_doo[w][x];
        a.ent_ds[eo] = __expf(sm.sl_s[w][x] - logZ) * (sm.sl_doo[w][x] - Delta);
      }
      const float fc = Mc == -INFINITY ? 0.f : __expf(Mc - logZ), fw = __expf(mw - logZ);
#pragma unroll
      for (int u = 0; u < EPL; ++u) {
        const float dqh = tau * fc * (B1[u] - Delta * B2[u]);
        a.dq[ro * D + lane * EPL + u] = tau * (fc * Bq[u] + fw * (A1[u] - Delta * A2[u])) + dqh;
        if (QCAL) a.dqhat[((static_cast<size_t>(b) * T_len + i) * Hq + h) * D + lane * EPL + u] = dqh;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ z
// Per (b, g, chunk c) and head: z = sum over the chunk's list entries of
// ds u_i (Q-Cal) and zb = sum ds.  Thread (part, q) sums the entries
// e = e_lo + part + P m (P = 256 / r parts, all G heads in registers); the
// parts are then added in part order.
__global__ void __launch_bounds__(kBT) bwd_z_kernel(BwdArgs a) {
  __shared__ float red[kBT][kMaxBwdG + 1];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int G = a.Hq / a.Hkv, C = a.T / kBK, K = a.K;
  const int r = a.r > 0 ? a.r : 1;  // with r = 0 the single column sums ds only
  const size_t pg = static_cast<size_t>(b) * a.Hkv + g;
  const int e_lo = a.inv_choff[pg * (C + 1) + c], e_hi = a.inv_choff[pg * (C + 1) + c + 1];
  const int32_t *list = a.inv_list + pg * static_cast<size_t>(a.T) * K;
  const float *ds = a.ent_ds + pg * static_cast<size_t>(a.T) * K * G;
  const int P = kBT / r, part = t / r, q = t % r;
  float acc[kMaxBwdG], accb[kMaxBwdG];
#pragma unroll
  for (int hh = 0; hh < kMaxBwdG; ++hh) acc[hh] = accb[hh] = 0.f;
  if (part < P) {
    for (int e = e_lo + part; e < e_hi; e += P) {
      const float uq = a.r > 0 ? a.u[(static_cast<size_t>(b) * a.T + (list[e] >> 5)) * a.r + q] : 0.f;
#pragma unroll
      for (int hh = 0; hh < kMaxBwdG; ++hh) {
        if (hh < G) {
          const float d = ds[static_cast<size_t>(e) * G + hh];
          acc[hh] += d * uq;
          accb[hh] += d;
        }
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < kMaxBwdG; ++hh) red[t][hh] = acc[hh];
  __syncthreads();
  if (a.r > 0 && t < a.r * G) {
    const int hh = t / a.r, qq = t % a.r;
    float s = 0.f;
    for (int p2 = 0; p2 < P; ++p2) s += red[p2 * r + qq][hh];
    a.zsum[((static_cast<size_t>(b) * a.Hq + g * G + hh) * C + c) * a.r + qq] = s;
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < kMaxBwdG; ++hh) red[t][hh] = accb[hh];
  __syncthreads();
  if (t < G) {  // column q = 0 of each part holds its ds sums
    float s = 0.f;
    for (int p2 = 0; p2 < P; ++p2) s += red[p2 * r][t];
    a.zb[(static_cast<size_t>(b) * a.Hq + g * G + t) * C + c] = s;
  }
}

// ------------------------------------------------------------------ keys (VALU)
template <int D>
struct KeySmem {
  float kt[kBK][D + 1];                  // the block's keys (fp32)
  float rq[kRowsPerBatch][D];            // a batch of rows: q and dO
  float rdo[kRowsPerBatch][D];
  float ra[kRowsPerBatch], rb[kRowsPerBatch], rds[kRowsPerBatch];
  int ri[kRowsPerBatch], rh[kRowsPerBatch], rwin[kRowsPerBatch];
  float dkp[kMaxBwdG][D];                // per head: tau sum ds q (the raw-q part of dk'_c)
  bwd::SummaryScratch<D> ss;
};

template <typename T, int D>
__global__ void __launch_bounds__(kBT)
bwd_keys_kernel(BwdArgs a) {
  __shared__ KeySmem<D> sm;
  const int kb = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int T_len = a.T, K = a.K, Hq = a.Hq, Hkv = a.Hkv, W = a.W, C = T_len / kBK;
  const int G = Hq / Hkv;
  const float tau = a.tau;
  constexpr int QD = D / 4;
  const int j = t >> 2, qd = t & 3;  // this thread: key j, elements [qd QD, qd QD + QD)
  const int j0 = kb * kBK, jj = j0 + j;
  const size_t pg = static_cast<size_t>(b) * Hkv + g;
  const T *kb_p = static_cast<const T *>(a.k) + pg * T_len * D;
  const T *vb_p = static_cast<const T *>(a.v) + pg * T_len * D;
  float kr[QD], vr[QD], dk[QD], dv[QD];
#pragma unroll
  for (int u = 0; u < QD; ++u) {
    const bool ok = jj < T_len;
    kr[u] = ok ? Elem<T>::load(kb_p, static_cast<size_t>(jj) * D + qd * QD + u) : 0.f;
    vr[u] = ok ? Elem<T>::load(vb_p, static_cast<size_t>(jj) * D + qd * QD + u) : 0.f;
    dk[u] = dv[u] = 0.f;
    sm.kt[j][qd * QD + u] = kr[u];
  }
  const bool full_chunk = kb < C;
  if (full_chunk)
    for (int x = t; x < G * D; x += kBT) sm.dkp[x / D][x % D] = 0.f;
  // the rows this block serves: every (i, h) whose window holds the block,
  // i in [j0, j0 + S + W - 2] with n_i S <= j0; then the chunk's entries
  const int iw_lo = j0, iw_hi = min(T_len - 1, j0 + kBK + W - 2);
  const int nwin = iw_hi >= iw_lo ? (iw_hi - iw_lo + 1) * G : 0;
  int e_lo = 0, e_n = 0;
  if (full_chunk && K > 0) {
    e_lo = a.inv_choff[pg * (C + 1) + kb];
    e_n = a.inv_choff[pg * (C + 1) + kb + 1] - e_lo;
  }
  const int nrows = nwin + e_n * G;
  const int *list = a.inv_list + pg * static_cast<size_t>(T_len) * K;
  const size_t ebase = pg * static_cast<size_t>(T_len) * K;
  for (int r0 = 0; r0 < nrows; r0 += kRowsPerBatch) {
    __syncthreads();
    // a batch of rows into LDS: row r -> (i, head) and its scalars
    if (t < kRowsPerBatch) {
      const int r = r0 + t;
      int i = 0, hh = 0, win = -1;
      if (r < nwin) {
        i = iw_lo + r / G;
        hh = r % G;
        win = (eligible_chunks(i, W, kBK) * kBK <= j0) ? 1 : -1;  // the block lies in i's window
        const size_t ro = (static_cast<size_t>(b) * Hq + g * G + hh) * T_len + i;
        if (win == 1) {
          sm.ra[t] = a.logz[ro];
          sm.rb[t] = a.delta[ro];
          sm.rds[t] = 0.f;
        }
      } else if (r < nrows) {
        const int e = e_lo + (r - nwin) / G;
        i = list[e] >> 5;
        hh = (r - nwin) % G;
        win = 0;
        const size_t eo = (ebase + e) * G + hh;
        sm.ra[t] = a.ent_lw[eo];
        sm.rb[t] = a.ent_doo[eo];
        sm.rds[t] = a.ent_ds[eo];
      }
      sm.ri[t] = i;
      sm.rh[t] = hh;
      sm.rwin[t] = win;
    }
    __syncthreads();
    for (int x = t; x < kRowsPerBatch * D; x += kBT) {
      const int r = x / D, e = x % D;
      if (sm.rwin[r] < 0) continue;
      const size_t ro = (static_cast<size_t>(b) * Hq + g * G + sm.rh[r]) * T_len + sm.ri[r];
      sm.rq[r][e] = Elem<T>::load(static_cast<const T *>(a.q), ro * D + e);
      sm.rdo[r][e] = Elem<T>::load(static_cast<const T *>(a.d_o), ro * D + e);
    }
    __syncthreads();
    for (int r = 0; r < kRowsPerBatch; ++r) {
      const int win = sm.rwin[r];
      if (win < 0) continue;  // uniform
      float l = 0.f, dov = 0.f;
#pragma unroll
      for (int u = 0; u < QD; ++u) {
        l += sm.rq[r][qd * QD + u] * kr[u];
        dov += sm.rdo[r][qd * QD + u] * vr[u];
      }
      l = tau * sum4(l);
      dov = sum4(dov);
      float cv, dl;
      if (win == 1) {  // window: u_j (dO.v_j - Delta), keys up to i
        cv = (jj <= sm.ri[r] && jj < T_len) ? __expf(l - sm.ra[r]) : 0.f;
        dl = cv * (dov - sm.rb[r]);
      } else {  // chunk entry: w_c P_cj (dO.v_j - dO.o_c)
        cv = __expf(l + sm.ra[r]);
        dl = cv * (dov - sm.rb[r]);
      }
#pragma unroll
      for (int u = 0; u < QD; ++u) {
        dv[u] += cv * sm.rdo[r][qd * QD + u];
        dk[u] += tau * dl * sm.rq[r][qd * QD + u];
      }
      // the raw-q part of the chunk's dk'_c: tau ds q (threads of key slot
      // hh keep head hh's sums)
      if (win == 0 && j == sm.rh[r]) {
#pragma unroll
        for (int u = 0; u < QD; ++u) sm.dkp[j][qd * QD + u] += tau * sm.rds[r] * sm.rq[r][qd * QD + u];
      }
    }
  }
  __syncthreads();
  if (full_chunk) bwd::summary_backward<T, D>(a, b, g, kb, sm.kt, kr, dk, sm.dkp, sm.ss);
  if (jj < T_len) {
#pragma unroll
    for (int u = 0; u < QD; ++u) {
      a.dk[(pg * T_len + jj) * D + qd * QD + u] = dk[u];
      a.dv[(pg * T_len + jj) * D + qd * QD + u] = dv[u];
    }
  }
}

// ------------------------------------------------------------------ launchers
template <typename T, int D>
static hipError_t bwd_t(const BwdArgs &a, hipStream_t st) {
  hipError_t e;
  const bool qcal = a.r > 0;
  const int ntok = a.B * a.T, HD = a.Hq * D;
  const T *h = static_cast<const T *>(a.h), *wd = static_cast<const T *>(a.w_down),
          *wu = static_cast<const T *>(a.w_up);
  if (qcal) {
    // u [ntok, r] = h [ntok, Dh] . W_down^T
    if ((e = gemm<T, T>(h, a.Dh, 1, wd, 1, a.Dh, a.u, a.r, 1, ntok, a.r, a.Dh, st, kBwdSplitDu, a.gpart)) !=
        hipSuccess)
      return e;
    // q_hat = q + u . W_up^T   (stored [B, Hq, T, D])
    if ((e = gemm<float, T, 1>(a.u, a.r, 1, wu, 1, a.r, a.qhat, 0, 0, ntok, HD, a.r, st, 1, nullptr,
                               static_cast<const T *>(a.q), a.Hq, a.T, D)) != hipSuccess)
      return e;
  }
  const int C = a.T / kBK, nqb = (a.T + kQBlk - 1) / kQBlk;
  if (a.K > 0 && C > 0) {
    bwd_inv_count_kernel<<<dim3(nqb, a.Hkv, a.B), kBT, 0, st>>>(a);
    bwd_inv_scan_kernel<<<dim3(a.Hkv, a.B), kBT, 0, st>>>(a, nqb);
    bwd_inv_fill_kernel<<<dim3(nqb, a.Hkv, a.B), kBT, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (bwd_rows_mfma_supported(a)) {
    if ((e = launch_bwd_rows_mfma(a, st)) != hipSuccess) return e;
  } else {
    const dim3 rows(a.T, a.Hkv, a.B);
    if (qcal)
      bwd_rows_kernel<T, D, true><<<rows, kBT, 0, st>>>(a);
    else
      bwd_rows_kernel<T, D, false><<<rows, kBT, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (C > 0 && a.K > 0) {
    bwd_z_kernel<<<dim3(C, a.Hkv, a.B), kBT, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (bwd_keys_mfma_supported(a)) {
    if ((e = launch_bwd_keys_mfma(a, st)) != hipSuccess) return e;
  } else {
    bwd_keys_kernel<T, D><<<dim3((a.T + kBK - 1) / kBK, a.Hkv, a.B), kBT, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (qcal) {
    // du [ntok, r] = dq_hat [ntok, Hq D] . W_up
    if ((e = gemm<float, T>(a.dqhat, HD, 1, wu, a.r, 1, a.du, a.r, 1, ntok, a.r, HD, st, kBwdSplitDu, a.gpart)) !=
        hipSuccess)
      return e;
    // dW_up [Hq D, r] = dq_hat^T . u      (long k = tokens: split)
    if ((e = gemm<float, float>(a.dqhat, 1, HD, a.u, a.r, 1, a.dw_up, a.r, 1, HD, a.r, ntok, st, kBwdSplitW,
                                a.gpart)) != hipSuccess)
      return e;
    // dW_down [r, Dh] = du^T . h
    if ((e = gemm<float, T>(a.du, 1, a.r, h, a.Dh, 1, a.dw_down, a.Dh, 1, a.r, a.Dh, ntok, st, kBwdSplitW, a.gpart)) !=
        hipSuccess)
      return e;
    // dh [ntok, Dh] = du . W_down
    if ((e = gemm<float, T>(a.du, a.r, 1, wd, a.Dh, 1, a.dh, a.Dh, 1, ntok, a.Dh, a.r, st)) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_backward(const BwdArgs &a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? bwd_t<uint16_t, 128>(a, st) : bwd_t<uint16_t, 64>(a, st);
  return a.d == 128 ? bwd_t<float, 128>(a, st) : bwd_t<float, 64>(a, st);
}

}  // namespace hils
