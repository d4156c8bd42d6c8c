// Backward pass of the HiLS-Attention prefill forward, for a fixed top-K
// selection (VALU kernels, fp32 accumulation).
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
//
// Kernels (all on the caller's stream):
//   [qcal]  u = W_down h, q_hat = q + W_up u                          (r > 0)
//   rows    one workgroup per (i, g, b), one wave per head (4 at a time):
//           two passes over the row's selected chunks and window blocks
//           (staged in LDS): the first gives logZ, Delta and per chunk its
//           log-weight and dO.o_c; the second the dl_j and dq.  Writes dq,
//           the per-row and per-slot values the key pass needs, and dq_hat.
//   lists   the inverse of the selection: for every (b, g, chunk) the
//           (query, slot) entries that selected it, ordered by query
//           (counted per 256-query block, no atomics on the order).
//   keys    one workgroup per 64-key block (b, g): every row whose window
//           covers the block, then (complete chunks) every entry of the
//           chunk's list with its G heads; thread (key, quarter of d) keeps
//           dk, dv in registers.  Then the chunk's summary backward.
//   [qcal]  du, dh, dW_down, dW_up.
// Every sum runs in a fixed order: the results are the same on every run.
#include "hils_common.h"
#include "launch.h"

namespace hils {

namespace {

constexpr int kBT = 256;     // threads per workgroup
constexpr int kBK = 64;      // keys per block (= chunk size S)
constexpr int kQBlk = 256;   // queries per block of the inverse-list build
constexpr int kRowsPerBatch = 8;

// Reduce over the 4 consecutive lanes 4m .. 4m+3.
__device__ __forceinline__ float sum4(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  return v;
}

// One row of a staged key / value tile, stored with one spare pair of
// elements per row so that lane j reading row j hits bank j + const.
template <typename T, int D>
struct Tile {
  static constexpr int kLD = D + (sizeof(T) == 2 ? 2 : 1);
  T x[kBK * kLD];
  __device__ __forceinline__ float at(int j, int e) const { return to_f(x[j * kLD + e]); }
  __device__ __forceinline__ static float to_f(float v) { return v; }
  __device__ __forceinline__ static float to_f(uint16_t v) { return bf16_to_f32(v); }
};

// Rows j0 .. j0 + 63 of a [T, D] matrix into a tile (rows past T are zero).
template <typename T, int D>
__device__ __forceinline__ void stage_tile(Tile<T, D> &tl, const T *src, int j0, int T_len) {
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte piece
  for (int p = threadIdx.x; p < kBK * D / EPV; p += kBT) {
    const int r = p / (D / EPV), s = p % (D / EPV);
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (j0 + r < T_len) u = *reinterpret_cast<const uint4 *>(src + static_cast<size_t>(j0 + r) * D + s * EPV);
    const T *e = reinterpret_cast<const T *>(&u);
#pragma unroll
    for (int x = 0; x < EPV; ++x) tl.x[r * Tile<T, D>::kLD + s * EPV + x] = e[x];
  }
}

}  // namespace

// ------------------------------------------------------------------ Q-Cal
// q_hat [B, Hq, T, D] fp32 = q + (W_up u)[h D + e], u [B*T, r] fp32.
template <typename T>
__global__ void __launch_bounds__(kBT)
bwd_qhat_kernel(const T *__restrict__ q, const T *__restrict__ w_up, const float *__restrict__ u,
                float *__restrict__ qhat, int Hq, int T_len, int D, int r, size_t total) {
  for (size_t x = blockIdx.x * static_cast<size_t>(kBT) + threadIdx.x; x < total;
       x += static_cast<size_t>(gridDim.x) * kBT) {
    const int e = static_cast<int>(x % D);
    const size_t row = x / D;  // (b, h, i)
    const int i = static_cast<int>(row % T_len), h = static_cast<int>((row / T_len) % Hq);
    const int b = static_cast<int>(row / (static_cast<size_t>(T_len) * Hq));
    const float *ur = u + (static_cast<size_t>(b) * T_len + i) * r;
    const T *wr = w_up + (static_cast<size_t>(h) * D + e) * r;
    float acc = 0.f;
    for (int a = 0; a < r; ++a) acc += Elem<T>::load(wr, a) * ur[a];
    qhat[x] = Elem<T>::load(q, x) + acc;
  }
}

// ------------------------------------------------------------------ rows
template <typename T, int D>
struct RowSmem {
  Tile<T, D> kt, vt;
  float qs[4][D], qhs[4][D], dos[4][D];
  float dls[4][kBK];                  // dl_j of the current block, per head
  float sl_m[4][32], sl_l[4][32];     // per selected chunk: max and sum of e^{l - max}
  float sl_doo[4][32], sl_s[4][32];   // dO.o_c and s_hat
  int sel[32];                        // the row's chunks (list order; -1: none)
};

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
  const T *kb = static_cast<const T *>(a.k) + (static_cast<size_t>(b) * Hkv + g) * T_len * D;
  const T *vb = static_cast<const T *>(a.v) + (static_cast<size_t>(b) * Hkv + g) * T_len * D;
  const T *ksum = static_cast<const T *>(a.k_sum);
  // the row's selection (an id outside [0, n_i) is no chunk)
  if (t < 32) {
    int c = -1;
    if (t < K) c = a.topk_idx[((static_cast<size_t>(b) * Hkv + g) * T_len + i) * K + t];
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
    // ---- pass 1: logZ, Delta; per chunk its statistics and dO.o_c
    float mw = -INFINITY, lw = 0.f, dw = 0.f;  // window: max, sum e^{l - mw}, sum e^{l - mw} dO.v
    for (int x = 0; x < K + nwb; ++x) {
      const bool chunk = x < K;
      if (chunk && sm.sel[x] < 0) continue;  // uniform across the workgroup
      const int j0 = chunk ? sm.sel[x] * kBK : w_lo + (x - K) * kBK;
      __syncthreads();  // the previous block's tiles are no longer read
      stage_tile<T, D>(sm.kt, kb, j0, T_len);
      stage_tile<T, D>(sm.vt, vb, j0, T_len);
      __syncthreads();
      if (act) {
        float l = 0.f, dov = 0.f;
        for (int e = 0; e < D; ++e) {
          l += sm.qs[w][e] * sm.kt.at(lane, e);
          dov += sm.dos[w][e] * sm.vt.at(lane, e);
        }
        l *= tau;
        if (chunk) {
          const float m = wave_max(l);
          const float p = __expf(l - m);
          const float lsum = wave_sum(p);
          const float doo = wave_sum(p * dov) / lsum;
          // s_hat = tau q_hat . k'_c + b'_c from the stored summary
          const int c = sm.sel[x];
          const size_t so = (static_cast<size_t>(b) * Hq + h) * C + c;
          float sp = 0.f;
#pragma unroll
          for (int u = 0; u < EPL; ++u) sp += sm.qhs[w][lane * EPL + u] * Elem<T>::load(ksum, so * D + lane * EPL + u);
          sp = wave_sum(sp);
          if (lane == 0) {
            sm.sl_m[w][x] = m;
            sm.sl_l[w][x] = lsum;
            sm.sl_doo[w][x] = doo;
            sm.sl_s[w][x] = tau * sp + a.b_sum[so];
          }
        } else {
          const int jj = j0 + lane;
          const float lm = jj <= i ? l : -INFINITY;
          const float mb = wave_max(lm);
          const float mn = fmaxf(mw, mb);
          const float e = jj <= i ? __expf(lm - mn) : 0.f;
          const float sc = mw == -INFINITY ? 0.f : __expf(mw - mn);
          lw = lw * sc + wave_sum(e);
          dw = dw * sc + wave_sum(e * dov);
          mw = mn;
        }
      }
    }
    __syncthreads();
    // ---- the joint normaliser, Delta, and the per-slot values
    float logZ = 0.f, Delta = 0.f;
    if (act) {
      float M = mw;
      for (int x = 0; x < K; ++x)
        if (sm.sel[x] >= 0) M = fmaxf(M, sm.sl_s[w][x]);
      float z = lw * __expf(mw - M);
      for (int x = 0; x < K; ++x)
        if (sm.sel[x] >= 0) z += __expf(sm.sl_s[w][x] - M);
      logZ = M + __logf(z);
      Delta = dw * __expf(mw - logZ);
      for (int x = 0; x < K; ++x)
        if (sm.sel[x] >= 0) Delta += __expf(sm.sl_s[w][x] - logZ) * sm.sl_doo[w][x];
      if (lane == 0) {
        a.logz[ro] = logZ;
        a.delta[ro] = Delta;
      }
      for (int x = lane; x < K; x += 64) {
        const bool ok = sm.sel[x] >= 0;
        const float wc = ok ? __expf(sm.sl_s[w][x] - logZ) : 0.f;
        // w_c P_cj = e^{l_j + lwt}: lwt = s_hat - logZ - max - log(sum)
        a.slot_lw[ro * K + x] = ok ? sm.sl_s[w][x] - logZ - sm.sl_m[w][x] - __logf(sm.sl_l[w][x]) : -INFINITY;
        a.slot_doo[ro * K + x] = ok ? sm.sl_doo[w][x] : 0.f;
        a.slot_ds[ro * K + x] = ok ? wc * (sm.sl_doo[w][x] - Delta) : 0.f;
      }
    }
    // ---- pass 2: dl_j of every block, dq
    float dq[EPL], dqh[EPL];
#pragma unroll
    for (int u = 0; u < EPL; ++u) dq[u] = dqh[u] = 0.f;
    for (int x = 0; x < K + nwb; ++x) {
      const bool chunk = x < K;
      if (chunk && sm.sel[x] < 0) continue;
      const int j0 = chunk ? sm.sel[x] * kBK : w_lo + (x - K) * kBK;
      __syncthreads();
      stage_tile<T, D>(sm.kt, kb, j0, T_len);
      stage_tile<T, D>(sm.vt, vb, j0, T_len);
      __syncthreads();
      if (act) {
        float l = 0.f, dov = 0.f;
        for (int e = 0; e < D; ++e) {
          l += sm.qs[w][e] * sm.kt.at(lane, e);
          dov += sm.dos[w][e] * sm.vt.at(lane, e);
        }
        l *= tau;
        float dl;
        if (chunk) {
          const float wc = __expf(sm.sl_s[w][x] - logZ);
          const float pw = wc * __expf(l - sm.sl_m[w][x]) / sm.sl_l[w][x];  // w_c P_cj
          dl = pw * (dov - sm.sl_doo[w][x]);
          // dq_hat += tau ds_c k'_c
          const int c = sm.sel[x];
          const size_t so = (static_cast<size_t>(b) * Hq + h) * C + c;
          const float ds = wc * (sm.sl_doo[w][x] - Delta);
#pragma unroll
          for (int u = 0; u < EPL; ++u) dqh[u] += tau * ds * Elem<T>::load(ksum, so * D + lane * EPL + u);
        } else {
          const int jj = j0 + lane;
          dl = jj <= i ? __expf(l - logZ) * (dov - Delta) : 0.f;
        }
        sm.dls[w][lane] = dl;
      }
      __syncthreads();
      if (act) {
        for (int j = 0; j < kBK; ++j) {
          const float dlj = sm.dls[w][j];
#pragma unroll
          for (int u = 0; u < EPL; ++u) dq[u] += dlj * sm.kt.at(j, lane * EPL + u);
        }
      }
    }
    if (act) {
#pragma unroll
      for (int u = 0; u < EPL; ++u) {
        a.dq[ro * D + lane * EPL + u] = tau * dq[u] + dqh[u];
        if (QCAL) a.dqhat[ro * D + lane * EPL + u] = dqh[u];
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ inverse lists
// For each (b, g) and chunk c, the entries (i, slot) with topk_idx[b,g,i,slot]
// == c (and c < n_i), ordered by i.  cnt [B, Hkv, nqb, C]: entries per
// 256-query block; qboff: their offset inside the chunk's list; choff
// [B, Hkv, C + 1]: each chunk's first entry; list [B, Hkv, T K]: i * 32 + slot.
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
  for (int k = 0; k < a.K; ++k) {
    const int c = ir[k];
    if (c < 0 || c >= n) continue;
    int rank = 0;
    for (int x = 0; x < (t >> 5); ++x) rank += __popc(sm.mask[c][x]);
    rank += __popc(sm.mask[c][t >> 5] & ((1u << (t & 31)) - 1u));
    const int pos = a.inv_choff[pg * (C + 1) + c] + a.inv_qboff[(pg * nqb + qb) * C + c] + rank;
    a.inv_list[pg * static_cast<size_t>(a.T) * a.K + pos] = i * 32 + k;
  }
}

// ------------------------------------------------------------------ keys
template <typename T, int D>
struct KeySmem {
  float kt[kBK][D + 1];                  // the block's keys (fp32)
  float rq[kRowsPerBatch][D];            // a batch of rows: q, dO, and q_hat (summary)
  float rdo[kRowsPerBatch][D];
  float rqh[kRowsPerBatch][D];
  float ra[kRowsPerBatch], rb[kRowsPerBatch], rds[kRowsPerBatch];
  int ri[kRowsPerBatch], rh[kRowsPerBatch], rwin[kRowsPerBatch];
  float red[4][kMaxBwdG];                   // cross-wave reductions
  float dkp[kMaxBwdG][D], dbp[kMaxBwdG];       // per head: dk'_c and db'_c of the chunk
  float qlm[D], kp[D], pl[kBK], dlj[kBK];
  float stat[4];
};

template <typename T, int D, bool QCAL>
__global__ void __launch_bounds__(kBT)
bwd_keys_kernel(BwdArgs a) {
  __shared__ KeySmem<T, D> sm;
  const int kb = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
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
  if (t < kMaxBwdG) sm.dbp[t] = 0.f;
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
  for (int r0 = 0; r0 < nrows; r0 += kRowsPerBatch) {
    __syncthreads();
    // a batch of rows into LDS: row r -> (i, head) and its scalars
    if (t < kRowsPerBatch) {
      const int r = r0 + t;
      int i = 0, hh = 0, win = -1, slot = 0;
      if (r < nwin) {
        i = iw_lo + r / G;
        hh = r % G;
        win = (eligible_chunks(i, W, kBK) * kBK <= j0) ? 1 : -1;  // the block lies in i's window
      } else if (r < nrows) {
        const int en = list[e_lo + (r - nwin) / G];
        i = en >> 5;
        slot = en & 31;
        hh = (r - nwin) % G;
        win = 0;
      }
      const size_t ro = (static_cast<size_t>(b) * Hq + g * G + hh) * T_len + i;
      sm.ri[t] = i;
      sm.rh[t] = hh;
      sm.rwin[t] = win;
      if (win == 1) {
        sm.ra[t] = a.logz[ro];
        sm.rb[t] = a.delta[ro];
        sm.rds[t] = 0.f;
      } else if (win == 0) {
        sm.ra[t] = a.slot_lw[ro * K + slot];
        sm.rb[t] = a.slot_doo[ro * K + slot];
        sm.rds[t] = a.slot_ds[ro * K + slot];
      }
    }
    __syncthreads();
    for (int x = t; x < kRowsPerBatch * D; x += kBT) {
      const int r = x / D, e = x % D;
      if (sm.rwin[r] < 0) continue;
      const size_t ro = (static_cast<size_t>(b) * Hq + g * G + sm.rh[r]) * T_len + sm.ri[r];
      sm.rq[r][e] = Elem<T>::load(static_cast<const T *>(a.q), ro * D + e);
      sm.rdo[r][e] = Elem<T>::load(static_cast<const T *>(a.d_o), ro * D + e);
      if (sm.rwin[r] == 0) sm.rqh[r][e] = QCAL ? a.qhat[ro * D + e] : sm.rq[r][e];
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
      // the chunk's summary gradients: dk'_c += tau ds q_hat, db'_c += ds
      // (threads of key slot hh keep head hh's sums)
      if (win == 0 && j == sm.rh[r]) {
#pragma unroll
        for (int u = 0; u < QD; ++u) sm.dkp[j][qd * QD + u] += tau * sm.rds[r] * sm.rqh[r][qd * QD + u];
        if (qd == 0) sm.dbp[j] += sm.rds[r];
      }
    }
  }
  __syncthreads();
  // ---- the chunk summary (Eq. 8) of each head of the group
  if (full_chunk) {
    for (int hh = 0; hh < G; ++hh) {
      const int h = g * G + hh;
      const size_t so = (static_cast<size_t>(b) * Hq + h) * C + kb;
      for (int x = t; x < D; x += kBT) sm.qlm[x] = Elem<T>::load(static_cast<const T *>(a.q_lm), so * D + x);
      __syncthreads();
      float l = 0.f;
#pragma unroll
      for (int u = 0; u < QD; ++u) l += sm.qlm[qd * QD + u] * kr[u];
      l = tau * sum4(l);
      // softmax over the 64 keys (4 lanes per key): block maximum and sum
      float m = wave_max(l);
      if (lane == 0) sm.red[wv][0] = m;
      __syncthreads();
      m = fmaxf(fmaxf(sm.red[0][0], sm.red[1][0]), fmaxf(sm.red[2][0], sm.red[3][0]));
      __syncthreads();
      const float ex = __expf(l - m);
      float s = wave_sum(ex) * 0.25f;  // each key counted by its 4 lanes
      float sl = wave_sum(ex * l) * 0.25f;
      if (lane == 0) {
        sm.red[wv][0] = s;
        sm.red[wv][1] = sl;
      }
      __syncthreads();
      const float z = sm.red[0][0] + sm.red[1][0] + sm.red[2][0] + sm.red[3][0];
      const float El = (sm.red[0][1] + sm.red[1][1] + sm.red[2][1] + sm.red[3][1]) / z;
      const float p = ex / z;
      if (qd == 0) sm.pl[j] = p;
      __syncthreads();
      // k' (unrounded) = sum_j p_j k_j, a fixed key order per element
      for (int e = t; e < D; e += kBT) {
        float acc = 0.f;
        for (int jk = 0; jk < kBK; ++jk) acc += sm.pl[jk] * sm.kt[jk][e];
        sm.kp[e] = acc;
      }
      __syncthreads();
      float proj = 0.f;
#pragma unroll
      for (int u = 0; u < QD; ++u) proj += sm.dkp[hh][qd * QD + u] * (kr[u] - sm.kp[qd * QD + u]);
      proj = sum4(proj);
      const float dl = p * (proj - sm.dbp[hh] * (l - El));
#pragma unroll
      for (int u = 0; u < QD; ++u) dk[u] += p * sm.dkp[hh][qd * QD + u] + tau * dl * sm.qlm[qd * QD + u];
      if (qd == 0) sm.dlj[j] = dl;
      __syncthreads();
      for (int e = t; e < D; e += kBT) {
        float acc = 0.f;
        for (int jk = 0; jk < kBK; ++jk) acc += sm.dlj[jk] * sm.kt[jk][e];
        a.dq_lm[so * D + e] = tau * acc;
      }
      __syncthreads();
    }
  }
  if (jj < T_len) {
#pragma unroll
    for (int u = 0; u < QD; ++u) {
      a.dk[(pg * T_len + jj) * D + qd * QD + u] = dk[u];
      a.dv[(pg * T_len + jj) * D + qd * QD + u] = dv[u];
    }
  }
}

// ------------------------------------------------------------------ Q-Cal weights
// du [B*T, r] = sum over heads of W_up[h D + e, :]^T dq_hat[b, h, i, e]:
// one workgroup per token, each thread a slice of the H_q D rows with all r
// sums in registers, then a fixed-order reduction over the threads.
template <typename T>
__global__ void __launch_bounds__(kBT)
bwd_du_kernel(const T *__restrict__ w_up, const float *__restrict__ dqhat, float *__restrict__ du, int Hq, int T_len,
              int D, int r) {
  __shared__ float part[kBT / 64][64];
  const int tok = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int b = tok / T_len, i = tok % T_len;
  float acc[64];
#pragma unroll
  for (int a = 0; a < 64; ++a) acc[a] = 0.f;
  for (int x = t; x < Hq * D; x += kBT) {
    const int h = x / D, e = x % D;
    const float g = dqhat[((static_cast<size_t>(b) * Hq + h) * T_len + i) * D + e];
    const T *wr = w_up + static_cast<size_t>(x) * r;
#pragma unroll
    for (int a = 0; a < 64; ++a)
      if (a < r) acc[a] += Elem<T>::load(wr, a) * g;
  }
#pragma unroll
  for (int a = 0; a < 64; ++a) {
    if (a < r) {
      const float v = wave_sum(acc[a]);
      if (lane == 0) part[wv][a] = v;
    }
  }
  __syncthreads();
  if (t < r) du[static_cast<size_t>(tok) * r + t] = part[0][t] + part[1][t] + part[2][t] + part[3][t];
}

// dW_up [Hq D, r]: entry (h D + e, a) = sum over tokens of dq_hat[b, h, i, e] u[b, i, a]
__global__ void __launch_bounds__(kBT)
bwd_dwup_kernel(const float *__restrict__ dqhat, const float *__restrict__ u, float *__restrict__ dwu, int B, int Hq,
                int T_len, int D, int r) {
  const int row = blockIdx.x * kBT + threadIdx.x, a = blockIdx.y;
  if (row >= Hq * D) return;
  const int h = row / D, e = row % D;
  float acc = 0.f;
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < T_len; ++i)
      acc += dqhat[((static_cast<size_t>(b) * Hq + h) * T_len + i) * D + e] * u[(static_cast<size_t>(b) * T_len + i) * r + a];
  dwu[static_cast<size_t>(row) * r + a] = acc;
}

// dW_down [r, Dh] = sum over tokens of du h;  dh [B*T, Dh] = du W_down
template <typename T>
__global__ void __launch_bounds__(kBT)
bwd_dwdown_kernel(const float *__restrict__ du, const T *__restrict__ hin, float *__restrict__ dwd, int ntok, int r,
                  int Dh) {
  const int f = blockIdx.x * kBT + threadIdx.x, a = blockIdx.y;
  if (f >= Dh) return;
  float acc = 0.f;
  for (int tok = 0; tok < ntok; ++tok) acc += du[static_cast<size_t>(tok) * r + a] * Elem<T>::load(hin, static_cast<size_t>(tok) * Dh + f);
  dwd[static_cast<size_t>(a) * Dh + f] = acc;
}

template <typename T>
__global__ void __launch_bounds__(kBT)
bwd_dh_kernel(const float *__restrict__ du, const T *__restrict__ w_down, float *__restrict__ dh, int ntok, int r,
              int Dh) {
  const size_t x = blockIdx.x * static_cast<size_t>(kBT) + threadIdx.x;
  if (x >= static_cast<size_t>(ntok) * Dh) return;
  const size_t tok = x / Dh;
  const int f = static_cast<int>(x % Dh);
  float acc = 0.f;
  for (int a = 0; a < r; ++a) acc += du[tok * r + a] * Elem<T>::load(w_down, static_cast<size_t>(a) * Dh + f);
  dh[x] = acc;
}

// ------------------------------------------------------------------ launchers
template <typename T, int D>
static hipError_t bwd_t(const BwdArgs &a, hipStream_t st) {
  hipError_t e;
  const bool qcal = a.r > 0;
  if (qcal) {
    e = launch_qcal_down(a.h, a.w_down, a.u, a.B * a.T, a.r, a.Dh, a.bf16, st);
    if (e != hipSuccess) return e;
    const size_t total = static_cast<size_t>(a.B) * a.Hq * a.T * D;
    bwd_qhat_kernel<T><<<static_cast<unsigned>((total + kBT - 1) / kBT < 65535 ? (total + kBT - 1) / kBT : 65535), kBT,
                         0, st>>>(static_cast<const T *>(a.q), static_cast<const T *>(a.w_up), a.u, a.qhat, a.Hq,
                                  a.T, D, a.r, total);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 rows(a.T, a.Hkv, a.B);
  if (qcal)
    bwd_rows_kernel<T, D, true><<<rows, kBT, 0, st>>>(a);
  else
    bwd_rows_kernel<T, D, false><<<rows, kBT, 0, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int C = a.T / kBK, nqb = (a.T + kQBlk - 1) / kQBlk;
  if (a.K > 0 && C > 0) {
    bwd_inv_count_kernel<<<dim3(nqb, a.Hkv, a.B), kBT, 0, st>>>(a);
    bwd_inv_scan_kernel<<<dim3(a.Hkv, a.B), kBT, 0, st>>>(a, nqb);
    bwd_inv_fill_kernel<<<dim3(nqb, a.Hkv, a.B), kBT, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 keys((a.T + kBK - 1) / kBK, a.Hkv, a.B);
  if (qcal)
    bwd_keys_kernel<T, D, true><<<keys, kBT, 0, st>>>(a);
  else
    bwd_keys_kernel<T, D, false><<<keys, kBT, 0, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (qcal) {
    const int ntok = a.B * a.T;
    bwd_du_kernel<T><<<ntok, kBT, 0, st>>>(static_cast<const T *>(a.w_up), a.dqhat, a.du, a.Hq, a.T, D, a.r);
    bwd_dwup_kernel<<<dim3((a.Hq * D + kBT - 1) / kBT, a.r), kBT, 0, st>>>(a.dqhat, a.u, a.dw_up, a.B, a.Hq, a.T, D, a.r);
    bwd_dwdown_kernel<T><<<dim3((a.Dh + kBT - 1) / kBT, a.r), kBT, 0, st>>>(a.du, static_cast<const T *>(a.h),
                                                                           a.dw_down, ntok, a.r, a.Dh);
    const size_t nh = static_cast<size_t>(ntok) * a.Dh;
    bwd_dh_kernel<T><<<static_cast<unsigned>((nh + kBT - 1) / kBT), kBT, 0, st>>>(
        a.du, static_cast<const T *>(a.w_down), a.dh, ntok, a.r, a.Dh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_backward(const BwdArgs &a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? bwd_t<uint16_t, 128>(a, st) : bwd_t<uint16_t, 64>(a, st);
  return a.d == 128 ? bwd_t<float, 128>(a, st) : bwd_t<float, 64>(a, st);
}

}  // namespace hils
