// Decode step of HiLS-Attention for one query per sequence (position
// seq_len-1), plus the dense causal-attention comparator.
//
// Method (picx.dev summary, Methodology 1-3, Eq. 7, Eq. 10; rcap.io
// pseudo-code): score every eligible chunk from its stored summary
// (s = tau q-hat.k' + b'), keep the top-K per GQA group by the max over the
// group's heads, attend inside each kept chunk and fuse with the sliding
// window under one normaliser.
//
// Launch structure (all on the caller's stream, no host round trip):
//   [qcal]  q-hat = q + W_up W_down h                      (only when r > 0)
//   D1      grid (P score slices + NW window units, H_kv, B)
//           score slice: stream CPB chunks' k'/b' of the G heads (the
//           dominant HBM stream), local top-K -> candidates in the
//           workspace; the last slice block of (b, g) to finish (atomic
//           ticket) merges all candidates into the final top-K.
//           window unit: 64 window keys -> online-softmax partial.
//   D2      grid (K chunk slots, H_kv, B): attend one selected chunk -> its
//           (s_hat, 1, o_c) partial; the last block of (b, g) combines the
//           chunk and window partials in a fixed order (deterministic).
#include "attn_unit.h"
#include "hils_common.h"
#include "launch.h"

namespace hils {

constexpr int kDecThreads = 256;
constexpr int kMaxCand = 4096;  // P * K candidates merged by one block

__device__ __forceinline__ int clamp_seq(const int32_t *seq_lens, int b, int Tmax, unsigned *err, bool count) {
  int s = seq_lens[b];
  if (s < 1 || s > Tmax) {
    if (count) atomicAdd(err, 1u);
    s = s < 1 ? 1 : Tmax;
  }
  return s;
}

// ------------------------------------------------------------------ Q-Cal (decode)
template <typename T, int D>
__global__ void __launch_bounds__(kDecThreads)
decode_qcal_kernel(const T *__restrict__ q, const T *__restrict__ h, const T *__restrict__ w_down,
                   const T *__restrict__ w_up, float *__restrict__ qhat, int Hq, int r, int Dh) {
  __shared__ float u[64];
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int a = wave; a < r; a += kDecThreads / 64) {
    float acc = 0.f;
    for (int e = lane; e < Dh; e += 64)
      acc += Elem<T>::load(w_down, static_cast<size_t>(a) * Dh + e) * Elem<T>::load(h, static_cast<size_t>(b) * Dh + e);
    acc = wave_sum(acc);
    if (lane == 0) u[a] = acc;
  }
  __syncthreads();
  for (int x = t; x < Hq * D; x += kDecThreads) {
    float acc = 0.f;
    for (int a = 0; a < r; ++a) acc += Elem<T>::load(w_up, static_cast<size_t>(x) * r + a) * u[a];
    qhat[static_cast<size_t>(b) * Hq * D + x] = Elem<T>::load(q, static_cast<size_t>(b) * Hq * D + x) + acc;
  }
}

// ------------------------------------------------------------------ D1
constexpr int kRowsMax = 4096;  // CPB * G rows of one score slice
struct D1Smem {
  union {
    struct {
      float qh[kMaxG * 128];
      float s[kRowsMax];  // per (chunk, head) score of the slice
      float sig[1024];
    } sc;
  };
  unsigned long long wkey[4][64];  // per-wave ranking scratch of wave_select
  uint32_t w_ord[4][64];
  int w_idx[4][64];
  int w_pos[4][64];
  int is_last;
};

// a score-slice block and a window-unit block never need both layouts
template <typename T, int D>
union D1Shared {
  D1Smem sc;
  UnitSmem<T, D> us;
};

// Per-slice top-K: wave 0 selects among the slice's chunks (NJ per lane).
template <int NJ>
__device__ __forceinline__ void slice_select(const DecodeArgs &a, D1Smem &sm, int nch, int c0, int G, size_t cbase) {
  const int lane = threadIdx.x & 63, K = a.K;
  uint32_t ord[NJ];
  int idx[NJ], rank[NJ];
  bool win[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int cl = lane + 64 * j;
    ord[j] = cl < nch ? orderable(sm.sc.sig[cl]) : 0u;
    idx[j] = c0 + cl;
  }
  wave_select<NJ>(ord, idx, K, win, rank, sm.wkey[0]);
  int nwin = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) nwin += __popcll(__ballot(win[j]));
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (win[j]) {
      const int cl = lane + 64 * j;
      publish(a.cand_key + cbase + rank[j], make_key(sm.sc.sig[cl], idx[j]));
      for (int hh = 0; hh < G; ++hh) publish(a.cand_s + (cbase + rank[j]) * G + hh, sm.sc.s[cl * G + hh]);
    }
  }
  for (int k = nwin + lane; k < K; k += 64) publish(a.cand_key + cbase + k, kNoKey);
}

// Merge of the P*K candidates of (b, g): each wave keeps its top-K, wave 0
// picks the final top-K from the waves' winners.
template <int NJ>
__device__ __forceinline__ void merge_select(const DecodeArgs &a, D1Smem &sm, int b, int g, int n) {
  // NJ candidates per lane: P * K <= 4 waves * 64 lanes * NJ
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, t = threadIdx.x;
  const int K = a.K, G = a.Hq / a.Hkv;
  const int total = a.P * K;
  const size_t cb0 = (static_cast<size_t>(b) * a.Hkv + g) * a.P * K;
  uint32_t ord[NJ];
  int idx[NJ], rank[NJ];
  bool win[NJ];
  unsigned long long key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int x = wave * 64 * NJ + j * 64 + lane;
    key[j] = x < total ? load_acquired(a.cand_key + cb0 + x) : kNoKey;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    ord[j] = static_cast<uint32_t>(key[j] >> 32);
    idx[j] = key[j] == kNoKey ? 0x7FFFFFFF : key_chunk(key[j]);
  }
  wave_select<NJ>(ord, idx, K, win, rank, sm.wkey[wave]);
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (win[j]) {
      sm.w_ord[wave][rank[j]] = ord[j];
      sm.w_idx[wave][rank[j]] = idx[j];
      sm.w_pos[wave][rank[j]] = wave * 64 * NJ + j * 64 + lane;
    }
  int nw = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) nw += __popcll(__ballot(win[j]));
  for (int k = nw + lane; k < 64; k += 64) sm.w_ord[wave][k] = 0u;
  __syncthreads();
  if (wave == 0) {
    uint32_t o2[2];
    int i2[2], p2[2], r2[2];
    bool w2[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int x = j * 64 + lane;  // x = wave * K + k
      const int ww = x / max(K, 1), kk = x % max(K, 1);
      const bool ok = K > 0 && ww < 4;
      o2[j] = ok ? sm.w_ord[ww][kk] : 0u;
      i2[j] = ok ? sm.w_idx[ww][kk] : 0x7FFFFFFF;
      p2[j] = ok ? sm.w_pos[ww][kk] : 0;
    }
    wave_select<2>(o2, i2, K, w2, r2, sm.wkey[0]);
    int nwin = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) nwin += __popcll(__ballot(w2[j]));
    const int keep = min(K, n);
    (void)keep;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (w2[j]) {
        // the winner's per-head scores: every load issued before any store
        float hs[kMaxG];
#pragma unroll
        for (int hh = 0; hh < kMaxG; ++hh)
          if (hh < G) hs[hh] = load_acquired(a.cand_s + (cb0 + p2[j]) * G + hh);
        a.topk_idx[(static_cast<size_t>(b) * a.Hkv + g) * K + r2[j]] = i2[j];
#pragma unroll
        for (int hh = 0; hh < kMaxG; ++hh)
          if (hh < G) a.topk_score[(static_cast<size_t>(b) * a.Hq + g * G + hh) * K + r2[j]] = hs[hh];
      }
    for (int k = nwin + lane; k < K; k += 64) {
      a.topk_idx[(static_cast<size_t>(b) * a.Hkv + g) * K + k] = -1;
      for (int hh = 0; hh < G; ++hh) a.topk_score[(static_cast<size_t>(b) * a.Hq + g * G + hh) * K + k] = -INFINITY;
    }
  }
  (void)t;
}

template <typename T, int D, bool QCAL, int SNJ, int MNJ>
__global__ void __launch_bounds__(kDecThreads)
decode_score_kernel(DecodeArgs a) {
  __shared__ D1Shared<T, D> shm;
  D1Smem &sm = shm.sc;
  UnitSmem<T, D> &us = shm.us;
  const int g = blockIdx.y, b = blockIdx.z, blk = blockIdx.x, t = threadIdx.x;
  const int G = a.Hq / a.Hkv, K = a.K;
  const int seq = clamp_seq(a.seq_lens, b, a.Tmax, a.err, blk == 0 && g == 0 && t == 0);
  const int i = seq - 1;
  const int n = eligible_chunks(i, a.W, a.S);
  const T *kc = static_cast<const T *>(a.k_cache) + (static_cast<size_t>(b) * a.Hkv + g) * a.Tmax * D;
  const T *vc = static_cast<const T *>(a.v_cache) + (static_cast<size_t>(b) * a.Hkv + g) * a.Tmax * D;

  if (blk >= a.P) {  // ---------------- window unit
    const int u = blk - a.P;
    const int j0 = n * a.S + u * kUnitKeys;
    float *rec = a.parts + ((static_cast<size_t>(b) * a.Hkv + g) * a.nslots + K + u) * G * (D + 2);
    if (j0 > i) {
      for (int hh = t; hh < G; hh += kDecThreads) { publish(rec + hh * (D + 2), -INFINITY); publish(rec + hh * (D + 2) + 1, 0.f); }
      return;
    }
    const int nk = min(kUnitKeys, i - j0 + 1);
    load_q_rows<T, D>(us, static_cast<const T *>(a.q) + (static_cast<size_t>(b) * a.Hq + g * G) * D, D, G);
    __syncthreads();
    constexpr int NP = pairs_per_thread<D>();
    float2 ou[NP];
    attend_unit<T, D>(us, kc + static_cast<size_t>(j0) * D, vc + static_cast<size_t>(j0) * D, nk, G, a.tau, ou);
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int pr = t + r * kUnitThreads, hh = pr / (D / 2), e2 = pr % (D / 2);
      if (hh < G) {
        float *rh = rec + hh * (D + 2);
        publish(rh + 2 + 2 * e2, ou[r].x);
        publish(rh + 3 + 2 * e2, ou[r].y);
        if (e2 == 0) { publish(rh, us.m[hh]); publish(rh + 1, us.l[hh]); }
      }
    }
    return;
  }

  // ---------------- score slice: chunks [c0, c0 + nch) of the G heads
  const int c0 = blk * a.CPB;
  const int nch = max(0, min(c0 + a.CPB, n) - c0);
  constexpr int LPH = D / 8;                         // lanes per (chunk, head) row, 8 elements each
  constexpr int RPP = static_cast<int>(sizeof(T)) / 2;  // 16-byte loads per 8-element piece
  constexpr int U = 8 / RPP;                         // pieces in flight per thread
  constexpr int RS = U * kDecThreads / LPH;          // rows per batch
  const int nrows = nch * G;
  const T *ks = static_cast<const T *>(a.k_sum);
  const size_t hbase = static_cast<size_t>(b) * a.Hq + g * G;
  for (int x = t; x < G * D; x += kDecThreads) {
    const size_t qo = hbase * D + x;
    sm.sc.qh[x] = QCAL ? a.qhat[qo] : Elem<T>::load(static_cast<const T *>(a.q), qo);
  }
  // Batches of RS rows, double buffered in registers: the loads of batch
  // n + 1 are in flight while batch n is reduced.
  // Branch-free: rows past the slice read its row 0 again (their dots are
  // never stored; chunk c0 exists even when the slice is empty), and every
  // lane of a row reads the row's b'.  A load under a
  // lane-dependent branch would make the compiler wait for every load in
  // flight at the branch's end.
  auto load_batch = [&](int rb, uint4 (&kv)[U * RPP], float (&bs)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = u * kDecThreads + t;
      const int row = rb + p / LPH, seg = p % LPH;
      const int rr = row < nrows ? row : 0;
      const int cl = rr / G, hh = rr % G;
      const size_t ro = (hbase + hh) * a.Cmax + c0 + cl;
#pragma unroll
      for (int r = 0; r < RPP; ++r) kv[u * RPP + r] = reinterpret_cast<const uint4 *>(ks + ro * D + seg * 8)[r];
      bs[u] = a.b_sum[ro];
    }
  };
  auto reduce_batch = [&](int rb, const uint4 (&kv)[U * RPP], const float (&bs)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = u * kDecThreads + t;
      const int row = rb + p / LPH, seg = p % LPH;
      const int hh = (row < nrows) ? row % G : 0;
      float kf[8];
      Elem<T>::load8(reinterpret_cast<const T *>(&kv[u * RPP]), kf);
      const float *qv = sm.sc.qh + hh * D + seg * 8;
      float part = 0.f;
#pragma unroll
      for (int x = 0; x < 8; ++x) part += qv[x] * kf[x];
      const float dot = dpp_group_sum<LPH>(part);
      if (seg == 0 && row < nrows) sm.sc.s[row] = a.tau * dot + bs[u];
    }
  };
  {
    // Every batch load is issued unconditionally (past the slice it re-reads
    // the slice's first rows, cached): the number of loads in flight is then
    // the same on every path, and each reduction waits only for its own batch.
    uint4 kvA[U * RPP], kvB[U * RPP];
    float bsA[U], bsB[U];
    load_batch(0, kvA, bsA);
    __syncthreads();  // q-hat in LDS; the first batch's loads stay in flight
    for (int rb = 0; rb < nrows; rb += 2 * RS) {
      load_batch(rb + RS, kvB, bsB);
      reduce_batch(rb, kvA, bsA);
      if (rb + RS >= nrows) break;
      load_batch(rb + 2 * RS, kvA, bsA);
      reduce_batch(rb + RS, kvB, bsB);
    }
  }
  __syncthreads();
  for (int cl = t; cl < nch; cl += kDecThreads) {
    float m = -INFINITY;
    for (int hh = 0; hh < G; ++hh) m = fmaxf(m, sm.sc.s[cl * G + hh]);
    sm.sc.sig[cl] = m;
  }
  __syncthreads();
  const size_t cbase = ((static_cast<size_t>(b) * a.Hkv + g) * a.P + blk) * K;
  if ((t >> 6) == 0 && K > 0) slice_select<SNJ>(a, sm, nch, c0, G, cbase);
  // ---------------- ticket: the last slice block of (b, g) merges
  {
    const unsigned before = arrive(a.count1 + b * a.Hkv + g);
    if (t == 0) sm.is_last = (before == static_cast<unsigned>(a.P - 1));
  }
  __syncthreads();
  if (!sm.is_last) return;
  if (K > 0) merge_select<MNJ>(a, sm, b, g, n);
  if (t == 0) reset_counter(a.count1 + b * a.Hkv + g);
}

// ------------------------------------------------------------------ combine
// Log-sum-exp combine of nslots partial records (m, l, o[D]) per head, in
// slot order, into o = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s.
// The records were published by other workgroups; all loads are issued
// before they are used.  scratch: >= 2 * nslots * G + G floats of LDS.
template <typename T, int D>
__device__ __forceinline__ void combine_slots(const float *recs, int nslots, int G, float *scratch, T *out) {
  const int t = threadIdx.x;
  float *w = scratch;                  // [nslots * G]: e^{m - M}
  float *lt = scratch + nslots * G;    // [G]: sum w * l
  for (int x = t; x < nslots * G; x += kDecThreads) {
    const float *rh = recs + static_cast<size_t>(x) * (D + 2);
    w[x] = load_acquired(rh);
    scratch[nslots * G + G + x] = load_acquired(rh + 1);
  }
  __syncthreads();
  for (int hh = t; hh < G; hh += kDecThreads) {
    float M = -INFINITY;
    for (int s = 0; s < nslots; ++s) M = fmaxf(M, w[s * G + hh]);
    float L = 0.f;
    for (int s = 0; s < nslots; ++s) {
      const float m = w[s * G + hh];
      const float e = (m == -INFINITY) ? 0.f : __expf(m - M);
      w[s * G + hh] = e;
      L += e * scratch[nslots * G + G + s * G + hh];
    }
    lt[hh] = L;
  }
  __syncthreads();
  for (int x = t; x < G * D; x += kDecThreads) {
    const int hh = x / D, e = x % D;
    float acc = 0.f;
    int s = 0;
    for (; s + 8 <= nslots; s += 8) {
      float o8[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) o8[q] = load_acquired(recs + (static_cast<size_t>(s + q) * G + hh) * (D + 2) + 2 + e);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc += w[(s + q) * G + hh] * o8[q];
    }
    for (; s < nslots; ++s) acc += w[s * G + hh] * load_acquired(recs + (static_cast<size_t>(s) * G + hh) * (D + 2) + 2 + e);
    Elem<T>::store(out, static_cast<size_t>(hh) * D + e, acc / lt[hh]);
  }
}

// ------------------------------------------------------------------ D2
template <typename T, int D>
__global__ void __launch_bounds__(kDecThreads)
decode_attend_kernel(DecodeArgs a) {
  __shared__ UnitSmem<T, D> us;
  __shared__ int is_last;
  const int g = blockIdx.y, b = blockIdx.z, slot = blockIdx.x, t = threadIdx.x;
  const int G = a.Hq / a.Hkv, K = a.K;
  const int seq = clamp_seq(a.seq_lens, b, a.Tmax, a.err, false);
  const int i = seq - 1;
  (void)i;
  float *recs = a.parts + (static_cast<size_t>(b) * a.Hkv + g) * a.nslots * G * (D + 2);
  if (slot < K) {
    float *rec = recs + static_cast<size_t>(slot) * G * (D + 2);
    const int c = a.topk_idx[(static_cast<size_t>(b) * a.Hkv + g) * K + slot];
    if (c < 0) {
      for (int hh = t; hh < G; hh += kDecThreads) { publish(rec + hh * (D + 2), -INFINITY); publish(rec + hh * (D + 2) + 1, 0.f); }
    } else {
      load_q_rows<T, D>(us, static_cast<const T *>(a.q) + (static_cast<size_t>(b) * a.Hq + g * G) * D, D, G);
      __syncthreads();
      const T *kc = static_cast<const T *>(a.k_cache) + ((static_cast<size_t>(b) * a.Hkv + g) * a.Tmax + static_cast<size_t>(c) * a.S) * D;
      const T *vc = static_cast<const T *>(a.v_cache) + ((static_cast<size_t>(b) * a.Hkv + g) * a.Tmax + static_cast<size_t>(c) * a.S) * D;
      constexpr int NP = pairs_per_thread<D>();
      float2 ou[NP];
      attend_unit<T, D>(us, kc, vc, a.S, G, a.tau, ou);
#pragma unroll
      for (int r = 0; r < NP; ++r) {
        const int pr = t + r * kUnitThreads, hh = pr / (D / 2), e2 = pr % (D / 2);
        if (hh < G) {
          float *rh = rec + hh * (D + 2);
          const float inv = 1.f / us.l[hh];
          publish(rh + 2 + 2 * e2, ou[r].x * inv);
          publish(rh + 3 + 2 * e2, ou[r].y * inv);
          if (e2 == 0) { publish(rh, a.topk_score[(static_cast<size_t>(b) * a.Hq + g * G + hh) * K + slot]); publish(rh + 1, 1.f); }
        }
      }
    }
  }
  {
    const unsigned before = arrive(a.count2 + b * a.Hkv + g);
    if (t == 0) is_last = (before == static_cast<unsigned>(a.nslot_blocks - 1));
  }
  __syncthreads();
  if (!is_last) return;
  // combine every slot (chunks 0..K-1, window units K..) in slot order
  combine_slots<T, D>(recs, a.nslots, G, reinterpret_cast<float *>(us.v),
                      static_cast<T *>(a.o) + (static_cast<size_t>(b) * a.Hq + g * G) * D);
  if (t == 0) reset_counter(a.count2 + b * a.Hkv + g);
}

// ------------------------------------------------------------------ dense comparator
template <typename T, int D>
__global__ void __launch_bounds__(kDecThreads)
dense_decode_kernel(DenseArgs a) {
  __shared__ UnitSmem<T, D> us;
  __shared__ int is_last;
  const int g = blockIdx.y, b = blockIdx.z, p = blockIdx.x, t = threadIdx.x;
  const int G = a.Hq / a.Hkv;
  const int seq = clamp_seq(a.seq_lens, b, a.Tmax, a.err, p == 0 && g == 0 && t == 0);
  const int i = seq - 1;
  float *recs = a.parts + (static_cast<size_t>(b) * a.Hkv + g) * a.P * G * (D + 2);
  float *rec = recs + static_cast<size_t>(p) * G * (D + 2);
  const int j_lo = p * a.L, j_hi = min(i + 1, (p + 1) * a.L);
  constexpr int NP = pairs_per_thread<D>();
  if (j_lo >= j_hi) {
    for (int hh = t; hh < G; hh += kDecThreads) { publish(rec + hh * (D + 2), -INFINITY); publish(rec + hh * (D + 2) + 1, 0.f); }
  } else {
    load_q_rows<T, D>(us, static_cast<const T *>(a.q) + (static_cast<size_t>(b) * a.Hq + g * G) * D, D, G);
    __syncthreads();
    const T *kc = static_cast<const T *>(a.k_cache) + (static_cast<size_t>(b) * a.Hkv + g) * a.Tmax * D;
    const T *vc = static_cast<const T *>(a.v_cache) + (static_cast<size_t>(b) * a.Hkv + g) * a.Tmax * D;
    PairAcc<D> acc;
    acc.init();
    float2 ou[NP];
    for (int j0 = j_lo; j0 < j_hi; j0 += kUnitKeys) {
      const int nk = min(kUnitKeys, j_hi - j0);
      attend_unit<T, D>(us, kc + static_cast<size_t>(j0) * D, vc + static_cast<size_t>(j0) * D, nk, G, a.tau, ou);
#pragma unroll
      for (int r = 0; r < NP; ++r) {
        const int pr = t + r * kUnitThreads, hh = pr / (D / 2);
        if (hh < G) acc.add(r, us.m[hh], us.l[hh], ou[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int pr = t + r * kUnitThreads, hh = pr / (D / 2), e2 = pr % (D / 2);
      if (hh < G) {
        float *rh = rec + hh * (D + 2);
        publish(rh + 2 + 2 * e2, acc.o[r].x);
        publish(rh + 3 + 2 * e2, acc.o[r].y);
        if (e2 == 0) { publish(rh, acc.m[r]); publish(rh + 1, acc.l[r]); }
      }
    }
  }
  {
    const unsigned before = arrive(a.count + b * a.Hkv + g);
    if (t == 0) is_last = (before == static_cast<unsigned>(a.P - 1));
  }
  __syncthreads();
  if (!is_last) return;
  combine_slots<T, D>(recs, a.P, G, reinterpret_cast<float *>(us.v),
                      static_cast<T *>(a.o) + (static_cast<size_t>(b) * a.Hq + g * G) * D);
  if (t == 0) reset_counter(a.count + b * a.Hkv + g);
}

// ------------------------------------------------------------------ launchers
template <typename T, int D, bool QCAL, int SNJ, int MNJ>
static void launch_d1(const DecodeArgs &a, hipStream_t st) {
  decode_score_kernel<T, D, QCAL, SNJ, MNJ><<<dim3(a.P + a.NW, a.Hkv, a.B), kDecThreads, 0, st>>>(a);
}

// slice width SNJ = CPB / 64 in {1, 4, 16}; merge width MNJ = P*K / 256 rounded up to {4, 8, 16}
template <typename T, int D, bool QCAL>
static void dispatch_d1(const DecodeArgs &a, hipStream_t st) {
  const int snj = a.CPB / 64, mnj_need = (a.P * a.K + kDecThreads - 1) / kDecThreads;
  const int mnj = mnj_need <= 4 ? 4 : (mnj_need <= 8 ? 8 : 16);
#define HILS_D1(S_, M_) \
  if (snj == S_ && mnj == M_) return launch_d1<T, D, QCAL, S_, M_>(a, st);
  HILS_D1(1, 4) HILS_D1(1, 8) HILS_D1(1, 16) HILS_D1(4, 4) HILS_D1(4, 8) HILS_D1(4, 16)
  HILS_D1(16, 4) HILS_D1(16, 8) HILS_D1(16, 16)
#undef HILS_D1
}

template <typename T, int D>
static hipError_t decode_t(const DecodeArgs &a, hipStream_t st) {
  if (a.r > 0) {
    decode_qcal_kernel<T, D><<<a.B, kDecThreads, 0, st>>>(
        static_cast<const T *>(a.q), static_cast<const T *>(a.h), static_cast<const T *>(a.w_down),
        static_cast<const T *>(a.w_up), a.qhat, a.Hq, a.r, a.Dh);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dispatch_d1<T, D, true>(a, st);
  } else {
    dispatch_d1<T, D, false>(a, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_attend_kernel<T, D><<<dim3(a.nslot_blocks, a.Hkv, a.B), kDecThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? decode_t<uint16_t, 128>(a, st) : decode_t<uint16_t, 64>(a, st);
  return a.d == 128 ? decode_t<float, 128>(a, st) : decode_t<float, 64>(a, st);
}

template <typename T, int D>
static hipError_t dense_t(const DenseArgs &a, hipStream_t st) {
  dense_decode_kernel<T, D><<<dim3(a.P, a.Hkv, a.B), kDecThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_dense_decode(const DenseArgs &a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? dense_t<uint16_t, 128>(a, st) : dense_t<uint16_t, 64>(a, st);
  return a.d == 128 ? dense_t<float, 128>(a, st) : dense_t<float, 64>(a, st);
}

}  // namespace hils
