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
//           score slice: stream 64 chunks' k'/b' of the G heads (the
//           dominant HBM stream) -> each chunk's group score sigma and
//           per-head scores in the workspace.
//           window unit: 64 window keys -> online-softmax partial.
//   D2      grid (K chunk slots, H_kv, B): every slot workgroup selects the
//           top-K from sigma (identically), attends the chunk of its rank
//           -> its (s_hat, 1, o_c) partial; the last block of (b, g)
//           combines the chunk and window partials in a fixed order
//           (deterministic).
#include "attn_unit.h"
#include "hils_common.h"
#include "launch.h"

namespace hils {

constexpr int kDecThreads = 256;

__device__ __forceinline__ int clamp_seq(const int32_t *seq_lens, int b, int Tmax, unsigned *err, bool count) {
  int s = seq_lens[b];
  if (s < 1 || s > Tmax) {
    if (count) atomicAdd(err, 1u);
    s = s < 1 ? 1 : Tmax;
  }
  return s;
}

// First row of the 64-key block j0 .. j0 + 63 of (b, g) (j0 a multiple of
// S = 64): in the contiguous cache [B, Hkv, Tmax, D], or in the page
// [num_pages, Hkv, S, D] that the block table gives for block j0 / S.  A page
// index outside [0, num_pages) gives nullptr (and, with count, one error).
template <typename T, int D>
__device__ __forceinline__ const T *kv_block(const DecodeArgs &a, const void *cache, int b, int g, int j0,
                                             bool count) {
  const T *base = static_cast<const T *>(cache);
  if (!a.block_table) return base + ((static_cast<size_t>(b) * a.Hkv + g) * a.Tmax + j0) * D;
  const int pg = a.block_table[static_cast<size_t>(b) * a.max_pages + j0 / a.S];
  if (pg < 0 || pg >= a.num_pages) {
    if (count) atomicAdd(a.err, 1u);
    return nullptr;
  }
  return base + (static_cast<size_t>(pg) * a.Hkv + g) * a.S * D;
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
constexpr int kCPB = 64;                    // chunks per score slice
constexpr int kRowsMax = kCPB * kMaxG;      // (chunk, head) rows of one slice
struct D1Smem {
  float qh[kMaxG * 128];
  float s[kRowsMax];  // per (chunk, head) score of the slice
};

// a score-slice block and a window-unit block never need both layouts
template <typename T, int D>
union D1Shared {
  D1Smem sc;
  UnitSmem<T, D> us;
};

// D1: score slices stream k'/b' of the group's heads and store every
// eligible chunk's group score sigma = max over the heads (and each head's
// own score); the selection runs in D2, after the kernel boundary.
template <typename T, int D, bool QCAL>
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
  if (blk >= a.P) {  // ---------------- window unit
    const int u = blk - a.P;
    const int j0 = n * a.S + u * kUnitKeys;
    float *rec = a.parts + ((static_cast<size_t>(b) * a.Hkv + g) * a.nslots + K + u) * G * (D + 2);
    const T *kb = j0 > i ? nullptr : kv_block<T, D>(a, a.k_cache, b, g, j0, t == 0);
    const T *vb = kb ? kv_block<T, D>(a, a.v_cache, b, g, j0, false) : nullptr;
    if (!vb) {  // past the query, or a page outside the pool: no keys
      for (int hh = t; hh < G; hh += kDecThreads) publish2(rec + hh * (D + 2), -INFINITY, 0.f);
      return;
    }
    const int nk = min(kUnitKeys, i - j0 + 1);
    load_q_rows<T, D>(us, static_cast<const T *>(a.q) + (static_cast<size_t>(b) * a.Hq + g * G) * D, D, G);
    __syncthreads();
    constexpr int NP = pairs_per_thread<D>();
    float2 ou[NP];
    attend_unit<T, D>(us, kb, vb, nk, G, a.tau, ou);
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int pr = t + r * kUnitThreads, hh = pr / (D / 2), e2 = pr % (D / 2);
      if (hh < G) {
        float *rh = rec + hh * (D + 2);
        publish2(rh + 2 + 2 * e2, ou[r].x, ou[r].y);
        if (e2 == 0) publish2(rh, us.m[hh], us.l[hh]);
      }
    }
    return;
  }

  // ---------------- score slice: chunks [c0, c0 + nch) of the G heads
  if (a.Cmax == 0) return;  // no chunk summary is stored (k_sum may be absent)
  const int c0 = blk * kCPB;
  const int nch = max(0, min(c0 + kCPB, n) - c0);
  constexpr int LPH = D / 8;                         // lanes per (chunk, head) row, 8 elements each
  constexpr int RPP = static_cast<int>(sizeof(T)) / 2;  // 16-byte loads per 8-element piece
  constexpr int U = 4 / RPP;                         // pieces in flight per thread (80 registers:
                                                     // five workgroups per CU, the whole grid at once)
  constexpr int RS = U * kDecThreads / LPH;          // rows per batch
  // rows are (head, chunk) in head-major order, row = hh * kCPB + cl: the 4
  // rows one load instruction covers are 1 KB of one head's contiguous
  // summaries
  const int nrows = nch > 0 ? G * kCPB : 0;
  const T *ks = static_cast<const T *>(a.k_sum);
  const size_t hbase = static_cast<size_t>(b) * a.Hq + g * G;
  // Batches of RS rows, double buffered in registers: the loads of batch
  // n + 1 are in flight while batch n is reduced.
  // Branch-free, and independent of n (a dependent load: the sequence
  // length): every row of the slice is read, its chunk clamped to the last
  // one stored, and rows past the slice read its row 0 again.  Only the
  // rows of eligible chunks are stored.  Every lane of a row reads the
  // row's b'.  A load under a lane-dependent branch would make the compiler
  // wait for every load in flight at the branch's end.
  auto load_batch = [&](int rb, uint4 (&kv)[U * RPP], float (&bs)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = u * kDecThreads + t;
      const int row = rb + p / LPH, seg = p % LPH;
      const int rr = row < G * kCPB ? row : 0;
      const int cl = rr & (kCPB - 1), hh = rr / kCPB;
      const size_t ro = (hbase + hh) * a.Cmax + min(c0 + cl, a.Cmax - 1);
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
      const int hh = (row < nrows) ? row / kCPB : 0;
      float kf[8];
      Elem<T>::load8(reinterpret_cast<const T *>(&kv[u * RPP]), kf);
      const float *qv = sm.qh + hh * D + seg * 8;
      float part = 0.f;
#pragma unroll
      for (int x = 0; x < 8; ++x) part += qv[x] * kf[x];
      const float dot = dpp_group_sum<LPH>(part);
      if (seg == 0 && row < nrows && (row & (kCPB - 1)) < nch) sm.s[row] = a.tau * dot + bs[u];
    }
  };
  {
    // Every batch load is issued unconditionally (past the slice it re-reads
    // the slice's first rows, cached): the number of loads in flight is then
    // the same on every path, and each reduction waits only for its own batch.
    uint4 kvA[U * RPP], kvB[U * RPP];
    float bsA[U], bsB[U];
    load_batch(0, kvA, bsA);
    // the query rows go to LDS while the first batch is in flight
    for (int x = t; x < G * D; x += kDecThreads) {
      const size_t qo = hbase * D + x;
      sm.qh[x] = QCAL ? a.qhat[qo] : Elem<T>::load(static_cast<const T *>(a.q), qo);
    }
    __syncthreads();
    for (int rb = 0; rb < nrows; rb += 2 * RS) {
      load_batch(rb + RS, kvB, bsB);
      reduce_batch(rb, kvA, bsA);
      if (rb + RS >= nrows) break;
      load_batch(rb + 2 * RS, kvA, bsA);
      reduce_batch(rb + RS, kvB, bsB);
    }
  }
  __syncthreads();
  // sigma and the per-head scores of the slice's chunks (hsc is chunk-major)
  const size_t bg = static_cast<size_t>(b) * a.Hkv + g;
  // (nch <= kCPB: the slice's chunks are the lanes of wave 0, whose maximum
  // is the slice's, for the selection's first bound)
  for (int cl = t; cl < nch; cl += kDecThreads) {
    float m = -INFINITY;
    for (int hh = 0; hh < G; ++hh) m = fmaxf(m, sm.s[hh * kCPB + cl]);
    a.sig[bg * a.Cmax + c0 + cl] = m;
  }
  if (t < 64) {
    float m = -INFINITY;
    if (t < nch)
      for (int hh = 0; hh < G; ++hh) m = fmaxf(m, sm.s[hh * kCPB + t]);
    m = wave_reduce_f32<1>(m);
    if (t == 0) a.smax[bg * a.P + blk] = m;
  }
  for (int x = t; x < nch * G; x += kDecThreads) a.hsc[(bg * a.Cmax + c0) * G + x] = sm.s[(x % G) * kCPB + x / G];
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
  float *lv = scratch + nslots * G + G;  // [nslots * G]: l
  // Loads first, in one round trip: (m, l) of every (slot, head), then the
  // o pairs of every slot for this thread's first output pair (8-byte
  // loads; no lane-dependent branch: a thread past the outputs re-reads
  // pair 0).  The (m, l) loads are older, so the weights wait only for them.
  constexpr int kPre = 32;
  const int nml = nslots * G, npairs = G * D / 2, npre = min(nslots, kPre);
  float2 ml[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int x = t + u * kDecThreads;
    ml[u] = load_acquired2(recs + static_cast<size_t>(x < nml ? x : 0) * (D + 2));
  }
  const int p0 = t < npairs ? t : 0;
  const int hh0 = p0 / (D / 2), e20 = p0 % (D / 2);
  float2 ov[kPre];
#pragma unroll
  for (int q = 0; q < kPre; ++q)
    if (q < npre) ov[q] = load_acquired2(recs + (static_cast<size_t>(q) * G + hh0) * (D + 2) + 2 + 2 * e20);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int x = t + u * kDecThreads;
    if (x < nml) { w[x] = ml[u].x; lv[x] = ml[u].y; }
  }
  for (int x = t + 2 * kDecThreads; x < nml; x += kDecThreads) {  // more than 2 per thread
    const float2 v = load_acquired2(recs + static_cast<size_t>(x) * (D + 2));
    w[x] = v.x;
    lv[x] = v.y;
  }
  __syncthreads();
  // weights e^{m - M} and the normaliser per head: one wave per head,
  // slots over lanes
  {
    const int lane = t & 63;
    for (int hh = t >> 6; hh < G; hh += kDecThreads / 64) {
      float mloc = -INFINITY;
      for (int s = lane; s < nslots; s += 64) mloc = fmaxf(mloc, w[s * G + hh]);
      const float M = wave_reduce_f32<1>(mloc);
      float lloc = 0.f;
      for (int s = lane; s < nslots; s += 64) {
        const float m = w[s * G + hh];
        const float e = (m == -INFINITY) ? 0.f : __expf(m - M);
        w[s * G + hh] = e;
        lloc += e * lv[s * G + hh];
      }
      const float L = wave_reduce_f32<2>(lloc);
      if (lane == 0) lt[hh] = L;
    }
  }
  __syncthreads();
  for (int p = t; p < npairs; p += kDecThreads) {
    const int hh = p / (D / 2), e2 = p % (D / 2);
    float2 acc = make_float2(0.f, 0.f);
    if (p == t) {
      // (the weights are read without a branch, so that the reads go out
      // together; past npre the term is skipped)
      float wq[kPre];
#pragma unroll
      for (int q = 0; q < kPre; ++q) wq[q] = w[(q < npre ? q : 0) * G + hh];
#pragma unroll
      for (int q = 0; q < kPre; ++q)
        if (q < npre) {
          acc.x += wq[q] * ov[q].x;
          acc.y += wq[q] * ov[q].y;
        }
    } else {
      for (int q = 0; q < npre; ++q) {
        const float2 v = load_acquired2(recs + (static_cast<size_t>(q) * G + hh) * (D + 2) + 2 + 2 * e2);
        acc.x += w[q * G + hh] * v.x;
        acc.y += w[q * G + hh] * v.y;
      }
    }
    for (int q = npre; q < nslots; ++q) {
      const float2 v = load_acquired2(recs + (static_cast<size_t>(q) * G + hh) * (D + 2) + 2 + 2 * e2);
      acc.x += w[q * G + hh] * v.x;
      acc.y += w[q * G + hh] * v.y;
    }
    const float inv = 1.f / lt[hh];
    Elem<T>::store2(out + static_cast<size_t>(hh) * D + 2 * e2, acc.x * inv, acc.y * inv);
  }
}

// ------------------------------------------------------------------ D2
constexpr int kSelVPT = 8;  // a 2048-score tile: D2 then fits four workgroups per CU (LDS, registers)
constexpr int kSelWaves = kDecThreads / 64;
constexpr int kSurvMax = 256;  // survivors the one-wave exact select takes (plus the kept winners)
constexpr int kSurvNJ = (kSurvMax + 32 + 63) / 64;
struct SelSmem {
  unsigned long long key[32];     // winners so far: (ordered score, ~chunk)
  unsigned long long sorted[32];  // final winners in rank order
  alignas(16) unsigned long long surv[kSurvMax + 32];
  uint32_t tw[kSelWaves];         // per-wave lower bound of the threshold
  uint32_t red[2][kSelWaves];     // per-wave partial sums / minima, double buffered
  uint32_t red2[2][kSelWaves];
  int nkey, nsurv, nslice;
  uint32_t sord[kDecThreads * kSelVPT];  // the tile's ordered scores (0 = none); or surviving slices
};

__device__ __forceinline__ unsigned long long sel_key(uint32_t ord, int c) {
  return (static_cast<unsigned long long>(ord) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(c));
}

// Sum (SUM) or minimum over the block of one value per wave (wave-uniform
// inputs); `slot` alternates between calls so one barrier per call suffices.
template <bool SUM>
__device__ __forceinline__ uint32_t block_reduce_waves(uint32_t v, uint32_t (&red)[2][kSelWaves], int &slot) {
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[slot][wave] = v;
  __syncthreads();
  uint32_t r = red[slot][0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) r = SUM ? r + red[slot][w] : min(r, red[slot][w]);
  slot ^= 1;
  return r;
}

__device__ __forceinline__ uint32_t wave_usum(uint32_t v) { return wave_reduce_u32<2>(v); }
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) { return wave_reduce_u32<0>(v); }

// Exact top-K of one tile with all threads: a bitwise search for the
// keep-th largest ordered score theta (counting with ballots, summed over
// the waves through LDS; it starts below the common leading bits of the
// smallest and largest candidate and stops once exactly `keep` scores are at
// or above the trial value), then every score above theta and the lowest
// chunks tied at theta.  Candidates: ord[] (0 = none) and the nprev winners
// kept from earlier tiles.  Leaves the winners, unordered, in ss.key[0..nkey).
__device__ __forceinline__ void tile_select_exact(const uint32_t (&ord)[kSelVPT], int tile0, int K, SelSmem &ss,
                                                  int &slot) {
  const int t = threadIdx.x;
  const int nprev = ss.nkey;
  const unsigned long long xkey = t < nprev ? ss.key[t] : 0ull;
  const uint32_t xo = static_cast<uint32_t>(xkey >> 32);
  const int xc = static_cast<int>(~static_cast<uint32_t>(xkey));
  uint32_t cnt = xo != 0u ? 1u : 0u, lo = xo != 0u ? xo : 0xFFFFFFFFu, hi = xo;
#pragma unroll
  for (int j = 0; j < kSelVPT; ++j) {
    cnt += ord[j] != 0u ? 1u : 0u;
    lo = min(lo, ord[j] != 0u ? ord[j] : 0xFFFFFFFFu);
    hi = max(hi, ord[j]);
  }
  const uint32_t avail = block_reduce_waves<true>(wave_usum(cnt), ss.red, slot);
  lo = block_reduce_waves<false>(wave_umin(lo), ss.red2, slot);
  hi = ~block_reduce_waves<false>(wave_umin(~hi), ss.red, slot);
  const int keep = min(K, static_cast<int>(avail));
  uint32_t theta = 0u;
  bool exact = false;
  if (keep > 0) {
    const uint32_t spread = lo ^ hi;
    const int top = spread ? 31 - __clz(spread) : -1;
    theta = top < 0 ? lo : (top == 31 ? 0u : lo & ~((2u << top) - 1u));
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t cand = theta | (1u << bit);
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < kSelVPT; ++j) c += __popcll(__ballot(ord[j] >= cand));
      c += __popcll(__ballot(xo >= cand && xo != 0u));
      const uint32_t tot = block_reduce_waves<true>(c, ss.red, slot);
      if (static_cast<int>(tot) >= keep) {
        theta = cand;
        if (static_cast<int>(tot) == keep) {
          exact = true;
          break;
        }
      }
    }
    if (top < 0) exact = static_cast<int>(avail) == keep;
  }
  uint32_t win = 0u;  // bit j: ord[j]
  uint32_t ngt = 0;
#pragma unroll
  for (int j = 0; j < kSelVPT; ++j) {
    const bool w = keep > 0 && ord[j] != 0u && (exact ? ord[j] >= theta : ord[j] > theta);
    win |= w ? (1u << j) : 0u;
    ngt += __popcll(__ballot(w));
  }
  bool xw = keep > 0 && xo != 0u && (exact ? xo >= theta : xo > theta);
  ngt += __popcll(__ballot(xw));
  int need = keep - static_cast<int>(block_reduce_waves<true>(ngt, ss.red, slot));
  while (need > 0) {  // uniform: every thread sees the same counts
    uint32_t best = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < kSelVPT; ++j)
      if (!((win >> j) & 1u) && ord[j] == theta && ord[j] != 0u)
        best = min(best, static_cast<uint32_t>(tile0 + j * kDecThreads + t));
    if (!xw && xo == theta && xo != 0u) best = min(best, static_cast<uint32_t>(xc));
    best = block_reduce_waves<false>(wave_umin(best), ss.red2, slot);
    if (best == 0xFFFFFFFFu) break;
#pragma unroll
    for (int j = 0; j < kSelVPT; ++j)
      if (static_cast<uint32_t>(tile0 + j * kDecThreads + t) == best && ord[j] == theta) win |= 1u << j;
    if (!xw && xo == theta && static_cast<uint32_t>(xc) == best) xw = true;
    --need;
  }
  __syncthreads();  // every thread has read ss.key / ss.nkey
  if (t == 0) ss.nkey = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kSelVPT; ++j)
    if ((win >> j) & 1u) ss.key[atomicAdd(&ss.nkey, 1)] = sel_key(ord[j], tile0 + j * kDecThreads + t);
  if (xw) ss.key[atomicAdd(&ss.nkey, 1)] = xkey;
  __syncthreads();
}

// The k-th largest of one ordered value per lane (0 = none), or 0 when
// fewer than k lanes hold a value: a bitwise search from below the common
// leading bits of the smallest and largest value, counting with ballots.
__device__ __forceinline__ uint32_t wave_kth_u32(uint32_t v, int k) {
  const int avail = __popcll(__ballot(v != 0u));
  if (k <= 0 || avail < k) return 0u;
  const uint32_t lo = wave_reduce_u32<0>(v != 0u ? v : 0xFFFFFFFFu), hi = wave_reduce_u32<1>(v);
  const uint32_t spread = lo ^ hi;
  if (!spread) return lo;
  const int top = 31 - __clz(spread);
  uint32_t theta = top == 31 ? 0u : lo & ~((2u << top) - 1u);
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = theta | (1u << bit);
    if (__popcll(__ballot(v >= cand)) >= k) theta = cand;
  }
  return theta;
}

// One wave selects the top-K of the tot survivor keys in ss.surv into
// ss.key (unordered; block_topk ranks them) and ss.nkey: the K-th largest
// key by a bitwise search over the 64-bit keys' ordered-score word, every
// key above it, and the lowest chunks tied at it.
template <int NJ>
__device__ __forceinline__ void select_survivors(SelSmem &ss, int tot, int K) {
  const int lane = threadIdx.x & 63;
  uint32_t so[NJ];
  int si[NJ];
  int avail = 0;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int x = j * 64 + lane;
    const unsigned long long kk = x < tot ? ss.surv[x] : 0ull;
    so[j] = static_cast<uint32_t>(kk >> 32);
    si[j] = x < tot ? static_cast<int>(~static_cast<uint32_t>(kk)) : 0x7FFFFFFF;
    avail += __popcll(__ballot(so[j] != 0u));
    lo = min(lo, so[j] != 0u ? so[j] : 0xFFFFFFFFu);
    hi = max(hi, so[j]);
  }
  const int keep = min(K, avail);
  lo = wave_reduce_u32<0>(lo);
  hi = wave_reduce_u32<1>(hi);
  uint32_t theta = 0u;
  bool exact = false;
  if (keep > 0) {
    const uint32_t spread = lo ^ hi;
    const int top = spread ? 31 - __clz(spread) : -1;
    theta = top < 0 ? lo : (top == 31 ? 0u : lo & ~((2u << top) - 1u));
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t cand = theta | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) cnt += __popcll(__ballot(so[j] >= cand));
      if (cnt >= keep) {
        theta = cand;
        if (cnt == keep) {
          exact = true;
          break;
        }
      }
    }
    if (top < 0) exact = avail == keep;
  }
  bool w[NJ];
  int ngt = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    w[j] = keep > 0 && so[j] != 0u && (exact ? so[j] >= theta : so[j] > theta);
    ngt += __popcll(__ballot(w[j]));
  }
  for (int need = keep - ngt; need > 0; --need) {  // ties at theta: lowest chunk first
    int best = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (!w[j] && so[j] == theta && so[j] != 0u) best = min(best, si[j]);
    best = static_cast<int>(wave_reduce_u32<0>(static_cast<uint32_t>(best)));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (!w[j] && so[j] == theta && si[j] == best) w[j] = true;
  }
  int base = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const unsigned long long m = __ballot(w[j]);
    const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
    if (w[j]) ss.key[base + below] = sel_key(so[j], si[j]);
    base += __popcll(m);
  }
  if (lane == 0) ss.nkey = base;
}

// Block-wide top-K of the group scores sigma[0..n) by (sigma desc, chunk
// asc), all kDecThreads threads, in tiles of kDecThreads * kSelVPT scores
// (2048 chunks; longer lists go through block_topk_sliced first).  Per tile:
//  1. a lower bound of the threshold: in a wave whose lanes' maxima include
//     at least K scores, the K-th largest lane maximum is exceeded or met by
//     K distinct scores, so it cannot lie above the tile's K-th largest
//     score; the largest such bound over the waves is taken;
//  2. the scores at or above it (typically a few dozen) and the winners kept
//     from earlier tiles are collected in LDS, and one wave selects exactly
//     among them (same order, same tie rule);
//  3. when too many scores pass (many equal scores), the tile falls back to
//     the exact block-wide search.
// On return ss.sorted[0..keep) holds the winners in rank order; returns keep.
__device__ __forceinline__ int block_topk(const float *sig, int n, int cmax, int K, SelSmem &ss) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int slot = 0;
  // loads without a lane-dependent branch, all issued before the first is
  // used; the first tile's go out before n is known (it follows from the
  // sequence length, itself a load): they read every stored score (past
  // cmax, sigma[0] again) and n masks them afterwards
  float sv[kSelVPT];
  if (cmax > 0) {
#pragma unroll
    for (int j = 0; j < kSelVPT; ++j) {
      const int c = j * kDecThreads + t;
      sv[j] = sig[c < cmax ? c : 0];
    }
  }
  if (t == 0) ss.nkey = 0;
  __syncthreads();
  for (int tile0 = 0; tile0 < n; tile0 += kDecThreads * kSelVPT) {
    if (tile0 > 0) {  // (past n, sigma[0] again)
#pragma unroll
      for (int j = 0; j < kSelVPT; ++j) {
        const int c = tile0 + j * kDecThreads + t;
        sv[j] = sig[c < n ? c : 0];
      }
    }
    uint32_t mx = 0u;
#pragma unroll
    for (int j = 0; j < kSelVPT; ++j) {
      const uint32_t o = tile0 + j * kDecThreads + t < n ? orderable(sv[j]) : 0u;  // 0: no candidate
      ss.sord[j * kDecThreads + t] = o;
      mx = max(mx, o);
    }
    // 1. per-wave bound: the K-th largest lane maximum (0 = no bound)
    {
      const uint32_t kth = wave_kth_u32(mx, K);
      if (lane == 0) ss.tw[wave] = kth;
    }
    if (t == 0) ss.nsurv = 0;
    __syncthreads();
    uint32_t bound = 1u;  // real scores are >= 1 in the ordered form
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) bound = max(bound, ss.tw[w]);
    // 2. survivors: scores >= bound (none of the others can be among the
    // tile's K largest), then the winners kept so far
    const int nprev = ss.nkey;
    {
      // (a thread holds a survivor only when its lane maximum reaches the bound)
      if (mx >= bound) {
        uint32_t sm = 0u;
#pragma unroll
        for (int j = 0; j < kSelVPT; ++j) sm |= ss.sord[j * kDecThreads + t] >= bound ? (1u << j) : 0u;
        int pos = atomicAdd(&ss.nsurv, __popc(sm));  // one LDS atomic per such thread
        while (sm) {
          const int j = __ffs(sm) - 1;
          sm &= sm - 1u;
          if (pos < kSurvMax) ss.surv[pos] = sel_key(ss.sord[j * kDecThreads + t], tile0 + j * kDecThreads + t);
          ++pos;
        }
      }
    }
    __syncthreads();
    const int ns = ss.nsurv;
    if (ns <= kSurvMax) {
      if (t < nprev) ss.surv[ns + t] = ss.key[t];
      __syncthreads();
      if (wave == 0) {
        const int tot = ns + nprev;
        if (tot <= 64)
          select_survivors<1>(ss, tot, K);
        else
          select_survivors<kSurvNJ>(ss, tot, K);
      }
      __syncthreads();
    } else {
      // 3. many scores at the bound: the exact block-wide search, on the
      // tile's scores read again
      uint32_t ord2[kSelVPT];
#pragma unroll
      for (int j = 0; j < kSelVPT; ++j) {
        const int c = tile0 + j * kDecThreads + t;
        const float v = sig[c < n ? c : 0];
        ord2[j] = c < n ? orderable(v) : 0u;
      }
      tile_select_exact(ord2, tile0, K, ss, slot);
    }
  }
  // rank the winners: position = number of larger keys
  const int keep = ss.nkey;
  if (t < keep) {
    const unsigned long long k0 = ss.key[t];
    int r = 0;
    for (int e = 0; e < keep; ++e) r += ss.key[e] > k0 ? 1 : 0;
    ss.sorted[r] = k0;
  }
  __syncthreads();
  return keep;
}

// After the survivors are in ss.surv[0 .. ss.nsurv) (a barrier behind):
// one wave selects exactly among them, and the winners are ranked into
// ss.sorted; too many survivors (many equal scores): block_topk on sig.
// Returns keep.
__device__ __forceinline__ int select_ranked(const float *sig, int n, int cmax, int K, SelSmem &ss) {
  const int t = threadIdx.x, wave = t >> 6;
  const int tot = ss.nsurv;
  if (tot > kSurvMax) return block_topk(sig, n, cmax, K, ss);
  if (tot <= 64) {
    // At most 64 survivors (the usual case): lane x of wave 0 takes
    // survivor x; its position in (score desc, chunk asc) order is the
    // number of larger keys (the keys are distinct: they hold the chunk),
    // and the first min(K, tot) positions are the winners.
    if (wave == 0) {
      const int lane = t & 63;
      const unsigned long long kx = lane < tot ? ss.surv[lane] : 0ull;
      const ulonglong2 *s2 = reinterpret_cast<const ulonglong2 *>(ss.surv);
      int r = 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const ulonglong2 w2 = s2[e];  // keys 2 e and 2 e + 1 (past tot: not counted)
        r += (2 * e < tot && w2.x > kx) ? 1 : 0;
        r += (2 * e + 1 < tot && w2.y > kx) ? 1 : 0;
      }
      if (lane < tot && r < K) ss.sorted[r] = kx;
    }
    __syncthreads();
    return min(K, tot);
  }
  if (wave == 0) {
    if (tot <= 64)
      select_survivors<1>(ss, tot, K);
    else
      select_survivors<kSurvNJ>(ss, tot, K);
  }
  __syncthreads();
  const int keep = ss.nkey;
  if (t < keep) {
    const unsigned long long k0 = ss.key[t];
    int r = 0;
    for (int e = 0; e < keep; ++e) r += ss.key[e] > k0 ? 1 : 0;
    ss.sorted[r] = k0;
  }
  __syncthreads();
  return keep;
}

// The same selection, narrowed first by the slices' maxima (each the largest
// group score of 64 consecutive chunks, stored by D1):
//  1. a lower bound of the threshold from the maxima, as in step 1 above:
//     K lanes whose maximum over their slices reaches it hold K distinct
//     chunks' scores at or above it;
//  2. only slices whose maximum reaches the bound can hold a winner; their
//     scores at or above the bound are the survivors;
//  3. one wave selects exactly among them.
// Too many surviving slices or scores (many equal scores): block_topk.
// The slice maxima come preloaded: smv[j] = the maximum of slice
// j * kDecThreads + t (any value past the stored slices).
constexpr int kSlicePT = 8;                          // slice maxima per thread
constexpr int kSliceMax = kDecThreads * kSelVPT;     // surviving slices kept (LDS: ss.sord)
__device__ __forceinline__ int block_topk_sliced(const float *sig, const float (&smv)[kSlicePT], int n, int cmax,
                                                 int K, SelSmem &ss) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int ns = (n + kCPB - 1) / kCPB;  // slices holding eligible chunks
  uint32_t mx = 0u, so[kSlicePT];
#pragma unroll
  for (int j = 0; j < kSlicePT; ++j) {
    const int s = j * kDecThreads + t;
    so[j] = s < ns ? orderable(smv[j]) : 0u;
    mx = max(mx, so[j]);
  }
  {
    const uint32_t kth = wave_kth_u32(mx, K);
    if (lane == 0) ss.tw[wave] = kth;
  }
  if (t == 0) {
    ss.nkey = 0;
    ss.nsurv = 0;
    ss.nslice = 0;
  }
  __syncthreads();
  uint32_t bound = 1u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) bound = max(bound, ss.tw[w]);
#pragma unroll
  for (int j = 0; j < kSlicePT; ++j) {
    if (so[j] >= bound) {
      const int p = atomicAdd(&ss.nslice, 1);
      if (p < kSliceMax) ss.sord[p] = static_cast<uint32_t>(j * kDecThreads + t);
    }
  }
  __syncthreads();
  const int nsl = ss.nslice;
  if (nsl > kSliceMax) return block_topk(sig, n, cmax, K, ss);
  // the surviving slices' scores: loads first, then the filter
  constexpr int kPT = 8;  // scores per thread per round
  for (int x0 = 0; x0 < nsl * kCPB; x0 += kDecThreads * kPT) {
    float v[kPT];
    int c[kPT];
#pragma unroll
    for (int j = 0; j < kPT; ++j) {
      const int x = x0 + j * kDecThreads + t;
      const int sl = x < nsl * kCPB ? static_cast<int>(ss.sord[x / kCPB]) : 0;
      c[j] = x < nsl * kCPB ? sl * kCPB + x % kCPB : n;
      v[j] = sig[c[j] < n ? c[j] : 0];
    }
#pragma unroll
    for (int j = 0; j < kPT; ++j) {
      const uint32_t o = c[j] < n ? orderable(v[j]) : 0u;
      if (o >= bound) {
        const int p = atomicAdd(&ss.nsurv, 1);
        if (p < kSurvMax) ss.surv[p] = sel_key(o, c[j]);
      }
    }
  }
  __syncthreads();
  return select_ranked(sig, n, cmax, K, ss);
}


// D2: every slot workgroup of (b, g) selects the top-K from the group scores
// (the same arithmetic in each, so they agree), slot 0 writes the lists,
// and slot k attends the chunk of rank k; the last workgroup combines the
// chunk and window partials in slot order.
template <typename T, int D>
__global__ void __launch_bounds__(kDecThreads)
decode_attend_kernel(DecodeArgs a) {
  __shared__ UnitSmem<T, D> us;
  __shared__ SelSmem ss;
  __shared__ int is_last;
  const int g = blockIdx.y, b = blockIdx.z, slot = blockIdx.x, t = threadIdx.x;
  const int G = a.Hq / a.Hkv, K = a.K;
  const size_t bg = static_cast<size_t>(b) * a.Hkv + g;
  float *recs = a.parts + bg * a.nslots * G * (D + 2);
  // The query rows (parked in LDS after the selection) and the slice maxima
  // go out before the sequence length (itself a load) is known, so that they
  // arrive with it; n masks the maxima afterwards.  (Loading every group
  // score here as well, to skip the survivors' dependent load, was slower:
  // the larger transfer delays the rest.)
  constexpr int QPT = (kMaxG * D + kDecThreads - 1) / kDecThreads;
  T qraw[QPT];  // raw: converted when parked, so that nothing waits for it before
  float smv[kSlicePT];
  const bool sliced = K > 0 && a.Cmax > kCPB * K;  // the slice maxima can be used
  const float *sig = a.sig + bg * a.Cmax;
  {
    // (no load under a branch, whose end would wait for it: past G * D a
    // thread reads element 0 again and does not park it; with K = 0 the
    // rows are read and not used)
    const T *qsrc = static_cast<const T *>(a.q) + (static_cast<size_t>(b) * a.Hq + g * G) * D;
#pragma unroll
    for (int r = 0; r < QPT; ++r) {
      const int x = t + r * kDecThreads;
      qraw[r] = qsrc[x < G * D ? x : 0];
    }
  }
  if (sliced) {
    const float *sx = a.smax + bg * a.P;
#pragma unroll
    for (int j = 0; j < kSlicePT; ++j) {
      const int x = j * kDecThreads + t;
      smv[j] = sx[x < a.P ? x : 0];
    }
  }
  const int seq = clamp_seq(a.seq_lens, b, a.Tmax, a.err, false);
  const int i = seq - 1;
  const int n = eligible_chunks(i, a.W, a.S);
  if (K > 0) {
    const int keep = !(n > kCPB * K && (n + kCPB - 1) / kCPB <= kSlicePT * kDecThreads)
                         ? block_topk(sig, n, a.Cmax, K, ss)
                         : block_topk_sliced(sig, smv, n, a.Cmax, K, ss);
#pragma unroll
    for (int r = 0; r < QPT; ++r) {
      const int x = t + r * kDecThreads;
      if (x < G * D) us.q[x / D][x % D] = Elem<T>::load(qraw, r);
    }
    __syncthreads();
    if (slot == 0) {
      // the lists: chunk ids, and each head's own score, in rank order
      for (int x = t; x < K; x += kDecThreads)
        a.topk_idx[bg * K + x] = x < keep ? static_cast<int>(~static_cast<uint32_t>(ss.sorted[x])) : -1;
      for (int x = t; x < K * G; x += kDecThreads) {
        const int k = x / G, hh = x % G;
        const int c = k < keep ? static_cast<int>(~static_cast<uint32_t>(ss.sorted[k])) : -1;
        a.topk_score[(static_cast<size_t>(b) * a.Hq + g * G + hh) * K + k] =
            c >= 0 ? a.hsc[(bg * a.Cmax + c) * G + hh] : -INFINITY;
      }
    }
    float *rec = recs + static_cast<size_t>(slot) * G * (D + 2);
    const int c = slot < keep ? static_cast<int>(~static_cast<uint32_t>(ss.sorted[slot])) : -1;
    const T *kc = c < 0 ? nullptr : kv_block<T, D>(a, a.k_cache, b, g, c * a.S, t == 0);
    const T *vc = kc ? kv_block<T, D>(a, a.v_cache, b, g, c * a.S, false) : nullptr;
    if (!vc) {  // no chunk of this rank, or its page is outside the pool
      for (int hh = t; hh < G; hh += kDecThreads) publish2(rec + hh * (D + 2), -INFINITY, 0.f);
    } else {
      constexpr int NP = pairs_per_thread<D>();
      float2 ou[NP];
      attend_unit<T, D>(us, kc, vc, a.S, G, a.tau, ou);
#pragma unroll
      for (int r = 0; r < NP; ++r) {
        const int pr = t + r * kUnitThreads, hh = pr / (D / 2), e2 = pr % (D / 2);
        if (hh < G) {
          float *rh = rec + hh * (D + 2);
          const float inv = 1.f / us.l[hh];
          publish2(rh + 2 + 2 * e2, ou[r].x * inv, ou[r].y * inv);
          if (e2 == 0) publish2(rh, a.hsc[(bg * a.Cmax + c) * G + hh], 1.f);
        }
      }
    }
  }
  {
    const unsigned before = arrive(a.count + b * a.Hkv + g);
    if (t == 0) is_last = (before == static_cast<unsigned>(a.nslot_blocks - 1));
  }
  __syncthreads();
  if (!is_last) return;
  // combine every slot (chunks 0..K-1, window units K..) in slot order
  combine_slots<T, D>(recs, a.nslots, G, reinterpret_cast<float *>(us.v),
                      static_cast<T *>(a.o) + (static_cast<size_t>(b) * a.Hq + g * G) * D);
  if (t == 0) reset_counter(a.count + b * a.Hkv + g);
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
    for (int hh = t; hh < G; hh += kDecThreads) publish2(rec + hh * (D + 2), -INFINITY, 0.f);
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
        publish2(rh + 2 + 2 * e2, acc.o[r].x, acc.o[r].y);
        if (e2 == 0) publish2(rh, acc.m[r], acc.l[r]);
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
template <typename T, int D>
static hipError_t decode_t(const DecodeArgs &a, hipStream_t st) {
  if (a.r > 0) {
    decode_qcal_kernel<T, D><<<a.B, kDecThreads, 0, st>>>(
        static_cast<const T *>(a.q), static_cast<const T *>(a.h), static_cast<const T *>(a.w_down),
        static_cast<const T *>(a.w_up), a.qhat, a.Hq, a.r, a.Dh);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    decode_score_kernel<T, D, true><<<dim3(a.P + a.NW, a.Hkv, a.B), kDecThreads, 0, st>>>(a);
  } else {
    decode_score_kernel<T, D, false><<<dim3(a.P + a.NW, a.Hkv, a.B), kDecThreads, 0, st>>>(a);
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
