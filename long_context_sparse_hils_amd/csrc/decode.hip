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
struct D1Smem {
  union {
    struct {
      float qh[kMaxG * 128];
      float s[1024 * 4];  // per (chunk, head) scores of the slice; CPB*G <= 4096
      float sig[1024];
    } sc;
    unsigned long long cand[kMaxCand];
  };
  unsigned long long red[4];
  int redx[4];
  int is_last;
};

// a score-slice block and a window-unit block never need both layouts
template <int D>
union D1Shared {
  D1Smem sc;
  UnitSmem<D> us;
};

template <typename T, int D, bool QCAL>
__global__ void __launch_bounds__(kDecThreads)
decode_score_kernel(DecodeArgs a) {
  __shared__ D1Shared<D> shm;
  D1Smem &sm = shm.sc;
  UnitSmem<D> &us = shm.us;
  const int g = blockIdx.y, b = blockIdx.z, blk = blockIdx.x, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
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

  // ---------------- score slice
  const int c0 = blk * a.CPB;
  const int c1 = min(c0 + a.CPB, n);
  const int nch = max(0, c1 - c0);
  for (int x = t; x < G * D; x += kDecThreads) {
    const size_t qo = (static_cast<size_t>(b) * a.Hq + g * G) * D + x;
    sm.sc.qh[x] = QCAL ? a.qhat[qo] : Elem<T>::load(static_cast<const T *>(a.q), qo);
  }
  __syncthreads();
  {
    constexpr int LPH = D / 8;      // lanes per (chunk, head) row
    constexpr int R = 64 / LPH;     // rows per wave load
    const int nrows = nch * G;
    const int seg = lane % LPH;
    const T *ks = static_cast<const T *>(a.k_sum);
    const size_t hbase = static_cast<size_t>(b) * a.Hq + g * G;
    constexpr int UN = 4;  // wave loads in flight per iteration
    for (int row0 = wave * R; row0 < nrows; row0 += 4 * R * UN) {
      float part[UN];
      int rows[UN];
#pragma unroll
      for (int uu = 0; uu < UN; ++uu) {
        const int row = row0 + uu * 4 * R + lane / LPH;
        rows[uu] = row;
        part[uu] = 0.f;
        if (row < nrows) {
          const int cl = row / G, hh = row % G;
          float kv[8];
          Elem<T>::load8(ks + ((hbase + hh) * a.Cmax + c0 + cl) * D + seg * 8, kv);
          const float *qv = sm.sc.qh + hh * D + seg * 8;
#pragma unroll
          for (int x = 0; x < 8; ++x) part[uu] += qv[x] * kv[x];
        }
      }
#pragma unroll
      for (int uu = 0; uu < UN; ++uu) {
        const float dot = group_sum<LPH>(part[uu]);
        const int row = rows[uu];
        if (seg == 0 && row < nrows) {
          const int cl = row / G, hh = row % G;
          sm.sc.s[row] = a.tau * dot + a.b_sum[(hbase + hh) * a.Cmax + c0 + cl];
        }
      }
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
  if (wave == 0) {
    const int keep = min(K, nch);
    unsigned long long prev = ~0ull;
    for (int k = 0; k < K; ++k) {
      unsigned long long best = kNoKey;
      if (k < keep) {
        for (int cl = lane; cl < nch; cl += 64) {
          const unsigned long long key = make_key(sm.sc.sig[cl], c0 + cl);
          if (key < prev && key > best) best = key;
        }
        best = wave_max_u64(best);
        prev = best;
      }
      if (lane == 0) publish(a.cand_key + cbase + k, best);
      if (best != kNoKey) {
        const int cl = key_chunk(best) - c0;
        for (int hh = lane; hh < G; hh += 64) publish(a.cand_s + (cbase + k) * G + hh, sm.sc.s[cl * G + hh]);
      }
    }
  }
  // ---------------- ticket: the last slice block of (b, g) merges
  {
    const unsigned before = arrive(a.count1 + b * a.Hkv + g);
    if (t == 0) sm.is_last = (before == static_cast<unsigned>(a.P - 1));
  }
  __syncthreads();
  if (!sm.is_last) return;
  const int total = a.P * K;
  const size_t cb0 = (static_cast<size_t>(b) * a.Hkv + g) * a.P * K;
  for (int x = t; x < total; x += kDecThreads) sm.cand[x] = load_acquired(a.cand_key + cb0 + x);
  __syncthreads();
  const int keep = min(K, n);
  unsigned long long prev = ~0ull;
  for (int k = 0; k < K; ++k) {
    if (k < keep) {
      unsigned long long best = kNoKey;
      int bx = -1;
      for (int x = t; x < total; x += kDecThreads) {
        const unsigned long long key = sm.cand[x];
        if (key < prev && key > best) { best = key; bx = x; }
      }
      unsigned long long wb = wave_max_u64(best);
      const unsigned long long ball = __ballot(best == wb && bx >= 0);
      const int src = ball ? __ffsll(static_cast<long long>(ball)) - 1 : 0;
      const int wx = __shfl(bx, src, 64);
      if (lane == 0) { sm.red[wave] = wb; sm.redx[wave] = wx; }
      __syncthreads();
      unsigned long long bb = sm.red[0];
      int bbx = sm.redx[0];
      for (int w = 1; w < kDecThreads / 64; ++w)
        if (sm.red[w] > bb) { bb = sm.red[w]; bbx = sm.redx[w]; }
      prev = bb;
      const int c = key_chunk(bb);
      if (t == 0) a.topk_idx[(static_cast<size_t>(b) * a.Hkv + g) * K + k] = c;
      for (int hh = t; hh < G; hh += kDecThreads)
        a.topk_score[(static_cast<size_t>(b) * a.Hq + g * G + hh) * K + k] =
            load_acquired(a.cand_s + (cb0 + bbx) * G + hh);
      __syncthreads();
    } else {
      if (t == 0) a.topk_idx[(static_cast<size_t>(b) * a.Hkv + g) * K + k] = -1;
      for (int hh = t; hh < G; hh += kDecThreads)
        a.topk_score[(static_cast<size_t>(b) * a.Hq + g * G + hh) * K + k] = -INFINITY;
    }
  }
  if (t == 0) reset_counter(a.count1 + b * a.Hkv + g);
}

// ------------------------------------------------------------------ D2
template <typename T, int D>
__global__ void __launch_bounds__(kDecThreads)
decode_attend_kernel(DecodeArgs a) {
  __shared__ UnitSmem<D> us;
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
  for (int x = t; x < G * D; x += kDecThreads) {
    const int hh = x / D, e = x % D;
    float m = -INFINITY, l = 0.f, o = 0.f;
    for (int s = 0; s < a.nslots; ++s) {
      const float *rh = recs + (static_cast<size_t>(s) * G + hh) * (D + 2);
      const float m2 = load_acquired(rh);
      if (m2 == -INFINITY) continue;
      const float l2 = load_acquired(rh + 1);
      const float o2 = load_acquired(rh + 2 + e);
      const float mn = fmaxf(m, m2);
      const float sa = (m == -INFINITY) ? 0.f : __expf(m - mn), sb = __expf(m2 - mn);
      o = o * sa + o2 * sb;
      l = l * sa + l2 * sb;
      m = mn;
    }
    Elem<T>::store(static_cast<T *>(a.o), (static_cast<size_t>(b) * a.Hq + g * G + hh) * D + e, o / l);
  }
  if (t == 0) reset_counter(a.count2 + b * a.Hkv + g);
}

// ------------------------------------------------------------------ dense comparator
template <typename T, int D>
__global__ void __launch_bounds__(kDecThreads)
dense_decode_kernel(DenseArgs a) {
  __shared__ UnitSmem<D> us;
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
  for (int x = t; x < G * D; x += kDecThreads) {
    const int hh = x / D, e = x % D;
    float m = -INFINITY, l = 0.f, o = 0.f;
    for (int s = 0; s < a.P; ++s) {
      const float *rh = recs + (static_cast<size_t>(s) * G + hh) * (D + 2);
      const float m2 = load_acquired(rh);
      if (m2 == -INFINITY) continue;
      const float l2 = load_acquired(rh + 1);
      const float o2 = load_acquired(rh + 2 + e);
      const float mn = fmaxf(m, m2);
      const float sa = (m == -INFINITY) ? 0.f : __expf(m - mn), sb = __expf(m2 - mn);
      o = o * sa + o2 * sb;
      l = l * sa + l2 * sb;
      m = mn;
    }
    Elem<T>::store(static_cast<T *>(a.o), (static_cast<size_t>(b) * a.Hq + g * G + hh) * D + e, o / l);
  }
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
