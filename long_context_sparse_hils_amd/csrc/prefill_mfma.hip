// Prefill hierarchical sparse attention on the MFMA units (bf16 operands,
// fp32 accumulation) -- HiLS-Attention, picx.dev summary, Methodology 2
// (Eq. 10) and 3 (query packing: M adjacent queries x G heads share the
// union of their selected chunks so that matrix tiles stay full).
//
// Workgroup = (tile of QT adjacent queries, KV head g, batch b), WAVES waves.
// Each wave owns 32 (query, head) rows = two 16-row MFMA tiles of
// 16/G queries x G heads, with fp32 output accumulators in registers.
//
// The workgroup walks a list of 64-key "items": first every chunk in the
// union of its queries' selections, then the 64-key blocks of the window
// band.  Each item's K (row-major, padded rows) and V (transposed to
// [d][key] while staging, padded rows) are staged once in LDS, double
// buffered, and shared by all waves.  Per item and row tile:
//   S^T = K Q^T           16x16x32 bf16 MFMA, keys in M, rows in N
//   chunk item:  p = softmax over the chunk's 64 keys (exact), scaled by the
//                fusion weight e^{s_hat - M_row}; rows that did not select
//                the chunk get weight 0
//   window item: online softmax (running max/sum per row) over the band,
//                masked to [n_i * S, i]
//   O^T += V^T P^T        16x16x32 bf16 MFMA, d in M, rows in N
// The key order inside S^T is permuted so that its accumulator layout is
// exactly the B-operand layout of the P^T product (no cross-lane moves).
// Row statistics start from M_row = max of the row's selected chunk scores
// and l_row = sum e^{s_hat - M_row}; one joint normaliser over chunks and
// window (Eq. 10's Z-hat_i).
#include "hils_common.h"
#include "launch.h"

namespace hils {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

constexpr int kItemKeys = 64;

template <int D, int G, int WAVES>
struct AttnCfg {
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kQPT = 16 / G;         // queries per 16-row tile
  static constexpr int kQPW = 2 * kQPT;       // queries per wave (two tiles)
  static constexpr int kQT = WAVES * kQPW;    // queries per workgroup
  static constexpr int kKS = D / 32;          // k-steps of S^T
  static constexpr int kDT = D / 16;          // d tiles of O^T
  static constexpr int kKLD = D + 8;          // padded K row (bf16)
  static constexpr int kVLD = kItemKeys + 8;  // padded V^T row (bf16)
  static constexpr int kPieces = kItemKeys * D / 8;  // 16-byte pieces per tensor per item
  static constexpr int kPPT = (kPieces + kThreads - 1) / kThreads;
};

template <int D, int G, int WAVES>
struct AttnSmem {
  using C = AttnCfg<D, G, WAVES>;
  uint16_t ks[2][kItemKeys * C::kKLD];
  uint16_t vt[2][D * C::kVLD];
  int16_t sel[C::kQT * 32];
  int16_t ulist[C::kQT * 32];
  uint32_t umask[256];
  int nunion;
};

// key held by S^T tile kt, row m (the permutation described above)
__device__ __forceinline__ int perm_key(int kt, int m) {
  return 32 * (kt >> 1) + 8 * (m >> 2) + 4 * (kt & 1) + (m & 3);
}

template <int D, int G, int WAVES>
__global__ void __launch_bounds__(WAVES * 64)
attn_prefill_mfma_kernel(AttnArgs a, int ntiles, int xcd_map) {
  using C = AttnCfg<D, G, WAVES>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  AttnSmem<D, G, WAVES> &sm = *reinterpret_cast<AttnSmem<D, G, WAVES> *>(smem_raw);

  const int T = a.T, K = a.K, S = a.S, W = a.W, Hq = a.Hq, Hkv = a.Hkv;
  const int C_chunks = T / S;
  // ---- workgroup -> (tile, g, b); heaviest (latest) tiles first, and the
  // tiles of one (b, g) on one XCD so its K/V stay in that XCD's L2
  int tile, g, b;
  {
    const int L = blockIdx.x;
    const int npairs = Hkv * a.B;
    int pair, slot;
    if (xcd_map) {
      const int xcd = L & 7, s = L >> 3;
      const int per = npairs / 8;           // pairs per XCD
      pair = xcd + 8 * (s / ntiles);
      slot = s % ntiles;
      (void)per;
    } else {
      pair = L / ntiles;
      slot = L % ntiles;
    }
    tile = ntiles - 1 - slot;
    g = pair % Hkv;
    b = pair / Hkv;
  }
  const int q0 = tile * C::kQT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;

  const uint16_t *qb = static_cast<const uint16_t *>(a.q);
  const uint16_t *kb = static_cast<const uint16_t *>(a.k) + (static_cast<size_t>(b) * Hkv + g) * T * D;
  const uint16_t *vb = static_cast<const uint16_t *>(a.v) + (static_cast<size_t>(b) * Hkv + g) * T * D;

  // ---- selection table and the union of selected chunks
  for (int x = tid; x < 256; x += C::kThreads) sm.umask[x] = 0u;
  __syncthreads();
  for (int x = tid; x < C::kQT * K; x += C::kThreads) {
    const int q = x / K, k = x % K, i = q0 + q;
    int c = -1;
    if (i < T) c = a.topk_idx[((static_cast<size_t>(b) * Hkv + g) * T + i) * K + k];
    sm.sel[q * 32 + k] = static_cast<int16_t>(c);
    if (c >= 0) atomicOr(&sm.umask[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  if (wave == 0) {
    const int nwords = (C_chunks + 31) >> 5;
    int base = 0;
    for (int w0 = 0; w0 < nwords; w0 += 64) {
      const int w = w0 + lane;
      const uint32_t bits = w < nwords ? sm.umask[w] : 0u;
      const int cnt = __popc(bits);
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      int pos = base + incl - cnt;
      uint32_t bb = bits;
      while (bb) {
        const int bit = __ffs(bb) - 1;
        bb &= bb - 1;
        sm.ulist[pos++] = static_cast<int16_t>(w * 32 + bit);
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) sm.nunion = base;
  }
  __syncthreads();
  const int nunion = sm.nunion;

  // window band of the tile: 64-key blocks from n_{first} * S to the last query
  const int i_first = q0, i_last = min(q0 + C::kQT - 1, T - 1);
  const int jw0 = eligible_chunks(i_first, W, S) * S;
  const int nwin = (i_last - jw0) / kItemKeys + 1;
  const int nitems = nunion + nwin;

  // ---- per-lane row identity for the two tiles
  int row_q[2], row_h[2];
  bool row_ok[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int q = wave * C::kQPW + t * C::kQPT + ln / G;
    row_q[t] = q;
    row_h[t] = g * G + (ln % G);
    row_ok[t] = (q0 + q) < T;
  }

  // ---- Q operands (B of S^T = K Q^T): lane holds row ln, d = 32 ks + 8 lg .. +8
  bf16x8 qop[2][C::kKS];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = q0 + row_q[t];
    const size_t qo = ((static_cast<size_t>(b) * Hq + row_h[t]) * T + (row_ok[t] ? i : 0)) * D;
#pragma unroll
    for (int s = 0; s < C::kKS; ++s) {
      uint4 u = row_ok[t] ? *reinterpret_cast<const uint4 *>(qb + qo + 32 * s + 8 * lg) : make_uint4(0, 0, 0, 0);
      qop[t][s] = as_bf16x8(u);
    }
  }

  // ---- row statistics from the selected chunk scores
  float m_row[2], l_row[2];
  f32x4 acc[2][C::kDT];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float mx = -INFINITY;
    const size_t so = ((static_cast<size_t>(b) * Hq + row_h[t]) * T + (q0 + row_q[t])) * K;
    if (row_ok[t])
      for (int k = 0; k < K; ++k)
        if (sm.sel[row_q[t] * 32 + k] >= 0) mx = fmaxf(mx, a.topk_score[so + k]);
    float l = 0.f;
    if (row_ok[t] && mx != -INFINITY)
      for (int k = 0; k < K; ++k)
        if (sm.sel[row_q[t] * 32 + k] >= 0) l += __expf(a.topk_score[so + k] - mx);
    m_row[t] = mx;
    l_row[t] = l;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) acc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- staging: item x -> LDS buffer
  auto item_key0 = [&](int x) -> int {
    return x < nunion ? static_cast<int>(sm.ulist[x]) * S : jw0 + (x - nunion) * kItemKeys;
  };
  uint4 pk[C::kPPT], pv[C::kPPT];
  auto fetch = [&](int x) {
    const int j0 = item_key0(x);
#pragma unroll
    for (int r = 0; r < C::kPPT; ++r) {
      const int p = tid + r * C::kThreads;
      const int key = p / (D / 8), seg = p % (D / 8);
      const bool ok = p < C::kPieces && (j0 + key) < T;
      const size_t off = static_cast<size_t>(j0 + key) * D + seg * 8;
      pk[r] = ok ? *reinterpret_cast<const uint4 *>(kb + off) : make_uint4(0, 0, 0, 0);
      pv[r] = ok ? *reinterpret_cast<const uint4 *>(vb + off) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int r = 0; r < C::kPPT; ++r) {
      const int p = tid + r * C::kThreads;
      if (p < C::kPieces) {
        const int key = p / (D / 8), seg = p % (D / 8);
        *reinterpret_cast<uint4 *>(&sm.ks[buf][key * C::kKLD + seg * 8]) = pk[r];
        const uint32_t w4[4] = {pv[r].x, pv[r].y, pv[r].z, pv[r].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.vt[buf][(seg * 8 + 2 * e) * C::kVLD + key] = static_cast<uint16_t>(w4[e] & 0xFFFFu);
          sm.vt[buf][(seg * 8 + 2 * e + 1) * C::kVLD + key] = static_cast<uint16_t>(w4[e] >> 16);
        }
      }
    }
  };

  if (nitems > 0) {
    fetch(0);
    stage(0);
  }
  __syncthreads();

  const float tau = a.tau;
  for (int x = 0; x < nitems; ++x) {
    const int buf = x & 1;
    if (x + 1 < nitems) fetch(x + 1);
    const bool is_chunk = x < nunion;
    const int j0 = item_key0(x);
    const int chunk = j0 / S;
    const uint16_t *ksb = sm.ks[buf];
    const uint16_t *vtb = sm.vt[buf];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // which rows take part
      int slot = -1;
      int lo = 0, hi = -1;  // valid key range of this row (window items)
      if (is_chunk) {
        if (row_ok[t])
          for (int k = 0; k < K; ++k)
            if (sm.sel[row_q[t] * 32 + k] == chunk) slot = k;
      } else if (row_ok[t]) {
        const int i = q0 + row_q[t];
        lo = max(j0, eligible_chunks(i, W, S) * S);
        hi = min(j0 + kItemKeys - 1, i);
      }
      const bool mine = is_chunk ? (slot >= 0) : (lo <= hi);
      if (__ballot(mine) == 0ull) continue;  // wave-uniform skip
      float alpha = -INFINITY;  // this row's fusion score for the chunk
      if (slot >= 0)
        alpha = a.topk_score[((static_cast<size_t>(b) * Hq + row_h[t]) * T + (q0 + row_q[t])) * K + slot];

      // S^T = K Q^T over the item's 64 keys (4 tiles of 16 keys)
      f32x4 st[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t *krow = ksb + perm_key(kt, ln) * C::kKLD + 8 * lg;
#pragma unroll
        for (int s = 0; s < C::kKS; ++s) {
          const uint4 u = *reinterpret_cast<const uint4 *>(krow + 32 * s);
          st[kt] = mfma16(as_bf16x8(u), qop[t][s], st[kt]);
        }
      }
      // softmax pieces: this lane holds keys perm_key(kt, 4 lg + i) of row ln
      float p[4][4];
      if (is_chunk) {
        float mc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) { p[kt][i] = tau * st[kt][i]; mc = fmaxf(mc, p[kt][i]); }
        mc = fmaxf(mc, __shfl_xor(mc, 16, 64));
        mc = fmaxf(mc, __shfl_xor(mc, 32, 64));
        float lc = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) { p[kt][i] = __expf(p[kt][i] - mc); lc += p[kt][i]; }
        lc += __shfl_xor(lc, 16, 64);
        lc += __shfl_xor(lc, 32, 64);
        const float w = (slot >= 0) ? __expf(alpha - m_row[t]) / lc : 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[kt][i] *= w;
      } else {
        float mb = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = j0 + perm_key(kt, 4 * lg + i);
            const float s = (j >= lo && j <= hi) ? tau * st[kt][i] : -INFINITY;
            p[kt][i] = s;
            mb = fmaxf(mb, s);
          }
        mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
        const float mn = fmaxf(m_row[t], mb);
        float ls = 0.f;
        if (mn == -INFINITY) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) p[kt][i] = 0.f;
        } else {
          const float sc = (m_row[t] == -INFINITY) ? 0.f : __expf(m_row[t] - mn);
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              p[kt][i] = (p[kt][i] == -INFINITY) ? 0.f : __expf(p[kt][i] - mn);
              ls += p[kt][i];
            }
          ls += __shfl_xor(ls, 16, 64);
          ls += __shfl_xor(ls, 32, 64);
          if (sc != 1.f) {
#pragma unroll
            for (int dt = 0; dt < C::kDT; ++dt) acc[t][dt] *= sc;
          }
          l_row[t] = l_row[t] * sc + ls;
          m_row[t] = mn;
        }
      }
      // P^T as the B operand: k-slot sl holds keys 32 sl + 8 lg .. +8
      bf16x8 pb[2];
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        uint4 u;
        u.x = pack_bf16x2(p[2 * sl][0], p[2 * sl][1]);
        u.y = pack_bf16x2(p[2 * sl][2], p[2 * sl][3]);
        u.z = pack_bf16x2(p[2 * sl + 1][0], p[2 * sl + 1][1]);
        u.w = pack_bf16x2(p[2 * sl + 1][2], p[2 * sl + 1][3]);
        pb[sl] = as_bf16x8(u);
      }
      // O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt) {
        const uint16_t *vrow = vtb + (16 * dt + ln) * C::kVLD + 8 * lg;
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const uint4 u = *reinterpret_cast<const uint4 *>(vrow + 32 * sl);
          acc[t][dt] = mfma16(as_bf16x8(u), pb[sl], acc[t][dt]);
        }
      }
    }
    // buffer buf ^ 1 was last read while computing item x-1, which every
    // thread finished before the barrier that ended that iteration
    if (x + 1 < nitems) stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: o = acc / l, lane holds d = 16 dt + 4 lg + (0..3) of row ln
  uint16_t *ob = static_cast<uint16_t *>(a.o);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (!row_ok[t]) continue;
    const float inv = 1.f / l_row[t];
    const size_t oo = ((static_cast<size_t>(b) * Hq + row_h[t]) * T + (q0 + row_q[t])) * D;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) {
      uint2 w;
      w.x = pack_bf16x2(acc[t][dt][0] * inv, acc[t][dt][1] * inv);
      w.y = pack_bf16x2(acc[t][dt][2] * inv, acc[t][dt][3] * inv);
      *reinterpret_cast<uint2 *>(ob + oo + 16 * dt + 4 * lg) = w;
    }
  }
}

template <int D, int G>
static hipError_t attn_mfma_t(const AttnArgs &a, hipStream_t st) {
  constexpr int WAVES = 8;
  using C = AttnCfg<D, G, WAVES>;
  const int ntiles = (a.T + C::kQT - 1) / C::kQT;
  const int npairs = a.Hkv * a.B;
  const int xcd_map = (npairs % 8 == 0) ? 1 : 0;
  const size_t smem = sizeof(AttnSmem<D, G, WAVES>);
  auto kern = attn_prefill_mfma_kernel<D, G, WAVES>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  kern<<<dim3(ntiles * npairs), C::kThreads, smem, st>>>(a, ntiles, xcd_map);
  return hipGetLastError();
}

bool attn_mfma_supported(const AttnArgs &a) {
  const int G = a.Hq / a.Hkv;
  return a.bf16 && (a.d == 64 || a.d == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) &&
         a.S == kItemKeys && a.K <= 32 && a.T / a.S <= 8192;
}

hipError_t launch_attn_mfma(const AttnArgs &a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
#define HILS_ATTN_CASE(DD, GG) \
  if (a.d == DD && G == GG) return attn_mfma_t<DD, GG>(a, st);
  HILS_ATTN_CASE(128, 4) HILS_ATTN_CASE(128, 1) HILS_ATTN_CASE(128, 2) HILS_ATTN_CASE(128, 8)
  HILS_ATTN_CASE(128, 16) HILS_ATTN_CASE(64, 4) HILS_ATTN_CASE(64, 1) HILS_ATTN_CASE(64, 2)
  HILS_ATTN_CASE(64, 8) HILS_ATTN_CASE(64, 16)
#undef HILS_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace hils
