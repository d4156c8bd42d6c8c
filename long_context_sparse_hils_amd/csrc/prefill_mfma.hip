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


constexpr int kItemKeys = 64;

template <int D, int G, int WAVES, int TPW>
struct AttnCfg {
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kQPT = 16 / G;         // queries per 16-row tile
  static constexpr int kQPW = TPW * kQPT;     // queries per wave (TPW tiles)
  static constexpr int kQT = WAVES * kQPW;    // queries per workgroup
  static constexpr int kKS = D / 32;          // k-steps of S^T
  static constexpr int kDT = D / 16;          // d tiles of O^T
  // K rows: D=128 unpadded with pieces XOR-swizzled (conflict-free operand
  // reads); D=64 padded rows
  static constexpr bool kSwz = (D == 128);
  static constexpr int kKLD = kSwz ? D : D + 8;
  static constexpr int kVLD = kItemKeys + 8;  // padded V^T row (bf16)
  static constexpr int kPieces = kItemKeys * D / 8;  // 16-byte pieces per tensor per item
  static constexpr int kPPT = (kPieces + kThreads - 1) / kThreads;
};

template <int D, int G, int WAVES, int TPW>
struct AttnSmem {
  using C = AttnCfg<D, G, WAVES, TPW>;
  uint16_t ks[2][kItemKeys * C::kKLD];
  uint16_t vt[2][D * C::kVLD];
  int16_t sel[32 * C::kQT];       // [slot][query]: selected chunk, -1 if none
  int16_t ulist[C::kQT * 32];
  float alpha[C::kQT * 32 * G];    // fusion score of (query, slot, head)
  int8_t slot_tab[2][C::kQT];      // per staged item: slot of its chunk in each query's selection, or -1
  float alpha_tab[2][C::kQT * G];  // per staged item: each (query, head)'s fusion score for it
  uint32_t umask[256];
  int nunion;
};

// key held by S^T tile kt, row m (the permutation described above)
__device__ __forceinline__ int perm_key(int kt, int m) {
  return 32 * (kt >> 1) + 8 * (m >> 2) + 4 * (kt & 1) + (m & 3);
}

// 16-byte piece pc of K row r is stored at piece pc ^ swz(r): the 16 rows
// one MFMA operand read touches ({0..3, 8..11, 16..19, 24..27} + const) then
// fall in 16 different bank groups.
__device__ __forceinline__ int k_swz(int r) { return (r & 3) | ((r >> 1) & 12); }

template <bool SWZ, int KLD>
__device__ __forceinline__ int k_off(int r, int pc) {
  return SWZ ? r * KLD + ((pc ^ k_swz(r)) << 3) : r * KLD + (pc << 3);
}

template <int D, int G, int WAVES, int TPW>
__global__ void __launch_bounds__(WAVES * 64)
attn_prefill_mfma_kernel(AttnArgs a, int ntiles, int xcd_map) {
  using C = AttnCfg<D, G, WAVES, TPW>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  AttnSmem<D, G, WAVES, TPW> &sm = *reinterpret_cast<AttnSmem<D, G, WAVES, TPW> *>(smem_raw);

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
    sm.sel[k * C::kQT + q] = static_cast<int16_t>(c);
    if (c >= 0) atomicOr(&sm.umask[c >> 5], 1u << (c & 31));
    for (int hh = 0; hh < G; ++hh)
      sm.alpha[(q * 32 + k) * G + hh] =
          c >= 0 ? a.topk_score[((static_cast<size_t>(b) * Hq + g * G + hh) * T + i) * K + k] : -INFINITY;
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
  int row_q[TPW], row_h[TPW];
  bool row_ok[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int q = wave * C::kQPW + t * C::kQPT + ln / G;
    row_q[t] = q;
    row_h[t] = g * G + (ln % G);
    row_ok[t] = (q0 + q) < T;
  }

  // ---- Q operands (B of S^T = K Q^T): lane holds row ln, d = 32 ks + 8 lg .. +8
  bf16x8 qop[TPW][C::kKS];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int i = q0 + row_q[t];
    const size_t qo = ((static_cast<size_t>(b) * Hq + row_h[t]) * T + (row_ok[t] ? i : 0)) * D;
#pragma unroll
    for (int s = 0; s < C::kKS; ++s) {
      uint4 u = row_ok[t] ? *reinterpret_cast<const uint4 *>(qb + qo + 32 * s + 8 * lg) : make_uint4(0, 0, 0, 0);
      qop[t][s] = as_bf16x8(u);
    }
  }

  // ---- row statistics from the selected chunk scores
  float m_row[TPW], l_row[TPW];
  f32x4 acc[TPW][C::kDT];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float mx = -INFINITY;
    const int hh = ln % G;
    if (row_ok[t])
      for (int k = 0; k < K; ++k)
        if (sm.sel[k * C::kQT + row_q[t]] >= 0) mx = fmaxf(mx, sm.alpha[(row_q[t] * 32 + k) * G + hh]);
    float l = 0.f;
    if (row_ok[t] && mx != -INFINITY)
      for (int k = 0; k < K; ++k)
        if (sm.sel[k * C::kQT + row_q[t]] >= 0) l += __expf(sm.alpha[(row_q[t] * 32 + k) * G + hh] - mx);
    m_row[t] = mx;
    l_row[t] = l;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) acc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- staging: item x -> LDS buffer
  auto item_key0 = [&](int x) -> int {
    return x < nunion ? static_cast<int>(sm.ulist[x]) * S : jw0 + (x - nunion) * kItemKeys;
  };
  // K: thread -> 16-byte pieces (key, piece) row-major; V: thread -> a pair
  // of keys x one 8-element piece, so the transposed [d][key] tile is written
  // with conflict-free 32-bit stores (one per d).
  constexpr int kVPairs = kItemKeys / 2 * (D / 8);          // (key pair, piece) units
  constexpr int kVPT = (kVPairs + C::kThreads - 1) / C::kThreads;
  uint4 pk[C::kPPT], pv[kVPT][2];
  auto fetch = [&](int x) {
    const int j0 = item_key0(x);
#pragma unroll
    for (int r = 0; r < C::kPPT; ++r) {
      const int p = tid + r * C::kThreads;
      const int key = p / (D / 8), seg = p % (D / 8);
      const bool ok = p < C::kPieces && (j0 + key) < T;
      pk[r] = ok ? *reinterpret_cast<const uint4 *>(kb + static_cast<size_t>(j0 + key) * D + seg * 8)
                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < kVPT; ++r) {
      const int p = tid + r * C::kThreads;
      const int kp = p % (kItemKeys / 2), seg = p / (kItemKeys / 2);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int key = 2 * kp + h2;
        const bool ok = p < kVPairs && (j0 + key) < T;
        pv[r][h2] = ok ? *reinterpret_cast<const uint4 *>(vb + static_cast<size_t>(j0 + key) * D + seg * 8)
                       : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // slot of item x's chunk in each query's selection (chunk items only)
  auto build_slots = [&](int x, int buf) {
    if (x < nunion) {
      const int c = sm.ulist[x];
      for (int q = tid; q < C::kQT; q += C::kThreads) {
        int sl = -1;
        for (int k = 0; k < K; ++k)
          if (sm.sel[k * C::kQT + q] == c) sl = k;
        sm.slot_tab[buf][q] = static_cast<int8_t>(sl);
        for (int hh = 0; hh < G; ++hh)
          sm.alpha_tab[buf][q * G + hh] = sl >= 0 ? sm.alpha[(q * 32 + sl) * G + hh] : -INFINITY;
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int r = 0; r < C::kPPT; ++r) {
      const int p = tid + r * C::kThreads;
      if (p < C::kPieces) {
        const int key = p / (D / 8), seg = p % (D / 8);
        *reinterpret_cast<uint4 *>(&sm.ks[buf][k_off<C::kSwz, C::kKLD>(key, seg)]) = pk[r];
      }
    }
#pragma unroll
    for (int r = 0; r < kVPT; ++r) {
      const int p = tid + r * C::kThreads;
      if (p < kVPairs) {
        const int kp = p % (kItemKeys / 2), seg = p / (kItemKeys / 2);
        const uint32_t a0[4] = {pv[r][0].x, pv[r][0].y, pv[r][0].z, pv[r][0].w};
        const uint32_t a1[4] = {pv[r][1].x, pv[r][1].y, pv[r][1].z, pv[r][1].w};
        uint32_t *vt32 = reinterpret_cast<uint32_t *>(sm.vt[buf]) + ((seg * 8 * C::kVLD + 2 * kp) >> 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // d = seg*8 + 2e: low halves of the two keys; d + 1: high halves
          vt32[(2 * e * C::kVLD) >> 1] = __builtin_amdgcn_perm(a1[e], a0[e], 0x05040100u);
          vt32[((2 * e + 1) * C::kVLD) >> 1] = __builtin_amdgcn_perm(a1[e], a0[e], 0x07060302u);
        }
      }
    }
  };

  if (nitems > 0) {
    fetch(0);
    stage(0);
    build_slots(0, 0);
  }
  __syncthreads();

  // per-lane LDS offsets of the S^T A operand (K rows).  For the permuted
  // key rows the XOR swizzle of row perm_key(kt, ln) is ln itself, so only
  // the key-tile term depends on kt (a compile-time constant).
  int koffb[C::kKS];
#pragma unroll
  for (int s = 0; s < C::kKS; ++s) {
    const int r0 = 8 * (ln >> 2) + (ln & 3);
    koffb[s] = C::kSwz ? r0 * C::kKLD + (((4 * s + lg) ^ ln) << 3) : r0 * C::kKLD + ((4 * s + lg) << 3);
  }

  const float tau = a.tau;
  const float tl2e = tau * 1.4426950408889634f;  // tau * log2(e)
  for (int x = 0; x < nitems; ++x) {
    const int buf = x & 1;
    if (x + 1 < nitems) fetch(x + 1);
    const bool is_chunk = x < nunion;
    const int j0 = item_key0(x);
    const uint16_t *ksb = sm.ks[buf];
    const uint16_t *vtb = sm.vt[buf];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      // which rows take part
      int slot = -1;
      int lo = 0, hi = -1;  // valid key range of this row (window items)
      if (is_chunk) {
        if (row_ok[t]) slot = sm.slot_tab[buf][row_q[t]];
      } else if (row_ok[t]) {
        const int i = q0 + row_q[t];
        lo = max(j0, eligible_chunks(i, W, S) * S);
        hi = min(j0 + kItemKeys - 1, i);
      }
      const bool mine = is_chunk ? (slot >= 0) : (lo <= hi);
      if (__ballot(mine) == 0ull) continue;  // wave-uniform skip
      float alpha = -INFINITY;  // this row's fusion score for the chunk
      if (slot >= 0) alpha = sm.alpha_tab[buf][row_q[t] * G + (ln % G)];

      // S^T = K Q^T over the item's 64 keys (4 tiles of 16 keys)
      f32x4 st[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // k-step outer, key tile inner; the scheduling barriers keep the
      // compiler from hoisting every operand load (register pressure)
#pragma unroll
      for (int s = 0; s < C::kKS; ++s) {
        uint4 u[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          u[kt] = *reinterpret_cast<const uint4 *>(ksb + koffb[s] + (32 * (kt >> 1) + 4 * (kt & 1)) * C::kKLD);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) st[kt] = mfma16(as_bf16x8(u[kt]), qop[t][s], st[kt]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // softmax pieces: this lane holds keys perm_key(kt, 4 lg + i) of row ln
      float p[4][4];
      if (is_chunk) {
        // exact softmax over the chunk's 64 keys: e = 2^{(s - max) tau log2 e}
        float mc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mc = fmaxf(mc, st[kt][i]);
        mc = fmaxf(mc, __shfl_xor(mc, 16, 64));
        mc = fmaxf(mc, __shfl_xor(mc, 32, 64));
        const float off = -mc * tl2e;
        float lc = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) { p[kt][i] = __builtin_amdgcn_exp2f(fmaf(st[kt][i], tl2e, off)); lc += p[kt][i]; }
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
          const float off = -mn * 1.4426950408889634f;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              p[kt][i] = (p[kt][i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(fmaf(p[kt][i], 1.4426950408889634f, off));
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
      for (int dt = 0; dt < C::kDT; dt += 2) {
        uint4 u[2][2];
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
          for (int sl = 0; sl < 2; ++sl)
            u[d2][sl] = *reinterpret_cast<const uint4 *>(vtb + (16 * (dt + d2) + ln) * C::kVLD + 8 * lg + 32 * sl);
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) acc[t][dt + d2] = mfma16(as_bf16x8(u[d2][sl]), pb[sl], acc[t][dt + d2]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // buffer buf ^ 1 was last read while computing item x-1, which every
    // thread finished before the barrier that ended that iteration
    if (x + 1 < nitems) {
      stage(buf ^ 1);
      build_slots(x + 1, buf ^ 1);
    }
    __syncthreads();
  }

  // ---- epilogue: o = acc / l, lane holds d = 16 dt + 4 lg + (0..3) of row ln
  uint16_t *ob = static_cast<uint16_t *>(a.o);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
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
  constexpr int WAVES = 8, TPW = 2;
  using C = AttnCfg<D, G, WAVES, TPW>;
  const int ntiles = (a.T + C::kQT - 1) / C::kQT;
  const int npairs = a.Hkv * a.B;
  const int xcd_map = (npairs % 8 == 0) ? 1 : 0;
  const size_t smem = sizeof(AttnSmem<D, G, WAVES, TPW>);
  auto kern = attn_prefill_mfma_kernel<D, G, WAVES, TPW>;
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
