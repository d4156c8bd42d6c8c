// Sliding-window term of the prefill hierarchical sparse attention on the
// MFMA units (bf16 operands, fp32 accumulation), and its fusion with the
// chunk terms -- HiLS-Attention, picx.dev summary, Methodology 2 (Eq. 10:
// one joint normaliser over the selected chunks and the window tokens).
//
// The chunk terms run first (prefill_chunks.hip): they leave in o each
// row's chunk part normalised by its chunk mass, and the chunk log-mass
// lse_C in the workspace.  This pass computes the window term of every row
// and combines the two.
//
// Workgroup = (32 consecutive queries, KV head g, batch b), 4 waves (one per
// SIMD) in under 80 KB of LDS, so that two workgroups share a CU and fill
// each other's barrier waits and softmax phases with MFMA work.  Each wave
// owns 32 (query, head) rows = two 16-row MFMA tiles of 16/G adjacent
// queries x G heads, with fp32 output accumulators in registers.  The
// workgroup walks the 64-key blocks of its window band: each block's K and
// V^T, in the MFMA operand order that one pass per call writes (every
// operand read is one wave-wide 1 KB piece), are staged in LDS straight from
// global memory, double buffered, and shared by all waves; each wave runs
// the tiles whose rows overlap the block:
//   S^T = K Q^T           16x16x32 bf16 MFMA, keys in M, rows in N
//   softmax against the row's reference maximum, masked to [n_i * S, i]
//                         only on blocks that cross a row's window edge
//   O^T += V^T P^T        16x16x32 bf16 MFMA, d in M, rows in N
// The key order inside S^T is permuted so that its accumulator layout is
// exactly the B-operand layout of the P^T product (no cross-lane moves):
// row m of S^T tile kt holds key 32 (kt >> 1) + 8 (m >> 2) + 4 (kt & 1) +
// (m & 3), the order in which the operand-order pass lays out K.
// A block moves the reference only when its own maximum exceeds it by more
// than kLazyRescale; numerator and denominator always share the reference,
// so the result does not depend on when it moves.
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
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyRescale = 8.f;  // natural-log units: probabilities stay below e^8

template <int D, int G, int WAVES, int TPW>
struct AttnCfg {
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kQPT = 16 / G;         // queries per 16-row tile
  static constexpr int kQPW = TPW * kQPT;     // queries per wave (TPW tiles)
  static constexpr int kQT = WAVES * kQPW;    // queries per workgroup
  static constexpr int kKS = D / 32;          // k-steps of S^T
  static constexpr int kDT = D / 16;          // d tiles of O^T
  static constexpr int kRowPieces = D / 8;    // 16-byte pieces per K row
  // one staged block = the K and V^T pieces of the operand order (1 KB each,
  // K pieces first), loaded straight into LDS
  static constexpr int kPiecesK = 4 * kKS, kPiecesV = 2 * kDT;
  static constexpr int kLoadsK = kPiecesK / WAVES;
  static constexpr int kLoadsV = kPiecesV / WAVES;
  static_assert(kLoadsK * WAVES == kPiecesK && kLoadsV * WAVES == kPiecesV, "pieces must split evenly over the waves");
};

template <int D, int G, int WAVES, int TPW>
struct AttnSmem {
  uint16_t ks[2][kItemKeys * D];   // K pieces in operand order (piece kt * D/32 + s at 512 kt + ...)
  uint16_t vt[2][D * kItemKeys];   // V^T pieces in operand order (piece 2 dt + sl)
};

// ------------------------------------------------------------------ one item
// Per-lane state of a wave's row tiles.
template <int D, int TPW>
struct RowState {
  bf16x8 qop[TPW][D / 32];   // Q as the B operand of S^T: row ln, d = 32 s + 8 lg .. +8
  f32x4 acc[TPW][D / 16];    // O^T: lane holds d = 16 dt + 4 lg + (0..3) of row ln
  float m_row[TPW], l_row[TPW];
};

// S^T = K Q^T of one 16-row tile; the operands of k-step s + 1 are read
// while the MFMAs of step s run, and the scheduling barrier keeps later reads
// from being hoisted further (registers).
template <int D>
__device__ __forceinline__ void tile_scores(const bf16x8 (&qop)[D / 32], const uint16_t *ksb, int lane8,
                                            f32x4 (&st)[4]) {
  constexpr int KS = D / 32;
  uint4 u[2][4];
  auto load_k = [&](uint4 (&dst)[4], int s) {  // K piece kt * KS + s
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) dst[kt] = *reinterpret_cast<const uint4 *>(ksb + (kt * KS + s) * 512 + lane8);
  };
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  load_k(u[0], 0);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (s + 1 < KS) load_k(u[(s + 1) & 1], s + 1);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) st[kt] = mfma16(as_bf16x8(u[s & 1][kt]), qop[s], st[kt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Softmax of one tile's S^T into the bf16 P^T operand (this lane holds keys
// 32 (kt >> 1) + 8 lg + 4 (kt & 1) + i of row ln) against the row's
// reference maximum m_row; when MASKED, only the lane's keys whose offset
// from 8 lg is at most lim count (see the window limit below).  The reference moves to
// the block's maximum only when that exceeds it by more than kLazyRescale,
// and the returned factor (1 otherwise) rescales the row's accumulator.
template <bool MASKED>
__device__ __forceinline__ float tile_softmax(const f32x4 (&st)[4], bf16x8 (&pb)[2], float &m_row, float &l_row,
                                              int lim, float tau, float tl2e) {
  float p[4][4];
  float mb = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = st[kt][i];
      // the key's offset from 8 lg, a constant
      if (MASKED) x = (32 * (kt >> 1) + 4 * (kt & 1) + i <= lim) ? x : -INFINITY;
      p[kt][i] = x;
      mb = fmaxf(mb, x);
    }
  mb = max_rows4(mb);
  const float cand = mb * tau;  // the block's largest logit of this row
  const bool move = cand > m_row + kLazyRescale;
  const float e = __expf(m_row - cand);  // 0 while m_row is -inf
  const float sc = move ? e : 1.f;
  const float ref = move ? cand : m_row;
  // ref stays -inf only when every key of the row is masked so far; any
  // finite offset then sends every masked logit to exp2(-inf) = 0
  const float off = (MASKED && ref == -INFINITY) ? 0.f : -ref * kLog2e;
  float ls = 0.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ex = __builtin_amdgcn_exp2f(fmaf(p[kt][i], tl2e, off));
      p[kt][i] = ex;
      ls += ex;
    }
  ls = sum_rows4(ls);
  l_row = l_row * sc + ls;
  m_row = ref;
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    uint4 u;
    u.x = pack_bf16x2(p[2 * sl][0], p[2 * sl][1]);
    u.y = pack_bf16x2(p[2 * sl][2], p[2 * sl][3]);
    u.z = pack_bf16x2(p[2 * sl + 1][0], p[2 * sl + 1][1]);
    u.w = pack_bf16x2(p[2 * sl + 1][2], p[2 * sl + 1][3]);
    pb[sl] = as_bf16x8(u);
  }
  return sc;
}

template <int D>
__device__ __forceinline__ void rescale_acc(f32x4 (&acc)[D / 16], float sc) {
  if (__ballot(sc != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] *= sc;
  }
}

// O^T += V^T P^T; the next d-tile pair's operands are read while this pair's
// MFMAs run
template <int D>
__device__ __forceinline__ void tile_pv(f32x4 (&acc)[D / 16], const bf16x8 (&pb)[2], const uint16_t *vtb, int lane8) {
  constexpr int DT = D / 16;
  uint4 v[2][2][2];
  auto load_v = [&](uint4 (&dst)[2][2], int dt) {  // V^T piece 2 (dt + d2) + sl
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
        dst[d2][sl] = *reinterpret_cast<const uint4 *>(vtb + (2 * (dt + d2) + sl) * 512 + lane8);
  };
  load_v(v[0], 0);
#pragma unroll
  for (int st2 = 0; st2 < DT / 2; ++st2) {
    const int dt = 2 * st2;
    if (st2 + 1 < DT / 2) load_v(v[(st2 + 1) & 1], dt + 2);
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) acc[dt + d2] = mfma16(as_bf16x8(v[st2 & 1][d2][sl]), pb[sl], acc[dt + d2]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Attend one staged block with one 16-row tile.
template <int D, bool MASKED>
__device__ __forceinline__ void attend_tile(const bf16x8 (&qop)[D / 32], f32x4 (&acc)[D / 16], float &m_row,
                                            float &l_row, const uint16_t *ksb, const uint16_t *vtb, int lane8,
                                            int lim, float tau, float tl2e) {
  f32x4 st[4];
  tile_scores<D>(qop, ksb, lane8, st);
  bf16x8 pb[2];
  const float sc = tile_softmax<MASKED>(st, pb, m_row, l_row, lim, tau, tl2e);
  rescale_acc<D>(acc, sc);
  tile_pv<D>(acc, pb, vtb, lane8);
}

// The same for a wave's two tiles at once: every K and V^T operand is read
// from LDS once and feeds both tiles' products (each accumulator sees the
// same products in the same order as in attend_tile), halving the LDS reads
// of the block, which the workgroups of a CU otherwise share at twice the
// rate the matrix units consume them.
template <int D>
__device__ __forceinline__ void tile_scores2(const bf16x8 (&q0)[D / 32], const bf16x8 (&q1)[D / 32],
                                             const uint16_t *ksb, int lane8, f32x4 (&s0)[4], f32x4 (&s1)[4]) {
  constexpr int KS = D / 32;
  uint4 u[2][4];
  auto load_k = [&](uint4 (&dst)[4], int s) {  // K piece kt * KS + s
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) dst[kt] = *reinterpret_cast<const uint4 *>(ksb + (kt * KS + s) * 512 + lane8);
  };
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    s0[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    s1[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  load_k(u[0], 0);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (s + 1 < KS) load_k(u[(s + 1) & 1], s + 1);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) s0[kt] = mfma16(as_bf16x8(u[s & 1][kt]), q0[s], s0[kt]);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) s1[kt] = mfma16(as_bf16x8(u[s & 1][kt]), q1[s], s1[kt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D>
__device__ __forceinline__ void tile_pv2(f32x4 (&acc0)[D / 16], f32x4 (&acc1)[D / 16], const bf16x8 (&p0)[2],
                                         const bf16x8 (&p1)[2], const uint16_t *vtb, int lane8) {
  constexpr int DT = D / 16;
  uint4 v[2][2][2];
  auto load_v = [&](uint4 (&dst)[2][2], int dt) {  // V^T piece 2 (dt + d2) + sl
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
        dst[d2][sl] = *reinterpret_cast<const uint4 *>(vtb + (2 * (dt + d2) + sl) * 512 + lane8);
  };
  load_v(v[0], 0);
#pragma unroll
  for (int st2 = 0; st2 < DT / 2; ++st2) {
    const int dt = 2 * st2;
    if (st2 + 1 < DT / 2) load_v(v[(st2 + 1) & 1], dt + 2);
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) acc0[dt + d2] = mfma16(as_bf16x8(v[st2 & 1][d2][sl]), p0[sl], acc0[dt + d2]);
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) acc1[dt + d2] = mfma16(as_bf16x8(v[st2 & 1][d2][sl]), p1[sl], acc1[dt + d2]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, bool MASKED>
__device__ __forceinline__ void attend_two(RowState<D, 2> &R, const uint16_t *ksb, const uint16_t *vtb, int lane8,
                                           const int (&lim)[2], float tau, float tl2e) {
  f32x4 s0[4], s1[4];
  tile_scores2<D>(R.qop[0], R.qop[1], ksb, lane8, s0, s1);
  bf16x8 p0[2], p1[2];
  const float sc0 = tile_softmax<MASKED>(s0, p0, R.m_row[0], R.l_row[0], lim[0], tau, tl2e);
  const float sc1 = tile_softmax<MASKED>(s1, p1, R.m_row[1], R.l_row[1], lim[1], tau, tl2e);
  rescale_acc<D>(R.acc[0], sc0);
  rescale_acc<D>(R.acc[1], sc1);
  tile_pv2<D>(R.acc[0], R.acc[1], p0, p1, vtb, lane8);
}

// Run the block for the wave's tiles that take part (bit t of `mask`).
template <int D, int TPW, bool MASKED>
__device__ __forceinline__ void run_item(int mask, RowState<D, TPW> &R, const uint16_t *ksb, const uint16_t *vtb,
                                         int lane8, const int (&lim)[TPW], float tau, float tl2e) {
  if constexpr (TPW == 2) {
    if (mask == 3) {
      attend_two<D, MASKED>(R, ksb, vtb, lane8, lim, tau, tl2e);
      return;
    }
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    if ((mask >> t) & 1)
      attend_tile<D, MASKED>(R.qop[t], R.acc[t], R.m_row[t], R.l_row[t], ksb, vtb, lane8, lim[t], tau, tl2e);
}

// ------------------------------------------------------------------ kernel
// One tile per wave: four waves per SIMD (two workgroups per CU), at most 128
// registers; two tiles per wave: two waves per SIMD, at most 256.
template <int D, int G, int WAVES, int TPW>
__global__ void __launch_bounds__(WAVES * 64, TPW == 1 ? 4 : 2)
attn_window_mfma_kernel(AttnArgs a, const uint16_t *__restrict__ ops, const uint16_t *__restrict__ ops_tail,
                        int ntiles, int xcd_map) {
  using C = AttnCfg<D, G, WAVES, TPW>;
  __shared__ AttnSmem<D, G, WAVES, TPW> sm;

  const int T = a.T, W = a.W, Hq = a.Hq, Hkv = a.Hkv;
  // ---- workgroup -> (tile, g, b); the tiles of one (b, g) on one XCD so
  // its K/V stay in that XCD's L2
  int tile, g, b;
  {
    const int L = blockIdx.x;
    int pair, slot;
    if (xcd_map) {
      const int xcd = L & 7, s = L >> 3;
      pair = xcd + 8 * (s / ntiles);
      slot = s % ntiles;
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
  // the pair's blocks in operand order: complete chunks, then the partial
  // block that ends a sequence whose length is not a multiple of 64
  const int nchunks = T / kItemKeys;
  constexpr int kBlockElems = (C::kPiecesK + C::kPiecesV) * 512;
  const uint16_t *opg = ops + (static_cast<size_t>(b) * Hkv + g) * nchunks * kBlockElems;
  const uint16_t *optail = ops_tail + (static_cast<size_t>(b) * Hkv + g) * kBlockElems;

  // ---- rows: tile t of this wave holds queries q0 + wave * kQPW + t * kQPT
  // + (0 .. kQPT - 1), lane column ln = (query ln / G, head g G + ln % G)
  const int row_h = g * G + (ln % G);
  int row_i[TPW];
  bool row_ok[TPW];
  RowState<D, TPW> R;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    row_i[t] = q0 + wave * C::kQPW + t * C::kQPT + ln / G;
    row_ok[t] = row_i[t] < T;
    // Q operands (B of S^T = K Q^T): lane holds row ln, d = 32 ks + 8 lg ..
    // +8; rows past T read the last query (their results are not stored)
    const size_t qo = ((static_cast<size_t>(b) * Hq + row_h) * T + min(row_i[t], T - 1)) * D;
#pragma unroll
    for (int s = 0; s < C::kKS; ++s) R.qop[t][s] = as_bf16x8(*reinterpret_cast<const uint4 *>(qb + qo + 32 * s + 8 * lg));
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) R.acc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    R.m_row[t] = -INFINITY;
    R.l_row[t] = 0.f;
  }
  // the rows' chunk log-mass, read now so that it has landed by the epilogue
  float lse_pre[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    lse_pre[t] = (a.lse_c && row_ok[t]) ? a.lse_c[(static_cast<size_t>(b) * Hq + row_h) * T + row_i[t]] : -INFINITY;

  // window band of the tile: 64-key blocks from n_{first} * S to the last query
  const int i_first = q0, i_last = min(q0 + C::kQT - 1, T - 1);
  const int jw0 = eligible_chunks(i_first, W, kItemKeys) * kItemKeys;
  const int nitems = (i_last - jw0) / kItemKeys + 1;

  // ---- staging: block x -> LDS buffer, straight from global memory.  Wave
  // w copies pieces w, w + WAVES, ... of the block (1 KB each, lane l's 16
  // bytes at byte 16 l), K pieces into ks, V^T pieces into vt.
  auto issue_loads = [&](int j0, int buf) {
    const int blk = j0 / kItemKeys;
    const uint16_t *src = (blk < nchunks ? opg + static_cast<size_t>(blk) * kBlockElems : optail) + lane * 8;
#pragma unroll
    for (int i = 0; i < C::kLoadsK; ++i) {
      const int piece = i * WAVES + wave;
      lds_dma16(src + piece * 512, lds_address(sm.ks[buf] + piece * 512));
    }
#pragma unroll
    for (int i = 0; i < C::kLoadsV; ++i) {
      const int piece = i * WAVES + wave;
      lds_dma16(src + (C::kPiecesK + piece) * 512, lds_address(sm.vt[buf] + piece * 512));
    }
  };
  // The rows' chunk parts (bf16, written into o by the chunk pass) for the
  // epilogue, into the idle buffer during the last block: the workgroup's
  // kQT G = 128 rows of 2 D bytes fill the K and V^T halves of one buffer
  // exactly (rows 0 .. 63, then 64 .. 127).  Row R's 16-byte piece p sits at
  // position p ^ (R mod pieces), so that the 16 rows one epilogue read
  // touches fall in 16 different bank groups.  Wave w loads its own rows
  // 32 w .. 32 w + 31, one 1 KB slice per instruction.
  constexpr int kPartPieces = 2 * D / 16;
  static_assert(C::kQT * G == 128 && 2 * kItemKeys * D == 128 * D, "the parts fill one staging buffer");
  auto part_row = [&](int t, int bufp, int R) -> uint16_t * {
    return (R < 64 ? sm.ks[bufp] : sm.vt[bufp]) + (R & 63) * D;
  };
  auto issue_parts = [&](int bufp) {
    const uint16_t *ob_in = static_cast<const uint16_t *>(a.o);
    constexpr int kRowsPerSlice = 1024 / (2 * D);
#pragma unroll
    for (int sl = 0; sl < 32 / kRowsPerSlice; ++sl) {
      const int R = wave * 32 + sl * kRowsPerSlice + lane / kPartPieces;  // this lane's row
      const int pp = lane % kPartPieces, pc = pp ^ (R % kPartPieces);
      const int t = (R >> 4) & (TPW - 1), c = R & 15;                      // its tile and column
      const int qi = min(q0 + wave * C::kQPW + t * C::kQPT + c / G, T - 1);
      const uint16_t *src = ob_in + ((static_cast<size_t>(b) * Hq + g * G + c % G) * T + qi) * D + pc * 8;
      lds_dma16(src, lds_address(part_row(t, bufp, wave * 32 + sl * kRowsPerSlice)));
    }
  };
  issue_loads(jw0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // every operand read: lane l's 16 bytes of a 1 KB piece
  const int lane8 = lane * 8;

  const float tau = a.tau;
  const float tl2e = tau * kLog2e;
  // one block: query i's window starts at n_i * S, a multiple of the block
  // size (S = 64): a block lies in it from its first key on, up to key i,
  // or not at all.  lim: the last key of the block the row takes, as a
  // lane-relative offset (key - j0 - 8 lg); -1 takes none.
  auto block = [&](int x) {
    const int buf = x & 1;
    const int j0 = jw0 + x * kItemKeys;
    int lim[TPW];
    int mask = 0;
    bool edge = false;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      lim[t] = -1;
      bool mine = false;
      if (row_ok[t]) {
        const int i = row_i[t];
        const int ws = eligible_chunks(i, W, kItemKeys) * kItemKeys;  // n_i * S
        mine = ws <= j0 && j0 <= i;
        const int hi = min(j0 + kItemKeys - 1, i);
        if (mine) lim[t] = hi - j0 - 8 * lg;
        // a row that does not take the whole block needs the mask
        edge = edge || !mine || hi != j0 + kItemKeys - 1;
      }
      if (__ballot(mine)) mask |= 1 << t;
    }
    if (__ballot(edge))
      run_item<D, TPW, true>(mask, R, sm.ks[buf], sm.vt[buf], lane8, lim, tau, tl2e);
    else
      run_item<D, TPW, false>(mask, R, sm.ks[buf], sm.vt[buf], lane8, lim, tau, tl2e);
  };
  // Block x + 1 loads into buffer (x + 1) & 1, last read in iteration
  // x - 1 (before the barrier that ended it).  The last block, peeled off
  // (the window always holds key i: nitems >= 1), loads the rows' chunk
  // parts for the epilogue into the buffer it leaves idle instead.
  for (int x = 0; x + 1 < nitems; ++x) {
    debug_sync();
    issue_loads(jw0 + (x + 1) * kItemKeys, (x & 1) ^ 1);
    block(x);
    // this wave's loads of block x + 1 have landed; after the barrier, all have
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  debug_sync();
  if (a.lse_c) issue_parts(nitems & 1);
  block(nitems - 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- epilogue: o = acc / l, lane holds d = 16 dt + 4 lg + (0..3) of row ln.
  // With a chunk pass before this one (a.lse_c), o holds each row's chunk
  // part normalised by its chunk mass e^{lse_C}: the two parts meet under
  // the joint normaliser,
  //   o = (acc e^{m} + o_C e^{lse_C}) / (l e^{m} + e^{lse_C}),
  // both scaled by e^{-max(m, lse_C)} (m, l: the row's window reference and
  // sum; the window always holds key i itself, so m is finite).
  // The chunk parts of both tiles, from the buffer the last block left
  // idle (a row without a chunk, lse_C = -inf, ignores what its slot holds).
  uint16_t *ob = static_cast<uint16_t *>(a.o);
  const int pbuf = nitems & 1;  // the buffer the last iteration did not read
  uint2 part[TPW][C::kDT];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int R = wave * 32 + t * 16 + ln;
    const uint16_t *pr = part_row(t, pbuf, R);
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) {
      const int pc = 2 * dt + (lg >> 1), pos = pc ^ (R % kPartPieces);
      part[t][dt] = a.lse_c ? *reinterpret_cast<const uint2 *>(pr + pos * 8 + (lg & 1) * 4) : make_uint2(0u, 0u);
    }
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if (!row_ok[t]) continue;
    const size_t ro = (static_cast<size_t>(b) * Hq + row_h) * T + row_i[t];
    const size_t oo = ro * D;
    float fw = 1.f, fc = 0.f, inv = 1.f / R.l_row[t];
    if (a.lse_c) {
      const float lc = lse_pre[t];
      const float mx = fmaxf(R.m_row[t], lc);
      fw = __expf(R.m_row[t] - mx);
      fc = lc == -INFINITY ? 0.f : __expf(lc - mx);
      inv = 1.f / (R.l_row[t] * fw + fc);
    }
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) {
      float c4[4] = {0.f, 0.f, 0.f, 0.f};
      if (fc != 0.f) {
        const uint2 pc = part[t][dt];
        c4[0] = __uint_as_float(pc.x << 16);
        c4[1] = __uint_as_float(pc.x & 0xFFFF0000u);
        c4[2] = __uint_as_float(pc.y << 16);
        c4[3] = __uint_as_float(pc.y & 0xFFFF0000u);
      }
      uint2 w;
      w.x = pack_bf16x2((R.acc[t][dt][0] * fw + c4[0] * fc) * inv, (R.acc[t][dt][1] * fw + c4[1] * fc) * inv);
      w.y = pack_bf16x2((R.acc[t][dt][2] * fw + c4[2] * fc) * inv, (R.acc[t][dt][3] * fw + c4[3] * fc) * inv);
      *reinterpret_cast<uint2 *>(ob + oo + 16 * dt + 4 * lg) = w;
    }
  }
}

// the chunk log-mass and block maxima of |v|, rounded up to 256 bytes
static size_t attn_chunk_meta_bytes(int B, int Hq, int Hkv, int T) {
  const size_t nblk = (static_cast<size_t>(T) + kItemKeys - 1) / kItemKeys;
  return ((static_cast<size_t>(B) * Hq * T + static_cast<size_t>(B) * Hkv * nblk) * sizeof(float) + 255) / 256 * 256;
}

// the 64-key blocks' K and V^T in operand order: every complete chunk, then
// one partial block per (b, g) pair (present whatever T, so that the layout
// does not depend on T mod 64)
static size_t attn_ops_bytes(int B, int Hkv, int T, int d) {
  return static_cast<size_t>(B) * Hkv * (T / kItemKeys) * kItemKeys * d * 2 * 2;
}
static size_t attn_ops_tail_bytes(int B, int Hkv, int d) {
  return static_cast<size_t>(B) * Hkv * kItemKeys * d * 2 * 2;
}

template <int D, int G>
static hipError_t attn_mfma_t(const AttnArgs &a_in, hipStream_t st) {
  constexpr int WAVES = 4, TPW = 2;
  using C = AttnCfg<D, G, WAVES, TPW>;
  const int ntiles = (a_in.T + C::kQT - 1) / C::kQT;
  const int npairs = a_in.Hkv * a_in.B;
  const int nblk = (a_in.T + kItemKeys - 1) / kItemKeys;
  // Every block's K and V^T in operand order (and its largest |v|) first.
  // Then the chunk terms (chunk-major, rows compacted per chunk): each row's
  // chunk part into o, its chunk log-mass into the workspace.  Then the
  // window band through the kernel above, which combines the two.  No query
  // has an eligible chunk when T - W < S.
  const bool chunks = a_in.K > 0 && eligible_chunks_host(a_in.T - 1, a_in.W, kItemKeys) > 0;
  uint8_t *ws = static_cast<uint8_t *>(a_in.vt_ws);
  float *lse = reinterpret_cast<float *>(ws);
  float *vmax = lse + static_cast<size_t>(a_in.B) * a_in.Hq * a_in.T;
  uint16_t *ops = reinterpret_cast<uint16_t *>(ws + attn_chunk_meta_bytes(a_in.B, a_in.Hq, a_in.Hkv, a_in.T));
  uint16_t *ops_tail = reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(ops) +
                                                    attn_ops_bytes(a_in.B, a_in.Hkv, a_in.T, D));
  uint8_t *ws_after_ops = reinterpret_cast<uint8_t *>(ops_tail) + attn_ops_tail_bytes(a_in.B, a_in.Hkv, D);
  hipError_t e = launch_kv_operand_order(a_in, ops, ops_tail, chunks && !attn_long_used(a_in.T, a_in.K) ? vmax : nullptr, st);
  if (e != hipSuccess) return e;
  AttnArgs a = a_in;
  a.lse_c = nullptr;
  if (chunks) {
    if (attn_long_used(a_in.T, a_in.K))
      e = launch_attn_long(a_in, ops, lse, ws_after_ops, st);
    else
      e = launch_attn_chunks(a_in, ops, lse, vmax, nblk, st);
    if (e != hipSuccess) return e;
    a.lse_c = lse;
  }
  // a (b, g) pair's K and V^T fit one XCD's 4 MB L2: keep each pair on one
  // XCD; longer sequences: every XCD works on the same pair at a time, so
  // that the blocks its queries read stay in the shared memory-side cache
  const bool pair_fits_l2 = static_cast<size_t>(a.T) * D * 2 * 2 <= (size_t{4} << 20);
  const int xcd_map = (npairs % 8 == 0 && pair_fits_l2) ? 1 : 0;
  attn_window_mfma_kernel<D, G, WAVES, TPW><<<dim3(ntiles * npairs), C::kThreads, 0, st>>>(a, ops, ops_tail, ntiles,
                                                                                           xcd_map);
  return hipGetLastError();
}

bool attn_mfma_supported(const AttnArgs &a) {
  const int G = a.Hq / a.Hkv;
  return a.bf16 && (a.d == 64 || a.d == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) &&
         a.S == kItemKeys && a.K <= 32 && a.T / a.S <= 8192;
}

// the chunk log-mass of every (b, query head, query) and the largest |v| of
// every 64-key block, then every block's K and V^T in operand order; for
// long sequences the chunk-major pass's lists and partial results
size_t attn_mfma_ws_bytes(int B, int Hq, int Hkv, int T, int d, int K) {
  return attn_chunk_meta_bytes(B, Hq, Hkv, T) + attn_ops_bytes(B, Hkv, T, d) + attn_ops_tail_bytes(B, Hkv, d) +
         attn_long_ws_bytes(B, Hq, Hkv, T, d, K);
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
