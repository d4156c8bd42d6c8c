// Prefill hierarchical sparse attention on the MFMA units (bf16 operands,
// fp32 accumulation) -- HiLS-Attention, picx.dev summary, Methodology 2
// (Eq. 10) and 3 (query packing: M queries x G heads share the union of
// their selected chunks so that matrix tiles stay full).
//
// Workgroup = (QT consecutive queries, KV head g, batch b), 4 waves (one per
// SIMD) in under 80 KB of LDS, so that two workgroups share a CU and fill
// each other's barrier waits and softmax phases with MFMA work.  Each wave
// owns 32 (query, head) rows = two 16-row MFMA tiles of 16/G queries x G
// heads, with fp32 output accumulators in registers; which queries share a
// tile comes from attn_plan_kernel (grouped by selection overlap).
//
// The workgroup walks a list of 64-key "items": first every chunk in the
// union of its queries' selections, then the 64-key blocks of the window
// band.  Each item's K (row-major, XOR-swizzled 16-byte pieces) and V^T
// ([d][key], padded rows; read from value tiles transposed once per call by
// a small kernel) are staged once in LDS, double buffered, and shared by all
// waves.  Per item, each wave runs only the row tiles that take part (one of
// their rows selected the chunk / overlaps the window block), one after the
// other:
//   S^T = K Q^T           16x16x32 bf16 MFMA, keys in M, rows in N
//   chunk item:  p = softmax over the chunk's 64 keys (exact), scaled by the
//                fusion weight e^{s_hat - M_row}; rows that did not select
//                the chunk get weight 0
//   window item: softmax against the row's reference maximum, masked to
//                [n_i * S, i] only on blocks that cross a row's window edge
//   O^T += V^T P^T        16x16x32 bf16 MFMA, d in M, rows in N
// The key order inside S^T is permuted so that its accumulator layout is
// exactly the B-operand layout of the P^T product (no cross-lane moves).
// Row statistics start from M_row = max of the row's selected chunk scores
// and l_row = sum e^{s_hat - M_row}; one joint normaliser over chunks and
// window (Eq. 10's Z-hat_i).  A window block moves M_row only when its own
// maximum exceeds M_row by more than kLazyRescale; numerator and denominator
// always share the reference, so the result does not depend on when it moves.
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
  static constexpr int kKMax = 32;            // largest top-K
  static constexpr int kLS = kKMax + 1;       // per-query list stride: slot kKMax is a sentinel
  static constexpr int kRowPieces = D / 8;    // 16-byte pieces per K row
  // one staged item = 64 K rows + D V^T rows of 128 bytes, loaded straight
  // into LDS in 1 KB wave-wide pieces
  static constexpr int kLoadsK = kItemKeys * D * 2 / 1024 / WAVES;
  static constexpr int kLoadsV = D * kItemKeys * 2 / 1024 / WAVES;
  static_assert(kLoadsK * WAVES * 1024 == kItemKeys * D * 2, "K item must split evenly over the waves");
};

template <int D, int G, int WAVES, int TPW>
struct AttnSmem {
  using C = AttnCfg<D, G, WAVES, TPW>;
  uint16_t ks[2][kItemKeys * D];   // K rows, 16-byte pieces XOR-swizzled per row
  uint16_t vt[2][D * kItemKeys];   // V^T rows, 16-byte pieces XOR-swizzled per row
  int16_t spos[C::kQT * C::kLS];     // per query: union positions of its chunks, ascending, then kNoPos
  int8_t sk[C::kQT * C::kLS];        // their slots in the query's top-K list (0 past the end)
  alignas(16) int16_t ulist[C::kQT * C::kKMax];  // union of selected chunks, ascending (first: the raw lists)
  uint32_t umask[256];
  int wbase[256];                    // union positions before each 32-chunk word
  int nunion;
};

constexpr int16_t kNoPos = 0x7FFF;  // cursor sentinel: no further selected chunk

// key held by S^T tile kt, row m (the permutation described above)
__device__ __forceinline__ int perm_key(int kt, int m) {
  return 32 * (kt >> 1) + 8 * (m >> 2) + 4 * (kt & 1) + (m & 3);
}

// XOR swizzle of the 16-byte pieces of K row r.  The 16 rows that one MFMA
// operand read touches (perm_key(kt, 0..15)) then fall in 16 different bank
// groups; for those rows the swizzle equals ln (D = 128) or ln >> 1 (D = 64).
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? ((r & 3) | ((r >> 1) & 12)) : (((r >> 1) & 1) | ((r >> 2) & 6));
}
// XOR swizzle of the 8 pieces of V^T row d: rows d and d ^ 1 share a 256-byte
// bank line, so the swizzle runs over d >> 1.
__device__ __forceinline__ int v_swz(int d) { return (d >> 1) & 7; }

// ------------------------------------------------------------------ V^T tiles
// v [B, Hkv, T, D] -> vt [B, Hkv, nblk, D, 64]: block blk holds keys
// 64 blk .. 64 blk + 63 transposed (keys at or past T are zero); vmax
// [B, Hkv, nblk] (when given): the largest |v| element of each block.
template <int D>
__global__ void __launch_bounds__(256)
vt_transpose_kernel(const uint16_t *__restrict__ v, uint16_t *__restrict__ vt, float *__restrict__ vmax, int T,
                    int nblk) {
  constexpr int LD = D + 2;  // padded row (4-byte aligned, spreads column reads over banks)
  __shared__ uint16_t tile[kItemKeys * LD];
  __shared__ uint32_t wmax[4];
  const int blk = blockIdx.x, pair = blockIdx.y;
  const uint16_t *src = v + static_cast<size_t>(pair) * T * D;
  const int j0 = blk * kItemKeys;
  uint32_t amax = 0u;  // |v| as bf16 bits: the order of non-negative floats
  for (int p = threadIdx.x; p < kItemKeys * D / 8; p += 256) {
    const int key = p / (D / 8), seg = p % (D / 8);
    const uint4 u = (j0 + key < T) ? *reinterpret_cast<const uint4 *>(src + static_cast<size_t>(j0 + key) * D + seg * 8)
                                   : make_uint4(0u, 0u, 0u, 0u);
    uint32_t *row = reinterpret_cast<uint32_t *>(tile + key * LD + seg * 8);
    row[0] = u.x; row[1] = u.y; row[2] = u.z; row[3] = u.w;
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = max(amax, max(w4[e] & 0x7FFFu, (w4[e] >> 16) & 0x7FFFu));
  }
  if (vmax) {
    amax = wave_reduce_u32<1>(amax);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  }
  __syncthreads();
  if (vmax && threadIdx.x == 0)
    vmax[static_cast<size_t>(pair) * nblk + blk] =
        bf16_to_f32(static_cast<uint16_t>(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]))));
  uint16_t *dst = vt + (static_cast<size_t>(pair) * nblk + blk) * D * kItemKeys;
  for (int p = threadIdx.x; p < D * kItemKeys / 8; p += 256) {
    const int d = p / 8, kp = p % 8;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = static_cast<uint32_t>(tile[(8 * kp + 2 * e) * LD + d]) |
             (static_cast<uint32_t>(tile[(8 * kp + 2 * e + 1) * LD + d]) << 16);
    *reinterpret_cast<uint4 *>(dst + d * kItemKeys + kp * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

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
__device__ __forceinline__ void tile_scores(const bf16x8 (&qop)[D / 32], const uint16_t *ksb, int koff,
                                            f32x4 (&st)[4]) {
  constexpr int KS = D / 32;
  uint4 u[2][4];
  auto load_k = [&](uint4 (&dst)[4], int s) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      dst[kt] = *reinterpret_cast<const uint4 *>(ksb + (koff ^ (32 * s)) + (32 * (kt >> 1) + 4 * (kt & 1)) * D);
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
// perm_key(kt, 4 lg + i) of row ln).  CHUNK: exact softmax over the chunk's
// 64 keys, scaled by the fusion weight wgt.  Otherwise a window block against
// the row's reference maximum m_row; when MASKED, only the lane's keys with
// perm_key(kt, 4 lg + i) - 8 lg <= lim count (see window_limit);
// the reference moves to the block's maximum only when that exceeds it by
// more than kLazyRescale, and the returned factor (1 otherwise) rescales the
// row's accumulator.
template <bool CHUNK, bool MASKED>
__device__ __forceinline__ float tile_softmax(const f32x4 (&st)[4], bf16x8 (&pb)[2], float &m_row, float &l_row,
                                              float wgt, int lim, float tau, float tl2e) {
  float p[4][4];
  float sc = 1.f;
  if (CHUNK) {
    float mc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mc = fmaxf(mc, st[kt][i]);
    mc = max_rows4(mc);
    const float off = -mc * tl2e;
    float lc = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[kt][i] = __builtin_amdgcn_exp2f(fmaf(st[kt][i], tl2e, off));
        lc += p[kt][i];
      }
    lc = sum_rows4(lc);
    const float w = wgt * __builtin_amdgcn_rcpf(lc);  // lc >= 1 (the maximum's term)
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
        float x = st[kt][i];
        // perm_key(kt, 4 lg + i) - 8 lg, a constant
        if (MASKED) x = (32 * (kt >> 1) + 4 * (kt & 1) + i <= lim) ? x : -INFINITY;
        p[kt][i] = x;
        mb = fmaxf(mb, x);
      }
    mb = max_rows4(mb);
    const float cand = mb * tau;  // the block's largest logit of this row
    const bool move = cand > m_row + kLazyRescale;
    const float e = __expf(m_row - cand);  // 0 while m_row is -inf
    sc = move ? e : 1.f;
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
  }
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
__device__ __forceinline__ void tile_pv(f32x4 (&acc)[D / 16], const bf16x8 (&pb)[2], const uint16_t *vtb, int voff) {
  constexpr int DT = D / 16;
  uint4 v[2][2][2];
  auto load_v = [&](uint4 (&dst)[2][2], int dt) {
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
        dst[d2][sl] = *reinterpret_cast<const uint4 *>(vtb + (voff ^ (32 * sl)) + 16 * (dt + d2) * kItemKeys);
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

// Attend one staged item with one 16-row tile.
template <int D, bool CHUNK, bool MASKED>
__device__ __forceinline__ void attend_tile(const bf16x8 (&qop)[D / 32], f32x4 (&acc)[D / 16], float &m_row,
                                            float &l_row, const uint16_t *ksb, const uint16_t *vtb, int koff,
                                            int voff, float wgt, int lim, float tau, float tl2e) {
  f32x4 st[4];
  tile_scores<D>(qop, ksb, koff, st);
  bf16x8 pb[2];
  const float sc = tile_softmax<CHUNK, MASKED>(st, pb, m_row, l_row, wgt, lim, tau, tl2e);
  if (!CHUNK) rescale_acc<D>(acc, sc);
  tile_pv<D>(acc, pb, vtb, voff);
}

// Run the item for the wave's tiles that take part (bit t of `mask`).
template <int D, int TPW, bool CHUNK, bool MASKED>
__device__ __forceinline__ void run_item(int mask, RowState<D, TPW> &R, const uint16_t *ksb, const uint16_t *vtb,
                                         int koff, int voff, const float (&wgt)[TPW], const int (&lim)[TPW], float tau,
                                         float tl2e) {
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    if ((mask >> t) & 1)
      attend_tile<D, CHUNK, MASKED>(R.qop[t], R.acc[t], R.m_row[t], R.l_row[t], ksb, vtb, koff, voff, wgt[t], lim[t],
                                    tau, tl2e);
}

// ------------------------------------------------------------------ query grouping
// Which QPT of a workgroup's QT queries share a 16-row tile.  A tile runs a
// chunk item when any of its queries selected the chunk, so tiles of
// queries with overlapping selections run fewer items: greedily, each tile
// starts from the lowest remaining query and takes, one at a time, the
// query whose chunks add the fewest to the tile's union (ties: the lower
// query).  Rows are independent, so every grouping gives the same outputs.
// One wave per workgroup tile (four per block, independent: no LDS, no
// barrier), lane q for query q, each query's chunks as a bit mask of the
// chunk ids in four registers (up to 128 chunks: T <= 8192 with S = 64); the
// forming tile's union in scalar registers (readlane), and lane s keeps the
// query chosen for row slot s.
// plan[(pair * ntiles + tile) * QT + s] is the local query of row slot
// s = tile_in_workgroup * QPT + query_in_tile.  More chunks, or workgroups
// of more than 64 queries, keep the identity.
template <int QT, int QPT>
__global__ void __launch_bounds__(256)
attn_plan_kernel(const int32_t *__restrict__ topk_idx, uint8_t *__restrict__ plan, int T, int K, int ntiles,
                 int nplans) {
  constexpr bool kGroup = QT <= 64 && QPT > 1;
  const int L = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (L >= nplans) return;
  const int tile = L % ntiles, pair = L / ntiles;
  const int q0 = tile * QT;
  uint8_t *out = plan + static_cast<size_t>(L) * QT;
  if (!kGroup || K <= 0 || K > 32 || T / kItemKeys > 128) {
    for (int x = lane; x < QT; x += 64) out[x] = static_cast<uint8_t>(x);
    return;
  }
  // this lane's query: its selected chunks as a 128-bit mask (past T: none)
  uint32_t mine[4] = {0u, 0u, 0u, 0u};
  {
    const bool ok = lane < QT && q0 + lane < T;
    const int32_t *row = topk_idx + (static_cast<size_t>(pair) * T + (ok ? q0 + lane : 0)) * K;
    // all loads in flight at once: 16-byte pieces when K is a multiple of 4
    // (rows are then 16-byte aligned), else single slots; pieces / slots past
    // K re-read the last one and count for nothing
    int cs[32];
    if ((K & 3) == 0) {
      const int4 *rv = reinterpret_cast<const int4 *>(row);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int4 x = rv[min(v, K / 4 - 1)];
        cs[4 * v] = x.x; cs[4 * v + 1] = x.y; cs[4 * v + 2] = x.z; cs[4 * v + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 32; ++k) cs[k] = row[min(k, K - 1)];
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int c = (ok && k < K) ? cs[k] : -1;
#pragma unroll
      for (int w = 0; w < 4; ++w) mine[w] |= (c >= 0 && (c >> 5) == w) ? (1u << (c & 31)) : 0u;
    }
  }
  unsigned long long rem = QT == 64 ? ~0ull : ((1ull << QT) - 1ull);
  int chosen = lane;  // the query of row slot `lane`
  for (int t = 0; t < QT / QPT; ++t) {
    const int seed = __ffsll(static_cast<long long>(rem)) - 1;
    rem &= ~(1ull << seed);
    chosen = lane == t * QPT ? seed : chosen;
    uint32_t u[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) u[w] = __builtin_amdgcn_readlane(mine[w], seed);
    for (int k = 1; k < QPT; ++k) {
      const bool cand = lane < QT && ((rem >> lane) & 1ull);
      const uint32_t cost =
          __popc(u[0] | mine[0]) + __popc(u[1] | mine[1]) + __popc(u[2] | mine[2]) + __popc(u[3] | mine[3]);
      const uint32_t key = wave_reduce_u32<0>(cand ? (cost << 8) | static_cast<uint32_t>(lane) : 0xFFFFFFFFu);
      const int best = static_cast<int>(__builtin_amdgcn_readfirstlane(key) & 0xFFu);
      rem &= ~(1ull << best);
      chosen = lane == t * QPT + k ? best : chosen;
#pragma unroll
      for (int w = 0; w < 4; ++w) u[w] |= __builtin_amdgcn_readlane(mine[w], best);
    }
  }
  if (lane < QT) out[lane] = static_cast<uint8_t>(chosen);
}

// ------------------------------------------------------------------ kernel
// One tile per wave: four waves per SIMD (two workgroups per CU), at most 128
// registers; two tiles per wave: two waves per SIMD, at most 256.
template <int D, int G, int WAVES, int TPW>
__global__ void __launch_bounds__(WAVES * 64, TPW == 1 ? 4 : 2)
attn_prefill_mfma_kernel(AttnArgs a, const uint8_t *__restrict__ plan, int ntiles, int xcd_map, int nblk) {
  using C = AttnCfg<D, G, WAVES, TPW>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  AttnSmem<D, G, WAVES, TPW> &sm = *reinterpret_cast<AttnSmem<D, G, WAVES, TPW> *>(smem_raw);
  // the rows' fusion scores [kQT * G * K] follow the struct
  float *wl = reinterpret_cast<float *>(smem_raw + sizeof(AttnSmem<D, G, WAVES, TPW>));

  const int T = a.T, K = a.K, W = a.W, Hq = a.Hq, Hkv = a.Hkv;
  const int C_chunks = T / kItemKeys;  // chunk size S = 64 on this path
  // ---- workgroup -> (tile, g, b); heaviest (latest) tiles first, and the
  // tiles of one (b, g) on one XCD so its K/V stay in that XCD's L2
  int tile, g, b, pair;
  {
    const int L = blockIdx.x;
    int slot;
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
  const uint16_t *kb = static_cast<const uint16_t *>(a.k) + (static_cast<size_t>(b) * Hkv + g) * T * D;
  const uint16_t *vtg = static_cast<const uint16_t *>(a.vt_ws) + (static_cast<size_t>(b) * Hkv + g) * nblk * D * kItemKeys;

  // ---- every global load of the set-up is issued here, at once, with
  // clamped indices and no lane-dependent branch (so that nothing waits for
  // one load before issuing the next): the rows' queries in the grouping of
  // attn_plan_kernel (first: the Q loads need them), the selections (query,
  // slot) of the tile, the rows' fusion scores, then the Q operands.
  int row_q[TPW];
  if (plan) {
    const uint8_t *pt = plan + (static_cast<size_t>(pair) * ntiles + tile) * C::kQT;
#pragma unroll
    for (int t = 0; t < TPW; ++t) row_q[t] = min(static_cast<int>(pt[wave * C::kQPW + t * C::kQPT + ln / G]), C::kQT - 1);
  } else {  // adjacent queries share a tile
#pragma unroll
    for (int t = 0; t < TPW; ++t) row_q[t] = wave * C::kQPW + t * C::kQPT + ln / G;
  }
  constexpr int kPairs = (C::kQT * C::kKMax + C::kThreads - 1) / C::kThreads;
  constexpr int kWPT = (C::kQT * G * C::kKMax + C::kThreads - 1) / C::kThreads;
  const int kc_max = K > 0 ? K - 1 : 0;
  int my_c[kPairs];
  float wv[kWPT];
  if (K > 0) {
    const int *idx_bg = a.topk_idx + (static_cast<size_t>(b) * Hkv + g) * T * K;
#pragma unroll
    for (int r = 0; r < kPairs; ++r) {
      const int x = tid + r * C::kThreads, q = x / C::kKMax, k = x % C::kKMax;
      my_c[r] = idx_bg[static_cast<size_t>(min(q0 + q, T - 1)) * K + min(k, kc_max)];
    }
    const float *tsc_b = a.topk_score + static_cast<size_t>(b) * Hq * T * K;
    const int total = C::kQT * G * K;
#pragma unroll
    for (int r = 0; r < kWPT; ++r) {
      const int x = tid + r * C::kThreads;
      const int xc = x < total ? x : 0;
      const int q = xc / (G * K), rem = xc % (G * K), hh = rem / K, k = rem % K;
      if (r * C::kThreads < total) wv[r] = tsc_b[(static_cast<size_t>(g * G + hh) * T + min(q0 + q, T - 1)) * K + k];
    }
  }
  // per-lane row identity for the tiles
  const int row_h = g * G + (ln % G);  // the same head in every tile
  bool row_ok[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) row_ok[t] = (q0 + row_q[t]) < T;
  RowState<D, TPW> R;
  // Q operands (B of S^T = K Q^T): lane holds row ln, d = 32 ks + 8 lg .. +8;
  // rows past T read the last query (their results are not stored)
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const size_t qo = ((static_cast<size_t>(b) * Hq + row_h) * T + min(q0 + row_q[t], T - 1)) * D;
#pragma unroll
    for (int s = 0; s < C::kKS; ++s) R.qop[t][s] = as_bf16x8(*reinterpret_cast<const uint4 *>(qb + qo + 32 * s + 8 * lg));
  }

  // ---- the union of the tile's selected chunks (bit mask -> ascending list)
  for (int x = tid; x < 256; x += C::kThreads) sm.umask[x] = 0u;
  __syncthreads();
  // the tile's fusion scores into LDS: wl[(q * G + hh) * K + k] =
  // topk_score[b, g G + hh, q0 + q, k], read by the row statistics and the
  // cursors below
  {
    const int total = C::kQT * G * K;
#pragma unroll
    for (int r = 0; r < kWPT; ++r) {
      const int x = tid + r * C::kThreads;
      if (r * C::kThreads < total && x < total) wl[x] = wv[r];
    }
  }
#pragma unroll
  for (int r = 0; r < kPairs; ++r) {
    const int x = tid + r * C::kThreads, q = x / C::kKMax, k = x % C::kKMax;
    // (an id outside the sequence's chunks counts as no chunk: the union
    // masks below are never indexed out of range)
    const int c = (q < C::kQT && k < K && q0 + q < T && my_c[r] < C_chunks) ? my_c[r] : -1;
    my_c[r] = c;
    if (q < C::kQT) sm.ulist[x] = static_cast<int16_t>(c);  // scratch copy of the raw lists
    if (c >= 0) atomicOr(&sm.umask[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  // ---- row statistics from the raw lists: M_row = max of the row's selected
  // chunk scores, l_row = sum of e^{s_hat - M_row} over them (every valid
  // slot counts), eight slots at a time with a running maximum
  int wrow[TPW];  // this row's fusion scores: wl + wrow[t], indexed by top-K slot
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    wrow[t] = (row_q[t] * G + (ln % G)) * K;
    const int16_t *raw = sm.ulist + row_q[t] * C::kKMax;
    float mx = -INFINITY, l = 0.f;
    for (int k0 = 0; k0 < K; k0 += 8) {
      const uint4 cw = *reinterpret_cast<const uint4 *>(raw + k0);
      const uint32_t cv[4] = {cw.x, cw.y, cw.z, cw.w};
      float sv[8];
      bool ok[8];
      float m8 = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = static_cast<int16_t>((cv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        ok[e] = (k0 + e < K) && c >= 0;
        sv[e] = wl[wrow[t] + min(k0 + e, K - 1)];
        m8 = ok[e] ? fmaxf(m8, sv[e]) : m8;
      }
      const float mn = fmaxf(mx, m8);
      float l8 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) l8 += ok[e] ? __expf(sv[e] - mn) : 0.f;
      l = (mx == -INFINITY ? 0.f : l * __expf(mx - mn)) + l8;
      mx = mn;
    }
    R.m_row[t] = mx;
    R.l_row[t] = l;
  }
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
      if (w < nwords) sm.wbase[w] = base + incl - cnt;
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) sm.nunion = base;
  }
  // ---- per query: its chunks' union positions in ascending order (= chunk
  // order), with their fusion scores.  Entry (q, k) takes rank
  //   #{valid c2 < c} + #{earlier valid c2 == c}        for a valid c,
  //   n_valid + #{earlier invalid entries}              otherwise,
  // a bijection onto 0 .. kKMax-1 (invalid ranks hold the sentinel).
#pragma unroll
  for (int r = 0; r < kPairs; ++r) {
    const int x = tid + r * C::kThreads, q = x / C::kKMax, k = x % C::kKMax;
    if (q >= C::kQT) continue;
    const int c = my_c[r];
    int below = 0, nvalid = 0, inv_before = 0;
    for (int k2 = 0; k2 < K; ++k2) {
      const int c2 = sm.ulist[q * C::kKMax + k2];
      nvalid += c2 >= 0;
      below += (c2 >= 0) & ((c2 < c) | ((c2 == c) & (k2 < k)));
      inv_before += (c2 < 0) & (k2 < k);
    }
    inv_before += max(0, k - K);  // entries k2 >= K are invalid too
    my_c[r] = c >= 0 ? below : -1 - (nvalid + inv_before);
  }
  __syncthreads();  // wbase, nunion ready; the raw lists are read no more
#pragma unroll
  for (int r = 0; r < kPairs; ++r) {
    const int x = tid + r * C::kThreads, q = x / C::kKMax, k = x % C::kKMax, i = q0 + q;
    if (q >= C::kQT) continue;
    (void)i;
    if (my_c[r] >= 0) {
      const int rank = my_c[r];
      const int c = sm.ulist[q * C::kKMax + k];
      const int upos = sm.wbase[c >> 5] + __popc(sm.umask[c >> 5] & ((1u << (c & 31)) - 1u));
      sm.spos[q * C::kLS + rank] = static_cast<int16_t>(upos);
      sm.sk[q * C::kLS + rank] = static_cast<int8_t>(k);
    } else {
      sm.spos[q * C::kLS + (-1 - my_c[r])] = kNoPos;
      sm.sk[q * C::kLS + (-1 - my_c[r])] = 0;
    }
  }
  for (int q = tid; q < C::kQT; q += C::kThreads) {
    sm.spos[q * C::kLS + C::kKMax] = kNoPos;
    sm.sk[q * C::kLS + C::kKMax] = 0;
  }
  __syncthreads();
  // the ascending union list (overwrites the scratch copy)
  if (wave == 0) {
    const int nwords = (C_chunks + 31) >> 5;
    for (int w = lane; w < nwords; w += 64) {
      int pos = sm.wbase[w];
      uint32_t bb = sm.umask[w];
      while (bb) {
        const int bit = __ffs(bb) - 1;
        bb &= bb - 1;
        sm.ulist[pos++] = static_cast<int16_t>(w * 32 + bit);
      }
    }
  }
  __syncthreads();
  const int nunion = sm.nunion;

  // window band of the tile: 64-key blocks from n_{first} * S to the last query
  const int i_first = q0, i_last = min(q0 + C::kQT - 1, T - 1);
  const int jw0 = eligible_chunks(i_first, W, kItemKeys) * kItemKeys;
  const int nwin = (i_last - jw0) / kItemKeys + 1;
  const int nitems = nunion + nwin;


  // ---- each row's cursor into its ascending selection list
  // cur[t]: LDS index of the row's next list entry (a list ends in kNoPos)
  int cur[TPW], nxt_pos[TPW];
  float nxt_alpha[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int qk = row_q[t] * C::kLS;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) R.acc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    cur[t] = qk;
    nxt_pos[t] = row_ok[t] ? sm.spos[qk] : kNoPos;
    nxt_alpha[t] = wl[wrow[t] + sm.sk[qk]];  // unused once the list has ended
  }

  // ---- staging: item x -> LDS buffer, straight from global memory.  Wave w
  // fills 1 KB slices w, w + WAVES, ... of each tensor; lane l's 16 bytes land
  // at byte 16 l of the slice, i.e. at one (row, physical piece) pair, and the
  // lane fetches the logical piece the swizzle puts there.
  auto issue_loads = [&](int j0, int buf) {
    const uint16_t *vsrc = vtg + static_cast<size_t>(j0 / kItemKeys) * D * kItemKeys;
#pragma unroll
    for (int i = 0; i < C::kLoadsK; ++i) {
      const int slice = i * WAVES + wave;
      const int sl = slice * 64 + lane;  // 16-byte slot
      const int r = sl / C::kRowPieces, pp = sl % C::kRowPieces;
      const int pc = pp ^ k_swz<D>(r);
      const int key = min(j0 + r, T - 1);  // rows past T are never used unmasked
      __builtin_amdgcn_global_load_lds(kb + static_cast<uint32_t>(key * D + pc * 8),
                                       (__attribute__((address_space(3))) void *)(sm.ks[buf] + slice * 512), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::kLoadsV; ++i) {
      const int slice = i * WAVES + wave;
      const int sl = slice * 64 + lane;
      const int d = sl / 8, pp = sl % 8;
      const int pc = pp ^ v_swz(d);
      __builtin_amdgcn_global_load_lds(vsrc + static_cast<uint32_t>(d * kItemKeys + pc * 8),
                                       (__attribute__((address_space(3))) void *)(sm.vt[buf] + slice * 512), 16, 0, 0);
    }
  };

  // the union list, 64 entries at a time in a register (lane l holds entry
  // ubase + l): an item's first key is a lane read, not an LDS round trip
  int ubase = 0;
  int ureg = lane < nunion ? sm.ulist[lane] : 0;
  auto union_key0 = [&](int x) -> int {
    if (x - ubase >= 64) {  // uniform: the next 64 entries
      ubase += 64;
      ureg = ubase + lane < nunion ? sm.ulist[ubase + lane] : 0;
    }
    return __builtin_amdgcn_readlane(ureg, x - ubase) * kItemKeys;
  };
  auto item_key0 = [&](int x) -> int { return x < nunion ? union_key0(x) : jw0 + (x - nunion) * kItemKeys; };
  int j0_cur = 0, j0_nxt = 0;
  if (nitems > 0) {
    j0_cur = item_key0(0);
    issue_loads(j0_cur, 0);
  }
  if (nitems > 1) j0_nxt = item_key0(1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // per-lane LDS offsets of the S^T A operand (K rows perm_key(kt, ln); their
  // swizzle does not depend on kt) and of the O^T A operand (V^T rows 16 dt + ln)
  // k-step s reads piece (4 s + lg) ^ swizzle = piece(0) ^ 4 s: offset koff ^ 32 s;
  // key slot sl reads piece (lg + 4 sl) ^ swizzle: offset voff ^ 32 sl
  const int r0 = 8 * (ln >> 2) + (ln & 3);
  const int koff = r0 * D + ((lg ^ k_swz<D>(r0)) << 3);
  const int voff = ln * kItemKeys + ((lg ^ v_swz(ln)) << 3);

  const float tau = a.tau;
  const float tl2e = tau * kLog2e;
  for (int x = 0; x < nitems; ++x) {
    const int buf = x & 1;
    // buffer buf ^ 1 was last read in iteration x - 1, before the barrier
    // that ended it
    if (x + 1 < nitems) issue_loads(j0_nxt, buf ^ 1);
    const int j0_nn = (x + 2 < nitems) ? item_key0(x + 2) : 0;
    const uint16_t *ksb = sm.ks[buf];
    const uint16_t *vtb = sm.vt[buf];
    const int j0 = j0_cur;
    float wgt[TPW];
    int lim[TPW];
    int mask = 0;
    if (x < nunion) {
      bool act[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        while (nxt_pos[t] < x) {  // a chunk listed twice: attended once
          ++cur[t];
          nxt_pos[t] = sm.spos[cur[t]];
          nxt_alpha[t] = wl[wrow[t] + sm.sk[cur[t]]];
        }
        act[t] = nxt_pos[t] == x;
        wgt[t] = act[t] ? __expf(nxt_alpha[t] - R.m_row[t]) : 0.f;
        lim[t] = 0;
        if (__ballot(act[t])) mask |= 1 << t;
      }
      run_item<D, TPW, true, false>(mask, R, ksb, vtb, koff, voff, wgt, lim, tau, tl2e);
      // rows that took their entry move on; the reads land during the
      // barrier wait instead of ahead of the tiles
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        cur[t] += act[t] ? 1 : 0;
        nxt_pos[t] = sm.spos[cur[t]];
        nxt_alpha[t] = wl[wrow[t] + sm.sk[cur[t]]];
      }
    } else {
      // Query i's window starts at n_i * S, a multiple of the block size
      // (S = 64): a block lies in it from its first key on, up to key i, or
      // not at all.  lim: the last key of the block the row takes, as a
      // lane-relative offset (key - j0 - 8 lg); -1 takes none.
      bool edge = false;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        wgt[t] = 0.f;
        lim[t] = -1;
        bool mine = false;
        if (row_ok[t]) {
          const int i = q0 + row_q[t];
          const int ws = (max(0, i - W + 1) >> 6) << 6;  // n_i * S
          mine = ws <= j0 && j0 <= i;
          const int hi = min(j0 + kItemKeys - 1, i);
          if (mine) lim[t] = hi - j0 - 8 * lg;
          // a row that does not take the whole block needs the mask
          edge = edge || !mine || hi != j0 + kItemKeys - 1;
        }
        if (__ballot(mine)) mask |= 1 << t;
      }
      if (__ballot(edge))
        run_item<D, TPW, false, true>(mask, R, ksb, vtb, koff, voff, wgt, lim, tau, tl2e);
      else
        run_item<D, TPW, false, false>(mask, R, ksb, vtb, koff, voff, wgt, lim, tau, tl2e);
    }
    j0_cur = j0_nxt;
    j0_nxt = j0_nn;
    // this wave's loads of item x + 1 have landed; after the barrier, all have
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: o = acc / l, lane holds d = 16 dt + 4 lg + (0..3) of row ln.
  // With a chunk pass before this one (a.lse_c), o holds each row's chunk
  // part normalised by its chunk mass e^{lse_C}: the two parts meet under
  // the joint normaliser,
  //   o = (acc e^{m} + o_C e^{lse_C}) / (l e^{m} + e^{lse_C}),
  // both scaled by e^{-max(m, lse_C)} (m, l: the row's window reference and
  // sum; the window always holds key i itself, so m is finite).
  uint16_t *ob = static_cast<uint16_t *>(a.o);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if (!row_ok[t]) continue;
    const size_t ro = (static_cast<size_t>(b) * Hq + row_h) * T + (q0 + row_q[t]);
    const size_t oo = ro * D;
    float fw = 1.f, fc = 0.f, inv = 1.f / R.l_row[t];
    if (a.lse_c) {
      const float lc = a.lse_c[ro];
      const float mx = fmaxf(R.m_row[t], lc);
      fw = __expf(R.m_row[t] - mx);
      fc = lc == -INFINITY ? 0.f : __expf(lc - mx);
      inv = 1.f / (R.l_row[t] * fw + fc);
    }
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) {
      float c4[4] = {0.f, 0.f, 0.f, 0.f};
      if (fc != 0.f) {
        const uint2 pc = *reinterpret_cast<const uint2 *>(ob + oo + 16 * dt + 4 * lg);
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

// value tiles (bf16), rounded up to 256 bytes
static size_t attn_vt_bytes(int B, int Hkv, int T, int d) {
  const size_t nblk = (static_cast<size_t>(T) + kItemKeys - 1) / kItemKeys;
  return (static_cast<size_t>(B) * Hkv * nblk * kItemKeys * d * 2 + 255) / 256 * 256;
}

template <int D, int G>
static hipError_t attn_mfma_t(const AttnArgs &a_in, hipStream_t st) {
  constexpr int WAVES = 4, TPW = 2;
  using C = AttnCfg<D, G, WAVES, TPW>;
  const int ntiles = (a_in.T + C::kQT - 1) / C::kQT;
  const int npairs = a_in.Hkv * a_in.B;
  const int nblk = (a_in.T + kItemKeys - 1) / kItemKeys;
  // The chunk terms first (chunk-major, rows compacted per chunk): each
  // row's chunk part into o, its chunk log-mass into the workspace after the
  // value tiles.  Then the window band through the kernel below, which
  // combines the two.  No query has an eligible chunk when T - W < S.
  const bool chunks = a_in.K > 0 && eligible_chunks_host(a_in.T - 1, a_in.W, kItemKeys) > 0;
  uint8_t *ws_after_vt = static_cast<uint8_t *>(a_in.vt_ws) + attn_vt_bytes(a_in.B, a_in.Hkv, a_in.T, D);
  float *lse = reinterpret_cast<float *>(ws_after_vt);
  float *vmax = lse + static_cast<size_t>(a_in.B) * a_in.Hq * a_in.T;
  uint16_t *ops = reinterpret_cast<uint16_t *>(ws_after_vt + attn_chunk_meta_bytes(a_in.B, a_in.Hq, a_in.Hkv, a_in.T));
  vt_transpose_kernel<D><<<dim3(nblk, npairs), 256, 0, st>>>(static_cast<const uint16_t *>(a_in.v),
                                                             static_cast<uint16_t *>(a_in.vt_ws),
                                                             chunks ? vmax : nullptr, a_in.T, nblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnArgs a = a_in;
  a.lse_c = nullptr;
  if (chunks) {
    e = launch_attn_chunks(a_in, ops, lse, vmax, nblk, st);
    if (e != hipSuccess) return e;
    a.lse_c = lse;
  }
  a.K = 0;
  a.topk_idx = nullptr;
  a.topk_score = nullptr;
  const uint8_t *plan = nullptr;
  // a (b, g) pair's K and V^T fit one XCD's 4 MB L2: keep each pair on one
  // XCD; longer sequences: every XCD works on the same pair at a time, so
  // that the chunks its queries gather stay in the shared memory-side cache
  const bool pair_fits_l2 = static_cast<size_t>(a.T) * D * 2 * 2 <= (size_t{4} << 20);
  const int xcd_map = (npairs % 8 == 0 && pair_fits_l2) ? 1 : 0;
  const size_t smem = sizeof(AttnSmem<D, G, WAVES, TPW>) + static_cast<size_t>(C::kQT) * G * a.K * sizeof(float);
  auto kern = attn_prefill_mfma_kernel<D, G, WAVES, TPW>;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(smem));
  if (e != hipSuccess) return e;
  kern<<<dim3(ntiles * npairs), C::kThreads, smem, st>>>(a, plan, ntiles, xcd_map, nblk);
  return hipGetLastError();
}

bool attn_mfma_supported(const AttnArgs &a) {
  const int G = a.Hq / a.Hkv;
  return a.bf16 && (a.d == 64 || a.d == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) &&
         a.S == kItemKeys && a.K <= 32 && a.T / a.S <= 8192;
}

// value tiles, then the chunk log-mass of every (b, query head, query) and
// the largest |v| of every 64-key block, then every complete chunk's K and
// V^T in operand order
size_t attn_mfma_ws_bytes(int B, int Hq, int Hkv, int T, int d) {
  const size_t chunks = static_cast<size_t>(B) * Hkv * (T / kItemKeys);
  return attn_vt_bytes(B, Hkv, T, d) + attn_chunk_meta_bytes(B, Hq, Hkv, T) + chunks * kItemKeys * d * 2 * 2;
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
