// Key-major pass of the HiLS-Attention backward on the matrix cores (bf16
// operands, fp32 accumulation): the key and value gradients of one 64-key
// block from every attention row that reads it, then the block's Eq. 8
// summary backward (picx.dev summary, Methodology 1 and 2).
//
// A row is a (query, head) pair that reads the block: through its sliding
// window (the queries i in [j0, j0 + S + W - 2]) or, for a complete chunk,
// through its top-K selection (the chunk's inverse list, every head of the
// group).  Per row the key pass needs q, dO and two scalars: the log-weight
// alpha (so that the row's weight of key j is e^{tau q.k_j + alpha}) and the
// value c its dO.v_j is compared against (Delta for window rows, dO.o_c for
// chunk rows).  The rows go through in tiles of 32; wave w owns keys
// 16 w .. 16 w + 15 and keeps them, and their values, in registers as MFMA
// B operands for the whole block:
//   S  = Q K^T     [32 rows x 16 keys]    16x16x32 bf16, rows in M
//   dP = dO V^T
//   P  = e^{tau S + alpha} (masked to keys <= i on window rows),
//   dS = tau P (dP - c)
//   dV^T += dO^T P,  dK^T += Q^T dS   [D x 16 keys], rows in K
// The tile rows are permuted in the S product (A row m of tile rt reads tile
// row 8 (m / 4) + 4 rt + m % 4), so that each lane's S accumulators are the
// 8 consecutive k slots of the B operand of the second products: P and dS go
// from accumulators to operands without leaving registers.  The second
// products need Q and dO transposed (8 consecutive rows of one d per lane),
// so each tile is staged in LDS twice, row-major and transposed (pairs of
// rows packed per 32-bit word).  The raw-q part of the summary gradient,
// tau sum ds q per head, is one more product per tile on the same Q^T
// operand: Q^T DS with DS[row][head] = ds of the row in its own head's
// column.
//
// The tile pipeline: while a tile computes, the next tile's q and dO rows
// load from HBM into registers and the tile after that looks up its rows
// (three slots of row data); the registers go to the other LDS buffer after
// the products.  Block y of the grid is the key block, so the blocks of the
// early chunks, which the most queries select, start first.
#include "bwd_common.h"

namespace hils {

namespace {

using bwd::kBK;
using bwd::kBT;

typedef __bf16 bf16x8k __attribute__((ext_vector_type(8)));
typedef float f32x4k __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4k mfma_k(const uint4 &a, const uint4 &b, const f32x4k &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8k, a), __builtin_bit_cast(bf16x8k, b), c, 0,
                                                 0, 0);
}

constexpr int kTR = 32;  // rows per tile
constexpr int kQP = 8;   // row-major tiles: rows D + 8 elements apart (16-byte reads spread over the banks)
constexpr int kTP = 40;  // transposed tiles: 32 rows + 8 elements per d

template <int D>
struct alignas(16) KmTiles {
  uint16_t qr[2][kTR][D + kQP];
  uint16_t dor[2][kTR][D + kQP];
  uint16_t qt[2][D][kTP];
  uint16_t dot[2][D][kTP];
};
template <int D>
struct KmEpi {
  float kt[kBK][D + 1];   // the block's keys (fp32)
  float dkb[kBK][D + 1];  // the key gradients from the rows
  float dkp[kMaxBwdG][D];
};
template <int D>
struct alignas(16) KmSmem {
  union {
    KmTiles<D> t;
    KmEpi<D> e;
  } u;
  long qoff[3][kTR];  // element offset of the row in q and dO (-1: padding)
  float alpha[3][kTR], cval[3][kTR], dsv[3][kTR];
  int limit[3][kTR];  // the last key the row reads (window rows: i)
  bwd::SummaryScratch<D> ss;
};

// A tile row's data, looked up by one of the first 32 threads.
struct RowMeta {
  long qoff;
  float alpha, cval, ds;
  int limit;
};

struct BlockRows {
  int iw_lo, nwin, nrows, e_lo, G;
  size_t ebase;
};

// Loads for list row r: window rows first (i-major, then head), then the
// chunk's entries with every head of the group.
__device__ __forceinline__ RowMeta row_meta(const BwdArgs &a, const BlockRows &br, int b, int g, int j0, int r) {
  RowMeta m{-1, -INFINITY, 0.f, 0.f, -1};
  const int G = br.G;
  if (r < br.nwin) {
    const int i = br.iw_lo + r / G, hh = r % G;
    if (eligible_chunks(i, a.W, kBK) * kBK <= j0) {  // the block lies in i's window (always, by the range)
      const size_t ro = (static_cast<size_t>(b) * a.Hq + g * G + hh) * a.T + i;
      m.qoff = static_cast<long>(ro) * a.d;
      m.alpha = -a.logz[ro];
      m.cval = a.delta[ro];
      m.limit = i;
    }
  } else if (r < br.nrows) {
    const int e = br.e_lo + (r - br.nwin) / G, hh = (r - br.nwin) % G;
    const size_t eo = (br.ebase + e) * G + hh;
    const int i = a.inv_list[br.ebase + e] >> 5;
    const size_t ro = (static_cast<size_t>(b) * a.Hq + g * G + hh) * a.T + i;
    m.qoff = static_cast<long>(ro) * a.d;
    m.alpha = a.ent_lw[eo];
    m.cval = a.ent_doo[eo];
    m.ds = a.ent_ds[eo];
    m.limit = 0x7fffffff;
  }
  return m;
}

}  // namespace

template <int D, int G>
__global__ void __launch_bounds__(256, 2)
bwd_keys_mfma_kernel(BwdArgs a) {
  __shared__ KmSmem<D> sm;
  constexpr int KS = D / 32, DT = D / 16, DTW = DT / 4;  // k-steps of S; d tiles; d tiles per wave (summary)
  constexpr int ITEMS = D / 64;                           // 16-byte row-pair pieces per thread and tile
  const int pair = blockIdx.x, kb = blockIdx.y;
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  // (the wave index is made a scalar so that no MFMA sits under a per-lane
  // mask: matrix instructions ignore EXEC)
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), ln = lane & 15, lg = lane >> 4;
  const int T_len = a.T, K = a.K, C = T_len / kBK;
  const float tau = a.tau;
  const int j0 = kb * kBK;
  const size_t pg = static_cast<size_t>(b) * a.Hkv + g;
  const uint16_t *kg = static_cast<const uint16_t *>(a.k) + pg * T_len * D;
  const uint16_t *vg = static_cast<const uint16_t *>(a.v) + pg * T_len * D;
  const uint16_t *qg = static_cast<const uint16_t *>(a.q), *og = static_cast<const uint16_t *>(a.d_o);
  // the wave's keys and values as B operands: key 16 w + ln, d = 32 s + 8 lg .. + 8
  const int key = j0 + 16 * w + ln;
  uint4 kop[KS], vop[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const bool ok = key < T_len;
    kop[s] = ok ? *reinterpret_cast<const uint4 *>(kg + static_cast<size_t>(key) * D + 32 * s + 8 * lg)
                : make_uint4(0u, 0u, 0u, 0u);
    vop[s] = ok ? *reinterpret_cast<const uint4 *>(vg + static_cast<size_t>(key) * D + 32 * s + 8 * lg)
                : make_uint4(0u, 0u, 0u, 0u);
  }
  BlockRows br;
  br.G = G;
  br.iw_lo = j0;
  const int iw_hi = min(T_len - 1, j0 + kBK + a.W - 2);
  br.nwin = iw_hi >= j0 ? (iw_hi - j0 + 1) * G : 0;
  br.e_lo = 0;
  int e_n = 0;
  const bool full_chunk = kb < C;
  if (full_chunk && K > 0) {
    br.e_lo = a.inv_choff[pg * (C + 1) + kb];
    e_n = a.inv_choff[pg * (C + 1) + kb + 1] - br.e_lo;
  }
  br.nrows = br.nwin + e_n * G;
  br.ebase = pg * static_cast<size_t>(T_len) * K;
  const int ntiles = (br.nrows + kTR - 1) / kTR;

  auto store_meta = [&](const RowMeta &m, int slot) {
    sm.qoff[slot][t] = m.qoff;
    sm.alpha[slot][t] = m.alpha;
    sm.cval[slot][t] = m.cval;
    sm.dsv[slot][t] = m.ds;
    sm.limit[slot][t] = m.limit;
  };
  // the q and dO rows of a tile: item x -> tensor, row pair pp, 8-element piece s
  uint4 stg[ITEMS][2];
  auto load_tile = [&](int slot) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int x = t + 256 * it, tensor = x / (16 * D / 8), rem = x % (16 * D / 8);
      const int pp = rem & 15, s = rem >> 4;
      const uint16_t *src = tensor ? og : qg;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const long o = sm.qoff[slot][2 * pp + h2];
        stg[it][h2] = o >= 0 ? *reinterpret_cast<const uint4 *>(src + o + 8 * s) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int x = t + 256 * it, tensor = x / (16 * D / 8), rem = x % (16 * D / 8);
      const int pp = rem & 15, s = rem >> 4;
      uint16_t(*rm)[D + kQP] = tensor ? sm.u.t.dor[buf] : sm.u.t.qr[buf];
      uint16_t(*tr)[kTP] = tensor ? sm.u.t.dot[buf] : sm.u.t.qt[buf];
      *reinterpret_cast<uint4 *>(&rm[2 * pp][8 * s]) = stg[it][0];
      *reinterpret_cast<uint4 *>(&rm[2 * pp + 1][8 * s]) = stg[it][1];
      const uint32_t r0[4] = {stg[it][0].x, stg[it][0].y, stg[it][0].z, stg[it][0].w};
      const uint32_t r1[4] = {stg[it][1].x, stg[it][1].y, stg[it][1].z, stg[it][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (r0[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, hi = (r1[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        *reinterpret_cast<uint32_t *>(&tr[8 * s + e][2 * pp]) = lo | (hi << 16);
      }
    }
  };

  f32x4k dv[DT], dk[DT], dkq[DTW];
#pragma unroll
  for (int x = 0; x < DT; ++x) dv[x] = dk[x] = f32x4k{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < DTW; ++x) dkq[x] = f32x4k{0.f, 0.f, 0.f, 0.f};

  // prologue: rows of tiles 0 and 1, tile 0 into buffer 0
  if (t < kTR) {
    store_meta(row_meta(a, br, b, g, j0, t), 0);
    store_meta(row_meta(a, br, b, g, j0, kTR + t), 1);
  }
  __syncthreads();
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int n = 0; n < ntiles; ++n) {
    const int mb = n % 3, buf = n & 1;
    // the rows of tile n + 2 and the q / dO of tile n + 1 (both land after the products)
    RowMeta nm;
    const bool meta_next = t < kTR && n + 2 < ntiles;
    if (meta_next) nm = row_meta(a, br, b, g, j0, (n + 2) * kTR + t);
    if (n + 1 < ntiles) load_tile((n + 1) % 3);
    // ---- S and dP
    f32x4k sacc[2], pacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) sacc[rt] = pacc[rt] = f32x4k{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int prow = 8 * (ln >> 2) + 4 * rt + (ln & 3);
        const uint4 aq = *reinterpret_cast<const uint4 *>(&sm.u.t.qr[buf][prow][32 * s + 8 * lg]);
        const uint4 ao = *reinterpret_cast<const uint4 *>(&sm.u.t.dor[buf][prow][32 * s + 8 * lg]);
        sacc[rt] = mfma_k(aq, kop[s], sacc[rt]);
        pacc[rt] = mfma_k(ao, vop[s], pacc[rt]);
      }
    }
    // ---- P and dS of rows 8 lg + 4 rt + j, key 16 w + ln: the B operands
    float pv[8], dsx[8];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int jx = 0; jx < 4; ++jx) {
        const int p = 8 * lg + 4 * rt + jx, e = 4 * rt + jx;
        const float P = key <= sm.limit[mb][p] ? __expf(tau * sacc[rt][jx] + sm.alpha[mb][p]) : 0.f;
        pv[e] = P;
        dsx[e] = tau * P * (pacc[rt][jx] - sm.cval[mb][p]);
      }
    const uint4 pb = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                                pack_bf16x2(pv[6], pv[7]));
    const uint4 db = make_uint4(pack_bf16x2(dsx[0], dsx[1]), pack_bf16x2(dsx[2], dsx[3]),
                                pack_bf16x2(dsx[4], dsx[5]), pack_bf16x2(dsx[6], dsx[7]));
    // the summary operand: ds of row p in column (head) p % G
    const bool summ = full_chunk && (n + 1) * kTR > br.nwin;
    uint4 dsh = make_uint4(0u, 0u, 0u, 0u);
    if (summ) {
      float hv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int p = 8 * lg + e;
        hv[e] = (ln < G && (p % G) == ln) ? sm.dsv[mb][p] : 0.f;
      }
      dsh = make_uint4(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]), pack_bf16x2(hv[4], hv[5]),
                       pack_bf16x2(hv[6], hv[7]));
    }
    // ---- dV^T += dO^T P, dK^T += Q^T dS (and the summary's Q^T DS)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint4 ao = *reinterpret_cast<const uint4 *>(&sm.u.t.dot[buf][16 * dt + ln][8 * lg]);
      const uint4 aq = *reinterpret_cast<const uint4 *>(&sm.u.t.qt[buf][16 * dt + ln][8 * lg]);
      dv[dt] = mfma_k(ao, pb, dv[dt]);
      dk[dt] = mfma_k(aq, db, dk[dt]);
    }
    // the wave's DTW d tiles of the summary product (dsh is zero on the
    // tiles without chunk entries, so the product may run there too)
    if (summ) {
#pragma unroll
      for (int x = 0; x < DTW; ++x) {
        const uint4 aq = *reinterpret_cast<const uint4 *>(&sm.u.t.qt[buf][16 * (DTW * w + x) + ln][8 * lg]);
        dkq[x] = mfma_k(aq, dsh, dkq[x]);
      }
    }
    if (n + 1 < ntiles) store_tile(buf ^ 1);
    if (meta_next) store_meta(nm, (n + 2) % 3);
    __syncthreads();
  }
  // ---- outputs: dV^T accumulator element j of tile dt is d = 16 dt + 4 lg + j, key 16 w + ln
  if (key < T_len) {
    float *dvo = a.dv + (pg * T_len + key) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4 *>(dvo + 16 * dt + 4 * lg) = make_float4(dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]);
  }
  if (!full_chunk) {
    if (key < T_len) {
      float *dko = a.dk + (pg * T_len + key) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<float4 *>(dko + 16 * dt + 4 * lg) =
            make_float4(dk[dt][0], dk[dt][1], dk[dt][2], dk[dt][3]);
    }
    return;  // uniform: the whole workgroup
  }
  // ---- the chunk's summary backward (fp32), on the thread-per-(key, quarter) layout
  // (the tile buffers are free: the last loop iteration ended with a barrier)
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const uint32_t kw[4] = {kop[s].x, kop[s].y, kop[s].z, kop[s].w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      sm.u.e.kt[16 * w + ln][32 * s + 8 * lg + e] = bf16_to_f32(static_cast<uint16_t>(kw[e >> 1] >> (16 * (e & 1))));
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int jx = 0; jx < 4; ++jx) sm.u.e.dkb[16 * w + ln][16 * dt + 4 * lg + jx] = dk[dt][jx];
  // Q^T DS accumulator of d tile dt = DTW w + x: element j is d = 16 dt + 4 lg + j, head ln
#pragma unroll
  for (int x = 0; x < DTW; ++x)
#pragma unroll
    for (int jx = 0; jx < 4; ++jx)
      if (ln < G) sm.u.e.dkp[ln][16 * (DTW * w + x) + 4 * lg + jx] = tau * dkq[x][jx];
  __syncthreads();
  constexpr int QD = D / 4;
  const int jk = t >> 2, qd = t & 3;
  float kr[QD], dkr[QD];
#pragma unroll
  for (int u = 0; u < QD; ++u) {
    kr[u] = sm.u.e.kt[jk][qd * QD + u];
    dkr[u] = sm.u.e.dkb[jk][qd * QD + u];
  }
  bwd::summary_backward<uint16_t, D>(a, b, g, kb, sm.u.e.kt, kr, dkr, sm.u.e.dkp, sm.ss);
  float *dko = a.dk + (pg * T_len + j0 + jk) * D + qd * QD;
#pragma unroll
  for (int u = 0; u < QD; u += 4) *reinterpret_cast<float4 *>(dko + u) = make_float4(dkr[u], dkr[u + 1], dkr[u + 2], dkr[u + 3]);
}

// ------------------------------------------------------------------ rows (MFMA)
// The query-major pass on the matrix cores: one workgroup per 16 / G
// consecutive queries of group g and batch b, their G heads the 16 columns of
// one tile (column = query i0 + col / G, head col % G).  The workgroup's
// blocks -- the union of its queries' selected chunks, each staged once, then
// the 64-key blocks covering their windows -- are staged in LDS one at a
// time (K row-major, V row-major, K^T), the next block's loads in flight
// while the current one computes; a column takes a chunk block only if its
// query selected that chunk, and from a window block only the keys of its
// own window.
// Wave w takes keys 16 w .. 16 w + 15 of each block:
//   S^T = K Q^T, dP^T = V dO^T        16x16x32 bf16, keys in M, heads in N
// and accumulates, per head, running sums over its own keys against one
// running reference R (the largest chunk score, raised by window logits
// past it):
//   V1 = sum_c e^{s_c - R} / Z_c sum_j e^{l_j - m_c} (dO.v_j - dO.o_c) k_j
//        + sum_window e^{l_j - R} dO.v_j k_j,
//   A2 = sum_window e^{l_j - R} k_j
// as K^T times a weight column: 16x16x16 bf16 products whose B operand is
// the lane's own accumulator entries (keys 4 lg .. 4 lg + 3 of column ln).
// The window weights enter as bf16 hi + lo pairs (V1 - Delta A2 cancels when
// the row's attention is sharp), the chunk weights, already differences, as
// one bf16 value.  A chunk's maximum, sum and dO.o_c are combined over the
// four waves through LDS; at the end the waves' window states and vectors
// are combined in wave order, so the result is the same on every run:
//   dq = tau sum_w e^{R_w - logZ} (V1_w - Delta A2_w) + dq_hat.
namespace {

typedef short bf16x4r __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4k mfma_16(const uint2 &a, const uint2 &b, const f32x4k &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4r, a), __builtin_bit_cast(bf16x4r, b), c,
                                                   0, 0, 0);
}

// bf16 hi part (round to nearest even) and the bf16 rounding of the rest
__device__ __forceinline__ void split_bf16(const float (&x)[4], uint2 &hi, uint2 &lo) {
  hi = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
  const float r0 = x[0] - __uint_as_float(hi.x << 16), r1 = x[1] - __uint_as_float(hi.x & 0xFFFF0000u);
  const float r2 = x[2] - __uint_as_float(hi.y << 16), r3 = x[3] - __uint_as_float(hi.y & 0xFFFF0000u);
  lo = make_uint2(pack_bf16x2(r0, r1), pack_bf16x2(r2, r3));
}

constexpr int kRP = 8;   // row-major tiles: rows D + 8 elements apart
constexpr int kTQ = 72;  // K^T tile: 64 keys + 8 per d row

template <int D>
struct alignas(16) RmTiles {
  uint16_t kr[kBK][D + kRP];
  uint16_t vr[kBK][D + kRP];
  uint16_t kt[D][kTQ];
};
template <int D, int QPW>
struct alignas(16) RmSmem {
  union {
    RmTiles<D> t;
    float vec[4][16][D + 4];  // the waves' row vectors for the final sum
  } u;
  float red[4][16][3];        // per wave and column: a chunk's max, sum, sum e dO.v over the wave's keys
  float fin[4][16][3];        // per wave and column: the window's max, sum, sum e dO.v
  float sl_s[32][16], sl_m[32][16], sl_z[32][16], sl_doo[32][16];  // per slot of the column's query, and column
  float row_lz[16], row_dl[16], row_mc[16];
  int sel[QPW][32];                            // each query's chunk per slot (-1: none)
  uint32_t umask[kMaxBwdChunks / 32];          // the chunks any query of the workgroup selected
  int wbase[kMaxBwdChunks / 32];
  int16_t ulist[kMaxBwdChunks];                // those chunks, ascending
  int8_t uslot[kMaxBwdChunks][16];             // per union chunk and column: the slot in the column's query's list, or -1
  int16_t blk[2 * kMaxBwdChunks + 4];          // staged blocks: union chunk u, or -1 - window block
  int nblk, nunion;
};

}  // namespace

template <int D, int G, bool QCAL>
__global__ void __launch_bounds__(256, 2)
bwd_rows_mfma_kernel(BwdArgs a) {
  constexpr int QPW = 16 / G;  // queries per workgroup: their G heads fill the tile's 16 columns
  __shared__ RmSmem<D, QPW> sm;
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int NKI = D / 64;  // (row pair, 8-element piece) items of K per thread; V: 2 NKI rows
  const int i0 = blockIdx.x * QPW, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), ln = lane & 15, lg = lane >> 4;
  const int T_len = a.T, K = a.K, Hq = a.Hq, Hkv = a.Hkv, C = T_len / kBK;
  const float tau = a.tau;
  // column ln of the tile: query i0 + ln / G, head ln % G (a query past T
  // is no query: it reads the last row and stores nothing); its window is
  // the keys [wlo_c, ic]
  const int cq = ln / G, ch = ln % G, ic = i0 + cq;
  const bool col_ok = ic < T_len;
  const int icc = col_ok ? ic : T_len - 1;
  const int wlo_c = eligible_chunks(icc, a.W, kBK) * kBK;
  // the workgroup's window blocks: from the first query's window start (the
  // smallest) to its last query
  const int i_last = min(i0 + QPW - 1, T_len - 1);
  const int w_lo = eligible_chunks(i0, a.W, kBK) * kBK;
  const int nwb = (i_last - w_lo) / kBK + 1;
  const size_t pg = static_cast<size_t>(b) * Hkv + g;
  const uint16_t *kg = static_cast<const uint16_t *>(a.k) + pg * T_len * D;
  const uint16_t *vg = static_cast<const uint16_t *>(a.v) + pg * T_len * D;
  const uint16_t *ksum = static_cast<const uint16_t *>(a.k_sum);
  // ---- each query's chunks, their union (each staged once), and per union
  // chunk and column the slot that chunk has in the column's query's list
  for (int x = t; x < QPW * 32; x += kBT) {
    const int q = x / 32, y = x % 32, iq = i0 + q;
    int c = -1;
    if (y < K && iq < T_len) {
      c = a.topk_idx[(pg * T_len + iq) * K + y];
      if (c < 0 || c >= eligible_chunks(iq, a.W, kBK)) c = -1;
    }
    sm.sel[q][y] = c;
  }
  for (int x = t; x < kMaxBwdChunks / 32; x += kBT) sm.umask[x] = 0u;
  for (int x = t; x < kMaxBwdChunks * 16 / 4; x += kBT) reinterpret_cast<int *>(&sm.uslot[0][0])[x] = -1;
  __syncthreads();
  for (int x = t; x < QPW * 32; x += kBT) {
    const int c = sm.sel[x / 32][x % 32];
    if (c >= 0) atomicOr(&sm.umask[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  if (t < 64) {  // union positions in ascending chunk order: prefix over the mask words (C <= 512)
    const int nw = (C + 31) >> 5;
    const uint32_t bits = t < nw ? sm.umask[t] : 0u;
    const int cnt = __popc(bits);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (t >= o) incl += y;
    }
    if (t < nw) sm.wbase[t] = incl - cnt;
    if (t == 63) sm.nunion = incl;
  }
  __syncthreads();
  for (int x = t; x < QPW * 32; x += kBT) {
    const int q = x / 32, y = x % 32, c = sm.sel[q][y];
    if (c >= 0) {
      const int u = sm.wbase[c >> 5] + __popc(sm.umask[c >> 5] & ((1u << (c & 31)) - 1u));
      sm.ulist[u] = static_cast<int16_t>(c);  // (the same value from every query that holds c)
#pragma unroll
      for (int h = 0; h < G; ++h) sm.uslot[u][q * G + h] = static_cast<int8_t>(y);
    }
  }
  const int nu = sm.nunion;
  for (int x = t; x < nu + nwb; x += kBT) sm.blk[x] = static_cast<int16_t>(x < nu ? x : -1 - (x - nu));
  // ---- the chunk scores s_hat = tau q_hat . k'_c + b'_c per (slot, column)
  for (int x = t; x < K * 16; x += kBT) {
    const int slot = x / 16, col = x % 16, q = col / G, hh = col % G, iq = i0 + q;
    const int c = iq < T_len ? sm.sel[q][slot] : -1;
    float s = -INFINITY;
    if (c >= 0) {
      const size_t ro = (static_cast<size_t>(b) * Hq + g * G + hh) * T_len + iq;
      const size_t so = (static_cast<size_t>(b) * Hq + g * G + hh) * C + c;
      float acc = 0.f;
      for (int e = 0; e < D; e += 8) {
        float kv[8];
        Elem<uint16_t>::load8(ksum + so * D + e, kv);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          acc += (QCAL ? a.qhat[ro * D + e + u] : bf16_to_f32(static_cast<const uint16_t *>(a.q)[ro * D + e + u])) * kv[u];
      }
      s = tau * acc + a.b_sum[so];
    }
    sm.sl_s[slot][col] = s;
  }
  __syncthreads();
  const int nb = nu + nwb;
  // this lane's column and its largest chunk score
  float Mc = -INFINITY;
  for (int x = 0; x < K; ++x) Mc = fmaxf(Mc, sm.sl_s[x][ln]);
  // Q and dO of the lane's column as B operands: d = 32 s + 8 lg .. + 8
  uint4 qop[KS], dop[KS];
  {
    const size_t ro = (static_cast<size_t>(b) * Hq + g * G + ch) * T_len + icc;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qop[s] = col_ok ? *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + ro * D + 32 * s + 8 * lg)
                      : make_uint4(0u, 0u, 0u, 0u);
      dop[s] = col_ok ? *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.d_o) + ro * D + 32 * s + 8 * lg)
                      : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // ---- staging: item it of K -> rows 2 pp, 2 pp + 1, piece s; V rows plain
  uint4 kst[NKI][2], vst[2 * NKI];
  auto block_j0 = [&](int x) { const int bb = sm.blk[x]; return bb >= 0 ? sm.ulist[bb] * kBK : w_lo - (1 + bb) * kBK; };
  auto load_block = [&](int j0) {
#pragma unroll
    for (int it = 0; it < NKI; ++it) {
      const int x = t + kBT * it, pp = x & 31, s = x >> 5;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int r = j0 + 2 * pp + h2;
        kst[it][h2] = r < T_len ? *reinterpret_cast<const uint4 *>(kg + static_cast<size_t>(r) * D + 8 * s)
                                : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int it = 0; it < 2 * NKI; ++it) {
      const int x = t + kBT * it, r = x / (D / 8), s = x % (D / 8);
      vst[it] = j0 + r < T_len ? *reinterpret_cast<const uint4 *>(vg + static_cast<size_t>(j0 + r) * D + 8 * s)
                               : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int it = 0; it < NKI; ++it) {
      const int x = t + kBT * it, pp = x & 31, s = x >> 5;
      *reinterpret_cast<uint4 *>(&sm.u.t.kr[2 * pp][8 * s]) = kst[it][0];
      *reinterpret_cast<uint4 *>(&sm.u.t.kr[2 * pp + 1][8 * s]) = kst[it][1];
      const uint32_t r0[4] = {kst[it][0].x, kst[it][0].y, kst[it][0].z, kst[it][0].w};
      const uint32_t r1[4] = {kst[it][1].x, kst[it][1].y, kst[it][1].z, kst[it][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (r0[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, hi = (r1[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        *reinterpret_cast<uint32_t *>(&sm.u.t.kt[8 * s + e][2 * pp]) = lo | (hi << 16);
      }
    }
#pragma unroll
    for (int it = 0; it < 2 * NKI; ++it) {
      const int x = t + kBT * it, r = x / (D / 8), s = x % (D / 8);
      *reinterpret_cast<uint4 *>(&sm.u.t.vr[r][8 * s]) = vst[it];
    }
  };

  f32x4k V1[DT], A2[DT];
#pragma unroll
  for (int x = 0; x < DT; ++x) V1[x] = A2[x] = f32x4k{0.f, 0.f, 0.f, 0.f};
  // this wave's reference and window sums for head ln (relative to R)
  float R = Mc, zw = 0.f, dw = 0.f;
  if (nb > 0) {
    load_block(block_j0(0));
    store_block();
  }
  __syncthreads();
  for (int x = 0; x < nb; ++x) {
    const int bb = sm.blk[x];
    const bool chunk = bb >= 0;
    const int j0 = block_j0(x);
    if (x + 1 < nb) load_block(block_j0(x + 1));
    // ---- S^T and dP^T of keys 16 w .. 16 w + 15
    f32x4k sacc = f32x4k{0.f, 0.f, 0.f, 0.f}, pacc = f32x4k{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 ak = *reinterpret_cast<const uint4 *>(&sm.u.t.kr[16 * w + ln][32 * s + 8 * lg]);
      const uint4 av = *reinterpret_cast<const uint4 *>(&sm.u.t.vr[16 * w + ln][32 * s + 8 * lg]);
      sacc = mfma_k(ak, qop[s], sacc);
      pacc = mfma_k(av, dop[s], pacc);
    }
    // element jx: key 16 w + 4 lg + jx of the block, head ln
    float l[4], dv[4];
#pragma unroll
    for (int jx = 0; jx < 4; ++jx) {
      l[jx] = tau * sacc[jx];
      dv[jx] = pacc[jx];
    }
    if (chunk) {
      float m = fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3]));
      m = max_rows4(m);
      float z = 0.f, dz = 0.f;
#pragma unroll
      for (int jx = 0; jx < 4; ++jx) {
        const float e = __expf(l[jx] - m);
        z += e;
        dz += e * dv[jx];
      }
      z = sum_rows4(z);
      dz = sum_rows4(dz);
      if (lg == 0) {
        sm.red[w][ln][0] = m;
        sm.red[w][ln][1] = z;
        sm.red[w][ln][2] = dz;
      }
      __syncthreads();
      // the chunk's statistics for column ln, combined over the waves in order
      float mc = sm.red[0][ln][0];
#pragma unroll
      for (int v = 1; v < 4; ++v) mc = fmaxf(mc, sm.red[v][ln][0]);
      float zc = 0.f, dzc = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float f = __expf(sm.red[v][ln][0] - mc);
        zc += f * sm.red[v][ln][1];
        dzc += f * sm.red[v][ln][2];
      }
      const float doo = dzc / zc;
      const int slot = sm.uslot[bb][ln];  // the chunk's slot in column ln's list; -1: not selected there
      if (w == 0 && lg == 0 && slot >= 0) {
        sm.sl_m[slot][ln] = mc;
        sm.sl_z[slot][ln] = zc;
        sm.sl_doo[slot][ln] = doo;
      }
      // (R >= s_hat of every selected chunk of column ln; a column that did
      // not select the chunk: weight 0)
      const float wgt = slot >= 0 ? __expf(sm.sl_s[slot][ln] - R) / zc : 0.f;
      float ed[4];
#pragma unroll
      for (int jx = 0; jx < 4; ++jx) ed[jx] = __expf(l[jx] - mc) * wgt * (dv[jx] - doo);
      const uint2 eb = make_uint2(pack_bf16x2(ed[0], ed[1]), pack_bf16x2(ed[2], ed[3]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 akt = *reinterpret_cast<const uint2 *>(&sm.u.t.kt[16 * dt + ln][16 * w + 4 * lg]);
        V1[dt] = mfma_16(akt, eb, V1[dt]);
      }
    } else {
      // keys of column ln's window, [wlo_c, ic]
      float lm[4];
      float mb = -INFINITY;
#pragma unroll
      for (int jx = 0; jx < 4; ++jx) {
        const int j = j0 + 16 * w + 4 * lg + jx;
        lm[jx] = (col_ok && j >= wlo_c && j <= ic) ? l[jx] : -INFINITY;
        mb = fmaxf(mb, lm[jx]);
      }
      mb = max_rows4(mb);
      const float rn = fmaxf(R, mb);
      // No branch around the update: the matrix products run for every
      // column whatever EXEC holds, so a column without keys in this block
      // (mb = -inf) takes weights 0 and rescale 1 and keeps its state.
      {
        const float sc = mb == -INFINITY ? 1.f : (R == -INFINITY ? 0.f : __expf(R - rn));
        float e[4], ed[4], ze = 0.f, zd = 0.f;
#pragma unroll
        for (int jx = 0; jx < 4; ++jx) {
          e[jx] = lm[jx] == -INFINITY ? 0.f : __expf(lm[jx] - rn);
          ed[jx] = e[jx] * dv[jx];
          ze += e[jx];
          zd += ed[jx];
        }
        zw = zw * sc + sum_rows4(ze);
        dw = dw * sc + sum_rows4(zd);
        R = rn;
        if (sc != 1.f) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            V1[dt] *= sc;
            A2[dt] *= sc;
          }
        }
        uint2 eh, el, dh, dl;
        split_bf16(e, eh, el);
        split_bf16(ed, dh, dl);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint2 akt = *reinterpret_cast<const uint2 *>(&sm.u.t.kt[16 * dt + ln][16 * w + 4 * lg]);
          V1[dt] = mfma_16(akt, dh, V1[dt]);
          V1[dt] = mfma_16(akt, dl, V1[dt]);
          A2[dt] = mfma_16(akt, eh, A2[dt]);
          A2[dt] = mfma_16(akt, el, A2[dt]);
        }
      }
    }
    __syncthreads();  // every wave is done with this block's tiles
    if (x + 1 < nb) store_block();
    __syncthreads();
  }
  // ---- the joint normaliser and Delta per head
  if (lg == 0) {
    sm.fin[w][ln][0] = R;
    sm.fin[w][ln][1] = zw;
    sm.fin[w][ln][2] = dw;
  }
  __syncthreads();
  if (t < 16) {  // column t: query i0 + t / G, head t % G
    const int col = t, q = t / G, hh = t % G, iq = i0 + q;
    float mc = -INFINITY;
    for (int x = 0; x < K; ++x) mc = fmaxf(mc, sm.sl_s[x][col]);
    float M = mc;
#pragma unroll
    for (int v = 0; v < 4; ++v) M = fmaxf(M, sm.fin[v][col][0]);
    float z = 0.f;
    for (int x = 0; x < K; ++x)
      if (sm.sel[q][x] >= 0) z += __expf(sm.sl_s[x][col] - M);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (sm.fin[v][col][0] != -INFINITY) z += sm.fin[v][col][1] * __expf(sm.fin[v][col][0] - M);
    const float lz = M + __logf(z);
    float dl = 0.f;
    for (int x = 0; x < K; ++x)
      if (sm.sel[q][x] >= 0) dl += __expf(sm.sl_s[x][col] - lz) * sm.sl_doo[x][col];
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (sm.fin[v][col][0] != -INFINITY) dl += sm.fin[v][col][2] * __expf(sm.fin[v][col][0] - lz);
    sm.row_lz[col] = lz;
    sm.row_dl[col] = dl;
    sm.row_mc[col] = mc;
    if (iq < T_len) {
      const size_t ro = (static_cast<size_t>(b) * Hq + g * G + hh) * T_len + iq;
      a.logz[ro] = lz;
      a.delta[ro] = dl;
    }
  }
  __syncthreads();
  // ---- each wave's row vectors into LDS (element j of d tile dt: d = 16 dt + 4 lg + j, head ln)
  {
    const float lz = sm.row_lz[ln], dl = sm.row_dl[ln];
    const float f = R == -INFINITY ? 0.f : __expf(R - lz);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jx = 0; jx < 4; ++jx) sm.u.vec[w][ln][16 * dt + 4 * lg + jx] = f * (V1[dt][jx] - dl * A2[dt][jx]);
  }
  __syncthreads();
  // ---- dq and dq_hat per (head, d); the list entries' values
  for (int x = t; x < 16 * D; x += kBT) {
    const int col = x / D, e = x % D, q = col / G, hh = col % G, iq = i0 + q, h = g * G + hh;
    if (iq >= T_len) continue;
    const float lz = sm.row_lz[col], dl = sm.row_dl[col], mc = sm.row_mc[col];
    float b1 = 0.f, b2 = 0.f;
    for (int y = 0; y < K; ++y) {
      const int c = sm.sel[q][y];
      if (c < 0) continue;
      const float sw = __expf(sm.sl_s[y][col] - mc);
      const float kp = bf16_to_f32(ksum[((static_cast<size_t>(b) * Hq + h) * C + c) * D + e]);
      b1 += sw * sm.sl_doo[y][col] * kp;
      b2 += sw * kp;
    }
    const float fc = mc == -INFINITY ? 0.f : __expf(mc - lz);
    const float dqh = tau * fc * (b1 - dl * b2);
    const float v = sm.u.vec[0][col][e] + sm.u.vec[1][col][e] + sm.u.vec[2][col][e] + sm.u.vec[3][col][e];
    const size_t ro = (static_cast<size_t>(b) * Hq + h) * T_len + iq;
    a.dq[ro * D + e] = tau * v + dqh;
    if (QCAL) a.dqhat[((static_cast<size_t>(b) * T_len + iq) * Hq + h) * D + e] = dqh;
  }
  for (int x = t; x < QPW * K * G; x += kBT) {
    const int q = x / (K * G), y = (x / G) % K, hh = x % G, col = q * G + hh, iq = i0 + q;
    if (iq >= T_len || sm.sel[q][y] < 0) continue;
    const int pos = a.inv_pos[(pg * T_len + iq) * K + y];
    const size_t eo = (pg * T_len * K + pos) * G + hh;
    const float lz = sm.row_lz[col];
    a.ent_lw[eo] = sm.sl_s[y][col] - lz - sm.sl_m[y][col] - __logf(sm.sl_z[y][col]);
    a.ent_doo[eo] = sm.sl_doo[y][col];
    a.ent_ds[eo] = __expf(sm.sl_s[y][col] - lz) * (sm.sl_doo[y][col] - sm.row_dl[col]);
  }
}

bool bwd_rows_mfma_supported(const BwdArgs &a) { return bwd_keys_mfma_supported(a); }

template <int D, int G>
static hipError_t rows_dg(const BwdArgs &a, hipStream_t st) {
  const dim3 grid((a.T + 16 / G - 1) / (16 / G), a.Hkv, a.B);  // 16 / G queries per workgroup
  if (a.r > 0)
    bwd_rows_mfma_kernel<D, G, true><<<grid, kBT, 0, st>>>(a);
  else
    bwd_rows_mfma_kernel<D, G, false><<<grid, kBT, 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
static hipError_t rows_d(const BwdArgs &a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return rows_dg<D, 1>(a, st);
    case 2: return rows_dg<D, 2>(a, st);
    case 4: return rows_dg<D, 4>(a, st);
    case 8: return rows_dg<D, 8>(a, st);
    default: return rows_dg<D, 16>(a, st);
  }
}

hipError_t launch_bwd_rows_mfma(const BwdArgs &a, hipStream_t st) {
  return a.d == 128 ? rows_d<128>(a, st) : rows_d<64>(a, st);
}

bool bwd_keys_mfma_supported(const BwdArgs &a) {
  const int G = a.Hq / a.Hkv;
  return a.bf16 && (a.d == 64 || a.d == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

template <int D>
static hipError_t keys_d(const BwdArgs &a, hipStream_t st) {
  const dim3 grid(a.B * a.Hkv, (a.T + kBK - 1) / kBK);
  switch (a.Hq / a.Hkv) {
    case 1: bwd_keys_mfma_kernel<D, 1><<<grid, kBT, 0, st>>>(a); break;
    case 2: bwd_keys_mfma_kernel<D, 2><<<grid, kBT, 0, st>>>(a); break;
    case 4: bwd_keys_mfma_kernel<D, 4><<<grid, kBT, 0, st>>>(a); break;
    case 8: bwd_keys_mfma_kernel<D, 8><<<grid, kBT, 0, st>>>(a); break;
    default: bwd_keys_mfma_kernel<D, 16><<<grid, kBT, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_keys_mfma(const BwdArgs &a, hipStream_t st) {
  return a.d == 128 ? keys_d<128>(a, st) : keys_d<64>(a, st);
}

}  // namespace hils
