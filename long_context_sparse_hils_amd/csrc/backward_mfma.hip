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
