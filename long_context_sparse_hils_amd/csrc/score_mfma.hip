// Prefill chunk scoring with Q-Cal and GQA top-K on the MFMA units --
// HiLS-Attention, picx.dev summary, Eq. 7 with Eq. 10's s-hat, Methodology 3
// (Q-Cal: q-hat = q + W_up W_down h; GQA: max over the group's heads), and
// the rcap.io pseudo-code's arg-top-K.
//
// The Q-Cal term is regrouped so that every product is a bf16 MFMA:
//   s = tau * (q . k' + u . m) + b',   u = W_down h (per token, r values),
//                                      m = W_up[h*d:(h+1)*d, :]^T k' (per head and chunk)
// q and k' are bf16 inputs (exact products); u and m are fp32 values carried
// as bf16 hi + lo pairs (u ~= u_hi + u_lo to ~2^-16 relative), multiplied as
// hi*hi + hi*lo + lo*hi.
//
// Kernels:
//   qcal_u_mfma      u[token, a]   MFMA GEMM over D_h  -> u_hi/u_lo [B*T, RP]
//   qcal_m           m[b, h, c, a] VALU (tiny)          -> m_hi/m_lo [B, Hq, C, RP]
//   score_topk_mfma  per (128 queries, KV head, batch), 8 waves of 16 queries,
//                    the latest (heaviest) query blocks first: items of 64
//                    chunks x one head of k', m and b' are staged once in LDS
//                    for all waves (double buffered, loaded straight from
//                    global memory); each wave forms S^T tiles of 16 chunks x
//                    16 queries per head.  Groups of at most 4 heads keep
//                    every head's score in registers (one pass); larger
//                    groups keep the group maximum and recompute the
//                    winners' per-head scores in a second pass (the same
//                    arithmetic, bit-identical).  Per query, a bitwise search
//                    for the K-th largest group score (counts from row sums
//                    of the 4 lanes of a query) and a rank pass order the
//                    winners by (score desc, chunk asc).
#include <type_traits>

#include "hils_common.h"
#include "launch.h"

namespace hils {

typedef __bf16 bf16x8s __attribute__((ext_vector_type(8)));
typedef float f32x4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4s mfma_s(const uint4 &a, const uint4 &b, const f32x4s &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8s, a), __builtin_bit_cast(bf16x8s, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ void split_bf16(float x, uint16_t &hi, uint16_t &lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// ------------------------------------------------------------------ u = W_down h
// A streaming GEMM over D_h: h (B*T x D_h) is read once and is the whole HBM
// traffic; W_down (r x D_h) is re-read from L2 by every workgroup.  One
// workgroup per 16 TT tokens; its 4 waves take quarters of D_h and add their
// partial (16 TT) x RP tiles through LDS.  Each wave holds TT token tiles,
// so one W_down operand serves TT MFMAs: the vector-memory requests, not
// HBM, bound this kernel, and W_down's share of them falls as 1 / TT.
template <int NT, int TT>  // output tiles of 16 (RP / 16); token tiles per wave
__device__ __forceinline__ void qcal_u_block(const uint16_t *__restrict__ h, const uint16_t *__restrict__ w_down,
                                             uint16_t *__restrict__ u_hi, uint16_t *__restrict__ u_lo, int Ntok, int r,
                                             int Dh, int bx, float (&part)[4][16 * TT][16 * NT + 1]) {
  constexpr int RP = 16 * NT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int tok0 = bx * 16 * TT;
  const uint16_t *hrow[TT];
  bool tok_ok[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    tok_ok[t] = tok0 + 16 * t + ln < Ntok;
    hrow[t] = h + static_cast<size_t>(tok_ok[t] ? tok0 + 16 * t + ln : 0) * Dh + 8 * lg;
  }
  const uint16_t *wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    wrow[nt] = 16 * nt + ln < r ? w_down + static_cast<size_t>(16 * nt + ln) * Dh + 8 * lg : nullptr;
  f32x4s acc[TT][NT];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[t][nt] = f32x4s{0.f, 0.f, 0.f, 0.f};
  // the wave's quarter of the 32-wide k-steps: a lane reads 16 bytes, the 4
  // lanes of a row 64 contiguous bytes per load
  const int nst = Dh / 32;
  const int s0 = nst * wave / 4, s1 = nst * (wave + 1) / 4;
  int s = s0;
  for (; s + 4 <= s1; s += 4) {
    uint4 av[4][TT], bv[4][NT];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 32 * (s + j);
#pragma unroll
      for (int t = 0; t < TT; ++t)
        av[j][t] = tok_ok[t] ? *reinterpret_cast<const uint4 *>(hrow[t] + e) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bv[j][nt] = wrow[nt] ? *reinterpret_cast<const uint4 *>(wrow[nt] + e) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[t][nt] = mfma_s(av[j][t], bv[j][nt], acc[t][nt]);
  }
  for (; s < s1; ++s) {
    const int e = 32 * s;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const uint4 av = tok_ok[t] ? *reinterpret_cast<const uint4 *>(hrow[t] + e) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[t][nt] = mfma_s(av, wrow[nt] ? *reinterpret_cast<const uint4 *>(wrow[nt] + e) : make_uint4(0, 0, 0, 0),
                            acc[t][nt]);
    }
  }
  // D[m = token 16 t + 4 lg + q][n = a = 16 nt + ln]
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) part[wave][16 * t + 4 * lg + q][16 * nt + ln] = acc[t][nt][q];
  __syncthreads();
  for (int x = threadIdx.x; x < 16 * TT * RP; x += 256) {
    const int tk = x / RP, aa = x % RP;
    if (tok0 + tk < Ntok) {
      const float v = (part[0][tk][aa] + part[1][tk][aa]) + (part[2][tk][aa] + part[3][tk][aa]);
      uint16_t hi, lo;
      split_bf16(v, hi, lo);
      const size_t o = static_cast<size_t>(tok0 + tk) * RP + aa;
      u_hi[o] = hi;
      u_lo[o] = lo;
    }
  }
}

// ------------------------------------------------------------------ m = W_up_h^T k'
// One workgroup per (32 chunks, query head, batch); W_up's head slice and
// the 32 summaries in LDS.  Thread (chunk t / 8, a4 = t % 8) forms the
// outputs a = 32 j + 4 a4 .. + 4 of its chunk.
template <int D>
struct QcalMSmem {
  float4 wu[D][16];  // [e][a / 4], zero for a >= r
  float kc[32][D + 1];
};
template <int D>
__device__ __forceinline__ void qcal_m_block(const uint16_t *__restrict__ k_sum, const uint16_t *__restrict__ w_up,
                                             uint16_t *__restrict__ m_hi, uint16_t *__restrict__ m_lo, int Hq, int C,
                                             int r, int RP, int bx, int h, int b, QcalMSmem<D> &ms) {
  float4 (&wu)[D][16] = ms.wu;
  float (&kc)[32][D + 1] = ms.kc;
  const int c0 = bx * 32, t = threadIdx.x;
  // The head's W_up slice (D x r, contiguous) and the 32 summaries
  // (32 x D, contiguous) are read with 16-byte loads, all issued before any
  // is used.
  constexpr int KV = 32 * D / 8 / 256;  // 16-byte pieces of k' per thread
  const int nw = D * r / 8;             // 16-byte pieces of the W_up slice (D is a multiple of 8)
  const uint16_t *wsl = w_up + static_cast<size_t>(h) * D * r;
  const uint16_t *ksl = k_sum + ((static_cast<size_t>(b) * Hq + h) * C + c0) * D;
  uint4 wv[4], kv[KV];  // nw <= D * 64 / 8 = 4 * 256 pieces for D = 128
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = t + 256 * j;
    wv[j] = x < nw ? *reinterpret_cast<const uint4 *>(wsl + 8 * x) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < KV; ++j) {
    const int x = t + 256 * j;
    kv[j] = c0 + (8 * x) / D < C ? *reinterpret_cast<const uint4 *>(ksl + 8 * x) : make_uint4(0, 0, 0, 0);
  }
  float *wuf = reinterpret_cast<float *>(&wu[0][0]);
  for (int x = t; x < D * 16; x += 256) wu[x / 16][x % 16] = make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = t + 256 * j;
    if (x < nw) {
      const uint32_t w4[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int flat = 8 * x + q, e = flat / r, aa = flat - e * r;
        wuf[e * 64 + aa] = bf16_to_f32(static_cast<uint16_t>(w4[q >> 1] >> (16 * (q & 1))));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KV; ++j) {
    const int x = t + 256 * j, cc = (8 * x) / D, e = (8 * x) % D;
    const uint32_t k4[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
#pragma unroll
    for (int q = 0; q < 8; ++q) kc[cc][e + q] = bf16_to_f32(static_cast<uint16_t>(k4[q >> 1] >> (16 * (q & 1))));
  }
  __syncthreads();
  const int cc = t >> 3, a4 = t & 7;
  if (c0 + cc >= C) return;
  const int NJ = RP / 32;
  float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 4
  for (int e = 0; e < D; ++e) {
    const float kv = kc[cc][e];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j < NJ) {
        const float4 w = wu[e][8 * j + a4];
        acc[j][0] += w.x * kv;
        acc[j][1] += w.y * kv;
        acc[j][2] += w.z * kv;
        acc[j][3] += w.w * kv;
      }
    }
  }
  const size_t o = ((static_cast<size_t>(b) * Hq + h) * C + c0 + cc) * RP;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j < NJ) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint16_t hi, lo;
        split_bf16(acc[j][q], hi, lo);
        m_hi[o + 32 * j + 4 * a4 + q] = hi;
        m_lo[o + 32 * j + 4 * a4 + q] = lo;
      }
    }
  }
}

// Both Q-Cal products in one launch: workgroups [0, nub) form u, the rest m
// (gmx chunk blocks x Hq x B).  The two are independent, so m's workgroups
// run beside u's stream instead of after it.
template <int NT, int TT, int D>
__global__ void __launch_bounds__(256, 3)
qcal_kernel(const uint16_t *__restrict__ h, const uint16_t *__restrict__ w_down, uint16_t *__restrict__ u_hi,
            uint16_t *__restrict__ u_lo, int Ntok, int Dh, const uint16_t *__restrict__ k_sum,
            const uint16_t *__restrict__ w_up, uint16_t *__restrict__ m_hi, uint16_t *__restrict__ m_lo, int Hq, int C,
            int r, int nub, int gmx) {
  __shared__ union {
    float part[4][16 * TT][16 * NT + 1];
    QcalMSmem<D> m;
  } sm;
  const int bx = blockIdx.x;
  if (bx < nub) {
    qcal_u_block<NT, TT>(h, w_down, u_hi, u_lo, Ntok, r, Dh, bx, sm.part);
  } else {
    const int y = bx - nub;
    qcal_m_block<D>(k_sum, w_up, m_hi, m_lo, Hq, C, r, 16 * NT, y % gmx, (y / gmx) % Hq, y / (gmx * Hq), sm.m);
  }
}

// ------------------------------------------------------------------ scores + top-K
constexpr int kScoreMaxC = 256;

// Shared memory of the score kernel: two staged items, then per wave the
// selection scratch.  An item holds one head's summaries k' (IC rows of D),
// Q-Cal projections m hi/lo (IC rows of RP) and entropies b' (IC floats) for
// IC consecutive chunks.  Rows of P 16-byte pieces are XOR-swizzled so that
// the 16 rows one MFMA operand read touches fall in 16 different bank groups.
template <int D, int NJ, int WAVES>
struct ScoreSelect {
  unsigned long long win[WAVES][16][32];  // per query: its winners' sort keys, compacted
  int8_t rtab[WAVES][16][64 * NJ]; // winner chunk -> its position in the query's list
};
struct ScoreItemLayout {
  int ks, mh, ml, bs, bytes;  // byte offsets inside one item, and its size
  __host__ __device__ ScoreItemLayout(int D, int IC, int RP) {
    ks = 0;
    mh = IC * D * 2;
    ml = mh + IC * RP * 2;
    bs = ml + IC * RP * 2;
    bytes = bs + IC * 4;
  }
};
// The two staged items share their space with the score write-out that
// follows the selection (256 K bytes per wave): whichever is larger.
__host__ __device__ inline int score_stage_area(int item_bytes, int waves, int K) {
  return 2 * item_bytes > waves * 256 * K ? 2 * item_bytes : waves * 256 * K;
}
template <int D, int NJ, int WAVES>
size_t score_smem_bytes(int IC, int RP, int K) {
  return static_cast<size_t>(score_stage_area(ScoreItemLayout(D, IC, RP).bytes, WAVES, K)) +
         sizeof(ScoreSelect<D, NJ, WAVES>);
}

// swizzled piece of logical piece pc in row r of a row of P pieces (P = 4, 8, 16)
__device__ __forceinline__ int score_swz(int r, int P) { return (r >> (P == 16 ? 0 : (P == 8 ? 1 : 2))) & (P - 1); }

// Workgroup = (WAVES x 16 queries, KV head g, batch b).  Lane (ln, lg) of a
// wave works on query ln; in an S^T tile of 16 chunks it holds chunks
// 16 ct + 4 lg + i (i < 4), so the group scores of one query live in the
// four lanes ln, ln + 16, ln + 32, ln + 48 (16 NJ values each), and the
// selection runs for the wave's 16 queries at once.
// HR = 4: the group has at most 4 heads and every head's scores stay in
// registers through the selection (one pass over the summaries); HR = 0:
// a second pass recomputes the winners' per-head scores.  QR = RP / 32 when
// known at compile time (0: no Q-Cal), else -1.
template <int D, int NJ, int WAVES, int IC, int HR, int QR>
__global__ void __launch_bounds__(WAVES * 64, 8 / WAVES)
score_topk_mfma_kernel(ScoreArgs a, const uint16_t *__restrict__ u_hi, const uint16_t *__restrict__ u_lo,
                       const uint16_t *__restrict__ m_hi, const uint16_t *__restrict__ m_lo, int RP_arg) {
  const int RP = QR >= 0 ? 32 * QR : RP_arg;
  constexpr int KS = D / 32;
  constexpr int QW = WAVES * 16;      // queries per workgroup
  constexpr int NT = 4 * NJ;          // chunk tiles of 16 (64 NJ chunks)
  constexpr int NV = 16 * NJ;         // candidate values per lane
  constexpr int TPI = IC / 16;        // chunk tiles per item
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const ScoreItemLayout lay(D, IC, RP);
  ScoreSelect<D, NJ, WAVES> &sm =
      *reinterpret_cast<ScoreSelect<D, NJ, WAVES> *>(smem_raw + score_stage_area(lay.bytes, WAVES, a.K));
  auto item_ks = [&](int buf) { return reinterpret_cast<uint16_t *>(smem_raw + buf * lay.bytes + lay.ks); };
  auto item_mh = [&](int buf) { return reinterpret_cast<uint16_t *>(smem_raw + buf * lay.bytes + lay.mh); };
  auto item_ml = [&](int buf) { return reinterpret_cast<uint16_t *>(smem_raw + buf * lay.bytes + lay.ml); };
  auto item_bs = [&](int buf) { return reinterpret_cast<float *>(smem_raw + buf * lay.bytes + lay.bs); };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int T = a.T, C = a.C, K = a.K, Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  // one-dimensional grid, query block slowest: the latest (heaviest: most
  // eligible chunks) query blocks of every (b, g) go first, so that the
  // light ones fill the tail
  const int npair = Hkv * a.B;
  const int xq = static_cast<int>(blockIdx.x) / npair, pair = static_cast<int>(blockIdx.x) % npair;
  const int g = pair % Hkv, b = pair / Hkv;
  const int nqb = (T + QW - 1) / QW;
  const int q_wg = (nqb - 1 - xq) * QW;
  const int qw0 = q_wg + wave * 16;  // the wave's first query
  const bool qcal = QR >= 0 ? QR > 0 : a.r > 0;
  const int i_me = qw0 + ln;         // this lane's query (B column)
  const bool q_ok = i_me < T;
  const int n_me = q_ok ? min(eligible_chunks(i_me, a.W, a.S), C) : 0;
  const int n_wave = qw0 < T ? min(eligible_chunks(min(qw0 + 15, T - 1), a.W, a.S), C) : 0;
  const int n_wg = min(eligible_chunks(min(q_wg + QW - 1, T - 1), a.W, a.S), C);
  const int nblk = (n_wg + IC - 1) / IC;          // chunk blocks of one head
  const int nitems = G * nblk;                    // head outer, chunk block inner

  uint4 uh[2], ul[2];  // this lane's query's u = W_down h as the B operand
#pragma unroll
  for (int s = 0; s < 2; ++s) { uh[s] = make_uint4(0, 0, 0, 0); ul[s] = make_uint4(0, 0, 0, 0); }
  if (qcal) {
    const size_t uo = (static_cast<size_t>(b) * T + (q_ok ? i_me : 0)) * RP + 8 * lg;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bool ok = q_ok && s < RP / 32;
      uh[s] = ok ? *reinterpret_cast<const uint4 *>(u_hi + uo + 32 * s) : make_uint4(0, 0, 0, 0);
      ul[s] = ok ? *reinterpret_cast<const uint4 *>(u_lo + uo + 32 * s) : make_uint4(0, 0, 0, 0);
    }
  }
  const uint16_t *qb = static_cast<const uint16_t *>(a.q);
  const uint16_t *ksb = static_cast<const uint16_t *>(a.k_sum);

  // ---- staging of item x = (head hh, chunk block cb) straight into LDS in
  // 1 KB wave-wide slices (lane l's 16 bytes land at byte 16 l of a slice);
  // the entropies go through a register of the last two waves
  constexpr int kPk = D / 8;              // pieces per k' row
  constexpr int kSlK = IC * D * 2 / 1024;  // k' slices
  const int Pm = RP / 8;                  // pieces per m row
  const int slm = qcal ? IC * RP * 2 / 1024 : 0;  // m slices (hi or lo)
  auto issue_item = [&](int x, int buf) {
    const int hh = x / nblk, cb = x % nblk;
    const int h = g * G + hh, c0 = cb * IC;
    const int nsl = kSlK + 2 * slm;
    for (int sl = wave; sl < nsl; sl += WAVES) {
      const uint16_t *src;
      uint16_t *dst;
      if (sl < kSlK) {
        const int slot = sl * 64 + lane, r = slot / kPk, pp = slot % kPk;
        const int c = min(c0 + r, C - 1);  // rows past C are never used
        src = ksb + ((static_cast<size_t>(b) * Hq + h) * C + c) * D + ((pp ^ score_swz(r, kPk)) << 3);
        dst = item_ks(buf) + sl * 512;
      } else {
        // (reached only with Q-Cal: slm, Pm > 0)
        const int slm1 = slm > 0 ? slm : 1, Pm1 = Pm > 0 ? Pm : 1;
        const int y = sl - kSlK, lohi = y / slm1, part = y % slm1;
        const int slot = part * 64 + lane, r = slot / Pm1, pp = slot % Pm1;
        const int c = min(c0 + r, C - 1);
        src = (lohi ? m_lo : m_hi) + ((static_cast<size_t>(b) * Hq + h) * C + c) * RP + ((pp ^ score_swz(r, Pm)) << 3);
        dst = (lohi ? item_ml(buf) : item_mh(buf)) + part * 512;
      }
      lds_dma16(src, lds_address(dst));
    }
    static_assert(IC == 64, "one entropy piece per lane");
    if (wave == WAVES - 1)  // rows past C are never used
      lds_dma4(a.b_sum + (static_cast<size_t>(b) * Hq + h) * C + min(c0 + lane, C - 1), lds_address(item_bs(buf)));
  };

  // Q operands of head hh: lane holds query ln, d = 32 s + 8 lg .. +8
  uint4 qv[KS];
  auto load_q = [&](uint4 (&dst)[KS], int hh) {
    const int h = g * G + hh;
    const size_t qo = ((static_cast<size_t>(b) * Hq + h) * T + (q_ok ? i_me : 0)) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s) dst[s] = q_ok ? *reinterpret_cast<const uint4 *>(qb + qo + 32 * s) : make_uint4(0, 0, 0, 0);
  };

  // s of chunk tile ctl of the staged item: lane holds chunks 16 ctl + 4 lg + i
  auto score_tile = [&](int buf, int ctl) -> f32x4s {
    const uint16_t *iks = item_ks(buf), *imh = item_mh(buf), *iml = item_ml(buf);
    const float *ibs = item_bs(buf);
    const int r = 16 * ctl + ln;  // A-operand row
    f32x4s acc = f32x4s{0.f, 0.f, 0.f, 0.f};
    uint4 av[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      av[s] = *reinterpret_cast<const uint4 *>(iks + r * D + (((4 * s + lg) ^ score_swz(r, kPk)) << 3));
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma_s(av[s], qv[s], acc);
    if (qcal) {
      for (int s = 0; s < RP / 32; ++s) {
        const int off = r * RP + (((4 * s + lg) ^ score_swz(r, Pm)) << 3);
        const uint4 mh = *reinterpret_cast<const uint4 *>(imh + off);
        const uint4 ml = *reinterpret_cast<const uint4 *>(iml + off);
        acc = mfma_s(mh, uh[s], acc);
        acc = mfma_s(mh, ul[s], acc);
        acc = mfma_s(ml, uh[s], acc);
      }
    }
    f32x4s sv;
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = a.tau * acc[i] + ibs[16 * ctl + 4 * lg + i];
    return sv;
  };

  // candidate v = 4 ct + i holds chunk 16 ct + 4 lg + i
  float sig[HR > 0 ? 1 : NV];                  // group maxima (HR = 0)
  float sc[HR > 0 ? HR : 1][HR > 0 ? NV : 1];  // per-head scores (HR = 4); the group max comes after
  int rank[HR > 0 ? 1 : NV];                   // winner positions for the second pass (HR = 0)
  if constexpr (HR == 0) {
#pragma unroll
    for (int v = 0; v < NV; ++v) { sig[v] = -INFINITY; rank[v] = -1; }
  }
  // (HR > 0: every sc[h2][v] with h2 < G and an eligible chunk is written by
  // pass 1 before it is read; the others are never read)

  // One pass over the items.  PASS 1: group maximum into sig (and, with HR,
  // each head's score into sc).  PASS 2 (HR = 0): each head's own score of
  // the winners into topk_score (the same arithmetic as pass 1, so the
  // values are bit-identical).
  // Item x + 1 streams into the other buffer while item x computes; the DMA
  // is invisible to the compiler's waits (its LDS reads of item x do not
  // wait for it) and each wave waits for its own loads before the barrier.
  auto run_pass = [&](bool pass2) {
    if (nitems > 0) issue_item(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int x = 0; x < nitems; ++x) {
      const int buf = x & 1;
      const int hh = x / nblk, cb = x % nblk;
      if (cb == 0) load_q(qv, hh);
      // buffer buf ^ 1 was last read in iteration x - 1, before its barrier
      debug_sync();
      if (x + 1 < nitems) issue_item(x + 1, buf ^ 1);
#pragma unroll
      for (int cbb = 0; cbb < NT / TPI + (NT % TPI ? 1 : 0); ++cbb) {
        if (cbb != cb) continue;
#pragma unroll
        for (int ctl = 0; ctl < TPI; ++ctl) {
          const int ct = cbb * TPI + ctl;
          if (ct >= NT) break;
          if (HR == 0 && 16 * ct >= n_wave) break;  // wave-uniform: no chunk of the tile is eligible
          const f32x4s sv = score_tile(buf, ctl);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (!pass2) {
              if constexpr (HR > 0) {
#pragma unroll
                for (int h2 = 0; h2 < HR; ++h2)
                  if (h2 == hh) sc[h2][4 * ct + i] = sv[i];
              } else {
                sig[4 * ct + i] = fmaxf(sig[4 * ct + i], sv[i]);
              }
            } else if constexpr (HR == 0) {
              if (rank[4 * ct + i] >= 0)
                a.topk_score[((static_cast<size_t>(b) * Hq + g * G + hh) * T + i_me) * K + rank[4 * ct + i]] = sv[i];
            }
          }
          // one tile's operand reads in flight at a time (registers)
          if (HR > 0) __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  };

  // ---- pass 1: group scores
  run_pass(false);

  // ---- selection for the wave's 16 queries at once (4 lanes per query)
  const int keep = min(K, n_me);
  uint32_t ord[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int c = 16 * (v >> 2) + 4 * lg + (v & 3);
    float gv;
    if constexpr (HR > 0) {
      gv = sc[0][v];
#pragma unroll
      for (int h2 = 1; h2 < HR; ++h2)
        if (h2 < G) gv = fmaxf(gv, sc[h2][v]);
    } else {
      gv = sig[v];
    }
    ord[v] = c < n_me ? orderable(gv) : 0u;  // 0 = below every real score
  }
  // Bitwise search for the largest theta with #{ord >= theta} >= keep.
  // theta lies between the smallest and the largest eligible value, so it
  // shares their common leading bits: the search starts below them (scores
  // of one query often agree in sign, exponent and the top mantissa bits).
  // A query stops as soon as exactly `keep` candidates are at or above the
  // trial value (its winners, no ties); otherwise theta ends as the keep-th
  // largest value, with ties at it.
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    hi = max(hi, ord[v]);
    lo = min(lo, ord[v] != 0u ? ord[v] : 0xFFFFFFFFu);
  }
  lo = umin_rows4(lo);
  hi = ~umin_rows4(~hi);
  const uint32_t spread = keep > 0 ? lo ^ hi : 0u;
  const int top = spread ? 31 - __clz(spread) : -1;  // highest bit where lo and hi differ
  uint32_t theta = keep > 0 ? (top == 31 ? 0u : lo & ~((2u << top) - 1u)) : 0u;
  bool done = keep == 0;
  if (!done && top < 0) {  // every eligible value of the query is equal
    theta = lo;
    done = n_me == keep;
  }
  bool open = !done && top >= 0;  // still searching
  for (int bit = 31; bit >= 0; --bit) {
    if (!__ballot(open)) break;                  // every query of the wave has its threshold
    if (!__ballot(open && bit <= top)) continue;  // inside every open query's common prefix
    const uint32_t cand = theta | (1u << bit);
    uint32_t cnt = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v) cnt += ord[v] >= cand ? 1u : 0u;
    cnt = usum_rows4(cnt);
    if (open && bit <= top && static_cast<int>(cnt) >= keep) {
      theta = cand;
      done = static_cast<int>(cnt) == keep;
      open = !done;
    }
  }
  // winners as a bit mask over the lane's candidates
  // winners as a bit mask over the lane's NV candidates (64 when NJ = 4)
  using WMask = typename std::conditional<(NV > 32), unsigned long long, uint32_t>::type;
  WMask winm = 0;
  uint32_t ngt = 0;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const bool w = keep > 0 && (done ? ord[v] >= theta : ord[v] > theta);
    winm |= w ? (WMask{1} << v) : WMask{0};
    ngt += w ? 1u : 0u;
  }
  // ties at theta (queries not done): the lowest chunks first, one per round
  int need_eq = keep - static_cast<int>(usum_rows4(ngt));
  while (__ballot(need_eq > 0)) {
    uint32_t mloc = 0xFFFFu;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint32_t c = 16 * (v >> 2) + 4 * lg + (v & 3);
      if (need_eq > 0 && !((winm >> v) & 1u) && ord[v] == theta && ord[v] != 0u) mloc = min(mloc, c);
    }
    const uint32_t m = umin_rows4(mloc);
    if (need_eq > 0) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const uint32_t c = 16 * (v >> 2) + 4 * lg + (v & 3);
        if (c == m) winm |= WMask{1} << v;
      }
      need_eq = m == 0xFFFFu ? 0 : need_eq - 1;
    }
  }
  // compact each query's winners (in lane-row order) into LDS; with HR,
  // each winner's per-head scores go beside it, into this wave's part of
  // the staging space (free after the last item): [query][position] x 4
  float4 *wsc = reinterpret_cast<float4 *>(smem_raw + wave * 256 * K);
  {
    uint32_t pos = uprefix_rows4(static_cast<uint32_t>(NV > 32 ? __popcll(winm) : __popc(static_cast<uint32_t>(winm))));
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if ((winm >> v) & 1u) {
        // key: ordered score above, 0xFFFF - chunk below (a larger key is
        // the higher score, then the lower chunk)
        sm.win[wave][ln][pos] = (static_cast<unsigned long long>(ord[v]) << 32) |
                                (0xFFFFu - static_cast<uint32_t>(16 * (v >> 2) + 4 * lg + (v & 3)));
        if constexpr (HR > 0) wsc[ln * K + pos] = make_float4(sc[0][v], sc[1][v], sc[2][v], sc[3][v]);
        ++pos;
      }
    }
  }
  // (LDS operations of one wave complete in order: no wait needed)
  __builtin_amdgcn_wave_barrier();
  debug_sync();
  // position of winner p among the query's winners by (score desc, chunk
  // asc); lane (ln, lg) ranks winners p = lg, lg + 4, ...
  {
    constexpr int PPL = 8;  // winners per lane (K <= 32); j < ceil(K / 4) used
    unsigned long long pk[PPL];
    int pr[PPL];
    float4 ps[HR > 0 ? PPL : 1];  // the winners' per-head scores (HR)
#pragma unroll
    for (int j = 0; j < PPL; ++j) {
      const int p = lg + 4 * j;
      pk[j] = (4 * j < K && p < keep) ? sm.win[wave][ln][p] : 0ull;
      if constexpr (HR > 0) ps[j] = (4 * j < K && p < keep) ? wsc[ln * K + p] : make_float4(0.f, 0.f, 0.f, 0.f);
      pr[j] = 0;
    }
    const ulonglong2 *row = reinterpret_cast<const ulonglong2 *>(&sm.win[wave][ln][0]);
    for (int e2 = 0; e2 < (K + 1) / 2; ++e2) {
      const ulonglong2 w2 = row[e2];  // entries 2 e2 and 2 e2 + 1
      const unsigned long long k0 = 2 * e2 < keep ? w2.x : 0ull;
      const unsigned long long k1 = 2 * e2 + 1 < keep ? w2.y : 0ull;
#pragma unroll
      for (int j = 0; j < PPL; ++j) {
        if (4 * j >= K) break;  // uniform
        pr[j] += (k0 > pk[j] ? 1 : 0) + (k1 > pk[j] ? 1 : 0);
      }
    }
    const size_t ibase = ((static_cast<size_t>(b) * Hkv + g) * T + i_me) * K;
#pragma unroll
    for (int j = 0; j < PPL; ++j) {
      const int p = lg + 4 * j;
      if (4 * j >= K) break;
      if (q_ok && p < keep) {
        const int c = 0xFFFF - static_cast<int>(pk[j] & 0xFFFFu);
        a.topk_idx[ibase + pr[j]] = c;
        sm.rtab[wave][ln][c] = static_cast<int8_t>(pr[j]);
      }
    }
    // padding of the lists past keep
    if (q_ok) {
      for (int k = keep + lg; k < K; k += 4) a.topk_idx[ibase + k] = -1;
      if constexpr (HR == 0) {
        for (int x = lg; x < G * (K - keep); x += 4) {
          const int hh = x / (K - keep), k = keep + x % (K - keep);
          a.topk_score[((static_cast<size_t>(b) * Hq + g * G + hh) * T + i_me) * K + k] = -INFINITY;
        }
      }
    }
    if constexpr (HR > 0) {
      // ---- each head's own score of the winners in list order: the
      // wave's lists [head][query][K] in LDS (over the parked scores, which
      // are in registers now), then one contiguous run per head: the 16
      // queries' lists of a head follow each other in topk_score
      __builtin_amdgcn_wave_barrier();
      debug_sync();
      float *wout = reinterpret_cast<float *>(wsc);
#pragma unroll
      for (int j = 0; j < PPL; ++j) {
        const int p = lg + 4 * j;
        if (4 * j >= K) break;
        if (p < keep) {
          const float s4[4] = {ps[j].x, ps[j].y, ps[j].z, ps[j].w};
#pragma unroll
          for (int h2 = 0; h2 < HR; ++h2)
            if (h2 < G) wout[(h2 * 16 + ln) * K + pr[j]] = s4[h2];
        }
      }
      for (int x = lg; x < G * (K - keep); x += 4) {
        const int hh = x / (K - keep), k = keep + x % (K - keep);
        wout[(hh * 16 + ln) * K + k] = -INFINITY;
      }
      __builtin_amdgcn_wave_barrier();
      debug_sync();
      const int nvalid = (qw0 < T ? min(16, T - qw0) : 0) * K;  // rows past T are not written
      for (int h2 = 0; h2 < G; ++h2) {
        float *dst = a.topk_score + ((static_cast<size_t>(b) * Hq + g * G + h2) * T + qw0) * K;
        for (int e = lane; e < nvalid; e += 64) dst[e] = wout[h2 * 16 * K + e];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  debug_sync();

  if constexpr (HR > 0) {
    // (the per-head scores were written with the lists above)
  } else {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = 16 * (v >> 2) + 4 * lg + (v & 3);
      rank[v] = ((winm >> v) & 1u) ? static_cast<int>(sm.rtab[wave][ln][c]) : -1;
    }
    // ---- pass 2: each head's own score of the winners
    run_pass(true);
  }
}

// ------------------------------------------------------------------ scores + top-K, long sequences
// More chunks than one pass of the kernel above keeps in registers (C up to
// 8192 per sequence): the summaries stream through in blocks of 64 chunks,
// every head of the group per block, and each query keeps a running top-K
// of keys (score, chunk) with every head's own score of the kept chunks.
//
// Lane (ln, lg) works on query ln of the wave's 16, as above; the running
// list of a query is spread over its four lanes, KPL slots each (slot s of
// row lg is list entry 4 s + lg; entries at or past K are never used).
// After each block the query's candidates above its current K-th key (the
// smallest kept key; empty slots hold key 0) replace that smallest entry one
// at a time, best first, so the list always holds the K largest keys seen.
// Keys are unique (the chunk is in the low word), so the result is the
// exact top-K by (score descending, chunk ascending) of all eligible chunks.

__device__ __forceinline__ unsigned long long umax64_rows4(unsigned long long v) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  auto rl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  auto rh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  unsigned long long x = (static_cast<unsigned long long>(rh[0]) << 32) | rl[0];
  unsigned long long y = (static_cast<unsigned long long>(rh[1]) << 32) | rl[1];
  v = x > y ? x : y;
  lo = static_cast<uint32_t>(v);
  hi = static_cast<uint32_t>(v >> 32);
  auto sl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  auto sh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  x = (static_cast<unsigned long long>(sh[0]) << 32) | sl[0];
  y = (static_cast<unsigned long long>(sh[1]) << 32) | sl[1];
  return x > y ? x : y;
}
__device__ __forceinline__ unsigned long long umin64_rows4(unsigned long long v) { return ~umax64_rows4(~v); }

template <int D, int WAVES, int KPL, int QR>
__global__ void __launch_bounds__(WAVES * 64)
score_topk_stream_kernel(ScoreArgs a, const uint16_t *__restrict__ u_hi, const uint16_t *__restrict__ u_lo,
                         const uint16_t *__restrict__ m_hi, const uint16_t *__restrict__ m_lo) {
  constexpr int RP = 32 * QR;  // Q-Cal rank padded to the MFMA k-step (0: no Q-Cal)
  constexpr int KS = D / 32;
  constexpr int IC = 64;         // chunks per block
  constexpr int QW = WAVES * 16;  // queries per workgroup
  constexpr int GM = 4;           // heads per group handled here
  constexpr unsigned long long kFull = ~0ull;  // a slot past K: never the smallest
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const ScoreItemLayout lay(D, IC, RP);
  auto item_ks = [&](int buf) { return reinterpret_cast<uint16_t *>(smem_raw + buf * lay.bytes + lay.ks); };
  auto item_mh = [&](int buf) { return reinterpret_cast<uint16_t *>(smem_raw + buf * lay.bytes + lay.mh); };
  auto item_ml = [&](int buf) { return reinterpret_cast<uint16_t *>(smem_raw + buf * lay.bytes + lay.ml); };
  auto item_bs = [&](int buf) { return reinterpret_cast<float *>(smem_raw + buf * lay.bytes + lay.bs); };
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int T = a.T, C = a.C, K = a.K, Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  // heaviest (latest) query blocks first, as above
  const int npair = Hkv * a.B;
  const int xq = static_cast<int>(blockIdx.x) / npair, pair = static_cast<int>(blockIdx.x) % npair;
  const int g = pair % Hkv, b = pair / Hkv;
  const int nqb = (T + QW - 1) / QW;
  const int q_wg = (nqb - 1 - xq) * QW;
  const int qw0 = q_wg + wave * 16;
  constexpr bool qcal = QR > 0;
  const int i_me = qw0 + ln;
  const bool q_ok = i_me < T;
  const int n_me = q_ok ? min(eligible_chunks(i_me, a.W, a.S), C) : 0;
  const int n_wave = qw0 < T ? min(eligible_chunks(min(qw0 + 15, T - 1), a.W, a.S), C) : 0;
  const int n_wg = min(eligible_chunks(min(q_wg + QW - 1, T - 1), a.W, a.S), C);
  const int nblk = (n_wg + IC - 1) / IC;
  const int nitems = nblk * G;  // block outer, head inner

  uint4 uh[2], ul[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) { uh[s] = make_uint4(0, 0, 0, 0); ul[s] = make_uint4(0, 0, 0, 0); }
  if (qcal) {
    const size_t uo = (static_cast<size_t>(b) * T + (q_ok ? i_me : 0)) * RP + 8 * lg;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bool ok = q_ok && s < RP / 32;
      uh[s] = ok ? *reinterpret_cast<const uint4 *>(u_hi + uo + 32 * s) : make_uint4(0, 0, 0, 0);
      ul[s] = ok ? *reinterpret_cast<const uint4 *>(u_lo + uo + 32 * s) : make_uint4(0, 0, 0, 0);
    }
  }
  const uint16_t *qb = static_cast<const uint16_t *>(a.q);
  const uint16_t *ksb = static_cast<const uint16_t *>(a.k_sum);
  // every head's Q operand: lane holds query ln, d = 32 s + 8 lg .. +8
  uint4 qv[GM][KS];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    const size_t qo = ((static_cast<size_t>(b) * Hq + g * G + min(hh, G - 1)) * T + (q_ok ? i_me : 0)) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qv[hh][s] = (q_ok && hh < G) ? *reinterpret_cast<const uint4 *>(qb + qo + 32 * s) : make_uint4(0, 0, 0, 0);
  }
  // The operands above are complete before the streaming loop: otherwise
  // the compiler, not knowing that a head's first product in an iteration
  // follows the same loads, waits for every memory operation in flight (the
  // staged item included) before it on every item.
  __builtin_amdgcn_s_waitcnt(0);

  // ---- staging of item x = (chunk block x / G, head x % G), as above
  constexpr int kPk = D / 8;
  constexpr int kSlK = IC * D * 2 / 1024;
  constexpr int Pm = RP / 8;
  constexpr int slm = IC * RP * 2 / 1024;
  // Slices sl = wave + WAVES k: a whole number per wave, k' slices first, so
  // each k is a k' or an m slice for every wave alike (no branch)
  constexpr int nsl = kSlK + 2 * slm;
  static_assert(nsl % WAVES == 0 && kSlK % WAVES == 0, "whole slices per wave");
  auto issue_item = [&](int x, int buf) {
    const int hh = x % G, cb = x / G;
    const int h = g * G + hh, c0 = cb * IC;
#pragma unroll
    for (int k = 0; k < nsl / WAVES; ++k) {
      const int sl = wave + WAVES * k;
      const uint16_t *src;
      uint16_t *dst;
      if (k < kSlK / WAVES) {
        const int slot = sl * 64 + lane, r = slot / kPk, pp = slot % kPk;
        const int c = min(c0 + r, C - 1);  // rows past C are never used
        src = ksb + ((static_cast<size_t>(b) * Hq + h) * C + c) * D + ((pp ^ score_swz(r, kPk)) << 3);
        dst = item_ks(buf) + sl * 512;
      } else {
        const int slm1 = slm > 0 ? slm : 1, Pm1 = Pm > 0 ? Pm : 1;
        const int y = sl - kSlK, lohi = y / slm1, part = y % slm1;
        const int slot = part * 64 + lane, r = slot / Pm1, pp = slot % Pm1;
        const int c = min(c0 + r, C - 1);
        src = (lohi ? m_lo : m_hi) + ((static_cast<size_t>(b) * Hq + h) * C + c) * RP + ((pp ^ score_swz(r, Pm)) << 3);
        dst = (lohi ? item_ml(buf) : item_mh(buf)) + part * 512;
      }
      lds_dma16(src, lds_address(dst));
    }
    if (wave == WAVES - 1)  // the entropies, one 4-byte piece per lane (rows past C are never used)
      lds_dma4(a.b_sum + (static_cast<size_t>(b) * Hq + h) * C + min(c0 + lane, C - 1), lds_address(item_bs(buf)));
  };
  // s of chunk tile ctl of the staged item for head hh
  auto score_tile = [&](int buf, int ctl, const uint4 (&qh)[KS]) -> f32x4s {
    const uint16_t *iks = item_ks(buf), *imh = item_mh(buf), *iml = item_ml(buf);
    const float *ibs = item_bs(buf);
    const int r = 16 * ctl + ln;
    f32x4s acc = f32x4s{0.f, 0.f, 0.f, 0.f};
    uint4 av[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      av[s] = *reinterpret_cast<const uint4 *>(iks + r * D + (((4 * s + lg) ^ score_swz(r, kPk)) << 3));
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma_s(av[s], qh[s], acc);
    if (qcal) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {  // RP / 32 of them (u, m registers stay unrolled)
        if (s >= RP / 32) break;
        const int off = r * RP + (((4 * s + lg) ^ score_swz(r, Pm)) << 3);
        const uint4 mh = *reinterpret_cast<const uint4 *>(imh + off);
        const uint4 ml = *reinterpret_cast<const uint4 *>(iml + off);
        acc = mfma_s(mh, uh[s], acc);
        acc = mfma_s(mh, ul[s], acc);
        acc = mfma_s(ml, uh[s], acc);
      }
    }
    f32x4s sv;
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = a.tau * acc[i] + ibs[16 * ctl + 4 * lg + i];
    return sv;
  };

  // the running list: slot s of this lane = entry 4 s + lg of the query's list
  unsigned long long skey[KPL];
  float ssc[KPL][GM];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    skey[s] = 4 * s + lg < K ? kNoKey : kFull;
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) ssc[s][hh] = -INFINITY;
  }
  unsigned long long theta = kNoKey;  // the query's smallest kept key
  float scb[GM][16];                  // this block's scores: candidate v = chunk 16 (v >> 2) + 4 lg + (v & 3)

  // Item x + 1 streams into the other buffer while item x computes (the
  // DMA is invisible to the compiler's waits, so LDS reads of item x do not
  // wait for it); each wave waits for its own loads before the barrier.
  // Item x + 2 is issued right after that barrier, into the buffer item x
  // leaves, so that it is in flight during the merge that may follow.
  if (nitems > 0) issue_item(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nitems > 1) issue_item(1, 1);
  for (int x = 0; x < nitems; ++x) {
    const int buf = x & 1;
    const int hh = x % G, cb = x / G;
    debug_sync();
    if (IC * cb < n_wave) {  // wave-uniform: some query of the wave has eligible chunks here
#pragma unroll
      for (int h2 = 0; h2 < GM; ++h2) {
        if (h2 != hh) continue;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const f32x4s sv = score_tile(buf, ct, qv[h2]);
#pragma unroll
          for (int i = 0; i < 4; ++i) scb[h2][4 * ct + i] = sv[i];
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // this wave's loads of item x + 1 (the only ones in flight) have landed;
    // after the barrier all have, and no wave reads item x's buffer any more
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    debug_sync();
    if (x + 2 < nitems) issue_item(x + 2, buf);
    if (hh != G - 1 || IC * cb >= n_wave) continue;
    // ---- block cb complete: merge its candidates into the running lists
    unsigned long long kv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = IC * cb + 16 * (v >> 2) + 4 * lg + (v & 3);
      float sg = scb[0][v];
#pragma unroll
      for (int h2 = 1; h2 < GM; ++h2)
        if (h2 < G) sg = fmaxf(sg, scb[h2][v]);
      kv[v] = c < n_me ? make_key(sg, c) : kNoKey;
    }
    // A lane's candidates are taken in descending key order (each round the
    // query takes the best of its lanes' best remaining ones), so the ones
    // still left are those below the last key the lane gave up (keys are
    // distinct: they hold the chunk).
    unsigned long long ceil_k = kFull;
    for (int round = 0; round < 64; ++round) {
      // this lane's best remaining candidate and its heads' scores (no test
      // against theta here: the query takes its best only if that is above
      // theta, and that best is then this lane's best)
      unsigned long long mb = kNoKey;
      float bs[GM];
#pragma unroll
      for (int h2 = 0; h2 < GM; ++h2) bs[h2] = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool take = kv[v] > mb && kv[v] < ceil_k;
        mb = take ? kv[v] : mb;
#pragma unroll
        for (int h2 = 0; h2 < GM; ++h2) bs[h2] = take ? scb[h2][v] : bs[h2];
      }
      const unsigned long long qbest = umax64_rows4(mb);
      const bool ins = qbest > theta;  // the query takes qbest this round
      if (!__ballot(ins)) break;
      const bool owner = ins && mb == qbest;
      ceil_k = owner ? mb : ceil_k;
#pragma unroll
      for (int h2 = 0; h2 < GM; ++h2) bs[h2] = max_rows4(owner ? bs[h2] : -INFINITY);
      // the slot to replace: the smallest key (= theta) of the lowest row holding it
      unsigned long long lmin = kFull;
      int lslot = 0;
#pragma unroll
      for (int s = 0; s < KPL; ++s) {
        const bool lt = skey[s] < lmin;
        lmin = lt ? skey[s] : lmin;
        lslot = lt ? s : lslot;
      }
      const uint32_t row_take = umin_rows4(lmin == theta ? static_cast<uint32_t>(lg) : 4u);
      const bool rep = ins && static_cast<uint32_t>(lg) == row_take;
#pragma unroll
      for (int s = 0; s < KPL; ++s) {
        const bool here = rep && s == lslot;
        skey[s] = here ? qbest : skey[s];
#pragma unroll
        for (int h2 = 0; h2 < GM; ++h2) ssc[s][h2] = here ? bs[h2] : ssc[s][h2];
      }
      unsigned long long m2 = kFull;
#pragma unroll
      for (int s = 0; s < KPL; ++s) m2 = skey[s] < m2 ? skey[s] : m2;
      theta = umin64_rows4(m2);
    }
  }

  // ---- the lists in selection order: an entry's position = number of the
  // query's kept keys above it (the staging buffers are free now)
  debug_sync();
  if (!q_ok) return;
  unsigned long long *lk = reinterpret_cast<unsigned long long *>(smem_raw) + (wave * 16 + ln) * (4 * KPL);
#pragma unroll
  for (int s = 0; s < KPL; ++s) lk[4 * s + lg] = skey[s] == kFull ? kNoKey : skey[s];
  __builtin_amdgcn_wave_barrier();
  const int keep = min(K, n_me);
  const size_t ibase = ((static_cast<size_t>(b) * Hkv + g) * T + i_me) * K;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const unsigned long long k0 = skey[s];
    if (k0 == kFull || k0 == kNoKey) continue;
    int rk = 0;
    for (int e = 0; e < 4 * KPL; ++e) rk += lk[e] > k0 ? 1 : 0;
    a.topk_idx[ibase + rk] = key_chunk(k0);
#pragma unroll
    for (int h2 = 0; h2 < GM; ++h2)
      if (h2 < G) a.topk_score[((static_cast<size_t>(b) * Hq + g * G + h2) * T + i_me) * K + rk] = ssc[s][h2];
  }
  for (int k = keep + lg; k < K; k += 4) a.topk_idx[ibase + k] = -1;
  for (int x = lg; x < G * (K - keep); x += 4) {
    const int h2 = x / (K - keep), k = keep + x % (K - keep);
    a.topk_score[((static_cast<size_t>(b) * Hq + g * G + h2) * T + i_me) * K + k] = -INFINITY;
  }
}

constexpr int kStreamMaxC = 8192;  // chunk ids fit the key's low word; 512K positions at S = 64

bool score_mfma_supported(const ScoreArgs &a) {
  const bool fits = a.C <= kScoreMaxC || (a.C <= kStreamMaxC && a.Hq / a.Hkv <= 4);
  return a.bf16 && (a.d == 64 || a.d == 128) && fits && a.K <= 32 && a.K > 0 &&
         (a.r == 0 || (a.Dh % 32 == 0 && a.r <= 64));
}

template <int D, int KPL, int QR>
static hipError_t launch_score_stream_q(const ScoreArgs &a, const uint16_t *u_hi, const uint16_t *u_lo,
                                        const uint16_t *m_hi, const uint16_t *m_lo, hipStream_t st) {
  constexpr int WAVES = 8;
  constexpr int RPa = 32 * QR;
  auto kern = score_topk_stream_kernel<D, WAVES, KPL, QR>;
  const size_t items = 2 * static_cast<size_t>(ScoreItemLayout(D, 64, RPa).bytes);
  const size_t lists = static_cast<size_t>(WAVES) * 16 * 4 * KPL * sizeof(unsigned long long);
  const size_t smem = items > lists ? items : lists;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem));
  if (e != hipSuccess) return e;
  kern<<<dim3((a.T + WAVES * 16 - 1) / (WAVES * 16) * a.Hkv * a.B), WAVES * 64, smem, st>>>(a, u_hi, u_lo, m_hi,
                                                                                            m_lo);
  return hipGetLastError();
}
template <int D, int KPL>
static hipError_t launch_score_stream(const ScoreArgs &a, const uint16_t *u_hi, const uint16_t *u_lo,
                                      const uint16_t *m_hi, const uint16_t *m_lo, int RPa, hipStream_t st) {
  if (RPa == 0) return launch_score_stream_q<D, KPL, 0>(a, u_hi, u_lo, m_hi, m_lo, st);
  if (RPa == 32) return launch_score_stream_q<D, KPL, 1>(a, u_hi, u_lo, m_hi, m_lo, st);
  return launch_score_stream_q<D, KPL, 2>(a, u_hi, u_lo, m_hi, m_lo, st);
}

size_t score_mfma_ws_bytes(int B, int T, int Hq, int C, int r) {
  if (r == 0) return 0;
  const int RP = r <= 32 ? 32 : 64;
  return 2 * sizeof(uint16_t) * (static_cast<size_t>(B) * T * RP + static_cast<size_t>(B) * Hq * C * RP) + 1024;
}

hipError_t launch_score_mfma(const ScoreArgs &a, hipStream_t st) {
  const int RP = a.r <= 32 ? 32 : 64;
  uint16_t *base = static_cast<uint16_t *>(a.ws);
  uint16_t *u_hi = base, *u_lo = u_hi + static_cast<size_t>(a.B) * a.T * RP;
  uint16_t *m_hi = u_lo + static_cast<size_t>(a.B) * a.T * RP;
  uint16_t *m_lo = m_hi + static_cast<size_t>(a.B) * a.Hq * a.C * RP;
  if (a.r > 0) {
    const int ntok = a.B * a.T;
    const uint16_t *hp = static_cast<const uint16_t *>(a.h), *wd = static_cast<const uint16_t *>(a.w_down);
    const uint16_t *ks = static_cast<const uint16_t *>(a.k_sum), *wu = static_cast<const uint16_t *>(a.w_up);
    const int gmx = (a.C + 31) / 32;  // (no complete chunk: nothing to project)
    const int nm = gmx * a.Hq * a.B;
#define HILS_QCAL(NT, TT, DD)                                                                                      \
  {                                                                                                               \
    const int nub = (ntok + 16 * (TT) - 1) / (16 * (TT));                                                         \
    qcal_kernel<NT, TT, DD><<<nub + nm, 256, 0, st>>>(hp, wd, u_hi, u_lo, ntok, a.Dh, ks, wu, m_hi, m_lo, a.Hq, \
                                                      a.C, a.r, nub, gmx);                                        \
  }
    if (RP == 32) {
      if (a.d == 128) HILS_QCAL(2, 2, 128) else HILS_QCAL(2, 2, 64)
    } else {
      if (a.d == 128) HILS_QCAL(4, 1, 128) else HILS_QCAL(4, 1, 64)
    }
#undef HILS_QCAL
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.C > kScoreMaxC) {  // long sequences: the streaming selection
    const int RPs = a.r > 0 ? RP : 0;
    if (a.d == 128)
      return a.K <= 16 ? launch_score_stream<128, 4>(a, u_hi, u_lo, m_hi, m_lo, RPs, st)
                       : launch_score_stream<128, 8>(a, u_hi, u_lo, m_hi, m_lo, RPs, st);
    return a.K <= 16 ? launch_score_stream<64, 4>(a, u_hi, u_lo, m_hi, m_lo, RPs, st)
                     : launch_score_stream<64, 8>(a, u_hi, u_lo, m_hi, m_lo, RPs, st);
  }
  // candidates per lane in the selection: ceil(C / 64) rounded to 1, 2 or 4
  const int nj = a.C <= 64 ? 1 : (a.C <= 128 ? 2 : 4);
  // groups of at most 4 heads keep every head's scores in registers (one
  // pass); items of 64 chunks
  const int hr = (a.Hq / a.Hkv <= 4 && nj <= 2) ? 4 : 0;
  const int RPa = a.r > 0 ? RP : 0;
  const int qr = RPa / 32;
#define HILS_SCORE(DD, NN, WW, HRR, QRR)                                                                    \
  if (a.d == DD && nj == NN && hr == HRR && (QRR < 0 || qr == QRR)) {                                     \
    auto kern = score_topk_mfma_kernel<DD, NN, WW, 64, HRR, QRR>;                                         \
    const size_t smem = score_smem_bytes<DD, NN, WW>(64, RPa, a.K);                                      \
    hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),                              \
                                        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem)); \
    if (e2 != hipSuccess) return e2;                                                                      \
    kern<<<dim3((a.T + WW * 16 - 1) / (WW * 16) * a.Hkv * a.B), WW * 64, smem, st>>>(a, u_hi, u_lo, m_hi, m_lo, RPa); \
    return hipGetLastError();                                                                             \
  }
  HILS_SCORE(128, 1, 4, 4, 0) HILS_SCORE(128, 1, 4, 4, 1) HILS_SCORE(128, 1, 4, 4, 2)
  HILS_SCORE(128, 2, 4, 4, 0) HILS_SCORE(128, 2, 4, 4, 1) HILS_SCORE(128, 2, 4, 4, 2)
  HILS_SCORE(64, 1, 4, 4, 0) HILS_SCORE(64, 1, 4, 4, 1) HILS_SCORE(64, 1, 4, 4, 2)
  HILS_SCORE(64, 2, 4, 4, 0) HILS_SCORE(64, 2, 4, 4, 1) HILS_SCORE(64, 2, 4, 4, 2)
  HILS_SCORE(128, 1, 8, 0, -1) HILS_SCORE(128, 2, 8, 0, -1) HILS_SCORE(128, 4, 4, 0, -1)
  HILS_SCORE(64, 1, 8, 0, -1) HILS_SCORE(64, 2, 8, 0, -1) HILS_SCORE(64, 4, 4, 0, -1)
#undef HILS_SCORE
  return hipErrorInvalidValue;  // no instantiation for this shape (score_mfma_supported excludes it)
}

}  // namespace hils
