// Chunk terms of the prefill for long sequences: chunk-major over the whole
// sequence (bf16 MFMA operands, fp32 accumulation) -- HiLS-Attention,
// picx.dev summary, Methodology 2 (Eq. 10: each selected chunk contributes
// its own softmax-normalised values, weighted by e^{s_hat} under the joint
// normaliser).
//
// Past a few hundred chunks the queries of a block select nearly disjoint
// chunks (at 512K tokens the 1024 selections of a 64-query block name ~480
// chunks), so a pass over query blocks loads a chunk's K and V for about
// one selection: ~15 KB of K/V per (query, slot) entry.  Here each chunk is
// loaded once for every query that selected it, and every entry costs its
// query rows, a partial result written and read back (~3 KB):
//   lists    per (b, g) and chunk, the (query, slot) entries that selected
//            it: counted per 256-query block in LDS, a scan, then placed by
//            an atomic cursor (the order inside a chunk's list is arbitrary
//            and nothing below depends on it);
//   chunks   one workgroup per (chunk, g, b).  Each wave holds the chunk's
//            K (permuted rows) and V^T in registers as MFMA A operands, read
//            from the operand-order copy, and runs 16-column tiles of the
//            chunk's entries x G heads: S^T = K Q^T, the exact softmax over
//            the chunk's 64 keys, O^T = V^T P^T, and the column's o_c
//            (normalised by its chunk mass, bf16) into the entry's own slot;
//   combine  one wave per row (b, h, i): the row's selected chunks in slot
//            order, weighted e^{s_hat - M} / L with M the largest selected
//            score and L the sum of e^{s_hat - M}, into o as the row's chunk
//            part, and lse_C = M + log L into the workspace -- what the
//            query-block pass leaves for the window pass.
// A column of an MFMA product depends only on that column's operands, so a
// partial does not depend on the tile it shares, and the combine sums in
// slot order: the result is the same on every run.  The sequence is taken
// in segments of queries so that the partials (B H_q K 2 d bytes per query)
// stay within a bounded workspace.
#include <algorithm>

#include "hils_common.h"
#include "launch.h"

namespace hils {

namespace {

constexpr int kLK = 64;    // keys per chunk (S)
constexpr int kLQB = 256;  // queries per block of the list build
constexpr int kLMaxC = 8192;
constexpr float kLL2e = 1.4426950408889634f;

typedef __bf16 bf16x8l __attribute__((ext_vector_type(8)));
typedef float f32x4l __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4l mfma_l(const uint4 &a, const uint4 &b, const f32x4l &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8l, a), __builtin_bit_cast(bf16x8l, b), c, 0,
                                                 0, 0);
}

inline size_t up256(size_t x) { return (x + 255) / 256 * 256; }

// Queries per segment: the segment's partials stay within kLongPartBytes.
int long_segment_queries(int B, int Hq, int K, int d, int T) {
  const size_t per_q = static_cast<size_t>(B) * Hq * K * d * 2;
  size_t sq = kLongPartBytes / per_q / kLQB * kLQB;
  if (sq < static_cast<size_t>(kLQB)) sq = kLQB;
  return static_cast<int>(sq < static_cast<size_t>(T) ? sq : T);
}

// Workspace of the long pass: per (b, g) pair the chunk counts, cursors and
// list offsets, then the segment's entry lists and its partials.
struct LongWs {
  int *cnt, *cur, *off, *list;
  uint16_t *part;
  int Sq;
  size_t bytes;
};

LongWs long_layout(uint8_t *base, int B, int Hq, int Hkv, int T, int d, int K) {
  LongWs L{};
  const size_t C = T / kLK, pairs = static_cast<size_t>(B) * Hkv;
  L.Sq = long_segment_queries(B, Hq, K, d, T);
  size_t o = 0;
  L.cnt = reinterpret_cast<int *>(base + o);
  o += up256(pairs * C * 4);
  L.cur = reinterpret_cast<int *>(base + o);
  o += up256(pairs * C * 4);
  L.off = reinterpret_cast<int *>(base + o);
  o += up256(pairs * (C + 1) * 4);
  L.list = reinterpret_cast<int *>(base + o);
  o += up256(pairs * L.Sq * K * 4);
  L.part = reinterpret_cast<uint16_t *>(base + o);
  o += up256(static_cast<size_t>(B) * Hq * L.Sq * K * d * 2);
  L.bytes = o;
  return L;
}

}  // namespace

// ------------------------------------------------------------------ lists
__global__ void __launch_bounds__(256) long_zero_kernel(int *p, size_t n) {
  for (size_t x = blockIdx.x * static_cast<size_t>(256) + threadIdx.x; x < n; x += static_cast<size_t>(gridDim.x) * 256)
    p[x] = 0;
}

// cnt[b, g, c] += the entries of this block's queries that selected chunk c
__global__ void __launch_bounds__(256) long_count_kernel(AttnArgs a, int q0, int nq, int *cnt) {
  __shared__ int hist[kLMaxC];
  const int g = blockIdx.y, b = blockIdx.z, t = threadIdx.x, C = a.T / kLK;
  for (int c = t; c < C; c += 256) hist[c] = 0;
  __syncthreads();
  const int i = q0 + blockIdx.x * kLQB + t;
  if (i < q0 + nq) {
    const int n = eligible_chunks(i, a.W, kLK);
    const int32_t *ir = a.topk_idx + ((static_cast<size_t>(b) * a.Hkv + g) * a.T + i) * a.K;
    for (int k = 0; k < a.K; ++k) {
      const int c = ir[k];
      if (c >= 0 && c < n) atomicAdd(&hist[c], 1);
    }
  }
  __syncthreads();
  int *cg = cnt + (static_cast<size_t>(b) * a.Hkv + g) * C;
  for (int c = t; c < C; c += 256)
    if (hist[c]) atomicAdd(&cg[c], hist[c]);
}

// off = exclusive prefix of cnt, the total at index C; cnt and cur back to 0
// for the next segment
__global__ void __launch_bounds__(256) long_scan_kernel(int C, int *cnt, int *cur, int *off) {
  __shared__ int part[256];
  const int pg = blockIdx.x, t = threadIdx.x;
  int *cg = cnt + static_cast<size_t>(pg) * C;
  int *ug = cur + static_cast<size_t>(pg) * C;
  int *og = off + static_cast<size_t>(pg) * (C + 1);
  const int per = (C + 255) / 256, c0 = t * per, c1 = min(C, c0 + per);
  int s = 0;
  for (int c = c0; c < c1; ++c) s += cg[c];
  part[t] = s;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int x = 0; x < 256; ++x) {
      const int v = part[x];
      part[x] = run;
      run += v;
    }
    og[C] = run;
  }
  __syncthreads();
  int run = part[t];
  for (int c = c0; c < c1; ++c) {
    og[c] = run;
    run += cg[c];
    cg[c] = 0;
    ug[c] = 0;
  }
}

// list[b, g][off[c] + cursor] = (i - q0) << 5 | slot.  The block places its
// own entries first (an LDS counter per chunk gives each entry its place in
// the block's run of that chunk), then reserves one run per chunk it holds
// with a single global atomic, all of them issued before any is used.  The
// order inside a chunk's list is not fixed; no result depends on it (each
// entry is one column of the chunk kernel's tiles, computed on its own).
constexpr int kLMaxK = 32;  // list slots per query handled here (top-K <= 32)
__global__ void __launch_bounds__(256) long_fill_kernel(AttnArgs a, int q0, int nq, const int *off, int *cur,
                                                        int *list) {
  __shared__ int run[kLMaxC];  // entries of the block per chunk, then where its run starts
  const int g = blockIdx.y, b = blockIdx.z, t = threadIdx.x, C = a.T / kLK;
  const size_t pg = static_cast<size_t>(b) * a.Hkv + g;
  for (int c = t; c < C; c += 256) run[c] = 0;
  __syncthreads();
  const int i = q0 + blockIdx.x * kLQB + t;
  const bool q_ok = i < q0 + nq;
  const int n = eligible_chunks(i, a.W, kLK);
  const int32_t *ir = a.topk_idx + (pg * a.T + (q_ok ? i : q0)) * a.K;
  // the query's list read first, without a branch (slots past K read slot
  // K - 1 again and are dropped): a load under a branch waits at its end
  int cc[kLMaxK], pos[kLMaxK];
#pragma unroll
  for (int k = 0; k < kLMaxK; ++k) cc[k] = ir[k < a.K ? k : a.K - 1];
#pragma unroll
  for (int k = 0; k < kLMaxK; ++k) {
    const int c = cc[k];
    const bool ok = q_ok && k < a.K && c >= 0 && c < n;
    cc[k] = ok ? c : -1;
    pos[k] = ok ? atomicAdd(&run[c], 1) : 0;
  }
  __syncthreads();
  // one reservation per chunk the block holds: the counts up to 32 per thread
  // (C <= 8192), the atomics issued together, their results used after
  constexpr int kPer = kLMaxC / 256;
  int base[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int c = t + 256 * r;
    const int h = c < C ? run[c] : 0;
    base[r] = h ? atomicAdd(&cur[pg * C + c], h) : 0;
  }
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int c = t + 256 * r;
    if (c < C) run[c] = off[pg * (C + 1) + c] + base[r];
  }
  __syncthreads();
  int *lg = list + pg * static_cast<size_t>(nq) * a.K;
#pragma unroll
  for (int k = 0; k < kLMaxK; ++k)
    if (cc[k] >= 0) lg[run[cc[k]] + pos[k]] = ((i - q0) << 5) | k;
}

// ------------------------------------------------------------------ chunks
// Tile t of the chunk covers entries (16/G) t .. (16/G) t + 16/G - 1 of its
// list; column ln is (entry ln / G, head ln % G).  Operand-order blocks of a
// chunk (1 KB, lane l = 16 lg + ln reads bytes 16 l ..): K block kt KS + s
// is K[key perm(kt, ln)][d = 32 s + 8 lg ..], V block 4 KS + 2 dt + sl is
// V^T[d = 16 dt + ln][keys 32 sl + 8 lg ..]; with the key permutation the
// S^T accumulators of tiles 2 sl and 2 sl + 1 are the P^T operand of slice sl.
template <int D, int G>
__global__ void __launch_bounds__(256)
long_chunk_kernel(AttnArgs a, const uint16_t *__restrict__ ops, int q0, int nq, const int *__restrict__ off,
                  const int *__restrict__ list, uint16_t *__restrict__ part) {
  constexpr int KS = D / 32, DT = D / 16, QPT = 16 / G;
  constexpr int kKB = 4 * KS, kVB = 2 * DT;
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int T = a.T, K = a.K, Hq = a.Hq, C = T / kLK;
  const size_t pg = static_cast<size_t>(b) * a.Hkv + g;
  const int e_lo = off[pg * (C + 1) + c], e_n = off[pg * (C + 1) + c + 1] - e_lo;
  const int ntile = (e_n + QPT - 1) / QPT;
  if (w >= ntile) return;  // uniform per wave (no chunk entries: every wave); no barriers below
  const uint16_t *opc = ops + (pg * C + c) * (kKB + kVB) * 512 + lane * 8;
  uint4 kop[4][KS], vop[DT][2];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int s = 0; s < KS; ++s) kop[kt][s] = *reinterpret_cast<const uint4 *>(opc + (kt * KS + s) * 512);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) vop[dt][sl] = *reinterpret_cast<const uint4 *>(opc + (kKB + 2 * dt + sl) * 512);
  const int *lst = list + pg * static_cast<size_t>(nq) * K + e_lo;
  const uint16_t *qb = static_cast<const uint16_t *>(a.q);
  const int hh = ln % G;
  const size_t hrow = static_cast<size_t>(b) * Hq + g * G + hh;  // this column's query head
  const float tl2e = a.tau * kLL2e;

  struct Col {
    uint4 qop[KS];
    size_t po;  // the entry's partial: row (b, h, i - q0), slot
    bool valid;
  };
  auto load_col = [&](Col &cl, int tile) {
    const int e = tile * QPT + ln / G;
    cl.valid = e < e_n;
    const int en = lst[min(e, e_n - 1)];
    const int iq = en >> 5, slot = en & 31;
    const uint16_t *qr = qb + (hrow * T + q0 + iq) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s) cl.qop[s] = *reinterpret_cast<const uint4 *>(qr + 32 * s);
    cl.po = (hrow * nq + iq) * K + slot;
  };
  auto compute = [&](const Col &cl) {
    f32x4l st[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4l{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) st[kt] = mfma_l(kop[kt][s], cl.qop[s], st[kt]);
    // exact softmax over the chunk's 64 keys of column ln
    float mc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) mc = fmaxf(mc, st[kt][j]);
    mc = max_rows4(mc);
    const float offs = -mc * tl2e;
    float p[4][4], lc = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[kt][j] = __builtin_amdgcn_exp2f(fmaf(st[kt][j], tl2e, offs));
        lc += p[kt][j];
      }
    const float inv = __builtin_amdgcn_rcpf(sum_rows4(lc));  // lc >= 1: the maximum's own term
    uint4 pb[2];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      pb[sl].x = pack_bf16x2(p[2 * sl][0] * inv, p[2 * sl][1] * inv);
      pb[sl].y = pack_bf16x2(p[2 * sl][2] * inv, p[2 * sl][3] * inv);
      pb[sl].z = pack_bf16x2(p[2 * sl + 1][0] * inv, p[2 * sl + 1][1] * inv);
      pb[sl].w = pack_bf16x2(p[2 * sl + 1][2] * inv, p[2 * sl + 1][3] * inv);
    }
    // O^T = V^T P^T: lane holds d = 16 dt + 4 lg + (0..3) of column ln
    uint16_t *pr = part + cl.po * D + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4l ot = f32x4l{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) ot = mfma_l(vop[dt][sl], pb[sl], ot);
      if (cl.valid)
        *reinterpret_cast<uint2 *>(pr + 16 * dt) = make_uint2(pack_bf16x2(ot[0], ot[1]), pack_bf16x2(ot[2], ot[3]));
    }
  };
  // the waves take tiles w, w + 4, ...; the next tile's entries and query
  // rows load while the current one computes
  Col ca, cb;
  int tile = w;
  load_col(ca, tile);
  while (true) {
    if (tile + 4 < ntile) load_col(cb, tile + 4);
    compute(ca);
    tile += 4;
    if (tile >= ntile) break;
    if (tile + 4 < ntile) load_col(ca, tile + 4);
    compute(cb);
    tile += 4;
    if (tile >= ntile) break;
  }
}

// ------------------------------------------------------------------ combine
// One wave per row (b, h, i) of the segment; lane holds d = EPL lane ..
// EPL lane + EPL - 1.  Lane k < K reads slot k's chunk and score; the
// partials of every selected slot load at once (KM slots unrolled).
template <int D, int KM>
__global__ void __launch_bounds__(256)
long_combine_kernel(AttnArgs a, int q0, int nq, const uint16_t *__restrict__ part, float *__restrict__ lse_out) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  const size_t row = blockIdx.x * static_cast<size_t>(4) + (threadIdx.x >> 6);  // (b, h, i - q0)
  const int Hq = a.Hq, G = a.Hq / a.Hkv, K = a.K, T = a.T;
  if (row >= static_cast<size_t>(a.B) * Hq * nq) return;  // uniform per wave
  const int iq = static_cast<int>(row % nq), h = static_cast<int>((row / nq) % Hq);
  const int b = static_cast<int>(row / (static_cast<size_t>(nq) * Hq)), i = q0 + iq;
  const int n = eligible_chunks(i, a.W, kLK);
  const size_t ro = (static_cast<size_t>(b) * Hq + h) * T + i;
  int c = -1;
  float s = -INFINITY;
  if (lane < K) {
    c = a.topk_idx[((static_cast<size_t>(b) * a.Hkv + h / G) * T + i) * K + lane];
    s = a.topk_score[ro * K + lane];
  }
  const bool ok = lane < K && c >= 0 && c < n;
  const float mx = wave_max(ok ? s : -INFINITY);
  if (mx == -INFINITY) {  // no chunk: the window pass takes the window alone
    if (lane == 0) lse_out[ro] = -INFINITY;
    return;
  }
  const float wk = ok ? __expf(s - mx) : 0.f;
  const float l = wave_sum(wk);
  const uint64_t sel = __ballot(ok);
  const uint16_t *pr = part + row * K * D + lane * EPL;
  uint32_t raw[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    raw[k] = 0u;
    if (k < K && ((sel >> k) & 1u)) {
      if constexpr (EPL == 2)
        raw[k] = *reinterpret_cast<const uint32_t *>(pr + static_cast<size_t>(k) * D);
      else
        raw[k] = pr[static_cast<size_t>(k) * D];
    }
  }
  float acc[EPL] = {};
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const float wq = __shfl(wk, k, 64);  // zero for a slot without a chunk
    acc[0] += wq * __uint_as_float(raw[k] << 16);
    if constexpr (EPL == 2) acc[1] += wq * __uint_as_float(raw[k] & 0xFFFF0000u);
  }
  const float inv = 1.f / l;
  uint16_t *o = static_cast<uint16_t *>(a.o) + ro * D + lane * EPL;
  if constexpr (EPL == 2)
    *reinterpret_cast<uint32_t *>(o) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  else
    o[0] = f32_to_bf16(acc[0] * inv);
  if (lane == 0) lse_out[ro] = mx + __logf(l);
}

// ------------------------------------------------------------------ launch
bool attn_long_used(int T, int K) { return K > 0 && T / kLK > kLongMinChunks; }

size_t attn_long_ws_bytes(int B, int Hq, int Hkv, int T, int d, int K) {
  if (!attn_long_used(T, K)) return 0;
  return long_layout(nullptr, B, Hq, Hkv, T, d, K).bytes;
}

template <int D, int G>
static hipError_t long_t(const AttnArgs &a, uint16_t *ops, float *lse, uint8_t *ws, hipStream_t st) {
  const int C = a.T / kLK, npairs = a.B * a.Hkv;
  const LongWs L = long_layout(ws, a.B, a.Hq, a.Hkv, a.T, D, a.K);
  hipError_t e;
  const size_t ncnt = static_cast<size_t>(npairs) * C;
  const unsigned zb = static_cast<unsigned>(std::min<size_t>((ncnt + 255) / 256, 4096));
  long_zero_kernel<<<zb, 256, 0, st>>>(L.cnt, ncnt);
  long_zero_kernel<<<zb, 256, 0, st>>>(L.cur, ncnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int q0 = 0; q0 < a.T; q0 += L.Sq) {
    const int nq = std::min(L.Sq, a.T - q0);
    const dim3 qg((nq + kLQB - 1) / kLQB, a.Hkv, a.B);
    long_count_kernel<<<qg, 256, 0, st>>>(a, q0, nq, L.cnt);
    long_scan_kernel<<<npairs, 256, 0, st>>>(C, L.cnt, L.cur, L.off);
    long_fill_kernel<<<qg, 256, 0, st>>>(a, q0, nq, L.off, L.cur, L.list);
    // chunks that a query of the segment can hold (the last query, the most)
    const int cmax = eligible_chunks_host(q0 + nq - 1, a.W, kLK);
    if (cmax > 0)
      long_chunk_kernel<D, G><<<dim3(cmax, a.Hkv, a.B), 256, 0, st>>>(a, ops, q0, nq, L.off, L.list, L.part);
    const size_t rows = static_cast<size_t>(a.B) * a.Hq * nq;
    const unsigned cb = static_cast<unsigned>((rows + 3) / 4);
    if (a.K <= 16)
      long_combine_kernel<D, 16><<<cb, 256, 0, st>>>(a, q0, nq, L.part, lse);
    else
      long_combine_kernel<D, 32><<<cb, 256, 0, st>>>(a, q0, nq, L.part, lse);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attn_long(const AttnArgs &a, uint16_t *ops, float *lse, uint8_t *ws, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
#define HILS_LONG_CASE(DD, GG) \
  if (a.d == DD && G == GG) return long_t<DD, GG>(a, ops, lse, ws, st);
  HILS_LONG_CASE(128, 4) HILS_LONG_CASE(128, 1) HILS_LONG_CASE(128, 2) HILS_LONG_CASE(128, 8)
  HILS_LONG_CASE(128, 16) HILS_LONG_CASE(64, 4) HILS_LONG_CASE(64, 1) HILS_LONG_CASE(64, 2)
  HILS_LONG_CASE(64, 8) HILS_LONG_CASE(64, 16)
#undef HILS_LONG_CASE
  return hipErrorInvalidValue;
}

}  // namespace hils
