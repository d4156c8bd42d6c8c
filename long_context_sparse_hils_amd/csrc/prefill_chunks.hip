// Chunk terms of the prefill hierarchical sparse attention, chunk-major with
// per-chunk row compaction (bf16 MFMA operands, fp32 accumulation) --
// HiLS-Attention, picx.dev summary, Methodology 2 (Eq. 10: each selected
// chunk contributes its own softmax-weighted values, scaled by e^{s_hat}
// over the joint normaliser) and 3 (query packing for the matrix units).
//
// The factorisation of Eq. 10 makes every (query, head, chunk) term
// independent once the chunk scores are known: the chunk's softmax is
// complete inside its 64 keys and its weight e^{s_hat - M} is fixed before
// any key is read.  So a workgroup that owns a block of QB queries of one
// KV head (QB x G query-head rows) walks the union of the chunks its queries
// selected, and for each chunk multiplies only the rows that selected it,
// packed densely into 16-row MFMA tiles (16/G queries x G heads).  On the 8K
// workload a block of 32 queries selects ~56 distinct chunks, each taken by
// ~8 of its queries: 84 % of the tile rows do useful work, against ~41 %
// when 4 adjacent queries share a tile over the union of their chunks.
//
// A wave takes one chunk at a time (an LDS ticket), holds its K (the A
// operand of S^T = K Q^T, keys permuted so that the S^T accumulator is the
// B operand of the next product) and its V^T (the A operand of
// O^T = V^T P^T) in registers, and runs the chunk's tiles (the next chunk's
// K and V^T load while the last tile of the current one computes):
//   S^T = K Q^T            16x16x32 bf16 MFMA, keys in M, rows in N
//   p   = softmax over the chunk's 64 keys, times w = e^{s_hat - M_row} / L_row
//   O^T = V^T P^T          16x16x32 bf16 MFMA
// and adds O^T into the rows' accumulators in LDS (the rows of one tile are
// distinct; tiles of other chunks, on other waves, may share rows).  M_row
// is the row's largest selected chunk score and L_row the sum of
// e^{s_hat - M_row} over its selected chunks, so each accumulator ends as
// the row's chunk part normalised by its chunk mass: a convex combination
// of value rows, bounded by the largest |v| of the block's chunks, B_v.
// The accumulators are therefore 32-bit fixed point with 2^30 / B_v units
// (the scale is folded into the fusion weight, each O^T element truncated
// to an integer and added with ds_add_u32, no overflow: |sum| <= ~1.01 B_v);
// integer addition does not depend on the order in which the waves arrive,
// and a row's terms do not depend on the tile it shares, so the result is
// the same on every run.  The quantum, B_v 2^-30, lies far below the bf16
// rounding of the outputs.  The epilogue writes each row's chunk part
// (bf16) into the output tensor and the chunk log-mass lse_C = M_row +
// log L_row into the workspace; the window pass then adds the
// sliding-window term under the joint normaliser and overwrites the output.
#include "hils_common.h"
#include "launch.h"

namespace hils {

namespace {

typedef __bf16 bf16x8c __attribute__((ext_vector_type(8)));
typedef float f32x4c __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4c mfma16c(const bf16x8c &a, const bf16x8c &b, const f32x4c &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8c as_bf16x8c(const uint4 &u) { return __builtin_bit_cast(bf16x8c, u); }

constexpr int kCK = 64;  // keys per chunk (S)
constexpr float kL2e = 1.4426950408889634f;

// key held by S^T tile kt, row m: within each 32-key step the two 16-key
// tiles interleave in groups of 4, so that lane group lg's accumulator rows
// of tiles 2 sl and 2 sl + 1 are keys 32 sl + 8 lg .. + 8, the B-operand
// slots of the P^T product
__device__ __forceinline__ int chunk_perm_key(int kt, int m) {
  return 32 * (kt >> 1) + 8 * (m >> 2) + 4 * (kt & 1) + (m & 3);
}

// Word offset of (row, d) in the LDS accumulators: rows D + 1 words apart,
// so that one ds_add over a tile (d = 16 dt + 4 lg + e, dt and e fixed)
// reaches bank (row + 4 lg + const) mod 64 -- spread over the banks by the
// tile's rows -- while each lane's 32 adds share one base address and differ
// only in the instruction's immediate offset.
template <int D>
__device__ __forceinline__ int acc_off(int row, int d) {
  return row * (D + 1) + d;
}

template <int D, int G, int QB, int K_MAX, int WAVES>
struct ChunkCfg {
  static constexpr int kRows = QB * G;
  static constexpr int kQPT = 16 / G;      // queries per 16-row tile
  static constexpr int kEnt = QB * K_MAX;  // (query, slot) entries of a block
  static constexpr int kWaves = WAVES;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKS = D / 32;       // k-steps of S^T
  static constexpr int kDT = D / 16;       // d tiles of O^T
};

template <int D, int G, int QB, int K_MAX, int WAVES>
struct ChunkSmem {
  using C = ChunkCfg<D, G, QB, K_MAX, WAVES>;
  int acc[C::kRows * (D + 1)];              // fixed point, 2^30 / B_v units (acc_off)
  float row_m[C::kRows], row_il[C::kRows];  // M_row, 1 / L_row
  uint32_t umask[256];                      // the block's chunk ids as a bit mask (C <= 8192)
  int wbase[256];                           // union positions before each 32-chunk word
  int ucnt[C::kEnt];                        // entries per union position
  int useg[C::kEnt];                        // their first place in slist
  int16_t ulist[C::kEnt];                   // chunk id of each union position, ascending
  uint16_t slist[C::kEnt];                  // entries grouped by chunk: query | slot << 8
  int nunion, next;
  float vscale, vunscale;                   // 2^30 / B_v and its inverse
};

}  // namespace

// ------------------------------------------------------------------ operand order
// Each 64-key block's K and V^T, written in the order the MFMA passes'
// operand loads consume them: 2 D / 16 pieces of 1 KB, piece i read by one
// wave-wide 16-byte load in which lane l = 16 lg + ln takes bytes
// 16 l .. 16 l + 15:
//   K piece  kt * (D/32) + s :  K[key chunk_perm_key(kt, ln)][d = 32 s + 8 lg .. + 8]
//   V piece  4 D/32 + 2 dt + sl: V[keys 32 sl + 8 lg .. + 8][d = 16 dt + ln]
// so every operand load reads 1 KB of consecutive bytes.  Complete chunks go
// to ops ([pair][chunk]); the partial block that ends a sequence whose
// length is not a multiple of 64 goes to ops_tail ([pair]), its keys past T
// zero.  vmax (when given) [pair][block]: each block's largest |v|.
template <int D>
__global__ void __launch_bounds__(256)
kv_operand_order_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, uint16_t *__restrict__ ops,
                        uint16_t *__restrict__ ops_tail, float *__restrict__ vmax, int T, int C, int nblk) {
  constexpr int LD = D + 2;  // padded V rows in LDS (spreads the column reads over banks)
  constexpr int KB = 4 * (D / 32), VB = 2 * (D / 16);
  __shared__ uint16_t vs[kCK * LD];
  __shared__ uint32_t wmax[4];
  const int c = blockIdx.x, pair = blockIdx.y, tid = threadIdx.x;
  const int nk = min(kCK, T - c * kCK);  // keys of the block inside the sequence
  const uint16_t *kc = k + (static_cast<size_t>(pair) * T + static_cast<size_t>(c) * kCK) * D;
  const uint16_t *vc = v + (static_cast<size_t>(pair) * T + static_cast<size_t>(c) * kCK) * D;
  uint16_t *out = c < C ? ops + (static_cast<size_t>(pair) * C + c) * (KB + VB) * 512
                        : ops_tail + static_cast<size_t>(pair) * (KB + VB) * 512;
  uint32_t amax = 0u;  // |v| as bf16 bits: the order of non-negative floats
  for (int p = tid; p < kCK * D / 8; p += 256) {  // V rows into LDS
    const int key = p / (D / 8), seg = p % (D / 8);
    const uint4 u = key < nk ? *reinterpret_cast<const uint4 *>(vc + key * D + seg * 8) : make_uint4(0u, 0u, 0u, 0u);
    uint32_t *row = reinterpret_cast<uint32_t *>(vs + key * LD + seg * 8);
    row[0] = u.x; row[1] = u.y; row[2] = u.z; row[3] = u.w;
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = max(amax, max(w4[e] & 0x7FFFu, (w4[e] >> 16) & 0x7FFFu));
  }
  for (int p = tid; p < KB * 64; p += 256) {  // K pieces: straight copies
    const int blk = p / 64, l = p % 64, ln = l & 15, lg = l >> 4;
    const int kt = blk / (D / 32), s = blk % (D / 32), key = chunk_perm_key(kt, ln);
    *reinterpret_cast<uint4 *>(out + p * 8) =
        key < nk ? *reinterpret_cast<const uint4 *>(kc + key * D + 32 * s + 8 * lg) : make_uint4(0u, 0u, 0u, 0u);
  }
  if (vmax) {
    amax = wave_reduce_u32<1>(amax);
    if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  }
  __syncthreads();
  if (vmax && tid == 0)
    vmax[static_cast<size_t>(pair) * nblk + c] =
        bf16_to_f32(static_cast<uint16_t>(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]))));
  for (int p = tid; p < VB * 64; p += 256) {  // V^T pieces from LDS
    const int blk = p / 64, l = p % 64, ln = l & 15, lg = l >> 4;
    const int dt = blk / 2, sl = blk % 2, d = 16 * dt + ln, key0 = 32 * sl + 8 * lg;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = static_cast<uint32_t>(vs[(key0 + 2 * e) * LD + d]) | (static_cast<uint32_t>(vs[(key0 + 2 * e + 1) * LD + d]) << 16);
    *reinterpret_cast<uint4 *>(out + (KB * 64 + p) * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int D, int G, int QB, int K_MAX, int WAVES>
__global__ void __launch_bounds__(WAVES * 64, 1)
attn_chunks_kernel(AttnArgs a, const uint16_t *__restrict__ ops, float *__restrict__ lse_out,
                   const float *__restrict__ vmax, int nblocks, int xcd_map, int nblk) {
  using C = ChunkCfg<D, G, QB, K_MAX, WAVES>;
  static_assert(QB <= 256, "query index must fit a byte");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  ChunkSmem<D, G, QB, K_MAX, WAVES> &sm = *reinterpret_cast<ChunkSmem<D, G, QB, K_MAX, WAVES> *>(smem_raw);

  const int T = a.T, K = a.K, W = a.W, Hq = a.Hq, Hkv = a.Hkv;
  const int C_chunks = T / kCK;
  int blk, pair;
  {
    const int L = blockIdx.x;
    int slot;
    if (xcd_map) {  // the blocks of one (b, g) on one XCD: its K/V stay in that L2
      const int xcd = L & 7, s = L >> 3;
      pair = xcd + 8 * (s / nblocks);
      slot = s % nblocks;
    } else {
      pair = L / nblocks;
      slot = L % nblocks;
    }
    blk = nblocks - 1 - slot;  // late queries (more chunks) first
  }
  const int g = pair % Hkv, b = pair / Hkv;
  const int q0 = blk * QB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int ln = lane & 15, lg = lane >> 4;

  const int32_t *idx_bg = a.topk_idx + static_cast<size_t>(pair) * T * K;
  const float *tsc_b = a.topk_score + static_cast<size_t>(b) * Hq * T * K;

  // ---- set-up.  Every global load is issued at once, with clamped indices
  // and no lane-dependent branch: the block's selections (entry (q, k)),
  // and for the row statistics each row's chunk ids and fusion scores, two
  // threads per row (thread t: row t / 2, list half t % 2).
  constexpr int kEPT = (C::kEnt + C::kThreads - 1) / C::kThreads;
  constexpr int KH = K_MAX / 2;
  static_assert(2 * C::kRows <= C::kThreads, "two threads per row");
  const int kmax = K - 1;
  int ec[kEPT];
#pragma unroll
  for (int r = 0; r < kEPT; ++r) {
    const int x = tid + r * C::kThreads, q = x / K_MAX, k = x % K_MAX;
    ec[r] = idx_bg[static_cast<size_t>(min(q0 + q, T - 1)) * K + min(k, kmax)];
  }
  const int rs_row = min(tid >> 1, C::kRows - 1), rs_k0 = (tid & 1) * KH;
  const int rs_q = rs_row / G, rs_hh = rs_row % G, rs_i = min(q0 + rs_q, T - 1);
  int rc[KH];
  float rv[KH];
#pragma unroll
  for (int k = 0; k < KH; ++k) {
    rc[k] = idx_bg[static_cast<size_t>(rs_i) * K + min(rs_k0 + k, kmax)];
    rv[k] = tsc_b[(static_cast<size_t>(g * G + rs_hh) * T + rs_i) * K + min(rs_k0 + k, kmax)];
  }
  // B_v of the block needs the largest |v| of every 64-key block it selects
  // (chunk ids below C <= 256 here: one pass covers longer sequences)
  float vpre[4] = {0.f, 0.f, 0.f, 0.f};
  const float *vm = vmax + static_cast<size_t>(pair) * nblk;
  if (tid < 64) {
#pragma unroll
    for (int j = 0; j < 4; ++j) vpre[j] = lane + 64 * j < C_chunks ? vm[lane + 64 * j] : 0.f;
  }
  for (int x = tid; x < 256; x += C::kThreads) sm.umask[x] = 0u;
  for (int x = tid; x < C::kEnt; x += C::kThreads) sm.ucnt[x] = 0;
  if (tid == 0) sm.next = 0;
  __syncthreads();
  // Entry (q, k) holds chunk c when q0 + q < T, k < K and 0 <= c < n_i (any
  // other id is no chunk).
#pragma unroll
  for (int r = 0; r < kEPT; ++r) {
    const int x = tid + r * C::kThreads, q = x / K_MAX, k = x % K_MAX;
    const int i = q0 + q;
    const bool ok = x < C::kEnt && k < K && i < T && ec[r] >= 0 && ec[r] < eligible_chunks(i, W, kCK);
    ec[r] = ok ? ec[r] : -1;
    if (ok) atomicOr(&sm.umask[ec[r] >> 5], 1u << (ec[r] & 31));
  }
  // ---- row statistics: M_row = largest selected chunk score of the row,
  // L_row = sum of e^{s_hat - M_row} over its selected chunks; lse_C of
  // the row to the workspace (-inf: no chunk).  The two halves of a row
  // meet by a lane swap.
  {
    const int i = q0 + rs_q, n = eligible_chunks(i, W, kCK);
    bool okk[KH];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      okk[k] = rs_k0 + k < K && i < T && rc[k] >= 0 && rc[k] < n;
      mx = okk[k] ? fmaxf(mx, rv[k]) : mx;
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    float l = 0.f;
    if (mx > -INFINITY) {
#pragma unroll
      for (int k = 0; k < KH; ++k) l += okk[k] ? __expf(rv[k] - mx) : 0.f;
    }
    l += __shfl_xor(l, 1, 64);
    if ((tid & 1) == 0 && (tid >> 1) < C::kRows) {
      if (i < T) lse_out[(static_cast<size_t>(b) * Hq + g * G + rs_hh) * T + i] = l > 0.f ? mx + __logf(l) : -INFINITY;
      sm.row_m[rs_row] = mx;
      sm.row_il[rs_row] = l > 0.f ? 1.f / l : 0.f;
    }
  }
  __syncthreads();
  // ---- clear the accumulators; union positions in ascending chunk order
  // (prefix over the mask words)
  for (int x = tid; x < C::kRows * (D + 1) / 4; x += C::kThreads)
    reinterpret_cast<int4 *>(sm.acc)[x] = make_int4(0, 0, 0, 0);
  if (tid < 64) {
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
  __syncthreads();
  // ---- entries per chunk: an LDS counter gives each entry its place inside
  // its chunk's group (the grouping only decides which rows share a tile)
  int eu[kEPT], es[kEPT];
#pragma unroll
  for (int r = 0; r < kEPT; ++r) {
    const int c = ec[r];
    eu[r] = -1;
    es[r] = 0;
    if (c >= 0) {
      const int u = sm.wbase[c >> 5] + __popc(sm.umask[c >> 5] & ((1u << (c & 31)) - 1u));
      eu[r] = u;
      es[r] = atomicAdd(&sm.ucnt[u], 1);
      sm.ulist[u] = static_cast<int16_t>(c);
    }
  }
  __syncthreads();
  const int nunion = sm.nunion;
  if (tid < 64) {  // exclusive prefix of the counts; B_v of the block's chunks
    int base = 0;
    float bv = 0.f;
    auto selected = [&](int c) { return (sm.umask[c >> 5] >> (c & 31)) & 1u; };
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j < C_chunks && selected(lane + 64 * j)) bv = fmaxf(bv, vpre[j]);
    for (int c = lane + 256; c < C_chunks; c += 64)
      if (selected(c)) bv = fmaxf(bv, vm[c]);
    for (int u0 = 0; u0 < nunion; u0 += 64) {
      const int u = u0 + lane;
      const int cnt = u < nunion ? sm.ucnt[u] : 0;
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      if (u < nunion) sm.useg[u] = base + incl - cnt;
      base += __shfl(incl, 63, 64);
    }
    // (a bound below 2^-90 is raised to it: the scale stays finite, and
    // chunk parts that small vanish)
    bv = fmaxf(wave_reduce_f32<1>(bv), 0x1p-90f);
    if (lane == 0) {
      sm.vscale = 0x1p30f / bv;
      sm.vunscale = bv * 0x1p-30f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kEPT; ++r) {
    if (eu[r] >= 0) {
      const int x = tid + r * C::kThreads, q = x / K_MAX, k = x % K_MAX;
      sm.slist[sm.useg[eu[r]] + es[r]] = static_cast<uint16_t>(q | (k << 8));
    }
  }
  __syncthreads();

  // ---- the chunks, one per wave at a time (an LDS ticket).  A wave holds
  // its chunk's K (permuted rows) and V^T rows as MFMA A operands in
  // registers and walks the chunk's tiles; loads run ahead of their use
  // across chunk boundaries: the next tile's query rows and fusion score
  // while the current tile computes, and on a chunk's last tile the next
  // chunk's K as soon as that tile's S^T has read K, its V^T as soon as the
  // tile's last product has read V^T.
  constexpr int kKB = 4 * C::kKS, kVB = 2 * C::kDT;  // 1 KB operand blocks of a chunk
  // the pair's operand-order blocks through a buffer resource: the block's
  // byte offset is a scalar (soffset), the lane's 16 bytes the vector offset
  // (no per-block address arithmetic on the vector unit)
  const __amdgpu_buffer_rsrc_t oprs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(ops + static_cast<size_t>(pair) * C_chunks * (kKB + kVB) * 512), static_cast<short>(0),
      C_chunks * (kKB + kVB) * 1024, kBufWord3);
  const uint32_t op_lane = lane * 16;
  auto op_block = [&](int byte_off) -> uint4 {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(oprs, op_lane, byte_off, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  const uint16_t *qb = static_cast<const uint16_t *>(a.q);
  const int s_slot = ln / G, hh = ln % G;  // this lane's column: query slot, head
  const float tl2e = a.tau * kL2e;
  const float vscale = sm.vscale;

  // a tile's column: its entry (clamped to the chunk's last one), the query
  // row as the B operand of S^T, and the row's fusion score
  struct Col {
    uint4 qop[C::kKS];
    float sh;
    int row;
    bool valid;
  };
  // the block's query rows and fusion scores from workgroup-uniform bases
  // with 32-bit per-lane offsets (head hh of the group: hh T rows further;
  // G T D < 2^32 for the sequences this pass takes)
  const char *qwg = reinterpret_cast<const char *>(qb + ((static_cast<size_t>(b) * Hq + g * G) * T + q0) * D);
  const char *swg = reinterpret_cast<const char *>(a.topk_score + ((static_cast<size_t>(b) * Hq + g * G) * T + q0) * K);
  const uint32_t qlane = (static_cast<uint32_t>(hh) * static_cast<uint32_t>(T) * D + 8 * lg) * 2;  // bytes
  const uint32_t slane = static_cast<uint32_t>(hh) * static_cast<uint32_t>(T) * static_cast<uint32_t>(K) * 4;
  auto load_col = [&](Col &cl, int seg0, int cnt, int t) {
    const int e = t * C::kQPT + s_slot;
    cl.valid = e < cnt;
    const int ent = sm.slist[seg0 + min(e, cnt - 1)];
    const uint32_t q = ent & 0xFF, k = ent >> 8;
    cl.row = q * G + hh;
    const uint32_t qo = qlane + q * (D * 2);
#pragma unroll
    for (int s = 0; s < C::kKS; ++s) cl.qop[s] = *reinterpret_cast<const uint4 *>(qwg + (qo + 64 * s));
    cl.sh = *reinterpret_cast<const float *>(swg + (slane + (q * static_cast<uint32_t>(K) + k) * 4));
  };
  uint4 kop[4][C::kKS], vop[C::kDT][2];
  auto load_k = [&](int c) {  // blocks kt * kKS + s of the chunk's operand order
    const int kc = c * (kKB + kVB) * 1024;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int s = 0; s < C::kKS; ++s) kop[kt][s] = op_block(kc + (kt * C::kKS + s) * 1024);
  };
  auto load_v = [&](int c) {  // blocks kKB + 2 dt + sl
    const int vc = (c * (kKB + kVB) + kKB) * 1024;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) vop[dt][sl] = op_block(vc + (2 * dt + sl) * 1024);
  };
  auto ticket = [&]() -> int {
    int x = 0;
    if (lane == 0) x = atomicAdd(&sm.next, 1);
    return __builtin_amdgcn_readfirstlane(__shfl(x, 0, 64));
  };
  // the current chunk: its entries and tile cursor
  int seg0 = 0, cnt = 1, ntile = 0, t = 0;
  bool live;
  Col ca, cb;
  {
    const int x = ticket();
    live = x < nunion;
    if (live) {
      const int c = __builtin_amdgcn_readfirstlane(sm.ulist[x]);  // uniform: one LDS slot
      seg0 = sm.useg[x];
      cnt = sm.ucnt[x];
      ntile = (cnt + C::kQPT - 1) / C::kQPT;
      load_k(c);
      load_v(c);
      load_col(ca, seg0, cnt, 0);
    }
  }
  // one tile with the column `use`; loads the next tile's column into `pre`
  auto step = [&](const Col &use, Col &pre) {
    const bool last = t + 1 == ntile;
    // The next tile's column loads go out first, on every path: the next
    // chunk's first column on a chunk's last tile (its ticket taken first),
    // the current chunk's first again when no chunk is left.  The same loads
    // in the same order on every path let the compiler count them exactly,
    // so the uses below wait only for loads of earlier steps (a load under a
    // branch makes it wait for every load in flight at the next use).
    int cn = 0, segn = seg0, cntn = cnt, tn = t + 1;
    bool more = false;
    if (last) {
      const int xn = ticket();
      more = xn < nunion;
      tn = 0;
      if (more) {
        cn = __builtin_amdgcn_readfirstlane(sm.ulist[xn]);  // uniform: one LDS slot
        segn = sm.useg[xn];
        cntn = sm.ucnt[xn];
      }
    }
    load_col(pre, segn, cntn, tn);
    // S^T = K Q^T: lane holds keys chunk_perm_key(kt, 4 lg + j) of column ln
    f32x4c st[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4c{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::kKS; ++s)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) st[kt] = mfma16c(as_bf16x8c(kop[kt][s]), as_bf16x8c(use.qop[s]), st[kt]);
    if (more) load_k(cn);  // the next chunk's K, once this tile's S^T has read K
    // exact softmax over the chunk's 64 keys, scaled by the fusion weight
    float mc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) mc = fmaxf(mc, st[kt][j]);
    mc = max_rows4(mc);
    const float off = -mc * tl2e;
    float p[4][4], lc = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[kt][j] = __builtin_amdgcn_exp2f(fmaf(st[kt][j], tl2e, off));
        lc += p[kt][j];
      }
    lc = sum_rows4(lc);  // >= 1: the maximum's own term
    // fusion weight e^{s_hat - M_row} / L_row, in accumulator units
    const float w = use.valid
                        ? __expf(use.sh - sm.row_m[use.row]) * sm.row_il[use.row] * vscale * __builtin_amdgcn_rcpf(lc)
                        : 0.f;
    bf16x8c pb[2];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      uint4 u;
      u.x = pack_bf16x2(p[2 * sl][0] * w, p[2 * sl][1] * w);
      u.y = pack_bf16x2(p[2 * sl][2] * w, p[2 * sl][3] * w);
      u.z = pack_bf16x2(p[2 * sl + 1][0] * w, p[2 * sl + 1][1] * w);
      u.w = pack_bf16x2(p[2 * sl + 1][2] * w, p[2 * sl + 1][3] * w);
      pb[sl] = as_bf16x8c(u);
    }
    // O^T = V^T P^T: lane holds d = 16 dt + 4 lg + (0..3) of column ln
    f32x4c ot[C::kDT];
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) {
      ot[dt] = f32x4c{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) ot[dt] = mfma16c(as_bf16x8c(vop[dt][sl]), pb[sl], ot[dt]);
    }
    if (more) load_v(cn);
    if (use.valid) {
      int *ar = sm.acc + acc_off<D>(use.row, 4 * lg);
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __hip_atomic_fetch_add(ar + 16 * dt + j, static_cast<int>(ot[dt][j]), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (!last) {
      ++t;
    } else if (more) {
      seg0 = segn;
      cnt = cntn;
      ntile = (cntn + C::kQPT - 1) / C::kQPT;
      t = 0;
    } else {
      live = false;
    }
  };
  while (live) {
    step(ca, cb);
    if (!live) break;
    step(cb, ca);
  }
  __syncthreads();

  // ---- epilogue: each row's chunk part (normalised by its chunk mass) as bf16
  uint16_t *ob = static_cast<uint16_t *>(a.o);
  const float vunscale = sm.vunscale;
  for (int p = tid; p < C::kRows * D / 8; p += C::kThreads) {
    const int row = p / (D / 8), seg = p % (D / 8);
    const int q = row / G, hr = row % G, i = q0 + q;
    if (i >= T) continue;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = static_cast<float>(sm.acc[acc_off<D>(row, seg * 8 + j)]) * vunscale;
    uint4 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    w.z = pack_bf16x2(v[4], v[5]);
    w.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4 *>(ob + ((static_cast<size_t>(b) * Hq + g * G + hr) * T + i) * D + seg * 8) = w;
  }
}

template <int D, int G, int QB, int K_MAX, int WAVES = 8>
static hipError_t chunks_t(const AttnArgs &a, uint16_t *ops, float *lse, const float *vmax, int nblk,
                           hipStream_t st) {
  using C = ChunkCfg<D, G, QB, K_MAX, WAVES>;
  const int nblocks = (a.T + QB - 1) / QB;
  const int npairs = a.B * a.Hkv;
  const bool pair_fits_l2 = static_cast<size_t>(a.T) * D * 2 * 2 <= (size_t{4} << 20);
  const int xcd_map = (npairs % 8 == 0 && pair_fits_l2) ? 1 : 0;
  const size_t smem = sizeof(ChunkSmem<D, G, QB, K_MAX, WAVES>);
  auto kern = attn_chunks_kernel<D, G, QB, K_MAX, WAVES>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  kern<<<dim3(nblocks * npairs), C::kThreads, smem, st>>>(a, ops, lse, vmax, nblocks, xcd_map, nblk);
  return hipGetLastError();
}

// One workgroup of 8 waves per CU (two per SIMD, so that one wave's softmax
// overlaps the other's products): QB x G = 256 rows (128 KB of
// accumulators at d = 128) for top-K up to 16, 128 rows up to 32 (the
// per-entry tables double); at most 64 queries per block.
template <int D, int G>
static hipError_t chunks_g(const AttnArgs &a, uint16_t *ops, float *lse, const float *vmax, int nblk,
                           hipStream_t st) {
  constexpr int QB16 = 256 / G > 64 ? 64 : 256 / G;
  constexpr int QB32 = 128 / G > 64 ? 64 : 128 / G;
  if (a.K <= 16) return chunks_t<D, G, QB16, 16>(a, ops, lse, vmax, nblk, st);
  return chunks_t<D, G, QB32, 32>(a, ops, lse, vmax, nblk, st);
}

hipError_t launch_kv_operand_order(const AttnArgs &a, uint16_t *ops, uint16_t *ops_tail, float *vmax, hipStream_t st) {
  const int C = a.T / kCK, nblk = (a.T + kCK - 1) / kCK;
  const dim3 grid(nblk, a.B * a.Hkv);
  const uint16_t *k = static_cast<const uint16_t *>(a.k), *v = static_cast<const uint16_t *>(a.v);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (a.d == 128)
    kv_operand_order_kernel<128><<<grid, 256, 0, st>>>(k, v, ops, ops_tail, vmax, a.T, C, nblk);
  else if (a.d == 64)
    kv_operand_order_kernel<64><<<grid, 256, 0, st>>>(k, v, ops, ops_tail, vmax, a.T, C, nblk);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attn_chunks(const AttnArgs &a, uint16_t *ops, float *lse, const float *vmax, int nblk,
                              hipStream_t st) {
  const int G = a.Hq / a.Hkv;
#define HILS_CHUNK_CASE(DD, GG) \
  if (a.d == DD && G == GG) return chunks_g<DD, GG>(a, ops, lse, vmax, nblk, st);
  HILS_CHUNK_CASE(128, 4) HILS_CHUNK_CASE(128, 1) HILS_CHUNK_CASE(128, 2) HILS_CHUNK_CASE(128, 8)
  HILS_CHUNK_CASE(128, 16) HILS_CHUNK_CASE(64, 4) HILS_CHUNK_CASE(64, 1) HILS_CHUNK_CASE(64, 2)
  HILS_CHUNK_CASE(64, 8) HILS_CHUNK_CASE(64, 16)
#undef HILS_CHUNK_CASE
  return hipErrorInvalidValue;
}

}  // namespace hils
