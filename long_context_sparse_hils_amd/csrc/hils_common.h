// Device helpers shared by the HiLS kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (one v_cvt_pk_bf16_f32 per pair)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.f) & 0xFFFFu);
}

// Element access for the two storage types: uint16_t = bf16 bits, float = f32.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t *p, size_t i, float v) { p[i] = f32_to_bf16(v); }
  // 8 consecutive elements (16-byte aligned)
  __device__ __forceinline__ static void load8(const uint16_t *p, float *o) {
    uint4 w = *reinterpret_cast<const uint4 *>(p);
    uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(a[i] << 16);
      o[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  }
  // 2 consecutive elements (4-byte aligned)
  __device__ __forceinline__ static void load2(const uint16_t *p, float *o) {
    uint32_t a = *reinterpret_cast<const uint32_t *>(p);
    o[0] = __uint_as_float(a << 16);
    o[1] = __uint_as_float(a & 0xFFFF0000u);
  }
  __device__ __forceinline__ static void store2(uint16_t *p, float a, float b) {
    *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(a, b);
  }
};
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float *p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float *p, size_t i, float v) { p[i] = v; }
  __device__ __forceinline__ static void load8(const float *p, float *o) {
    float4 a = reinterpret_cast<const float4 *>(p)[0];
    float4 b = reinterpret_cast<const float4 *>(p)[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
  __device__ __forceinline__ static void load2(const float *p, float *o) {
    float2 a = *reinterpret_cast<const float2 *>(p);
    o[0] = a.x; o[1] = a.y;
  }
  __device__ __forceinline__ static void store2(float *p, float a, float b) {
    *reinterpret_cast<float2 *>(p) = make_float2(a, b);
  }
};

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
// reduce inside aligned groups of `width` lanes (width a power of two <= 64)
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sums inside aligned groups of 8 or 16 lanes with DPP lane moves (no LDS
// traffic): xor-1 and xor-2 inside quads, then mirror inside 8 and 16 lanes.
template <int width>
__device__ __forceinline__ float dpp_group_sum(float v) {
  static_assert(width == 8 || width == 16, "width");
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  if (width == 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  return v;
}

// Reductions over the four lanes l, l^16, l^32, l^48 with the gfx950 row
// swaps (v_permlane16_swap / v_permlane32_swap: plain VALU moves, no LDS).
// Called with the same register as both operands, a swap returns the value
// and its partner's in every lane.
__device__ __forceinline__ float max_rows4(float v) {
  const uint32_t b = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const uint32_t c = __float_as_uint(v);
  auto s = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_rows4(float v) {
  const uint32_t b = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const uint32_t c = __float_as_uint(v);
  auto s = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ uint32_t usum_rows4(uint32_t v) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = r[0] + r[1];
  auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return s[0] + s[1];
}
__device__ __forceinline__ uint32_t umin_rows4(uint32_t v) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min(static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1]));
  auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min(static_cast<uint32_t>(s[0]), static_cast<uint32_t>(s[1]));
}
// Exclusive prefix sum over the rows4 group in row order (row = lane >> 4).
// After a 16-swap every lane holds its pair's (even row, odd row) values;
// after a 32-swap of the pair sums, (rows 0+1, rows 2+3).
__device__ __forceinline__ uint32_t uprefix_rows4(uint32_t v) {
  const int row = (threadIdx.x & 63) >> 4;
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  const uint32_t pair = r[0] + r[1];
  auto s = __builtin_amdgcn_permlane32_swap(pair, pair, false, false);
  return ((row & 1) ? static_cast<uint32_t>(r[0]) : 0u) + ((row & 2) ? static_cast<uint32_t>(s[0]) : 0u);
}

// Whole-wave min / max / sum of a uint32 without LDS traffic: DPP moves
// inside each row of 16 lanes (xor 1, xor 2, then the half-row and row
// mirrors), then the row swaps across the four rows.
template <int OP, int CTRL>
__device__ __forceinline__ uint32_t dpp_combine(uint32_t v) {
  const uint32_t o = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xF, 0xF, false));
  return OP == 0 ? min(v, o) : OP == 1 ? max(v, o) : v + o;
}
template <int OP>  // 0: min, 1: max, 2: sum
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  v = dpp_combine<OP, 0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_combine<OP, 0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_combine<OP, 0x141>(v);  // row_half_mirror
  v = dpp_combine<OP, 0x140>(v);  // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  const uint32_t a = r[0], b = r[1];
  v = OP == 0 ? min(a, b) : OP == 1 ? max(a, b) : a + b;
  auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  const uint32_t c = q[0], d = q[1];
  return OP == 0 ? min(c, d) : OP == 1 ? max(c, d) : c + d;
}

// The same over floats (max or sum).
template <int OP, int CTRL>
__device__ __forceinline__ float dpp_combine_f(float v) {
  const float o = __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
  return OP == 1 ? fmaxf(v, o) : v + o;
}
template <int OP>  // 1: max, 2: sum
__device__ __forceinline__ float wave_reduce_f32(float v) {
  v = dpp_combine_f<OP, 0xB1>(v);
  v = dpp_combine_f<OP, 0x4E>(v);
  v = dpp_combine_f<OP, 0x141>(v);
  v = dpp_combine_f<OP, 0x140>(v);
  return OP == 1 ? max_rows4(v) : sum_rows4(v);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

// ---------------------------------------------------------------- selection keys
// A 64-bit key whose unsigned order is (score descending, chunk ascending):
// high word = order-preserving image of the float, low word = ~chunk.
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ unsigned long long make_key(float score, int chunk) {
  return (static_cast<unsigned long long>(orderable(score)) << 32) |
         static_cast<uint32_t>(~static_cast<uint32_t>(chunk));
}
__device__ __forceinline__ int key_chunk(unsigned long long k) {
  return static_cast<int>(~static_cast<uint32_t>(k & 0xFFFFFFFFu));
}
constexpr unsigned long long kNoKey = 0ull;  // below every real key

// Cross-workgroup hand-off without whole-cache maintenance.  The L2 of one
// XCD is not coherent with the others', and a device-scope fence writes back
// and invalidates the whole L2 of the XCD.  Instead, data handed to another
// workgroup is written with device-scope atomic stores (written through to
// the coherent memory side), each thread waits for its stores before the
// workgroup barrier that precedes the ticket, and the workgroup that takes the
// last ticket reads the data with device-scope atomic loads.  Both move two
// adjacent floats (8-byte aligned) at a time.
__device__ __forceinline__ void publish2(float *p, float x, float y) {
  const unsigned long long v = static_cast<unsigned long long>(__float_as_uint(x)) |
                               (static_cast<unsigned long long>(__float_as_uint(y)) << 32);
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_acquired2(const float *p) {
  const unsigned long long v =
      __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32)));
}
// Call from every thread after its publish2() stores: returns, in thread 0 of
// the workgroup, the number of workgroups that arrived before this one.
__device__ __forceinline__ unsigned arrive(unsigned *counter) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unsigned before = 0;
  if (threadIdx.x == 0) before = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return before;
}
__device__ __forceinline__ void reset_counter(unsigned *counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// ---------------------------------------------------------------- race check
// A library built with -DHILS_DEBUG_SYNC (libhils_debug_sync.so) serialises
// every LDS hand-off that the kernels otherwise leave to ordering: each LDS
// DMA waits for itself, and debug_sync() adds a full memory wait and a
// workgroup barrier where a buffer is refilled or a wave reuses LDS after
// its own earlier phase.  Results must be bit-identical with and without
// it.  Call sites are reached by every wave of the workgroup the same number
// of times (the control flow of a neighbouring __syncthreads, or the kernel's
// top level), never after a return that only some waves take.
__device__ __forceinline__ void debug_sync() {
#ifdef HILS_DEBUG_SYNC
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#endif
}

// Word 3 of a raw buffer resource for gfx9 (32-bit data format, so that
// untyped loads return data; no swizzle, no index stride).
constexpr int kBufWord3 = 0x00020000;

// ---------------------------------------------------------------- LDS DMA
// A wave-wide load from global memory straight into LDS: lane l's bytes
// (16 or 4) land at LDS byte address lds_base + size * l, lds_base being
// wave-uniform (M0).  Issued as inline assembly so that the compiler's wait
// insertion does not tie later LDS reads of other buffers to it (with the
// builtin it waits for every DMA in flight before the next LDS read, which
// serialises a multi-buffered pipeline).  The caller therefore waits
// itself: s_waitcnt vmcnt before the barrier that publishes the buffer.
// The kernels that use it issue no other loads into registers while DMAs
// are in flight unless they wait for everything first, so the compiler's
// own waits stay exact or conservative.
__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p)));
}
// M0 (the LDS base of the DMA) is saved and restored inside the statement:
// the compiler reserves it and does not expect it to change.
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory");
#ifdef HILS_DEBUG_SYNC
  __builtin_amdgcn_s_waitcnt(0);
#endif
}
__device__ __forceinline__ void lds_dma4(const void *src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory");
#ifdef HILS_DEBUG_SYNC
  __builtin_amdgcn_s_waitcnt(0);
#endif
}

// R1 partition: complete chunks before query i's window
__device__ __forceinline__ int eligible_chunks(int i, int W, int S) {
  int w0 = i - W + 1;
  return w0 > 0 ? w0 / S : 0;
}

}  // namespace hils
