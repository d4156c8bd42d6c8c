// Streaming-read reference for measurements (libhils_hbm_ref.so, not part of
// the libhils C ABI): a plain kernel that reads n bytes once with 16-byte
// loads, the rate a kernel reading a known number of bytes can be set
// against at that size.  Small reads stay below the 8 TB/s peak (launch,
// ramp-up and the tail of the grid), so a decode step that reads a few
// hundred MB is compared with a read of its own size.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Each thread reads U 16-byte pieces a grid stride apart per step (all U in
// flight together), then the remainder one at a time.  The XOR of the data
// decides a store that never happens for the all-ones fill the caller uses,
// so the loads cannot be dropped and nothing is written.
template <int U>
__global__ void __launch_bounds__(256) hbm_read_kernel(const v4u *__restrict__ p, size_t n16, uint32_t never,
                                                        uint32_t *__restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const v4u v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == never) sink[threadIdx.x] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16, 16-byte aligned) at device address `p`
// with `blocks` workgroups of 256 threads, `unroll` (4 or 8) loads in flight
// per thread, on `stream`.  `never` is a value the XOR of every thread's
// data does not take; `sink` (256 uint32, device) receives a store only if
// it does.  Returns a hipError_t; hipErrorInvalidValue for bad arguments.
extern "C" int hbm_ref_read(const void *p, size_t bytes, int blocks, int unroll, uint32_t never, void *sink,
                            void *stream) {
  if (!p || !sink || bytes % 16 || reinterpret_cast<uintptr_t>(p) % 16 || blocks <= 0 ||
      (unroll != 4 && unroll != 8))
    return hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const v4u *src = static_cast<const v4u *>(p);
  uint32_t *out = static_cast<uint32_t *>(sink);
  if (unroll == 4)
    hbm_read_kernel<4><<<blocks, 256, 0, st>>>(src, n16, never, out);
  else
    hbm_read_kernel<8><<<blocks, 256, 0, st>>>(src, n16, never, out);
  return hipGetLastError();
}
