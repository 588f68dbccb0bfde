// ceiling.hip -- measurement helper, not part of the MatMulNBits ABI: a plain streaming read
// of a device buffer, the practical ceiling a one-launch decode GEMV of the same byte count
// can reach on this GPU (launch, ramp-up and drain included).  Built into its own library
// (libmnb_ceiling.so), which only the benchmark loads.
//
// Each thread issues U independent 16-byte loads (global_load_dwordx4), U * 256 * 16 bytes
// per workgroup, strided by the grid so that every wave's loads are 1 KiB contiguous; the
// loaded words are folded with XOR into a value that is stored only if it equals a
// constant no data here produces, so the loads stay live and nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u4v *p, size_t n16, uint32_t *sink) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  u4v v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = t + (size_t)u * stride;
    v[u] = i < n16 ? p[i] : u4v{0u, 0u, 0u, 0u};
  }
  uint32_t r = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) r ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (r == 0x9E3779B9u) sink[blockIdx.x & 255] = r;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16, 16-byte aligned) from `p` on `stream` with U loads per
// thread (U in 1, 2, 4, 8); `sink` is a device buffer of 256 words that is never written by
// real data.  Returns 0, or -1 for bad arguments, or the HIP error code of the launch.
int mnb_ceiling_stream_read(const void *p, size_t bytes, int loads_per_thread, void *sink, void *stream) {
  if (!p || !sink || (bytes & 15) || ((uintptr_t)p & 15) || bytes == 0) return -1;
  const size_t n16 = bytes / 16;
  const int U = loads_per_thread;
  if (U != 1 && U != 2 && U != 4 && U != 8) return -1;
  const size_t per_wg = (size_t)256 * U;
  const size_t grid = (n16 + per_wg - 1) / per_wg;
  if (grid > 0x7fffffff) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const u4v *src = static_cast<const u4v *>(p);
  uint32_t *k = static_cast<uint32_t *>(sink);
  switch (U) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3((unsigned)grid), dim3(256), 0, s, src, n16, k); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3((unsigned)grid), dim3(256), 0, s, src, n16, k); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3((unsigned)grid), dim3(256), 0, s, src, n16, k); break;
    default: hipLaunchKernelGGL(stream_read_kernel<8>, dim3((unsigned)grid), dim3(256), 0, s, src, n16, k); break;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
