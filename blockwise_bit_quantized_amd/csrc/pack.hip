// pack.hip -- weight packer and unpacker (2-, 4- and 8-bit codes) for the 64-row
// interleaved layout described in common.h, plus the fill used for K == 0.
//
// The packer plays the role of the offline "new transposed initializers" of onnxruntime
// PR #33800 ("Fuse DQ->MatMulNBits for shared initializers and skip outer-scope weights",
// Description): it reads already-quantized codes, block scales and zero points once and
// writes the layout the matmul kernels stream.  One thread per (group, block, row).
#include <algorithm>

#include "common.h"

namespace mnb {
namespace {

// KN: codes [K, N] and scales / zero points [K/32, N] (the DequantizeLinear layout, blocks
// along the first axis) instead of [N, K] and [N, K/32]
template <int BITS, bool KN>
__global__ __launch_bounds__(256) void pack_kernel(PackParams p) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)p.NG * p.KB * kGroup;
  if (idx >= total) return;
  const int r = (int)(idx % kGroup);
  const long tile = idx / kGroup;
  const int kb = (int)(tile % p.KB);
  const int g = (int)(tile / p.KB);
  const int n = g * kGroup + r;
  const bool ok = n < p.N;
  u4_t c0 = {0u, 0u, 0u, 0u}, c1 = {0u, 0u, 0u, 0u};
  if (ok && !KN) {
    const uint8_t *src = p.codes + (size_t)n * p.K + (size_t)kb * kBlock;
    c0 = *reinterpret_cast<const u4_t *>(src);
    c1 = *reinterpret_cast<const u4_t *>(src + 16);
  } else if (ok) {
    // column n of the block's 32 rows: consecutive threads read consecutive bytes
    const uint8_t *src = p.codes + (size_t)kb * kBlock * p.N + n;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      c0[k >> 2] |= (uint32_t)src[(size_t)k * p.N] << (8 * (k & 3));
      c1[k >> 2] |= (uint32_t)src[(size_t)(k + 16) * p.N] << (8 * (k & 3));
    }
  }
  // block-parameter index of row n (scales, zero points)
  auto bidx = [&](int nn) -> size_t { return KN ? (size_t)kb * p.N + nn : (size_t)nn * p.KB + kb; };
  auto code = [&](int k) -> uint32_t {  // code k (0..31) of this row-block
    const u4_t &v = k < 16 ? c0 : c1;
    const int kk = k & 15;
    return (v[kk >> 2] >> (8 * (kk & 3))) & 0xffu;
  };
  if constexpr (BITS == 2) {
    // two blocks per 16-byte chunk: this block fills half h = kb % 2 (and clears the other
    // half when it is the last block of an odd count)
    u2_t out;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w |= (code(16 * j + 2 * i) & 3u) << (2 * i);
        w |= (code(16 * j + 2 * i + 1) & 3u) << (16 + 2 * i);
      }
      out[j] = w;
    }
    const int KB2 = (p.KB + 1) / 2;
    uint8_t *dst = p.wq + (((size_t)g * KB2 + kb / 2) * kGroup + r) * 16 + 8 * (kb & 1);
    *reinterpret_cast<u2_t *>(dst) = out;
    if ((kb & 1) == 0 && kb + 1 == p.KB) *reinterpret_cast<u2_t *>(dst + 8) = u2_t{0u, 0u};
  } else if constexpr (BITS == 4) {
    u4_t out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w |= (code(8 * j + 2 * i) & 0xFu) << (4 * i);
        w |= (code(8 * j + 2 * i + 1) & 0xFu) << (16 + 4 * i);
      }
      out[j] = w;
    }
    *reinterpret_cast<u4_t *>(p.wq + ((size_t)tile * kGroup + r) * 16) = out;
  } else {
    *reinterpret_cast<u4_t *>(p.wq + (((size_t)tile * 2 + 0) * kGroup + r) * 16) = c0;
    *reinterpret_cast<u4_t *>(p.wq + (((size_t)tile * 2 + 1) * kGroup + r) * 16) = c1;
  }
  p.sc[(size_t)tile * kGroup + r] = ok ? p.scales[bidx(n)] : (uint16_t)0;
  if (p.zp) {
    if constexpr (BITS == 2) {
      if ((r & 3) == 0) {
        uint32_t b = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          if (n + d < p.N) b |= (p.zp[bidx(n + d)] & 3u) << (2 * d);
        p.zpp[(size_t)tile * 16 + (r >> 2)] = (uint8_t)b;
      }
    } else if constexpr (BITS == 4) {
      if ((r & 1) == 0) {
        const uint32_t z0 = ok ? (p.zp[bidx(n)] & 0xFu) : 0u;
        const uint32_t z1 = (n + 1 < p.N) ? (p.zp[bidx(n + 1)] & 0xFu) : 0u;
        p.zpp[(size_t)tile * 32 + (r >> 1)] = (uint8_t)(z0 | (z1 << 4));
      }
    } else {
      p.zpp[(size_t)tile * kGroup + r] = ok ? p.zp[bidx(n)] : (uint8_t)0;
    }
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void unpack_kernel(PackParams p, uint8_t *codes, uint16_t *scales,
                                                     uint8_t *zp) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;   // over N * KB
  if (idx >= (long)p.N * p.KB) return;
  const int n = (int)(idx / p.KB), kb = (int)(idx % p.KB);
  const int g = n / kGroup, r = n % kGroup;
  const size_t tile = (size_t)g * p.KB + kb;
  u4_t o0, o1;
  if constexpr (BITS == 2) {
    const int KB2 = (p.KB + 1) / 2;
    const u2_t w = *reinterpret_cast<const u2_t *>(p.wq + (((size_t)g * KB2 + kb / 2) * kGroup + r) * 16 + 8 * (kb & 1));
    uint32_t b[32];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        b[16 * j + 2 * i] = (w[j] >> (2 * i)) & 3u;
        b[16 * j + 2 * i + 1] = (w[j] >> (16 + 2 * i)) & 3u;
      }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o0[q] = b[4 * q] | (b[4 * q + 1] << 8) | (b[4 * q + 2] << 16) | (b[4 * q + 3] << 24);
      o1[q] = b[16 + 4 * q] | (b[16 + 4 * q + 1] << 8) | (b[16 + 4 * q + 2] << 16) | (b[16 + 4 * q + 3] << 24);
    }
  } else if constexpr (BITS == 4) {
    const u4_t w = *reinterpret_cast<const u4_t *>(p.wq + (tile * kGroup + r) * 16);
    uint32_t b[32];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[8 * j + 2 * i] = (w[j] >> (4 * i)) & 0xFu;
        b[8 * j + 2 * i + 1] = (w[j] >> (16 + 4 * i)) & 0xFu;
      }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o0[q] = b[4 * q] | (b[4 * q + 1] << 8) | (b[4 * q + 2] << 16) | (b[4 * q + 3] << 24);
      o1[q] = b[16 + 4 * q] | (b[16 + 4 * q + 1] << 8) | (b[16 + 4 * q + 2] << 16) | (b[16 + 4 * q + 3] << 24);
    }
  } else {
    o0 = *reinterpret_cast<const u4_t *>(p.wq + ((tile * 2 + 0) * kGroup + r) * 16);
    o1 = *reinterpret_cast<const u4_t *>(p.wq + ((tile * 2 + 1) * kGroup + r) * 16);
  }
  uint8_t *dst = codes + (size_t)n * p.K + (size_t)kb * kBlock;
  *reinterpret_cast<u4_t *>(dst) = o0;
  *reinterpret_cast<u4_t *>(dst + 16) = o1;
  scales[(size_t)n * p.KB + kb] = p.sc[tile * kGroup + r];
  if (zp && p.zp) {
    if constexpr (BITS == 2) zp[(size_t)n * p.KB + kb] = (p.zp[tile * 16 + (r >> 2)] >> (2 * (r & 3))) & 3u;
    else if constexpr (BITS == 4) zp[(size_t)n * p.KB + kb] = (p.zp[tile * 32 + (r >> 1)] >> (4 * (r & 1))) & 0xFu;
    else zp[(size_t)n * p.KB + kb] = p.zp[tile * kGroup + r];
  }
}

// Y[m, n] = bias[n], or 0 without a bias (K == 0: empty packed weights)
__global__ __launch_bounds__(256) void fill_kernel(uint16_t *Y, const uint16_t *bias, long n, int N) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (!bias) {
    const long nv = n / 8;
    if (i < nv) reinterpret_cast<u4_t *>(Y)[i] = u4_t{0u, 0u, 0u, 0u};
    if (i < n - nv * 8) Y[nv * 8 + i] = 0;
    return;
  }
  for (long e = i; e < n; e += (long)gridDim.x * 256) Y[e] = bias[e % N];
}

}  // namespace

hipError_t launch_pack(int bits, bool kn, const PackParams &p, hipStream_t s) {
  const long total = (long)p.NG * p.KB * kGroup;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (bits == 2 && !kn) hipLaunchKernelGGL((pack_kernel<2, false>), grid, dim3(256), 0, s, p);
  else if (bits == 2) hipLaunchKernelGGL((pack_kernel<2, true>), grid, dim3(256), 0, s, p);
  else if (bits == 4 && !kn) hipLaunchKernelGGL((pack_kernel<4, false>), grid, dim3(256), 0, s, p);
  else if (bits == 4) hipLaunchKernelGGL((pack_kernel<4, true>), grid, dim3(256), 0, s, p);
  else if (!kn) hipLaunchKernelGGL((pack_kernel<8, false>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((pack_kernel<8, true>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_unpack(int bits, const PackParams &p, uint8_t *codes, uint16_t *scales, uint8_t *zp,
                         hipStream_t s) {
  const long total = (long)p.N * p.KB;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (bits == 2) hipLaunchKernelGGL(unpack_kernel<2>, grid, dim3(256), 0, s, p, codes, scales, zp);
  else if (bits == 4) hipLaunchKernelGGL(unpack_kernel<4>, grid, dim3(256), 0, s, p, codes, scales, zp);
  else hipLaunchKernelGGL(unpack_kernel<8>, grid, dim3(256), 0, s, p, codes, scales, zp);
  return hipGetLastError();
}

hipError_t launch_fill(uint16_t *Y, const uint16_t *bias, int M, int N, hipStream_t s) {
  const long n = (long)M * N;
  const long work = bias ? std::min<long>(n, 1L << 22) : std::max<long>(n / 8, n % 8);
  if (work == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, Y, bias, n, N);
  return hipGetLastError();
}

}  // namespace mnb
