// tproj.hip -- LoRA down-projection T[M, 32] = X[M, K] . A[K, 32] for the prefill path
// (and for decode when T is computed in its own launch).  T is stored in fp16, rounded
// once from FP32 accumulation, and is read by the GEMM epilogue as an MFMA operand.
//
// onnxruntime PR #33370 ("[WebGPU] Fuse rank-32 quantized LoRA with MatMulNBits"), commit
// list: fuse_up computes T first, then the base GEMM with an integrated T*Bt^T epilogue;
// a later commit keeps a "K-parallel narrow-N" path for this projection.  Here: the output
// is only 32 wide, so the grid is (32-row M tiles) x (K parts of 512); each wave runs
// v_mfma_f32_32x32x16_f16 over 128 k; the four waves meet in LDS and the K parts meet in
// the workspace, where the last arriving workgroup of an M tile adds them in part order.
#include "common.h"

namespace mnb {
namespace {

template <int KIND>  // 1: F16 A, 2: INT8 A with block-32 fp16 scales
__global__ __launch_bounds__(256) void tproj_kernel(TprojParams p) {
  __shared__ float red[4][kRank * kRank];
  __shared__ int last_sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int mt = blockIdx.x / p.parts;
  const int part = blockIdx.x - mt * p.parts;
  const int kbeg = part * p.kp;
  const int kend = min(p.K, kbeg + p.kp);
  const int mrow = mt * 32 + (lane & 31);
  const int hk = 8 * (lane >> 5);            // this lane's 8 k within a 16-k step
  const int r = lane & 31;

  f16x_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  for (int kk = kbeg + wave * 16; kk < kend; kk += 64) {
    const int k = kk + hk;
    h8_t a, b;
    if (mrow < p.M) {
      a = *reinterpret_cast<const h8_t *>(reinterpret_cast<const _Float16 *>(p.X) + (size_t)mrow * p.K + k);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = (_Float16)0.f;
    }
    if constexpr (KIND == 1) {
      const _Float16 *A = static_cast<const _Float16 *>(p.A);
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = A[(size_t)(k + e) * kRank + r];
    } else {
      const int8_t *A = static_cast<const int8_t *>(p.A);
      const float s = h2f(p.sA[(size_t)(k / kBlock) * kRank + r]);
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = (_Float16)((float)A[(size_t)(k + e) * kRank + r] * s);
    }
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
  }
  // accumulator layout of a 32x32 MFMA tile: column = lane % 32,
  // row = 8*(v/4) + 4*(lane/32) + v%4 for register v
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int i = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    red[wave][i * kRank + r] = acc[v];
  }
  __syncthreads();
  float sum[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q;
    sum[q] = red[0][e] + red[1][e] + red[2][e] + red[3][e];
  }
  if (p.parts == 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int m = mt * 32 + e / kRank;
      if (m < p.M) p.t16[(size_t)m * kRank + (e % kRank)] = __builtin_bit_cast(uint16_t, (_Float16)sum[q]);
    }
    return;
  }
  const size_t mpad = (size_t)p.MT * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q;
    p.tpart[((size_t)part * mpad + mt * 32) * kRank + e] = sum[q];
  }
  fence_release();
  __syncthreads();
  if (tid == 0) {
    const int old = atomic_add_agent(&p.cnt[mt], 1);
    last_sh = (old == p.parts - 1);
    if (last_sh) atomic_store_agent(&p.cnt[mt], 0);
  }
  __syncthreads();
  if (!last_sh) return;
  fence_acquire();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q;
    float t = 0.f;
    for (int pp = 0; pp < p.parts; ++pp) t += p.tpart[((size_t)pp * mpad + mt * 32) * kRank + e];
    const int m = mt * 32 + e / kRank;
    if (m < p.M) p.t16[(size_t)m * kRank + (e % kRank)] = __builtin_bit_cast(uint16_t, (_Float16)t);
  }
}

}  // namespace

hipError_t launch_tproj(int lora, const TprojParams &p, hipStream_t s) {
  const int grid = p.MT * p.parts;
  if (lora == 1) hipLaunchKernelGGL(tproj_kernel<1>, dim3(grid), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(tproj_kernel<2>, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mnb
