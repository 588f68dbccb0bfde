// tproj.hip -- LoRA down-projection T = X[M, K] . A[K, 32] for the prefill path (and for
// decode when T runs in its own launch).  The output is FP32 partial sums per K-part,
// tpart[part][m][r]; the consumer (GEMM or GEMV epilogue) adds the parts in part order.
//
// onnxruntime PR #33370 ("[WebGPU] Fuse rank-32 quantized LoRA with MatMulNBits"), commit
// list: fuse_up computes T first, then the base GEMM with an integrated T*Bt^T epilogue;
// a later commit keeps a "K-parallel narrow-N" path for this projection.  Here the output
// is only 32 wide, so the grid is (32-row M tiles) x (K parts of kp).  Per workgroup:
//  * the A-part [kp, 32] is read once with 16-byte loads and written transposed into LDS
//    (8x8 half tiles transposed in registers, one ds_write_b128 per rank row), so the
//    MFMA B operand (8 consecutive k of one rank) is a single ds_read_b128;
//  * each wave owns kp/4 consecutive k and issues all of its X loads (MFMA A operand,
//    8 consecutive k of one row per lane) before waiting on anything;
//  * v_mfma_f32_32x32x16_f16 per 16 k; the four waves meet in LDS in fixed order.
// No counters and no cross-workgroup waits.
#include "common.h"

namespace mnb {
namespace {

// KIND 1: F16 A, 2: INT8 A with block-32 fp16 scales; KP: K per part (256, 512 or 1024,
// see tproj_kp)
template <int KIND, int KP>
__global__ __launch_bounds__(256) void tproj_kernel(TprojParams p) {
  constexpr int kKP = KP;
  constexpr int kStepsPerWave = kKP / 4 / 16;
  constexpr int kLdA = kKP + 8;       // halfs per transposed A row (pad keeps lanes on distinct banks)
  static_assert(kRank * kLdA * 2 >= 4 * 1024 * 4, "the cross-wave sum reuses the A buffer");
  __shared__ __attribute__((aligned(16))) _Float16 sAT[kRank * kLdA];   // 66 KB at KP = 1024
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int mt = blockIdx.x / p.parts;
  const int part = blockIdx.x - mt * p.parts;
  const int kbeg = part * kKP;
  const int kend = min(p.K, kbeg + kKP);
  const int mrow = mt * 32 + (lane & 31);
  const bool mok = mrow < p.M;
  const int hk = 8 * (lane >> 5);

  // X operand loads for this wave's k range (all issued first)
  const int kw = kbeg + wave * (kKP / 4);
  const _Float16 *xr = reinterpret_cast<const _Float16 *>(p.X) + (size_t)(mok ? mrow : 0) * p.K;
  h8_t xa[kStepsPerWave];
#pragma unroll
  for (int s = 0; s < kStepsPerWave; ++s) {
    const int k = kw + 16 * s + hk;
    xa[s] = *reinterpret_cast<const h8_t *>(xr + (k < kend ? k : 0));
  }

  // A part -> LDS transposed: thread handles 8x8 tiles (k octet, r octet)
  constexpr int kTiles = kKP / 8 * 4;
#pragma unroll
  for (int t = tid; t < kTiles; t += 256) {
    const int ko = t >> 2, ro = t & 3;
    const int k0 = kbeg + ko * 8;
    uint32_t v[8][4];   // v[row e][dword d] = halves (r = 2d, 2d+1) of A[k0+e][8*ro ..]
    if (k0 < kend) {
      if constexpr (KIND == 1) {
        const uint16_t *A = static_cast<const uint16_t *>(p.A);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const u4_t a = *reinterpret_cast<const u4_t *>(A + (size_t)(k0 + e) * kRank + ro * 8);
#pragma unroll
          for (int d = 0; d < 4; ++d) v[e][d] = a[d];
        }
      } else {
        const int8_t *A = static_cast<const int8_t *>(p.A);
        const u4_t sv = *reinterpret_cast<const u4_t *>(p.sA + (size_t)(k0 / kBlock) * kRank + ro * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint2 a = *reinterpret_cast<const uint2 *>(A + (size_t)(k0 + e) * kRank + ro * 8);
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t bytes = d < 2 ? a.x : a.y;
            const int8_t lo = (int8_t)((bytes >> (16 * (d & 1))) & 0xff);
            const int8_t hi = (int8_t)((bytes >> (16 * (d & 1) + 8)) & 0xff);
            const h2_t s2 = as_h2(sv[d]);
            const h2_t q = {(_Float16)((float)lo * (float)s2[0]), (_Float16)((float)hi * (float)s2[1])};
            v[e][d] = as_u32(q);
          }
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int d = 0; d < 4; ++d) v[e][d] = 0u;
    }
    // transpose: rank row rr = 2d + h gets k = e (8 halves) -> one 16-byte store
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u4_t o;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint32_t lo = (v[2 * e2][d] >> (16 * h)) & 0xffffu;
          const uint32_t hi = (v[2 * e2 + 1][d] >> (16 * h)) & 0xffffu;
          o[e2] = lo | (hi << 16);
        }
        *reinterpret_cast<u4_t *>(&sAT[(ro * 8 + 2 * d + h) * kLdA + ko * 8]) = o;
      }
  }
  __syncthreads();

  f16x_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  const int r = lane & 31;
#pragma unroll
  for (int s = 0; s < kStepsPerWave; ++s) {
    const int k = kw + 16 * s;
    if (k < kend) {
      const h8_t b = *reinterpret_cast<const h8_t *>(&sAT[r * kLdA + (k - kbeg) + hk]);
      h8_t a = xa[s];
      if (!mok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (_Float16)0.f;
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
    }
  }
  __syncthreads();   // sAT no longer needed: reuse it for the cross-wave sum
  float *red = reinterpret_cast<float *>(sAT);   // [4][32*32]
  // accumulator layout of a 32x32 MFMA tile: column = lane % 32,
  // row = 8*(v/4) + 4*(lane/32) + v%4 for register v
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int i = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    red[wave * 1024 + i * kRank + r] = acc[v];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q;
    const float sum = red[e] + red[1024 + e] + red[2048 + e] + red[3072 + e];
    const int m = mt * 32 + e / kRank;
    if (m < p.M) {
      float *dst = p.tpart + ((size_t)part * p.M + m) * kRank + (e % kRank);
      if (p.reduce) __hip_atomic_store(dst, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else *dst = sum;
    }
  }
  if (!p.reduce) return;
  // The workgroup that counts itself last for this M tile adds the parts in part order
  // (the order is fixed, so the sum does not depend on which workgroup arrives last) and
  // writes T once; it resets the counter for the next call.  No fences: the partials above
  // were written with device-coherent stores, which write through the XCD's L2, and each
  // thread waits until its stores are acknowledged before the workgroup counts itself; the
  // last workgroup reads the partials with device-coherent loads, which bypass its L2, after
  // its count has returned.  (Agent-scope fences write back and invalidate a whole L2 on
  // this part; the fenced version took 16.2 against 14.9 us per 8 x 4096 x 4096 call.)
  __shared__ int last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    last = __hip_atomic_fetch_add(&p.ctrl[ctrl_tproj_word(mt)], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           p.parts - 1;
  __syncthreads();
  if (!last) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q;
    const int m = mt * 32 + e / kRank;
    if (m < p.M) {
      const float *src = p.tpart + (size_t)m * kRank + (e % kRank);
      float v[4];
      float t = 0.f;
      int pp = 0;
      for (; pp + 4 <= p.parts; pp += 4) {     // four loads in flight, added in order
#pragma unroll
        for (int u = 0; u < 4; ++u)
          v[u] = __hip_atomic_load(src + (size_t)(pp + u) * p.M * kRank, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int u = 0; u < 4; ++u) t += v[u];
      }
      for (; pp < p.parts; ++pp)
        t += __hip_atomic_load(src + (size_t)pp * p.M * kRank, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      p.tfinal[(size_t)m * kRank + (e % kRank)] = t;
    }
  }
  if (tid == 0) __hip_atomic_store(&p.ctrl[ctrl_tproj_word(mt)], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// K per part: above M = 16 512 (the GEMM adds up to 8 parts with their loads issued before
// its ring starts; measured 1-2 us faster per prefill call than 1024, 256 slower); for
// M <= 16 (whose parts the projection adds itself) 1024, or 256 when that would give fewer
// than 128 workgroups
int tproj_kp(int M, int K) {
  if (M > kRowsMaxM) return 512;
  return (((long)M + 31) / 32) * ((K + 1023) / 1024) < 128 ? 256 : 1024;
}
int tproj_parts(int M, int K) {
  const int kp = tproj_kp(M, K);
  return (K + kp - 1) / kp;
}

hipError_t launch_tproj(int lora, const TprojParams &p, hipStream_t s) {
  const int grid = p.MT * p.parts;
  const int kp = tproj_kp(p.M, p.K);
  if (lora == 1) {
    if (kp == 256) hipLaunchKernelGGL((tproj_kernel<1, 256>), dim3(grid), dim3(256), 0, s, p);
    else if (kp == 512) hipLaunchKernelGGL((tproj_kernel<1, 512>), dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((tproj_kernel<1, 1024>), dim3(grid), dim3(256), 0, s, p);
  } else {
    if (kp == 256) hipLaunchKernelGGL((tproj_kernel<2, 256>), dim3(grid), dim3(256), 0, s, p);
    else if (kp == 512) hipLaunchKernelGGL((tproj_kernel<2, 512>), dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((tproj_kernel<2, 1024>), dim3(grid), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace mnb
