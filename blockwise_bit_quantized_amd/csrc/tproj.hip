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
//  * each thread issues its A loads, then its wave's X loads (MFMA A operand, 8
//    consecutive k of one row per lane; a wave owns kp/4 consecutive k), before waiting
//    on anything: loads return in issue order, so the transposes run while X streams in
//    (at 1024 x 4096 the stamped A phase went from 1.9 to 1.0 us of a ~3.9 us pass);
//  * v_mfma_f32_32x32x16_f16 per 16 k, all B operands read from LDS first, one chain in
//    k order; the four waves meet in LDS in fixed order.
// No cross-workgroup waits (with `reduce`, an arrival counter per M tile picks the
// workgroup that adds the parts).
#include "common.h"

namespace mnb {
namespace {

typedef float f4_t __attribute__((ext_vector_type(4)));
// cache-policy operand of the buffer-load builtins for an agent-scope coherent load: sc1
constexpr int kCoherentSc1 = 16;

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

  const int kw = kbeg + wave * (kKP / 4);

  // 1. this thread's 8x8 tiles (k octet, r octet) of the A part, raw, into registers.  They
  //    are issued before X: a wave's loads return in issue order, so the transposes below
  //    run while X is still streaming in instead of after it.
  constexpr int kTiles = kKP / 8 * 4;
  constexpr int kTilesPerThread = (kTiles + 255) / 256;
  u4_t araw[kTilesPerThread][8];       // F16: row e of the tile; INT8: .xy = row e's 8 bytes
  u4_t asc[kTilesPerThread];           // INT8: the tile's 8 block scales
#pragma unroll
  for (int i = 0; i < kTilesPerThread; ++i) {
    const int t = tid + 256 * i;
    const int ko = t >> 2, ro = t & 3;
    const int k0 = kbeg + ko * 8;
    if (t < kTiles && k0 < kend) {
      if constexpr (KIND == 1) {
        const uint16_t *A = static_cast<const uint16_t *>(p.A);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          araw[i][e] = *reinterpret_cast<const u4_t *>(A + (size_t)(k0 + e) * kRank + ro * 8);
      } else {
        const int8_t *A = static_cast<const int8_t *>(p.A);
        asc[i] = *reinterpret_cast<const u4_t *>(p.sA + (size_t)(k0 / kBlock) * kRank + ro * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint2 a = *reinterpret_cast<const uint2 *>(A + (size_t)(k0 + e) * kRank + ro * 8);
          araw[i][e] = u4_t{a.x, a.y, 0u, 0u};
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) araw[i][e] = u4_t{0u, 0u, 0u, 0u};
      asc[i] = u4_t{0u, 0u, 0u, 0u};
    }
  }

  // 2. X operand loads for this wave's k range (8 consecutive k of one row per lane)
  const _Float16 *xr = reinterpret_cast<const _Float16 *>(p.X) + (size_t)(mok ? mrow : 0) * p.K;
  h8_t xa[kStepsPerWave];
#pragma unroll
  for (int s = 0; s < kStepsPerWave; ++s) {
    const int k = kw + 16 * s + hk;
    xa[s] = *reinterpret_cast<const h8_t *>(xr + (k < kend ? k : 0));
  }

  // 3. A part -> LDS transposed, so that the MFMA B operand (8 consecutive k of one rank) is
  //    a single ds_read_b128
#pragma unroll
  for (int i = 0; i < kTilesPerThread; ++i) {
    const int t = tid + 256 * i;
    if (t >= kTiles) continue;
    const int ko = t >> 2, ro = t & 3;
    uint32_t v[8][4];   // v[row e][dword d] = halves (r = 2d, 2d+1) of A[k0+e][8*ro ..]
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (KIND == 1) {
#pragma unroll
        for (int d = 0; d < 4; ++d) v[e][d] = araw[i][e][d];
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t bytes = d < 2 ? araw[i][e][0] : araw[i][e][1];
          const int8_t lo = (int8_t)((bytes >> (16 * (d & 1))) & 0xff);
          const int8_t hi = (int8_t)((bytes >> (16 * (d & 1) + 8)) & 0xff);
          const h2_t s2 = as_h2(asc[i][d]);
          const h2_t q = {(_Float16)((float)lo * (float)s2[0]), (_Float16)((float)hi * (float)s2[1])};
          v[e][d] = as_u32(q);
        }
      }
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

  // 4. this wave's k-steps inside the part (a wave-uniform count): all B operands read
  //    first, then one MFMA chain in k order
  const int nst = __builtin_amdgcn_readfirstlane(min(kStepsPerWave, max(0, (kend - kw + 15) / 16)));
  f16x_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  const int r = lane & 31;
  h8_t bq[kStepsPerWave];
#pragma unroll
  for (int s = 0; s < kStepsPerWave; ++s)
    if (s < nst) bq[s] = *reinterpret_cast<const h8_t *>(&sAT[r * kLdA + (kw - kbeg) + 16 * s + hk]);
#pragma unroll
  for (int s = 0; s < kStepsPerWave; ++s) {
    if (s < nst) {
      h8_t a = xa[s];
      if (!mok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (_Float16)0.f;
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bq[s], acc, 0, 0, 0);
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
  // Thread tid adds 4 consecutive ranks of one row (row tid / 8 of the tile) over the parts,
  // in part order: 16-byte device-coherent loads (sc1: they miss in this XCD's L2 rather
  // than hit a stale line), up to kB parts in flight at once.  Measured per small-M call
  // against one dword per lane and part, four parts at a time: 0.3-1.6 us faster at 10
  // and 16 parts, 0.15 us slower at 8 (8192 x 2048, M <= 8); dwords with every part in
  // flight were slower than both.  The 32-bit offsets reach parts * M * 128 bytes, below
  // 2^31 for the M <= 16 that reduce (K < 2^25).
  const int m = mt * 32 + (tid >> 3);
  if (m < p.M) {
    constexpr int kB = 16;
    const auto rt = buffer_rsrc(p.tpart, (long)p.parts * p.M * kRank * 4);
    const uint32_t off = ((uint32_t)m * kRank + (tid & 7) * 4) * 4u;
    const uint32_t pstride = (uint32_t)p.M * kRank * 4u;
    f4_t tot = {0.f, 0.f, 0.f, 0.f};
    for (int pp = 0; pp < p.parts; pp += kB) {
      const int n = min(kB, p.parts - pp);  // wave-uniform: scalar branches, no lane masks
      f4_t v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (u < n) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rt, off + (uint32_t)(pp + u) * pstride, 0, kCoherentSc1);
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (u < n) tot += v[u];
    }
    *reinterpret_cast<f4_t *>(p.tfinal + (size_t)m * kRank + (tid & 7) * 4) = tot;
  }
  if (tid == 0) __hip_atomic_store(&p.ctrl[ctrl_tproj_word(mt)], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// K per part: above M = 16 512 (the GEMM adds up to 8 parts with their loads issued before
// its ring starts; measured 1-2 us faster per prefill call than 1024, 256 slower).  Up to
// 16 rows and K <= 2048, 256 or 512: at most 4 parts, which the small-M GEMV loads ahead of
// its weight stream and adds itself, with no reduction round trips in the projection
// (8192 x 2048 with an F16 adapter at M = 2-16: 1.1-1.3 us faster per call than 8 parts
// reduced).  Longer K: 1024, or 256 when that would give fewer than 128 workgroups, and the
// projection reduces the parts (`reduce`): 4 parts of 1024 k measured 0.2-0.4 us faster at
// 4096 x 4096 but 1.3-2.1 us slower with the INT8 adapter of 9728 x 2560 (3 workgroups,
// each converting 1024 rows of A).
int tproj_kp(int M, int K) {
  if (M > kRowsMaxM) return 512;
  if (K <= 2048) return K <= 1024 ? 256 : 512;
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
