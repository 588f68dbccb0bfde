// gemm.hip -- prefill path of MatMulNBits (M > 1): FP16 MFMA GEMM over weights that are
// dequantized once per workgroup into LDS, with the rank-32 LoRA up-projection T.B run
// as two extra MFMA k-steps on the same accumulators before the fp16 store.
//
// onnxruntime PR #33370 ("[WebGPU] Fuse rank-32 quantized LoRA with MatMulNBits"), commit
// list: prefill (fuse_up) computes T first, then the base GEMM "with an integrated
// T * Bt^T epilogue"; a later commit names it the "fused LoRA-up output stage".
//
// Tile: 128 x 128 outputs per workgroup of 4 waves (2 x 2, 64 x 64 each as 2 x 2
// v_mfma_f32_32x32x16_f16 blocks), K step 64 (two quantization blocks), LDS double buffer:
//   global -> registers (X 64 B per thread; W 16 or 32 B of codes + scale + zero point)
//   registers -> dequantize (q - z) * s to fp16 (exact subtraction, one rounding) -> LDS
//   LDS -> MFMA operands (ds_read_b128; rows padded to 144 B so 8 consecutive lanes hit
//   distinct banks)
// The next step's global loads are issued before this step's MFMAs; one barrier per step.
// Without an adapter the two epilogue k-steps are skipped, so the base accumulation order
// is the same in every variant and a zero adapter reproduces the base output bitwise.
#include "common.h"

namespace mnb {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;    // halfs per LDS row
constexpr int LDT = kRank + 8; // halfs per LDS row of the epilogue operands

template <int BITS, bool HAS_ZP, int LORA>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  constexpr int C = BITS / 4;
  __shared__ __attribute__((aligned(16))) _Float16 sX[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) _Float16 sW[2][BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile order: consecutive workgroup ids go to different XCDs, so give each XCD
  // a contiguous range of tiles (M fastest) that shares weight columns in its L2.
  const int ntiles = p.MT * p.NT;
  int tile = blockIdx.x;
  if ((ntiles & 7) == 0) tile = (blockIdx.x & 7) * (ntiles >> 3) + (blockIdx.x >> 3);
  const int mt = tile % p.MT, nt = tile / p.MT;
  const int m0 = mt * BM, n0 = nt * BN;

  // this thread's share of the global loads
  const int xr = tid >> 1, xc = (tid & 1) * 32;
  const bool xrow_ok = (m0 + xr) < p.M;
  const _Float16 *xsrc = reinterpret_cast<const _Float16 *>(p.X) + (size_t)(xrow_ok ? m0 + xr : 0) * p.K + xc;
  const int wblk = tid >> 7, wrr = tid & 127;
  const int wg = (n0 >> 6) + (wrr >> 6), wr = wrr & 63;
  const bool wrow_ok = wg < p.NG;
  const int nsteps = (p.KB + 1) / 2;

  u4_t xreg[4];
  u4_t creg[C];
  uint32_t sreg = 0, zreg = 0;
  const u4_t zero4 = {0u, 0u, 0u, 0u};

  auto gload = [&](int step) {
    const int k0 = step * BK;
    const bool xok = xrow_ok && (k0 + xc) < p.K;
#pragma unroll
    for (int q = 0; q < 4; ++q) xreg[q] = xok ? *reinterpret_cast<const u4_t *>(xsrc + k0 + 8 * q) : zero4;
    const int kb = 2 * step + wblk;
    const bool ok = wrow_ok && kb < p.KB;
    const size_t t = (size_t)wg * p.KB + kb;
#pragma unroll
    for (int c = 0; c < C; ++c)
      creg[c] = ok ? *reinterpret_cast<const u4_t *>(p.wq + ((t * C + c) * kGroup + wr) * 16) : zero4;
    sreg = ok ? p.sc[t * kGroup + wr] : 0u;
    if constexpr (HAS_ZP) {
      if constexpr (BITS == 4) zreg = ok ? (p.zp[t * 32 + (wr >> 1)] >> ((wr & 1) * 4)) & 0xFu : 0u;
      else zreg = ok ? p.zp[t * kGroup + wr] : 0u;
    }
  };

  auto sstore = [&](int buf) {
    u4_t *dx = reinterpret_cast<u4_t *>(&sX[buf][xr * LDK + xc]);
#pragma unroll
    for (int q = 0; q < 4; ++q) dx[q] = xreg[q];
    const uint32_t z = HAS_ZP ? zreg : (1u << (BITS - 1));
    const _Float16 zz = (_Float16)(float)(1024u + z);
    const h2_t zz2 = {zz, zz};
    const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)sreg);
    const h2_t s2 = {s, s};
    u4_t out[4];
    if constexpr (BITS == 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[j][i] = as_u32((nib_pair(creg[0][j], i) - zz2) * s2);
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 8 * c + 2 * j;   // dword index of k = 16c + 4j within the block
          out[d >> 2][d & 3] = as_u32((byte_pair_lo(creg[c][j]) - zz2) * s2);
          out[(d + 1) >> 2][(d + 1) & 3] = as_u32((byte_pair_hi(creg[c][j]) - zz2) * s2);
        }
    }
    u4_t *dw = reinterpret_cast<u4_t *>(&sW[buf][wrr * LDK + wblk * 32]);
#pragma unroll
    for (int q = 0; q < 4; ++q) dw[q] = out[q];
  };

  f16x_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  const int arow = (lane & 31);
  const int akof = 8 * (lane >> 5);
  if (nsteps > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) gload(s + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      h8_t af[2], bf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = *reinterpret_cast<const h8_t *>(&sX[buf][(wm * 64 + mb * 32 + arow) * LDK + kk * 16 + akof]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bf[nb] = *reinterpret_cast<const h8_t *>(&sW[buf][(wn * 64 + nb * 32 + arow) * LDK + kk * 16 + akof]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
    }
    if (s + 1 < nsteps) sstore(buf ^ 1);
    __syncthreads();
  }

  if constexpr (LORA != 0) {
    // epilogue operands: T tile [128 m][32 r] and B tile transposed to [128 n][32 r]
    _Float16 *sT = &sX[0][0];
    _Float16 *sB = &sW[0][0];
    {
      const int row = tid >> 1, hh = (tid & 1) * 16;
      const int m = m0 + row;
      u4_t v0 = zero4, v1 = zero4;
      if (m < p.M) {
        v0 = *reinterpret_cast<const u4_t *>(p.t16 + (size_t)m * kRank + hh);
        v1 = *reinterpret_cast<const u4_t *>(p.t16 + (size_t)m * kRank + hh + 8);
      }
      *reinterpret_cast<u4_t *>(&sT[row * LDT + hh]) = v0;
      *reinterpret_cast<u4_t *>(&sT[row * LDT + hh + 8]) = v1;
    }
    {
      const int r = tid >> 3, nc = (tid & 7) * 16;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int n = n0 + nc + e;
        _Float16 v = (_Float16)0.f;
        if (n < p.N) {
          if constexpr (LORA == 1) {
            v = __builtin_bit_cast(_Float16, static_cast<const uint16_t *>(p.B)[(size_t)r * p.N + n]);
          } else {
            v = (_Float16)((float)static_cast<const int8_t *>(p.B)[(size_t)r * p.N + n] * h2f(p.sB[n]));
          }
        }
        sB[(nc + e) * LDT + r] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRank / 16; ++kk) {
      h8_t af[2], bf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = *reinterpret_cast<const h8_t *>(&sT[(wm * 64 + mb * 32 + arow) * LDT + kk * 16 + akof]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bf[nb] = *reinterpret_cast<const h8_t *>(&sB[(wn * 64 + nb * 32 + arow) * LDT + kk * 16 + akof]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
    }
  }

  // store: accumulator register v of a 32x32 block holds row 8*(v/4) + 4*(lane/32) + v%4,
  // column lane % 32
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = n0 + wn * 64 + nb * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < p.M && n < p.N)
          p.Y[(size_t)m * p.N + n] = __builtin_bit_cast(uint16_t, (_Float16)acc[mb][nb][v]);
      }
    }
}

template <int BITS, bool HAS_ZP>
hipError_t launch2(int lora, const GemmParams &p, hipStream_t s) {
  const dim3 grid(p.MT * p.NT), block(256);
  switch (lora) {
    case 0: hipLaunchKernelGGL((gemm_kernel<BITS, HAS_ZP, 0>), grid, block, 0, s, p); break;
    case 1: hipLaunchKernelGGL((gemm_kernel<BITS, HAS_ZP, 1>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((gemm_kernel<BITS, HAS_ZP, 2>), grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int bits, bool has_zp, int lora, const GemmParams &p, hipStream_t s) {
  if (bits == 4) return has_zp ? launch2<4, true>(lora, p, s) : launch2<4, false>(lora, p, s);
  return has_zp ? launch2<8, true>(lora, p, s) : launch2<8, false>(lora, p, s);
}

}  // namespace mnb
