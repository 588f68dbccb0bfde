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
// Global loads run two K-steps ahead of the MFMAs (two register stages, the loop unrolled
// by two so stages are chosen at compile time); one barrier per step.
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

  // this thread's share of the global loads.  Every load is unconditional from a valid
  // (clamped) address; out-of-range data is masked when it is written to LDS, so no wait
  // is ever placed between issuing a load and the MFMAs of the current step.
  const int xr = tid >> 1, xc = (tid & 1) * 32;
  const bool xrow_ok = (m0 + xr) < p.M;
  const _Float16 *X = reinterpret_cast<const _Float16 *>(p.X);
  const _Float16 *xsrc = X + (size_t)(xrow_ok ? m0 + xr : 0) * p.K + xc;
  const int wblk = tid >> 7, wrr = tid & 127;
  const int wg = (n0 >> 6) + (wrr >> 6), wr = wrr & 63;
  const bool wrow_ok = wg < p.NG;
  const int nsteps = (p.KB + 1) / 2;

  // register stages: global -> stage (two K-steps ahead) -> LDS (one step ahead) -> MFMA
  struct Stage {
    u4_t x[4];
    u4_t c[C];
    uint32_t s, z;
    bool xok, wok;
  };
  const u4_t zero4 = {0u, 0u, 0u, 0u};

  auto gload = [&](Stage &st, int step) {
    const bool live = step < nsteps;               // past the end: masked, from a valid address
    step = live ? step : 0;
    const int k0 = step * BK;
    st.xok = live && xrow_ok && (k0 + xc) < p.K;
    const _Float16 *xp = st.xok ? xsrc + k0 : X;
#pragma unroll
    for (int q = 0; q < 4; ++q) st.x[q] = *reinterpret_cast<const u4_t *>(xp + 8 * q);
    const int kb = 2 * step + wblk;
    st.wok = live && wrow_ok && kb < p.KB;
    const size_t t = st.wok ? (size_t)wg * p.KB + kb : 0;
#pragma unroll
    for (int c = 0; c < C; ++c) st.c[c] = *reinterpret_cast<const u4_t *>(p.wq + ((t * C + c) * kGroup + wr) * 16);
    st.s = p.sc[t * kGroup + wr];
    st.z = 0;
    if constexpr (HAS_ZP) {
      if constexpr (BITS == 4) st.z = p.zp[t * 32 + (wr >> 1)];
      else st.z = p.zp[t * kGroup + wr];
    }
  };

  auto sstore = [&](const Stage &st, int buf) {
    u4_t *dx = reinterpret_cast<u4_t *>(&sX[buf][xr * LDK + xc]);
#pragma unroll
    for (int q = 0; q < 4; ++q) dx[q] = st.xok ? st.x[q] : zero4;
    uint32_t z = 1u << (BITS - 1);
    if constexpr (HAS_ZP) z = BITS == 4 ? (st.z >> ((wr & 1) * 4)) & 0xFu : st.z;
    const _Float16 zz = (_Float16)(float)(1024u + z);
    const h2_t zz2 = {zz, zz};
    const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)(st.wok ? st.s : 0u));
    const h2_t s2 = {sv, sv};
    u4_t out[4];
    if constexpr (BITS == 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[j][i] = as_u32((nib_pair(st.c[0][j], i) - zz2) * s2);
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 8 * c + 2 * j;   // dword index of k = 16c + 4j within the block
          out[d >> 2][d & 3] = as_u32((byte_pair_lo(st.c[c][j]) - zz2) * s2);
          out[(d + 1) >> 2][(d + 1) & 3] = as_u32((byte_pair_hi(st.c[c][j]) - zz2) * s2);
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
  Stage sa, sb;                       // even steps use sa, odd steps use sb
  gload(sa, 0);
  gload(sb, 1);
  // LoRA epilogue operands, fetched before the main loop so their latency is hidden:
  // T rows (sum of the FP32 K-part partials, in part order) and this thread's slice of B.
  float tsum[16];
  u4_t braw[2];
  uint32_t bsc[8];
  bool bvec = false;
  const int trow = tid >> 1, thh = (tid & 1) * 16;
  const int br = tid >> 3, bnc = (tid & 7) * 16;
  if constexpr (LORA != 0) {
    const int m = m0 + trow;
    const size_t mrow = m < p.M ? (size_t)m : 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) tsum[e] = 0.f;
    // up to four parts in flight at once (clamped part index, masked), then any rest
    float4 tv[4][4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int pc = pp < p.tparts ? pp : 0;
      const float *src = p.tpart + ((size_t)pc * p.M + mrow) * kRank + thh;
#pragma unroll
      for (int q = 0; q < 4; ++q) tv[pp][q] = *reinterpret_cast<const float4 *>(src + 4 * q);
    }
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      if (pp < p.tparts) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          tsum[4 * q + 0] += tv[pp][q].x;
          tsum[4 * q + 1] += tv[pp][q].y;
          tsum[4 * q + 2] += tv[pp][q].z;
          tsum[4 * q + 3] += tv[pp][q].w;
        }
      }
    }
    for (int pp = 4; pp < p.tparts; ++pp) {
      const float *src = p.tpart + ((size_t)pp * p.M + mrow) * kRank + thh;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4 *>(src + 4 * q);
        tsum[4 * q + 0] += v.x;
        tsum[4 * q + 1] += v.y;
        tsum[4 * q + 2] += v.z;
        tsum[4 * q + 3] += v.w;
      }
    }
    const int n = n0 + bnc;
    if constexpr (LORA == 1) {
      bvec = (p.N % 8) == 0 && n + 16 <= p.N;
      if (bvec) {
        const uint16_t *src = static_cast<const uint16_t *>(p.B) + (size_t)br * p.N + n;
        braw[0] = *reinterpret_cast<const u4_t *>(src);
        braw[1] = *reinterpret_cast<const u4_t *>(src + 8);
      }
    } else {
      bvec = (p.N % 16) == 0 && n + 16 <= p.N;
      if (bvec) {
        braw[0] = *reinterpret_cast<const u4_t *>(static_cast<const int8_t *>(p.B) + (size_t)br * p.N + n);
        const u4_t s0 = *reinterpret_cast<const u4_t *>(p.sB + n);
        const u4_t s1 = *reinterpret_cast<const u4_t *>(p.sB + n + 8);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bsc[q] = s0[q];
          bsc[4 + q] = s1[q];
        }
      }
    }
  }

  auto mfma_step = [&](int buf) {
    h8_t af[BK / 16][2], bf[BK / 16][2];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[kk][mb] = *reinterpret_cast<const h8_t *>(&sX[buf][(wm * 64 + mb * 32 + arow) * LDK + kk * 16 + akof]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bf[kk][nb] = *reinterpret_cast<const h8_t *>(&sW[buf][(wn * 64 + nb * 32 + arow) * LDK + kk * 16 + akof]);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[kk][mb], bf[kk][nb], acc[mb][nb], 0, 0, 0);
  };

  // The pair loop is branch-free (a trailing odd step runs masked with zero data), so
  // the loads of one stage stay in flight across the other stage's MFMAs.
  sstore(sa, 0);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    gload(sa, s + 2);        // even step s: LDS buffer 0 holds step s, stage sb step s+1
    mfma_step(0);
    sstore(sb, 1);
    __syncthreads();
    gload(sb, s + 3);        // odd step s+1: LDS buffer 1 holds step s+1, stage sa step s+2
    mfma_step(1);
    sstore(sa, 0);
    __syncthreads();
  }

  if constexpr (LORA != 0) {
    // epilogue operands: T tile [128 m][32 r] (fp16, rounded once from the FP32 sum) and
    // the B tile transposed to [128 n][32 r]
    _Float16 *sT = &sX[0][0];
    _Float16 *sB = &sW[0][0];
    {
      u4_t o[2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const h2_t hv = {(_Float16)tsum[8 * q + 2 * d], (_Float16)tsum[8 * q + 2 * d + 1]};
          o[q][d] = as_u32(hv);
        }
      *reinterpret_cast<u4_t *>(&sT[trow * LDT + thh]) = o[0];
      *reinterpret_cast<u4_t *>(&sT[trow * LDT + thh + 8]) = o[1];
    }
    {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int n = n0 + bnc + e;
        _Float16 v = (_Float16)0.f;
        if (bvec) {
          if constexpr (LORA == 1) {
            v = as_h2(braw[e >> 3][(e & 7) >> 1])[e & 1];
          } else {
            const int8_t b8 = (int8_t)((braw[0][e >> 2] >> (8 * (e & 3))) & 0xff);
            v = (_Float16)((float)b8 * (float)as_h2(bsc[e >> 1])[e & 1]);
          }
        } else if (n < p.N) {
          if constexpr (LORA == 1) {
            v = __builtin_bit_cast(_Float16, static_cast<const uint16_t *>(p.B)[(size_t)br * p.N + n]);
          } else {
            v = (_Float16)((float)static_cast<const int8_t *>(p.B)[(size_t)br * p.N + n] * h2f(p.sB[n]));
          }
        }
        sB[(bnc + e) * LDT + br] = v;
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
