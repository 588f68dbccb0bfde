// gemv_rows.hip -- small-M path of MatMulNBits (2 <= M <= 16): one HBM pass over the packed
// weights serves all M rows, with dequantization in registers and FP32 accumulation; the
// rank-32 LoRA term comes from the T projection launch (FP32 partials per K-part) and is
// added in the epilogue.
//
// onnxruntime PR #33370 ("[WebGPU] Fuse rank-32 quantized LoRA with MatMulNBits"), commit
// list: the path is chosen per matrix by its row count M ("per-matrix row dimension"), and
// fuse_up (M > 1) computes T first and adds T * Bt^T after the base product.  A weight
// matrix read once for a few rows is bound by HBM like the M == 1 decode, so it keeps the
// decode GEMV's structure instead of an MFMA tile (whose 128-row X tile would be mostly
// padding):
//  * a workgroup of 8 waves owns 64/Q rows of one 64-row group over the whole of K; one
//    wave load of 16 B per lane covers 64/Q rows x Q chunk-columns of the packed layout;
//  * the X values of the MR rows that the round's loads need are staged into the wave's
//    own LDS area, so the exact fp16 (q - z) pairs built once per weight word are dotted
//    (v_dot2_f32_f16) with MR rows of X;
//  * block partials are scaled once in FP32; lanes sharing a row meet by lane exchange,
//    waves through LDS, in fixed order.
#include "common.h"

namespace mnb {
namespace {

enum { LORA_NONE = 0, LORA_F16 = 1, LORA_Q8 = 2 };
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kXHalfs = 4096;    // MR x (X halfs per wave per round) <= this: 8 KB of LDS per wave

template <int BITS, int MR, int Q, int LPW>
__global__ __launch_bounds__(kThreads) void gemv_rows_kernel(GemvParams p, int lora) {
  constexpr int R = kGroup / Q;     // rows per workgroup
  constexpr int KPC = BITS == 2 ? 64 : 32 / (BITS / 4);   // k per chunk: 64, 32 or 16
  constexpr int XW = LPW * Q * KPC; // halfs of X one wave needs per round and row
  static_assert(MR * XW <= kXHalfs, "X staging size");
  __shared__ float red[MR][kWaves][kGroup];
  __shared__ __attribute__((aligned(16))) _Float16 xs[kWaves][MR][XW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bid = blockIdx.x;
  const int m0 = blockIdx.y * MR;
  // Q siblings of a 64-row group on one XCD (ids 8 apart), as in the M == 1 GEMV
  int wgi = bid;
  if (Q > 1 && (p.NG & 7) == 0) {
    const int x = bid & 7, u = bid >> 3;
    wgi = (x + 8 * (u / Q)) * Q + (u % Q);
  }
  const int g = wgi / Q;
  const int rowoff = (wgi - g * Q) * R;
  const int rl = lane % R;              // row within this workgroup
  const int qi = lane / R;              // chunk-column slot within a wave load
  const int row = rowoff + rl;          // row within the 64-row group
  const int n = g * kGroup + row;       // this lane's output column
  const bool has_zp = p.zp != nullptr;

  const int ncc = chunk_cols(BITS, p.KB); // chunk-columns per row
  const int nloads = (ncc + Q - 1) / Q; // wave loads per workgroup
  const size_t tile0 = (size_t)g * p.KB;
  const _Float16 *X = reinterpret_cast<const _Float16 *>(p.X);

  float acc[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) acc[r] = 0.f;

  for (int l0 = 0; l0 < nloads; l0 += kWaves * LPW) {
    const int lend = min(nloads, l0 + kWaves * LPW);
    // 1. weight stream: all of this wave's loads of the round (clamped addresses)
    u4_t cw[LPW];
    uint32_t sraw[LPW], zraw[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int l = l0 + wave + kWaves * i;
      const int cc = l * Q + qi;
      const bool ok = l < lend && cc < ncc;
      const int ccl = ok ? cc : 0;
      cw[i] = *reinterpret_cast<const u4_t *>(p.wq + (((size_t)g * ncc + ccl) * kGroup + row) * 16);
      if constexpr (BITS == 2) {
        // two blocks per chunk: scales (0 for a block past K) and zero points of both
        const int kb0 = 2 * ccl, kb1 = min(2 * ccl + 1, p.KB - 1);
        const uint32_t s1 = 2 * ccl + 1 < p.KB ? p.sc[(tile0 + kb1) * kGroup + row] : 0u;
        sraw[i] = p.sc[(tile0 + kb0) * kGroup + row] | (s1 << 16);
        zraw[i] = 2u | (2u << 8);
        if (has_zp) {
          const int sh = (row & 3) * 2;
          zraw[i] = ((p.zp[(tile0 + kb0) * 16 + (row >> 2)] >> sh) & 3u) |
                    (((uint32_t)(p.zp[(tile0 + kb1) * 16 + (row >> 2)] >> sh) & 3u) << 8);
        }
      } else {
        const size_t tile = tile0 + ccl / (BITS / 4);
        sraw[i] = p.sc[tile * kGroup + row];
        zraw[i] = 1u << (BITS - 1);
        if (has_zp) {
          if constexpr (BITS == 4) zraw[i] = (p.zp[tile * 32 + (row >> 1)] >> ((row & 1) * 4)) & 0xFu;
          else zraw[i] = p.zp[tile * kGroup + row];
        }
      }
    }
    // 2. this wave's X for MR rows: slot j = i*Q + qi holds the KPC values of
    //    chunk-column (l0 + wave + kWaves*i)*Q + qi (16 B per lane, clamped past the end;
    //    rows past M read row M-1 and are never stored)
    constexpr int kPieces = XW / 8;
    for (int pc = lane; pc < MR * kPieces; pc += 64) {
      const int r = pc / kPieces, pp = pc - r * kPieces;
      const int j = pp / (KPC / 8), sub = pp % (KPC / 8);
      const int i = j / Q, q = j % Q;
      const int cc = (l0 + wave + kWaves * i) * Q + q;
      const int k = cc * KPC + sub * 8;
      const bool kin = cc < ncc && k < p.K;     // (2-bit: past K in the last chunk -> zeros)
      const _Float16 *xrow = X + (size_t)min(m0 + r, p.M - 1) * p.K;
      u4_t xv = *reinterpret_cast<const u4_t *>(xrow + (kin ? k : 0));
      if (!kin) xv = u4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u4_t *>(&xs[wave][r][pp * 8]) = xv;
    }
    // 3. arithmetic: exact (q - z) pairs once per word, dotted with MR rows of X
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int l = l0 + wave + kWaves * i;
      const int cc = l * Q + qi;
      if (l < lend && cc < ncc) {
        if constexpr (BITS == 2) {
          // two blocks of 32 k = 16 pairs each
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const h2_t zzh = as_h2((((zraw[i] >> (8 * h)) & 3u) * 0x00010001u) | 0x64006400u);
            h2_t d[16];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int e = 0; e < 8; ++e) d[8 * j + e] = crumb_pair(cw[i][2 * h + j], e) - zzh;
            const float sh = h2f((uint16_t)(sraw[i] >> (16 * h)));
#pragma unroll
            for (int r = 0; r < MR; ++r) {
              const u4_t *xv = reinterpret_cast<const u4_t *>(&xs[wave][r][(i * Q + qi) * KPC + 32 * h]);
              float q0 = 0.f, q1 = 0.f;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const u4_t x4 = xv[j];
                q0 = __builtin_amdgcn_fdot2(d[4 * j], as_h2(x4[0]), q0, false);
                q1 = __builtin_amdgcn_fdot2(d[4 * j + 1], as_h2(x4[1]), q1, false);
                q0 = __builtin_amdgcn_fdot2(d[4 * j + 2], as_h2(x4[2]), q0, false);
                q1 = __builtin_amdgcn_fdot2(d[4 * j + 3], as_h2(x4[3]), q1, false);
              }
              acc[r] = fmaf(q0 + q1, sh, acc[r]);
            }
          }
          continue;
        }
        const h2_t zz2 = as_h2((zraw[i] * 0x00010001u) | 0x64006400u);   // 1024 + z, both halves
        if constexpr (BITS == 4) {
          // 4-bit: one chunk = one block = 32 k = 16 pairs
          h2_t d[16];
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) d[4 * j + e] = nib_pair(cw[i][j], e) - zz2;
#pragma unroll
          for (int r = 0; r < MR; ++r) {
            const u4_t *xv = reinterpret_cast<const u4_t *>(&xs[wave][r][(i * Q + qi) * KPC]);
            float q0 = 0.f, q1 = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const u4_t x4 = xv[j];
              q0 = __builtin_amdgcn_fdot2(d[4 * j], as_h2(x4[0]), q0, false);
              q1 = __builtin_amdgcn_fdot2(d[4 * j + 1], as_h2(x4[1]), q1, false);
              q0 = __builtin_amdgcn_fdot2(d[4 * j + 2], as_h2(x4[2]), q0, false);
              q1 = __builtin_amdgcn_fdot2(d[4 * j + 3], as_h2(x4[3]), q1, false);
            }
            acc[r] = fmaf(q0 + q1, h2f((uint16_t)sraw[i]), acc[r]);
          }
        } else {
          // 8-bit: 16 k = 8 pairs
          h2_t d[8];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            d[2 * jj] = byte_pair_lo(cw[i][jj]) - zz2;
            d[2 * jj + 1] = byte_pair_hi(cw[i][jj]) - zz2;
          }
#pragma unroll
          for (int r = 0; r < MR; ++r) {
            const u4_t *xv = reinterpret_cast<const u4_t *>(&xs[wave][r][(i * Q + qi) * KPC]);
            const u4_t x0 = xv[0], x1 = xv[1];
            float q0 = 0.f, q1 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              q0 = __builtin_amdgcn_fdot2(d[e], as_h2(x0[e]), q0, false);
              q1 = __builtin_amdgcn_fdot2(d[4 + e], as_h2(x1[e]), q1, false);
            }
            acc[r] = fmaf(q0 + q1, h2f((uint16_t)sraw[i]), acc[r]);
          }
        }
      }
    }
  }
  // lanes sharing a row, then waves, in fixed order
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    float a = acc[r];
    if constexpr (Q >= 8) a += __shfl_xor(a, 8);
    if constexpr (Q >= 4) a += __shfl_xor(a, 16);
    if constexpr (Q >= 2) a += __shfl_xor(a, 32);
    red[r][wave][lane] = a;
  }
  __syncthreads();
  if (wave != 0) return;

  // LoRA: this lane's column of B, and T rows from the T projection (FP32 partials per
  // K-part, added in part order), T[r] broadcast from lane r
  uint32_t bpk[kRank / 2];
  float bscale = 1.f;
  const bool active = lane < R && n < p.N;
  if (lora != LORA_NONE) {
    const size_t nb = active ? n : 0;
    if (lora == LORA_F16) {
      const uint16_t *Bp = static_cast<const uint16_t *>(p.B);
#pragma unroll
      for (int r = 0; r < kRank; r += 2)
        bpk[r / 2] = Bp[(size_t)r * p.N + nb] | ((uint32_t)Bp[(size_t)(r + 1) * p.N + nb] << 16);
    } else {
      const uint8_t *Bp = static_cast<const uint8_t *>(p.B);
#pragma unroll
      for (int r = 0; r < kRank; r += 2)
        bpk[r / 2] = Bp[(size_t)r * p.N + nb] | ((uint32_t)Bp[(size_t)(r + 1) * p.N + nb] << 16);
      bscale = h2f(p.sB[nb]);
    }
  }
  for (int r = 0; r < MR; ++r) {
    const int m = m0 + r;
    if (m >= p.M) break;
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) total += red[r][w][rl];
    float lsum = 0.f;
    if (lora != LORA_NONE) {
      const float *src = p.tin + (size_t)m * kRank + (lane & 31);
      float tv = 0.f;
      for (int pp = 0; pp < p.tparts; ++pp) tv += src[(size_t)pp * p.tmpad * kRank];
#pragma unroll
      for (int rr = 0; rr < kRank; ++rr) {
        const float tr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tv), rr));
        float b;
        if (lora == LORA_F16) b = (float)__builtin_bit_cast(_Float16, (uint16_t)(bpk[rr / 2] >> (16 * (rr & 1))));
        else b = (float)(int8_t)((bpk[rr / 2] >> (16 * (rr & 1))) & 0xff);
        lsum = fmaf(tr, b, lsum);
      }
      lsum *= bscale;
    }
    float y = total + lsum;
    if (p.bias && active) y += h2f(p.bias[n]);
    if (active) p.Y[(size_t)m * p.N + n] = __builtin_bit_cast(uint16_t, (_Float16)y);
  }
}

template <int BITS, int MR, int Q>
hipError_t launch_q(const GemvParams &p, int lora, int lpw, int gx, int gy, hipStream_t s) {
  constexpr int KPC = BITS == 2 ? 64 : 32 / (BITS / 4);
  constexpr int kCap = kXHalfs / (MR * Q * KPC);   // largest LPW whose X staging fits
  constexpr int kCapP2 = kCap >= 8 ? 8 : kCap >= 4 ? 4 : kCap >= 2 ? 2 : 1;
  const int want = lpw <= 1 ? 1 : lpw <= 2 ? 2 : lpw <= 4 ? 4 : 8;   // one round if it fits
  const int use = want < kCapP2 ? want : kCapP2;                      // else several rounds
  const dim3 grid(gx, gy), block(kThreads);
  switch (use) {
    case 8: hipLaunchKernelGGL((gemv_rows_kernel<BITS, MR, Q, (kCapP2 >= 8 ? 8 : 1)>), grid, block, 0, s, p, lora); break;
    case 4: hipLaunchKernelGGL((gemv_rows_kernel<BITS, MR, Q, (kCapP2 >= 4 ? 4 : 1)>), grid, block, 0, s, p, lora); break;
    case 2: hipLaunchKernelGGL((gemv_rows_kernel<BITS, MR, Q, (kCapP2 >= 2 ? 2 : 1)>), grid, block, 0, s, p, lora); break;
    default: hipLaunchKernelGGL((gemv_rows_kernel<BITS, MR, Q, 1>), grid, block, 0, s, p, lora); break;
  }
  return hipGetLastError();
}

template <int BITS, int MR>
hipError_t launch_mr(const GemvParams &p, int lora, int lpw, int gx, int gy, hipStream_t s) {
  switch (p.q) {
    case 1: return launch_q<BITS, MR, 1>(p, lora, lpw, gx, gy, s);
    case 2: return launch_q<BITS, MR, 2>(p, lora, lpw, gx, gy, s);
    case 4: return launch_q<BITS, MR, 4>(p, lora, lpw, gx, gy, s);
    default: return launch_q<BITS, MR, 8>(p, lora, lpw, gx, gy, s);
  }
}

template <int BITS>
hipError_t launch_bits(const GemvParams &p, int lora, int mr, int lpw, int gx, int gy, hipStream_t s) {
  if (mr <= 4) return launch_mr<BITS, 4>(p, lora, lpw, gx, gy, s);
  if (mr <= 8 || BITS == 2) return launch_mr<BITS, 8>(p, lora, lpw, gx, gy, s);
  if constexpr (BITS != 2) return launch_mr<BITS, 16>(p, lora, lpw, gx, gy, s);
  return hipErrorInvalidValue;
}

}  // namespace

// rows per workgroup; 2-bit stops at 8 (its 64-k chunks would not fit 16 rows of X in LDS)
int gemv_rows_mr(int M, int bits) { return M <= 4 ? 4 : (M <= 8 || bits == 2 ? 8 : 16); }

hipError_t launch_gemv_rows(int bits, int lora, const GemvParams &p, int grid_x, hipStream_t s) {
  const int mr = gemv_rows_mr(p.M, bits);
  const int ncc = chunk_cols(bits, p.KB);
  const int nloads = (ncc + p.q - 1) / p.q;
  const int lpw = (nloads + kWaves - 1) / kWaves;
  const int gy = (int)(((long)p.M + mr - 1) / mr);
  if (bits == 2) return launch_bits<2>(p, lora, mr, lpw, grid_x, gy, s);
  return bits == 4 ? launch_bits<4>(p, lora, mr, lpw, grid_x, gy, s) : launch_bits<8>(p, lora, mr, lpw, grid_x, gy, s);
}

}  // namespace mnb
