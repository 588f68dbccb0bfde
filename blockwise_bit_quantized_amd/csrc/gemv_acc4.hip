// gemv_acc4.hip -- MatMulNBits at accuracy level 4: the base product takes int8
// block-quantized activations and integer dot products (v_dot4_i32_i8), the rank-32 LoRA
// term keeps the unquantized FP16 X (T from the T projection launch).
//
// onnxruntime PR #33370 ("[WebGPU] Fuse rank-32 quantized LoRA with MatMulNBits"), commit
// list: the base product may use int8-quantized activations, T is computed from the
// unquantized FP16 X; PR #33800
// ("Fuse DQ->MatMulNBits ...", Description): the lm_head runs at the default accuracy level
// 4.  The pages give no quantization rule; the one used (per row, per block of 32 along
// K): amax = max |x| in FP32, inv = 127 / amax, q = rint(x * inv) clamped to [-127, 127],
// sx = amax / 127, all FP32 with round to nearest even; an all-zero block has q = 0.
//
// Per workgroup (8 waves, MR X rows -- 4 when M > 1, K <= 4096 and the grid is wide, else
// 1 -- and 64/Q weight rows of one 64-row group, as the decode GEMV), so the weights stream
// once per MR rows:
//  * each thread loads its 16-byte pieces of the X row first, then the weight stream;
//  * the X rows are quantized into LDS: four threads share a block (max and sum by lane
//    exchange); the int8 codes are stored in the byte order the weight codes unpack to
//    (4-bit: (w & 0x0F0F0F0F) holds k 0, 4, 1, 5 of a word, (w >> 4) & .. k 2, 6, 3, 7;
//    2-bit: (w >> 2e) & 0x03030303 holds k 2e, 8+2e, 2e+1, 9+2e; 8-bit: natural order),
//    with sx per block and the code sum per 16 k;
//  * per 16-byte chunk and X row: exact int32 sums of q_w * q_x by v_dot4_i32_i8 (8-bit
//    codes as q - 128; the unpacked code words are shared by the rows), minus
//    z_eff * sum(q_x) (z_eff = z, or z - 128 for 8-bit), so the partial is the exact
//    integer sum of (q - z) * q_x; it is scaled once by sx * s in FP32.
#include "common.h"

namespace mnb {
namespace {

enum { LORA_NONE = 0, LORA_F16 = 1, LORA_Q8 = 2 };
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

// byte position of k within its 32-k block in the quantized-X layout of each code width
template <int BITS>
__device__ __forceinline__ int xq_pos(int t) {
  if constexpr (BITS == 4) {          // word j = t / 8: bytes x0 x4 x1 x5 | x2 x6 x3 x7
    const int j = t >> 3, u = t & 7;
    return 8 * j + 2 * (u & 3) + (u >> 2);
  } else if constexpr (BITS == 2) {   // word j = t / 16: groups e of x 2e, 8+2e, 2e+1, 9+2e
    const int j = t >> 4, u = t & 15;
    return 16 * j + 4 * ((u & 7) >> 1) + (u >= 8 ? 1 : 0) + ((u & 1) ? 2 : 0);
  } else {
    return t;
  }
}

template <int BITS, bool HAS_ZP, int LORA, int Q, int LPW, int MR>
__global__ __launch_bounds__(kThreads) void gemv_acc4_kernel(GemvParams p) {
  constexpr int R = kGroup / Q;                                   // rows per workgroup
  constexpr int KPC = BITS == 2 ? 64 : 32 / (BITS / 4);           // k per chunk
  constexpr int KM = MR == 1 ? kAcc4MaxK : kAcc4MultiRowMaxK;     // K capacity per X row
  __shared__ float red[kWaves][MR][kGroup];
  __shared__ __attribute__((aligned(16))) int8_t xq[MR * KM];     // quantized X rows
  __shared__ float sxs[MR * KM / 32];                             // sx per block
  __shared__ int sqs[MR * KM / 16];                               // sum of codes per 16 k

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = blockIdx.y * MR;                                 // first X row
  const int nrows = min(MR, p.M - m0);
  int wgi = blockIdx.x;
  if (Q > 1 && (p.NG & 7) == 0) {
    const int x = wgi & 7, u = wgi >> 3;
    wgi = (x + 8 * (u / Q)) * Q + (u % Q);
  }
  const int g = wgi / Q;
  const int rowoff = (wgi - g * Q) * R;
  const int rl = lane % R, qi = lane / R;
  const int row = rowoff + rl;
  const int n = g * kGroup + row;
  const int ncc = chunk_cols(BITS, p.KB);
  const int nloads = (ncc + Q - 1) / Q;
  const size_t tile0 = (size_t)g * p.KB;
  const _Float16 *X = reinterpret_cast<const _Float16 *>(p.X);

  // 1. this thread's X pieces (8 halfs each) first: their wait then does not wait for the
  //    weight stream issued after them.  Piece pc is piece pc % (K/8) of row m0 + pc / (K/8)
  //    (a block's four pieces never straddle two rows, as K % 32 == 0)
  constexpr int kMaxPieces = MR * KM / 8 / kThreads;
  const int rpieces = p.K / 8;
  const int npieces = nrows * rpieces;
  u4_t xv[kMaxPieces];
#pragma unroll
  for (int i = 0; i < kMaxPieces; ++i) {
    if (i * kThreads >= npieces) break;       // uniform: passes past the last piece
    const int pc = tid + i * kThreads;
    const int pcl = pc < npieces ? pc : 0;
    const int r = pcl / rpieces;
    xv[i] = *reinterpret_cast<const u4_t *>(X + (size_t)(m0 + r) * p.K + 8 * (pcl - r * rpieces));
  }

  float acc[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) acc[r] = 0.f;
  for (int l0 = 0; l0 < nloads; l0 += kWaves * LPW) {
    const int lend = min(nloads, l0 + kWaves * LPW);
    // 2. weight stream of the round
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
        const int kb0 = 2 * ccl, kb1 = min(2 * ccl + 1, p.KB - 1);
        const uint32_t s1 = 2 * ccl + 1 < p.KB ? p.sc[(tile0 + kb1) * kGroup + row] : 0u;
        sraw[i] = p.sc[(tile0 + kb0) * kGroup + row] | (s1 << 16);
        zraw[i] = 2u | (2u << 8);
        if constexpr (HAS_ZP) {
          const int sh = (row & 3) * 2;
          zraw[i] = ((p.zp[(tile0 + kb0) * 16 + (row >> 2)] >> sh) & 3u) |
                    (((uint32_t)(p.zp[(tile0 + kb1) * 16 + (row >> 2)] >> sh) & 3u) << 8);
        }
      } else {
        const size_t tile = tile0 + ccl / (BITS / 4);
        sraw[i] = p.sc[tile * kGroup + row];
        zraw[i] = 1u << (BITS - 1);
        if constexpr (HAS_ZP) {
          if constexpr (BITS == 4) zraw[i] = (p.zp[tile * 32 + (row >> 1)] >> ((row & 1) * 4)) & 0xFu;
          else zraw[i] = p.zp[tile * kGroup + row];
        }
      }
    }

    // 3. quantize the X row into LDS (first round only); four consecutive threads hold
    //    the four pieces of a block
    if (l0 == 0) {
#pragma unroll
      for (int i = 0; i < kMaxPieces; ++i) {
        if (i * kThreads >= npieces) break;
        const int pc = tid + i * kThreads;
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const h2_t h = as_h2(xv[i][e]);
          v[2 * e] = (float)h[0];
          v[2 * e + 1] = (float)h[1];
        }
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        const float inv = amax > 0.f ? 127.f / amax : 0.f;
        int sum = 0;
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          q[e] = (int)fminf(fmaxf(rintf(v[e] * inv), -127.f), 127.f);
          sum += q[e];
        }
        sum += __shfl_xor(sum, 1);     // the 16 k of this piece and its neighbour
        if (pc < npieces) {
          const int r = pc / rpieces, lp = pc - r * rpieces;
          const int kb = lp >> 2, t0 = 8 * (lp & 3);
#pragma unroll
          for (int e = 0; e < 8; ++e) xq[r * KM + 32 * kb + xq_pos<BITS>(t0 + e)] = (int8_t)q[e];
          if ((lp & 1) == 0) sqs[r * (KM / 16) + (lp >> 1)] = sum;
          if ((lp & 3) == 0) sxs[r * (KM / 32) + kb] = amax / 127.f;
        }
      }
      __syncthreads();
    }

    // 4. integer dot products per chunk, one FP32 scaling per block
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int l = l0 + wave + kWaves * i;
      const int cc = l * Q + qi;
      if (l < lend && cc < ncc) {
        const int k0 = cc * KPC;                      // first k of the chunk
        if constexpr (BITS == 4) {
          const int kb = cc;
          int wlo[4], whi[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            wlo[j] = (int)(cw[i][j] & 0x0F0F0F0Fu);
            whi[j] = (int)((cw[i][j] >> 4) & 0x0F0F0F0Fu);
          }
          const float s = h2f((uint16_t)sraw[i]);
#pragma unroll
          for (int r = 0; r < MR; ++r) {
            if (r < nrows) {
              const int *xw = reinterpret_cast<const int *>(xq + r * KM + k0);
              int isum = 0;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                isum = __builtin_amdgcn_sdot4(wlo[j], xw[2 * j], isum, false);
                isum = __builtin_amdgcn_sdot4(whi[j], xw[2 * j + 1], isum, false);
              }
              const int *sq = sqs + r * (KM / 16);
              const int part = isum - (int)zraw[i] * (sq[2 * kb] + sq[2 * kb + 1]);
              acc[r] = fmaf((float)part, sxs[r * (KM / 32) + kb] * s, acc[r]);
            }
          }
        } else if constexpr (BITS == 2) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int kb = 2 * cc + h;
            if (kb < p.KB) {
              int wc[2][4];
#pragma unroll
              for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) wc[j][e] = (int)((cw[i][2 * h + j] >> (2 * e)) & 0x03030303u);
              const int z = (int)((zraw[i] >> (8 * h)) & 0xFFu);
              const float s = h2f((uint16_t)(sraw[i] >> (16 * h)));
#pragma unroll
              for (int r = 0; r < MR; ++r) {
                if (r < nrows) {
                  const int *xw = reinterpret_cast<const int *>(xq + r * KM + k0);
                  int isum = 0;
#pragma unroll
                  for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) isum = __builtin_amdgcn_sdot4(wc[j][e], xw[8 * h + 4 * j + e], isum, false);
                  const int *sq = sqs + r * (KM / 16);
                  const int part = isum - z * (sq[2 * kb] + sq[2 * kb + 1]);
                  acc[r] = fmaf((float)part, sxs[r * (KM / 32) + kb] * s, acc[r]);
                }
              }
            }
          }
        } else {
          const int kb = cc >> 1;
          int wc[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) wc[j] = (int)(cw[i][j] ^ 0x80808080u);
          const float s = h2f((uint16_t)sraw[i]);
#pragma unroll
          for (int r = 0; r < MR; ++r) {
            if (r < nrows) {
              const int *xw = reinterpret_cast<const int *>(xq + r * KM + k0);
              int isum = 0;
#pragma unroll
              for (int j = 0; j < 4; ++j) isum = __builtin_amdgcn_sdot4(wc[j], xw[j], isum, false);
              const int part = isum - ((int)zraw[i] - 128) * sqs[r * (KM / 16) + cc];
              acc[r] = fmaf((float)part, sxs[r * (KM / 32) + kb] * s, acc[r]);
            }
          }
        }
      }
    }
  }

  // lanes sharing a row, then waves, in fixed order
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    if constexpr (Q >= 8) acc[r] += __shfl_xor(acc[r], 8);
    if constexpr (Q >= 4) acc[r] += __shfl_xor(acc[r], 16);
    if constexpr (Q >= 2) acc[r] += __shfl_xor(acc[r], 32);
    red[wave][r][lane] = acc[r];
  }
  __syncthreads();
  if (wave != 0) return;

  const bool active = lane < R && n < p.N;
  const size_t nb = active ? n : 0;
  float bscale = 1.f;
  if constexpr (LORA == LORA_Q8) bscale = h2f(p.sB[nb]);
  for (int xr = 0; xr < nrows; ++xr) {
    const int m = m0 + xr;
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) total += red[w][xr][rl];
    float lora = 0.f;
    if constexpr (LORA != LORA_NONE) {
      // T (FP32 partials per K-part of the projection launch, added in part order) from
      // the unquantized FP16 X; this lane's column of B
      const float *src = p.tin + (size_t)m * kRank + (lane & 31);
      float tv = 0.f;
      for (int pp = 0; pp < p.tparts; ++pp) tv += src[(size_t)pp * p.tmpad * kRank];
#pragma unroll
      for (int r = 0; r < kRank; ++r) {
        const float tr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tv), r));
        float b;
        if constexpr (LORA == LORA_F16) b = h2f(static_cast<const uint16_t *>(p.B)[(size_t)r * p.N + nb]);
        else b = (float)static_cast<const int8_t *>(p.B)[(size_t)r * p.N + nb];
        lora = fmaf(tr, b, lora);
      }
      lora *= bscale;
    }
    if (active) {
      float y = total + lora;
      if (p.bias) y += h2f(p.bias[n]);
      p.Y[(size_t)m * p.N + n] = __builtin_bit_cast(uint16_t, (_Float16)y);
    }
  }
}

template <int BITS, bool HAS_ZP, int LORA, int Q, int MR>
hipError_t launch_m4(const GemvParams &p, int lpw, int gx, int gy, hipStream_t s) {
  const dim3 grid(gx, gy), block(kThreads);
  if (lpw <= 2) hipLaunchKernelGGL((gemv_acc4_kernel<BITS, HAS_ZP, LORA, Q, 2, MR>), grid, block, 0, s, p);
  else if (lpw <= 4) hipLaunchKernelGGL((gemv_acc4_kernel<BITS, HAS_ZP, LORA, Q, 4, MR>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((gemv_acc4_kernel<BITS, HAS_ZP, LORA, Q, 8, MR>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <int BITS, bool HAS_ZP, int LORA, int Q>
hipError_t launch_q4(const GemvParams &p, int lpw, int gx, int gy, hipStream_t s) {
  // gy counts X rows; a workgroup row takes acc4_rows_mr of them
  const int mr = acc4_rows_mr(p.M, p.N, p.K);
  if (mr == 4) return launch_m4<BITS, HAS_ZP, LORA, Q, 4>(p, lpw, gx, (gy + 3) / 4, s);
  return launch_m4<BITS, HAS_ZP, LORA, Q, 1>(p, lpw, gx, gy, s);
}

template <int BITS, bool HAS_ZP, int LORA>
hipError_t launch_l4(const GemvParams &p, int lpw, int gx, int gy, hipStream_t s) {
  switch (p.q) {
    case 1: return launch_q4<BITS, HAS_ZP, LORA, 1>(p, lpw, gx, gy, s);
    case 2: return launch_q4<BITS, HAS_ZP, LORA, 2>(p, lpw, gx, gy, s);
    case 4: return launch_q4<BITS, HAS_ZP, LORA, 4>(p, lpw, gx, gy, s);
    default: return launch_q4<BITS, HAS_ZP, LORA, 8>(p, lpw, gx, gy, s);
  }
}

template <int BITS, bool HAS_ZP>
hipError_t launch_z4(int lora, const GemvParams &p, int lpw, int gx, int gy, hipStream_t s) {
  switch (lora) {
    case LORA_NONE: return launch_l4<BITS, HAS_ZP, LORA_NONE>(p, lpw, gx, gy, s);
    case LORA_F16: return launch_l4<BITS, HAS_ZP, LORA_F16>(p, lpw, gx, gy, s);
    default: return launch_l4<BITS, HAS_ZP, LORA_Q8>(p, lpw, gx, gy, s);
  }
}

template <int BITS>
hipError_t launch_b4(bool has_zp, int lora, const GemvParams &p, int lpw, int gx, int gy, hipStream_t s) {
  return has_zp ? launch_z4<BITS, true>(lora, p, lpw, gx, gy, s) : launch_z4<BITS, false>(lora, p, lpw, gx, gy, s);
}

}  // namespace

// X rows per workgroup row: 4 when there are several rows, they fit the LDS budget
// (K <= kAcc4MultiRowMaxK) and one row group alone fills the chip (>= 256 workgroups), so
// the weights stream once per 4 rows; else 1.  (8 rows measured slower: their registers
// leave room for one workgroup per CU.)
int acc4_rows_mr(int M, int N, int K) {
  const long wgs = ((long)N + kGroup - 1) / kGroup * gemv_rows_split(N, false);
  return M >= 2 && K <= kAcc4MultiRowMaxK && wgs >= 256 ? 4 : 1;
}

namespace {

// Accuracy level 4 for the prefill GEMM: X' = fp16(q * sx) for every row and block of 32
// along K, with q and sx decided exactly as the GEMV path above does (FP32 amax, 127 / amax,
// rint, clamp, amax / 127), so that the MFMA GEMM multiplies the block-quantized
// activations.  Four threads per block (8 values each, 16-byte loads and stores); the
// block's amax is combined across the four lanes by shuffles.
__global__ __launch_bounds__(256) void acc4_xquant_kernel(const uint16_t *X, uint16_t *Xq, long nblocks) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long blk = t >> 2;
  const bool in = blk < nblocks;
  u4_t raw = u4_t{0u, 0u, 0u, 0u};
  if (in) raw = *reinterpret_cast<const u4_t *>(X + 8 * t);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)as_h2(raw[e >> 1])[e & 1];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));      // the four lanes of a block are adjacent
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const float inv = amax > 0.f ? 127.f / amax : 0.f;
  const float sx = amax / 127.f;
  u4_t out;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const float q0 = fminf(fmaxf(rintf(v[e] * inv), -127.f), 127.f);
    const float q1 = fminf(fmaxf(rintf(v[e + 1] * inv), -127.f), 127.f);
    const h2_t h = {(_Float16)(q0 * sx), (_Float16)(q1 * sx)};
    out[e >> 1] = as_u32(h);
  }
  if (in) *reinterpret_cast<u4_t *>(Xq + 8 * t) = out;
}

}  // namespace

hipError_t launch_acc4_xquant(const uint16_t *X, uint16_t *Xq, int M, int K, hipStream_t s) {
  if (K % kBlock) return hipErrorInvalidValue;
  const long nblocks = (long)M * (K / kBlock);
  const long threads = 4 * nblocks;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(acc4_xquant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, X, Xq, nblocks);
  return hipGetLastError();
}

hipError_t launch_gemv_acc4(int bits, bool has_zp, int lora, const GemvParams &p, int grid_x, int grid_y,
                            hipStream_t s) {
  if (p.K > kAcc4MaxK || p.K % kBlock) return hipErrorInvalidValue;
  const int ncc = chunk_cols(bits, p.KB);
  const int nloads = (ncc + p.q - 1) / p.q;
  const int lpw = (nloads + kWaves - 1) / kWaves;
  if (bits == 2) return launch_b4<2>(has_zp, lora, p, lpw, grid_x, grid_y, s);
  if (bits == 4) return launch_b4<4>(has_zp, lora, p, lpw, grid_x, grid_y, s);
  return launch_b4<8>(has_zp, lora, p, lpw, grid_x, grid_y, s);
}

}  // namespace mnb
