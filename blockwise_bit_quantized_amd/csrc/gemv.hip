// gemv.hip -- decode path of MatMulNBits (M == 1; also any M when forced): one HBM pass
// over the packed weights with dequantization in registers, FP32 accumulation, and the
// rank-32 LoRA term fused in the same launch.
//
// Operation (onnxruntime PR #33370 "[WebGPU] Fuse rank-32 quantized LoRA with
// MatMulNBits", commit list: decode uses base + T followed by base + T*Bt^T, sharing the
// decode GEMV reduction; here both steps run in one launch):
//   y[n] = sum_kb s[n,kb] * sum_{k in kb} x[k] * (q[n,k] - z[n,kb])  +  sum_r t[r] * b[r,n]
//   t[r] = sum_k x[k] * a[k,r]
//
// Work decomposition (gfx950, wave64):
//  * a workgroup of 4 waves owns one 64-row group and one K-part of `bpp` blocks; lane l
//    owns row 64g + l, so one 16-byte load per lane streams 1 KiB of contiguous codes and
//    no cross-lane reduction is needed for the base sum;
//  * wave w takes blocks kb_beg + w, + 4, ...; all of a wave's loads (codes, scale, zero
//    point) are issued before any arithmetic so the whole problem is in flight at once;
//  * X is wave-uniform per block (scalar loads); (q - z) is formed exactly in fp16 and
//    dotted with X pairs by v_dot2_f32_f16; the block partial is scaled once in FP32;
//  * the 4 wave partials are summed through LDS in fixed order; with split > 1 the parts
//    of a group meet in the workspace and the last arriving workgroup (one device-scope
//    counter per group) adds them in part order, so results do not depend on timing;
//  * in-pass T: the first `gt` workgroups of the grid compute T over K-slices and publish
//    partials; the last of them adds the partials in slice order and raises a flag.  The
//    epilogue of each group waits on that flag (bounded) only after its base sum is done.
//    Those workgroups are dispatched first and never wait, so the wait always ends.
#include "common.h"

namespace mnb {
namespace {

enum { LORA_NONE = 0, LORA_F16 = 1, LORA_Q8 = 2 };
enum { T_INPASS = 0, T_PRECOMP = 1 };

// One in-pass T slice: t_j[r] = sum_{k in slice j} x[k] * a[k,r]  (M == 1).
template <int LORA>
__device__ void t_slice(const GemvParams &p, int j, float (*tsh)[32]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kbeg = j * p.kt;
  const int kend = min(p.K, kbeg + p.kt);
  const _Float16 *x = reinterpret_cast<const _Float16 *>(p.X);
  if constexpr (LORA == LORA_F16) {
    // a wave step covers 16 k-rows of A (1 KiB): lane -> (k = k0 + lane/4, 8 ranks)
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const int r8 = (lane & 3) * 8;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int k0 = kbeg + wave * 16; k0 < kend; k0 += 64) {
      const int k = k0 + (lane >> 2);
      const u4_t a = *reinterpret_cast<const u4_t *>(A + (size_t)k * kRank + r8);
      const float xv = (float)x[k];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const h2_t ap = as_h2(a[e]);
        acc[2 * e] = fmaf(xv, (float)ap[0], acc[2 * e]);
        acc[2 * e + 1] = fmaf(xv, (float)ap[1], acc[2 * e + 1]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] += __shfl_xor(acc[e], 4);
      acc[e] += __shfl_xor(acc[e], 8);
      acc[e] += __shfl_xor(acc[e], 16);
      acc[e] += __shfl_xor(acc[e], 32);
    }
    if (lane < 4) {
#pragma unroll
      for (int e = 0; e < 8; ++e) tsh[wave][lane * 8 + e] = acc[e];
    }
  } else {
    // INT8 A: a wave step covers 32 k-rows (1 KiB): lane -> (k = k0 + lane/2, 16 ranks)
    const int8_t *A = static_cast<const int8_t *>(p.A);
    const int r16 = (lane & 1) * 16;
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    for (int k0 = kbeg + wave * 32; k0 < kend; k0 += 128) {
      const int k = k0 + (lane >> 1);
      const u4_t a = *reinterpret_cast<const u4_t *>(A + (size_t)k * kRank + r16);
      const u4_t s0 = *reinterpret_cast<const u4_t *>(p.sA + (size_t)(k / kBlock) * kRank + r16);
      const u4_t s1 = *reinterpret_cast<const u4_t *>(p.sA + (size_t)(k / kBlock) * kRank + r16 + 8);
      const float xv = (float)x[k];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int8_t v = (int8_t)((a[e >> 2] >> (8 * (e & 3))) & 0xff);
        const uint32_t sw = (e < 8) ? s0[e >> 1] : s1[(e - 8) >> 1];
        const float s = (float)as_h2(sw)[e & 1];
        acc[e] = fmaf(xv, (float)v * s, acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc[e] += __shfl_xor(acc[e], 2);
      acc[e] += __shfl_xor(acc[e], 4);
      acc[e] += __shfl_xor(acc[e], 8);
      acc[e] += __shfl_xor(acc[e], 16);
      acc[e] += __shfl_xor(acc[e], 32);
    }
    if (lane < 2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) tsh[wave][lane * 16 + e] = acc[e];
    }
  }
  __syncthreads();
  if (wave == 0) {
    if (lane < 32) p.tpart[(size_t)j * kRank + lane] = tsh[0][lane] + tsh[1][lane] + tsh[2][lane] + tsh[3][lane];
    fence_release();
    int old = 0;
    if (lane == 0) old = atomic_add_agent(&p.ctrl[CTRL_TCOUNT], 1);
    old = __shfl(old, 0);
    if (old == p.gt - 1) {
      fence_acquire();
      if (lane < 32) {
        float t = 0.f;
        for (int q = 0; q < p.gt; ++q) t += p.tpart[(size_t)q * kRank + lane];
        p.tfin[lane] = t;
      }
      fence_release();
      if (lane == 0) atomic_store_agent(&p.ctrl[CTRL_TFLAG], 1);
    }
  }
  __syncthreads();
}

template <int BITS, bool HAS_ZP, int LORA, int TMODE, int BPW>
__global__ __launch_bounds__(256) void gemv_kernel(GemvParams p) {
  constexpr int C = BITS / 4;                // 16-byte chunks per block and row
  __shared__ float red[4][kGroup];
  __shared__ float tsh[4][kRank];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int bid = blockIdx.x;
  if constexpr (LORA != LORA_NONE && TMODE == T_INPASS) {
    if (bid < p.gt) {
      t_slice<LORA>(p, bid, tsh);
      return;
    }
    bid -= p.gt;
  }
  const int m = blockIdx.y;
  const int g = bid / p.split;
  const int part = bid - g * p.split;
  const int kb_beg = part * p.bpp;
  const int kb_end = min(p.KB, kb_beg + p.bpp);
  const _Float16 *xrow = reinterpret_cast<const _Float16 *>(p.X) + (size_t)m * p.K;
  const size_t tile0 = (size_t)g * p.KB;

  float acc = 0.f;
  for (int kb0 = kb_beg + wave; kb0 < kb_end; kb0 += 4 * BPW) {
    u4_t cw[BPW][C];
    uint32_t sraw[BPW];
    uint32_t zraw[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int kb = kb0 + 4 * i;
      if (kb < kb_end) {
        const size_t tile = tile0 + kb;
#pragma unroll
        for (int c = 0; c < C; ++c)
          cw[i][c] = *reinterpret_cast<const u4_t *>(p.wq + ((tile * C + c) * kGroup + lane) * 16);
        sraw[i] = p.sc[tile * kGroup + lane];
        if constexpr (HAS_ZP) {
          if constexpr (BITS == 4) zraw[i] = (p.zp[tile * 32 + (lane >> 1)] >> ((lane & 1) * 4)) & 0xFu;
          else zraw[i] = p.zp[tile * kGroup + lane];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int kb = kb0 + 4 * i;
      if (kb < kb_end) {
        const uint32_t *xw = reinterpret_cast<const uint32_t *>(xrow + (size_t)kb * kBlock);
        const uint32_t z = HAS_ZP ? zraw[i] : (1u << (BITS - 1));
        const _Float16 zz = (_Float16)(float)(1024u + z);      // exact: 1024 + z < 2048
        const h2_t zz2 = {zz, zz};
        float p0 = 0.f, p1 = 0.f;
        if constexpr (BITS == 4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t w = cw[i][0][j];
            p0 = __builtin_amdgcn_fdot2(nib_pair(w, 0) - zz2, as_h2(xw[4 * j + 0]), p0, false);
            p1 = __builtin_amdgcn_fdot2(nib_pair(w, 1) - zz2, as_h2(xw[4 * j + 1]), p1, false);
            p0 = __builtin_amdgcn_fdot2(nib_pair(w, 2) - zz2, as_h2(xw[4 * j + 2]), p0, false);
            p1 = __builtin_amdgcn_fdot2(nib_pair(w, 3) - zz2, as_h2(xw[4 * j + 3]), p1, false);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t w = cw[i][c][j];
              p0 = __builtin_amdgcn_fdot2(byte_pair_lo(w) - zz2, as_h2(xw[8 * c + 2 * j]), p0, false);
              p1 = __builtin_amdgcn_fdot2(byte_pair_hi(w) - zz2, as_h2(xw[8 * c + 2 * j + 1]), p1, false);
            }
        }
        acc = fmaf(p0 + p1, h2f((uint16_t)sraw[i]), acc);
      }
    }
  }

  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float total = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
  const int n = g * kGroup + lane;
  const size_t npad = (size_t)p.NG * kGroup;

  if (p.split > 1) {
    p.part[(size_t)part * npad + n] = total;
    fence_release();
    int old = 0;
    if (lane == 0) old = atomic_add_agent(&p.cnt[g], 1);
    old = __shfl(old, 0);
    if (old != p.split - 1) return;
    if (lane == 0) atomic_store_agent(&p.cnt[g], 0);
    fence_acquire();
    total = 0.f;
    for (int q = 0; q < p.split; ++q) total += p.part[(size_t)q * npad + n];
  }

  float lora = 0.f;
  if constexpr (LORA != LORA_NONE) {
    // B column of this lane's output (independent of T: issued before any wait)
    float bcol[kRank];
    if (n < p.N) {
#pragma unroll
      for (int r = 0; r < kRank; ++r) {
        if constexpr (LORA == LORA_F16) bcol[r] = h2f(static_cast<const uint16_t *>(p.B)[(size_t)r * p.N + n]);
        else bcol[r] = (float)static_cast<const int8_t *>(p.B)[(size_t)r * p.N + n];
      }
    } else {
#pragma unroll
      for (int r = 0; r < kRank; ++r) bcol[r] = 0.f;
    }
    float tv;
    if constexpr (TMODE == T_INPASS) {
      int spins = 0;
      bool ok = true;
      while (atomic_load_agent(&p.ctrl[CTRL_TFLAG]) == 0) {
        if (++spins > kSpinLimit) { ok = false; break; }
        __builtin_amdgcn_s_sleep(2);
      }
      tv = ok ? p.tfin[lane & 31] : __builtin_nanf("");
      if (!ok && lane == 0) atomic_store_agent(&p.ctrl[CTRL_ERROR], 1);
      int done = 0;
      if (lane == 0) done = atomic_add_agent(&p.ctrl[CTRL_TDONE], 1);
      done = __shfl(done, 0);
      if (done == p.NG - 1 && lane == 0) {      // every epilogue has read T: reset
        atomic_store_agent(&p.ctrl[CTRL_TFLAG], 0);
        atomic_store_agent(&p.ctrl[CTRL_TCOUNT], 0);
        atomic_store_agent(&p.ctrl[CTRL_TDONE], 0);
      }
    } else {
      tv = h2f(p.t16[(size_t)m * kRank + (lane & 31)]);
    }
#pragma unroll
    for (int r = 0; r < kRank; ++r) {
      const float tr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tv), r));
      lora = fmaf(tr, bcol[r], lora);
    }
    if constexpr (LORA == LORA_Q8) lora *= (n < p.N) ? h2f(p.sB[n]) : 0.f;
  }
  if (n < p.N) {
    const _Float16 y = (_Float16)(total + lora);
    p.Y[(size_t)m * p.N + n] = __builtin_bit_cast(uint16_t, y);
  }
}

template <int BITS, bool HAS_ZP, int LORA, int TMODE>
hipError_t launch4(const GemvParams &p, int bpw, int gx, int gy, hipStream_t s) {
  if (bpw <= 4)
    hipLaunchKernelGGL((gemv_kernel<BITS, HAS_ZP, LORA, TMODE, 4>), dim3(gx, gy), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((gemv_kernel<BITS, HAS_ZP, LORA, TMODE, 8>), dim3(gx, gy), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int BITS, bool HAS_ZP>
hipError_t launch3(int lora, int tmode, const GemvParams &p, int bpw, int gx, int gy, hipStream_t s) {
  switch (lora) {
    case LORA_NONE: return launch4<BITS, HAS_ZP, LORA_NONE, T_PRECOMP>(p, bpw, gx, gy, s);
    case LORA_F16:
      return tmode == T_INPASS ? launch4<BITS, HAS_ZP, LORA_F16, T_INPASS>(p, bpw, gx, gy, s)
                               : launch4<BITS, HAS_ZP, LORA_F16, T_PRECOMP>(p, bpw, gx, gy, s);
    default:
      return tmode == T_INPASS ? launch4<BITS, HAS_ZP, LORA_Q8, T_INPASS>(p, bpw, gx, gy, s)
                               : launch4<BITS, HAS_ZP, LORA_Q8, T_PRECOMP>(p, bpw, gx, gy, s);
  }
}

}  // namespace

hipError_t launch_gemv(int bits, bool has_zp, int lora, int tmode, const GemvParams &p,
                       int grid_x, int grid_y, hipStream_t s) {
  const int bpw = (p.bpp + 3) / 4;
  if (bits == 4)
    return has_zp ? launch3<4, true>(lora, tmode, p, bpw, grid_x, grid_y, s)
                  : launch3<4, false>(lora, tmode, p, bpw, grid_x, grid_y, s);
  return has_zp ? launch3<8, true>(lora, tmode, p, bpw, grid_x, grid_y, s)
                : launch3<8, false>(lora, tmode, p, bpw, grid_x, grid_y, s);
}

}  // namespace mnb
