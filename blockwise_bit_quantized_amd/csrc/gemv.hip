// gemv.hip -- decode path of MatMulNBits (M == 1; any M when forced): one HBM pass over
// the packed 2-, 4- or 8-bit weights with dequantization in registers, FP32 accumulation,
// and the rank-32 LoRA term fused into the same launch.
//
// Operation (onnxruntime PR #33370 "[WebGPU] Fuse rank-32 quantized LoRA with
// MatMulNBits", commit list: decode computes base + T and then base + T*Bt^T, sharing the
// decode GEMV reduction; here both happen in one launch):
//   y[n] = sum_kb s[n,kb] * sum_{k in kb} x[k] * (q[n,k] - z[n,kb])  +  sum_r t[r] * b[r,n]
//   t[r] = sum_k x[k] * a[k,r]
//
// Work decomposition (gfx950, wave64, kWaves waves per workgroup):
//  * a workgroup owns R = 64/Q rows of one 64-row group over the whole of K, so no partial
//    sums leave the workgroup.  One wave load of 16 B per lane covers R rows x Q
//    chunk-columns (Q contiguous segments of R*16 B inside the 1 KiB chunks of the packed
//    layout); Q is chosen so the grid has enough workgroups to spread over the 256 CUs;
//  * every wave issues all of its code, scale and zero-point loads first; the X slice the
//    workgroup needs is staged into LDS meanwhile, so the only memory round trip before
//    the arithmetic is the weight stream itself;
//  * (q - z) is formed exactly in fp16 and dotted with X pairs by v_dot2_f32_f16; each
//    chunk's partial is scaled once in FP32.  The Q lanes that share a row are combined by
//    lane exchange, the waves through LDS, both in fixed order;
//  * in-pass T: the first `gt` workgroups of the grid compute T over K-slices of `kt` rows.
//    Each slice is written as 32 (value, tag) 64-bit words with device-coherent stores,
//    where the tag identifies this call (a per-call epoch kept in the workspace, never 0),
//    into kTReplicas copies, so that the readers spread over many lines.  Each row
//    workgroup has one extra wave that carries no weight loads: it polls one word of its
//    copy (the last slice's first word), then reads all the words, accepts them
//    when every tag matches (no fences: the tags make a stale or early read detectable),
//    adds the slices in slice order and leaves T in LDS for the epilogue.  The slice
//    workgroups are dispatched first and never wait, so every bounded wait ends.  Every
//    workgroup reports that it has read the epoch through a two-level count (kDoneGroups
//    counters, then one) issued right after that read; the last arrival resets the counts
//    and advances the epoch.
#include <algorithm>

#include "common.h"

namespace mnb {
namespace {

enum { LORA_NONE = 0, LORA_F16 = 1, LORA_Q8 = 2 };
enum { T_INPASS = 0, T_PRECOMP = 1 };
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxSlicesUnrolled = 16;
constexpr int kTSliceMax = 256;     // k rows per in-pass T slice (the host passes kt <= this)

__device__ __forceinline__ uint32_t call_tag(uint32_t epoch) { return (epoch & 0x7fffffffu) + 1u; }
__device__ __forceinline__ unsigned long long tagged(float v, uint32_t tag) {
  return (unsigned long long)__builtin_bit_cast(uint32_t, v) | ((unsigned long long)tag << 32);
}

// sum_{j < n} src[j * stride], in j order.  The first U loads are issued together (from
// clamped addresses) before any is consumed, so they cost one memory round trip.
template <int U>
__device__ __forceinline__ float sum_parts(const float *src, size_t stride, int n) {
  float v[U];
#pragma unroll
  for (int j = 0; j < U; ++j) v[j] = src[(size_t)(j < n ? j : 0) * stride];
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < U; ++j)
    if (j < n) t += v[j];
  for (int j = U; j < n; ++j) t += src[(size_t)j * stride];
  return t;
}

// In-pass T for rank r (lanes 0..31): sum over the gt slices of the tagged words, in slice
// order; false if some slice of this call has not landed yet.  Lanes 32..63 load nothing.
__device__ __forceinline__ bool gather_t(const unsigned long long *tw, int gt, uint32_t tag, int lane, float &t) {
  if (lane >= kRank) {
    t = 0.f;
    return true;
  }
  unsigned long long v[kMaxSlicesUnrolled];
#pragma unroll
  for (int j = 0; j < kMaxSlicesUnrolled; ++j)
    if (j < gt) v[j] = __hip_atomic_load(tw + (size_t)j * kRank + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool ok = true;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxSlicesUnrolled; ++j)
    if (j < gt) {
      ok = ok && (uint32_t)(v[j] >> 32) == tag;
      s += __builtin_bit_cast(float, (uint32_t)v[j]);
    }
  for (int j = kMaxSlicesUnrolled; j < gt; ++j) {
    const unsigned long long w =
        __hip_atomic_load(tw + (size_t)j * kRank + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ok = ok && (uint32_t)(w >> 32) == tag;
    s += __builtin_bit_cast(float, (uint32_t)w);
  }
  t = s;
  return ok;
}

// Epoch count: every workgroup of an in-pass launch (slices and rows) arrives once, right
// after it has read the call epoch, on the counter of its group (id % kDoneGroups, one
// 256-byte line each); after its own work it checks the value it got back, and the last
// arrival of a group adds the group to the second-level count, whose last arrival resets
// both levels and advances the epoch.  So the epoch moves only once every workgroup of the
// launch holds this call's tag, and the round trips overlap the weight stream instead of
// delaying the epilogue.
__device__ __forceinline__ int epoch_arrive(const GemvParams &p, int id) {
  return __hip_atomic_fetch_add(&p.ctrl[ctrl_done_word(id % kDoneGroups)], 1, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void epoch_leave(const GemvParams &p, int id, int old, uint32_t tag) {
  const int total = p.gt + p.nepi;
  const int grp = id % kDoneGroups;
  const int members = (total - grp + kDoneGroups - 1) / kDoneGroups;
  const int groups = min(kDoneGroups, total);
  if (old != members - 1) return;
  __hip_atomic_store(&p.ctrl[ctrl_done_word(grp)], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__hip_atomic_fetch_add(&p.ctrl[CTRL_TDONE], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == groups - 1) {
    __hip_atomic_store(&p.ctrl[CTRL_TDONE], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.ctrl[CTRL_EPOCH], (int)tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One in-pass T slice: words[j][r] = (sum_{k in slice j} x[k] * a[k,r], tag)   (M == 1)
template <int LORA>
__device__ void t_slice(const GemvParams &p, int j, float (*tsh)[kRank]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t tag = call_tag(__hip_atomic_load((const uint32_t *)&p.ctrl[CTRL_EPOCH], __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT));
  int arrived = 0;
  if (threadIdx.x == 0) arrived = epoch_arrive(p, blockIdx.x);
  const int kbeg = j * p.kt;
  const int kend = min(p.K, kbeg + p.kt);
  const _Float16 *x = reinterpret_cast<const _Float16 *>(p.X);
  if (wave >= kWaves) {
    // the workgroup's extra wave (it exists for the row workgroups) only joins the barrier
  } else if constexpr (LORA == LORA_F16) {
    // a wave step covers 16 k-rows of A (1 KiB): lane -> (k = k0 + lane/4, 8 ranks); the
    // slice's steps are unrolled so every load is in flight before the first FMA
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const int r8 = (lane & 3) * 8;
    constexpr int kSteps = kTSliceMax / (16 * kWaves);
    u4_t a[kSteps];
    _Float16 xv[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int k0 = kbeg + wave * 16 + i * 16 * kWaves;
      const int k = k0 < kend ? k0 + (lane >> 2) : 0;
      a[i] = *reinterpret_cast<const u4_t *>(A + (size_t)k * kRank + r8);
      xv[i] = x[k];
      if (k0 >= kend) {           // past the slice: contributes exactly nothing
        a[i] = u4_t{0u, 0u, 0u, 0u};
        xv[i] = (_Float16)0.f;
      }
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int i = 0; i < kSteps; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const h2_t ap = as_h2(a[i][e]);
        acc[2 * e] = fmaf((float)xv[i], (float)ap[0], acc[2 * e]);
        acc[2 * e + 1] = fmaf((float)xv[i], (float)ap[1], acc[2 * e + 1]);
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
    constexpr int kSteps = kTSliceMax / (32 * kWaves) > 0 ? kTSliceMax / (32 * kWaves) : 1;
    u4_t a[kSteps], s0[kSteps], s1[kSteps];
    _Float16 xv[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int k0 = kbeg + wave * 32 + i * 32 * kWaves;
      const int k = k0 < kend ? k0 + (lane >> 1) : 0;
      a[i] = *reinterpret_cast<const u4_t *>(A + (size_t)k * kRank + r16);
      s0[i] = *reinterpret_cast<const u4_t *>(p.sA + (size_t)(k / kBlock) * kRank + r16);
      s1[i] = *reinterpret_cast<const u4_t *>(p.sA + (size_t)(k / kBlock) * kRank + r16 + 8);
      xv[i] = x[k];
      if (k0 >= kend) {
        a[i] = u4_t{0u, 0u, 0u, 0u};
        xv[i] = (_Float16)0.f;
      }
    }
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int i = 0; i < kSteps; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int8_t v = (int8_t)((a[i][e >> 2] >> (8 * (e & 3))) & 0xff);
        const uint32_t sw = (e < 8) ? s0[i][e >> 1] : s1[i][(e - 8) >> 1];
        const float sc = (float)as_h2(sw)[e & 1];
        acc[e] = fmaf((float)xv[i], (float)v * sc, acc[e]);
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
  if (wave == 0 && lane < kRank) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += tsh[w][lane];
    const unsigned long long word = tagged(t, tag);
#pragma unroll
    for (int c = 0; c < kTReplicas; ++c)
      __hip_atomic_store(p.tword + ((size_t)c * p.gt + j) * kRank + lane, word, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x == 0) epoch_leave(p, blockIdx.x, arrived, tag);
}

template <int BITS, bool HAS_ZP, int LORA, int TMODE, int Q, int LPW>
__global__ __launch_bounds__(kThreads + 64) void gemv_kernel(GemvParams p) {
  constexpr int R = kGroup / Q;     // rows per workgroup
  constexpr int KPC = BITS == 2 ? 64 : 32 / (BITS / 4);   // k per chunk: 64, 32 or 16
  constexpr int XW = LPW * Q * KPC; // halfs of X one wave needs per round
  constexpr bool kTWave = LORA != LORA_NONE && TMODE == T_INPASS;
  __shared__ float red[kWaves][kGroup];
  __shared__ float tsh[kWaves][kRank];
  __shared__ float tfin[kRank];
  __shared__ __attribute__((aligned(16))) _Float16 xs[kWaves][XW];   // per-wave X slices

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int bid = blockIdx.x;
  if constexpr (kTWave) {
    if (bid < p.gt) {
      t_slice<LORA>(p, bid, tsh);
      return;
    }
    bid -= p.gt;
  }
  const int m = blockIdx.y;
  // The Q workgroups of one 64-row group read disjoint 128/Q-byte pieces of the same
  // 128-byte scale lines (and zero-point and B lines).  Workgroups are dealt to the 8 XCDs by id modulo 8,
  // so give the Q siblings ids 8 apart: they then share one XCD and its L2 fetches each
  // line once instead of Q times.
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
  const bool active = wave == 0 && lane < R && n < p.N;

  if constexpr (kTWave) {
    if (wave == kWaves) {
      // T wave: carries no weight loads.  It reads the call epoch and counts itself, polls
      // one word of its replica of the slices, reads the tagged words of all slices and
      // leaves T in LDS for the epilogue.  Its loads share the CU's memory pipeline with
      // the weight stream, so they return behind the workgroup's weight loads.
      const uint32_t tag = call_tag(__hip_atomic_load((const uint32_t *)&p.ctrl[CTRL_EPOCH], __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT));
      int arrived = 0;
      if (lane == 0) arrived = epoch_arrive(p, blockIdx.x);
      const unsigned long long *rep = p.tword + (size_t)(bid % kTReplicas) * p.gt * kRank;
      // hint: one lane polls the first word of the last slice (dispatched last, so as a
      // rule done last); the gather below checks every tag anyway.  A single word per
      // poll keeps the uncached polling traffic of hundreds of workgroups small.
      int spins = 0;
      for (; spins < p.spin_limit; ++spins) {
        const bool seen = lane != 0 ||
                          (uint32_t)(__hip_atomic_load(rep + (size_t)(p.gt - 1) * kRank, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT) >> 32) == tag;
        if (__all(seen)) break;
        __builtin_amdgcn_s_sleep(8);
      }
      float tv = 0.f;
      bool ok = false;
      for (; spins <= p.spin_limit && !ok; ++spins) {
        ok = __all(gather_t(rep, p.gt, tag, lane, tv));
        if (!ok) __builtin_amdgcn_s_sleep(1);
      }
      if (!ok) {
        tv = __builtin_nanf("");
        if (lane == 0) atomic_store_agent(&p.ctrl[CTRL_ERROR], 1);
      }
      if (lane < kRank) tfin[lane] = tv;
      __syncthreads();
      if (lane == 0) epoch_leave(p, blockIdx.x, arrived, tag);
      return;
    }
  }

  const int ncc = chunk_cols(BITS, p.KB); // chunk-columns per row
  const int nloads = (ncc + Q - 1) / Q; // wave loads per workgroup
  const _Float16 *xrow = reinterpret_cast<const _Float16 *>(p.X) + (size_t)m * p.K;
  const size_t tile0 = (size_t)g * p.KB;

  // LoRA: this lane's column of B, loaded with the weight stream (independent of T)
  uint32_t bpk[kRank / 2];
  float bscale = 0.f;
  if constexpr (LORA != LORA_NONE) {
    if (wave == 0) {
      const size_t nb = active ? n : 0;
      if constexpr (LORA == LORA_F16) {
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
  }

  float acc = 0.f;
  // rounds of up to kWaves*LPW wave loads (one round at the decode workloads)
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
        // two blocks per chunk: both scales in one word (0 for a block past K), both
        // zero-point bytes in the low two bytes
        const int kb0 = 2 * ccl, kb1 = min(2 * ccl + 1, p.KB - 1);
        const uint32_t s1 = 2 * ccl + 1 < p.KB ? p.sc[(tile0 + kb1) * kGroup + row] : 0u;
        sraw[i] = p.sc[(tile0 + kb0) * kGroup + row] | (s1 << 16);
        zraw[i] = 0;
        if constexpr (HAS_ZP)
          zraw[i] = p.zp[(tile0 + kb0) * 16 + (row >> 2)] | ((uint32_t)p.zp[(tile0 + kb1) * 16 + (row >> 2)] << 8);
      } else {
        const size_t tile = tile0 + ccl / (BITS / 4);
        sraw[i] = p.sc[tile * kGroup + row];
        zraw[i] = 0;
        if constexpr (HAS_ZP) {
          if constexpr (BITS == 4) zraw[i] = p.zp[tile * 32 + (row >> 1)];
          else zraw[i] = p.zp[tile * kGroup + row];
        }
      }
    }
    // 2. this wave's X: slot j = i*Q + qi holds the KPC values of chunk-column
    //    (l0 + wave + kWaves*i)*Q + qi, loaded 16 B per lane (clamped past the end)
    constexpr int kPieces = XW / 8;
#pragma unroll
    for (int pc = lane; pc < kPieces; pc += 64) {
      const int j = pc / (KPC / 8), sub = pc % (KPC / 8);
      const int i = j / Q, q = j % Q;
      const int cc = (l0 + wave + kWaves * i) * Q + q;
      // (2-bit: the second block of the last chunk of an odd block count lies past K; its
      // X is staged as zeros, its scale is 0)
      const int k = cc * KPC + sub * 8;
      const bool kin = cc < ncc && k < p.K;
      u4_t xv = *reinterpret_cast<const u4_t *>(xrow + (kin ? k : 0));
      if (!kin) xv = u4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u4_t *>(&xs[wave][pc * 8]) = xv;
    }
    // 3. arithmetic (xs[wave] is written and read by this wave only: LDS order suffices)
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int l = l0 + wave + kWaves * i;
      const int cc = l * Q + qi;
      if (l < lend && cc < ncc) {
        const uint32_t *xw = reinterpret_cast<const uint32_t *>(&xs[wave][(i * Q + qi) * KPC]);
        if constexpr (BITS == 2) {
          // two blocks; in each 32-bit word the four 2-bit field pairs of a byte are taken
          // in place (v_bfi_b32): pair e comes out as 4^e (q - z), exact, into its own
          // accumulator pe, which a power-of-two FP32 rescale puts back exactly
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            uint32_t z = 2u;
            if constexpr (HAS_ZP) z = ((zraw[i] >> (8 * h)) >> ((row & 3) * 2)) & 3u;
            float pe[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const u4_t xa = *reinterpret_cast<const u4_t *>(xw + 16 * h + 8 * j);
              const u4_t xb = *reinterpret_cast<const u4_t *>(xw + 16 * h + 8 * j + 4);
              const uint32_t w = cw[i][2 * h + j], w8 = w >> 8;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t mask = 0x00030003u << (2 * e);
                const h2_t zz = as_h2(((z << (2 * e)) * 0x00010001u) | 0x64006400u);   // 1024 + 4^e z
                pe[e] = __builtin_amdgcn_fdot2(as_h2(bfi(mask, w, 0x64006400u)) - zz, as_h2(xa[e]), pe[e], false);
                pe[e] = __builtin_amdgcn_fdot2(as_h2(bfi(mask, w8, 0x64006400u)) - zz, as_h2(xb[e]), pe[e], false);
              }
            }
            const float blk = pe[0] + pe[1] * 0.25f + pe[2] * 0.0625f + pe[3] * 0.015625f;
            acc = fmaf(blk, h2f((uint16_t)(sraw[i] >> (16 * h))), acc);
          }
          continue;
        }
        uint32_t z = 1u << (BITS - 1);
        if constexpr (HAS_ZP) z = BITS == 4 ? (zraw[i] >> ((row & 1) * 4)) & 0xFu : zraw[i];
        const h2_t zz2 = as_h2((z * 0x00010001u) | 0x64006400u);   // 1024 + z, both halves
        float p0 = 0.f, p1 = 0.f;
        if constexpr (BITS == 4) {
          // pairs 1 and 3 come out as 16 (q - z) (nib_hi16): p1 holds 16x its terms, which
          // the power-of-two rescale below undoes exactly
          const h2_t zz16 = as_h2((z * 0x00100010u) | 0x64006400u);   // 1024 + 16 z
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u4_t xv = *reinterpret_cast<const u4_t *>(xw + 4 * j);
            const uint32_t w = cw[i][j], w8 = w >> 8;
            p0 = __builtin_amdgcn_fdot2(nib_lo(w) - zz2, as_h2(xv[0]), p0, false);
            p1 = __builtin_amdgcn_fdot2(nib_hi16(w) - zz16, as_h2(xv[1]), p1, false);
            p0 = __builtin_amdgcn_fdot2(nib_lo(w8) - zz2, as_h2(xv[2]), p0, false);
            p1 = __builtin_amdgcn_fdot2(nib_hi16(w8) - zz16, as_h2(xv[3]), p1, false);
          }
          p1 *= 0.0625f;
        } else {
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            const u4_t xv = *reinterpret_cast<const u4_t *>(xw + 2 * j);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const uint32_t w = cw[i][j + jj];
              p0 = __builtin_amdgcn_fdot2(byte_pair_lo(w) - zz2, as_h2(xv[2 * jj]), p0, false);
              p1 = __builtin_amdgcn_fdot2(byte_pair_hi(w) - zz2, as_h2(xv[2 * jj + 1]), p1, false);
            }
          }
        }
        acc = fmaf(p0 + p1, h2f((uint16_t)sraw[i]), acc);
      }
    }
  }
  // lanes sharing a row, then waves, in fixed order
  if constexpr (Q >= 8) acc += __shfl_xor(acc, 8);
  if constexpr (Q >= 4) acc += __shfl_xor(acc, 16);
  if constexpr (Q >= 2) acc += __shfl_xor(acc, 32);
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) total += red[w][rl];

  float lora = 0.f;
  if constexpr (LORA != LORA_NONE) {
    float tv;
    if constexpr (TMODE == T_INPASS) {
      tv = tfin[lane & 31];
    } else {
      // T from the T-projection launch: FP32 partials per K-part, added in part order
      tv = sum_parts<8>(p.tin + (size_t)m * kRank + (lane & 31), (size_t)p.tmpad * kRank, p.tparts);
    }
#pragma unroll
    for (int r = 0; r < kRank; ++r) {
      const float tr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tv), r));
      float b;
      if constexpr (LORA == LORA_F16) b = (float)__builtin_bit_cast(_Float16, (uint16_t)(bpk[r / 2] >> (16 * (r & 1))));
      else b = (float)(int8_t)((bpk[r / 2] >> (16 * (r & 1))) & 0xff);
      lora = fmaf(tr, b, lora);
    }
    if constexpr (LORA == LORA_Q8) lora *= bscale;
  }
  if (active) {
    float y = total + lora;
    if (p.bias) y += h2f(p.bias[n]);
    p.Y[(size_t)m * p.N + n] = __builtin_bit_cast(uint16_t, (_Float16)y);
  }
}

template <int BITS, bool HAS_ZP, int LORA, int TMODE, int Q>
hipError_t launch5(const GemvParams &p, int lpw, int gx, int gy, size_t lds, hipStream_t s) {
  (void)lds;
  const int nt = kThreads + ((LORA != LORA_NONE && TMODE == T_INPASS) ? 64 : 0);
  if (lpw <= 2)
    hipLaunchKernelGGL((gemv_kernel<BITS, HAS_ZP, LORA, TMODE, Q, 2>), dim3(gx, gy), dim3(nt), 0, s, p);
  else if (lpw <= 4)
    hipLaunchKernelGGL((gemv_kernel<BITS, HAS_ZP, LORA, TMODE, Q, 4>), dim3(gx, gy), dim3(nt), 0, s, p);
  else
    hipLaunchKernelGGL((gemv_kernel<BITS, HAS_ZP, LORA, TMODE, Q, 8>), dim3(gx, gy), dim3(nt), 0, s, p);
  return hipGetLastError();
}

template <int BITS, bool HAS_ZP, int LORA, int TMODE>
hipError_t launch4(const GemvParams &p, int lpw, int gx, int gy, size_t lds, hipStream_t s) {
  switch (p.q) {
    case 1: return launch5<BITS, HAS_ZP, LORA, TMODE, 1>(p, lpw, gx, gy, lds, s);
    case 2: return launch5<BITS, HAS_ZP, LORA, TMODE, 2>(p, lpw, gx, gy, lds, s);
    case 4: return launch5<BITS, HAS_ZP, LORA, TMODE, 4>(p, lpw, gx, gy, lds, s);
    default: return launch5<BITS, HAS_ZP, LORA, TMODE, 8>(p, lpw, gx, gy, lds, s);
  }
}

template <int BITS, bool HAS_ZP>
hipError_t launch3(int lora, int tmode, const GemvParams &p, int lpw, int gx, int gy, size_t lds, hipStream_t s) {
  switch (lora) {
    case LORA_NONE: return launch4<BITS, HAS_ZP, LORA_NONE, T_PRECOMP>(p, lpw, gx, gy, lds, s);
    case LORA_F16:
      return tmode == T_INPASS ? launch4<BITS, HAS_ZP, LORA_F16, T_INPASS>(p, lpw, gx, gy, lds, s)
                               : launch4<BITS, HAS_ZP, LORA_F16, T_PRECOMP>(p, lpw, gx, gy, lds, s);
    default:
      return tmode == T_INPASS ? launch4<BITS, HAS_ZP, LORA_Q8, T_INPASS>(p, lpw, gx, gy, lds, s)
                               : launch4<BITS, HAS_ZP, LORA_Q8, T_PRECOMP>(p, lpw, gx, gy, lds, s);
  }
}

int loads_per_wave(int K, int bits, int q) {
  const int ncc = chunk_cols(bits, K / kBlock);
  const int nloads = (ncc + q - 1) / q;
  const int lpw = (nloads + kWaves - 1) / kWaves;
  return lpw <= 2 ? 2 : (lpw <= 4 ? 4 : 8);
}

}  // namespace

// Rows per workgroup = 64 / q: the smallest q in {1, 2, 4, 8} that gives at least 512 row
// workgroups (two per CU), or 256 when the launch also computes T in-pass: the T slices'
// loads then compete with fewer weight streams, and T arrives earlier (measured on the
// 8192 x 2048 decode: 6.5 us at 256 against 6.9 us at 512; base-only 4.97 us at 512
// against 5.29 us at 256).
int gemv_rows_split(int N, bool inpass_t) {
  const int NG = (int)(((long)N + kGroup - 1) / kGroup);
  const int target = inpass_t ? 256 : 512;
  int q = 1;
  while (q < 8 && NG * q < target) q *= 2;
  return q;
}


size_t gemv_lds_bytes(int K, int bits, int q) {
  const int lpw = loads_per_wave(K, bits, q);
  const int ncc = chunk_cols(bits, K / kBlock);
  const int nloads = (ncc + q - 1) / q;
  const int per_round = std::min(nloads, kWaves * lpw);
  const int kpc = bits == 2 ? 64 : 32 / (bits / 4);
  return (size_t)per_round * q * kpc * sizeof(uint16_t);
}

hipError_t launch_gemv(int bits, bool has_zp, int lora, int tmode, const GemvParams &p, int grid_x, int grid_y,
                       hipStream_t s) {
  const int lpw = loads_per_wave(p.K, bits, p.q);
  const size_t lds = gemv_lds_bytes(p.K, bits, p.q);
  if (bits == 2)
    return has_zp ? launch3<2, true>(lora, tmode, p, lpw, grid_x, grid_y, lds, s)
                  : launch3<2, false>(lora, tmode, p, lpw, grid_x, grid_y, lds, s);
  if (bits == 4)
    return has_zp ? launch3<4, true>(lora, tmode, p, lpw, grid_x, grid_y, lds, s)
                  : launch3<4, false>(lora, tmode, p, lpw, grid_x, grid_y, lds, s);
  return has_zp ? launch3<8, true>(lora, tmode, p, lpw, grid_x, grid_y, lds, s)
                : launch3<8, false>(lora, tmode, p, lpw, grid_x, grid_y, lds, s);
}

}  // namespace mnb
