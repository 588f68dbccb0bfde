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
//  * every wave issues its X slice and then all of its code, scale and zero-point loads
//    before it waits on anything, so the only memory round trip before the arithmetic is
//    the weight stream itself.  The weight streams are read through buffer descriptors
//    that end at the group's last block (the hardware range check returns zeros past it),
//    so no lane computes a clamped address: the address work per load is one add;
//  * arithmetic is what bounds this kernel once its single round trip has landed (the
//    dequantization runs after the data arrives, on every SIMD at once), so each pair of
//    codes costs one v_bfi_b32 (codes into fp16 mantissas: 1024 + q, or 1024 + 16 q /
//    1024 + 4^e q for fields taken in place) and one v_dot2_f32_f16 against X.  The
//    offsets and the zero point leave the inner loop: each block subtracts C + z S once,
//    with S the block's X sum and C its X sum weighted by the fields' offsets, both
//    computed while X is staged (default zero point: one number).  Each chunk's partial is
//    scaled once in FP32.  The Q lanes that share a row are combined by lane exchange, the
//    waves through LDS, both in fixed order;
//  * in-pass T: the first `gt` workgroups of the grid compute T over K-slices of `kt` rows.
//    Each slice is written as 32 (value, tag) 64-bit words with device-coherent stores,
//    where the tag identifies this call (a per-call epoch kept in the workspace, never 0),
//    into kTReplicas copies, so that the readers spread over many lines.  Each row
//    workgroup has one extra wave that carries no weight loads: it reads all the words of
//    its copy until every tag matches (no fences: the tags make a stale or early read
//    detectable), adds the slices in slice order and leaves T in LDS for the epilogue.  The slice
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

// Lane exchanges for sums (each returns the partner lane's value): xor 1 and xor 2 by DPP
// quad permutes, xor 8 and xor 16 by ds_swizzle (bit-mask mode inside 32 lanes), xor 32 by
// ds_bpermute.  None needs the generic shuffle's width bookkeeping.
__device__ __forceinline__ float lane_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}
template <int MASK>
__device__ __forceinline__ float lane_xor_swz(float v) {
  static_assert(MASK > 0 && MASK < 32, "ds_swizzle exchanges inside 32 lanes");
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), (MASK << 10) | 0x1F));
}
__device__ __forceinline__ float lane_xor32(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, v)));
}

// LoRA term of this lane's row: sum_r t[r] * b[r] in r order, with t[r] in LDS (lane r
// reads it, then each is broadcast by v_readlane) and b[r] packed two per word (F16, or
// INT8 in the low byte of each half with the column scale `bs` applied once at the end).
// (A form that reads t as 16-byte LDS broadcasts into four accumulators measured 0.3 us
// slower per 8192 x 2048 call.)
template <int LORA>
__device__ __forceinline__ float lora_dot(const float *t, const uint32_t *bpk, float bs) {
  const float tv = t[threadIdx.x & 31];
  float lora = 0.f;
#pragma unroll
  for (int r = 0; r < kRank; ++r) {
    const float tr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tv), r));
    float b;
    if constexpr (LORA == LORA_F16) b = (float)__builtin_bit_cast(_Float16, (uint16_t)(bpk[r / 2] >> (16 * (r & 1))));
    else b = (float)(int8_t)((bpk[r / 2] >> (16 * (r & 1))) & 0xff);
    lora = fmaf(tr, b, lora);
  }
  if constexpr (LORA == LORA_Q8) lora *= bs;
  return lora;
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
  __shared__ __attribute__((aligned(16))) _Float16 xs[kWaves][XW];   // per-wave X slices
  __shared__ float2 xsum[kWaves][XW / 8 / (BITS == 8 ? 2 : 4)];       // per-block X sums (C, S)
  __shared__ __attribute__((aligned(16))) float tfin[kRank];              // T for the epilogue

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
      // T wave: carries no weight loads.  It reads the call epoch and counts itself, then
      // reads the tagged words of all slices of its replica until every tag is this call's,
      // and leaves T in LDS for the epilogue.  Each read of the words is the poll: a
      // separate one-word poll before the read cost one more memory round trip between the
      // slices landing and T being in hand (4096 x 4096 M = 1: 6.87 -> 6.50 us), while the
      // extra polling traffic (gt x 256 B per read per workgroup) goes to lines that stay
      // in the device cache.  Its loads share the CU's memory pipeline with the weight
      // stream, so they return behind the workgroup's weight loads.
      const uint32_t tag = call_tag(__hip_atomic_load((const uint32_t *)&p.ctrl[CTRL_EPOCH], __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT));
      int arrived = 0;
      if (lane == 0) arrived = epoch_arrive(p, blockIdx.x);
      const unsigned long long *rep = p.tword + (size_t)(bid % kTReplicas) * p.gt * kRank;
      int spins = 0;
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
  // Per-lane byte offsets inside one wave load's window (Q chunk-columns, this lane's row);
  // the uniform part of each load's offset is added per load.  Codes, scales and zero points
  // are read through buffer descriptors that end at the group's last block, so a lane whose
  // chunk-column lies past the row (K not a multiple of Q chunk-columns), and every load of a
  // slot past the last wave load, reads zeros; its X is staged as zeros too, so it adds
  // exactly nothing.
  constexpr int kZpLane = BITS == 4 ? 32 : (BITS == 8 ? 64 : 16);   // zero-point bytes per block
  const uint32_t w_lane = (uint32_t)(qi * kGroup + row) * 16u;
  uint32_t s_lane, z_lane;
  if constexpr (BITS == 4) {
    s_lane = (uint32_t)(qi * kGroup + row) * 2u;
    z_lane = (uint32_t)(qi * kZpLane + (row >> 1));
  } else if constexpr (BITS == 8) {
    s_lane = (uint32_t)((qi >> 1) * kGroup + row) * 2u;
    z_lane = (uint32_t)((qi >> 1) * kZpLane + row);
  } else {
    s_lane = (uint32_t)(2 * qi * kGroup + row) * 2u;
    z_lane = (uint32_t)(2 * qi * kZpLane + (row >> 2));
  }
  // X: piece pc (8 halfs, 16 B) of this wave's slots; its byte offset minus the uniform
  // (l0 + wave) * Q * KPC * 2 part, and the correction slot it contributes to
  constexpr int kPieces = XW / 8;
  constexpr int kPiecesPerChunk = KPC / 8;
  constexpr int kPiecesPerSum = BITS == 8 ? 2 : 4;       // one sum per 32-k block (8-bit: per chunk)


  // LoRA: this lane's column of B, loaded ahead of the weight stream (independent of T)
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
    const int c0 = l0 * Q;                                   // first chunk-column of the round
    const int kb0 = BITS == 4 ? c0 : (BITS == 8 ? c0 / 2 : 2 * c0);   // its first block
    const auto rw = buffer_rsrc(p.wq + ((size_t)g * ncc + c0) * kGroup * 16, (long)(ncc - c0) * kGroup * 16);
    const auto rs = buffer_rsrc(p.sc + ((size_t)g * p.KB + kb0) * kGroup, (long)(p.KB - kb0) * kGroup * 2);
    const auto rz = buffer_rsrc(HAS_ZP ? p.zp + ((size_t)g * p.KB + kb0) * kZpLane : p.wq,
                                HAS_ZP ? (long)(p.KB - kb0) * kZpLane : 0);
    // 1. X first (its loads return first), then this wave's weight stream
    u4_t xv[(kPieces + 63) / 64];
    {
      const auto rx = buffer_rsrc(xrow, (long)p.K * 2);
#pragma unroll
      for (int t = 0; t < (kPieces + 63) / 64; ++t) {
        const int pc = lane + 64 * t;
        const int j = pc / kPiecesPerChunk, sub = pc % kPiecesPerChunk;
        const int cc = (l0 + wave + kWaves * (j / Q)) * Q + j % Q;
        const uint32_t off = pc < kPieces ? (uint32_t)(cc * KPC + sub * 8) * 2u : 0x7ffffff0u;
        xv[t] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
      }
    }
    u4_t cw[LPW];
    uint32_t sraw[LPW], zraw[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const uint32_t rel = (uint32_t)(wave + kWaves * i);    // load index within the round
      cw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane + rel * (Q * kGroup * 16), 0, 0);
      if constexpr (BITS == 4) {
        sraw[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, s_lane + rel * (Q * kGroup * 2), 0, 0);
        zraw[i] = HAS_ZP ? __builtin_amdgcn_raw_buffer_load_b8(rz, z_lane + rel * (Q * kZpLane), 0, 0) : 0u;
      } else if constexpr (BITS == 8) {
        const uint32_t tl = (rel * Q) >> 1;                  // block of the load (Q = 1: two loads per block)
        sraw[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, s_lane + tl * (kGroup * 2), 0, 0);
        zraw[i] = HAS_ZP ? __builtin_amdgcn_raw_buffer_load_b8(rz, z_lane + tl * kZpLane, 0, 0) : 0u;
      } else {
        // two blocks per chunk: both scales in one word, both zero-point bytes in the low two
        const uint32_t so = s_lane + rel * (Q * kGroup * 4), zo = z_lane + rel * (Q * kZpLane * 2);
        sraw[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0) |
                  ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, so + kGroup * 2, 0, 0) << 16);
        zraw[i] = HAS_ZP ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, zo, 0, 0) |
                               ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, zo + kZpLane, 0, 0) << 8)
                         : 0u;
      }
    }
    // 2. X to LDS, with each block's X sums: the codes enter the dot products as 1024 + q
    //    (and 1024 + 16 q or 1024 + 4^e q for the in-place fields), so every block subtracts
    //    C + z S once, where S is the block's X sum and C the X sum weighted by each field's
    //    offset (default zero point: C + z S is one number, folded into the constants).
    //    xsum[wave] is written and read by this wave only: LDS order suffices.
#pragma unroll
    for (int t = 0; t < (kPieces + 63) / 64; ++t) {
      const int pc = lane + 64 * t;
      if (pc < kPieces) *reinterpret_cast<u4_t *>(&xs[wave][pc * 8]) = xv[t];
      constexpr float zd = (float)(1 << (BITS - 1));          // default zero point
      const float zc = HAS_ZP ? 0.f : zd;
      float c = 0.f, s = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // field offset of word e of the piece: 4-bit 1024, 64 (the 16x fields, rescaled);
        // 8-bit 1024; 2-bit 1024 / 4^e
        const float off = BITS == 8 ? 1024.f : (BITS == 4 ? ((e & 1) ? 64.f : 1024.f) : 1024.f / (float)(1 << (2 * e)));
        const _Float16 k = (_Float16)(off + zc);
        c = __builtin_amdgcn_fdot2(as_h2(xv[t][e]), h2_t{k, k}, c, false);
        if constexpr (HAS_ZP) s = __builtin_amdgcn_fdot2(as_h2(xv[t][e]), h2_t{(_Float16)1.f, (_Float16)1.f}, s, false);
      }
      c += lane_xor1(c);
      if constexpr (HAS_ZP) s += lane_xor1(s);
      if constexpr (kPiecesPerSum == 4) {
        c += lane_xor2(c);
        if constexpr (HAS_ZP) s += lane_xor2(s);
      }
      if (pc < kPieces && pc % kPiecesPerSum == 0) xsum[wave][pc / kPiecesPerSum] = make_float2(c, s);
    }
    // 3. arithmetic: a slot past the last wave load is skipped (the condition is uniform)
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int l = l0 + wave + kWaves * i;
      if (l < nloads) {
        const int slot = i * Q + qi;
        const uint32_t *xw = reinterpret_cast<const uint32_t *>(&xs[wave][slot * KPC]);
        if constexpr (BITS == 2) {
          // two blocks; in each 32-bit word the four 2-bit field pairs of a byte are taken
          // in place (v_bfi_b32): pair e comes out as 1024 + 4^e q into its own
          // accumulator pe, which a power-of-two FP32 rescale puts back exactly
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float2 cs = xsum[wave][2 * slot + h];
            float pe[4] = {-cs.x, 0.f, 0.f, 0.f};
            if constexpr (HAS_ZP) pe[0] = fmaf(-(float)(((zraw[i] >> (8 * h)) >> ((row & 3) * 2)) & 3u), cs.y, -cs.x);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const u4_t xa = *reinterpret_cast<const u4_t *>(xw + 16 * h + 8 * j);
              const u4_t xb = *reinterpret_cast<const u4_t *>(xw + 16 * h + 8 * j + 4);
              const uint32_t w = cw[i][2 * h + j], w8 = w >> 8;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t mask = 0x00030003u << (2 * e);
                pe[e] = __builtin_amdgcn_fdot2(as_h2(bfi(mask, w, 0x64006400u)), as_h2(xa[e]), pe[e], false);
                pe[e] = __builtin_amdgcn_fdot2(as_h2(bfi(mask, w8, 0x64006400u)), as_h2(xb[e]), pe[e], false);
              }
            }
            const float blk = fmaf(pe[3], 0.015625f, fmaf(pe[2], 0.0625f, fmaf(pe[1], 0.25f, pe[0])));
            acc = fmaf(blk, h2f((uint16_t)(sraw[i] >> (16 * h))), acc);
          }
          continue;
        }
        const float2 cs = xsum[wave][slot];
        float p0 = -cs.x, p1 = 0.f;
        if constexpr (HAS_ZP) {
          const uint32_t z = BITS == 4 ? (zraw[i] >> ((row & 1) * 4)) & 0xFu : zraw[i];
          p0 = fmaf(-(float)z, cs.y, -cs.x);
        }
        if constexpr (BITS == 4) {
          // fields 1 and 3 of each half are taken in place as 1024 + 16 q (nib_hi16): p1
          // holds 16x its terms, which the power-of-two rescale below undoes exactly
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u4_t x4 = *reinterpret_cast<const u4_t *>(xw + 4 * j);
            const uint32_t w = cw[i][j], w8 = w >> 8;
            p0 = __builtin_amdgcn_fdot2(nib_lo(w), as_h2(x4[0]), p0, false);
            p1 = __builtin_amdgcn_fdot2(nib_hi16(w), as_h2(x4[1]), p1, false);
            p0 = __builtin_amdgcn_fdot2(nib_lo(w8), as_h2(x4[2]), p0, false);
            p1 = __builtin_amdgcn_fdot2(nib_hi16(w8), as_h2(x4[3]), p1, false);
          }
          acc = fmaf(fmaf(p1, 0.0625f, p0), h2f((uint16_t)sraw[i]), acc);
        } else {
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            const u4_t x4 = *reinterpret_cast<const u4_t *>(xw + 2 * j);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const uint32_t w = cw[i][j + jj];
              p0 = __builtin_amdgcn_fdot2(byte_pair_lo(w), as_h2(x4[2 * jj]), p0, false);
              p1 = __builtin_amdgcn_fdot2(byte_pair_hi(w), as_h2(x4[2 * jj + 1]), p1, false);
            }
          }
          acc = fmaf(p0 + p1, h2f((uint16_t)sraw[i]), acc);
        }
      }
    }
  }

  // lanes sharing a row, then waves, in fixed order
  if constexpr (Q >= 8) acc += lane_xor_swz<8>(acc);
  if constexpr (Q >= 4) acc += lane_xor_swz<16>(acc);
  if constexpr (Q >= 2) acc += lane_xor32(acc, lane);
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) total += red[w][rl];

  float lora = 0.f;
  if constexpr (LORA != LORA_NONE) {
    if constexpr (!kTWave) {
      // T from the T-projection launch: FP32 partials per K-part, added in part order
      const float tv = sum_parts<8>(p.tin + (size_t)m * kRank + (lane & 31), (size_t)p.tmpad * kRank, p.tparts);
      if (lane < kRank) tfin[lane] = tv;     // read back below by this wave only: LDS order suffices
    }
    lora = lora_dot<LORA>(tfin, bpk, bscale);
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
  else if (lpw <= 6)
    hipLaunchKernelGGL((gemv_kernel<BITS, HAS_ZP, LORA, TMODE, Q, 6>), dim3(gx, gy), dim3(nt), 0, s, p);
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
  return lpw <= 2 ? 2 : (lpw <= 4 ? 4 : (lpw <= 6 ? 6 : 8));
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
