// gemm.hip -- prefill path of MatMulNBits (M > 1): FP16 MFMA GEMM whose 2-, 4- or 8-bit
// weight operand is dequantized straight into MFMA operand registers, with the rank-32
// LoRA up-projection T.B run as two extra MFMA k-steps on the same accumulators before the
// fp16 store.
//
// onnxruntime PR #33370 ("[WebGPU] Fuse rank-32 quantized LoRA with MatMulNBits"), commit
// list: prefill (fuse_up) computes T first, then the base GEMM "with an integrated
// T * Bt^T epilogue"; a later commit names it the "fused LoRA-up output stage".
//
// Tile: 128 x 128 outputs per workgroup of 4 waves, K step 64 (two quantization blocks).
// Wave w owns the column half nh = w & 1 (64 columns = one packed 64-row group) and the
// block kh = w >> 1 of every K-step, and runs the MFMAs of its 128 x 64 piece over that
// block's 32 k (4 x 2 v_mfma_f32_32x32x16_f16 blocks, two k16 steps).  So every weight is
// dequantized exactly once, by the wave that multiplies it, directly into the B-operand
// registers -- no fp16 weight tile goes through LDS -- and each X operand read from LDS
// feeds two MFMAs.  After the K loop the two waves of a column half (K halves of the same
// 64 columns) each finish half of the row blocks: each hands the other half of its partials
// to its partner through LDS, adds the LoRA term and then the partner's partial on its own
// rows (fixed order: the result does not depend on timing), and stores that quarter.
//
// Memory pipeline.  Each K-step's inputs travel by direct-to-LDS loads
// (buffer_load_dwordx4 / _dword ... lds) into a 4-slot ring, three steps ahead of the MFMAs,
// so the load latency (L2 / Infinity Cache / HBM) hides behind three steps of matrix work
// without holding any of it in registers.  With 128-row tiles the ring is filled by four
// load waves (one per SIMD, beside the compute wave whose loads it issues), so the compute
// waves' instruction streams hold no global loads: a wave that issues its own loads issues
// no MFMAs while it waits to get them accepted, and one wave per SIMD moves only about half
// the bytes per clock that the CU's load path carries with two.  64-row tiles (two
// workgroups per CU) issue their own loads.
//   * the X tile (128 rows x 64 halfs), shared by all waves: each 16-byte chunk is
//     fetched into slot position chunk ^ ((row >> 1) & 7) (an XOR swizzle chosen through
//     the source address, since a DMA writes lanes consecutively), so MFMA operand reads
//     of 16 consecutive rows (256 bytes, one pass over the 64 LDS banks) hit distinct
//     banks without padding;
//   * the codes, scales and zero points of the wave's own 64 rows and block; without load
//     waves the wave later reads only bytes its own lanes fetched, so it waits only on its
//     own load counter (with them, the step barrier publishes these as well).  Every lane issues every direct load (lanes past the useful ones fetch
//     copies): loads narrower than 4 bytes, or under a lane mask, are not used.
// One step ahead of its MFMAs each wave dequantizes (q - z) * s (exact subtraction, one
// rounding) from the ring into registers.  Waits are explicit (s_waitcnt vmcnt for the
// loads, then one barrier per step for the shared X tile); the compiler is kept from moving
// memory accesses across the barrier.  Steps past the end issue loads from
// clamped addresses into free slots, so every step has the same loads in flight; loop
// iterations that load only steps before the last one skip the clamps.
// Without an adapter the two epilogue k-steps are skipped, so the base accumulation order
// is the same in every variant and a zero adapter reproduces the base output bitwise.
// Each wave's finished quarter is staged in LDS and stored as whole row pieces (16 bytes
// per lane, 128 contiguous bytes per row), not as the accumulator layout's 8 bytes in each
// of 32 rows.
#include <type_traits>
#include "common.h"

namespace mnb {
namespace {

constexpr int BN = 128, BK = 64;   // tile columns and K-step; the tile rows BMT are 128 or 64
constexpr int kThreads = 256;
constexpr int LDT = kRank + 8; // halfs per LDS row of the epilogue operands
// ring depth: loads run kSlots - 1 steps ahead (measured: 6 slots at 128 rows, 5 steps
// ahead, gave the same times)
constexpr int kSlots = 4;

template <int BMT, int C>
struct Slot {
  static constexpr int kX = 0;
  static constexpr int kCodesWave = C * 1024;         // 64 rows x 16 B x C chunks
  static constexpr int kCodes = BMT * BK * 2;         // after the X tile of one step
  static constexpr int kScale = kCodes + 4 * kCodesWave;   // per wave 256 B: 64 scales, twice
  static constexpr int kZp = kScale + 4 * 256;             // per wave 256 B: 32 or 64 B, repeated
  static constexpr int kBytes = kZp + 4 * 256;
};
template <int BMT, int C>
struct Lds {
  static constexpr int kBytes = kSlots * Slot<BMT, C>::kBytes;
  static constexpr int kRed = 2 * BMT * 64 * 4;                  // the kh = 1 partials
  static constexpr int kEpiOff = kRed;                           // epilogue operands after them
  static_assert(kSlots % 2 == 0, "the main loop alternates two B operand sets");
  static_assert(kBytes <= (BMT == 128 ? 160 : 80) * 1024, "LDS budget (two workgroups per CU at 64 rows)");
  static_assert(kEpiOff + (BMT + BN) * LDT * 2 <= kBytes, "epilogue buffers fit the ring");
};

typedef __attribute__((address_space(3))) void lds_void;
// Direct-to-LDS load of 16 or 4 bytes per lane (lane i lands at dst + i * size) through a
// buffer descriptor: address = descriptor base + soff (SGPR, per step) + voff (VGPR,
// loop-invariant), so a step costs no vector address arithmetic.  A plain device function,
// so kernel templates instantiate for the host pass as well.  The
// descriptors here span 2^31 - 1 bytes: every address is valid by construction, no range
// check is relied on.
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t *dst, int size) {
  lds_void *d = (lds_void *)(dst);
  if (size == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, voff, soff, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wide_rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}

// s_waitcnt with vmcnt = N (gfx9 encoding: vmcnt bits 3:0 and 15:14), other counters free
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// all of this wave's LDS accesses done, then the workgroup barrier; the asm memory clobber
// keeps the compiler from moving memory accesses across it
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

template <int BITS, bool HAS_ZP, int LORA, int BMT>
__global__ __launch_bounds__(BMT == 128 ? 2 * kThreads : kThreads, BMT == 64 ? 2 : 1) void gemm_kernel(GemmParams p) {
  // 128-row tiles: waves 4-7 are load waves.  Load wave 4 + w issues, for compute wave w,
  // the ring loads that wave w would issue (the same addresses: every per-wave quantity
  // below is computed from w), plus the LoRA operands, and arrives at every barrier the
  // compute waves do; the compute waves issue no global loads in the K loop.
  constexpr bool LW = BMT == 128;
  constexpr int C = BITS == 8 ? 2 : 1;       // 16-byte code chunks per wave and step
  constexpr int MB = BMT / 32;               // 32-row MFMA blocks per wave
  constexpr int XQ = BMT / 32;               // X loads per wave and step (1 KiB each)
  using SL = Slot<BMT, C>;
  constexpr int kLdsBytes = Lds<BMT, C>::kBytes;
  constexpr int kEpiOff = Lds<BMT, C>::kEpiOff;
  // direct loads per wave per step: 4 X, C codes, 1 scale, 1 zero point
  constexpr int kLoadsPerStep = XQ + C + 1 + (HAS_ZP ? 1 : 0);
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];

  const int tid = threadIdx.x & (kThreads - 1);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = LW && __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8) != 0;
  const int nh = wave & 1;                   // column half: one packed 64-row group
  const int kh = wave >> 1;                  // block of the K-step
  const int l32 = lane & 31, hi = lane >> 5;

  // XCD-aware order: workgroup ids are dealt to the 8 XCDs by id modulo 8.  Without K
  // splitting, XCD x takes the 2-D block (x % 2, x / 2) of a 2 x 4 partition of the tile
  // grid, so its L2 fetches half of X and a quarter of the weights (against all of X with
  // column strips: 31% fewer L2 fills at 1024 x 4096 x 4096, same time).  Otherwise each
  // XCD takes a contiguous range of (K range, tile) items, M fastest, sharing weight
  // columns.  With a tail split, the head (tiles below tail0, whole K) is mapped that way
  // and the workgroups after it take (K range, tail tile) items, tiles fastest; tiles are
  // numbered M fastest, so the tail is the last column strips.
  const int ntiles = p.MT * p.NT;
  const bool tailw = p.tsplits > 1 && (int)blockIdx.x >= p.tail0;
  int ks, tile, mt, nt, nranges;
  if (tailw) {
    const int ntail = ntiles - p.tail0;
    const int u = blockIdx.x - p.tail0;
    ks = u / ntail;
    tile = p.tail0 + (u - ks * ntail);
    nranges = p.tsplits;
    mt = tile % p.MT;
    nt = tile / p.MT;
  } else {
    const int nhead = p.tsplits > 1 ? p.tail0 : ntiles;
    const int nwg = nhead * p.splits;
    int item = blockIdx.x;
    if ((nwg & 7) == 0) item = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    ks = item / nhead;
    tile = item - ks * nhead;
    nranges = p.splits;
    mt = tile % p.MT;
    nt = tile / p.MT;
    const int nth = nhead / p.MT;             // head column strips (when the head is whole strips)
    if (p.splits == 1 && nhead % p.MT == 0 && (p.MT & 1) == 0 && (nth & 3) == 0) {
      const int x = blockIdx.x & 7, u = blockIdx.x >> 3;
      const int bm = p.MT >> 1, bn = nth >> 2;
      mt = (x & 1) * bm + u % bm;
      nt = (x >> 1) * bn + u / bm;
    }
  }
  const int m0 = mt * BMT, n0 = nt * BN;
  // K-steps [sbase, sbase + nsteps) of the (KB + 1) / 2; the host picks `splits` and
  // `tsplits` so that every range is non-empty
  const int tsteps = (p.KB + 1) / 2;
  const int sps = (tsteps + nranges - 1) / nranges;
  const int sbase = ks * sps;
  const int nsteps = min(tsteps, sbase + sps) - sbase;
  // the LoRA term is added once, by the first K range
  const bool lora_here = LORA != 0 && ks == 0;

  const int wg = (n0 >> 6) + nh;             // packed row group of this wave
  const bool wrow_ok = wg < p.NG;

  // ---- direct-to-LDS loads of one step into one ring slot: X rows (two halves), then the
  // wave's codes, scales and zero points ----
  // Addresses are a wave-uniform base plus a loop-invariant 32-bit lane offset, so the
  // direct loads use the scalar-base form and a step costs no vector address arithmetic.
  // X chunk load q of this wave covers tile rows r0 = (BMT/4) wave + 8 q .. r0 + 7 (8 lanes
  // per row): uniform base row min(m0 + r0, M - 1); lane offset = (its row, clamped to
  // M - 1, minus the base row) * 2K bytes + 16 c, with chunk c = position ^ ((r >> 1) & 7)
  // of the swizzle (at most 7 * 2K + 112 bytes; K < 2^25 is checked by the host)
  const uint8_t *X = reinterpret_cast<const uint8_t *>(p.X);
  const uint8_t *xrow[XQ];
  uint32_t xoff[XQ], xoffr[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int r0 = (BMT / 4) * wave + 8 * q;
    const int rb = min(m0 + r0, p.M - 1);
    const int r = r0 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    xrow[q] = X + (size_t)rb * p.K * 2;
    xoff[q] = (uint32_t)(min(m0 + r, p.M - 1) - rb) * (uint32_t)p.K * 2u + (uint32_t)c * 16u;
    // with an odd block count the last step's second block lies past K: its chunks
    // (c >= 4) re-read the first block (any valid address; the block's scales are 0)
    xoffr[q] = xoff[q] - (c >= 4 ? 64u : 0u);
  }
  __amdgpu_buffer_rsrc_t xr[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) xr[q] = wide_rsrc(xrow[q]);
  auto issue_x = [&](int step, int slot, int half) {
    const int sv = sbase + (step < nsteps ? step : nsteps - 1);   // past the end: a valid address
    const bool ragged = 2 * sv + 1 >= p.KB;
    uint8_t *base = smem + slot * SL::kBytes;
    const uint32_t so = (uint32_t)sv * BK * 2;
    if (ragged) {
#pragma unroll
      for (int q = half * (XQ / 2); q < (half + 1) * (XQ / 2); ++q)
        dma_buf(xr[q], xoffr[q], so, base + SL::kX + ((BMT / 4) * wave + 8 * q) * 128, 16);
    } else {
#pragma unroll
      for (int q = half * (XQ / 2); q < (half + 1) * (XQ / 2); ++q)
        dma_buf(xr[q], xoff[q], so, base + SL::kX + ((BMT / 4) * wave + 8 * q) * 128, 16);
    }
  };
  // per-lane byte offsets of the weight loads; descriptors based at this wave's packed row
  // group (row group 0 when the group lies past N: any valid address, never used)
  const uint32_t lo16 = (uint32_t)lane * 16u, lo_sc = (uint32_t)l32 * 4u;
  const uint32_t lo_zp = 4u * (uint32_t)(BITS == 2 ? (lane & 3) : BITS == 4 ? (lane & 7) : (lane & 15));
  constexpr int kZpB = BITS == 2 ? 16 : BITS == 4 ? 32 : kGroup;   // zero-point bytes per block
  const size_t wgb = wrow_ok ? (size_t)wg : 0;
  const auto wr = wide_rsrc(p.wq + wgb * (BITS == 2 ? (size_t)tsteps : (size_t)p.KB * C) * kGroup * 16);
  const auto sr = wide_rsrc(reinterpret_cast<const uint8_t *>(p.sc) + wgb * p.KB * kGroup * 2);
  const auto zr = wide_rsrc(HAS_ZP ? p.zp + wgb * p.KB * kZpB : p.wq);
  auto issue_w = [&](int step, int slot) {
    const int sv = sbase + (step < nsteps ? step : nsteps - 1);
    uint8_t *base = smem + slot * SL::kBytes;
    const int kb = 2 * sv + kh;
    const bool ok = wrow_ok && kb < p.KB;
    const uint32_t kbo = ok ? (uint32_t)kb : 0u;
    if constexpr (BITS == 2) {
      // one chunk holds both blocks of the step (each wave uses its half)
      dma_buf(wr, lo16, wrow_ok ? (uint32_t)sv * kGroup * 16 : 0u, base + SL::kCodes + wave * SL::kCodesWave, 16);
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c)
        dma_buf(wr, lo16, (kbo * C + c) * kGroup * 16, base + SL::kCodes + wave * SL::kCodesWave + c * 1024, 16);
    }
    dma_buf(sr, lo_sc, kbo * kGroup * 2, base + SL::kScale + wave * 256, 4);
    if constexpr (HAS_ZP) dma_buf(zr, lo_zp, kbo * kZpB, base + SL::kZp + wave * 256, 4);
  };
  auto issue = [&](int step, int slot) {
    issue_x(step, slot, 0);
    issue_x(step, slot, 1);
    issue_w(step, slot);
  };
  // The same loads for a step before the last one of the range (so neither past the end
  // nor ragged, and its blocks lie before KB): no clamps or selects, offsets linear in the
  // step.
  const uint32_t kb_base = wrow_ok ? (uint32_t)(2 * sbase + kh) : 0u, kb_inc = wrow_ok ? 2u : 0u;
  auto issue_x_mid = [&](int step, int slot, int half) {
    uint8_t *base = smem + slot * SL::kBytes;
    const uint32_t so = (uint32_t)(sbase + step) * BK * 2;
#pragma unroll
    for (int q = half * (XQ / 2); q < (half + 1) * (XQ / 2); ++q)
      dma_buf(xr[q], xoff[q], so, base + SL::kX + ((BMT / 4) * wave + 8 * q) * 128, 16);
  };
  auto issue_w_mid = [&](int step, int slot) {
    uint8_t *base = smem + slot * SL::kBytes;
    const uint32_t kbo = kb_base + (uint32_t)step * kb_inc;
    if constexpr (BITS == 2) {
      dma_buf(wr, lo16, (kbo >> 1) * kGroup * 16, base + SL::kCodes + wave * SL::kCodesWave, 16);
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c)
        dma_buf(wr, lo16, (kbo * C + c) * kGroup * 16, base + SL::kCodes + wave * SL::kCodesWave + c * 1024, 16);
    }
    dma_buf(sr, lo_sc, kbo * kGroup * 2, base + SL::kScale + wave * 256, 4);
    if constexpr (HAS_ZP) dma_buf(zr, lo_zp, kbo * kZpB, base + SL::kZp + wave * 256, 4);
  };

  // ---- dequantize this wave's block of one step into B operands [nb][kk] ----
  // The k index of an MFMA is a summation index, so any assignment of the block's k to
  // (k16 step kk, lane half hi) works if X uses the same one.  Here (kk, hi) takes the 8 k
  // of 8-k chunk 2 * hi + kk: for 4-bit codes that is word 2 * hi + kk of the row's
  // 16-byte chunk (pair i of a word = k 2i, 2i+1 of its 8), for 8-bit codes bytes
  // 8 * kk .. 8 * kk + 7 of the row's 16-byte chunk hi, so a lane reads one contiguous
  // piece and needs no selects.  B operand: lane holds 8 consecutive k of column l32;
  // column = weight row 32 * nb + l32.
  struct Raw {
    u4_t cw[2];          // 4-bit: words (2hi, 2hi+1) in [0], [1]; 8-bit: chunk hi; 2-bit: word hi in [0]
    uint32_t sraw[2], zb[2];
  };
  auto dq_read = [&](int slot, Raw &rw) {
    const uint8_t *base = smem + slot * SL::kBytes;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int r = 32 * nb + l32;
      if constexpr (BITS == 2) {
        // word hi of this wave's block kh: k 16 hi .. 16 hi + 15 of the block
        rw.cw[nb][0] = *reinterpret_cast<const uint32_t *>(base + SL::kCodes + wave * SL::kCodesWave + r * 16 + 8 * kh +
                                                            4 * hi);
      } else if constexpr (BITS == 4) {
        const u2_t w2 = *reinterpret_cast<const u2_t *>(base + SL::kCodes + wave * SL::kCodesWave + r * 16 + hi * 8);
        rw.cw[nb][0] = w2[0];
        rw.cw[nb][1] = w2[1];
      } else {
        rw.cw[nb] = *reinterpret_cast<const u4_t *>(base + SL::kCodes + wave * SL::kCodesWave + hi * 1024 + r * 16);
      }
      rw.sraw[nb] = *reinterpret_cast<const uint16_t *>(base + SL::kScale + wave * 256 + r * 2);
      rw.zb[nb] = 0;
      if constexpr (HAS_ZP)
        rw.zb[nb] = BITS == 2   ? base[SL::kZp + wave * 256 + (r >> 2)]
                    : BITS == 4 ? base[SL::kZp + wave * 256 + (r >> 1)]
                                : base[SL::kZp + wave * 256 + r];
    }
  };
  auto dq_compute = [&](int step, const Raw &rw, int nb, u4_t (&bo)[2][2]) {
    const bool wok = wrow_ok && 2 * (sbase + step) + kh < p.KB;
    const int r = 32 * nb + l32;
    uint32_t z = 1u << (BITS - 1);
    if constexpr (HAS_ZP)
      z = BITS == 2 ? (rw.zb[nb] >> ((r & 3) * 2)) & 3u : BITS == 4 ? (rw.zb[nb] >> ((r & 1) * 4)) & 0xFu : rw.zb[nb];
    // binary16 of 1024 + z is 0x6400 | z (z < 1024): both halves at once, one v_perm_b32
    // (bytes z, 0x64, z, 0x64; 8-bit z up to 255 sits in the low byte alone)
    const h2_t zz2 = as_h2(__builtin_amdgcn_perm(0x64646464u, z, 0x04000400u));
    // the scale in both halves (bytes 0, 1, 0, 1 of the raw word), 0 past K
    const h2_t s2 = as_h2(__builtin_amdgcn_perm(0u, wok ? rw.sraw[nb] : 0u, 0x01000100u));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if constexpr (BITS == 2) {
        // byte kk of each half of the word: fields (2e, 2e+1) -> the pair k = 8 kk + 2e,
        // + 1 of this wave's 16; (q - z) exact, times s rounded once
        const uint32_t v = rw.cw[nb][0] >> (8 * kk);
#pragma unroll
        for (int e = 0; e < 4; ++e) bo[nb][kk][e] = as_u32((crumb_pair(v, e) - zz2) * s2);
      } else if constexpr (BITS == 4) {
        // Nibbles 0 and 2 of each half sit in mantissa bits 0-3 (after a shift by 8 for
        // 2): OR-ing 0x6400 gives 1024 + q, and minus (1024 + z) that is q - z, exact.
        // Nibbles 1 and 3 are taken in place, at bits 4-7: 1024 + 16 q.  One fused
        // multiply-add takes it to (1024 + 16 q) / 16 - (64 + z) = q - z: every term is
        // exact and so is the small integer result.  Both kinds are then multiplied by the
        // same s, so each weight is (q - z) s rounded once, for every finite scale
        // (subnormal ones included).
        const h2_t nz64 = h2_t{(_Float16)960.f, (_Float16)960.f} - zz2;   // 960 - (1024 + z) = -(64 + z), exact
        const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
        const uint32_t w = rw.cw[nb][kk];
        const uint32_t w8 = w >> 8;
        bo[nb][kk][0] = as_u32((as_h2(bfi(0x000F000Fu, w, 0x64006400u)) - zz2) * s2);
        bo[nb][kk][1] = as_u32(__builtin_elementwise_fma(as_h2(bfi(0x00F000F0u, w, 0x64006400u)), sixteenth, nz64) * s2);
        bo[nb][kk][2] = as_u32((as_h2(bfi(0x000F000Fu, w8, 0x64006400u)) - zz2) * s2);
        bo[nb][kk][3] = as_u32(__builtin_elementwise_fma(as_h2(bfi(0x00F000F0u, w8, 0x64006400u)), sixteenth, nz64) * s2);
      } else {
        const uint32_t w0 = rw.cw[nb][2 * kk], w1 = rw.cw[nb][2 * kk + 1];
        bo[nb][kk][0] = as_u32((byte_pair_lo(w0) - zz2) * s2);
        bo[nb][kk][1] = as_u32((byte_pair_hi(w0) - zz2) * s2);
        bo[nb][kk][2] = as_u32((byte_pair_lo(w1) - zz2) * s2);
        bo[nb][kk][3] = as_u32((byte_pair_hi(w1) - zz2) * s2);
      }
    }
  };

  // LoRA epilogue operands, fetched first (ordinary loads that complete ahead of the ring
  // loads): T rows (FP32 K-part partials, added in part order) and this thread's B slice.
  // Two threads per tile row: for 64-row tiles only waves 0 and 1 load T, and only the
  // parts that exist (the others' loads would be wasted L2 traffic in every tile).
  float tsum[16];
  u4_t braw[2];
  uint32_t bsc[8];
  bool bvec = false;
  const int trow = tid >> 1, thh = (tid & 1) * 16;
  const bool t_loader = trow < BMT;            // wave-uniform
  const int br = tid >> 3, bnc = (tid & 7) * 16;
  constexpr int kTPartsAhead = 8;            // T parts loaded before the ring starts
  // (with load waves these are theirs: B here, the T parts one per step of their loop)
  float4 tv[LW ? 1 : kTPartsAhead][4];
  float4 tw[2][4];                           // load waves: T parts in flight, two steps deep
  if (lora_here && (!LW || loader)) {
    const size_t mrow = (size_t)min(m0 + trow, p.M - 1);
    if constexpr (!LW) {
      if (t_loader) {
#pragma unroll
        for (int pp = 0; pp < kTPartsAhead; ++pp) {
          if (pp < p.tparts) {
            const float *src = p.tpart + ((size_t)pp * p.M + mrow) * kRank + thh;
#pragma unroll
            for (int q = 0; q < 4; ++q) tv[pp][q] = *reinterpret_cast<const float4 *>(src + 4 * q);
          }
        }
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

  _Float16 *sT = reinterpret_cast<_Float16 *>(smem + kEpiOff);
  _Float16 *sB = sT + BMT * LDT;
  auto write_lora_operands = [&]() {
    // epilogue operands: T tile [BMT m][32 r] (fp16, rounded once from the FP32 sum) and
    // the B tile transposed to [128 n][32 r]
    u4_t o[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const h2_t hv = {(_Float16)tsum[8 * q + 2 * d], (_Float16)tsum[8 * q + 2 * d + 1]};
        o[q][d] = as_u32(hv);
      }
    if (trow < BMT) {
      *reinterpret_cast<u4_t *>(&sT[trow * LDT + thh]) = o[0];
      *reinterpret_cast<u4_t *>(&sT[trow * LDT + thh + 8]) = o[1];
    }
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
    };
  if constexpr (LW) {
    if (loader) {
      // the ring's first kSlots - 1 steps; steps 0 and 1 landed before the first barrier
      if (lora_here) {
#pragma unroll
        for (int e = 0; e < 16; ++e) tsum[e] = 0.f;
      }
#pragma unroll
      for (int st = 0; st < kSlots - 1; ++st) issue(st, st);
      wait_vmcnt<(kSlots - 3) * kLoadsPerStep>();
      lds_barrier();
      // load waves: step s + kSlots - 1 into the slot freed by the previous barrier, then
      // wait until step s + 2 has landed (the compute waves read its weights right after
      // this step's barrier, its X one step later).  The T parts of the LoRA term come one
      // per step, in part order, each added two steps after it is issued (by then the wait
      // for a later ring step has covered it).
      auto lstep = [&](int s, auto buf_c) {
        constexpr int b = decltype(buf_c)::value;
        const bool tl = lora_here && t_loader;
        if (tl && s >= 2 && s - 2 < p.tparts) {
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            tsum[4 * q + 0] += tw[b][q].x;
            tsum[4 * q + 1] += tw[b][q].y;
            tsum[4 * q + 2] += tw[b][q].z;
            tsum[4 * q + 3] += tw[b][q].w;
          }
        }
        const bool tnew = lora_here && s < p.tparts;   // uniform: the wait below counts its loads
        if (tnew) {
          const float *src = p.tpart + ((size_t)s * p.M + (size_t)min(m0 + trow, p.M - 1)) * kRank + thh;
  #pragma unroll
          for (int q = 0; q < 4; ++q) tw[b][q] = *reinterpret_cast<const float4 *>(src + 4 * q);
        }
        issue(s + kSlots - 1, (s + kSlots - 1) % kSlots);
        if (tnew) wait_vmcnt<(kSlots - 3) * kLoadsPerStep + 4>();
        else wait_vmcnt<(kSlots - 3) * kLoadsPerStep>();
        lds_barrier();
      };
      constexpr std::integral_constant<int, 0> kB0{};
      constexpr std::integral_constant<int, 1> kB1{};
      int s = 0;
      for (; s + 1 < nsteps; s += 2) {
        lstep(s, kB0);
        lstep(s + 1, kB1);
      }
      if (s < nsteps) lstep(s, kB0);
      wait_vmcnt<0>();
      if (lora_here && t_loader) {
        // the parts issued in the last two steps, then any beyond the K range's steps
  #pragma unroll
        for (int d = 2; d >= 1; --d) {
          const int pp = nsteps - d;
          if (pp >= 0 && pp < p.tparts) {
            const int b = pp & 1;
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 v = b ? tw[1][q] : tw[0][q];
              tsum[4 * q + 0] += v.x;
              tsum[4 * q + 1] += v.y;
              tsum[4 * q + 2] += v.z;
              tsum[4 * q + 3] += v.w;
            }
          }
        }
        for (int pp = nsteps; pp < p.tparts; ++pp) {
          const float *src = p.tpart + ((size_t)pp * p.M + (size_t)min(m0 + trow, p.M - 1)) * kRank + thh;
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4 *>(src + 4 * q);
            tsum[4 * q + 0] += v.x;
            tsum[4 * q + 1] += v.y;
            tsum[4 * q + 2] += v.z;
            tsum[4 * q + 3] += v.w;
          }
        }
      }

      wait_vmcnt<0>();
      lds_barrier();                        // the compute waves' last step
      if (lora_here) write_lora_operands();
      __syncthreads();                      // the compute waves' epilogue barrier
      return;
    }
  }

  f16x_t acc[MB][2];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  // ---- X operands of this wave's block of one K-step: the first k16 half right after
  // the barrier that publishes the step, the second from the same slot once the step's
  // first MFMAs are issued (the slot is reused only after the step's own barrier), so
  // only half of the reads stand between the barrier and the first MFMA ----
  auto read_a_kk = [&](int slot, h8_t (&af)[2][MB], int kk) {
    const uint8_t *xs = smem + slot * SL::kBytes + SL::kX;
    const int c = 4 * kh + 2 * hi + kk;        // 8-k chunk of the step (see the B operand)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = mb * 32 + l32;
      af[kk][mb] = *reinterpret_cast<const h8_t *>(xs + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
    }
  };
  auto read_a = [&](int slot, h8_t (&af)[2][MB]) {
    read_a_kk(slot, af, 0);
    read_a_kk(slot, af, 1);
  };
  // ---- a quarter of this wave's block of one K-step: k16 step kk, row blocks 2h, 2h+1 ----
  auto mfma_q = [&](const h8_t (&af)[2][MB], const u4_t (&bo)[2][2], int kk, int h) {
#pragma unroll
    for (int mb = h * (MB / 2); mb < (h + 1) * (MB / 2); ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8_t, bo[nb][kk]), af[kk][mb],
                                                             acc[mb][nb], 0, 0, 0);
  };

  // ---- prologue: steps 0 .. kSlots - 2 in flight, step 0 dequantized ----
  u4_t bcur[2][2], bnext[2][2];
  h8_t acur[2][MB];
  if constexpr (LW) {
    {
      lds_barrier();                        // steps 0 and 1 (X and weights) are in LDS
      Raw rw;
      dq_read(0, rw);
      dq_compute(0, rw, 0, bcur);
      dq_compute(0, rw, 1, bcur);
      read_a(0, acur);
    }
  } else {
  #pragma unroll
    for (int st = 0; st < kSlots - 1; ++st) issue(st, st);
    if (lora_here) {
  #pragma unroll
      for (int e = 0; e < 16; ++e) tsum[e] = 0.f;
  #pragma unroll
      for (int pp = 0; pp < kTPartsAhead; ++pp) {
        if (t_loader && pp < p.tparts) {
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            tsum[4 * q + 0] += tv[pp][q].x;
            tsum[4 * q + 1] += tv[pp][q].y;
            tsum[4 * q + 2] += tv[pp][q].z;
            tsum[4 * q + 3] += tv[pp][q].w;
          }
        }
      }
      for (int pp = kTPartsAhead; t_loader && pp < p.tparts; ++pp) {
        const float *src = p.tpart + ((size_t)pp * p.M + (size_t)min(m0 + trow, p.M - 1)) * kRank + thh;
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = *reinterpret_cast<const float4 *>(src + 4 * q);
          tsum[4 * q + 0] += v.x;
          tsum[4 * q + 1] += v.y;
          tsum[4 * q + 2] += v.z;
          tsum[4 * q + 3] += v.w;
        }
      }
    }
    wait_vmcnt<(kSlots - 2) * kLoadsPerStep>();   // own loads of step 0 have landed
    {
      Raw rw;
      dq_read(0, rw);
      dq_compute(0, rw, 0, bcur);
      dq_compute(0, rw, 1, bcur);
    }
    lds_barrier();                          // step 0's X tile (all waves) is in LDS
    read_a(0, acur);

  }

  // ---- main loop: step s computes; step s+1 is dequantized; step s+3 is loaded ----
  // Source order is issue order (scheduling barriers keep the compiler from regrouping):
  // the step's 16 MFMAs come in quarters with the next step's dequantization arithmetic
  // between them, so the VALU work runs while the matrix core is busy.
  // slot: s mod kSlots, a compile-time constant at every call
  // mid: the step issued here (s + kSlots - 1) is before the range's last step
  auto body = [&](auto mid_c, int s, u4_t (&bc)[2][2], u4_t (&bn)[2][2], const int slot) {
    constexpr bool mid = decltype(mid_c)::value;
    const int ls = (slot + kSlots - 1) % kSlots;
    const int ns = (slot + 1) % kSlots;
    if constexpr (!LW) wait_vmcnt<(kSlots - 3) * kLoadsPerStep>();   // own loads of step s+1 have landed (later ones may not)
    Raw rw;
    dq_read(ns, rw);                      // past the end: unused, from a loaded slot
    __builtin_amdgcn_sched_barrier(0);
    mfma_q(acur, bc, 0, 0);
    read_a_kk(slot, acur, 1);             // this step's second k16 half, from its own slot
    if constexpr (LW) {
    } else if constexpr (mid) issue_x_mid(s + kSlots - 1, ls, 0);
    else issue_x(s + kSlots - 1, ls, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_q(acur, bc, 0, 1);
    dq_compute(s + 1, rw, 0, bn);
    __builtin_amdgcn_sched_barrier(0);
    mfma_q(acur, bc, 1, 0);
    if constexpr (LW) {
    } else if constexpr (mid) {
      issue_x_mid(s + kSlots - 1, ls, 1);
      issue_w_mid(s + kSlots - 1, ls);
    } else {
      issue_x(s + kSlots - 1, ls, 1);
      issue_w(s + kSlots - 1, ls);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfma_q(acur, bc, 1, 1);
    dq_compute(s + 1, rw, 1, bn);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();                        // step s+1's X ready for all; slot s free
    read_a_kk(ns, acur, 0);               // past the end: unused
  };
  // unrolled by the ring depth, so ring slots are compile-time constants
  // (first the iterations whose loads are all for steps before the last: s + 2 kSlots - 2
  // <= nsteps - 2)
  constexpr std::integral_constant<bool, true> kMid{};
  constexpr std::integral_constant<bool, false> kEdge{};
  int s = 0;
  for (; s + 2 * kSlots <= nsteps; s += kSlots) {
#pragma unroll
    for (int i = 0; i < kSlots; i += 2) {
      body(kMid, s + i, bcur, bnext, i);
      body(kMid, s + i + 1, bnext, bcur, i + 1);
    }
  }
  for (; s + kSlots - 1 < nsteps; s += kSlots) {
#pragma unroll
    for (int i = 0; i < kSlots; i += 2) {
      body(kEdge, s + i, bcur, bnext, i);
      body(kEdge, s + i + 1, bnext, bcur, i + 1);
    }
  }
#pragma unroll
  for (int i = 0; i < kSlots - 1; i += 2) {   // at most kSlots - 1 steps remain
    if (s + i < nsteps) body(kEdge, s + i, bcur, bnext, i);
    if (i + 1 < kSlots - 1 && s + i + 1 < nsteps) body(kEdge, s + i + 1, bnext, bcur, i + 1);
  }

  wait_vmcnt<0>();                        // the trailing loads into free slots are done
  lds_barrier();

  // ---- epilogue: the two waves of a column half (kh = 0, 1) hold K-half partials of the
  // same 64 columns over all tile rows.  Each keeps half of the row blocks (own: kh MBH ..
  // kh MBH + MBH - 1) and hands the other half to its partner (wave ^ 2) through LDS, so
  // both finish, convert and store a quarter of the tile. ----
  // Accumulator register v of block [mb][nb] holds tile row 32 mb + lane % 32 and tile
  // column 64 nh + 32 nb + 8 (v / 4) + 4 (lane / 32) + v % 4 (the MFMAs computed Y^T blocks,
  // weights as the row operand): four consecutive columns per register quad.
  constexpr int MBH = MB / 2;
  constexpr int kGive = MBH * 2 * 4;         // float4 per lane handed over (MBH blocks x 2 nb x 4)
  float4 *red = reinterpret_cast<float4 *>(smem);
  static_assert(4 * kGive * 64 * 16 <= Lds<BMT, C>::kRed, "handed-over partials fit their region");
  // (the block offsets are compile-time constants in both instances, so the accumulators
  // stay in registers)
  auto give = [&](auto give_c) {
    constexpr int give0 = decltype(give_c)::value;
#pragma unroll
    for (int b = 0; b < MBH; ++b)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          red[(wave * kGive + (b * 2 + nb) * 4 + v4) * 64 + lane] =
              float4{acc[give0 + b][nb][4 * v4], acc[give0 + b][nb][4 * v4 + 1], acc[give0 + b][nb][4 * v4 + 2],
                     acc[give0 + b][nb][4 * v4 + 3]};
  };
  if (!loader) {
    if (kh == 0) give(std::integral_constant<int, MBH>{});
    else give(std::integral_constant<int, 0>{});
  }
  if (!LW && lora_here) write_lora_operands();
  __syncthreads();

  // own row blocks: + the LoRA term (two MFMA k-steps of 16 over the rank), then + the
  // partner's partial; the sum is ((own K half + T B) + other K half) in FP32
  const int own0 = kh * MBH;
  float y[MBH][2][16];
  const float4 *mine = red + (size_t)(wave ^ 2) * kGive * 64;   // the partner's hand-over
  auto finish = [&](auto own_c) {
    constexpr int ob = decltype(own_c)::value;   // first own block
    if (lora_here) {
      const int akof = 8 * hi;
#pragma unroll
      for (int kk = 0; kk < kRank / 16; ++kk) {
        h8_t af[MBH], bf[2];
#pragma unroll
        for (int b = 0; b < MBH; ++b)
          af[b] = *reinterpret_cast<const h8_t *>(&sT[((ob + b) * 32 + l32) * LDT + kk * 16 + akof]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          bf[nb] = *reinterpret_cast<const h8_t *>(&sB[(nh * 64 + nb * 32 + l32) * LDT + kk * 16 + akof]);
#pragma unroll
        for (int b = 0; b < MBH; ++b)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[ob + b][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[nb], af[b], acc[ob + b][nb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int b = 0; b < MBH; ++b)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const float4 o = mine[((b * 2 + nb) * 4 + v4) * 64 + lane];
          y[b][nb][4 * v4] = acc[ob + b][nb][4 * v4] + o.x;
          y[b][nb][4 * v4 + 1] = acc[ob + b][nb][4 * v4 + 1] + o.y;
          y[b][nb][4 * v4 + 2] = acc[ob + b][nb][4 * v4 + 2] + o.z;
          y[b][nb][4 * v4 + 3] = acc[ob + b][nb][4 * v4 + 3] + o.w;
        }
  };
  if (kh == 0) finish(std::integral_constant<int, 0>{});
  else finish(std::integral_constant<int, MBH>{});

  // The partner's hand-over region is read by this wave alone, and its reads precede
  // these writes in LDS order: it stages this wave's quarter of the tile (MBH 32 rows x 64
  // columns), which the wave then stores as whole row pieces.  16-byte chunks are swizzled
  // by row so that the 32 rows of one write spread over the banks.
  uint8_t *stage = reinterpret_cast<uint8_t *>(smem) + (size_t)(wave ^ 2) * kGive * 64 * 16;
  const int mrow0 = m0 + own0 * 32;          // first tile row of this wave's quarter
  const int ncol0 = n0 + nh * 64;            // first column
  if (nranges > 1) {
    // this K range's FP32 partial (256-byte rows, 16 chunks); the reduction launch adds the
    // ranges in order, and the bias
#pragma unroll
    for (int b = 0; b < MBH; ++b)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = b * 32 + l32, ch = 8 * nb + 2 * j + hi;
          *reinterpret_cast<float4 *>(stage + r * 256 + ((ch ^ (r & 15)) << 4)) =
              float4{y[b][nb][4 * j], y[b][nb][4 * j + 1], y[b][nb][4 * j + 2], y[b][nb][4 * j + 3]};
        }
    const int c16 = lane & 15;
    float *dst0;
    size_t pitch;
    if (tailw) {
      // tail tile: the whole BMT x 128 partial, compact (rows and columns past M and N are
      // written too and never read)
      dst0 = p.ypart + ((size_t)ks * (ntiles - p.tail0) + (tile - p.tail0)) * (BMT * BN) + (size_t)own0 * 32 * BN +
             nh * 64;
      pitch = BN;
    } else {
      dst0 = p.ypart + (size_t)ks * p.M * p.N + (size_t)mrow0 * p.N + ncol0;
      pitch = p.N;
    }
    const bool vec = tailw || (p.N & 3) == 0;
#pragma unroll
    for (int pass = 0; pass < MBH * 8; ++pass) {
      const int r = pass * 4 + (lane >> 4);
      const float4 v = *reinterpret_cast<const float4 *>(stage + r * 256 + ((c16 ^ (r & 15)) << 4));
      if (!tailw && (mrow0 + r >= p.M || ncol0 + 4 * c16 >= p.N)) continue;
      float *dst = dst0 + (size_t)r * pitch + 4 * c16;
      if (vec && (tailw || ncol0 + 4 * c16 + 4 <= p.N)) {
        *reinterpret_cast<float4 *>(dst) = v;
      } else {
        const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (ncol0 + 4 * c16 + e < p.N) dst[e] = e4[e];
      }
    }
    return;
  }
  // whole K: + bias in FP32, one rounding to fp16 (128-byte rows, 8 chunks)
  if (p.bias) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = ncol0 + nb * 32 + 8 * j + 4 * hi + e;
          const float bv = n < p.N ? h2f(p.bias[n]) : 0.f;
#pragma unroll
          for (int b = 0; b < MBH; ++b) y[b][nb][4 * j + e] += bv;
        }
  }
#pragma unroll
  for (int b = 0; b < MBH; ++b)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = b * 32 + l32, ch = 4 * nb + j;
        const h2_t lo = {(_Float16)y[b][nb][4 * j], (_Float16)y[b][nb][4 * j + 1]};
        const h2_t hi2 = {(_Float16)y[b][nb][4 * j + 2], (_Float16)y[b][nb][4 * j + 3]};
        *reinterpret_cast<u2_t *>(stage + r * 128 + ((ch ^ (r & 7)) << 4) + 8 * hi) = u2_t{as_u32(lo), as_u32(hi2)};
      }
  const bool vec = (p.N & 7) == 0;
  const int c8 = lane & 7;
#pragma unroll
  for (int pass = 0; pass < MBH * 4; ++pass) {
    const int r = pass * 8 + (lane >> 3);
    const int m = mrow0 + r, n = ncol0 + 8 * c8;
    const u4_t v = *reinterpret_cast<const u4_t *>(stage + r * 128 + ((c8 ^ (r & 7)) << 4));
    if (m >= p.M || n >= p.N) continue;
    uint16_t *dst = p.Y + (size_t)m * p.N + n;
    if (vec && n + 8 <= p.N) {
      *reinterpret_cast<u4_t *>(dst) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < p.N) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// Y = fp16(sum over the K ranges of the FP32 partials, in range order, + bias): four
// consecutive outputs per thread when N % 4 == 0, else one
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *part, int splits, const uint16_t *bias,
                                                            uint16_t *Y, int M, int N) {
  const long MN = (long)M * N;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if ((N & 3) == 0) {
    const long e = 4 * i;
    if (e >= MN) return;
    float4 v[kMaxSplits];
#pragma unroll
    for (int k = 0; k < kMaxSplits; ++k)
      if (k < splits) v[k] = *reinterpret_cast<const float4 *>(part + k * MN + e);
    float4 y = v[0];
#pragma unroll
    for (int k = 1; k < kMaxSplits; ++k)
      if (k < splits) {
        y.x += v[k].x;
        y.y += v[k].y;
        y.z += v[k].z;
        y.w += v[k].w;
      }
    if (bias) {
      const int n = (int)(e % N);
      y.x += h2f(bias[n]);
      y.y += h2f(bias[n + 1]);
      y.z += h2f(bias[n + 2]);
      y.w += h2f(bias[n + 3]);
    }
    const h2_t lo = {(_Float16)y.x, (_Float16)y.y};
    const h2_t hi = {(_Float16)y.z, (_Float16)y.w};
    *reinterpret_cast<u2_t *>(Y + e) = u2_t{as_u32(lo), as_u32(hi)};
  } else {
    if (i >= MN) return;
    float y = part[i];
    for (int k = 1; k < splits; ++k) y += part[k * MN + i];
    if (bias) y += h2f(bias[i % N]);
    Y[i] = __builtin_bit_cast(uint16_t, (_Float16)y);
  }
}

// Tail tiles: Y = fp16(sum over the tsplits K ranges of the compact FP32 partials
// [tsplits, tail tiles, bm, 128], in range order, + bias).  One thread per four
// consecutive columns of a tile row.
__global__ __launch_bounds__(256) void tail_reduce_kernel(const float *part, int splits, const uint16_t *bias,
                                                          uint16_t *Y, int M, int N, int MT, int tail0, int ntail,
                                                          int bm) {
  const int per_tile = bm * (BN / 4);            // float4 per tile
  const long g = (long)blockIdx.x * 256 + threadIdx.x;
  if (g >= (long)ntail * per_tile) return;
  const int t = (int)(g / per_tile), w = (int)(g - (long)t * per_tile);
  const int r = w / (BN / 4), c4 = w - r * (BN / 4);
  const int tile = tail0 + t;
  const int m = (tile % MT) * bm + r, n = (tile / MT) * BN + 4 * c4;
  if (m >= M || n >= N) return;
  const size_t stride = (size_t)ntail * per_tile;   // float4 between consecutive ranges
  const float4 *src = reinterpret_cast<const float4 *>(part) + (size_t)t * per_tile + w;
  float4 v[kMaxSplits];
#pragma unroll
  for (int k = 0; k < kMaxSplits; ++k)
    if (k < splits) v[k] = src[(size_t)k * stride];
  float y[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
  for (int k = 1; k < kMaxSplits; ++k)
    if (k < splits) {
      y[0] += v[k].x;
      y[1] += v[k].y;
      y[2] += v[k].z;
      y[3] += v[k].w;
    }
  uint16_t *dst = Y + (size_t)m * N + n;
  if ((N & 3) == 0) {
    if (bias) {
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] += h2f(bias[n + e]);
    }
    const h2_t lo = {(_Float16)y[0], (_Float16)y[1]};
    const h2_t hi = {(_Float16)y[2], (_Float16)y[3]};
    *reinterpret_cast<u2_t *>(dst) = u2_t{as_u32(lo), as_u32(hi)};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < N) dst[e] = __builtin_bit_cast(uint16_t, (_Float16)(bias ? y[e] + h2f(bias[n + e]) : y[e]));
  }
}

template <int BITS, bool HAS_ZP>
hipError_t launch2(int lora, const GemmParams &p, hipStream_t s) {
  const int ntiles = p.MT * p.NT;
  const dim3 grid(p.tsplits > 1 ? p.tail0 + (ntiles - p.tail0) * p.tsplits : ntiles * p.splits);
  const dim3 block(p.bm == 64 ? kThreads : 2 * kThreads);   // 128-row tiles: 4 compute + 4 load waves
  if (p.bm == 64) {
    switch (lora) {
      case 0: hipLaunchKernelGGL((gemm_kernel<BITS, HAS_ZP, 0, 64>), grid, block, 0, s, p); break;
      case 1: hipLaunchKernelGGL((gemm_kernel<BITS, HAS_ZP, 1, 64>), grid, block, 0, s, p); break;
      default: hipLaunchKernelGGL((gemm_kernel<BITS, HAS_ZP, 2, 64>), grid, block, 0, s, p); break;
    }
    return hipGetLastError();
  }
  switch (lora) {
    case 0: hipLaunchKernelGGL((gemm_kernel<BITS, HAS_ZP, 0, 128>), grid, block, 0, s, p); break;
    case 1: hipLaunchKernelGGL((gemm_kernel<BITS, HAS_ZP, 1, 128>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((gemm_kernel<BITS, HAS_ZP, 2, 128>), grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

// Tile rows.  128-row tiles (one workgroup per CU, with load waves) dequantize each weight
// once per 128 rows; 64-row tiles dequantize it twice as often but run two workgroups per
// CU, whose loads, waits and matrix work interleave.  Measured: 128 wins when the tiles fill
// whole rounds of the 256 CUs (1024 x 4096: 56 against 60 us), and from M = 256 up when all
// of them fit one round, K split to fill it (x 4096 x 4096 with the adapter: M = 256 / 384 /
// 512 29.4 / 34.6 / 38.1 against 28.7 / 31.2 / 34.2 us; M = 32 / 64 / 128 lose: 16.6 / 17.6 /
// 25.1 against 17.4 / 20.1 / 25.3); 64 wins when the last round of 128-row tiles would be at
// most half full (1024 x 9728 at M = 512: 59 against 74 us).
int gemm_bm(int M, int N) {
  const long t128 = (((long)M + 127) / 128) * (((long)N + BN - 1) / BN);
  const long rem = t128 % kCUs;
  return (rem == 0 || rem > kCUs / 2 || (t128 <= kCUs && M >= 256)) ? 128 : 64;
}

hipError_t launch_gemm(int bits, bool has_zp, int lora, const GemmParams &p, hipStream_t s) {
  if (p.splits < 1 || p.splits > kMaxSplits || (p.bm != 64 && p.bm != 128)) return hipErrorInvalidValue;
  const int ntiles = p.MT * p.NT;
  if (p.tsplits < 1 || p.tsplits > kMaxSplits ||
      (p.tsplits > 1 && (p.splits != 1 || p.tail0 < 1 || p.tail0 >= ntiles)))
    return hipErrorInvalidValue;
  const hipError_t e = bits == 2   ? (has_zp ? launch2<2, true>(lora, p, s) : launch2<2, false>(lora, p, s))
                       : bits == 4 ? (has_zp ? launch2<4, true>(lora, p, s) : launch2<4, false>(lora, p, s))
                                   : (has_zp ? launch2<8, true>(lora, p, s) : launch2<8, false>(lora, p, s));
  if (e != hipSuccess) return e;
  if (p.tsplits > 1) {
    const int ntail = ntiles - p.tail0;
    const long work = (long)ntail * p.bm * (BN / 4);
    hipLaunchKernelGGL(tail_reduce_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, p.ypart,
                       p.tsplits, p.bias, p.Y, p.M, p.N, p.MT, p.tail0, ntail, p.bm);
    return hipGetLastError();
  }
  if (p.splits == 1) return e;
  const long MN = (long)p.M * p.N;
  const long work = (p.N & 3) == 0 ? MN / 4 : MN;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, p.ypart, p.splits,
                     p.bias, p.Y, p.M, p.N);
  return hipGetLastError();
}

// K ranges per output tile.  The grid holds one 128 x 128 tile per CU at a time, so a
// shape with fewer tiles than CUs (small M) leaves CUs idle for the whole K loop, and a
// tile count just above a multiple of the CU count leaves a short last round.  Splitting
// K into S ranges multiplies the workgroups by S at the price of S FP32 partial outputs
// written and read once more by a reduction launch.  S minimises the estimate
//   rounds(tiles * S) * steps(S) * t_step  +  [S > 1] (t_launch + partial bytes / bandwidth)
// with t_step ~0.8 us per 64-k step of a tile, t_launch ~2 us and ~6 TB/s for the
// partials (they stay in the Infinity Cache at these sizes); at least 2 K-steps per range.
namespace {
struct Plan {
  int splits, tsplits, tail0;
};

// The uniform split (every tile as S K ranges) and the tail split (only the last round's
// tiles, as t ranges) from one cost model: a K-step costs 0.8 us per round of resident
// workgroups, or 0.5 us for 64-row workgroups alone on their CUs (a sparse last round).  A
// uniform split adds 3.5 us plus its partial traffic (written once, read by the reduction)
// at 4 TB/s, fitted to 640 x 4096 x 4096 (3 ranges of all 160 tiles: 54.1 us; whole: 43.2
// us); a tail split adds 2 us plus its smaller partial traffic at 6 TB/s (its measured times
// match that within 1 us).  The tail split replaces the uniform choice when predicted 3%
// faster.
Plan gemm_plan(int M, int N, int K) {
  const int bm = gemm_bm(M, N);
  const long ntiles = (((long)M + bm - 1) / bm) * (((long)N + BN - 1) / BN);
  const int tsteps = (K / kBlock + 1) / 2;
  Plan plan{1, 1, (int)ntiles};
  if (ntiles <= 0 || tsteps <= 0) return plan;
  const long slots = bm == 64 ? 2 * kCUs : kCUs;     // workgroups resident at once
  double best_us = 1e30;
  for (int S = 1; S <= kMaxSplits; ++S) {
    const int sps = (tsteps + S - 1) / S;
    if (S > 1 && sps < 2) break;
    if ((tsteps + sps - 1) / sps != S) continue;     // some range would be empty
    const double rounds = (double)((ntiles * S + slots - 1) / slots);
    double us = rounds * sps * 0.8;
    if (S > 1) us += 3.5 + (2.0 * S + 0.5) * 4.0 * (double)M * N / 4e6;
    if (us < best_us * 0.97) {
      best_us = us;
      plan.splits = S;
    }
  }
  const long full = ntiles / slots, rem = ntiles % slots;
  if (full == 0 || rem == 0 || tsteps < 4) return plan;
  auto step_us = [&](long wgs) { return bm == 64 && wgs <= kCUs ? 0.5 : 0.8; };
  const double head_us = full * tsteps * 0.8;
  if (plan.splits == 1) best_us = head_us + tsteps * step_us(rem);   // the whole last round
  int best_t = 1;
  for (int t = 2; t <= kMaxSplits; ++t) {
    if (rem * t > slots) break;
    const int sps = (tsteps + t - 1) / t;
    if (sps < 2) break;
    if ((tsteps + sps - 1) / sps != t) continue;
    const double us = head_us + sps * step_us(rem * t) + 2.0 + (2.0 * t + 0.5) * 4.0 * (double)rem * bm * BN / 6e6;
    if (us < best_us * 0.97) {
      best_us = us;
      best_t = t;
    }
  }
  if (best_t > 1) plan = Plan{1, best_t, (int)(full * slots)};
  return plan;
}
}  // namespace

int gemm_splits(int M, int N, int K) { return gemm_plan(M, N, K).splits; }

// Tail split.  Without K splitting, a grid of `ntiles` tiles over `slots` resident
// workgroups runs floor(ntiles / slots) full rounds and a last, partly filled one that still
// takes a whole round's K loop.  Splitting only the last round's tiles into t K ranges
// (partials for those tiles alone, one reduction over their outputs) shortens that round.
// Measured: 1024 x 9728 x 2560 at M = 512 (608 tiles of 64 x 128, the last 96 as 5 ranges)
// 57.0 -> 51.6 us; at M = 1024 its last 192 tiles run alone on their CUs, a split gained
// nothing and the model leaves them whole.
int gemm_tail_splits(int M, int N, int K, int *tail0) {
  const Plan plan = gemm_plan(M, N, K);
  *tail0 = plan.tail0;
  return plan.tsplits;
}

}  // namespace mnb
