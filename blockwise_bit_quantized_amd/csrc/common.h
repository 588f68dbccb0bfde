// common.h -- types, packed-layout geometry and launch parameters shared by the libmnb
// kernels (gfx950 / CDNA4, wave64).
//
// Packed layout (this library's own; the pages fix only "2/4/8-bit codes in blocks of 32
// along K with an FP16 scale and an optional zero point per block"):
//   * weight rows are grouped by 64 (NG = ceil(N/64) groups, padded rows are zero);
//   * K is split in KB = K/32 blocks; a row holds CC 16-byte chunk-columns: CC = 2*KB
//     (8-bit, half a block each), KB (4-bit, one block), ceil(KB/2) (2-bit, two blocks);
//   * chunk (g, cc, r) lives at byte (((g*CC + cc)*64 + r) * 16), so one wave64 load
//     instruction of 16 B per lane reads 1 KiB of contiguous codes (64 rows of one
//     chunk-column);
//   * 4-bit chunk: 32-bit word j (bytes 4j..4j+3, little-endian) holds k = 8j..8j+7 with
//     nibble i = k 8j+2i (bits 4i..4i+3) and nibble 4+i = k 8j+2i+1 (bits 16+4i..).  The
//     mask 0x000F000F applied to (word >> 4i) then yields the pair (k, k+1) in the two
//     16-bit halves, which is exactly the packed-fp16 pair order of natural X;
//   * 8-bit chunk c: byte b holds k = 16c + b;
//   * 2-bit chunk cc: bytes 8h..8h+7 hold block 2cc + h (zero past KB); in it, word j
//     (bytes 4j..4j+3) holds k = 16j..16j+15 with 2-bit field i (bits 2i..2i+1) = k
//     16j+2i and field 8+i (bits 16+2i..) = k 16j+2i+1, so (word >> 2i) & 0x00030003 is
//     the natural pair (k, k+1) again;
//   * scales fp16 at ((g*KB + kb)*64 + r); zero points (4-bit) two per byte at
//     ((g*KB + kb)*32 + r/2), low nibble for even r; (8-bit) one byte at ((g*KB+kb)*64 + r);
//     (2-bit) four per byte at ((g*KB + kb)*16 + r/4), bits 2*(r%4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mnb {

constexpr int kGroup = 64;   // weight rows per interleaved group (= wave64 lanes)
constexpr int kBlock = 32;   // quantization block along K
constexpr int kRank = 32;    // LoRA rank supported by the kernels
constexpr int kCUs = 256;    // MI355X compute units (planning constant)

// 16-byte chunk-columns per row of KB blocks
__host__ __device__ __forceinline__ int chunk_cols(int bits, int KB) {
  return bits == 2 ? (KB + 1) / 2 : KB * (bits / 4);
}

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f16x_t __attribute__((ext_vector_type(16)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }
__device__ __forceinline__ uint32_t as_u32(h2_t v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Raw buffer descriptor over [base, base + bytes) (gfx9-family word 3: 32-bit data format,
// no swizzle, stride 0).  A buffer load whose byte offset lies at or past `bytes` returns
// zeros instead of touching memory; `bytes` is clamped to [0, 2^31 - 1].  The offsets
// passed with it are VGPR offsets (the range check covers them), the SGPR offset is 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, long bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// Device-scope (all XCDs) store of a flag word, written through the L2 (no fence: agent-
// scope fences write back and invalidate a whole L2 on this part).
__device__ __forceinline__ void atomic_store_agent(int *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Convert 4-bit codes to fp16 pairs: 0x6400 is 1024.0 in binary16, so OR-ing a 4-bit
// code into the low mantissa bits gives exactly 1024 + code; subtracting 1024 + z (also
// exact) yields the exact integer (code - z).
__device__ __forceinline__ h2_t nib_pair(uint32_t w, int i) {
  return as_h2(((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u);
}
// (x & mask) | (c & ~mask) in one v_bfi_b32 (the compiler splits the folded form into two)
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t x, uint32_t c) {
  uint32_t d;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(d) : "s"(mask), "v"(x), "v"(c));
  return d;
}
// Shift-free variant for 4-bit words: nibbles 0 and 2 of each half (after a shift by 8 for
// 2) sit in mantissa bits 0-3, giving 1024 + q; nibbles 1 and 3 are taken in place at
// bits 4-7, giving 1024 + 16 q, whose difference with 1024 + 16 z is 16 (q - z), exact.
__device__ __forceinline__ h2_t nib_lo(uint32_t w) { return as_h2(bfi(0x000F000Fu, w, 0x64006400u)); }
__device__ __forceinline__ h2_t nib_hi16(uint32_t w) { return as_h2(bfi(0x00F000F0u, w, 0x64006400u)); }
// 2-bit codes: field pair e (bits 2e.. of each half) as 1024 + q, both halves
__device__ __forceinline__ h2_t crumb_pair(uint32_t w, int e) {
  return as_h2(((w >> (2 * e)) & 0x00030003u) | 0x64006400u);
}
// Same for two 8-bit codes (bytes b0, b1 of w -> halves), via v_perm_b32 with the
// constant byte 0x64 taken from the first operand.
__device__ __forceinline__ h2_t byte_pair_lo(uint32_t w) {
  return as_h2(__builtin_amdgcn_perm(0x64646464u, w, 0x04010400u));
}
__device__ __forceinline__ h2_t byte_pair_hi(uint32_t w) {
  return as_h2(__builtin_amdgcn_perm(0x64646464u, w, 0x04030402u));
}

// Control area at the start of the workspace (its layout depends on no shape):
//   * 64 words: the in-pass T call epoch, the count of done-groups that have finished
//     reading T and a sticky error word;
//   * kDoneGroups counters of the in-pass launch's workgroups that have read the epoch,
//     one per 256-byte line so that the increments of different groups do not queue on
//     one address.
// Every counter is back to zero when a call ends.  The in-pass T slices are written in
// kTReplicas copies (32 words of FP32 value | call tag << 32 per slice), so that the row
// workgroups' reads spread over many lines.
enum { CTRL_EPOCH = 0, CTRL_TDONE = 1, CTRL_ERROR = 2, CTRL_WORDS = 64 };
constexpr int kDoneGroups = 16;
constexpr int kCtrlLineInts = 64;                                        // 256 B
constexpr int kTReplicas = 16;
// arrival counters of the T projection's K-parts, one per 32-row M tile (M <= 32768 rows)
constexpr int kTprojCounters = 1024;
constexpr size_t kCtrlBytes = (size_t)(1 + kDoneGroups) * kCtrlLineInts * sizeof(int) + kTprojCounters * sizeof(int);
__device__ __forceinline__ int ctrl_tproj_word(int mt) { return (1 + kDoneGroups) * kCtrlLineInts + mt; }
__device__ __forceinline__ int ctrl_done_word(int group) { return (1 + group) * kCtrlLineInts; }

// Bounded wait for the in-pass T handoff; on expiry the kernel records CTRL_ERROR and
// uses NaN for T so the failure is visible in Y rather than hanging the device.
constexpr int kSpinLimit = 1 << 22;

// ----------------------------------------------------------------------------------------
// Launch parameter blocks
// ----------------------------------------------------------------------------------------

struct GemvParams {
  const uint16_t *X;      // [M, K]
  const uint8_t *wq;      // packed codes
  const uint16_t *sc;     // packed scales
  const uint8_t *zp;      // packed zero points or null
  const void *A;          // adapter factors (kind-dependent)
  const uint16_t *sA;
  const void *B;
  const uint16_t *sB;
  uint16_t *Y;            // [M, N]
  const uint16_t *bias;   // fp16 [N] broadcast bias or null
  int M, N, K, NG, KB;
  int q;                  // chunk-columns per wave load; a workgroup owns 64/q rows
  int gt;                 // in-pass T: number of T-slice workgroups (first in the grid)
  int kt;                 // in-pass T: k rows per slice
  int nepi;               // in-pass T: number of row workgroups (the launch has gt + nepi)
  int spin_limit;         // in-pass T: polls before a row workgroup gives up (-1: at once)
  int tparts;             // precomputed T: number of K-part partials
  int tmpad;              // precomputed T: rows per partial (= M of the T launch)
  int *ctrl;              // control words
  const float *tin;       // precomputed T partials [tparts, tmpad, 32]
  unsigned long long *tword;  // in-pass T: [kTReplicas, gt, 32] slice words (FP32 value | call tag << 32)
};

struct TprojParams {
  const uint16_t *X;
  const void *A;
  const uint16_t *sA;
  float *tpart;           // [parts, M, 32] FP32 partial sums
  float *tfinal;          // [M, 32] FP32 sum over the parts (when `reduce`)
  int *ctrl;              // control words (arrival counters per M tile)
  int M, K, MT, parts, reduce;
};

struct GemmParams {
  const uint16_t *X;
  const uint8_t *wq;
  const uint16_t *sc;
  const uint8_t *zp;
  const void *B;
  const uint16_t *sB;
  const float *tpart;     // T partials [tparts, M, 32]
  uint16_t *Y;
  const uint16_t *bias;   // fp16 [N] broadcast bias or null
  float *ypart;           // splits > 1: FP32 partial outputs [splits, M, N];
                          // tsplits > 1: the tail tiles' partials [tsplits, tail tiles, bm, 128]
  int M, N, K, NG, KB, MT, NT, tparts;
  int splits;             // K ranges per output tile (1: the workgroup stores Y itself)
  int bm;                 // tile rows: 128 or 64
  int tail0;              // tsplits > 1: tiles from tail0 on (the last round) split K ...
  int tsplits;            // ... into tsplits ranges; 1: no tail split
};

struct PackParams {
  const uint8_t *codes;
  const uint16_t *scales;
  const uint8_t *zp;
  uint8_t *wq;
  uint16_t *sc;
  uint8_t *zpp;
  int N, K, NG, KB;
};

// Host-side launchers (each returns hipGetLastError() of its launch).
hipError_t launch_gemv(int bits, bool has_zp, int lora, int tmode, const GemvParams &p,
                       int grid_x, int grid_y, hipStream_t s);
// small M (2..16) on the matrix cores: 16 weight rows per workgroup, grid 4 * NG
hipError_t launch_gemv_mfma(int bits, int lora, const GemvParams &p, hipStream_t s);
bool gemv_mfma_wide(int M, int N, int K, int bits);   // the one-workgroup-per-row-group form
// accuracy level 4 (int8 block-quantized activations for the base product), any M
constexpr int kAcc4MaxK = 16384;
constexpr int kAcc4MultiRowMaxK = 4096;       // K limit of the 4-rows-per-workgroup form
int acc4_rows_mr(int M, int N, int K);        // X rows per workgroup row (1 or 4)
// accuracy level 4 on the GEMM path: Xq = fp16(block-quantized X), [M, K]
hipError_t launch_acc4_xquant(const uint16_t *X, uint16_t *Xq, int M, int K, hipStream_t s);
hipError_t launch_gemv_acc4(int bits, bool has_zp, int lora, const GemvParams &p, int grid_x, int grid_y,
                            hipStream_t s);
hipError_t launch_tproj(int lora, const TprojParams &p, hipStream_t s);
hipError_t launch_gemm(int bits, bool has_zp, int lora, const GemmParams &p, hipStream_t s);
int gemm_splits(int M, int N, int K);         // K ranges per output tile of the prefill GEMM
// K ranges of the tail tiles (1: none) when every tile otherwise runs whole; sets *tail0
int gemm_tail_splits(int M, int N, int K, int *tail0);
int gemm_bm(int M, int N);                    // tile rows of the prefill GEMM (64 or 128)
constexpr int kMaxSplits = 16;
// K limit: the GEMM's direct loads go through buffer descriptors whose 32-bit offsets reach
// one packed row group's codes (8-bit: 64 K bytes) and, for X, up to 8 rows (16 K + 112
// bytes); both stay below 2^31 - 1 for K < 2^25
constexpr int kMaxK = 1 << 25;
hipError_t launch_pack(int bits, bool kn, const PackParams &p, hipStream_t s);  // kn: [K, N] source
hipError_t launch_unpack(int bits, const PackParams &p, uint8_t *codes, uint16_t *scales,
                         uint8_t *zp, hipStream_t s);
hipError_t launch_fill(uint16_t *Y, const uint16_t *bias, int M, int N, hipStream_t s);

// planning helpers shared by the dispatcher and the launchers
int gemv_rows_split(int N, bool inpass_t);    // q: 1, 2, 4 or 8
int tproj_parts(int M, int K);                 // K parts of the T projection
// largest M of the small-M path (the matrix-core GEMV): measured against the MFMA GEMM (K
// split over workgroups, 64-row tiles) on the four workload weight sets, cold, it is faster
// at every M up to 16 (8192 x 2048 int4 + LoRA at M = 8: 10.3 against 15.7 us; 49152 x 576
// int8: 11.5 against 12.4 us; 9728 x 2560 with INT8 adapters at M = 16: 20.2 against 20.3)
constexpr int kSmallM = 16;
constexpr int kRowsMaxM = 16;                  // largest M the small-M path takes (its MFMA's rows)

}  // namespace mnb
