// gemv_mfma.hip -- small-M path of MatMulNBits (2 <= M <= 16) on the matrix cores: one HBM
// pass over the packed weights serves all M rows; each weight is dequantized once into an
// fp16 MFMA operand and multiplied with up to 16 X rows by v_mfma_f32_16x16x32_f16.
//
// onnxruntime PR #33370 ("[WebGPU] Fuse rank-32 quantized LoRA with MatMulNBits"), commit
// list: the path is chosen per matrix by its row count M, and fuse_up (M > 1) computes T
// first and adds T * Bt^T after the base product.  A matrix read once for a few rows is
// bound by HBM like the M == 1 decode, so the weight stream keeps the decode GEMV's shape;
// what changes is the arithmetic.  Dotting every unpacked weight with each of M rows costs
// M v_dot2 per pair of codes, which for M = 8 is ~4 us of VALU issue per SIMD at the
// 49152 x 576 int8 lm_head; here a pair costs 3 VALU operations (extract, subtract, scale)
// whatever M is, and the products run on the matrix core:
//  * a workgroup of 8 waves owns 16 rows of one 64-row group (the MFMA's 16 columns) over
//    the whole of K.  One wave load of 16 B per lane covers the 16 rows x 4 chunk-columns;
//    lane l holds row l % 16 of chunk-column 4 * load + l / 16;
//  * the MFMA's B operand is 8 consecutive k of one row per lane, lane group l / 16 giving
//    k group l / 16 of the instruction.  Each lane feeds 8 k of its own chunk at a time, so
//    one instruction sums over 4 chunk-columns' k ranges: the k order of the contraction is
//    permuted, the same permutation on both operands (X is staged in LDS by chunk-column).
//    The scale is folded into each fp16 weight ((q - z) s, rounded once), so blocks may mix
//    inside one instruction;
//  * X rows (up to 16: the MFMA's 16 rows) are staged into the wave's LDS area by
//    chunk-column, with a 16-byte pad per row so that the A-operand reads of 16 rows hit
//    distinct banks; rows past M read zeros and their outputs are not stored;
//  * waves meet in LDS in fixed order; the LoRA term (T from the projection launch) is one
//    more MFMA: T rows (fp16, rounded once from the FP32 sum over parts) by the B columns.
#include "common.h"

namespace mnb {
namespace {

enum { LORA_NONE = 0, LORA_F16 = 1, LORA_Q8 = 2 };
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsWG = 16;   // weight rows per workgroup: the MFMA's 16 columns
constexpr int kQ = 4;         // chunk-columns per wave load: one per 16-lane group

typedef float f4_t __attribute__((ext_vector_type(4)));

template <int BITS>
struct Shape {
  static constexpr int KPC = BITS == 2 ? 64 : 32 / (BITS / 4);        // k per chunk
  static constexpr int LPW = BITS == 4 ? 2 : (BITS == 8 ? 4 : 1);      // loads per wave per round
  static constexpr int kZpB = BITS == 4 ? 32 : (BITS == 8 ? 64 : 16);  // zero-point bytes per block
  static constexpr int kRowH = KPC + 8;                                 // X row pitch in LDS (halfs)
};

__device__ __forceinline__ h8_t cat4(h2_t a, h2_t b, h2_t c, h2_t d) {
  return h8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One wave load's chunk (16 B per lane: 32, 16 or 64 codes of row `row`) dequantized into
// fp16 (q - z) s, each rounded once, and multiplied by the X rows of its k range: `xslot` is
// the LDS slot of the lane's chunk-column (X row m at m * pitch halfs, MR rows), and lane l
// supplies X row l % 16 (zeros past M) to the A operand.
template <int BITS>
__device__ __forceinline__ void slot_mfma(f4_t &acc, const u4_t cw, uint32_t sraw, uint32_t zraw, bool has_zp,
                                          int row, const _Float16 *xslot, int pitch, int MR, int M) {
  const int xm = threadIdx.x & 15;
  const _Float16 *xa = xslot + (xm < MR ? xm : 0) * pitch;
  auto a_op = [&](int s8) -> h8_t {
    h8_t a = *reinterpret_cast<const h8_t *>(xa + 8 * s8);
    if (xm >= M) a = h8_t{};
    return a;
  };
  if constexpr (BITS == 4) {
    const uint32_t z = has_zp ? (zraw >> ((row & 1) * 4)) & 0xFu : 8u;
    const h2_t zz2 = as_h2((z * 0x00010001u) | 0x64006400u);           // 1024 + z
    const h2_t nz64 = as_h2(((z << 4) * 0x00010001u) | 0xD400D400u);   // -(64 + z)
    const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2_t s2 = as_h2((sraw & 0xffffu) * 0x00010001u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = cw[j], w8 = w >> 8;
      const h8_t b = cat4((nib_lo(w) - zz2) * s2, __builtin_elementwise_fma(nib_hi16(w), sixteenth, nz64) * s2,
                          (nib_lo(w8) - zz2) * s2, __builtin_elementwise_fma(nib_hi16(w8), sixteenth, nz64) * s2);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op(j), b, acc, 0, 0, 0);
    }
  } else if constexpr (BITS == 8) {
    const uint32_t z = has_zp ? zraw & 0xffu : 128u;
    const h2_t zz2 = as_h2((z * 0x00010001u) | 0x64006400u);
    const h2_t s2 = as_h2((sraw & 0xffffu) * 0x00010001u);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t w0 = cw[2 * j], w1 = cw[2 * j + 1];
      const h8_t b = cat4((byte_pair_lo(w0) - zz2) * s2, (byte_pair_hi(w0) - zz2) * s2,
                          (byte_pair_lo(w1) - zz2) * s2, (byte_pair_hi(w1) - zz2) * s2);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op(j), b, acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t z = has_zp ? ((zraw >> (8 * h)) >> ((row & 3) * 2)) & 3u : 2u;
      const h2_t zz2 = as_h2((z * 0x00010001u) | 0x64006400u);
      const h2_t s2 = as_h2(((sraw >> (16 * h)) & 0xffffu) * 0x00010001u);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w = cw[2 * h + j];
#pragma unroll
        for (int e4 = 0; e4 < 2; ++e4) {
          const h8_t b = cat4((crumb_pair(w, 4 * e4) - zz2) * s2, (crumb_pair(w, 4 * e4 + 1) - zz2) * s2,
                              (crumb_pair(w, 4 * e4 + 2) - zz2) * s2, (crumb_pair(w, 4 * e4 + 3) - zz2) * s2);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op(4 * h + 2 * j + e4), b, acc, 0, 0, 0);
        }
      }
    }
  }
}

// The end of a 16 x 16 output tile (X rows 4 (lane / 16) .. + 3 of weight row n, FP32 in
// `total`): plus the LoRA term, one more MFMA -- T rows as the A operand (row lane % 16,
// ranks 8 (lane / 16) .., fp16 rounded once from the FP32 sum over parts) by the B column as
// the B operand (INT8 B is exact in fp16; its column scale multiplies the product) -- plus
// the bias, stored as fp16 for the rows below M.
// T parts of the projection launch for the epilogue lane (X row lane % 16, ranks
// 8 (lane / 16) .. + 7): in the 16-row form with an adapter the first kTPre are loaded when
// the kernel starts, ahead of the weight stream, so their round trip passes with it (the
// projection keeps its parts to at most 4 when K allows, and reduces them itself beyond
// that); their registers are live throughout, so the form is instantiated without them for
// calls with one part or none, and the one-group form loads T in its epilogue
constexpr int kTPre = 4;
struct TPre {
  float4 v[kTPre][2];
};
__device__ __forceinline__ void t_prefetch(const GemvParams &p, int lora, int M, TPre &t) {
  const int lane = threadIdx.x & 63;
  const int tm = lane & 15, r0 = 8 * (lane >> 4);
  if (lora == LORA_NONE || tm >= M) return;
#pragma unroll
  for (int pp = 0; pp < kTPre; ++pp) {
    if (pp >= p.tparts) break;
    const float *src = p.tin + ((size_t)pp * p.tmpad + tm) * kRank + r0;
    t.v[pp][0] = *reinterpret_cast<const float4 *>(src);
    t.v[pp][1] = *reinterpret_cast<const float4 *>(src + 4);
  }
}

__device__ __forceinline__ void finish_tile(const GemvParams &p, int lora, f4_t total, int n, int M, const TPre *tp) {
  const int lane = threadIdx.x & 63;
  if (lora != LORA_NONE) {
    const int tm = lane & 15, r0 = 8 * (lane >> 4);
    float tv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (tm < M) {
      // the parts in part order: the prefetched ones, then any beyond them
      auto add = [&](const float4 &a, const float4 &b) {
        tv[0] += a.x; tv[1] += a.y; tv[2] += a.z; tv[3] += a.w;
        tv[4] += b.x; tv[5] += b.y; tv[6] += b.z; tv[7] += b.w;
      };
      int pp = 0;
      if (tp) {
#pragma unroll
        for (int q = 0; q < kTPre; ++q)
          if (q < p.tparts) add(tp->v[q][0], tp->v[q][1]);
        pp = kTPre;
      }
      for (; pp < p.tparts; ++pp) {
        const float *src = p.tin + ((size_t)pp * p.tmpad + tm) * kRank + r0;
        add(*reinterpret_cast<const float4 *>(src), *reinterpret_cast<const float4 *>(src + 4));
      }
    }
    h8_t ta, tb;
#pragma unroll
    for (int e = 0; e < 8; ++e) ta[e] = (_Float16)tv[e];
    const size_t nb = n < p.N ? n : 0;
    float bscale = 1.f;
    if (lora == LORA_F16) {
      const uint16_t *Bp = static_cast<const uint16_t *>(p.B);
#pragma unroll
      for (int e = 0; e < 8; ++e) tb[e] = __builtin_bit_cast(_Float16, Bp[(size_t)(r0 + e) * p.N + nb]);
    } else {
      const int8_t *Bp = static_cast<const int8_t *>(p.B);
#pragma unroll
      for (int e = 0; e < 8; ++e) tb[e] = (_Float16)Bp[(size_t)(r0 + e) * p.N + nb];
      bscale = h2f(p.sB[nb]);
    }
    const f4_t lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(ta, tb, f4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    total += lo * bscale;
  }
  if (n < p.N) {
    const float bias = p.bias ? h2f(p.bias[n]) : 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * (lane >> 4) + v;
      if (m < M) p.Y[(size_t)m * p.N + n] = __builtin_bit_cast(uint16_t, (_Float16)(total[v] + bias));
    }
  }
}

template <int BITS, int MR, bool TP>
__global__ __launch_bounds__(kThreads) void gemv_mfma_kernel(GemvParams p, int lora) {
  using S = Shape<BITS>;
  constexpr int KPC = S::KPC, LPW = S::LPW, kRowH = S::kRowH, kZpB = S::kZpB;
  constexpr int kSlotH = MR * kRowH;                         // one chunk-column's X rows
  __shared__ __attribute__((aligned(16))) _Float16 xs[kWaves][LPW * kQ * kSlotH];
  __shared__ f4_t red[kWaves][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the kQ sibling workgroups of a 64-row group on one XCD (ids 8 apart), as in the decode
  int wgi = blockIdx.x;
  if ((p.NG & 7) == 0) {
    const int x = wgi & 7, u = wgi >> 3;
    wgi = (x + 8 * (u / kQ)) * kQ + (u % kQ);
  }
  const int g = wgi / kQ;
  const int rowoff = (wgi - g * kQ) * kRowsWG;
  const int nl = lane & 15;              // MFMA column: this lane's weight row in the workgroup
  const int gq = lane >> 4;              // k group: the chunk-column slot of a wave load
  const int row = rowoff + nl;
  const int n = g * kGroup + row;
  const int M = p.M;
  const bool has_zp = p.zp != nullptr;
  const int ncc = chunk_cols(BITS, p.KB);
  const int nloads = (ncc + kQ - 1) / kQ;

  // per-lane byte offsets inside one wave load's window (see the decode GEMV)
  const uint32_t w_lane = (uint32_t)(gq * kGroup + row) * 16u;
  uint32_t s_lane, z_lane;
  if constexpr (BITS == 4) {
    s_lane = (uint32_t)(gq * kGroup + row) * 2u;
    z_lane = (uint32_t)(gq * kZpB + (row >> 1));
  } else if constexpr (BITS == 8) {
    s_lane = (uint32_t)((gq >> 1) * kGroup + row) * 2u;
    z_lane = (uint32_t)((gq >> 1) * kZpB + row);
  } else {
    s_lane = (uint32_t)(2 * gq * kGroup + row) * 2u;
    z_lane = (uint32_t)(2 * gq * kZpB + (row >> 2));
  }
  // all of X through one descriptor: a piece of a row past M, or of k past K, reads zeros
  const auto rx = buffer_rsrc(p.X, (long)M * p.K * 2);
  TPre tpre;                               // wave 0 finishes the tile: its T parts first
  if constexpr (TP)
    if (wave == 0) t_prefetch(p, lora, M, tpre);

  f4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int l0 = 0; l0 < nloads; l0 += kWaves * LPW) {
    const int c0 = l0 * kQ;
    const int kb0 = BITS == 4 ? c0 : (BITS == 8 ? c0 / 2 : 2 * c0);
    const auto rw = buffer_rsrc(p.wq + ((size_t)g * ncc + c0) * kGroup * 16, (long)(ncc - c0) * kGroup * 16);
    const auto rs = buffer_rsrc(p.sc + ((size_t)g * p.KB + kb0) * kGroup, (long)(p.KB - kb0) * kGroup * 2);
    const auto rz = buffer_rsrc(has_zp ? p.zp + ((size_t)g * p.KB + kb0) * kZpB : p.wq,
                                has_zp ? (long)(p.KB - kb0) * kZpB : 0);
    // 1. X pieces of this wave's slots (slot j = i * kQ + q holds chunk-column
    //    (l0 + wave + kWaves * i) * kQ + q): piece = (slot, X row m, 8 halfs)
    constexpr int kPieces = LPW * kQ * MR * (KPC / 8);
    constexpr int kIter = (kPieces + 63) / 64;
    u4_t xv[kIter];
#pragma unroll
    for (int t = 0; t < kIter; ++t) {
      const int pc = lane + 64 * t;
      const int sub = pc % (KPC / 8), rest = pc / (KPC / 8);
      const int m = rest % MR, j = rest / MR;
      const int cc = (l0 + wave + kWaves * (j / kQ)) * kQ + j % kQ;
      const int k = cc * KPC + sub * 8;
      const bool in = pc < kPieces && m < M && k < p.K;
      xv[t] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? (uint32_t)((size_t)m * p.K + k) * 2u : 0x7ffffff0u, 0, 0);
    }
    // 2. this wave's weight stream (a slot past the last load reads zeros)
    u4_t cw[LPW];
    uint32_t sraw[LPW], zraw[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const uint32_t rel = (uint32_t)(wave + kWaves * i);
      cw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane + rel * (kQ * kGroup * 16), 0, 0);
      if constexpr (BITS == 4) {
        sraw[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, s_lane + rel * (kQ * kGroup * 2), 0, 0);
        zraw[i] = has_zp ? __builtin_amdgcn_raw_buffer_load_b8(rz, z_lane + rel * (kQ * kZpB), 0, 0) : 0u;
      } else if constexpr (BITS == 8) {
        const uint32_t tl = rel * (kQ / 2);                  // block of the load's chunk-column 0
        sraw[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, s_lane + tl * (kGroup * 2), 0, 0);
        zraw[i] = has_zp ? __builtin_amdgcn_raw_buffer_load_b8(rz, z_lane + tl * kZpB, 0, 0) : 0u;
      } else {
        const uint32_t so = s_lane + rel * (kQ * kGroup * 4), zo = z_lane + rel * (kQ * kZpB * 2);
        sraw[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0) |
                  ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, so + kGroup * 2, 0, 0) << 16);
        zraw[i] = has_zp ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, zo, 0, 0) |
                               ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, zo + kZpB, 0, 0) << 8)
                         : 0u;
      }
    }
    // 3. X to LDS (written and read by this wave only: LDS order suffices)
#pragma unroll
    for (int t = 0; t < kIter; ++t) {
      const int pc = lane + 64 * t;
      const int sub = pc % (KPC / 8), rest = pc / (KPC / 8);
      const int m = rest % MR, j = rest / MR;
      if (pc < kPieces) *reinterpret_cast<u4_t *>(&xs[wave][j * kSlotH + m * kRowH + sub * 8]) = xv[t];
    }
    // 4. dequantize each weight once ((q - z) s, rounded once) and multiply with the X rows
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      if (l0 + wave + kWaves * i >= nloads) continue;        // uniform
      slot_mfma<BITS>(acc, cw[i], sraw[i], zraw[i], has_zp, row, &xs[wave][(i * kQ + gq) * kSlotH], kRowH, MR, M);
    }
  }

  // waves meet in LDS, in fixed order; wave 0 finishes: lane l holds the outputs of X rows
  // 4 (l / 16) .. + 3 for weight row l % 16
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f4_t total = red[0][lane];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) total += red[w][lane];

  finish_tile(p, lora, total, n, M, TP ? &tpre : nullptr);
}

// Short K and many row groups: a workgroup owns one 64-row group, with X for all of K (at
// most LPW * 4 chunk-columns) staged once per workgroup.  With up to 8 X rows it has 8
// waves: waves w and w + 4 own rows 16 w .. 16 w + 15 and take the even and the odd wave
// loads of those rows, and the odd half's partial sums reach the even half through LDS
// (added in that order).  With 16 X rows it has 4 waves, each over the whole of K.  Every
// wave issues all of its loads before it waits on anything.  A wave's loads in flight are
// what bounds this form: on the 49152 x 576 int8 lm_head (9 wave loads per row) splitting
// each row slice over two waves took M = 2-8 from 10.7 to 9.6 us; at 16 X rows (larger
// staging and MFMA operands per wave) a timing copy of the split without the halves' sum
// (so at best) was slower, 11.1 -> 12.2 us.  (With 8
// waves splitting K over 16 rows instead, a 576-k row gives each 16-row workgroup 9 wave
// loads for 8 waves and 4 workgroups per 64 rows: the lm_head then ran 3072 small
// workgroups in four dispatch rounds.)
template <int BITS, int MR, int LPW>
__global__ __launch_bounds__(MR <= 8 ? 512 : 256) void gemv_mfma_wide_kernel(GemvParams p, int lora) {
  using S = Shape<BITS>;
  constexpr int KPC = S::KPC, kRowH = S::kRowH, kZpB = S::kZpB;
  constexpr int kSlotH = MR * kRowH;
  constexpr int kCC = LPW * kQ;                              // chunk-columns of X staged
  constexpr int kHalves = MR <= 8 ? 2 : 1;                   // waves per 16-row slice
  constexpr int kNT = 256 * kHalves;                         // threads
  __shared__ __attribute__((aligned(16))) _Float16 xs[kCC * kSlotH];
  __shared__ f4_t red[kHalves == 2 ? 4 : 1][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave >> 2;                                // 0 with kHalves == 1
  const int g = blockIdx.x;
  const int nl = lane & 15, gq = lane >> 4;
  const int row = (wave & 3) * kRowsWG + nl;
  const int n = g * kGroup + row;
  const int M = p.M;
  const bool has_zp = p.zp != nullptr;
  const int ncc = chunk_cols(BITS, p.KB);
  const int nloads = (ncc + kQ - 1) / kQ;                    // <= LPW (the host's choice)

  const uint32_t w_lane = (uint32_t)(gq * kGroup + row) * 16u;
  uint32_t s_lane, z_lane;
  if constexpr (BITS == 4) {
    s_lane = (uint32_t)(gq * kGroup + row) * 2u;
    z_lane = (uint32_t)(gq * kZpB + (row >> 1));
  } else if constexpr (BITS == 8) {
    s_lane = (uint32_t)((gq >> 1) * kGroup + row) * 2u;
    z_lane = (uint32_t)((gq >> 1) * kZpB + row);
  } else {
    s_lane = (uint32_t)(2 * gq * kGroup + row) * 2u;
    z_lane = (uint32_t)(2 * gq * kZpB + (row >> 2));
  }
  const auto rx = buffer_rsrc(p.X, (long)M * p.K * 2);
  const auto rw = buffer_rsrc(p.wq + (size_t)g * ncc * kGroup * 16, (long)ncc * kGroup * 16);
  const auto rs = buffer_rsrc(p.sc + (size_t)g * p.KB * kGroup, (long)p.KB * kGroup * 2);
  const auto rz = buffer_rsrc(has_zp ? p.zp + (size_t)g * p.KB * kZpB : p.wq, has_zp ? (long)p.KB * kZpB : 0);

  // 1. X pieces (chunk-column, X row m, 8 halfs) over the workgroup's threads
  constexpr int kPieces = kCC * MR * (KPC / 8);
  constexpr int kIter = (kPieces + kNT - 1) / kNT;
  u4_t xv[kIter];
#pragma unroll
  for (int t = 0; t < kIter; ++t) {
    const int pc = threadIdx.x + kNT * t;
    const int sub = pc % (KPC / 8), rest = pc / (KPC / 8);
    const int m = rest % MR, cc = rest / MR;
    const int k = cc * KPC + sub * 8;
    const bool in = pc < kPieces && m < M && k < p.K;
    xv[t] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? (uint32_t)((size_t)m * p.K + k) * 2u : 0x7ffffff0u, 0, 0);
  }
  // 2. this wave's weight stream: wave load i covers chunk-columns 4 i .. 4 i + 3 of its
  //    rows (with two halves, this wave's loads are those with i % 2 == half)
  u4_t cw[LPW];
  uint32_t sraw[LPW], zraw[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    if (kHalves == 2 && (i & 1) != half) continue;           // uniform
    const uint32_t rel = (uint32_t)i;
    cw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane + rel * (kQ * kGroup * 16), 0, 0);
    if constexpr (BITS == 4) {
      sraw[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, s_lane + rel * (kQ * kGroup * 2), 0, 0);
      zraw[i] = has_zp ? __builtin_amdgcn_raw_buffer_load_b8(rz, z_lane + rel * (kQ * kZpB), 0, 0) : 0u;
    } else if constexpr (BITS == 8) {
      const uint32_t tl = rel * (kQ / 2);
      sraw[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, s_lane + tl * (kGroup * 2), 0, 0);
      zraw[i] = has_zp ? __builtin_amdgcn_raw_buffer_load_b8(rz, z_lane + tl * kZpB, 0, 0) : 0u;
    } else {
      const uint32_t so = s_lane + rel * (kQ * kGroup * 4), zo = z_lane + rel * (kQ * kZpB * 2);
      sraw[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0) |
                ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, so + kGroup * 2, 0, 0) << 16);
      zraw[i] = has_zp ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, zo, 0, 0) |
                             ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, zo + kZpB, 0, 0) << 8)
                       : 0u;
    }
  }
  // 3. X to LDS, shared by the waves
#pragma unroll
  for (int t = 0; t < kIter; ++t) {
    const int pc = threadIdx.x + kNT * t;
    const int sub = pc % (KPC / 8), rest = pc / (KPC / 8);
    const int m = rest % MR, cc = rest / MR;
    if (pc < kPieces) *reinterpret_cast<u4_t *>(&xs[cc * kSlotH + m * kRowH + sub * 8]) = xv[t];
  }
  __syncthreads();
  // 4. dequantize each weight once and multiply with the X rows
  f4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    if (i >= nloads || (kHalves == 2 && (i & 1) != half)) continue;   // uniform
    slot_mfma<BITS>(acc, cw[i], sraw[i], zraw[i], has_zp, row, &xs[(i * kQ + gq) * kSlotH], kRowH, MR, M);
  }
  if constexpr (kHalves == 2) {
    // the odd loads' partial sums to the even half, added in that order
    if (half) red[wave & 3][lane] = acc;
    __syncthreads();
    if (half) return;
    acc += red[wave][lane];
  }
  finish_tile(p, lora, acc, n, M, nullptr);
}

template <int BITS, bool TP>
void launch_bits_tp(const GemvParams &p, int lora, int gx, hipStream_t s) {
  if (p.M <= 8) hipLaunchKernelGGL((gemv_mfma_kernel<BITS, 8, TP>), dim3(gx), dim3(kThreads), 0, s, p, lora);
  else hipLaunchKernelGGL((gemv_mfma_kernel<BITS, 16, TP>), dim3(gx), dim3(kThreads), 0, s, p, lora);
}
template <int BITS>
hipError_t launch_bits(const GemvParams &p, int lora, int gx, hipStream_t s) {
  // the prefetch only where there are parts to add: its registers cost occupancy (with them
  // 9728 x 2560 at M <= 8 fits two workgroups per CU, not three, and ran two rounds)
  if (lora != LORA_NONE && p.tparts > 1) launch_bits_tp<BITS, true>(p, lora, gx, s);
  else launch_bits_tp<BITS, false>(p, lora, gx, s);
  return hipGetLastError();
}

template <int BITS, int MR>
hipError_t launch_wide_mr(const GemvParams &p, int lora, int nloads, hipStream_t s) {
  const dim3 block(MR <= 8 ? 512 : 256);                    // the kernel's two halves at up to 8 X rows
  if (nloads <= 8) hipLaunchKernelGGL((gemv_mfma_wide_kernel<BITS, MR, 8>), dim3(p.NG), block, 0, s, p, lora);
  else if (nloads <= 9) hipLaunchKernelGGL((gemv_mfma_wide_kernel<BITS, MR, 9>), dim3(p.NG), block, 0, s, p, lora);
  else if (nloads <= 12) hipLaunchKernelGGL((gemv_mfma_wide_kernel<BITS, MR, 12>), dim3(p.NG), block, 0, s, p, lora);
  else hipLaunchKernelGGL((gemv_mfma_wide_kernel<BITS, MR, 16>), dim3(p.NG), block, 0, s, p, lora);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_wide(const GemvParams &p, int lora, int nloads, hipStream_t s) {
  return p.M <= 8 ? launch_wide_mr<BITS, 8>(p, lora, nloads, s) : launch_wide_mr<BITS, 16>(p, lora, nloads, s);
}

}  // namespace

// The wide form when the rows are many and short: at least 256 row groups (one workgroup
// each), at most 16 wave loads per row (a 576-k int8 row has 9, instantiated exactly: three
// idle loads of the next size up cost 0.7 us there at M = 8) and X staging within 64 KiB
// (room for two workgroups per CU); else 8 waves split K.
bool gemv_mfma_wide(int M, int N, int K, int bits) {
  const int NG = (int)(((long)N + kGroup - 1) / kGroup);
  const int nloads = (chunk_cols(bits, K / kBlock) + kQ - 1) / kQ;
  const int lpw = nloads <= 8 ? 8 : (nloads <= 9 ? 9 : (nloads <= 12 ? 12 : 16));
  const int mr = M <= 8 ? 8 : 16;
  const int kpc = bits == 2 ? 64 : 32 / (bits / 4);
  const long lds = (long)lpw * kQ * mr * (kpc + 8) * 2;
  return NG >= 256 && nloads <= 16 && lds <= 65536;
}

// p.M in [1, 16]
hipError_t launch_gemv_mfma(int bits, int lora, const GemvParams &p, hipStream_t s) {
  if (p.M < 1 || p.M > kRowsMaxM) return hipErrorInvalidValue;
  if (gemv_mfma_wide(p.M, p.N, p.K, bits)) {
    const int nloads = (chunk_cols(bits, p.KB) + kQ - 1) / kQ;
    if (bits == 2) return launch_wide<2>(p, lora, nloads, s);
    return bits == 4 ? launch_wide<4>(p, lora, nloads, s) : launch_wide<8>(p, lora, nloads, s);
  }
  const int gx = p.NG * kQ;
  if (bits == 2) return launch_bits<2>(p, lora, gx, s);
  return bits == 4 ? launch_bits<4>(p, lora, gx, s) : launch_bits<8>(p, lora, gx, s);
}

}  // namespace mnb
