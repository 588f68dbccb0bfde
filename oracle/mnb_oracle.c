/*
 * mnb_oracle.c -- plain, slow, obviously correct CPU oracle for MatMulNBits with an
 * optional rank-32 LoRA term.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load this library; the product path never
 * does.  It shares no code, header, table or constant generator with the HIP library.
 *
 * What it computes (FP64 throughout):
 *
 *   w[n,k]   = (q[n,k] - z[n,k/32]) * s[n,k/32]
 *   base     = X . w^T                         (sum over k in ascending order)
 *   t[m,r]   = sum_k X[m,k] * a[k,r]           (LoRA down-projection)
 *   lora     = t . b                           (LoRA up-projection, sum over r ascending)
 *   Y        = base + lora                     (Y = base when the adapter is empty)
 *
 * Sources, by page and section:
 *  - "Fuse DQ->MatMulNBits for shared initializers and skip outer-scope weights"
 *    (onnxruntime PR #33800), Description and Tests: the fused MatMulNBits output is
 *    compared against the unfused DequantizeLinear -> MatMul graph, so MatMulNBits is
 *    DequantizeLinear followed by MatMul.  DequantizeLinear is (x - zero_point) * scale
 *    (the ONNX operator definition), applied here per block of 32 along K.
 *  - "[WebGPU] Fuse rank-32 quantized LoRA with MatMulNBits" (onnxruntime PR #33370),
 *    commit list: INT4/block-32 base weights, rank-32 adapters, "base + T * Bt^T" with
 *    T = X * A, and empty adapters executing only the base projection; Description:
 *    rank-32 block-32 INT8 adapters.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - default zero point (zp pointer NULL) = 2^(bits-1): 8 for 4-bit, 128 for 8-bit;
 *  - INT8 adapters are symmetric int8 values times an fp16 scale per block of 32 along
 *    each factor's contraction axis: a[k,r] = vA[k,r] * sA[k/32, r],
 *    b[r,n] = vB[r,n] * sB[r/32, n];
 *  - an adapter is empty when kind == 0, rank == 0, or A or B is NULL.
 *
 * The packed device layout (mnbo_pack / mnbo_unpack) is this project's own layout; it is
 * implemented here independently from its prose description:
 *  - rows are grouped by 64 (NG = ceil(N/64)), padded rows hold code 0, scale 0, zp 0;
 *  - KB = K/32 blocks; for 4 and 8 bits each block of one row is C = bits/4 chunks of
 *    16 bytes, and wq chunk (g, kb, c, r) sits at byte ((((g*KB + kb)*C + c)*64 + r) * 16);
 *  - 2-bit: one 16-byte chunk holds two consecutive blocks of one row: chunk (g, kb2, r),
 *    kb2 < KB2 = ceil(KB/2), sits at byte (((g*KB2 + kb2)*64 + r) * 16); its bytes 8h..8h+7
 *    hold block 2*kb2 + h (all zero when that block is past KB).  Within a block's 8 bytes,
 *    bytes 4j..4j+3 form a little-endian word (j = 0, 1) whose 2-bit field i (bits
 *    2i..2i+1, i = 0..7) holds k = 16j + 2i and whose field 8+i (bits 16+2i..) holds
 *    k = 16j + 2i + 1;
 *  - 4-bit chunk: 32 codes k = 0..31 of the block; bytes 4j..4j+3 form a little-endian
 *    32-bit word whose nibble i (bits 4i..4i+3, i = 0..3) holds k = 8j + 2i and whose
 *    nibble 4+i (bits 16+4i..) holds k = 8j + 2i + 1;
 *  - 8-bit chunk c: byte b holds k = 16c + b;
 *  - scales: fp16 element ((g*KB + kb)*64 + r);
 *  - zero points: 4-bit byte ((g*KB + kb)*32 + r/2), low nibble for even r, high for odd r;
 *    8-bit byte ((g*KB + kb)*64 + r); 2-bit byte ((g*KB + kb)*16 + r/4), bits
 *    2*(r%4)..2*(r%4)+1.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC.  MNBO_MUTATION=<n> plants one
 * deliberate mistake (see the switch in each function); it exists so that the pin tests
 * can show that each such mistake is caught.  The normal build has MNBO_MUTATION=0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef MNBO_MUTATION
#define MNBO_MUTATION 0
#endif

#define BLK 32
#define GROUP 64

int mnbo_mutation(void) { return MNBO_MUTATION; }

/* IEEE 754 binary16 -> double, from the format definition: sign, 5-bit exponent with
 * bias 15, 10-bit fraction; exponent 0 is subnormal (fraction * 2^-24); 31 is inf/NaN. */
static double h2d(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0) v = ldexp((double)f, -24);
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexp((double)(f + 1024), e - 25);
  return sign ? -v : v;
}

/* double -> binary16 with round-to-nearest, ties to even. */
static uint16_t d2h(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  if (isnan(v)) return 0x7e00;
  double a = fabs(v);
  if (a >= 65520.0) return sign | 0x7c00;           /* halfway to 2^16 rounds up (odd max) */
  if (a < ldexp(1.0, -14)) {                         /* subnormal range, quantum 2^-24 */
    double q = rint(ldexp(a, 24));                   /* rint: current mode = nearest-even */
    return sign | (uint16_t)q;                       /* q == 1024 is the smallest normal */
  }
  int e;
  frexp(a, &e);                                      /* a in [2^(e-1), 2^e) */
  double q = rint(ldexp(a, 11 - e));                 /* 11-bit significand in [1024, 2048] */
  int E = e + 14;
  if (q >= 2048.0) { q = 1024.0; E += 1; }
  if (E >= 31) return sign | 0x7c00;
  return sign | (uint16_t)(E << 10) | (uint16_t)((int)q - 1024);
}

void mnbo_f16_to_f64(const uint16_t *h, double *d, long n) {
  for (long i = 0; i < n; ++i) d[i] = h2d(h[i]);
}

void mnbo_f64_to_f16(const double *d, uint16_t *h, long n) {
  for (long i = 0; i < n; ++i) h[i] = d2h(d[i]);
}

static int default_zp(int bits) {
#if MNBO_MUTATION == 6
  (void)bits;
  return 0;                                          /* planted: wrong default zero point */
#else
  return 1 << (bits - 1);
#endif
}

/* Step 2 of the definition: w[n,k] = (q - z) * s, one block of 32 along K per scale. */
static double dequant(const uint8_t *codes, const uint16_t *scales, const uint8_t *zp,
                      int N, int K, int bits, int n, int k) {
  int KB = K / BLK;
  int kb = k / BLK;
#if MNBO_MUTATION == 4
  kb = (kb + 1) % KB;                                /* planted: off-by-one block index */
#endif
  long si = (long)n * KB + kb;
#if MNBO_MUTATION == 3
  si = (long)kb * N + n;                             /* planted: transposed scale index */
#endif
  double q = (double)codes[(long)n * K + k];
  double z = zp ? (double)zp[(long)n * KB + kb] : (double)default_zp(bits);
  double s = h2d(scales[si]);
#if MNBO_MUTATION == 1
  return (q + z) * s;                                /* planted: zero point sign */
#else
  return (q - z) * s;
#endif
}

/* LoRA factor entries, F16 (kind 1) or block-32 INT8 (kind 2). */
static double lora_a(int kind, const void *A, const uint16_t *sA, int K, int k, int r) {
  long idx = (long)k * 32 + r;
#if MNBO_MUTATION == 5
  idx = (long)r * K + k;                             /* planted: A read transposed */
#endif
  if (kind == 1) return h2d(((const uint16_t *)A)[idx]);
  int sr = r;
#if MNBO_MUTATION == 10
  sr = 0;                                            /* planted: scale ignores the rank column */
#endif
  return (double)((const int8_t *)A)[idx] * h2d(sA[(long)(k / BLK) * 32 + sr]);
}

static double lora_b(int kind, const void *B, const uint16_t *sB, int N, int r, int n) {
  long idx = (long)r * N + n;
#if MNBO_MUTATION == 9
  idx = (long)n * 32 + r;                            /* planted: B read transposed */
#endif
  if (kind == 1) return h2d(((const uint16_t *)B)[idx]);
  return (double)((const int8_t *)B)[idx] * h2d(sB[(long)(r / BLK) * N + n]);
}

/*
 * Accuracy level 4 (int8 activations for the base product; on the PR #33370 page's commit
 * list the base product may take int8-quantized activations while T is still computed
 * from the unquantized FP16 X, and the PR #33800 page runs its lm_head at the default
 * accuracy level 4).  The pages give no
 * quantization rule; the reading taken here, per row and per block of 32 along K:
 *   amax = max |x|  (FP32; every binary16 is exact in it)
 *   amax == 0: every code 0;  else inv = 127 / amax, q = rint(x * inv) clamped to
 *   [-127, 127] (FP32 division and multiplication, round to nearest even), sx = amax / 127
 *   x' = q * sx  (exact in FP64), and the base product uses x' in place of x.
 */
static void quantize_block_acc4(const uint16_t *xh, double *xq) {
  float amax = 0.0f;
  for (int j = 0; j < BLK; ++j) {
    float a = fabsf((float)h2d(xh[j]));
    if (a > amax) amax = a;
  }
  if (amax == 0.0f) {
    for (int j = 0; j < BLK; ++j) xq[j] = 0.0;
    return;
  }
#if MNBO_MUTATION == 13
  volatile float inv = 128.0f / amax;                /* planted: 128 levels instead of 127 */
#else
  volatile float inv = 127.0f / amax;
#endif
  volatile float sx = amax / 127.0f;
  for (int j = 0; j < BLK; ++j) {
    volatile float prod = (float)h2d(xh[j]) * inv;
    float q = rintf(prod);
    if (q > 127.0f) q = 127.0f;
    if (q < -127.0f) q = -127.0f;
    xq[j] = (double)q * (double)sx;
  }
}

/*
 * Y[m,n] (FP64, row-major [M,N]).  X [M,K] binary16; codes [N,K] one per byte; scales
 * [N,K/32] binary16; zp [N,K/32] or NULL; kind 0 none / 1 F16 / 2 INT8; rank 0 or 32;
 * acc_level 0 (exact FP16 activations) or 4 (int8 activations for the base, above).
 * Returns 0, or -1 on unsupported arguments.
 */
int mnbo_matmul(int M, int N, int K, int bits, const uint16_t *X, const uint8_t *codes,
                const uint16_t *scales, const uint8_t *zp, int kind, int rank, const void *A,
                const uint16_t *A_scales, const void *B, const uint16_t *B_scales,
                const uint16_t *bias, double *Y, int acc_level) {
  if (acc_level != 0 && acc_level != 4) return -1;
  if (M < 0 || N < 0 || K < 0 || K % BLK) return -1;
  if (bits != 2 && bits != 4 && bits != 8) return -1;
  int has_lora = kind != 0 && rank != 0 && A != NULL && B != NULL;
  if (has_lora && (rank != 32 || (kind != 1 && kind != 2))) return -1;
  if (has_lora && kind == 2 && (A_scales == NULL || B_scales == NULL)) return -1;
#if MNBO_MUTATION == 2
  has_lora = 0;                                      /* planted: LoRA term dropped */
#endif
  if (M == 0 || N == 0) return 0;

  /* step 1: x = (double)X, exact */
  double *x = (double *)malloc(sizeof(double) * ((size_t)M * K + 1));
  for (long i = 0; i < (long)M * K; ++i) {
#if MNBO_MUTATION == 8
    long m = i / K, k = i % K;                       /* planted: X read transposed */
    x[i] = h2d(X[k * M + m]);
#else
    x[i] = h2d(X[i]);
#endif
  }

  /* step 1b (accuracy level 4): the base product's activations are quantized per block */
  double *xb = x;
  if (acc_level == 4) {
    xb = (double *)malloc(sizeof(double) * ((size_t)M * K + 1));
    for (int m = 0; m < M; ++m)
      for (int b = 0; b < K / BLK; ++b)
        quantize_block_acc4(X + (long)m * K + (long)b * BLK, xb + (long)m * K + (long)b * BLK);
  }

  /* step 2: dequantize W to FP64 */
  double *w = (double *)malloc(sizeof(double) * ((size_t)N * K + 1));
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) w[(long)n * K + k] = dequant(codes, scales, zp, N, K, bits, n, k);

  /* step 3: base = X . w^T, ascending k */
#pragma omp parallel for collapse(2) schedule(static)
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) {
      const double *xr = xb + (long)m * K, *wr = w + (long)n * K;
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += xr[k] * wr[k];
      Y[(long)m * N + n] = acc;
    }

  /* step 4: Y += (X . a) . b */
  if (has_lora) {
    double *a = (double *)malloc(sizeof(double) * (size_t)K * 32 + 8);
    double *b = (double *)malloc(sizeof(double) * (size_t)32 * N + 8);
    double *t = (double *)malloc(sizeof(double) * (size_t)M * 32 + 8);
    for (int k = 0; k < K; ++k)
      for (int r = 0; r < 32; ++r) a[k * 32 + r] = lora_a(kind, A, A_scales, K, k, r);
    for (int r = 0; r < 32; ++r)
      for (int n = 0; n < N; ++n) b[(long)r * N + n] = lora_b(kind, B, B_scales, N, r, n);
    for (int m = 0; m < M; ++m)
      for (int r = 0; r < 32; ++r) {
        double acc = 0.0;
#if MNBO_MUTATION == 14
        for (int k = 0; k < K; ++k) acc += xb[(long)m * K + k] * a[k * 32 + r];   /* planted: T from quantized X */
#else
        for (int k = 0; k < K; ++k) acc += x[(long)m * K + k] * a[k * 32 + r];
#endif
        t[m * 32 + r] = acc;
      }
#pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < M; ++m)
      for (int n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int r = 0; r < 32; ++r) acc += t[m * 32 + r] * b[(long)r * N + n];
        Y[(long)m * N + n] += acc;
      }
    free(a);
    free(b);
    free(t);
  }

  /* step 5: Y[m, n] += bias[n], the optional broadcast bias of MatMulNBits (the PR #33370
     page, commit list: empty packed weights give zeros or the broadcast bias) */
  if (bias != NULL)
    for (int m = 0; m < M; ++m)
      for (int n = 0; n < N; ++n) {
#if MNBO_MUTATION == 11
        Y[(long)m * N + n] += h2d(bias[m % N]);       /* planted: bias indexed by the row */
#else
        Y[(long)m * N + n] += h2d(bias[n]);
#endif
      }
  if (xb != x) free(xb);
  free(x);
  free(w);
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Packed device layout                                                                  */
/* ------------------------------------------------------------------------------------ */

static int bits_ok(int bits) { return bits == 2 || bits == 4 || bits == 8; }

int mnbo_packed_sizes(int N, int K, int bits, int has_zp, long *wq, long *sc, long *zpb) {
  if (N < 0 || K < 0 || K % BLK || !bits_ok(bits)) return -1;
  long NG = (N + GROUP - 1) / GROUP, KB = K / BLK;
  *wq = bits == 2 ? NG * ((KB + 1) / 2) * GROUP * 16 : NG * KB * GROUP * 16 * (bits / 4);
  *sc = NG * KB * GROUP * 2;
  *zpb = has_zp ? NG * KB * GROUP * bits / 8 : 0;
  return 0;
}

/* byte offset of the 4-bit code k (0..31) inside its 16-byte chunk, and its nibble shift */
static void nib_pos(int k, int *byte, int *shift) {
  int j = k / 8, within = k % 8;
  int i = within / 2, hi_half = within % 2;          /* even k -> low 16 bits, odd -> high */
  int bit = (hi_half ? 16 : 0) + 4 * i;
#if MNBO_MUTATION == 7
  bit = 4 * within;                                  /* planted: natural nibble order */
#endif
  *byte = 4 * j + bit / 8;
  *shift = bit % 8;
}

/* byte offset of the 2-bit code k (0..31) of block kb inside its 16-byte chunk, and its
   shift; the chunk is (kb / 2) */
static void crumb_pos(int kb, int k, int *byte, int *shift) {
  int j = k / 16, within = k % 16;
  int i = within / 2, odd = within % 2;
  int bit = (odd ? 16 : 0) + 2 * i;
  *byte = 8 * (kb % 2) + 4 * j + bit / 8;
  *shift = bit % 8;
}

int mnbo_pack(int N, int K, int bits, const uint8_t *codes, const uint16_t *scales,
              const uint8_t *zp, uint8_t *wq, uint16_t *sc, uint8_t *zpp) {
  long wqb, scb, zpb;
  if (mnbo_packed_sizes(N, K, bits, zp != NULL, &wqb, &scb, &zpb)) return -1;
  int NG = (N + GROUP - 1) / GROUP, KB = K / BLK, C = bits / 4, KB2 = (KB + 1) / 2;
  memset(wq, 0, (size_t)wqb);
  memset(sc, 0, (size_t)scb);
  if (zp && zpp) memset(zpp, 0, (size_t)zpb);
  for (int g = 0; g < NG; ++g)
    for (int kb = 0; kb < KB; ++kb)
      for (int r = 0; r < GROUP; ++r) {
        int n = g * GROUP + r;
        if (n >= N) continue;                        /* padded rows stay zero */
        long tile = (long)g * KB + kb;
        for (int kk = 0; kk < BLK; ++kk) {
          uint8_t q = codes[(long)n * K + kb * BLK + kk];
          if (bits == 2) {
            int byte, shift;
            crumb_pos(kb, kk, &byte, &shift);
            wq[(((long)g * KB2 + kb / 2) * GROUP + r) * 16 + byte] |= (uint8_t)((q & 3) << shift);
          } else if (bits == 4) {
            int byte, shift;
            nib_pos(kk, &byte, &shift);
            wq[((tile * C + 0) * GROUP + r) * 16 + byte] |= (uint8_t)((q & 0xf) << shift);
          } else {
            int c = kk / 16, b = kk % 16;
            wq[((tile * C + c) * GROUP + r) * 16 + b] = q;
          }
        }
        sc[tile * GROUP + r] = scales[(long)n * KB + kb];
        if (zp && zpp) {
          uint8_t z = zp[(long)n * KB + kb];
          if (bits == 2) zpp[tile * 16 + r / 4] |= (uint8_t)((z & 3) << (2 * (r % 4)));
          else if (bits == 4) zpp[tile * 32 + r / 2] |= (uint8_t)((z & 0xf) << (4 * (r % 2)));
          else zpp[tile * 64 + r] = z;
        }
      }
  return 0;
}

/*
 * Packing from the DequantizeLinear layout: codes [K, N], scales and zero points [K/32, N]
 * (blocks along K, the weight's first axis), as DequantizeLinear -> MatMul holds them.
 * The PR #33800 page ("Fuse DQ->MatMulNBits ...", Description) fuses that pair into
 * MatMulNBits by writing new, transposed initializers; here: transpose to [N, K] and
 * [N, K/32], then pack as above.
 */
int mnbo_pack_kn(int N, int K, int bits, const uint8_t *codes_kn, const uint16_t *scales_kn,
                 const uint8_t *zp_kn, uint8_t *wq, uint16_t *sc, uint8_t *zpp) {
  if (N < 0 || K < 0 || K % BLK || !bits_ok(bits)) return -1;
  int KB = K / BLK;
  uint8_t *codes = malloc((size_t)N * K + 1);
  uint16_t *scales = malloc(((size_t)N * KB + 1) * sizeof(uint16_t));
  uint8_t *zp = zp_kn ? malloc((size_t)N * KB + 1) : NULL;
  if (!codes || !scales || (zp_kn && !zp)) {
    free(codes);
    free(scales);
    free(zp);
    return -1;
  }
  for (int k = 0; k < K; ++k)
    for (int n = 0; n < N; ++n) codes[(long)n * K + k] = codes_kn[(long)k * N + n];
  for (int kb = 0; kb < KB; ++kb)
    for (int n = 0; n < N; ++n) {
#if MNBO_MUTATION == 12
      scales[(long)n * KB + kb] = scales_kn[(long)n * KB + kb];   /* planted: scales not transposed */
#else
      scales[(long)n * KB + kb] = scales_kn[(long)kb * N + n];
#endif
      if (zp) zp[(long)n * KB + kb] = zp_kn[(long)kb * N + n];
    }
  int rc = mnbo_pack(N, K, bits, codes, scales, zp, wq, sc, zpp);
  free(codes);
  free(scales);
  free(zp);
  return rc;
}

int mnbo_unpack(int N, int K, int bits, const uint8_t *wq, const uint16_t *sc, const uint8_t *zpp,
                uint8_t *codes, uint16_t *scales, uint8_t *zp) {
  if (N < 0 || K < 0 || K % BLK || !bits_ok(bits)) return -1;
  int KB = K / BLK, C = bits / 4, KB2 = (KB + 1) / 2;
  for (int n = 0; n < N; ++n) {
    int g = n / GROUP, r = n % GROUP;
    for (int kb = 0; kb < KB; ++kb) {
      long tile = (long)g * KB + kb;
      for (int kk = 0; kk < BLK; ++kk) {
        uint8_t q;
        if (bits == 2) {
          int byte, shift;
          crumb_pos(kb, kk, &byte, &shift);
          q = (wq[(((long)g * KB2 + kb / 2) * GROUP + r) * 16 + byte] >> shift) & 3;
        } else if (bits == 4) {
          int byte, shift;
          nib_pos(kk, &byte, &shift);
          q = (wq[((tile * C + 0) * GROUP + r) * 16 + byte] >> shift) & 0xf;
        } else {
          q = wq[((tile * C + kk / 16) * GROUP + r) * 16 + kk % 16];
        }
        codes[(long)n * K + kb * BLK + kk] = q;
      }
      scales[(long)n * KB + kb] = sc[tile * GROUP + r];
      if (zp && zpp) {
        if (bits == 2) zp[(long)n * KB + kb] = (zpp[tile * 16 + r / 4] >> (2 * (r % 4))) & 3;
        else if (bits == 4) zp[(long)n * KB + kb] = (zpp[tile * 32 + r / 2] >> (4 * (r % 2))) & 0xf;
        else zp[(long)n * KB + kb] = zpp[tile * 64 + r];
      }
    }
  }
  return 0;
}
