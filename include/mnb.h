/*
 * mnb.h -- C ABI of libmnb: MatMulNBits with an optional fused rank-32 LoRA term, for one
 * AMD Instinct MI355X (gfx950).
 *
 *   Y[M,N] = X[M,K] . deq(W)^T  +  (X . A) . B
 *   deq(W)[n,k] = (q[n,k] - z[n,k/32]) * s[n,k/32]
 *
 * The operation is the one described on the onnxruntime pull-request pages
 * "[WebGPU] Fuse rank-32 quantized LoRA with MatMulNBits" (PR #33370: commit list and
 * Description -- INT4 block-32 base weights, replaceable rank-32 FP16 or block-32 INT8
 * adapters, base + (X.A).B, empty adapters run the base projection only) and
 * "Fuse DQ->MatMulNBits for shared initializers and skip outer-scope weights" (PR #33800:
 * Description -- MatMulNBits equals DequantizeLinear followed by MatMul; 8-bit weights with
 * block scales and uint8 zero points for a tied lm_head).  Both pages run MatMulNBits with
 * 2-, 4- and 8-bit weights (PR #33370's file list and its split-out empty-weights change test
 * 2/4/8-bit cases); all three widths are supported here.
 *
 * Conventions for every call:
 *  - fp16 tensors are IEEE binary16 bit patterns, passed as (const) void *.
 *  - Tensor pointers are DEVICE pointers unless the argument says "host".
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued on it and
 *    never synchronised by the library; device faults surface at the caller's next
 *    synchronisation, as for any HIP call.
 *  - The caller owns every buffer.  The library allocates no device memory and keeps no
 *    per-call state, except the counters inside the caller's workspace (see
 *    mnb_workspace_bytes).
 *  - Arguments are validated before anything is enqueued; an invalid call returns a
 *    status and has no effect.
 *  - Tensor pointers must be 16-byte aligned (MNB_ERR_MISALIGNED otherwise).
 *  - Dimensions are int; the library rejects negative values (MNB_ERR_INVALID_ARG).
 */
#ifndef MNB_H
#define MNB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Unsupported settings return errors rather than failing on the device, as
 * the PR #33370 page's empty-weight change does for malformed shapes and the PagedAttention
 * pages do with their not-implemented statuses. */
enum {
  MNB_OK = 0,
  MNB_ERR_INVALID_ARG = 1,  /* negative size, NULL required pointer, bad enum */
  MNB_ERR_UNSUPPORTED = 2,  /* bits not 2/4/8, block not 32, K % 32 != 0, K >= 2^25, rank not 0/32,
                               or a launch grid past INT_MAX: ceil(M/64) * ceil(N/128) * 16 or
                               ceil(M/32) * ceil(K/256) */
  MNB_ERR_MISALIGNED = 3,   /* a tensor pointer is not 16-byte aligned */
  MNB_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than mnb_workspace_bytes() */
  MNB_ERR_ALIAS = 5,        /* Y overlaps an input or the workspace */
  MNB_ERR_HIP = 6,          /* a HIP runtime call failed (no device, launch failure) */
  MNB_ERR_HANDOFF = 7,      /* mnb_workspace_error: an in-pass T handoff gave up (outputs NaN) */
  MNB_ERR_TOO_LARGE = 8     /* mnb_matmul_noalloc: workspace need exceeds MNB_NOALLOC_SCRATCH_BYTES */
};

/* Adapter kinds (PR #33370: FP16 rank-32 adapters; block-32 INT8 adapters). */
enum { MNB_ADAPTER_NONE = 0, MNB_ADAPTER_F16 = 1, MNB_ADAPTER_Q8 = 2 };

/* Path override (PR #33370 keeps explicit fuse_down / fuse_up overrides so that the two
 * can be compared; here the override names the kernel family). */
enum { MNB_PATH_AUTO = 0, MNB_PATH_GEMV = 1, MNB_PATH_GEMM = 2 };

/* Option flags. */
enum {
  /* Decode (GEMV, M == 1) with an adapter normally computes T = X.A inside the same launch
   * as the base product.  This flag computes T in a separate launch first (two launches,
   * the structure of the pages' fuse_down), for comparison. */
  MNB_FLAG_T_SEPARATE = 1,
  /* Accuracy level 4: the base product takes int8 activations, quantized per row and per
   * block of 32 along K (amax = max |x|, q = rint(x * (127 / amax)) clamped to +-127,
   * scale amax / 127, FP32); the LoRA term keeps the FP16 X (PR #33370 commit list:
   * int8-quantized activations for the base product while T uses the unquantized FP16 X;
   * PR #33800 Description: the lm_head at the default accuracy level 4).  T comes from the
   * projection launch when there is an adapter.  Up to 16 rows (or with MNB_PATH_GEMV) the
   * GEMV family runs integer dot products on the codes (requires K <= 16384, else
   * MNB_ERR_UNSUPPORTED); above 16 rows (or with MNB_PATH_GEMM) a pre-pass writes
   * q * sx rounded to fp16 into the workspace and the MFMA GEMM multiplies it. */
  MNB_FLAG_ACC4 = 2,
  /* Test hook for the failure path of the decode's in-pass T handoff: the row workgroups
   * give up on T without waiting, exactly as when their bounded wait (about 2^22 polls)
   * expires, so the call's outputs are NaN and the workspace's error word is set (see
   * mnb_workspace_error).  Only the in-pass decode reads it; never set it for real work. */
  MNB_FLAG_FAIL_HANDOFF = 4
};

/*
 * A LoRA adapter, replaceable per call (PR #33370 Description: adapters remain replaceable;
 * base weights are unchanged).  The adapter is EMPTY -- the call computes the base
 * projection only -- when the pointer to this struct is NULL, kind == MNB_ADAPTER_NONE,
 * rank == 0, A == NULL or B == NULL (PR #33370 commit list: empty adapters execute only the
 * base projection; zero-sized adapter defaults).  Otherwise rank must be 32.
 *
 *   kind F16: A      fp16 [K, 32] row-major (rank index fastest)
 *             B      fp16 [32, N] row-major (column index fastest)
 *             A_scales, B_scales unused
 *   kind Q8 : A      int8 [K, 32] row-major,  A_scales fp16 [K/32, 32]
 *             B      int8 [32, N] row-major,  B_scales fp16 [1, N]
 *             a[k,r] = A[k,r] * A_scales[k/32, r];  b[r,n] = B[r,n] * B_scales[r/32, n]
 *             (symmetric int8 values, one fp16 scale per block of 32 along each factor's
 *             contraction axis: the "rank-32 block-32 INT8 adapters" of PR #33370)
 */
typedef struct mnb_adapter {
  int kind;
  int rank;
  const void *A;
  const void *A_scales;
  const void *B;
  const void *B_scales;
} mnb_adapter;

typedef struct mnb_options {
  int path;   /* MNB_PATH_* */
  int flags;  /* MNB_FLAG_* */
} mnb_options;

/*
 * Sizes in bytes of the packed weight buffers for an N x K weight (host only, no device
 * call).  block must be 32; bits 2, 4 or 8; has_zp selects whether a zero-point buffer
 * exists.  No page defines this call or the byte layout: the pages fix only the content (2-,
 * 4- or 8-bit codes in blocks of 32 along K, an fp16 scale and an optional zero point per
 * block).  Layout (this library's own): rows grouped by 64 (padded), K in blocks of 32:
 *   wq: ceil(N/64) * CC * 64 * 16 bytes, CC = 16-byte chunks per row = (K/32) * bits/4
 *       for 4 and 8 bits, ceil((K/32) / 2) for 2 bits (two blocks per chunk)
 *   sc: ceil(N/64) * (K/32) * 64 * 2 bytes
 *   zp: ceil(N/64) * (K/32) * 64 * bits/8 bytes, or 0 without zero points
 */
int mnb_packed_sizes(int N, int K, int bits, int block, int has_zp,
                     size_t *wq_bytes, size_t *sc_bytes, size_t *zp_bytes);

/*
 * Pack an already-quantized weight into the device layout (the role of the offline
 * "transposed initializers" of PR #33800's TransposeDQWeightsForMatMulNBits; here the input
 * is already [N, K]).
 *   codes  uint8 [N, K], one code per byte, value < 2^bits (higher bits are ignored)
 *   scales fp16  [N, K/32]
 *   zp     uint8 [N, K/32] or NULL (then no zero-point buffer is written and the default
 *          zero point 2^(bits-1) applies at matmul time)
 *   wq, sc, zpp  outputs sized by mnb_packed_sizes (zpp ignored when zp is NULL)
 * Rows beyond N in the last 64-row group are written as code 0, scale 0, zero point 0, so
 * they contribute 0.  Deterministic: packing the same input twice gives identical bytes.
 */
int mnb_pack(const uint8_t *codes, const void *scales, const uint8_t *zp, int N, int K,
             int bits, int block, void *wq, void *sc, void *zpp, void *stream);

/*
 * mnb_pack from the DequantizeLinear layout that a DequantizeLinear -> MatMul pair holds:
 * the weight's first axis is K and the blocks of 32 run along it.  This is the offline
 * transposition of PR #33800's TransposeDQWeightsForMatMulNBits ("Fuse DQ->MatMulNBits for
 * shared initializers and skip outer-scope weights", Description: the fusion reads the
 * original initializers and adds transposed ones), done on the device.
 *   codes_kn   uint8 [K, N], one code per byte, value < 2^bits
 *   scales_kn  fp16  [K/32, N]
 *   zp_kn      uint8 [K/32, N] or NULL (default zero point 2^(bits-1))
 *   wq, sc, zpp, stream, status codes: as mnb_pack; the output bytes are identical to
 *   mnb_pack of the transposed tensors.  All pointers 16-byte aligned.
 */
int mnb_pack_kn(const uint8_t *codes_kn, const void *scales_kn, const uint8_t *zp_kn, int N,
                int K, int bits, int block, void *wq, void *sc, void *zpp, void *stream);

/* Inverse of mnb_pack (for round-trip checks).  zp may be NULL iff zpp is NULL.  No page
 * defines it: it inverts this library's own packed layout (see mnb_packed_sizes). */
int mnb_unpack(const void *wq, const void *sc, const void *zpp, int N, int K, int bits,
               int block, uint8_t *codes, void *scales, uint8_t *zp, void *stream);

/*
 * Workspace bytes needed by mnb_matmul / mnb_matmul_ex for these sizes, for any path, any
 * adapter kind and any flags (host only).  No page defines a workspace: it is this library's own
 * scratch, passed in by the caller so that the library allocates nothing.  Returns 0 for
 * M or N <= 0 and for sizes every call rejects (K % 32 != 0, K >= 2^25, grids past INT_MAX).  The workspace holds partial sums (among them the prefill
 * GEMM's FP32 partial outputs when it splits K over several workgroups per output tile),
 * the LoRA down-projection T, accuracy level 4's block-quantized X for the GEMM path
 * (fp16 [M, K]) and a few counters.  It must be ZERO-FILLED before its first use; every call that
 * completes leaves its counters at zero again, so one workspace can be reused by
 * consecutive calls on one stream.  Calls that overlap in time must not share a workspace.
 */
size_t mnb_workspace_bytes(int M, int N, int K, int bits, int rank);

/*
 * Reports and clears the workspace's sticky error word.  The decode's in-pass T handoff
 * (M == 1 with an adapter, one launch) bounds every wait; when a row workgroup's wait
 * expires it writes NaN for its outputs and sets this word instead of hanging.  Waits for
 * `stream` (so it is not for use under graph capture), then reads and clears the word.
 * Returns MNB_OK, MNB_ERR_HANDOFF if the word was set since the last query,
 * MNB_ERR_INVALID_ARG for a NULL workspace, or MNB_ERR_HIP.
 */
int mnb_workspace_error(void *workspace, void *stream);

/*
 * Y[M,N] = X . deq(W)^T (+ (X.A).B), fp16 output rounded to nearest even once, from FP32
 * accumulation.
 *   X      fp16 [M, K] row-major
 *   wq, sc, zpp   packed by mnb_pack (zpp NULL: default zero point 2^(bits-1), i.e. 2 for
 *                 2-bit, 8 for 4-bit, 128 for 8-bit)
 *   ad     adapter or NULL (see mnb_adapter for when it counts as empty)
 *   Y      fp16 [M, N] row-major; must not overlap X, wq, sc, zpp, the adapter or the
 *          workspace (MNB_ERR_ALIAS)
 *   bits 2, 4 or 8, block 32, K % 32 == 0, K < 2^25
 *   workspace, ws_bytes   see mnb_workspace_bytes
 * M == 0 or N == 0: nothing is enqueued, MNB_OK.  K == 0: Y is filled with zeros.
 * Path (PR #33370 commit list, auto mode by the row count M): M == 1 runs the decode GEMV
 * with T computed in the same launch; 2 <= M <= 16 the T projection, then a GEMV that
 * streams the weights once for all rows and multiplies them with the rows on the matrix
 * cores; M > 16 the T projection, then the MFMA GEMM with the LoRA term in its epilogue.
 */
int mnb_matmul(const void *X, const void *wq, const void *sc, const void *zpp,
               const mnb_adapter *ad, void *Y, int M, int N, int K, int bits, int block,
               void *workspace, size_t ws_bytes, void *stream);

/* mnb_matmul with options (opt NULL = defaults: automatic path, no flags). */
int mnb_matmul_ex(const void *X, const void *wq, const void *sc, const void *zpp,
                  const mnb_adapter *ad, void *Y, int M, int N, int K, int bits, int block,
                  void *workspace, size_t ws_bytes, void *stream, const mnb_options *opt);

/*
 * mnb_matmul_ex plus MatMulNBits' optional broadcast bias: Y[m,n] = ... + bias[n], added in
 * FP32 before the single rounding.  bias: fp16 [N] on the device, 16-byte aligned, or NULL
 * (then identical to mnb_matmul_ex); it must not overlap Y (MNB_ERR_ALIAS).  With K == 0
 * (empty packed weights) Y is the broadcast bias, or zeros without one (the PR #33370
 * page, commit list: empty packed weights keep the logical output shape and give zeros or
 * the broadcast bias).
 */
int mnb_matmul_bias(const void *X, const void *wq, const void *sc, const void *zpp,
                    const mnb_adapter *ad, const void *bias, void *Y, int M, int N, int K,
                    int bits, int block, void *workspace, size_t ws_bytes, void *stream,
                    const mnb_options *opt);

/*
 * Describe, without any device call, the kernels mnb_matmul_ex would launch for these
 * arguments (host only): writes a NUL-terminated text such as
 * "gemv_b4_zpdef_f16_inpass grid=256x1 split=2" into buf (at most buf_len bytes).
 * has_adapter_kind is the effective adapter kind (0 when empty).  Returns a status.
 */
int mnb_describe_route(int M, int N, int K, int bits, int has_zp, int has_adapter_kind,
                       const mnb_options *opt, char *buf, size_t buf_len);

/*
 * mnb_matmul_bias without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The call allocates nothing (no hipMalloc, no hipFree, no allocating library
 * routine); its workspace is a static device array of MNB_NOALLOC_SCRATCH_BYTES inside the
 * library, one copy per device, held from the library's load until the process ends.
 *   - Arguments and results as mnb_matmul_bias (opt may be NULL).
 *   - A call whose workspace (mnb_workspace_bytes) would exceed the array returns
 *     MNB_ERR_TOO_LARGE and enqueues nothing; use mnb_matmul_bias with a caller workspace.
 *   - The first call on a device looks the array up and zeroes its counters with a kernel
 *     on `stream` (no memset), ahead of its own kernels.
 *   - Every call on a device shares that device's array, which keeps the last call's
 *     contents: calls on one device that overlap in time (several streams, threads or
 *     concurrently replayed graphs) race and give wrong results; consecutive calls on one
 *     stream are fine.
 *   - The in-pass T handoff's error word lives in the array and is not reported; a handoff
 *     that gives up still writes NaN outputs.
 */
#define MNB_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int mnb_matmul_noalloc(const void *X, const void *wq, const void *sc, const void *zpp,
                       const mnb_adapter *ad, const void *bias, void *Y, int M, int N, int K,
                       int bits, int block, void *stream, const mnb_options *opt);

/* Static text for a status code. */
const char *mnb_status_string(int status);

/* ABI version (major * 100 + minor): 101 adds mnb_matmul_bias, 102 mnb_pack_kn, 103
 * mnb_workspace_error and MNB_FLAG_FAIL_HANDOFF, 104 mnb_matmul_noalloc. */
int mnb_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MNB_H */
