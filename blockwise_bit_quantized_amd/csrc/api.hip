// api.hip -- the exported C ABI of libmnb (declared in include/mnb.h): argument
// validation, the M-based dispatcher, workspace layout and kernel launches.
//
// Dispatch (onnxruntime PR #33370 "[WebGPU] Fuse rank-32 quantized LoRA with
// MatMulNBits", commit list: the automatic mode selects the prefill path for M > 1 and the
// decode path for M == 1 on each invocation, from X's row count; a one-token prompt uses
// the decode path; explicit overrides are kept for comparisons).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <climits>
#include <mutex>

#include "common.h"
#include "mnb.h"

using namespace mnb;

// Scratch of mnb_matmul_noalloc: a workspace inside the library, for callers that cannot
// allocate.  Each device that loads the library holds its own copy until the process ends.
// Host code never uses this name as an address: the per-device address comes from
// hipGetSymbolAddress (scratch_for).
static __device__ __align__(256) unsigned char scratch[MNB_NOALLOC_SCRATCH_BYTES];

namespace {

// Zero the control area's counters (every word but the call epoch, which must only grow:
// the in-pass T words left by earlier calls carry earlier tags) -- a kernel, not a memset,
// so that a graph capturing the first call replays correctly.
__global__ void scratch_init_kernel(int *ctrl) {
  const int n = (int)(kCtrlBytes / sizeof(int));
  for (int i = 1 + (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += (int)(gridDim.x * blockDim.x))
    ctrl[i] = 0;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device (guarded by g_scratch_mu)

// The scratch address for the device of `s`: looked up once per device, with that device
// current, and its counters zeroed by a kernel on `s` before the first call uses it.
int scratch_for(hipStream_t s, void **out) {
  int dev = 0;
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return MNB_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MNB_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return MNB_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MNB_ERR_HIP;
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess && p) {
      hipLaunchKernelGGL(scratch_init_kernel, dim3(8), dim3(256), 0, s, static_cast<int *>(p));
      e = hipGetLastError();
    }
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return MNB_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MNB_OK;
}

enum { LORA_NONE = 0, LORA_F16 = 1, LORA_Q8 = 2 };

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }
// ceil(a / b) for a >= 0, b >= 1 (64-bit sum: a may be INT_MAX)
int cdiv(int a, int b) { return (int)(((long)a + b - 1) / b); }

// ---- plan -------------------------------------------------------------------------------

constexpr int kTSliceRows = 256;  // in-pass T: K rows per slice workgroup

// Workspace: a fixed control area first (its offsets depend on nothing, so a zeroed
// workspace stays valid for calls of any shape), then data regions that need no
// initialisation.
struct WsLayout {
  size_t ctrl, tinpass, tproj, tfinal, xq, ypart, total;
  int gt, tparts, tmt, splits, tsplits, tail0;
};

WsLayout ws_layout(int M, int N, int K, int rank) {
  WsLayout w{};
  w.gt = cdiv(K, kTSliceRows);
  w.tparts = std::max(1, tproj_parts(M, K));
  w.tmt = cdiv(M, 32);
  size_t off = align_up(kCtrlBytes);
  w.ctrl = 0;
  w.tinpass = off;
  if (rank) off += align_up((size_t)kTReplicas * w.gt * kRank * sizeof(unsigned long long));
  w.tproj = off;
  if (rank) off += align_up((size_t)w.tparts * M * kRank * sizeof(float));
  w.tfinal = off;
  if (rank) off += align_up((size_t)M * kRank * sizeof(float));
  // accuracy level 4 on the GEMM path: the block-quantized X, fp16 [M, K]
  w.xq = off;
  off += align_up((size_t)M * K * 2);
  // prefill GEMM with K split into ranges: FP32 partial outputs [splits, M, N]; or with
  // only the last round's tiles split: their partials [tsplits, tail tiles, bm, 128]
  w.splits = gemm_splits(M, N, K);
  w.tsplits = gemm_tail_splits(M, N, K, &w.tail0);
  w.ypart = off;
  if (w.splits > 1) off += align_up((size_t)w.splits * M * N * sizeof(float));
  if (w.tsplits > 1) {
    const int bm = gemm_bm(M, N);
    const size_t ntail = (size_t)cdiv(M, bm) * cdiv(N, 128) - w.tail0;
    off += align_up((size_t)w.tsplits * ntail * bm * 128 * sizeof(float));
  }
  w.total = off;
  return w;
}

struct Route {
  int path;      // MNB_PATH_GEMV / MNB_PATH_GEMM
  int lora;      // LORA_*
  int tmode;     // 0 in-pass, 1 precomputed by the T projection launch
  bool tproj;
  bool acc4;     // block-quantized int8 activations for the base product
};

Route route(int M, int lora, const mnb_options *opt) {
  Route r{};
  const int path = opt ? opt->path : MNB_PATH_AUTO;
  const int flags = opt ? opt->flags : 0;
  // automatic rule: the GEMV family for M <= kSmallM (M == 1 decode, the small-M
  // matrix-core variant above it: both stream the weights once), the MFMA GEMM above
  r.path = path != MNB_PATH_AUTO ? path : (M <= kSmallM ? MNB_PATH_GEMV : MNB_PATH_GEMM);
  // the small-M kernel reads all of X through one 32-bit buffer range
  static_assert((long)kRowsMaxM * kMaxK * 2 <= INT_MAX, "X of the small-M kernel exceeds one buffer range");
  r.lora = lora;
  r.tmode = 1;
  r.tproj = false;
  r.acc4 = (flags & MNB_FLAG_ACC4) != 0;
  if (r.acc4) {
    // the GEMV family (integer dot products) up to kRowsMaxM rows; above, the MFMA GEMM on
    // the block-quantized X; T always from the projection launch and the unquantized X
    if (path == MNB_PATH_AUTO) r.path = M <= kRowsMaxM ? MNB_PATH_GEMV : MNB_PATH_GEMM;
    r.tproj = lora != 0;
    return r;
  }
  if (lora) {
    if (r.path == MNB_PATH_GEMV && M == 1 && !(flags & MNB_FLAG_T_SEPARATE)) r.tmode = 0;
    else r.tproj = true;
  }
  return r;
}

// ---- validation ---------------------------------------------------------------------------

bool misaligned(const void *p) { return p && ((uintptr_t)p & 15u); }

struct Range {
  const void *p;
  size_t n;
};
bool overlap(const void *a, size_t an, Range b) {
  if (!a || !b.p || an == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + an;
}

int effective_lora(const mnb_adapter *ad) {
  if (!ad || ad->kind == MNB_ADAPTER_NONE || ad->rank == 0 || !ad->A || !ad->B) return LORA_NONE;
  return ad->kind == MNB_ADAPTER_F16 ? LORA_F16 : LORA_Q8;
}

int check_common(int M, int N, int K, int bits, int block) {
  if (M < 0 || N < 0 || K < 0) return MNB_ERR_INVALID_ARG;
  if (bits != 2 && bits != 4 && bits != 8) return MNB_ERR_UNSUPPORTED;
  if (block != kBlock || K % kBlock) return MNB_ERR_UNSUPPORTED;
  if (K >= kMaxK) return MNB_ERR_UNSUPPORTED;
  // every launch's grid fits an int: 64 x 128 GEMM tiles with up to kMaxSplits K ranges
  // each, and 32-row T-projection tiles with up to ceil(K / 256) K parts each
  if ((long)cdiv(M, 64) * cdiv(N, 128) * kMaxSplits > INT_MAX) return MNB_ERR_UNSUPPORTED;
  if ((long)cdiv(M, 32) * cdiv(K, 256) > INT_MAX) return MNB_ERR_UNSUPPORTED;
  return MNB_OK;
}

// check_ws false: every check but the workspace's (mnb_matmul_noalloc checks its own)
int validate(const void *X, const void *wq, const void *sc, const void *zpp, const mnb_adapter *ad,
             const void *bias, const void *Y, int M, int N, int K, int bits, int block, const void *ws,
             size_t ws_bytes, const mnb_options *opt, bool check_ws = true) {
  int st = check_common(M, N, K, bits, block);
  if (st) return st;
  if (opt) {
    if (opt->path < MNB_PATH_AUTO || opt->path > MNB_PATH_GEMM) return MNB_ERR_INVALID_ARG;
    if (opt->flags & ~(MNB_FLAG_T_SEPARATE | MNB_FLAG_ACC4 | MNB_FLAG_FAIL_HANDOFF)) return MNB_ERR_INVALID_ARG;
    if ((opt->flags & MNB_FLAG_ACC4) && K > kAcc4MaxK &&
        (opt->path == MNB_PATH_GEMV || (opt->path == MNB_PATH_AUTO && M <= kRowsMaxM)))
      return MNB_ERR_UNSUPPORTED;   // the GEMV family's LDS holds at most kAcc4MaxK quantized X
  }
  if (ad) {
    if (ad->kind < MNB_ADAPTER_NONE || ad->kind > MNB_ADAPTER_Q8 || ad->rank < 0) return MNB_ERR_INVALID_ARG;
  }
  const int lora = effective_lora(ad);
  if (lora && ad->rank != kRank) return MNB_ERR_UNSUPPORTED;
  if (lora == LORA_Q8 && (!ad->A_scales || !ad->B_scales)) return MNB_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return MNB_OK;
  if (!Y) return MNB_ERR_INVALID_ARG;
  if (K > 0 && (!X || !wq || !sc)) return MNB_ERR_INVALID_ARG;
  if (misaligned(X) || misaligned(wq) || misaligned(sc) || misaligned(zpp) || misaligned(Y) || misaligned(ws) ||
      misaligned(bias))
    return MNB_ERR_MISALIGNED;
  if (lora && (misaligned(ad->A) || misaligned(ad->B) || misaligned(ad->A_scales) || misaligned(ad->B_scales)))
    return MNB_ERR_MISALIGNED;
  if (K > 0 && check_ws) {
    const size_t need = mnb_workspace_bytes(M, N, K, bits, lora ? kRank : 0);
    if (need > 0 && (!ws || ws_bytes < need)) return MNB_ERR_WORKSPACE;
  }
  size_t wqb = 0, scb = 0, zpb = 0;
  mnb_packed_sizes(N, K, bits, block, zpp != nullptr, &wqb, &scb, &zpb);
  const size_t ybytes = (size_t)M * N * 2;
  Range ins[] = {{X, (size_t)M * K * 2}, {wq, wqb}, {sc, scb}, {zpp, zpb}, {ws, ws_bytes},
                 {lora ? ad->A : nullptr, (size_t)K * kRank * (lora == LORA_F16 ? 2 : 1)},
                 {lora ? ad->B : nullptr, (size_t)kRank * N * (lora == LORA_F16 ? 2 : 1)},
                 {lora == LORA_Q8 ? ad->A_scales : nullptr, (size_t)(K / kBlock) * kRank * 2},
                 {lora == LORA_Q8 ? ad->B_scales : nullptr, (size_t)N * 2},
                 {bias, (size_t)N * 2}};
  for (const Range &r : ins)
    if (overlap(Y, ybytes, r)) return MNB_ERR_ALIAS;
  return MNB_OK;
}

void describe(char *buf, size_t len, int M, int N, int K, int bits, int has_zp, const Route &r) {
  const WsLayout w = ws_layout(M, N, K, r.lora ? kRank : 0);
  const char *ln = r.lora == LORA_NONE ? "none" : (r.lora == LORA_F16 ? "f16" : "q8");
  char tp[160] = "";
  if (r.tproj) snprintf(tp, sizeof tp, "tproj_%s grid=%d parts=%d; ", ln, w.tmt * w.tparts, w.tparts);
  if (r.acc4 && r.path == MNB_PATH_GEMM) {
    // block quantization of X, then the GEMM below on it
    const size_t n = strlen(tp);
    snprintf(tp + n, sizeof tp - n, "acc4_xquant grid=%ld; ", ((long)M * (K / kBlock) * 4 + 255) / 256);
  }
  if (r.acc4 && r.path == MNB_PATH_GEMV) {
    const int NG = cdiv(N, kGroup);
    const int q = gemv_rows_split(N, false);
    const int mr = acc4_rows_mr(M, N, K);
    snprintf(buf, len, "%sgemv_acc4_b%d_zp%s_%s grid=%dx%d rows=%d q=%d mr=%d", tp, bits, has_zp ? "x" : "def", ln,
             NG * q, cdiv(M, mr), kGroup / q, q, mr);
  } else if (r.path == MNB_PATH_GEMV && M > 1 && M <= kRowsMaxM) {
    if (gemv_mfma_wide(M, N, K, bits))
      snprintf(buf, len, "%sgemv_mfma_wide_b%d_zp%s_%s grid=%d rows=64 mr=%d", tp, bits, has_zp ? "x" : "def", ln,
               cdiv(N, kGroup), M <= 8 ? 8 : 16);
    else
      snprintf(buf, len, "%sgemv_mfma_b%d_zp%s_%s grid=%d rows=16 mr=%d", tp, bits, has_zp ? "x" : "def", ln,
               cdiv(N, kGroup) * 4, M <= 8 ? 8 : 16);
  } else if (r.path == MNB_PATH_GEMV) {
    const int NG = cdiv(N, kGroup);
    const int extra = (r.lora && r.tmode == 0) ? w.gt : 0;
    const int q = gemv_rows_split(N, extra > 0);
    snprintf(buf, len, "%sgemv_b%d_zp%s_%s_%s grid=%dx%d rows=%d q=%d gt=%d", tp, bits, has_zp ? "x" : "def", ln,
             r.lora ? (r.tmode == 0 ? "inpass" : "tprecomp") : "base", NG * q + extra, M, kGroup / q, q, extra);
  } else {
    const int bm = gemm_bm(M, N);
    const int ntiles = cdiv(M, bm) * cdiv(N, 128);   // fits: check_common bounds the grid
    if (w.tsplits > 1)
      snprintf(buf, len, "%sgemm_b%d_zp%s_%s grid=%d tile=%dx128x64 splits=1 tail=%dx%d", tp, bits,
               has_zp ? "x" : "def", ln, w.tail0 + (ntiles - w.tail0) * w.tsplits, bm, ntiles - w.tail0, w.tsplits);
    else
      snprintf(buf, len, "%sgemm_b%d_zp%s_%s grid=%d tile=%dx128x64 splits=%d", tp, bits, has_zp ? "x" : "def", ln,
               ntiles * w.splits, bm, w.splits);
  }
}

// both packers: kn selects the [K, N] (DequantizeLinear) source layout
int pack_any(const uint8_t *codes, const void *scales, const uint8_t *zp, int N, int K, int bits, int block,
             void *wq, void *sc, void *zpp, void *stream, bool kn) {
  int st = check_common(0, N, K, bits, block);
  if (st) return st;
  if (N == 0 || K == 0) return MNB_OK;
  if (!codes || !scales || !wq || !sc || (zp && !zpp)) return MNB_ERR_INVALID_ARG;
  if (misaligned(codes) || misaligned(scales) || misaligned(zp) || misaligned(wq) || misaligned(sc) ||
      (zp && misaligned(zpp)))
    return MNB_ERR_MISALIGNED;
  PackParams p{codes, static_cast<const uint16_t *>(scales), zp, static_cast<uint8_t *>(wq),
               static_cast<uint16_t *>(sc), static_cast<uint8_t *>(zpp), N, K, cdiv(N, kGroup), K / kBlock};
  if (!zp) p.zpp = nullptr;
  return launch_pack(bits, kn, p, static_cast<hipStream_t>(stream)) == hipSuccess ? MNB_OK : MNB_ERR_HIP;
}

bool log_enabled() {
  static int v = -1;
  if (v < 0) {
    const char *e = getenv("MNB_LOG");
    v = (e && *e && *e != '0') ? 1 : 0;
  }
  return v == 1;
}

}  // namespace

extern "C" {

int mnb_version(void) { return 104; }

const char *mnb_status_string(int status) {
  switch (status) {
    case MNB_OK: return "MNB_OK";
    case MNB_ERR_INVALID_ARG: return "MNB_ERR_INVALID_ARG: invalid argument";
    case MNB_ERR_UNSUPPORTED: return "MNB_ERR_UNSUPPORTED: unsupported setting (bits 2/4/8, block 32, K%32==0, rank 0/32)";
    case MNB_ERR_MISALIGNED: return "MNB_ERR_MISALIGNED: tensor pointer not 16-byte aligned";
    case MNB_ERR_WORKSPACE: return "MNB_ERR_WORKSPACE: workspace missing or too small";
    case MNB_ERR_ALIAS: return "MNB_ERR_ALIAS: output overlaps an input or the workspace";
    case MNB_ERR_HIP: return "MNB_ERR_HIP: HIP runtime error";
    case MNB_ERR_HANDOFF: return "MNB_ERR_HANDOFF: an in-pass T handoff gave up, its outputs are NaN";
    case MNB_ERR_TOO_LARGE:
      return "MNB_ERR_TOO_LARGE: the call needs more workspace than mnb_matmul_noalloc's static scratch "
             "(MNB_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown mnb status";
  }
}

int mnb_packed_sizes(int N, int K, int bits, int block, int has_zp, size_t *wq_bytes, size_t *sc_bytes,
                     size_t *zp_bytes) {
  const int st = check_common(0, N, K, bits, block);
  if (st) return st;
  const size_t tiles = (size_t)cdiv(N, kGroup) * (K / kBlock);
  if (wq_bytes) *wq_bytes = (size_t)cdiv(N, kGroup) * chunk_cols(bits, K / kBlock) * kGroup * 16;
  if (sc_bytes) *sc_bytes = tiles * kGroup * 2;
  if (zp_bytes) *zp_bytes = has_zp ? tiles * kGroup * bits / 8 : 0;
  return MNB_OK;
}

size_t mnb_workspace_bytes(int M, int N, int K, int bits, int rank) {
  (void)bits;
  if (M <= 0 || N <= 0 || K < 0) return 0;
  if (check_common(M, N, K, 4, kBlock) != MNB_OK) return 0;   // no call accepts these sizes
  return ws_layout(M, N, K, rank ? kRank : 0).total;
}

int mnb_workspace_error(void *workspace, void *stream) {
  if (!workspace) return MNB_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int *word = static_cast<int *>(workspace) + CTRL_ERROR;   // the control area starts the workspace
  int v = 0;
  const int zero = 0;
  if (hipMemcpyAsync(&v, word, sizeof v, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MNB_ERR_HIP;
  if (v == 0) return MNB_OK;
  if (hipMemcpyAsync(word, &zero, sizeof zero, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MNB_ERR_HIP;
  return MNB_ERR_HANDOFF;
}

int mnb_pack(const uint8_t *codes, const void *scales, const uint8_t *zp, int N, int K, int bits, int block,
             void *wq, void *sc, void *zpp, void *stream) {
  return pack_any(codes, scales, zp, N, K, bits, block, wq, sc, zpp, stream, false);
}

int mnb_pack_kn(const uint8_t *codes_kn, const void *scales_kn, const uint8_t *zp_kn, int N, int K, int bits,
                int block, void *wq, void *sc, void *zpp, void *stream) {
  return pack_any(codes_kn, scales_kn, zp_kn, N, K, bits, block, wq, sc, zpp, stream, true);
}


int mnb_unpack(const void *wq, const void *sc, const void *zpp, int N, int K, int bits, int block,
               uint8_t *codes, void *scales, uint8_t *zp, void *stream) {
  int st = check_common(0, N, K, bits, block);
  if (st) return st;
  if ((zp == nullptr) != (zpp == nullptr)) return MNB_ERR_INVALID_ARG;
  if (N == 0 || K == 0) return MNB_OK;
  if (!wq || !sc || !codes || !scales) return MNB_ERR_INVALID_ARG;
  if (misaligned(codes) || misaligned(scales) || misaligned(zp) || misaligned(wq) || misaligned(sc) ||
      misaligned(zpp))
    return MNB_ERR_MISALIGNED;
  PackParams p{nullptr, nullptr, static_cast<const uint8_t *>(zpp), const_cast<uint8_t *>(static_cast<const uint8_t *>(wq)),
               const_cast<uint16_t *>(static_cast<const uint16_t *>(sc)), nullptr, N, K, cdiv(N, kGroup), K / kBlock};
  return launch_unpack(bits, p, codes, static_cast<uint16_t *>(scales), zp, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? MNB_OK
             : MNB_ERR_HIP;
}

int mnb_describe_route(int M, int N, int K, int bits, int has_zp, int has_adapter_kind, const mnb_options *opt,
                       char *buf, size_t buf_len) {
  int st = check_common(M, N, K, bits, kBlock);
  if (st) return st;
  if (has_adapter_kind < 0 || has_adapter_kind > 2 || !buf || buf_len == 0) return MNB_ERR_INVALID_ARG;
  if (opt && (opt->path < 0 || opt->path > 2 ||
              (opt->flags & ~(MNB_FLAG_T_SEPARATE | MNB_FLAG_ACC4 | MNB_FLAG_FAIL_HANDOFF))))
    return MNB_ERR_INVALID_ARG;
  if (opt && (opt->flags & MNB_FLAG_ACC4) && K > kAcc4MaxK &&
      (opt->path == MNB_PATH_GEMV || (opt->path == MNB_PATH_AUTO && M <= kRowsMaxM)))
    return MNB_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) {
    snprintf(buf, buf_len, "noop");
    return MNB_OK;
  }
  if (K == 0) {
    snprintf(buf, buf_len, "fill");
    return MNB_OK;
  }
  describe(buf, buf_len, M, N, K, bits, has_zp, route(M, has_adapter_kind, opt));
  return MNB_OK;
}

int mnb_matmul_ex(const void *X, const void *wq, const void *sc, const void *zpp, const mnb_adapter *ad, void *Y,
                  int M, int N, int K, int bits, int block, void *workspace, size_t ws_bytes, void *stream,
                  const mnb_options *opt) {
  return mnb_matmul_bias(X, wq, sc, zpp, ad, nullptr, Y, M, N, K, bits, block, workspace, ws_bytes, stream, opt);
}

int mnb_matmul_bias(const void *X, const void *wq, const void *sc, const void *zpp, const mnb_adapter *ad,
                    const void *bias, void *Y, int M, int N, int K, int bits, int block, void *workspace,
                    size_t ws_bytes, void *stream, const mnb_options *opt) {
  int st = validate(X, wq, sc, zpp, ad, bias, Y, M, N, K, bits, block, workspace, ws_bytes, opt);
  if (st) return st;
  if (M == 0 || N == 0) return MNB_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t *Yh = static_cast<uint16_t *>(Y);
  const uint16_t *bh = static_cast<const uint16_t *>(bias);
  if (K == 0) return launch_fill(Yh, bh, M, N, s) == hipSuccess ? MNB_OK : MNB_ERR_HIP;

  const int lora = effective_lora(ad);
  const Route r = route(M, lora, opt);
  const WsLayout w = ws_layout(M, N, K, lora ? kRank : 0);
  char *ws = static_cast<char *>(workspace);
  const int NG = cdiv(N, kGroup), KB = K / kBlock;
  const bool has_zp = zpp != nullptr;
  if (log_enabled()) {
    char b[256];
    describe(b, sizeof b, M, N, K, bits, has_zp, r);
    fprintf(stderr, "[mnb] M=%d N=%d K=%d bits=%d: %s\n", M, N, K, bits, b);
  }

  // T projection output: FP32 partials per K-part; consumers read `tparts` parts.  For
  // 2 <= M <= 16 and K <= 2048 the parts are at most 4, which the small-M GEMV loads ahead
  // of its weight stream and adds itself; more parts are reduced by the projection
  // (per-tile arrival counter; device-coherent stores and loads, no fences).  Above 16 rows the reduction costs more than the
  // consumer's part loads it saves (measured for every M: 1024 x 4096 x 4096 49.7 -> 54.1
  // us), so the projection uses 512-k parts and the GEMM adds them (eight loads in flight,
  // then one at a time); the M == 1 GEMV adds up to 8 with its loads in flight together.
  float *tproj_out = lora ? reinterpret_cast<float *>(ws + w.tproj) : nullptr;
  int tparts = w.tparts;
  if (r.tproj) {
    const int reduce = w.tparts > 4 && w.tmt <= kTprojCounters && M > 1 && M <= kRowsMaxM;
    TprojParams tp{static_cast<const uint16_t *>(X), ad->A, static_cast<const uint16_t *>(ad->A_scales), tproj_out,
                   reinterpret_cast<float *>(ws + w.tfinal), reinterpret_cast<int *>(ws + w.ctrl),
                   M, K, w.tmt, w.tparts, reduce};
    if (launch_tproj(lora, tp, s) != hipSuccess) return MNB_ERR_HIP;
    if (reduce) {
      tproj_out = tp.tfinal;
      tparts = 1;
    }
  }

  if (r.path == MNB_PATH_GEMV) {
    GemvParams p{};
    p.X = static_cast<const uint16_t *>(X);
    p.wq = static_cast<const uint8_t *>(wq);
    p.sc = static_cast<const uint16_t *>(sc);
    p.zp = static_cast<const uint8_t *>(zpp);
    if (lora) {
      p.A = ad->A;
      p.sA = static_cast<const uint16_t *>(ad->A_scales);
      p.B = ad->B;
      p.sB = static_cast<const uint16_t *>(ad->B_scales);
    }
    p.Y = Yh;
    p.bias = bh;
    p.N = N;
    p.K = K;
    p.NG = NG;
    p.KB = KB;
    p.gt = (lora && r.tmode == 0) ? w.gt : 0;
    p.q = gemv_rows_split(N, p.gt > 0);
    p.kt = kTSliceRows;
    p.nepi = NG * p.q;
    p.spin_limit = (opt && (opt->flags & MNB_FLAG_FAIL_HANDOFF)) ? -1 : kSpinLimit;
    p.tparts = tparts;
    p.tmpad = M;
    p.ctrl = reinterpret_cast<int *>(ws + w.ctrl);
    p.tin = tproj_out;
    p.tword = reinterpret_cast<unsigned long long *>(ws + w.tinpass);
    if (r.acc4) {
      // accuracy level 4: 4 X rows per workgroup row (M > 1, K <= 4096, wide grid) or one
      // (T from the projection launch); grid rows count X rows here, the launcher groups them
      p.gt = 0;
      p.q = gemv_rows_split(N, false);
      for (int m0 = 0; m0 < M; m0 += 65535) {
        const int mc = std::min(65535, M - m0);
        GemvParams q = p;
        q.X = p.X + (size_t)m0 * K;
        q.Y = p.Y + (size_t)m0 * N;
        if (tproj_out) q.tin = tproj_out + (size_t)m0 * kRank;
        q.M = mc;
        if (launch_gemv_acc4(bits, has_zp, lora, q, NG * p.q, mc, s) != hipSuccess) return MNB_ERR_HIP;
      }
      return MNB_OK;
    }
    if (M > 1 && M <= kRowsMaxM) {
      // small M: one pass over the weights for all rows on the matrix cores (T from the
      // projection launch; X of up to 16 rows fits one 32-bit buffer range at every K)
      p.M = M;
      p.gt = 0;
      p.q = 4;
      if (launch_gemv_mfma(bits, lora, p, s) != hipSuccess) return MNB_ERR_HIP;
      return MNB_OK;
    }
    // rows in chunks that respect the grid's y limit (the in-pass T path has M == 1)
    const int kMaxY = 65535;
    for (int m0 = 0; m0 < M; m0 += kMaxY) {
      const int mc = std::min(kMaxY, M - m0);
      GemvParams q = p;
      q.X = p.X + (size_t)m0 * K;
      q.Y = p.Y + (size_t)m0 * N;
      if (tproj_out) q.tin = tproj_out + (size_t)m0 * kRank;
      q.M = mc;
      const int gx = NG * p.q + p.gt;
      if (launch_gemv(bits, has_zp, lora, r.tmode, q, gx, mc, s) != hipSuccess) return MNB_ERR_HIP;
    }
    return MNB_OK;
  }

  GemmParams g{};
  g.X = static_cast<const uint16_t *>(X);
  if (r.acc4) {
    // accuracy level 4: the GEMM multiplies the block-quantized X (T above used the X given)
    uint16_t *xq = reinterpret_cast<uint16_t *>(ws + w.xq);
    if (launch_acc4_xquant(g.X, xq, M, K, s) != hipSuccess) return MNB_ERR_HIP;
    g.X = xq;
  }
  g.wq = static_cast<const uint8_t *>(wq);
  g.sc = static_cast<const uint16_t *>(sc);
  g.zp = static_cast<const uint8_t *>(zpp);
  if (lora) {
    g.B = ad->B;
    g.sB = static_cast<const uint16_t *>(ad->B_scales);
  }
  g.tpart = tproj_out;
  g.tparts = tparts;
  g.bias = bh;
  g.Y = Yh;
  g.M = M;
  g.N = N;
  g.K = K;
  g.NG = NG;
  g.KB = KB;
  g.bm = gemm_bm(M, N);
  g.MT = cdiv(M, g.bm);
  g.NT = cdiv(N, 128);
  g.splits = w.splits;
  g.tsplits = w.tsplits;
  g.tail0 = w.tail0;
  g.ypart = reinterpret_cast<float *>(ws + w.ypart);
  return launch_gemm(bits, has_zp, lora, g, s) == hipSuccess ? MNB_OK : MNB_ERR_HIP;
}

int mnb_matmul(const void *X, const void *wq, const void *sc, const void *zpp, const mnb_adapter *ad, void *Y, int M,
               int N, int K, int bits, int block, void *workspace, size_t ws_bytes, void *stream) {
  return mnb_matmul_ex(X, wq, sc, zpp, ad, Y, M, N, K, bits, block, workspace, ws_bytes, stream, nullptr);
}

int mnb_matmul_noalloc(const void *X, const void *wq, const void *sc, const void *zpp, const mnb_adapter *ad,
                       const void *bias, void *Y, int M, int N, int K, int bits, int block, void *stream,
                       const mnb_options *opt) {
  // everything the workspace does not decide, first (no device call on an invalid call)
  int st = validate(X, wq, sc, zpp, ad, bias, Y, M, N, K, bits, block, nullptr, 0, opt, false);
  if (st) return st;
  if (M == 0 || N == 0) return MNB_OK;
  const size_t need = mnb_workspace_bytes(M, N, K, bits, effective_lora(ad) ? kRank : 0);
  if (need > MNB_NOALLOC_SCRATCH_BYTES) return MNB_ERR_TOO_LARGE;
  void *ws = nullptr;
  st = scratch_for(static_cast<hipStream_t>(stream), &ws);
  if (st) return st;
  return mnb_matmul_bias(X, wq, sc, zpp, ad, bias, Y, M, N, K, bits, block, ws, MNB_NOALLOC_SCRATCH_BYTES, stream,
                         opt);
}

}  // extern "C"
