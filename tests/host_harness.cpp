// Host-side checks of libmnb's planning and validation, for the sanitizer run
// (tests/test_sanitizers.py builds it with the library's sources compiled host-only under
// AddressSanitizer and UndefinedBehaviorSanitizer; no GPU is used):
//  - every host-only call (packed sizes, workspace bytes, route descriptions) over a sweep
//    of shapes up to the int limits, all widths, zero-point modes, adapter kinds and
//    options;
//  - every validation path of the matmul and pack calls with fake, never-dereferenced
//    pointers: each returns its status before any device call.
// Exit status 0 and "host harness: N calls" on success; a sanitizer finding aborts.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "mnb.h"

namespace {

long g_calls = 0;
int g_fail = 0;

void expect(int got, int want, const char *what) {
  ++g_calls;
  if (got != want) {
    std::fprintf(stderr, "host harness: %s returned %d, expected %d\n", what, got, want);
    ++g_fail;
  }
}

void *fake(int i) { return reinterpret_cast<void *>((uintptr_t)(i + 1) << 40); }

}  // namespace

int main() {
  const int dims[] = {0, 1, 2, 3, 4, 5, 8, 16, 17, 31, 32, 63, 64, 65, 127, 128, 129, 255, 256, 257, 896, 1000,
                      1024, 2048, 2560, 4096, 8192, 9728, 49152, 65535, 65536, 1 << 20, 1 << 24, INT_MAX / 2,
                      INT_MAX - 63, INT_MAX};
  const int ks[] = {0, 32, 64, 96, 160, 576, 896, 1024, 2048, 2560, 4096, 8192, 16384, 16416, 1 << 20,
                    (1 << 25) - 32, 1 << 25, (1 << 28) - 32, 1 << 28, INT_MAX - 31, -32};
  const int bits_list[] = {2, 4, 8, 3};
  char buf[256];

  // packed sizes: every shape, width and zero-point mode
  for (int N : dims)
    for (int K : ks)
      for (int bits : bits_list)
        for (int zp = 0; zp < 2; ++zp) {
          size_t a = 0, b = 0, c = 0;
          (void)mnb_packed_sizes(N, K, bits, 32, zp, &a, &b, &c);
          ++g_calls;
        }

  // workspace bytes and route descriptions: every row count, shape, adapter kind and option
  const mnb_options opts[] = {{MNB_PATH_AUTO, 0},
                              {MNB_PATH_GEMV, 0},
                              {MNB_PATH_GEMM, 0},
                              {MNB_PATH_GEMV, MNB_FLAG_T_SEPARATE},
                              {MNB_PATH_AUTO, MNB_FLAG_ACC4},
                              {MNB_PATH_GEMV, MNB_FLAG_ACC4 | MNB_FLAG_FAIL_HANDOFF},
                              {7, 0},
                              {MNB_PATH_AUTO, 64}};
  for (int M : dims)
    for (int N : dims)
      for (int K : ks)
        for (int bits : bits_list) {
          (void)mnb_workspace_bytes(M, N, K, bits, 32);
          (void)mnb_workspace_bytes(M, N, K, bits, 0);
          g_calls += 2;
          for (int kind = 0; kind < 3; ++kind)
            for (const mnb_options &o : opts) {
              (void)mnb_describe_route(M, N, K, bits, kind == 1, kind, &o, buf, sizeof buf);
              ++g_calls;
            }
          (void)mnb_describe_route(M, N, K, bits, 1, 0, nullptr, buf, 8);   // truncated text
          ++g_calls;
        }

  // validation of the matmul calls: each case returns before any device call
  void *X = fake(0), *WQ = fake(1), *SC = fake(2), *ZP = fake(3), *Y = fake(4), *WS = fake(5), *A = fake(6),
       *B = fake(7), *BIAS = fake(8);
  const size_t big = (size_t)1 << 34;
  mnb_adapter f16{MNB_ADAPTER_F16, 32, A, nullptr, B, nullptr};
  mnb_adapter q8_noscale{MNB_ADAPTER_Q8, 32, A, nullptr, B, nullptr};
  mnb_adapter rank16{MNB_ADAPTER_F16, 16, A, nullptr, B, nullptr};
  mnb_adapter badkind{9, 32, A, nullptr, B, nullptr};
  mnb_options bad_path{5, 0}, bad_flags{0, 1 << 10}, acc4_gemv{MNB_PATH_GEMV, MNB_FLAG_ACC4};
  for (int M : {1, 3, 64, 1024})
    for (int N : {1, 70, 4096})
      for (int K : {32, 4096}) {
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, Y, M, N, K, 3, 32, WS, big, nullptr, nullptr),
               MNB_ERR_UNSUPPORTED, "bits 3");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, Y, M, N, K, 4, 64, WS, big, nullptr, nullptr),
               MNB_ERR_UNSUPPORTED, "block 64");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, Y, M, N, K + 16, 4, 32, WS, big, nullptr, nullptr),
               MNB_ERR_UNSUPPORTED, "K % 32");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, Y, -M, N, K, 4, 32, WS, big, nullptr, nullptr),
               MNB_ERR_INVALID_ARG, "negative M");
        expect(mnb_matmul_bias(nullptr, WQ, SC, ZP, nullptr, nullptr, Y, M, N, K, 4, 32, WS, big, nullptr, nullptr),
               MNB_ERR_INVALID_ARG, "X NULL");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, (char *)Y + 8, M, N, K, 4, 32, WS, big, nullptr,
                               nullptr),
               MNB_ERR_MISALIGNED, "Y misaligned");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, Y, M, N, K, 4, 32, nullptr, 0, nullptr, nullptr),
               MNB_ERR_WORKSPACE, "no workspace");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, X, M, N, K, 4, 32, WS, big, nullptr, nullptr),
               MNB_ERR_ALIAS, "Y over X");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, Y, Y, M, N, K, 4, 32, WS, big, nullptr, nullptr),
               MNB_ERR_ALIAS, "Y over bias");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, &rank16, nullptr, Y, M, N, K, 4, 32, WS, big, nullptr, nullptr),
               MNB_ERR_UNSUPPORTED, "rank 16");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, &q8_noscale, nullptr, Y, M, N, K, 4, 32, WS, big, nullptr, nullptr),
               MNB_ERR_INVALID_ARG, "Q8 without scales");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, &badkind, nullptr, Y, M, N, K, 4, 32, WS, big, nullptr, nullptr),
               MNB_ERR_INVALID_ARG, "adapter kind");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, &f16, nullptr, B, M, N, K, 4, 32, WS, big, nullptr, nullptr),
               MNB_ERR_ALIAS, "Y over B");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, Y, M, N, K, 4, 32, WS, big, nullptr, &bad_path),
               MNB_ERR_INVALID_ARG, "path");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, Y, M, N, K, 4, 32, WS, big, nullptr, &bad_flags),
               MNB_ERR_INVALID_ARG, "flags");
        // the GEMV family's LDS holds at most 16384 quantized X values per row (the GEMM
        // path takes accuracy level 4 at any K)
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, Y, M, N, K + 16384, 4, 32, WS, big, nullptr,
                               &acc4_gemv),
               MNB_ERR_UNSUPPORTED, "ACC4 on the GEMV path past its K limit");
        expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, BIAS, Y, 0, N, K, 4, 32, WS, big, nullptr, nullptr), MNB_OK,
               "M == 0");
        expect(mnb_matmul_noalloc(X, WQ, SC, ZP, nullptr, nullptr, Y, M, N, K + 16, 4, 32, nullptr, nullptr),
               MNB_ERR_UNSUPPORTED, "noalloc K % 32");
        expect(mnb_matmul_noalloc(X, WQ, SC, ZP, nullptr, nullptr, X, M, N, K, 4, 32, nullptr, nullptr),
               MNB_ERR_ALIAS, "noalloc Y over X");
      }
  expect(mnb_matmul_noalloc(X, WQ, SC, nullptr, nullptr, nullptr, Y, 256, 12288, 16384, 4, 32, nullptr, nullptr),
         MNB_ERR_TOO_LARGE, "noalloc beyond the scratch");
  expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, Y, INT_MAX, INT_MAX, 32, 4, 32, WS, big, nullptr, nullptr),
         MNB_ERR_UNSUPPORTED, "int-limit shape: its grid does not fit an int");
  expect(mnb_matmul_bias(X, WQ, SC, ZP, nullptr, nullptr, Y, 1 << 20, 1 << 16, 4096, 4, 32, WS, 16, nullptr, nullptr),
         MNB_ERR_WORKSPACE, "large shape, small workspace");

  // packing validation
  expect(mnb_pack(static_cast<uint8_t *>(X), SC, nullptr, 64, 33, 4, 32, WQ, SC, nullptr, nullptr),
         MNB_ERR_UNSUPPORTED, "pack K % 32");
  expect(mnb_pack(nullptr, SC, nullptr, 64, 64, 4, 32, WQ, SC, nullptr, nullptr), MNB_ERR_INVALID_ARG,
         "pack codes NULL");
  expect(mnb_pack_kn(static_cast<uint8_t *>(X) + 1, SC, nullptr, 64, 64, 4, 32, WQ, SC, nullptr, nullptr),
         MNB_ERR_MISALIGNED, "pack_kn misaligned");
  expect(mnb_unpack(WQ, SC, ZP, 64, 64, 8, 32, static_cast<uint8_t *>(X), SC, nullptr, nullptr),
         MNB_ERR_INVALID_ARG, "unpack zp mismatch");
  for (int st = -1; st < 12; ++st) {
    const char *s = mnb_status_string(st);
    expect(s != nullptr && std::strlen(s) > 0, 1, "status string");
  }

  std::printf("host harness: %ld calls, %d failures\n", g_calls, g_fail);
  return g_fail ? 1 : 0;
}
