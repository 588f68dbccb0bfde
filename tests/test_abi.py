"""Host-side checks of the C ABI that need no GPU.

 - libmnb.so loads and exports every function include/mnb.h declares;
 - packed sizes agree with the oracle's independent implementation of the layout;
 - argument validation returns the documented status before any HIP call (these calls
   use fake, never-dereferenced pointer values and launch nothing);
 - the dispatcher's route description follows the automatic rule (M == 1 decode GEMV
   with in-pass T; M > 1 T projection + MFMA GEMM) and the overrides.
"""
from __future__ import annotations

import os
import re

import pytest

import oracle
from _util import ROOT, ensure_lib

mnb = ensure_lib()


def header_functions():
    text = open(os.path.join(ROOT, "include", "mnb.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mnb_[a-z_]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = header_functions()
    for n in ("mnb_pack", "mnb_pack_kn", "mnb_unpack", "mnb_matmul", "mnb_matmul_ex", "mnb_matmul_bias",
              "mnb_workspace_bytes", "mnb_packed_sizes", "mnb_status_string", "mnb_describe_route",
              "mnb_version", "mnb_workspace_error", "mnb_matmul_noalloc"):
        assert n in names


def test_every_declared_symbol_is_exported():
    for name in header_functions():
        assert hasattr(mnb.lib, name), name                      # ctypes dlsym
        assert callable(getattr(mnb, name)), name                # binding uses the same names


def test_version_and_status_strings():
    assert mnb.mnb_version() == 104
    for st in range(9):
        assert mnb.mnb_status_string(st).startswith("MNB_")
    assert "unknown" in mnb.mnb_status_string(99)


@pytest.mark.parametrize("N,K,bits,zp", [(1, 32, 4, 1), (64, 64, 8, 0), (65, 96, 4, 1), (896, 896, 4, 1),
                                          (8192, 2048, 4, 0), (49152, 576, 8, 1), (9728, 2560, 4, 0)])
def test_packed_sizes_match_oracle_layout(N, K, bits, zp):
    st, wq, sc, zpb = mnb.mnb_packed_sizes(N, K, bits, 32, zp)
    assert st == 0
    assert (wq, sc, zpb) == oracle.packed_sizes(N, K, bits, zp)


def test_packed_sizes_rejects():
    assert mnb.mnb_packed_sizes(64, 33, 4, 32, 0)[0] == mnb.MNB_ERR_UNSUPPORTED
    assert mnb.mnb_packed_sizes(64, 64, 3, 32, 0)[0] == mnb.MNB_ERR_UNSUPPORTED
    assert mnb.mnb_packed_sizes(64, 64, 4, 64, 0)[0] == mnb.MNB_ERR_UNSUPPORTED
    assert mnb.mnb_packed_sizes(64, 1 << 25, 4, 32, 0)[0] == mnb.MNB_ERR_UNSUPPORTED   # K < 2^25
    assert mnb.mnb_packed_sizes(64, (1 << 25) - 32, 4, 32, 0)[0] == mnb.MNB_OK
    assert mnb.mnb_packed_sizes(-1, 64, 4, 32, 0)[0] == mnb.MNB_ERR_INVALID_ARG


def test_workspace_bytes():
    assert mnb.mnb_workspace_bytes(0, 64, 64, 4, 32) == 0
    a = mnb.mnb_workspace_bytes(1, 8192, 2048, 4, 0)
    b = mnb.mnb_workspace_bytes(1, 8192, 2048, 4, 32)
    c = mnb.mnb_workspace_bytes(1024, 4096, 4096, 4, 32)
    assert 0 < a < b and c > b
    assert a % 256 == 0 and c % 256 == 0


# fake device addresses: 16-byte aligned, far apart, never dereferenced by validation
BASE = 1 << 40
X, WQ, SC, ZP, Y, WS, A, B = (BASE * (i + 1) for i in range(8))


def call(M=1, N=64, K=64, bits=4, block=32, x=X, wq=WQ, sc=SC, zp=ZP, y=Y, ws=WS, ws_bytes=1 << 30, ad=None,
         opt=None):
    return mnb.mnb_matmul_ex(x, wq, sc, zp, ad, y, M, N, K, bits, block, ws, ws_bytes, None, opt)


def test_validation_status_codes():
    E = mnb
    assert call(bits=3) == E.MNB_ERR_UNSUPPORTED
    assert call(block=64) == E.MNB_ERR_UNSUPPORTED
    assert call(K=48) == E.MNB_ERR_UNSUPPORTED
    assert call(K=1 << 25) == E.MNB_ERR_UNSUPPORTED
    assert call(M=-1) == E.MNB_ERR_INVALID_ARG
    assert call(N=-5) == E.MNB_ERR_INVALID_ARG
    assert call(x=None) == E.MNB_ERR_INVALID_ARG
    assert call(y=None) == E.MNB_ERR_INVALID_ARG
    assert call(wq=None) == E.MNB_ERR_INVALID_ARG
    assert call(x=X + 2) == E.MNB_ERR_MISALIGNED
    assert call(y=Y + 8) == E.MNB_ERR_MISALIGNED
    assert call(ws=None) == E.MNB_ERR_WORKSPACE
    assert call(ws_bytes=16) == E.MNB_ERR_WORKSPACE
    assert call(y=X) == E.MNB_ERR_ALIAS
    assert call(y=WS + 4096) == E.MNB_ERR_ALIAS
    assert call(opt=mnb.mnb_options(7, 0)) == E.MNB_ERR_INVALID_ARG
    assert call(opt=mnb.mnb_options(0, 8)) == E.MNB_ERR_INVALID_ARG
    assert call(ad=mnb.mnb_adapter(1, 16, A, None, B, None)) == E.MNB_ERR_UNSUPPORTED
    assert call(ad=mnb.mnb_adapter(2, 32, A, None, B, None)) == E.MNB_ERR_INVALID_ARG
    assert call(ad=mnb.mnb_adapter(5, 32, A, None, B, None)) == E.MNB_ERR_INVALID_ARG
    assert call(ad=mnb.mnb_adapter(1, 32, A + 4, None, B, None)) == E.MNB_ERR_MISALIGNED
    assert call(y=B, ad=mnb.mnb_adapter(1, 32, A, None, B, None)) == E.MNB_ERR_ALIAS


BIAS = BASE * 9


def call_bias(bias=BIAS, y=Y, M=1, N=64, K=64, ws=WS):
    return mnb.mnb_matmul_bias(X, WQ, SC, ZP, None, bias, y, M, N, K, 4, 32, ws, 1 << 30, None, None)


def test_bias_validation_status_codes():
    assert call_bias(bias=BIAS + 2) == mnb.MNB_ERR_MISALIGNED
    assert call_bias(bias=BIAS + 8) == mnb.MNB_ERR_MISALIGNED
    assert call_bias(y=BIAS) == mnb.MNB_ERR_ALIAS                  # Y over the bias
    assert call_bias(bias=Y + 64) == mnb.MNB_ERR_ALIAS             # bias inside Y [1, 64]


def test_degenerate_sizes_enqueue_nothing():
    # M == 0 or N == 0 returns before any device call, even with NULL tensors
    assert call(M=0, x=None, y=None, wq=None, sc=None, ws=None) == 0
    assert call(N=0, x=None, y=None, wq=None, sc=None, ws=None) == 0


def test_pack_validation():
    P = 1 << 41
    assert mnb.mnb_pack(P, P * 2, None, 64, 33, 4, 32, P * 3, P * 4, None, None) == mnb.MNB_ERR_UNSUPPORTED
    assert mnb.mnb_pack(P + 1, P * 2, None, 64, 64, 4, 32, P * 3, P * 4, None, None) == mnb.MNB_ERR_MISALIGNED
    assert mnb.mnb_pack(None, P * 2, None, 64, 64, 4, 32, P * 3, P * 4, None, None) == mnb.MNB_ERR_INVALID_ARG
    assert mnb.mnb_pack(P, P * 2, P * 5, 64, 64, 4, 32, P * 3, P * 4, None, None) == mnb.MNB_ERR_INVALID_ARG
    assert mnb.mnb_pack(None, None, None, 0, 64, 4, 32, None, None, None, None) == 0
    assert mnb.mnb_unpack(P, P, P, 64, 64, 8, 32, P, P, None, None) == mnb.MNB_ERR_INVALID_ARG
    for f in (mnb.mnb_pack, mnb.mnb_pack_kn):     # the DQ-layout packer validates the same way
        assert f(P, P * 2, None, 64, 33, 4, 32, P * 3, P * 4, None, None) == mnb.MNB_ERR_UNSUPPORTED
        assert f(P, P * 2 + 2, None, 64, 64, 4, 32, P * 3, P * 4, None, None) == mnb.MNB_ERR_MISALIGNED
        assert f(P, P * 2, None, 64, 64, 3, 32, P * 3, P * 4, None, None) == mnb.MNB_ERR_UNSUPPORTED
        assert f(P, None, None, 64, 64, 4, 32, P * 3, P * 4, None, None) == mnb.MNB_ERR_INVALID_ARG
        assert f(None, None, None, 64, 0, 4, 32, None, None, None, None) == 0


def route(M, N=4096, K=4096, bits=4, zp=1, kind=1, path=0, flags=0):
    st, text = mnb.mnb_describe_route(M, N, K, bits, zp, kind, mnb.mnb_options(path, flags))
    assert st == 0
    return text


def test_gemm_k_split_rule():
    """K is split only when the tiles leave CUs idle: none at 1024x4096 (256 tiles of 128
    rows) or for the batched prefill (64-row tiles, two workgroups per CU), several ranges at
    M = 256 and below; every range is non-empty, and the workspace grows by the FP32
    partials."""
    assert route(1024).endswith("tile=128x128x64 splits=1")
    # the batched prefill: 1216 tiles over 512 slots; its last 192 run alone on their CUs,
    # where splitting their K gains nothing, so all run whole
    assert route(1024, N=9728, K=2560, kind=2).endswith("tile=64x128x64 splits=1")
    # at M = 512 (608 tiles) only the last round's 96 tiles split K; at 1280x4096x4096 the
    # tail split (128 tiles in 2) replaces a uniform split in 2 of all 640 tiles; at 1536 the
    # last 256 tiles run alone on their CUs and stay whole
    assert route(512, N=9728, K=2560, kind=2).endswith("tile=64x128x64 splits=1 tail=96x2")
    assert route(1280).endswith("tile=64x128x64 splits=1 tail=128x2")
    assert route(1536).endswith("tile=64x128x64 splits=1")
    # a uniform split costs its partial traffic: none for 160 tiles of 128 rows at M = 640
    assert route(640).endswith("tile=128x128x64 splits=1")
    # a tail split needs at least one full round and a last one with room for the ranges
    assert " tail=" not in route(2048) and " tail=" not in route(1024, N=9728, K=256, kind=2)
    assert mnb.mnb_workspace_bytes(512, 9728, 2560, 4, 0) >= 2 * 96 * 64 * 128 * 4
    for M in (256, 64):
        assert int(route(M).rsplit("splits=", 1)[1]) > 1
    for M, N, K in ((300, 130, 800), (40, 136, 1056), (1, 64, 32), (129, 257, 320)):
        text = route(M, N=N, K=K, path=2)
        S = int(text.rsplit("splits=", 1)[1])
        steps = (K // 32 + 1) // 2
        sps = -(-steps // S)
        assert 1 <= S <= 16 and (S - 1) * sps < steps, (M, N, K, S)
    assert mnb.mnb_workspace_bytes(256, 4096, 4096, 4, 0) >= 2 * 256 * 4096 * 4
    # no partials at 1024 x 4096: the control area and accuracy level 4's quantized X [M, K]
    assert mnb.mnb_workspace_bytes(1024, 4096, 4096, 4, 0) < (1 << 20) + 1024 * 4096 * 2


def test_accuracy_level4_route_and_validation():
    A4 = mnb.MNB_FLAG_ACC4
    assert route(1, flags=A4).startswith("tproj_f16") and "gemv_acc4_b4_zpx_f16" in route(1, flags=A4)
    assert route(1, kind=0, flags=A4).startswith("gemv_acc4_b4_zpx_none")
    assert "gemv_acc4" in route(16, flags=A4) and "gemv_acc4" in route(5, bits=8, kind=0, flags=A4)
    assert "gemv_acc4_b2" in route(3, bits=2, flags=A4, path=1) and "gemv_acc4" in route(1024, flags=A4, path=1)
    # above 16 rows (or with the GEMM path forced): the block quantization of X, then the GEMM
    for r in (route(17, flags=A4), route(1024, flags=A4), route(4, flags=A4, path=2)):
        assert r.startswith("tproj_f16") and "; acc4_xquant grid=" in r and "; gemm_b4_zpx_f16" in r, r
    assert route(1024, kind=0, flags=A4).startswith("acc4_xquant grid=2048; gemm_b4_zpx_none")   # 4 threads per block
    # 4 X rows per workgroup row when the grid is wide and K <= 4096, else one
    assert route(8, N=49152, K=576, bits=8, kind=0, flags=A4).endswith("grid=768x2 rows=64 q=1 mr=4")
    assert route(13, flags=A4).endswith("grid=512x4 rows=8 q=8 mr=4")
    assert route(1, flags=A4).endswith("mr=1") and route(8, K=4128, flags=A4).endswith("grid=512x8 rows=8 q=8 mr=1")
    assert route(3, N=896, K=896, flags=A4).endswith("grid=112x3 rows=8 q=8 mr=1")
    st, _ = mnb.mnb_describe_route(1, 64, 16416, 4, 1, 1, mnb.mnb_options(0, A4))
    assert st == mnb.MNB_ERR_UNSUPPORTED                                    # GEMV family, K above 16384
    st, _ = mnb.mnb_describe_route(17, 64, 16416, 4, 1, 1, mnb.mnb_options(0, A4))
    assert st == mnb.MNB_OK                                                 # the GEMM takes any K
    assert call(K=16416, opt=mnb.mnb_options(0, A4)) == mnb.MNB_ERR_UNSUPPORTED
    assert call(opt=mnb.mnb_options(0, 8)) == mnb.MNB_ERR_INVALID_ARG      # unknown flag
    # the handoff failure hook is a known flag (the GPU tests exercise it)
    st, _ = mnb.mnb_describe_route(1, 8192, 2048, 4, 0, 1, mnb.mnb_options(0, mnb.MNB_FLAG_FAIL_HANDOFF))
    assert st == mnb.MNB_OK
    assert mnb.mnb_workspace_error(None, None) == mnb.MNB_ERR_INVALID_ARG


def test_dispatcher_rule():
    # M == 1: decode GEMV with in-pass T; 2 <= M <= 16: the small-M matrix-core GEMV after
    # the T projection (one 64-row group per workgroup when the rows are many and short,
    # else 16 rows per workgroup); M > 16: T projection + MFMA GEMM
    assert route(1).startswith("gemv_b4_zpx_f16_inpass")
    assert route(1, kind=0).startswith("gemv_b4_zpx_none_base")
    assert route(2).startswith("tproj_f16") and "gemv_mfma_b4_zpx_f16 grid=256 rows=16 mr=8" in route(2)
    assert "gemv_mfma_b4" in route(5) and "mr=8" in route(5)
    assert "gemv_mfma_b4" in route(9) and "mr=16" in route(9)
    assert "gemv_mfma_b4" in route(16) and "mr=16" in route(16)
    assert route(17).startswith("tproj_f16") and "gemm_b4_zpx_f16" in route(17)
    assert route(1024, kind=2).startswith("tproj_q8") and "gemm_b4_zpx_q8" in route(1024, kind=2)
    assert route(4, N=49152, K=576, bits=8, kind=0) == "gemv_mfma_wide_b8_zpx_none grid=768 rows=64 mr=8"
    assert route(16, N=49152, K=576, bits=8, kind=0) == "gemv_mfma_wide_b8_zpx_none grid=768 rows=64 mr=16"
    # the wide form needs >= 256 row groups, <= 16 wave loads per row and X within 64 KiB
    assert "gemv_mfma_b8" in route(8, N=16320, K=576, bits=8, kind=0)        # 255 row groups
    assert "gemv_mfma_wide_b8" in route(8, N=16321, K=576, bits=8, kind=0)   # 256
    assert "gemv_mfma_b4" in route(8, N=49152, K=2080, bits=4, kind=0)       # 17 wave loads
    assert "gemv_mfma_wide_b2" in route(8, N=49152, K=2048, bits=2, kind=0)
    assert "gemv_mfma_b2" in route(16, N=49152, K=2048, bits=2, kind=0)      # X staging 72 KiB
    # at the largest K every small-M X still fits one 32-bit buffer range (16 * 2K < 2^31)
    assert "gemv_mfma_b4" in route(16, K=(1 << 25) - 32) and "gemv_mfma" in route(15, K=(1 << 25) - 32, path=1)
    # overrides, as the pages keep explicit path overrides for comparisons
    assert route(1, path=2).startswith("tproj_f16") and "gemm" in route(1, path=2)
    assert route(7, path=2).startswith("tproj_f16") and "gemm" in route(7, path=2)
    assert route(7, path=1).startswith("tproj_f16") and "gemv_mfma_b4_zpx_f16" in route(7, path=1)
    assert route(40, path=1).startswith("tproj_f16") and "gemv_b4_zpx_f16_tprecomp" in route(40, path=1)
    assert "tprecomp" in route(1, flags=1) and route(1, flags=1).startswith("tproj")
    assert route(0) == "noop" and route(3, K=0) == "fill"


def test_gemv_grid_covers_the_chip():
    # decode: 64/q rows per workgroup with the smallest q in {1, 2, 4, 8} that gives at least
    # 512 row workgroups (two per CU), or 256 when T is computed in the same launch, plus
    # the T-slice workgroups (K/256 of them)
    for N, K, bits in ((8192, 2048, 4), (4096, 4096, 4), (49152, 576, 8), (896, 896, 4), (1024, 16384, 4),
                       (8192, 2048, 2)):
        for kind, target in ((1, 256), (0, 512)):
            t = route(1, N=N, K=K, bits=bits, zp=0, kind=kind)
            grid = int(re.search(r"grid=(\d+)x1", t).group(1))
            q = int(re.search(r" q=(\d+)", t).group(1))
            gt = int(re.search(r"gt=(\d+)", t).group(1))
            ng = (N + 63) // 64
            want = next(qq for qq in (1, 2, 4, 8) if ng * qq >= target or qq == 8)
            assert q == want, (N, K, bits, kind, q, want)
            assert gt == ((K + 255) // 256 if kind else 0) and grid == ng * q + gt


# ------------------------------------------------------------------------------------------
# the torch binding's own checks (CPU tensors; every case fails before any library call)
# ------------------------------------------------------------------------------------------

def test_workspace_cache_is_per_device_and_stream():
    """Calls that may overlap must not share a workspace: the binding's cache keeps one
    buffer per (device, stream), reuses it on that stream and grows it on demand."""
    import torch
    made = []

    def alloc(n):
        made.append(n)
        return torch.zeros(n, dtype=torch.uint8)

    c = mnb.WorkspaceCache(alloc)
    a = c.get(0, 0x1000, 256)
    b = c.get(0, 0x2000, 256)
    d = c.get(1, 0x1000, 256)
    assert len({a.data_ptr(), b.data_ptr(), d.data_ptr()}) == 3 and len(c) == 3
    assert c.get(0, 0x1000, 100) is a                  # same stream: reused
    big = c.get(0, 0x1000, 4096)                       # grows, replaces that stream's buffer only
    assert big.numel() == 4096 and c.get(0, 0x2000, 256) is b and len(c) == 3
    assert made == [256, 256, 256, 4096]


def test_binding_rejects_bad_tensors_before_the_library():
    import torch
    K, N = 64, 96
    pw = mnb.PackedWeight(torch.zeros(mnb.mnb_packed_sizes(N, K, 4, 32, 0)[1], dtype=torch.uint8),
                          torch.zeros(mnb.mnb_packed_sizes(N, K, 4, 32, 0)[2] // 2, dtype=torch.float16),
                          None, N, K, 4)
    X = torch.zeros((4, K), dtype=torch.float16)
    with pytest.raises(TypeError):
        mnb.matmul(X.float(), pw)                                         # X not fp16
    with pytest.raises(ValueError):
        mnb.matmul(torch.zeros((K, 4), dtype=torch.float16).t(), pw)      # X not contiguous
    with pytest.raises(ValueError):
        mnb.matmul(X, pw, out=torch.zeros((4, N - 1), dtype=torch.float16))   # out too small
    with pytest.raises(ValueError):
        mnb.matmul(X, pw, bias=torch.zeros(N + 1, dtype=torch.float16))   # bias not [N]
    short = mnb.PackedWeight(pw.wq[:-16], pw.sc, None, N, K, 4)
    with pytest.raises(ValueError):
        mnb.matmul(X, short)                                              # packed codes too short
    bad_a = mnb.Adapter(mnb.MNB_ADAPTER_F16, torch.zeros((K, 16), dtype=torch.float16),
                        torch.zeros((32, N), dtype=torch.float16))
    with pytest.raises(ValueError):
        mnb.matmul(X, pw, bad_a)                                          # A not [K, 32]
    q8 = mnb.Adapter(mnb.MNB_ADAPTER_Q8, torch.zeros((K, 32), dtype=torch.int8),
                     torch.zeros((32, N), dtype=torch.int8))
    with pytest.raises(ValueError):
        mnb.matmul(X, pw, q8)                                             # INT8 adapter without scales
    with pytest.raises(TypeError):
        mnb.pack(torch.zeros((N, K), dtype=torch.int32), torch.zeros((N, K // 32), dtype=torch.float16), None, 4)


def test_noalloc_validation_before_any_device_call():
    """mnb_matmul_noalloc validates like mnb_matmul_bias (no workspace argument) and refuses
    a call whose workspace would exceed its static scratch, before touching the device."""
    def na(M=1, N=64, K=64, bits=4, x=X, y=Y, ad=None, opt=None):
        return mnb.mnb_matmul_noalloc(x, WQ, SC, ZP, ad, None, y, M, N, K, bits, 32, None, opt)
    assert na(bits=3) == mnb.MNB_ERR_UNSUPPORTED
    assert na(M=-1) == mnb.MNB_ERR_INVALID_ARG
    assert na(x=None) == mnb.MNB_ERR_INVALID_ARG
    assert na(y=Y + 8) == mnb.MNB_ERR_MISALIGNED
    assert na(y=X) == mnb.MNB_ERR_ALIAS
    assert na(M=0, x=None, y=None) == mnb.MNB_OK
    big = (256, 12288, 16384)                     # K split into FP32 partials: 48 MiB of workspace
    assert mnb.mnb_workspace_bytes(*big, 4, 0) > mnb.MNB_NOALLOC_SCRATCH_BYTES
    assert na(*big) == mnb.MNB_ERR_TOO_LARGE
    assert "MNB_ERR_TOO_LARGE" in mnb.mnb_status_string(mnb.MNB_ERR_TOO_LARGE)
