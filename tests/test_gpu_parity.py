"""GPU parity: the HIP path (through the C ABI) against the FP64 oracle.

Bars: packing and indexing bit-exact; exact-arithmetic cases bit-exact; FP16 outputs within
max-abs 2e-2 and normwise relative 1e-2 of the oracle (FP32 accumulation).  The five
workloads run at their full sizes in the launch configuration the benchmark times, every
output element compared (the oracle takes a few seconds for M = 1024).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from _util import compare, ensure_lib, f16_to_f64, same_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mnb = ensure_lib()
DEV = torch.device("cuda:0")


# ------------------------------------------------------------------------------------------
# marshalling
# ------------------------------------------------------------------------------------------

def t16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.float16)).to(DEV)


def tu8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def ti8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int8)).to(DEV)


def dev_weight(case):
    zp = tu8(case["zp"]) if case.get("zp") is not None else None
    return mnb.pack(tu8(case["codes"]), t16(case["scales"]), zp, case["bits"])


def dev_adapter(ad):
    if ad is None:
        return None
    if ad["kind"] == "f16":
        return mnb.Adapter(mnb.MNB_ADAPTER_F16, t16(ad["A"]), t16(ad["B"]), rank=ad.get("rank", 32))
    return mnb.Adapter(mnb.MNB_ADAPTER_Q8, ti8(ad["A"]), ti8(ad["B"]), t16(ad["A_scales"]), t16(ad["B_scales"]),
                       rank=ad.get("rank", 32))


def run(case, path=0, flags=0, pw=None, ad="case", X=None):
    pw = pw or dev_weight(case)
    a = dev_adapter(case.get("adapter")) if ad == "case" else ad
    Xd = t16(case["X"]) if X is None else X
    bias = t16(case["bias"]) if case.get("bias") is not None else None
    Y = mnb.matmul(Xd, pw, a, path=path, flags=flags, bias=bias)
    torch.cuda.synchronize()
    return Y.cpu().numpy().view(np.uint16)


def rows_case(case, rows):
    return dict(case, X=case["X"][rows], M=len(rows))


PATHS = [(0, 0, "auto"), (1, 0, "gemv"), (1, 1, "gemv_tsep"), (2, 0, "gemm")]


# ------------------------------------------------------------------------------------------
# packing (bit-exact)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("N,K,bits,zp", [(1, 32, 4, True), (64, 64, 4, False), (100, 96, 8, True),
                                          (130, 160, 4, True), (896, 896, 4, True), (8192, 2048, 4, False),
                                          (49152, 576, 8, True), (257, 1024, 8, False), (70, 96, 2, True),
                                          (130, 160, 2, False), (8192, 2048, 2, True), (5, 32, 2, True)])
def test_pack_matches_oracle_bytes(N, K, bits, zp):
    case = si.make_random(11, 1, N, K, bits, zp, None)
    pw = dev_weight(case)
    torch.cuda.synchronize()
    wq, sc, zpp = oracle.pack(case["codes"], case["scales"], case["zp"], N, K, bits)
    assert np.array_equal(pw.wq.cpu().numpy(), wq)
    assert np.array_equal(pw.sc.cpu().numpy().view(np.uint16), sc)
    if zp:
        assert np.array_equal(pw.zp.cpu().numpy(), zpp)
    codes, scales, z2 = mnb.unpack(pw)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), case["codes"])
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), case["scales"])
    if zp:
        assert np.array_equal(z2.cpu().numpy(), case["zp"])


@pytest.mark.parametrize("N,K,bits,zp", [(1, 32, 4, True), (70, 96, 4, False), (100, 96, 8, True),
                                          (130, 160, 4, True), (49152, 576, 8, True), (4096, 4096, 4, True),
                                          (257, 1024, 8, False), (66, 96, 2, True), (4096, 4096, 2, False)])
def test_pack_from_dq_layout_matches_oracle_bytes(N, K, bits, zp):
    """mnb_pack_kn ([K, N] codes, [K/32, N] scales and zero points, as DequantizeLinear
    holds them; the 576 x 49152 int8 case is the tied lm_head's own layout) against the
    oracle, byte for byte, and against mnb_pack of the transposed tensors."""
    case = si.make_random(21, 1, N, K, bits, zp, None)
    ckn = np.ascontiguousarray(case["codes"].T)
    skn = np.ascontiguousarray(case["scales"].T)
    zkn = np.ascontiguousarray(case["zp"].T) if zp else None
    pw = mnb.pack_kn(tu8(ckn), t16(skn), tu8(zkn) if zp else None, bits)
    ref = dev_weight(case)
    torch.cuda.synchronize()
    want = oracle.pack_kn(ckn, skn, zkn, N, K, bits)
    assert same_bits(pw.wq.cpu().numpy(), want[0])
    assert same_bits(pw.sc.cpu().numpy().view(np.uint16), want[1])
    if zp:
        assert same_bits(pw.zp.cpu().numpy(), want[2])
    assert torch.equal(pw.wq, ref.wq) and torch.equal(pw.sc.view(torch.int16), ref.sc.view(torch.int16))


def test_pack_is_deterministic():
    case = si.make_random(12, 1, 300, 256, 4, True, None)
    a, b = dev_weight(case), dev_weight(case)
    torch.cuda.synchronize()
    assert torch.equal(a.wq, b.wq) and torch.equal(a.sc.view(torch.int16), b.sc.view(torch.int16))


# ------------------------------------------------------------------------------------------
# the five workloads at full size
# ------------------------------------------------------------------------------------------

def test_cfg1_tiny_decode():
    case = si.make_config(1)
    compare(run(case), oracle.matmul(case), what="cfg1")


@pytest.mark.parametrize("with_adapter", [True, False], ids=["lora", "empty"])
def test_cfg2_decode(with_adapter):
    case = si.make_config(2, adapter=with_adapter)
    ref = oracle.matmul(case)
    compare(run(case), ref, what="cfg2")
    if with_adapter:
        compare(run(case, flags=mnb.MNB_FLAG_T_SEPARATE), ref, what="cfg2 T separate")


def test_cfg3_prefill_and_dispatcher_rows():
    case = si.make_config(3)
    pw = dev_weight(case)
    Y = run(case, pw=pw)
    ref = oracle.matmul(case)
    compare(Y, ref, what="cfg3 M=1024, all rows")
    # same weights, M = 256 and M = 1 as prefix rows of X (GEMM and GEMV by the dispatcher)
    c256 = si.make_config(3, M=256)
    compare(run(c256, pw=pw), ref[:256], what="cfg3 M=256")
    c1 = si.make_config(3, M=1)
    compare(run(c1, pw=pw), ref[:1], what="cfg3 M=1")


@pytest.mark.parametrize("M", [1, 8])
def test_cfg4_lm_head(M):
    case = si.make_config(4, M=M)
    compare(run(case), oracle.matmul(case), what="cfg4 M=%d" % M)


def test_cfg5_batched_prefill_q8():
    case = si.make_config(5)
    Y = run(case)
    compare(Y, oracle.matmul(case), what="cfg5 all rows")
    # the zero half of B: those columns equal the base-only output bitwise
    base = run(case, ad=None)
    half = case["N"] // 2
    assert same_bits(Y[:, half:], base[:, half:])
    assert not same_bits(Y[:, :half], base[:, :half])


# ------------------------------------------------------------------------------------------
# small shapes: every variant, every path, ragged tails
# ------------------------------------------------------------------------------------------

SHAPES = [(1, 64, 32), (1, 100, 96), (1, 1, 32), (3, 130, 160), (7, 32, 64), (2, 200, 1024), (129, 257, 320),
          (256, 384, 512), (1, 4096, 4096), (16, 96, 256), (9, 70, 192), (5, 513, 128), (17, 64, 96),
          (1, 64, 16384), (3, 100, 8192)]   # long K: several load rounds, 64 T slices or parts


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("zp", [True, False], ids=["zp", "zpdef"])
@pytest.mark.parametrize("adapter", [None, "f16", "q8"], ids=["base", "f16", "q8"])
def test_small_shapes_all_paths(bits, zp, adapter):
    for i, (M, N, K) in enumerate(SHAPES):
        case = si.make_random(40 + i, M, N, K, bits, zp, adapter)
        ref = oracle.matmul(case)
        pw = dev_weight(case)
        for path, flags, name in PATHS:
            compare(run(case, path, flags, pw=pw), ref, what="%s M=%d N=%d K=%d" % (name, M, N, K))


# decode shapes for the X-range test: one 64-row group (8 chunk-columns per wave load and a
# ragged last load at K = 96), ragged K against the load width, the decode width, and a
# 625-group lm_head-like shape (one chunk-column per wave load); M = 3 takes the small-M path
X_RANGE_SHAPES = [(1, 64, 96), (1, 200, 1056), (1, 8192, 2080), (1, 40000, 576), (3, 200, 1056)]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("zp", [True, False], ids=["zp", "zpdef"])
@pytest.mark.parametrize("x_std,s_lo,s_hi", [(1e-3, 0.01, 0.02), (30.0, 1e-4, 1e-3)], ids=["small_x", "large_x"])
def test_decode_x_range(bits, zp, x_std, s_lo, s_hi):
    """The decode path enters the codes as 1024 + q (and 1024 + 16 q, 1024 + 4^e q for the
    fields taken in place) and subtracts each block's offset-weighted X sum once, so its
    block sums pass through values near 1024 * sum(X).  X from 1e-3 to 30 in spread, with
    one value per 32-k block raised 40-fold (an outlier the block sum carries), against the
    oracle.  The weight scales are then scaled down (once, as fp16) until the largest output
    is at most 8, where the fp16 output rounding stays far below the max-abs bar; the
    adapter (whose T is an ordinary FP32 product) rides along with the small X only."""
    for i, (M, N, K) in enumerate(X_RANGE_SHAPES):
        adapter = "f16" if i % 2 and x_std < 1 else None
        case = si.make_random(300 + i, M, N, K, bits, zp, adapter, s_lo=s_lo, s_hi=s_hi, x_std=x_std)
        x = case["X"].view(np.float16).astype(np.float32)
        x[:, 7::32] *= 40.0
        case["X"] = np.clip(x, -60000, 60000).astype(np.float16).view(np.uint16)
        ref = oracle.matmul(case)
        peak = float(np.abs(ref).max())
        if peak > 8.0:
            sc = case["scales"].view(np.float16).astype(np.float32) * np.float32(8.0 / peak)
            case["scales"] = sc.astype(np.float16).view(np.uint16)
            ref = oracle.matmul(case)
        pw = dev_weight(case)
        for path in (0, 1):
            compare(run(case, path, 0, pw=pw), ref, what="path %d M=%d N=%d K=%d" % (path, M, N, K))


# small-M matrix-core GEMV, both forms: 16 rows per workgroup (8 waves splitting K), and one
# 64-row group per workgroup when the rows are many and short (>= 256 row groups, <= 16 wave
# loads per row); ragged N (last row group partial) and K (wave loads past the row), X rows
# 2..16 (the MFMA's rows past M padded).  The one-group form at up to 8 X rows splits each
# row slice's wave loads over two waves: odd load counts (9, 5, 3 at 8, 4, 2 bits for
# K = 576: uneven halves) and a single load (K = 64: the odd half has none)
SMALL_M_SHAPES = [(2, 200, 1056), (5, 130, 96), (9, 16400, 576), (16, 16400, 160), (3, 20000, 2080),
                  (5, 16400, 576), (2, 16400, 64)]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("zp", [True, False], ids=["zp", "zpdef"])
@pytest.mark.parametrize("adapter", [None, "f16", "q8"], ids=["base", "f16", "q8"])
def test_small_m_matrix_core_forms(bits, zp, adapter):
    forms = set()
    for i, (M, N, K) in enumerate(SMALL_M_SHAPES):
        case = si.make_random(500 + i, M, N, K, bits, zp, adapter)
        kind = {None: 0, "f16": 1, "q8": 2}[adapter]
        st, text = mnb.mnb_describe_route(M, N, K, bits, int(zp), kind, None)
        assert st == 0 and "gemv_mfma" in text, text
        forms.add("wide" in text)
        ref = oracle.matmul(case)
        compare(run(case, 0, 0), ref, what="%s M=%d N=%d K=%d" % (text, M, N, K))
    assert forms == {True, False}, "both forms exercised"


# T projection part layouts: the part reduction in the projection (2 <= M <= 16, K > 2048)
# across its 16-part load batches with a ragged last part, both 8-row blocks of a 16-row
# tile, the 1024-k parts (two A tiles per thread); up to 4 parts added by the small-M GEMV
# from its prefetch (K <= 2048, ragged last part, both X-row forms); and the parts the GEMM
# adds (M > 16, ragged)
TPROJ_CASES = [(5, 136, 4640, "f16", 19), (5, 136, 4640, "q8", 19), (16, 200, 8192, "q8", 32),
               (2, 64, 131072, "f16", 128), (6, 136, 2016, "f16", 4), (9, 200, 1056, "q8", 3),
               (40, 96, 2592, "q8", 6)]


@pytest.mark.parametrize("M,N,K,adapter,parts", TPROJ_CASES)
def test_t_projection_parts(M, N, K, adapter, parts):
    kind = {"f16": 1, "q8": 2}[adapter]
    _, desc = mnb.mnb_describe_route(M, N, K, 4, 1, kind, None)
    assert "parts=%d;" % parts in desc, desc
    case = si.make_random(260 + M, M, N, K, 4, True, adapter)
    ref = oracle.matmul(case)
    peak = float(np.abs(ref).max())
    if peak > 8.0:
        # long K: scales shrunk so that the fp16 outputs' own rounding stays below the
        # absolute bound (|y| <= 8: half an ulp is at most 2^-8)
        sc = case["scales"].view(np.float16).astype(np.float32) * np.float32(8.0 / peak)
        case["scales"] = sc.astype(np.float16).view(np.uint16)
        ref = oracle.matmul(case)
    compare(run(case), ref, what="%s M=%d N=%d K=%d" % (adapter, M, N, K))


SPLIT_SHAPES = [(40, 136, 1056), (300, 130, 800), (2, 200, 1024), (200, 1000, 2080)]


@pytest.mark.parametrize("adapter", [None, "f16"], ids=["base", "f16"])
def test_gemm_tile_rows_both(adapter):
    """Both tile heights: 128-row tiles when they fill the CUs' rounds (and most of a
    last one), 64-row tiles otherwise; the 128-row tiles' load waves also with K ranges of
    one step (K = 32) and two steps, the second ragged (K = 96)."""
    for i, (M, N, K, bm) in enumerate([(256, 12800, 512, 128), (200, 200, 320, 64), (1024, 4096, 256, 128),
                                       (1024, 4096, 32, 128), (1024, 4096, 96, 128)]):
        _, desc = mnb.mnb_describe_route(M, N, K, 4, 1, 1 if adapter else 0)
        assert "tile=%dx128x64" % bm in desc, desc
        case = si.make_random(210 + i, M, N, K, 4, True, adapter, bias=i == 1)
        rows = [0, 1, 63, 64, 127, 128, M - 1]
        compare(run(case)[rows], oracle.matmul(rows_case(case, rows)), what="tiles M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("adapter", [None, "f16", "q8"], ids=["base", "f16", "q8"])
def test_gemm_load_waves_split_k(bits, adapter):
    """128-row tiles, whose load waves issue the ring's loads and fetch the LoRA operands
    (B, and the T parts one per step), with K split over 3 ranges (11, 11 and 10 steps; the
    first range adds the LoRA term) and a ragged last row tile: every output checked."""
    M, N, K = 134, 9728, 4096
    kind = {None: 0, "f16": 1, "q8": 2}[adapter]
    _, desc = mnb.mnb_describe_route(M, N, K, bits, 1, kind)
    assert "tile=128x128x64 splits=3" in desc, desc
    case = si.make_random(270 + bits, M, N, K, bits, True, adapter)
    ref = oracle.matmul(case)
    peak = float(np.abs(ref).max())
    if peak > 8.0:
        # scales shrunk so that the fp16 outputs' own rounding stays below the absolute
        # bound (|y| <= 8: half an ulp is at most 2^-8)
        sc = case["scales"].view(np.float16).astype(np.float32) * np.float32(8.0 / peak)
        case["scales"] = sc.astype(np.float16).view(np.uint16)
        ref = oracle.matmul(case)
    compare(run(case), ref, what="%s M=%d N=%d K=%d" % (desc, M, N, K))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("adapter", [None, "f16", "q8"], ids=["base", "f16", "q8"])
def test_gemm_split_k_ranges(bits, adapter):
    """Shapes with fewer 128x128 tiles than CUs: the GEMM splits K into ranges (odd block
    counts, ragged M and N, N % 4 != 0 for the scalar reduction) and must still match."""
    for i, (M, N, K) in enumerate(SPLIT_SHAPES):
        _, desc = mnb.mnb_describe_route(M, N, K, bits, 1, {None: 0, "f16": 1, "q8": 2}[adapter],
                                         mnb.mnb_options(2, 0))
        assert not desc.endswith(" splits=1"), desc
        case = si.make_random(190 + i, M, N, K, bits, i % 2 == 0, adapter, bias=i >= 2)
        rows = list(range(M)) if M <= 64 else [0, 1, 127, 128, M - 1]
        compare(run(case, 2, 0)[rows], oracle.matmul(rows_case(case, rows)), what="split M=%d N=%d K=%d" % (M, N, K))


LOOP_SHAPES = [(1024, 4096, 1056), (1024, 4096, 544), (1024, 4096, 512)]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("adapter", [None, "f16"], ids=["base", "f16"])
def test_gemm_whole_k_loop_paths(bits, adapter):
    """128-row tiles over whole K, so that one K range runs both forms of the main loop (the
    iterations whose loads are all before the last step, then the clamped ones and the
    tail): 17 steps with an odd block count (the last step ragged), 9 steps (odd), 8 steps;
    rows sampled in every 32-row block of a tile, i.e. from every wave's quarter of the
    epilogue."""
    for i, (M, N, K) in enumerate(LOOP_SHAPES):
        _, desc = mnb.mnb_describe_route(M, N, K, bits, 1, 1 if adapter else 0, mnb.mnb_options(2, 0))
        assert desc.endswith("tile=128x128x64 splits=1"), desc
        case = si.make_random(250 + i, M, N, K, bits, i != 1, adapter, bias=i == 2)
        rows = [0, 1, 31, 32, 63, 64, 95, 96, 127, 128, 300, 511, 512, 700, M - 33, M - 1]
        compare(run(case, 2, 0)[rows], oracle.matmul(rows_case(case, rows)), what="loop M=%d N=%d K=%d" % (M, N, K))


TAIL_SHAPES = [(1000, 4202, 1056), (960, 4354, 1056), (1000, 4100, 640)]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("adapter", [None, "f16", "q8"], ids=["base", "f16", "q8"])
def test_gemm_tail_split(bits, adapter):
    """Shapes whose last round of tiles is mostly empty: only those tiles split K (odd
    block counts, ragged M, N % 4 != 0 for the scalar reduction, a head that ends inside a
    column strip) and must still match."""
    for i, (M, N, K) in enumerate(TAIL_SHAPES):
        _, desc = mnb.mnb_describe_route(M, N, K, bits, 1, {None: 0, "f16": 1, "q8": 2}[adapter],
                                         mnb.mnb_options(2, 0))
        assert " tail=" in desc, desc
        case = si.make_random(230 + i, M, N, K, bits, i % 2 == 0, adapter, bias=i == 1)
        rows = [0, 1, 63, 64, 511, 512, M - 65, M - 1]
        compare(run(case, 2, 0)[rows], oracle.matmul(rows_case(case, rows)), what="tail M=%d N=%d K=%d" % (M, N, K))


# ------------------------------------------------------------------------------------------
# bit-exact pins on the GPU
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("bits,zp", [(4, True), (4, False), (8, True), (8, False), (2, True), (2, False)])
def test_one_hot_bit_exact(bits, zp):
    """X = rows of the identity: each output is one dequantized weight rounded once."""
    N, K = 200, 256
    case = si.make_random(60 + bits, K, N, K, bits, zp, None)
    X = np.eye(K, dtype=np.float16).view(np.uint16)
    c = dict(case, X=X, M=K)
    want = oracle.f64_to_f16(oracle.matmul(c))
    pw = dev_weight(c)
    for path, flags, name in PATHS:
        assert same_bits(run(c, path, flags, pw=pw), want), name


def small_scales(rng, shape):
    """fp16 bit patterns spread over the subnormals and [2^-14, 2^-10): the range where a
    scale divided by 16 is no longer an exact fp16 value."""
    s = rng.integers(0x0400, 0x1400, size=shape).astype(np.uint16)
    sub = rng.random(shape) < 0.25
    s[sub] = rng.integers(0x0001, 0x0400, size=int(sub.sum())).astype(np.uint16)
    return s


@pytest.mark.parametrize("bits,zp", [(4, True), (4, False), (8, True), (2, True)])
def test_one_hot_small_scales_bit_exact(bits, zp):
    """One-hot X with scales below 2^-10 and subnormal scales: each output is the single
    weight (q - z) * s rounded once to fp16, on every path (the dequantized weight of the
    MFMA operand must round once for every finite scale)."""
    N, K = 200, 256
    case = si.make_random(260 + bits, K, N, K, bits, zp, None)
    scales = small_scales(np.random.default_rng(261 + bits), case["scales"].shape)
    X = np.eye(K, dtype=np.float16).view(np.uint16)
    c = dict(case, X=X, M=K, scales=scales)
    want = oracle.f64_to_f16(oracle.matmul(c))
    pw = dev_weight(c)
    for path, flags, name in PATHS:
        assert same_bits(run(c, path, flags, pw=pw), want), name


def exact_case(seed, M, N, K, bits, zp, kind, bias=False):
    """Inputs whose every product and partial sum is exact in FP32 (P-e)."""
    r = np.random.default_rng(seed)
    X = np.zeros((M, K), np.float16)
    for m in range(M):
        ks = r.choice(K, size=min(8, K), replace=False)
        X[m, ks] = r.choice([-2.0, -1.0, 1.0, 2.0], size=len(ks))
    z = {2: r.integers(0, 4, size=(N, K // 32)), 4: r.integers(0, 16, size=(N, K // 32)),
         8: r.integers(100, 157, size=(N, K // 32))}[bits]
    zfull = np.repeat(z if zp else np.full_like(z, 2 ** (bits - 1)), 32, axis=1)
    codes = (np.clip(zfull + r.integers(-15, 16, size=(N, K)), 0, 2 ** bits - 1)).astype(np.uint8)
    scales = np.full((N, K // 32), 0x3000, np.uint16)                  # 2^-3
    ad = None
    if kind == "f16":
        ad = dict(kind="f16", A=si.to_f16_bits(r.integers(-3, 4, size=(K, 32)) * 0.25),
                  B=si.to_f16_bits(r.integers(-3, 4, size=(32, N)) * 0.25))
    elif kind == "q8":
        ad = dict(kind="q8", A=r.integers(-3, 4, size=(K, 32)).astype(np.int8),
                  A_scales=np.full((K // 32, 32), 0x3400, np.uint16),       # 2^-2
                  B=r.integers(-3, 4, size=(32, N)).astype(np.int8),
                  B_scales=np.full((1, N), 0x3400, np.uint16))
    b = si.to_f16_bits(r.integers(-64, 65, size=N) * 0.125) if bias else None
    return dict(M=M, N=N, K=K, bits=bits, X=X.view(np.uint16), codes=codes, scales=scales,
                zp=z.astype(np.uint8) if zp else None, adapter=ad, bias=b)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("kind", [None, "f16", "q8"], ids=["base", "f16", "q8"])
@pytest.mark.parametrize("M", [1, 5, 130])
def test_exact_arithmetic_bit_exact(bits, kind, M):
    case = exact_case(70 + M + bits, M, 192, 320, bits, True, kind)
    want = oracle.f64_to_f16(oracle.matmul(case))
    pw = dev_weight(case)
    for path, flags, name in PATHS:
        assert same_bits(run(case, path, flags, pw=pw), want), name


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("kind", [None, "f16", "q8"], ids=["base", "f16", "q8"])
@pytest.mark.parametrize("M", [1, 5, 130])
def test_exact_arithmetic_small_scales_bit_exact(bits, kind, M):
    """Exact arithmetic with scales below 2^-10 (normal and subnormal, with low mantissa
    bits set) and |q - z| <= 1, so every weight is an fp16 value; adapters scaled by 2^-8
    keep every sum exact in FP32: each output is the exact value rounded once."""
    r = np.random.default_rng(270 + M + bits)
    case = exact_case(270 + M + bits, M, 192, 320, bits, True, kind)
    zfull = np.repeat(case["zp"], 32, axis=1).astype(np.int64)
    codes = np.clip(zfull + r.integers(-1, 2, size=zfull.shape), 0, 2 ** bits - 1).astype(np.uint8)
    scales = r.choice(np.array([0x0401, 0x0403, 0x07FF, 0x0C05, 0x13FF, 0x0001, 0x0155, 0x03FF], np.uint16),
                      size=case["scales"].shape)
    ad = case["adapter"]
    if ad is not None and ad["kind"] == "f16":
        ad = dict(ad, A=si.to_f16_bits(si.f16_bits_to_f32(ad["A"]) * 2.0 ** -6),
                  B=si.to_f16_bits(si.f16_bits_to_f32(ad["B"]) * 2.0 ** -6))
    elif ad is not None:
        ad = dict(ad, A_scales=np.full_like(ad["A_scales"], 0x1C00),      # 2^-8
                  B_scales=np.full_like(ad["B_scales"], 0x1C00))
    c = dict(case, codes=codes, scales=scales, adapter=ad)
    want = oracle.f64_to_f16(oracle.matmul(c))
    pw = dev_weight(c)
    for path, flags, name in PATHS:
        assert same_bits(run(c, path, flags, pw=pw), want), name


@pytest.mark.parametrize("kind", [None, "f16", "q8"], ids=["base", "f16", "q8"])
@pytest.mark.parametrize("M", [1, 6, 16, 130])
def test_exact_arithmetic_with_bias_bit_exact(kind, M):
    """Bias multiples of 2^-3 keep every sum exact: each output is the exact value rounded once."""
    for bits in (2, 4, 8):
        case = exact_case(170 + M + bits, M, 200, 320, bits, bits != 8, kind, bias=True)
        want = oracle.f64_to_f16(oracle.matmul(case))
        pw = dev_weight(case)
        for path, flags, name in PATHS:
            assert same_bits(run(case, path, flags, pw=pw), want), "%s bits=%d" % (name, bits)


BIAS_SHAPES = [(1, 64, 32), (1, 100, 96), (3, 130, 160), (8, 257, 320), (13, 96, 256), (16, 70, 192),
               (129, 257, 320), (1, 4096, 2048), (5, 16400, 576)]   # the last: the one-group small-M form


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("adapter", [None, "f16", "q8"], ids=["base", "f16", "q8"])
def test_bias_small_shapes_all_paths(bits, adapter):
    for i, (M, N, K) in enumerate(BIAS_SHAPES):
        case = si.make_random(150 + i, M, N, K, bits, i % 2 == 0, adapter, bias=True)
        ref = oracle.matmul(case)
        pw = dev_weight(case)
        for path, flags, name in PATHS:
            compare(run(case, path, flags, pw=pw), ref, what="bias %s M=%d N=%d K=%d" % (name, M, N, K))


def test_empty_weights_give_broadcast_bias():
    """K == 0: Y is the bias broadcast over rows, bit for bit, on every path; without a
    bias it is zeros (empty packed weights keep the output shape)."""
    for M, N in [(1, 1), (3, 70), (5, 4099), (64, 1000)]:
        case = si.make_random(160 + M, M, N, 32, 4, False, None, bias=True)
        bias = t16(case["bias"])
        X = torch.zeros((M, 0), dtype=torch.float16, device=DEV)
        pw = mnb.PackedWeight(torch.zeros(16, dtype=torch.uint8, device=DEV),
                              torch.zeros(8, dtype=torch.float16, device=DEV), None, N, 0, 4)
        want = np.broadcast_to(case["bias"], (M, N))
        empty = dict(case, K=0, X=np.zeros((M, 0), np.uint16), codes=np.zeros((N, 0), np.uint8),
                     scales=np.zeros((N, 0), np.uint16))
        assert same_bits(oracle.f64_to_f16(oracle.matmul(empty)), want)
        for path, flags, name in PATHS:
            Y = mnb.matmul(X, pw, None, path=path, flags=flags, bias=bias)
            torch.cuda.synchronize()
            assert same_bits(Y.cpu().numpy().view(np.uint16), want), "%s M=%d N=%d" % (name, M, N)
            Y = mnb.matmul(X, pw, None, path=path, flags=flags)
            torch.cuda.synchronize()
            assert bool((Y == 0).all()), name


@pytest.mark.parametrize("M", [1, 64])
def test_empty_and_zero_adapter_equal_base_bitwise(M):
    case = si.make_random(80 + M, M, 320, 512, 4, True, "f16")
    pw = dev_weight(case)
    for path, flags, name in PATHS:
        base = run(case, path, flags, pw=pw, ad=None)
        ad = case["adapter"]
        A, B = t16(ad["A"]), t16(ad["B"])
        zA, zB = torch.zeros_like(A), torch.zeros_like(B)
        variants = [mnb.Adapter(mnb.MNB_ADAPTER_F16, A, B, rank=0),
                    mnb.Adapter(mnb.MNB_ADAPTER_NONE, A, B),
                    mnb.Adapter(mnb.MNB_ADAPTER_F16, None, B),
                    mnb.Adapter(mnb.MNB_ADAPTER_F16, zA, B),
                    mnb.Adapter(mnb.MNB_ADAPTER_F16, A, zB)]
        for v in variants:
            assert same_bits(run(case, path, flags, pw=pw, ad=v), base), name
        assert not same_bits(run(case, path, flags, pw=pw), base), name


def test_code_equal_zero_point_gives_zero():
    for bits in (2, 4, 8):
        case = si.make_random(90 + bits, 3, 130, 256, bits, True, "f16")
        codes = np.repeat(case["zp"], 32, axis=1).astype(np.uint8)
        c = dict(case, codes=codes)
        pw = dev_weight(c)
        for path, flags, name in PATHS:
            y = run(c, path, flags, pw=pw, ad=None)
            assert np.all(f16_to_f64(y) == 0.0), name
            compare(run(c, path, flags, pw=pw), oracle.matmul(c), what=name)


def test_default_zero_point_equals_explicit():
    for bits in (2, 4, 8):
        case = si.make_random(95 + bits, 3, 130, 256, bits, False, "q8")
        explicit = dict(case, zp=np.full(case["scales"].shape, 2 ** (bits - 1), np.uint8))
        for path, flags, name in PATHS:
            assert same_bits(run(case, path, flags), run(explicit, path, flags)), name


# ------------------------------------------------------------------------------------------
# accuracy level 4 (int8 block-quantized activations for the base product)
# ------------------------------------------------------------------------------------------

# M > 1 with K <= 4096 and >= 256 workgroups runs 4 X rows per workgroup row (N >= 4096:
# M = 8, 6 and 13, the last with K = 4096, its largest K, and a ragged last group); the
# narrow shapes and K > 4096 one row per workgroup row
ACC4_SHAPES = [(1, 64, 32), (1, 100, 96), (3, 130, 160), (1, 8192, 2048), (2, 200, 1024), (130, 257, 320),
               (9, 70, 192), (1, 49152, 576), (1, 64, 16384), (8, 49152, 576), (13, 4096, 4096), (6, 4096, 640),
               (3, 72, 4128)]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("adapter", [None, "f16", "q8"], ids=["base", "f16", "q8"])
def test_acc4_against_oracle(bits, adapter):
    for i, (M, N, K) in enumerate(ACC4_SHAPES):
        if bits != 8 and N == 49152:
            continue
        case = si.make_random(300 + i, M, N, K, bits, i % 2 == 1, adapter, bias=i % 3 == 2)
        rows = list(range(M)) if M <= 16 else [0, 1, 63, 64, M - 1]
        ref4 = oracle.matmul(dict(rows_case(case, rows), acc_level=4))
        pw = dev_weight(case)
        for path in (0, 1, 2):           # auto, the GEMV family, the GEMM on the quantized X
            y = run(case, path, mnb.MNB_FLAG_ACC4, pw=pw)
            compare(y[rows], ref4, what="acc4 path=%d M=%d N=%d K=%d" % (path, M, N, K))


@pytest.mark.parametrize("cfg", [3, 5])
def test_acc4_prefill_workloads(cfg):
    """Accuracy level 4 at the prefill workloads (the GEMM on the block-quantized X, T from the
    unquantized X): every output against the oracle at level 4."""
    case = si.make_config(cfg)
    assert "acc4_xquant" in mnb.mnb_describe_route(case["M"], case["N"], case["K"], case["bits"],
                                                   case["zp"] is not None, 1 if cfg == 3 else 2,
                                                   mnb.mnb_options(0, mnb.MNB_FLAG_ACC4))[1]
    y = run(case, 0, mnb.MNB_FLAG_ACC4)
    compare(y, oracle.matmul(dict(case, acc_level=4)), what="acc4 cfg%d" % cfg)


def acc4_exact_case(seed, M, N, K, bits, zp, kind):
    """Activations that block quantization represents exactly (c * 2^-e, max |c| = 127)
    and weights, adapters and scales that keep every sum exact: the result is unique."""
    case = exact_case(seed, M, N, K, bits, zp, kind)
    r = np.random.default_rng(seed + 1)
    X = np.zeros((M, K))
    for m in range(M):
        for b in range(K // 32):
            if (m + b) % 5 == 2:
                continue
            c = r.integers(-127, 128, size=32)
            c[r.integers(0, 32)] = 127
            X[m, 32 * b:32 * b + 32] = c * 2.0 ** -int(r.integers(8, 11))
    if kind == "f16":
        # A nonzero in 4 rows of one block per rank column, so that T = X.A (one power of two
        # times at most 4 products of 7-bit and 2-bit integers) is exact in fp16 as well: the
        # GEMM path rounds T to an fp16 MFMA operand, the GEMV family keeps it in FP32
        A = np.zeros((K, 32))
        b0 = int(r.integers(0, K // 32))
        for col in range(32):
            ks = 32 * b0 + r.choice(32, size=4, replace=False)
            A[ks, col] = r.integers(-3, 4, size=4) * 0.25
        case["adapter"] = dict(case["adapter"], A=si.to_f16_bits(A))
    return dict(case, X=si.to_f16_bits(X))


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("kind", [None, "f16"], ids=["base", "f16"])
@pytest.mark.parametrize("M", [1, 6, 11, 40])
def test_acc4_exact_bit_exact(bits, kind, M):
    """On exactly representable activations accuracy level 4 is lossless: GPU == oracle at
    level 4 == oracle at level 0, bit for bit, on every path (M = 40 routes to the GEMM)."""
    N = 4096 if M == 11 else 192           # M = 11 takes 4 X rows per workgroup row
    case = acc4_exact_case(500 + 10 * bits + M, M, N, 320, bits, bits != 8, kind)
    want = oracle.f64_to_f16(oracle.matmul(dict(case, acc_level=4)))
    assert same_bits(want, oracle.f64_to_f16(oracle.matmul(case)))
    pw = dev_weight(case)
    for path in (0, 1, 2):
        assert same_bits(run(case, path, mnb.MNB_FLAG_ACC4, pw=pw), want), path


def test_acc4_differs_from_fp16_activations():
    """On random activations the quantization is visible (and within its tolerance of the
    FP16-activation result), so the flag really selects the int8 path."""
    case = si.make_random(333, 1, 4096, 2048, 4, True, None)
    pw = dev_weight(case)
    y4 = run(case, 0, mnb.MNB_FLAG_ACC4, pw=pw)
    y0 = run(case, 0, 0, pw=pw)
    assert not same_bits(y4, y0)
    compare(y4, oracle.matmul(case), max_abs=0.1, max_rel=0.02, what="acc4 vs fp16 activations")


# ------------------------------------------------------------------------------------------
# degenerate sizes, determinism, workspace reuse
# ------------------------------------------------------------------------------------------

def test_degenerate_sizes():
    case = si.make_random(100, 4, 70, 64, 4, True, "f16")
    pw = dev_weight(case)
    X = t16(case["X"])
    sentinel = torch.full((4, 70), 7.0, dtype=torch.float16, device=DEV)
    ws = mnb.workspace(DEV, 1 << 20)
    # M == 0: nothing written
    st = mnb.mnb_matmul(X.data_ptr(), pw.wq.data_ptr(), pw.sc.data_ptr(), pw.zp.data_ptr(), None,
                        sentinel.data_ptr(), 0, 70, 64, 4, 32, ws.data_ptr(), ws.numel(), 0)
    torch.cuda.synchronize()
    assert st == 0 and bool((sentinel == 7.0).all())
    # K == 0: zeros
    st = mnb.mnb_matmul(X.data_ptr(), pw.wq.data_ptr(), pw.sc.data_ptr(), None, None,
                        sentinel.data_ptr(), 4, 70, 0, 4, 32, ws.data_ptr(), ws.numel(), 0)
    torch.cuda.synchronize()
    assert st == 0 and bool((sentinel == 0).all())


def test_determinism_and_workspace_reuse():
    shapes = [(1, 8192, 2048, 4, False, "f16"), (1024, 1024, 1024, 4, True, "f16"), (1, 896, 896, 4, True, "q8"),
              (1, 49152, 576, 8, True, None), (3, 300, 512, 8, False, "f16")]
    cases = [si.make_random(110 + i, *s) for i, s in enumerate(shapes)]
    first = [run(c) for c in cases]
    for _ in range(3):                       # interleaved shapes share one workspace
        for c, y0 in zip(cases, first):
            assert np.array_equal(run(c), y0)
    for c, y0 in zip(cases, first):
        rows = list(range(c["M"])) if c["M"] <= 8 else [0, 5, c["M"] - 1]
        compare(y0[rows], oracle.matmul(rows_case(c, rows)), what="reuse %s" % (c["M"],))


def test_graph_replay_matches_eager():
    """Calls captured in a HIP graph (decode with the in-pass T handoff, small M with the T
    parts added by the small-M GEMV and with the T reduction in the projection, split-K
    prefill, a prefill whose last round of tiles splits K, accuracy level 4 with one and with
    four X rows per workgroup and on the GEMM path) give, on every replay, exactly the eager
    results, with eager calls on the same workspace between the replays: the library
    enqueues no memset and keeps its per-call state (the T epoch, the counters) in the
    workspace."""
    specs = [(1, 4096, 2048, 4, False, "f16", 0), (3, 1000, 1024, 4, True, "q8", 0),
             (200, 512, 1024, 8, True, "f16", 0), (1000, 4100, 640, 4, False, "f16", 0),
             (1, 896, 896, 4, True, None, mnb.MNB_FLAG_ACC4), (6, 4096, 640, 4, True, "f16", mnb.MNB_FLAG_ACC4),
             (300, 640, 512, 4, True, "f16", mnb.MNB_FLAG_ACC4), (3, 1000, 2560, 4, True, "q8", 0)]
    assert mnb.mnb_describe_route(6, 4096, 640, 4, 1, 1, mnb.mnb_options(0, mnb.MNB_FLAG_ACC4))[1].endswith("mr=4")
    assert "parts=4;" in mnb.mnb_describe_route(3, 1000, 1024, 4, 1, 2)[1]      # added by the GEMV
    assert "parts=10;" in mnb.mnb_describe_route(3, 1000, 2560, 4, 1, 2)[1]     # reduced in the projection
    assert " tail=" in mnb.mnb_describe_route(1000, 4100, 640, 4, 0, 1)[1]
    ws = torch.zeros(max(mnb.mnb_workspace_bytes(M, N, K, b, 32) for M, N, K, b, *_ in specs), dtype=torch.uint8,
                     device=DEV)
    calls = []
    for i, (M, N, K, bits, zp, ad, fl) in enumerate(specs):
        c = si.make_random(600 + i, M, N, K, bits, zp, ad, bias=i == 2)
        pw = dev_weight(c)
        a = dev_adapter(c["adapter"])
        X = t16(c["X"])
        b = t16(c["bias"]) if c.get("bias") is not None else None
        Y = torch.empty((M, N), dtype=torch.float16, device=DEV)
        calls.append((X, pw, a, fl, b, Y))
    def run_all():
        for X, pw, a, fl, b, Y in calls:
            mnb.matmul(X, pw, a, flags=fl, out=Y, ws=ws, bias=b)
    run_all()
    torch.cuda.synchronize()
    eager = [Y.clone() for *_, Y in calls]
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        run_all()
    for rep in range(4):
        for *_, Y in calls:
            Y.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        for (*_, Y), y0 in zip(calls, eager):
            assert torch.equal(Y.view(torch.int16), y0.view(torch.int16)), rep
        run_all()                                  # eager work on the same workspace between replays
        torch.cuda.synchronize()


def test_workspace_counters_return_to_zero():
    """The in-pass T handoff and the T projection's part reduction leave every counter of
    the workspace's control area at zero, never set the error word, and advance the epoch
    once per in-pass call."""
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    cases = [si.make_random(130, 1, 4096, 2048, 4, False, "f16"),      # in-pass T
             si.make_random(131, 4, 1000, 4096, 4, True, "q8"),        # small M: T reduced in the projection
             si.make_random(132, 2, 640, 9216, 8, False, "f16"),       # more than 4 T parts
             si.make_random(133, 1, 896, 896, 8, True, "q8")]          # in-pass T again
    inpass = 0
    for rep in range(3):
        for c in cases:
            pw = dev_weight(c)
            a = dev_adapter(c["adapter"])
            Y = torch.empty((c["M"], c["N"]), dtype=torch.float16, device=DEV)
            mnb.matmul(t16(c["X"]), pw, a, out=Y, ws=ws)
            inpass += c["M"] == 1
    torch.cuda.synchronize()
    ctrl = ws[:8448].cpu().numpy().view(np.int32)
    epoch, tdone, err = int(ctrl[0]), int(ctrl[1]), int(ctrl[2])
    assert err == 0 and tdone == 0
    # epoch: the tag of the last in-pass call, i.e. one past the previous tag per call
    assert epoch == inpass
    assert not ctrl[3:].any(), np.nonzero(ctrl[3:])[0][:8] + 3


def test_handoff_failure_reports_and_recovers():
    """The failure path of the in-pass decode handoff, forced from the host
    (MNB_FLAG_FAIL_HANDOFF: the row workgroups give up on T at once, as when their bounded
    wait expires): every output is NaN, the workspace's error word is reported once and
    cleared, the counters still return to zero and the next call is correct."""
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    c = si.make_random(140, 1, 4096, 2048, 4, False, "f16")
    pw = dev_weight(c)
    a = dev_adapter(c["adapter"])
    X = t16(c["X"])
    Y = torch.empty((1, c["N"]), dtype=torch.float16, device=DEV)
    assert mnb.workspace_error(ws) == mnb.MNB_OK
    mnb.matmul(X, pw, a, flags=mnb.MNB_FLAG_FAIL_HANDOFF, out=Y, ws=ws)
    torch.cuda.synchronize()
    assert torch.isnan(Y.float()).all()
    assert mnb.workspace_error(ws) == mnb.MNB_ERR_HANDOFF
    assert mnb.workspace_error(ws) == mnb.MNB_OK
    mnb.matmul(X, pw, a, out=Y, ws=ws)
    torch.cuda.synchronize()
    compare(Y.cpu().numpy().view(np.uint16), oracle.matmul(c), what="decode after a forced handoff failure")
    ctrl = ws[:8448].cpu().numpy().view(np.int32)
    assert int(ctrl[1]) == 0 and int(ctrl[2]) == 0 and not ctrl[3:].any()
