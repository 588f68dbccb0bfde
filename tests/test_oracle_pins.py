"""Pins for the CPU oracle: each checks it against something other than itself.

 - exact rational brute force on tiny inputs (fractions.Fraction);
 - the DequantizeLinear -> MatMul route through numpy's float64 matmul, the equivalence
   the page "Fuse DQ->MatMulNBits for shared initializers and skip outer-scope weights"
   (Description, Tests) states;
 - the closed form of that page's repro (codes 0, zero point 3, scale 0.02);
 - one-hot activations, which reduce the product to a single dequantized weight;
 - invariants: code == zero point gives exactly 0, an empty or zero adapter equals the
   base-only result bitwise ("[WebGPU] Fuse rank-32 quantized LoRA with MatMulNBits",
   commit list: empty adapters execute only the base projection), superposition of base
   and adapter, the default zero point, INT8 adapters equal to F16 adapters holding the
   same values;
 - binary16 conversion against numpy for every bit pattern and for rounding ties;
 - hand-derived bytes of the packed layout, and pack/unpack round trips;
 - packing from the DequantizeLinear layout ([K, N]) against numpy's transpose, and the
   same page's repro packed from its own layout.

``test_planted_mistakes_are_caught`` rebuilds the oracle with each deliberate mistake of
mnb_oracle.c (zero-point sign, dropped LoRA term, transposed operands, wrong block or
scale index, wrong default zero point, wrong nibble order, bias by row, untransposed
DQ-layout scales) and checks that at least one pin fails for each.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = os.path.join(HERE, "golden")


# ------------------------------------------------------------------------------------------
# independent helpers (exact arithmetic and numpy routes; no oracle code)
# ------------------------------------------------------------------------------------------

def _f16(bits) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _frac_matrix(vals) -> list:
    return [[Fraction(float(v)) for v in row] for row in np.atleast_2d(vals)]


def exact_result(case) -> list:
    """Exact rational Y for a tiny case, straight from DequantizeLinear then MatMul."""
    M, N, K, bits = case["M"], case["N"], case["K"], case["bits"]
    X = _frac_matrix(_f16(case["X"]))
    S = _frac_matrix(_f16(case["scales"]))
    codes = case["codes"]
    zp = case.get("zp")
    W = [[(int(codes[n, k]) - (int(zp[n, k // 32]) if zp is not None else 2 ** (bits - 1)))
          * S[n][k // 32] for k in range(K)] for n in range(N)]
    Y = [[sum(X[m][k] * W[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
    ad = case.get("adapter")
    if ad is not None:
        if ad["kind"] == "f16":
            A = _frac_matrix(_f16(ad["A"]))
            B = _frac_matrix(_f16(ad["B"]))
        else:
            sA = _frac_matrix(_f16(ad["A_scales"]))
            sB = _frac_matrix(_f16(ad["B_scales"]))
            A = [[int(ad["A"][k, r]) * sA[k // 32][r] for r in range(32)] for k in range(K)]
            B = [[int(ad["B"][r, n]) * sB[r // 32][n] for n in range(N)] for r in range(32)]
        T = [[sum(X[m][k] * A[k][r] for k in range(K)) for r in range(32)] for m in range(M)]
        for m in range(M):
            for n in range(N):
                Y[m][n] += sum(T[m][r] * B[r][n] for r in range(32))
    if case.get("bias") is not None:
        bias = [Fraction(float(v)) for v in _f16(case["bias"])]
        for m in range(M):
            for n in range(N):
                Y[m][n] += bias[n]
    return Y


def abs_terms(case) -> np.ndarray:
    """sum |x| |w| (+ |x| |a| |b|): the scale of rounding error for a plain FP64 sum."""
    X = np.abs(_f16(case["X"]))
    z = case["zp"].astype(np.float64) if case.get("zp") is not None else np.full(
        case["scales"].shape, 2.0 ** (case["bits"] - 1))
    W = np.abs((case["codes"].astype(np.float64) - np.repeat(z, 32, axis=1))
               * np.repeat(_f16(case["scales"]), 32, axis=1))
    tot = X @ W.T
    ad = case.get("adapter")
    if ad is not None:
        A, B = numpy_adapter(ad, case["K"], case["N"])
        tot = tot + (X @ np.abs(A)) @ np.abs(B)
    return tot


def numpy_adapter(ad, K, N):
    if ad["kind"] == "f16":
        return _f16(ad["A"]), _f16(ad["B"])
    A = ad["A"].astype(np.float64) * np.repeat(_f16(ad["A_scales"]), 32, axis=0)
    B = ad["B"].astype(np.float64) * np.repeat(_f16(ad["B_scales"]), 32, axis=0)
    return A, B


def numpy_dq_matmul(case) -> np.ndarray:
    """DequantizeLinear (numpy broadcasting) followed by numpy's float64 matmul."""
    bits = case["bits"]
    q = case["codes"].astype(np.float64)
    z = case["zp"].astype(np.float64) if case.get("zp") is not None else np.full(
        case["scales"].shape, 2.0 ** (bits - 1))
    W = (q - np.repeat(z, 32, axis=1)) * np.repeat(_f16(case["scales"]), 32, axis=1)
    X = _f16(case["X"])
    Y = X @ W.T
    if case.get("adapter") is not None:
        A, B = numpy_adapter(case["adapter"], case["K"], case["N"])
        Y = Y + (X @ A) @ B
    if case.get("bias") is not None:
        Y = Y + _f16(case["bias"])[None, :]
    return Y


# ------------------------------------------------------------------------------------------
# pins: each takes the oracle library so the mutation test can run them on planted copies
# ------------------------------------------------------------------------------------------

TINY = [  # (seed, M, N, K, bits, zp, adapter, bias)
    (1, 1, 5, 32, 4, True, None, False),
    (2, 2, 8, 64, 4, False, "f16", False),
    (3, 3, 7, 64, 8, True, "q8", True),
    (4, 2, 6, 32, 8, False, None, True),
    (5, 1, 3, 64, 4, True, "q8", False),
    (6, 2, 4, 32, 4, True, "f16", True),
    (7, 2, 5, 64, 2, True, "f16", False),
    (8, 1, 6, 96, 2, False, "q8", True),
]


def pin_exact_bruteforce(lib):
    for seed, M, N, K, bits, zp, ad, bias in TINY:
        case = si.make_random(seed, M, N, K, bits, zp, ad, bias=bias)
        ex = exact_result(case)
        got = oracle.matmul(case, lib)
        bound = 1e-13 * (abs_terms(case) + (np.abs(_f16(case["bias"]))[None, :] if bias else 0)) + 1e-300
        for m in range(M):
            for n in range(N):
                err = abs(Fraction(float(got[m, n])) - ex[m][n])
                assert err <= Fraction(float(bound[m, n])), (seed, m, n, float(err))


def pin_numpy_dq_matmul(lib):
    for seed, (M, N, K, bits, zp, ad, bias) in enumerate([(3, 70, 96, 4, True, "f16", False),
                                                          (2, 65, 160, 8, True, "q8", True),
                                                          (4, 33, 64, 4, False, "q8", False),
                                                          (1, 130, 128, 8, False, None, True),
                                                          (2, 67, 224, 2, True, "f16", True),
                                                          (3, 40, 96, 2, False, None, False)]):
        case = si.make_random(100 + seed, M, N, K, bits, zp, ad, bias=bias)
        got = oracle.matmul(case, lib)
        ref = numpy_dq_matmul(case)
        scale = abs_terms(case) + (np.abs(_f16(case["bias"]))[None, :] if bias else 0)
        assert np.all(np.abs(got - ref) <= 1e-12 * scale + 1e-300), seed


def pin_empty_weights_bias(lib):
    """K == 0 (empty packed weights): Y is the broadcast bias exactly, or zeros (PR #33370
    page, commit list: the output keeps its logical shape and holds zeros or the bias)."""
    r = np.random.default_rng(9)
    for M, N, bits in ((3, 5, 4), (1, 70, 8), (2, 9, 2)):
        bias = r.standard_normal(N).astype(np.float16).view(np.uint16)
        case = dict(M=M, N=N, K=0, bits=bits, X=np.zeros((M, 0), np.uint16),
                    codes=np.zeros((N, 0), np.uint8), scales=np.zeros((N, 0), np.uint16), zp=None,
                    adapter=None, bias=bias)
        got = oracle.matmul(case, lib)
        assert np.array_equal(got, np.broadcast_to(_f16(bias), (M, N)))
        case["bias"] = None
        assert not oracle.matmul(case, lib).any()


def pin_p5_closed_form(lib):
    kv = {}
    for line in open(os.path.join(GOLD, "p5_constant_codes.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            kv[k] = int(v, 0)
    K, N, bits = kv["K"], kv["N"], kv["bits"]
    s = Fraction(kv["scale_exact_numerator"], kv["scale_exact_denominator"])
    assert Fraction(float(_f16(np.uint16(kv["scale_f16"])))) == s
    M = 3
    r = np.random.default_rng(7)
    X = si.to_f16_bits(r.standard_normal((M, K)))
    case = dict(M=M, N=N, K=K, bits=bits, X=X,
                codes=np.full((N, K), kv["code"], np.uint8),
                scales=np.full((N, K // 32), kv["scale_f16"], np.uint16),
                zp=np.full((N, K // 32), kv["zero_point"], np.uint8), adapter=None)
    got = oracle.matmul(case, lib)
    Xf = _frac_matrix(_f16(X))
    for m in range(M):
        want = -3 * s * sum(Xf[m])
        assert np.all(got[m] == got[m, 0])                      # identical columns
        bound = 1e-13 * float(3 * s * sum(abs(v) for v in Xf[m]))
        assert abs(Fraction(float(got[m, 0])) - want) <= Fraction(bound)


def pin_one_hot(lib):
    for bits, zp in ((4, True), (4, False), (8, True), (8, False), (2, True), (2, False)):
        N, K = 67, 96
        case = si.make_random(200 + bits, 1, N, K, bits, zp, None)
        for k in (0, 1, 2, 7, 8, 15, 16, 31, 32, 33, 63, 64, K - 1):
            for xv in (1.0, -0.5, 2.0 ** -10):
                X = np.zeros((1, K), np.float16)
                X[0, k] = xv
                c = dict(case, X=X.view(np.uint16))
                got = oracle.matmul(c, lib)[0]
                z = case["zp"][:, k // 32].astype(np.float64) if zp else 2.0 ** (bits - 1)
                want = xv * (case["codes"][:, k].astype(np.float64) - z) * _f16(case["scales"][:, k // 32])
                assert np.array_equal(got, want), (bits, zp, k)


def pin_code_equals_zero_point(lib):
    for bits, zp in ((4, True), (8, True), (4, False), (8, False), (2, True), (2, False)):
        case = si.make_random(300 + bits, 3, 40, 96, bits, zp, "f16")
        z = case["zp"] if zp else np.full(case["scales"].shape, 2 ** (bits - 1), np.uint8)
        codes = np.repeat(z, 32, axis=1).astype(np.uint8)
        base = oracle.matmul(dict(case, codes=codes, adapter=None), lib)
        assert np.all(base == 0.0)
        withl = oracle.matmul(dict(case, codes=codes), lib)
        A, B = numpy_adapter(case["adapter"], case["K"], case["N"])
        lo = (_f16(case["X"]) @ A) @ B
        assert np.allclose(withl, lo, rtol=1e-12, atol=1e-15)
        assert np.any(withl != 0.0)


def pin_empty_and_zero_adapter(lib):
    case = si.make_random(400, 2, 50, 64, 4, True, "f16")
    base = oracle.matmul(dict(case, adapter=None), lib)
    ad = case["adapter"]
    empties = [dict(ad, rank=0), dict(ad, A_null=True), dict(ad, B_null=True),
               dict(ad, A=np.zeros_like(ad["A"])), dict(ad, B=np.zeros_like(ad["B"]))]
    for e in empties:
        assert np.array_equal(oracle.matmul(dict(case, adapter=e), lib), base)
    full = oracle.matmul(case, lib)
    assert not np.array_equal(full, base)


def pin_superposition(lib):
    for bits, ad in ((4, "f16"), (8, "q8")):
        case = si.make_random(500 + bits, 3, 45, 128, bits, True, ad)
        full = oracle.matmul(case, lib)
        base = oracle.matmul(dict(case, adapter=None), lib)
        codes0 = np.repeat(case["zp"], 32, axis=1).astype(np.uint8)
        lora = oracle.matmul(dict(case, codes=codes0), lib)
        assert np.all(np.abs(full - (base + lora)) <= 1e-12 * abs_terms(case) + 1e-300)


def pin_default_zero_point(lib):
    for bits in (2, 4, 8):
        case = si.make_random(600 + bits, 2, 30, 64, bits, False, None)
        explicit = dict(case, zp=np.full(case["scales"].shape, 2 ** (bits - 1), np.uint8))
        assert np.array_equal(oracle.matmul(case, lib), oracle.matmul(explicit, lib))


def pin_q8_equals_f16(lib):
    K, N = 96, 40
    r = np.random.default_rng(8)
    vA = r.integers(-127, 128, size=(K, 32)).astype(np.int8)
    vB = r.integers(-127, 128, size=(32, N)).astype(np.int8)
    sA = si.to_f16_bits(2.0 ** r.integers(-12, -6, size=(K // 32, 32)))
    sB = si.to_f16_bits(2.0 ** r.integers(-12, -6, size=(1, N)))
    Af = vA.astype(np.float64) * np.repeat(_f16(sA), 32, axis=0)      # fp16-exact values
    Bf = vB.astype(np.float64) * _f16(sB)
    case = si.make_random(700, 2, N, K, 4, True, None)
    q8 = dict(case, adapter=dict(kind="q8", A=vA, A_scales=sA, B=vB, B_scales=sB))
    f16 = dict(case, adapter=dict(kind="f16", A=si.to_f16_bits(Af), B=si.to_f16_bits(Bf)))
    assert np.array_equal(_f16(si.to_f16_bits(Af)), Af)
    assert np.array_equal(oracle.matmul(q8, lib), oracle.matmul(f16, lib))


def _read_pack_examples():
    ex, cur = [], None
    for line in open(os.path.join(GOLD, "pack_layout_examples.txt")):
        t = line.split()
        if not t or t[0].startswith("#"):
            continue
        if t[0] == "example":
            cur = dict(name=t[1], N=int(t[3]), K=int(t[5]), bits=int(t[7]), wq=[], sc=[], zp=[])
            ex.append(cur)
        elif t[0] == "wq_size":
            cur["wq_size"] = int(t[1])
        else:
            cur[t[0]].append((int(t[1]), [int(v, 16) for v in t[2:]]))
    return ex


def pack_example_inputs(name):
    if name == "A":
        k = np.arange(32)
        codes = np.stack([k % 16, 15 - k % 16]).astype(np.uint8)
        return codes, np.array([[0x3C00], [0x4000]], np.uint16), np.array([[3], [12]], np.uint8)
    if name == "C":
        n, k = np.arange(5)[:, None], np.arange(96)[None, :]
        codes = ((k + n) % 4).astype(np.uint8)
        scales = np.repeat((0x3C00 + np.arange(5))[:, None], 3, axis=1).astype(np.uint16)
        zp = np.repeat((np.arange(5) % 4)[:, None], 3, axis=1).astype(np.uint8)
        return codes, scales, zp
    codes = (100 + np.arange(32)).astype(np.uint8)[None, :]
    return codes, np.array([[0x2E66]], np.uint16), np.array([[128]], np.uint8)


def pin_pack_layout(lib):
    for ex in _read_pack_examples():
        codes, scales, zp = pack_example_inputs(ex["name"])
        wq, sc, zpp = oracle.pack(codes, scales, zp, ex["N"], ex["K"], ex["bits"], lib)
        assert wq.size == ex["wq_size"]
        for off, vals in ex["wq"]:
            assert list(wq[off:off + len(vals)]) == vals, (ex["name"], off)
        for off, vals in ex["sc"]:
            assert list(sc[off:off + len(vals)]) == vals
        for off, vals in ex["zp"]:
            assert list(zpp[off:off + len(vals)]) == vals


def pin_pack_roundtrip(lib):
    for bits in (2, 4, 8):
        for N, K, zp in ((1, 32, True), (64, 64, False), (130, 96, True), (200, 32, True)):
            case = si.make_random(800 + N, 1, N, K, bits, zp, None)
            wq, sc, zpp = oracle.pack(case["codes"], case["scales"], case["zp"], N, K, bits, lib)
            c2, s2, z2 = oracle.unpack(wq, sc, zpp, N, K, bits, lib)
            assert np.array_equal(c2, case["codes"]) and np.array_equal(s2, case["scales"])
            if zp:
                assert np.array_equal(z2, case["zp"])


def pin_pack_from_dq_layout(lib):
    """Packing from the DequantizeLinear layout (codes [K, N], scales / zero points
    [K/32, N]; PR #33800 page, Description: the fusion writes transposed initializers)
    equals packing numpy's transpose of the same tensors, byte for byte."""
    r = np.random.default_rng(12)
    for N, K, bits, zp in ((70, 96, 4, True), (33, 64, 8, True), (5, 160, 4, False), (130, 32, 8, False),
                           (66, 96, 2, True), (3, 32, 2, False)):
        codes_kn = r.integers(0, 1 << bits, size=(K, N), dtype=np.uint8)
        scales_kn = r.integers(0x1000, 0x3C00, size=(K // 32, N)).astype(np.uint16)
        zp_kn = r.integers(0, 1 << bits, size=(K // 32, N)).astype(np.uint8) if zp else None
        got = oracle.pack_kn(codes_kn, scales_kn, zp_kn, N, K, bits, lib)
        want = oracle.pack(np.transpose(codes_kn), np.transpose(scales_kn),
                           None if zp_kn is None else np.transpose(zp_kn), N, K, bits, lib)
        for g, w in zip(got, want):
            assert (g is None and w is None) or np.array_equal(g, w)


def pin_p5_closed_form_dq_layout(lib):
    """The PR #33800 repro in its own DequantizeLinear layout (w_q [K, N] = 0, scalar scale
    0.02 and zero point 3, broadcast to every block): packed from [K, N], every output is
    -3 * s * sum_k x[k], the same in every column."""
    kv = {}
    for line in open(os.path.join(GOLD, "p5_constant_codes.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            kv[k] = int(v, 0)
    K, N, bits = kv["K"], kv["N"], kv["bits"]
    s = Fraction(kv["scale_exact_numerator"], kv["scale_exact_denominator"])
    wq, sc, zpp = oracle.pack_kn(np.full((K, N), kv["code"], np.uint8),
                                 np.full((K // 32, N), kv["scale_f16"], np.uint16),
                                 np.full((K // 32, N), kv["zero_point"], np.uint8), N, K, bits, lib)
    codes, scales, zp = oracle.unpack(wq, sc, zpp, N, K, bits, lib)
    M = 2
    X = si.to_f16_bits(np.random.default_rng(8).standard_normal((M, K)))
    got = oracle.matmul(dict(M=M, N=N, K=K, bits=bits, X=X, codes=codes, scales=scales, zp=zp,
                             adapter=None), lib)
    Xf = _frac_matrix(_f16(X))
    for m in range(M):
        want = -3 * s * sum(Xf[m])
        assert np.all(got[m] == got[m, 0])
        bound = 1e-13 * float(3 * s * sum(abs(v) for v in Xf[m]))
        assert abs(Fraction(float(got[m, 0])) - want) <= Fraction(bound)


def _acc4_representable_x(r, M, K):
    """X whose every block is c * 2^-e with integer |c| <= 127, max |c| = 127 (or all zero):
    then 127 / amax = 2^e and amax / 127 = 2^-e exactly, so block quantization is lossless."""
    X = np.zeros((M, K), np.float64)
    for m in range(M):
        for b in range(K // 32):
            if (m + b) % 7 == 3:
                continue                                   # an all-zero block
            c = r.integers(-127, 128, size=32)
            c[r.integers(0, 32)] = 127 * (1 if r.integers(0, 2) else -1)
            X[m, 32 * b:32 * b + 32] = c * 2.0 ** -int(r.integers(7, 13))
    return si.to_f16_bits(X)


def pin_acc4_lossless_when_representable(lib):
    """Accuracy level 4 on activations that block quantization represents exactly equals
    the FP16-activation result bit for bit (same products, same order)."""
    r = np.random.default_rng(44)
    for bits, zp, ad in ((4, True, "f16"), (8, True, None), (2, False, "q8"), (4, False, None)):
        case = si.make_random(440 + bits, 3, 37, 160, bits, zp, ad)
        case["X"] = _acc4_representable_x(r, 3, 160)
        assert np.array_equal(oracle.matmul(dict(case, acc_level=4), lib), oracle.matmul(case, lib))


def pin_acc4_error_bound(lib):
    """Round-to-nearest block quantization moves each activation by at most half a step
    (sx / 2, sx = amax / 127 in FP32): |Y4 - Y| <= sum_k |w[n,k]| sx(k) / 2, and it does move
    random activations."""
    for bits, zp in ((4, True), (8, True), (2, False)):
        case = si.make_random(450 + bits, 3, 41, 192, bits, zp, None)
        y0 = oracle.matmul(case, lib)
        y4 = oracle.matmul(dict(case, acc_level=4), lib)
        x = _f16(case["X"])
        amax = np.abs(x.reshape(3, -1, 32)).max(axis=2).astype(np.float32)
        step = np.repeat((amax / np.float32(127.0)).astype(np.float64), 32, axis=1)        # [M, K]
        z = case["zp"].astype(np.float64) if zp else np.full(case["scales"].shape, 2.0 ** (bits - 1))
        W = np.abs((case["codes"] - np.repeat(z, 32, axis=1)) * np.repeat(_f16(case["scales"]), 32, axis=1))
        bound = (step / 2) @ W.T
        assert np.all(np.abs(y4 - y0) <= bound * (1 + 1e-9) + 1e-12)
        assert np.any(y4 != y0)


def pin_acc4_lora_uses_fp16_x(lib):
    """With all codes equal to their zero points the base is exactly 0 at any accuracy
    level, so accuracy level 4 leaves exactly the LoRA term, which takes the original FP16
    X (PR #33370 page, commit list)."""
    for kind in ("f16", "q8"):
        case = si.make_random(460, 2, 30, 96, 4, True, kind)
        case["codes"] = np.repeat(case["zp"], 32, axis=1).astype(np.uint8)
        assert np.array_equal(oracle.matmul(dict(case, acc_level=4), lib), oracle.matmul(case, lib))


PINS = [pin_exact_bruteforce, pin_numpy_dq_matmul, pin_p5_closed_form, pin_one_hot,
        pin_code_equals_zero_point, pin_empty_and_zero_adapter, pin_superposition,
        pin_default_zero_point, pin_q8_equals_f16, pin_pack_layout, pin_pack_roundtrip,
        pin_empty_weights_bias, pin_pack_from_dq_layout, pin_p5_closed_form_dq_layout,
        pin_acc4_lossless_when_representable, pin_acc4_error_bound, pin_acc4_lora_uses_fp16_x]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.load())


# ------------------------------------------------------------------------------------------
# binary16 conversion against numpy (a library routine)
# ------------------------------------------------------------------------------------------

def test_f16_decode_every_pattern():
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f64(allb)
    want = allb.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_f16_round_nearest_even():
    allb = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    v = allb.view(np.float16).astype(np.float64)
    nxt = np.append(v[1:], 65536.0)
    mids = (v + nxt) / 2                                          # exact ties
    r = np.random.default_rng(3)
    samples = np.concatenate([v, mids, -mids, mids * (1 + 2.0 ** -40), mids * (1 - 2.0 ** -40),
                              r.standard_normal(20000) * 10.0 ** r.integers(-9, 5, 20000),
                              [0.0, -0.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -25, 2.0 ** -26]])
    got = oracle.f64_to_f16(samples)
    want = samples.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------------------------------
# mutation check: every planted mistake is caught by at least one pin
# ------------------------------------------------------------------------------------------

MUTATIONS = {1: "zero-point sign", 2: "LoRA term dropped", 3: "scale index transposed",
             4: "block index off by one", 5: "A transposed", 6: "default zero point 0",
             7: "natural nibble order", 8: "X transposed", 9: "B transposed",
             10: "INT8 A scale ignores rank column", 11: "bias indexed by the row",
             12: "DQ-layout scales not transposed", 13: "acc4 with 128 levels",
             14: "acc4 T from quantized X"}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS), ids=lambda m: MUTATIONS[m])
def test_planted_mistakes_are_caught(mutation, tmp_path):
    path = obuild.build(mutation=mutation, out=str(tmp_path / ("liboracle_m%d.so" % mutation)))
    lib = oracle.load(path)
    assert lib.mnbo_mutation() == mutation
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "mutation %d (%s) passed every pin" % (mutation, MUTATIONS[mutation])
