"""Seeded synthetic inputs for MatMulNBits with an optional rank-32 LoRA term.

This module is the only code shared by the CPU oracle side (tests, cpu baseline)
and the GPU side (tests, bench). It draws random numbers and shapes them into the
logical tensors of the operation; it holds none of the operation's arithmetic
(no dequantization, no products, no packing).

Logical tensors (all little-endian numpy arrays):
  X       uint16 [M, K]      IEEE binary16 bit patterns of the activations
  codes   uint8  [N, K]      one quantized weight code per byte, value < 2**bits
  scales  uint16 [N, K/32]   binary16 bit patterns, one scale per block of 32 along K
  zp      uint8  [N, K/32]   one zero point per block, or None (default zero point)
  adapter dict or None:
    kind 'f16': A uint16 [K, 32], B uint16 [32, N]   (binary16 bit patterns)
    kind 'q8' : A int8 [K, 32] + A_scales uint16 [K/32, 32],
                B int8 [32, N] + B_scales uint16 [1, N]

The workloads follow the shapes of the projections discussed on the pages (the
onnxruntime pull requests "[WebGPU] Fuse rank-32 quantized LoRA with
MatMulNBits" and "Fuse DQ->MatMulNBits for shared initializers and skip
outer-scope weights"): a 896x896 tiny decode, an 8192x2048 MLP up-projection, a
4096x4096 prefill projection, the 49152x576 tied lm_head, and a 9728x2560
batched prefill with block-32 INT8 adapters.  The models and datasets those
pages measure are not available; these seeded tensors stand in for them.

Random bounds are half-open on the high side (numpy ``integers(lo, hi)``), so
the largest code 2**bits - 1 occurs.
"""
from __future__ import annotations

import numpy as np

SEED_ROOT = 20261202
RANK = 32
BLOCK = 32

# tensor ids for the seed sequence
_T_X, _T_CODES, _T_SCALES, _T_ZP, _T_A, _T_B = range(6)


def rng_for(cfg: int, tensor_id: int, extra: int = 0) -> np.random.Generator:
    """A generator that depends only on (cfg, tensor_id, extra)."""
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, cfg, tensor_id, extra]))


def to_f16_bits(a) -> np.ndarray:
    """Round float data to binary16 (round-to-nearest-even, numpy) and return the bit patterns."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32).astype(np.float16)).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def normal_f16(rng, shape, std=1.0) -> np.ndarray:
    return to_f16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def uniform_f16(rng, shape, lo, hi) -> np.ndarray:
    return to_f16_bits(rng.uniform(lo, hi, size=shape).astype(np.float32))


def quantize_q8_blocks(vals: np.ndarray, axis: int):
    """Symmetric int8 blocks of 32 along ``axis`` (data generation for the Q8 adapters).

    Per block: s = fp16(max|v| / 127), q = clip(rint(v / s), -127, 127); an all-zero
    block gets s = 0 and q = 0.  Returns (int8 codes, uint16 scale bits) with the
    scale array shaped like ``vals`` but with ``axis`` divided by 32.
    """
    v = np.moveaxis(np.asarray(vals, dtype=np.float32), axis, 0)
    n0 = v.shape[0]
    assert n0 % BLOCK == 0
    vb = v.reshape(n0 // BLOCK, BLOCK, *v.shape[1:])
    amax = np.abs(vb).max(axis=1)
    s16 = (amax / np.float32(127.0)).astype(np.float16)
    s32 = s16.astype(np.float32)
    safe = np.where(s32 > 0, s32, np.float32(1.0))
    q = np.rint(vb / safe[:, None]).clip(-127, 127)
    q = np.where(s32[:, None] > 0, q, 0).astype(np.int8)
    q = np.moveaxis(q.reshape(v.shape), 0, axis)
    s16 = np.moveaxis(s16, 0, axis)
    return np.ascontiguousarray(q), np.ascontiguousarray(s16).view(np.uint16)


# --------------------------------------------------------------------------------------
# The five workloads.
# --------------------------------------------------------------------------------------

CONFIGS = {
    1: dict(name="tiny decode 896x896 int4 explicit-zp + F16 LoRA", M=1, N=896, K=896, bits=4,
            s_lo=0.001, s_hi=0.02, zp=(0, 16), adapter="f16"),
    2: dict(name="decode GEMV 8192x2048 int4 default-zp + F16 LoRA", M=1, N=8192, K=2048, bits=4,
            s_lo=0.001, s_hi=0.02, zp=None, adapter="f16"),
    3: dict(name="prefill GEMM 1024x4096x4096 int4 explicit-zp + F16 LoRA", M=1024, N=4096, K=4096,
            bits=4, s_lo=0.001, s_hi=0.02, zp=(0, 16), adapter="f16"),
    4: dict(name="tied lm_head 49152x576 int8 explicit-zp, no adapter", M=8, N=49152, K=576, bits=8,
            s_lo=1e-4, s_hi=4e-3, zp=(100, 157), adapter=None),
    5: dict(name="batched prefill 1024x9728x2560 int4 default-zp + Q8 LoRA (half-zero B)", M=1024,
            N=9728, K=2560, bits=4, s_lo=0.001, s_hi=0.02, zp=None, adapter="q8"),
}


def make_weights(cfg: int, N: int, K: int, bits: int, s_lo: float, s_hi: float, zp):
    """codes [N,K], scales [N,K/32] (fp16 bits), zp [N,K/32] or None."""
    assert K % BLOCK == 0
    codes = rng_for(cfg, _T_CODES).integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    scales = uniform_f16(rng_for(cfg, _T_SCALES), (N, K // BLOCK), s_lo, s_hi)
    zpa = None
    if zp is not None:
        zpa = rng_for(cfg, _T_ZP).integers(zp[0], zp[1], size=(N, K // BLOCK), dtype=np.uint8)
    return codes, scales, zpa


def make_adapter(cfg: int, kind, N: int, K: int, half_zero_b: bool = False):
    if kind is None:
        return None
    a_f = rng_for(cfg, _T_A).standard_normal((K, RANK), dtype=np.float32) * np.float32(0.02)
    b_f = rng_for(cfg, _T_B).standard_normal((RANK, N), dtype=np.float32) * np.float32(0.02)
    if kind == "f16":
        return dict(kind="f16", A=to_f16_bits(a_f), B=to_f16_bits(b_f))
    if kind == "q8":
        qa, sa = quantize_q8_blocks(a_f, axis=0)          # blocks of 32 along K
        qb, sb = quantize_q8_blocks(b_f, axis=0)          # one block of 32 along r per column
        if half_zero_b:
            qb[:, N // 2:] = 0                            # B zero in the upper half of the columns
        return dict(kind="q8", A=qa, A_scales=sa, B=qb, B_scales=sb)
    raise ValueError(kind)


def make_config(cfg: int, M: int | None = None, adapter: str | None | bool = True):
    """All inputs of one workload.  ``M`` overrides the row count (prefix rows of the
    same X); ``adapter=False`` drops the adapter, a string forces a kind."""
    c = CONFIGS[cfg]
    Mx = c["M"] if M is None else M
    Mgen = max(Mx, c["M"])
    X = normal_f16(rng_for(cfg, _T_X), (Mgen, c["K"]))[:Mx]
    codes, scales, zp = make_weights(cfg, c["N"], c["K"], c["bits"], c["s_lo"], c["s_hi"], c["zp"])
    kind = c["adapter"] if adapter is True else (None if adapter is False else adapter)
    ad = make_adapter(cfg, kind, c["N"], c["K"], half_zero_b=(cfg == 5))
    return dict(cfg=cfg, name=c["name"], M=Mx, N=c["N"], K=c["K"], bits=c["bits"],
                X=np.ascontiguousarray(X), codes=codes, scales=scales, zp=zp, adapter=ad)


def make_random(seed: int, M: int, N: int, K: int, bits: int, with_zp: bool, adapter=None,
                s_lo=None, s_hi=None, x_std=1.0, bias=False):
    """Generic seeded case for tests (shapes not tied to a workload).  Scales default to the
    decode/prefill range U[0.001, 0.02] for 4-bit (and 2-bit) and the lm_head range
    U[1e-4, 4e-3] for 8-bit weights; for 8-bit with K > 576 the range shrinks by sqrt(576/K) so that the
    output spread stays at the lm_head's (sigma(Y) ~ 4), inside the range where the fp16
    output rounding (half an ulp) stays well below the 2e-2 max-abs tolerance."""
    if s_lo is None:
        s_lo, s_hi = (0.001, 0.02) if bits in (2, 4) else (1e-4, 4e-3)
        if bits == 8 and K > 576:
            f = float(np.sqrt(576.0 / K))
            s_lo, s_hi = s_lo * f, s_hi * f
    r = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, 1000, seed, M, N, K, bits]))
    X = normal_f16(r, (M, K), std=x_std)
    codes = r.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    scales = uniform_f16(r, (N, K // BLOCK), s_lo, s_hi)
    zp = r.integers(0, 1 << bits, size=(N, K // BLOCK), dtype=np.uint8) if with_zp else None
    ad = None
    if adapter == "f16":
        ad = dict(kind="f16", A=normal_f16(r, (K, RANK), 0.02), B=normal_f16(r, (RANK, N), 0.02))
    elif adapter == "q8":
        a_f = r.standard_normal((K, RANK), dtype=np.float32) * np.float32(0.02)
        b_f = r.standard_normal((RANK, N), dtype=np.float32) * np.float32(0.02)
        qa, sa = quantize_q8_blocks(a_f, 0)
        qb, sb = quantize_q8_blocks(b_f, 0)
        ad = dict(kind="q8", A=qa, A_scales=sa, B=qb, B_scales=sb)
    case = dict(M=M, N=N, K=K, bits=bits, X=X, codes=codes, scales=scales, zp=zp, adapter=ad)
    if bias:   # broadcast bias fp16 [N] ~ N(0, 0.5), drawn after everything else
        case["bias"] = normal_f16(r, (N,), std=0.5)
    return case
