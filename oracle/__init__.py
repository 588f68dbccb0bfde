"""CPU oracle for MatMulNBits (+ rank-32 LoRA), FP64.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product path (``blockwise_bit_quantized_amd``) never does, and
nothing here imports the product package.  See ``mnb_oracle.c`` for the definition it
follows and the pages it cites.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_P = C.c_void_p
_libs: dict[str, C.CDLL] = {}


def load(path: str | None = None) -> C.CDLL:
    """Load (building if absent) the oracle library, or a mutated copy at ``path``.  The
    environment variable MNB_ORACLE_LIB names another build of it (the sanitizer build)."""
    path = path or os.environ.get("MNB_ORACLE_LIB") or _build.LIB
    if path in _libs:
        return _libs[path]
    if path == _build.LIB and (not os.path.exists(path) or
                               os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
        _build.build()          # absent, or older than its source (a CPU build of seconds)
    lib = C.CDLL(path)
    lib.mnbo_matmul.argtypes = [C.c_int] * 4 + [_P] * 4 + [C.c_int, C.c_int] + [_P] * 6 + [C.c_int]
    lib.mnbo_matmul.restype = C.c_int
    lib.mnbo_pack.argtypes = [C.c_int] * 3 + [_P] * 6
    lib.mnbo_pack.restype = C.c_int
    lib.mnbo_pack_kn.argtypes = [C.c_int] * 3 + [_P] * 6
    lib.mnbo_pack_kn.restype = C.c_int
    lib.mnbo_unpack.argtypes = [C.c_int] * 3 + [_P] * 6
    lib.mnbo_unpack.restype = C.c_int
    lib.mnbo_packed_sizes.argtypes = [C.c_int] * 4 + [C.POINTER(C.c_long)] * 3
    lib.mnbo_packed_sizes.restype = C.c_int
    lib.mnbo_f16_to_f64.argtypes = [_P, _P, C.c_long]
    lib.mnbo_f64_to_f16.argtypes = [_P, _P, C.c_long]
    lib.mnbo_mutation.restype = C.c_int
    _libs[path] = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_P)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def f16_to_f64(bits, lib=None) -> np.ndarray:
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float64)
    (lib or load()).mnbo_f16_to_f64(_ptr(b), _ptr(out), b.size)
    return out


def f64_to_f16(vals, lib=None) -> np.ndarray:
    v = _c(vals, np.float64)
    out = np.empty(v.shape, np.uint16)
    (lib or load()).mnbo_f64_to_f16(_ptr(v), _ptr(out), v.size)
    return out


def matmul(case: dict, lib=None) -> np.ndarray:
    """FP64 Y[M,N] for a case dict (see ``seeded_inputs``); ``acc_level`` 4 selects int8
    block-quantized activations for the base product."""
    lib = lib or load()
    M, N, K, bits = case["M"], case["N"], case["K"], case["bits"]
    X = _c(case["X"], np.uint16)
    codes = _c(case["codes"], np.uint8)
    scales = _c(case["scales"], np.uint16)
    zp = _c(case.get("zp"), np.uint8)
    ad = case.get("adapter")
    kind, rank, A, sA, B, sB = 0, 0, None, None, None, None
    if ad is not None:
        kind = {"f16": 1, "q8": 2}[ad["kind"]]
        rank = ad.get("rank", 32)
        if ad["kind"] == "f16":
            A, B = _c(ad["A"], np.uint16), _c(ad["B"], np.uint16)
        else:
            A, B = _c(ad["A"], np.int8), _c(ad["B"], np.int8)
            sA, sB = _c(ad["A_scales"], np.uint16), _c(ad["B_scales"], np.uint16)
        if ad.get("A_null"):
            A = None
        if ad.get("B_null"):
            B = None
    bias = _c(case.get("bias"), np.uint16)
    Y = np.zeros((M, N), np.float64)
    rc = lib.mnbo_matmul(M, N, K, bits, _ptr(X), _ptr(codes), _ptr(scales), _ptr(zp), kind, rank,
                         _ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(bias), _ptr(Y), int(case.get("acc_level", 0)))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return Y


def packed_sizes(N, K, bits, has_zp, lib=None):
    lib = lib or load()
    a, b, c = C.c_long(), C.c_long(), C.c_long()
    if lib.mnbo_packed_sizes(N, K, bits, int(bool(has_zp)), C.byref(a), C.byref(b), C.byref(c)):
        raise ValueError("bad sizes")
    return a.value, b.value, c.value


def pack(codes, scales, zp, N, K, bits, lib=None):
    """(wq uint8[...], sc uint16[...], zp uint8[...] or None) in the device layout."""
    lib = lib or load()
    wqb, scb, zpb = packed_sizes(N, K, bits, zp is not None, lib)
    wq = np.zeros(wqb, np.uint8)
    sc = np.zeros(scb // 2, np.uint16)
    zpp = np.zeros(zpb, np.uint8) if zp is not None else None
    rc = lib.mnbo_pack(N, K, bits, _ptr(_c(codes, np.uint8)), _ptr(_c(scales, np.uint16)),
                       _ptr(_c(zp, np.uint8)), _ptr(wq), _ptr(sc), _ptr(zpp))
    if rc:
        raise ValueError("pack failed")
    return wq, sc, zpp


def pack_kn(codes_kn, scales_kn, zp_kn, N, K, bits, lib=None):
    """Pack from the DequantizeLinear layout: codes [K, N], scales / zero points [K/32, N]."""
    lib = lib or load()
    wqb, scb, zpb = packed_sizes(N, K, bits, zp_kn is not None, lib)
    wq = np.zeros(wqb, np.uint8)
    sc = np.zeros(scb // 2, np.uint16)
    zpp = np.zeros(zpb, np.uint8) if zp_kn is not None else None
    rc = lib.mnbo_pack_kn(N, K, bits, _ptr(_c(codes_kn, np.uint8)), _ptr(_c(scales_kn, np.uint16)),
                          _ptr(_c(zp_kn, np.uint8)), _ptr(wq), _ptr(sc), _ptr(zpp))
    if rc:
        raise ValueError("pack_kn failed")
    return wq, sc, zpp


def unpack(wq, sc, zpp, N, K, bits, lib=None):
    lib = lib or load()
    codes = np.zeros((N, K), np.uint8)
    scales = np.zeros((N, K // 32), np.uint16)
    zp = np.zeros((N, K // 32), np.uint8) if zpp is not None else None
    rc = lib.mnbo_unpack(N, K, bits, _ptr(_c(wq, np.uint8)), _ptr(_c(sc, np.uint16)),
                         _ptr(_c(zpp, np.uint8)), _ptr(codes), _ptr(scales), _ptr(zp))
    if rc:
        raise ValueError("unpack failed")
    return codes, scales, zp
