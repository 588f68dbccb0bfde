"""Shared test helpers: building on demand, GPU marshalling and the parity comparison."""
from __future__ import annotations

import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# tolerance for FP16 outputs accumulated in FP32, against the FP64 oracle
MAX_ABS = 2e-2
MAX_REL = 1e-2


def ensure_lib():
    """Import the binding, building libmnb.so first only if it is absent."""
    path = os.path.join(ROOT, "blockwise_bit_quantized_amd", "libmnb.so")
    if not os.path.exists(path):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_mnb_build", os.path.join(ROOT, "blockwise_bit_quantized_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
    import blockwise_bit_quantized_amd as mnb
    return mnb


def f16_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def compare(y16_bits, ref: np.ndarray, max_abs=MAX_ABS, max_rel=MAX_REL, what=""):
    """Element-by-element check of GPU fp16 output against the FP64 oracle.

    max-abs: max |Y - y| <= max_abs; relative (normwise): max |Y - y| / max |y| <= max_rel.
    Returns a dict of the measured errors; raises AssertionError with them on failure.
    """
    y = f16_to_f64(y16_bits)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    d = np.abs(y - ref)
    bad = ~np.isfinite(y)
    assert not bad.any(), "%s: %d non-finite outputs" % (what, int(bad.sum()))
    maxabs = float(d.max()) if d.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    rel = maxabs / scale if scale > 0 else maxabs
    stats = dict(maxabs=maxabs, rel=rel, n=int(d.size),
                 l2rel=float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)) if d.size else 0.0)
    assert maxabs <= max_abs and rel <= max_rel, "%s: %s" % (what, stats)
    return stats


def same_bits(a, b) -> bool:
    """Bitwise equality of fp16 bit patterns, treating +0 and -0 as equal."""
    a = np.asarray(a, np.uint16).copy()
    b = np.asarray(b, np.uint16).copy()
    a[a == 0x8000] = 0
    b[b == 0x8000] = 0
    return bool(np.array_equal(a, b))
