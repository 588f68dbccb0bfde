"""Python binding of libmnb: MatMulNBits with a fused rank-32 LoRA term on MI355X (gfx950).

The C ABI (``include/mnb.h``) is exposed under its own names (``mnb_pack``,
``mnb_matmul`` ...) taking plain integers for device pointers and the stream.  The
convenience wrappers (``pack``, ``unpack``, ``matmul``) only marshal torch tensors into
those calls: every step of the computation runs in the HIP kernels of ``libmnb.so``.
Importing this package fails if ``libmnb.so`` has not been built (there is no fallback).

Operation (onnxruntime PR #33370 "[WebGPU] Fuse rank-32 quantized LoRA with MatMulNBits";
PR #33800 "Fuse DQ->MatMulNBits for shared initializers and skip outer-scope weights"):
    Y[M,N] = X[M,K] . deq(W)^T + (X . A) . B [+ bias[N]],
    deq(W)[n,k] = (q[n,k] - z[n,k/32]) * s[n,k/32]
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmnb.so")

MNB_OK, MNB_ERR_INVALID_ARG, MNB_ERR_UNSUPPORTED, MNB_ERR_MISALIGNED = 0, 1, 2, 3
MNB_ERR_WORKSPACE, MNB_ERR_ALIAS, MNB_ERR_HIP, MNB_ERR_HANDOFF, MNB_ERR_TOO_LARGE = 4, 5, 6, 7, 8
MNB_NOALLOC_SCRATCH_BYTES = 32 << 20
MNB_ADAPTER_NONE, MNB_ADAPTER_F16, MNB_ADAPTER_Q8 = 0, 1, 2
MNB_PATH_AUTO, MNB_PATH_GEMV, MNB_PATH_GEMM = 0, 1, 2
MNB_FLAG_T_SEPARATE, MNB_FLAG_ACC4, MNB_FLAG_FAIL_HANDOFF = 1, 2, 4


class mnb_adapter(C.Structure):
    _fields_ = [("kind", C.c_int), ("rank", C.c_int), ("A", C.c_void_p), ("A_scales", C.c_void_p),
                ("B", C.c_void_p), ("B_scales", C.c_void_p)]


class mnb_options(C.Structure):
    _fields_ = [("path", C.c_int), ("flags", C.c_int)]


def _hip_runtimes() -> set:
    """Paths of every HIP runtime library mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {line.split()[-1] for line in f if "libamdhip64" in line and "/" in line}
    except OSError:
        return set()


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmnb.so is not built (%s); run `python blockwise_bit_quantized_amd/build.py`"
                          % LIB_PATH)
    # torch ships its own HIP runtime with the same soname as the system one.  Loading torch
    # first makes libmnb bind to that runtime, so device memory, streams and kernels of both
    # live in one runtime; loading libmnb first would leave two runtimes in the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = C.CDLL(LIB_PATH)
    runtimes = {os.path.realpath(p) for p in _hip_runtimes()}
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded (%s); import torch before loading libmnb"
                          % ", ".join(sorted(runtimes)))
    P, I, S = C.c_void_p, C.c_int, C.c_size_t
    lib.mnb_packed_sizes.argtypes = [I, I, I, I, I, C.POINTER(S), C.POINTER(S), C.POINTER(S)]
    lib.mnb_pack.argtypes = [P, P, P, I, I, I, I, P, P, P, P]
    lib.mnb_pack_kn.argtypes = [P, P, P, I, I, I, I, P, P, P, P]
    lib.mnb_unpack.argtypes = [P, P, P, I, I, I, I, P, P, P, P]
    lib.mnb_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.mnb_workspace_bytes.restype = S
    lib.mnb_workspace_error.argtypes = [P, P]
    lib.mnb_matmul.argtypes = [P, P, P, P, C.POINTER(mnb_adapter), P, I, I, I, I, I, P, S, P]
    lib.mnb_matmul_ex.argtypes = [P, P, P, P, C.POINTER(mnb_adapter), P, I, I, I, I, I, P, S, P,
                                  C.POINTER(mnb_options)]
    lib.mnb_matmul_bias.argtypes = [P, P, P, P, C.POINTER(mnb_adapter), P, P, I, I, I, I, I, P, S, P,
                                    C.POINTER(mnb_options)]
    lib.mnb_matmul_noalloc.argtypes = [P, P, P, P, C.POINTER(mnb_adapter), P, P, I, I, I, I, I, P,
                                       C.POINTER(mnb_options)]
    lib.mnb_describe_route.argtypes = [I, I, I, I, I, I, C.POINTER(mnb_options), C.c_char_p, S]
    lib.mnb_status_string.argtypes = [I]
    lib.mnb_status_string.restype = C.c_char_p
    lib.mnb_version.argtypes = []
    for f in ("mnb_packed_sizes", "mnb_pack", "mnb_pack_kn", "mnb_unpack", "mnb_matmul", "mnb_matmul_ex",
              "mnb_matmul_bias", "mnb_matmul_noalloc", "mnb_describe_route", "mnb_version",
              "mnb_workspace_error"):
        getattr(lib, f).restype = I
    return lib


lib = _load()

# ---------------------------------------------------------------------------------------
# The C ABI under its own names (integers for pointers and the stream)
# ---------------------------------------------------------------------------------------


def mnb_version() -> int:
    return lib.mnb_version()


def mnb_status_string(status: int) -> str:
    return lib.mnb_status_string(status).decode()


def mnb_packed_sizes(N, K, bits, block, has_zp):
    a, b, c = C.c_size_t(), C.c_size_t(), C.c_size_t()
    st = lib.mnb_packed_sizes(N, K, bits, block, int(bool(has_zp)), C.byref(a), C.byref(b), C.byref(c))
    return st, a.value, b.value, c.value


def mnb_pack(codes, scales, zp, N, K, bits, block, wq, sc, zpp, stream) -> int:
    return lib.mnb_pack(codes, scales, zp, N, K, bits, block, wq, sc, zpp, stream)


def mnb_pack_kn(codes_kn, scales_kn, zp_kn, N, K, bits, block, wq, sc, zpp, stream) -> int:
    return lib.mnb_pack_kn(codes_kn, scales_kn, zp_kn, N, K, bits, block, wq, sc, zpp, stream)


def mnb_unpack(wq, sc, zpp, N, K, bits, block, codes, scales, zp, stream) -> int:
    return lib.mnb_unpack(wq, sc, zpp, N, K, bits, block, codes, scales, zp, stream)


def mnb_workspace_bytes(M, N, K, bits, rank) -> int:
    return lib.mnb_workspace_bytes(M, N, K, bits, rank)


def mnb_workspace_error(workspace, stream) -> int:
    return lib.mnb_workspace_error(workspace, stream)


def mnb_matmul(X, wq, sc, zpp, ad, Y, M, N, K, bits, block, workspace, ws_bytes, stream) -> int:
    return lib.mnb_matmul(X, wq, sc, zpp, C.byref(ad) if ad is not None else None, Y, M, N, K, bits,
                          block, workspace, ws_bytes, stream)


def mnb_matmul_ex(X, wq, sc, zpp, ad, Y, M, N, K, bits, block, workspace, ws_bytes, stream, opt) -> int:
    return lib.mnb_matmul_ex(X, wq, sc, zpp, C.byref(ad) if ad is not None else None, Y, M, N, K, bits,
                             block, workspace, ws_bytes, stream, C.byref(opt) if opt is not None else None)


def mnb_matmul_bias(X, wq, sc, zpp, ad, bias, Y, M, N, K, bits, block, workspace, ws_bytes, stream,
                    opt) -> int:
    return lib.mnb_matmul_bias(X, wq, sc, zpp, C.byref(ad) if ad is not None else None, bias, Y, M, N, K,
                               bits, block, workspace, ws_bytes, stream,
                               C.byref(opt) if opt is not None else None)


def mnb_matmul_noalloc(X, wq, sc, zpp, ad, bias, Y, M, N, K, bits, block, stream, opt) -> int:
    return lib.mnb_matmul_noalloc(X, wq, sc, zpp, C.byref(ad) if ad is not None else None, bias, Y, M, N, K,
                                  bits, block, stream, C.byref(opt) if opt is not None else None)


def mnb_describe_route(M, N, K, bits, has_zp, adapter_kind, opt=None):
    buf = C.create_string_buffer(256)
    st = lib.mnb_describe_route(M, N, K, bits, int(bool(has_zp)), adapter_kind,
                                C.byref(opt) if opt is not None else None, buf, 256)
    return st, buf.value.decode()


# ---------------------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------------------


def _check(st: int):
    if st != MNB_OK:
        raise RuntimeError(mnb_status_string(st))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    import torch
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t, name, dtype, shape=None, dev=None, min_numel=None):
    """Argument check only (no arithmetic): dtype, contiguity, device and shape, so that the
    library never reads or writes past a tensor's storage."""
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dev is not None and t.device != dev:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s holds %d elements, needs at least %d" % (name, t.numel(), min_numel))


@dataclass
class PackedWeight:
    wq: object          # torch.uint8 device tensor
    sc: object          # torch.float16 device tensor (scale bit patterns)
    zp: object          # torch.uint8 device tensor or None (default zero point)
    N: int
    K: int
    bits: int

    def check(self, dev):
        import torch
        st, wqb, scb, zpb = mnb_packed_sizes(self.N, self.K, self.bits, 32, self.zp is not None)
        _check(st)
        _need(self.wq, "packed codes", torch.uint8, dev=dev, min_numel=wqb)
        _need(self.sc, "packed scales", torch.float16, dev=dev, min_numel=scb // 2)
        if self.zp is not None:
            _need(self.zp, "packed zero points", torch.uint8, dev=dev, min_numel=zpb)


@dataclass
class Adapter:
    kind: int           # MNB_ADAPTER_F16 or MNB_ADAPTER_Q8
    A: object
    B: object
    A_scales: object = None
    B_scales: object = None
    rank: int = 32

    def struct(self) -> mnb_adapter:
        return mnb_adapter(self.kind, self.rank, _ptr(self.A), _ptr(self.A_scales), _ptr(self.B),
                           _ptr(self.B_scales))

    def is_empty(self) -> bool:
        return self.kind == MNB_ADAPTER_NONE or self.rank == 0 or self.A is None or self.B is None

    def check(self, N, K, dev):
        """Shapes and dtypes of a non-empty adapter (rank 32; the library rejects others)."""
        import torch
        if self.is_empty() or self.rank != 32:
            return
        r = self.rank
        if self.kind == MNB_ADAPTER_F16:
            _need(self.A, "adapter A", torch.float16, (K, r), dev)
            _need(self.B, "adapter B", torch.float16, (r, N), dev)
        elif self.kind == MNB_ADAPTER_Q8:
            _need(self.A, "adapter A", torch.int8, (K, r), dev)
            _need(self.B, "adapter B", torch.int8, (r, N), dev)
            if self.A_scales is None or self.B_scales is None:
                raise ValueError("an INT8 adapter needs A_scales and B_scales")
            _need(self.A_scales, "adapter A_scales", torch.float16, (K // 32, r), dev)
            _need(self.B_scales, "adapter B_scales", torch.float16, None, dev, N)
            if self.B_scales.numel() != N:
                raise ValueError("adapter B_scales must hold N = %d values" % N)


def pack(codes, scales, zp, bits: int) -> PackedWeight:
    """Pack device tensors codes uint8 [N,K], scales fp16 [N,K/32], zp uint8 [N,K/32] | None."""
    import torch
    N, K = codes.shape
    dev = codes.device
    _need(codes, "codes", torch.uint8, (N, K), dev)
    _need(scales, "scales", torch.float16, (N, K // 32), dev)
    if zp is not None:
        _need(zp, "zp", torch.uint8, (N, K // 32), dev)
    st, wqb, scb, zpb = mnb_packed_sizes(N, K, bits, 32, zp is not None)
    _check(st)
    wq = torch.empty(wqb, dtype=torch.uint8, device=dev)
    sc = torch.empty(scb // 2, dtype=torch.float16, device=dev)
    zpp = torch.empty(zpb, dtype=torch.uint8, device=dev) if zp is not None else None
    _check(mnb_pack(_ptr(codes), _ptr(scales), _ptr(zp), N, K, bits, 32, _ptr(wq), _ptr(sc), _ptr(zpp),
                    _stream(dev)))
    return PackedWeight(wq, sc, zpp, N, K, bits)


def pack_kn(codes_kn, scales_kn, zp_kn, bits: int) -> PackedWeight:
    """Pack from the DequantizeLinear layout: codes uint8 [K,N], scales fp16 [K/32,N],
    zp uint8 [K/32,N] | None (device tensors)."""
    import torch
    K, N = codes_kn.shape
    dev = codes_kn.device
    _need(codes_kn, "codes_kn", torch.uint8, (K, N), dev)
    _need(scales_kn, "scales_kn", torch.float16, (K // 32, N), dev)
    if zp_kn is not None:
        _need(zp_kn, "zp_kn", torch.uint8, (K // 32, N), dev)
    st, wqb, scb, zpb = mnb_packed_sizes(N, K, bits, 32, zp_kn is not None)
    _check(st)
    wq = torch.empty(wqb, dtype=torch.uint8, device=dev)
    sc = torch.empty(scb // 2, dtype=torch.float16, device=dev)
    zpp = torch.empty(zpb, dtype=torch.uint8, device=dev) if zp_kn is not None else None
    _check(mnb_pack_kn(_ptr(codes_kn), _ptr(scales_kn), _ptr(zp_kn), N, K, bits, 32, _ptr(wq), _ptr(sc),
                       _ptr(zpp), _stream(dev)))
    return PackedWeight(wq, sc, zpp, N, K, bits)


def unpack(pw: PackedWeight):
    import torch
    dev = pw.wq.device
    pw.check(dev)
    codes = torch.empty((pw.N, pw.K), dtype=torch.uint8, device=dev)
    scales = torch.empty((pw.N, pw.K // 32), dtype=torch.float16, device=dev)
    zp = torch.empty((pw.N, pw.K // 32), dtype=torch.uint8, device=dev) if pw.zp is not None else None
    _check(mnb_unpack(_ptr(pw.wq), _ptr(pw.sc), _ptr(pw.zp), pw.N, pw.K, pw.bits, 32, _ptr(codes),
                      _ptr(scales), _ptr(zp), _stream(dev)))
    return codes, scales, zp


class WorkspaceCache:
    """Zero-initialised workspaces, one per (device index, stream handle).

    The library keeps per-call counters and the in-pass T epoch inside the workspace, so
    calls that may overlap in time must not share one (include/mnb.h); calls on different
    streams may overlap, calls on one stream do not.  Keying by stream gives each stream
    its own buffer.  `alloc(nbytes)` returns a zero-filled uint8 tensor."""

    def __init__(self, alloc):
        self._alloc = alloc
        self._bufs = {}

    def get(self, dev_index: int, stream: int, nbytes: int):
        key = (int(dev_index), int(stream))
        ws = self._bufs.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = self._alloc(max(nbytes, 1))
            self._bufs[key] = ws
        return ws

    def __len__(self):
        return len(self._bufs)


_ws_caches: dict = {}


def workspace(dev, nbytes: int, stream=None):
    """A zero-initialised workspace of at least ``nbytes`` for ``dev`` and ``stream`` (the
    device's current stream by default), reused by later calls on that stream."""
    import torch
    index = dev.index if dev.index is not None else torch.cuda.current_device()
    if stream is None:
        stream = torch.cuda.current_stream(index)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    cache = _ws_caches.get(index)
    if cache is None:
        d = torch.device("cuda", index)
        cache = _ws_caches[index] = WorkspaceCache(lambda n: torch.zeros(n, dtype=torch.uint8, device=d))
    return cache.get(index, handle, nbytes)


def workspace_error(ws) -> int:
    """Reports and clears the workspace's error word: MNB_ERR_HANDOFF if an in-pass T
    handoff gave up since the last query (its outputs are NaN), else MNB_OK.  Waits for
    the current stream of the workspace's device."""
    return mnb_workspace_error(_ptr(ws), _stream(ws.device))


def _matmul_args(X, pw, adapter, out, bias):
    import torch
    if X.dim() != 2:
        raise ValueError("X must be 2-D [M, K]")
    M, K = X.shape
    if K != pw.K:
        raise ValueError("X has K=%d, weight has K=%d" % (K, pw.K))
    dev = X.device
    _need(X, "X", torch.float16, (M, K), dev)
    pw.check(dev)
    if adapter is not None:
        adapter.check(pw.N, K, dev)
    if bias is not None:
        _need(bias, "bias", torch.float16, None, dev, pw.N)
        if bias.numel() != pw.N:
            raise ValueError("bias must hold N = %d values" % pw.N)
    Y = out if out is not None else torch.empty((M, pw.N), dtype=torch.float16, device=dev)
    _need(Y, "out", torch.float16, (M, pw.N), dev)
    return M, K, dev, Y


def matmul_noalloc(X, pw: PackedWeight, adapter: Adapter | None = None, path: int = MNB_PATH_AUTO,
                   flags: int = 0, out=None, bias=None):
    """matmul through mnb_matmul_noalloc: the library's static per-device scratch instead of
    a workspace (no device allocation in the call when ``out`` is given).  Calls that
    overlap in time on one device must not be made."""
    M, K, dev, Y = _matmul_args(X, pw, adapter, out, bias)
    ad = adapter.struct() if adapter is not None else None
    _check(mnb_matmul_noalloc(_ptr(X), _ptr(pw.wq), _ptr(pw.sc), _ptr(pw.zp), ad, _ptr(bias), _ptr(Y), M,
                              pw.N, K, pw.bits, 32, _stream(dev), mnb_options(path, flags)))
    return Y


def matmul(X, pw: PackedWeight, adapter: Adapter | None = None, path: int = MNB_PATH_AUTO,
           flags: int = 0, out=None, ws=None, bias=None):
    """Y = X . deq(W)^T (+ (X.A).B) (+ bias) for a device fp16 X [M, K] and an optional fp16
    bias [N]; returns fp16 Y [M, N].

    Without ``ws`` the call uses the workspace cached for the current stream of X's device;
    under graph capture a workspace must be passed (a cached one would be allocated and
    zeroed inside the capture)."""
    import torch
    M, K, dev, Y = _matmul_args(X, pw, adapter, out, bias)
    need = mnb_workspace_bytes(M, pw.N, K, pw.bits, 32 if adapter is not None else 0)
    if ws is None:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("pass ws= under graph capture (a zeroed workspace owned by the caller)")
        ws = workspace(dev, need)
    _need(ws, "workspace", torch.uint8, None, dev, need)
    ad = adapter.struct() if adapter is not None else None
    opt = mnb_options(path, flags)
    _check(mnb_matmul_bias(_ptr(X), _ptr(pw.wq), _ptr(pw.sc), _ptr(pw.zp), ad, _ptr(bias), _ptr(Y), M,
                           pw.N, K, pw.bits, 32, _ptr(ws), ws.numel(), _stream(dev), opt))
    return Y
