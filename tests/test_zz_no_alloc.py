"""mnb_matmul_noalloc (its workspace is the library's static per-device scratch) against
mnb_matmul_bias with a caller workspace, through the C ABI: the same kernels run, so the
outputs must be equal bit for bit.  Each case makes two calls in a row on one stream, the
second with a smaller input; the scratch keeps the first call's contents."""
from __future__ import annotations

import numpy as np
import pytest

import seeded_inputs as si
from _util import ensure_lib, same_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mnb = ensure_lib()
DEV = torch.device("cuda:0")


def t16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.float16)).to(DEV)


def prepare(spec, seed):
    M, N, K, bits, zp, kind = spec
    c = si.make_random(seed, M, N, K, bits, zp, kind, bias=seed % 2 == 0)
    z = torch.from_numpy(c["zp"]).to(DEV) if c["zp"] is not None else None
    pw = mnb.pack(torch.from_numpy(c["codes"]).to(DEV), t16(c["scales"]), z, bits)
    ad = c["adapter"]
    if ad is None:
        a = None
    elif ad["kind"] == "f16":
        a = mnb.Adapter(mnb.MNB_ADAPTER_F16, t16(ad["A"]), t16(ad["B"]))
    else:
        a = mnb.Adapter(mnb.MNB_ADAPTER_Q8, torch.from_numpy(ad["A"]).to(DEV), torch.from_numpy(ad["B"]).to(DEV),
                        t16(ad["A_scales"]), t16(ad["B_scales"]))
    bias = t16(c["bias"]) if c.get("bias") is not None else None
    return dict(X=t16(c["X"]), pw=pw, ad=a, bias=bias, M=M, N=N, K=K, bits=bits)


def noalloc(call, Y, stream):
    pw, a, bias = call["pw"], call["ad"], call["bias"]
    return mnb.mnb_matmul_noalloc(call["X"].data_ptr(), pw.wq.data_ptr(), pw.sc.data_ptr(),
                                  pw.zp.data_ptr() if pw.zp is not None else None,
                                  a.struct() if a is not None else None,
                                  bias.data_ptr() if bias is not None else None, Y.data_ptr(),
                                  call["M"], call["N"], call["K"], call["bits"], 32, stream, None)


def with_workspace(call):
    ws = torch.zeros(mnb.mnb_workspace_bytes(call["M"], call["N"], call["K"], call["bits"], 32),
                     dtype=torch.uint8, device=DEV)
    Y = mnb.matmul(call["X"], call["pw"], call["ad"], out=None, ws=ws, bias=call["bias"])
    torch.cuda.synchronize()
    return Y.cpu().numpy().view(np.uint16)


# (first call, second call with a smaller input): in-pass decode, prefill (T projection +
# GEMM), split-K prefill with FP32 partials, small M with the T reduction counters
PAIRS = [
    ((1, 8192, 2048, 4, False, "f16"), (1, 896, 896, 4, True, "f16")),
    ((1024, 4096, 4096, 4, True, "f16"), (64, 320, 512, 4, True, "q8")),
    ((256, 4096, 4096, 4, True, "f16"), (40, 136, 1056, 4, True, None)),
    ((3, 1000, 1024, 4, True, "q8"), (2, 200, 512, 8, False, "f16")),
    ((1, 49152, 576, 8, True, None), (1, 4096, 2048, 2, False, "q8")),
]


@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_equals_workspace_call(pair):
    first, second = (prepare(spec, 700 + 10 * pair + i) for i, spec in enumerate(PAIRS[pair]))
    assert mnb.mnb_workspace_bytes(first["M"], first["N"], first["K"], first["bits"], 32) <= \
        mnb.MNB_NOALLOC_SCRATCH_BYTES
    want = [with_workspace(first), with_workspace(second)]
    stream = torch.cuda.current_stream(DEV).cuda_stream
    for rep in range(2):                      # the second round starts from a used scratch
        Y1 = torch.full((first["M"], first["N"]), 7.0, dtype=torch.float16, device=DEV)
        Y2 = torch.full((second["M"], second["N"]), 7.0, dtype=torch.float16, device=DEV)
        torch.cuda.synchronize()
        assert noalloc(first, Y1, stream) == mnb.MNB_OK
        assert noalloc(second, Y2, stream) == mnb.MNB_OK      # back to back on one stream
        torch.cuda.synchronize()
        assert same_bits(Y1.cpu().numpy().view(np.uint16), want[0]), (pair, rep, "first")
        assert same_bits(Y2.cpu().numpy().view(np.uint16), want[1]), (pair, rep, "second")


def test_noalloc_refuses_what_the_scratch_cannot_hold():
    big = (256, 12288, 16384)                  # K split into FP32 partials: 48 MiB of workspace
    assert mnb.mnb_workspace_bytes(*big, 4, 0) > mnb.MNB_NOALLOC_SCRATCH_BYTES
    X = torch.zeros(big[:1] + big[2:], dtype=torch.float16, device=DEV)
    Y = torch.full(big[:2], 7.0, dtype=torch.float16, device=DEV)
    _, wqb, scb, _ = mnb.mnb_packed_sizes(big[1], big[2], 4, 32, 0)
    wq = torch.zeros(wqb, dtype=torch.uint8, device=DEV)
    sc = torch.zeros(scb // 2, dtype=torch.float16, device=DEV)
    st = mnb.mnb_matmul_noalloc(X.data_ptr(), wq.data_ptr(), sc.data_ptr(), None, None, None, Y.data_ptr(),
                                *big, 4, 32, torch.cuda.current_stream(DEV).cuda_stream, None)
    torch.cuda.synchronize()
    assert st == mnb.MNB_ERR_TOO_LARGE
    assert bool((Y == 7.0).all())
