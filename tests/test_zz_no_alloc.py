"""The allocation-free split-K entry point (gemm_fp16_tn_splitk_noalloc),
called through the C-ABI, against the workspace entry point it mirrors
(gemm_fp16_tn_splitk): the same kernels, so the same bits; two calls in a
row on the library's fixed scratch, the second with a smaller input, and
the rejection of a plan larger than the scratch."""
import sys

import numpy as np
import pytest

import oracle
import stage_pipelined_mainloop_amd as sg
from stage_pipelined_mainloop_amd import _lib, inputs

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(M, N, K, s, a, b, noalloc):
    d = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = _lib.lib().gemm_fp16_tn_splitk_noalloc(M, N, K, 1.0, a.data_ptr(), b.data_ptr(),
                                                    d.data_ptr(), s, stream)
    else:
        need = sg.gemm_fp16_tn_splitk_workspace_bytes(M, N, K, s)
        ws = torch.full((max(need, 16),), 0x7F, dtype=torch.uint8, device=DEV)
        st = _lib.lib().gemm_fp16_tn_splitk(M, N, K, 1.0, a.data_ptr(), b.data_ptr(),
                                            d.data_ptr(), s, ws.data_ptr(), ws.numel(), stream)
    torch.cuda.synchronize()
    assert st == _lib.SG_OK, _lib.sg_status_string(st)
    return d


def test_noalloc_matches_the_workspace_entry_on_two_calls():
    # a 64-tile grid cut 4 ways (256 partials: the whole scratch), then a
    # smaller ragged one cut 3 ways on the scratch the first call left behind
    for (M, N, K, s) in [(2048, 2048, 4096, 4), (1000, 1032, 1000, 3)]:
        print(f"[case] noalloc {M}x{N}x{K} splits={s}", flush=True)
        sys.stdout.flush()
        A, B = inputs.operands(M, N, K, 3100 + K)
        a, b = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
        want = _run(M, N, K, s, a, b, noalloc=False)
        got = _run(M, N, K, s, a, b, noalloc=True)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (M, N, K, s)
        rep = oracle.check(got.cpu().numpy(), oracle.gemm_tn_f64(A, B), K)
        assert rep.ok, str(rep)


def test_noalloc_rejects_plans_beyond_its_scratch():
    # 64 tiles cut 8 ways need 512 partial tiles (128 MiB): refused before
    # any launch, D untouched
    M = N = 2048
    K = 4096
    assert sg.gemm_fp16_tn_splitk_workspace_bytes(M, N, K, 8) > 64 << 20
    a = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    b = torch.zeros((N, K), dtype=torch.float16, device=DEV)
    d = torch.full((M, N), 3.0, dtype=torch.float16, device=DEV)
    st = _lib.lib().gemm_fp16_tn_splitk_noalloc(M, N, K, 1.0, a.data_ptr(), b.data_ptr(),
                                                d.data_ptr(), 8, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == _lib.SG_ERR_SHAPE
    assert bool((d == 3.0).all())
