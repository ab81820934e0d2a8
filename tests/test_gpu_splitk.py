"""GPU parity of the split-K entry point (gemm_fp16_tn_splitk) against the
CPU oracle, through the C-ABI.

Every output element is compared (|D - D_ref| <= 2 ulp16(|D_ref|) +
1e-4 sqrt(K), finite), on grids with fewer tiles than one round of resident
workgroups (every tile cut along K), on grids with whole rounds plus a
part-full one (whole tiles and cut tiles in one launch), with M, N and K
tails, split counts that do and do not divide the K tiles, and runs of a
single K tile.  The run-order reduction makes the result independent of
which run finishes first: repeated calls must agree bit for bit, whatever
the workspace held before."""
import math
import sys

import numpy as np
import pytest

import oracle
import stage_pipelined_mainloop_amd as sg
from stage_pipelined_mainloop_amd import inputs

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def split_call(a, b, M, N, K, splits, alpha=1.0, ws=None):
    """One gemm_fp16_tn_splitk call into a NaN-filled D, with a workspace
    full of NaN bit patterns (its contents on entry must not matter)."""
    need = sg.gemm_fp16_tn_splitk_workspace_bytes(M, N, K, splits)
    if ws is None:
        ws = torch.full((max(need, 256),), 0xFF, dtype=torch.uint8, device=DEV)
    d = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    sg.gemm_fp16_tn_splitk(M, N, K, alpha, a.data_ptr(), b.data_ptr(), d.data_ptr(), splits,
                           ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return d, ws, need


@pytest.mark.parametrize("shape,splits", [
    ((2048, 2048, 8192), (2, 3, 4)),          # 64 tiles: every tile cut
    ((2056, 1032, 1000), (2, 4, 7, 16)),      # M, N tails; K = 15 tiles + 40
    ((300, 264, 520), (2, 5, 9, 12)),         # 9 K tiles: 9 and 12 give runs of one tile
    ((4352, 4352, 1024), (3, 7)),             # 289 tiles: 256 whole, 33 cut
    ((264, 8, 136), (3,)),                    # N = 8, K tail inside the last run
    ((81920, 256, 256), (2, 4)),              # the tall shape: 320 tiles, 64 cut
])
def test_split_runs_match_the_oracle(shape, splits):
    M, N, K = shape
    A, B = inputs.operands(M, N, K, 2100 + K)
    a, b = to_dev(A), to_dev(B)
    say(f"[case] splitk oracle {shape}")
    ref = oracle.gemm_tn_f64(A, B)
    for s in splits:
        say(f"[case] splitk {shape} splits={s}")
        d, ws, need = split_call(a, b, M, N, K, s)
        assert need > 0, (shape, s)
        rep = oracle.check(d.cpu().numpy(), ref, K)
        assert rep.ok, (shape, s, str(rep))
        # a second call on the same (now used) workspace: bit for bit the same
        d2, _, _ = split_call(a, b, M, N, K, s, ws=ws)
        assert torch.equal(d2.view(torch.int16), d.view(torch.int16)), (shape, s)


def test_split_line_alignment_selects_schedule():
    # K % 64 == 0: with A and B on 128-byte lines the pieces run schedule
    # 10, with A 16 bytes past a line schedule 12; the same runs in the same
    # order give the same bits, and both
    # match the oracle in every element (M and N tails, uneven runs)
    M, N, K = 2056, 1040, 1024
    A, B = inputs.operands(M, N, K, 2999)
    ref = oracle.gemm_tn_f64(A, B)
    a, b = to_dev(A), to_dev(B)
    flat = torch.empty(M * K + 64, dtype=torch.float16, device=DEV)
    a16 = flat[8:8 + M * K].view(M, K)
    a16.copy_(a)
    assert a.data_ptr() % 128 == 0 and b.data_ptr() % 128 == 0 and a16.data_ptr() % 128 == 16
    for s in (3, 16):
        outs = []
        for x, label in ((a, "lines"), (a16, "16 bytes past a line")):
            say(f"[case] splitk alignment {label} splits={s}")
            d, _, need = split_call(x, b, M, N, K, s)
            assert need > 0
            rep = oracle.check(d.cpu().numpy(), ref, K)
            assert rep.ok, (label, s, str(rep))
            outs.append(d)
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), s


def test_6144_square_remainder_form_and_split():
    # 576 tiles: two whole rounds and a quarter round.  The library's call
    # runs the whole rounds as 256x256 tiles and the quarter round as 256
    # quarters of 128x128 (no split); the split call with 4 runs cuts the
    # quarter round along K instead.  Both against the oracle in every
    # element, through the Python entry and the C-ABI
    M = N = 6144
    K = 4096
    A, B = inputs.operands(M, N, K, 2201)
    a, b = to_dev(A), to_dev(B)
    assert sg.gemm_fp16_tn_splitk_splits(M, N, K) == 1
    assert sg.gemm_fp16_tn_remainder_quarters(M, N, K) == 256
    ref = oracle.gemm_tn_f64(A, B)
    say("[case] 6144^2 x 4096 library call (remainder form)")
    d = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    sg.gemm(a, b, out=d)
    torch.cuda.synchronize()
    rep = oracle.check(d.cpu().numpy(), ref, K)
    assert rep.ok, str(rep)
    say("[case] 6144^2 x 4096 split x4")
    d2, _, need = split_call(a, b, M, N, K, 4)
    assert need > 0
    rep = oracle.check(d2.cpu().numpy(), ref, K)
    assert rep.ok, str(rep)


@pytest.mark.parametrize("K", [512, 2048, 16384])
def test_split_ksweep_library_choice(K):
    # the K-sweep grid (64 tiles of 256 x 256) through the Python entry's
    # default choice, every element
    A, B = inputs.ksweep(K)
    a, b = to_dev(A), to_dev(B)
    d = torch.full((2048, 2048), float("nan"), dtype=torch.float16, device=DEV)
    say(f"[case] splitk ksweep K={K} library splits={sg.gemm_fp16_tn_splitk_splits(2048, 2048, K)}")
    sg.gemm(a, b, out=d)
    torch.cuda.synchronize()
    rep = oracle.check(d.cpu().numpy(), oracle.gemm_tn_f64(A, B), K)
    assert rep.ok, (K, str(rep))


@pytest.mark.parametrize("alpha", [-1.0, 0.5, -0.375])
def test_split_alpha_and_zero_sums(alpha):
    M, N, K = 520, 264, 1032
    A, B = inputs.operands(M, N, K, 2301)
    A[7] = 0.0
    A[300] = -0.0
    a, b = to_dev(A), to_dev(B)
    ref = oracle.gemm_tn_f64(A, B, alpha)
    say(f"[case] splitk alpha={alpha}")
    d, _, _ = split_call(a, b, M, N, K, 4, alpha=alpha)
    h = d.cpu().numpy()
    assert np.array_equal(h[[7, 300]].view(np.uint16), ref[[7, 300]].view(np.uint16))
    rep = oracle.check(h, ref, K)
    assert rep.ok, str(rep)


def test_split_counts_that_need_no_workspace():
    # one K tile (nothing to cut) and splits = 1 run the plain call
    for (M, N, K, s) in [(300, 264, 64, 4), (300, 264, 520, 1), (512, 512, 8, 3)]:
        say(f"[case] splitk no-op split {(M, N, K, s)}")
        assert sg.gemm_fp16_tn_splitk_workspace_bytes(M, N, K, s) == 0
        A, B = inputs.operands(M, N, K, 2401 + K)
        a, b = to_dev(A), to_dev(B)
        d = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        sg.gemm_fp16_tn_splitk(M, N, K, 1.0, a.data_ptr(), b.data_ptr(), d.data_ptr(), s, 0, 0,
                               torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        rep = oracle.check(d.cpu().numpy(), oracle.gemm_tn_f64(A, B), K)
        assert rep.ok, str(rep)


def test_split_canary_bands():
    # D and the workspace inside NaN / 0xAB guard bands: nothing outside them
    # changes, every element of D is written
    M, N, K, s = 520, 264, 1032, 4
    A, B = inputs.operands(M, N, K, 2501)
    a, b = to_dev(A), to_dev(B)
    need = sg.gemm_fp16_tn_splitk_workspace_bytes(M, N, K, s)
    guard = 4096
    dbuf = torch.full((M * N + 2 * guard,), float("nan"), dtype=torch.float16, device=DEV)
    wbuf = torch.full((need + 2 * guard,), 0xAB, dtype=torch.uint8, device=DEV)
    d = dbuf[guard:guard + M * N]
    say("[case] splitk canary")
    sg.gemm_fp16_tn_splitk(M, N, K, 1.0, a.data_ptr(), b.data_ptr(), d.data_ptr(), s,
                           wbuf[guard:].data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    host = dbuf.cpu().numpy()
    pattern = np.float16(np.nan).view(np.uint16)
    assert np.all(host[:guard].view(np.uint16) == pattern)
    assert np.all(host[guard + M * N:].view(np.uint16) == pattern)
    w = wbuf.cpu().numpy()
    assert np.all(w[:guard] == 0xAB) and np.all(w[guard + need:] == 0xAB)
    rep = oracle.check(host[guard:guard + M * N].reshape(M, N), oracle.gemm_tn_f64(A, B), K)
    assert rep.ok, str(rep)


def test_split_graph_replays_and_streams():
    # replays of a captured split call (two kernels; its workspace from the
    # graph's pool) and calls on two streams at once, each with its own
    # cached workspace, all equal to the eager result bit for bit
    M, N, K = 1024, 1024, 8192
    A, B = inputs.operands(M, N, K, 2601)
    a, b = to_dev(A), to_dev(B)
    assert sg.gemm_fp16_tn_splitk_splits(M, N, K) > 1
    say("[case] splitk graph / streams")
    eager = sg.gemm(a, b)
    torch.cuda.synchronize()
    rep = oracle.check(eager.cpu().numpy(), oracle.gemm_tn_f64(A, B), K)
    assert rep.ok, str(rep)
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(2):
            sg.gemm(a, b, out=out)
    for r in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), r
        tmp = sg.gemm(a, b)
        torch.cuda.synchronize()
        assert torch.equal(tmp.view(torch.int16), eager.view(torch.int16)), r
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = sg.gemm(a, b)
        with torch.cuda.stream(s2):
            o2 = sg.gemm(a, b)
        outs += [o1, o2]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), eager.view(torch.int16))


def test_library_split_choice():
    # the split counts the cost model picks for shapes whose timings it was
    # fitted to (1: the plain call); every compiled choice must run
    expect = {(2048, 2048, 16384): 4, (2048, 2048, 8192): 1, (6144, 6144, 4096): 1,
              (2048, 2048, 2048): 1, (2048, 2048, 512): 1, (3072, 3072, 4096): 1,
              (8192, 8192, 8192): 1, (8000, 7936, 8200): 1, (81920, 256, 256): 1,
              (4096, 4096, 128): 1}
    for shape, s in expect.items():
        assert sg.gemm_fp16_tn_splitk_splits(*shape) == s, shape
    assert sg.gemm_fp16_tn_splitk_splits(4352, 4352, 4096) == 1       # the remainder form instead
    assert sg.gemm_fp16_tn_remainder_quarters(4352, 4352, 4096) == 132
    assert sg.gemm_fp16_tn_splitk_splits(1024, 1024, 8192) > 1


def test_split_random_shapes_counts_and_alpha():
    # seeded random cases: any M, N and K tail, any split count 2..16, any
    # alpha; every element, and the allocation-free entry point's bits equal
    # to the workspace entry point's
    g = np.random.Generator(np.random.PCG64(5151))
    for case in range(30):
        M = int(g.integers(1, 1300))
        N = 8 * int(g.integers(1, 170))
        K = 8 * int(g.integers(1, 260))
        s = int(g.integers(2, 17))
        alpha = float(np.float32(g.choice([1.0, 0.5, -1.25, 1.0 / 3.0, 2.0 ** -7])))
        A = g.uniform(-1, 1, (M, K)).astype(np.float16)
        B = g.uniform(-1, 1, (N, K)).astype(np.float16)
        say(f"[case] splitk random {case}: {M}x{N}x{K} splits={s} alpha={alpha}")
        a, b = to_dev(A), to_dev(B)
        d, _, need = split_call(a, b, M, N, K, s, alpha=alpha)
        rep = oracle.check(d.cpu().numpy(), oracle.gemm_tn_f64(A, B, alpha), K)
        assert rep.ok, (case, M, N, K, s, alpha, str(rep))
        if need <= 64 << 20:
            d2 = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
            sg.gemm_fp16_tn_splitk_noalloc(M, N, K, alpha, a.data_ptr(), b.data_ptr(), d2.data_ptr(),
                                           s, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            assert torch.equal(d2.view(torch.int16), d.view(torch.int16)), case


def test_split_edge_cases():
    # K at the documented limit 2^21 (minus a tail) cut into 16 runs of 2048
    # K tiles: per-piece offsets and buffer ranges come closest to 2^31 here
    M, N, K = 264, 24, (1 << 21) - 8
    g = np.random.Generator(np.random.PCG64(903))
    A = g.uniform(-1, 1, (M, K)).astype(np.float16)
    B = g.uniform(-1, 1, (N, K)).astype(np.float16)
    say(f"[case] splitk max K {M}x{N}x{K}")
    d, _, need = split_call(to_dev(A), to_dev(B), M, N, K, 16)
    assert need == 2 * 16 * 256 * 256 * 4
    rep = oracle.check(d.cpu().numpy(), oracle.gemm_tn_f64(A, B), K)
    assert rep.ok, str(rep)
    # K = 0 through the split entry point: the empty sum, +0 for alpha < 0
    # too, no workspace needed
    say("[case] splitk K=0")
    a = torch.zeros((300, 0), dtype=torch.float16, device=DEV)
    b = torch.zeros((264, 0), dtype=torch.float16, device=DEV)
    d = torch.full((300, 264), float("nan"), dtype=torch.float16, device=DEV)
    sg.gemm_fp16_tn_splitk(300, 264, 0, -2.0, a.data_ptr(), b.data_ptr(), d.data_ptr(), 4, 0, 0,
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert bool((d.view(torch.int16) == 0).all())
