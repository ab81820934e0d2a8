"""GPU parity of the HIP path against the CPU oracle.

Every call goes through the C-ABI (libstagegemm.so) via the thin binding.
Inputs are the seeded generators of stage_pipelined_mainloop_amd.inputs; the
expected values come only from oracle/.  Bound per element:
|D - D_ref| <= 2 ulp16(|D_ref|) + 1e-4 sqrt(K), every element finite.

Small shapes, and the full-size workloads 4096^3, 8192^3 (the benchmarked
call), 8000x7936x8200, 4096x4096x128, 81920x256x256 and the K-sweep
(M = N = 2048, every K, every stage count of both tile families), are
compared element by element in full.  Exactly zero sums are compared by bit
pattern (+0 for either sign of alpha).
"""
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


def to_dev(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def run_gemm(A, B, alpha=None, config=None):
    a, b = to_dev(A), to_dev(B)
    d = torch.full((A.shape[0], B.shape[0]), float("nan"), dtype=torch.float16, device=DEV)
    sg.gemm(a, b, out=d, alpha=alpha, config=config)
    torch.cuda.synchronize()
    return d


def full_check(A, B, alpha=None, config=None, label=""):
    K = A.shape[1]
    say(f"[case] full {label} M={A.shape[0]} N={B.shape[0]} K={K} alpha={alpha} cfg={config}")
    d = run_gemm(A, B, alpha, config).cpu().numpy()
    ref = oracle.gemm_tn_f64(A, B, 1.0 if alpha is None else alpha)
    rep = oracle.check(d, ref, K)
    assert rep.ok, f"{label}: {rep}"
    return d


def sample_lines(n, extra_seed, count=6):
    base = [0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, 257, 511, 512, n // 2,
            n - 257, n - 256, n - 129, n - 128, n - 33, n - 32, n - 2, n - 1]
    g = np.random.Generator(np.random.PCG64(extra_seed))
    base += list(g.integers(0, n, count))
    return sorted({int(v) for v in base if 0 <= v < n})


def sampled_check(A, B, d_dev, alpha, label, seed=0):
    M, K = A.shape
    N = B.shape[0]
    say(f"[case] sampled {label} M={M} N={N} K={K} alpha={alpha}")
    assert bool(torch.isfinite(d_dev).all()), f"{label}: non-finite output"
    rows = sample_lines(M, 1000 + seed)
    cols = sample_lines(N, 2000 + seed)
    d = d_dev.cpu().numpy()
    rr = np.repeat(rows, N)
    rc = np.tile(np.arange(N), len(rows))
    cr = np.repeat(np.arange(M), len(cols))
    cc = np.tile(cols, M)
    r = np.concatenate([rr, cr])
    c = np.concatenate([rc, cc])
    ref = oracle.gemm_tn_f64_at(A, B, r, c, 1.0 if alpha is None else alpha)
    rep = oracle.check(d[r, c], ref, K)
    assert rep.ok, f"{label}: {rep} at (row {r[rep.argmax]}, col {c[rep.argmax]})"


VARIANTS = [c.as_tuple() for c in sg.configs()]
SHORTK = [c for c in VARIANTS if c[5] == 4]


def runs(cfg, K):
    """Whether a compiled variant takes this K: the short-K schedule (4)
    needs the whole K extent in its ring (K <= stages * tile_k)."""
    return cfg is None or cfg[5] != 4 or K <= cfg[2] * cfg[3]


# ---------------------------------------------------------------------------
# small shapes, full comparison

def test_square256_default_and_every_variant():
    A, B = inputs.workload("square256")
    full_check(A, B, label="square256 default")
    for cfg in VARIANTS:
        if runs(cfg, 256):
            full_check(A, B, config=cfg, label=f"square256 {cfg}")


@pytest.mark.parametrize("shape", [(300, 264, 200), (257, 136, 40), (1, 8, 8), (129, 520, 1000),
                                   (512, 512, 8)])
def test_every_variant_on_ragged_shapes(shape):
    M, N, K = shape
    A, B = inputs.operands(M, N, K, 300 + M)
    for cfg in VARIANTS:
        if runs(cfg, K):
            full_check(A, B, config=cfg, label=f"ragged {shape} {cfg}")


@pytest.mark.parametrize("cfg", [None, (128, 128, 32, 3, 4, 1), (256, 256, 32, 5, 8, 1),
                                 (256, 256, 64, 2, 8, 1), (256, 256, 32, 3, 8, 0),
                                 (128, 128, 64, 3, 4, 1), (256, 256, 64, 2, 8, 2),
                                 (128, 128, 64, 2, 4, 3), (256, 256, 64, 2, 8, 3),
                                 (128, 128, 64, 2, 4, 4), (256, 256, 64, 2, 8, 5),
                                 (256, 256, 64, 2, 8, 7), (256, 256, 64, 3, 8, 8),
                                 (256, 256, 64, 2, 4, 10), (256, 256, 64, 3, 4, 11),
                                 (256, 256, 64, 3, 4, 12), (128, 128, 64, 4, 4, 14)])
def test_tiny_shape_grid(cfg):
    # every M, N and K tail against every tile boundary of the variant
    say(f"[case] tiny grid cfg={cfg}")
    g = np.random.Generator(np.random.PCG64(17))
    for M in (1, 2, 33, 127, 129, 255, 257, 300):
        for N in (8, 16, 136, 248, 264):
            for K in (8, 24, 40, 72, 136):
                A = g.uniform(-1, 1, (M, K)).astype(np.float16)
                B = g.uniform(-1, 1, (N, K)).astype(np.float16)
                if not runs(cfg, K):
                    continue
                d = run_gemm(A, B, config=cfg).cpu().numpy()
                rep = oracle.check(d, oracle.gemm_tn_f64(A, B), K)
                assert rep.ok, (M, N, K, cfg, str(rep))


@pytest.mark.parametrize("shape,cfg", [((4352, 4352, 264), None),
                                       ((4352, 4104, 200), (256, 256, 64, 2, 8, 1)),
                                       ((4352, 4104, 200), (256, 256, 64, 2, 8, 7)),
                                       ((4352, 4104, 200), (256, 256, 64, 3, 8, 8)),
                                       ((4352, 4104, 200), (256, 256, 64, 2, 4, 10)),
                                       ((4352, 4360, 4104), (256, 256, 64, 2, 4, 10)),
                                       ((4352, 4104, 200), (256, 256, 64, 3, 4, 11)),
                                       ((4352, 4360, 4104), (256, 256, 64, 3, 4, 11)),
                                       ((4352, 4104, 200), (256, 256, 64, 3, 4, 12)),
                                       ((4352, 4360, 4104), (256, 256, 64, 3, 4, 12)),
                                       ((4352, 4104, 200), (128, 128, 64, 4, 4, 14)),
                                       ((2056, 2312, 4104), (128, 128, 64, 4, 4, 14)),
                                       ((2304, 2304, 520), (128, 128, 32, 4, 4, 1)),
                                       ((2304, 2312, 1000), (256, 256, 32, 3, 8, 0)),
                                       ((4352, 4360, 336), (256, 256, 64, 2, 8, 2)),
                                       ((4352, 4360, 336), (128, 128, 32, 3, 4, 3)),
                                       ((4352, 4360, 200), (128, 128, 64, 2, 4, 3))])
def test_k_tail_on_grids_of_several_rounds(shape, cfg):
    # more than 256 workgroups (several rounds per CU, M and N tails) with a
    # ragged last K tile in every workgroup's loop
    M, N, K = shape
    A, B = inputs.operands(M, N, K, 500 + K)
    full_check(A, B, config=cfg, label=f"several rounds {shape}")


def test_operand_line_alignment_selects_schedule():
    # with K % 64 == 0 the library runs schedule 10 when A and B start on
    # 128-byte lines and schedule 12 when A starts 16 bytes past one; both
    # are compared with the oracle element by element, and with each other
    # bit for bit (same MFMA, same K order)
    M, N, K = 4104, 4096, 1088
    A, B = inputs.operands(M, N, K, 4096 + 11)
    ref = oracle.gemm_tn_f64(A, B)
    a, b = to_dev(A), to_dev(B)
    assert a.data_ptr() % 128 == 0 and b.data_ptr() % 128 == 0
    flat = torch.empty(M * K + 64, dtype=torch.float16, device=DEV)
    a16 = flat[8:8 + M * K].view(M, K)
    a16.copy_(a)
    assert a16.data_ptr() % 128 == 16
    outs = []
    for x, label in ((a, "lines"), (a16, "16 bytes past a line")):
        say(f"[case] alignment {label} {M}x{N}x{K}")
        d = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        sg.gemm(x, b, out=d)
        torch.cuda.synchronize()
        rep = oracle.check(d.cpu().numpy(), ref, K)
        assert rep.ok, (label, str(rep))
        outs.append(d)
    assert torch.equal(outs[0], outs[1])
    assert sg._lib.sg_select_config(M, N, K).as_tuple() == (256, 256, 64, 2, 4, 10)


@pytest.mark.parametrize("shape", [(4352, 4104, 1088), (4360, 4352, 1088), (81920, 256, 1088)])
def test_remainder_form(shape):
    # grids of more than one round of 256x256 tiles with a last round at
    # most a quarter full: the library's call runs the whole rounds as
    # 256x256 tiles and each remaining tile as four 128x128 quarters
    # (quarters past N or M end at once).  Every element against the
    # oracle, and bit for bit against the 256x256 tiled kernel alone (same
    # MFMA, same K order); with alpha, and with beta and C
    M, N, K = shape
    q = sg.gemm_fp16_tn_remainder_quarters(M, N, K)
    assert q > 0, (shape, q)
    A, B = inputs.operands(M, N, K, 2700 + K)
    a32 = float(np.float32(0.375))
    say(f"[case] remainder form {shape} quarters={q}")
    d = full_check(A, B, alpha=a32, label=f"remainder {shape}")
    tiled = run_gemm(A, B, alpha=a32, config=(256, 256, 64, 2, 4, 10)).cpu().numpy()
    assert np.array_equal(d.view(np.uint16), tiled.view(np.uint16))
    Cm = inputs.matrix(M, N, 2800 + N, "normal")
    b32 = float(np.float32(-0.5))
    dd = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    sg.gemm(to_dev(A), to_dev(B), out=dd, alpha=a32, beta=b32, C=to_dev(Cm))
    torch.cuda.synchronize()
    rep = oracle.check(dd.cpu().numpy(), oracle.gemm_tn_f64_beta(A, B, Cm, a32, b32), K)
    assert rep.ok, str(rep)


PERSISTENT = [c for c in VARIANTS if c[5] == 3]


@pytest.mark.parametrize("shape", [(4200, 4104, 200), (4200, 4104, 8), (4224, 4112, 72),
                                   (2056, 4104, 136)])
def test_persistent_workgroups_loop_over_tiles(shape):
    # more output tiles than resident workgroups: each workgroup of the
    # persistent schedule runs several tiles through one ring, with M, N and
    # K tails, one-tile K loops (K = 8) and tiles whose K loop is shorter
    # than the ring
    M, N, K = shape
    A, B = inputs.operands(M, N, K, 1100 + K)
    say(f"[case] persistent {shape}")
    ref = oracle.gemm_tn_f64(A, B)
    assert PERSISTENT
    for cfg in PERSISTENT:
        say(f"[case] persistent {shape} {cfg}")
        d = run_gemm(A, B, config=cfg).cpu().numpy()
        rep = oracle.check(d, ref, K)
        assert rep.ok, (cfg, str(rep))


@pytest.mark.parametrize("alpha", [None, -1.0, -0.375])
@pytest.mark.parametrize("cfg", [None] + PERSISTENT[:2] + SHORTK +
                         [(256, 256, 64, 2, 8, 7), (256, 256, 64, 3, 8, 8),
                          (256, 256, 64, 2, 4, 10), (256, 256, 64, 3, 4, 11),
                          (256, 256, 64, 3, 4, 12), (128, 128, 64, 4, 4, 14)])
def test_k_zero_every_schedule(cfg, alpha):
    # the empty sum is +0 (bit pattern 0) for either sign of alpha
    say(f"[case] K=0 {cfg} alpha={alpha}")
    A = np.zeros((1100, 0), np.float16)
    B = np.zeros((1032, 0), np.float16)
    d = run_gemm(A, B, alpha=alpha, config=cfg).cpu().numpy()
    assert np.all(d.view(np.uint16) == 0)


@pytest.mark.parametrize("alpha", [-1.0, -0.375, 1.0])
def test_zero_sums_are_plus_zero_every_variant(alpha):
    # rows whose sum is exactly zero (all-zero, signed zeros, products that
    # cancel) must give the oracle's bit patterns (+0) for negative alpha too;
    # the other rows are compared within the tolerance
    M, N, K = 300, 264, 136
    A, B = inputs.operands(M, N, K, 1901)
    A[5] = 0.0
    A[70] = -0.0
    A[171] = 0.0
    A[171, :8] = [1, -1, 0.5, -0.5, 0.25, -0.25, 2, -2]      # cancels against B's first...
    B[:, :8] = np.float16(0.75)                              # ...8 columns of equal value
    ref = oracle.gemm_tn_f64(A, B, alpha)
    zero_rows = [5, 70, 171]
    assert np.all(ref[zero_rows].view(np.uint16) == 0)
    for cfg in [None] + VARIANTS:
        if not runs(cfg, K):
            continue
        say(f"[case] zero sums alpha={alpha} {cfg}")
        d = run_gemm(A, B, alpha=alpha, config=cfg).cpu().numpy()
        assert np.array_equal(d[zero_rows].view(np.uint16), ref[zero_rows].view(np.uint16)), cfg
        rep = oracle.check(d, ref, K)
        assert rep.ok, (cfg, str(rep))


@pytest.mark.parametrize("shape,cfg", [((40, 16, 1 << 21), None), ((8, 1 << 21, 8), None),
                                       ((264, 24, (1 << 21) - 8), None),
                                       ((264, 24, (1 << 21) - 8), (256, 256, 64, 3, 8, 8)),
                                       ((264, 24, 1 << 21), (256, 256, 64, 2, 4, 10)),
                                       ((264, 24, (1 << 21) - 8), (256, 256, 64, 3, 4, 11)),
                                       ((264, 24, (1 << 21) - 8), (256, 256, 64, 3, 4, 12)),
                                       ((136, 24, (1 << 21) - 8), (128, 128, 64, 4, 4, 14))])
def test_maximum_k_and_n(shape, cfg):
    # K and N at the documented limit 2^21: per-workgroup buffer ranges and
    # offsets come closest to 2^31 here (the last case with 256-row A and B
    # ranges of the split-load ping-pong: 1 GiB each)
    M, N, K = shape
    g = np.random.Generator(np.random.PCG64(901))
    A = g.uniform(-1, 1, (M, K)).astype(np.float16)
    B = g.uniform(-1, 1, (N, K)).astype(np.float16)
    full_check(A, B, config=cfg, label=f"limit {shape}")


def test_k_zero_writes_zeros():
    say("[case] K=0")
    A = np.zeros((70, 0), np.float16)
    B = np.zeros((24, 0), np.float16)
    d = run_gemm(A, B).cpu().numpy()
    assert np.all(d.view(np.uint16) == 0)


def test_empty_m_or_n_leaves_output_untouched():
    say("[case] M=0 / N=0")
    a = torch.zeros((0, 16), dtype=torch.float16, device=DEV)
    b = torch.zeros((8, 16), dtype=torch.float16, device=DEV)
    out = sg.gemm(a, b)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 8)


@pytest.mark.parametrize("cfg,shape", [(None, (300, 264, 136)), ((128, 128, 32, 4, 4, 1), (300, 264, 136)),
                                       ((256, 256, 32, 4, 8, 1), (300, 264, 136)),
                                       ((256, 256, 32, 4, 8, 0), (300, 264, 136)),
                                       ((256, 256, 64, 2, 8, 2), (300, 264, 136)),
                                       ((128, 128, 64, 2, 4, 3), (4200, 4104, 72)),
                                       ((256, 256, 64, 2, 8, 3), (4200, 4104, 72)),
                                       ((128, 128, 64, 2, 4, 4), (300, 264, 128)),
                                       ((128, 128, 64, 2, 4, 4), (4200, 4104, 72)),
                                       ((256, 256, 64, 2, 8, 5), (300, 264, 136)),
                                       ((256, 256, 64, 2, 8, 7), (300, 264, 136)),
                                       ((256, 256, 64, 3, 8, 8), (300, 264, 136)),
                                       ((256, 256, 64, 2, 4, 10), (300, 264, 136)),
                                       ((256, 256, 64, 3, 4, 11), (300, 264, 136)),
                                       ((256, 256, 64, 3, 4, 12), (300, 264, 136)),
                                       ((128, 128, 64, 4, 4, 14), (300, 264, 136))])
def test_canary_guard_bands(cfg, shape):
    # D sits inside a larger buffer filled with a NaN pattern; nothing outside
    # D may change and every element of D must be written
    M, N, K = shape
    say(f"[case] canary cfg={cfg}")
    A, B = inputs.operands(M, N, K, 77)
    guard = 4096
    buf = torch.full((M * N + 2 * guard,), float("nan"), dtype=torch.float16, device=DEV)
    d = buf[guard:guard + M * N].view(M, N)
    sg.gemm(to_dev(A), to_dev(B), out=d, config=cfg)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    pattern = np.float16(np.nan).view(np.uint16)
    assert np.all(host[:guard].view(np.uint16) == pattern)
    assert np.all(host[guard + M * N:].view(np.uint16) == pattern)
    rep = oracle.check(host[guard:guard + M * N].reshape(M, N), oracle.gemm_tn_f64(A, B), K)
    assert rep.ok, str(rep)


@pytest.mark.parametrize("alpha", [1.0, 0.5, -2.0, 1.0 / 3.0, 1e-3])
def test_alpha_values(alpha):
    A, B = inputs.operands(384, 392, 520, 91)
    a32 = float(np.float32(alpha))
    # the library's choice, and the large-shape kernel on the same operands
    for cfg in (None, (256, 256, 64, 3, 8, 8), (256, 256, 64, 2, 4, 10), (256, 256, 64, 3, 4, 11),
                (256, 256, 64, 3, 4, 12)):
        full_check(A, B, alpha=a32, config=cfg, label=f"alpha {alpha} {cfg}")


@pytest.mark.parametrize("shape", [(300, 264, 200), (4352, 520, 264), (256, 256, 0),
                                   (20480, 256, 256), (3848, 3840, 136), (4096, 4104, 256)])
@pytest.mark.parametrize("alpha,beta", [(1.0, 1.0), (0.5, -0.75), (-1.0, 0.3), (0.0, 2.0)])
def test_beta_c(shape, alpha, beta):
    # (20480, 256, 256): without C the library picks the persistent schedule;
    # with C it must fall back to a tiled variant.  (3848, 3840, 136) takes
    # the 256 x 256 tiles, with M and N tails; (4096, 4104, 256) the same
    # tiles on the one-wave schedule (K % 64 == 0), with an N tail.
    M, N, K = shape
    say(f"[case] beta {shape} alpha={alpha} beta={beta}")
    A, B = inputs.operands(M, N, K, 600 + M + K)
    Cm = inputs.matrix(M, N, 700 + N, "normal")
    a32, b32 = float(np.float32(alpha)), float(np.float32(beta))
    c_dev = to_dev(Cm)
    d = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    sg.gemm(to_dev(A), to_dev(B), out=d, alpha=a32, beta=b32, C=c_dev)
    torch.cuda.synchronize()
    rep = oracle.check(d.cpu().numpy(), oracle.gemm_tn_f64_beta(A, B, Cm, a32, b32), K)
    assert rep.ok, str(rep)
    # in place: C is D
    d2 = to_dev(Cm)
    sg.gemm(to_dev(A), to_dev(B), out=d2, alpha=a32, beta=b32, C=d2)
    torch.cuda.synchronize()
    assert torch.equal(d2.view(torch.int16), d.view(torch.int16))


def test_beta_zero_does_not_read_c():
    say("[case] beta zero with NaN C")
    A, B = inputs.operands(300, 264, 200, 801)
    nanc = torch.full((300, 264), float("nan"), dtype=torch.float16, device=DEV)
    d = torch.empty((300, 264), dtype=torch.float16, device=DEV)
    a, b = to_dev(A), to_dev(B)          # keep the tensors alive across the launch
    sg._lib.gemm_fp16_tn_alpha_beta(300, 264, 200, 0.5, 0.0, a.data_ptr(), b.data_ptr(),
                                    nanc.data_ptr(), d.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rep = oracle.check(d.cpu().numpy(), oracle.gemm_tn_f64(A, B, 0.5), 200)
    assert rep.ok, str(rep)


def test_alpha_one_is_bitwise_plain():
    A, B = inputs.operands(256, 256, 264, 93)
    d1 = run_gemm(A, B).cpu().numpy()
    d2 = run_gemm(A, B, alpha=1.0).cpu().numpy()
    assert np.array_equal(d1.view(np.uint16), d2.view(np.uint16))


def test_identity_and_permutation_exact():
    say("[case] identity / permutation")
    K = 512
    A, _ = inputs.operands(300, K, K, 95)
    eye = np.eye(K, dtype=np.float16)
    d = run_gemm(A, eye).cpu().numpy()
    assert np.array_equal(d.view(np.uint16), A.view(np.uint16))
    perm = np.random.Generator(np.random.PCG64(3)).permutation(K)
    P = np.zeros((K, K), np.float16)
    P[np.arange(K), perm] = 1.0
    d = run_gemm(A, P).cpu().numpy()
    assert np.array_equal(d.view(np.uint16), A[:, perm].view(np.uint16))


def test_all_ones_k8200():
    say("[case] all ones K=8200")
    A = np.ones((260, 8200), np.float16)
    B = np.ones((136, 8200), np.float16)
    d = run_gemm(A, B).cpu().numpy()
    assert np.all(d == np.float16(8200))


def test_deterministic_and_stream():
    A, B = inputs.operands(1024, 1024, 1024, 97)
    a, b = to_dev(A), to_dev(B)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        d1 = sg.gemm(a, b)
        d2 = sg.gemm(a, b)
    s.synchronize()
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
    rep = oracle.check(d1.cpu().numpy(), oracle.gemm_tn_f64(A, B), 1024)
    assert rep.ok, str(rep)


# ---------------------------------------------------------------------------
# the workloads at full size, sampled comparison

def test_attention_scores_full():
    # Q, K 4096 x 128 N(0,1), S = Q K^T / sqrt(128)
    A, B = inputs.workload("attn_scores")
    alpha = float(np.float32(1.0 / math.sqrt(128.0)))
    full_check(A, B, alpha=alpha, label="attn_scores")


def test_square4096():
    # every element against the oracle (about 2 s of fp64 on 16 host cores)
    A, B = inputs.workload("square4096")
    d = run_gemm(A, B)
    assert bool(torch.isfinite(d).all())
    say("[case] full square4096 (oracle on all 16.8M outputs)")
    rep = oracle.check(d.cpu().numpy(), oracle.gemm_tn_f64(A, B), 4096)
    assert rep.ok, str(rep)


@pytest.mark.parametrize("K", inputs.KSWEEP_K)
def test_ksweep_every_stage_count(K):
    # every element of every variant (each stage count of both tile
    # families, and the library's own choice) against one oracle run per K
    A, B = inputs.ksweep(K)
    a, b = to_dev(A), to_dev(B)
    say(f"[case] ksweep K={K}: oracle on all 4.2M outputs")
    ref = oracle.gemm_tn_f64(A, B)
    for cfg in [None] + VARIANTS:
        if cfg is not None and (cfg[:2] not in ((128, 128), (256, 256)) or not runs(cfg, K)):
            continue
        say(f"[case] ksweep K={K} {cfg}")
        d = torch.full((2048, 2048), float("nan"), dtype=torch.float16, device=DEV)
        sg.gemm(a, b, out=d, config=cfg)
        torch.cuda.synchronize()
        rep = oracle.check(d.cpu().numpy(), ref, K)
        assert rep.ok, (K, cfg, str(rep))


def test_square8192():
    # the benchmarked call, every element against the oracle (1.1 TFLOP of
    # fp64 on the host: about 16 s on 16 cores)
    A, B = inputs.workload("square8192")
    d = run_gemm(A, B)
    assert bool(torch.isfinite(d).all())
    say("[case] full square8192 (oracle on all 67M outputs)")
    rep = oracle.check(d.cpu().numpy(), oracle.gemm_tn_f64(A, B), 8192)
    assert rep.ok, str(rep)


def test_graph_replays_match_eager():
    # the launch path makes no allocation, memset or host synchronisation, so
    # it can be captured into a HIP graph: replays, with eager work between
    # them, must reproduce the eager result bit for bit (tiled, persistent
    # and short-K kernels, the remainder form's two kernels, schedule 14, and
    # the 256^3 call that bench.py replays from a graph)
    for (M, N, K) in [(4096, 4096, 512), (2048, 1024, 512), (20480, 256, 256), (4096, 2048, 128),
                      (256, 256, 256), (4352, 4104, 1088), (2048, 2048, 1024)]:
        say(f"[case] graph {M}x{N}x{K}")
        A, B = inputs.operands(M, N, K, 1500 + K)
        a, b = to_dev(A), to_dev(B)
        eager = sg.gemm(a, b)
        torch.cuda.synchronize()
        out = torch.empty_like(eager)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            sg.gemm(a, b, out=out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(3):                 # several steps in one graph
                sg.gemm(a, b, out=out)
        for r in range(4):
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), (M, N, K, r)
            tmp = sg.gemm(a, b)                # eager work between the replays
            torch.cuda.synchronize()
            assert torch.equal(tmp.view(torch.int16), eager.view(torch.int16))


@pytest.mark.parametrize("shape", [(4096, 4096, 128), (2048, 2048, 16384), (4352, 4104, 1088)])
def test_bench_launch_function_replays_from_a_graph(shape):
    # bench.py times launch-bound calls by replaying a captured graph of the
    # library call it builds (short-K, split-K with its workspace, the
    # remainder form): the graph must hold the kernels, so a replay rewrites
    # D with the eager result
    import os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    M, N, K = shape
    say(f"[case] bench launch function in a graph {shape}")
    A, B = inputs.operands(M, N, K, 2300 + K)
    a, b = to_dev(A), to_dev(B)
    d = torch.empty((M, N), dtype=torch.float16, device=DEV)
    fn, _, _ = bench.library_call(M, N, K, a, b, d, None)
    fn()
    torch.cuda.synchronize()
    eager = d.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(2):
        d.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.view(torch.int16), eager.view(torch.int16)), shape


def test_calls_from_several_host_threads():
    # host threads, each on its own stream, call the tiled (split-load
    # ping-pong), persistent, short-K and attention entry points at once; the
    # launchers share only per-device caches, and every result must equal the
    # one the same call gives alone, bit for bit
    import threading
    cases = [((3072, 3080, 520), 1701), ((20480, 256, 256), 1703), ((4096, 2048, 128), 1705)]
    ops = []
    for (M, N, K), seed in cases:
        A, B = inputs.operands(M, N, K, seed)
        a, b = to_dev(A), to_dev(B)
        ops.append(lambda a=a, b=b: sg.gemm(a, b))
    gen = torch.Generator().manual_seed(1707)
    q, k, v = (torch.randn((4, 512, 128), generator=gen).half().cuda() for _ in range(3))
    ops.append(lambda: sg.attention(q, k, v, splits=2))
    alone = []
    for op in ops:
        alone.append(op())
        torch.cuda.synchronize()
    results, errors = {}, []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [ops[i]() for _ in range(4)]
            s.synchronize()
            results[i] = outs
        except Exception as e:             # reported from the main thread
            errors.append((i, repr(e)))

    say("[case] host threads")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(ops))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    for i, ref in enumerate(alone):
        for r, out in enumerate(results[i]):
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (i, r)


def test_two_streams_concurrently():
    # independent calls on three streams at once (two persistent launches
    # competing for the same CUs, and the one-wave schedule 12, whose
    # workgroups take a whole CU's LDS) each match the oracle
    A1, B1 = inputs.operands(20480, 256, 256, 1601)
    A2, B2 = inputs.operands(2048, 2048, 1024, 1603)
    A3, B3 = inputs.operands(3072, 3080, 520, 1605)
    a1, b1, a2, b2 = to_dev(A1), to_dev(B1), to_dev(A2), to_dev(B2)
    a3, b3 = to_dev(A3), to_dev(B3)
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = sg.gemm(a1, b1)
        with torch.cuda.stream(s2):
            o2 = sg.gemm(a2, b2)
        with torch.cuda.stream(s3):
            o3 = sg.gemm(a3, b3)
        outs.append((o1, o2, o3))
    torch.cuda.synchronize()
    assert sg._lib.sg_select_config(3072, 3080, 520).as_tuple() == (256, 256, 64, 3, 4, 12)
    ref1 = oracle.gemm_tn_f64(A1, B1)
    ref2 = oracle.gemm_tn_f64(A2, B2)
    ref3 = oracle.gemm_tn_f64(A3, B3)
    for o1, o2, o3 in outs:
        assert oracle.check(o1.cpu().numpy(), ref1, 256).ok
        assert oracle.check(o2.cpu().numpy(), ref2, 1024).ok
        assert oracle.check(o3.cpu().numpy(), ref3, 520).ok


def test_tall_skinny_81920():
    # every element, for the library's choice and every persistent variant
    A, B = inputs.workload("tall81920")
    ref = oracle.gemm_tn_f64(A, B)
    for cfg in [None] + PERSISTENT:
        say(f"[case] full tall81920 {cfg}")
        d = run_gemm(A, B, config=cfg).cpu().numpy()
        rep = oracle.check(d, ref, 256)
        assert rep.ok, (cfg, str(rep))


@pytest.mark.parametrize("shape", [(4096, 4096, 128), (1000, 1032, 120), (264, 8, 8), (520, 4104, 64)])
def test_short_k_schedule(shape):
    # whole K extent in the ring, epilogue per row block: K up to the ring,
    # with M, N and K tails
    M, N, K = shape
    A, B = inputs.operands(M, N, K, 1300 + K, "normal")
    alpha = float(np.float32(1.0 / math.sqrt(K)))
    ref = oracle.gemm_tn_f64(A, B, alpha)
    assert SHORTK
    for cfg in SHORTK:
        if not runs(cfg, K):
            continue
        say(f"[case] short-K {shape} {cfg}")
        d = run_gemm(A, B, alpha=alpha, config=cfg).cpu().numpy()
        rep = oracle.check(d, ref, K)
        assert rep.ok, (cfg, str(rep))


@pytest.mark.parametrize("shape", [(2048, 2048, 128), (4104, 4096, 64), (8192, 8200, 128),
                                   (81920, 256, 128), (81928, 256, 64)])
def test_short_loop_tile_orders(shape):
    # the short-K and persistent kernels walk their tiles row-major where A
    # and B fit in one XCD's L2 (4 MiB) and XCD-renumbered where they do
    # not (8192 x 8200 x 128 is just past it; 81928 rows give a tile count
    # that is not a multiple of 8, which the renumbering leaves alone); the
    # library's own choice among them too, every element
    M, N, K = shape
    A, B = inputs.operands(M, N, K, 2100 + K, "uniform")
    ref = oracle.gemm_tn_f64(A, B)
    for cfg in [None, (128, 128, 64, 2, 4, 3), (128, 128, 64, 2, 4, 4)]:
        say(f"[case] short-loop order {shape} {cfg}")
        d = run_gemm(A, B, config=cfg).cpu().numpy()
        rep = oracle.check(d, ref, K)
        assert rep.ok, (cfg, str(rep))


def test_attention_scores_persistent():
    A, B = inputs.workload("attn_scores")
    alpha = float(np.float32(1.0 / math.sqrt(128.0)))
    ref = oracle.gemm_tn_f64(A, B, alpha)
    for cfg in PERSISTENT:
        say(f"[case] attn_scores {cfg}")
        d = run_gemm(A, B, alpha=alpha, config=cfg).cpu().numpy()
        rep = oracle.check(d, ref, 128)
        assert rep.ok, (cfg, str(rep))


def test_ragged8000():
    # not a tile multiple in any dimension: every element against the oracle
    A, B = inputs.workload("ragged8000")
    d = run_gemm(A, B)
    assert bool(torch.isfinite(d).all())
    say("[case] full ragged8000 (oracle on all 63.5M outputs)")
    rep = oracle.check(d.cpu().numpy(), oracle.gemm_tn_f64(A, B), 8200)
    assert rep.ok, str(rep)


@pytest.mark.parametrize("shape", [(3072, 3080, 520), (40960, 256, 2056), (2600, 2560, 1032)])
def test_selection_refit_shapes(shape):
    # shapes whose tile family the fitted round-cost model decides: mid-size
    # squares and a tall shape with a long K loop go to 256x256 tiles
    # (schedule 12: K % 64 != 0), 2600 x 2560 to 128x128 tiles; every element
    M, N, K = shape
    A, B = inputs.operands(M, N, K, 1500 + K)
    cfg = sg._lib.sg_select_config(M, N, K).as_tuple()
    want = (128, 128, 64, 2, 4, 1) if M == 2600 else (256, 256, 64, 3, 4, 12)
    assert cfg == want, (shape, cfg)
    full_check(A, B, label=f"refit {shape} -> {cfg}")


def test_random_shapes_variants_and_alpha():
    # seeded random cases beyond the fixed grids: any M, N and K tail, any
    # compiled variant that takes the K, any alpha; every element
    g = np.random.Generator(np.random.PCG64(4242))
    for case in range(40):
        M = int(g.integers(1, 700))
        N = 8 * int(g.integers(1, 80))
        K = 8 * int(g.integers(0, 80))
        cands = [c for c in VARIANTS if runs(c, K)]
        cfg = cands[int(g.integers(0, len(cands)))]
        alpha = float(np.float32(g.choice([1.0, 0.5, -1.25, 1.0 / 3.0, 2.0 ** -7])))
        A = g.uniform(-1, 1, (M, K)).astype(np.float16)
        B = g.uniform(-1, 1, (N, K)).astype(np.float16)
        say(f"[case] random {case}: {M}x{N}x{K} cfg={cfg} alpha={alpha}")
        d = run_gemm(A, B, alpha, cfg).cpu().numpy()
        rep = oracle.check(d, oracle.gemm_tn_f64(A, B, alpha), K)
        assert rep.ok, (case, M, N, K, cfg, alpha, str(rep))
