"""GPU parity of the fused attention forward (attention_fp16_fwd) against the
oracle's fp64 attention, O = softmax(alpha Q K^T) V.

Tolerance, derived from the arithmetic (the pages give none): the scores are
fp32 sums of exact fp16 products and the exponentials are fp32, both far
below the other terms; the probabilities enter P V rounded to fp16 (relative
error <= 2^-11 each) while the row sum uses them unrounded, and P V adds N
fp32 terms.  With w = sum_j p_j |v_jc| (from the oracle) the output error is
at most (2^-11 + N 2^-24) w, plus the final rounding of O.  The check allows
twice that:  |O - O_ref| <= 2 ulp16(|O_ref|) + 2 (2^-11 + N 2^-24) w."""
import math

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


def qkv(H, M, N, seed, scale=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    Q = (scale * g.standard_normal((H, M, 128))).astype(np.float16)
    K = g.standard_normal((H, N, 128)).astype(np.float16)
    V = g.standard_normal((H, N, 128)).astype(np.float16)
    return Q, K, V


def gpu_attention(Q, K, V, alpha, splits=None):
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (Q, K, V))
    o = torch.full(q.shape, float("nan"), dtype=torch.float16, device=DEV)
    ws = None
    if splits is not None and splits > 1:
        # scratch contents on entry must not matter
        H, M, N = Q.shape[0], Q.shape[1], K.shape[1]
        need = sg.attention_fp16_workspace_bytes(H, M, N, 128, splits)
        ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    sg.attention(q, k, v, alpha=alpha, out=o, splits=splits, workspace=ws)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def check(Q, K, V, alpha, label, splits=None):
    N = K.shape[-2]
    say(f"[case] attention {label} Q{Q.shape} N={N} alpha={alpha} splits={splits}")
    O = gpu_attention(Q, K, V, alpha, splits).astype(np.float64)
    ref, w = oracle.attention_f64(Q, K, V, alpha, with_bound=True)
    ref = ref.astype(np.float64)
    assert np.all(np.isfinite(O)), label
    bound = 2 * oracle.ulp16(np.abs(ref)) + 2 * (2.0 ** -11 + N * 2.0 ** -24) * w
    err = np.abs(O - ref)
    excess = err - bound
    say(f"         max |err| {err.max():.3g}, max |err| / bound {float((err / bound).max()):.3f}")
    assert excess.max() <= 0, (label, float(excess.max()), np.unravel_index(excess.argmax(), O.shape))
    return O, ref


@pytest.mark.parametrize("H,M,N", [(1, 1, 1), (1, 37, 1), (1, 128, 64), (2, 129, 65), (1, 300, 63),
                                   (3, 200, 200), (1, 64, 1000), (2, 513, 777)])
def test_small_and_ragged(H, M, N):
    Q, K, V = qkv(H, M, N, 4000 + M + N)
    check(Q, K, V, float(np.float32(1.0 / math.sqrt(128))), f"ragged {H}x{M}x{N}")


def test_one_key_is_its_value_row():
    # softmax over one key is exactly 1: O = v (bitwise)
    Q, K, V = qkv(2, 150, 1, 4101)
    O = gpu_attention(Q, K, V, 0.3)
    assert np.array_equal(O.view(np.uint16), np.broadcast_to(V, O.shape).view(np.uint16))


@pytest.mark.parametrize("scale", [0.0, 0.05, 4.0])
def test_flat_and_sharp_softmax(scale):
    # alpha scale 0: uniform weights (mean of V); large: nearly one-hot rows,
    # where the running maximum changes between key tiles
    Q, K, V = qkv(1, 256, 640, 4103 + int(10 * scale))
    check(Q, K, V, float(np.float32(scale)), f"scale {scale}")


@pytest.mark.parametrize("alpha,N", [(-0.0884, 700), (-1.5, 130), (0.0, 100), (-0.0, 1)])
def test_negative_and_zero_alpha(alpha, N):
    # alpha < 0: the largest scaled score comes from the smallest score;
    # alpha = 0 with a ragged last key tile: uniform weights over the N keys
    Q, K, V = qkv(2, 160, N, 4111 + N)
    check(Q, K, V, float(np.float32(alpha)), f"alpha {alpha} N={N}")


@pytest.mark.parametrize("top", [4.0, 30.0])
def test_growing_scores(top):
    # key rows scaled up along the sequence, so a row's maximum keeps rising
    # from tile to tile: by less than the rescale threshold (top 4) or far
    # beyond it (top 30), both with and without a rescale of O
    Q, K, V = qkv(1, 256, 1500, 4113 + int(top))
    K = (K.astype(np.float64) * np.linspace(1.0, top, 1500)[None, :, None]).astype(np.float16)
    check(Q, K, V, float(np.float32(1.0 / math.sqrt(128))), f"growing to x{top}")


@pytest.mark.parametrize("H,M,N,splits", [(1, 300, 1000, 1), (1, 300, 1000, 2), (1, 300, 1000, 5),
                                          (2, 129, 65, 2), (1, 37, 200, 4), (1, 200, 130, 100),
                                          (3, 256, 4096, 16), (1, 1, 1, 3)])
def test_split_keys(H, M, N, splits):
    # keys cut into runs merged afterwards; more splits than key tiles are
    # lowered to one run per tile
    Q, K, V = qkv(H, M, N, 4115 + M + N + splits)
    check(Q, K, V, float(np.float32(1.0 / math.sqrt(128))), f"split {splits}", splits=splits)


def test_split_growing_and_negative():
    # runs with very different maxima (keys scaled up along the sequence),
    # and alpha < 0
    Q, K, V = qkv(1, 256, 1500, 4117)
    K = (K.astype(np.float64) * np.linspace(1.0, 30.0, 1500)[None, :, None]).astype(np.float16)
    check(Q, K, V, float(np.float32(1.0 / math.sqrt(128))), "split growing", splits=6)
    check(Q, K, V, -0.0884, "split negative", splits=6)


def test_split_choice_and_workspace_reuse():
    # the library's choice on this device: one head of 4096 queries is 32
    # row blocks, far from two per CU; sixteen heads already fill the device
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s1 = sg.attention_fp16_splits(1, 4096, 4096, 128)
    assert 1 <= s1 <= 64
    if cus == 256:
        assert s1 == 8                                 # the fastest measured on MI355X
        assert sg.attention_fp16_splits(16, 4096, 4096, 128) == 1
    assert sg.attention_fp16_splits(1, 4096, 40, 128) == 1    # one key tile
    # one workspace, two calls of different shapes back to back
    need = sg.attention_fp16_workspace_bytes(2, 512, 2000, 128, 8)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
    outs = []
    for H, M, N in ((2, 512, 2000), (1, 100, 700)):
        Q, K, V = qkv(H, M, N, 4119 + N)
        q, k, v = (torch.from_numpy(x).to(DEV) for x in (Q, K, V))
        o = sg.attention(q, k, v, alpha=0.09, splits=8, workspace=ws)
        outs.append((o, Q, K, V))
    torch.cuda.synchronize()
    for o, Q, K, V in outs:
        ref, w = oracle.attention_f64(Q, K, V, 0.09, with_bound=True)
        bound = 2 * oracle.ulp16(np.abs(ref.astype(np.float64))) + 2 * (2.0 ** -11 + K.shape[1] * 2.0 ** -24) * w
        assert np.all(np.abs(o.cpu().numpy().astype(np.float64) - ref.astype(np.float64)) <= bound)


@pytest.mark.parametrize("H,M,N", [(64, 1024, 300), (256, 200, 77), (260, 129, 64)])
def test_wide_workgroups(H, M, N):
    # grids whose 256-row workgroups fill every CU take the 8-wave kernel
    # (ragged M inside a 256-row block included)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert H * -(-M // 256) >= cus
    Q, K, V = qkv(H, M, N, 4121 + H)
    check(Q, K, V, float(np.float32(1.0 / math.sqrt(128))), f"wide {H}x{M}x{N}")
    check(Q, K, V, -0.07, f"wide {H}x{M}x{N} alpha<0")


def test_sixteen_heads_sampled_rows():
    # the 16-head 4096 x 4096 x 128 shape the bench times: every output
    # finite, 48 sampled rows per head against the oracle
    H, M, N = 16, 4096, 4096
    Q, K, V = qkv(H, M, N, 4123)
    alpha = float(np.float32(1.0 / math.sqrt(128)))
    say(f"[case] attention 16 heads full, sampled rows")
    O = gpu_attention(Q, K, V, alpha).astype(np.float64)
    assert np.all(np.isfinite(O))
    g = np.random.Generator(np.random.PCG64(4125))
    rows = np.sort(np.concatenate([[0, 255, 256, M - 1], g.choice(M, 44, replace=False)]))
    ref, w = oracle.attention_f64(np.ascontiguousarray(Q[:, rows]), K, V, alpha, with_bound=True)
    ref = ref.astype(np.float64)
    bound = 2 * oracle.ulp16(np.abs(ref)) + 2 * (2.0 ** -11 + N * 2.0 ** -24) * w
    err = np.abs(O[:, rows] - ref)
    say(f"         max |err| {err.max():.3g}, max |err| / bound {float((err / bound).max()):.3f}")
    assert np.all(err <= bound)


def test_attention_config_full():
    # the attention-score workload's Q and K (4096 x 128, N(0,1)) with a V of
    # the same shape, alpha = fp32(1/sqrt(128)); every output against the oracle
    Q, K = inputs.workload("attn_scores")
    V = inputs.matrix(4096, 128, 4105, "normal")
    for splits in (None, 1):
        check(Q[None], K[None], V[None], float(np.float32(1.0 / math.sqrt(128))), "4096x4096x128",
              splits=splits)


def test_multi_head():
    Q, K, V = qkv(8, 1024, 1024, 4107)
    check(Q, K, V, float(np.float32(1.0 / math.sqrt(128))), "8 heads 1024x1024")


def test_deterministic():
    Q, K, V = qkv(2, 300, 500, 4109)
    a = gpu_attention(Q, K, V, 0.1)
    b = gpu_attention(Q, K, V, 0.1)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_empty_and_unsupported():
    q = torch.zeros((1, 0, 128), dtype=torch.float16, device=DEV)
    k = torch.zeros((1, 8, 128), dtype=torch.float16, device=DEV)
    assert sg.attention(q, k, k).shape == (1, 0, 128)
    q64 = torch.zeros((1, 8, 64), dtype=torch.float16, device=DEV)
    with pytest.raises(sg.SgError):
        sg.attention(q64, q64, q64)


def test_graph_replays_match_eager():
    # no allocation, memset or host synchronisation on the launch path (the
    # split call's workspace is the caller's): captured into a HIP graph,
    # replays with eager work between them reproduce the eager result bit for
    # bit, for the 4-wave, 8-wave and split kernels
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for (H, M, N, splits) in [(2, 300, 700, 1), (cus, 256, 200, 1), (1, 512, 2048, 4)]:
        say(f"[case] attention graph H={H} M={M} N={N} splits={splits}")
        Q, K, V = qkv(H, M, N, 4127 + N)
        q, k, v = (torch.from_numpy(x).to(DEV) for x in (Q, K, V))
        need = max(sg.attention_fp16_workspace_bytes(H, M, N, 128, splits), 16)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        eager = sg.attention(q, k, v, alpha=0.09, splits=splits, workspace=ws)
        torch.cuda.synchronize()
        out = torch.empty_like(eager)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            sg.attention(q, k, v, alpha=0.09, out=out, splits=splits, workspace=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sg.attention(q, k, v, alpha=0.09, out=out, splits=splits, workspace=ws)
        for r in range(4):
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), (H, M, N, splits, r)
            tmp = sg.attention(q, k, v, alpha=0.09, splits=splits, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(tmp.view(torch.int16), eager.view(torch.int16))


def test_two_streams_concurrently():
    # a split call and a wide call on two streams at once, each with its own
    # workspace, both match the oracle
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Q1, K1, V1 = qkv(1, 1024, 3000, 4129)
    Q2, K2, V2 = qkv(cus, 256, 100, 4131)
    d1 = [torch.from_numpy(x).to(DEV) for x in (Q1, K1, V1)]
    d2 = [torch.from_numpy(x).to(DEV) for x in (Q2, K2, V2)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws1 = torch.empty(sg.attention_fp16_workspace_bytes(1, 1024, 3000, 128, 6), dtype=torch.uint8, device=DEV)
    outs = []
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = sg.attention(*d1, alpha=0.1, splits=6, workspace=ws1)
        with torch.cuda.stream(s2):
            o2 = sg.attention(*d2, alpha=0.1)
        outs.append((o1, o2))
        s1.synchronize()                               # ws1 is reused by the next iteration
    torch.cuda.synchronize()
    for (Q, K, V), idx in (((Q1, K1, V1), 0), ((Q2, K2, V2), 1)):
        ref, w = oracle.attention_f64(Q, K, V, 0.1, with_bound=True)
        ref = ref.astype(np.float64)
        bound = 2 * oracle.ulp16(np.abs(ref)) + 2 * (2.0 ** -11 + K.shape[1] * 2.0 ** -24) * w
        for pair in outs:
            err = np.abs(pair[idx].cpu().numpy().astype(np.float64) - ref)
            assert np.all(err <= bound), idx


def test_random_shapes_alpha_and_splits():
    # seeded random cases: heads, ragged M and N, alpha of either sign and
    # size, the library's split count or a random one up to the key tiles
    g = np.random.Generator(np.random.PCG64(4343))
    for case in range(24):
        H = int(g.integers(1, 4))
        M = int(g.integers(1, 420))
        N = int(g.integers(1, 900))
        alpha = float(np.float32(g.choice([1.0 / math.sqrt(128), -1.0 / math.sqrt(128), 0.02, -0.3])))
        ntiles = (N + 63) // 64
        splits = None if g.integers(0, 3) == 0 else int(g.integers(1, min(ntiles, 8) + 1))
        Q, K, V = qkv(H, M, N, 5000 + case, scale=float(g.choice([0.5, 1.0, 2.0])))
        check(Q, K, V, alpha, f"random {case}", splits=splits)
