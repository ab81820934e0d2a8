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


def gpu_attention(Q, K, V, alpha):
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (Q, K, V))
    o = torch.full(q.shape, float("nan"), dtype=torch.float16, device=DEV)
    sg.attention(q, k, v, alpha=alpha, out=o)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def check(Q, K, V, alpha, label):
    N = K.shape[-2]
    say(f"[case] attention {label} Q{Q.shape} N={N} alpha={alpha}")
    O = gpu_attention(Q, K, V, alpha).astype(np.float64)
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


def test_attention_config_full():
    # the attention-score workload's Q and K (4096 x 128, N(0,1)) with a V of
    # the same shape, alpha = fp32(1/sqrt(128)); every output against the oracle
    Q, K = inputs.workload("attn_scores")
    V = inputs.matrix(4096, 128, 4105, "normal")
    check(Q[None], K[None], V[None], float(np.float32(1.0 / math.sqrt(128))), "4096x4096x128")


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
