"""GPU parity of the forward pass (fa_fwd / fa_fwd_f32) against the float64 oracle.

Every comparison feeds the oracle the float64 upcast of exactly the values the
GPU received.  Tolerances (max abs over all compared elements): O within 2e-2
for bf16 outputs and 1e-5 for fp32 inputs; lse within 1e-3.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_10_amd as fa
from oracle import naive_fwd, naive_fwd_rows
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu


def _s32(x):
    """The scale as the kernels receive it: a float32, widened for the oracle."""
    return float(np.float32(x))

TOL_BF16 = 2e-2
TOL_F32 = 1e-5
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")
    fa.load_library()


def _say(*a):
    print(*a, flush=True)


def _run(q, k, v, causal, scale, prefill_nan=True):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    B, H, N, d = q.shape
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    if prefill_nan:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    if q.dtype == torch.float32:
        fa.fa_fwd_f32(qd, kd, vd, o, lse, causal, scale)
    else:
        fa.fa_fwd(qd, kd, vd, o, lse, causal, scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _f64(t):
    return t.float().numpy().astype(np.float64)


SMALL_N = [1, 2, 63, 65, 127, 129, 257, 1000]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SMALL_N)
def test_bf16_small_and_ragged(N, causal, d):
    _say(f"[fwd bf16] N={N} d={d} causal={causal}")
    q, k, v = make_inputs(2, 3, N, d, torch.bfloat16, seed=100 + N)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(q, k, v, causal, scale)
    ro, rl = naive_fwd(_f64(q), _f64(k), _f64(v), _s32(scale), causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    eo = np.max(np.abs(o - ro))
    el = np.max(np.abs(lse - rl))
    _say(f"   max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL_BF16 and el <= TOL_LSE


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 31, 33, 129, 256, 300])
def test_f32_small_and_ragged(N, causal, d):
    _say(f"[fwd f32] N={N} d={d} causal={causal}")
    q, k, v = make_inputs(1, 2, N, d, torch.float32, seed=200 + N)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(q, k, v, causal, scale)
    ro, rl = naive_fwd(_f64(q), _f64(k), _f64(v), _s32(scale), causal)
    eo = np.max(np.abs(o - ro))
    el = np.max(np.abs(lse - rl))
    _say(f"   max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL_F32 and el <= TOL_LSE


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_grid_that_fills_the_gpu(causal, d):
    """fa_fwd_f32 on a grid of at least one 128-query tile per CU (4 x 32
    heads x 300 rows: 384 tiles), where the tile kernel runs rather than the
    key-split kernel the small cases above take: sampled whole heads."""
    _say(f"[fwd f32 large grid] d={d} causal={causal}")
    q, k, v = make_inputs(4, 32, 300, d, torch.float32, seed=260 + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(q, k, v, causal, scale)
    worst_o = worst_l = 0.0
    for (b, h) in [(0, 0), (1, 7), (2, 17), (3, 31)]:
        ro, rl = naive_fwd(_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _s32(scale), causal)
        worst_o = max(worst_o, float(np.max(np.abs(o[b, h] - ro))))
        worst_l = max(worst_l, float(np.max(np.abs(lse[b, h] - rl))))
    _say(f"   max|dO|={worst_o:.3e} max|dlse|={worst_l:.3e}")
    assert worst_o <= TOL_F32 and worst_l <= TOL_LSE


def test_single_head_fp32_workload_full():
    """Single-head fp32 workload at full size (1 x 1 x 256 x 64, non-causal)."""
    w = WORKLOADS["single_head_fp32_n256"]
    q, k, v = workload_inputs(w)
    o, lse = _run(q, k, v, False, w.scale)
    ro, rl = naive_fwd(_f64(q), _f64(k), _f64(v), _s32(w.scale), False)
    eo = np.max(np.abs(o - ro))
    _say(f"[{w.name}] max|dO|={eo:.3e} max|dlse|={np.max(np.abs(lse - rl)):.3e}")
    assert eo <= TOL_F32
    assert np.max(np.abs(lse - rl)) <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_gpt2_medium_workload_full(causal):
    """GPT-2-medium shape (8 x 16 x 1024 x 64, every 7th query row x4): every
    output element against the oracle."""
    w = WORKLOADS["gpt2_medium_n1024"]
    q, k, v = workload_inputs(w)
    _say(f"[{w.name}] causal={causal}")
    o, lse = _run(q, k, v, causal, w.scale)
    ro, rl = naive_fwd(_f64(q), _f64(k), _f64(v), _s32(w.scale), causal)
    eo = np.max(np.abs(o - ro))
    el = np.max(np.abs(lse - rl))
    _say(f"   max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL_BF16 and el <= TOL_LSE


def _sampled_check(w, causal, heads, rows_per_head=48, seed=0):
    q, k, v = workload_inputs(w)
    o, lse = _run(q, k, v, causal, w.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(seed)
    N = w.N
    worst_o = worst_l = 0.0
    for (b, h) in heads:
        pos = np.unique(np.concatenate([
            [0, 1, 63, 64, 127, 128, N - 1],
            rng.integers(0, N, size=rows_per_head)]))
        ro, rl = naive_fwd_rows(_f64(q[b, h, pos]), _f64(k[b, h]), _f64(v[b, h]),
                                _s32(w.scale), causal, pos)
        worst_o = max(worst_o, float(np.max(np.abs(o[b, h, pos] - ro))))
        worst_l = max(worst_l, float(np.max(np.abs(lse[b, h, pos] - rl))))
    _say(f"   sampled max|dO|={worst_o:.3e} max|dlse|={worst_l:.3e}")
    assert worst_o <= TOL_BF16 and worst_l <= TOL_LSE
    return q, k, v, o, lse


def test_llama8b_workload_sampled():
    """Llama-3.1-8B shape (1 x 32 x 4096 x 128, causal), sampled rows of several
    heads against the oracle, in the bench's launch configuration."""
    w = WORKLOADS["llama8b_n4096"]
    _say(f"[{w.name}]")
    _sampled_check(w, True, [(0, 0), (0, 7), (0, 19), (0, 31)])


def _full_heads_check(w, causal, heads):
    """Every element of the listed heads against the oracle, in the bench's
    launch configuration (the whole workload in one call)."""
    q, k, v = workload_inputs(w)
    o, lse = _run(q, k, v, causal, w.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    worst_o = worst_l = 0.0
    for (b, h) in heads:
        ro, rl = naive_fwd(_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _s32(w.scale), causal)
        eo = float(np.max(np.abs(o[b, h] - ro)))
        el = float(np.max(np.abs(lse[b, h] - rl)))
        _say(f"   head ({b},{h}) max|dO|={eo:.3e} max|dlse|={el:.3e}")
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
    assert worst_o <= TOL_BF16 and worst_l <= TOL_LSE


def test_llama8b_workload_full_heads_one_per_xcd():
    """Llama-3.1-8B shape (1 x 32 x 4096 x 128, causal): every element of eight
    whole heads, 0, 4, .., 28 -- the grid order gives XCD x the heads 4x..4x+3,
    so these run on eight different XCDs."""
    w = WORKLOADS["llama8b_n4096"]
    _say(f"[{w.name}] full heads")
    _full_heads_check(w, True, [(0, h) for h in range(0, 32, 4)])


def test_long_context_n16384_full_head():
    """Long-context shape (1 x 8 x 16384 x 128, causal): every element of one
    whole head (head 5, the one XCD 5 owns)."""
    w = WORKLOADS["long_context_n16384"]
    _say(f"[{w.name}] full head")
    _full_heads_check(w, True, [(0, 5)])


@pytest.mark.parametrize("name", ["long_context_n16384", "long_context_n32768"])
def test_long_context_sampled(name):
    w = WORKLOADS[name]
    _say(f"[{name}]")
    _sampled_check(w, True, [(0, 0), (0, 5)], rows_per_head=24)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_zero_queries_full_size(causal, d):
    """Q = 0 at a full-size shape: P is uniform over the visible keys, so O_i is
    the mean of those V rows and lse_i = log(count) (exact closed form)."""
    N = 4096
    _, k, v = make_inputs(1, 2, N, d, torch.bfloat16, seed=7)
    q = torch.zeros_like(k)
    o, lse = _run(q, k, v, causal, 1.0 / math.sqrt(d))
    vv = _f64(v)
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(vv, axis=2) / cnt[None, None, :, None] if causal else \
        np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
    assert np.max(np.abs(o - mean)) <= TOL_BF16
    assert np.max(np.abs(lse - np.log(cnt)[None, None, :])) <= TOL_LSE


def test_output_in_convex_hull_full_size():
    w = WORKLOADS["llama8b_n4096"]
    q, k, v = make_inputs(1, 4, w.N, w.d, torch.bfloat16, seed=11)
    o, _ = _run(q, k, v, True, w.scale)
    vv = _f64(v)
    cmax = np.maximum.accumulate(vv, axis=2)
    cmin = np.minimum.accumulate(vv, axis=2)
    slack = 1e-2
    assert np.all(o <= cmax + slack) and np.all(o >= cmin - slack)


def test_large_scores_finite():
    """Scores far past fp32's exp overflow point stay finite and correct."""
    q, k, v = make_inputs(1, 2, 300, 64, torch.bfloat16, seed=12)
    q = (q.float() * 24).to(torch.bfloat16)
    o, lse = _run(q, k, v, True, 1.0)
    ro, rl = naive_fwd(_f64(q), _f64(k), _f64(v), 1.0, True)
    assert np.max(rl) > 100
    assert np.max(np.abs(o - ro)) <= TOL_BF16
    assert np.max(np.abs(lse - rl)) <= TOL_LSE


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_running_max_grows_every_tile(causal, d):
    """Key blocks of 64 with growing norm: the running max rises by ~10 natural
    units per tile, so the rescale by exp(m_old - m_new) fires tile after tile
    (P2 section 2), and the last block jumps by thousands of units (a
    probability formed against the old max would overflow fp32)."""
    N = 700
    q, k, v = make_inputs(1, 2, N, d, torch.bfloat16, seed=15)
    grow = torch.tensor([1.0 + 0.5 * (j // 64) for j in range(N)])
    grow[640:] *= 20.0
    k = (k.float() * grow[None, None, :, None]).to(torch.bfloat16)
    o, lse = _run(q, k, v, causal, 1.0)
    ro, rl = naive_fwd(_f64(q), _f64(k), _f64(v), 1.0, causal)
    jumps = np.diff(rl[0, 0, ::64])
    _say(f"   lse at every 64th row: {np.round(rl[0, 0, ::64], 1)}")
    assert np.max(rl) > 1000
    assert np.max(np.abs(o - ro)) <= TOL_BF16
    assert np.max(np.abs(lse - rl)) <= TOL_LSE * max(1.0, np.max(np.abs(rl)) / 1000)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 2.0])
def test_unusual_scales(scale):
    q, k, v = make_inputs(1, 2, 200, 64, torch.bfloat16, seed=13)
    for causal in (False, True):
        o, lse = _run(q, k, v, causal, scale)
        ro, rl = naive_fwd(_f64(q), _f64(k), _f64(v), _s32(scale), causal)
        assert np.max(np.abs(o - ro)) <= TOL_BF16
        assert np.max(np.abs(lse - rl)) <= TOL_LSE


def test_forward_is_deterministic():
    w = WORKLOADS["gpt2_medium_n1024"]
    q, k, v = (t.cuda() for t in make_inputs(2, 4, 1024, 64, torch.bfloat16, seed=14))
    o1, l1 = fa.forward(q, k, v, True, w.scale)
    o2, l2 = fa.forward(q, k, v, True, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_is_noop():
    q = torch.empty((2, 3, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.forward(q, q, q, True)
    assert o.shape == q.shape and lse.shape == (2, 3, 0)
