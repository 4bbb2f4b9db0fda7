"""GPU parity of the head-dimension-256 forward (fa_fwd, fa_fwd_gqa and
fa_fwd_kv at d = 256) against the float64 oracle.

d = 256 runs its own kernels (32-key tiles; causal with an even number of
query tiles: balanced pairs of tiles, the heavy one split over two wave
groups and merged); the operation
and the tolerances are those of the other forwards: O within 2e-2 (bf16
output), lse within 1e-3, max abs over every element.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_10_amd as fa
from oracle import naive_fwd, naive_fwd_gqa, naive_fwd_kv
from workloads import make_gqa_inputs, make_inputs

pytestmark = pytest.mark.gpu


def _s32(x):
    """The scale as the kernels receive it: a float32, widened for the oracle."""
    return float(np.float32(x))

TOL = 2e-2
TOL_LSE = 1e-3
D = 256


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")
    fa.load_library()


def _say(*a):
    print(*a, flush=True)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _cmp(o, lse, ro, rl):
    eo = float(np.max(np.abs(_f64(o) - ro)))
    el = float(np.max(np.abs(_f64(lse) - rl)))
    _say(f"   max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert eo <= TOL and el <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 31, 33, 129, 256, 257, 1000, 2048])
def test_d256_forward(N, causal):
    _say(f"[d256 fwd] N={N} causal={causal}")
    q, k, v = make_inputs(2, 3, N, D, torch.bfloat16, seed=1000 + N)
    scale = 1 / math.sqrt(D)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal, scale)
    torch.cuda.synchronize()
    _cmp(o, lse, *naive_fwd(_f64(q), _f64(k), _f64(v), _s32(scale), causal))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [300, 512])
def test_d256_forward_gqa(N, causal):
    q, k, v = make_gqa_inputs(1, 8, 2, N, D, seed=1100 + N)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal, 0.07)
    torch.cuda.synchronize()
    _cmp(o, lse, *naive_fwd_gqa(_f64(q), _f64(k), _f64(v), _s32(0.07), causal))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 3000), (40, 700), (300, 100), (256, 700), (1000, 1030)])
def test_d256_forward_kv(nq, nk, causal):
    _say(f"[d256 kv] Nq={nq} Nk={nk} causal={causal}")
    q = make_gqa_inputs(1, 4, 2, nq, D, seed=1200 + nq)[0]
    k, v = make_gqa_inputs(1, 4, 2, nk, D, seed=1300 + nk)[1:]
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal, 1 / math.sqrt(D))
    torch.cuda.synchronize()
    ro, rl = naive_fwd_kv(_f64(q), _f64(k), _f64(v), _s32(1 / math.sqrt(D)), causal)
    live = np.isfinite(rl)
    go, gl = _f64(o), _f64(lse)
    assert np.all(go[~live] == 0) and np.all(gl[~live] == -np.inf)
    eo = float(np.max(np.abs(go - ro)))
    el = float(np.max(np.abs(gl[live] - rl[live]))) if live.any() else 0.0
    _say(f"   max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL and el <= TOL_LSE


def test_d256_large_sampled():
    """[1, 16, 4096, 256] causal: sampled rows of every head."""
    from oracle import naive_fwd_rows
    q, k, v = make_inputs(1, 16, 4096, D, torch.bfloat16, seed=1400)
    scale = 1 / math.sqrt(D)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), True, scale)
    torch.cuda.synchronize()
    go, gl = _f64(o), _f64(lse)
    rng = np.random.default_rng(1)
    wo = wl = 0.0
    for h in range(16):
        rows = np.unique(np.concatenate([[0, 127, 128, 4095], rng.integers(0, 4096, 12)]))
        ro, rl = naive_fwd_rows(_f64(q[0, h, rows]), _f64(k[0, h]), _f64(v[0, h]), _s32(scale), True,
                                rows)
        wo = max(wo, float(np.max(np.abs(go[0, h, rows] - ro))))
        wl = max(wl, float(np.max(np.abs(gl[0, h, rows] - rl))))
    _say(f"[d256 4096 sampled] max|dO|={wo:.3e} max|dlse|={wl:.3e}")
    assert wo <= TOL and wl <= TOL_LSE


def test_d256_causal_pairs_full_heads():
    """[1, 16, 4096, 256] causal, every row of three heads (one per pair
    position: heads on different XCDs) -- the balanced pair kernel, whose
    heavy tiles are split between two wave groups and merged -- against the
    oracle."""
    from oracle import naive_fwd_rows
    q, k, v = make_inputs(1, 16, 4096, D, torch.bfloat16, seed=1500)
    scale = 1 / math.sqrt(D)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), True, scale)
    torch.cuda.synchronize()
    go, gl = _f64(o), _f64(lse)
    rows = np.arange(4096)
    for h in (0, 7, 15):
        ro, rl = naive_fwd_rows(_f64(q[0, h]), _f64(k[0, h]), _f64(v[0, h]), _s32(scale), True, rows)
        eo = float(np.max(np.abs(go[0, h] - ro)))
        el = float(np.max(np.abs(gl[0, h] - rl)))
        _say(f"[d256 pairs head {h}] max|dO|={eo:.3e} max|dlse|={el:.3e}")
        assert eo <= TOL and el <= TOL_LSE


# --- backward at d = 256 -----------------------------------------------------------

def _bwd_check(q, k, v, do, causal, scale):
    from oracle import naive_bwd_kv
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal, scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, causal, scale)
    torch.cuda.synchronize()
    ref = naive_bwd_kv(_f64(q), _f64(k), _f64(v), _f64(do), _s32(scale), causal)
    tol = max(TOL, 2.0 ** -7 * max(float(np.max(np.abs(r))) for r in ref))
    errs = [float(np.max(np.abs(_f64(g) - r))) for g, r in zip((dq, dk, dv), ref)]
    _say(f"   max|d dQ|={errs[0]:.3e} |d dK|={errs[1]:.3e} |d dV|={errs[2]:.3e} (tol {tol:.3e})")
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
    assert max(errs) <= tol


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 129, 300])
def test_d256_backward(N, causal):
    _say(f"[d256 bwd] N={N} causal={causal}")
    q, k, v, do = make_inputs(1, 2, N, D, torch.bfloat16, seed=1500 + N, with_do=True)
    _bwd_check(q, k, v, do, causal, 1 / math.sqrt(D))


@pytest.mark.parametrize("causal", [False, True])
def test_d256_backward_gqa_and_lengths(causal):
    q = make_gqa_inputs(1, 4, 2, 150, D, seed=1600, with_do=True)
    k, v = make_gqa_inputs(1, 4, 2, 400, D, seed=1601)[1:]
    _bwd_check(q[0], k, v, q[3], causal, 1 / math.sqrt(D))


def test_d256_backward_bench_shape_every_head():
    """[1, 16, 4096, 256] causal, the inputs the bench times (fa_fwd then
    fa_bwd, seed 9): every element of dQ, dK and dV of every head against the
    oracle, 2e-2."""
    from oracle import naive_bwd
    q, k, v, do = make_gqa_inputs(1, 16, 16, 4096, D, seed=9, with_do=True)
    scale = 1 / 16.0
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o = torch.empty_like(qd)
    lse = torch.empty((1, 16, 4096), dtype=torch.float32, device="cuda")
    fa.fa_fwd(qd, kd, vd, o, lse, True, scale)
    dq, dk, dv = (torch.full_like(qd, float("nan")) for _ in range(3))
    ws = torch.full((fa.fa_bwd_workspace_size(1, 16, 4096, D),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    fa.fa_bwd(qd, kd, vd, o, dod, lse, dq, dk, dv, ws, True, scale)
    torch.cuda.synchronize()
    worst = 0.0
    for h in range(16):
        ref = naive_bwd(_f64(q[0, h]), _f64(k[0, h]), _f64(v[0, h]), _f64(do[0, h]), _s32(scale),
                        True)
        errs = [float(np.max(np.abs(_f64(g[0, h]) - r))) for g, r in zip((dq, dk, dv), ref)]
        _say(f"   head {h}: max|d dQ|={errs[0]:.3e} |d dK|={errs[1]:.3e} |d dV|={errs[2]:.3e}")
        worst = max(worst, max(errs))
    assert worst <= TOL
