"""GPU parity of grouped-query attention (fa_fwd_gqa, fa_bwd_gqa) against the
float64 oracle (``naive_fwd_gqa`` / ``naive_bwd_gqa``).

H query heads share Hkv key/value heads; query head h reads key/value head
h // (H / Hkv).  Tolerances as for plain attention: O, dQ, dK, dV within 2e-2
(bf16 outputs), lse within 1e-3, max abs over every element.  dK and dV of a
shared head sum H / Hkv query heads' contributions, so their magnitude grows
with the group; where a reference gradient passes O(1) the bar is also at
least one bf16 ulp of the largest reference magnitude (rounding the exact
gradient to bf16 already moves it by half of that).
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_10_amd as fa
from oracle import naive_bwd_gqa, naive_fwd_gqa, naive_fwd_rows
from workloads import make_gqa_inputs

pytestmark = pytest.mark.gpu


def _s32(x):
    """The scale as the kernels receive it: a float32, widened for the oracle."""
    return float(np.float32(x))

TOL = 2e-2
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")
    fa.load_library()


def _say(*a):
    print(*a, flush=True)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _fwd(q, k, v, causal, scale):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    B, H, N, d = q.shape
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd_gqa(qd, kd, vd, o, lse, causal, scale)
    torch.cuda.synchronize()
    return o, lse


CASES = [(4, 1), (4, 2), (8, 2), (6, 3)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 257, 700])
@pytest.mark.parametrize("H,Hkv", CASES)
def test_gqa_forward(H, Hkv, N, causal, d):
    _say(f"[gqa fwd] H={H} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v = make_gqa_inputs(2, H, Hkv, N, d, seed=300 + N + H + Hkv)
    scale = 1.0 / math.sqrt(d)
    o, lse = _fwd(q, k, v, causal, scale)
    ro, rl = naive_fwd_gqa(_f64(q), _f64(k), _f64(v), _s32(scale), causal)
    eo = float(np.max(np.abs(_f64(o) - ro)))
    el = float(np.max(np.abs(_f64(lse) - rl)))
    _say(f"   max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert eo <= TOL and el <= TOL_LSE


def _bwd(q, k, v, do, o, lse, causal, scale, split):
    """fa_bwd_gqa with the plain workspace (no head split) or the one
    fa_bwd_kv_workspace_size asks for (the split the plan picks)."""
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    nb = (fa.fa_bwd_kv_workspace_size(B, H, Hkv, N, N, d) if split
          else fa.fa_bwd_workspace_size(B, H, N, d))
    ws = torch.full((max(1, nb),), 0xFF, dtype=torch.uint8, device="cuda")
    fa.fa_bwd_gqa(qd, kd, vd, o, dod, lse, dq, dk, dv, ws, causal, scale)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 257, 700])
@pytest.mark.parametrize("H,Hkv", CASES)
def test_gqa_backward(H, Hkv, N, causal, d, split):
    """Small shapes, where the plan deals every query head of a group to its
    own workgroup when the workspace allows (split=True)."""
    _say(f"[gqa bwd] H={H} Hkv={Hkv} N={N} d={d} causal={causal} split={split}")
    q, k, v, do = make_gqa_inputs(2, H, Hkv, N, d, seed=400 + N + H + Hkv, with_do=True)
    scale = 1.0 / math.sqrt(d)
    o, lse = _fwd(q, k, v, causal, scale)
    dq, dk, dv = _bwd(q, k, v, do, o, lse, causal, scale, split)
    ref = naive_bwd_gqa(_f64(q), _f64(k), _f64(v), _f64(do), _s32(scale), causal)
    tol = max(TOL, 2.0 ** -7 * max(float(np.max(np.abs(r))) for r in ref))
    errs = [float(np.max(np.abs(_f64(g) - r))) for g, r in zip((dq, dk, dv), ref)]
    _say(f"   max|d dQ|={errs[0]:.3e} |d dK|={errs[1]:.3e} |d dV|={errs[2]:.3e} (tol {tol:.3e})")
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
    assert max(errs) <= tol


def test_gqa_matches_plain_attention_on_repeated_heads():
    """fa_fwd_gqa on K/V with Hkv heads equals fa_fwd on K/V whose heads are
    repeated over each group, bit for bit (the same kernel arithmetic)."""
    q, k, v = make_gqa_inputs(1, 8, 2, 1000, 128, seed=7)
    o, lse = _fwd(q, k, v, True, 1 / math.sqrt(128))
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o2, lse2 = fa.forward(q.cuda(), kr.cuda(), vr.cuda(), True, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_llama8b_gqa_shape_sampled():
    """Llama-3.1-8B's attention shape with its real head sharing (32 query heads
    over 8 key/value heads, N = 4096, d = 128, causal): sampled rows of every
    fourth query head against the oracle."""
    B, H, Hkv, N, d = 1, 32, 8, 4096, 128
    q, k, v = make_gqa_inputs(B, H, Hkv, N, d, seed=6)
    scale = 1 / math.sqrt(d)
    o, lse = _fwd(q, k, v, True, scale)
    o = _f64(o)
    lse = _f64(lse)
    rng = np.random.default_rng(0)
    worst_o = worst_l = 0.0
    for h in range(0, H, 3):
        g = h // (H // Hkv)
        rows = np.unique(np.concatenate([[0, 1, 255, 256, N - 1],
                                         rng.integers(0, N, 24)]))
        ro, rl = naive_fwd_rows(_f64(q[0, h, rows]), _f64(k[0, g]), _f64(v[0, g]), _s32(scale),
                                True, rows)
        worst_o = max(worst_o, float(np.max(np.abs(o[0, h, rows] - ro))))
        worst_l = max(worst_l, float(np.max(np.abs(lse[0, h, rows] - rl))))
    _say(f"[llama8b gqa 32/8] max|dO|={worst_o:.3e} max|dlse|={worst_l:.3e}")
    assert worst_o <= TOL and worst_l <= TOL_LSE


def test_llama8b_gqa_backward():
    """Backward at Llama-3.1-8B's attention shape with its head sharing (32
    query heads over 8 key/value heads, N = 4096, d = 128, causal) in the
    benchmark's launch configuration (head split on): the last key/value head
    (query heads 28..31) against the oracle, every element; then, over all
    heads, the split against the unsplit kernel: dQ bit for bit (the same
    query-tile kernel), dK and dV within one bf16 ulp of each element plus
    2^-16 of the tensor's largest magnitude (the split only changes the float32
    summation order, which moves a sum that cancels by a few float32 ulps of
    its terms)."""
    B, H, Hkv, N, d = 1, 32, 8, 4096, 128
    q, k, v, do = make_gqa_inputs(B, H, Hkv, N, d, seed=6, with_do=True)
    scale = 1 / math.sqrt(d)
    assert (fa.fa_bwd_kv_workspace_size(B, H, Hkv, N, N, d)
            > fa.fa_bwd_workspace_size(B, H, N, d))
    o, lse = _fwd(q, k, v, True, scale)
    got = _bwd(q, k, v, do, o, lse, True, scale, True)
    plain = _bwd(q, k, v, do, o, lse, True, scale, False)
    assert torch.equal(got[0], plain[0])
    for a, b in zip(got[1:], plain[1:]):
        a, b = a.float(), b.float()
        assert torch.isfinite(a).all()
        bound = 2.0 ** -7 * torch.maximum(a.abs(), b.abs()) + 2.0 ** -16 * b.abs().max()
        excess = ((a - b).abs() - bound).max().item()
        _say(f"   split vs unsplit: max diff {(a - b).abs().max().item():.3e}, "
             f"worst excess over the bound {excess:.3e}")
        assert excess <= 0
    ref = naive_bwd_gqa(_f64(q[:, 28:]), _f64(k[:, 7:]), _f64(v[:, 7:]), _f64(do[:, 28:]),
                        _s32(scale), True)
    tol = max(TOL, 2.0 ** -7 * max(float(np.max(np.abs(r))) for r in ref))
    errs = [float(np.max(np.abs(_f64(g) - r)))
            for g, r in zip((got[0][:, 28:], got[1][:, 7:], got[2][:, 7:]), ref)]
    _say(f"[llama8b gqa bwd] max|d dQ|={errs[0]:.3e} |d dK|={errs[1]:.3e} "
         f"|d dV|={errs[2]:.3e} (tol {tol:.3e})")
    assert max(errs) <= tol
