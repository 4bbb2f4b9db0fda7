"""GPU parity on seeded random problem shapes: the combinations the fixed
cases do not enumerate.

Forty configurations are drawn once from a fixed seed: head dimension 64, 128
or 256; batch 1-2; 1-2 key/value heads with 1, 2 or 4 query heads each; query
and key lengths 1-400, equal in half of the cases; causal or not; a scale of
either sign.  Each runs the forward through the entry point its shape calls
for (``fa_fwd``, ``fa_fwd_gqa`` or ``fa_fwd_kv``), NaN-prefilled outputs,
against ``naive_fwd_kv``; every other one also runs the backward (``fa_bwd``,
``fa_bwd_gqa`` or ``fa_bwd_kv``) against ``naive_bwd_kv``; twelve more run
fp32 inputs through ``fa_fwd_f32`` against ``naive_fwd``.  Tolerances: 2e-2
on O and 1e-3 on the lse of rows that see a key (rows that see none must be
O = 0, lse = -inf); the gradients within max(2e-2, 2^-7 max|ref|), one bf16
ulp of the largest reference magnitude -- the bar the grouped-head and
different-length backward tests use, since gradients summed over a group's
query heads can pass O(1) -- plus, for dQ and dK, each element's first-order
budget of the forward's bf16 output entering D = rowsum(dO * O)
(``budgets.d_term_bounds_kv``; at scales well above 1/sqrt(d) the scores are
large and that term is what separates the GPU from the float64 oracle).
"""


import numpy as np
import pytest
import torch

import exact_tiled_attention_10_amd as fa
from budgets import d_term_bounds_kv
from oracle import naive_bwd_kv, naive_fwd_kv, visible_mask_kv
from workloads import make_gqa_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2
TOL_LSE = 1e-3


def _draw(count=40, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        d = int(rng.choice([64, 128, 256], p=[0.4, 0.4, 0.2]))
        B = int(rng.integers(1, 3))
        Hkv = int(rng.integers(1, 3))
        H = Hkv * int(rng.choice([1, 2, 4]))
        nq = int(rng.integers(1, 401))
        nk = nq if rng.random() < 0.5 else int(rng.integers(1, 401))
        causal = bool(rng.random() < 0.5)
        scale = float(rng.uniform(0.05, 0.3)) * (-1.0 if rng.random() < 0.15 else 1.0)
        out.append((i, d, B, H, Hkv, nq, nk, causal, round(scale, 4), i % 2 == 0))
    return out


CASES = _draw()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")
    fa.load_library()


def _say(*a):
    print(*a, flush=True)


def _s32(x):
    return float(np.float32(x))


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", CASES, ids=[f"c{c[0]}" for c in CASES])
def test_random_shape(case):
    i, d, B, H, Hkv, nq, nk, causal, scale, with_bwd = case
    _say(f"[random {i}] d={d} B={B} H={H} Hkv={Hkv} Nq={nq} Nk={nk} causal={causal} "
         f"scale={scale} bwd={with_bwd}")
    q, _, _, do = make_gqa_inputs(B, H, Hkv, nq, d, seed=1000 + i, with_do=True)
    _, k, v = make_gqa_inputs(B, H, Hkv, nk, d, seed=2000 + i)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, nq), float("nan"), dtype=torch.float32, device="cuda")
    if nq == nk and H == Hkv:
        kind = "plain"
        fa.fa_fwd(qd, kd, vd, o, lse, causal, scale)
    elif nq == nk:
        kind = "gqa"
        fa.fa_fwd_gqa(qd, kd, vd, o, lse, causal, scale)
    else:
        kind = "kv"
        nb = fa.fa_fwd_kv_workspace_size(B, H, Hkv, nq, nk, d)
        ws = torch.empty((nb,), dtype=torch.uint8, device="cuda") if nb else None
        fa.fa_fwd_kv(qd, kd, vd, o, lse, ws, causal, scale)
    torch.cuda.synchronize()
    ro, rl = naive_fwd_kv(_f64(q), _f64(k), _f64(v), _s32(scale), causal)
    go, gl = _f64(o), _f64(lse)
    live = visible_mask_kv(nq, nk, causal).any(axis=1)
    assert np.all(np.isfinite(go))
    assert np.all(go[..., ~live, :] == 0) and np.all(gl[..., ~live] == -np.inf)
    eo = float(np.max(np.abs(go - ro)))
    el = float(np.max(np.abs(gl[..., live] - rl[..., live]))) if live.any() else 0.0
    _say(f"   {kind}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL and el <= TOL_LSE
    if not with_bwd:
        return
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    if kind == "plain":
        ws = torch.empty((fa.fa_bwd_workspace_size(B, H, nq, d),), dtype=torch.uint8,
                         device="cuda")
        fa.fa_bwd(qd, kd, vd, o, dod, lse, dq, dk, dv, ws, causal, scale)
    else:
        ws = torch.empty((max(1, fa.fa_bwd_kv_workspace_size(B, H, Hkv, nq, nk, d)),),
                         dtype=torch.uint8, device="cuda")
        if kind == "gqa":
            fa.fa_bwd_gqa(qd, kd, vd, o, dod, lse, dq, dk, dv, ws, causal, scale)
        else:
            fa.fa_bwd_kv(qd, kd, vd, o, dod, lse, dq, dk, dv, ws, causal, scale)
    torch.cuda.synchronize()
    ref = naive_bwd_kv(_f64(q), _f64(k), _f64(v), _f64(do), _s32(scale), causal)
    tol = max(TOL, 2.0 ** -7 * max(float(np.max(np.abs(r))) if r.size else 0.0 for r in ref))
    errs = [float(np.max(np.abs(_f64(g) - r))) if r.size else 0.0
            for g, r in zip((dq, dk, dv), ref)]
    _say(f"   bwd: max|d dQ|={errs[0]:.3e} |d dK|={errs[1]:.3e} |d dV|={errs[2]:.3e} "
         f"(tol {tol:.3e})")
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
    bq, bk = d_term_bounds_kv(_f64(q), _f64(k), _f64(v), _f64(do), _s32(scale), causal)
    for g, r, bnd in zip((dq, dk, dv), ref, (bq, bk, 0.0)):
        assert np.max(np.abs(_f64(g) - r) - (tol + bnd)) <= 0.0


def _draw_f32(count=12, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 5))
        n = int(rng.integers(1, 401))
        causal = bool(rng.random() < 0.5)
        scale = float(rng.uniform(0.05, 0.3)) * (-1.0 if rng.random() < 0.15 else 1.0)
        out.append((i, d, B, H, n, causal, round(scale, 4)))
    return out


CASES_F32 = _draw_f32()


@pytest.mark.parametrize("case", CASES_F32, ids=[f"f{c[0]}" for c in CASES_F32])
def test_random_shape_fp32(case):
    """fp32 inputs (``fa_fwd_f32``) on twelve seeded random shapes: O within
    1e-5, lse within 1e-3."""
    from oracle import naive_fwd
    from workloads import make_inputs
    i, d, B, H, n, causal, scale = case
    _say(f"[random fp32 {i}] d={d} B={B} H={H} N={n} causal={causal} scale={scale}")
    q, k, v = make_inputs(B, H, n, d, torch.float32, seed=3000 + i)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, n), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd_f32(qd, kd, vd, o, lse, causal, scale)
    torch.cuda.synchronize()
    ro, rl = naive_fwd(_f64(q), _f64(k), _f64(v), _s32(scale), causal)
    eo = float(np.max(np.abs(_f64(o) - ro)))
    el = float(np.max(np.abs(_f64(lse) - rl)))
    _say(f"   max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= 1e-5 and el <= TOL_LSE
