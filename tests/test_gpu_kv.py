"""GPU parity of the forward with different query and key lengths
(fa_fwd_kv: cross-attention and decode against a key/value cache) against the
float64 oracle ``naive_fwd_kv``.

Causal masking aligns the queries with the END of the keys: query i sees key
j iff j <= i + (Nk - Nq).  A query that sees no key has O = 0 and lse = -inf
exactly.  Small query counts (decode) take the split-key path: ranges of keys
on separate workgroups, merged by their log-sum-exps.  Tolerances as for the
plain forward: O within 2e-2 (bf16 output), lse within 1e-3.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_10_amd as fa
from oracle import naive_fwd_kv, visible_mask_kv
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


def _inputs(B, H, Hkv, Nq, Nk, d, seed):
    """q from a [B, H, Nq, d] draw, k and v from a [B, Hkv, Nk, d] draw."""
    q, _, _ = make_gqa_inputs(B, H, Hkv, Nq, d, seed=seed)
    _, k, v = make_gqa_inputs(B, H, Hkv, Nk, d, seed=seed + 7919)
    return q, k, v


def _run(q, k, v, causal, scale, use_ws=True):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    nb = fa.fa_fwd_kv_workspace_size(B, H, k.shape[1], Nq, Nk, d)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda") if (nb and use_ws) else None
    if nb and not use_ws:
        pytest.skip("this shape needs a workspace")
    fa.fa_fwd_kv(qd, kd, vd, o, lse, ws, causal, scale)
    torch.cuda.synchronize()
    return o, lse, nb


def _check(q, k, v, causal, scale, o, lse):
    ro, rl = naive_fwd_kv(_f64(q), _f64(k), _f64(v), _s32(scale), causal)
    go, gl = _f64(o), _f64(lse)
    live = visible_mask_kv(q.shape[2], k.shape[2], causal).any(axis=1)
    assert np.all(go[..., ~live, :] == 0) and np.all(gl[..., ~live] == -np.inf)
    eo = float(np.max(np.abs(go - ro))) if go.size else 0.0
    el = float(np.max(np.abs(gl[..., live] - rl[..., live]))) if live.any() else 0.0
    _say(f"   max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert np.all(np.isfinite(go))
    assert eo <= TOL and el <= TOL_LSE


SHAPES = [(1, 1), (1, 63), (1, 4096), (5, 700), (64, 97), (300, 1000), (257, 4096),
          (1000, 300), (129, 1)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", SHAPES)
def test_kv_forward(nq, nk, causal, d):
    _say(f"[kv fwd] Nq={nq} Nk={nk} d={d} causal={causal}")
    q, k, v = _inputs(2, 2, 2, nq, nk, d, seed=500 + nq + nk)
    scale = 1 / math.sqrt(d)
    o, lse, nb = _run(q, k, v, causal, scale)
    _say(f"   workspace {nb} bytes")
    _check(q, k, v, causal, scale, o, lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv,nq,nk", [(8, 2, 1, 2048), (8, 1, 3, 777), (6, 3, 200, 500)])
def test_kv_forward_gqa(H, Hkv, nq, nk, causal):
    _say(f"[kv fwd gqa] H={H} Hkv={Hkv} Nq={nq} Nk={nk} causal={causal}")
    q, k, v = _inputs(1, H, Hkv, nq, nk, 128, seed=600 + nq)
    o, lse, _ = _run(q, k, v, causal, 1 / math.sqrt(128))
    _check(q, k, v, causal, 1 / math.sqrt(128), o, lse)


def test_kv_no_keys():
    """Nk = 0: every row is empty (O = 0, lse = -inf)."""
    q, k, v = _inputs(1, 2, 2, 5, 0, 64, seed=1)
    o, lse, _ = _run(q, k, v, True, 0.125)
    assert torch.all(o == 0) and torch.all(lse == float("-inf"))


def test_kv_equal_lengths_match_fa_fwd():
    """Nq = Nk with enough query tiles to fill the GPU (no key split) takes
    the same kernel path as fa_fwd: identical bits."""
    q, k, v = _inputs(1, 64, 64, 1024, 1024, 128, seed=2)
    o, lse, nb = _run(q, k, v, True, 1 / math.sqrt(128))
    assert nb == 0
    o2, lse2 = fa.forward(q.cuda(), k.cuda(), v.cuda(), True, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_kv_split_and_unsplit_agree():
    """A shape the library splits (few query tiles) against the same rows
    computed in a launch with enough heads that it does not split."""
    q, k, v = _inputs(1, 4, 4, 600, 600, 128, seed=2)
    o, lse, nb = _run(q, k, v, True, 1 / math.sqrt(128))
    assert nb > 0
    _check(q, k, v, True, 1 / math.sqrt(128), o, lse)


def test_llama8b_decode_against_long_cache():
    """One new token per sequence against a 32k-token cache in Llama-3.1-8B's
    attention shape (32 query heads over 8 key/value heads, d = 128): the
    split-key path, every output against the oracle."""
    B, H, Hkv, Nq, Nk, d = 2, 32, 8, 1, 32768, 128
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, seed=3)
    o, lse, nb = _run(q, k, v, True, 1 / math.sqrt(d))
    _say(f"[llama8b decode] workspace {nb} bytes")
    assert nb > 0
    _check(q, k, v, True, 1 / math.sqrt(d), o, lse)


# --- backward (fa_bwd_kv) ------------------------------------------------------

def _bwd(q, k, v, do, causal, scale):
    o, lse, _ = _run(q, k, v, causal, scale)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    ws = torch.full((max(1, fa.fa_bwd_kv_workspace_size(B, H, Hkv, Nq, Nk, d)),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    fa.fa_bwd_kv(qd, kd, vd, o, dod, lse, dq, dk, dv, ws, causal, scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check_grads(q, k, v, do, causal, scale, got):
    from oracle import naive_bwd_kv
    ref = naive_bwd_kv(_f64(q), _f64(k), _f64(v), _f64(do), _s32(scale), causal)
    # one bf16 ulp of the largest reference magnitude, never below 2e-2 (the
    # summed gradients of shared key/value heads can pass O(1))
    tol = max(TOL, 2.0 ** -7 * max(float(np.max(np.abs(r))) if r.size else 0.0 for r in ref))
    errs = [float(np.max(np.abs(_f64(g) - r))) if r.size else 0.0 for g, r in zip(got, ref)]
    _say(f"   max|d dQ|={errs[0]:.3e} |d dK|={errs[1]:.3e} |d dV|={errs[2]:.3e} (tol {tol:.3e})")
    for g in got:
        assert torch.isfinite(g).all()
    assert max(errs) <= tol


BWD_SHAPES = [(1, 300), (5, 700), (64, 97), (300, 1000), (1000, 300), (129, 1), (257, 600)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", BWD_SHAPES)
def test_kv_backward(nq, nk, causal, d):
    _say(f"[kv bwd] Nq={nq} Nk={nk} d={d} causal={causal}")
    q, k, v = _inputs(2, 2, 2, nq, nk, d, seed=700 + nq + nk)
    do = make_gqa_inputs(2, 2, 2, nq, d, seed=900 + nq, with_do=True)[3]
    got = _bwd(q, k, v, do, causal, 1 / math.sqrt(d))
    _check_grads(q, k, v, do, causal, 1 / math.sqrt(d), got)


@pytest.mark.parametrize("causal", [False, True])
def test_kv_backward_gqa(causal):
    _say(f"[kv bwd gqa] causal={causal}")
    q, k, v = _inputs(1, 8, 2, 200, 520, 64, seed=11)
    do = make_gqa_inputs(1, 8, 2, 200, 64, seed=12, with_do=True)[3]
    got = _bwd(q, k, v, do, causal, 0.125)
    _check_grads(q, k, v, do, causal, 0.125, got)


def test_kv_backward_no_queries_zeroes_key_gradients():
    k, v = _inputs(1, 2, 2, 3, 70, 64, seed=13)[1:]
    kd, vd = k.cuda(), v.cuda()
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    st = fa.load_library().fa_bwd_kv(None, kd.data_ptr(), vd.data_ptr(), None, None, None, None,
                                     dk.data_ptr(), dv.data_ptr(), None, 0, 1, 2, 2, 0, 70, 64,
                                     1, 0.125, None)
    torch.cuda.synchronize()
    assert st == fa.FA_OK
    assert torch.all(dk == 0) and torch.all(dv == 0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv,nq,nk", [(8, 2, 8, 5000), (8, 1, 4, 3001), (8, 1, 5, 3001),
                                         (4, 4, 32, 900), (2, 1, 1, 1)])
def test_kv_decode_packed_rows(H, Hkv, nq, nk, causal, d):
    """The packed-rows decode kernel: group * Nq rows of one key/value head in
    one wave (exactly 32 rows: 8 x 4; one past: 8 x 5 takes the tile kernel),
    with key splits and bottom-right causal positions."""
    _say(f"[kv decode] H={H} Hkv={Hkv} Nq={nq} Nk={nk} d={d} causal={causal}")
    q, k, v = _inputs(2, H, Hkv, nq, nk, d, seed=3000 + nq + nk)
    o, lse, nb = _run(q, k, v, causal, 1 / math.sqrt(d))
    _say(f"   workspace {nb} bytes")
    _check(q, k, v, causal, 1 / math.sqrt(d), o, lse)
