"""GPU tests of the launch contract: every entry point enqueues its kernels on
the stream it is given (no allocation, no memset, no synchronisation inside),
so the calls run on any stream and can be recorded into a HIP graph.

* side stream: the forward and the backward issued on a created stream
  (default priority) give the same O, lse, dK and dV as on the default stream,
  bit for bit, and dQ within the stated tolerance of the oracle (at d = 64 dQ
  is a sum of float atomics, whose order is not fixed);
* graph: the four calls of a training step (``fa_fwd`` ->
  ``fa_bwd_preprocess`` -> ``fa_bwd_main`` -> ``fa_bwd_finalize``) captured
  once in a ``torch.cuda.CUDAGraph`` and replayed three times, the outputs
  NaN-filled and the workspace set to 0xFF by eager work between replays
  (so every replay must rewrite every output and re-zero its own dQ
  accumulator); each replay against the eager run, bit for bit where the
  kernels are deterministic, and every gradient against the oracle;
* graph: one decoding token through ``fa_fwd_kv``'s split-key path (its
  workspace written by one kernel and merged by the next) replayed the same
  way.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_10_amd as fa
from oracle import naive_bwd, naive_fwd
from workloads import make_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2
TOL_LSE = 1e-3


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


def _buffers(q):
    B, H, N, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    ws = torch.full((fa.fa_bwd_workspace_size(B, H, N, d),), 0xFF, dtype=torch.uint8,
                    device=q.device)
    return o, lse, dq, dk, dv, ws


def _oracle_check(q, k, v, do, scale, causal, o, lse, dq, dk, dv, tag):
    qf, kf, vf, dof = (_f64(t) for t in (q, k, v, do))
    ro, rl = naive_fwd(qf, kf, vf, _s32(scale), causal)
    rq, rk, rv = naive_bwd(qf, kf, vf, dof, _s32(scale), causal)
    errs = [float(np.abs(_f64(g) - r).max()) for g, r in ((o, ro), (dq, rq), (dk, rk), (dv, rv))]
    el = float(np.abs(_f64(lse) - rl).max())
    _say(f"   {tag}: O {errs[0]:.3e} lse {el:.3e} dQ {errs[1]:.3e} dK {errs[2]:.3e} "
         f"dV {errs[3]:.3e}")
    assert max(errs) <= TOL and el <= TOL_LSE


@pytest.mark.parametrize("d", [64, 128])
def test_side_stream_matches_default_stream(d):
    B, H, N, causal = 2, 4, 300, True
    scale = 1.0 / math.sqrt(d)
    _say(f"[side stream] B={B} H={H} N={N} d={d} causal")
    q, k, v, do = (t.cuda() for t in make_inputs(B, H, N, d, torch.bfloat16, seed=310 + d,
                                                   with_do=True))
    ref = _buffers(q)
    fa.fa_fwd(q, k, v, ref[0], ref[1], causal, scale)
    fa.fa_bwd(q, k, v, ref[0], do, ref[1], ref[2], ref[3], ref[4], ref[5], causal, scale)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = _buffers(q)
        fa.fa_fwd(q, k, v, got[0], got[1], causal, scale, stream=side)
        fa.fa_bwd(q, k, v, got[0], do, got[1], got[2], got[3], got[4], got[5], causal, scale,
                  stream=side)
    side.synchronize()
    torch.cuda.current_stream().wait_stream(side)
    for name, a, b in (("O", got[0], ref[0]), ("lse", got[1], ref[1]), ("dK", got[3], ref[3]),
                       ("dV", got[4], ref[4])):
        assert torch.equal(a, b), f"{name} differs between the side and the default stream"
    if d != 64:
        assert torch.equal(got[2], ref[2]), "dQ differs between the side and the default stream"
    _oracle_check(q, k, v, do, scale, causal, got[0], got[1], got[2], got[3], got[4], "side")


@pytest.mark.parametrize("d", [64, 128])
def test_graph_replays_of_the_staged_step(d):
    B, H, N, causal = 1, 4, 1024, True
    scale = 1.0 / math.sqrt(d)
    _say(f"[graph] B={B} H={H} N={N} d={d} causal")
    q, k, v, do = (t.cuda() for t in make_inputs(B, H, N, d, torch.bfloat16, seed=320 + d,
                                                   with_do=True))
    o, lse, dq, dk, dv, ws = _buffers(q)

    def step():
        fa.fa_fwd(q, k, v, o, lse, causal, scale)
        fa.fa_bwd_preprocess(o, do, lse, ws)
        fa.fa_bwd_main(q, k, v, do, dk, dv, ws, causal, scale)
        fa.fa_bwd_finalize(dq, ws, q, k, v, do, causal, scale)

    step()   # eager
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o, lse, dq, dk, dv)]
    _oracle_check(q, k, v, do, scale, causal, *eager, "eager")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "lse", "dQ", "dK", "dV"), (o, lse, dq, dk, dv), eager):
            if name == "dQ" and d == 64:
                continue
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager run"
        _oracle_check(q, k, v, do, scale, causal, o, lse, dq, dk, dv, f"replay {rep}")


def test_graph_replays_of_split_key_decode():
    """One decoding token of 32 query heads over 8 key/value heads (d = 128,
    4096 cached keys, batch 2) through ``fa_fwd_kv`` -- the split-key kernel
    writing the caller's workspace and the merge reading it -- captured once
    and replayed three times with NaN-filled outputs and a 0xFF workspace
    between replays: each replay bit-identical to the eager run, and against
    the oracle."""
    from oracle import naive_fwd_kv
    from workloads import make_gqa_inputs
    B, H, Hkv, Nk, d = 2, 32, 8, 4096, 128
    scale = 1.0 / math.sqrt(d)
    _say(f"[graph decode] B={B} H={H} Hkv={Hkv} Nk={Nk} d={d}")
    q = make_gqa_inputs(B, H, Hkv, 1, d, seed=330, with_do=False)[0].cuda()
    _, k, v = (t.cuda() for t in make_gqa_inputs(B, H, Hkv, Nk, d, seed=331))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, 1), float("nan"), dtype=torch.float32, device="cuda")
    nb = fa.fa_fwd_kv_workspace_size(B, H, Hkv, 1, Nk, d)
    assert nb > 0, "the decode shape should take the split-key path"
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    fa.fa_fwd_kv(q, k, v, o, lse, ws, True, scale)
    torch.cuda.synchronize()
    eager = (o.clone(), lse.clone())
    ro, rl = naive_fwd_kv(_f64(q), _f64(k), _f64(v), _s32(scale), True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_fwd_kv(q, k, v, o, lse, ws, True, scale)
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager[0]) and torch.equal(lse, eager[1]), f"replay {rep}"
        eo = float(np.abs(_f64(o) - ro).max())
        el = float(np.abs(_f64(lse) - rl).max())
        _say(f"   replay {rep}: O {eo:.3e} lse {el:.3e}")
        assert eo <= TOL and el <= TOL_LSE
