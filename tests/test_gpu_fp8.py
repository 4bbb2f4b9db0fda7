"""GPU parity of the fp8 forward (fa_fwd_fp8: OCP e4m3 inputs, d = 128)
against the float64 oracle evaluated on the dequantised inputs.

Error budget (this path's own; the bf16 bar of 2e-2 does not apply):
the kernel rounds each probability p to e4m3 before the P V product.  An
e4m3 normal carries 3 mantissa bits (relative rounding error <= 2^-4); below
2^-6 the spacing is 2^-9 (absolute error <= 2^-10, and never more than p
itself, which rounding to zero loses).  The kernel's probabilities are
scaled so the largest of a row is >= 1 (its sum l >= 1), so in probability
units the error of each p_ij is at most 2^-4 P_ij + min(P_ij, 2^-10).  With
the unrounded fp32 sum as the denominator, each output element therefore
satisfies
    |O_id - ref_id| <= sum_j (2^-4 P_ij + min(P_ij, 2^-10)) |v_jd|
                       + 2^-8 |ref_id| + 1e-4
(the second term is the bf16 rounding of O, the last fp32 accumulation).
The bound is evaluated from the oracle's P and checked element by element.
lse is formed from the unrounded probabilities in fp32: within 1e-3 as for
the bf16 path, except where the scores themselves are large: the fp32
accumulation of a d-term dot product is only good to the classical bound
d * 2^-24 * sum_c |scale q_ic k_jc|, which passes 1e-3 for the stress case
with scale 2.0 (scores near 100).  The lse bar is the larger of the two.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_10_amd as fa
from oracle import e4m3_decode, naive_fwd_fp8, naive_probs
from workloads import make_fp8_inputs

pytestmark = pytest.mark.gpu

TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")
    fa.load_library()


def _say(*a):
    print(*a, flush=True)


def _run(q8, k8, v8, sq, sk, sv, causal, scale):
    B, H, N, d = q8.shape
    qd, kd, vd = (t.cuda() for t in (q8, k8, v8))
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd_fp8(qd, kd, vd, o, lse, sq, sk, sv, causal, scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(q8, k8, v8, sq, sk, sv, causal, scale):
    o, lse = _run(q8, k8, v8, sq, sk, sv, causal, scale)
    qn, kn, vn = (x.numpy() for x in (q8, k8, v8))
    ro, rl = naive_fwd_fp8(qn, kn, vn, sq, sk, sv, scale, causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    worst = 0.0
    for b in range(q8.shape[0]):
        for h in range(q8.shape[1]):
            p = naive_probs(sq * e4m3_decode(qn[b, h]), sk * e4m3_decode(kn[b, h]), scale,
                            causal)
            av = np.abs(sv * e4m3_decode(vn[b, h]))
            bound = (2.0 ** -4 * p + np.minimum(p, 2.0 ** -10)) @ av
            bound += 2.0 ** -8 * np.abs(ro[b, h]) + 1e-4
            err = np.abs(o[b, h] - ro[b, h])
            worst = max(worst, float(np.max(err / bound)))
            assert np.all(err <= bound), (b, h, float(np.max(err - bound)))
    el = float(np.max(np.abs(lse - rl)))
    tol_lse = TOL_LSE
    for b in range(q8.shape[0]):
        for h in range(q8.shape[1]):
            aq = np.abs(sq * e4m3_decode(qn[b, h]))
            ak = np.abs(sk * e4m3_decode(kn[b, h]))
            dot = abs(scale) * float(np.max(aq @ ak.T)) if aq.size and ak.size else 0.0
            tol_lse = max(tol_lse, q8.shape[-1] * 2.0 ** -24 * dot)
    _say(f"   max err / bound = {worst:.3f}; max|O err|={np.max(np.abs(o - ro)):.3e};"
         f" max|dlse|={el:.3e} (bar {tol_lse:.2e})")
    assert el <= tol_lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 127, 129, 300, 1000])
def test_fp8_forward(N, causal):
    _say(f"[fp8 fwd] N={N} causal={causal}")
    q8, k8, v8, sq, sk, sv = make_fp8_inputs(2, 2, N, 128, seed=2000 + N)
    _check(q8, k8, v8, sq, sk, sv, causal, 1 / math.sqrt(128))


def test_fp8_forward_negative_scale_and_peaked_rows():
    """A negative score factor (sign flip of the e4m3 query bytes) and a large
    one (near one-hot rows, the largest per-element rounding)."""
    q8, k8, v8, sq, sk, sv = make_fp8_inputs(1, 2, 200, 128, seed=2100)
    _check(q8, k8, v8, sq, sk, sv, True, -0.2)
    _check(q8, k8, v8, sq, sk, sv, False, 2.0)


def test_fp8_llama8b_shape_sampled_heads():
    """[1, 32, 4096, 128] causal (the Llama-3.1-8B attention shape): heads 0
    and 31 checked in full against the bound."""
    B, H, N, d = 1, 32, 4096, 128
    q8, k8, v8, sq, sk, sv = make_fp8_inputs(B, H, N, d, seed=2200)
    o, lse = _run(q8, k8, v8, sq, sk, sv, True, 1 / math.sqrt(d))
    for h in (0, 31):
        qn, kn, vn = (x[0, h].numpy() for x in (q8, k8, v8))
        ro, rl = naive_fwd_fp8(qn, kn, vn, sq, sk, sv, 1 / math.sqrt(d), True)
        p = naive_probs(sq * e4m3_decode(qn), sk * e4m3_decode(kn), 1 / math.sqrt(d), True)
        bound = (2.0 ** -4 * p + np.minimum(p, 2.0 ** -10)) @ np.abs(sv * e4m3_decode(vn))
        bound += 2.0 ** -8 * np.abs(ro) + 1e-4
        err = np.abs(o[0, h] - ro)
        _say(f"[fp8 4096] head {h}: max err / bound = {np.max(err / bound):.3f},"
             f" max|dlse| = {np.max(np.abs(lse[0, h] - rl)):.3e}")
        assert np.all(err <= bound)
        assert np.max(np.abs(lse[0, h] - rl)) <= TOL_LSE
