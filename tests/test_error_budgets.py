"""The backward tests' D-term budget (tests/budgets.py) checked on the CPU: it
must cover what the forward's bf16 rounding does to dQ and dK through
D = rowsum(dO * O).  Simulated here in float64: probabilities rounded to bf16
before the P V product, the output rounded to bf16, D formed from it, and the
gradients of the softmax-Jacobian form dS = P (dP - D) (exact in D, so first
order is exact) compared with the exact ones."""

import numpy as np
import pytest
import torch

from budgets import BF16_U, d_term_bounds, d_term_bounds_kv
from oracle import kv_head_of, naive_bwd, naive_bwd_kv, naive_probs, softmax_rows, visible_mask_kv


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def _grads_with_d(q, k, v, do, scale, causal, D):
    P = naive_probs(q, k, scale, causal)
    dP = do @ v.T
    dS = P * (dP - D[:, None])
    return scale * dS @ k, scale * dS.T @ q


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale,boost", [(0.125, 1.0), (0.125, 4.0), (0.5, 1.0), (-0.2, 1.0)])
def test_d_term_budget_covers_bf16_output(causal, scale, boost):
    rng = np.random.default_rng(7)
    N, d = 96, 32
    q, k, v, do = (_bf16(rng.standard_normal((N, d))) for _ in range(4))
    q[6::7] *= boost                       # the boosted rows of the GPT-2-medium workload
    P = naive_probs(q, k, scale, causal)
    O = P @ v
    o_hat = _bf16(_bf16(P) @ v)            # probabilities, then the output, in bf16
    D = np.sum(do * O, axis=1)
    D_hat = np.sum(do * o_hat, axis=1)
    dq, dk = _grads_with_d(q, k, v, do, scale, causal, D)
    dq_h, dk_h = _grads_with_d(q, k, v, do, scale, causal, D_hat)
    # the D form agrees with the oracle's softmax Jacobian
    ref = naive_bwd(q, k, v, do, scale, causal)
    assert np.max(np.abs(dq - ref[0])) < 1e-9 and np.max(np.abs(dk - ref[1])) < 1e-9
    bq, bk = d_term_bounds(q, k, v, do, scale, causal)
    assert np.all(np.abs(dq_h - dq) <= bq + 1e-12)
    assert np.all(np.abs(dk_h - dk) <= bk + 1e-12)
    # and it is not vacuous: the bound is within a small factor of the worst
    # simulated effect where that effect is largest
    if boost > 1:
        assert np.max(bk) < 64 * np.max(np.abs(dk_h - dk))


def test_d_term_budget_is_zero_without_scale():
    rng = np.random.default_rng(8)
    q, k, v, do = (rng.standard_normal((20, 8)) for _ in range(4))
    bq, bk = d_term_bounds(q, k, v, do, 0.0, True)
    assert not bq.any() and not bk.any()
    assert BF16_U == 2.0 ** -8


def test_kv_budget_equals_square_budget_on_square_heads():
    rng = np.random.default_rng(9)
    q, k, v, do = (rng.standard_normal((1, 2, 40, 16)) for _ in range(4))
    bq, bk = d_term_bounds_kv(q, k, v, do, 0.3, True)
    for h in range(2):
        rq, rk = d_term_bounds(q[0, h], k[0, h], v[0, h], do[0, h], 0.3, True)
        np.testing.assert_allclose(bq[0, h], rq, rtol=1e-12, atol=0)
        np.testing.assert_allclose(bk[0, h], rk, rtol=1e-12, atol=0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk,scale", [(24, 70, 0.3), (70, 24, -0.27), (33, 33, 0.5)])
def test_kv_budget_covers_bf16_output(causal, nq, nk, scale):
    """Grouped heads (4 query heads over 2 key/value heads) and different
    lengths: the same float64 simulation of the forward's bf16 probabilities
    and output entering D, against the bound."""
    rng = np.random.default_rng(10)
    B, H, Hkv, d = 1, 4, 2, 32
    q = _bf16(rng.standard_normal((B, H, nq, d)))
    do = _bf16(rng.standard_normal((B, H, nq, d)))
    k = _bf16(rng.standard_normal((B, Hkv, nk, d)))
    v = _bf16(rng.standard_normal((B, Hkv, nk, d)))
    mask = visible_mask_kv(nq, nk, causal)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dq_h = np.zeros(q.shape)
    dk_h = np.zeros(k.shape)
    for h in range(H):
        g = kv_head_of(h, H, Hkv)
        P = softmax_rows(np.where(mask, scale * (q[0, h] @ k[0, g].T), -np.inf))
        O = P @ v[0, g]
        o_hat = _bf16(_bf16(P) @ v[0, g])
        dP = do[0, h] @ v[0, g].T
        for D, gq, gk in ((np.sum(do[0, h] * O, axis=1), dq, dk),
                          (np.sum(do[0, h] * o_hat, axis=1), dq_h, dk_h)):
            dS = P * (dP - D[:, None])
            gq[0, h] = scale * dS @ k[0, g]
            gk[0, g] += scale * dS.T @ q[0, h]
    ref = naive_bwd_kv(q, k, v, do, scale, causal)
    assert np.max(np.abs(dq - ref[0])) < 1e-9 and np.max(np.abs(dk - ref[1])) < 1e-9
    bq, bk = d_term_bounds_kv(q, k, v, do, scale, causal)
    assert np.all(np.abs(dq_h - dq) <= bq + 1e-12)
    assert np.all(np.abs(dk_h - dk) <= bk + 1e-12)
