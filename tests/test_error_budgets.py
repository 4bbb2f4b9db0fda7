"""The backward tests' D-term budget (tests/budgets.py) checked on the CPU: it
must cover what the forward's bf16 rounding does to dQ and dK through
D = rowsum(dO * O).  Simulated here in float64: probabilities rounded to bf16
before the P V product, the output rounded to bf16, D formed from it, and the
gradients of the softmax-Jacobian form dS = P (dP - D) (exact in D, so first
order is exact) compared with the exact ones."""

import numpy as np
import pytest
import torch

from budgets import BF16_U, d_term_bounds
from oracle import naive_bwd, naive_probs


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
