"""Pins for the float64 CPU oracle (no GPU).

The oracle is checked against things other than itself: the worked examples
the source pages print (fixtures under tests/golden/, each carrying its
citation), the tile / FLOP / traffic tables they print, closed forms, invariants
of the definition, a library routine in float64, central finite differences,
and agreement between the two independent CPU implementations.  A planted
mistake (no rescale) shows the worked-example pin catches the classic bug.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (causal_tile_counts, naive_bwd, naive_fwd, naive_probs,
                    online_normaliser, softmax_rows, tiled_bwd, tiled_fwd)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _matches_printed(value, printed, decimals):
    """True when ``value`` rounds to the printed figure (half-unit slack)."""
    value = np.asarray(value, dtype=np.float64)
    printed = np.asarray(printed, dtype=np.float64)
    return bool(np.all(np.abs(value - printed) <= 0.5 * 10.0 ** -decimals + 1e-12))


# ---------------------------------------------------------------------------
# worked examples
# ---------------------------------------------------------------------------

def test_first_principles_three_by_three():
    g = _golden("first_principles_3x3.json")
    q, k, v = (np.array(g[x], dtype=np.float64) for x in ("Q", "K", "V"))
    # S: scores with scale 1 are exact small integers; recovered from the
    # probabilities' logs up to the row constant, then checked against P.
    p = naive_probs(q, k, g["scale"])
    assert _matches_printed(p, g["P"], g["P_decimals"])
    o, lse = naive_fwd(q, k, v, g["scale"])
    assert _matches_printed(o, g["O"], g["O_decimals"])
    # the printed S reproduces the oracle's probabilities exactly
    s = np.array(g["S"], dtype=np.float64)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    np.testing.assert_allclose(p, e / e.sum(axis=1, keepdims=True), rtol=0,
                               atol=1e-15)
    # saved statistic: shift invariance makes r of [101,100,102] the same as
    # that of row 1 [1,0,2]; lse_1 = 2 + log r.
    r = math.exp(lse[0] - 2.0)
    assert _matches_printed(r, g["shifted_row_final_r"], g["r_decimals"])
    # resurrection from the saved statistics: P_12 = exp(S_12 - L_1)
    j = g["resurrected_index"]
    assert _matches_printed(math.exp(s[0, j] - lse[0]), g["resurrected_weight"], 3)
    # the shifted row streamed one element at a time ends at m=102, r=1.5032
    m, l, _ = online_normaliser(g["shifted_row"], 1)
    assert m == g["shifted_row_final_m"]
    assert _matches_printed(l, g["shifted_row_final_r"], g["r_decimals"])
    # the tiled variant lands on the same numbers at every block shape
    for bq in (1, 2, 3):
        for bk in (1, 2, 3):
            ot, lt, _ = tiled_fwd(q, k, v, g["scale"], block_q=bq, block_k=bk)
            np.testing.assert_allclose(ot[0, 0], o, rtol=0, atol=1e-15)
            np.testing.assert_allclose(lt[0, 0], lse, rtol=0, atol=1e-15)


def test_first_principles_softmax_rows():
    g = _golden("first_principles_3x3.json")
    for ex in g["softmax_examples"]:
        assert _matches_printed(softmax_rows(np.array([ex["row"]], float))[0],
                                ex["softmax"], 3)
    # shift invariance: [101,100,102] has row 1's weights
    sh = softmax_rows(np.array([g["shifted_row"]], float))[0]
    assert _matches_printed(sh, g["P"][0], 3)


def test_refresh3_rebase_stream():
    g = _golden("refresh3_rebase_stream.json")
    m, l, trace = online_normaliser(g["logits"], g["block"])
    assert len(trace) == len(g["blocks"])
    for got, want in zip(trace, g["blocks"]):
        for key, val in want.items():
            assert _matches_printed(got[key], val, g["decimals"]), (key, got, want)
    # the streamed sum equals the one-shot sum of exp(x - max)
    x = np.array(g["logits"])
    one_shot = float(np.sum(np.exp(x - x.max())))
    assert _matches_printed(one_shot, g["one_shot_sum"], g["decimals"])
    assert abs(l - one_shot) < 1e-15


def test_from_scratch_four_by_two():
    g = _golden("from_scratch_4x2.json")
    q, k, v = (np.array(g[x], dtype=np.float64) for x in ("Q", "K", "V"))
    row, dec = g["row"], g["decimals"]
    trace = []
    o, lse, _ = tiled_fwd(q, k, v, g["scale"], block_q=4, block_k=g["block"],
                          trace=trace)
    assert [t["k0"] for t in trace] == [0, 2]
    s1, s2 = trace
    assert s1["m"][0, 0, row, 0] == g["after_block_1"]["m"]
    assert _matches_printed(s1["l"][0, 0, row, 0], g["after_block_1"]["l"], dec)
    assert _matches_printed(s1["acc"][0, 0, row], g["after_block_1"]["acc"], dec)
    assert s2["m"][0, 0, row, 0] == g["after_block_2"]["m"]
    corr = math.exp(g["after_block_1"]["m"] - g["after_block_2"]["m"])
    assert _matches_printed(corr, g["after_block_2"]["correction"], dec)
    assert _matches_printed(s2["l"][0, 0, row, 0], g["after_block_2"]["l"], dec)
    assert _matches_printed(s2["acc"][0, 0, row], g["after_block_2"]["acc"], dec)
    assert _matches_printed(o[0, 0, row], g["O"], dec)
    # the plain definition gives the same row
    on, _ = naive_fwd(q, k, v, g["scale"])
    assert _matches_printed(on[row], g["O"], dec)
    # scores of that row are the printed ones
    np.testing.assert_array_equal(q[row] @ k.T, g["scores"])


def test_planted_no_rescale_is_caught():
    """The classic bug (history not rebased when the max moves) reproduces the
    page's wrong answer, and the worked-example pin rejects it."""
    g = _golden("from_scratch_4x2.json")
    q, k, v = (np.array(g[x], dtype=np.float64) for x in ("Q", "K", "V"))
    row = g["row"]
    bad, _, _ = tiled_fwd(q, k, v, g["scale"], block_q=4, block_k=g["block"],
                          _no_rescale=True)
    assert _matches_printed(bad[0, 0, row], g["no_rescale_O"],
                            g["no_rescale_decimals"])
    assert not _matches_printed(bad[0, 0, row], g["O"], g["decimals"])


# ---------------------------------------------------------------------------
# printed tables: causal tile counts, FLOPs, traffic
# ---------------------------------------------------------------------------

def test_refresh3_causal_tile_counts():
    g = _golden("refresh3_causal_tiles.json")
    n = g["n"]
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, n, 2))
    for r in g["rows"]:
        b = r["block"]
        _, _, c = tiled_fwd(q, q, q, 1.0, causal=True, block_q=b, block_k=b)
        assert c["tiles_computed"] == r["computed"]
        assert c["blocks_skipped"] == r["skipped"]
        assert causal_tile_counts(n, b) == (r["computed"], r["skipped"])
        frac = c["blocks_skipped"] / (c["blocks_skipped"] + c["tiles_computed"])
        assert round(100 * frac) == r["percent"]
        nb = n // b
        assert c["blocks_skipped"] * 2 * nb == (nb - 1) * (nb * nb)


def test_refresh3_flops_and_traffic():
    g = _golden("refresh3_flops_traffic.json")
    rng = np.random.default_rng(1)
    for r in g["rows"]:
        n = r["n"]
        q = rng.standard_normal((1, g["heads"], n, g["d"]))
        k = rng.standard_normal((1, g["heads"], n, g["d"]))
        v = rng.standard_normal((1, g["heads"], n, g["d"]))
        _, _, c = tiled_fwd(q, k, v, 0.125, causal=False, block_q=g["block"],
                            block_k=g["block"], elem_bytes=g["elem_bytes"])
        assert round(c["matmul_flops"] / 1e9, 1) == r["flops_noncausal_G"]
        assert c["hbm_bytes"] / 2 ** 20 == r["tiled_traffic_MiB"]
        assert n // g["block"] == r["kv_rereads"]
        # naive FLOPs: the same expression over the whole matrix
        assert c["matmul_flops"] == 2 * (2 * g["heads"] * n * n * g["d"])
        _, _, cc = tiled_fwd(q, k, v, 0.125, causal=True, block_q=g["block"],
                             block_k=g["block"], elem_bytes=g["elem_bytes"])
        assert round(cc["matmul_flops"] / 1e9, 1) == r["flops_causal_G"]
        nb = n // g["block"]
        assert cc["matmul_flops"] * 2 * nb == c["matmul_flops"] * (nb + 1)


# ---------------------------------------------------------------------------
# agreement, library special case, closed forms, invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("blocks", [(8, 8), (3, 3), (8, 3), (5, 7)])
def test_tiled_equals_naive(causal, blocks):
    rng = np.random.default_rng(42)
    for n in (64, 67):
        q, k, v = (rng.standard_normal((2, 2, n, 16)) for _ in range(3))
        q[0, 0, 5] *= 6.0                      # a later key block holds the max
        k[0, 0, n - 2] = 4.0 * q[0, 0, 5]
        on, ln = naive_fwd(q, k, v, 0.25, causal)
        ot, lt, _ = tiled_fwd(q, k, v, 0.25, causal, *blocks)
        assert np.max(np.abs(on - ot)) < 1e-14
        assert np.max(np.abs(ln - lt)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_naive_matches_library_sdpa_float64(causal):
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((2, 3, 50, 8)) for _ in range(3))
    o, _ = naive_fwd(q, k, v, 0.3, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=0.3).numpy()
    assert np.max(np.abs(o - ref)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((2, 40, 6))
    p = naive_probs(q * 5, k, 1.0, causal)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(p >= 0)
    if causal:
        assert np.all(np.triu(p, 1) == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_prefix_means(causal):
    """Q = 0 makes every visible score 0: P is uniform over the visible keys,
    O_i is the mean of those V rows and lse_i = log(count)."""
    rng = np.random.default_rng(4)
    n = 37
    q = np.zeros((n, 8))
    k, v = rng.standard_normal((2, n, 8))
    o, lse = naive_fwd(q, k, v, 0.5, causal)
    for i in range(n):
        cnt = i + 1 if causal else n
        np.testing.assert_allclose(o[i], v[:cnt].mean(axis=0), atol=1e-14)
        assert abs(lse[i] - math.log(cnt)) < 1e-14


def test_output_in_convex_hull_of_values():
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((3, 60, 16))
    for causal in (False, True):
        o, _ = naive_fwd(q * 3, k, v, 1.0, causal)
        for i in range(60):
            vis = v[: i + 1] if causal else v
            assert np.all(o[i] <= vis.max(axis=0) + 1e-12)
            assert np.all(o[i] >= vis.min(axis=0) - 1e-12)


def test_row_shift_invariance():
    """Adding u to every key row adds scale*q_i.u to row i's scores: O is
    unchanged and lse moves by exactly that constant."""
    rng = np.random.default_rng(6)
    q, k, v = rng.standard_normal((3, 30, 8))
    u = rng.standard_normal(8)
    for causal in (False, True):
        o1, l1 = naive_fwd(q, k, v, 0.7, causal)
        o2, l2 = naive_fwd(q, k + u, v, 0.7, causal)
        np.testing.assert_allclose(o1, o2, atol=1e-13)
        np.testing.assert_allclose(l2 - l1, 0.7 * (q @ u), atol=1e-12)


def test_large_scores_stay_finite():
    """Row maxima far past float32's exp overflow point (88.7) still give a
    finite, correct answer (the max subtraction is present)."""
    rng = np.random.default_rng(8)
    q, k, v = rng.standard_normal((3, 32, 8))
    q *= 60.0
    o, lse = naive_fwd(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.max(lse) > 200
    ot, lt, _ = tiled_fwd(q, k, v, 1.0, block_q=8, block_k=8)
    assert np.max(np.abs(o - ot[0, 0])) < 1e-12


def test_hostile_rows_online_normaliser():
    """Rows of 2048 logits stretched x8 (range ~58), streamed at several block
    sizes: the streamed sum equals the one-shot sum and softmax rows sum to 1."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 2048)) * 8.0
    for row in x:
        one_shot = np.sum(np.exp(row - row.max()))
        for block in (64, 128, 512, 2048):
            m, l, _ = online_normaliser(row, block)
            assert m == row.max()
            assert abs(l / one_shot - 1) < 1e-13
    np.testing.assert_allclose(softmax_rows(x).sum(axis=1), 1.0, atol=1e-14)


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    rng = np.random.default_rng(10)
    n, d, scale = 6, 3, 0.6
    q, k, v, do = rng.standard_normal((4, n, d))
    dq, dk, dv = naive_bwd(q, k, v, do, scale, causal)

    def loss(qq, kk, vv):
        o, _ = naive_fwd(qq, kk, vv, scale, causal)
        return float(np.sum(o * do))

    h = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        fd = np.empty_like(arr)
        for idx in np.ndindex(*arr.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=0, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_library_autograd_float64(causal):
    rng = np.random.default_rng(11)
    q, k, v, do = (rng.standard_normal((2, 2, 33, 8)) for _ in range(4))
    dq, dk, dv = naive_bwd(q, k, v, do, 0.4, causal)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv,
                                                         is_causal=causal,
                                                         scale=0.4)
    o.backward(torch.from_numpy(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_backward_equals_jacobian_backward(causal):
    """The recomputing backward (P from lse, D = rowsum(dO*O)) equals the
    Jacobian form; also checks the identity sum_k P_ik dP_ik = dO_i . O_i."""
    rng = np.random.default_rng(12)
    n = 45
    q, k, v, do = (rng.standard_normal((1, 2, n, 16)) for _ in range(4))
    o, lse = naive_fwd(q, k, v, 0.25, causal)
    ref = naive_bwd(q, k, v, do, 0.25, causal)
    for blocks in ((8, 8), (16, 5), (7, 16)):
        got = tiled_bwd(q, k, v, o, lse, do, 0.25, causal, *blocks)
        for a, b in zip(got, ref):
            assert np.max(np.abs(a - b)) < 1e-12
    p = naive_probs(q[0, 0], k[0, 0], 0.25, causal)
    dp = do[0, 0] @ v[0, 0].T
    np.testing.assert_allclose(np.sum(p * dp, axis=1),
                               np.sum(do[0, 0] * o[0, 0], axis=1), atol=1e-12)


def test_empty_sequence():
    z = np.zeros((1, 2, 0, 8))
    o, lse = naive_fwd(z, z, z, 1.0)
    assert o.shape == (1, 2, 0, 8) and lse.shape == (1, 2, 0)
    dq, dk, dv = naive_bwd(z, z, z, z, 1.0)
    assert dq.shape == z.shape


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_match_full_oracle(causal):
    """The sampled-rows form used for full-size checks equals the full pass."""
    from oracle import naive_fwd_rows
    rng = np.random.default_rng(13)
    q, k, v = rng.standard_normal((3, 70, 8))
    o, lse = naive_fwd(q, k, v, 0.5, causal)
    pos = np.array([0, 3, 31, 32, 69])
    o_r, l_r = naive_fwd_rows(q[pos], k, v, 0.5, causal, pos)
    np.testing.assert_allclose(o_r, o[pos], atol=1e-14)
    np.testing.assert_allclose(l_r, lse[pos], atol=1e-14)



def _autograd_f64(q, k, v, do, scale, causal):
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                         scale=scale)
    o.backward(torch.from_numpy(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_backward_rows_match_library_autograd(causal):
    """The row-wise backward used for full-size checks: each row's dQ, and the
    rows' parts of dK and dV summed over a partition of all rows, equal torch's
    float64 autograd of its own SDPA (a library routine)."""
    from oracle import naive_bwd_rows
    rng = np.random.default_rng(14)
    n, d, scale = 41, 8, 0.35
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    gq, gk, gv = _autograd_f64(q, k, v, do, scale, causal)
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    for part in (np.arange(0, 13), np.array([13, 20, 40]), np.arange(14, 20),
                 np.arange(21, 40)):
        dq_r, dk_p, dv_p = naive_bwd_rows(q[part], k, v, do[part], scale, causal, part)
        assert np.max(np.abs(dq_r - gq[part])) < 1e-12
        dk += dk_p
        dv += dv_p
    assert np.max(np.abs(dk - gk)) < 1e-12
    assert np.max(np.abs(dv - gv)) < 1e-12
    # a subset of keys returns the same parts as the full set
    keys = np.array([0, 7, 40])
    _, dk_s, dv_s = naive_bwd_rows(q[:13], k, v, do[:13], scale, causal, np.arange(13), keys)
    _, dk_f, dv_f = naive_bwd_rows(q[:13], k, v, do[:13], scale, causal, np.arange(13))
    np.testing.assert_array_equal(dk_s, dk_f[keys])
    np.testing.assert_array_equal(dv_s, dv_f[keys])


def test_causal_last_rows_carry_whole_gradients_of_last_keys():
    """Under causal masking the last t keys are seen only by the last t queries,
    so those rows' parts are the keys' complete dK and dV (the form the
    maximum-length GPU check uses)."""
    from oracle import naive_bwd_rows
    rng = np.random.default_rng(15)
    n, d, t, scale = 50, 8, 6, 0.3
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    _, gk, gv = _autograd_f64(q, k, v, do, scale, True)
    rows = np.arange(n - t, n)
    _, dk_p, dv_p = naive_bwd_rows(q[rows], k, v, do[rows], scale, True, rows, rows)
    assert np.max(np.abs(dk_p - gk[rows])) < 1e-12
    assert np.max(np.abs(dv_p - gv[rows])) < 1e-12
    # and the same keys with one row fewer are not complete
    _, dk_m, _ = naive_bwd_rows(q[rows[1:]], k, v, do[rows[1:]], scale, True, rows[1:], rows)
    assert np.max(np.abs(dk_m - gk[rows])) > 1e-6

# --- grouped-query attention -------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 1), (8, 4)])
def test_gqa_matches_library_sdpa_and_autograd_float64(causal, H, Hkv):
    """torch's float64 SDPA with enable_gqa (a library routine that repeats each
    key/value head over consecutive query heads) and its autograd pin the
    head map h -> h // (H // Hkv) and the summed dK, dV of a shared head."""
    from oracle import naive_bwd_gqa, naive_fwd_gqa
    rng = np.random.default_rng(21)
    q = rng.standard_normal((2, H, 29, 8))
    k, v = (rng.standard_normal((2, Hkv, 29, 8)) for _ in range(2))
    do = rng.standard_normal(q.shape)
    o, _ = naive_fwd_gqa(q, k, v, 0.35, causal)
    dq, dk, dv = naive_bwd_gqa(q, k, v, do, 0.35, causal)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=0.35, enable_gqa=True)
    ref.backward(torch.from_numpy(do))
    assert np.max(np.abs(o - ref.detach().numpy())) < 1e-13
    for mine, r in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(mine - r.numpy())) < 1e-12


def test_gqa_with_one_query_head_per_kv_head_is_plain_attention():
    from oracle import naive_bwd_gqa, naive_fwd_gqa
    rng = np.random.default_rng(22)
    q, k, v, do = (rng.standard_normal((1, 3, 20, 8)) for _ in range(4))
    for a, b in zip(naive_fwd_gqa(q, k, v, 0.5, True), naive_fwd(q, k, v, 0.5, True)):
        assert np.array_equal(a, b)
    for a, b in zip(naive_bwd_gqa(q, k, v, do, 0.5, True),
                    naive_bwd(q, k, v, do, 0.5, True)):
        assert np.array_equal(a, b)


def test_gqa_rejects_a_head_count_the_kv_heads_do_not_divide():
    from oracle import naive_fwd_gqa
    z = np.zeros((1, 3, 4, 8))
    with pytest.raises(ValueError):
        naive_fwd_gqa(z, np.zeros((1, 2, 4, 8)), np.zeros((1, 2, 4, 8)), 1.0)


# --- queries and keys of different lengths (bottom-right causal) -----------------

def _sdpa_lower_right(q, k, v, do, scale, causal):
    from torch.nn.attention.bias import causal_lower_right
    import warnings
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")   # the library warns about rows with no key
        mask = causal_lower_right(q.shape[-2], k.shape[-2]) if causal else None
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                             scale=scale)
    o.backward(torch.from_numpy(do))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 37), (5, 37), (16, 64), (37, 37), (40, 19)])
def test_kv_matches_library_sdpa_lower_right_float64(nq, nk, causal):
    """torch's float64 SDPA with its lower-right causal bias (a library routine)
    pins the alignment j <= i + (Nk - Nq), forward and gradients."""
    from oracle import naive_bwd_kv, naive_fwd_kv, visible_mask_kv
    rng = np.random.default_rng(31)
    q = rng.standard_normal((2, 3, nq, 8))
    k, v = (rng.standard_normal((2, 3, nk, 8)) for _ in range(2))
    do = rng.standard_normal(q.shape)
    o, lse = naive_fwd_kv(q, k, v, 0.45, causal)
    dq, dk, dv = naive_bwd_kv(q, k, v, do, 0.45, causal)
    ro, rdq, rdk, rdv = _sdpa_lower_right(q, k, v, do, 0.45, causal)
    live = visible_mask_kv(nq, nk, causal).any(axis=1)
    # rows with visible keys agree with the library; empty rows are 0 / -inf
    assert np.max(np.abs(o[..., live, :] - ro[..., live, :])) < 1e-13
    assert np.all(o[..., ~live, :] == 0) and np.all(lse[..., ~live] == -np.inf)
    assert np.all(np.isfinite(lse[..., live]))
    for mine, ref in ((dq, rdq), (dk, rdk), (dv, rdv)):
        ref = np.nan_to_num(ref)
        assert np.max(np.abs(mine - ref)) < 1e-12


def test_kv_with_equal_lengths_is_plain_attention():
    from oracle import naive_bwd_kv, naive_fwd_kv
    rng = np.random.default_rng(32)
    q, k, v, do = (rng.standard_normal((1, 2, 23, 8)) for _ in range(4))
    for causal in (False, True):
        for a, b in zip(naive_fwd_kv(q, k, v, 0.3, causal), naive_fwd(q, k, v, 0.3, causal)):
            assert np.max(np.abs(a - b)) < 1e-14
        for a, b in zip(naive_bwd_kv(q, k, v, do, 0.3, causal),
                        naive_bwd(q, k, v, do, 0.3, causal)):
            assert np.max(np.abs(a - b)) < 1e-13


def test_kv_gqa_matches_library_on_repeated_heads():
    from oracle import naive_fwd_kv
    rng = np.random.default_rng(33)
    q = rng.standard_normal((1, 6, 9, 8))
    k, v = (rng.standard_normal((1, 2, 30, 8)) for _ in range(2))
    o, _ = naive_fwd_kv(q, k, v, 0.5, True)
    kr, vr = (np.repeat(x, 3, axis=1) for x in (k, v))
    ro, _, _, _ = _sdpa_lower_right(q, kr, vr, np.zeros_like(q), 0.5, True)
    assert np.max(np.abs(o - ro)) < 1e-13


def test_kv_block_merge_law():
    """Attention over all keys equals the merge of two disjoint key blocks by
    their log-sum-exps ("Flash Attention, From First Principles", "The
    scaffold"): lse = log(e^lse1 + e^lse2), O = (e^lse1 O1 + e^lse2 O2) / e^lse.
    This pins lse as the natural log-sum-exp of the scaled scores."""
    from oracle import naive_fwd_kv
    rng = np.random.default_rng(34)
    q = rng.standard_normal((1, 1, 4, 8)) * 3
    k, v = (rng.standard_normal((1, 1, 50, 8)) for _ in range(2))
    o, lse = naive_fwd_kv(q, k, v, 0.7, False)
    o1, l1 = naive_fwd_kv(q, k[:, :, :21], v[:, :, :21], 0.7, False)
    o2, l2 = naive_fwd_kv(q, k[:, :, 21:], v[:, :, 21:], 0.7, False)
    lm = np.logaddexp(l1, l2)
    om = (np.exp(l1 - lm)[..., None] * o1 + np.exp(l2 - lm)[..., None] * o2)
    assert np.max(np.abs(lm - lse)) < 1e-13
    assert np.max(np.abs(om - o)) < 1e-13
    # a single query row: lse is log sum_j exp(scale q.k_j), computed directly
    direct = np.log(np.sum(np.exp(0.7 * (k[0, 0] @ q[0, 0, 2]))))
    assert abs(direct - lse[0, 0, 2]) < 1e-12


def test_kv_decode_row_sees_every_key():
    from oracle import naive_fwd_kv
    rng = np.random.default_rng(35)
    q = rng.standard_normal((1, 2, 1, 8))
    k, v = (rng.standard_normal((1, 2, 40, 8)) for _ in range(2))
    for a, b in zip(naive_fwd_kv(q, k, v, 0.5, True), naive_fwd_kv(q, k, v, 0.5, False)):
        assert np.array_equal(a, b)


# --- e4m3 inputs -------------------------------------------------------------------

def test_e4m3_decode_matches_the_format_and_the_library():
    """Spot values of the OCP e4m3 format, and every one of the 256 codes
    against torch's float8_e4m3fn conversion (a library routine)."""
    from oracle import e4m3_decode
    spots = {0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6,
             0x07: 7 * 2.0 ** -9, 0xB8: -1.0, 0x00: 0.0, 0x3C: 1.5}
    for code, val in spots.items():
        assert e4m3_decode(code) == val, hex(code)
    assert np.isnan(e4m3_decode(0x7F)) and np.isnan(e4m3_decode(0xFF))
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = e4m3_decode(codes)
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.all(both_nan | (ref == mine))


def test_fp8_oracle_is_attention_of_the_dequantised_inputs():
    from oracle import naive_fwd_fp8
    from workloads import make_fp8_inputs
    q8, k8, v8, sq, sk, sv = make_fp8_inputs(1, 2, 40, 16, seed=3)
    o, lse = naive_fwd_fp8(q8.numpy(), k8.numpy(), v8.numpy(), sq, sk, sv, 0.25, True)
    deq = [x.view(torch.float8_e4m3fn).to(torch.float64) * s
           for x, s in ((q8, sq), (k8, sk), (v8, sv))]
    ref = torch.nn.functional.scaled_dot_product_attention(*deq, is_causal=True, scale=0.25)
    assert np.max(np.abs(o - ref.numpy())) < 1e-13
