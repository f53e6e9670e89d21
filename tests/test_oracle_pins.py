"""Pins of the CPU oracle to facts the pages and mathematics fix (no GPU).

Each test ties the oracle to something other than itself: a hand-worked
example, an algebraic identity, a closed form, a textbook routine, a
distributional law, or brute force by explicit loops on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import ndtr

from oracle import sol_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BLK = orc.BLOCK


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# Hand-worked example (tests/golden/hand_worked_4blocks.json)
# ----------------------------------------------------------------------------

def _hand_inputs():
    d, n = 4, 256
    k = np.zeros((n, d))
    q = np.zeros((n, d))
    v = np.zeros((n, d))
    even = (np.arange(BLK) % 2) == 0
    blk = lambda j: slice(j * BLK, (j + 1) * BLK)
    k[blk(0)] = np.where(even[:, None], [2, 0, 1, 0], [2, 0, -1, 0])
    k[blk(1)] = [0, 2, 0, 0]
    k[blk(2)] = [-2, 0, 0, 0]
    k[blk(3)] = [0, 0, 0, 0]
    q[blk(0)] = np.where(even[:, None], [1, 0, 2, 0], [1, 0, -2, 0])
    q[blk(1)] = [0, 1, 0, 0]
    q[blk(2)] = [0, 0, 0, 1]
    q[blk(3)] = [-1, 0, 0, 0]
    v[blk(0)] = np.where(even[:, None], [2, 0, 0, 0], [0, 0, 0, 0])
    v[blk(1)] = [0, 1, 0, 0]
    v[blk(2)] = [0, 0, 1, 0]
    v[blk(3)] = [0, 0, 0, 1]
    return q, k, v


def _ev(expr):
    return eval(expr, {"__builtins__": {}}, {"e": math.e, "sqrt": math.sqrt})


@pytest.mark.parametrize("route_dtype", [np.float64, np.float32])
def test_hand_worked_example(route_dtype):
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_4blocks.json")))
    q, k, v = _hand_inputs()
    exp = g["expected"]
    for corr, key in ((True, "out_correction_on"), (False, "out_correction_off")):
        r = orc.sol_attention_head(q, k, v, g["beta"], corr, route_dtype=route_dtype)
        np.testing.assert_allclose(r["s_hat"], [[_ev(x) for x in row] for row in exp["s_hat"]],
                                   atol=1e-7)
        np.testing.assert_allclose(r["mu"], [_ev(x) for x in exp["mu"]], atol=1e-7)
        np.testing.assert_allclose(r["sigma"], [_ev(x) for x in exp["sigma"]], atol=1e-7)
        np.testing.assert_array_equal(r["mask"], np.array(exp["mask"], dtype=bool))
        out = r["out"]
        want = exp[key]
        rows = {"block0_even": out[0], "block0_odd": out[1], "block1": out[64],
                "block2": out[128], "block3": out[192]}
        for name, got in rows.items():
            np.testing.assert_allclose(got, [_ev(x) for x in want[name]], rtol=1e-12, atol=1e-15,
                                       err_msg=f"{key}/{name}")
        # every row of a block with identical rows agrees with its first row
        for b in (1, 2, 3):
            np.testing.assert_allclose(out[b * BLK:(b + 1) * BLK], np.repeat(out[b * BLK][None], BLK, 0),
                                       rtol=0, atol=0)


# ----------------------------------------------------------------------------
# Closed-form mu/sigma == brute-force row mean/std (the identity the method relies on)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d,nb,seed", [(64, 37, 1), (128, 100, 2), (16, 5, 3)])
def test_closed_form_equals_bruteforce(d, nb, seed):
    rng = _rng(seed)
    # non-centred, correlated keys so that m != 0 and C is dense
    mix = rng.standard_normal((d, d))
    k = (rng.standard_normal((nb * BLK, d)) @ mix) + rng.standard_normal(d) * 3.0
    q = rng.standard_normal((nb * BLK, d)) @ mix.T + 1.0
    kbar = orc.block_means(k)
    qbar = orc.block_means(q)
    s_hat = orc.proxy_scores(qbar, kbar)
    mu_bf, sd_bf = orc.row_mean_std(s_hat)
    m, C = orc.key_summary_moments(kbar)
    mu_cf, sd_cf = orc.closed_form_mean_std(qbar, m, C)
    np.testing.assert_allclose(mu_cf, mu_bf, rtol=1e-9, atol=1e-9 * np.abs(s_hat).max())
    np.testing.assert_allclose(sd_cf, sd_bf, rtol=1e-9)
    # C is a covariance: symmetric and positive semi-definite
    np.testing.assert_allclose(C, C.T, rtol=0, atol=1e-12 * np.abs(C).max())
    assert np.linalg.eigvalsh(C).min() > -1e-9 * np.abs(C).max()


def test_block_means_bruteforce_loop():
    rng = _rng(4)
    x = rng.standard_normal((3 * BLK, 5))
    got = orc.block_means(x)
    for j in range(3):
        for c in range(5):
            s = 0.0
            for t in range(BLK):
                s += x[j * BLK + t, c]
            assert abs(got[j, c] - s / BLK) < 1e-13


# ----------------------------------------------------------------------------
# beta -> -inf is dense softmax attention; the correction is then a no-op
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("correction", [True, False])
def test_dense_limit(correction):
    rng = _rng(5)
    n, d = 6 * BLK, 32
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    r = orc.sol_attention_head(q, k, v, -math.inf, correction, route_dtype=np.float64)
    assert r["mask"].all()
    np.testing.assert_allclose(r["out"], orc.dense_attention(q, k, v), rtol=1e-12, atol=1e-13)


def test_dense_attention_textbook_loop():
    """The dense routine itself against explicit per-row loops on a tiny case."""
    rng = _rng(6)
    n, d = 7, 3
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    got = orc.dense_attention(q, k, v)
    for r in range(n):
        logits = [sum(q[r, c] * k[t, c] for c in range(d)) / math.sqrt(d) for t in range(n)]
        w = [math.exp(x) for x in logits]
        z = sum(w)
        for c in range(d):
            assert abs(got[r, c] - sum(w[t] * v[t, c] for t in range(n)) / z) < 1e-12


# ----------------------------------------------------------------------------
# kept fraction ~ 1 - Phi(beta) when the standardised proxies are Gaussian
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0, 1.5, 2.0])
def test_kept_fraction_gaussian(beta):
    """Keys constant inside each block with k_bar_j ~ N(0, I) make every proxy row
    exactly Gaussian across j (q_bar_i fixed), so the pooled kept fraction must be
    close to 1 - Phi(beta) ([IT] 'Una soglia per ogni riga')."""
    rng = _rng(7)
    d, nb, nq, heads = 64, 2048, 32, 16
    kept = 0
    total = 0
    for _ in range(heads):
        kbar = rng.standard_normal((nb, d))
        k = np.repeat(kbar, BLK, axis=0)                 # constant keys inside each block
        # independent query directions per block, so that rows are (nearly) independent samples
        qtok = np.repeat(rng.standard_normal((nq, d)), BLK, 0) + 0.1 * rng.standard_normal((nq * BLK, d))
        qbar = orc.block_means(qtok)
        s_hat = orc.proxy_scores(qbar.astype(np.float32), orc.block_means(k).astype(np.float32))
        mu, sd = orc.row_mean_std(s_hat)
        mask = orc.select_blocks(s_hat, orc.thresholds(mu, sd, beta))
        kept += mask.sum()
        total += mask.size
    frac = kept / total
    assert abs(frac - (1.0 - ndtr(beta))) < 0.005, (frac, 1.0 - ndtr(beta))


# ----------------------------------------------------------------------------
# The correction (virtual tokens) is exact when every block is constant
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("beta", [-0.5, 0.5, 1.0, 2.0, math.inf])
def test_correction_exact_for_constant_blocks(beta):
    """If all 64 keys of every key block are equal and all 64 queries of every
    query block are equal, each exact logit equals the block proxy s_hat_ij, so
    the corrected output must equal dense attention for any beta ([IT]
    'Scegliere mentre si calcola': zeroth-order term with the block-mean key)."""
    rng = _rng(8)
    nb, d = 9, 16
    q = np.repeat(rng.standard_normal((nb, d)), BLK, axis=0)
    k = np.repeat(rng.standard_normal((nb, d)), BLK, axis=0)
    v = rng.standard_normal((nb * BLK, d))              # values need not be constant
    r = orc.sol_attention_head(q, k, v, beta, True, route_dtype=np.float64)
    if beta == math.inf:
        assert not r["mask"].any()
    else:
        assert r["mask"].any() and not r["mask"].all()
    np.testing.assert_allclose(r["out"], orc.dense_attention(q, k, v), rtol=1e-11, atol=1e-12)


def test_correction_only_is_pooled_attention():
    """beta = +inf with the correction: every block is virtual, and each row of
    query block i equals dense attention of q_bar_i over the block summaries
    (k_bar_j, v_bar_j), the 64-fold multiplicity cancelling."""
    rng = _rng(9)
    nb, d = 12, 8
    q, k, v = (rng.standard_normal((nb * BLK, d)) for _ in range(3))
    r = orc.sol_attention_head(q, k, v, math.inf, True, route_dtype=np.float64)
    assert not r["mask"].any()
    pooled = orc.dense_attention(orc.block_means(q), orc.block_means(k), orc.block_means(v))
    np.testing.assert_allclose(r["out"], np.repeat(pooled, BLK, axis=0), rtol=1e-12, atol=1e-13)


def test_correction_off_empty_rows_are_zero():
    rng = _rng(10)
    q, k, v = (rng.standard_normal((4 * BLK, 8)) for _ in range(3))
    r = orc.sol_attention_head(q, k, v, math.inf, False, route_dtype=np.float64)
    assert not r["out"].any()


@pytest.mark.parametrize("beta,correction", [(0.0, True), (1.0, True), (1.0, False), (math.inf, True)])
def test_constant_values_reproduce_the_constant(beta, correction):
    """Softmax weights (exact and virtual) are a convex combination: V == c gives c."""
    rng = _rng(11)
    n, d = 5 * BLK, 6
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    c = rng.standard_normal(d)
    v = np.tile(c, (n, 1))
    r = orc.sol_attention_head(q, k, v, beta, correction, route_dtype=np.float64)
    rows = np.repeat(r["kept"] > 0, BLK) if not correction else np.ones(n, bool)
    np.testing.assert_allclose(r["out"][rows], np.tile(c, (rows.sum(), 1)), rtol=1e-12, atol=1e-13)


def test_zero_sigma_keeps_nothing():
    """Identical key blocks give a constant proxy row: sigma = 0, tau = mu, and the
    strict test keeps no block ([IT] threshold equation, strict '>')."""
    rng = _rng(12)
    kb = rng.standard_normal((1, 8))
    k = np.tile(kb, (4 * BLK, 1))
    q = rng.standard_normal((4 * BLK, 8))
    v = rng.standard_normal((4 * BLK, 8))
    r = orc.sol_attention_head(q, k, v, 0.0, True, route_dtype=np.float64)
    assert np.all(r["sigma"] == 0)
    assert not r["mask"].any()


# ----------------------------------------------------------------------------
# Invariances of the selection (properties of tau = mu + beta*sigma)
# ----------------------------------------------------------------------------

def _mask(q, k, beta):
    return orc.sol_attention_head(q, k, np.zeros_like(k), beta, False, route_dtype=np.float64)["mask"]


def test_mask_invariances():
    rng = _rng(13)
    nb, d = 20, 16
    q = rng.standard_normal((nb * BLK, d)) + np.repeat(rng.standard_normal((nb, d)), BLK, 0)
    k = rng.standard_normal((nb * BLK, d)) + np.repeat(rng.standard_normal((nb, d)), BLK, 0)
    beta = 0.7
    base = _mask(q, k, beta)
    assert base.any() and not base.all()
    # positive scaling of the keys
    np.testing.assert_array_equal(_mask(q, 3.7 * k, beta), base)
    # translation of every key by one vector shifts each proxy row by a constant
    np.testing.assert_array_equal(_mask(q, k + rng.standard_normal(d), beta), base)
    # the same orthogonal rotation on queries and keys
    rot, _ = np.linalg.qr(rng.standard_normal((d, d)))
    np.testing.assert_array_equal(_mask(q @ rot, k @ rot, beta), base)
    # permuting key blocks permutes the mask columns
    perm = rng.permutation(nb)
    kp = k.reshape(nb, BLK, d)[perm].reshape(-1, d)
    np.testing.assert_array_equal(_mask(q, kp, beta), base[:, perm])
    # permuting tokens inside a key block changes nothing
    kt = k.reshape(nb, BLK, d)[:, rng.permutation(BLK)].reshape(-1, d)
    np.testing.assert_array_equal(_mask(q, kt, beta), base)


def test_output_invariant_under_joint_rotation():
    rng = _rng(14)
    nb, d = 6, 8
    q, k, v = (rng.standard_normal((nb * BLK, d)) for _ in range(3))
    rot, _ = np.linalg.qr(rng.standard_normal((d, d)))
    a = orc.sol_attention_head(q, k, v, 0.5, True, route_dtype=np.float64)
    b = orc.sol_attention_head(q @ rot, k @ rot, v, 0.5, True, route_dtype=np.float64)
    np.testing.assert_array_equal(a["mask"], b["mask"])
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------
# Brute force by explicit loops on a tiny random input
# ----------------------------------------------------------------------------

def _loop_reference(q, k, v, beta, correction):
    """Per-token loops straight from the definitions (independent of the vectorised oracle)."""
    n, d = len(q), len(q[0])
    nb = n // BLK
    mean = lambda x, j, c: sum(x[j * BLK + t][c] for t in range(BLK)) / BLK
    qb = [[mean(q, i, c) for c in range(d)] for i in range(nb)]
    kb = [[mean(k, j, c) for c in range(d)] for j in range(nb)]
    vb = [[mean(v, j, c) for c in range(d)] for j in range(nb)]
    out = [[0.0] * d for _ in range(n)]
    for i in range(nb):
        s = [sum(qb[i][c] * kb[j][c] for c in range(d)) / math.sqrt(d) for j in range(nb)]
        mu = sum(s) / nb
        sd = math.sqrt(sum((x - mu) ** 2 for x in s) / nb)
        tau = mu + beta * sd
        keep = [x > tau for x in s]
        for r in range(i * BLK, (i + 1) * BLK):
            terms = []                       # (logit, multiplicity, value vector)
            for j in range(nb):
                if keep[j]:
                    for t in range(j * BLK, (j + 1) * BLK):
                        lg = sum(q[r][c] * k[t][c] for c in range(d)) / math.sqrt(d)
                        terms.append((lg, 1.0, v[t]))
                elif correction:
                    terms.append((s[j], float(BLK), vb[j]))
            if not terms:
                continue
            mx = max(t[0] for t in terms)
            den = sum(m * math.exp(lg - mx) for lg, m, _ in terms)
            for c in range(d):
                out[r][c] = sum(m * math.exp(lg - mx) * val[c] for lg, m, val in terms) / den
    return np.array(out)


@pytest.mark.parametrize("beta,correction", [(0.3, True), (0.3, False), (-0.4, True)])
def test_bruteforce_loops_tiny(beta, correction):
    rng = _rng(15)
    n, d = 4 * BLK, 3
    q = rng.standard_normal((n, d)) + np.repeat(rng.standard_normal((4, d)), BLK, 0)
    k = rng.standard_normal((n, d)) + np.repeat(rng.standard_normal((4, d)), BLK, 0)
    v = rng.standard_normal((n, d))
    got = orc.sol_attention_head(q, k, v, beta, correction, route_dtype=np.float64)["out"]
    want = _loop_reference(q.tolist(), k.tolist(), v.tolist(), beta, correction)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_query_block_subset_matches_full():
    rng = _rng(16)
    n, d = 10 * BLK, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    full = orc.sol_attention_head(q, k, v, 0.5, True)
    sub = orc.sol_attention_head(q, k, v, 0.5, True, query_blocks=[7, 2])
    np.testing.assert_array_equal(sub["mask"], full["mask"][[7, 2]])
    np.testing.assert_array_equal(sub["out"][:BLK], full["out"][7 * BLK:8 * BLK])
    np.testing.assert_array_equal(sub["out"][BLK:], full["out"][2 * BLK:3 * BLK])


def test_rejects_bad_inputs():
    with pytest.raises(ValueError):
        orc.block_means(np.zeros((65, 4)))
    with pytest.raises(ValueError):
        orc.thresholds(np.zeros(2), np.ones(2), float("nan"))


# ---- routing baselines: top-k and top-p ------------------------------------

def _subsets(n):
    import itertools
    for m in range(n + 1):
        for c in itertools.combinations(range(n), m):
            yield c


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topk_is_the_best_k_subset(seed):
    """Brute force over every subset of a tiny row: the kept set has exactly k blocks and
    the largest score sum of all k-subsets; with integer scores ties resolve to lower j."""
    rng = _rng(40 + seed)
    s = rng.integers(-3, 4, size=(5, 7)).astype(np.float64)
    for k in range(0, 9):
        keep = orc.select_topk(s, k)
        kk = min(k, 7)
        assert (keep.sum(1) == kk).all()
        for i in range(s.shape[0]):
            best = max(sum(s[i, list(c)]) for c in _subsets(7) if len(c) == kk)
            assert sum(s[i, keep[i]]) == best
            # among equal scores at the boundary, the lower index is kept
            kept_idx = np.flatnonzero(keep[i])
            dropped = np.flatnonzero(~keep[i])
            for a in kept_idx:
                for b in dropped:
                    assert s[i, a] > s[i, b] or (s[i, a] == s[i, b] and a < b)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topp_is_the_smallest_set_reaching_p(seed):
    """Brute force over every subset of a tiny row: the kept set reaches probability mass p,
    no smaller set does, and it holds the highest scores."""
    rng = _rng(50 + seed)
    s = rng.standard_normal((4, 7))
    prob = np.exp(s - s.max(1, keepdims=True))
    prob /= prob.sum(1, keepdims=True)
    for p in (0.05, 0.3, 0.5, 0.77, 0.95, 0.999):
        keep = orc.select_topp(s, p)
        for i in range(s.shape[0]):
            m = keep[i].sum()
            assert prob[i, keep[i]].sum() >= p - 1e-12
            smallest = min(len(c) for c in _subsets(7) if prob[i, list(c)].sum() >= p - 1e-12)
            assert m == smallest
            assert s[i, keep[i]].min() >= s[i, ~keep[i]].max(initial=-np.inf)


def test_topp_flat_row_keeps_ceil_p_n():
    """A flat proxy row spreads the probability evenly: top-p keeps ceil(p * n_b) blocks,
    the upper end of the range the pages give; a dominant block alone reaches p."""
    s = np.zeros((1, 8))
    for p, want in ((0.125, 1), (0.5, 4), (0.625, 5), (1.0, 8)):
        assert orc.select_topp(s, p).sum() == want
    s = np.array([[20.0, 0.0, 0.0, 0.0]])
    assert orc.select_topp(s, 0.9).tolist() == [[True, False, False, False]]


def test_topk_topp_monotone():
    rng = _rng(60)
    s = rng.standard_normal((6, 40))
    prev = np.zeros_like(s, dtype=bool)
    for k in range(0, 41, 5):
        cur = orc.select_topk(s, k)
        assert (cur >= prev).all()
        prev = cur
    prev = np.zeros_like(s, dtype=bool)
    for p in (0.1, 0.3, 0.6, 0.9):
        cur = orc.select_topp(s, p)
        assert (cur >= prev).all()
        prev = cur


# ---- per-row correction logit ----------------------------------------------

@pytest.mark.parametrize("beta", [-0.3, 0.4, 1.2, math.inf])
def test_row_correction_exact_for_constant_key_blocks(beta):
    """Per-row form: if the 64 keys of every key block are equal, each virtual token is the
    real token, so the corrected output equals dense attention for any beta, whatever the
    queries ([IT] 'Scegliere mentre si calcola': every token of an excluded block takes the
    block-mean key). The block-level form is not exact here (its logit ignores q_r - q_bar_i)."""
    rng = _rng(70)
    nb, d = 9, 16
    q = rng.standard_normal((nb * BLK, d)) + np.repeat(rng.standard_normal((nb, d)), BLK, axis=0)
    k = np.repeat(rng.standard_normal((nb, d)), BLK, axis=0)
    v = rng.standard_normal((nb * BLK, d))
    dense = orc.dense_attention(q, k, v)
    r = orc.sol_attention_head(q, k, v, beta, True, route_dtype=np.float64, correction_form="row")
    np.testing.assert_allclose(r["out"], dense, rtol=1e-11, atol=1e-12)
    if beta != -0.3:
        blk = orc.sol_attention_head(q, k, v, beta, True, route_dtype=np.float64)
        assert np.abs(blk["out"] - dense).max() > 1e-6


def test_row_correction_equals_block_for_constant_query_blocks():
    """With constant query blocks q_r = q_bar_i, the per-row logit is the block proxy."""
    rng = _rng(71)
    nb, d = 7, 8
    q = np.repeat(rng.standard_normal((nb, d)), BLK, axis=0)
    k = rng.standard_normal((nb * BLK, d))
    v = rng.standard_normal((nb * BLK, d))
    for beta in (0.0, 0.8):
        a = orc.sol_attention_head(q, k, v, beta, True, route_dtype=np.float64, correction_form="row")
        b = orc.sol_attention_head(q, k, v, beta, True, route_dtype=np.float64)
        np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-13)


def test_row_correction_only_is_attention_over_summaries():
    """beta = +inf with the per-row correction: each row attends to the block summaries
    (k_bar_j, v_bar_j), the multiplicity 64 cancelling: dense attention of q_r over them."""
    rng = _rng(72)
    nb, d = 6, 5
    q, k, v = (rng.standard_normal((nb * BLK, d)) for _ in range(3))
    r = orc.sol_attention_head(q, k, v, math.inf, True, route_dtype=np.float64, correction_form="row")
    kb, vb = orc.block_means(k), orc.block_means(v)
    np.testing.assert_allclose(r["out"], orc.dense_attention(q, kb, vb), rtol=1e-11, atol=1e-12)
    with pytest.raises(ValueError):
        orc.sol_attention_head(q, k, v, 1.0, True, correction_form="tokens")


# ---- joint attention with an exact text segment ------------------------------

def test_text_segment_rows_and_columns_exact():
    """Text key blocks are kept by every query block, text query rows equal dense attention,
    and a text segment covering the whole sequence gives dense attention."""
    rng = _rng(80)
    nb, d, T = 12, 8, 3
    q, k, v = (rng.standard_normal((nb * BLK, d)) for _ in range(3))
    r = orc.sol_attention_head(q, k, v, 1.5, True, route_dtype=np.float64, text_blocks=T)
    assert r["mask"][:, nb - T:].all() and r["mask"][nb - T:, :].all()
    plain = orc.sol_attention_head(q, k, v, 1.5, True, route_dtype=np.float64)
    assert (r["mask"] >= plain["mask"]).all()
    dense = orc.dense_attention(q, k, v)
    np.testing.assert_allclose(r["out"][(nb - T) * BLK:], dense[(nb - T) * BLK:], rtol=1e-11, atol=1e-12)
    full = orc.sol_attention_head(q, k, v, 2.5, False, route_dtype=np.float64, text_blocks=nb)
    np.testing.assert_allclose(full["out"], dense, rtol=1e-11, atol=1e-12)
