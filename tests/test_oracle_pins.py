"""Pins of the float64 oracle against facts the pages and the mathematics fix.

Each test names the plausible mistake it would catch. None of these re-types the
oracle's own formula: they compare against textbook routines (scipy), brute force over
tiny inputs, closed forms and invariants.
"""
import itertools

import numpy as np
import pytest
import scipy.optimize
import scipy.special

from oracle import am_oracle as O

RNG = np.random.default_rng(1234)


def _qkv(n, T, d, rng=RNG, qscale=1.0):
    Q = rng.standard_normal((n, d)) * qscale
    K = rng.standard_normal((T, d)) * rng.lognormal(0, 0.5, d)
    V = rng.standard_normal((T, d))
    return Q, K, V


def _loop_stats(Q, K, V, scale, causal, group):
    """Per-query brute force with scipy's textbook softmax/logsumexp."""
    n, T = Q.shape[0], K.shape[0]
    lse = np.empty(n)
    Oo = np.empty((n, V.shape[1]))
    P = np.zeros((n, T))
    for i in range(n):
        nv = (i // group + 1) if causal else T
        s = np.array([scale * float(np.dot(Q[i], K[j])) for j in range(nv)])
        lse[i] = scipy.special.logsumexp(s)
        p = scipy.special.softmax(s)
        Oo[i] = p @ V[:nv]
        P[i, :nv] = p
    return lse, Oo, P


# ---------------------------------------------------------------------------- S1 / S2
@pytest.mark.parametrize("causal,group", [(False, 1), (True, 1), (True, 4), (False, 4)])
def test_stats_match_textbook_softmax(causal, group):
    # catches: missing scale, transposed operand, causal off-by-one, wrong lse base
    T, d = 13, 8
    n = T * group
    Q, K, V = _qkv(n, T, d)
    scale = 1 / np.sqrt(d)
    lse, Oo, stats = O.full_cache_stats(Q, K, V, scale, causal, group)
    lse2, O2, P = _loop_stats(Q, K, V, scale, causal, group)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Oo, O2, rtol=1e-12, atol=1e-12)
    # per-key statistics by brute force over the full probability matrix
    np.testing.assert_allclose(stats[0], P.sum(0), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(stats[1], (P ** 2).sum(0), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(stats[2], P.max(0), rtol=1e-12, atol=1e-15)
    # MAX mode is Eq. 6: max over queries of softmax(s K q)_i (non-causal case)
    if not causal:
        sm = scipy.special.softmax(scale * Q @ K.T, axis=1)
        np.testing.assert_allclose(O.key_score(stats, "max", n), sm.max(0), rtol=1e-12)
    np.testing.assert_allclose(O.key_score(stats, "rms", n), np.sqrt((P ** 2).mean(0)), rtol=1e-12)
    np.testing.assert_allclose(O.key_score(stats, "mean", n), P.mean(0), rtol=1e-12)


def test_stats_chunked_equals_single_block():
    # catches: chunk-boundary bugs in the query loop (budget forces many chunks)
    Q, K, V = _qkv(300, 50, 8)
    a = O.full_cache_stats(Q, K, V, 0.3, True, 3)
    import oracle.am_oracle as mod
    saved = mod._chunks
    try:
        mod._chunks = lambda n, T, budget=0: [(0, n)]
        b = O.full_cache_stats(Q, K, V, 0.3, True, 3)
    finally:
        mod._chunks = saved
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13)
    for x, y in zip(a[2], b[2]):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-16)


def test_shift_invariance_and_value_linearity():
    # adding c to every score of a row: O unchanged, lse shifted by c (catches max-shift bugs)
    Q, K, V = _qkv(20, 30, 6)
    scale = 0.37
    c = 5.0
    Q2 = np.hstack([Q, np.full((20, 1), c / scale)])
    K2 = np.hstack([K, np.ones((30, 1))])
    l1, O1, _ = O.full_cache_stats(Q, K, V, scale)
    l2, O2, _ = O.full_cache_stats(Q2, K2, V, scale)
    np.testing.assert_allclose(l2, l1 + c, atol=1e-12)
    np.testing.assert_allclose(O2, O1, atol=1e-12)
    _, O3, _ = O.full_cache_stats(Q, K, 2.5 * V, scale)
    np.testing.assert_allclose(O3, 2.5 * O1, atol=1e-12)


def test_large_scores_do_not_overflow():
    # scores near 700 would overflow exp without the max shift
    Q, K, V = _qkv(5, 7, 4)
    l, Oo, _ = O.full_cache_stats(Q * 400, K, V, 1.0)
    l2, O2, _ = _loop_stats(Q * 400, K, V, 1.0, False, 1)
    np.testing.assert_allclose(l, l2, rtol=1e-14)
    np.testing.assert_allclose(Oo, O2, atol=1e-12)


def test_attention_rows_matches_full():
    Q, K, V = _qkv(40, 10, 4)
    lse, Oo, _ = O.full_cache_stats(Q, K, V, 0.5, True, 4)
    rows = np.array([0, 3, 17, 39])
    l2, O2 = O.attention_rows(Q, K, V, 0.5, rows, True, 4)
    np.testing.assert_allclose(l2, lse[rows], atol=1e-13)
    np.testing.assert_allclose(O2, Oo[rows], atol=1e-13)


# ---------------------------------------------------------------------------- S3
def test_select_top_bruteforce_and_ties():
    # I4(a): idx = lexicographically smallest argmax over all t-subsets of the score sum
    rng = np.random.default_rng(7)
    for trial in range(30):
        T = int(rng.integers(2, 11))
        t = int(rng.integers(1, min(4, T) + 1))
        sc = rng.integers(0, 4, T).astype(float) / 3.0  # many exact ties
        best, best_set = -1.0, None
        for S in itertools.combinations(range(T), t):  # lexicographic order
            v = sc[list(S)].sum()
            if v > best + 1e-15:
                best, best_set = v, S
        got = O.select_top(sc, t)
        assert list(got) == sorted(best_set), (sc, t, got, best_set)
        assert np.all(np.diff(got) > 0)


def test_select_top_tie_goes_to_lower_index():
    sc = np.array([0.5, 0.9, 0.5, 0.5, 0.1])
    assert list(O.select_top(sc, 2)) == [0, 1]
    assert list(O.select_top(sc, 3)) == [0, 1, 2]


# ---------------------------------------------------------------------------- S5 NNLS
def _bruteforce_nnls(M, b):
    """Enumerate every support, solve unconstrained LS on it, keep feasible minimum."""
    t = M.shape[1]
    best, bw = np.inf, None
    for mask in itertools.product([0, 1], repeat=t):
        S = np.flatnonzero(mask)
        w = np.zeros(t)
        if S.size:
            w[S] = np.linalg.lstsq(M[:, S], b, rcond=None)[0]
        if np.any(w < -1e-12):
            continue
        w = np.maximum(w, 0)
        f = np.sum((M @ w - b) ** 2)
        if f < best - 1e-14:
            best, bw = f, w
    return bw, best


def test_nnls_bruteforce_tiny():
    # I4(b): the active-set NNLS equals enumeration of all 2^t supports
    rng = np.random.default_rng(11)
    for trial in range(40):
        n = int(rng.integers(3, 25))
        t = int(rng.integers(1, 5))
        M = rng.standard_normal((n, t))
        if trial % 2:
            M = np.abs(M)
        b = rng.standard_normal(n) + (trial % 3 == 0) * 2
        w, _ = O.fit_beta(M, b)
        wb, fb = _bruteforce_nnls(M, b)
        f = np.sum((M @ w - b) ** 2)
        assert f <= fb * (1 + 1e-10) + 1e-12
        np.testing.assert_allclose(M @ w, M @ wb, atol=1e-8)
        assert np.all(w >= 0)


def test_nnls_matches_scipy_and_kkt():
    # textbook routine (scipy's Lawson-Hanson) on medium problems; I3 KKT holds
    rng = np.random.default_rng(5)
    for n, t in [(200, 30), (500, 64), (100, 80)]:
        M = np.abs(rng.standard_normal((n, t))) ** 2
        b = np.ones(n) + 0.3 * rng.standard_normal(n)
        w, beta = O.fit_beta(M, b)
        ws, _ = scipy.optimize.nnls(M, b)
        np.testing.assert_allclose(M @ w, M @ ws, atol=1e-8)
        G, h = M.T @ M, M.T @ b
        assert O.nnls_kkt_residual(G, h, w) <= 1e-9 * np.abs(h).max()
        assert np.all(np.isneginf(beta[w == 0]))
        np.testing.assert_allclose(np.exp(beta[w > 0]), w[w > 0], rtol=1e-14)


def test_nnls_rank_deficient_unique_mass():
    # duplicated columns: w is not unique, but M w is (I6 / reading A7)
    rng = np.random.default_rng(9)
    M = np.abs(rng.standard_normal((60, 5)))
    M = np.hstack([M, M[:, :2]])
    b = np.ones(60)
    w, _ = O.fit_beta(M, b)
    ws, _ = scipy.optimize.nnls(M, b)
    np.testing.assert_allclose(M @ w, M @ ws, atol=1e-9)
    assert O.nnls_kkt_residual(M.T @ M, M.T @ b, w) <= 1e-9


def test_nnls_box_bounds_and_kkt():
    rng = np.random.default_rng(3)
    M = np.abs(rng.standard_normal((80, 10)))
    b = 1 + rng.standard_normal(80)
    lo, hi = np.exp(-3), np.exp(3)
    w, _ = O.fit_beta(M, b, lo, hi)
    assert np.all(w >= lo - 1e-12) and np.all(w <= hi + 1e-12)
    assert O.nnls_kkt_residual(M.T @ M, M.T @ b, w, lo, hi) <= 1e-8


# ---------------------------------------------------------------------------- S7 ridge
def test_ridge_equals_stacked_lstsq_for_every_subset():
    # I4(c): (A^T A + lam I)^-1 A^T Y equals QR least squares on [A; sqrt(lam) I]
    rng = np.random.default_rng(21)
    A_full = np.abs(rng.standard_normal((20, 6)))
    Y = rng.standard_normal((20, 3))
    for lam in (0.0, 1e-3, 0.5):
        for t in range(1, 4):
            for S in itertools.combinations(range(6), t):
                A = A_full[:, S]
                C = O.fit_values(A, Y, lam)
                stacked = np.vstack([A, np.sqrt(lam) * np.eye(t)])
                rhs = np.vstack([Y, np.zeros((t, 3))])
                C2 = np.linalg.lstsq(stacked, rhs, rcond=None)[0]
                np.testing.assert_allclose(C, C2, rtol=1e-9, atol=1e-10)


def test_t1_closed_forms():
    # I5: t = 1 -> w = m.1 / m.m and C_v = a^T Y / (a^T a + lam), a = 0/1 visibility
    rng = np.random.default_rng(4)
    T, d, group = 9, 4, 2
    Q, K, V = _qkv(T * group, T, d, rng)
    r = O.compact_head(Q, K, V, 1, 0.5, True, group, ridge_lambda=0.01)
    m = r["M"][:, 0]
    assert r["w"][0] == pytest.approx(m.sum() / (m @ m), rel=1e-12)
    a = (m > 0).astype(float)
    np.testing.assert_allclose(r["A"][:, 0], a, atol=0)
    np.testing.assert_allclose(r["Cv"][0], a @ r["O"] / (a @ a + 0.01), rtol=1e-12)


# ---------------------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal,group", [(False, 1), (True, 2)])
def test_I1_full_budget_reproduces_cache(causal, group):
    # with t = T, C_k = K, beta = 0, C_v = V the evaluator gives back O and lse exactly,
    # and the fits recover w = 1 and (lambda = 0) C_v = V
    rng = np.random.default_rng(31)
    T, d = 12, 6
    n = max(T * group, 3 * T)
    n -= n % group
    Q, K, V = _qkv(n, T, d, rng)
    sc = 1 / np.sqrt(d)
    lse, Oo, _ = O.full_cache_stats(Q, K, V, sc, causal, group)
    logz, A = O.compacted_attention(Q, K, np.arange(T), np.zeros(T), V, sc, causal, group)
    np.testing.assert_allclose(logz, lse, atol=1e-12)
    np.testing.assert_allclose(A, Oo, atol=1e-12)
    r = O.compact_head(Q, K, V, T, sc, causal, group, ridge_lambda=0.0)
    assert list(r["idx"]) == list(range(T))
    np.testing.assert_allclose(r["w"], 1.0, atol=1e-9)
    np.testing.assert_allclose(r["Cv"], V, atol=1e-7)
    assert r["r_mass"] < 1e-18 and r["r_out"] < 1e-14


def test_I2_zero_query_mass():
    # q = 0: every score is 0, so Z = number of visible keys (log T non-causal) and the
    # compacted mass is sum_j exp(beta_j) over the visible compacted keys
    rng = np.random.default_rng(8)
    T, d = 10, 4
    Q = np.zeros((T * 2, d))
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    lse, _, _ = O.full_cache_stats(Q, K, V, 0.5)
    np.testing.assert_allclose(lse, np.log(T), atol=1e-14)
    lse_c, _, _ = O.full_cache_stats(Q, K, V, 0.5, True, 2)
    np.testing.assert_allclose(lse_c, np.log(np.arange(2 * T) // 2 + 1), atol=1e-14)
    beta = rng.standard_normal(4)
    idx = np.array([0, 3, 5, 9])
    logz, _ = O.compacted_attention(Q, K[idx], idx, beta, V[idx], 0.5)
    np.testing.assert_allclose(logz, np.log(np.exp(beta).sum()), atol=1e-14)
    # and the fit: constant rows, so NNLS reaches zero residual with sum(w) = T
    r = O.compact_head(Q, K, V, 4, 0.5)
    assert r["r_mass"] < 1e-20
    assert r["w"].sum() == pytest.approx(T, rel=1e-10)


def test_I6_permutation_equivariance():
    rng = np.random.default_rng(12)
    Q, K, V = _qkv(30, 15, 5, rng)
    perm = rng.permutation(15)
    a = O.compact_head(Q, K, V, 4, 0.4)
    b = O.compact_head(Q, K[perm], V[perm], 4, 0.4)
    inv = np.argsort(perm)
    np.testing.assert_allclose(b["score"][inv], a["score"], rtol=1e-12)
    assert sorted(perm[b["idx"]]) == list(a["idx"])
    assert b["r_mass"] == pytest.approx(a["r_mass"], rel=1e-8)
    assert b["r_out"] == pytest.approx(a["r_out"], rel=1e-8)


def test_residuals_agree_with_evaluator():
    # the fitted design residuals equal the evaluator's (Eq. 2-4) residuals
    rng = np.random.default_rng(2)
    Q, K, V = _qkv(64, 20, 6, rng)
    for causal, group in [(False, 1), (True, 4)]:
        Qg = Q if not causal else Q[:80] if Q.shape[0] >= 80 else np.vstack([Q, Q[:16]])
        r = O.compact_head(Qg, K, V, 5, 0.4, causal, group)
        logz, A = O.compacted_attention(Qg, r["Ck"], r["idx"], r["beta"], r["Cv"], 0.4, causal, group)
        rm, ro = O.residuals(r["lse"], r["O"], logz, A)
        assert rm == pytest.approx(r["r_mass"], rel=1e-9)
        assert ro == pytest.approx(r["r_out"], rel=1e-9)


def test_absolute_mass_mode_is_row_weighting():
    # the absolute form weights equation i by Z_i: with an exact fit available (t = T)
    # both forms give w = 1; otherwise the absolute optimum is the weighted LS optimum
    rng = np.random.default_rng(17)
    T, d = 8, 4
    Q, K, V = _qkv(40, T, d, rng)
    ra = O.compact_head(Q, K, V, T, 0.5, mass="absolute", ridge_lambda=0.0)
    np.testing.assert_allclose(ra["w"], 1.0, atol=1e-8)
    lse, _, _ = O.full_cache_stats(Q, K, V, 0.5)
    idx = np.array([1, 4, 6])
    Mr, _ = O.mass_design(Q, K[idx], idx, lse, 0.5, mode="relative")
    Ma, ba = O.mass_design(Q, K[idx], idx, lse, 0.5, mode="absolute")
    z = np.exp(lse - lse.max())
    np.testing.assert_allclose(Ma, Mr * z[:, None], rtol=1e-12)
    wa, _ = O.fit_beta(Ma, ba)
    ws, _ = scipy.optimize.nnls(Mr * z[:, None], z)
    np.testing.assert_allclose(Ma @ wa, Ma @ ws, atol=1e-10)


# --------------------------------------------------------------------------------------
# cache attention with appended entries (Latent Compaction §3.1 Eq. 2-5, App. A.2)
# --------------------------------------------------------------------------------------
def _cache_case(rng, n=37, t=23, m=11, d=8, group=2):
    Q = rng.standard_normal((n, d))
    Ck = rng.standard_normal((t, d))
    Cv = rng.standard_normal((t, d))
    bias = rng.standard_normal(t)
    keypos = np.sort(rng.choice(3 * t, size=t, replace=False))
    Kn = rng.standard_normal((m, d))
    Vn = rng.standard_normal((m, d))
    return Q, Ck, Cv, bias, keypos, Kn, Vn


@pytest.mark.parametrize("causal,new_causal,nvalid", [(False, True, None), (True, True, 17),
                                                      (True, False, 23), (False, False, 5)])
def test_cache_attention_is_one_softmax_over_both_sets(causal, new_causal, nvalid):
    """Eq. 5 equals a single softmax over the document slots (biased, masked) and the new
    entries (unbiased, causal): computed here directly on the concatenation."""
    rng = np.random.default_rng(11)
    Q, Ck, Cv, bias, keypos, Kn, Vn = _cache_case(rng)
    n, t, m, g, scale = Q.shape[0], Ck.shape[0], Kn.shape[0], 2, 0.4
    out, lz, lz1 = O.cache_attention(Q, Ck, Cv, bias, scale, keypos=keypos, nvalid=nvalid,
                                     causal=causal, group=g, Kn=Kn, Vn=Vn, new_causal=new_causal)
    s = np.concatenate([scale * Q @ Ck.T + bias, scale * Q @ Kn.T], axis=1)
    ok = np.ones_like(s, dtype=bool)
    if nvalid is not None:
        ok[:, nvalid:t] = False
    pos = np.arange(n) // g
    if causal:
        ok[:, :t] &= keypos[None, :] <= pos[:, None]
    if new_causal:
        ok[:, t:] &= np.arange(m)[None, :] <= pos[:, None]
    s = np.where(ok, s, -np.inf)
    ref_lz = scipy.special.logsumexp(s, axis=1)
    ref_out = np.exp(s - ref_lz[:, None]) @ np.concatenate([Cv, Vn])
    np.testing.assert_allclose(lz, ref_lz, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    ref_lz1 = scipy.special.logsumexp(s[:, :t], axis=1)
    np.testing.assert_allclose(lz1, ref_lz1, rtol=0, atol=1e-12)


def test_bias_is_log_multiplicity():
    """A slot with bias log r weighs exactly like r unbiased copies of its key and value."""
    rng = np.random.default_rng(12)
    Q, Ck, Cv, _, _, _, _ = _cache_case(rng, t=6)
    r = np.array([1, 3, 1, 2, 5, 1])
    rep_k, rep_v = np.repeat(Ck, r, axis=0), np.repeat(Cv, r, axis=0)
    out_b, lz_b, _ = O.cache_attention(Q, Ck, Cv, np.log(r), 0.7)
    out_r, lz_r, _ = O.cache_attention(Q, rep_k, rep_v, np.zeros(r.sum()), 0.7)
    np.testing.assert_allclose(out_b, out_r, atol=1e-12)
    np.testing.assert_allclose(lz_b, lz_r, atol=1e-12)


def test_cache_attention_hand_example():
    """d = 1, q = 1, scale 1. Document: keys 0, 0 with biases 0, log 3 and values 1, 5, so
    Z_cmp = 1 + 3 = 4 and A_cmp = (1 + 15) / 4 = 4. New entry: key log 4, value -2, so
    Z_new = 4 and A_new = -2. Eq. 5: A = (4 * 4 + 4 * (-2)) / 8 = 1 and log Z = log 8."""
    out, lz, lz1 = O.cache_attention(np.ones((1, 1)), np.zeros((2, 1)), np.array([[1.0], [5.0]]),
                                     np.array([0.0, np.log(3.0)]), 1.0,
                                     Kn=np.array([[np.log(4.0)]]), Vn=np.array([[-2.0]]))
    assert abs(out[0, 0] - 1.0) < 1e-14
    assert abs(lz[0] - np.log(8.0)) < 1e-14
    assert abs(lz1[0] - np.log(4.0)) < 1e-14


def test_cache_attention_empty_branches():
    rng = np.random.default_rng(13)
    Q, Ck, Cv, bias, keypos, Kn, Vn = _cache_case(rng)
    # no new entries: the document branch alone
    out, lz, lz1 = O.cache_attention(Q, Ck, Cv, bias, 0.5)
    l = O.biased_scores(Q, Ck, bias, np.ones((Q.shape[0], Ck.shape[0]), bool), 0.5)
    d_lz = O.log_normalizer(l)
    d_out = O.attention_output(l, d_lz, Cv)
    np.testing.assert_array_equal(out, d_out)
    np.testing.assert_array_equal(lz, d_lz)
    # no valid slot: the new branch alone (unbiased causal attention over Kn)
    out, lz, lz1 = O.cache_attention(Q, Ck, Cv, bias, 0.5, nvalid=0, Kn=Kn, Vn=Vn, group=4)
    assert np.all(lz1 == -np.inf)
    ref_lse, ref_O, _ = O.full_cache_stats(Q, Kn, Vn, 0.5, causal=True, group=4)
    np.testing.assert_allclose(lz, ref_lse, atol=1e-12)
    np.testing.assert_allclose(out, ref_O, atol=1e-12)
    # both empty: -inf and zero rows
    out, lz, _ = O.cache_attention(Q, Ck, Cv, bias, 0.5, nvalid=0)
    assert np.all(lz == -np.inf) and np.all(out == 0.0)


def test_unbiased_cache_attention_is_plain_attention():
    rng = np.random.default_rng(14)
    Q, Ck, Cv, _, _, _, _ = _cache_case(rng)
    out, lz, _ = O.cache_attention(Q, Ck, Cv, np.zeros(Ck.shape[0]), 0.3)
    lse, Oref, _ = O.full_cache_stats(Q, Ck, Cv, 0.3)
    np.testing.assert_allclose(lz, lse, atol=1e-12)
    np.testing.assert_allclose(out, Oref, atol=1e-12)


def test_combine_weights_sum_to_one_and_commute():
    rng = np.random.default_rng(15)
    o1, o2 = rng.standard_normal((2, 9, 4))
    l1 = rng.standard_normal(9) * 5
    l2 = rng.standard_normal(9) * 5
    l2[3] = -np.inf
    a, la = O.merge_log_space(o1, l1, o2, l2)
    b, lb = O.merge_log_space(o2, l2, o1, l1)
    np.testing.assert_allclose(a, b, atol=1e-13)
    np.testing.assert_array_equal(la, lb)
    np.testing.assert_allclose(a[3], o1[3], atol=1e-15)
    # equal normalizers: the plain average, and log Z grows by log 2
    c, lc = O.merge_log_space(o1, l1, o2, l1)
    np.testing.assert_allclose(c, 0.5 * (o1 + o2), atol=1e-13)
    np.testing.assert_allclose(lc, l1 + np.log(2.0), atol=1e-13)


# --------------------------------------------------------------------------------------
# fast variants ("Compaction" blog: redistribution beta, direct values)
# --------------------------------------------------------------------------------------
def _loop_redistribute(Q, Ck, idx, lse, scale, causal, group):
    n, t = Q.shape[0], Ck.shape[0]
    m = [0.0] * t
    missing = 0.0
    for i in range(n):
        cmp_mass = 0.0
        for j in range(t):
            if not causal or idx[j] <= i // group:
                e = float(np.exp(scale * float(Q[i] @ Ck[j])))
                m[j] += e / n
                cmp_mass += e
        missing += (float(np.exp(lse[i])) - cmp_mass) / n
    return np.array([np.log((m[j] + missing / t) / m[j]) for j in range(t)])


@pytest.mark.parametrize("causal,group", [(False, 1), (True, 2)])
def test_redistribute_beta_bruteforce(causal, group):
    rng = np.random.default_rng(16)
    T, d = 20, 6
    n = group * T
    Q, K, V = _qkv(n, T, d, rng)
    lse, _, _ = O.full_cache_stats(Q, K, V, 0.5, causal, group)
    idx = np.array([0, 3, 4, 9, 15, 19])
    got = O.redistribute_beta(Q, K[idx], idx, lse, 0.5, causal, group)
    ref = _loop_redistribute(Q, K[idx], idx, lse, 0.5, causal, group)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal,group", [(False, 1), (True, 3)])
def test_redistribute_beta_conserves_mean_mass(causal, group):
    """With the redistributed biases the compacted cache's mass averaged over the reference
    queries equals the full cache's (the missing mass is handed back in full)."""
    rng = np.random.default_rng(17)
    T, d = 64, 8
    n = group * T
    Q, K, V = _qkv(n, T, d, rng)
    lse, _, _ = O.full_cache_stats(Q, K, V, 0.4, causal, group)
    idx = np.sort(rng.choice(T, size=12, replace=False))
    idx[0] = 0
    beta = O.redistribute_beta(Q, K[idx], idx, lse, 0.4, causal, group)
    logz, _ = O.compacted_attention(Q, K[idx], idx, beta, V[idx], 0.4, causal, group)
    np.testing.assert_allclose(np.exp(logz).mean(), np.exp(lse).mean(), rtol=1e-12)
    assert np.all(beta >= 0.0)   # the compacted keys never hold more than the full cache


def test_redistribute_beta_full_budget_is_zero():
    rng = np.random.default_rng(18)
    Q, K, V = _qkv(30, 30, 5, rng)
    lse, _, _ = O.full_cache_stats(Q, K, V, 0.6, True, 1)
    beta = O.redistribute_beta(Q, K, np.arange(30), lse, 0.6, True, 1)
    np.testing.assert_allclose(beta, 0.0, atol=1e-12)


def test_direct_values_are_the_selected_rows():
    V = np.arange(24.0).reshape(8, 3)
    np.testing.assert_array_equal(O.direct_values(V, [1, 4, 6]), V[[1, 4, 6]])


# --------------------------------------------------------------------------------------
# two-pass selection ("Compaction" blog, §Choosing C_k, Attempt #3)
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("causal,group", [(False, 1), (True, 2)])
def test_two_pass_with_full_shortlist_and_all_queries_is_full_selection(causal, group):
    rng = np.random.default_rng(21)
    T, d = 48, 8
    n = group * T
    Q, K, V = _qkv(n, T, d, rng)
    lse, _, st = O.full_cache_stats(Q, K, V, 0.5, causal, group)
    full = O.select_top(O.key_score(st, "rms", n), 10)
    idx, lse_s = O.select_two_pass(Q, K, np.arange(n), 10, 5, 0.5, causal, group)   # 50 >= T
    np.testing.assert_array_equal(idx, full)
    np.testing.assert_allclose(lse_s, lse, atol=1e-12)


def _loop_two_pass(Q, K, sub, t, k_mult, scale, causal, group):
    n, T = Q.shape[0], K.shape[0]

    def stats(rows, keys):
        sq = np.zeros(len(keys))
        lse = np.zeros(len(rows))
        for a, i in enumerate(rows):
            vis = [b for b, j in enumerate(keys) if not causal or j <= i // group]
            sc = {b: scale * float(Q[i] @ K[keys[b]]) for b in vis}
            m = max(sc.values())
            z = sum(np.exp(v - m) for v in sc.values())
            lse[a] = m + np.log(z)
            for b, v in sc.items():
                sq[b] += float(np.exp(v - lse[a])) ** 2
        return sq, lse

    sq1, _ = stats(list(sub), list(range(T)))
    r1 = np.sqrt(sq1 / len(sub))
    short = sorted(sorted(range(T), key=lambda j: (-r1[j], j))[: min(k_mult * t, T)])
    sq2, lse2 = stats(list(range(n)), short)
    r2 = np.sqrt(sq2 / n)
    loc = sorted(sorted(range(len(short)), key=lambda b: (-r2[b], b))[:t])
    return np.array([short[b] for b in loc]), lse2


@pytest.mark.parametrize("causal,group", [(False, 1), (True, 3)])
def test_two_pass_bruteforce(causal, group):
    rng = np.random.default_rng(22)
    T, d = 30, 6
    n = group * T
    Q, K, V = _qkv(n, T, d, rng)
    sub = np.sort(rng.choice(n, size=12, replace=False))
    idx, lse_s = O.select_two_pass(Q, K, sub, 4, 2, 0.7, causal, group)
    ref_idx, ref_lse = _loop_two_pass(Q, K, sub, 4, 2, 0.7, causal, group)
    np.testing.assert_array_equal(idx, ref_idx)
    np.testing.assert_allclose(lse_s, ref_lse, atol=1e-12)


def test_two_pass_shortlist_mass_is_a_lower_bound():
    rng = np.random.default_rng(23)
    Q, K, V = _qkv(80, 80, 8, rng)
    lse, _, _ = O.full_cache_stats(Q, K, V, 0.5, True, 1)
    idx, lse_s = O.select_two_pass(Q, K, np.arange(0, 80, 5), 6, 2, 0.5, True, 1)
    assert np.all(lse_s <= lse + 1e-12)
    assert np.all(np.diff(idx) > 0) and idx.size == 6


def test_rows_that_see_no_key_subset():
    """With a key subset at later positions, early causal rows see nothing: lse = -inf, a
    zero output row, and no contribution to any key's statistics."""
    rng = np.random.default_rng(24)
    Q, K, V = _qkv(20, 20, 4, rng)
    keypos = np.array([5, 9, 14])
    lse, Oo, (cs, cq, cm) = O.full_cache_stats(Q, K[keypos], V[keypos], 0.5, True, 1,
                                               keypos=keypos)
    assert np.all(lse[:5] == -np.inf) and np.all(Oo[:5] == 0.0)
    l2, O2, (s2, q2, m2) = O.full_cache_stats(Q[5:], K[keypos], V[keypos], 0.5, True, 1,
                                              rows=np.arange(5, 20), keypos=keypos)
    np.testing.assert_allclose(lse[5:], l2, atol=1e-13)
    np.testing.assert_allclose(cs, s2, atol=1e-13)
    np.testing.assert_allclose(cq, q2, atol=1e-13)


# --------------------------------------------------------------------------------------
# anchor + diversifier initialization (Latent Compaction §3.2, Eq. 6-7)
# --------------------------------------------------------------------------------------
def test_select_anchors_first_entry_and_ties():
    sc = np.array([0.0, 5.0, 3.0, 5.0, 9.0, 1.0])
    np.testing.assert_array_equal(O.select_anchors(sc, 3), [0, 1, 4])   # 9, then 5 at 1 (lower)
    np.testing.assert_array_equal(O.select_anchors(sc, 1), [0])
    sc[0] = 100.0                                                       # entry 0 never counted twice
    np.testing.assert_array_equal(O.select_anchors(sc, 2), [0, 4])


def test_farthest_first_on_a_line():
    """Points 0, 1, ..., 10 on a line, starting from {0}: 10 is farthest (100); then 5
    (25 to both ends); then 2, 3, 7 and 8 tie at 4 and the lower index 2 wins; then 7 and 8
    tie at 4 and 7 wins (worked by hand below)."""
    K = np.arange(11.0)[:, None]
    seq = O.farthest_first(K, [0], 5)
    # after {0, 10, 5}: mindists 1:1 2:4 3:4 4:1 6:1 7:4 8:4 9:1 -> first max index 2
    # after {0, 10, 5, 2}: 3:1 7:4 8:4 -> 7
    np.testing.assert_array_equal(seq, [0, 10, 5, 2, 7])


def _loop_fft(K, start, M):
    seq = list(start)
    while len(seq) < M:
        best, bi = -1.0, -1
        for i in range(len(K)):
            if i in seq:
                continue
            dmin = min(float(((K[i] - K[j]) ** 2).sum()) for j in seq)
            if dmin > best:
                best, bi = dmin, i
        seq.append(bi)
    return seq


def test_farthest_first_bruteforce_and_radius_monotone():
    rng = np.random.default_rng(31)
    K = rng.standard_normal((40, 5))
    seq = O.farthest_first(K, [0, 7], 15)
    np.testing.assert_array_equal(seq, _loop_fft(K, [0, 7], 15))
    # the distance of each newly added key to the set never increases (Gonzalez)
    radii = [min(((K[seq[s]] - K[j]) ** 2).sum() for j in seq[:s]) for s in range(2, 15)]
    assert all(a >= b - 1e-12 for a, b in zip(radii, radii[1:]))


def test_anchor_diverse_init_budget():
    rng = np.random.default_rng(32)
    Q, K, V = _qkv(64, 64, 8, rng)
    seq, idx = O.anchor_diverse_init(Q, K, 16, 0.5, True, 1)
    assert seq.size == 16 and np.unique(seq).size == 16 and 0 in seq
    np.testing.assert_array_equal(idx, np.sort(seq))
    _, _, st = O.full_cache_stats(Q, K, V, 0.5, True, 1, want_O=False)
    np.testing.assert_array_equal(np.sort(seq[:4]), O.select_anchors(O.key_score(st, "max", 64), 4))


# --------------------------------------------------------------------------------------
# stage-1 attention fitting (Latent Compaction §3.3 Eq. 8, AdamW)
# --------------------------------------------------------------------------------------
def _stage1_case(rng, causal=True, group=2):
    T, d, t = 40, 6, 9
    n = group * T
    Q, K, V = _qkv(n, T, d, rng)
    lse, Of, _ = O.full_cache_stats(Q, K, V, 0.5, causal, group)
    keypos = np.sort(np.concatenate([[0], rng.choice(np.arange(1, T), t - 1, replace=False)]))
    return Q, K, V, lse, Of, keypos


@pytest.mark.parametrize("causal,group", [(True, 2), (False, 1)])
def test_stage1_gradient_matches_finite_differences(causal, group):
    rng = np.random.default_rng(41)
    Q, K, V, lse, Of, kp = _stage1_case(rng, causal, group)
    Ck = K[kp] + 0.1 * rng.standard_normal(K[kp].shape)
    Cv = V[kp] + 0.1 * rng.standard_normal(V[kp].shape)
    b = 0.3 * rng.standard_normal(kp.size)
    sa, sz = O.teacher_scales(Of, lse, group)
    rows = O.stage1_rows(rng.integers(0, Q.shape[0] // group, size=7), group)
    L, dCk, dCv, db = O.stage1_loss_grad(Q, rows, Ck, Cv, b, kp, Of, lse, sa, sz, 0.5, causal, group)
    h = 1e-6
    for X, dX in ((Ck, dCk), (Cv, dCv), (b, db)):
        for idx in [tuple(rng.integers(0, s) for s in X.shape) for _ in range(6)]:
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args = [Ck, Cv, b]
            which = [Ck is X, Cv is X, b is X].index(True)
            args_p, args_m = list(args), list(args)
            args_p[which], args_m[which] = Xp, Xm
            Lp = O.stage1_loss_grad(Q, rows, *args_p, kp, Of, lse, sa, sz, 0.5, causal, group)[0]
            Lm = O.stage1_loss_grad(Q, rows, *args_m, kp, Of, lse, sa, sz, 0.5, causal, group)[0]
            assert abs((Lp - Lm) / (2 * h) - dX[idx]) <= 1e-6 * (1 + abs(dX[idx]))


def test_stage1_loss_is_zero_on_the_full_cache():
    """With every key as a slot, the original values and zero biases, the compacted branch
    is the full cache: Eq. 8 is zero and so is its gradient."""
    rng = np.random.default_rng(42)
    Q, K, V, lse, Of, _ = _stage1_case(rng)
    kp = np.arange(K.shape[0])
    sa, sz = O.teacher_scales(Of, lse, 2)
    L, dCk, dCv, db = O.stage1_loss_grad(Q, np.arange(Q.shape[0]), K, V, np.zeros(kp.size), kp,
                                         Of, lse, sa, sz, 0.5, True, 2)
    assert L < 1e-24 and np.abs(dCk).max() < 1e-12 and np.abs(dCv).max() < 1e-12


def test_adamw_first_step_closed_form():
    """From zero moments the bias-corrected ratio is g / (|g| + eps): each coordinate moves
    by lr times its gradient's sign (after the decoupled decay)."""
    th = np.array([1.0, -2.0, 0.5])
    g = np.array([3.0, -1e-3, 0.0])
    new, m, v = O.adamw_step(th, g, np.zeros(3), np.zeros(3), 1, 1e-2, 0.1)
    ref = th * (1 - 1e-3) - 1e-2 * g / (np.abs(g) + 1e-8)
    np.testing.assert_allclose(new, ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(m, 0.1 * g)
    np.testing.assert_allclose(v, 0.001 * g * g)


def test_stage1_fit_lowers_the_loss_and_freezes():
    rng = np.random.default_rng(43)
    Q, K, V, lse, Of, kp = _stage1_case(rng)
    samples = rng.integers(0, Q.shape[0] // 2, size=(60, 16))
    frozen = np.zeros(kp.size, dtype=bool)
    frozen[[0, 3]] = True
    Ck, Cv, b, losses = O.stage1_fit(Q, K[kp], V[kp], np.zeros(kp.size), kp, Of, lse, samples,
                                     0.5, True, 2, lr=1e-2, trainable=~frozen)
    sa, sz = O.teacher_scales(Of, lse, 2)
    rows = np.arange(Q.shape[0])
    before = O.stage1_loss_grad(Q, rows, K[kp], V[kp], np.zeros(kp.size), kp, Of, lse, sa, sz,
                                0.5, True, 2)[0]
    after = O.stage1_loss_grad(Q, rows, Ck, Cv, b, kp, Of, lse, sa, sz, 0.5, True, 2)[0]
    assert after < 0.8 * before
    np.testing.assert_array_equal(Ck[frozen], K[kp][frozen])
    np.testing.assert_array_equal(b[frozen], 0.0)


# --------------------------------------------------------------------------------------
# hand-worked cases: teacher statistics, Eq. 8's averaging, the KKT checker
# --------------------------------------------------------------------------------------
def test_teacher_scales_hand_worked():
    """Two query heads (group 2, rows alternate heads). Head 0's outputs are the channel
    values {1, 3, 3, 5}: mean 3, population variance (4 + 0 + 0 + 4) / 4 = 2, std sqrt(2)
    (ddof = 1 would give sqrt(8/3)); its log-normalizers {0, 4} have population std 2
    (ddof = 1: 2 sqrt 2). Head 1 is constant in both, so both stds are 0 and the floor of
    1e-4 applies to the standard deviation itself (a floor on the variance would give
    1e-2). Pooling the heads would mix {1, 3, 3, 5} with {2, 2, 2, 2}."""
    O_full = np.array([[1.0, 3.0], [2.0, 2.0], [3.0, 5.0], [2.0, 2.0]])
    lse = np.array([0.0, 7.0, 4.0, 7.0])
    sa, sz = O.teacher_scales(O_full, lse, 2)
    np.testing.assert_allclose(sa, [np.sqrt(2.0), 1e-4], rtol=1e-15, atol=0)
    np.testing.assert_allclose(sz, [2.0, 1e-4], rtol=1e-15, atol=0)


def test_stage1_loss_hand_worked():
    """Eq. 8 on two rows, d = 2, one slot: with t = 1 the softmax is 1, so A = C_v for every
    row and log Z = scale k . q + b. Rows q0 = (1, 0), q1 = (0, 1); slot key (2, 0), value
    (1, 2), bias 0.5, scale 0.5: log Z = (1.5, 0.5). Targets O = ((0, 0), (1, 1)) and
    lse = (0.5, 0.5), with sa = 2 and sz = 0.5 given.
      output term: ((1/2)^2 + (2/2)^2 + 0^2 + (1/2)^2) / (N d = 4)  = 1.5 / 4  = 0.375
      log Z term:  ((1/0.5)^2 + 0^2) / (N = 2)                        = 4 / 2    = 2
      L = 2.375 (dividing the output term by N alone would give 2.75, summing the log Z
      term instead of averaging 4.375).
    Gradients: dL/db = (2 * 1 / 0.25 + 0) / 2 = 4; dL/dC_v = 2 / (sa^2 N d) * sum of the
    output errors = (1/8) * (1, 3); dL/dC_k = (2 * 1 / (0.25 * 2)) * scale * q0 = (2, 0)."""
    Q = np.array([[1.0, 0.0], [0.0, 1.0]])
    Ck = np.array([[2.0, 0.0]])
    Cv = np.array([[1.0, 2.0]])
    b = np.array([0.5])
    O_full = np.array([[0.0, 0.0], [1.0, 1.0]])
    lse = np.array([0.5, 0.5])
    L, dCk, dCv, db = O.stage1_loss_grad(Q, np.arange(2), Ck, Cv, b, np.zeros(1, np.int64),
                                         O_full, lse, np.array([2.0]), np.array([0.5]), 0.5)
    assert L == pytest.approx(2.375, rel=1e-15)
    np.testing.assert_allclose(db, [4.0], rtol=1e-15)
    np.testing.assert_allclose(dCv, [[0.125, 0.375]], rtol=1e-15)
    np.testing.assert_allclose(dCk, [[2.0, 0.0]], rtol=1e-15, atol=1e-15)


def test_kkt_residual_flags_non_optimal_points():
    """G = diag(2, 1), h = (2, 1): the optimum w = (1, 1) is interior. Hand-computed
    violations of g = G w - h:
      interior, w = (0.5, 1): g = (-1, 0), both free -> |g_0| = 1;
      lower bound, w = (0, 1): g = (-2, 0), w_0 at 0 needs g_0 >= 0 -> 2;
      lower bound met, h = (-2, 1), w = (0, 1): g = (2, 0) -> 0 (the optimum);
      upper bound hi = 0.5, w = (0.5, 0.5): g = (-1, -0.5), both at hi need g <= 0 -> 0;
      upper bound, h = (0.5, 0.2), w = (0.5, 0.5): g = (0.5, 0.3) at hi -> 0.5;
      infeasible, w = (1.25, 1) with hi = 1.2: outside the box by 0.05."""
    G = np.diag([2.0, 1.0])
    h = np.array([2.0, 1.0])
    assert O.nnls_kkt_residual(G, h, np.array([1.0, 1.0])) == 0.0
    assert O.nnls_kkt_residual(G, h, np.array([0.5, 1.0])) == pytest.approx(1.0, rel=1e-15)
    assert O.nnls_kkt_residual(G, h, np.array([0.0, 1.0])) == pytest.approx(2.0, rel=1e-15)
    assert O.nnls_kkt_residual(G, np.array([-2.0, 1.0]), np.array([0.0, 1.0])) == 0.0
    assert O.nnls_kkt_residual(G, h, np.array([0.5, 0.5]), 0.0, 0.5) == 0.0
    assert O.nnls_kkt_residual(G, np.array([0.5, 0.2]), np.array([0.5, 0.5]), 0.0, 0.5) == \
        pytest.approx(0.5, rel=1e-15)
    assert O.nnls_kkt_residual(G, np.array([2.5, 1.0]), np.array([1.25, 1.0]), 0.0, 1.2) == \
        pytest.approx(0.05, rel=1e-12)
    # a positive lower bound: w_0 sits at lo = 0.25 with g_0 = 0.5 - 2 < 0 -> 1.5
    assert O.nnls_kkt_residual(G, h, np.array([0.25, 1.0]), 0.25) == pytest.approx(1.5, rel=1e-15)


def test_output_residual_from_stats_equals_direct():
    """The expansion ||A C - Y||^2 = ||A C||^2 - 2 <C, A^T Y> + ||Y||^2 against the direct
    residual, for the optimum and for an arbitrary C."""
    rng = np.random.default_rng(71)
    A = np.abs(rng.standard_normal((300, 12)))
    A /= A.sum(axis=1, keepdims=True)
    Y = rng.standard_normal((300, 5))
    AtY, yy = O.value_fit_stats(A, Y)
    for C in (O.fit_values(A, Y, 1e-3), rng.standard_normal((12, 5))):
        assert O.output_residual_from_stats(A, C, AtY, yy) == \
            pytest.approx(O.output_residual(A, Y, C), rel=1e-10)
