"""Float64 CPU oracle for per-KV-head attention-matching KV compaction.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP path; both sides receive the same seeded inputs.

What is computed, per head problem (all arithmetic in float64; bf16 inputs are upcast
exactly before they arrive here):

  S1  full-cache statistics. Scores s_ij = scale * q_i . k_j over the keys visible to query
      i; lse_i = log sum_j exp(s_ij); O_i = sum_j exp(s_ij - lse_i) v_j.
      ("Latent Compaction with Test-Time Training", §3 Preliminaries, Eq. 1: attention
      output A(q) and normalizer Z(q); App. A.2 "Normalizer Computation and Storage":
      masked scores, logsumexp and softmax in a wider float type.)
  S2  per-key attention statistics of p_ij = exp(s_ij - lse_i): the column sum, sum of
      squares and maximum over queries. The selection score is the RMS over queries by
      default (same paper, App. A.3: the Attention Matching baseline uses RMS
      attention-based key selection); MEAN and MAX (Eq. 6) are options.
  S3  C_k = the t keys of highest score ("Compaction" blog, §Fast KV Compaction via
      Attention Matching, step 1; C_k is a subset of K). Ties go to the lower key index;
      indices are returned ascending because compacted entries keep their positions
      (Latent Compaction, §3.1 "Handling Subsequent Tokens": no renumbering).
  S4/S5  beta from the mass equations by non-negative least squares on w = exp(beta)
      (blog, §Choosing beta, mass-matching equation for every reference query). The
      default divides equation i by its full-cache mass Z_i, so the design entries are
      M_ij = p_{i, idx_j} and the target is 1; the literal (absolute) form is an option.
  S6/S7  C_v from the output equations by ridge least squares (blog, §Choosing C_v):
      A_i = softmax over the visible selected keys of (scale q_i . C_k + beta), and
      C_v = argmin ||A C - O||_F^2 + lambda ||C||_F^2.
  E   the compacted attention itself, to evaluate any (idx, beta, C_v): biased scores
      l(q) = scale K_cmp q + b (Latent Compaction §3.1, Eq. 2), output Eq. 3 and
      normalizer Z_cmp = 1^T exp(l) (Eq. 4), plus the residuals compared in parity.
  C   attention through a compacted cache followed by ordinary appended entries (Latent
      Compaction §3.1 Eq. 2-5; App. A.2, attention over a compacted cache plus new
      tokens): each entry set gives masked, biased scores (Eq. 2), a log-normalizer
      (Eq. 4) and an output (Eq. 3), and the two sets are merged by Eq. 5 in log space.
  F   the fast variants of the "Compaction" blog: beta by uniform redistribution of the
      missing mass (§Choosing beta) and direct values C_v = V[idx] (§Choosing C_v).
  I   anchor + diversifier initialization (Latent Compaction §3.2): anchors by maximum
      attention (Eq. 6) plus the first entry, diversifiers by farthest-first traversal
      (Eq. 7).
  G   stage-1 attention fitting (Latent Compaction §3.3, Eq. 8; App. A.2 sampling and
      AdamW): the compacted keys, values and biases move by AdamW on the standardized
      output and log-normalizer errors of sampled query positions.

Readings where the pages are silent (each is listed with its reason in the design notes):
masked entries are excluded (weight exp(-inf) = 0), and an entry set a row cannot see
at all has log Z = -inf and takes no weight in Eq. 5 (key 0 is visible to every query of
the full cache, so its rows always see one); the RMS divisor is n for every key; w_j = 0 gives beta_j = -inf; a query with no visible
selected key contributes a zero row to A; lambda is absolute on the summed normal
equations; natural log/exp throughout, with the 1/sqrt(d) scale applied to q.k.

Parity pins live in tests/test_oracle_*.py. The weights w themselves are parity unpinned
on rank-deficient designs (the minimiser is not unique there; the fitted mass vector Mw
is, and that is what is pinned and compared).
"""
from __future__ import annotations

import numpy as np
import scipy.linalg
import scipy.optimize
import scipy.special

SCORE_MODES = ("rms", "mean", "max")
MASS_MODES = ("relative", "absolute")


# --------------------------------------------------------------------------------------
# visibility
# --------------------------------------------------------------------------------------
def visible(rows: np.ndarray, keys: np.ndarray, causal: bool, group: int) -> np.ndarray:
    """Boolean [len(rows), len(keys)]: key position keys[j] is visible to query rows[i].

    Causal workloads place query i at position i // group (group = query heads per KV
    head, queries ordered position-major) and let it see keys at positions <= its own
    (Latent Compaction §3 Preliminaries: the index set I of causally visible entries).
    """
    rows = np.asarray(rows)
    keys = np.asarray(keys)
    if not causal:
        return np.ones((rows.size, keys.size), dtype=bool)
    return keys[None, :] <= (rows // group)[:, None]


def _chunks(n: int, T: int, budget: int = 1 << 24):
    step = max(1, min(n, budget // max(T, 1)))
    for a in range(0, n, step):
        yield a, min(n, a + step)


# --------------------------------------------------------------------------------------
# S1 + S2: full-cache statistics
# --------------------------------------------------------------------------------------
def full_cache_stats(Q, K, V, scale, causal=False, group=1, want_O=True, rows=None,
                     keypos=None):
    """lse [n], O [n, d] (or None) and per-key (sum p, sum p^2, max p) over queries.

    Q [n, d], K and V [T, d], all float64. p_ij = exp(s_ij - lse_i) for visible pairs, 0
    otherwise. Queries are processed in chunks only to bound memory. `rows` gives the
    query indices (positions) of the rows of Q when Q is a subset of a problem's queries;
    `keypos` the original positions of the rows of K when K is a subset of the keys.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    n, T = Q.shape[0], K.shape[0]
    lse = np.empty(n)
    O = np.empty((n, V.shape[1])) if want_O else None
    colsum = np.zeros(T)
    colsq = np.zeros(T)
    colmax = np.zeros(T)
    keys = np.arange(T) if keypos is None else np.asarray(keypos)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    for a, b in _chunks(n, T):
        s = scale * (Q[a:b] @ K.T)
        vis = visible(rows[a:b], keys, causal, group)
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1)
        m = np.where(np.isfinite(m), m, 0.0)   # a row that sees no key: lse = -inf, p = 0
        with np.errstate(divide="ignore"):
            lse[a:b] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
        p = np.where(vis, np.exp(s - np.where(np.isfinite(lse[a:b]), lse[a:b], 0.0)[:, None]), 0.0)
        if want_O:
            O[a:b] = p @ V
        colsum += p.sum(axis=0)
        colsq += (p * p).sum(axis=0)
        np.maximum(colmax, p.max(axis=0), out=colmax)
    return lse, O, (colsum, colsq, colmax)


def attention_rows(Q, K, V, scale, rows, causal=False, group=1):
    """lse and O for selected query rows only (used to sample large problems)."""
    rows = np.asarray(rows)
    s = scale * (np.asarray(Q, np.float64)[rows] @ np.asarray(K, np.float64).T)
    s = np.where(visible(rows, np.arange(K.shape[0]), causal, group), s, -np.inf)
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    O = np.exp(s - lse[:, None]) @ np.asarray(V, np.float64)
    return lse, O


def key_score(stats, mode: str, n: int) -> np.ndarray:
    """Selection statistic per key: RMS (default), MEAN or MAX of p over the n queries."""
    colsum, colsq, colmax = stats
    if mode == "rms":
        return np.sqrt(colsq / n)
    if mode == "mean":
        return colsum / n
    if mode == "max":
        return colmax.copy()
    raise ValueError(mode)


# --------------------------------------------------------------------------------------
# S3: top-t selection
# --------------------------------------------------------------------------------------
def select_top(score: np.ndarray, t: int) -> np.ndarray:
    """Indices of the t largest scores (ties -> lower index), returned ascending."""
    score = np.asarray(score)
    order = np.lexsort((np.arange(score.size), -score))
    return np.sort(order[:t]).astype(np.int64)


# --------------------------------------------------------------------------------------
# S4: the mass design
# --------------------------------------------------------------------------------------
def mass_design(Q, Ck, idx, lse, scale, causal=False, group=1, mode="relative", rows=None):
    """Design matrix M [n, t] and target b [n] of the mass equations.

    Mass equation for query i: sum_j exp(s_i,c_j + beta_j) ~= Z_i (blog, §Choosing beta).
    relative: divide by Z_i  -> M_ij = exp(s_i,c_j - lse_i), b_i = 1.
    absolute: divide by exp(c), c = max_i lse_i -> M_ij = exp(s_i,c_j - c), b_i = exp(lse_i - c).
    Compacted keys keep their positions, so the causal mask uses idx. `rows` gives the query
    indices of the rows of Q when Q is a subset of a problem's queries.
    """
    Q = np.asarray(Q, np.float64)
    s = scale * (Q @ np.asarray(Ck, np.float64).T)
    rows = np.arange(Q.shape[0]) if rows is None else np.asarray(rows)
    vis = visible(rows, np.asarray(idx), causal, group)
    if mode == "relative":
        M = np.where(vis, np.exp(np.where(vis, s, 0.0) - lse[:, None]), 0.0)
        b = np.ones(Q.shape[0])
    elif mode == "absolute":
        c = lse.max()
        M = np.where(vis, np.exp(np.where(vis, s, 0.0) - c), 0.0)
        b = np.exp(lse - c)
    else:
        raise ValueError(mode)
    return M, b


# --------------------------------------------------------------------------------------
# S5: non-negative least squares
# --------------------------------------------------------------------------------------
def nnls_gram(G: np.ndarray, h: np.ndarray, tol: float | None = None):
    """Lawson-Hanson active-set NNLS on the normal equations.

    Minimises f(w) = 1/2 w^T G w - h^T w over w >= 0, where G = M^T M and h = M^T b, which
    is 1/2 ||M w - b||^2 up to a constant. The passive set P holds the free variables;
    each outer step frees the variable with the largest dual u_j = (h - G w)_j, and the
    inner loop steps toward the unconstrained minimiser on P, dropping variables that
    reach zero, until that minimiser is strictly positive.
    """
    G = np.asarray(G, np.float64)
    h = np.asarray(h, np.float64)
    t = h.size
    if tol is None:
        tol = 1e-12 * max(1.0, float(np.abs(h).max())) * max(1.0, float(np.abs(np.diag(G)).max()))
    # An interior optimum: if the unconstrained minimiser is strictly positive it is feasible,
    # hence optimal for the constrained problem too (the KKT conditions hold with every
    # variable free). Verified, not assumed.
    try:
        z = scipy.linalg.cho_solve(scipy.linalg.cho_factor(G, lower=True, check_finite=False), h,
                                   check_finite=False)
        if np.all(np.isfinite(z)) and np.all(z > 0) and nnls_kkt_residual(G, h, z) <= tol * 1e3:
            return z
    except np.linalg.LinAlgError:
        pass
    w = np.zeros(t)
    P = np.zeros(t, dtype=bool)
    barred = np.zeros(t, dtype=bool)
    u = h - G @ w
    for _ in range(4 * t + 10):
        cand = (~P) & (~barred) & (u > tol)
        if not cand.any():
            break
        j = int(np.argmax(np.where(cand, u, -np.inf)))
        P[j] = True
        for _inner in range(4 * t + 10):
            ip = np.flatnonzero(P)
            z = np.zeros(t)
            z[ip] = _spd_solve(G[np.ix_(ip, ip)], h[ip])
            if np.all(z[ip] > 0):
                w = z
                break
            neg = ip[z[ip] <= 0]
            alpha = np.min(w[neg] / (w[neg] - z[neg]))
            w = w + alpha * (z - w)
            drop = P & (w <= 1e-300)
            drop[neg[np.argmin(w[neg] / (w[neg] - z[neg]))]] = True
            P &= ~drop
            w[~P] = 0.0
            if not P.any():
                break
        u = h - G @ w
        # a freed variable that could not stay positive is numerically dependent
        if not P[j]:
            barred[j] = True
        else:
            barred[:] = False
    return w


def _spd_solve(A, b):
    try:
        c = scipy.linalg.cho_factor(A, lower=True, check_finite=False)
        x = scipy.linalg.cho_solve(c, b, check_finite=False)
        if np.all(np.isfinite(x)):
            return x
    except np.linalg.LinAlgError:
        pass
    return np.linalg.lstsq(A, b, rcond=None)[0]


def nnls_box(M, b, lo: float, hi: float):
    """Bounded least squares min ||M w - b|| over lo <= w <= hi (textbook BVLS)."""
    r = scipy.optimize.lsq_linear(M, b, bounds=(lo, hi), method="bvls", tol=1e-14,
                                  max_iter=10 * M.shape[1] + 100)
    return r.x


def fit_beta(M, b, lo: float = 0.0, hi: float = np.inf):
    """w = argmin_{lo<=w<=hi} ||M w - b||^2 and beta = log w (w = 0 -> -inf)."""
    if lo == 0.0 and np.isinf(hi):
        G = M.T @ M
        h = M.T @ b
        w = nnls_gram(G, h)
    else:
        w = nnls_box(M, b, lo, hi)
    with np.errstate(divide="ignore"):
        beta = np.log(w)
    return w, beta


def nnls_kkt_residual(G, h, w, lo: float = 0.0, hi: float = np.inf) -> float:
    """Largest violation of the box-NNLS optimality conditions, g = G w - h.

    Free variables need g_j = 0; variables at the lower bound need g_j >= 0; variables at
    the upper bound need g_j <= 0; and lo <= w <= hi.
    """
    g = G @ w - h
    atlo = w <= lo + 1e-300 if lo == 0 else np.isclose(w, lo, rtol=1e-12, atol=0)
    athi = np.isfinite(hi) & np.isclose(w, hi, rtol=1e-12, atol=0)
    free = ~atlo & ~athi
    v = 0.0
    if free.any():
        v = max(v, float(np.abs(g[free]).max()))
    if atlo.any():
        v = max(v, float(np.maximum(-g[atlo], 0).max()))
    if np.any(athi):
        v = max(v, float(np.maximum(g[athi], 0).max()))
    v = max(v, float(np.maximum(lo - w, 0).max()), float(np.maximum(w - hi, 0).max()))
    return v


# --------------------------------------------------------------------------------------
# S6 + S7: the value fit
# --------------------------------------------------------------------------------------
def value_design(M, w):
    """A_i = (w * M_i) / (M_i . w): the compacted softmax weights with beta = log w.

    Rows with no visible selected key of positive weight are zero.
    """
    Dm = M @ w
    num = M * w[None, :]
    A = np.zeros_like(M)
    ok = Dm > 0
    A[ok] = num[ok] / Dm[ok, None]
    return A


def fit_values(A, Y, lam: float):
    """C_v = (A^T A + lam I)^{-1} A^T Y by Cholesky and two triangular solves."""
    t = A.shape[1]
    G = A.T @ A + lam * np.eye(t)
    R = A.T @ Y
    c = scipy.linalg.cho_factor(G, lower=True)
    return scipy.linalg.cho_solve(c, R)


# --------------------------------------------------------------------------------------
# E: compacted attention and residuals
# --------------------------------------------------------------------------------------
def compacted_attention(Q, Ck, idx, beta, Cv, scale, causal=False, group=1):
    """log Z_cmp [n] and A_cmp [n, d] of the biased compacted cache (Eq. 2-4)."""
    Q = np.asarray(Q, np.float64)
    l = scale * (Q @ np.asarray(Ck, np.float64).T) + np.asarray(beta, np.float64)[None, :]
    vis = visible(np.arange(Q.shape[0]), np.asarray(idx), causal, group)
    l = np.where(vis, l, -np.inf)
    m = l.max(axis=1)
    fin = np.isfinite(m)
    logz = np.full(Q.shape[0], -np.inf)
    A = np.zeros((Q.shape[0], np.asarray(Cv).shape[1]))
    if fin.any():
        lf = l[fin] - m[fin, None]
        e = np.exp(lf)
        z = e.sum(axis=1)
        logz[fin] = m[fin] + np.log(z)
        A[fin] = (e / z[:, None]) @ np.asarray(Cv, np.float64)
    return logz, A


# --------------------------------------------------------------------------------------
# C: cache attention with appended entries, and the log-space combination
# --------------------------------------------------------------------------------------
def biased_scores(Q, keys, bias, valid, scale):
    """Eq. 2 with the entry mask: l_ij = scale * q_i . k_j + bias_j where valid[i, j], and
    -inf (excluded) elsewhere. bias None means an unbiased set of entries."""
    l = scale * (np.asarray(Q, np.float64) @ np.asarray(keys, np.float64).T)
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return np.where(np.broadcast_to(valid, l.shape), l, -np.inf)


def log_normalizer(l):
    """Eq. 4 in log form: log Z_i = log sum_j exp(l_ij) over the entries that are not
    -inf; a row with none gets -inf (scipy's logsumexp, which returns -inf there)."""
    return scipy.special.logsumexp(l, axis=1)


def attention_output(l, logz, values):
    """Eq. 3: A_i = sum_j exp(l_ij - log Z_i) v_j; a row with log Z = -inf is zero."""
    out = np.zeros((l.shape[0], np.asarray(values).shape[1]))
    fin = np.isfinite(logz)
    if fin.any():
        out[fin] = np.exp(l[fin] - logz[fin, None]) @ np.asarray(values, np.float64)
    return out


def merge_log_space(out1, logz1, out2, logz2):
    """Eq. 5 for two disjoint entry sets, weighted in log space: log Z = log(Z1 + Z2) and
    A = (Z1 A1 + Z2 A2) / (Z1 + Z2). A set whose log Z is -inf takes no weight; rows where
    both are -inf keep -inf and a zero output."""
    logz = np.logaddexp(logz1, logz2)
    out = np.zeros_like(np.asarray(out1, np.float64))
    fin = np.isfinite(logz)
    w1 = np.exp(logz1[fin] - logz[fin])
    w2 = np.exp(logz2[fin] - logz[fin])
    out[fin] = w1[:, None] * out1[fin] + w2[:, None] * out2[fin]
    return out, logz


def cache_attention(Q, Ck, Cv, bias, scale, keypos=None, nvalid=None, causal=False, group=1,
                    Kn=None, Vn=None, new_causal=True, rows=None):
    """Attention of queries Q through a compacted cache (Ck, Cv, bias) and optional new
    entries (Kn, Vn) appended after it.

    Document slot j is valid when j < nvalid and, for causal problems, when its original
    position keypos[j] <= i // group. New entry j is visible to query i when
    j <= i // group (new_causal) or always. `rows` gives the query indices of the rows of Q
    when Q is a subset. Returns (out [n, d], log Z [n], log Z_cmp [n]).
    """
    n = np.asarray(Q).shape[0]
    t = np.asarray(Ck).shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    slots = np.arange(t)
    valid = np.ones((n, t), dtype=bool)
    if nvalid is not None:
        valid &= (slots < nvalid)[None, :]
    if causal:
        valid &= visible(rows, np.asarray(keypos), True, group)
    l1 = biased_scores(Q, Ck, bias, valid, scale)           # document slots (Eq. 2)
    lz1 = log_normalizer(l1)                                 # Eq. 4
    out1 = attention_output(l1, lz1, Cv)                     # Eq. 3
    if Kn is None or np.asarray(Kn).shape[0] == 0:
        return out1, lz1.copy(), lz1
    m = np.asarray(Kn).shape[0]
    nvis = visible(rows, np.arange(m), bool(new_causal), group)
    l2 = biased_scores(Q, Kn, None, nvis, scale)            # appended entries, no bias
    lz2 = log_normalizer(l2)
    out2 = attention_output(l2, lz2, Vn)
    out, lz = merge_log_space(out1, lz1, out2, lz2)          # Eq. 5
    return out, lz, lz1


# --------------------------------------------------------------------------------------
# F: fast variants (no fits)
# --------------------------------------------------------------------------------------
def redistribute_beta(Q, Ck, idx, lse, scale, causal=False, group=1):
    """beta by uniform redistribution of the missing mass ("Compaction" blog, §Choosing beta).

    m_j   = (1/n) sum_i exp(s_{i, c_j}) over the queries that see c_j,
    Delta = (1/n) sum_i [Z_i - sum_j exp(s_{i, c_j})] with Z_i = exp(lse_i) the mass of
            query i over the reference key set (the full cache, or a shortlist),
    beta_j = log((m_j + Delta / t) / m_j).
    Every selected key receives the same share Delta / t of the mass the compacted keys miss.
    """
    Q = np.asarray(Q, np.float64)
    lse = np.asarray(lse, np.float64)
    n, t = Q.shape[0], np.asarray(Ck).shape[0]
    c = lse.max()   # common factor e^c of every mass; beta does not depend on it
    e = np.zeros((n, t))
    for a, b in _chunks(n, t):
        s = scale * (Q[a:b] @ np.asarray(Ck, np.float64).T)
        vis = visible(np.arange(a, b), np.asarray(idx), causal, group)
        e[a:b] = np.where(vis, np.exp(np.where(vis, s, 0.0) - c), 0.0)
    m = e.sum(axis=0) / n
    # Delta is a mass (the compacted keys are a subset of the reference set): a negative
    # value can only be rounding, and is taken as 0
    delta = max((np.exp(lse - c).sum() - e.sum()) / n, 0.0)
    return np.log((m + delta / t) / m)


def select_two_pass(Q, K, sub, t, k_mult, scale, causal=False, group=1, mode="rms"):
    """Two-pass key selection ("Compaction" blog, §Choosing C_k, Attempt #3).

    Pass 1 scores every key against the query subset `sub` (ascending query indices; the
    statistic's divisor is the subset size) and keeps the k_mult * t best keys as a
    shortlist (all T if fewer). Pass 2 scores the shortlist against all n queries, with
    each query's softmax normalized over the shortlist keys it sees, and keeps the t best.
    Returns (idx [t] ascending original key indices, lse over the shortlist [n]).
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    n, T = Q.shape[0], K.shape[0]
    sub = np.asarray(sub)
    _, _, st1 = full_cache_stats(Q[sub], K, K, scale, causal, group, want_O=False, rows=sub)
    short = select_top(key_score(st1, mode, sub.size), min(k_mult * t, T))
    lse_s, _, st2 = full_cache_stats(Q, K[short], K[short], scale, causal, group, want_O=False,
                                     keypos=short)
    loc = select_top(key_score(st2, mode, n), t)
    return short[loc], lse_s


def select_anchors(score, n_anchor):
    """Anchors (Latent Compaction §3.2 "Budget Allocation"): the first document entry and the
    n_anchor - 1 highest-scoring remaining entries (ties to the lower index), ascending.
    `score` is the maximum teacher attention of Eq. 6 (key_score "max")."""
    score = np.asarray(score, np.float64)
    if n_anchor <= 1:
        return np.array([0], dtype=np.int64)[:max(n_anchor, 0)]
    rest = np.arange(1, score.size)
    order = rest[np.lexsort((rest, -score[1:]))]
    return np.sort(np.concatenate([[0], order[: n_anchor - 1]])).astype(np.int64)


def farthest_first(K, start, M):
    """Farthest-first traversal (Latent Compaction §3.2, Eq. 7; Gonzalez 1985): starting from
    the index set `start`, repeatedly add the key i not yet chosen that maximizes
    min_{j chosen} ||k_i - k_j||^2 (ties to the lower index) until M keys are chosen.
    Returns the chosen indices in order (start first, in the given order)."""
    K = np.asarray(K, np.float64)
    seq = [int(j) for j in start]
    chosen = np.zeros(K.shape[0], dtype=bool)
    chosen[seq] = True
    dist = np.full(K.shape[0], np.inf)
    for j in seq:
        dist = np.minimum(dist, ((K - K[j]) ** 2).sum(axis=1))
    while len(seq) < min(M, K.shape[0]):
        cand = np.where(chosen, -np.inf, dist)
        j = int(np.argmax(cand))       # first index of the maximum
        seq.append(j)
        chosen[j] = True
        dist = np.minimum(dist, ((K - K[j]) ** 2).sum(axis=1))
    return np.array(seq, dtype=np.int64)


def anchor_diverse_init(Q, K, M, scale, causal=False, group=1, n_anchor=None):
    """Anchor + diversifier initialization of an M-slot budget: M / 4 anchors (at least
    the first entry) by Eq. 6, the rest by farthest-first traversal (Eq. 7) from them.
    Returns (order of selection, indices ascending)."""
    n_anchor = max(1, M // 4) if n_anchor is None else n_anchor
    _, _, st = full_cache_stats(Q, K, K, scale, causal, group, want_O=False)
    anchors = select_anchors(key_score(st, "max", np.asarray(Q).shape[0]), n_anchor)
    seq = farthest_first(K, anchors, M)
    return seq, np.sort(seq)


def teacher_scales(O_full, lse_full, group):
    """Per query head g (rows i with i % group == g): the population standard deviation of
    the full-cache outputs over positions and channels, and of the log-normalizers over
    positions, each floored at 1e-4 (Latent Compaction §3.3: fixed teacher statistics).
    The means cancel in Eq. 8's differences and are not needed."""
    O_full = np.asarray(O_full, np.float64)
    lse_full = np.asarray(lse_full, np.float64)
    g = np.arange(O_full.shape[0]) % group
    sa = np.array([max(O_full[g == q].std(), 1e-4) for q in range(group)])
    sz = np.array([max(lse_full[g == q].std(), 1e-4) for q in range(group)])
    return sa, sz


def stage1_rows(positions, group):
    """The query rows of sampled positions: every query head of each position."""
    positions = np.asarray(positions, dtype=np.int64)
    return (positions[:, None] * group + np.arange(group)[None, :]).ravel()


def stage1_loss_grad(Q, rows, Ck, Cv, b, keypos, O_full, lse_full, sa, sz, scale, causal=False,
                     group=1):
    """Eq. 8 on the query rows `rows` and its gradient with respect to (Ck, Cv, b).

    A = softmax(l) Cv and log Z = logsumexp(l) with l = scale Ck q + b over the visible
    slots (Eq. 2-4); L = mean over rows and channels of ((A - A_full) / sa_g)^2 + mean over
    rows of ((log Z - log Z_full) / sz_g)^2, g the row's query head. Rows that see no slot
    are left out of both means. Returns (L, dCk, dCv, db)."""
    Q = np.asarray(Q, np.float64)[rows]
    Ck = np.asarray(Ck, np.float64)
    Cv = np.asarray(Cv, np.float64)
    b = np.asarray(b, np.float64)
    Y = np.asarray(O_full, np.float64)[rows]
    lz_t = np.asarray(lse_full, np.float64)[rows]
    g = np.asarray(rows) % group
    vis = visible(np.asarray(rows), np.asarray(keypos), causal, group)
    keep = vis.any(axis=1)
    Q, Y, lz_t, g, vis = Q[keep], Y[keep], lz_t[keep], g[keep], vis[keep]
    N, d = Q.shape[0], Cv.shape[1]
    s = np.where(vis, scale * Q @ Ck.T + b[None, :], -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    P = e / z
    lz = (m + np.log(z))[:, 0]
    A = P @ Cv
    wa = 1.0 / sa[g] ** 2
    wz = 1.0 / sz[g] ** 2
    L = float((wa[:, None] * (A - Y) ** 2).sum() / (N * d) + (wz * (lz - lz_t) ** 2).sum() / N)
    dA = 2.0 * wa[:, None] * (A - Y) / (N * d)
    dlz = 2.0 * wz * (lz - lz_t) / N
    dCv = P.T @ dA
    dP = dA @ Cv.T
    dS = P * (dP - (dA * A).sum(axis=1, keepdims=True) + dlz[:, None])
    db = dS.sum(axis=0)
    dCk = scale * dS.T @ Q
    return L, dCk, dCv, db


def adamw_step(theta, grad, m, v, step, lr, wd, beta1=0.9, beta2=0.999, eps=1e-8):
    """One AdamW update (decoupled weight decay first), step counted from 1. Returns the new
    (theta, m, v)."""
    m = beta1 * m + (1.0 - beta1) * grad
    v = beta2 * v + (1.0 - beta2) * grad * grad
    mh = m / (1.0 - beta1 ** step)
    vh = v / (1.0 - beta2 ** step)
    theta = theta * (1.0 - lr * wd) - lr * mh / (np.sqrt(vh) + eps)
    return theta, m, v


def stage1_fit(Q, Ck, Cv, b, keypos, O_full, lse_full, samples, scale, causal=False, group=1,
               lr=3e-3, wd=1e-2, trainable=None):
    """Stage-1 attention fitting: for each row of `samples` (sampled positions of one update),
    Eq. 8's gradient on those positions' query rows and one AdamW update of the trainable
    slots' keys, values and biases (frozen slots keep theirs). Returns (Ck, Cv, b, losses)."""
    sa, sz = teacher_scales(O_full, lse_full, group)
    params = [np.asarray(x, np.float64).copy() for x in (Ck, Cv, b)]
    mom = [np.zeros_like(x) for x in params]
    vel = [np.zeros_like(x) for x in params]
    t = params[0].shape[0]
    mask = np.ones(t, dtype=bool) if trainable is None else np.asarray(trainable, dtype=bool)
    losses = []
    for k, pos in enumerate(samples, start=1):
        L, *grads = stage1_loss_grad(Q, stage1_rows(pos, group), *params, keypos, O_full,
                                     lse_full, sa, sz, scale, causal, group)
        losses.append(L)
        for i in range(3):
            th, mm, vv = adamw_step(params[i], grads[i], mom[i], vel[i], k, lr, wd)
            sel = mask if params[i].ndim == 1 else mask[:, None]
            params[i] = np.where(sel, th, params[i])
            mom[i] = np.where(sel, mm, mom[i])
            vel[i] = np.where(sel, vv, vel[i])
    return params[0], params[1], params[2], np.array(losses)


def direct_values(V, idx):
    """C_v = V[idx] as float64 (blog, §Choosing C_v: the selected keys keep their values)."""
    return np.asarray(V, np.float64)[np.asarray(idx)]


def residuals(lse, O, logz_cmp, A_cmp):
    """R_mass = mean_i (Z_cmp,i / Z_i - 1)^2 and R_out = sum ||A_cmp - O||^2 / sum ||O||^2."""
    ratio = np.exp(logz_cmp - lse)
    r_mass = float(np.mean((ratio - 1.0) ** 2))
    r_out = float(((A_cmp - O) ** 2).sum() / (O ** 2).sum())
    return r_mass, r_out


def mass_residual(M, b, w) -> float:
    """||M w - b||^2 / n for the relative design (b = 1) or the absolute one."""
    r = M @ w - b
    return float(r @ r / M.shape[0])


def output_residual(A, Y, Cv) -> float:
    """||A C_v - Y||_F^2 / ||Y||_F^2."""
    R = A @ Cv - Y
    return float((R * R).sum() / (Y * Y).sum())


def value_fit_stats(A, Y):
    """(A^T Y, ||Y||_F^2): what the output residual of any C_v needs besides A itself, since
    ||A C - Y||^2 = ||A C||^2 - 2 <C, A^T Y> + ||Y||^2. Lets a large problem's targets Y be
    summarized once instead of kept."""
    Y = np.asarray(Y, np.float64)
    return np.asarray(A, np.float64).T @ Y, float((Y * Y).sum())


def output_residual_from_stats(A, Cv, AtY, yy) -> float:
    """The output residual ||A C_v - Y||_F^2 / ||Y||_F^2 from value_fit_stats(A, Y)."""
    AC = np.asarray(A, np.float64) @ np.asarray(Cv, np.float64)
    return float(((AC * AC).sum() - 2.0 * (np.asarray(Cv, np.float64) * AtY).sum() + yy) / yy)


# --------------------------------------------------------------------------------------
# the whole per-head pipeline
# --------------------------------------------------------------------------------------
def fit_selected(Q, K, lse, O, idx, scale, causal=False, group=1, mass="relative", w_lo=0.0,
                 w_hi=np.inf, ridge_lambda=1e-3, rows=None):
    """S4..S7 on a given key set: the mass design and beta (NNLS on w), then the value
    design and C_v (ridge), with both residuals. lse and O are the full-cache targets of
    the rows of Q (query indices `rows` when Q is a subset of a problem's queries)."""
    Q = np.asarray(Q, np.float64)
    idx = np.asarray(idx, np.int64)
    Ck = np.asarray(K, np.float64)[idx]
    M, b = mass_design(Q, Ck, idx, lse, scale, causal, group, mass, rows)
    w, beta = fit_beta(M, b, w_lo, w_hi)
    A = value_design(M, w)
    Cv = fit_values(A, O, ridge_lambda)
    return dict(idx=idx, Ck=Ck, M=M, b=b, w=w, beta=beta, A=A, Cv=Cv,
                r_mass=mass_residual(M, b, w), r_out=output_residual(A, O, Cv))


def compact_head(Q, K, V, t, scale, causal=False, group=1, score="rms", mass="relative",
                 w_lo=0.0, w_hi=np.inf, ridge_lambda=1e-3, idx=None):
    """S1..S7 for one head. Returns a dict with every intermediate the parity tests use.

    If idx is given, selection is skipped and the fits run on that key set.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n = Q.shape[0]
    lse, O, stats = full_cache_stats(Q, K, V, scale, causal, group)
    sc = key_score(stats, score, n)
    if idx is None:
        idx = select_top(sc, t)
    r = fit_selected(Q, K, lse, O, idx, scale, causal, group, mass, w_lo, w_hi, ridge_lambda)
    r.update(lse=lse, O=O, stats=stats, score=sc)
    return r
