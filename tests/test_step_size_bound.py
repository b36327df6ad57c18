"""The NNLS kernels take their step size 1/L from a Collatz-Wielandt bound: for a matrix A
with no negative entry and any positive vector u, max_i (A u)_i / u_i is at least A's
largest eigenvalue. The kernels form A = D^-1 G D^-1 from the Gram G = M^T M of a
nonnegative design (D = sqrt(diag G), empty rows left at zero), start u at all ones, take
two steps u <- A u + 2^-10 u and use the ratio bound of the third product times 1 + 2^-10.
This checks that rule, as written here in float64, against the largest eigenvalue on the
matrices it can meet: Grams of random nonnegative designs (with empty columns, a duplicated
column, a dominant rank-one part, an identity-like one), so that a step size below
1 / lambda_max cannot come out of it."""
import numpy as np
import pytest


def cw_bound(G):
    d = np.sqrt(np.diag(G))
    di = np.where(d > 0, 1.0 / np.where(d > 0, d, 1.0), 0.0)
    A = di[:, None] * G * di[None, :]
    u = np.ones(G.shape[0])
    for _ in range(2):
        u = A @ u + 2.0 ** -10 * u
    return (A @ u / u).max() * (1 + 2.0 ** -10), A


def designs():
    rng = np.random.default_rng(11)
    yield "random", rng.random((400, 60))
    M = rng.random((300, 50))
    M[:, [3, 17, 40]] = 0.0                       # keys no query gives weight
    yield "empty_columns", M
    M = rng.random((200, 30))
    M[:, 7] = M[:, 2]                             # a duplicated key
    yield "duplicate_column", M
    x = rng.random(500)
    yield "rank_one_dominant", np.outer(x, rng.random(40)) + 1e-3 * rng.random((500, 40))
    M = np.eye(64) + 1e-6 * rng.random((64, 64))  # nearly orthogonal columns
    yield "nearly_orthogonal", M
    # softmax-like rows: most mass on one column per row (the attention designs)
    S = rng.normal(size=(800, 80)) * 3.0
    P = np.exp(S - S.max(axis=1, keepdims=True))
    yield "softmax_rows", P / P.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("name,M", list(designs()), ids=[n for n, _ in designs()])
def test_step_size_bound_covers_the_largest_eigenvalue(name, M):
    G = M.T @ M
    L, A = cw_bound(G)
    lam = np.linalg.eigvalsh(A)[-1]
    assert L >= lam * (1 - 1e-12), (L, lam)
    # and it is a usable step size, not a loose one (the kernels' steps would slow down)
    assert L <= 2.0 * lam, (L, lam)


def test_step_size_bound_is_exact_for_a_diagonal_gram():
    G = np.diag(np.arange(1.0, 9.0))              # scaled to the identity: lambda_max = 1
    L, _ = cw_bound(G)
    assert L == pytest.approx(1 + 2.0 ** -10, rel=1e-12)
