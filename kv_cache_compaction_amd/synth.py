"""Seeded synthetic inputs for the compaction path (random draws and dtype rounding only).

This module holds none of the method's arithmetic: it draws keys, queries and values for
one head problem and rounds them to the input dtype. Tests, the benchmark and the smoke
check feed the same arrays to the HIP path and to the float64 checker.

Recipe per head problem (a stand-in for context-prefill queries and keys of a real model,
as the "Compaction" blog's §Speeding up Attention Matching describes them):
  * channel scales s_c ~ LogNormal(0, 0.5), one per head dimension;
  * keys K[j, c] = s_c * z, z ~ N(0, 1);
  * exactly floor(0.01 T) "needle" key rows, chosen without replacement, scaled x3; with
    ``extra_needles`` a further, disjoint floor(0.001 T) rows scaled x4;
  * exactly floor(n / 2) queries, chosen by a seeded permutation, are K[j] + N(0, 0.5^2)
    with j uniform over all T keys (also under a causal mask); the rest are N(0, 1);
  * values V ~ N(0, 1);
  * normals are drawn in float32 from numpy's PCG64 generator seeded with
    SeedSequence([SEED0, workload index, layer, doc, kv_head]);
  * bf16 workloads round the float32 draws to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np

from .configs import WORKLOADS, Workload

SEED0 = 20260212


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def workload_index(w: Workload) -> int:
    for i, x in enumerate(WORKLOADS):
        if x.name.split("_small")[0] == w.name.split("_small")[0]:
            return i
    return 99


def head_rng(w: Workload, h: int, seed0: int = SEED0) -> np.random.Generator:
    layer, doc, kv = w.seed_path(h)
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed0, workload_index(w), layer, doc, kv])))


def draw_head_f32(w: Workload, h: int, seed0: int = SEED0):
    """Q [n, d], K [T, d], V [T, d] as float32 draws for head problem h (before rounding)."""
    rng = head_rng(w, h, seed0)
    T, n, d = w.T, w.n, w.d
    s = rng.lognormal(0.0, 0.5, size=d).astype(np.float32)
    K = rng.standard_normal((T, d), dtype=np.float32) * s
    n_needle = int(0.01 * T)
    perm = rng.permutation(T)
    needles = perm[:n_needle]
    K[needles] *= np.float32(3.0)
    if w.extra_needles:
        n_extra = int(0.001 * T)
        K[perm[n_needle:n_needle + n_extra]] *= np.float32(4.0)
    Q = rng.standard_normal((n, d), dtype=np.float32)
    qperm = rng.permutation(n)
    kd = qperm[: n // 2]
    src = rng.integers(0, T, size=kd.size)
    Q[kd] = K[src] + np.float32(0.5) * rng.standard_normal((kd.size, d), dtype=np.float32)
    V = rng.standard_normal((T, d), dtype=np.float32)
    return Q, K, V


def make_head(w: Workload, h: int, seed0: int = SEED0):
    """Inputs of head problem h in the workload's dtype.

    Returns (Q, K, V) as float32 arrays for "f32" workloads, or as uint16 bf16 bit patterns
    for "bf16" workloads.
    """
    Q, K, V = draw_head_f32(w, h, seed0)
    if w.dtype == "bf16":
        return bf16_bits(Q), bf16_bits(K), bf16_bits(V)
    return Q, K, V


def make_batch(w: Workload, heads=None, seed0: int = SEED0):
    """Stacked inputs [h, rows, d] for the listed head problems (default: all)."""
    hs = range(w.heads) if heads is None else list(heads)
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    H = len(hs)
    Q = np.empty((H, w.n, w.d), dt)
    K = np.empty((H, w.T, w.d), dt)
    V = np.empty((H, w.T, w.d), dt)
    for i, h in enumerate(hs):
        Q[i], K[i], V[i] = make_head(w, h, seed0)
    return Q, K, V


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of generated inputs (bf16 bits are upcast exactly)."""
    if dtype == "bf16":
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def make_cache_case(seed: int, heads: int, n: int, T: int, t: int, m: int, d: int,
                    dtype: str = "bf16", ragged: bool = True):
    """A compacted cache and appended entries for the cache-attention calls (random draws).

    Per head: keys and queries follow the recipe above on a T-key document; the slots are a
    sorted random subset of t document positions (position 0 always kept), with values
    Cv ~ N(0, 1) and biases ~ N(0, 0.5^2) in float32 (stand-ins for fitted ones); nvalid is
    drawn in [t / 2, t] when ragged (else t); m new entries follow the same key/value
    recipe. Returns Q [h, n, d], Ck [h, t, d], Cv, bias, keypos, nvalid, Kn, Vn [h, m, d];
    Q, Ck, Kn, Vn in the input dtype (uint16 bf16 bits for "bf16").
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED0, 7, seed])))
    Q = np.empty((heads, n, d), np.float32)
    Ck = np.empty((heads, t, d), np.float32)
    Kn = np.empty((heads, m, d), np.float32)
    Vn = rng.standard_normal((heads, m, d), dtype=np.float32)
    Cv = rng.standard_normal((heads, t, d), dtype=np.float32)
    bias = (0.5 * rng.standard_normal((heads, t))).astype(np.float32)
    keypos = np.empty((heads, t), np.int32)
    nvalid = np.full(heads, t, np.int32)
    for h in range(heads):
        s = rng.lognormal(0.0, 0.5, size=d).astype(np.float32)
        K = rng.standard_normal((T, d), dtype=np.float32) * s
        pos = np.sort(rng.choice(np.arange(1, T), size=t - 1, replace=False)) if t > 1 else \
            np.zeros(0, np.int64)
        keypos[h] = np.concatenate([[0], pos]).astype(np.int32)
        Ck[h] = K[keypos[h]]
        Kn[h] = rng.standard_normal((m, d), dtype=np.float32) * s
        Q[h] = rng.standard_normal((n, d), dtype=np.float32)
        half = rng.permutation(n)[: n // 2]
        Q[h, half] = K[rng.integers(0, T, size=half.size)] + \
            np.float32(0.5) * rng.standard_normal((half.size, d), dtype=np.float32)
        if ragged:
            nvalid[h] = rng.integers(max(1, t // 2), t + 1)
    if dtype == "bf16":
        Q, Ck, Kn, Vn = (bf16_bits(x) for x in (Q, Ck, Kn, Vn))
    return Q, Ck, Cv, bias, keypos, nvalid, Kn, Vn


def make_heldout_queries(w: Workload, heads=None, K=None, seed: int = 1):
    """A second query set for the same caches (held-out evaluation): the query recipe above
    (half of the rows near random keys) from its own seeded stream. K is the batch's key
    array as generated (bf16 bits or float32); returns Q [h, n, d] in the workload dtype."""
    hs = range(w.heads) if heads is None else list(heads)
    Kf = as_f64(K, w.dtype).astype(np.float32)
    out = np.empty((len(hs), w.n, w.d), np.float32)
    for i, h in enumerate(hs):
        rng = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([SEED0, 8, workload_index(w), h, seed])))
        Q = rng.standard_normal((w.n, w.d), dtype=np.float32)
        kd = rng.permutation(w.n)[: w.n // 2]
        src = rng.integers(0, w.T, size=kd.size)
        Q[kd] = Kf[i][src] + np.float32(0.5) * rng.standard_normal((kd.size, w.d), dtype=np.float32)
        out[i] = Q
    return bf16_bits(out) if w.dtype == "bf16" else out


def query_subset(w: Workload, heads=None, s: int = 256, seed: int = 1):
    """The two-pass method's random query subset: s distinct query indices per head, drawn
    uniformly without replacement from its own seeded stream, ascending, int32 [h, s]."""
    hs = range(w.heads) if heads is None else list(heads)
    out = np.empty((len(hs), s), np.int32)
    for i, h in enumerate(hs):
        rng = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([SEED0, 9, workload_index(w), h, seed])))
        out[i] = np.sort(rng.choice(w.n, size=s, replace=False))
    return out


def stage1_samples(n_pos: int, steps: int, S: int = 128, pool: int = 4096, seed: int = 1):
    """Positions of the stage-1 updates (Latent Compaction App. A.2): a pool of at most
    `pool` evenly spaced positions (floor(k * n_pos / pool)) out of n_pos, then S positions
    per update drawn uniformly with replacement from it, from their own seeded stream,
    shared by every head. Returns int32 [steps, S]."""
    base = np.arange(n_pos) if n_pos <= pool else (np.arange(pool) * n_pos) // pool
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED0, 10, n_pos, seed])))
    return base[rng.integers(0, base.size, size=(steps, S))].astype(np.int32)
