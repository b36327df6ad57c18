"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

Every workload runs through one am_compact_head call over all of its heads. The float64
oracle then checks what it can afford on the host. For sampled heads it checks
everything: lse, outputs, key scores, the selection rule, and the residuals of the
fitted cache, evaluated with the oracle's own compacted attention. For sampled query
rows it checks lse and outputs one by one. Where a full oracle pass is out of reach (the
128K-key head), it checks properties that hold at any size."""
import math
import time

import numpy as np
import pytest

import kv_cache_compaction_amd as amc
from kv_cache_compaction_amd import synth
from kv_cache_compaction_amd.configs import BY_NAME, WORKLOADS
from oracle import am_oracle as O
from tests.gpu_util import check_selection, f64, row_rel_err, to_dev

pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def _run(w):
    _log(f"{w.name}: generating {w.heads} heads")
    Q, K, V = synth.make_batch(w)
    dQ, dK, dV = (to_dev(x, w.dtype) for x in (Q, K, V))
    out = amc.compact_head(dQ, dK, dV, w.t, causal=w.causal, group=w.group,
                           options=amc.make_options(ridge_lambda=w.ridge_lambda))
    import torch
    g = {k: (v.cpu().numpy() if v.dtype != torch.bfloat16 else None) for k, v in out.items()}
    _log(f"{w.name}: GPU done")
    return Q, K, V, g


def _check_rows(w, Q, K, V, g, h, rows):
    q, k, v = (f64(x[h], w.dtype) for x in (Q, K, V))
    l_ref, O_ref = O.attention_rows(q, k, v, w.scale, rows, w.causal, w.group)
    assert np.max(np.abs(g["lse"][h][rows] - l_ref)) <= 1e-3
    tol = 2e-2 if w.dtype == "bf16" else 1e-4
    assert row_rel_err(g["O"][h][rows].astype(np.float64), O_ref).max() <= tol


def _check_head_fully(w, Q, K, V, g, h):
    q, k, v = (f64(x[h], w.dtype) for x in (Q, K, V))
    r = O.compact_head(q, k, v, w.t, w.scale, w.causal, w.group, ridge_lambda=w.ridge_lambda)
    assert np.max(np.abs(g["lse"][h] - r["lse"])) <= 1e-3
    tol = 2e-2 if w.dtype == "bf16" else 1e-4
    assert row_rel_err(g["O"][h].astype(np.float64), r["O"]).max() <= tol
    err = np.abs(g["score"][h] - r["score"]) - (1e-4 * r["score"] + 1e-9 * r["score"].max())
    assert err.max() <= 0
    idx = g["idx"][h].astype(np.int64)
    overlap = check_selection(idx, r["score"], w.t)
    logz, A = O.compacted_attention(q, k[idx], idx, g["beta"][h].astype(np.float64),
                                    g["Cv"][h].astype(np.float64), w.scale, w.causal, w.group)
    rm, ro = O.residuals(r["lse"], r["O"], logz, A)
    f = 1.01 if np.array_equal(idx, r["idx"]) else 1.05
    assert rm <= f * r["r_mass"] + 1e-6, (rm, r["r_mass"])
    assert ro <= f * r["r_out"] + 1e-6, (ro, r["r_out"])
    assert g["resid"][0][h] == pytest.approx(rm, rel=2e-3, abs=1e-7)
    assert g["resid"][1][h] == pytest.approx(ro, rel=2e-2, abs=1e-6)
    _log(f"{w.name} head {h}: overlap {overlap:.4f}, mass resid {rm:.5f} "
         f"(oracle {r['r_mass']:.5f}), output resid {ro:.5f} (oracle {r['r_out']:.5f})")


@pytest.mark.parametrize("name,heads", [("docs64x8_T2k", [0, 137, 300, 511]),
                                        ("layers36x8_T4k_gqa4", [0, 143, 287])])
def test_many_heads_full_size(name, heads):
    w = BY_NAME[name]
    Q, K, V, g = _run(w)
    assert np.all(g["status"] == 0)
    for h in heads:
        _check_head_fully(w, Q, K, V, g, h)
    rng = np.random.default_rng(1)
    for h in rng.choice(w.heads, 16, replace=False):
        _check_rows(w, Q, K, V, g, int(h), rng.choice(w.n, 16, replace=False))


def test_causal_long_layer_full_size():
    w = BY_NAME["causal8_T32k_gqa4"]
    Q, K, V, g = _run(w)
    assert np.all(g["status"] == 0)
    rng = np.random.default_rng(2)
    for h in range(w.heads):
        rows = np.concatenate([[0, 1, 2, 3, w.n - 1], rng.choice(w.n, 27, replace=False)])
        _check_rows(w, Q, K, V, g, h, rows)
    _check_head_fully(w, Q, K, V, g, 5)


def test_single_long_head_full_size():
    """128K keys: the full float64 pass takes minutes on the host, so sampled rows plus
    properties that hold at any size."""
    import torch
    w = BY_NAME["single_head_T128k"]
    Q, K, V, g = _run(w)
    assert np.all(g["status"] == 0)
    rng = np.random.default_rng(3)
    _check_rows(w, Q, K, V, g, 0, rng.choice(w.n, 96, replace=False))
    # mean scores of each query row sum to 1, so the MEAN statistic sums to 1 over keys
    dQ, dK, dV = (to_dev(x, w.dtype) for x in (Q, K, V))
    _, _, mean = amc.targets(dQ, dK, dV, score="mean", want_O=False)
    assert float(mean.double().sum()) == pytest.approx(1.0, rel=1e-4)
    # selection: ascending, unique, and every selected score >= every unselected one
    idx = g["idx"][0].astype(np.int64)
    sc = g["score"][0]
    assert np.all(np.diff(idx) > 0)
    mask = np.zeros(w.T, bool)
    mask[idx] = True
    assert sc[mask].min() >= sc[~mask].max()
    # fitted cache on sampled queries: the compacted attention of the GPU's (idx, beta, Cv),
    # evaluated by the oracle, against the full cache on the same rows
    q, k, v = (f64(x[0], w.dtype) for x in (Q, K, V))
    rows = rng.choice(w.n, 1024, replace=False)
    l_ref, O_ref = O.attention_rows(q, k, v, w.scale, rows)
    logz, A = O.compacted_attention(q[rows], k[idx], idx, g["beta"][0].astype(np.float64),
                                    g["Cv"][0].astype(np.float64), w.scale)
    rm, ro = O.residuals(l_ref, O_ref, logz, A)
    _log(f"{w.name}: sampled mass resid {rm:.5f} (GPU full {g['resid'][0][0]:.5f}), "
         f"sampled output resid {ro:.5f} (GPU full {g['resid'][1][0]:.5f})")
    # the sample estimates the full residuals the library reports
    assert rm == pytest.approx(float(g["resid"][0][0]), rel=0.3)
    assert ro == pytest.approx(float(g["resid"][1][0]), rel=0.3)
    del torch
