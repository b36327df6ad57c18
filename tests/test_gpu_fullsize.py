"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

Every workload runs through one am_compact_head call over all of its heads. The float64
oracle then checks what it can afford on the host. For sampled heads it checks
everything: lse, outputs, key scores, the selection rule, and the residuals of the
fitted cache, evaluated with the oracle's own compacted attention. For sampled query
rows it checks lse and outputs one by one. The 128K-key head, whose float64 pass takes
minutes, is checked against stored oracle results in test_gpu_golden.py."""
import math
import time

import numpy as np
import pytest

import kv_cache_compaction_amd as amc
from kv_cache_compaction_amd import synth
from kv_cache_compaction_amd.configs import BY_NAME, WORKLOADS
from oracle import am_oracle as O
from tests.gpu_util import check_selection, f64, oracle_optimum_on, row_rel_err, to_dev

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
    om, oo, refit = oracle_optimum_on(q, k, r, idx, w)
    assert rm <= 1.01 * om + 1e-12, (rm, om, refit)
    assert ro <= 1.01 * oo + 1e-12, (ro, oo, refit)
    assert g["resid"][0][h] == pytest.approx(rm, rel=2e-3, abs=1e-7)
    assert g["resid"][1][h] == pytest.approx(ro, rel=2e-2, abs=1e-6)
    _log(f"{w.name} head {h}: overlap {overlap:.4f}, mass resid {rm:.5f} (oracle {om:.5f} on "
         f"the GPU's keys, {r['r_mass']:.5f} on its own), output resid {ro:.5f} (oracle "
         f"{oo:.5f}, {r['r_out']:.5f}){' (refit)' if refit else ''}")


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
