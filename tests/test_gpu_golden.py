"""The 128K-key workload (one KV head, T = n = 131072, t = 4096) against stored float64
oracle results (tests/golden/single_head_T128k.npz, written on the CPU by
tests/golden/make_single_head_T128k.py from the oracle alone).

What is compared, in the launch configuration bench.py times (one am_compact_head call):
  - every key's score (1e-4 relative, plus 1e-9 of the largest) and every query's lse
    (1e-3 absolute) against the stored oracle values; outputs on sampled rows against the
    oracle computed here;
  - the selection against the oracle's scores by the near-tie rule;
  - both fits on the oracle's key set, through am_fit_beta_nnls and am_fit_values_ols
    (the latter on the oracle's beta): residuals within 1% of the oracle's optimum,
    evaluated in float64. The stored A^T Y of the oracle's value design gives the output
    residual of any C_v on that design without the 64 MiB of outputs; the value fit takes
    the library's own outputs as its targets (they match the oracle's per row within the
    bf16 tolerance, and the fit's optimum moves by far less than 1% with them);
  - the NNLS runs on 256 workgroups that keep only 7 of their 16 rows of G in LDS (the
    schedule query shows it), and its KKT residual is small;
  - when the library selects the oracle's keys, the end-to-end residuals of its own
    (beta, C_v) within 1% of the oracle's.
"""
import os
import time

import numpy as np
import pytest

import kv_cache_compaction_amd as amc
from kv_cache_compaction_amd import synth
from kv_cache_compaction_amd.configs import BY_NAME
from oracle import am_oracle as O
from tests.gpu_util import check_selection, f64, row_rel_err, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "single_head_T128k.npz")


def _log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def test_single_long_head_against_golden():
    import torch
    w = BY_NAME["single_head_T128k"]
    gold = np.load(GOLDEN)
    idx_or = gold["idx"].astype(np.int64)
    lse_or = gold["lse"]
    _log(f"{w.name}: generating inputs")
    Q, K, V = synth.make_batch(w)
    dQ, dK, dV = (to_dev(x, w.dtype) for x in (Q, K, V))
    out = amc.compact_head(dQ, dK, dV, w.t, options=amc.make_options(ridge_lambda=w.ridge_lambda))
    g = {k: (v.cpu().numpy() if v.dtype != torch.bfloat16 else None) for k, v in out.items()}
    _log(f"{w.name}: GPU step done, status {g['status']}")
    assert np.all(g["status"] == 0)
    q, k, v = (f64(x[0], w.dtype) for x in (Q, K, V))

    # full-cache statistics
    assert np.max(np.abs(g["lse"][0] - lse_or)) <= 1e-3
    sc = gold["score"]
    err = np.abs(g["score"][0] - sc) - (1e-4 * sc + 1e-9 * sc.max())
    assert err.max() <= 0, float(err.max())
    rows = np.random.default_rng(3).choice(w.n, 96, replace=False)
    l_ref, O_ref = O.attention_rows(q, k, v, w.scale, rows)
    assert np.max(np.abs(l_ref - lse_or[rows])) <= 1e-9   # the stored lse is the oracle's
    assert row_rel_err(g["O"][0][rows].astype(np.float64), O_ref).max() <= 2e-2
    idx_g = g["idx"][0].astype(np.int64)
    overlap = check_selection(idx_g, sc, w.t)
    _log(f"{w.name}: statistics and selection match (overlap {overlap:.5f})")

    # the NNLS schedule at this size reads part of G from memory at every step
    plan = amc.fit_beta_plan(1, w.n, w.T, w.d, w.t)
    _log(f"{w.name}: NNLS plan {plan}")
    assert plan["workgroups_per_head"] > 1
    assert 0 < plan["lds_rows_per_workgroup"] < plan["rows_per_workgroup"]

    # both fits on the oracle's key set
    ck = torch.from_numpy(np.ascontiguousarray(K[0][idx_or])[None].view(np.int16)).view(
        torch.bfloat16).cuda()
    didx = torch.from_numpy(idx_or[None].astype(np.int32)).cuda()
    dlse = torch.from_numpy(lse_or[None].astype(np.float32)).cuda()
    beta, wv, res, st, kkt, its = (x.cpu().numpy() for x in amc.fit_beta_nnls(
        dQ, ck, didx, dlse, T=w.T, diagnostics=True))
    assert st[0] == 0
    M, b = O.mass_design(q, k[idx_or], idx_or, lse_or, w.scale)
    rg = O.mass_residual(M, b, wv[0].astype(np.float64))
    _log(f"{w.name}: mass resid on the oracle's keys {rg:.6g} (oracle {float(gold['r_mass']):.6g}),"
         f" kkt {kkt[0]:.3g}, {its[0]} steps")
    assert rg <= 1.01 * float(gold["r_mass"]) + 1e-12
    assert res[0] == pytest.approx(rg, rel=2e-3, abs=1e-7)
    assert kkt[0] <= 1e-3 and 0 < its[0] < 500
    w_or = gold["w"]
    with np.errstate(divide="ignore"):
        beta_or = np.log(w_or).astype(np.float32)
    A = O.value_design(M, w_or)
    del M
    Cv, ores, st = (x.cpu().numpy() for x in amc.fit_values_ols(
        dQ, ck, didx, torch.from_numpy(beta_or[None]).cuda(), out["O"], T=w.T,
        ridge_lambda=w.ridge_lambda))
    assert st[0] == 0
    ro = O.output_residual_from_stats(A, Cv[0].astype(np.float64), gold["AtY"].astype(np.float64),
                                      float(gold["yy"]))
    del A
    _log(f"{w.name}: output resid on the oracle's keys and beta {ro:.6g} "
         f"(oracle {float(gold['r_out']):.6g})")
    assert ro <= 1.01 * float(gold["r_out"]) + 1e-12

    # end to end, when the key sets agree (the oracle's refit on another key set needs the
    # full outputs and a 4096-key NNLS in float64, minutes on the host)
    logz, Acmp = O.compacted_attention(q, k[idx_g], idx_g, g["beta"][0].astype(np.float64),
                                       g["Cv"][0].astype(np.float64), w.scale)
    rm_e, ro_e = O.residuals(lse_or, g["O"][0].astype(np.float64), logz, Acmp)
    _log(f"{w.name}: end to end mass resid {rm_e:.6g}, output resid {ro_e:.6g} (against the "
         f"library's outputs); keys {'equal to' if np.array_equal(idx_g, idx_or) else 'differ from'}"
         f" the oracle's")
    assert float(g["resid"][0][0]) == pytest.approx(rm_e, rel=2e-3, abs=1e-7)
    if np.array_equal(idx_g, idx_or):
        assert rm_e <= 1.01 * float(gold["r_mass"]) + 1e-12
        assert ro_e <= 1.01 * float(gold["r_out"]) + 1e-12
