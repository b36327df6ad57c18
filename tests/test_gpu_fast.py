"""GPU parity of the "Compaction" blog's fast variants (beta by uniform redistribution,
direct values) and of the held-out evaluation, against the float64 oracle on the same
seeded inputs, through the C ABI. Key sets come from the oracle so both sides work on the
same compacted keys."""
import numpy as np
import pytest

import kv_cache_compaction_amd as amc
from kv_cache_compaction_amd import synth
from kv_cache_compaction_amd.configs import WORKLOADS, Workload, small_variant
from oracle import am_oracle as O
from tests.gpu_util import f64, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    (WORKLOADS[0], [0]),
    (small_variant(WORKLOADS[2], heads=2, T=1024), [0, 1]),
    (small_variant(WORKLOADS[3], heads=2, T=1024), [0, 1]),
    (Workload("ragged_causal_g3", 2, 64, 333, 999, 45, "bf16", True, 3), [0, 1]),
    (Workload("big_t_causal_g4", 2, 128, 1536, 6144, 384, "bf16", True, 4), [0, 1]),
    (Workload("f32_causal_d128", 1, 128, 500, 500, 70, "f32", True, 1), [0]),
    (Workload("t1", 1, 128, 300, 300, 1, "bf16", False, 1), [0]),
]


F32_MAX = float(np.finfo(np.float32).max)


def _check_mass_resid(got, ref):
    """The library reports residuals in fp32: values beyond its range come back as inf
    (redistribution can hand keys of tiny mass very large biases)."""
    got = float(got)
    if ref >= F32_MAX:
        assert got == np.inf
    else:
        assert abs(got - ref) <= 2e-3 * ref + 1e-7, (got, ref)


def _setup(w, heads):
    import torch
    Q, K, V = synth.make_batch(w, heads)
    refs = []
    for i in range(len(heads)):
        q, k, v = (f64(x[i], w.dtype) for x in (Q, K, V))
        lse, Oref, stats = O.full_cache_stats(q, k, v, w.scale, w.causal, w.group)
        idx = O.select_top(O.key_score(stats, "rms", w.n), w.t)
        refs.append(dict(q=q, k=k, v=v, lse=lse, O=Oref, idx=idx))
    idx = torch.from_numpy(np.stack([r["idx"] for r in refs]).astype(np.int32)).cuda()
    Ck = to_dev(np.stack([K[i][r["idx"]] for i, r in enumerate(refs)]), w.dtype)
    return Q, K, V, refs, idx, Ck


@pytest.mark.parametrize("w,heads", CASES, ids=[c[0].name for c in CASES])
def test_beta_redistribute_matches_oracle(w, heads):
    print(f"case {w.name}", flush=True)
    Q, K, V, refs, idx, Ck = _setup(w, heads)
    dQ = to_dev(Q, w.dtype)
    lse, _, _ = amc.targets(dQ, to_dev(K, w.dtype), None, causal=w.causal, group=w.group,
                            want_O=False, want_score=False)
    beta, wv, res = amc.beta_redistribute(dQ, Ck, idx, lse, causal=w.causal, group=w.group, T=w.T)
    beta, wv, res = beta.cpu().numpy(), wv.cpu().numpy(), res.cpu().numpy()
    for i, r in enumerate(refs):
        ref = O.redistribute_beta(r["q"], r["k"][r["idx"]], r["idx"], r["lse"], w.scale, w.causal,
                                  w.group)
        assert np.all(np.isfinite(beta[i]))
        # beta_j = log(m_j + Delta / t) - log m_j moves by dDelta / (t m_j + Delta) when
        # Delta does. The GPU's lse (abs. error ~3e-5) and fp32 exponentials bound
        # |dDelta| by 5e-5 of the mean reference mass; the comparison allows that plus 1e-4.
        c = r["lse"].max()
        s = w.scale * r["q"] @ r["k"][r["idx"]].T
        vis = O.visible(np.arange(w.n), r["idx"], w.causal, w.group)
        m = np.where(vis, np.exp(np.where(vis, s, 0.0) - c), 0.0).sum(axis=0) / w.n
        total = np.exp(r["lse"] - c).sum() / w.n
        delta = max(total - m.sum(), 0.0)
        tol = 1e-4 + 5e-5 * total / (w.t * m + delta)
        err = np.abs(beta[i] - ref)
        assert np.all(err <= tol), f"beta error {err.max():.3e} (worst margin {(err / tol).max():.2f})"
        well = (tol < 1e-3) & (ref < np.log(F32_MAX))
        np.testing.assert_allclose(wv[i][well], np.exp(ref[well]), rtol=2e-3)
        assert np.all(wv[i][ref > np.log(F32_MAX) + 1e-3] == np.inf)   # w = e^beta beyond fp32
        # mass residual of the GPU's beta, evaluated by the oracle
        logz, _ = O.compacted_attention(r["q"], r["k"][r["idx"]], r["idx"], beta[i].astype(np.float64),
                                        r["v"][r["idx"]], w.scale, w.causal, w.group)
        r_mass = float(np.mean((np.exp(logz - r["lse"]) - 1.0) ** 2))
        _check_mass_resid(res[i], r_mass)


@pytest.mark.parametrize("beta_mode,value_mode", [("redistribute", "direct"),
                                                  ("redistribute", "fit"), ("nnls", "direct")])
def test_compact_head_fast_variants(beta_mode, value_mode):
    import torch
    w = small_variant(WORKLOADS[3], heads=2, T=1024)
    Q, K, V = synth.make_batch(w, [0, 1])
    dQ, dK, dV = (to_dev(x, w.dtype) for x in (Q, K, V))
    opts = amc.make_options(beta=beta_mode, values=value_mode, ridge_lambda=w.ridge_lambda)
    out = amc.compact_head(dQ, dK, dV, w.t, causal=w.causal, group=w.group, options=opts)
    base = amc.compact_head(dQ, dK, dV, w.t, causal=w.causal, group=w.group,
                            options=amc.make_options(ridge_lambda=w.ridge_lambda))
    torch.cuda.synchronize()
    assert torch.equal(out["idx"], base["idx"])
    assert int(out["status"].abs().sum()) == 0
    if beta_mode == "redistribute":
        b2, _, _ = amc.beta_redistribute(dQ, out["Ck"], out["idx"], out["lse"], causal=w.causal,
                                         group=w.group, T=w.T)
        assert torch.equal(out["beta"], b2)
    else:
        assert torch.equal(out["beta"], base["beta"])
    idx = out["idx"].cpu().numpy()
    Cv = out["Cv"].cpu().numpy()
    beta = out["beta"].cpu().numpy().astype(np.float64)
    res = out["resid"].cpu().numpy()
    for i in range(2):
        q, k, v = (f64(x[i], w.dtype) for x in (Q, K, V))
        lse, Oref, _ = O.full_cache_stats(q, k, v, w.scale, w.causal, w.group)
        if value_mode == "direct":
            np.testing.assert_array_equal(Cv[i], v[idx[i]].astype(np.float32))
        logz, A = O.compacted_attention(q, k[idx[i]], idx[i], beta[i], Cv[i].astype(np.float64),
                                        w.scale, w.causal, w.group)
        r_mass, r_out = O.residuals(lse, Oref, logz, A)
        _check_mass_resid(res[0, i], r_mass)
        assert abs(res[1, i] - r_out) <= 2e-2 * r_out + 1e-6


@pytest.mark.parametrize("w,heads", [(small_variant(WORKLOADS[3], heads=2, T=1024), [0, 1]),
                                     (Workload("ragged_g3_d64", 2, 64, 333, 999, 45, "bf16", True, 3), [0, 1]),
                                     (WORKLOADS[0], [0])],
                         ids=["causal_g4", "ragged_g3_d64", "f32_d64"])
def test_eval_residuals_on_heldout_queries(w, heads):
    """A compaction fitted on the reference queries, evaluated on a second seeded query set
    against the same cache: GPU residuals against the oracle's evaluator."""
    Q, K, V = synth.make_batch(w, heads)
    Qh = synth.make_heldout_queries(w, heads, K, seed=3)
    dQ, dK, dV, dQh = (to_dev(x, w.dtype) for x in (Q, K, V, Qh))
    out = amc.compact_head(dQ, dK, dV, w.t, causal=w.causal, group=w.group,
                           options=amc.make_options(ridge_lambda=w.ridge_lambda))
    res = amc.eval_residuals(dQh, dK, dV, out["idx"], out["Ck"], out["beta"], out["Cv"],
                             causal=w.causal, group=w.group).cpu().numpy()
    idx = out["idx"].cpu().numpy()
    beta = out["beta"].cpu().numpy().astype(np.float64)
    Cv = out["Cv"].cpu().numpy().astype(np.float64)
    for i in range(len(heads)):
        qh, k, v = (f64(x[i], w.dtype) for x in (Qh, K, V))
        lse, Oref, _ = O.full_cache_stats(qh, k, v, w.scale, w.causal, w.group)
        logz, A = O.compacted_attention(qh, k[idx[i]], idx[i], beta[i], Cv[i], w.scale, w.causal,
                                        w.group)
        r_mass, r_out = O.residuals(lse, Oref, logz, A)
        tol = 2e-2 if w.dtype == "bf16" else 1e-3
        _check_mass_resid(res[0, i], r_mass)
        assert abs(res[1, i] - r_out) <= tol * r_out + 1e-6
