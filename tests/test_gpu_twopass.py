"""GPU parity of the two-pass key selection and of the blog's two-pass method (two-pass
selection, redistributed beta, direct values), against the float64 oracle, through the
C ABI."""
import numpy as np
import pytest

import kv_cache_compaction_amd as amc
from kv_cache_compaction_amd import synth
from kv_cache_compaction_amd.configs import WORKLOADS, Workload, small_variant
from oracle import am_oracle as O
from tests.gpu_util import check_selection, f64, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    (small_variant(WORKLOADS[3], heads=2, T=1024), [0, 1], 256, 4),
    (small_variant(WORKLOADS[2], heads=2, T=1024), [0, 1], 256, 3),
    (Workload("ragged_causal_g3", 2, 64, 333, 999, 45, "bf16", True, 3), [0, 1], 100, 5),
    (Workload("f32_causal_d128", 1, 128, 500, 500, 70, "f32", True, 1), [0], 64, 2),
    (WORKLOADS[0], [0], 128, 4),
]


def _pass_scores(q, k, sub, short, w, mode="rms"):
    """The two stages' statistics from the oracle, for the near-tie rule."""
    _, _, st1 = O.full_cache_stats(q[sub], k, k, w.scale, w.causal, w.group, want_O=False,
                                   rows=sub)
    _, _, st2 = O.full_cache_stats(q, k[short], k[short], w.scale, w.causal, w.group, want_O=False,
                                   keypos=short)
    return O.key_score(st1, mode, sub.size), O.key_score(st2, mode, q.shape[0])


@pytest.mark.parametrize("w,heads,s,k_mult", CASES, ids=[c[0].name for c in CASES])
def test_select_two_pass_matches_oracle(w, heads, s, k_mult):
    import torch
    print(f"case {w.name}", flush=True)
    Q, K, V = synth.make_batch(w, heads)
    sub = synth.query_subset(w, heads, s)
    idx, Ck, Vs, lse = amc.select_two_pass(to_dev(Q, w.dtype), to_dev(K, w.dtype),
                                           torch.from_numpy(sub).cuda(), w.t,
                                           V=to_dev(V, w.dtype), k_mult=k_mult, causal=w.causal,
                                           group=w.group)
    idx, lse = idx.cpu().numpy(), lse.cpu().numpy()
    raw = lambda x: x.view(torch.int16).numpy().view(np.uint16) if w.dtype == "bf16" else x.numpy()
    Ck, Vs = raw(Ck.cpu()), raw(Vs.cpu())
    kt = min(k_mult * w.t, w.T)
    for i in range(len(heads)):
        q, k = f64(Q[i], w.dtype), f64(K[i], w.dtype)
        ref_idx, ref_lse = O.select_two_pass(q, k, sub[i], w.t, k_mult, w.scale, w.causal, w.group)
        sc1 = O.key_score(O.full_cache_stats(q[sub[i]], k, k, w.scale, w.causal, w.group,
                                             want_O=False, rows=sub[i])[2], "rms", s)
        short = O.select_top(sc1, kt)
        np.testing.assert_array_equal(Ck[i], K[i][idx[i]])
        np.testing.assert_array_equal(Vs[i], V[i][idx[i]])
        assert np.all(np.diff(idx[i]) > 0)
        # the shortlist is unique unless pass 1 has a near tie at its threshold (then the
        # GPU may keep another key there and the second stage differs legitimately)
        order = np.lexsort((np.arange(w.T), -sc1))
        clear = kt >= w.T or sc1[order[kt - 1]] - sc1[order[kt]] > 1e-4 * sc1[order[kt - 1]]
        assert clear, "seeded case has a pass-1 near tie; choose another subset seed"
        _, sc2 = _pass_scores(q, k, sub[i], short, w)
        # the selection, as positions in the shortlist, obeys the near-tie rule on pass 2
        loc = np.searchsorted(short, idx[i])
        assert np.all(short[np.minimum(loc, kt - 1)] == idx[i]), "selected keys outside the shortlist"
        check_selection(loc, sc2, w.t)
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(lse[i]), fin)
        assert np.max(np.abs(lse[i][fin] - ref_lse[fin]), initial=0.0) <= 1e-3


def test_two_pass_full_shortlist_all_queries_equals_one_pass():
    import torch
    w = small_variant(WORKLOADS[3], heads=2, T=1024)
    Q, K, V = synth.make_batch(w, [0, 1])
    dQ, dK, dV = (to_dev(x, w.dtype) for x in (Q, K, V))
    sub = torch.arange(w.n, dtype=torch.int32).repeat(2, 1).contiguous().cuda()
    idx, _, _, lse = amc.select_two_pass(dQ, dK, sub, w.t, k_mult=w.T // w.t, causal=w.causal,
                                         group=w.group)
    lse_full, _, sc = amc.targets(dQ, dK, dV, causal=w.causal, group=w.group)
    idx_full, _, _ = amc.select_keys(sc, dK, w.t)
    assert torch.equal(idx, idx_full)
    assert torch.allclose(lse, lse_full, rtol=0, atol=1e-4)


def test_compact_two_pass_chain():
    import torch
    w = small_variant(WORKLOADS[3], heads=2, T=1024)
    Q, K, V = synth.make_batch(w, [0, 1])
    dQ, dK, dV = (to_dev(x, w.dtype) for x in (Q, K, V))
    sub = torch.from_numpy(synth.query_subset(w, [0, 1], 256)).cuda()
    out = amc.compact_two_pass(dQ, dK, dV, sub, w.t, k_mult=4, causal=w.causal, group=w.group)
    idx, Ck, _, lse = amc.select_two_pass(dQ, dK, sub, w.t, k_mult=4, causal=w.causal,
                                          group=w.group)
    assert torch.equal(out["idx"], idx) and torch.equal(out["Ck"], Ck)
    beta, _, res = amc.beta_redistribute(dQ, Ck, idx, lse, causal=w.causal, group=w.group, T=w.T)
    assert torch.equal(out["beta"], beta)
    assert torch.equal(out["resid"][0], res)
    assert torch.all(out["resid"][1] == -1)
    ref_cv = np.stack([f64(V[i], w.dtype)[idx[i].cpu().numpy()] for i in range(2)]).astype(np.float32)
    np.testing.assert_array_equal(out["Cv"].cpu().numpy(), ref_cv)
