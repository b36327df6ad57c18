"""GPU parity of the score passes (lse, outputs, per-key scores) and of the top-t select,
against the float64 oracle on the same seeded inputs, through the C ABI."""
import numpy as np
import pytest

import kv_cache_compaction_amd as amc
from kv_cache_compaction_amd import synth
from kv_cache_compaction_amd.configs import WORKLOADS, Workload, small_variant
from oracle import am_oracle as O
from tests.gpu_util import check_selection, f64, row_rel_err, to_dev

pytestmark = pytest.mark.gpu


def _raw(x, dtype):
    import torch
    return x.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else x.numpy()


def _case(w: Workload, heads):
    Q, K, V = synth.make_batch(w, heads)
    return Q, K, V


CASES = [
    # (workload, head subset) -- full workload 0, subsets of the others at reduced size
    (WORKLOADS[0], [0]),
    (WORKLOADS[1], [0, 1, 511]),
    (small_variant(WORKLOADS[2], heads=2, T=1024), [0, 1]),
    (small_variant(WORKLOADS[3], heads=2, T=1024), [0, 1]),
    (small_variant(WORKLOADS[4], T=8192), [0]),
    # ragged shapes: T and n off the tile sizes, d = 64 in bf16, odd GQA group
    (Workload("ragged_bf16", 2, 128, 1000, 777, 37, "bf16", False, 1), [0, 1]),
    (Workload("ragged_causal_g3", 2, 64, 333, 999, 10, "bf16", True, 3), [0, 1]),
    (Workload("ragged_f32_d128", 1, 128, 200, 200, 7, "f32", True, 1), [0]),
    (Workload("tiny", 1, 64, 1, 1, 1, "bf16", False, 1), [0]),
    (Workload("tiny_causal", 1, 128, 3, 12, 2, "f32", True, 4), [0]),
    # a head count that splits evenly over the eight XCDs (whole heads per XCD), every head
    (Workload("heads16_causal_g2", 16, 64, 300, 600, 20, "bf16", True, 2), list(range(16))),
]


@pytest.mark.parametrize("w,heads", CASES, ids=[c[0].name for c in CASES])
def test_targets_and_selection(w, heads):
    print(f"case {w.name} heads={heads}", flush=True)
    Q, K, V = _case(w, heads)
    dQ, dK, dV = (to_dev(x, w.dtype) for x in (Q, K, V))
    for mode in ("rms", "mean", "max"):
        lse, Og, sc = amc.targets(dQ, dK, dV, causal=w.causal, group=w.group, score=mode)
        idx, Ck, Vs = amc.select_keys(sc, dK, w.t, dV, want_vsel=True)
        lse, Og, sc, idx = (x.cpu().numpy() for x in (lse, Og, sc, idx))
        Ck, Vs = Ck.cpu(), Vs.cpu()
        for i in range(len(heads)):
            q, k, v = (f64(x[i], w.dtype) for x in (Q, K, V))
            l_ref, O_ref, stats = O.full_cache_stats(q, k, v, w.scale, w.causal, w.group)
            s_ref = O.key_score(stats, mode, w.n)
            assert np.max(np.abs(lse[i] - l_ref)) <= 1e-3
            tol = 2e-2 if w.dtype == "bf16" else 1e-4
            err = row_rel_err(Og[i].astype(np.float64), O_ref)
            assert err.max() <= tol, f"O row error {err.max():.3e}"
            err_s = np.abs(sc[i] - s_ref) - (1e-4 * s_ref + 1e-9 * s_ref.max())
            assert err_s.max() <= 0, f"{mode} score error beyond 1e-4 relative: {err_s.max():.3e}"
            check_selection(idx[i], s_ref, w.t)
            # gathered rows are bit-exact copies
            ki = idx[i].astype(np.int64)
            raw_k = K[i][ki]
            raw_v = V[i][ki]
            ck, vs = _raw(Ck[i], w.dtype), _raw(Vs[i], w.dtype)
            np.testing.assert_array_equal(ck, raw_k)
            np.testing.assert_array_equal(vs, raw_v)


@pytest.mark.parametrize("T,t", [(1, 1), (100, 1), (100, 100), (4097, 1000), (131072, 4096),
                                 (2048, 64)])
def test_select_is_exact_on_given_scores(T, t):
    """Integer work: on the same fp32 scores the select is bit-exact with the oracle's rule,
    including heavy ties (ties go to the lower index)."""
    import torch
    rng = np.random.default_rng(T + t)
    heads = 3
    sc = rng.random((heads, T)).astype(np.float32)
    sc[1] = np.round(sc[1] * 7) / 7             # many exact ties
    sc[2] = 0.25                                 # all equal
    sc[2, ::5] = 0.5
    K = rng.integers(0, 60000, (heads, T, 64)).astype(np.uint16)
    dK = to_dev(K, "bf16")
    idx, Ck, _ = amc.select_keys(torch.from_numpy(sc).cuda(), dK, t)
    idx = idx.cpu().numpy()
    for i in range(heads):
        ref = O.select_top(sc[i].astype(np.float64), t)
        np.testing.assert_array_equal(idx[i], ref)
    np.testing.assert_array_equal(Ck.cpu().view(torch.int16).numpy().view(np.uint16),
                                  np.stack([K[i][idx[i]] for i in range(heads)]))


def test_targets_deterministic():
    import torch
    w = small_variant(WORKLOADS[3], heads=2, T=512)
    Q, K, V = _case(w, [0, 1])
    dQ, dK, dV = (to_dev(x, w.dtype) for x in (Q, K, V))
    a = amc.targets(dQ, dK, dV, causal=True, group=4)
    b = amc.targets(dQ, dK, dV, causal=True, group=4)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
