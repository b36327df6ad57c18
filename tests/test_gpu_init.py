"""GPU parity of the anchor + diversifier initialization (Latent Compaction §3.2, Eq. 6-7)
against the float64 oracle, through the C ABI. Anchors follow the selection near-tie rule
on the maximum-attention score; each traversal step must pick a key whose distance to the
chosen set (float64, recomputed from the GPU's own earlier picks) is the largest up to a
relative 1e-5, and the sequence equals the oracle's where no such near tie occurs."""
import numpy as np
import pytest

import kv_cache_compaction_amd as amc
from kv_cache_compaction_amd import synth
from kv_cache_compaction_amd.configs import WORKLOADS, Workload, small_variant
from oracle import am_oracle as O
from tests.gpu_util import check_selection, f64, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    (small_variant(WORKLOADS[3], heads=2, T=1024), [0, 1], 64),
    (WORKLOADS[0], [0], 32),
    (Workload("ragged_causal_g3", 2, 64, 333, 999, 45, "bf16", True, 3), [0, 1], 45),
    (Workload("f32_d128", 1, 128, 700, 700, 90, "f32", False, 1), [0], 90),
    (Workload("tiny", 1, 64, 5, 5, 2, "bf16", False, 1), [0], 5),
]


def _check_head(k, q, w, M, order, idx, na, rel=1e-5):
    T = k.shape[0]
    _, _, st = O.full_cache_stats(q, k, k, w.scale, w.causal, w.group, want_O=False)
    amax = O.key_score(st, "max", q.shape[0])
    forced = amax.copy()
    forced[0] = np.inf
    anchors = order[:na]
    assert np.all(np.diff(anchors) > 0) and anchors[0] == 0
    if na > 1:
        check_selection(anchors, forced, na)
    np.testing.assert_array_equal(idx, np.sort(order))
    assert np.unique(order).size == M
    # every traversal step takes a farthest remaining key (float64 on the GPU's own set)
    dist = np.full(T, np.inf)
    chosen = np.zeros(T, dtype=bool)
    for j in order[:na]:
        dist = np.minimum(dist, ((k - k[j]) ** 2).sum(axis=1))
        chosen[j] = True
    exact = True
    for s in range(na, M):
        cand = np.where(chosen, -np.inf, dist)
        best = cand.max()
        j = order[s]
        assert not chosen[j], f"step {s} repeats key {j}"
        assert dist[j] >= best * (1 - rel) - 1e-6, f"step {s}: {dist[j]} vs best {best}"
        second = np.sort(cand)[-2] if T - s > 1 else -np.inf
        exact = exact and (best - second > rel * best)
        dist = np.minimum(dist, ((k - k[j]) ** 2).sum(axis=1))
        chosen[j] = True
    return anchors, exact


@pytest.mark.parametrize("w,heads,M", CASES, ids=[c[0].name for c in CASES])
def test_init_anchor_diverse_matches_oracle(w, heads, M):
    print(f"case {w.name}", flush=True)
    Q, K, V = synth.make_batch(w, heads)
    idx, order, status = amc.init_anchor_diverse(to_dev(Q, w.dtype), to_dev(K, w.dtype), M,
                                                 causal=w.causal, group=w.group)
    idx, order, status = idx.cpu().numpy(), order.cpu().numpy(), status.cpu().numpy()
    assert np.all(status == 0)
    na = max(1, M // 4)
    for i in range(len(heads)):
        q, k = f64(Q[i], w.dtype), f64(K[i], w.dtype)
        anchors, exact = _check_head(k, q, w, M, order[i], idx[i], na)
        ref_seq = O.farthest_first(k, anchors, M)
        if exact:   # no near tie along the way: the sequence is unique
            np.testing.assert_array_equal(order[i], ref_seq)


def test_init_anchor_diverse_headline_size():
    """8 heads x 32768 keys, M = 256 (64 anchors, 192 diversifiers), 131072 causal GQA-4
    reference queries: the traversal checked step by step on two heads."""
    w = WORKLOADS[3]
    Q, K, V = synth.make_batch(w)
    M = 256
    idx, order, status = amc.init_anchor_diverse(to_dev(Q, w.dtype), to_dev(K, w.dtype), M,
                                                 causal=w.causal, group=w.group)
    order, idx, status = order.cpu().numpy(), idx.cpu().numpy(), status.cpu().numpy()
    assert np.all(status == 0)
    for i in (0, 7):
        k = f64(K[i], w.dtype)
        np.testing.assert_array_equal(idx[i], np.sort(order[i]))
        assert order[i][0] == 0 and np.unique(order[i]).size == M
        dist = np.full(w.T, np.inf)
        chosen = np.zeros(w.T, dtype=bool)
        for j in order[i][:64]:
            dist = np.minimum(dist, ((k - k[j]) ** 2).sum(axis=1))
            chosen[j] = True
        for s in range(64, M):
            j = order[i][s]
            best = np.where(chosen, -np.inf, dist).max()
            assert not chosen[j] and dist[j] >= best * (1 - 1e-5) - 1e-6
            dist = np.minimum(dist, ((k - k[j]) ** 2).sum(axis=1))
            chosen[j] = True


def test_traversal_repeats_bit_exactly():
    """8192 keys per head span several co-resident workgroups that agree on each next key at
    a per-head barrier (candidate slots exchanged at device scope): three runs must give the
    same order."""
    w = Workload("traversal_4x8k", 4, 128, 8192, 8192, 256, "bf16", False, 1)
    Q, K, V = synth.make_batch(w)
    dQ, dK = to_dev(Q, w.dtype), to_dev(K, w.dtype)
    runs = [amc.init_anchor_diverse(dQ, dK, 128, causal=w.causal, group=w.group) for _ in range(3)]
    assert np.all(runs[0][2].cpu().numpy() == 0)
    for r in runs[1:]:
        np.testing.assert_array_equal(runs[0][1].cpu().numpy(), r[1].cpu().numpy())
        np.testing.assert_array_equal(runs[0][0].cpu().numpy(), r[0].cpu().numpy())
