"""The seeded generator: determinism, recipe counts and bf16 rounding."""
import numpy as np
import torch

from kv_cache_compaction_amd import synth
from kv_cache_compaction_amd.configs import WORKLOADS, small_variant


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 37,
                        np.array([1.00390625, 1.01171875, -3.0e-39, 65504.0], np.float32)])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.bf16_to_f32(ours),
                                  torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_deterministic_and_distinct_heads():
    w = small_variant(WORKLOADS[1], heads=3, T=256)
    a = synth.make_batch(w)
    b = synth.make_batch(w)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0][0], a[0][1])


def test_recipe_counts():
    w = small_variant(WORKLOADS[4], T=1000)
    Q, K, V = synth.draw_head_f32(w, 0)
    assert Q.shape == (w.n, w.d) and K.shape == (w.T, w.d)
    # needle rows have ~3x (or 4x) the typical row norm
    nrm = np.linalg.norm(K / np.median(np.linalg.norm(K, axis=1)), axis=1)
    assert int((nrm > 2.2).sum()) == int(0.01 * w.T) + int(0.001 * w.T)
    # exactly half of the queries sit close to some key
    d2 = ((Q * Q).sum(1)[:, None] - 2 * Q @ K.T + (K * K).sum(1)[None, :]).min(1)
    # a key-derived query is 0.5 * N(0, 1) away from its key: |noise|^2 ~ 0.25 d
    assert abs(int((d2 < 0.5 * w.d).sum()) - w.n // 2) <= w.n // 50


def test_workload_pair_counts():
    assert WORKLOADS[3].visible_pairs_per_head() == 2 * 32768 * (32768 + 1)
    assert WORKLOADS[4].visible_pairs() == 131072 ** 2
    assert WORKLOADS[1].visible_pairs() == 512 * 2048 * 2048
