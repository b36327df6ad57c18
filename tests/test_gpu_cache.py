"""GPU parity of attention through a compacted cache with appended entries and of the
log-space merge (Latent Compaction §3.1 Eq. 2-5), against the float64 oracle on the same
seeded inputs, through the C ABI."""
import numpy as np
import pytest

import kv_cache_compaction_amd as amc
from kv_cache_compaction_amd import synth
from oracle import am_oracle as O
from tests.gpu_util import f64, row_rel_err, to_dev

pytestmark = pytest.mark.gpu

# (name, seed, heads, n, T, t, m, d, dtype, causal, group, new_causal, ragged)
CASES = [
    ("doc_causal_g4", 1, 2, 4 * 1000, 1000, 100, 0, 128, "bf16", True, 4, True, False),
    ("doc_and_new_causal", 2, 2, 4 * 300, 2000, 150, 300, 128, "bf16", False, 4, True, True),
    ("causal_doc_and_new", 3, 2, 4 * 257, 900, 130, 257, 128, "bf16", True, 4, True, True),
    ("f32_d64_all_visible", 4, 1, 333, 500, 77, 50, 64, "f32", False, 1, False, True),
    ("bf16_d64_ragged", 5, 3, 2 * 95, 400, 65, 95, 64, "bf16", False, 2, True, True),
    ("f32_d128_causal", 6, 1, 3 * 70, 300, 33, 70, 128, "f32", True, 3, True, True),
    ("tiny", 7, 1, 1, 4, 1, 1, 64, "bf16", False, 1, True, False),
]


def _run(case, nvalid_override=None):
    name, seed, h, n, T, t, m, d, dt, causal, g, newc, ragged = case
    Q, Ck, Cv, bias, kp, nv, Kn, Vn = synth.make_cache_case(seed, h, n, T, t, m, d, dt, ragged)
    if nvalid_override is not None:
        nv = np.asarray(nvalid_override, np.int32)
    import torch
    dQ, dCk = to_dev(Q, dt), to_dev(Ck, dt)
    dCv, dbias = torch.from_numpy(Cv).cuda(), torch.from_numpy(bias).cuda()
    dkp, dnv = torch.from_numpy(kp).cuda(), torch.from_numpy(nv).cuda()
    dKn = to_dev(Kn, dt) if m else None
    dVn = to_dev(Vn, dt) if m else None
    out, lse, lz1 = amc.cache_attention(dQ, dCk, dCv, dbias, keypos=dkp, nvalid=dnv, Kn=dKn,
                                        Vn=dVn, new_causal=newc, causal=causal, group=g,
                                        want_lse_cmp=True)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(d)
    res = []
    for i in range(h):
        ref = O.cache_attention(f64(Q[i], dt), f64(Ck[i], dt), Cv[i].astype(np.float64),
                                bias[i].astype(np.float64), scale, keypos=kp[i], nvalid=nv[i],
                                causal=causal, group=g,
                                Kn=f64(Kn[i], dt) if m else None, Vn=f64(Vn[i], dt) if m else None,
                                new_causal=newc)
        res.append(ref)
    return (out.cpu().numpy(), lse.cpu().numpy(), lz1.cpu().numpy()), res, dt


def _compare(got, refs, dt):
    out, lse, lz1 = got
    tol = 2e-2 if dt == "bf16" else 1e-4
    for i, (r_out, r_lz, r_lz1) in enumerate(refs):
        fin = np.isfinite(r_lz)
        assert np.array_equal(np.isfinite(lse[i]), fin), "empty rows must give -inf"
        assert np.max(np.abs(lse[i][fin] - r_lz[fin]), initial=0.0) <= 1e-3
        fin1 = np.isfinite(r_lz1)
        assert np.array_equal(np.isfinite(lz1[i]), fin1)
        assert np.max(np.abs(lz1[i][fin1] - r_lz1[fin1]), initial=0.0) <= 1e-3
        err = row_rel_err(out[i][fin].astype(np.float64), r_out[fin])
        assert err.max(initial=0.0) <= tol, f"output row error {err.max():.3e}"
        assert np.all(out[i][~fin] == 0.0)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cache_attention_matches_oracle(case):
    print(f"case {case[0]}", flush=True)
    got, refs, dt = _run(case)
    _compare(got, refs, dt)


def test_cache_attention_empty_slots_and_rows():
    """A head with no valid slot reduces to the new branch; under a causal document mask
    with no new entries, queries before every slot position get -inf and zero rows."""
    case = ("mixed", 8, 3, 2 * 200, 600, 40, 200, 128, "bf16", False, 2, True, True)
    got, refs, dt = _run(case, nvalid_override=[0, 40, 17])
    _compare(got, refs, dt)
    name, seed, h, n, T, t, m, d, dt, causal, g, newc, ragged = case
    Q, Ck, Cv, bias, kp, nv, Kn, Vn = synth.make_cache_case(9, 1, 2 * 600, T, t, 0, d, dt, False)
    kp = kp + 50   # slot positions 50.. : queries at positions < 50 see no slot
    import torch
    out, lse = amc.cache_attention(to_dev(Q, dt), to_dev(Ck, dt), torch.from_numpy(Cv).cuda(),
                                   torch.from_numpy(bias).cuda(), keypos=torch.from_numpy(kp).cuda(),
                                   causal=True, group=2)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    ref = O.cache_attention(f64(Q[0], dt), f64(Ck[0], dt), Cv[0].astype(np.float64),
                            bias[0].astype(np.float64), 1 / np.sqrt(d), keypos=kp[0], causal=True,
                            group=2)
    assert np.all(lse[0, :100] == -np.inf) and np.all(out[0, :100] == 0.0)
    _compare((out, lse, lse), [ref], dt)   # no new entries: log Z = log Z_cmp


def test_attention_merge_matches_oracle_and_in_place():
    import torch
    rng = np.random.default_rng(5)
    h, n, d = 3, 1000, 128
    O1 = rng.standard_normal((h, n, d)).astype(np.float32)
    O2 = rng.standard_normal((h, n, d)).astype(np.float32)
    l1 = (5 * rng.standard_normal((h, n))).astype(np.float32)
    l2 = (5 * rng.standard_normal((h, n))).astype(np.float32)
    l1[0, :10] = -np.inf
    l2[1, :10] = -np.inf
    l1[2, :5] = -np.inf
    l2[2, :5] = -np.inf
    O1[2, :5] = 0.0
    O2[2, :5] = 0.0
    d1, d2 = torch.from_numpy(O1).cuda(), torch.from_numpy(O2).cuda()
    e1, e2 = torch.from_numpy(l1).cuda(), torch.from_numpy(l2).cuda()
    out, lse = amc.attention_merge(d1, e1, d2, e2)
    ref_out = np.zeros((h, n, d))
    ref_l = np.zeros((h, n))
    for i in range(h):
        ref_out[i], ref_l[i] = O.merge_log_space(O1[i].astype(np.float64), l1[i].astype(np.float64),
                                                  O2[i].astype(np.float64), l2[i].astype(np.float64))
    lse = lse.cpu().numpy()
    assert np.array_equal(np.isfinite(lse), np.isfinite(ref_l))
    fin = np.isfinite(ref_l)
    np.testing.assert_allclose(lse[fin], ref_l[fin], rtol=0, atol=2e-6 * (1 + np.abs(ref_l[fin])).max())
    np.testing.assert_allclose(out.cpu().numpy(), ref_out, rtol=0, atol=2e-6)
    # in place into the first operand
    amc.attention_merge(d1, e1, d2, e2, out=d1, lse_out=e1)
    np.testing.assert_allclose(d1.cpu().numpy(), ref_out, rtol=0, atol=2e-6)
    assert np.array_equal(np.isfinite(e1.cpu().numpy()), np.isfinite(ref_l))


def test_cache_attention_sampled_rows_at_serving_size():
    """8 heads, 1024 slots selected from a 32K-key document, 4096 appended tokens with GQA 4
    (16384 queries per head): sampled rows against the oracle."""
    import torch
    h, T, t, m, d, g = 8, 32768, 1024, 4096, 128, 4
    n = g * m
    Q, Ck, Cv, bias, kp, nv, Kn, Vn = synth.make_cache_case(10, h, n, T, t, m, d, "bf16", False)
    out, lse = amc.cache_attention(to_dev(Q, "bf16"), to_dev(Ck, "bf16"), torch.from_numpy(Cv).cuda(),
                                   torch.from_numpy(bias).cuda(), Kn=to_dev(Kn, "bf16"),
                                   Vn=to_dev(Vn, "bf16"), new_causal=True, group=g)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(8), np.linspace(0, n - 1, 120).astype(np.int64),
                                     np.arange(n - 8, n)]))
    for i in (0, 5):
        r_out, r_lz, _ = O.cache_attention(f64(Q[i][rows], "bf16"), f64(Ck[i], "bf16"),
                                           Cv[i].astype(np.float64), bias[i].astype(np.float64),
                                           1 / np.sqrt(d), group=g, Kn=f64(Kn[i], "bf16"),
                                           Vn=f64(Vn[i], "bf16"), new_causal=True, rows=rows)
        assert np.max(np.abs(lse[i][rows] - r_lz)) <= 1e-3
        assert row_rel_err(out[i][rows].astype(np.float64), r_out).max() <= 2e-2
