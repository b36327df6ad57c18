"""GPU parity of stage-1 attention fitting (Latent Compaction §3.3 Eq. 8, App. A.2) against
the float64 oracle, through the C ABI: the loss and its gradients at one set of sampled
positions, and the loss trajectory and parameters after several AdamW updates with frozen
slots.

Tolerances: the GPU evaluates the forward and backward passes in fp32 with sums of at most
max(t, d, N) terms; with unit-scale inputs their rounding stays near 1e-6 relative, so
gradients must agree to 1e-3 of the largest gradient entry of the head and losses to 1e-4
relative. Adam divides each gradient by its running RMS, so a parameter whose gradient is
near zero relative to fp32 rounding may step in the other direction; the parameters after
k updates must therefore agree to within 0.05 lr k per entry (each Adam step moves an
entry by about lr), and frozen slots must keep their values exactly."""
import numpy as np
import pytest

import kv_cache_compaction_amd as amc
from kv_cache_compaction_amd import synth
from oracle import am_oracle as O
from tests.gpu_util import f64, to_dev

pytestmark = pytest.mark.gpu

# (name, heads, d, T, t, group, causal, dtype, S)
CASES = [
    ("causal_g2_d64", 2, 64, 512, 96, 2, True, "bf16", 37),
    ("causal_g4_d128", 2, 128, 300, 45, 4, True, "bf16", 29),
    ("noncausal_f32_d128", 1, 128, 256, 70, 1, False, "f32", 128),
    ("causal_g3_d64_f32", 1, 64, 200, 17, 3, True, "f32", 5),
    ("causal_g2_t2100_d64", 1, 64, 4096, 2100, 2, True, "bf16", 40),   # rows beyond registers
    ("single_slot_f32", 1, 128, 64, 1, 1, False, "f32", 16),
]


def _case(name, heads, d, T, t, group, causal, dtype, seed=0):
    n = group * T
    Q, Ck, Cv, bias, keypos, _, _, _ = synth.make_cache_case(seed, heads, n, T, t, 0, d, dtype,
                                                             ragged=False)
    # the full cache's keys and values behind the slots: the slots plus the rest of the
    # document drawn on the same scale (the oracle gives the targets)
    rng = np.random.default_rng(1234 + seed)
    Qf = f64(Q, dtype)
    Ckf = f64(Ck, dtype)
    scale = 1.0 / np.sqrt(d)
    Kfull = np.empty((heads, T, d))
    Vfull = rng.standard_normal((heads, T, d))
    Ofull = np.empty((heads, n, d))
    lfull = np.empty((heads, n))
    for h in range(heads):
        Kfull[h] = rng.standard_normal((T, d)) * Ckf[h].std(axis=0)
        Kfull[h, keypos[h]] = Ckf[h]
        Vfull[h, keypos[h]] = Cv[h]
        lfull[h], Ofull[h], _ = O.full_cache_stats(Qf[h], Kfull[h], Vfull[h], scale, causal,
                                                   group, want_O=True)
    return Q, Qf, Ckf, Cv.astype(np.float64), bias.astype(np.float64), keypos, \
        Ofull.astype(np.float32), lfull.astype(np.float32), scale


def _dev_params(Ckf, Cv, bias):
    import torch
    return (torch.from_numpy(Ckf.astype(np.float32)).cuda(),
            torch.from_numpy(Cv.astype(np.float32)).cuda(),
            torch.from_numpy(bias.astype(np.float32)).cuda())


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_stage1_loss_grad_matches_oracle(case):
    import torch
    name, heads, d, T, t, group, causal, dtype, S = case
    print(f"case {name}", flush=True)
    Q, Qf, Ckf, Cv, bias, keypos, Ofull, lfull, scale = _case(*case[:8])
    samples = synth.stage1_samples(T, 1, S)[0]
    samples[0] = 0   # position 0 sees only slot 0 (or nothing), a degenerate row
    p = amc.stage1_loss_grad(to_dev(Q, dtype), torch.from_numpy(Ofull).cuda(),
                             torch.from_numpy(lfull).cuda(), torch.from_numpy(samples).cuda(),
                             *_dev_params(Ckf, Cv, bias),
                             keypos=torch.from_numpy(keypos).cuda() if causal else None,
                             causal=causal, group=group, scale=scale)
    L, gCk, gCv, gb = (x.cpu().numpy().astype(np.float64) for x in p)
    rows = O.stage1_rows(samples, group)
    for h in range(heads):
        sa, sz = O.teacher_scales(Ofull[h], lfull[h], group)
        ref = O.stage1_loss_grad(Qf[h], rows, Ckf[h], Cv[h], bias[h], keypos[h], Ofull[h],
                                 lfull[h], sa, sz, scale, causal, group)
        assert abs(L[h] - ref[0]) <= 1e-4 * abs(ref[0]), (h, L[h], ref[0])
        for got, want, nm in zip((gCk[h], gCv[h], gb[h]), ref[1:], ("dCk", "dCv", "db")):
            tol = 1e-3 * np.abs(want).max()
            err = np.abs(got - want).max()
            assert err <= tol, f"{name} head {h} {nm}: max err {err} > {tol}"


def test_stage1_no_visible_rows():
    """Every sampled position precedes all slots but none: the loss and gradients are zero
    (rows that see no slot are left out)."""
    import torch
    case = ("causal_late_slots", 1, 64, 256, 20, 2, True, "bf16")
    Q, Qf, Ckf, Cv, bias, keypos, Ofull, lfull, scale = _case(*case)
    keypos = np.sort(np.random.default_rng(5).choice(np.arange(128, 256), 20, replace=False))
    keypos = keypos.astype(np.int32)[None]
    samples = np.arange(0, 100, 3, dtype=np.int32)
    L, gCk, gCv, gb = amc.stage1_loss_grad(
        to_dev(Q, "bf16"), torch.from_numpy(Ofull).cuda(), torch.from_numpy(lfull).cuda(),
        torch.from_numpy(samples).cuda(), *_dev_params(Ckf, Cv, bias),
        keypos=torch.from_numpy(keypos).cuda(), causal=True, group=2, scale=scale)
    assert float(L[0]) == 0.0
    for g in (gCk, gCv, gb):
        assert torch.count_nonzero(g).item() == 0


@pytest.mark.parametrize("case", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_stage1_fit_matches_oracle(case):
    import torch
    name, heads, d, T, t, group, causal, dtype, S = case
    print(f"case {name}", flush=True)
    Q, Qf, Ckf, Cv, bias, keypos, Ofull, lfull, scale = _case(*case[:8], seed=3)
    steps, lr, wd = 8, 3e-3, 1e-2
    samples = synth.stage1_samples(T, steps, S, seed=2)
    trainable = np.random.default_rng(7).random((heads, t)) < 0.3   # anchors/diversifiers
    trainable[:, 0] = True
    Ck0, Cv0, b0 = _dev_params(Ckf, Cv, bias)
    Ck1, Cv1, b1, losses = amc.fit_stage1(
        to_dev(Q, dtype), torch.from_numpy(Ofull).cuda(), torch.from_numpy(lfull).cuda(),
        torch.from_numpy(samples).cuda(), Ck0, Cv0, b0,
        keypos=torch.from_numpy(keypos).cuda() if causal else None,
        trainable=torch.from_numpy(trainable).cuda(), lr=lr, wd=wd, causal=causal,
        group=group, scale=scale)
    got = [x.cpu().numpy().astype(np.float64) for x in (Ck1, Cv1, b1)]
    losses = losses.cpu().numpy().astype(np.float64)
    start = [x.cpu().numpy().astype(np.float64) for x in (Ck0, Cv0, b0)]
    for h in range(heads):
        rCk, rCv, rb, rl = O.stage1_fit(Qf[h], start[0][h], start[1][h], start[2][h],
                                        keypos[h], Ofull[h], lfull[h], samples, scale, causal,
                                        group, lr, wd, trainable[h])
        np.testing.assert_allclose(losses[:, h], rl, rtol=2e-3, atol=0)
        fz = ~trainable[h]
        for g, r, s0, nm in zip(got, (rCk, rCv, rb), start, ("Ck", "Cv", "b")):
            np.testing.assert_array_equal(g[h][fz], s0[h][fz])
            err = np.abs(g[h] - r).max()
            print(f"head {h} {nm}: max |gpu - oracle| {err:.3e}", flush=True)
            assert err <= 0.05 * lr * steps, f"{name} head {h} {nm}: {err}"
        # the updates descend: the loss over every position (the oracle's, on the GPU's
        # fitted parameters) is below the starting one
        sa, sz = O.teacher_scales(Ofull[h], lfull[h], group)
        every = O.stage1_rows(np.arange(T), group)
        before = O.stage1_loss_grad(Qf[h], every, start[0][h], start[1][h], start[2][h],
                                    keypos[h], Ofull[h], lfull[h], sa, sz, scale, causal,
                                    group)[0]
        after = O.stage1_loss_grad(Qf[h], every, got[0][h], got[1][h], got[2][h], keypos[h],
                                   Ofull[h], lfull[h], sa, sz, scale, causal, group)[0]
        assert after < before, (before, after)


def test_stage1_loss_grad_full_size():
    """The timed configuration: 8 heads of 131072 queries (GQA 4, causal, 32768 positions),
    1024 slots, 128 positions per update. The targets are synthetic arrays of the right
    shape (the fit only reads them), so the oracle evaluates each head exactly."""
    import torch
    heads, d, T, t, group, S = 8, 128, 32768, 1024, 4, 128
    n = T * group
    rng = np.random.default_rng(77)
    Qb = synth.bf16_bits(rng.standard_normal((heads, n, d), dtype=np.float32))
    Ofull = (0.3 * rng.standard_normal((heads, n, d), dtype=np.float32)).astype(np.float32)
    lfull = (8.0 + 2.0 * rng.standard_normal((heads, n))).astype(np.float32)
    Ck = rng.standard_normal((heads, t, d)).astype(np.float32)
    Cv = rng.standard_normal((heads, t, d)).astype(np.float32)
    bias = (0.5 * rng.standard_normal((heads, t))).astype(np.float32)
    keypos = np.stack([np.sort(rng.choice(T, t, replace=False)) for _ in range(heads)])
    keypos[:, 0] = 0
    keypos = keypos.astype(np.int32)
    samples = synth.stage1_samples(T, 1, S)[0]
    scale = 1.0 / np.sqrt(d)
    dQ = to_dev(Qb, "bf16")
    L, gCk, gCv, gb = amc.stage1_loss_grad(
        dQ, torch.from_numpy(Ofull).cuda(), torch.from_numpy(lfull).cuda(),
        torch.from_numpy(samples).cuda(), torch.from_numpy(Ck).cuda(),
        torch.from_numpy(Cv).cuda(), torch.from_numpy(bias).cuda(),
        keypos=torch.from_numpy(keypos).cuda(), causal=True, group=group, scale=scale)
    L, gCk, gCv, gb = (x.cpu().numpy().astype(np.float64) for x in (L, gCk, gCv, gb))
    del dQ
    rows = O.stage1_rows(samples, group)
    Qf = synth.bf16_to_f32(Qb[:, rows]).astype(np.float64)   # only the sampled rows
    full_rows = np.zeros((n, d))   # the oracle indexes queries by row; only `rows` are read
    for h in range(heads):
        sa, sz = O.teacher_scales(Ofull[h], lfull[h], group)
        full_rows[rows] = Qf[h]
        ref = O.stage1_loss_grad(full_rows, rows, Ck[h].astype(np.float64),
                                 Cv[h].astype(np.float64), bias[h].astype(np.float64),
                                 keypos[h], Ofull[h], lfull[h], sa, sz, scale, True, group)
        assert abs(L[h] - ref[0]) <= 1e-4 * abs(ref[0]), (h, L[h], ref[0])
        for got, want, nm in zip((gCk[h], gCv[h], gb[h]), ref[1:], ("dCk", "dCv", "db")):
            err = np.abs(got - want).max()
            assert err <= 1e-3 * np.abs(want).max(), f"head {h} {nm}: max err {err}"


def test_stage1_fit_all_frozen_and_zero_rate():
    """No trainable slot, or a zero learning rate with zero decay: every parameter keeps its
    value exactly, while the losses are still evaluated (equal to the oracle's first)."""
    import torch
    case = CASES[0]
    name, heads, d, T, t, group, causal, dtype, S = case
    Q, Qf, Ckf, Cv, bias, keypos, Ofull, lfull, scale = _case(*case[:8], seed=5)
    samples = synth.stage1_samples(T, 3, S, seed=4)
    args = dict(keypos=torch.from_numpy(keypos).cuda(), causal=causal, group=group, scale=scale)
    Ck0, Cv0, b0 = _dev_params(Ckf, Cv, bias)
    for kw in (dict(trainable=torch.zeros((heads, t), dtype=torch.bool).cuda()),
               dict(lr=0.0, wd=0.0)):
        Ck1, Cv1, b1, losses = amc.fit_stage1(
            to_dev(Q, dtype), torch.from_numpy(Ofull).cuda(), torch.from_numpy(lfull).cuda(),
            torch.from_numpy(samples).cuda(), Ck0, Cv0, b0, **args, **kw)
        assert torch.equal(Ck1, Ck0) and torch.equal(Cv1, Cv0) and torch.equal(b1, b0)
        for h in range(heads):
            sa, sz = O.teacher_scales(Ofull[h], lfull[h], group)
            ref = O.stage1_loss_grad(Qf[h], O.stage1_rows(samples[0], group), Ckf[h], Cv[h],
                                     bias[h], keypos[h], Ofull[h], lfull[h], sa, sz, scale,
                                     causal, group)[0]
            got = losses.cpu().numpy()[:, h]
            assert np.all(np.isfinite(got))
            assert abs(got[0] - ref) <= 1e-4 * abs(ref)
