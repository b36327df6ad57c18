"""The C ABI on the host: the library loads, exports what include/am.h declares, and
rejects bad arguments before any device work (no GPU is touched by these tests)."""
import ctypes
import math

import pytest

import kv_cache_compaction_amd as amc

FAKE = 0x10000  # aligned, never dereferenced: validation fails before any launch


def P(**kw):
    base = dict(heads=2, n=256, T=128, d=128, causal=0, group=1, scale=1 / math.sqrt(128),
                dtype=amc.AM_BF16)
    base.update(kw)
    return amc.AmProblem(base["heads"], base["n"], base["T"], base["d"], base["causal"],
                         base["group"], base["scale"], base["dtype"])


def test_exports_every_declared_symbol():
    L = amc.lib()
    names = amc.header_functions()
    assert {"am_targets", "am_select_keys", "am_fit_beta_nnls", "am_fit_values_ols",
            "am_compact_head", "am_workspace_bytes", "am_status_str", "am_abi_version",
            "am_default_options"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings():
    assert amc.lib().am_abi_version() == amc.ABI_VERSION == 4
    assert amc.status_str(0) == "ok"
    assert amc.status_str(-3) == "workspace too small"
    assert amc.status_str(7) == "unknown status"


def test_default_options():
    o = amc.AmOptions()
    amc.lib().am_default_options(ctypes.byref(o))
    assert o.score == 0 and o.mass == 0 and o.w_lo == 0 and math.isinf(o.w_hi)
    assert o.nnls_max_iter == 500 and o.ridge_lambda == pytest.approx(1e-3)
    assert o.beta == 0 and o.values == 0


def test_workspace_sizes():
    p = P()
    for which in range(5):
        assert amc.workspace_bytes(p, 16, which) >= 0
    assert amc.workspace_bytes(p, 0, amc.CALL_TARGETS) > 0
    assert amc.workspace_bytes(P(d=96), 16, amc.CALL_TARGETS) == 0      # unsupported d
    assert amc.workspace_bytes(p, 0, amc.CALL_FIT_BETA) == 0            # t < 1
    assert amc.workspace_bytes(p, 129, amc.CALL_FIT_BETA) == 0          # t > T


def _targets(p, Q=FAKE, K=FAKE, V=FAKE, lse=FAKE, O=FAKE, sc=FAKE, mode=0, ws=FAKE, nb=1 << 40):
    return amc.lib().am_targets(ctypes.byref(p) if p is not None else None, Q, K, V, lse, O, sc,
                                mode, ws, nb, None)


def test_targets_validation():
    assert _targets(None) == amc.AM_ERR_INVALID_ARG
    assert _targets(P(), Q=None) == amc.AM_ERR_INVALID_ARG
    assert _targets(P(), lse=None) == amc.AM_ERR_INVALID_ARG
    assert _targets(P(), V=None) == amc.AM_ERR_INVALID_ARG          # O wanted without V
    assert _targets(P(), K=FAKE + 8) == amc.AM_ERR_INVALID_ARG      # misaligned
    assert _targets(P(d=96)) == amc.AM_ERR_UNSUPPORTED
    assert _targets(P(heads=0)) == amc.AM_ERR_INVALID_ARG
    assert _targets(P(n=0)) == amc.AM_ERR_INVALID_ARG
    assert _targets(P(group=0)) == amc.AM_ERR_INVALID_ARG
    assert _targets(P(causal=1, group=4, n=100, T=50)) == amc.AM_ERR_INVALID_ARG
    assert _targets(P(scale=-1.0)) == amc.AM_ERR_INVALID_ARG
    assert _targets(P(scale=float("nan"))) == amc.AM_ERR_INVALID_ARG
    assert _targets(P(dtype=5)) == amc.AM_ERR_INVALID_ARG
    assert _targets(P(), mode=3) == amc.AM_ERR_INVALID_ARG
    assert _targets(P(), nb=16) == amc.AM_ERR_WORKSPACE
    assert _targets(P(), ws=None) == amc.AM_ERR_WORKSPACE


def test_select_validation():
    L = amc.lib()
    p = P()
    f = lambda t, **kw: L.am_select_keys(ctypes.byref(p), kw.get("sc", FAKE), t, FAKE,
                                         kw.get("V", FAKE), kw.get("idx", FAKE), FAKE,
                                         kw.get("Vs", None), None, 0, None)
    assert f(0) == amc.AM_ERR_INVALID_ARG
    assert f(129) == amc.AM_ERR_INVALID_ARG
    assert f(4, sc=None) == amc.AM_ERR_INVALID_ARG
    assert f(4, idx=FAKE + 4) == amc.AM_ERR_INVALID_ARG
    assert f(4, V=None, Vs=FAKE) == amc.AM_ERR_INVALID_ARG


def test_fit_validation():
    L = amc.lib()
    p = P()
    o = amc.make_options()
    fb = lambda t, opt, nb=1 << 40, **kw: L.am_fit_beta_nnls(
        ctypes.byref(p), FAKE, FAKE, FAKE, kw.get("lse", FAKE), t, ctypes.byref(opt)
        if opt is not None else None, FAKE, None, None, kw.get("kkt"), kw.get("iters"), None,
        FAKE, nb, None)
    assert fb(0, o) == amc.AM_ERR_INVALID_ARG
    assert fb(4, None) == amc.AM_ERR_INVALID_ARG
    assert fb(4, o, lse=None) == amc.AM_ERR_INVALID_ARG
    assert fb(4, amc.make_options(w_lo=2.0, w_hi=1.0)) == amc.AM_ERR_INVALID_ARG
    assert fb(4, amc.make_options(w_lo=-1.0)) == amc.AM_ERR_INVALID_ARG
    assert fb(4, amc.make_options(nnls_max_iter=0)) == amc.AM_ERR_INVALID_ARG
    assert fb(4, amc.make_options(score="max", mass="absolute", ridge_lambda=-1.0)) == amc.AM_ERR_INVALID_ARG
    assert fb(4, o, nb=8) == amc.AM_ERR_WORKSPACE
    assert fb(4, o, kkt=FAKE + 4) == amc.AM_ERR_INVALID_ARG     # misaligned diagnostics
    assert fb(4, o, iters=FAKE + 8) == amc.AM_ERR_INVALID_ARG
    assert fb(4, o, nb=8, kkt=FAKE, iters=FAKE) == amc.AM_ERR_WORKSPACE
    plan = amc.AmNnlsPlan()
    assert L.am_fit_beta_plan(ctypes.byref(p), 0, ctypes.byref(plan)) == amc.AM_ERR_INVALID_ARG
    assert L.am_fit_beta_plan(ctypes.byref(p), 4, None) == amc.AM_ERR_INVALID_ARG
    assert L.am_fit_beta_plan(ctypes.byref(P(d=96)), 4, ctypes.byref(plan)) == \
        amc.AM_ERR_UNSUPPORTED
    fv = lambda t, lam, nb=1 << 40: L.am_fit_values_ols(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE,
                                                       FAKE, t, lam, FAKE, None, None, FAKE, nb,
                                                       None)
    assert fv(4, -1.0) == amc.AM_ERR_INVALID_ARG
    assert fv(4, float("inf")) == amc.AM_ERR_INVALID_ARG
    assert fv(200, 1e-3) == amc.AM_ERR_INVALID_ARG
    assert fv(4, 1e-3, nb=8) == amc.AM_ERR_WORKSPACE
    fc = lambda t, nb: L.am_compact_head(ctypes.byref(p), FAKE, FAKE, FAKE, t, ctypes.byref(o),
                                         FAKE, FAKE, FAKE, FAKE, None, None, None, None, None,
                                         FAKE, nb, None)
    assert fc(4, 8) == amc.AM_ERR_WORKSPACE
    assert fc(0, 1 << 40) == amc.AM_ERR_INVALID_ARG
    # the allocation-free variant: problems beyond its fixed scratch are refused, invalid
    # ones get am_compact_head's error, and neither launches anything
    fn = lambda pp, t: L.am_compact_head_noalloc(ctypes.byref(pp), FAKE, FAKE, FAKE, t,
                                                 ctypes.byref(o), FAKE, FAKE, FAKE, FAKE, None,
                                                 None, None, None, None, None)
    big = P(heads=8, n=1 << 20, T=1 << 16, causal=1, group=16)
    assert amc.workspace_bytes(big, 64, amc.CALL_COMPACT) > amc.NOALLOC_SCRATCH_BYTES
    assert fn(big, 64) == amc.AM_ERR_WORKSPACE
    assert fn(p, 0) == amc.AM_ERR_INVALID_ARG
    assert fn(P(d=96), 4) == amc.AM_ERR_UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 64)
    with pytest.raises(TypeError):
        amc.targets(q, q, q)


def test_new_calls_validation():
    L = amc.lib()
    p = P()
    ws = amc.workspace_bytes(p, 16, amc.CALL_CACHE_ATTENTION)
    assert ws > 0
    assert amc.workspace_bytes(p, 16, amc.CALL_BETA_REDIST) > 0
    assert amc.workspace_bytes(p, 16, amc.CALL_EVAL) > amc.workspace_bytes(p, 16, amc.CALL_BETA_REDIST)
    # cache attention: m < 0, bad new_causal, missing keypos under causal, small workspace
    args = dict(Q=FAKE, Ck=FAKE, Cv=FAKE, bias=FAKE, keypos=None, nvalid=None, m=4, Kn=FAKE,
                Vn=FAKE, nc=1, out=FAKE, lse=FAKE, lz=None, ws=FAKE, nb=1 << 40)

    def ca(pp, **kw):
        a = dict(args, **kw)
        return L.am_cache_attention(ctypes.byref(pp), a["Q"], a["Ck"], a["Cv"], a["bias"],
                                    a["keypos"], a["nvalid"], a["m"], a["Kn"], a["Vn"], a["nc"],
                                    a["out"], a["lse"], a["lz"], a["ws"], a["nb"], None)
    assert ca(p, m=-1) == amc.AM_ERR_INVALID_ARG
    assert ca(p, nc=2) == amc.AM_ERR_INVALID_ARG
    assert ca(P(causal=1), keypos=None) == amc.AM_ERR_INVALID_ARG
    assert ca(p, Kn=None) == amc.AM_ERR_INVALID_ARG
    assert ca(p, nb=16) == amc.AM_ERR_WORKSPACE
    assert ca(p, Q=FAKE + 4) == amc.AM_ERR_INVALID_ARG
    assert ca(P(d=96)) == amc.AM_ERR_UNSUPPORTED
    # merge: d must be a positive multiple of 4
    assert L.am_attention_merge(10, 6, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == amc.AM_ERR_INVALID_ARG
    assert L.am_attention_merge(10, 8, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == amc.AM_ERR_INVALID_ARG
    assert L.am_attention_merge(0, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == amc.AM_OK
    # redistribution and evaluation: t range, workspace
    assert L.am_beta_redistribute(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, None,
                                  FAKE, 1 << 40, None) == amc.AM_ERR_INVALID_ARG
    assert L.am_beta_redistribute(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 16, FAKE, None, None,
                                  FAKE, 16, None) == amc.AM_ERR_WORKSPACE
    assert L.am_eval_residuals(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 129,
                               FAKE, FAKE, 1 << 40, None) == amc.AM_ERR_INVALID_ARG
    assert L.am_eval_residuals(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 16,
                               FAKE, FAKE, 1 << 40, None) == amc.AM_ERR_INVALID_ARG


def test_option_modes_validated():
    L = amc.lib()
    p = P()
    o = amc.make_options()
    o.beta = 5
    assert L.am_compact_head(ctypes.byref(p), FAKE, FAKE, FAKE, 16, ctypes.byref(o), FAKE, FAKE,
                             FAKE, FAKE, None, None, None, None, None, FAKE, 1 << 40,
                             None) == amc.AM_ERR_INVALID_ARG
    o = amc.make_options(values="direct")
    o.values = -1
    assert L.am_compact_head(ctypes.byref(p), FAKE, FAKE, FAKE, 16, ctypes.byref(o), FAKE, FAKE,
                             FAKE, FAKE, None, None, None, None, None, FAKE, 1 << 40,
                             None) == amc.AM_ERR_INVALID_ARG


def test_stage1_validation():
    L = amc.lib()
    p = P(n=256, T=32, group=2, causal=1)
    assert L.am_stage1_workspace_bytes(ctypes.byref(p), 16) > 0
    assert L.am_stage1_workspace_bytes(ctypes.byref(p), 0) == 0
    assert L.am_stage1_workspace_bytes(ctypes.byref(P(n=255, T=32, group=2)), 16) == 0
    big = 1 << 40

    def fit(pp, S=16, steps=4, lr=3e-3, wd=1e-2, keypos=FAKE, Ck=FAKE, nb=big, samples=FAKE):
        return L.am_fit_stage1(ctypes.byref(pp), FAKE, FAKE, FAKE, keypos, samples, S, steps,
                               None, lr, wd, Ck, FAKE, FAKE, None, FAKE, nb, None)
    assert fit(p, steps=0) == amc.AM_ERR_INVALID_ARG
    assert fit(p, S=0) == amc.AM_ERR_INVALID_ARG
    assert fit(p, lr=-1.0) == amc.AM_ERR_INVALID_ARG
    assert fit(p, wd=float("nan")) == amc.AM_ERR_INVALID_ARG
    assert fit(p, keypos=None) == amc.AM_ERR_INVALID_ARG       # causal needs positions
    assert fit(p, Ck=None) == amc.AM_ERR_INVALID_ARG
    assert fit(p, samples=FAKE + 4) == amc.AM_ERR_INVALID_ARG  # misaligned
    assert fit(p, nb=64) == amc.AM_ERR_WORKSPACE
    assert fit(P(n=256, T=32, group=2, d=96)) == amc.AM_ERR_UNSUPPORTED
    assert L.am_stage1_loss_grad(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE,
                                 FAKE, None, FAKE, None, FAKE, FAKE, big,
                                 None) == amc.AM_ERR_INVALID_ARG   # gCv missing
    assert L.am_stage1_loss_grad(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE,
                                 FAKE, None, FAKE, FAKE, FAKE, FAKE, 8,
                                 None) == amc.AM_ERR_WORKSPACE
