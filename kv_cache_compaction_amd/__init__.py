"""Attention-matching KV compaction on MI355X: Python binding of the C ABI (libamc.so).

The functions mirror include/am.h one to one. They only marshal arguments: every step of
the path runs in the library's gfx950 kernels. PyTorch supplies device memory (outputs and
workspace are torch tensors) and the stream (torch's current stream). If the library is
missing, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libamc.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "am.h")

AM_OK, AM_ERR_INVALID_ARG, AM_ERR_UNSUPPORTED, AM_ERR_WORKSPACE, AM_ERR_DEVICE = 0, -1, -2, -3, -4
AM_F32, AM_BF16 = 0, 1
SCORE_MODES = {"rms": 0, "mean": 1, "max": 2}
MASS_MODES = {"relative": 0, "absolute": 1}
(CALL_TARGETS, CALL_SELECT, CALL_FIT_BETA, CALL_FIT_VALUES, CALL_COMPACT, CALL_CACHE_ATTENTION,
 CALL_BETA_REDIST, CALL_EVAL, CALL_INIT) = range(9)
BETA_MODES = {"nnls": 0, "redistribute": 1}
VALUE_MODES = {"fit": 0, "direct": 1}
ABI_VERSION = 4
HEAD_NNLS_NOT_CONVERGED, HEAD_CHOL_PIVOT, HEAD_NONFINITE, HEAD_TIMEOUT = 1, 2, 4, 8


class AmProblem(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int64), ("n", ctypes.c_int64), ("T", ctypes.c_int64),
                ("d", ctypes.c_int64), ("causal", ctypes.c_int32), ("group", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int)]


class AmOptions(ctypes.Structure):
    _fields_ = [("score", ctypes.c_int), ("mass", ctypes.c_int), ("w_lo", ctypes.c_float),
                ("w_hi", ctypes.c_float), ("nnls_max_iter", ctypes.c_int32),
                ("nnls_tol", ctypes.c_float), ("ridge_lambda", ctypes.c_float),
                ("beta", ctypes.c_int), ("values", ctypes.c_int)]


class AmNnlsPlan(ctypes.Structure):
    _fields_ = [("workgroups_per_head", ctypes.c_int32), ("launches", ctypes.c_int32),
                ("heads_per_launch", ctypes.c_int32), ("rows_per_workgroup", ctypes.c_int32),
                ("lds_rows_per_workgroup", ctypes.c_int32)]


class AmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} ({status})")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_PROTOS = {
    "am_abi_version": (ctypes.c_int, []),
    "am_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "am_default_options": (None, [ctypes.POINTER(AmOptions)]),
    "am_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(AmProblem), ctypes.c_int64, ctypes.c_int]),
    "am_targets": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P, _P, _P, _P, ctypes.c_int,
                                  _P, ctypes.c_size_t, _P]),
    "am_select_keys": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, ctypes.c_int64, _P, _P, _P, _P,
                                      _P, _P, ctypes.c_size_t, _P]),
    "am_fit_beta_nnls": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P, _P, ctypes.c_int64,
                                        ctypes.POINTER(AmOptions), _P, _P, _P, _P, _P, _P, _P,
                                        ctypes.c_size_t, _P]),
    "am_fit_beta_plan": (ctypes.c_int, [ctypes.POINTER(AmProblem), ctypes.c_int64,
                                        ctypes.POINTER(AmNnlsPlan)]),
    "am_fit_values_ols": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P, _P, _P,
                                         ctypes.c_int64, ctypes.c_float, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]),
    "am_compact_head": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P, ctypes.c_int64,
                                       ctypes.POINTER(AmOptions), _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _P, ctypes.c_size_t, _P]),
    "am_compact_head_noalloc": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P,
                                               ctypes.c_int64, ctypes.POINTER(AmOptions), _P, _P,
                                               _P, _P, _P, _P, _P, _P, _P, _P]),
    "am_cache_attention": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P, _P, _P, _P,
                                          ctypes.c_int64, _P, _P, ctypes.c_int32, _P, _P, _P,
                                          _P, ctypes.c_size_t, _P]),
    "am_attention_merge": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _P, _P, _P,
                                          _P]),
    "am_beta_redistribute": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P, _P,
                                            ctypes.c_int64, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "am_select_two_pass": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P, _P, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int32, ctypes.c_int, _P, _P, _P,
                                          _P, _P, ctypes.c_size_t, _P]),
    "am_compact_two_pass": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P, _P, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int32, ctypes.c_int, _P, _P, _P,
                                           _P, _P, _P, ctypes.c_size_t, _P]),
    "am_two_pass_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(AmProblem), ctypes.c_int64,
                                                      ctypes.c_int64, ctypes.c_int32,
                                                      ctypes.c_int32]),
    "am_init_anchor_diverse": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, ctypes.c_int64,
                                              ctypes.c_int64, _P, _P, _P, _P, ctypes.c_size_t,
                                              _P]),
    "am_eval_residuals": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_int64, _P, _P, ctypes.c_size_t, _P]),
    "am_stage1_loss_grad": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P, _P, _P,
                                           ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _P,
                                           ctypes.c_size_t, _P]),
    "am_fit_stage1": (ctypes.c_int, [ctypes.POINTER(AmProblem), _P, _P, _P, _P, _P, ctypes.c_int64,
                                     ctypes.c_int64, _P, ctypes.c_float, ctypes.c_float, _P, _P,
                                     _P, _P, _P, ctypes.c_size_t, _P]),
    "am_stage1_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(AmProblem), ctypes.c_int64]),
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/am.h declares."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[a-z_]+\s*\*?\s+)+\*?(am_[a-z_]+)\s*\(", txt, re.M)))


def status_str(s: int) -> str:
    return lib().am_status_str(s).decode()


def _check(s: int, what: str):
    if s != AM_OK:
        raise AmError(s, what)


# ------------------------------------------------------------------------------------------
# marshalling helpers
# ------------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return AM_BF16
    if t.dtype == torch.float32:
        return AM_F32
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _need(t, name, *, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def make_problem(Q, K, *, causal=False, group=1, scale=None) -> AmProblem:
    h, n, d = Q.shape
    h2, T, d2 = K.shape
    if h2 != h or d2 != d:
        raise ValueError("Q [h, n, d] and K [h, T, d] disagree")
    if Q.dtype != K.dtype:
        raise TypeError("Q and K must share a dtype")
    return AmProblem(h, n, T, d, int(bool(causal)), int(group),
                     float(1.0 / math.sqrt(d) if scale is None else scale), _dtype_code(Q))


def make_options(score="rms", mass="relative", w_lo=0.0, w_hi=math.inf, nnls_max_iter=500,
                 nnls_tol=1e-6, ridge_lambda=1e-3, beta="nnls", values="fit") -> AmOptions:
    return AmOptions(SCORE_MODES[score], MASS_MODES[mass], w_lo, w_hi, nnls_max_iter, nnls_tol,
                     ridge_lambda, BETA_MODES[beta], VALUE_MODES[values])


def workspace_bytes(p: AmProblem, t: int, which: int) -> int:
    return int(lib().am_workspace_bytes(ctypes.byref(p), t, which))


def _workspace(p, t, which, device):
    torch = _torch()
    nb = max(workspace_bytes(p, t, which), 256)
    return torch.empty(nb, dtype=torch.uint8, device=device), nb


# ------------------------------------------------------------------------------------------
# the five calls
# ------------------------------------------------------------------------------------------
def targets(Q, K, V=None, *, causal=False, group=1, scale=None, score="rms", want_O=True,
            want_score=True):
    """lse [h, n], O [h, n, d] (or None) and key_score [h, T] (or None)."""
    torch = _torch()
    _need(Q, "Q"); _need(K, "K")
    p = make_problem(Q, K, causal=causal, group=group, scale=scale)
    if want_O:
        _need(V, "V", dtype=Q.dtype, shape=K.shape)
    dev = Q.device
    lse = torch.empty((p.heads, p.n), dtype=torch.float32, device=dev)
    O = torch.empty((p.heads, p.n, p.d), dtype=torch.float32, device=dev) if want_O else None
    sc = torch.empty((p.heads, p.T), dtype=torch.float32, device=dev) if want_score else None
    ws, nb = _workspace(p, 0, CALL_TARGETS, dev)
    _check(lib().am_targets(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V) if want_O else None,
                            _ptr(lse), _ptr(O), _ptr(sc), SCORE_MODES[score], _ptr(ws), nb,
                            _stream()), "am_targets")
    return lse, O, sc


def select_keys(key_score, K, t, V=None, *, want_vsel=False):
    """idx [h, t] int32 ascending, C_k [h, t, d] and (optionally) V[idx]."""
    torch = _torch()
    _need(K, "K")
    h, T, d = K.shape
    _need(key_score, "key_score", dtype=torch.float32, shape=(h, T))
    p = AmProblem(h, 1, T, d, 0, 1, 1.0 / math.sqrt(d), _dtype_code(K))
    idx = torch.empty((h, t), dtype=torch.int32, device=K.device)
    Ck = torch.empty((h, t, d), dtype=K.dtype, device=K.device)
    Vs = None
    if want_vsel:
        _need(V, "V", dtype=K.dtype, shape=K.shape)
        Vs = torch.empty_like(Ck)
    _check(lib().am_select_keys(ctypes.byref(p), _ptr(key_score), t, _ptr(K), _ptr(V), _ptr(idx),
                                _ptr(Ck), _ptr(Vs), None, 0, _stream()), "am_select_keys")
    return idx, Ck, Vs


def fit_beta_nnls(Q, Ck, idx, lse, *, causal=False, group=1, scale=None, options=None,
                  T=None, diagnostics=False):
    """beta [h, t], w [h, t], mass residual [h], head status [h]; with diagnostics=True also
    the relative KKT residual [h] (f32) and the projected-gradient step count [h] (int32)."""
    torch = _torch()
    _need(Q, "Q"); _need(Ck, "Ck", dtype=Q.dtype)
    h, n, d = Q.shape
    t = Ck.shape[1]
    _need(idx, "idx", dtype=torch.int32, shape=(h, t))
    _need(lse, "lse", dtype=torch.float32, shape=(h, n))
    Tk = T if T is not None else (n // group if causal else max(t, 1))
    p = AmProblem(h, n, Tk, d, int(bool(causal)), int(group),
                  float(1.0 / math.sqrt(d) if scale is None else scale), _dtype_code(Q))
    o = options or make_options()
    dev = Q.device
    beta = torch.empty((h, t), dtype=torch.float32, device=dev)
    w = torch.empty((h, t), dtype=torch.float32, device=dev)
    res = torch.empty((h,), dtype=torch.float32, device=dev)
    st = torch.empty((h,), dtype=torch.int32, device=dev)
    kkt = torch.empty((h,), dtype=torch.float32, device=dev) if diagnostics else None
    its = torch.empty((h,), dtype=torch.int32, device=dev) if diagnostics else None
    ws, nb = _workspace(p, t, CALL_FIT_BETA, dev)
    _check(lib().am_fit_beta_nnls(ctypes.byref(p), _ptr(Q), _ptr(Ck), _ptr(idx), _ptr(lse), t,
                                  ctypes.byref(o), _ptr(beta), _ptr(w), _ptr(res), _ptr(kkt),
                                  _ptr(its), _ptr(st), _ptr(ws), nb, _stream()),
           "am_fit_beta_nnls")
    if diagnostics:
        return beta, w, res, st, kkt, its
    return beta, w, res, st


def fit_beta_plan(heads, n, T, d, t, *, causal=False, group=1, dtype="bf16"):
    """How the NNLS of such a problem is scheduled on the current device (a dict of
    am_nnls_plan's fields)."""
    p = AmProblem(heads, n, T, d, int(bool(causal)), int(group), float(1.0 / math.sqrt(d)),
                  AM_BF16 if dtype == "bf16" else AM_F32)
    out = AmNnlsPlan()
    _check(lib().am_fit_beta_plan(ctypes.byref(p), t, ctypes.byref(out)), "am_fit_beta_plan")
    return {f: getattr(out, f) for f, _ in AmNnlsPlan._fields_}


def fit_values_ols(Q, Ck, idx, beta, O, *, causal=False, group=1, scale=None, ridge_lambda=1e-3,
                   T=None):
    """C_v [h, t, d] f32, output residual [h], head status [h]."""
    torch = _torch()
    _need(Q, "Q"); _need(Ck, "Ck", dtype=Q.dtype)
    h, n, d = Q.shape
    t = Ck.shape[1]
    _need(idx, "idx", dtype=torch.int32, shape=(h, t))
    _need(beta, "beta", dtype=torch.float32, shape=(h, t))
    _need(O, "O", dtype=torch.float32, shape=(h, n, d))
    Tk = T if T is not None else (n // group if causal else max(t, 1))
    p = AmProblem(h, n, Tk, d, int(bool(causal)), int(group),
                  float(1.0 / math.sqrt(d) if scale is None else scale), _dtype_code(Q))
    dev = Q.device
    Cv = torch.empty((h, t, d), dtype=torch.float32, device=dev)
    res = torch.empty((h,), dtype=torch.float32, device=dev)
    st = torch.empty((h,), dtype=torch.int32, device=dev)
    ws, nb = _workspace(p, t, CALL_FIT_VALUES, dev)
    _check(lib().am_fit_values_ols(ctypes.byref(p), _ptr(Q), _ptr(Ck), _ptr(idx), _ptr(beta),
                                   _ptr(O), t, float(ridge_lambda), _ptr(Cv), _ptr(res), _ptr(st),
                                   _ptr(ws), nb, _stream()), "am_fit_values_ols")
    return Cv, res, st


def compact_head(Q, K, V, t, *, causal=False, group=1, scale=None, options=None,
                 want_stats=True):
    """The whole path. Returns a dict of idx, Ck, beta, Cv, resid [2, h], status [h] and,
    with want_stats, lse, O and score."""
    torch = _torch()
    _need(Q, "Q"); _need(K, "K"); _need(V, "V", dtype=K.dtype, shape=K.shape)
    p = make_problem(Q, K, causal=causal, group=group, scale=scale)
    o = options or make_options()
    dev = Q.device
    h, n, T, d = p.heads, p.n, p.T, p.d
    out = dict(
        idx=torch.empty((h, t), dtype=torch.int32, device=dev),
        Ck=torch.empty((h, t, d), dtype=Q.dtype, device=dev),
        beta=torch.empty((h, t), dtype=torch.float32, device=dev),
        Cv=torch.empty((h, t, d), dtype=torch.float32, device=dev),
        resid=torch.empty((2, h), dtype=torch.float32, device=dev),
        status=torch.empty((h,), dtype=torch.int32, device=dev),
    )
    if want_stats:
        out["lse"] = torch.empty((h, n), dtype=torch.float32, device=dev)
        out["O"] = torch.empty((h, n, d), dtype=torch.float32, device=dev)
        out["score"] = torch.empty((h, T), dtype=torch.float32, device=dev)
    ws, nb = _workspace(p, t, CALL_COMPACT, dev)
    g = out.get
    _check(lib().am_compact_head(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), t, ctypes.byref(o),
                                 _ptr(out["idx"]), _ptr(out["Ck"]), _ptr(out["beta"]),
                                 _ptr(out["Cv"]), _ptr(g("lse")), _ptr(g("O")), _ptr(g("score")),
                                 _ptr(out["resid"]), _ptr(out["status"]), _ptr(ws), nb, _stream()),
           "am_compact_head")
    return out


NOALLOC_SCRATCH_BYTES = 128 << 20   # AM_NOALLOC_SCRATCH_BYTES of include/am.h


def compact_head_noalloc(Q, K, V, t, *, causal=False, group=1, scale=None, options=None,
                         want_stats=True):
    """compact_head through am_compact_head_noalloc: the library's fixed scratch array
    instead of a workspace (the outputs are still allocated here, by the caller)."""
    torch = _torch()
    _need(Q, "Q"); _need(K, "K"); _need(V, "V", dtype=K.dtype, shape=K.shape)
    p = make_problem(Q, K, causal=causal, group=group, scale=scale)
    o = options or make_options()
    dev = Q.device
    h, n, T, d = p.heads, p.n, p.T, p.d
    out = dict(
        idx=torch.empty((h, t), dtype=torch.int32, device=dev),
        Ck=torch.empty((h, t, d), dtype=Q.dtype, device=dev),
        beta=torch.empty((h, t), dtype=torch.float32, device=dev),
        Cv=torch.empty((h, t, d), dtype=torch.float32, device=dev),
        resid=torch.empty((2, h), dtype=torch.float32, device=dev),
        status=torch.empty((h,), dtype=torch.int32, device=dev),
    )
    if want_stats:
        out["lse"] = torch.empty((h, n), dtype=torch.float32, device=dev)
        out["O"] = torch.empty((h, n, d), dtype=torch.float32, device=dev)
        out["score"] = torch.empty((h, T), dtype=torch.float32, device=dev)
    g = out.get
    _check(lib().am_compact_head_noalloc(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), t,
                                         ctypes.byref(o), _ptr(out["idx"]), _ptr(out["Ck"]),
                                         _ptr(out["beta"]), _ptr(out["Cv"]), _ptr(g("lse")),
                                         _ptr(g("O")), _ptr(g("score")), _ptr(out["resid"]),
                                         _ptr(out["status"]), _stream()),
           "am_compact_head_noalloc")
    return out


def cache_attention(Q, Ck, Cv, bias, *, keypos=None, nvalid=None, Kn=None, Vn=None,
                    new_causal=True, causal=False, group=1, scale=None, want_lse_cmp=False):
    """Attention through a compacted cache (slots Ck, Cv f32, bias f32; optional original
    positions keypos for causal masking and per-head slot counts nvalid) followed by new
    entries Kn, Vn. Returns out [h, n, d], lse [h, n] and, with want_lse_cmp, log Z_cmp."""
    torch = _torch()
    _need(Q, "Q"); _need(Ck, "Ck")
    p = make_problem(Q, Ck, causal=causal, group=group, scale=scale)
    h, n, t, d = p.heads, p.n, p.T, p.d
    _need(Cv, "Cv", dtype=torch.float32, shape=(h, t, d))
    _need(bias, "bias", dtype=torch.float32, shape=(h, t))
    if keypos is not None:
        _need(keypos, "keypos", dtype=torch.int32, shape=(h, t))
    if nvalid is not None:
        _need(nvalid, "nvalid", dtype=torch.int32, shape=(h,))
    m = 0
    if Kn is not None:
        _need(Kn, "Kn", dtype=Q.dtype)
        m = Kn.shape[1]
        _need(Vn, "Vn", dtype=Q.dtype, shape=Kn.shape)
        if Kn.shape[0] != h or Kn.shape[2] != d:
            raise ValueError("Kn must be [h, m, d]")
    dev = Q.device
    out = torch.empty((h, n, d), dtype=torch.float32, device=dev)
    lse = torch.empty((h, n), dtype=torch.float32, device=dev)
    lz1 = torch.empty((h, n), dtype=torch.float32, device=dev) if want_lse_cmp else None
    ws, nb = _workspace(p, m, CALL_CACHE_ATTENTION, dev)
    _check(lib().am_cache_attention(ctypes.byref(p), _ptr(Q), _ptr(Ck), _ptr(Cv), _ptr(bias),
                                    _ptr(keypos), _ptr(nvalid), m, _ptr(Kn) if m else None,
                                    _ptr(Vn) if m else None, int(bool(new_causal)), _ptr(out),
                                    _ptr(lse), _ptr(lz1), _ptr(ws), nb, _stream()),
           "am_cache_attention")
    return (out, lse, lz1) if want_lse_cmp else (out, lse)


def attention_merge(O1, lse1, O2, lse2, *, out=None, lse_out=None):
    """Log-space merge of two attention results over disjoint entry sets (Eq. 5).
    O1, O2 [..., d] f32 and lse1, lse2 [...] f32; returns (out, lse)."""
    torch = _torch()
    for x, nm in ((O1, "O1"), (O2, "O2"), (lse1, "lse1"), (lse2, "lse2")):
        _need(x, nm, dtype=torch.float32)
    if O1.shape != O2.shape or lse1.shape != lse2.shape or tuple(O1.shape[:-1]) != tuple(lse1.shape):
        raise ValueError("O1, O2 [..., d] and lse1, lse2 [...] must agree")
    d = O1.shape[-1]
    rows = lse1.numel()
    out = torch.empty_like(O1) if out is None else out
    lse_out = torch.empty_like(lse1) if lse_out is None else lse_out
    _need(out, "out", dtype=torch.float32, shape=O1.shape)
    _need(lse_out, "lse_out", dtype=torch.float32, shape=lse1.shape)
    _check(lib().am_attention_merge(rows, d, _ptr(O1), _ptr(lse1), _ptr(O2), _ptr(lse2), _ptr(out),
                                    _ptr(lse_out), _stream()), "am_attention_merge")
    return out, lse_out


def beta_redistribute(Q, Ck, idx, lse, *, causal=False, group=1, scale=None, T=None):
    """beta by uniform redistribution of the missing mass; returns (beta, w, mass_resid).
    T (full-cache keys) is only used to describe the problem (causal needs n == group * T)."""
    torch = _torch()
    _need(Q, "Q"); _need(Ck, "Ck")
    h, n, d = Q.shape
    t = Ck.shape[1]
    _need(idx, "idx", dtype=torch.int32, shape=(h, t))
    _need(lse, "lse", dtype=torch.float32, shape=(h, n))
    T = T if T is not None else (n // group if causal else max(t, 1))
    p = AmProblem(h, n, T, d, int(bool(causal)), int(group),
                  float(1.0 / math.sqrt(d) if scale is None else scale), _dtype_code(Q))
    dev = Q.device
    beta = torch.empty((h, t), dtype=torch.float32, device=dev)
    w = torch.empty((h, t), dtype=torch.float32, device=dev)
    res = torch.empty((h,), dtype=torch.float32, device=dev)
    ws, nb = _workspace(p, t, CALL_BETA_REDIST, dev)
    _check(lib().am_beta_redistribute(ctypes.byref(p), _ptr(Q), _ptr(Ck), _ptr(idx), _ptr(lse), t,
                                      _ptr(beta), _ptr(w), _ptr(res), _ptr(ws), nb, _stream()),
           "am_beta_redistribute")
    return beta, w, res


def eval_residuals(Q, K, V, idx, Ck, beta, Cv, *, causal=False, group=1, scale=None):
    """[2, h] mass and output residuals of a compacted cache on the queries Q."""
    torch = _torch()
    _need(Q, "Q"); _need(K, "K"); _need(V, "V", dtype=K.dtype, shape=K.shape)
    p = make_problem(Q, K, causal=causal, group=group, scale=scale)
    h, t, d = p.heads, Ck.shape[1], p.d
    _need(Ck, "Ck", dtype=Q.dtype, shape=(h, t, d))
    _need(idx, "idx", dtype=torch.int32, shape=(h, t))
    _need(beta, "beta", dtype=torch.float32, shape=(h, t))
    _need(Cv, "Cv", dtype=torch.float32, shape=(h, t, d))
    res = torch.empty((2, h), dtype=torch.float32, device=Q.device)
    ws, nb = _workspace(p, t, CALL_EVAL, Q.device)
    _check(lib().am_eval_residuals(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _ptr(Ck),
                                   _ptr(beta), _ptr(Cv), t, _ptr(res), _ptr(ws), nb, _stream()),
           "am_eval_residuals")
    return res


def _two_pass_setup(Q, K, sub, t, k_mult, causal, group, scale, compact):
    torch = _torch()
    _need(Q, "Q"); _need(K, "K")
    p = make_problem(Q, K, causal=causal, group=group, scale=scale)
    _need(sub, "sub", dtype=torch.int32)
    if sub.dim() != 2 or sub.shape[0] != p.heads:
        raise ValueError("sub must be [h, s]")
    s = sub.shape[1]
    nb = int(lib().am_two_pass_workspace_bytes(ctypes.byref(p), t, s, int(k_mult), int(compact)))
    if nb == 0:
        raise AmError(AM_ERR_INVALID_ARG, "am_two_pass_workspace_bytes")
    ws = torch.empty(nb, dtype=torch.uint8, device=Q.device)
    return p, s, ws, nb


def select_two_pass(Q, K, sub, t, *, V=None, k_mult=4, score="rms", causal=False, group=1,
                    scale=None):
    """Two-pass selection from the query subset sub [h, s] (ascending int32 indices).
    Returns idx [h, t], Ck [h, t, d], V_sel (or None) and lse over the shortlist [h, n]."""
    torch = _torch()
    p, s, ws, nb = _two_pass_setup(Q, K, sub, t, k_mult, causal, group, scale, 0)
    h, n, d = p.heads, p.n, p.d
    idx = torch.empty((h, t), dtype=torch.int32, device=Q.device)
    Ck = torch.empty((h, t, d), dtype=Q.dtype, device=Q.device)
    Vs = None
    if V is not None:
        _need(V, "V", dtype=K.dtype, shape=K.shape)
        Vs = torch.empty_like(Ck)
    lse = torch.empty((h, n), dtype=torch.float32, device=Q.device)
    _check(lib().am_select_two_pass(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(sub), s, t,
                                    int(k_mult), SCORE_MODES[score], _ptr(idx), _ptr(Ck), _ptr(Vs),
                                    _ptr(lse), _ptr(ws), nb, _stream()), "am_select_two_pass")
    return idx, Ck, Vs, lse


def compact_two_pass(Q, K, V, sub, t, *, k_mult=4, score="rms", causal=False, group=1,
                     scale=None):
    """The blog's two-pass method: two-pass selection, redistributed beta, direct values.
    Returns a dict of idx, Ck, beta, Cv and resid [2, h] (row 1 is -1: not computed)."""
    torch = _torch()
    _need(V, "V", dtype=K.dtype, shape=K.shape)
    p, s, ws, nb = _two_pass_setup(Q, K, sub, t, k_mult, causal, group, scale, 1)
    h, d = p.heads, p.d
    out = dict(idx=torch.empty((h, t), dtype=torch.int32, device=Q.device),
               Ck=torch.empty((h, t, d), dtype=Q.dtype, device=Q.device),
               beta=torch.empty((h, t), dtype=torch.float32, device=Q.device),
               Cv=torch.empty((h, t, d), dtype=torch.float32, device=Q.device),
               resid=torch.empty((2, h), dtype=torch.float32, device=Q.device))
    _check(lib().am_compact_two_pass(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(sub), s, t,
                                     int(k_mult), SCORE_MODES[score], _ptr(out["idx"]),
                                     _ptr(out["Ck"]), _ptr(out["beta"]), _ptr(out["Cv"]),
                                     _ptr(out["resid"]), _ptr(ws), nb, _stream()),
           "am_compact_two_pass")
    return out


def init_anchor_diverse(Q, K, M, *, n_anchor=None, causal=False, group=1, scale=None):
    """Anchor + diversifier initialization of an M-slot budget (n_anchor defaults to M // 4,
    at least 1). Returns idx [h, M] ascending, the selection order [h, M] and status [h]."""
    torch = _torch()
    _need(Q, "Q"); _need(K, "K")
    p = make_problem(Q, K, causal=causal, group=group, scale=scale)
    na = max(1, M // 4) if n_anchor is None else int(n_anchor)
    dev = Q.device
    idx = torch.empty((p.heads, M), dtype=torch.int32, device=dev)
    order = torch.empty((p.heads, M), dtype=torch.int32, device=dev)
    status = torch.empty((p.heads,), dtype=torch.int32, device=dev)
    ws, nb = _workspace(p, M, CALL_INIT, dev)
    _check(lib().am_init_anchor_diverse(ctypes.byref(p), _ptr(Q), _ptr(K), M, na, _ptr(idx),
                                        _ptr(order), _ptr(status), _ptr(ws), nb, _stream()),
           "am_init_anchor_diverse")
    return idx, order, status


def _stage1_setup(Q, O_full, lse_full, keypos, Ck, Cv, bias, samples, causal, group, scale):
    torch = _torch()
    _need(Q, "Q")
    h, n, d = Q.shape
    _need(O_full, "O_full", dtype=torch.float32, shape=(h, n, d))
    _need(lse_full, "lse_full", dtype=torch.float32, shape=(h, n))
    _need(Ck, "Ck", dtype=torch.float32)
    t = Ck.shape[1]
    if Ck.dim() != 3 or Ck.shape[0] != h or Ck.shape[2] != d:
        raise ValueError("Ck must be [h, t, d]")
    _need(Cv, "Cv", dtype=torch.float32, shape=(h, t, d))
    _need(bias, "bias", dtype=torch.float32, shape=(h, t))
    if keypos is not None:
        _need(keypos, "keypos", dtype=torch.int32, shape=(h, t))
    _need(samples, "samples", dtype=torch.int32)
    S = samples.shape[-1]
    p = AmProblem(h, n, t, d, int(bool(causal)), int(group),
                  float(1.0 / math.sqrt(d) if scale is None else scale), _dtype_code(Q))
    nb = int(lib().am_stage1_workspace_bytes(ctypes.byref(p), S))
    if nb == 0:
        raise AmError(AM_ERR_INVALID_ARG, "am_stage1_workspace_bytes")
    ws = torch.empty(nb, dtype=torch.uint8, device=Q.device)
    return p, S, ws, nb


def stage1_loss_grad(Q, O_full, lse_full, samples, Ck, Cv, bias, *, keypos=None, causal=False,
                     group=1, scale=None):
    """Stage-1 loss [h] and its gradients (dCk, dCv, dbias) at the positions samples [S]
    (int32), for f32 parameters Ck, Cv [h, t, d] and bias [h, t]."""
    torch = _torch()
    p, S, ws, nb = _stage1_setup(Q, O_full, lse_full, keypos, Ck, Cv, bias, samples, causal,
                                 group, scale)
    if samples.dim() != 1:
        raise ValueError("samples must be [S]")
    loss = torch.empty((p.heads,), dtype=torch.float32, device=Q.device)
    gCk, gCv, gb = torch.empty_like(Ck), torch.empty_like(Cv), torch.empty_like(bias)
    _check(lib().am_stage1_loss_grad(ctypes.byref(p), _ptr(Q), _ptr(O_full), _ptr(lse_full),
                                     _ptr(keypos), _ptr(samples), S, _ptr(Ck), _ptr(Cv),
                                     _ptr(bias), _ptr(loss), _ptr(gCk), _ptr(gCv), _ptr(gb),
                                     _ptr(ws), nb, _stream()), "am_stage1_loss_grad")
    return loss, gCk, gCv, gb


def fit_stage1(Q, O_full, lse_full, samples, Ck, Cv, bias, *, keypos=None, trainable=None,
               lr=3e-3, wd=1e-2, causal=False, group=1, scale=None):
    """Stage-1 fitting: one AdamW update per row of samples [steps, S] (int32 positions).
    Ck, Cv, bias are copied to f32 and returned fitted with the per-update losses
    [steps, h]; trainable [h, t] (bool or uint8) freezes the slots where it is 0."""
    torch = _torch()
    Ck = Ck.to(torch.float32).contiguous().clone()
    Cv = Cv.to(torch.float32).contiguous().clone()
    bias = bias.to(torch.float32).contiguous().clone()
    p, S, ws, nb = _stage1_setup(Q, O_full, lse_full, keypos, Ck, Cv, bias, samples, causal,
                                 group, scale)
    if samples.dim() != 2:
        raise ValueError("samples must be [steps, S]")
    steps = samples.shape[0]
    tr = None
    if trainable is not None:
        tr = trainable.to(torch.uint8).contiguous()
        if tuple(tr.shape) != (p.heads, p.T):
            raise ValueError("trainable must be [h, t]")
    loss = torch.empty((steps, p.heads), dtype=torch.float32, device=Q.device)
    _check(lib().am_fit_stage1(ctypes.byref(p), _ptr(Q), _ptr(O_full), _ptr(lse_full),
                               _ptr(keypos), _ptr(samples), S, steps, _ptr(tr), float(lr),
                               float(wd), _ptr(Ck), _ptr(Cv), _ptr(bias), _ptr(loss), _ptr(ws),
                               nb, _stream()), "am_fit_stage1")
    return Ck, Cv, bias, loss
