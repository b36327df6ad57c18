"""Benchmark of the attention-matching compaction path on one MI355X.

One step is one am_compact_head call over the whole batch of the workload: full-cache
statistics (flash pass + column-score pass), top-t selection, the beta fit and the
value fit, with inputs already resident in HBM. The headline workload is the long
causal GQA layer (8 KV heads, T = 32768 keys, 131072 queries per KV head, t = 1024).

value = causally visible query-key pairs of the batch / step time (pairs/s).
roofline = the flash pass (the dominant kernel): 4 d flops per visible pair (Q K^T and
P V on bf16 MFMA) over its average duration, timed with HIP events on the stream the
library launches on, against the bf16 dense MFMA peak.
cpu_baseline = the float64 oracle, stage by stage (S1 targets, S2 scores, S3 selection,
S4+S5 beta fit, S6+S7 value fit), on a bounded sample: 24576 evenly spaced query rows of
head 0 with every key they see; its whole-step rate is reported beside the GPU's, with the
host's CPU model, BLAS thread count and library versions.
next = the adjacent rows, timed on the same inputs: the fast pipeline (redistributed beta,
direct values), the two-pass method (256-query subset, shortlist of 4t keys, then the fast
fits), the anchor + diversifier initialization of a t/4-slot budget, the held-out
evaluation, and attention through the compacted cache with 4096
appended tokens (GQA 4) merged in log space. The pairs/s of the pipelines count the
full workload's visible pairs (the work they stand in for), not the pairs they score.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "query·key pairs/sec (and TFLOP/s, % MFMA peak) per KV head at T=32K, 32×"
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3    # MI355X fp32 (used for fp32-input workloads)
HBM_PEAK_GBS = 8000.0


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "flash_fwd_causal8_T32k_gqa4_traffic.txt")


def flash_traffic(workload: str):
    """HBM bytes per flash-pass launch from the committed counter profile, or None when the
    profile is for another workload or the kernel source changed since it was taken."""
    import hashlib
    if workload != "causal8_T32k_gqa4" or not os.path.exists(TRAFFIC_PROFILE):
        return None
    kv = {}
    for line in open(TRAFFIC_PROFILE):
        if ":" in line and not line.startswith((" ", "#")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    src = os.path.join(ROOT, kv.get("source", ""))
    if not os.path.isfile(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("source_sha256"):
        return None
    return float(kv["traffic_bytes_per_launch"])


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_calls(torch, fn, reps, warm=True):
    """Average ms of fn() over reps calls, bracketed by events on the current stream; with
    warm, after one untimed call (first-launch costs of the call's kernels stay out)."""
    e0, e1 = _events(torch)
    if warm:
        fn()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def host_info():
    """CPU model, BLAS library and thread count, numpy/scipy versions of the host."""
    import numpy as np
    import scipy
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = {}
    try:
        import threadpoolctl
        for d in threadpoolctl.threadpool_info():
            if d.get("user_api") == "blas":
                blas = {"blas": f"{d.get('internal_api')} {d.get('version')}",
                        "blas_threads": d.get("num_threads")}
                break
    except Exception:   # threadpoolctl missing or failing: report what is known
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count(), **blas,
            "numpy": np.__version__, "scipy": scipy.__version__}


def cpu_baseline(w, Q, K, V, rows_max=24576):
    """The float64 oracle stage by stage on a bounded sample of the workload: m evenly
    spaced query rows of head 0 with every key they see. S1 = lse and outputs
    (attention_rows), S2 = the per-key statistics (a second pass over the same scores, as
    the device does), S3 = top-t on the sample's RMS scores, S4+S5 = mass design + NNLS,
    S6+S7 = value design + ridge solve, both on the sample rows. Returns the whole-step
    rate (sample pairs / the five stages' time), per-stage seconds and host metadata."""
    import numpy as np

    from kv_cache_compaction_amd import synth
    from oracle import am_oracle as O

    q = synth.as_f64(Q[0], w.dtype)
    k = synth.as_f64(K[0], w.dtype)
    v = synth.as_f64(V[0], w.dtype)
    m = min(w.n, rows_max)
    rows = np.linspace(0, w.n - 1, m).astype(np.int64)
    pairs = int((rows // w.group + 1).sum()) if w.causal else m * w.T
    st = {}
    t0 = time.perf_counter()
    lse, Oo = O.attention_rows(q, k, v, w.scale, rows, w.causal, w.group)
    st["S1"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    _, _, stats = O.full_cache_stats(q[rows], k, k, w.scale, w.causal, w.group, want_O=False,
                                     rows=rows)
    st["S2"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    idx = O.select_top(O.key_score(stats, "rms", m), w.t)
    st["S3"] = time.perf_counter() - t0
    fits = m >= 8 * w.t   # fewer rows than that leave the NNLS rank-deficient and slow
    if fits:
        t0 = time.perf_counter()
        M, b = O.mass_design(q[rows], k[idx], idx, lse, w.scale, w.causal, w.group, rows=rows)
        wv, _ = O.fit_beta(M, b)
        st["S4+S5"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        O.fit_values(O.value_design(M, wv), Oo, w.ridge_lambda)
        st["S6+S7"] = time.perf_counter() - t0
    total = sum(st.values())
    info = host_info()
    return {"value": pairs / total, "unit": "pairs/s",
            "cores": info.get("blas_threads") or info["cpu_count"], "kind": "oracle",
            "sample": f"head 0, {m} evenly spaced query rows with every key they see "
                      f"({pairs} visible pairs), all five stages in float64 "
                      f"({'S1-S7' if fits else 'S1-S3 only'}), {total:.1f} s",
            "stages_s": st, "host": info}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="causal8_T32k_gqa4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run one plain 256 MiB device copy; hardware "
                         "byte counters of that copy calibrate the HBM traffic of the kernels")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the per-head problems shard across GPUs without communication)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_compaction_amd as amc
    from kv_cache_compaction_amd import synth
    from kv_cache_compaction_amd.configs import BY_NAME

    w = BY_NAME[args.workload]
    torch.cuda.set_device(0)
    t0 = time.time()
    Q, K, V = synth.make_batch(w)
    print(f"[bench] generated {w.name} inputs in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    if w.dtype == "bf16":
        dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        dev = lambda x: torch.from_numpy(x).cuda()
    dQ, dK, dV = dev(Q), dev(K), dev(V)
    opts = amc.make_options(ridge_lambda=w.ridge_lambda)

    step = lambda: amc.compact_head(dQ, dK, dV, w.t, causal=w.causal, group=w.group,
                                    options=opts, want_stats=False)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ms = time_calls(torch, step, args.steps, warm=False)   # the warmup steps ran above
    wall = (time.perf_counter() - t_wall) / args.steps * 1e3
    print(f"[bench] {args.steps} steps: {ms:.3f} ms/step (events), {wall:.3f} ms/step (wall)",
          file=sys.stderr, flush=True)

    pairs = w.visible_pairs()
    flops_flash = 4 * w.d * pairs
    flops_scores = 6 * w.d * pairs
    # stage timings (separate calls, same inputs)
    ms_flash = time_calls(torch, lambda: amc.targets(dQ, dK, dV, causal=w.causal, group=w.group,
                                                     want_score=False), 3)
    ms_targets = time_calls(torch, lambda: amc.targets(dQ, dK, dV, causal=w.causal,
                                                       group=w.group), 3)
    lse, Og, sc = amc.targets(dQ, dK, dV, causal=w.causal, group=w.group)
    ms_select = time_calls(torch, lambda: amc.select_keys(sc, dK, w.t), 5)
    idx, Ck, _ = amc.select_keys(sc, dK, w.t)
    ms_beta = time_calls(torch, lambda: amc.fit_beta_nnls(dQ, Ck, idx, lse, causal=w.causal,
                                                          group=w.group, options=opts, T=w.T), 2)
    beta, _, _, _, nnls_kkt, nnls_steps = amc.fit_beta_nnls(dQ, Ck, idx, lse, causal=w.causal,
                                                            group=w.group, options=opts, T=w.T,
                                                            diagnostics=True)
    ms_values = time_calls(torch, lambda: amc.fit_values_ols(dQ, Ck, idx, beta, Og,
                                                             causal=w.causal, group=w.group,
                                                             ridge_lambda=w.ridge_lambda, T=w.T), 2)
    # adjacent rows: the fast variants and the compacted cache in use
    fast_opts = amc.make_options(beta="redistribute", values="direct")
    ms_fast = time_calls(torch, lambda: amc.compact_head(dQ, dK, dV, w.t, causal=w.causal,
                                                         group=w.group, options=fast_opts,
                                                         want_stats=False), 3)
    ms_redist = time_calls(torch, lambda: amc.beta_redistribute(dQ, Ck, idx, lse, causal=w.causal,
                                                                group=w.group, T=w.T), 5)
    full = amc.compact_head(dQ, dK, dV, w.t, causal=w.causal, group=w.group, options=opts,
                            want_stats=False)
    Qh = synth.make_heldout_queries(w, None, K, seed=3)
    dQh = dev(Qh)
    ms_eval = time_calls(torch, lambda: amc.eval_residuals(dQh, dK, dV, full["idx"], full["Ck"],
                                                           full["beta"], full["Cv"],
                                                           causal=w.causal, group=w.group), 2)
    sub = torch.from_numpy(synth.query_subset(w, None, 256)).cuda()
    ms_two = time_calls(torch, lambda: amc.compact_two_pass(dQ, dK, dV, sub, w.t, k_mult=4,
                                                            causal=w.causal, group=w.group), 3)
    M_init = w.t // 4   # the anchor + diversifier share of a t-slot budget
    ms_init = time_calls(torch, lambda: amc.init_anchor_diverse(dQ, dK, M_init, causal=w.causal,
                                                                group=w.group), 2)
    m_new, g_new = min(4096, w.T), 4
    n_new = g_new * m_new
    Qn = synth.make_heldout_queries(
        type(w)("appended_queries", w.heads, w.d, m_new, n_new, w.t, w.dtype, True, g_new), None,
        K[:, :m_new], seed=5)
    _, _, _, _, _, _, Kn, Vn = synth.make_cache_case(11, w.heads, 1, 64, 1, m_new, w.d, w.dtype,
                                                     False)
    dQn, dKn, dVn = dev(Qn), dev(Kn), dev(Vn)
    cache = lambda: amc.cache_attention(dQn, full["Ck"], full["Cv"], full["beta"], Kn=dKn, Vn=dVn,
                                        new_causal=True, group=g_new)
    ms_cache = time_calls(torch, cache, 5)
    cache_pairs = w.heads * (n_new * w.t + g_new * m_new * (m_new + 1) // 2)
    # stage-1 attention fitting of the compacted cache. The fitting queries stand in for
    # teacher queries that follow the document: a pool of 4096 evenly spaced positions (every
    # query head of each), seeing the whole cache (no mask), with full-cache targets from an
    # unmasked targets pass over the pool; 128 pool positions per update, a quarter of the
    # slots trainable
    S1, s1_updates, pool = 128, 50, 4096
    n_pos = w.n // w.group
    pool_pos = (np.arange(min(pool, n_pos)) * n_pos) // min(pool, n_pos)
    pool_rows = torch.from_numpy((pool_pos[:, None] * w.group + np.arange(w.group)).ravel()).cuda()
    Qp = dQ[:, pool_rows].contiguous()
    lse_p, Op, _ = amc.targets(Qp, dK, dV, causal=False, group=w.group, want_score=False)
    s1_samples = torch.from_numpy(synth.stage1_samples(pool_pos.size, s1_updates, S1)).cuda()
    s1_train = torch.from_numpy(np.random.default_rng(0).random((w.heads, w.t)) < 0.25).cuda()
    s1 = lambda: amc.fit_stage1(Qp, Op, lse_p, s1_samples, full["Ck"], full["Cv"], full["beta"],
                                trainable=s1_train, causal=False, group=w.group)
    ms_s1 = time_calls(torch, s1, 2)
    s1_flops = 10 * w.heads * S1 * w.group * w.t * w.d * s1_updates
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    achieved = flops_flash / (ms_flash * 1e-3) / 1e12
    score_tflops = flops_scores / (ms_targets * 1e-3) / 1e12

    if args.calibrate_copy:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] calibration copy: 268435456 bytes read, 268435456 bytes written",
              file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the float64 oracle on a bounded sample (host cores)",
              file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, Q, K, V)
        cpu["gpu_over_oracle"] = (pairs / (ms * 1e-3)) / cpu["value"]

    def per_head(x, digits):
        v = x.detach().double().cpu().numpy()
        f = (lambda a: int(a)) if digits == 0 else (lambda a: float(f"{a:.{digits}g}"))
        if v.size <= 16:
            return [f(a) for a in v.tolist()]
        return {"min": f(v.min()), "mean": float(f"{v.mean():.4g}"), "max": f(v.max())}

    out = {
        "metric": METRIC,
        "value": pairs / (ms * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "heads": w.heads, "d": w.d, "T": w.T, "n": w.n, "t": w.t,
                   "causal": w.causal, "group": w.group, "visible_pairs": pairs},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": flash_traffic(w.name),
                     "kernel": "flash_fwd_kernel (with the 0.1% V transpose in the timed call)"},
        "cpu_baseline": cpu,
        "stages_ms": {"flash_pass": ms_flash, "score_passes": ms_targets, "select": ms_select,
                      "fit_beta": ms_beta, "fit_values": ms_values},
        "score_passes": {"pairs_per_s": pairs / (ms_targets * 1e-3),
                         "tflops": score_tflops, "mfma_frac": score_tflops / peak},
        # from the library's own outputs on this workload: the fits' relative residuals and
        # status, and the NNLS's relative KKT residual and step count (per head up to 16
        # heads, else min / mean / max)
        "fits": {"mass_resid": per_head(full["resid"][0], 7),
                 "out_resid": per_head(full["resid"][1], 7),
                 "status_nonzero": int((full["status"] != 0).sum().item()),
                 "nnls_kkt_rel": per_head(nnls_kkt, 3),
                 "nnls_steps": per_head(nnls_steps, 0)},
        "next": {
            "fast_pipeline": {"ms_per_step": ms_fast, "pairs_per_s": pairs / (ms_fast * 1e-3),
                              "options": "beta=redistribute, values=direct",
                              "beta_redistribute_ms": ms_redist},
            "two_pass_pipeline": {"ms_per_step": ms_two, "pairs_per_s": pairs / (ms_two * 1e-3),
                                  "options": "256 query subset, shortlist 4t, redistributed "
                                             "beta, direct values"},
            "init_anchor_diverse": {"ms": ms_init, "M": M_init, "anchors": max(1, M_init // 4),
                                    "note": "maximum-attention pass over all pairs + "
                                            "farthest-first traversal"},
            "heldout_eval": {"ms": ms_eval, "queries_per_head": w.n,
                             "pairs_per_s": pairs / (ms_eval * 1e-3)},
            "stage1_fit": {"ms_per_update": ms_s1 / s1_updates, "updates_timed": s1_updates,
                           "positions_per_update": S1, "rows_per_update": S1 * w.group,
                           "slots": w.t, "trainable_frac": 0.25,
                           "fp32_tflops": s1_flops / (ms_s1 * 1e-3) / 1e12,
                           "pool_positions": int(pool_pos.size),
                           "note": "one call = teacher statistics over the pool + "
                                   f"{s1_updates} AdamW updates; pool queries see every slot"},
            "cache_attention": {"ms": ms_cache, "slots": w.t, "appended": m_new,
                                "queries_per_head": n_new, "visible_pairs": cache_pairs,
                                "tflops": 4 * w.d * cache_pairs / (ms_cache * 1e-3) / 1e12,
                                "mfma_frac": 4 * w.d * cache_pairs / (ms_cache * 1e-3) / 1e12
                                / peak},
        },
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
