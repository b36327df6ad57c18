"""Writes single_head_T128k.npz: float64 oracle results for the 128K-key workload
(one KV head, T = n = 131072, d = 128, bf16 inputs, t = 4096, ridge 1e-3), so that the GPU
parity test at that size can compare against the oracle without the oracle's minutes-long
full pass on the GPU host.

Only the oracle (oracle/am_oracle.py) and the seeded input generator are used. Stored:
  score [T] f64   the RMS selection statistic of every key (S2)
  lse   [n] f64   every query's full-cache log-normalizer (S1)
  idx   [t] i32   the oracle's selection (S3)
  w     [t] f64   the oracle's NNLS weights on that selection (S5)
  r_mass, r_out   the oracle's mass and output residuals at its optimum (S5, S7)
  AtY  [t, d] f32, yy   value_fit_stats of the oracle's value design on (idx, w) and the
                  full-cache outputs: with them the output residual of any C_v fitted on
                  (idx, w) is evaluated without the outputs themselves
  kkt             the KKT residual of the oracle's w (in the units of M^T M)

Run from the repository root: python tests/golden/make_single_head_T128k.py
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from kv_cache_compaction_amd import synth  # noqa: E402
from kv_cache_compaction_amd.configs import BY_NAME  # noqa: E402
from oracle import am_oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "single_head_T128k.npz")


def main():
    w = BY_NAME["single_head_T128k"]
    t0 = time.time()
    Q, K, V = synth.make_head(w, 0)
    q, k, v = (synth.as_f64(x, w.dtype) for x in (Q, K, V))
    print(f"inputs {time.time() - t0:.1f} s", flush=True)
    r = O.compact_head(q, k, v, w.t, w.scale, w.causal, w.group, ridge_lambda=w.ridge_lambda)
    print(f"oracle compaction {time.time() - t0:.1f} s: r_mass {r['r_mass']:.6g} "
          f"r_out {r['r_out']:.6g}", flush=True)
    AtY, yy = O.value_fit_stats(r["A"], r["O"])
    G = r["M"].T @ r["M"]
    kkt = O.nnls_kkt_residual(G, r["M"].T @ r["b"], r["w"])
    np.savez_compressed(OUT, score=r["score"], lse=r["lse"], idx=r["idx"].astype(np.int32),
                        w=r["w"], r_mass=r["r_mass"], r_out=r["r_out"],
                        AtY=AtY.astype(np.float32), yy=yy, kkt=kkt)
    print(f"wrote {OUT} ({os.path.getsize(OUT) / 1e6:.1f} MB) after {time.time() - t0:.1f} s; "
          f"kkt {kkt:.3g}, zero weights {(r['w'] == 0).sum()}", flush=True)


if __name__ == "__main__":
    main()
