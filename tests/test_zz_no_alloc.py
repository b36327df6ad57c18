"""am_compact_head_noalloc (the library's fixed scratch array instead of a workspace)
against am_compact_head on the same inputs: every output bit-identical, on two calls in a
row of which the second is smaller, then on a problem that needs the multi-workgroup
NNLS and the stored-design Gram path (t > 256)."""
import numpy as np
import pytest

import kv_cache_compaction_amd as amc
from kv_cache_compaction_amd import synth
from kv_cache_compaction_amd.configs import Workload
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu

CASES = [
    Workload("noalloc_causal_g4", 4, 128, 2048, 8192, 64, "bf16", True, 4),   # first call
    Workload("noalloc_small", 2, 64, 512, 512, 32, "bf16", False, 1),         # smaller
    Workload("noalloc_big_t", 2, 128, 2048, 2048, 300, "bf16", False, 1),     # t > 256
]


def _run(w):
    import torch
    print(f"case {w.name}", flush=True)
    Q, K, V = synth.make_batch(w)
    dQ, dK, dV = (to_dev(x, w.dtype) for x in (Q, K, V))
    p = amc.make_problem(dQ, dK, causal=w.causal, group=w.group)
    need = amc.workspace_bytes(p, w.t, amc.CALL_COMPACT)
    assert 0 < need <= amc.NOALLOC_SCRATCH_BYTES, need
    ref = amc.compact_head(dQ, dK, dV, w.t, causal=w.causal, group=w.group)
    got = amc.compact_head_noalloc(dQ, dK, dV, w.t, causal=w.causal, group=w.group)
    torch.cuda.synchronize()
    assert np.all(got["status"].cpu().numpy() == 0)
    for k in ref:
        assert torch.equal(ref[k], got[k]), (w.name, k)


def test_noalloc_two_calls_second_smaller():
    _run(CASES[0])
    _run(CASES[1])


def test_noalloc_multiworkgroup_fit():
    _run(CASES[2])


def test_noalloc_rejects_problems_beyond_its_scratch():
    import torch
    w = Workload("noalloc_too_big", 8, 128, 4096, 65536, 64, "bf16", True, 16)
    dQ = torch.zeros((w.heads, w.n, w.d), dtype=torch.bfloat16, device="cuda")
    dK = torch.zeros((w.heads, w.T, w.d), dtype=torch.bfloat16, device="cuda")
    p = amc.make_problem(dQ, dK, causal=True, group=16)
    assert amc.workspace_bytes(p, w.t, amc.CALL_COMPACT) > amc.NOALLOC_SCRATCH_BYTES
    with pytest.raises(amc.AmError) as e:
        amc.compact_head_noalloc(dQ, dK, dK, w.t, causal=True, group=16)
    assert e.value.status == amc.AM_ERR_WORKSPACE
