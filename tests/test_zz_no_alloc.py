"""The no-allocation entry point (abg_biased_mqa_fwd_ex_noalloc) against the
entry point with a caller's workspace (abg_biased_mqa_fwd_ex), through the
C ABI: two calls in a row, the second smaller than the first (so that it runs
on what the first left in the library's scratch array), each equal to the
workspace call and within the bf16 tolerance of the oracle; no device memory
is allocated by the calls."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import to_host, upload
from long_context_biased_amd import (AbgError, NOALLOC_SCRATCH_BYTES, biased_mqa_fwd,
                                     biased_mqa_fwd_ex_noalloc, pair_bias_project, workloads)
from parity import attention_ok

pytestmark = pytest.mark.gpu

# (S, q rows (start, stop), kv_splits, cap): the first a 2048-position
# sequence in 4 key ranges with the cap (partials 33.8 MB), the second
# smaller: 45 queries at an offset of a 1000-position sequence in 4 ranges of
# 4 tiles, the last partial, without the cap (the log-sum-exp merge).
CALLS = [(2048, (0, 2048), 4, 5.0), (1000, (16, 61), 4, 0.0)]


def _inputs(S, rows, cap, seed):
    L = workloads.make_custom(B=1, S=S, dtype="bf16", C=16, seed=seed, qkv_std=1.0, bias_std=2.0)
    L.cap = cap
    t = upload(L)
    bias = pair_bias_project(t["pair"], t["weight"])
    q = t["q"][:, rows[0]:rows[1]].contiguous()
    return L, t, bias, q


def test_noalloc_matches_the_workspace_entry_point():
    outs = []
    for n, (S, rows, z, cap) in enumerate(CALLS):
        print(f"  no-alloc call {n}: S={S} rows={rows} kv_splits={z} cap={cap}", flush=True)
        L, t, bias, q = _inputs(S, rows, cap, seed=4400 + S)
        ref = biased_mqa_fwd(q, t["k"], t["v"], bias, scale=L.scale, softcap=cap,
                             q_offset=rows[0], kv_splits=z)
        out = torch.full_like(ref, float("nan"))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        free0, _ = torch.cuda.mem_get_info()
        biased_mqa_fwd_ex_noalloc(q, t["k"], t["v"], bias, out, scale=L.scale, softcap=cap,
                                  q_offset=rows[0], kv_splits=z)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        assert torch.cuda.max_memory_allocated() == before
        if n > 0:  # the scratch array is resident from the first call on
            assert free0 == free1, (free0, free1)
        # the same kernels on the same inputs: identical bits
        assert torch.equal(out, ref), float((out.float() - ref.float()).abs().max())
        got = to_host(out)
        ref64 = oracle.attention_rows(L.q, L.k, L.v, oracle.project_pair_bias(L.pair, L.weight),
                                      np.arange(rows[0], rows[1]), scale=L.scale, cap=cap, batch=0)
        ok, ma, rel = attention_ok(got[0], ref64, "bf16")
        print(f"    vs oracle: max-abs {ma:.3g} rel-L2 {rel:.3g}", flush=True)
        assert ok, f"max-abs {ma:.3g} rel-L2 {rel:.3g}"
        outs.append(out)


def test_noalloc_rejects_more_partials_than_its_scratch():
    L, t, bias, q = _inputs(8192, (0, 8192), 5.0, seed=4500)
    out = torch.empty_like(q)
    with pytest.raises(AbgError) as e:
        biased_mqa_fwd_ex_noalloc(q, t["k"], t["v"], bias, out, softcap=5.0, kv_splits=8)
    assert e.value.status == 2 and str(NOALLOC_SCRATCH_BYTES) in str(e.value)
    # one key range needs no scratch at all
    biased_mqa_fwd_ex_noalloc(q, t["k"], t["v"], bias, out, softcap=5.0, kv_splits=1)
    ref = biased_mqa_fwd(q, t["k"], t["v"], bias, softcap=5.0)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
