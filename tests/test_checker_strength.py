"""The parity checker must reject plausible wrong kernels at every workload
shape.  CPU only.

At the workloads' own input distribution the attention output is small
(|out| ~ 1e-2 at S = 2,048), so the contract's max-abs bounds alone (2e-2
for bf16 inputs, 1e-4 for float32) would accept an all-zero output or a
kernel without the soft-cap.  ``parity.attention_ok`` therefore also bounds
the relative L2 error, and every workload is also checked on its hot
companion (q, k, v ~ N(0, 1), bias x 2).  This test computes four wrong
outputs with float64 arithmetic written out here -- all zeros, no soft-cap,
the compact bias tiled instead of repeated, the Q.K term dropped -- and
requires each to fail the checker on the regular inputs or on the hot
companion, at the same query rows the GPU tests check.
"""

import numpy as np
import pytest

import oracle
from long_context_biased_amd import workloads
from parity import attention_ok, sample_rows

MUTANTS = ["zeros", "no_cap", "tile_bias", "drop_qk"]


def _rows_f64(layer, bias64, rows, b, mutation=None):
    """Output rows [len(rows), Hq, Dv] of batch item b, dense float64."""
    q = oracle.as_f64(layer.q[b])           # [S, Hq, Dk]
    k = oracle.as_f64(layer.k[b, :, 0, :])  # [S, Dk]
    v = oracle.as_f64(layer.v[b, :, 0, :])  # [S, Dv]
    bias = bias64[layer.bias_index[b]] if bias64.ndim == 4 else bias64
    S = q.shape[0]
    P = bias.shape[-1]
    i = np.asarray(rows)[:, None]
    j = np.arange(S)[None, :]
    if mutation == "tile_bias":
        bi, bj = i % P, j % P
    else:
        bi, bj = i // 16, j // 16
    out = np.empty((len(rows), q.shape[1], v.shape[1]))
    for h in range(q.shape[1]):
        x = bias[h][bi, bj]
        if mutation != "drop_qk":
            x = x + layer.scale * (q[rows, h, :] @ k.T)
        L = x if mutation == "no_cap" else layer.cap * np.tanh(x / layer.cap)
        e = np.exp(L - L.max(axis=1, keepdims=True))
        out[:, h, :] = (e / e.sum(axis=1, keepdims=True)) @ v
    if mutation == "zeros":
        out[:] = 0.0
    return out


@pytest.mark.parametrize("name", ["tiny", "mid", "full", "variant", "stress", "stress_f32"])
def test_checker_rejects_wrong_kernels(name):
    rejected = {m: [] for m in MUTANTS}
    for hot in (False, True):
        L = workloads.make_layer(name, hot=hot)
        bias64 = oracle.project_pair_bias(L.pair, L.weight)
        rows = np.arange(L.S) if L.S <= 512 else sample_rows(L.S, seed=3, extra=8)
        items = (0, 1) if L.B > 1 else (0,)  # ref and alt item of the first pair
        for b in items:
            truth = oracle.attention_rows(L.q, L.k, L.v, bias64, rows, scale=L.scale,
                                          cap=L.cap, bias_index=L.bias_index, batch=b)
            # the unmutated rows written out here are the oracle's
            assert np.allclose(_rows_f64(L, bias64, rows, b), truth, rtol=1e-10, atol=1e-13)
            for m in MUTANTS:
                ok, _, _ = attention_ok(_rows_f64(L, bias64, rows, b, m), truth, L.dtype)
                if not ok:
                    rejected[m].append((hot, b))
    print(f"  {name}: " + "; ".join(f"{m} rejected by {rejected[m]}" for m in MUTANTS), flush=True)
    missed = [m for m in MUTANTS if not rejected[m]]
    assert not missed, f"{name}: the checker accepts {missed}"
