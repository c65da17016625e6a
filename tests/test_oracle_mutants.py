"""Plant plausible mistakes in a copy of the oracle's arithmetic and require
every one of them to fail at least one pin: evidence that the pins would
catch such a mistake in the oracle itself.  CPU only.

``mutant_attention(mutation=None)`` is the oracle's dense computation written
out once more with switches; with no mutation it must equal the oracle.
"""

import math

import numpy as np
import pytest

import oracle
import oracle_pins as pins

ATTN_MUTATIONS = [
    "drop_bias", "tile_bias", "transpose_bias", "cap_outside_bias", "no_cap",
    "cap_without_div", "cap_without_mul", "scale_on_bias", "no_scale",
    "softmax_over_queries", "shifted_block", "block_8", "bias_sign",
    "drop_qk", "bias_head_0", "bias_head_reversed", "value_shift",
    "no_normalisation", "bias_batch_0", "query_head_0", "exp_of_cap_only",
    "sqrt_scale",
]

#: Pins that restate the definition (scalar loops, the tiled recurrence); a
#: mutant must also fail at least one pin outside this set.
RESTATING_PINS = {"pin_brute_force", "pin_tiled_recurrence"}


def mutant_attention(q, k, v, bias, *, scale, cap, bias_index=None, mutation=None):
    B, S, Hq, _ = q.shape
    Dv = v.shape[-1]
    out = np.empty((B, S, Hq, Dv))
    for b in range(B):
        bi = b if bias_index is None else int(bias_index[b])
        if mutation == "bias_batch_0":
            bi = 0
        kb = oracle.as_f64(k[b, :, 0, :])
        vb = oracle.as_f64(v[b, :, 0, :])
        if mutation == "value_shift":
            vb = np.roll(vb, 1, axis=0)
        for h in range(Hq):
            hb = h
            if mutation == "bias_head_0":
                hb = 0
            elif mutation == "bias_head_reversed":
                hb = Hq - 1 - h
            cb = np.asarray(bias, dtype=np.float64)[bi, hb]
            if mutation == "transpose_bias":
                cb = cb.T
            if mutation == "tile_bias":
                dense = np.tile(cb, (16, 16))[:S, :S]
            elif mutation == "block_8":
                dense = np.repeat(np.repeat(cb, 8, 0), 8, 1)
                dense = np.pad(dense, ((0, max(0, S - dense.shape[0])),
                                       (0, max(0, S - dense.shape[1]))), mode="edge")[:S, :S]
            elif mutation == "shifted_block":
                dense = np.repeat(np.repeat(cb, 16, 0), 16, 1)
                dense = np.roll(dense, 1, axis=1)[:S, :S]
            else:
                dense = np.repeat(np.repeat(cb, 16, 0), 16, 1)[:S, :S]
            qh = oracle.as_f64(q[b, :, 0 if mutation == "query_head_0" else h, :])
            qk = qh @ kb.T
            if mutation == "drop_qk":
                qk = 0 * qk
            if mutation == "drop_bias":
                dense = 0 * dense
            if mutation == "bias_sign":
                dense = -dense
            if mutation == "scale_on_bias":
                x = scale * (qk + dense)
            elif mutation == "no_scale":
                x = qk + dense
            elif mutation == "sqrt_scale":
                x = math.sqrt(scale) * qk + dense
            else:
                x = scale * qk + dense
            if cap == 0.0 or mutation == "no_cap":
                L = x
            elif mutation == "cap_outside_bias":
                L = cap * np.tanh((x - dense) / cap) + dense
            elif mutation == "cap_without_div":
                L = cap * np.tanh(x)
            elif mutation == "cap_without_mul":
                L = np.tanh(x / cap)
            elif mutation == "exp_of_cap_only":
                L = cap * np.tanh(x / cap) + 0.5 * x
            else:
                L = cap * np.tanh(x / cap)
            axis = 0 if mutation == "softmax_over_queries" else 1
            m = L.max(axis=axis, keepdims=True)
            e = np.exp(L - m)
            if mutation == "no_normalisation":
                p = e
            else:
                p = e / e.sum(axis=axis, keepdims=True)
            out[b, :, h, :] = p @ vb
    return out


def _bind(mutation):
    def attn(q, k, v, bias, *, scale, cap, bias_index=None):
        return mutant_attention(q, k, v, bias, scale=scale, cap=cap,
                                bias_index=bias_index, mutation=mutation)
    return attn


def test_unmutated_copy_equals_oracle():
    q, k, v, bias = pins._rand_case(700, B=2, S=80, Hq=4, Dk=16, Dv=8, bias_std=2.0)
    for cap in (5.0, 0.0):
        a = mutant_attention(q, k, v, bias, scale=0.3, cap=cap)
        b = oracle.attention(q, k, v, bias, scale=0.3, cap=cap)
        assert np.max(np.abs(a - b)) <= 1e-13


@pytest.mark.parametrize("mutation", ATTN_MUTATIONS)
def test_attention_mutant_is_caught(mutation):
    attn = _bind(mutation)
    failed = []
    for pin in pins.ATTENTION_PINS:
        try:
            ok, _ = pin(attn)
        except Exception as exc:  # a crash counts as caught, but name it
            ok = False
            _ = exc
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"mutation {mutation!r} passed every pin"
    assert set(failed) - RESTATING_PINS, (
        f"mutation {mutation!r} is caught only by {failed}")


PROJ_MUTATIONS = ["transpose_pair", "no_moveaxis_fix", "weight_row_0", "sum_over_rows",
                  "drop_last_channel", "heads_reversed"]


def mutant_project(pair, w, mutation=None):
    pair = np.asarray(pair, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if mutation == "transpose_pair":
        pair = np.swapaxes(pair, -2, -3)
    if mutation == "weight_row_0":
        w = np.broadcast_to(w[:1], w.shape)
    if mutation == "drop_last_channel":
        pair = pair[..., :-1]
        w = w[:-1]
    if mutation == "heads_reversed":
        w = w[:, ::-1]
    y = pair @ w
    if mutation == "sum_over_rows":
        y = np.broadcast_to(y.sum(axis=-3, keepdims=True), y.shape)
    if mutation == "no_moveaxis_fix":
        return np.swapaxes(y, -1, -3)  # [.., H, P(r), P(p)]: rows and columns swapped
    return np.moveaxis(y, -1, -3)


@pytest.mark.parametrize("mutation", PROJ_MUTATIONS)
def test_projection_mutant_is_caught(mutation):
    failed = []
    for pin in pins.PROJECTION_PINS:
        try:
            ok, _ = pin(lambda p, w: mutant_project(p, w, mutation))
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"projection mutation {mutation!r} passed every pin"


def test_unmutated_projection_equals_oracle():
    r = np.random.default_rng(3)
    pair = r.standard_normal((2, 5, 5, 7))
    w = r.standard_normal((7, 8))
    assert np.max(np.abs(mutant_project(pair, w) - oracle.project_pair_bias(pair, w))) < 1e-14
