"""The oracle against its pins (closed forms, a library routine, invariants,
brute force, the tiled recurrence).  CPU only."""

import numpy as np
import pytest

import oracle
import oracle_pins as pins


def oracle_attn(q, k, v, bias, *, scale, cap, bias_index=None):
    return oracle.attention(q, k, v, bias, scale=scale, cap=cap, bias_index=bias_index)


def oracle_project(pair, w):
    return oracle.project_pair_bias(pair, w)


@pytest.mark.parametrize("pin", pins.ATTENTION_PINS, ids=lambda f: f.__name__)
def test_attention_pin(pin):
    ok, detail = pin(oracle_attn)
    assert ok, detail


@pytest.mark.parametrize("pin", pins.PROJECTION_PINS, ids=lambda f: f.__name__)
def test_projection_pin(pin):
    ok, detail = pin(oracle_project)
    assert ok, detail


def test_expand_bias_is_repeat_not_tile():
    """Materialised repetition equals the bias looked up by floor division of
    both positions, bit for bit, and differs from tiling."""
    bias = np.random.default_rng(7).standard_normal((3, 5, 4))
    dense = oracle.expand_bias(bias, 80, 64)
    i = np.arange(80)[:, None]
    j = np.arange(64)[None, :]
    looked_up = bias[:, i // 16, j // 16]
    assert np.array_equal(dense, looked_up)
    tiled = np.tile(bias, (1, 16, 16))[:, :80, :64]
    assert not np.array_equal(dense, tiled)


def test_attention_rows_matches_full():
    """Row subsets (used at full size) equal the corresponding rows of the full
    computation, bit for bit."""
    q, k, v, bias = pins._rand_case(600, B=2, S=128, Hq=8, Dk=16, Dv=16, bias_std=2.0)
    full = oracle.attention(q, k, v, bias, scale=0.25, cap=5.0, row_block=48)
    rows = np.array([0, 15, 16, 63, 64, 127])
    part = oracle.attention_rows(q, k, v, bias, rows, scale=0.25, cap=5.0, batch=1)
    assert np.allclose(part, full[1, rows], rtol=0, atol=1e-15)
    # a length off the 16-position cell (P = ceil(S/16)), against the brute force
    q, k, v, bias = pins._rand_case(601, B=1, S=37, Hq=2, Dk=4, Dv=4, bias_std=2.0)
    rows = np.array([0, 15, 16, 31, 32, 36])
    part = oracle.attention_rows(q, k, v, bias, rows, scale=0.5, cap=5.0, batch=0)
    brute = np.array(oracle.attention_brute(q, k, v, bias, scale=0.5, cap=5.0))[0, rows]
    assert np.allclose(part, brute, rtol=0, atol=1e-12)


def test_row_given_bias_row_matches_brute_force():
    """The one-position entry (the query's compact bias row only, for
    sequences whose whole bias does not fit on the host) against the scalar
    brute force, on a length off the 16-position cell, with and without the
    cap, BF16 inputs included."""
    for seed, S, cap, bf16 in ((610, 37, 5.0, False), (611, 64, 0.0, False), (612, 50, 2.0, True)):
        q, k, v, bias = pins._rand_case(seed, B=1, S=S, Hq=3, Dk=4, Dv=5, bias_std=2.0)
        if bf16:
            from long_context_biased_amd.workloads import f32_to_bf16_bits
            q, k, v = (f32_to_bf16_bits(np.asarray(x, dtype=np.float32)) for x in (q, k, v))
        brute = np.array(oracle.attention_brute(q, k, v, bias, scale=0.5, cap=cap))[0]
        for i in (0, 15, 16, S - 1):
            row = oracle.attention_row_given_bias_row(q[0, i], k[0, :, 0], v[0, :, 0],
                                                      bias[0][:, i // 16, :], scale=0.5, cap=cap)
            assert np.allclose(row, brute[i], rtol=0, atol=1e-12), (seed, i)


def test_bf16_decoding_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x3C00], dtype=np.uint16)
    vals = oracle.as_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0
    assert vals[2] == 3.140625
    assert vals[3] == 2.0 ** -133          # smallest subnormal bf16
    assert vals[4] == (2 - 2 ** -7) * 2.0 ** 127
    assert vals[5] == 2.0 ** -7
