"""Seeded workload generator (determinism, recipe) and the stored oracle
regression fixture.  CPU only."""

import hashlib
import json
import math
import os

import numpy as np
import pytest

import oracle
from long_context_biased_amd import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def _digest(layer):
    h = hashlib.sha256()
    for a in (layer.q, layer.k, layer.v, layer.pair, layer.weight):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_generator_is_deterministic():
    a = workloads.make_layer("mid", S=256)
    b = workloads.make_layer("mid", S=256)
    assert _digest(a) == _digest(b)
    c = workloads.make_layer("mid", S=256, hot=True)
    assert _digest(a) != _digest(c)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5],
                 dtype=np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    back = oracle.as_f64(bits)
    # ties go to the even mantissa; above-tie rounds up
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5]


def test_tiny_recipe():
    L = workloads.make_layer("tiny")
    assert L.q.dtype == np.float32 and L.q.shape == (1, 512, 8, 128)
    assert L.pair.shape == (1, 32, 32, 8) and np.array_equal(L.weight, np.eye(8))
    assert abs(L.q.std() * math.sqrt(128) - 1) < 0.01
    assert abs(L.pair.std() - 1) < 0.02


def test_variant_recipe():
    L = workloads.make_layer("variant", S=4160)
    assert L.q.shape[0] == 8 and L.bias_group == 2 and L.pair.shape[0] == 4
    q = oracle.as_f64(L.q)
    lo, hi = workloads.VARIANT_ROWS
    for pi in range(4):
        ref, alt = q[2 * pi], q[2 * pi + 1]
        diff_rows = np.nonzero(np.abs(ref - alt).max(axis=(1, 2)))[0]
        assert diff_rows.min() == lo and diff_rows.max() == hi
    # different pairs are different draws
    assert not np.array_equal(q[0], q[2])


def test_golden_tiny_rows():
    with open(os.path.join(HERE, "golden", "tiny_oracle_rows.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        hot = case["workload"].endswith("_hot")
        L = workloads.make_layer("tiny", hot=hot)
        bias = oracle.project_pair_bias(L.pair, L.weight)
        out = oracle.attention_rows(L.q, L.k, L.v, bias, case["rows"], scale=L.scale, cap=L.cap)
        assert np.allclose(out[:, :, :8], np.array(case["out"]), rtol=1e-12, atol=1e-15)
        assert np.allclose(out.sum(-1), np.array(case["row_sums"]), rtol=1e-12, atol=1e-15)
