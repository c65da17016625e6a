"""Seeded synthetic inputs for biased multi-query attention.

This module only draws random numbers and rounds them to the input dtype; it
holds none of the attention arithmetic.  The GPU path and the CPU oracle are
both fed from here, so they see bit-identical inputs.

No real AlphaGenome activations or pair representations are available, so
the workloads stand in for them with the shapes of the web page "Making
Full-Context AlphaGenome Fit on an RTX 3090" (section "Why stock
FlashAttention was not a drop-in replacement": Q [B,S,8,128], K and V
[B,S,1,D], a compact bias with one cell per 16 positions) at the full
1,048,576-bp context (8,192 positions of 128 bp):

=========  ==  ======  ====  =====  ============================================
name       B   S       P     dtype  content
=========  ==  ======  ====  =====  ============================================
tiny       1   512     32    f32    q,k,v ~ N(0,1)/sqrt(128); compact bias
                                    [32,32,8] ~ N(0,1) given directly (a pair
                                    representation with C = 8 and W = I_8)
mid        1   2048    128   bf16   pair [128,128,128] ~ N(0,1); W [128,8] with
                                    variance 1/128
full       1   8192    512   bf16   9 independent seeded layers (one per
                                    transformer block), each like mid
variant    8   8192    512   bf16   4 ref/alt pairs; alt = ref + noise of
                                    variance 0.1 on positions 4090..4101 of q,
                                    k and v; one pair representation per pair,
                                    one W for the layer
stress     1   16384   1024  bf16   like full (one layer); also in f32
=========  ==  ======  ====  =====  ============================================

"hot" companions (``hot=True``) draw q, k, v ~ N(0,1) and double the bias, so
that the outputs are O(1) and the soft-cap bends the logits; they exist to
give the parity checks teeth.

Every array is drawn in float32 with numpy's PCG64 from a fixed seed in the
order q, k, v, pair, W, noise; BF16 inputs are the round-to-nearest-even
upper halves of those float32 values, stored as ``uint16`` bit patterns.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

HQ = 8
DK = 128
DV = 128
CAP = 5.0
BLOCK = 16

#: Seeds per workload; layer / pair index is added.  Hot companions add 100000.
SEEDS = {"tiny": 1000, "mid": 2000, "full": 3000, "variant": 4000,
         "stress": 5000, "stress_f32": 6000}
HOT_SEED_OFFSET = 100000

#: Positions whose q, k, v differ between ref and alt in the variant workload.
VARIANT_ROWS = (4090, 4101)  # inclusive
VARIANT_NOISE_VAR = 0.1
#: W ~ N(0, 1/128): the second argument read as a variance (fan-in scale),
#: which makes the projected bias ~ N(0, 1) like the tiny workload's bias.
W_VAR = 1.0 / 128.0


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    B: int
    S: int
    dtype: str          # "bf16" or "f32"
    C: int              # pair channels
    layers: int = 1
    pairs: int = 1      # distinct pair representations (variant: 4)

    @property
    def P(self) -> int:
        return -(-self.S // BLOCK)


SHAPES = {
    "tiny": Shape("tiny", 1, 512, "f32", C=8),
    "mid": Shape("mid", 1, 2048, "bf16", C=128),
    "full": Shape("full", 1, 8192, "bf16", C=128, layers=9),
    "variant": Shape("variant", 8, 8192, "bf16", C=128, pairs=4),
    "stress": Shape("stress", 1, 16384, "bf16", C=128),
    "stress_f32": Shape("stress_f32", 1, 16384, "f32", C=128),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


@dataclasses.dataclass
class Layer:
    """Inputs of one attention call.

    q [B,S,8,128], k [B,S,1,128], v [B,S,1,128]; pair [Bp,P,P,C] and
    weight [C,8] (uint16 BF16 bits or float32).  ``bias_group`` batch items
    share one pair representation (variant: 2, ref and alt).
    """
    name: str
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    pair: np.ndarray
    weight: np.ndarray
    bias_group: int = 1
    scale: float = 1.0 / math.sqrt(DK)
    cap: float = CAP

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def S(self) -> int:
        return self.q.shape[1]

    @property
    def bias_index(self) -> np.ndarray:
        return np.arange(self.B) // self.bias_group


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def make_layer(name: str, layer: int = 0, *, hot: bool = False,
               S: Optional[int] = None, Dv: int = DV) -> Layer:
    """Inputs of layer ``layer`` of workload ``name``.

    ``S`` overrides the sequence length (tests use short versions of a
    workload with the same recipe); ``Dv`` the value width (192 is the
    released checkpoint's; the workloads are stated with 128).
    """
    shp = SHAPES[name]
    S = shp.S if S is None else S
    P = -(-S // BLOCK)  # a last cell shorter than 16 keeps its row and column
    seed = SEEDS[name] + layer + (HOT_SEED_OFFSET if hot else 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    qkv_std = 1.0 if hot else 1.0 / math.sqrt(DK)
    bias_mult = 2.0 if hot else 1.0
    B = shp.B
    n_pairs = shp.pairs
    group = B // n_pairs
    f32 = np.float32

    def normal(shape, std):
        return (rng.standard_normal(shape, dtype=f32) * f32(std)).astype(f32)

    # Ref items are drawn first; alt items are filled in below.
    q = np.empty((B, S, HQ, DK), f32)
    k = np.empty((B, S, 1, DK), f32)
    v = np.empty((B, S, 1, Dv), f32)
    for pi in range(n_pairs):
        q[pi * group] = normal((S, HQ, DK), qkv_std)
        k[pi * group] = normal((S, 1, DK), qkv_std)
        v[pi * group] = normal((S, 1, Dv), qkv_std)

    if name == "tiny":
        # Compact bias [P,P,8] given directly = pair with C = 8, W = I_8.
        pair = normal((1, P, P, HQ), bias_mult)
        weight = np.eye(HQ, dtype=f32)
    else:
        pair = normal((n_pairs, P, P, shp.C), 1.0)
        weight = normal((shp.C, HQ), math.sqrt(W_VAR) * bias_mult)

    if group > 1:
        lo, hi = VARIANT_ROWS
        lo, hi = min(lo, S - 1), min(hi, S - 1)
        std = math.sqrt(VARIANT_NOISE_VAR)
        for pi in range(n_pairs):
            for a in range(1, group):
                dst = pi * group + a
                q[dst] = q[pi * group]
                k[dst] = k[pi * group]
                v[dst] = v[pi * group]
                n = hi - lo + 1
                q[dst, lo:hi + 1] += normal((n, HQ, DK), std)
                k[dst, lo:hi + 1] += normal((n, 1, DK), std)
                v[dst, lo:hi + 1] += normal((n, 1, Dv), std)

    dt = shp.dtype
    return Layer(name=name, dtype=dt, q=_cast(q, dt), k=_cast(k, dt),
                 v=_cast(v, dt), pair=_cast(pair, dt), weight=_cast(weight, dt),
                 bias_group=group)


def make_custom(*, B: int, S: int, dtype: str, C: int = 16, seed: int = 0,
                qkv_std: float = 1.0, bias_std: float = 1.0, Dv: int = DV,
                n_pairs: Optional[int] = None) -> Layer:
    """Free-form seeded inputs for edge-case tests (any B, S; one pair per
    batch item unless ``n_pairs`` says otherwise)."""
    n_pairs = B if n_pairs is None else n_pairs
    rng = np.random.Generator(np.random.PCG64(seed))
    f32 = np.float32
    P = -(-S // BLOCK)  # a last cell shorter than 16 keeps its row and column
    q = rng.standard_normal((B, S, HQ, DK), dtype=f32) * f32(qkv_std)
    k = rng.standard_normal((B, S, 1, DK), dtype=f32) * f32(qkv_std)
    v = rng.standard_normal((B, S, 1, Dv), dtype=f32) * f32(qkv_std)
    pair = rng.standard_normal((n_pairs, P, P, C), dtype=f32)
    weight = rng.standard_normal((C, HQ), dtype=f32) * f32(bias_std / math.sqrt(C))
    return Layer(name="custom", dtype=dtype, q=_cast(q, dtype), k=_cast(k, dtype),
                 v=_cast(v, dtype), pair=_cast(pair, dtype),
                 weight=_cast(weight, dtype), bias_group=B // n_pairs)


def lattice_pair(p0: int, p1: int, P: int, C: int, xp=np, device=None):
    """Rows p0 .. p1 - 1 of a [P, P, C] pair representation on an integer
    lattice, for lengths whose random inputs would not fit a host: entry
    (p, r, c) is k / 64 with k = (37 p + 101 r + 29 c + 13 (p r mod 257)
    + 7 (r c mod 61)) mod 256 - 128, an integer in [-128, 128).

    Integer arithmetic, so numpy (``xp=np``) and torch (``xp=torch``, on
    ``device``) produce the same float32 values, and every value is exact in
    bf16.  Returns float32 [p1 - p0, P, C]."""
    if xp is np:
        def idx(lo, hi, shape):
            return np.arange(lo, hi, dtype=np.int64).reshape(shape)
    else:
        def idx(lo, hi, shape):
            return xp.arange(lo, hi, dtype=xp.int64, device=device).reshape(shape)
    p = idx(p0, p1, (-1, 1, 1))
    r = idx(0, P, (1, -1, 1))
    c = idx(0, C, (1, 1, -1))
    k = (37 * p + 101 * r + 29 * c + 13 * ((p * r) % 257) + 7 * ((r * c) % 61)) % 256 - 128
    return (k.astype(np.float32) if xp is np else k.to(xp.float32)) / 64.0


def make_qkv(*, B: int, S: int, dtype: str, seed: int, qkv_std: float = 1.0):
    """q [B,S,8,128], k and v [B,S,1,128] ~ N(0, qkv_std^2), drawn in that
    order from PCG64(seed) in float32 and cast to ``dtype``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f32 = np.float32
    q = rng.standard_normal((B, S, HQ, DK), dtype=f32) * f32(qkv_std)
    k = rng.standard_normal((B, S, 1, DK), dtype=f32) * f32(qkv_std)
    v = rng.standard_normal((B, S, 1, DV), dtype=f32) * f32(qkv_std)
    return _cast(q, dtype), _cast(k, dtype), _cast(v, dtype)
