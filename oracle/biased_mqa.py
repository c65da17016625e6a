"""Dense float64 definition of AlphaGenome-style biased multi-query attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed, following [AG3090]:

* Shapes, section "Why stock FlashAttention was not a drop-in replacement":
  Q is [B, S, Hq, Dk], K is [B, S, 1, Dk] and V is [B, S, 1, Dv]; the one K/V
  head is shared by every query head (multi-query attention).
* The per-head pair bias comes from a compact pair representation that is
  projected per head and repeated 16 times along both sequence axes, section
  "Profiling pointed at one very large object".  The compact bias has one cell
  per 16 positions per axis and each cell covers a 16 x 16 square, section
  "Why stock FlashAttention ...".  The 16 is also the ratio of the 2,048-bp
  pair resolution to the 128-bp transformer resolution ([AGDNA]).
* The logit equation of that section: the scaled dot product plus the bias
  cell of the two positions, soft-capped by cap * tanh(x / cap) with cap 5,
  the bias inside the cap and the 1/sqrt(128) scale on the dot product only.
* Softmax over keys, then a weighted sum of V rows (same section, list of
  requirements).  Matrix products there are BF16 with FP32 accumulation; the
  oracle takes the exact input values (BF16 inputs are decoded exactly) and
  does every step in float64.
* The tiled online softmax of section "Online softmax, one block at a time"
  (running max m, denominator d, numerator n, output n / d) is the same
  softmax up to rounding order; ``tiled_attention`` writes that recurrence out
  so the two can be compared.

Readings where the page leaves a step open (each is listed in the design
notes of the repository):
* the projection is linear, with no bias term, normalisation or activation;
* a soft-cap value of 0 means "no cap" (L = x), used for the invariants;
* the bias is float64 here and float32 on the GPU (accumulated, never rounded
  to BF16).
"""

from __future__ import annotations

import numpy as np

#: Positions per compact bias cell along each axis ([AG3090] section "Why stock
#: FlashAttention was not a drop-in replacement"; [AGDNA] 2,048 bp / 128 bp).
BIAS_BLOCK = 16


def as_f64(x) -> np.ndarray:
    """Exact float64 value of an input array.

    ``uint16`` arrays are BF16 bit patterns (the upper half of an IEEE float32),
    decoded exactly; any float array is converted with ``astype``.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def project_pair_bias(pair, weight) -> np.ndarray:
    """Per-head compact bias from a compact pair representation.

    ``pair`` is [P, P, C] (or [Bp, P, P, C]) and ``weight`` is [C, H].
    Returns ``bias[h, p, r] = sum_c pair[p, r, c] * weight[c, h]`` as
    [H, P, P] (or [Bp, H, P, P]).  [AG3090] section "Profiling pointed at one
    very large object": the compact pair representation is projected to the
    attention bias before the 16x repetition.  Plain linear map (reading).
    """
    pair = as_f64(pair)
    weight = as_f64(weight)
    return np.moveaxis(pair @ weight, -1, -3)


def expand_bias(bias, s_q: int, s_k: int) -> np.ndarray:
    """Dense bias by nearest-neighbour repetition of each compact cell.

    ``bias`` is [..., P_q, P_k]; every cell is repeated over a 16 x 16 square
    (``np.repeat`` along both axes, not ``np.tile``), then cut to
    [..., s_q, s_k].  [AG3090] section "Why stock FlashAttention ...": the
    bias of positions (i, j) is the cell (floor(i/16), floor(j/16)).
    """
    b = np.repeat(as_f64(bias), BIAS_BLOCK, axis=-2)
    b = np.repeat(b, BIAS_BLOCK, axis=-1)
    return b[..., :s_q, :s_k]


def soft_cap(x, cap: float) -> np.ndarray:
    """cap * tanh(x / cap); ``cap == 0`` means no cap (identity)."""
    if cap == 0.0:
        return x
    return cap * np.tanh(x / cap)


def logits(q_h, k, bias_dense, scale: float, cap: float) -> np.ndarray:
    """Logit equation of [AG3090] for one head.

    ``q_h`` [Sq, Dk], ``k`` [Sk, Dk], ``bias_dense`` [Sq, Sk]:
    ``L = cap * tanh((scale * q_h @ k.T + bias_dense) / cap)``.
    """
    x = scale * (as_f64(q_h) @ as_f64(k).T) + bias_dense
    return soft_cap(x, cap)


def softmax_two_pass(L) -> np.ndarray:
    """Row softmax over the last axis: max, then exp(L - max) / sum."""
    m = np.max(L, axis=-1, keepdims=True)
    e = np.exp(L - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _bias_for_item(bias, bias_index, b):
    bias = np.asarray(bias) if not isinstance(bias, np.ndarray) else bias
    if bias.ndim == 3:
        return bias
    idx = b if bias_index is None else int(bias_index[b])
    return bias[idx]


def attention_rows(q, k, v, bias, rows, *, scale: float, cap: float,
                   bias_index=None, batch=0, heads=None) -> np.ndarray:
    """Output rows of one batch item, computed densely.

    ``q`` [B, S, Hq, Dk], ``k`` [B, S, 1, Dk], ``v`` [B, S, 1, Dv] (arrays of
    float or BF16 bits), ``bias`` [H, P, P] or [Bb, H, P, P] with
    ``bias_index[b]`` naming the bias of batch item b (default: b).
    ``rows`` are query positions.  Returns [len(rows), len(heads), Dv].

    Steps: materialise the repeated bias rows, the full logit rows of every
    selected query against all S keys, the soft-cap, a two-pass softmax, then
    the weighted sum of V.  Nothing is tiled.
    """
    rows = np.asarray(rows, dtype=np.int64)
    S = q.shape[1]
    Hq = q.shape[2]
    heads = list(range(Hq)) if heads is None else list(heads)
    kb = as_f64(k[batch, :, 0, :])
    vb = as_f64(v[batch, :, 0, :])
    bias_b = as_f64(_bias_for_item(bias, bias_index, batch))
    out = np.empty((rows.size, len(heads), vb.shape[-1]), dtype=np.float64)
    for n, h in enumerate(heads):
        # Repeat the compact rows, then pick the selected query positions.
        dense_rows = np.repeat(bias_b[h], BIAS_BLOCK, axis=0)[rows]
        dense_rows = np.repeat(dense_rows, BIAS_BLOCK, axis=1)[:, :S]
        L = logits(q[batch, rows, h, :], kb, dense_rows, scale, cap)
        out[:, n, :] = softmax_two_pass(L) @ vb
    return out


def attention_row_given_bias_row(q_row, k, v, bias_row, *, scale: float,
                                 cap: float) -> np.ndarray:
    """Output of one query position from its compact bias row alone.

    ``q_row`` [Hq, Dk], ``k`` [S, Dk], ``v`` [S, Dv] (float or BF16 bits) and
    ``bias_row`` [Hq, P], the compact bias row of the query's cell
    (``bias[h, i // 16, :]``).  The steps of ``attention_rows`` for one
    position: repeat the row 16 times along the keys, the logit equation,
    the soft-cap, a two-pass softmax and the weighted sum of V.  It lets a
    check reach positions of sequences whose whole compact bias would not fit
    in host memory.  Returns [Hq, Dv].
    """
    kb = as_f64(k)
    vb = as_f64(v)
    S = kb.shape[0]
    br = as_f64(bias_row)
    q_row = np.asarray(q_row)
    out = np.empty((q_row.shape[0], vb.shape[-1]), dtype=np.float64)
    for h in range(q_row.shape[0]):
        dense = np.repeat(br[h][None, :], BIAS_BLOCK, axis=1)[:, :S]
        L = logits(q_row[h][None, :], kb, dense, scale, cap)
        out[h] = (softmax_two_pass(L) @ vb)[0]
    return out


def attention(q, k, v, bias, *, scale: float, cap: float, bias_index=None,
              row_block: int = 1024) -> np.ndarray:
    """Full output [B, S, Hq, Dv] in float64.

    Loops over batch items and blocks of ``row_block`` query positions only to
    bound memory; every block is computed densely by ``attention_rows``.
    """
    B, S, Hq, _ = q.shape
    Dv = v.shape[-1]
    out = np.empty((B, S, Hq, Dv), dtype=np.float64)
    for b in range(B):
        for r0 in range(0, S, row_block):
            rows = np.arange(r0, min(S, r0 + row_block))
            out[b, rows] = attention_rows(q, k, v, bias, rows, scale=scale,
                                          cap=cap, bias_index=bias_index,
                                          batch=b)
    return out


def tiled_attention(q, k, v, bias, *, scale: float, cap: float,
                    bias_index=None, tile: int = 64) -> np.ndarray:
    """The online-softmax recurrence of [AG3090] section "Online softmax, one
    block at a time", in float64, for checking that it equals the dense
    definition.

    For every query row it keeps the running maximum m, denominator d and
    numerator n, walks the keys in tiles of ``tile`` positions, and after each
    tile with maximum m_t sets m' = max(m, m_t), d' = d e^(m - m') +
    sum_j e^(L_j - m'), n' = n e^(m - m') + sum_j e^(L_j - m') V_j.  The output
    is n / d.  The bias of a tile is read as the compact cell
    (floor(i/16), floor(j/16)) of each position pair instead of a dense copy.
    """
    B, S, Hq, _ = q.shape
    Dv = v.shape[-1]
    out = np.empty((B, S, Hq, Dv), dtype=np.float64)
    pos = np.arange(S)
    for b in range(B):
        kb = as_f64(k[b, :, 0, :])
        vb = as_f64(v[b, :, 0, :])
        bias_b = as_f64(_bias_for_item(bias, bias_index, b))
        for h in range(Hq):
            qh = as_f64(q[b, :, h, :])
            m = np.full(S, -np.inf)
            d = np.zeros(S)
            n = np.zeros((S, Dv))
            for j0 in range(0, S, tile):
                cols = pos[j0:j0 + tile]
                cell = bias_b[h][np.ix_(pos // BIAS_BLOCK, cols // BIAS_BLOCK)]
                x = scale * (qh @ kb[cols].T) + cell
                L = soft_cap(x, cap)
                m_new = np.maximum(m, L.max(axis=1))
                alpha = np.exp(m - m_new)
                w = np.exp(L - m_new[:, None])
                d = d * alpha + w.sum(axis=1)
                n = n * alpha[:, None] + w @ vb[cols]
                m = m_new
            out[b, :, h, :] = n / d[:, None]
    return out
