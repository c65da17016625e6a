"""Pins for the CPU oracle: checks against things other than the oracle itself.

Every pin takes an attention implementation ``attn(q, k, v, bias, scale=,
cap=, bias_index=)`` returning float64 [B, S, Hq, Dv] (``bias`` is
[Bb, Hq, P, P]), and returns ``(ok, detail)``.  ``tests/test_oracle_pins.py``
requires every pin to pass for the oracle; ``tests/test_oracle_mutants.py``
plants plausible mistakes in a copy of the oracle's arithmetic and requires
each one to fail at least one pin, so the pins are known to have teeth.

Sources of the pinned facts (web page "Making Full-Context AlphaGenome Fit on
an RTX 3090", abbreviated [AG3090]):
* closed forms that follow from the logit equation and softmax in section
  "Why stock FlashAttention was not a drop-in replacement" when the logits
  take values chosen by construction (artanh cases below);
* a library routine: float64 ``torch.nn.functional.scaled_dot_product_attention``
  with an additive mask is the uncapped special case;
* invariants of softmax attention (shift invariance without the cap, one key,
  equal values, rows summing to one, permutations inside a 16-position bias
  cell, linearity in V, independence of heads and batch items);
* brute force (scalar loops) on tiny shapes;
* the tiled recurrence of section "Online softmax, one block at a time",
  which must equal the dense result.
"""

from __future__ import annotations

import math

import numpy as np

import oracle

CAP = 5.0
TIGHT = 1e-11


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand_case(seed, B=1, S=64, Hq=8, Dk=8, Dv=8, qkv_std=1.0, bias_std=1.0, Bb=None):
    r = _rng(seed)
    P = (S + 15) // 16
    Bb = B if Bb is None else Bb
    q = r.standard_normal((B, S, Hq, Dk))
    k = r.standard_normal((B, S, 1, Dk))
    v = r.standard_normal((B, S, 1, Dv))
    bias = r.standard_normal((Bb, Hq, P, P)) * bias_std
    return q * qkv_std, k * qkv_std, v, bias


def _close(a, b, tol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    return err <= tol * scale, err


# --------------------------------------------------------------------------
# Brute force on tiny shapes
# --------------------------------------------------------------------------
def pin_brute_force(attn):
    # lengths off the 16-position cell (7, 23, 40) pin a last cell that is
    # shorter than 16 positions: the brute force indexes the compact bias by
    # integer division and never builds the repeated bias
    for seed, (S, Hq, D, cap) in enumerate([(16, 1, 4, CAP), (32, 2, 4, CAP),
                                            (48, 8, 4, 1.5), (32, 3, 8, 0.0),
                                            (7, 2, 4, CAP), (23, 1, 4, CAP),
                                            (40, 2, 4, 1.5)]):
        q, k, v, bias = _rand_case(100 + seed, B=2, S=S, Hq=Hq, Dk=D, Dv=D + 1,
                                   qkv_std=1.5, bias_std=2.0)
        scale = 1.0 / math.sqrt(D)
        got = attn(q, k, v, bias, scale=scale, cap=cap)
        ref = np.array(oracle.attention_brute(q, k, v, bias, scale=scale, cap=cap))
        ok, err = _close(got, ref, TIGHT)
        if not ok:
            return False, f"brute S={S} Hq={Hq} cap={cap}: err {err:.3g}"
    return True, ""


# --------------------------------------------------------------------------
# Library routine: uncapped attention with an additive mask
# --------------------------------------------------------------------------
def _sdpa(q, k, v, bias, scale, bias_index=None):
    import torch
    B, S, Hq, Dk = q.shape
    out = np.empty((B, S, Hq, v.shape[-1]))
    for b in range(B):
        bi = b if bias_index is None else int(bias_index[b])
        tq = torch.from_numpy(np.ascontiguousarray(q[b].transpose(1, 0, 2)))
        tk = torch.from_numpy(np.ascontiguousarray(k[b, :, 0, :]))[None].expand(Hq, S, Dk)
        tv = torch.from_numpy(np.ascontiguousarray(v[b, :, 0, :]))[None].expand(Hq, S, -1)
        # repeat_interleave: each compact cell covers 16 consecutive positions.
        tb = torch.from_numpy(bias[bi])
        tb = tb.repeat_interleave(16, dim=1).repeat_interleave(16, dim=2)[:, :S, :S]
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.contiguous(), tv.contiguous(), attn_mask=tb.contiguous(), scale=scale)
        out[b] = o.numpy().transpose(1, 0, 2)
    return out


def pin_sdpa_uncapped(attn):
    for seed, (B, S, Hq, D) in enumerate([(1, 64, 8, 16), (2, 80, 3, 8), (1, 128, 8, 128)]):
        q, k, v, bias = _rand_case(200 + seed, B=B, S=S, Hq=Hq, Dk=D, Dv=D,
                                   qkv_std=1.0, bias_std=2.0)
        scale = 1.0 / math.sqrt(D)
        ref = _sdpa(q, k, v, bias, scale)
        ok, err = _close(attn(q, k, v, bias, scale=scale, cap=0.0), ref, TIGHT)
        if not ok:
            return False, f"sdpa uncapped S={S}: err {err:.3g}"
        # cap -> infinity equals the uncapped softmax
        ok, err = _close(attn(q, k, v, bias, scale=scale, cap=1e7), ref, 1e-9)
        if not ok:
            return False, f"cap->inf S={S}: err {err:.3g}"
    return True, ""


# --------------------------------------------------------------------------
# Closed forms of the soft-cap (artanh construction)
# --------------------------------------------------------------------------
def artanh(t):
    """artanh(t) = ln((1+t)/(1-t)) / 2, written from its definition."""
    return 0.5 * math.log((1.0 + t) / (1.0 - t))


def _closed_form_blocks(t_table, v):
    """Expected output when every logit of (query block p, key block r) is
    CAP * t_table[p][r]: weights exp(CAP t) per key, 16 keys per block."""
    Pq, Pk = t_table.shape
    S = v.shape[0]
    out = np.empty((S, v.shape[1]))
    for i in range(S):
        p = i // 16
        w = np.array([math.exp(CAP * t_table[p, j // 16]) for j in range(S)])
        out[i] = (w[:, None] * v).sum(0) / w.sum()
    return out


def pin_cap_closed_form(attn):
    """q = 0, bias cell = CAP * artanh(t): every logit of the cell is CAP * t,
    so the weights are known in closed form (no tanh evaluated)."""
    r = _rng(300)
    S, Hq, D = 64, 2, 8
    P = S // 16
    t = r.uniform(-0.95, 0.95, size=(Hq, P, P))
    bias = np.vectorize(lambda x: CAP * artanh(x))(t)[None]
    q = np.zeros((1, S, Hq, D))
    k = r.standard_normal((1, S, 1, D))
    v = r.standard_normal((1, S, 1, D))
    got = attn(q, k, v, bias, scale=1.0 / math.sqrt(D), cap=CAP)
    for h in range(Hq):
        ref = _closed_form_blocks(t[h], v[0, :, 0, :])
        ok, err = _close(got[0, :, h, :], ref, TIGHT)
        if not ok:
            return False, f"cap closed form head {h}: err {err:.3g}"
    return True, ""


def pin_bias_inside_cap(attn):
    """q_i = sqrt(Dk) e_0 and k_j = kappa_block(j) e_0, so scale * q.k is
    kappa of j's block; with bias = CAP artanh(t) - kappa the capped logit is
    CAP * t exactly when the bias sits inside the cap and the scale multiplies
    the dot product only."""
    r = _rng(301)
    S, Hq, D = 64, 2, 128
    P = S // 16
    t = r.uniform(-0.9, 0.9, size=(Hq, P, P))
    kappa = r.uniform(-2.0, 2.0, size=P)
    q = np.zeros((1, S, Hq, D))
    q[..., 0] = math.sqrt(D)
    k = np.zeros((1, S, 1, D))
    k[0, :, 0, 0] = np.repeat(kappa, 16)
    bias = np.empty((1, Hq, P, P))
    for h in range(Hq):
        for p in range(P):
            for j in range(P):
                bias[0, h, p, j] = CAP * artanh(t[h, p, j]) - kappa[j]
    v = r.standard_normal((1, S, 1, D))
    got = attn(q, k, v, bias, scale=1.0 / math.sqrt(D), cap=CAP)
    for h in range(Hq):
        ref = _closed_form_blocks(t[h], v[0, :, 0, :])
        ok, err = _close(got[0, :, h, :], ref, 1e-10)
        if not ok:
            return False, f"bias inside cap head {h}: err {err:.3g}"
    return True, ""


def pin_small_logit_limit(attn):
    """cap tanh(x/cap) = x - x^3 / (3 cap^2) + O(x^5): for |x| <= 1e-2 the
    capped and uncapped outputs differ by at most ~1e-7 relative."""
    q, k, v, bias = _rand_case(302, S=64, Hq=2, Dk=8, Dv=8, qkv_std=0.03, bias_std=0.004)
    a = attn(q, k, v, bias, scale=0.3, cap=CAP)
    b = attn(q, k, v, bias, scale=0.3, cap=0.0)
    ok, err = _close(a, b, 2e-7)
    if not ok:
        return False, f"small-logit limit err {err:.3g}"
    # and they are not identical: the cap does act.
    if np.array_equal(a, b):
        return False, "cap has no effect"
    return True, ""


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------
def pin_row_constant_uncapped(attn):
    """Without the cap, adding a constant to a compact bias row (all keys of
    query block p) leaves the softmax unchanged.  With the cap it does not."""
    q, k, v, bias = _rand_case(400, S=64, Hq=3, Dk=8, Dv=8, bias_std=1.5)
    c = _rng(401).standard_normal(bias.shape[:-1])[..., None] * 3.0
    a = attn(q, k, v, bias, scale=0.35, cap=0.0)
    b = attn(q, k, v, bias + c, scale=0.35, cap=0.0)
    ok, err = _close(a, b, TIGHT)
    if not ok:
        return False, f"row constant (uncapped) err {err:.3g}"
    a = attn(q, k, v, bias, scale=0.35, cap=CAP)
    b = attn(q, k, v, bias + c, scale=0.35, cap=CAP)
    if np.max(np.abs(a - b)) < 1e-3:
        return False, "row constant does not change the capped output"
    return True, ""


def pin_single_key(attn):
    """One key: the only weight is 1 and the output is that value row."""
    r = _rng(402)
    q = r.standard_normal((2, 1, 8, 16))
    k = r.standard_normal((2, 1, 1, 16))
    v = r.standard_normal((2, 1, 1, 16))
    bias = r.standard_normal((2, 8, 1, 1)) * 3
    for cap in (CAP, 0.0):
        out = attn(q, k, v, bias, scale=0.25, cap=cap)
        ref = np.broadcast_to(v, out.shape)
        ok, err = _close(out, ref, 1e-14)
        if not ok:
            return False, f"single key cap={cap}: err {err:.3g}"
    return True, ""


def pin_equal_values(attn):
    """All value rows equal to u: the output is u for every query and head."""
    q, k, v, bias = _rand_case(403, S=96, Hq=8, Dk=16, Dv=16, qkv_std=2.0, bias_std=2.0)
    u = _rng(404).standard_normal(16)
    v[:] = u
    out = attn(q, k, v, bias, scale=0.25, cap=CAP)
    ok, err = _close(out, np.broadcast_to(u, out.shape), 1e-13)
    return ok, ("" if ok else f"equal values err {err:.3g}")


def pin_weights_sum_to_one(attn):
    """With V = identity columns (Dv = S, v_j = e_j), the output rows are the
    attention weights themselves: non-negative and summing to one."""
    q, k, v, bias = _rand_case(405, S=48, Hq=2, Dk=8, Dv=8, qkv_std=1.0, bias_std=2.0)
    v = np.eye(48)[None, :, None, :]
    out = attn(q, k, v, bias, scale=0.5, cap=CAP)
    if np.min(out) < 0:
        return False, "negative weight"
    ok, err = _close(out.sum(-1), np.ones(out.shape[:-1]), 1e-13)
    return ok, ("" if ok else f"weights sum err {err:.3g}")


def pin_block_permutation(attn):
    """Keys permuted inside their 16-block (with their V rows) leave the output
    unchanged; queries permuted inside a 16-block permute the output rows."""
    q, k, v, bias = _rand_case(406, S=64, Hq=4, Dk=8, Dv=8, qkv_std=1.0, bias_std=2.0)
    r = _rng(407)
    perm = np.concatenate([16 * b + r.permutation(16) for b in range(4)])
    base = attn(q, k, v, bias, scale=0.4, cap=CAP)
    out = attn(q, k[:, perm], v[:, perm], bias, scale=0.4, cap=CAP)
    ok, err = _close(out, base, TIGHT)
    if not ok:
        return False, f"key permutation err {err:.3g}"
    out = attn(q[:, perm], k, v, bias, scale=0.4, cap=CAP)
    ok, err = _close(out, base[:, perm], TIGHT)
    if not ok:
        return False, f"query permutation err {err:.3g}"
    # a permutation across blocks does change the output
    cross = np.roll(np.arange(64), 16)
    out = attn(q, k[:, cross], v[:, cross], bias, scale=0.4, cap=CAP)
    if np.max(np.abs(out - base)) < 1e-6:
        return False, "cross-block permutation had no effect"
    return True, ""


def pin_linearity_in_v(attn):
    q, k, v, bias = _rand_case(408, S=64, Hq=2, Dk=8, Dv=8)
    v2 = _rng(409).standard_normal(v.shape)
    a = attn(q, k, v + 2.0 * v2, bias, scale=0.4, cap=CAP)
    b = attn(q, k, v, bias, scale=0.4, cap=CAP) + 2.0 * attn(q, k, v2, bias, scale=0.4, cap=CAP)
    ok, err = _close(a, b, TIGHT)
    return ok, ("" if ok else f"linearity err {err:.3g}")


def pin_independence(attn):
    """Changing q of one head changes only that head; changing one batch item's
    inputs changes only that item; a query row change touches only that row."""
    q, k, v, bias = _rand_case(410, B=2, S=64, Hq=4, Dk=8, Dv=8, bias_std=2.0)
    base = attn(q, k, v, bias, scale=0.4, cap=CAP)
    q2 = q.copy()
    q2[:, :, 2, :] += 1.0
    out = attn(q2, k, v, bias, scale=0.4, cap=CAP)
    d = np.abs(out - base).max(axis=(0, 1, 3))
    if d[2] < 1e-6 or np.delete(d, 2).max() > 0:
        return False, f"head independence {d}"
    k2 = k.copy()
    k2[1] += 0.5
    out = attn(q, k2, v, bias, scale=0.4, cap=CAP)
    d = np.abs(out - base).max(axis=(1, 2, 3))
    if d[0] > 0 or d[1] < 1e-6:
        return False, f"batch independence {d}"
    q3 = q.copy()
    q3[0, 37] += 1.0
    out = attn(q3, k, v, bias, scale=0.4, cap=CAP)
    d = np.abs(out - base).max(axis=(2, 3))[0]
    if d[37] < 1e-6 or np.delete(d, 37).max() > 0:
        return False, "query-row independence"
    return True, ""


def pin_bias_index(attn):
    """Items mapped to the same compact bias by ``bias_index`` equal a run with
    that bias given per item."""
    q, k, v, bias = _rand_case(411, B=4, S=32, Hq=2, Dk=8, Dv=8, bias_std=2.0, Bb=2)
    idx = np.array([0, 0, 1, 1])
    a = attn(q, k, v, bias, scale=0.4, cap=CAP, bias_index=idx)
    b = attn(q, k, v, bias[idx], scale=0.4, cap=CAP)
    ok, err = _close(a, b, 0.0)
    if not ok:
        return False, f"bias_index err {err:.3g}"
    return True, ""


def pin_mean_closed_form(attn):
    """q = 0 and bias = 0: every logit is 0, so every output row is the mean of
    the value rows."""
    r = _rng(412)
    S = 80
    q = np.zeros((1, S, 8, 16))
    k = r.standard_normal((1, S, 1, 16))
    v = r.standard_normal((1, S, 1, 16))
    bias = np.zeros((1, 8, 5, 5))
    out = attn(q, k, v, bias, scale=0.25, cap=CAP)
    ok, err = _close(out, np.broadcast_to(v[0, :, 0, :].mean(0), out.shape), 1e-13)
    return ok, ("" if ok else f"mean closed form err {err:.3g}")


def pin_tiled_recurrence(attn):
    """The online-softmax recurrence (tiles of 64 and of 16 keys) equals the
    dense definition up to rounding order."""
    for seed, cap in ((413, CAP), (414, 0.0)):
        q, k, v, bias = _rand_case(seed, B=2, S=192, Hq=3, Dk=16, Dv=12,
                                   qkv_std=1.2, bias_std=2.0)
        dense = attn(q, k, v, bias, scale=0.3, cap=cap)
        for tile in (64, 16):
            tiled = oracle.tiled_attention(q, k, v, bias, scale=0.3, cap=cap, tile=tile)
            ok, err = _close(tiled, dense, TIGHT)
            if not ok:
                return False, f"tiled({tile}) vs dense cap={cap}: err {err:.3g}"
    return True, ""


ATTENTION_PINS = [
    pin_brute_force, pin_sdpa_uncapped, pin_cap_closed_form, pin_bias_inside_cap,
    pin_small_logit_limit, pin_row_constant_uncapped, pin_single_key,
    pin_equal_values, pin_weights_sum_to_one, pin_block_permutation,
    pin_linearity_in_v, pin_independence, pin_bias_index, pin_mean_closed_form,
    pin_tiled_recurrence,
]


# --------------------------------------------------------------------------
# Projection pins: project(pair [Bp,P,P,C] or [P,P,C], weight [C,H])
# --------------------------------------------------------------------------
def pin_projection_brute(project):
    r = _rng(500)
    for P, C, H in ((4, 3, 8), (5, 16, 2)):
        pair = r.standard_normal((P, P, C))
        w = r.standard_normal((C, H))
        ok, err = _close(project(pair, w), np.array(oracle.project_brute(pair, w)), 1e-13)
        if not ok:
            return False, f"projection brute P={P} C={C}: err {err:.3g}"
    return True, ""


def pin_projection_identity(project):
    """W = I: the bias of head h is channel h of the pair representation."""
    pair = _rng(501).standard_normal((6, 6, 8))
    out = project(pair, np.eye(8))
    ok, err = _close(out, pair.transpose(2, 0, 1), 0.0)
    return ok, ("" if ok else f"identity projection err {err:.3g}")


def pin_projection_one_hot(project):
    """A pair representation that is one-hot in channel c at cell (p, r)
    projects to W[c, :] at (p, r) and to zero elsewhere."""
    C, H, P = 12, 8, 5
    w = _rng(502).standard_normal((C, H))
    pair = np.zeros((P, P, C))
    pair[3, 1, 7] = 1.0
    out = project(pair, w)
    ref = np.zeros((H, P, P))
    ref[:, 3, 1] = w[7]
    ok, err = _close(out, ref, 0.0)
    return ok, ("" if ok else f"one-hot projection err {err:.3g}")


def pin_projection_batched(project):
    """A batch of pair representations projects item by item."""
    r = _rng(503)
    pair = r.standard_normal((3, 4, 4, 6))
    w = r.standard_normal((6, 8))
    out = project(pair, w)
    for b in range(3):
        ok, err = _close(out[b], np.array(oracle.project_brute(pair[b], w)), 1e-13)
        if not ok:
            return False, f"batched projection item {b}: err {err:.3g}"
    return True, ""


PROJECTION_PINS = [pin_projection_brute, pin_projection_identity,
                   pin_projection_one_hot, pin_projection_batched]
