"""Pins of the oracle's error-bound helpers (CPU only).

The backward parity bounds use the oracle's D-sensitivities eq, ek (from
_d_sensitivity), and the windowed KV cache is checked against the oracle's
retained_mask.  Both are pinned here against things other than themselves:

  * _d_sensitivity: with every key vector equal to the ones vector, each row's
    softmax is uniform over its visible set, so w_t and eq_t = scale w_t have
    a closed form written out below from the visible set; shifting the
    oracle backward's D_t by eps w_t moves dQ and dK by at most eps eq and
    eps ek, and by exactly that much when q, k have one sign per component.
    (The training backward of the operator: "CoWindow Attention: Full Causal
    Coverage Is a Collective Property", Abstract.)
  * retained_mask: the keys a decode cache must still hold after position t
    (Abstract: lower decode memory; the pattern is position arithmetic, news
    page mechanism paragraph) have the closed form
        j <= t and (j < S or t - j < W or
                    (L > 0 and t - j < W + (b+1) L and j + W + b L < n_max)),
    b the head's window index: a later query t' in [t, n_max) sees j through
    the band iff [j + W + bL, j + W + (b+1)L) meets [t, n_max).
"""

import numpy as np
import pytest

import oracle.cowa_oracle as O

CASES = [
    (40, 4, 2, 16, dict(sink=2, window=5, h=4, off=1)),
    (33, 3, 3, 8, dict(sink=0, window=1, h=2, off=0)),
    (48, 2, 1, 16, dict(sink=3, window=7, h=4, off=0, mode=O.MODE_CAUSAL)),
]


def _inputs(seed, N, Hq, Hkv, d, ones_k=False, positive_q=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((1, N, Hq, d))
    k = rng.standard_normal((1, N, Hkv, d))
    v = rng.standard_normal((1, N, Hkv, d))
    do = rng.standard_normal((1, N, Hq, d))
    if ones_k:
        k = np.ones_like(k)
    if positive_q:
        q = np.abs(q) + 0.1
    return q, k, v, do


def _pattern(N, kw):
    return O.Pattern(N, kw["sink"], kw["window"], 0, kw["h"], kw["off"], kw.get("mode", 0))


def _closed_form_w(v, do, p, N, Hq, Hkv):
    """w_t for uniform rows: sum_c |dO_tc| (mean_vis |v_jc| + |mean_vis v_jc|)."""
    G = Hq // Hkv
    w = np.zeros((N, Hq))
    for hq in range(Hq):
        h = hq // G
        g = p.kv_head_offset + h
        for t in range(N):
            keys = O.decode_visible_keys(t, g, p)
            vv = v[0, keys, h]
            w[t, hq] = (np.abs(do[0, t, hq]) * (np.abs(vv).mean(axis=0) +
                                                 np.abs(vv.mean(axis=0)))).sum()
    return w


@pytest.mark.parametrize("case", CASES)
def test_d_sensitivity_closed_form_for_uniform_rows(case):
    N, Hq, Hkv, d, kw = case
    p = _pattern(N, kw)
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = _inputs(1, N, Hq, Hkv, d, ones_k=True)
    eq = O.attention_backward(q, k, v, do, p, scale, magnitudes=True)[6]
    w = _closed_form_w(v, do, p, N, Hq, Hkv)
    np.testing.assert_allclose(eq[0], scale * w[:, :, None] * np.ones(d), rtol=1e-12, atol=0)


@pytest.mark.parametrize("case", CASES)
def test_d_shift_bound_is_attained(case):
    """q > 0 componentwise and k = 1: a shift of D_t by eps w_t moves every
    dQ and dK element by exactly eps eq and eps ek."""
    N, Hq, Hkv, d, kw = case
    p = _pattern(N, kw)
    scale = 1.0 / np.sqrt(d)
    eps = 1e-3
    q, k, v, do = _inputs(2, N, Hq, Hkv, d, ones_k=True, positive_q=True)
    ref = O.attention_backward(q, k, v, do, p, scale, magnitudes=True)
    w = _closed_form_w(v, do, p, N, Hq, Hkv)
    sh = O.attention_backward(q, k, v, do, p, scale, d_shift=eps * w[None])
    np.testing.assert_allclose(np.abs(sh[0] - ref[0]), eps * ref[6], rtol=1e-8, atol=1e-15)
    np.testing.assert_allclose(np.abs(sh[1] - ref[1]), eps * ref[7], rtol=1e-8, atol=1e-15)


@pytest.mark.parametrize("case", CASES)
def test_d_shift_bound_holds_in_general(case):
    """Random q, k and shifts of either sign with |shift_t| <= eps w_t: the
    gradients move by at most eps eq, eps ek.  w_t is read off eq_t as
    eq_t / (scale sum_j P_tj |k_j|), the sum being the oracle forward with
    |k| as the values, and is checked against its definition
    sum_c |dO_tc| (sum_j P_tj |v_jc| + |O_tc|) built from oracle forwards."""
    N, Hq, Hkv, d, kw = case
    p = _pattern(N, kw)
    scale = 1.0 / np.sqrt(d)
    eps = 1e-3
    q, k, v, do = _inputs(3, N, Hq, Hkv, d)
    ref = O.attention_backward(q, k, v, do, p, scale, magnitudes=True)
    # w_t from eq_t / (scale sum_j P_tj |k_j|): recover sum_j P |k| from the
    # oracle's forward with |k| as the values
    o_absk, _ = O.attention(q, k, np.abs(k), p, scale)
    w = np.zeros((N, Hq))
    for hq in range(Hq):
        w[:, hq] = ref[6][0, :, hq, 0] / (scale * o_absk[0, :, hq, 0])
    rng = np.random.Generator(np.random.PCG64(9))
    shift = eps * w[None] * rng.uniform(-1, 1, size=w.shape)[None]
    sh = O.attention_backward(q, k, v, do, p, scale, d_shift=shift)
    assert (np.abs(sh[0] - ref[0]) <= eps * ref[6] * (1 + 1e-9) + 1e-15).all()
    assert (np.abs(sh[1] - ref[1]) <= eps * ref[7] * (1 + 1e-9) + 1e-15).all()
    # and w_t really is the same quantity as the closed form's ingredients:
    # sum_c |dO_tc| (sum_j P_tj |v_jc| + |O_tc|), with P and O from the forward
    o_absv, _ = O.attention(q, k, np.abs(v), p, scale)
    o, _ = O.attention(q, k, v, p, scale)
    for hq in range(Hq):
        want = (np.abs(do[0, :, hq]) * (o_absv[0, :, hq] + np.abs(o[0, :, hq]))).sum(axis=1)
        np.testing.assert_allclose(w[:, hq], want, rtol=1e-10)


RET_PATTERNS = [
    (64, dict(sink=3, window=5, h=4, off=0)),
    (61, dict(sink=0, window=1, h=4, off=0)),
    (50, dict(sink=60, window=2, h=2, off=0)),
    (64, dict(sink=2, window=4, h=8, off=0, n_bands=2)),
    (40, dict(sink=2, window=6, h=4, off=0, mode=O.MODE_SINK_LOCAL)),
]


def _retained_closed_form(n_max, g, p):
    t = np.arange(n_max)[:, None]
    j = np.arange(n_max)[None, :]
    L = O.resolved_band(p)
    b = O.band_index(g, p)
    keep = (j < p.sink) | (t - j < p.window)
    if L > 0:
        keep |= (t - j < p.window + (b + 1) * L) & (j + p.window + b * L < n_max)
    return (j <= t) & keep


@pytest.mark.parametrize("case", RET_PATTERNS)
def test_retained_mask_closed_form(case):
    n_max, kw = case
    p = O.Pattern(n_max, kw["sink"], kw["window"], 0, kw["h"], kw["off"], kw.get("mode", 0),
                  kw.get("n_bands", 0))
    for g in range(kw["h"]):
        assert np.array_equal(O.retained_mask(n_max, g, p), _retained_closed_form(n_max, g, p)), g
