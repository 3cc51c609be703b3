"""Pattern variants on the same plan and kernels (CPU): sliding-window
attention with sinks (no long-range window) and the duplicated-window
ablation (m distinct long-range windows over the KV heads).

Pins of the oracle come from the pages' descriptions of the two patterns;
the host plan is compared bit for bit with the oracle's own enumeration."""

import ctypes

import numpy as np
import pytest

import oracle.cowa_oracle as O
from oracle.cowa_oracle import MODE_COWA, MODE_SINK_LOCAL, Pattern
from structured_sparse_attention_cowa_amd import binding as C


def test_sink_local_row_counts_match_swa_with_sinks():
    """SWA(w, 4) on the SWA-with-sinks page: a total window of w keys, 4 of
    them the first positions (sinks), the other w - 4 the most recent keys.
    As a pattern: S = 4, W = w - 4, no band; every row sees min(t + 1, w)
    keys, the first min(t + 1, 4) positions among them."""
    w = 64
    for n in (40, 64, 200, 1000):
        p = Pattern(n_ctx=n, sink=4, window=w - 4, h_kv_global=4, mode=MODE_SINK_LOCAL)
        for g in range(4):
            m = O.visible_mask(n, n, g, p)
            t = np.arange(n)
            assert np.array_equal(m.sum(axis=1), np.minimum(t + 1, w))
            assert m[:, :4][np.arange(n) >= 3].all()
            assert [O.visible_count(int(tt), g, p) for tt in (0, n - 1)] == [1, min(n, w)]


def test_sink_local_is_the_band_free_cowa():
    """CoWA with n_ctx <= W has no band (L = 0); the sink-local mode gives the
    same sets at any n_ctx, for every head."""
    n = 300
    for S, Wd in ((0, 16), (5, 40), (7, 1)):
        a = Pattern(n_ctx=n, sink=S, window=Wd, h_kv_global=4, mode=MODE_SINK_LOCAL)
        b = Pattern(n_ctx=Wd, sink=S, window=Wd, h_kv_global=4, mode=MODE_COWA)
        assert O.resolved_band(a) == 0 and O.resolved_band(b) == 0
        for g in range(4):
            assert np.array_equal(O.visible_mask(n, n, g, a), O.visible_mask(n, n, g, b))


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_duplicated_windows_coverage(m):
    """The ablation spreads m distinct long-range windows over 8 KV heads at
    fixed per-head width: beyond the shared windows, a distance in one of the
    first m bands is seen by exactly 8/m heads and any farther distance by
    none; with m = 8 the pattern is CoWA's (full causal coverage)."""
    n, S, Wd, H = 1000, 3, 20, 8
    p = Pattern(n_ctx=n, sink=S, window=Wd, h_kv_global=H, n_bands=m)
    L = O.resolved_band(p)
    assert L == -(-(n - Wd) // H)
    shared = O.visible_mask(n, n, 0, Pattern(n_ctx=Wd, sink=S, window=Wd, h_kv_global=H))
    count = sum(O.visible_mask(n, n, g, p).astype(int) for g in range(H))
    t = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    dist = t - j
    far = (dist >= Wd) & (j >= S)
    assert (count[shared] == H).all()
    inside = far & (dist < Wd + m * L)
    assert (count[inside] == H // m).all()
    assert (count[far & ~inside] == 0).all()
    if m == H:
        cowa = Pattern(n_ctx=n, sink=S, window=Wd, h_kv_global=H)
        for g in range(H):
            assert np.array_equal(O.visible_mask(n, n, g, p), O.visible_mask(n, n, g, cowa))


def test_one_distinct_window_gives_every_head_the_same_set():
    p = Pattern(n_ctx=500, sink=2, window=30, h_kv_global=8, n_bands=1)
    m0 = O.visible_mask(500, 500, 0, p)
    for g in range(1, 8):
        assert np.array_equal(O.visible_mask(500, 500, g, p), m0)


def pat(**kw):
    base = dict(n_ctx=1024, sink=16, window=128, band=0, h_kv_global=4, kv_head_offset=0, mode=0,
                n_bands=0)
    base.update(kw)
    return C.make_pattern(**base), O.Pattern(**base)


@pytest.mark.parametrize("kw", [dict(mode=2), dict(n_bands=1), dict(n_bands=2),
                                dict(n_bands=2, kv_head_offset=1), dict(n_bands=3, n_ctx=1000)])
@pytest.mark.parametrize("bm,bn", [(256, 64), (64, 128), (16, 16)])
def test_variant_plans_bit_exact(lib, kw, bm, bn):
    hkv = 4 - kw.get("kv_head_offset", 0)
    cp, op = pat(**kw)
    n = op.n_ctx
    rp, col, fl = C.cowa_plan(cp, n, hkv, bm, bn)
    orp, ocol, ofl = O.tile_lists(n, hkv, op, bm, bn, method="bruteforce")
    assert np.array_equal(rp, orp) and np.array_equal(col, ocol) and np.array_equal(fl, ofl)
    rp, col, fl = C.cowa_plan_kv(cp, n, hkv, bm, bn)
    orp, ocol, ofl = O.tile_lists_kv(n, hkv, op, bm, bn, method="bruteforce")
    assert np.array_equal(rp, orp) and np.array_equal(col, ocol) and np.array_equal(fl, ofl)


@pytest.mark.parametrize("m", [1, 2, 4])
def test_variant_plan_8k_fast_enumeration(lib, m):
    cp, op = pat(n_ctx=8192, sink=64, window=1024, h_kv_global=8, n_bands=m)
    rp, col, fl = C.cowa_plan(cp, 8192, 8, 256, 64)
    orp, ocol, ofl = O.tile_lists(8192, 8, op, 256, 64, method="fast")
    assert np.array_equal(rp, orp) and np.array_equal(col, ocol) and np.array_equal(fl, ofl)


def test_variant_pattern_validation(lib):
    L = C.load()
    out = ctypes.c_int64()
    for kw in (dict(n_bands=-1), dict(n_bands=5), dict(mode=3)):
        cp, _ = pat(**kw)
        assert L.cowa_plan_size(ctypes.byref(cp), 1024, 4, 256, 64, ctypes.byref(out)) == \
            C.COWA_ERR_INVALID_ARG, kw
    cp, _ = pat(mode=2)
    assert C.cowa_band_length(cp) == 0
    cp, _ = pat(n_bands=2)
    assert C.cowa_band_length(cp) == 224  # the width stays ceil((N - W) / H_kv_global)
