"""CPU tests of the windowed KV cache layout: the rings the library reserves
hold every key a later decode step can read (brute force from the oracle's
visibility), are no larger than needed, and bad calls are rejected."""

import ctypes

import numpy as np
import pytest

import oracle.cowa_oracle as O
from structured_sparse_attention_cowa_amd import binding as C


@pytest.mark.parametrize("kw", [
    dict(n_ctx=600, sink=5, window=30, h_kv_global=4),
    dict(n_ctx=600, sink=0, window=1, h_kv_global=8),
    dict(n_ctx=600, sink=7, window=40, h_kv_global=4, n_bands=2),
    dict(n_ctx=600, sink=4, window=60, h_kv_global=4, mode=2),
    dict(n_ctx=300, sink=3, window=20, h_kv_global=4),   # queries past n_ctx (n_max 900)
])
def test_rings_hold_exactly_what_later_queries_read(lib, kw):
    n_max = 900
    H = kw["h_kv_global"]
    cp = C.make_pattern(**kw)
    op = O.Pattern(**kw)
    rows, total = C.cowa_kv_window_rows(cp, H, n_max)
    S = min(kw["sink"], n_max)
    assert total == rows.sum() and (rows >= S).all()
    for g in range(H):
        R = int(rows[g]) - S
        keep = O.retained_mask(n_max, g, op)
        t = np.arange(n_max)[:, None]
        j = np.arange(n_max)[None, :]
        nonsink = keep & (j >= S)
        # every key still needed is within the ring's reach (no two share a row)
        assert not (nonsink & (t - j >= R)).any(), g
        # and no larger than the most keys ever needed at once (when the cache
        # is long enough for some query to have a full ring of later readers;
        # near the cache's end fewer keys are needed, and the ring is an
        # upper bound)
        most = nonsink.sum(axis=1).max()
        assert most == R if S + 2 * R <= n_max else most <= R, g


def test_ring_rows_at_the_decode_workload(lib):
    cp = C.make_pattern(131072, 128, 8192, 0, 8, 0, 0)
    rows, total = C.cowa_kv_window_rows(cp, 8, 131072)
    # head g keeps 128 sink rows and W + (g+1) L = 8192 + (g+1) 15360 ring rows,
    # capped at the cache size
    assert list(rows) == [min(128 + 8192 + (g + 1) * 15360, 131072) for g in range(8)]
    assert total == 619392
    # one tensor-parallel rank (a single KV head at offset g) keeps rows[g]
    cp0 = C.make_pattern(131072, 128, 8192, 0, 8, 0, 0)
    assert C.cowa_kv_window_rows(cp0, 1, 131072)[1] == 23680


def test_window_validation(lib):
    L = C.load()
    out = ctypes.c_int64()
    cpc = C.make_pattern(1000, 4, 64, 0, 4, 0, 1)
    assert L.cowa_kv_window_rows(ctypes.byref(cpc), 4, 1000, None, ctypes.byref(out)) == \
        C.COWA_ERR_UNSUPPORTED
    cp = C.make_pattern(1000, 4, 64, 0, 4, 0, 0)
    assert L.cowa_kv_window_rows(ctypes.byref(cp), 4, 0, None, ctypes.byref(out)) == \
        C.COWA_ERR_INVALID_ARG
    rows, total = C.cowa_kv_window_rows(cp, 4, 1000)
    fake = ctypes.c_void_p(0x1000)
    small = (ctypes.c_int64 * 8)(1, 1, 1, 1, 1, 1, total * 128 - 1, total * 128)
    assert L.cowa_kv_window_fill(ctypes.byref(cp), fake, fake, fake, fake, fake, 2, 4, 128, 1000,
                                 small, None) == C.COWA_ERR_INVALID_ARG
    st = (ctypes.c_int64 * 6)(8, 8, 8, 8, total * 128, total * 128)
    assert L.cowa_kv_window_append(ctypes.byref(cp), fake, fake, fake, fake, fake, 2, 4, 96,
                                   1000, st, None) == C.COWA_ERR_UNSUPPORTED
    dst = (ctypes.c_int64 * 6)(1, 1, total * 128 - 8, total * 128, 1, 1)
    assert L.cowa_decode_window(ctypes.byref(cp), fake, fake, fake, fake, fake, 1, fake, 2, 8, 4,
                                128, 1000, dst, 0.1, ctypes.c_void_p(0x100000), 1 << 30,
                                None) == C.COWA_ERR_INVALID_ARG
