"""The kernels' visibility arithmetic, compiled for the host, against the
oracle's element predicate (CPU only).

Partial tiles are masked on the device with the 64-bit masks
row_visible_bits (query t, keys base..base+63: prefill forward and dQ) and
col_visible_bits (key j, queries base..base+63: dK/dV); the decode kernels
walk the key ranges of row_ranges.  tests/host_shim.cpp builds these very
header functions with g++; here every bit and every range is compared with
oracle.visible / oracle.decode_visible_keys ("Splitting long-range windows
across KV heads beats duplicating them at lower cost", mechanism paragraph;
"CoWindow Attention: Full Causal Coverage Is a Collective Property",
Abstract).  The library's cowa_visible_ranges export is checked the same way
at the 128K decode workload's drawn lengths."""

import numpy as np
import pytest

import oracle.cowa_oracle as O
from structured_sparse_attention_cowa_amd import binding as C
from structured_sparse_attention_cowa_amd import workloads as W
from tests import host_shim

PATTERNS = [
    O.Pattern(1024, 16, 128, 0, 4, 0, 0),
    O.Pattern(1000, 7, 100, 0, 8, 0, 0),
    O.Pattern(777, 0, 1, 0, 4, 0, 0),
    O.Pattern(512, 200, 3, 0, 2, 0, 0),
    O.Pattern(300, 400, 1, 0, 2, 0, 0),
    O.Pattern(1024, 16, 128, 0, 4, 0, O.MODE_CAUSAL),
    O.Pattern(1024, 4, 60, 0, 4, 0, O.MODE_SINK_LOCAL),
    O.Pattern(1024, 16, 64, 0, 8, 0, 0, 2),
    O.Pattern(131072, 128, 8192, 0, 8, 0, 0),
]


def _hp_args(p, g):
    return (p.sink, p.window, O.resolved_band(p), O.band_index(g, p),
            1 if p.mode == O.MODE_CAUSAL else 0)


def _rows_of_interest(p):
    L = O.resolved_band(p)
    ts = [0, 1, 2, 3, 63, 64, 65, p.sink - 1, p.sink, p.sink + 1, p.window - 1, p.window,
          p.window + 1, p.n_ctx - 1]
    for b in range(p.h_kv_global + 1):
        e = p.window + b * L
        ts += [e - 1, e, e + 1, e + 63, e + 64, e + p.sink, e + p.sink + 1]
    return sorted({t for t in ts if 0 <= t < p.n_ctx})


def _bases(t, p, span):
    """Tile bases (multiples of 4, as the kernels use) whose 64 keys or
    queries cover the edges of row t's windows."""
    L = O.resolved_band(p)
    edges = [0, p.sink, t, t - p.window + 1]
    edges += [t - p.window - b * L + 1 for b in range(p.h_kv_global + 1)]
    out = set()
    for e in edges:
        for base in range(e - span, e + span, 4):
            if base >= 0:
                out.add(base - base % 4)
    return sorted(out)


@pytest.mark.parametrize("pi", range(len(PATTERNS)))
def test_row_masks_equal_predicate(pi):
    lib = host_shim.load()
    p = PATTERNS[pi]
    o = np.arange(64)
    for g in range(p.h_kv_global):
        args = _hp_args(p, g)
        for t in _rows_of_interest(p):
            for base in _bases(t, p, 80):
                m = lib.shim_row_visible_bits(*args, t, base)
                got = np.array([(m >> int(i)) & 1 for i in o], dtype=bool)
                want = O.visible(t, base + o, g, p)
                assert np.array_equal(got, want), (p, g, t, base)


@pytest.mark.parametrize("pi", range(len(PATTERNS)))
def test_col_masks_equal_predicate(pi):
    lib = host_shim.load()
    p = PATTERNS[pi]
    o = np.arange(64)
    L = O.resolved_band(p)
    for g in range(p.h_kv_global):
        args = _hp_args(p, g)
        keys = sorted({0, 1, p.sink - 1, p.sink, p.sink + 1, 100, p.n_ctx // 2, p.n_ctx - 1})
        for j in (k for k in keys if 0 <= k < p.n_ctx):
            # query tiles around the key's diagonal and every window edge
            edges = [j, j + p.window - 1, j + p.window]
            edges += [j + p.window + b * L + s for b in range(p.h_kv_global + 1) for s in (-1, 0)]
            bases = sorted({max(0, e + s) // 4 * 4 for e in edges for s in range(-72, 72, 4)})
            for base in bases:
                m = lib.shim_col_visible_bits(*args, base, j)
                got = np.array([(m >> int(i)) & 1 for i in o], dtype=bool)
                want = O.visible(base + o, j, g, p)
                assert np.array_equal(got, want), (p, g, j, base)


def _keys_of(ranges):
    parts = [np.arange(a, b) for a, b in ranges]
    return np.concatenate(parts)


@pytest.mark.parametrize("pi", range(len(PATTERNS) - 1))
def test_row_ranges_equal_oracle_keys_every_row(pi):
    """row_ranges (host build) and cowa_visible_ranges (the library) give
    disjoint ascending ranges whose keys are exactly the oracle's, for every
    row of the small patterns and every head."""
    lib = host_shim.load()
    p = PATTERNS[pi]
    cp = C.make_pattern(p.n_ctx, p.sink, p.window, p.band, p.h_kv_global, 0, p.mode, p.n_bands)
    lo, hi = host_shim.int_array(3), host_shim.int_array(3)
    for g in range(p.h_kv_global):
        args = _hp_args(p, g)
        for t in range(p.n_ctx):
            lib.shim_row_ranges(*args, t, lo, hi)
            r = [(lo[i], hi[i]) for i in range(3)]
            assert r == C.cowa_visible_ranges(cp, g, t)
            assert all(a <= b for a, b in r)
            keys = _keys_of(r)
            assert np.all(np.diff(keys) > 0)  # disjoint and ascending
            assert np.array_equal(keys, O.decode_visible_keys(t, g, p)), (g, t)


def test_visible_ranges_at_decode_workload():
    """cowa_visible_ranges at the 128K decode workload's drawn lengths and at
    lengths where the sequence start meets each band edge, every head."""
    w = W.D128K
    p = O.Pattern(w.n_ctx, w.sink, w.window, 0, w.h_kv_global)
    cp = C.make_pattern(w.n_ctx, w.sink, w.window, 0, w.h_kv_global, 0, 0)
    L = O.resolved_band(p)
    lens = [int(x) for x in W.decode_lens(w)] + [1, 2, w.sink, w.sink + 1, w.n_max]
    lens += [w.window + g * L + s for g in range(w.h_kv_global + 1) for s in (0, 1)]
    for n in sorted({x for x in lens if 1 <= x <= w.n_max}):
        for g in range(w.h_kv_global):
            r = C.cowa_visible_ranges(cp, g, n - 1)
            assert np.array_equal(_keys_of(r), O.decode_visible_keys(n - 1, g, p)), (n, g)


def test_visible_ranges_rejects_bad_arguments():
    cp = C.make_pattern(1024, 16, 128, 0, 4, 2, 0)
    for h, t in ((-1, 5), (2, 5), (0, -1)):
        with pytest.raises(C.CowaError):
            C.cowa_visible_ranges(cp, h, t)
    assert C.cowa_visible_ranges(cp, 1, 0) == [(0, 1), (1, 1), (1, 1)]
