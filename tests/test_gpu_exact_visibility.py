"""Exact, key-by-key visibility parity of the GPU kernels at full size.

With Q = 0 every visible score is 0, so each head's softmax is uniform over
its own visible set ("Splitting long-range windows across KV heads beats
duplicating them at lower cost", paragraph on what CoWA does not claim; the
set itself from the mechanism paragraph and "CoWindow Attention: Full Causal
Coverage Is a Collective Property", Abstract).  Then exp(LSE) is the number
of visible keys and O * count is the sum of their value rows.  The value rows
are 0/1 position codes (the binary digits of the position and of a hash of
it, exact in bf16): the kernels' fp32 sums of them are exact integers, so
every row's count and code sums are compared as integers with the oracle's
visible_code_sums.  One key more or less, a shifted band, a missing sink or a
swapped key changes them (tests/test_exact_visibility.py shows this on the
oracle), which the O <= 2e-2 and LSE <= 1e-3 tolerances of random-data
parity cannot see at 23,680 visible keys.  Every row of every head is
checked.  Decode caches hold NaN at and after each length, so a read past it
shows up as well."""

import numpy as np
import pytest

import oracle.cowa_oracle as O
from structured_sparse_attention_cowa_amd import binding as C
from structured_sparse_attention_cowa_amd import workloads as W
from tests.gpu_helpers import Prefill, bits_to_dev

pytestmark = pytest.mark.gpu

NC = W.N_POSITION_CODES
# Code sums: |O * count - sum| <= SUM_TOL.  The fp32 sums of 0/1 codes are
# exact integers; only the final division (and in decode the log-sum-exp
# weights of the chunks) round, by relative errors of a few 1e-7 to 2e-6,
# i.e. well below 0.45 for sums up to 65536.  Two visible sets of equal size
# whose code sums agree within 0.45 agree exactly: exchanging one key for
# another changes some binary digit's sum by 1.
SUM_TOL = 0.45


def lse_tolerance(counts):
    """|LSE - ln(count)| allowed per row: 0.45 of the distance to ln(count + 1),
    so that a row seeing one key more or less always fails.  At 131072 keys
    this is 3.4e-6, about four units in the last place of an fp32 LSE near 12
    (the kernels' fp32 logarithm is off by about two)."""
    c = np.asarray(counts, np.float64)
    return 0.45 * np.log1p(1.0 / c)


def check_exact(o, lse, counts, sums, what):
    """o [R, H, >=NC] fp32 (rows x query heads), lse [H, R]; counts [R],
    sums [R, NC] (the heads of o all use these)."""
    lse = np.asarray(lse, np.float64)
    assert np.isfinite(lse).all(), f"{what}: non-finite LSE"
    assert counts.min() >= 1 and counts.max() <= 1 << 17
    err = np.abs(lse - np.log(counts.astype(np.float64))[None, :])
    bad = err > lse_tolerance(counts)[None, :]
    if bad.any():
        h, r = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: head {h} row {r}: exp(LSE) = {np.exp(lse[h, r]):.4f}, "
                             f"visible count {counts[r]} (LSE error {err[h, r]:.2e})")
    s = np.asarray(o[:, :, :NC], np.float64) * counts[:, None, None]
    bad = np.abs(s - sums[:, None, :]) > SUM_TOL
    if bad.any():
        r, h, c = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: row {r} head {h} code {c}: O * count = {s[r, h, c]:.4f},"
                             f" oracle sum {sums[r, c]}")
    return float((err / lse_tolerance(counts)[None, :]).max())


def _zero_rest(o, what):
    import torch
    assert bool((o[..., NC:] == 0).all()), f"{what}: nonzero output beyond the codes"
    assert bool(torch.isfinite(o).all()), f"{what}: non-finite O"


def _prefill_exact(x, sink, window, h_kv_global, offset=0, mode=0, n_ctx=None, n_bands=0,
                   what=""):
    pf = Prefill(x, sink, window, h_kv_global, offset, mode, n_ctx, "f32", n_bands)
    print(f"[exact prefill] {what} N={pf.N} B={pf.B} Hq={pf.Hq} Hkv={pf.Hkv} d={pf.d} "
          f"g0={offset} mode={mode}", flush=True)
    pf.run()
    import torch
    torch.cuda.synchronize()
    _zero_rest(pf.o, what)
    o = pf.o[..., :NC].cpu().numpy()
    lse = pf.lse.cpu().numpy()
    G = pf.Hq // pf.Hkv
    for b in range(pf.B):
        for h in range(pf.Hkv):
            codes = W.position_codes(np.arange(pf.N), b * pf.Hkv + h).astype(np.int64)
            cnt, sums = O.visible_code_sums(np.arange(pf.N), offset + h, pf.opattern, codes)
            hs = slice(h * G, (h + 1) * G)
            check_exact(o[b, :, hs], lse[b, hs], cnt, sums, f"{what} b={b} h={h}")


_X128 = {}


def _x128():
    w = W.P128K
    if "x" not in _X128:
        _X128["x"] = W.zero_query_inputs(41, w.B, w.N, w.H_q, w.H_kv, w.d)
    return _X128["x"]


@pytest.mark.parametrize("g", range(8))
def test_exact_prefill_128k_rank(lib, g):
    """Every row and query head of the 128K single-rank prefill, each global
    KV head g = 0..7 (the eight tensor-parallel ranks)."""
    w = W.P128K
    _prefill_exact(_x128(), w.sink, w.window, w.h_kv_global, offset=g, what=f"128K g={g}")


def test_exact_prefill_128k_causal(lib):
    w = W.P128K
    _prefill_exact(_x128(), w.sink, w.window, w.h_kv_global, mode=1, what="128K causal")


@pytest.mark.parametrize("mode", [0, 1])
def test_exact_prefill_32k(lib, mode):
    """The 32K workload shape (40 query heads over 8 KV heads), CoWA and
    full-causal mode; each KV head has its own codes."""
    w = W.P32K
    x = W.zero_query_inputs(42, w.B, w.N, w.H_q, w.H_kv, w.d)
    _prefill_exact(x, w.sink, w.window, w.h_kv_global, mode=mode, what=f"32K mode={mode}")


def test_exact_prefill_8k(lib):
    w = W.P8K
    x = W.zero_query_inputs(43, w.B, w.N, w.H_q, w.H_kv, w.d)
    _prefill_exact(x, w.sink, w.window, w.h_kv_global, what="8K")


def test_exact_prefill_tiny_d64(lib):
    w = W.TINY
    x = W.zero_query_inputs(44, w.B, w.N, w.H_q, w.H_kv, w.d)
    _prefill_exact(x, w.sink, w.window, w.h_kv_global, what="tiny")


@pytest.mark.parametrize("case", [
    (1000, 8, 2, 128, dict(sink=7, window=100, h_kv_global=8, offset=5)),
    (2049, 6, 3, 64, dict(sink=0, window=1, h_kv_global=4, offset=1)),
    (777, 4, 1, 128, dict(sink=5, window=60, h_kv_global=4, mode=2)),
    (1500, 8, 4, 128, dict(sink=16, window=64, h_kv_global=8, n_bands=2, offset=4)),
    (300, 2, 1, 128, dict(sink=400, window=1, h_kv_global=2)),
])
def test_exact_prefill_edge_shapes(lib, case):
    """Ragged lengths, band-only, sink + local only, duplicated windows and a
    sink longer than the sequence."""
    N, Hq, Hkv, d, kw = case
    x = W.zero_query_inputs(45, 2, N, Hq, Hkv, d)
    _prefill_exact(x, what=f"edge N={N}", **kw)


def test_exact_prefill_varlen(lib):
    """Packed sequences: positions restart at 0 in each, so each sequence's
    rows see exactly its own keys under the pattern."""
    import torch
    lens = np.array([1000, 1, 0, 2500, 300, 4097], np.int64)
    Hq, Hkv, d = 8, 2, 128
    S, Wd, H, off = 16, 128, 8, 3
    T, max_len = int(lens.sum()), int(lens.max())
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    k = np.zeros((T, Hkv, d), np.uint16)
    v = np.zeros((T, Hkv, d), np.uint16)
    rng = np.random.Generator(np.random.PCG64(46))
    k[:] = W.to_bf16_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32))
    for i, n in enumerate(lens):
        for h in range(Hkv):
            v[cu[i]:cu[i + 1], h] = W.position_code_rows(int(n), d, i * Hkv + h)
    p = C.make_pattern(max_len, S, Wd, 0, H, off, 0)
    op = O.Pattern(max_len, S, Wd, 0, H, off, 0)
    bm, bn = C.cowa_fwd_block_sizes(d)
    rp, col, fl = [torch.from_numpy(a).cuda() for a in C.cowa_plan(p, max_len, Hkv, bm, bn)]
    q = torch.zeros((T, Hq, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full((T, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[exact varlen] lens={list(lens)}", flush=True)
    C.cowa_fwd_varlen(p, rp, col, fl, col.numel(), bm, bn, q, bits_to_dev(k), bits_to_dev(v),
                      o, lse, torch.from_numpy(cu).cuda(), max_len, 1.0 / np.sqrt(d))
    torch.cuda.synchronize()
    _zero_rest(o, "varlen")
    o_h, lse_h = o[..., :NC].cpu().numpy(), lse.cpu().numpy()
    G = Hq // Hkv
    for i, n in enumerate(lens):
        if n == 0:
            continue
        a, b = int(cu[i]), int(cu[i + 1])
        for h in range(Hkv):
            codes = W.position_codes(np.arange(n), i * Hkv + h).astype(np.int64)
            cnt, sums = O.visible_code_sums(np.arange(n), off + h, op, codes)
            hs = slice(h * G, (h + 1) * G)
            check_exact(o_h[a:b, hs], lse_h[hs, a:b], cnt, sums, f"varlen seq {i} h={h}")


# ---------------- decode ----------------


def _decode_caches(B, n_max, Hkv, d, lens, seed):
    """K ~ N(0,1) drawn on the device, V = position codes (salt b * Hkv + h);
    both NaN at and after each length."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    k = torch.empty((B, n_max, Hkv, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    for b in range(B):
        k[b].copy_(torch.randn((n_max, Hkv, d), generator=gen, device="cuda"))
        rows = np.stack([W.position_code_rows(n_max, d, b * Hkv + h) for h in range(Hkv)],
                        axis=1)
        v[b].copy_(bits_to_dev(rows))
        k[b, int(lens[b]):] = float("nan")
        v[b, int(lens[b]):] = float("nan")
    return k, v


def _decode_expected(lens, Hkv, n_max, op):
    cnts = np.zeros((len(lens), Hkv), np.int64)
    sums = np.zeros((len(lens), Hkv, NC), np.int64)
    for b, L in enumerate(lens):
        t = int(L) - 1
        for h in range(Hkv):
            keys = O.decode_visible_keys(t, op.kv_head_offset + h, op)
            codes = W.position_codes(keys, b * Hkv + h).astype(np.int64)
            cnts[b, h] = len(keys)
            sums[b, h] = codes.sum(axis=0)
    return cnts, sums


def _check_decode(o, lse, cnts, sums, G, what):
    import torch
    assert bool(torch.isfinite(o).all()), f"{what}: non-finite O"
    assert bool((o[..., NC:] == 0).all()), f"{what}: nonzero output beyond the codes"
    o_h = o[..., :NC].cpu().numpy()
    lse_h = lse.cpu().numpy()
    B, Hkv = cnts.shape
    for b in range(B):
        for h in range(Hkv):
            hs = slice(h * G, (h + 1) * G)
            check_exact(o_h[b:b + 1, hs], lse_h[b, hs][:, None], cnts[b, h:h + 1],
                        sums[b, h][None, :], f"{what} b={b} h={h}")


def _run_decode(p, q, k, v, lens, Hkv, n_max, d, window=False):
    import torch
    B, Hq = q.shape[0], q.shape[1]
    ws = torch.full((C.cowa_decode_workspace_size(p, B, Hq, Hkv, d, n_max),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    sl = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    if window:
        _, total = C.cowa_kv_window_rows(p, Hkv, n_max)
        kw = torch.full((B, total, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        vw = torch.full_like(kw, float("nan"))
        C.cowa_kv_window_fill(p, k, v, sl, kw, vw)
        C.cowa_decode_window(p, q, kw, vw, sl, o, lse, Hkv, n_max, 1.0 / np.sqrt(d), ws)
    else:
        C.cowa_decode(p, q, k, v, sl, o, lse, 1.0 / np.sqrt(d), ws)
    torch.cuda.synchronize()
    return o, lse


_D128 = {}


def _decode128():
    w = W.D128K
    if "x" not in _D128:
        lens = W.decode_lens(w)
        k, v = _decode_caches(w.B, w.n_max, w.H_kv, w.d, lens, 47)
        _D128["x"] = (lens, k, v)
    return _D128["x"]


@pytest.mark.parametrize("variant", ["cowa", "causal", "window"])
def test_exact_decode_128k_workload(lib, variant):
    """All 16 sequences and all 40 query heads of the 128K decode workload
    (the drawn lengths), on the full caches (CoWA and full-causal mode) and
    on the windowed caches filled from them."""
    import torch
    w = W.D128K
    lens, k, v = _decode128()
    mode = 1 if variant == "causal" else 0
    p = C.make_pattern(w.n_ctx, w.sink, w.window, 0, w.h_kv_global, 0, mode)
    op = O.Pattern(w.n_ctx, w.sink, w.window, 0, w.h_kv_global, 0, mode)
    q = torch.zeros((w.B, w.H_q, w.d), dtype=torch.bfloat16, device="cuda")
    print(f"[exact decode] 128K {variant} lens={list(lens)}", flush=True)
    o, lse = _run_decode(p, q, k, v, lens, w.H_kv, w.n_max, w.d, window=variant == "window")
    cnts, sums = _decode_expected(lens, w.H_kv, w.n_max, op)
    _check_decode(o, lse, cnts, sums, w.H_q // w.H_kv, f"decode128k {variant}")


def test_exact_decode_128k_band_edges(lib):
    """Lengths where the sequence start crosses each band edge of the 128K
    pattern (key 0 at the first or last distance of band g), the shortest and
    the longest length."""
    import torch
    w = W.D128K
    L = C.cowa_band_length(C.make_pattern(w.n_ctx, w.sink, w.window, 0, w.h_kv_global, 0, 0))
    lens = [1, 2, w.sink, w.sink + 1, w.window, w.window + 1, w.n_max]
    for g in range(w.h_kv_global):
        e = w.window + g * L
        lens += [e, e + 1, e + L, e + L + 1]
    lens = np.array(sorted(set(min(x, w.n_max) for x in lens)), np.int32)
    B = len(lens)
    k, v = _decode_caches(B, w.n_max, w.H_kv, w.d, lens, 48)
    p = C.make_pattern(w.n_ctx, w.sink, w.window, 0, w.h_kv_global, 0, 0)
    op = O.Pattern(w.n_ctx, w.sink, w.window, 0, w.h_kv_global, 0, 0)
    q = torch.zeros((B, w.H_q, w.d), dtype=torch.bfloat16, device="cuda")
    print(f"[exact decode] band-edge lens={list(lens)}", flush=True)
    o, lse = _run_decode(p, q, k, v, lens, w.H_kv, w.n_max, w.d)
    cnts, sums = _decode_expected(lens, w.H_kv, w.n_max, op)
    _check_decode(o, lse, cnts, sums, w.H_q // w.H_kv, "decode band edges")


@pytest.mark.parametrize("kw", [dict(sink=5, window=37, h=4, off=0, n_max=700),
                                dict(sink=0, window=1, h=4, off=1, n_max=515),
                                dict(sink=16, window=64, h=8, off=6, n_max=1030, n_bands=4)])
def test_exact_decode_every_length(lib, kw):
    """Small patterns, one sequence for every length 1..n_max: every split of
    the visible ranges into chunks, every wrap of the windowed ring."""
    import torch
    n_max, Hkv, d = kw["n_max"], 2, 64
    Hq = 2 * Hkv
    lens = np.arange(1, n_max + 1, dtype=np.int32)
    B = len(lens)
    k, v = _decode_caches(B, n_max, Hkv, d, lens, 49)
    p = C.make_pattern(n_max, kw["sink"], kw["window"], 0, kw["h"], kw["off"], 0,
                       kw.get("n_bands", 0))
    op = O.Pattern(n_max, kw["sink"], kw["window"], 0, kw["h"], kw["off"], 0, kw.get("n_bands", 0))
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    cnts, sums = _decode_expected(lens, Hkv, n_max, op)
    for window in (False, True):
        print(f"[exact decode] every length {kw} window={window}", flush=True)
        o, lse = _run_decode(p, q, k, v, lens, Hkv, n_max, d, window=window)
        _check_decode(o, lse, cnts, sums, Hq // Hkv, f"every length window={window}")
