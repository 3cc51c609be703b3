"""Plain fp64 CPU oracle for CoWindow Attention (CoWA).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module.  The GPU library
never calls it and shares no code with it: this file has its own visibility
predicate, its own interval and tile enumeration, and a dense masked softmax.

Sources (pages are cited by title and paragraph; they carry no numbered
sections, equations or listings):

  [SF] "Splitting long-range windows across KV heads beats duplicating them at
       lower cost" (skillfed.io news, 2026-09-30).  Second paragraph: all KV
       heads share a near-diagonal window and a prefix-sink window; the rest
       of the causal history is cut into non-overlapping long-range intervals,
       one per KV head; the pattern is position arithmetic only.  Paragraph
       "What CoWA does not claim": every head applies softmax over its own
       visible set.  Sixth paragraph: global KV-head indexing keeps the bands
       complementary across tensor-parallel ranks.
  [AB] "CoWindow Attention: Full Causal Coverage Is a Collective Property",
       Abstract (newx.sg paper page; same text on the acceptodds.com ICLR 2027
       submission page): complementary long-range windows partition the
       remaining history and, with the shared windows, their union gives full
       causal coverage; FullAttn is the dense comparison.

Readings where the pages give no formula:

  * Band partition.  The pages state the structure but no formula.  This
    oracle fixes: with L = ceil((N_ctx - W) / H_kv_global) when N_ctx > W and
    L = 0 otherwise, KV head with global index g sees keys at query-to-key
    distance t - j in the half-open interval [W + g*L, W + (g+1)*L).
  * Shared windows: the sink is keys j < S, the local window is distances
    t - j < W (so W keys including the diagonal).  Both are intersected with
    causality j <= t.
  * A key reachable through several windows counts once (set union).
  * GQA: query head hq uses local KV head h = hq // G with G = H_q / H_kv_local;
    its global index is g = kv_head_offset + h.
  * Decode: the new token's K/V are already in the cache, so the query
    position is t = len - 1.
  * LSE is the natural-log log-sum-exp of the scaled scores over the visible
    set.

Parity status: the visibility predicate, interval form, tile lists and the
masked softmax are pinned by the CPU tests (hand-derived 16-token grid,
coverage/disjointness invariants, closed-form pair counts, reductions to
textbook dense causal softmax, closed-form band-only case, softmax identities
checked against scipy).  The backward (attention_backward and its row- and
key-sampled forms) is pinned by float64 autograd where CoWA reduces to dense
causal attention, central finite differences of the forward, GQA sums of
single-head problems and invariance to a common shift of the value rows.
The error-bound helpers: the D-sensitivity (_d_sensitivity, eq, ek) by its
closed form when every row's softmax is uniform and by shifting D in the
backward (the bound holds, and is attained when q, k have one sign); the KV
retention mask (brute force over all later queries) by its closed form.
visible_code_sums (zero-query attention as integer sums) by the dense
predicate and the merged interval form.  Numeric O/LSE
values for the benchmark workloads are not printed by the pages; for those
the definition below plus the reductions above are the pins.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

MODE_COWA = 0
MODE_CAUSAL = 1
MODE_SINK_LOCAL = 2


@dataclass(frozen=True)
class Pattern:
    """Position-only pattern parameters ([SF] second paragraph; [AB] Abstract).

    n_ctx: context length the band width is derived from.
    sink: S, keys j < S are shared by every head.
    window: W, distances t - j < W are shared by every head.
    band: L; a value <= 0 means "derive from n_ctx, window, h_kv_global".
    h_kv_global: number of KV heads across all tensor-parallel ranks.
    kv_head_offset: global index of this rank's first KV head ([SF] sixth
        paragraph: bands follow the global KV-head index).
    mode: MODE_COWA, MODE_CAUSAL (dense causal FullAttn, [AB] Abstract) or
        MODE_SINK_LOCAL (sink and local windows only: sliding-window attention
        with sinks, the band-less pattern of the [BH] page).
    n_bands: number of distinct long-range windows shared out over the
        h_kv_global heads ([SF] ablation paragraph: 1, 2, 4 or 8 distinct
        windows over 8 KV heads at fixed per-head width).  0 means
        h_kv_global (CoWA proper).  Head g takes window g mod n_bands, of
        width L as above (the page does not say which head takes which).
    """

    n_ctx: int
    sink: int
    window: int
    band: int = 0
    h_kv_global: int = 1
    kv_head_offset: int = 0
    mode: int = MODE_COWA
    n_bands: int = 0


def band_length(n_ctx: int, window: int, h_kv_global: int) -> int:
    """L = ceil((N_ctx - W) / H_kv_global) if N_ctx > W else 0 (band reading)."""
    if n_ctx <= window:
        return 0
    rest = n_ctx - window
    # integer ceiling division, written out
    q, r = divmod(rest, h_kv_global)
    return q + (1 if r else 0)


def resolved_band(p: Pattern) -> int:
    """Band width L; 0 (no band) in MODE_SINK_LOCAL."""
    if p.mode == MODE_SINK_LOCAL:
        return 0
    return p.band if p.band > 0 else band_length(p.n_ctx, p.window, p.h_kv_global)


def band_index(g: int, p: Pattern) -> int:
    """Which long-range window global KV head g takes: g itself for CoWA,
    g mod n_bands for the duplicated-window ablation."""
    m = p.n_bands if p.n_bands > 0 else p.h_kv_global
    return g % m


def visible(t, j, g, p: Pattern):
    """Element predicate vis_g(t, j) (broadcasting over numpy arrays).

    CoWA: j <= t and (j < S or t - j < W or W + g*L <= t - j < W + (g+1)*L).
    Causal mode: j <= t.
    """
    t = np.asarray(t, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    dist = t - j
    causal = (dist >= 0) & (j >= 0)
    if p.mode == MODE_CAUSAL:
        return causal
    L = resolved_band(p)
    in_sink = j < p.sink
    in_local = dist < p.window
    if L > 0:
        bi = band_index(g, p)
        lo = p.window + bi * L
        hi = p.window + (bi + 1) * L
        in_band = (dist >= lo) & (dist < hi)
    else:
        in_band = np.zeros(np.broadcast(t, j).shape, dtype=bool)
    return causal & (in_sink | in_local | in_band)


def visible_mask(n_rows: int, n_keys: int, g: int, p: Pattern) -> np.ndarray:
    """Dense boolean [n_rows, n_keys] mask for small sizes."""
    t = np.arange(n_rows)[:, None]
    j = np.arange(n_keys)[None, :]
    return np.broadcast_to(visible(t, j, g, p), (n_rows, n_keys)).copy()


def visible_intervals(t: int, g: int, p: Pattern):
    """Row t's visible keys as sorted, disjoint, non-adjacent [a, b) intervals.

    A second, independent derivation of the same set: each window is turned
    into a key interval and the intervals are merged.
    """
    if t < 0:
        return []
    ivs = []
    if p.mode == MODE_CAUSAL:
        ivs.append((0, t + 1))
    else:
        L = resolved_band(p)
        if p.sink > 0:
            ivs.append((0, min(p.sink, t + 1)))
        ivs.append((max(0, t - p.window + 1), t + 1))
        if L > 0:
            # distances [W+bL, W+(b+1)L)  <=>  keys (t-W-(b+1)L, t-W-bL], b the
            # head's window index
            bi = band_index(g, p)
            a = t - (p.window + (bi + 1) * L) + 1
            b = t - (p.window + bi * L) + 1
            a, b = max(a, 0), min(b, t + 1)
            if a < b:
                ivs.append((a, b))
    ivs = sorted(iv for iv in ivs if iv[0] < iv[1])
    merged = []
    for a, b in ivs:
        if merged and a <= merged[-1][1]:
            merged[-1] = (merged[-1][0], max(merged[-1][1], b))
        else:
            merged.append((a, b))
    return merged


def visible_count(t: int, g: int, p: Pattern) -> int:
    return sum(b - a for a, b in visible_intervals(t, g, p))


# --------------------------------------------------------------------------
# Tile lists (the plan).  Tile (qi, kj) covers rows [qi*BM, (qi+1)*BM) and keys
# [kj*BN, (kj+1)*BN).  Listed iff any element is visible, full iff all BM*BN
# elements are visible (a tile reaching past N is therefore never full).
# Rows of the CSR are ordered (h_local, qi); columns ascend.
# --------------------------------------------------------------------------


def _csr_from_counts(counts_per_head, bm, bn):
    row_ptr = [0]
    cols = []
    flags = []
    for counts in counts_per_head:
        for qi in range(counts.shape[0]):
            nz = np.nonzero(counts[qi])[0]
            cols.extend(int(c) for c in nz)
            flags.extend(1 if counts[qi, c] == bm * bn else 0 for c in nz)
            row_ptr.append(len(cols))
    return (np.asarray(row_ptr, dtype=np.int32), np.asarray(cols, dtype=np.int32),
            np.asarray(flags, dtype=np.uint8))


def tile_counts_bruteforce(n: int, g: int, p: Pattern, bm: int, bn: int) -> np.ndarray:
    """Visible-element count per tile by materialising the element mask."""
    nqt = -(-n // bm)
    nkt = -(-n // bn)
    m = np.zeros((nqt * bm, nkt * bn), dtype=bool)
    m[:n, :n] = visible_mask(n, n, g, p)
    return m.reshape(nqt, bm, nkt, bn).sum(axis=(1, 3)).astype(np.int64)


def tile_counts_intervals(n: int, g: int, p: Pattern, bm: int, bn: int) -> np.ndarray:
    """Visible-element count per tile from per-row intervals (large N).

    For each query tile, a difference array over key positions counts how many
    of its rows see each key; summing that over a key tile's BN positions
    gives the tile's visible-element count.
    """
    nqt = -(-n // bm)
    nkt = -(-n // bn)
    counts = np.zeros((nqt, nkt), dtype=np.int64)
    for qi in range(nqt):
        diff = np.zeros(nkt * bn + 1, dtype=np.int64)
        for t in range(qi * bm, min((qi + 1) * bm, n)):
            for a, b in visible_intervals(t, g, p):
                diff[a] += 1
                diff[b] -= 1
        per_key = np.cumsum(diff[:-1])
        counts[qi] = per_key.reshape(nkt, bn).sum(axis=1)
    return counts


def row_windows(t, g: int, p: Pattern):
    """Visible keys of query positions t (int array) as disjoint [a, b) key
    intervals, one array pair per window: sink, then band minus sink, then
    local window minus the other two (a >= b: empty).  The same windows as
    visible_intervals, written per window instead of merged, so that plain
    interval sums count each key once.  Causal mode: one interval [0, t+1)."""
    t = np.asarray(t, dtype=np.int64)
    if p.mode == MODE_CAUSAL:
        return [(np.zeros_like(t), t + 1)]
    L = resolved_band(p)
    sink_b = np.minimum(p.sink, t + 1)
    sink = (np.zeros_like(t), sink_b)
    loc_a = np.maximum(np.maximum(0, t - p.window + 1), sink_b)
    loc = (loc_a, np.maximum(t + 1, loc_a))
    ivs = [sink, loc]
    if L > 0:
        bi = band_index(g, p)
        ba = np.maximum(t - (p.window + (bi + 1) * L) + 1, sink_b)
        bb = np.minimum(t - (p.window + bi * L) + 1, loc_a)
        bb = np.maximum(bb, ba)
        ivs.append((ba, bb))
    return ivs


def tile_counts_intervals_fast(n: int, g: int, p: Pattern, bm: int, bn: int) -> np.ndarray:
    """Same as tile_counts_intervals, vectorised over rows (for 32K-128K).

    Each window of row t is an interval [a_t, b_t) (row_windows, made
    disjoint) so that plain +1/-1 difference marks count each key once.
    """
    nqt = -(-n // bm)
    nkt = -(-n // bn)
    ivs = row_windows(np.arange(n, dtype=np.int64), g, p)
    counts = np.zeros((nqt, nkt), dtype=np.int64)
    for qi in range(nqt):
        r0, r1 = qi * bm, min((qi + 1) * bm, n)
        diff = np.zeros(nkt * bn + 1, dtype=np.int64)
        for a, b in ivs:
            aa, bb = a[r0:r1], b[r0:r1]
            keep = aa < bb
            np.add.at(diff, aa[keep], 1)
            np.add.at(diff, bb[keep], -1)
        per_key = np.cumsum(diff[:-1])
        counts[qi] = per_key.reshape(nkt, bn).sum(axis=1)
    return counts


def visible_code_sums(rows, g: int, p: Pattern, codes: np.ndarray):
    """Per query position t in rows: the number of keys head g sees and the
    sum of codes[j] over those keys (codes: integer array [n_keys, c], keys
    0..n_keys-1, n_keys > max(rows)).

    This is the exact outcome of attention with a zero query: every visible
    score is 0, so the softmax is uniform over the visible set ([SF] paragraph
    on what CoWA does not claim: each head's softmax runs over its own visible
    set), LSE = ln(count) and O * count = sum of the visible value rows.
    Computed from row_windows with prefix sums over keys.
    Returns counts int64 [R] and sums int64 [R, c]."""
    rows = np.asarray(rows, dtype=np.int64)
    codes = np.asarray(codes)
    prefix = np.zeros((codes.shape[0] + 1, codes.shape[1]), dtype=np.int64)
    np.cumsum(codes, axis=0, out=prefix[1:])
    counts = np.zeros(len(rows), dtype=np.int64)
    sums = np.zeros((len(rows), codes.shape[1]), dtype=np.int64)
    for a, b in row_windows(rows, g, p):
        b = np.maximum(a, b)
        counts += b - a
        sums += prefix[b] - prefix[a]
    return counts, sums


def tile_lists(n: int, h_kv_local: int, p: Pattern, bm: int, bn: int, method: str = "auto"):
    """CSR visible-tile lists for local heads 0..h_kv_local-1 (global g = offset + h)."""
    if method == "auto":
        method = "bruteforce" if n <= 4096 else "fast"
    fn = {"bruteforce": tile_counts_bruteforce, "intervals": tile_counts_intervals,
          "fast": tile_counts_intervals_fast}[method]
    per_head = [fn(n, p.kv_head_offset + h, p, bm, bn) for h in range(h_kv_local)]
    return _csr_from_counts(per_head, bm, bn)


def tile_lists_kv(n: int, h_kv_local: int, p: Pattern, bm: int, bn: int, method: str = "auto"):
    """Key-major visible-tile lists (for the backward pass over key tiles).

    Rows of the CSR are ordered (h_local, kj); columns are the query tiles qi,
    ascending; flags as in tile_lists (1 when all BM*BN elements are visible).
    """
    if method == "auto":
        method = "bruteforce" if n <= 4096 else "fast"
    fn = {"bruteforce": tile_counts_bruteforce, "intervals": tile_counts_intervals,
          "fast": tile_counts_intervals_fast}[method]
    per_head = [fn(n, p.kv_head_offset + h, p, bm, bn).T for h in range(h_kv_local)]
    return _csr_from_counts(per_head, bm, bn)


# --------------------------------------------------------------------------
# Attention: dense masked softmax over each head's own visible set
# ([SF] "What CoWA does not claim"), in float64.
# --------------------------------------------------------------------------


def _masked_softmax_rows(qrows, keys, vals, rows_t, g, p: Pattern, scale):
    """qrows [R, d], keys/vals [J, d] (keys 0..J-1), rows_t [R] positions.

    Returns O [R, d] and LSE [R] (natural log).
    """
    s = (qrows @ keys.T) * scale
    mask = visible(rows_t[:, None], np.arange(keys.shape[0])[None, :], g, p)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    lsum = e.sum(axis=1)
    lse = m + np.log(lsum)
    w = np.exp(s - lse[:, None])
    return w @ vals, lse


def attention(q, k, v, p: Pattern, scale: float, rows=None, heads=None, row_block: int = 256):
    """CoWA (or causal) prefill attention, fp64.

    q [B, N, H_q, d]; k, v [B, N, H_kv_local, d] (any float dtype, widened to
    float64).  rows: optional sorted array of query positions to compute (all
    if None).  heads: optional list of query heads (all if None).
    Returns O [B, len(rows), len(heads), d] and LSE [B, len(heads), len(rows)].
    """
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    out = np.zeros((B, len(rows), len(heads), d), dtype=np.float64)
    lse = np.zeros((B, len(heads), len(rows)), dtype=np.float64)
    for b in range(B):
        for hi, hq in enumerate(heads):
            h = hq // G
            g = p.kv_head_offset + h
            for r0 in range(0, len(rows), row_block):
                rt = rows[r0:r0 + row_block]
                J = int(rt.max()) + 1
                qr = np.asarray(q[b, rt, hq], dtype=np.float64)
                kk = np.asarray(k[b, :J, h], dtype=np.float64)
                vv = np.asarray(v[b, :J, h], dtype=np.float64)
                o, l_ = _masked_softmax_rows(qr, kk, vv, rt, g, p, scale)
                out[b, r0:r0 + len(rt), hi] = o
                lse[b, hi, r0:r0 + len(rt)] = l_
    return out, lse


def decode(q, k_cache, v_cache, lens, p: Pattern, scale: float):
    """Single-token decode, fp64: query position t_b = lens[b] - 1, keys 0..t_b.

    q [B, H_q, d]; caches [B, N_max, H_kv_local, d]; lens [B].
    Returns O [B, H_q, d] and LSE [B, H_q].
    """
    B, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    for b in range(B):
        t = int(lens[b]) - 1
        rt = np.asarray([t], dtype=np.int64)
        for hq in range(Hq):
            h = hq // G
            g = p.kv_head_offset + h
            kk = np.asarray(k_cache[b, :t + 1, h], dtype=np.float64)
            vv = np.asarray(v_cache[b, :t + 1, h], dtype=np.float64)
            o, l_ = _masked_softmax_rows(np.asarray(q[b, hq][None, :], dtype=np.float64),
                                         kk, vv, rt, g, p, scale)
            out[b, hq] = o[0]
            lse[b, hq] = l_[0]
    return out, lse


def decode_visible_keys(t: int, g: int, p: Pattern) -> np.ndarray:
    """Sorted key positions visible to a decode query at position t."""
    parts = [np.arange(a, b) for a, b in visible_intervals(t, g, p)]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def retained_mask(n_max: int, g: int, p: Pattern) -> np.ndarray:
    """R[t, j] = key j <= t is visible to some query t' with t <= t' < n_max.

    What a decode cache must still hold for head g after the token at
    position t has been appended ([NX] Abstract: lower decode memory; the
    pattern is fixed by positions, so later queries are known in advance).
    Brute force over the dense mask: a suffix OR over query rows.
    """
    m = visible_mask(n_max, n_max, g, p)
    later = np.logical_or.accumulate(m[::-1], axis=0)[::-1]
    return later & (np.arange(n_max)[None, :] <= np.arange(n_max)[:, None])


def visible_pairs(n: int, g: int, p: Pattern) -> int:
    """Sum over rows t < n of |vis_g(t)| (element-level work of one head)."""
    return int(sum(visible_count(t, g, p) for t in range(n)))


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


# --------------------------------------------------------------------------
# Backward pass (the pages' training operator, [AB] Abstract: forward and
# backward latency at 128K).  Gradients of sum(O * dO), i.e. the
# vector-Jacobian product of the per-head masked softmax attention.
#   P_tj  = exp(scale * s_tj - LSE_t) on the visible set, 0 elsewhere
#   dV_j  = sum_t P_tj dO_t            (summed over the query heads of the group)
#   dP_tj = dO_t . v_j
#   D_t   = sum_c dO_tc O_tc           (= sum_j P_tj dP_tj)
#   dS_tj = P_tj (dP_tj - D_t)
#   dQ_t  = scale sum_j dS_tj k_j
#   dK_j  = scale sum_t dS_tj q_t      (summed over the query heads of the group)
# --------------------------------------------------------------------------


def attention_backward(q, k, v, do, p: Pattern, scale: float, magnitudes: bool = False,
                       d_shift=None):
    """Full backward in float64 for moderate sizes (dense per head).

    d_shift: optional [B, N, H_q] array added to D_t before dS is formed (an
    error in D, to measure how the gradients respond to one; None: exact).

    With magnitudes=True it also returns, for each gradient, the sum of the
    absolute values of the terms it is the sum of (scale sum_j |dS_tj| |k_j|,
    scale sum_t |dS_tj| |q_t|, sum_t P_tj |dO_t|): the scale against which a
    rounding error of each term is measured; and the sensitivities of dQ and
    dK to an error in D_t of relative size 1 in every term of D's inputs:
      w_t  = sum_c |dO_tc| (sum_j P_tj |v_jc| + |O_tc|)
      eq_t = scale w_t sum_j P_tj |k_j|,  ek_j = scale sum_t P_tj w_t |q_t|.
    (An O computed with relative errors u in P and stored with relative error
    u moves D_t by at most u w_t.)  Returns dq, dk, dv, mq, mk, mv, eq, ek."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    mq, mk, mv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    eq, ek = np.zeros_like(q), np.zeros_like(k)
    t = np.arange(N)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            g = p.kv_head_offset + h
            mask = visible(t[:, None], t[None, :], g, p)
            s = (q[b, :, hq] @ k[b, :, h].T) * scale
            s = np.where(mask, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            lse = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
            P = np.exp(s - lse)
            o = P @ v[b, :, h]
            dP = do[b, :, hq] @ v[b, :, h].T
            D = (do[b, :, hq] * o).sum(axis=1, keepdims=True)
            if d_shift is not None:
                D = D + np.asarray(d_shift, np.float64)[b, :, hq][:, None]
            dS = P * (dP - D)
            dq[b, :, hq] = scale * dS @ k[b, :, h]
            dk[b, :, h] += scale * dS.T @ q[b, :, hq]
            dv[b, :, h] += P.T @ do[b, :, hq]
            if magnitudes:
                aS = np.abs(dS)
                mq[b, :, hq] = scale * aS @ np.abs(k[b, :, h])
                mk[b, :, h] += scale * aS.T @ np.abs(q[b, :, hq])
                mv[b, :, h] += P.T @ np.abs(do[b, :, hq])
                w = _d_sensitivity(P, v[b, :, h], o, do[b, :, hq])
                eq[b, :, hq] = scale * w[:, None] * (P @ np.abs(k[b, :, h]))
                ek[b, :, h] += scale * P.T @ (w[:, None] * np.abs(q[b, :, hq]))
    if magnitudes:
        return dq, dk, dv, mq, mk, mv, eq, ek
    return dq, dk, dv


def _d_sensitivity(P, v, o, do):
    """w_t = sum_c |dO_tc| (sum_j P_tj |v_jc| + |O_tc|) for the rows of P."""
    return (np.abs(do) * (P @ np.abs(v) + np.abs(o))).sum(axis=1)


def backward_rows_dq(q, k, v, do, p: Pattern, scale: float, rows, heads=None,
                     magnitudes: bool = False):
    """dQ for selected query rows only (each row needs only its own softmax);
    magnitudes=True also returns mq and eq (as in attention_backward) for
    those rows."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    rows = np.asarray(rows, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    out = np.zeros((B, len(rows), len(heads), d))
    mag = np.zeros_like(out)
    esens = np.zeros_like(out)
    for b in range(B):
        for hi, hq in enumerate(heads):
            h = hq // G
            g = p.kv_head_offset + h
            J = int(rows.max()) + 1
            kk = np.asarray(k[b, :J, h], np.float64)
            vv = np.asarray(v[b, :J, h], np.float64)
            qq = np.asarray(q[b, rows, hq], np.float64)
            dd = np.asarray(do[b, rows, hq], np.float64)
            mask = visible(rows[:, None], np.arange(J)[None, :], g, p)
            s = np.where(mask, (qq @ kk.T) * scale, -np.inf)
            m = s.max(axis=1, keepdims=True)
            lse = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
            P = np.exp(s - lse)
            o = P @ vv
            dP = dd @ vv.T
            D = (dd * o).sum(axis=1, keepdims=True)
            out[b, :, hi] = scale * (P * (dP - D)) @ kk
            if magnitudes:
                mag[b, :, hi] = scale * np.abs(P * (dP - D)) @ np.abs(kk)
                w = _d_sensitivity(P, vv, o, dd)
                esens[b, :, hi] = scale * w[:, None] * (P @ np.abs(kk))
    if magnitudes:
        return out, mag, esens
    return out


def backward_keys_dkdv(q, k, v, do, p: Pattern, scale: float, keys, heads_kv=None,
                       magnitudes: bool = False):
    """dK, dV for selected key positions: sums over every row that sees them
    (practical for keys near the end of the sequence or at small N);
    magnitudes=True also returns mk, mv and ek (as in attention_backward)."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    keys = np.asarray(keys, dtype=np.int64)
    heads_kv = list(range(Hkv)) if heads_kv is None else list(heads_kv)
    dk = np.zeros((B, len(keys), len(heads_kv), d))
    dv = np.zeros((B, len(keys), len(heads_kv), d))
    mk, mv, ek = np.zeros_like(dk), np.zeros_like(dv), np.zeros_like(dk)
    for b in range(B):
        for hi, h in enumerate(heads_kv):
            g = p.kv_head_offset + h
            # rows that can see any selected key
            rows = np.arange(int(keys.min()), N)
            vis_any = visible(rows[:, None], keys[None, :], g, p).any(axis=1)
            rows = rows[vis_any]
            if len(rows) == 0:
                continue
            J = int(rows.max()) + 1
            kk = np.asarray(k[b, :J, h], np.float64)
            vv = np.asarray(v[b, :J, h], np.float64)
            for hq in range(h * G, (h + 1) * G):
                for r0 in range(0, len(rows), 256):
                    rt = rows[r0:r0 + 256]
                    qq = np.asarray(q[b, rt, hq], np.float64)
                    dd = np.asarray(do[b, rt, hq], np.float64)
                    mask = visible(rt[:, None], np.arange(J)[None, :], g, p)
                    s = np.where(mask, (qq @ kk.T) * scale, -np.inf)
                    m = s.max(axis=1, keepdims=True)
                    lse = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
                    P = np.exp(s - lse)
                    o = P @ vv
                    D = (dd * o).sum(axis=1, keepdims=True)
                    Pk = P[:, keys]
                    dPk = dd @ vv[keys].T
                    dSk = Pk * (dPk - D)
                    dk[b, :, hi] += scale * dSk.T @ qq
                    dv[b, :, hi] += Pk.T @ dd
                    if magnitudes:
                        mk[b, :, hi] += scale * np.abs(dSk).T @ np.abs(qq)
                        mv[b, :, hi] += Pk.T @ np.abs(dd)
                        w = _d_sensitivity(P, vv, o, dd)
                        ek[b, :, hi] += scale * Pk.T @ (w[:, None] * np.abs(qq))
    if magnitudes:
        return dk, dv, mk, mv, ek
    return dk, dv
