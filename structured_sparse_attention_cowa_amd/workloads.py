"""Seeded synthetic workloads for the CoWA operator (shapes, draws, bf16 rounding).

This module holds the workload definitions and the random-input generators
shared by the tests, the smoke check and the benchmark.  It contains none of
the method's arithmetic: no visibility rule, no band derivation, no softmax.
The band width each workload states is recorded as a plain number so that the
tests can check the derivation against it.

Inputs are drawn as float32 from numpy's PCG64 generator and rounded once to
bfloat16 (round to nearest, ties to even).  Both the GPU path and the fp64
oracle consume the rounded values, so parity measures kernel error, not input
quantisation.  The 128K decode cache (two 4 GiB bf16 tensors) is drawn on the
device with torch's seeded generator instead; the oracle then reads the rows
it needs back to the host.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BF16_NAN_BITS = 0x7FC0


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(to_bf16_bits(x))


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    N: int
    H_q: int
    H_kv: int            # KV heads held by this GPU
    d: int
    sink: int
    window: int
    h_kv_global: int
    stated_band: int     # L as the workload definition states it
    seed: int
    offsets: tuple = (0,)  # global KV-head offsets to run
    q_dist: str = "normal"       # "normal" | "rms1.5"
    k_dist: str = "normal"       # "normal" | "peaky5pct"


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    n_max: int
    n_ctx: int
    H_q: int
    H_kv: int
    d: int
    sink: int
    window: int
    h_kv_global: int
    stated_band: int
    seed: int
    len_lo: int
    len_hi: int          # inclusive
    offsets: tuple = (0,)


TINY = PrefillWorkload("tiny-1k", B=1, N=1024, H_q=8, H_kv=4, d=64, sink=16, window=128,
                       h_kv_global=4, stated_band=224, seed=1)
P8K = PrefillWorkload("prefill-8k", B=2, N=8192, H_q=32, H_kv=8, d=128, sink=64, window=1024,
                      h_kv_global=8, stated_band=896, seed=2, k_dist="peaky5pct")
P32K = PrefillWorkload("prefill-32k", B=1, N=32768, H_q=40, H_kv=8, d=128, sink=128,
                       window=4096, h_kv_global=8, stated_band=3584, seed=3, q_dist="rms1.5")
P128K = PrefillWorkload("prefill-128k-rank", B=1, N=131072, H_q=5, H_kv=1, d=128, sink=128,
                        window=8192, h_kv_global=8, stated_band=15360, seed=4,
                        offsets=tuple(range(8)))
D128K = DecodeWorkload("decode-128k", B=16, n_max=131072, n_ctx=131072, H_q=40, H_kv=8, d=128,
                       sink=128, window=8192, h_kv_global=8, stated_band=15360, seed=5,
                       len_lo=98304, len_hi=131072)

PREFILL_WORKLOADS = (TINY, P8K, P32K, P128K)


@dataclass(frozen=True)
class VarlenWorkload:
    """Packed prefill: n_seqs sequences with lengths uniform on [len_lo, len_hi]
    (integers, drawn first), the 32K workload's heads and pattern."""
    name: str
    n_seqs: int
    len_lo: int
    len_hi: int
    n_ctx: int
    H_q: int
    H_kv: int
    d: int
    sink: int
    window: int
    h_kv_global: int
    seed: int

    def lengths(self) -> np.ndarray:
        rng = np.random.Generator(np.random.PCG64(self.seed))
        return rng.integers(self.len_lo, self.len_hi, endpoint=True, size=self.n_seqs)


VARLEN32K = VarlenWorkload("varlen-32k", n_seqs=8, len_lo=4096, len_hi=32768, n_ctx=32768,
                           H_q=40, H_kv=8, d=128, sink=128, window=4096, h_kv_global=8, seed=6)


@dataclass
class PrefillInputs:
    q_bits: np.ndarray   # uint16 [B, N, H_q, d]
    k_bits: np.ndarray   # uint16 [B, N, H_kv, d]
    v_bits: np.ndarray
    extra: dict = field(default_factory=dict)

    def q(self):
        return bf16_bits_to_f32(self.q_bits)

    def k(self):
        return bf16_bits_to_f32(self.k_bits)

    def v(self):
        return bf16_bits_to_f32(self.v_bits)


def prefill_inputs(w: PrefillWorkload, n_override: int | None = None) -> PrefillInputs:
    """Q, K, V for a prefill workload (draw order: Q, K, V, then the K scaling mask).

    q_dist "rms1.5": each query vector is rescaled to root-mean-square 1.5.
    k_dist "peaky5pct": each key vector (b, j, h) is multiplied by 4 with
    probability 0.05 (before rounding; x4 is exact in bf16).
    """
    N = w.N if n_override is None else n_override
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q = rng.standard_normal((w.B, N, w.H_q, w.d), dtype=np.float32)
    k = rng.standard_normal((w.B, N, w.H_kv, w.d), dtype=np.float32)
    v = rng.standard_normal((w.B, N, w.H_kv, w.d), dtype=np.float32)
    if w.q_dist == "rms1.5":
        rms = np.sqrt(np.mean(q.astype(np.float64) ** 2, axis=-1, keepdims=True))
        q = (q / rms * 1.5).astype(np.float32)
    if w.k_dist == "peaky5pct":
        hot = rng.random((w.B, N, w.H_kv), dtype=np.float64) < 0.05
        k = np.where(hot[..., None], k * np.float32(4.0), k).astype(np.float32)
    return PrefillInputs(to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v))


def random_prefill(seed, B, N, H_q, H_kv, d, scale_q=1.0):
    """Generic N(0,1) inputs for edge-case tests (any shape)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, N, H_q, d), dtype=np.float32) * np.float32(scale_q)
    k = rng.standard_normal((B, N, H_kv, d), dtype=np.float32)
    v = rng.standard_normal((B, N, H_kv, d), dtype=np.float32)
    return PrefillInputs(to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v))


def hot_key_prefill(seed, B, N, H_q, H_kv, d, hot):
    """Inputs whose scores jump late in a row: every query gets the common
    direction u = (1, ..., 1) / sqrt(d) added with weight 2, and the keys at
    the positions in `hot` (a dict position -> gain) are replaced by gain * u,
    so their scores are about 2 * gain above the typical N(0, d) score spread.
    Rows see the hot keys only once their tiles come up, after ordinary ones."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = np.full(d, 1.0 / np.sqrt(d), dtype=np.float32)
    q = rng.standard_normal((B, N, H_q, d), dtype=np.float32) + np.float32(2.0) * u
    k = rng.standard_normal((B, N, H_kv, d), dtype=np.float32)
    v = rng.standard_normal((B, N, H_kv, d), dtype=np.float32)
    for j, gain in hot.items():
        k[:, j, :, :] = np.float32(gain) * u
    return PrefillInputs(to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v))


# Position codes: value rows that identify their key position.  With a zero
# query every visible score is equal, so an output row is the mean of the
# value rows of exactly the visible keys; with 0/1 codes (exact in bf16) the
# product of that mean and the visible count is an integer the fp32 sums
# reproduce exactly, which makes the visible set checkable key by key.
POSITION_CODE_BITS = 18      # positions below 2^18
N_POSITION_CODES = 2 * POSITION_CODE_BITS + 1
BF16_ONE_BITS = 0x3F80


def position_codes(j, salt: int = 0) -> np.ndarray:
    """0/1 codes of key positions j: uint8 [len(j), N_POSITION_CODES].

    Columns 0..17: the bits of j.  Columns 18..35: the bits of a
    multiplicative hash of (j, salt) (a different code per head or sequence
    when salt differs).  Column 36: the constant 1."""
    j = np.asarray(j, dtype=np.uint64)
    nb = POSITION_CODE_BITS
    h = ((j + np.uint64(salt) * np.uint64(1 << nb)) * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)
    h = h >> np.uint64(32 - nb)
    out = np.zeros((len(j), N_POSITION_CODES), dtype=np.uint8)
    for c in range(nb):
        out[:, c] = (j >> np.uint64(c)) & np.uint64(1)
        out[:, nb + c] = (h >> np.uint64(c)) & np.uint64(1)
    out[:, 2 * nb] = 1
    return out


def position_code_rows(n: int, d: int, salt: int = 0) -> np.ndarray:
    """Value rows [n, d] as bf16 bits: the position codes of keys 0..n-1 in the
    first N_POSITION_CODES dimensions, zero in the rest."""
    assert d >= N_POSITION_CODES and n <= (1 << POSITION_CODE_BITS)
    out = np.zeros((n, d), dtype=np.uint16)
    out[:, :N_POSITION_CODES] = position_codes(np.arange(n), salt) * np.uint16(BF16_ONE_BITS)
    return out


def zero_query_inputs(seed, B, N, H_q, H_kv, d) -> PrefillInputs:
    """Q = 0, K ~ N(0,1) (seeded), V = position codes, salt b * H_kv + h for
    sequence b and local KV head h."""
    rng = np.random.Generator(np.random.PCG64(seed))
    k = to_bf16_bits(rng.standard_normal((B, N, H_kv, d), dtype=np.float32))
    v = np.zeros((B, N, H_kv, d), dtype=np.uint16)
    for b in range(B):
        for h in range(H_kv):
            v[b, :, h] = position_code_rows(N, d, b * H_kv + h)
    return PrefillInputs(np.zeros((B, N, H_q, d), dtype=np.uint16), k, v)


def grad_output(seed, B, N, H_q, d) -> np.ndarray:
    """Upstream gradient dO for the backward: N(0,1), bf16 bits [B, N, H_q, d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return to_bf16_bits(rng.standard_normal((B, N, H_q, d), dtype=np.float32))


def decode_lens(w: DecodeWorkload) -> np.ndarray:
    """Cached lengths, integers uniform on [len_lo, len_hi] (drawn first)."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    return rng.integers(w.len_lo, w.len_hi, endpoint=True, size=w.B).astype(np.int32)


def decode_query(w: DecodeWorkload) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(w.seed))
    rng.integers(w.len_lo, w.len_hi, endpoint=True, size=w.B)  # same stream position
    return to_bf16_bits(rng.standard_normal((w.B, w.H_q, w.d), dtype=np.float32))


def decode_cache_host(seed, B, n_max, H_kv, d, lens, poison=True):
    """Small decode caches on the host: N(0,1) below each length, NaN at and after it."""
    rng = np.random.Generator(np.random.PCG64(seed))
    k = to_bf16_bits(rng.standard_normal((B, n_max, H_kv, d), dtype=np.float32))
    v = to_bf16_bits(rng.standard_normal((B, n_max, H_kv, d), dtype=np.float32))
    if poison:
        for b in range(B):
            k[b, int(lens[b]):] = BF16_NAN_BITS
            v[b, int(lens[b]):] = BF16_NAN_BITS
    return k, v


def decode_cache_device(w: DecodeWorkload, lens: np.ndarray, device="cuda"):
    """Full-size decode caches drawn on the device (torch seeded generator).

    K and V are [B, n_max, H_kv, d] bf16, N(0,1) below each sequence's
    length and NaN at and after it, so any read past a length shows up as NaN.
    """
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    shape = (w.B, w.n_max, w.H_kv, w.d)
    caches = []
    for _ in range(2):
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        for b in range(w.B):  # per sequence, to bound the fp32 temporary
            t[b].copy_(torch.randn(shape[1:], generator=gen, device=device,
                                   dtype=torch.float32))
            t[b, int(lens[b]):] = float("nan")
        caches.append(t)
    return caches[0], caches[1]


def varlen_device(w: VarlenWorkload, device="cuda"):
    """Packed Q [T, H_q, d], K, V [T, H_kv, d] bf16, N(0,1), drawn on the device
    with torch's generator seeded w.seed (in the order Q, K, V), and
    cu_seqlens int32 [n_seqs + 1] on the device; T = sum of w.lengths()."""
    import torch

    lens = w.lengths()
    T = int(lens.sum())
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    q = torch.randn((T, w.H_q, w.d), generator=gen, device=device).to(torch.bfloat16)
    k = torch.randn((T, w.H_kv, w.d), generator=gen, device=device).to(torch.bfloat16)
    v = torch.randn((T, w.H_kv, w.d), generator=gen, device=device).to(torch.bfloat16)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(device)
    return q, k, v, cu
