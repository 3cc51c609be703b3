"""GPU tests of the windowed KV cache for decode.

cowa_decode_window on caches packed by cowa_kv_window_fill (and grown by
cowa_kv_window_append) must give exactly the bits cowa_decode gives on the
full caches (same kernel, same chunking, only the rows it reads move), and
both must match the fp64 oracle.  Full caches hold NaN past each length, so a
read of a wrong position shows."""

import numpy as np
import pytest

import oracle.cowa_oracle as O
from structured_sparse_attention_cowa_amd import binding as C
from structured_sparse_attention_cowa_amd import workloads as W
from tests.gpu_helpers import bits_to_dev, check_close

pytestmark = pytest.mark.gpu


def _decode_both(p, qd, kc, vc, kw, vw, sl, Hkv, n_max, scale):
    import torch
    B, Hq, d = qd.shape
    ws = torch.zeros(C.cowa_decode_workspace_size(p, B, Hq, Hkv, d, n_max), dtype=torch.uint8,
                     device="cuda")
    o1 = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    l1 = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    o2, l2 = o1.clone(), l1.clone()
    C.cowa_decode(p, qd, kc, vc, sl, o1, l1, scale, ws)
    C.cowa_decode_window(p, qd, kw, vw, sl, o2, l2, Hkv, n_max, scale, ws)
    torch.cuda.synchronize()
    return o1.cpu().numpy(), l1.cpu().numpy(), o2.cpu().numpy(), l2.cpu().numpy()


CASES = [
    dict(kw=dict(sink=16, window=64, h_kv_global=8, kv_head_offset=3), Hkv=2, G=4, d=128),
    dict(kw=dict(sink=0, window=1, h_kv_global=4), Hkv=4, G=1, d=128),
    dict(kw=dict(sink=7, window=100, h_kv_global=4, n_bands=2), Hkv=4, G=2, d=64),
    dict(kw=dict(sink=4, window=60, h_kv_global=4, mode=2), Hkv=2, G=5, d=128),
    dict(kw=dict(sink=128, window=512, h_kv_global=2), Hkv=2, G=8, d=128),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: str(c["kw"]))
def test_window_fill_then_decode(lib, case):
    import torch
    n_max, B = 3000, 5
    Hkv, d = case["Hkv"], case["d"]
    Hq = Hkv * case["G"]
    lens = np.array([1, 17, 700, 2999, 3000], np.int32)
    rng = np.random.Generator(np.random.PCG64(601))
    q_bits = W.to_bf16_bits(rng.standard_normal((B, Hq, d), dtype=np.float32))
    kb, vb = W.decode_cache_host(602, B, n_max, Hkv, d, lens)
    p = C.make_pattern(n_max, **case["kw"])
    rows, total = C.cowa_kv_window_rows(p, Hkv, n_max)
    kc, vc = bits_to_dev(kb), bits_to_dev(vb)
    kw = torch.full((B, total, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vw = torch.full((B, total, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    sl = torch.from_numpy(lens).cuda()
    print(f"[kvwin] {case} rows={list(rows)} of {n_max} per head", flush=True)
    C.cowa_kv_window_fill(p, kc, vc, sl, kw, vw)
    scale = 1.0 / np.sqrt(d)
    o1, l1, o2, l2 = _decode_both(p, bits_to_dev(q_bits), kc, vc, kw, vw, sl, Hkv, n_max, scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    op = O.Pattern(n_max, **case["kw"])
    o_ref, lse_ref = O.decode(W.bf16_bits_to_f32(q_bits), W.bf16_bits_to_f32(kb),
                              W.bf16_bits_to_f32(vb), lens, op, scale)
    check_close(o2, l2, o_ref, lse_ref, f"window decode {case['kw']}")


@pytest.mark.parametrize("case", CASES[:3], ids=lambda c: str(c["kw"]))
def test_window_append_steps(lib, case):
    """Fill at the starting lengths, then append one token per step; every
    step's windowed decode equals the full-cache decode bit for bit."""
    import torch
    n_max, B, steps = 2000, 3, 40
    Hkv, d = case["Hkv"], case["d"]
    Hq = Hkv * case["G"]
    len0 = np.array([3, 500, 1900], np.int32)
    rng = np.random.Generator(np.random.PCG64(603))
    kb, vb = W.decode_cache_host(604, B, n_max, Hkv, d, len0 + steps)
    p = C.make_pattern(n_max, **case["kw"])
    _, total = C.cowa_kv_window_rows(p, Hkv, n_max)
    kc, vc = bits_to_dev(kb), bits_to_dev(vb)
    kw = torch.zeros((B, total, d), dtype=torch.bfloat16, device="cuda")
    vw = torch.zeros((B, total, d), dtype=torch.bfloat16, device="cuda")
    C.cowa_kv_window_fill(p, kc, vc, torch.from_numpy(len0).cuda(), kw, vw)
    scale = 1.0 / np.sqrt(d)
    ar = torch.arange(B, device="cuda")
    print(f"[kvwin append] {case}", flush=True)
    for s in range(steps):
        lens = len0 + s + 1
        sl = torch.from_numpy(lens).cuda()
        pos = torch.from_numpy((lens - 1).astype(np.int64)).cuda()
        C.cowa_kv_window_append(p, kc[ar, pos].contiguous(), vc[ar, pos].contiguous(), sl, kw,
                                vw, n_max)
        q_bits = W.to_bf16_bits(rng.standard_normal((B, Hq, d), dtype=np.float32))
        o1, l1, o2, l2 = _decode_both(p, bits_to_dev(q_bits), kc, vc, kw, vw, sl, Hkv, n_max,
                                      scale)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), f"step {s}"
    op = O.Pattern(n_max, **case["kw"])
    o_ref, lse_ref = O.decode(W.bf16_bits_to_f32(q_bits), W.bf16_bits_to_f32(kb),
                              W.bf16_bits_to_f32(vb), lens, op, scale)
    check_close(o2, l2, o_ref, lse_ref, f"window append {case['kw']}")


def test_window_decode_128k_workload(lib):
    """The 128K decode workload on windowed caches: the same bits as the full
    caches at about 0.59 of their memory."""
    import torch
    w = W.D128K
    lens = W.decode_lens(w)
    q_bits = W.decode_query(w)
    kc, vc = W.decode_cache_device(w, lens)
    p = C.make_pattern(w.n_ctx, w.sink, w.window, 0, w.h_kv_global, 0, 0)
    rows, total = C.cowa_kv_window_rows(p, w.H_kv, w.n_max)
    assert total / (w.H_kv * w.n_max) < 0.6
    kw = torch.empty((w.B, total, w.d), dtype=torch.bfloat16, device="cuda")
    vw = torch.empty((w.B, total, w.d), dtype=torch.bfloat16, device="cuda")
    sl = torch.from_numpy(lens).cuda()
    C.cowa_kv_window_fill(p, kc, vc, sl, kw, vw)
    o1, l1, o2, l2 = _decode_both(p, bits_to_dev(q_bits), kc, vc, kw, vw, sl, w.H_kv, w.n_max,
                                  1.0 / np.sqrt(w.d))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.isfinite(o2).all()
