"""cowa_decode_noalloc (the library's own scratch, for callers that cannot
allocate) against cowa_decode (a caller workspace): the same kernels, so the
outputs must agree bit for bit, on two calls in a row, the second with a
smaller problem than the first (the shared scratch keeps the first call's
partials, which must not leak into the second)."""

import numpy as np
import pytest

import oracle.cowa_oracle as O
from structured_sparse_attention_cowa_amd import binding as C
from structured_sparse_attention_cowa_amd import workloads as W
from tests.gpu_helpers import bits_to_dev, check_close

pytestmark = pytest.mark.gpu


def _both(p, q, k, v, lens, d):
    import torch
    B, Hq = q.shape[0], q.shape[1]
    n_max, Hkv = k.shape[1], k.shape[2]
    sl = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    scale = 1.0 / np.sqrt(d)
    ws = torch.full((C.cowa_decode_workspace_size(p, B, Hq, Hkv, d, n_max),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    o1 = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    l1 = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    C.cowa_decode(p, q, k, v, sl, o1, l1, scale, ws)
    C.cowa_decode_noalloc(p, q, k, v, sl, o2, l2, scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), "O differs"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "LSE differs"
    return o2.cpu().numpy(), l2.cpu().numpy()


def test_noalloc_equals_decode_two_calls(lib):
    # call 1: the 128K decode workload (B=16, H_q=40, H_kv=8, d=128)
    w = W.D128K
    lens = W.decode_lens(w)
    q_bits = W.decode_query(w)
    k, v = W.decode_cache_device(w, lens)
    p = C.make_pattern(w.n_ctx, w.sink, w.window, 0, w.h_kv_global, 0, 0)
    print(f"[noalloc] call 1: 128K decode workload lens={list(lens)}", flush=True)
    o, lse = _both(p, bits_to_dev(q_bits), k, v, lens, w.d)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    del k, v
    # call 2: a smaller problem (fewer sequences, heads and splits, d = 64)
    B, n_max, Hq, Hkv, d, S, Wd, H, off = 3, 1500, 4, 2, 64, 8, 100, 4, 1
    lens2 = np.array([1, 777, 1500], np.int32)
    rng = np.random.Generator(np.random.PCG64(91))
    qb = W.to_bf16_bits(rng.standard_normal((B, Hq, d), dtype=np.float32))
    kb, vb = W.decode_cache_host(92, B, n_max, Hkv, d, lens2)
    p2 = C.make_pattern(n_max, S, Wd, 0, H, off, 0)
    print(f"[noalloc] call 2: B={B} n_max={n_max} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    o2, lse2 = _both(p2, bits_to_dev(qb), bits_to_dev(kb), bits_to_dev(vb), lens2, d)
    op = O.Pattern(n_max, S, Wd, 0, H, off, 0)
    o_ref, lse_ref = O.decode(W.bf16_bits_to_f32(qb), W.bf16_bits_to_f32(kb),
                              W.bf16_bits_to_f32(vb), lens2, op, 1.0 / np.sqrt(d))
    check_close(o2, lse2, o_ref, lse_ref, "noalloc call 2")


def test_noalloc_rejects_oversized_problem(lib):
    """A problem whose partials exceed the scratch is refused before launch."""
    import torch
    w = W.D128K
    p = C.make_pattern(w.n_ctx, w.sink, w.window, 0, w.h_kv_global, 0, 0)
    B = 64
    assert C.cowa_decode_workspace_size(p, B, w.H_q, w.H_kv, w.d, w.n_max) > \
        C.COWA_DECODE_SCRATCH_BYTES
    q = torch.zeros((B, w.H_q, w.d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, 1, w.H_kv, w.d), dtype=torch.bfloat16, device="cuda").expand(
        B, w.n_max, w.H_kv, w.d)  # stride 0 along positions: refused before any read
    sl = torch.ones(B, dtype=torch.int32, device="cuda")
    o = torch.empty((B, w.H_q, w.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, w.H_q), dtype=torch.float32, device="cuda")
    with pytest.raises(C.CowaError) as e:
        C.cowa_decode_noalloc(p, q, k, k, sl, o, lse, 0.1)
    assert e.value.status == C.COWA_ERR_SCRATCH_LIMIT
