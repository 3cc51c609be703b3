"""The entry points take any element strides with a contiguous head dimension:
prefill, backward and decode on head-major storage ([B, H, N, d] viewed as
[B, N, H, d]) give the same bits as on the contiguous layout."""

import numpy as np
import pytest

from structured_sparse_attention_cowa_amd import binding as C
from structured_sparse_attention_cowa_amd import workloads as W
from tests.gpu_helpers import bits_to_dev

pytestmark = pytest.mark.gpu


def _head_major(t):
    """The same values in [B, H, N, d] storage, viewed as [B, N, H, d]."""
    return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


def _empty_head_major(shape, dtype):
    import torch
    B, N, H, d = shape
    return torch.full((B, H, N, d), float("nan"), dtype=dtype, device="cuda").permute(0, 2, 1, 3)


def test_prefill_and_backward_on_head_major_storage(lib):
    import torch
    B, N, Hq, Hkv, d = 2, 700, 8, 2, 128
    x = W.random_prefill(901, B, N, Hq, Hkv, d)
    q, k, v = bits_to_dev(x.q_bits), bits_to_dev(x.k_bits), bits_to_dev(x.v_bits)
    do = bits_to_dev(W.grad_output(902, B, N, Hq, d))
    p = C.make_pattern(N, 16, 128, 0, 4, 1)
    bm, bn = C.cowa_fwd_block_sizes(d)
    bmk, bnk = C.cowa_bwd_block_sizes(d)
    rp, col, fl = [torch.from_numpy(a).cuda() for a in C.cowa_plan(p, N, Hkv, bm, bn)]
    rpk, colk, flk = [torch.from_numpy(a).cuda() for a in C.cowa_plan_kv(p, N, Hkv, bmk, bnk)]
    ws = torch.empty(C.cowa_bwd_workspace_size(p, B, Hq, Hkv, N), dtype=torch.uint8, device="cuda")
    scale = 1.0 / np.sqrt(d)

    def run(q, k, v, do, alloc):
        o = alloc((B, N, Hq, d), torch.float32)
        lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device="cuda")
        dq = alloc((B, N, Hq, d), torch.float32)
        dk = alloc((B, N, Hkv, d), torch.float32)
        dv = alloc((B, N, Hkv, d), torch.float32)
        C.cowa_fwd(p, rp, col, fl, col.numel(), bm, bn, q, k, v, o, lse, scale)
        C.cowa_bwd(p, rp, col, fl, col.numel(), bm, bn, rpk, colk, flk, colk.numel(), bmk, bnk,
                   q, k, v, o, do, lse, dq, dk, dv, scale, ws)
        torch.cuda.synchronize()
        return [t.contiguous().cpu().numpy() for t in (o, lse, dq, dk, dv)]

    def contiguous(shape, dtype):
        return torch.full(shape, float("nan"), dtype=dtype, device="cuda")

    print("[layouts] prefill + backward, contiguous vs head-major", flush=True)
    ref = run(q, k, v, do, contiguous)
    qh, kh, vh, doh = (_head_major(t) for t in (q, k, v, do))
    assert not qh.is_contiguous() and qh.stride(2) == N * d
    got = run(qh, kh, vh, doh, _empty_head_major)
    for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), ref, got):
        assert np.isfinite(a).all(), name
        assert np.array_equal(a, b), f"{name} differs on head-major storage"


def test_decode_on_head_major_cache(lib):
    import torch
    B, Hq, Hkv, d, n_max = 3, 8, 2, 128, 3000
    lens = np.array([3000, 1, 1777], np.int32)
    x = W.random_prefill(903, B, n_max, Hkv, Hkv, d)  # cache values, [B, n_max, Hkv, d]
    kc, vc = bits_to_dev(x.k_bits), bits_to_dev(x.v_bits)
    q = bits_to_dev(W.random_prefill(904, B, 1, Hq, Hkv, d).q_bits[:, 0])
    p = C.make_pattern(4096, 16, 256, 0, 4, 2)
    ws = torch.empty(C.cowa_decode_workspace_size(p, B, Hq, Hkv, d, n_max), dtype=torch.uint8,
                     device="cuda")
    sl = torch.from_numpy(lens).cuda()

    def run(k, v):
        o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        C.cowa_decode(p, q, k, v, sl, o, lse, 1.0 / np.sqrt(d), ws)
        torch.cuda.synchronize()
        return o.cpu().numpy(), lse.cpu().numpy()

    print("[layouts] decode, contiguous vs head-major cache", flush=True)
    o1, l1 = run(kc, vc)
    o2, l2 = run(_head_major(kc), _head_major(vc))
    assert np.isfinite(o1).all() and np.isfinite(l1).all()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
