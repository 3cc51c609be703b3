"""The entry points allocate nothing, synchronise nothing and issue no memory
fills, so a caller can capture them in a HIP graph (a serving loop's decode
step, a training step's attention).  A captured prefill + decode + backward is
replayed several times with eager work and synchronisations in between; every
replay must reproduce the eager results bit for bit."""

import numpy as np
import pytest

from structured_sparse_attention_cowa_amd import binding as C
from structured_sparse_attention_cowa_amd import workloads as W
from tests.gpu_helpers import Backward, bits_to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(lib):
    import torch
    # prefill + backward on a ragged small problem, decode on a small cache
    x = W.random_prefill(501, 1, 700, 8, 2, 128)
    bw = Backward(x, 16, 64, 4, offset=1, n_ctx=700)
    B, Hq, Hkv, d, n_max = 3, 8, 2, 128, 3000
    rng = np.random.Generator(np.random.PCG64(502))
    lens = np.array([1, 1777, 3000], np.int32)
    q_bits = W.to_bf16_bits(rng.standard_normal((B, Hq, d), dtype=np.float32))
    kb, vb = W.decode_cache_host(503, B, n_max, Hkv, d, lens)
    pd = C.make_pattern(n_max, 16, 64, 0, 4, 1, 0)
    ws = torch.empty(C.cowa_decode_workspace_size(pd, B, Hq, Hkv, d, n_max), dtype=torch.uint8,
                     device="cuda")
    qd, kc, vc = bits_to_dev(q_bits), bits_to_dev(kb), bits_to_dev(vb)
    sl = torch.from_numpy(lens).cuda()
    od = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lsed = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

    def work():
        bw.run()  # forward (O, LSE) then backward (dQ, dK, dV)
        C.cowa_decode(pd, qd, kc, vc, sl, od, lsed, 1.0 / np.sqrt(d), ws)

    outs = lambda: [t.clone() for t in (bw.pf.o, bw.pf.lse, bw.dq, bw.dk, bw.dv, od, lsed)]
    work()
    torch.cuda.synchronize()
    ref = outs()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (bw.pf.o, bw.pf.lse, bw.dq, bw.dk, bw.dv, od, lsed):
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "decode o", "decode lse"), ref,
                              outs()):
            assert torch.equal(a, b), f"replay {rep}: {name}"


def test_graph_replays_match_eager_varlen(lib):
    """The packed forward and backward captured together (a training step on
    a packed batch), replayed against their eager results."""
    import torch
    lens = np.array([700, 0, 33, 1500, 256], np.int64)
    T, max_len = int(lens.sum()), int(lens.max())
    Hq, Hkv, d = 8, 2, 64
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    x = W.random_prefill(504, 1, T, Hq, Hkv, d)
    q, k, v = bits_to_dev(x.q_bits[0]), bits_to_dev(x.k_bits[0]), bits_to_dev(x.v_bits[0])
    do = bits_to_dev(W.grad_output(505, 1, T, Hq, d)[0])
    p = C.make_pattern(max_len, 16, 128, 0, 4, 2)
    bm, bn = C.cowa_fwd_block_sizes(d)
    bmk, bnk = C.cowa_bwd_block_sizes(d)
    rp, col, fl = [torch.from_numpy(a).cuda() for a in C.cowa_plan(p, max_len, Hkv, bm, bn)]
    rpk, colk, flk = [torch.from_numpy(a).cuda()
                      for a in C.cowa_plan_kv(p, max_len, Hkv, bmk, bnk)]
    ws = torch.empty(C.cowa_bwd_workspace_size(p, len(lens), Hq, Hkv, max_len),
                     dtype=torch.uint8, device="cuda")
    fws = torch.empty(C.cowa_fwd_workspace_size(len(lens), max_len, Hkv, d), dtype=torch.uint8,
                      device="cuda")
    o = torch.empty((T, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    dq = torch.empty((T, Hq, d), dtype=torch.bfloat16, device="cuda")
    dk = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device="cuda")
    dv = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / np.sqrt(d)

    def work():
        C.cowa_fwd_varlen(p, rp, col, fl, col.numel(), bm, bn, q, k, v, o, lse, cu, max_len,
                          scale, workspace=fws)
        C.cowa_bwd_varlen(p, rp, col, fl, col.numel(), bm, bn, rpk, colk, flk, colk.numel(),
                          bmk, bnk, q, k, v, o, do, lse, dq, dk, dv, cu, max_len, scale, ws)

    tensors = (o, lse, dq, dk, dv)
    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in tensors]
    assert all(torch.isfinite(t.float()).all() for t in ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in tensors:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), ref, tensors):
            assert torch.equal(a, b), f"replay {rep}: {name}"
