"""GPU parity of the packed (varlen) backward: sequences of different lengths
in one call, after the packed GPU forward, each sequence's dQ, dK, dV against
the fp64 oracle's backward of that sequence alone (the element-wise bounds of
tests/gpu_helpers.py for a backward that takes the GPU forward's O and LSE)."""

import numpy as np
import pytest

import oracle.cowa_oracle as O
from structured_sparse_attention_cowa_amd import binding as C
from structured_sparse_attention_cowa_amd import workloads as W
from tests.gpu_helpers import D_REL_FWD, OUT_REL_BF16, bits_to_dev, check_grad

pytestmark = pytest.mark.gpu


def _run(lens, Hq, Hkv, d, kw, seed, g_dtype):
    import torch
    lens = np.asarray(lens, np.int64)
    T = int(lens.sum())
    max_len = int(lens.max())
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = W.random_prefill(seed, 1, T, Hq, Hkv, d)
    do_bits = W.grad_output(seed + 1, 1, T, Hq, d)[0]
    p = C.make_pattern(kw.get("n_ctx", max_len), kw["sink"], kw["window"], 0, kw["h"],
                       kw.get("off", 0), kw.get("mode", 0), kw.get("n_bands", 0))
    bm, bn = C.cowa_fwd_block_sizes(d)
    bmk, bnk = C.cowa_bwd_block_sizes(d)
    rp, col, fl = [torch.from_numpy(a).cuda() for a in C.cowa_plan(p, max_len, Hkv, bm, bn)]
    rpk, colk, flk = [torch.from_numpy(a).cuda()
                      for a in C.cowa_plan_kv(p, max_len, Hkv, bmk, bnk)]
    q, k, v = bits_to_dev(x.q_bits[0]), bits_to_dev(x.k_bits[0]), bits_to_dev(x.v_bits[0])
    do = bits_to_dev(do_bits)
    o = torch.full((T, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    gdt = torch.float32 if g_dtype == "f32" else torch.bfloat16
    dq = torch.full((T, Hq, d), float("nan"), dtype=gdt, device="cuda")
    dk = torch.full((T, Hkv, d), float("nan"), dtype=gdt, device="cuda")
    dv = torch.full((T, Hkv, d), float("nan"), dtype=gdt, device="cuda")
    ws = torch.full((C.cowa_bwd_workspace_size(p, len(lens), Hq, Hkv, max_len),), 0xFF,
                    dtype=torch.uint8, device="cuda")  # no initialisation needed
    cu_d = torch.from_numpy(cu).cuda()
    scale = 1.0 / np.sqrt(d)
    print(f"[bwd varlen] lens={list(lens)} Hq={Hq} Hkv={Hkv} d={d} {kw} g={g_dtype}", flush=True)
    C.cowa_fwd_varlen(p, rp, col, fl, col.numel(), bm, bn, q, k, v, o, lse, cu_d, max_len, scale)
    C.cowa_bwd_varlen(p, rp, col, fl, col.numel(), bm, bn, rpk, colk, flk, colk.numel(), bmk,
                      bnk, q, k, v, o, do, lse, dq, dk, dv, cu_d, max_len, scale, ws)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy() for t in (dq, dk, dv)]
    return x, do_bits, p, cu, got, scale


CASES = [
    ([1, 17, 255, 256, 257, 1000, 64], 8, 4, 128, dict(sink=16, window=128, h=4), "f32"),
    ([700, 3, 1500, 129], 10, 2, 64, dict(sink=5, window=100, h=8, off=3), "bf16"),
    ([300, 900, 40], 4, 2, 128, dict(sink=8, window=64, h=4, mode=1), "f32"),
    ([512, 1024, 77], 6, 3, 128, dict(sink=8, window=64, h=4, n_bands=2, n_ctx=1024), "f32"),
    # empty sequences inside the batch get no rows and disturb no others
    ([0, 300, 0, 0, 129, 0], 4, 2, 128, dict(sink=8, window=64, h=4, off=1), "f32"),
    # the longest sequence's sink key tile has its step list split into parts;
    # the shorter sequences take the leading part of the same plan rows
    ([6400, 100, 3000], 4, 1, 64, dict(sink=32, window=64, h=8), "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[0]) for c in CASES])
def test_bwd_varlen_against_oracle(lib, case):
    lens, Hq, Hkv, d, kw, g_dtype = case
    x, do_bits, p, cu, (dq, dk, dv), scale = _run(lens, Hq, Hkv, d, kw, 811, g_dtype)
    op = O.Pattern(p.n_ctx, p.sink, p.window, 0, p.h_kv_global, p.kv_head_offset, p.mode,
                   p.n_bands)
    do = W.bf16_bits_to_f32(do_bits).astype(np.float64)
    out = OUT_REL_BF16 if g_dtype == "bf16" else 0.0
    for i, n in enumerate(lens):
        a, b = int(cu[i]), int(cu[i + 1])
        if n == 0:
            continue
        rq, rk, rv, mq, mk, mv, eq, ek = O.attention_backward(
            x.q()[:, a:b], x.k()[:, a:b], x.v()[:, a:b], do[None, a:b], op, scale,
            magnitudes=True)
        what = f"varlen seq {i} (n={n})"
        r = [check_grad(dq[None, a:b], rq, mq, eq, what + " dQ", D_REL_FWD, out),
             check_grad(dk[None, a:b], rk, mk, ek, what + " dK", D_REL_FWD, out),
             check_grad(dv[None, a:b], rv, mv, np.zeros_like(mv), what + " dV", D_REL_FWD, out)]
        print(f"[bwd varlen] {what} worst error / bound: {r[0]:.3f} {r[1]:.3f} {r[2]:.3f}",
              flush=True)
