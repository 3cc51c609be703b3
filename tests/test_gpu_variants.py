"""GPU parity of the pattern variants against the fp64 oracle: sliding-window
attention with sinks (COWA_MODE_SINK_LOCAL) and the duplicated-window
ablation (n_bands distinct long-range windows), through the same plan,
forward, decode and backward entry points."""

import numpy as np
import pytest

import oracle.cowa_oracle as O
from structured_sparse_attention_cowa_amd import binding as C
from structured_sparse_attention_cowa_amd import workloads as W
from tests.gpu_helpers import (D_REL_EXACT, Backward, Prefill, bits_to_dev, check_close,
                               check_grad, sample_rows)

pytestmark = pytest.mark.gpu

VARIANTS = [dict(mode=2), dict(n_bands=1), dict(n_bands=2), dict(n_bands=2, offset=1)]


def _ids(v):
    return "-".join(f"{k}{x}" for k, x in v.items())


@pytest.mark.parametrize("v", VARIANTS, ids=_ids)
def test_variant_prefill_full(lib, v):
    x = W.random_prefill(401, 2, 1000, 6, 3, 128)
    off = v.get("offset", 0)
    pf = Prefill(x, 16, 128, 4, offset=off, mode=v.get("mode", 0), n_bands=v.get("n_bands", 0))
    print(f"[variant fwd] {v}", flush=True)
    pf.run()
    o, lse = pf.result()
    o_ref, lse_ref = pf.oracle()
    check_close(o, lse, o_ref, lse_ref, f"variant {v}")


@pytest.mark.parametrize("v", [dict(mode=2), dict(n_bands=2), dict(n_bands=4)], ids=_ids)
def test_variant_prefill_8k_sampled(lib, v):
    """The ablation's setting: 8 KV heads at 8K (1, 2, 4, 8 distinct windows)."""
    w = W.P8K
    x = W.prefill_inputs(w)
    pf = Prefill(x, w.sink, w.window, w.h_kv_global, mode=v.get("mode", 0),
                 n_bands=v.get("n_bands", 0))
    print(f"[variant fwd 8k] {v}", flush=True)
    pf.run()
    o, lse = pf.result()
    rows = sample_rows(w.N, w.window, w.sink, w.stated_band, w.h_kv_global, 12, 55)
    heads = [0, 5, 17, 31]
    o_ref, lse_ref = pf.oracle(rows=rows, heads=heads)
    check_close(o[:, rows][:, :, heads], lse[:, heads][:, :, rows], o_ref, lse_ref, f"8k {v}")


@pytest.mark.parametrize("v", VARIANTS, ids=_ids)
def test_variant_decode(lib, v):
    import torch
    B, n_max, Hq, Hkv, d = 4, 3000, 8, 2, 128
    off = v.get("offset", 0)
    rng = np.random.Generator(np.random.PCG64(402))
    lens = np.array([1, 700, 2999, 3000], np.int32)
    q_bits = W.to_bf16_bits(rng.standard_normal((B, Hq, d), dtype=np.float32))
    kb, vb = W.decode_cache_host(403, B, n_max, Hkv, d, lens)
    mode, nb = v.get("mode", 0), v.get("n_bands", 0)
    p = C.make_pattern(n_max, 16, 256, 0, 4, off, mode, nb)
    ws = torch.zeros(C.cowa_decode_workspace_size(p, B, Hq, Hkv, d, n_max), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    print(f"[variant decode] {v}", flush=True)
    C.cowa_decode(p, bits_to_dev(q_bits), bits_to_dev(kb), bits_to_dev(vb),
                  torch.from_numpy(lens).cuda(), o, lse, 1.0 / np.sqrt(d), ws)
    torch.cuda.synchronize()
    op = O.Pattern(n_max, 16, 256, 0, 4, off, mode, nb)
    o_ref, lse_ref = O.decode(W.bf16_bits_to_f32(q_bits), W.bf16_bits_to_f32(kb),
                              W.bf16_bits_to_f32(vb), lens, op, 1.0 / np.sqrt(d))
    check_close(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"decode {v}")


@pytest.mark.parametrize("v", VARIANTS, ids=_ids)
def test_variant_backward_full(lib, v):
    x = W.random_prefill(404, 1, 900, 6, 3, 128)
    bw = Backward(x, 16, 128, 4, offset=v.get("offset", 0), mode=v.get("mode", 0),
                  n_bands=v.get("n_bands", 0))
    print(f"[variant bwd] {v}", flush=True)
    bw.set_oracle_forward()
    bw.run_bwd()
    dq, dk, dv = bw.result()
    rq, rk, rv, mq, mk, mv, eq, ek = bw.oracle_full()
    check_grad(dq, rq, mq, eq, f"{v} dQ", D_REL_EXACT)
    check_grad(dk, rk, mk, ek, f"{v} dK", D_REL_EXACT)
    check_grad(dv, rv, mv, np.zeros_like(mv), f"{v} dV", D_REL_EXACT)
