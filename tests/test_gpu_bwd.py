"""GPU parity of cowa_bwd against the fp64 oracle (through the C ABI).

Small shapes compare every gradient element against element-wise bounds
derived from the kernels' roundings (tests/gpu_helpers.py): with the oracle's
O and LSE as the backward's inputs (the backward kernels alone), and after
the GPU forward (training as it runs).  The large workloads run the GPU
forward and backward at full size and compare sampled query rows (dQ),
sampled keys (dK, dV) and sums over all keys that hold at any size."""

import numpy as np
import pytest

from structured_sparse_attention_cowa_amd import workloads as W
from tests.gpu_helpers import D_REL_EXACT, D_REL_FWD, GRAD_REL, OUT_REL_BF16, Backward, \
    check_grad, sample_rows

pytestmark = pytest.mark.gpu


def _full(x, S, Wd, H, off=0, mode=0, o_dtype="f32", g_dtype="f32", gpu_forward=False,
          what=""):
    """Every gradient element against the oracle.  By default the backward
    takes the oracle's O and LSE (the tight bound isolates the backward
    kernels); gpu_forward=True runs the GPU forward first, as in training."""
    bw = Backward(x, S, Wd, H, off, mode, o_dtype=o_dtype, g_dtype=g_dtype)
    pf = bw.pf
    print(f"[bwd] {what} B={pf.B} N={pf.N} Hq={pf.Hq} Hkv={pf.Hkv} S={S} W={Wd} H={H} "
          f"off={off} mode={mode} o={o_dtype} g={g_dtype} gpu_forward={gpu_forward}",
          flush=True)
    if gpu_forward:
        pf.run()
    else:
        bw.set_oracle_forward()
    bw.run_bwd()
    dq, dk, dv = bw.result()
    rq, rk, rv, mq, mk, mv, eq, ek = bw.oracle_full()
    d_rel = D_REL_FWD if gpu_forward else D_REL_EXACT
    out = OUT_REL_BF16 if g_dtype == "bf16" else 0.0
    r = [check_grad(dq, rq, mq, eq, f"{what} dQ", d_rel, out),
         check_grad(dk, rk, mk, ek, f"{what} dK", d_rel, out),
         check_grad(dv, rv, mv, np.zeros_like(mv), f"{what} dV", d_rel, out)]
    print(f"[bwd] {what} worst error / bound: dQ {r[0]:.3f} dK {r[1]:.3f} dV {r[2]:.3f}",
          flush=True)
    return bw


def test_bwd_tiny_shape_full(lib):
    # the tiny workload's shape and pattern at d = 128
    x = W.random_prefill(201, 1, 1024, 8, 4, 128)
    _full(x, 16, 128, 4, what="tiny-d128")


def test_bwd_ragged_offset_gqa5(lib):
    x = W.random_prefill(202, 2, 1000, 10, 2, 128)
    _full(x, 16, 128, 4, off=1, what="ragged-gqa5")


def test_bwd_causal_mode(lib):
    x = W.random_prefill(203, 1, 777, 4, 2, 128)
    _full(x, 8, 64, 4, mode=1, what="causal")


@pytest.mark.parametrize("N,S,Wd,H,off,Hq,Hkv", [
    (1, 0, 1, 1, 0, 2, 1),        # single token
    (17, 2, 4, 4, 0, 8, 4),       # worked ragged case
    (64, 3, 10, 2, 1, 2, 1),      # exactly one query tile
    (65, 3, 10, 2, 1, 2, 1),      # one row past a tile
    (129, 0, 1, 8, 3, 4, 2),      # band only, ragged key tile
    (300, 40, 400, 4, 0, 4, 4),   # window covers all (L = 0)
    (520, 520, 1, 2, 0, 2, 2),    # sink covers all
    (640, 3, 10, 1, 0, 4, 1),     # one global head: dense causal
])
def test_bwd_edge_shapes(lib, N, S, Wd, H, off, Hq, Hkv):
    x = W.random_prefill(300 + N, 2, N, Hq, Hkv, 128)
    _full(x, S, Wd, H, off, what=f"edge N={N}")


@pytest.mark.parametrize("o_dtype,g_dtype", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
def test_bwd_after_gpu_forward(lib, o_dtype, g_dtype):
    x = W.random_prefill(204, 1, 1024, 8, 2, 128)
    _full(x, 16, 128, 4, off=2, o_dtype=o_dtype, g_dtype=g_dtype, gpu_forward=True,
          what=f"e2e o={o_dtype}")


@pytest.mark.parametrize("gpu_forward,g_dtype", [(False, "f32"), (True, "bf16")])
def test_bwd_tiny_workload_d64(lib, gpu_forward, g_dtype):
    # the tiny workload itself (d = 64, its pattern), every gradient element
    w = W.TINY
    x = W.prefill_inputs(w)
    _full(x, w.sink, w.window, w.h_kv_global, g_dtype=g_dtype, gpu_forward=gpu_forward,
          what=f"tiny-d64 gpu_forward={gpu_forward}")


@pytest.mark.parametrize("N,S,Wd,H,off,Hq,Hkv", [
    (17, 2, 4, 4, 0, 8, 4),       # ragged, shorter than one tile
    (129, 0, 1, 8, 3, 4, 2),      # band only, ragged key tile
    (1000, 16, 128, 4, 1, 10, 2), # GQA 5, ragged
])
def test_bwd_edge_shapes_d64(lib, N, S, Wd, H, off, Hq, Hkv):
    x = W.random_prefill(400 + N, 2, N, Hq, Hkv, 64)
    _full(x, S, Wd, H, off, what=f"d64 N={N}")


def test_bwd_split_sink_tiles_d64(lib):
    # 100 query tiles x 4 heads see the sink key tile: its step list is cut into
    # parts whose fp32 partials are summed by the reduction kernel
    x = W.random_prefill(411, 1, 6400, 4, 1, 64)
    from structured_sparse_attention_cowa_amd import binding as C
    cp = C.make_pattern(6400, 32, 64, 0, 8, 0)
    assert C.cowa_bwd_workspace_size(cp, 1, 4, 1, 6400) > 2 * (4 * 6400 * 4)
    _full(x, 32, 64, 8, what="d64 split sink tiles")


def test_bwd_2k_full(lib):
    x = W.random_prefill(205, 1, 2048, 6, 2, 128)
    _full(x, 64, 256, 8, off=5, what="2k")


def test_bwd_deterministic(lib):
    x = W.random_prefill(206, 1, 1500, 4, 2, 128)
    bw = Backward(x, 16, 128, 4)
    bw.run()
    a = bw.result()
    bw.dq.fill_(0)
    bw.dk.fill_(0)
    bw.dv.fill_(0)
    bw.run_bwd()
    b = bw.result()
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def _dv_sum_property(bw, dv, what):
    """sum_j dV_j = sum over the group's heads and all rows of dO_t (each row's
    probabilities sum to 1); the roundings of P bound the error by
    GRAD_REL sum |dO_t|."""
    pf = bw.pf
    G = pf.Hq // pf.Hkv
    do = bw.dout().astype(np.float64).reshape(pf.B, pf.N, pf.Hkv, G, pf.d)
    want = do.sum(axis=(1, 3))
    bound = GRAD_REL * np.abs(do).sum(axis=(1, 3)) + 1e-3
    got = dv.astype(np.float64).sum(axis=1)
    assert (np.abs(got - want) <= bound).all(), f"{what}: sum of dV differs from sum of dO"


def _dk_sum_property(bw, dk, what):
    """sum_j dK_j = scale sum_t q_t sum_j dS_tj = 0 (sum_j dS_tj = 0 per row)."""
    s = dk.astype(np.float64).sum(axis=1)
    a = np.abs(dk.astype(np.float64)).sum(axis=1)
    assert (np.abs(s) <= 1e-2 * a + 1e-3).all(), f"{what}: sum of dK is not ~0"


def _sampled(w, x, off, mode, n_rows, n_keys, seed, heads_kv=None, what=""):
    """GPU forward then backward at the workload's full size; sampled rows and
    keys against the oracle (bound with the forward's D error), plus the sum
    properties over all keys."""
    bw = Backward(x, w.sink, w.window, w.h_kv_global, off, mode, n_ctx=w.N, do_seed=seed)
    print(f"[bwd] {w.name} {what} off={off} mode={mode}", flush=True)
    bw.run()
    dq, dk, dv = bw.result()
    pf = bw.pf
    rows = sample_rows(w.N, w.window, w.sink, w.stated_band, w.h_kv_global, n_rows, seed)
    rq, mq, eq = bw.oracle_rows(rows)
    rq_w = check_grad(dq[:, rows], rq, mq, eq, f"{w.name} dQ rows", D_REL_FWD)
    # keys near the end are seen only by local-window rows, so the oracle
    # sums few rows
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    keys = np.unique(np.concatenate([[w.N - 1, w.N - 2, w.N - 64, w.N - 128, w.N - 129],
                                     rng.integers(w.N - 512, w.N, n_keys)]))
    hk = list(range(pf.Hkv)) if heads_kv is None else heads_kv
    rk, rv, mk, mv, ek = bw.oracle_keys(keys, hk)
    rk_w = check_grad(dk[:, keys][:, :, hk], rk, mk, ek, f"{w.name} dK keys", D_REL_FWD)
    rv_w = check_grad(dv[:, keys][:, :, hk], rv, mv, np.zeros_like(mv), f"{w.name} dV keys")
    _dv_sum_property(bw, dv, w.name)
    _dk_sum_property(bw, dk, w.name)
    print(f"[bwd] {w.name} worst error / bound: dQ {rq_w:.3f} dK {rk_w:.3f} dV {rv_w:.3f}",
          flush=True)
    return bw, dq, dk, dv


def test_bwd_8k_workload_sampled(lib):
    w = W.P8K
    x = W.prefill_inputs(w)
    bw, dq, dk, dv = _sampled(w, x, 0, 0, 16, 24, 91, heads_kv=[0, 7])
    # the sink key 0 and a key mid-sequence, for one KV head: every row that
    # sees them enters the oracle's sum
    keys = np.array([0, 63, 64, 4000])
    rk, rv, mk, mv, ek = bw.oracle_keys(keys, [3])
    check_grad(dk[:, keys][:, :, [3]], rk, mk, ek, "8k dK sink/mid keys", D_REL_FWD)
    check_grad(dv[:, keys][:, :, [3]], rv, mv, np.zeros_like(mv), "8k dV sink/mid keys")


def test_bwd_32k_causal_mode_sampled(lib):
    w = W.P32K
    x = W.prefill_inputs(w)
    _sampled(w, x, 0, 1, 8, 16, 92, heads_kv=[2], what="causal")


@pytest.mark.parametrize("g", [0, 3, 7])
def test_bwd_128k_rank_sampled(lib, g):
    w = W.P128K
    x = W.prefill_inputs(w)
    _sampled(w, x, g, 0, 12, 16, 93 + g)
