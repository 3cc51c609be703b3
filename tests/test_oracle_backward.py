"""Pins for the oracle's backward pass: torch autograd on float64 SDPA where
CoWA reduces to dense causal attention, central finite differences on the
16-token CoWA pattern, and agreement of the row/key-sampled forms with the
full backward."""

import numpy as np
import pytest
import torch

import oracle.cowa_oracle as O
from oracle.cowa_oracle import Pattern, MODE_CAUSAL
from structured_sparse_attention_cowa_amd import workloads as W


def sdpa_grads(q, k, v, do, scale):
    B, N, Hq, d = q.shape
    G = Hq // k.shape[2]
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    kk = kt.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vv = vt.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qt.permute(0, 2, 1, 3), kk, vv,
                                                         is_causal=True, scale=scale)
    (o.permute(0, 2, 1, 3) * torch.tensor(do, dtype=torch.float64)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("case", ["sink_plus_window", "one_global_head", "causal_mode"])
def test_backward_reduces_to_dense_causal_autograd(case):
    B, N, Hq, Hkv, d = 2, 80, 4, 2, 16
    x = W.random_prefill(3, B, N, Hq, Hkv, d)
    q, k, v = x.q(), x.k(), x.v()
    if case == "one_global_head":
        x = W.random_prefill(3, B, N, Hq, 1, d)
        q, k, v = x.q(), x.k(), x.v()
        p = Pattern(n_ctx=N, sink=3, window=9, h_kv_global=1)
    elif case == "sink_plus_window":
        p = Pattern(n_ctx=N, sink=30, window=50, h_kv_global=4)
    else:
        p = Pattern(n_ctx=N, sink=3, window=9, h_kv_global=4, mode=MODE_CAUSAL)
    do = np.random.Generator(np.random.PCG64(4)).standard_normal(q.shape)
    dq, dk, dv = O.attention_backward(q, k, v, do, p, 0.3)
    rq, rk, rv = sdpa_grads(q, k, v, do, 0.3)
    for a, r in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, r, rtol=0, atol=1e-11)


def test_backward_finite_differences_cowa_pattern():
    B, N, Hq, Hkv, d = 1, 16, 8, 4, 4
    rng = np.random.Generator(np.random.PCG64(5))
    q = rng.standard_normal((B, N, Hq, d))
    k = rng.standard_normal((B, N, Hkv, d))
    v = rng.standard_normal((B, N, Hkv, d))
    do = rng.standard_normal((B, N, Hq, d))
    p = Pattern(n_ctx=16, sink=2, window=4, h_kv_global=4)
    scale = 0.7

    def loss(q_, k_, v_):
        o, _ = O.attention(q_, k_, v_, p, scale)
        return float((o * do).sum())

    dq, dk, dv = O.attention_backward(q, k, v, do, p, scale)
    eps = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        direction = rng.standard_normal(arr.shape)
        plus = arr + eps * direction
        minus = arr - eps * direction
        args_p = {"q": q, "k": k, "v": v}
        args_m = dict(args_p)
        args_p[name] = plus
        args_m[name] = minus
        fd = (loss(args_p["q"], args_p["k"], args_p["v"]) -
              loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        assert abs(fd - float((grad * direction).sum())) < 1e-7, name


def test_backward_sampled_forms_match_full():
    B, N, Hq, Hkv, d = 1, 300, 4, 2, 8
    x = W.random_prefill(6, B, N, Hq, Hkv, d)
    q, k, v = x.q(), x.k(), x.v()
    do = np.random.Generator(np.random.PCG64(7)).standard_normal(q.shape)
    p = Pattern(n_ctx=N, sink=5, window=30, h_kv_global=4, kv_head_offset=2)
    dq, dk, dv = O.attention_backward(q, k, v, do, p, 0.25)
    rows = np.array([0, 7, 64, 250, 299])
    dq_s = O.backward_rows_dq(q, k, v, do, p, 0.25, rows)
    np.testing.assert_allclose(dq_s, dq[:, rows], rtol=0, atol=1e-12)
    keys = np.array([0, 3, 200, 298, 299])
    dk_s, dv_s = O.backward_keys_dkdv(q, k, v, do, p, 0.25, keys)
    np.testing.assert_allclose(dk_s, dk[:, keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_s, dv[:, keys], rtol=0, atol=1e-12)


def test_backward_gqa_sums_query_heads():
    # with G query heads per KV head, dK/dV are the sums of the per-head
    # gradients of G independent single-head problems
    B, N, G, d = 1, 64, 3, 8
    x = W.random_prefill(8, B, N, G, 1, d)
    q, k, v = x.q(), x.k(), x.v()
    do = np.random.Generator(np.random.PCG64(9)).standard_normal(q.shape)
    p = Pattern(n_ctx=N, sink=2, window=7, h_kv_global=2, kv_head_offset=1)
    dq, dk, dv = O.attention_backward(q, k, v, do, p, 0.4)
    sk = np.zeros_like(dk)
    sv = np.zeros_like(dv)
    for hq in range(G):
        a, b_, c = O.attention_backward(q[:, :, hq:hq + 1], k, v, do[:, :, hq:hq + 1], p, 0.4)
        np.testing.assert_allclose(a[:, :, 0], dq[:, :, hq], rtol=0, atol=1e-12)
        sk += b_
        sv += c
    np.testing.assert_allclose(sk, dk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(sv, dv, rtol=0, atol=1e-12)


def test_kv_tile_lists_are_the_transpose():
    p = Pattern(n_ctx=1000, sink=16, window=128, h_kv_global=4, kv_head_offset=1)
    rp, col, fl = O.tile_lists(1000, 2, p, 64, 128)
    rpt, colt, flt = O.tile_lists_kv(1000, 2, p, 64, 128)
    nqt, nkt = -(-1000 // 64), -(-1000 // 128)
    for h in range(2):
        a = {}
        for qi in range(nqt):
            r = h * nqt + qi
            for e in range(rp[r], rp[r + 1]):
                a[(qi, int(col[e]))] = int(fl[e])
        bt = {}
        for kj in range(nkt):
            r = h * nkt + kj
            cols = list(colt[rpt[r]:rpt[r + 1]])
            assert cols == sorted(cols)
            for e in range(rpt[r], rpt[r + 1]):
                bt[(int(colt[e]), kj)] = int(flt[e])
        assert a == bt


def test_backward_magnitudes():
    """The term-magnitude sums bound each gradient (triangle inequality), equal
    it when every term has one sign (dV with dO >= 0 is sum_t P_tj dO_t, all
    terms >= 0), and the sampled forms return the same magnitudes."""
    B, N, Hq, Hkv, d = 1, 200, 4, 2, 8
    x = W.random_prefill(10, B, N, Hq, Hkv, d)
    q, k, v = x.q(), x.k(), x.v()
    rng = np.random.Generator(np.random.PCG64(11))
    do = rng.standard_normal(q.shape)
    p = Pattern(n_ctx=N, sink=4, window=20, h_kv_global=4, kv_head_offset=1)
    dq, dk, dv, mq, mk, mv, eq, ek = O.attention_backward(q, k, v, do, p, 0.3,
                                                          magnitudes=True)
    for g, m in ((dq, mq), (dk, mk), (dv, mv)):
        assert (m >= np.abs(g) - 1e-12).all()
        assert (m > np.abs(g) + 1e-6).any()  # signs do cancel somewhere
    assert (eq > 0).all() and (ek[:, :N] > 0).all()
    do_pos = np.abs(do)
    _, _, dv_p, _, _, mv_p, _, _ = O.attention_backward(q, k, v, do_pos, p, 0.3,
                                                        magnitudes=True)
    np.testing.assert_allclose(mv_p, dv_p, rtol=1e-13, atol=0)
    rows = np.array([0, 5, 99, 199])
    dq_s, mq_s, eq_s = O.backward_rows_dq(q, k, v, do, p, 0.3, rows, magnitudes=True)
    np.testing.assert_allclose(mq_s, mq[:, rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(eq_s, eq[:, rows], rtol=1e-12, atol=0)
    keys = np.array([0, 3, 150, 199])
    _, _, mk_s, mv_s, ek_s = O.backward_keys_dkdv(q, k, v, do, p, 0.3, keys, magnitudes=True)
    np.testing.assert_allclose(mk_s, mk[:, keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(mv_s, mv[:, keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ek_s, ek[:, keys], rtol=1e-12, atol=0)


def test_backward_invariant_to_a_common_shift_of_v():
    """Adding one vector c to every value row moves O_t and dP_tj by dO_t.c
    and D_t by the same amount, so dS, dQ and dK do not change; dV does not
    depend on V.  A dropped or mis-signed D term breaks this."""
    B, N, Hq, Hkv, d = 1, 60, 4, 2, 8
    x = W.random_prefill(12, B, N, Hq, Hkv, d)
    q, k, v = x.q(), x.k(), x.v()
    rng = np.random.Generator(np.random.PCG64(13))
    do = rng.standard_normal(q.shape)
    p = Pattern(n_ctx=N, sink=2, window=6, h_kv_global=2)
    c = 3.0 * rng.standard_normal(d)
    a = O.attention_backward(q, k, v, do, p, 0.5)
    b = O.attention_backward(q, k, v + c, do, p, 0.5)
    for u, w in zip(a, b):
        np.testing.assert_allclose(u, w, rtol=0, atol=1e-11)
    assert np.abs(a[0]).max() > 0.1
