"""Helpers shared by the GPU parity tests: run the library through the C ABI
and compare with the fp64 oracle at the stated tolerances."""

from __future__ import annotations

import numpy as np

import oracle.cowa_oracle as O
from structured_sparse_attention_cowa_amd import binding as C
from structured_sparse_attention_cowa_amd import workloads as W

# Acceptance: O max-abs <= 2e-2; LSE |diff| <= 1e-3 * max(1, |LSE_ref|).
O_TOL = 2e-2
LSE_REL = 1e-3
# Backward tolerance, element-wise, from the arithmetic of the kernels: every
# gradient element is a sum of terms P_tj dO_t or scale dS_tj (k_j or q_t),
# and the kernels round each P and dS once to bf16 (8-bit significand, unit
# roundoff u = 2^-8) before an exact bf16 product and an fp32 sum.  D_t =
# dO_t . O_t enters every dS_tj of a row with the same sign, so an error in O
# (the forward's own bf16 rounding of P, and O's storage) moves dQ and dK by
# up to that relative error times the oracle's D-sensitivities eq, ek.
# Bounds:
#   |err| <= GRAD_REL * m + D_REL_FWD * e   (O and LSE from the GPU forward)
#   |err| <= GRAD_REL * m + D_REL_EXACT * e (O and LSE from the oracle: only
#            fp32 rounding of O and fp32 sums remain in D and dP)
# with m the sum of the terms' absolute values.  Each constant is twice the
# rounding it covers: 2u = 2^-7 for bf16 roundings, and 2^-12 for fp32 sums of
# 128 products (128 * 2^-24 = 2^-17) with room to spare.  A single-term sum
# (a key seen by one row) can reach the full u, so the factor 2 is the only
# headroom.  Gradients stored in bf16 add u |ref| (as 2u |ref|).
GRAD_REL = 2.0 ** -7
D_REL_FWD = 2.0 ** -7
D_REL_EXACT = 2.0 ** -12
OUT_REL_BF16 = 2.0 ** -7


def check_close(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O"
    assert np.isfinite(lse_gpu).all(), f"{what}: non-finite LSE"
    err_o = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    err_l = np.abs(lse_gpu - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
    err_l = float(err_l.max()) if err_l.size else 0.0
    assert err_o <= O_TOL, f"{what}: O max-abs error {err_o:.3e} > {O_TOL}"
    assert err_l <= LSE_REL, f"{what}: LSE error {err_l:.3e} > {LSE_REL}"
    return err_o, err_l


def bits_to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class Prefill:
    """Device-resident prefill problem: inputs, plan and outputs."""

    def __init__(self, x: W.PrefillInputs, sink, window, h_kv_global, offset=0, mode=0,
                 n_ctx=None, o_dtype="f32", n_bands=0):
        import torch
        self.x = x
        B, N, Hq, d = x.q_bits.shape
        Hkv = x.k_bits.shape[2]
        self.B, self.N, self.Hq, self.Hkv, self.d = B, N, Hq, Hkv, d
        self.pattern = C.make_pattern(n_ctx or N, sink, window, 0, h_kv_global, offset, mode,
                                      n_bands)
        self.opattern = O.Pattern(n_ctx or N, sink, window, 0, h_kv_global, offset, mode,
                                  n_bands)
        self.bm, self.bn = C.cowa_fwd_block_sizes(d)
        rp, col, fl = C.cowa_plan(self.pattern, N, Hkv, self.bm, self.bn)
        self.nnz = len(col)
        self.rp = torch.from_numpy(rp).cuda()
        self.col = torch.from_numpy(col if len(col) else np.zeros(1, np.int32)).cuda()
        self.fl = torch.from_numpy(fl if len(fl) else np.zeros(1, np.uint8)).cuda()
        self.q = bits_to_dev(x.q_bits)
        self.k = bits_to_dev(x.k_bits)
        self.v = bits_to_dev(x.v_bits)
        odt = torch.float32 if o_dtype == "f32" else torch.bfloat16
        self.o = torch.empty((B, N, Hq, d), dtype=odt, device="cuda")
        self.lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
        self.ws = torch.empty(C.cowa_fwd_workspace_size(B, N, Hkv, d), dtype=torch.uint8,
                              device="cuda")
        self.scale = 1.0 / np.sqrt(d)

    def run(self, stream=None):
        C.cowa_fwd(self.pattern, self.rp, self.col, self.fl, self.nnz, self.bm, self.bn,
                   self.q, self.k, self.v, self.o, self.lse, self.scale, stream, self.ws)

    def result(self):
        import torch
        torch.cuda.synchronize()
        return self.o.float().cpu().numpy(), self.lse.cpu().numpy()

    def oracle(self, rows=None, heads=None):
        return O.attention(self.x.q(), self.x.k(), self.x.v(), self.opattern, self.scale,
                           rows=rows, heads=heads)


def sample_rows(N, window, sink, band, h_kv_global, n_random, seed):
    """Boundary rows of every window and band plus a seeded random sample."""
    rng = np.random.Generator(np.random.PCG64(seed))
    edges = [0, 1, 2, 63, 64, 127, 128, N - 1, N - 2, N - 64, N - 128]
    for base in [sink, window] + [window + g * band for g in range(h_kv_global + 1)]:
        edges += [base - 1, base, base + 1, base + 127, base + 128]
    r = np.concatenate([np.asarray(edges), rng.integers(0, N, n_random)])
    return np.unique(r[(r >= 0) & (r < N)])


def check_grad(gpu, ref, m, e, what="", d_rel=D_REL_EXACT, out_rel=0.0):
    """Element-wise |gpu - ref| <= GRAD_REL m + d_rel e (+ out_rel |ref| for
    gradients stored in bf16).  Returns the largest ratio of error to bound."""
    gpu = np.asarray(gpu, dtype=np.float64)
    assert np.isfinite(gpu).all(), f"{what}: non-finite gradient"
    if ref.size == 0:
        return 0.0
    bound = GRAD_REL * m + d_rel * e + out_rel * np.abs(ref) + 1e-30
    ratio = np.abs(gpu - ref) / bound
    worst = float(ratio.max())
    i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert worst <= 1.0, (f"{what}: error {abs(gpu[i] - ref[i]):.3e} at {i} exceeds bound "
                          f"{bound[i]:.3e} (ref {ref[i]:.3e}, m {m[i]:.3e}, e {e[i]:.3e})")
    return worst


class Backward:
    """Device-resident backward problem: a Prefill (run first for O and LSE),
    the upstream gradient, both plans, the workspace and the gradients."""

    def __init__(self, x: W.PrefillInputs, sink, window, h_kv_global, offset=0, mode=0,
                 n_ctx=None, o_dtype="f32", g_dtype="f32", do_seed=1, n_bands=0):
        import torch
        self.pf = pf = Prefill(x, sink, window, h_kv_global, offset, mode, n_ctx, o_dtype,
                               n_bands)
        B, N, Hq, Hkv, d = pf.B, pf.N, pf.Hq, pf.Hkv, pf.d
        self.do_bits = W.grad_output(do_seed, B, N, Hq, d)
        self.do = bits_to_dev(self.do_bits)
        self.bm_kv, self.bn_kv = C.cowa_bwd_block_sizes(d)
        rp, col, fl = C.cowa_plan_kv(pf.pattern, N, Hkv, self.bm_kv, self.bn_kv)
        self.nnz_kv = len(col)
        self.rp_kv = torch.from_numpy(rp).cuda()
        self.col_kv = torch.from_numpy(col if len(col) else np.zeros(1, np.int32)).cuda()
        self.fl_kv = torch.from_numpy(fl if len(fl) else np.zeros(1, np.uint8)).cuda()
        # the workspace needs no initialisation: start it as NaN bytes
        self.ws = torch.full((C.cowa_bwd_workspace_size(pf.pattern, B, Hq, Hkv, N),), 0xFF,
                             dtype=torch.uint8, device="cuda")
        gdt = torch.float32 if g_dtype == "f32" else torch.bfloat16
        self.dq = torch.full((B, N, Hq, d), float("nan"), dtype=gdt, device="cuda")
        self.dk = torch.full((B, N, Hkv, d), float("nan"), dtype=gdt, device="cuda")
        self.dv = torch.full((B, N, Hkv, d), float("nan"), dtype=gdt, device="cuda")

    def run_bwd(self, stream=None):
        pf = self.pf
        C.cowa_bwd(pf.pattern, pf.rp, pf.col, pf.fl, pf.nnz, pf.bm, pf.bn, self.rp_kv,
                   self.col_kv, self.fl_kv, self.nnz_kv, self.bm_kv, self.bn_kv, pf.q, pf.k,
                   pf.v, pf.o, self.do, pf.lse, self.dq, self.dk, self.dv, pf.scale, self.ws,
                   stream)

    def run(self):
        self.pf.run()
        self.run_bwd()

    def set_oracle_forward(self):
        """Use the oracle's O and LSE (fp64 rounded to fp32) as the backward's
        forward inputs, so that only the backward kernels' rounding remains."""
        import torch
        pf = self.pf
        o, lse = pf.oracle()
        pf.o = torch.from_numpy(o.astype(np.float32)).cuda()
        pf.lse = torch.from_numpy(lse.astype(np.float32)).cuda()

    def result(self):
        import torch
        torch.cuda.synchronize()
        return (self.dq.float().cpu().numpy(), self.dk.float().cpu().numpy(),
                self.dv.float().cpu().numpy())

    def dout(self):
        return W.bf16_bits_to_f32(self.do_bits)

    def oracle_full(self):
        x = self.pf.x
        return O.attention_backward(x.q(), x.k(), x.v(), self.dout(), self.pf.opattern,
                                    self.pf.scale, magnitudes=True)

    def oracle_rows(self, rows, heads=None):
        x = self.pf.x
        return O.backward_rows_dq(x.q(), x.k(), x.v(), self.dout(), self.pf.opattern,
                                  self.pf.scale, rows, heads, magnitudes=True)

    def oracle_keys(self, keys, heads_kv=None):
        x = self.pf.x
        return O.backward_keys_dkdv(x.q(), x.k(), x.v(), self.dout(), self.pf.opattern,
                                    self.pf.scale, keys, heads_kv, magnitudes=True)
