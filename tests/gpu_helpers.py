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
                 n_ctx=None, o_dtype="f32"):
        import torch
        self.x = x
        B, N, Hq, d = x.q_bits.shape
        Hkv = x.k_bits.shape[2]
        self.B, self.N, self.Hq, self.Hkv, self.d = B, N, Hq, Hkv, d
        self.pattern = C.make_pattern(n_ctx or N, sink, window, 0, h_kv_global, offset, mode)
        self.opattern = O.Pattern(n_ctx or N, sink, window, 0, h_kv_global, offset, mode)
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
        self.scale = 1.0 / np.sqrt(d)

    def run(self, stream=None):
        C.cowa_fwd(self.pattern, self.rp, self.col, self.fl, self.nnz, self.bm, self.bn,
                   self.q, self.k, self.v, self.o, self.lse, self.scale, stream)

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
