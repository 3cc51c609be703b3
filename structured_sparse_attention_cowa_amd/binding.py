"""ctypes binding of libcowa (include/cowa.h): argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are
torch tensors on the GPU (torch supplies device memory and streams); the work
itself runs in the library's HIP kernels.  There is no fallback: if the
library is not built, load() raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcowa.so")

COWA_OK = 0
COWA_ERR_INVALID_ARG = 1
COWA_ERR_UNSUPPORTED = 2
COWA_ERR_WORKSPACE = 3
COWA_ERR_PLAN_MISMATCH = 4
COWA_ERR_HIP = 5
COWA_ERR_CAPACITY = 6
COWA_ERR_SCRATCH_LIMIT = 7
COWA_DECODE_SCRATCH_BYTES = 32 << 20
COWA_MODE_COWA = 0
COWA_MODE_CAUSAL = 1
COWA_MODE_SINK_LOCAL = 2
COWA_DTYPE_BF16 = 0
COWA_DTYPE_F32 = 1

EXPORTED = ("cowa_status_str", "cowa_band_length", "cowa_fwd_block_sizes", "cowa_plan_size",
            "cowa_plan", "cowa_fwd", "cowa_decode_workspace_size", "cowa_decode",
            "cowa_bwd_block_sizes", "cowa_plan_kv_size", "cowa_plan_kv",
            "cowa_bwd_workspace_size", "cowa_bwd", "cowa_bwd_varlen", "cowa_kv_window_rows",
            "cowa_kv_window_fill", "cowa_kv_window_append", "cowa_decode_window",
            "cowa_fwd_varlen", "cowa_visible_ranges", "cowa_decode_noalloc",
            "cowa_fwd_workspace_size")


class CowaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {cowa_status_str(status)} (status {status})")


class cowa_pattern(ctypes.Structure):
    _fields_ = [("n_ctx", ctypes.c_int32), ("sink", ctypes.c_int32), ("window", ctypes.c_int32),
                ("band", ctypes.c_int32), ("h_kv_global", ctypes.c_int32),
                ("kv_head_offset", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("n_bands", ctypes.c_int32)]


def make_pattern(n_ctx, sink, window, band=0, h_kv_global=1, kv_head_offset=0,
                 mode=COWA_MODE_COWA, n_bands=0) -> cowa_pattern:
    return cowa_pattern(n_ctx, sink, window, band, h_kv_global, kv_head_offset, mode, n_bands)


_lib = None


def load():
    """Load libcowa.so from the package directory (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libcowa.so not built at {LIB_PATH}; run "
                           "python -m structured_sparse_attention_cowa_amd.build")
    # torch ships its own HIP runtime (same soname as the system one).  Loading
    # torch first makes libcowa bind to that runtime, so device pointers and
    # stream handles from torch are valid inside the library.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    _check_single_hip_runtime()
    P = ctypes.POINTER
    i32, i64, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    pat = P(cowa_pattern)
    lib.cowa_status_str.restype = ctypes.c_char_p
    lib.cowa_status_str.argtypes = [ctypes.c_int]
    lib.cowa_band_length.restype = i32
    lib.cowa_band_length.argtypes = [pat]
    lib.cowa_fwd_block_sizes.restype = ctypes.c_int
    lib.cowa_fwd_block_sizes.argtypes = [i32, P(i32), P(i32)]
    lib.cowa_plan_size.restype = ctypes.c_int
    lib.cowa_plan_size.argtypes = [pat, i32, i32, i32, i32, P(i64)]
    lib.cowa_plan.restype = ctypes.c_int
    lib.cowa_plan.argtypes = [pat, i32, i32, i32, i32, vp, vp, vp, i64]
    lib.cowa_fwd.restype = ctypes.c_int
    lib.cowa_fwd.argtypes = [pat, vp, vp, vp, i64, i32, i32, vp, vp, vp, vp, i32, vp,
                             i32, i32, i32, i32, i32, P(i64), f32, vp, ctypes.c_size_t, vp]
    lib.cowa_fwd_workspace_size.restype = ctypes.c_int
    lib.cowa_fwd_workspace_size.argtypes = [i32, i32, i32, i32, P(ctypes.c_size_t)]
    lib.cowa_decode_workspace_size.restype = ctypes.c_int
    lib.cowa_decode_workspace_size.argtypes = [pat, i32, i32, i32, i32, i32, P(ctypes.c_size_t)]
    lib.cowa_decode.restype = ctypes.c_int
    lib.cowa_decode.argtypes = [pat, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32,
                                P(i64), f32, vp, ctypes.c_size_t, vp]
    lib.cowa_bwd_block_sizes.restype = ctypes.c_int
    lib.cowa_bwd_block_sizes.argtypes = [i32, P(i32), P(i32)]
    lib.cowa_plan_kv_size.restype = ctypes.c_int
    lib.cowa_plan_kv_size.argtypes = [pat, i32, i32, i32, i32, P(i64)]
    lib.cowa_plan_kv.restype = ctypes.c_int
    lib.cowa_plan_kv.argtypes = [pat, i32, i32, i32, i32, vp, vp, vp, i64]
    lib.cowa_bwd_workspace_size.restype = ctypes.c_int
    lib.cowa_bwd_workspace_size.argtypes = [pat, i32, i32, i32, i32, P(ctypes.c_size_t)]
    lib.cowa_bwd.restype = ctypes.c_int
    lib.cowa_bwd.argtypes = [pat, vp, vp, vp, i64, i32, i32, vp, vp, vp, i64, i32, i32,
                             vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, i32,
                             i32, i32, i32, i32, i32, P(i64), f32, vp, ctypes.c_size_t, vp]
    lib.cowa_bwd_varlen.restype = ctypes.c_int
    lib.cowa_bwd_varlen.argtypes = [pat, vp, vp, vp, i64, i32, i32, vp, vp, vp, i64, i32, i32,
                                    vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, i32,
                                    vp, i32, i32, i32, i32, i32, i32, P(i64), f32, vp,
                                    ctypes.c_size_t, vp]
    lib.cowa_kv_window_rows.restype = ctypes.c_int
    lib.cowa_kv_window_rows.argtypes = [pat, i32, i32, vp, P(i64)]
    lib.cowa_kv_window_fill.restype = ctypes.c_int
    lib.cowa_kv_window_fill.argtypes = [pat, vp, vp, vp, vp, vp, i32, i32, i32, i32, P(i64), vp]
    lib.cowa_kv_window_append.restype = ctypes.c_int
    lib.cowa_kv_window_append.argtypes = [pat, vp, vp, vp, vp, vp, i32, i32, i32, i32, P(i64),
                                          vp]
    lib.cowa_decode_window.restype = ctypes.c_int
    lib.cowa_decode_window.argtypes = [pat, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32,
                                       P(i64), f32, vp, ctypes.c_size_t, vp]
    lib.cowa_decode_noalloc.restype = ctypes.c_int
    lib.cowa_decode_noalloc.argtypes = [pat, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32,
                                        i32, P(i64), f32, vp]
    lib.cowa_visible_ranges.restype = ctypes.c_int
    lib.cowa_visible_ranges.argtypes = [pat, i32, i32, P(i32), P(i32)]
    lib.cowa_fwd_varlen.restype = ctypes.c_int
    lib.cowa_fwd_varlen.argtypes = [pat, vp, vp, vp, i64, i32, i32, vp, vp, vp, vp, i32, vp, vp,
                                    i32, i32, i32, i32, i32, i32, P(i64), f32, vp,
                                    ctypes.c_size_t, vp]
    _lib = lib
    return lib


def _check_single_hip_runtime():
    """Two HIP runtimes in one process cannot share streams or allocations."""
    try:
        maps = open("/proc/self/maps").read()
    except OSError:
        return
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    if len(libs) > 1:
        raise RuntimeError(f"two HIP runtimes are loaded in this process: {sorted(libs)}")


def _check(st: int, where: str):
    if st != COWA_OK:
        raise CowaError(st, where)


def cowa_status_str(status: int) -> str:
    return load().cowa_status_str(int(status)).decode()


def cowa_band_length(p: cowa_pattern) -> int:
    return int(load().cowa_band_length(ctypes.byref(p)))


def cowa_fwd_block_sizes(d: int):
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(load().cowa_fwd_block_sizes(d, ctypes.byref(bm), ctypes.byref(bn)),
           "cowa_fwd_block_sizes")
    return bm.value, bn.value


def cowa_visible_ranges(p: cowa_pattern, h: int, t: int):
    """[(lo, hi)] * 3: sink, long-range window and local window of row t."""
    lo, hi = (ctypes.c_int32 * 3)(), (ctypes.c_int32 * 3)()
    _check(load().cowa_visible_ranges(ctypes.byref(p), h, t, lo, hi), "cowa_visible_ranges")
    return [(lo[i], hi[i]) for i in range(3)]


def cowa_plan_size(p: cowa_pattern, n: int, h_kv_local: int, block_m: int, block_n: int) -> int:
    nnz = ctypes.c_int64()
    _check(load().cowa_plan_size(ctypes.byref(p), n, h_kv_local, block_m, block_n,
                                 ctypes.byref(nnz)), "cowa_plan_size")
    return nnz.value


def cowa_plan(p: cowa_pattern, n: int, h_kv_local: int, block_m: int, block_n: int):
    """Returns (row_ptr int32, col int32, flags uint8) host arrays."""
    nnz = cowa_plan_size(p, n, h_kv_local, block_m, block_n)
    nqt = -(-n // block_m)
    row_ptr = np.zeros(h_kv_local * nqt + 1, dtype=np.int32)
    col = np.zeros(max(nnz, 1), dtype=np.int32)
    flags = np.zeros(max(nnz, 1), dtype=np.uint8)
    _check(load().cowa_plan(ctypes.byref(p), n, h_kv_local, block_m, block_n,
                            row_ptr.ctypes.data, col.ctypes.data, flags.ctypes.data, nnz),
           "cowa_plan")
    return row_ptr, col[:nnz], flags[:nnz]


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _strides(t, ndim_keep):
    if t.stride(-1) != 1:
        raise ValueError("the last (head-dim) axis must be contiguous")
    return list(t.stride()[:ndim_keep])


def _o_dtype(o):
    import torch
    if o.dtype == torch.bfloat16:
        return COWA_DTYPE_BF16
    if o.dtype == torch.float32:
        return COWA_DTYPE_F32
    raise TypeError("o must be bfloat16 or float32")


def cowa_fwd_workspace_size(B: int, N: int, H_kv_local: int, d: int) -> int:
    n = ctypes.c_size_t()
    _check(load().cowa_fwd_workspace_size(B, N, H_kv_local, d, ctypes.byref(n)),
           "cowa_fwd_workspace_size")
    return n.value


def _fwd_workspace(workspace, B, N, Hkv, d, device):
    """(pointer, bytes) of the caller's workspace, or of a new uint8 device
    tensor of the required size when workspace is None (callers that must not
    allocate per call, such as graph capture, pass their own)."""
    import torch
    if workspace is None:
        workspace = torch.empty(cowa_fwd_workspace_size(B, N, Hkv, d), dtype=torch.uint8,
                                device=device)
    return workspace, workspace.data_ptr(), workspace.numel() * workspace.element_size()


def cowa_fwd(p: cowa_pattern, row_ptr, col, flags, nnz: int, block_m: int, block_n: int,
             q, k, v, o, lse, softmax_scale: float, stream=None, workspace=None):
    """Prefill forward.  q/o [B,N,H_q,d], k/v [B,N,H_kv,d] (bf16), lse [B,H_q,N] fp32;
    workspace: a device tensor of at least cowa_fwd_workspace_size(B, N, H_kv, d)
    bytes, or None for a new one."""
    import torch
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q, k, v must be bfloat16 GPU tensors")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, N, Hkv, d) or tuple(v.shape) != (B, N, Hkv, d):
        raise ValueError("k and v must be [B, N, H_kv, d] matching q")
    if tuple(o.shape) != (B, N, Hq, d) or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("o must be [B, N, H_q, d] and lse [B, H_q, N]")
    strides = (ctypes.c_int64 * 12)(*(_strides(q, 3) + _strides(k, 3) + _strides(v, 3)
                                      + _strides(o, 3)))
    ws, ws_ptr, ws_bytes = _fwd_workspace(workspace, B, N, Hkv, d, q.device)
    st = load().cowa_fwd(ctypes.byref(p), row_ptr.data_ptr(), col.data_ptr(), flags.data_ptr(),
                         nnz, block_m, block_n, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                         o.data_ptr(), _o_dtype(o), lse.data_ptr(), B, N, Hq, Hkv, d,
                         strides, float(softmax_scale), ws_ptr, ws_bytes, _stream_ptr(stream))
    _check(st, "cowa_fwd")


def cowa_decode_workspace_size(p: cowa_pattern, B: int, H_q: int, H_kv_local: int, d: int,
                               n_max: int) -> int:
    n = ctypes.c_size_t()
    _check(load().cowa_decode_workspace_size(ctypes.byref(p), B, H_q, H_kv_local, d, n_max,
                                             ctypes.byref(n)), "cowa_decode_workspace_size")
    return n.value


def cowa_decode(p: cowa_pattern, q, k_cache, v_cache, cache_seqlens, o, lse,
                softmax_scale: float, workspace, stream=None):
    """Decode.  q/o [B,H_q,d]; caches [B,n_max,H_kv,d] bf16; seqlens int32[B]; lse [B,H_q]."""
    import torch
    for t in (q, k_cache, v_cache):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q and caches must be bfloat16 GPU tensors")
    if cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda:
        raise TypeError("cache_seqlens must be an int32 GPU tensor")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    B, Hq, d = q.shape
    _, n_max, Hkv, _ = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[0] != B:
        raise ValueError("caches must be [B, n_max, H_kv, d]")
    if tuple(o.shape) != (B, Hq, d) or tuple(lse.shape) != (B, Hq):
        raise ValueError("o must be [B, H_q, d] and lse [B, H_q]")
    strides = (ctypes.c_int64 * 10)(*(_strides(q, 2) + _strides(k_cache, 3)
                                      + _strides(v_cache, 3) + _strides(o, 2)))
    st = load().cowa_decode(ctypes.byref(p), q.data_ptr(), k_cache.data_ptr(),
                            v_cache.data_ptr(), cache_seqlens.data_ptr(), o.data_ptr(),
                            _o_dtype(o), lse.data_ptr(), B, Hq, Hkv, d, n_max, strides,
                            float(softmax_scale), workspace.data_ptr(), workspace.numel()
                            * workspace.element_size(), _stream_ptr(stream))
    _check(st, "cowa_decode")


def cowa_decode_noalloc(p: cowa_pattern, q, k_cache, v_cache, cache_seqlens, o, lse,
                        softmax_scale: float, stream=None):
    """cowa_decode with the library's own scratch (no workspace argument);
    tensors as cowa_decode.  Marshalling only: allocates nothing."""
    import torch
    for t in (q, k_cache, v_cache):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q and caches must be bfloat16 GPU tensors")
    if cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda:
        raise TypeError("cache_seqlens must be an int32 GPU tensor")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    B, Hq, d = q.shape
    _, n_max, Hkv, _ = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[0] != B:
        raise ValueError("caches must be [B, n_max, H_kv, d]")
    if tuple(o.shape) != (B, Hq, d) or tuple(lse.shape) != (B, Hq):
        raise ValueError("o must be [B, H_q, d] and lse [B, H_q]")
    strides = (ctypes.c_int64 * 10)(*(_strides(q, 2) + _strides(k_cache, 3)
                                      + _strides(v_cache, 3) + _strides(o, 2)))
    st = load().cowa_decode_noalloc(ctypes.byref(p), q.data_ptr(), k_cache.data_ptr(),
                                    v_cache.data_ptr(), cache_seqlens.data_ptr(), o.data_ptr(),
                                    _o_dtype(o), lse.data_ptr(), B, Hq, Hkv, d, n_max, strides,
                                    float(softmax_scale), _stream_ptr(stream))
    _check(st, "cowa_decode_noalloc")


def cowa_bwd_block_sizes(d: int):
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(load().cowa_bwd_block_sizes(d, ctypes.byref(bm), ctypes.byref(bn)),
           "cowa_bwd_block_sizes")
    return bm.value, bn.value


def cowa_plan_kv_size(p: cowa_pattern, n: int, h_kv_local: int, block_m: int,
                      block_n: int) -> int:
    nnz = ctypes.c_int64()
    _check(load().cowa_plan_kv_size(ctypes.byref(p), n, h_kv_local, block_m, block_n,
                                    ctypes.byref(nnz)), "cowa_plan_kv_size")
    return nnz.value


def cowa_plan_kv(p: cowa_pattern, n: int, h_kv_local: int, block_m: int, block_n: int):
    """Key-major lists: (row_ptr int32 [h_kv_local * nkt + 1], col int32, flags uint8)."""
    nnz = cowa_plan_kv_size(p, n, h_kv_local, block_m, block_n)
    nkt = -(-n // block_n)
    row_ptr = np.zeros(h_kv_local * nkt + 1, dtype=np.int32)
    col = np.zeros(max(nnz, 1), dtype=np.int32)
    flags = np.zeros(max(nnz, 1), dtype=np.uint8)
    _check(load().cowa_plan_kv(ctypes.byref(p), n, h_kv_local, block_m, block_n,
                               row_ptr.ctypes.data, col.ctypes.data, flags.ctypes.data, nnz),
           "cowa_plan_kv")
    return row_ptr, col[:nnz], flags[:nnz]


def cowa_bwd_workspace_size(p: cowa_pattern, B: int, H_q: int, H_kv_local: int, N: int) -> int:
    n = ctypes.c_size_t()
    _check(load().cowa_bwd_workspace_size(ctypes.byref(p), B, H_q, H_kv_local, N,
                                          ctypes.byref(n)), "cowa_bwd_workspace_size")
    return n.value


def cowa_bwd(p: cowa_pattern, row_ptr, col, flags, nnz: int, block_m: int, block_n: int,
             row_ptr_kv, col_kv, flags_kv, nnz_kv: int, block_m_kv: int, block_n_kv: int,
             q, k, v, o, dout, lse, dq, dk, dv, softmax_scale: float, workspace, stream=None):
    """Backward.  q/dout/dq [B,N,H_q,d], k/v/dk/dv [B,N,H_kv,d], o the forward
    output (bf16 or fp32), lse [B,H_q,N] fp32; dq, dk, dv share one dtype."""
    import torch
    for t in (q, k, v, dout):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q, k, v, dout must be bfloat16 GPU tensors")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    if not (dq.dtype == dk.dtype == dv.dtype):
        raise TypeError("dq, dk, dv must share one dtype")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    for t in (k, v, dk, dv):
        if tuple(t.shape) != (B, N, Hkv, d):
            raise ValueError("k, v, dk, dv must be [B, N, H_kv, d]")
    for t in (o, dout, dq):
        if tuple(t.shape) != (B, N, Hq, d):
            raise ValueError("o, dout, dq must be [B, N, H_q, d]")
    if tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be [B, H_q, N]")
    strides = (ctypes.c_int64 * 24)(*(sum((_strides(t, 3) for t in (q, k, v, o, dout, dq, dk,
                                                                       dv)), [])))
    st = load().cowa_bwd(ctypes.byref(p), row_ptr.data_ptr(), col.data_ptr(), flags.data_ptr(),
                         nnz, block_m, block_n, row_ptr_kv.data_ptr(), col_kv.data_ptr(),
                         flags_kv.data_ptr(), nnz_kv, block_m_kv, block_n_kv, q.data_ptr(),
                         k.data_ptr(), v.data_ptr(), o.data_ptr(), _o_dtype(o),
                         dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                         dv.data_ptr(), _o_dtype(dq), B, N, Hq, Hkv, d, strides,
                         float(softmax_scale), workspace.data_ptr(),
                         workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    _check(st, "cowa_bwd")


def cowa_bwd_varlen(p: cowa_pattern, row_ptr, col, flags, nnz: int, block_m: int, block_n: int,
                    row_ptr_kv, col_kv, flags_kv, nnz_kv: int, block_m_kv: int,
                    block_n_kv: int, q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens,
                    max_seqlen: int, softmax_scale: float, workspace, stream=None):
    """Packed backward: q/o/dout/dq [T, H_q, d], k/v/dk/dv [T, H_kv, d], lse [H_q, T]
    (cowa_fwd_varlen's), cu_seqlens int32 [n_seqs + 1] on the device; both plans
    are built for n = max_seqlen."""
    import torch
    for t in (q, k, v, dout):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q, k, v, dout must be bfloat16 GPU tensors")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
        raise TypeError("cu_seqlens must be an int32 GPU tensor")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    if not (dq.dtype == dk.dtype == dv.dtype):
        raise TypeError("dq, dk, dv must share one dtype")
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    for t in (k, v, dk, dv):
        if tuple(t.shape) != (T, Hkv, d):
            raise ValueError("k, v, dk, dv must be [T, H_kv, d]")
    for t in (o, dout, dq):
        if tuple(t.shape) != (T, Hq, d):
            raise ValueError("o, dout, dq must be [T, H_q, d]")
    if tuple(lse.shape) != (Hq, T):
        raise ValueError("lse must be [H_q, T]")
    strides = (ctypes.c_int64 * 16)(*(sum((_strides(t, 2) for t in (q, k, v, o, dout, dq, dk,
                                                                       dv)), [])))
    st = load().cowa_bwd_varlen(ctypes.byref(p), row_ptr.data_ptr(), col.data_ptr(),
                                flags.data_ptr(), nnz, block_m, block_n, row_ptr_kv.data_ptr(),
                                col_kv.data_ptr(), flags_kv.data_ptr(), nnz_kv, block_m_kv,
                                block_n_kv, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                o.data_ptr(), _o_dtype(o), dout.data_ptr(), lse.data_ptr(),
                                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _o_dtype(dq),
                                cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, max_seqlen, T, Hq,
                                Hkv, d, strides, float(softmax_scale), workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(),
                                _stream_ptr(stream))
    _check(st, "cowa_bwd_varlen")


def cowa_kv_window_rows(p: cowa_pattern, h_kv_local: int, n_max: int):
    """(rows per local head as an int32 array, rows per sequence)."""
    rows = np.zeros(h_kv_local, dtype=np.int32)
    total = ctypes.c_int64()
    _check(load().cowa_kv_window_rows(ctypes.byref(p), h_kv_local, n_max, rows.ctypes.data,
                                      ctypes.byref(total)), "cowa_kv_window_rows")
    return rows, total.value


def _win_stride(t):
    assert t.dim() == 3 and t.stride(2) == 1 and t.stride(1) == t.shape[2], \
        "windowed caches are [B, rows, d] with contiguous rows"
    return t.stride(0)


def cowa_kv_window_fill(p: cowa_pattern, k_cache, v_cache, cache_seqlens, k_win, v_win,
                        stream=None):
    """Pack full caches [B, n_max, H_kv, d] into windowed caches [B, rows, d]."""
    B, n_max, Hkv, d = k_cache.shape
    strides = (ctypes.c_int64 * 8)(*(_strides(k_cache, 3) + _strides(v_cache, 3)
                                     + [_win_stride(k_win), _win_stride(v_win)]))
    _check(load().cowa_kv_window_fill(ctypes.byref(p), k_cache.data_ptr(), v_cache.data_ptr(),
                                      cache_seqlens.data_ptr(), k_win.data_ptr(),
                                      v_win.data_ptr(), B, Hkv, d, n_max, strides,
                                      _stream_ptr(stream)), "cowa_kv_window_fill")


def cowa_kv_window_append(p: cowa_pattern, k_new, v_new, cache_seqlens, k_win, v_win, n_max,
                          stream=None):
    """Write k_new, v_new [B, H_kv, d] at position cache_seqlens - 1."""
    B, Hkv, d = k_new.shape
    strides = (ctypes.c_int64 * 6)(*(_strides(k_new, 2) + _strides(v_new, 2)
                                     + [_win_stride(k_win), _win_stride(v_win)]))
    _check(load().cowa_kv_window_append(ctypes.byref(p), k_new.data_ptr(), v_new.data_ptr(),
                                        cache_seqlens.data_ptr(), k_win.data_ptr(),
                                        v_win.data_ptr(), B, Hkv, d, n_max, strides,
                                        _stream_ptr(stream)), "cowa_kv_window_append")


def cowa_decode_window(p: cowa_pattern, q, k_win, v_win, cache_seqlens, o, lse, h_kv_local,
                       n_max, softmax_scale: float, workspace, stream=None):
    """Decode against windowed caches [B, rows, d]; q/o [B, H_q, d], lse [B, H_q]."""
    import torch
    if q.dtype != torch.bfloat16 or k_win.dtype != torch.bfloat16:
        raise TypeError("q and windowed caches must be bfloat16")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    B, Hq, d = q.shape
    strides = (ctypes.c_int64 * 6)(*(_strides(q, 2) + [_win_stride(k_win), _win_stride(v_win)]
                                     + _strides(o, 2)))
    _check(load().cowa_decode_window(ctypes.byref(p), q.data_ptr(), k_win.data_ptr(),
                                     v_win.data_ptr(), cache_seqlens.data_ptr(), o.data_ptr(),
                                     _o_dtype(o), lse.data_ptr(), B, Hq, h_kv_local, d, n_max,
                                     strides, float(softmax_scale), workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(),
                                     _stream_ptr(stream)), "cowa_decode_window")


def cowa_fwd_varlen(p: cowa_pattern, row_ptr, col, flags, nnz: int, block_m: int, block_n: int,
                    q, k, v, o, lse, cu_seqlens, max_seqlen: int, softmax_scale: float,
                    stream=None, workspace=None):
    """Packed prefill: q/o [T, H_q, d], k/v [T, H_kv, d], lse [H_q, T], cu_seqlens
    int32 [n_seqs + 1] on the device; the plan is built for n = max_seqlen;
    workspace as for cowa_fwd with B = n_seqs, N = max_seqlen."""
    import torch
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q, k, v must be bfloat16 GPU tensors")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
        raise TypeError("cu_seqlens must be an int32 GPU tensor")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if tuple(lse.shape) != (Hq, T) or tuple(o.shape) != (T, Hq, d):
        raise ValueError("o must be [T, H_q, d] and lse [H_q, T]")
    strides = (ctypes.c_int64 * 8)(*(_strides(q, 2) + _strides(k, 2) + _strides(v, 2)
                                     + _strides(o, 2)))
    ws, ws_ptr, ws_bytes = _fwd_workspace(workspace, cu_seqlens.numel() - 1, max_seqlen, Hkv,
                                          d, q.device)
    st = load().cowa_fwd_varlen(ctypes.byref(p), row_ptr.data_ptr(), col.data_ptr(),
                                flags.data_ptr(), nnz, block_m, block_n, q.data_ptr(),
                                k.data_ptr(), v.data_ptr(), o.data_ptr(), _o_dtype(o),
                                lse.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                                max_seqlen, T, Hq, Hkv, d, strides, float(softmax_scale),
                                ws_ptr, ws_bytes, _stream_ptr(stream))
    _check(st, "cowa_fwd_varlen")
