"""Builds tests/host_shim.cpp with g++ (the kernels' integer helpers compiled
for the host) and loads it with ctypes; used by the CPU tests."""

from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "structured_sparse_attention_cowa_amd", "csrc")

_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    out_dir = tempfile.mkdtemp(prefix="cowa_host_shim_")
    so = os.path.join(out_dir, "libcowa_host_shim.so")
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-Wall",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(HERE, "host_shim.cpp"), "-o", so]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host shim build failed:\n{r.stdout}{r.stderr}")
    lib = ctypes.CDLL(so)
    i32, i64, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    P32 = ctypes.POINTER(i32)
    lib.shim_row_visible_bits.restype = u64
    lib.shim_row_visible_bits.argtypes = [i32] * 7
    lib.shim_col_visible_bits.restype = u64
    lib.shim_col_visible_bits.argtypes = [i32] * 7
    lib.shim_row_ranges.restype = None
    lib.shim_row_ranges.argtypes = [i32] * 6 + [P32, P32]
    lib.shim_xcd_logical.restype = i32
    lib.shim_xcd_logical.argtypes = [i32, i32, i32]
    lib.shim_xcd_chunk.restype = i32
    lib.shim_xcd_chunk.argtypes = [i64, i64, i64]
    lib.shim_xcd_grid.restype = i64
    lib.shim_xcd_grid.argtypes = [i64, i32]
    lib.shim_swz_both.restype = i32
    lib.shim_swz_both.argtypes = [i32, i32]
    lib.shim_plain_offsets.restype = None
    lib.shim_plain_offsets.argtypes = [i32, i32, P32]
    lib.shim_tr_offsets.restype = None
    lib.shim_tr_offsets.argtypes = [i32, i32, P32]
    lib.shim_load_row.restype = i32
    lib.shim_load_row.argtypes = [i32, i32]
    lib.shim_load_col.restype = i32
    lib.shim_load_col.argtypes = [i32, i32]
    for name in ("shim_swz_tr8", "shim_tr16_position", "shim_hdm_load_row", "shim_hdm_load_chunk"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [i32]
    lib.shim_hdm_read_offsets.restype = None
    lib.shim_hdm_read_offsets.argtypes = [i32, i32, P32]
    _lib = lib
    return lib


def int_array(n):
    return (ctypes.c_int32 * n)()
