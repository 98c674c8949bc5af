"""Seeded synthetic inputs for the CSA2 hot path (shared by both sides).

Holds none of the method's arithmetic.  Integer-valued tensors (indexer
queries and keys, FP4 code bytes, power-of-two E4M3 scale bytes) come from the
counter hash in ``gen.h`` and can be produced on the host (``gen_host.c``) or
directly in device memory (``gen_dev.hip``) with identical values.  fp32
N(0,1) tensors come from numpy's ``default_rng([seed, tensor])``; window K/V
bytes are those normals rounded to E4M3FN by torch's CPU cast.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libgen_host.so")
DEV_LIB = os.path.join(_HERE, "libgen_dev.so")

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build():
    """Compile the host (gcc) and device (hipcc, gfx950) generator libraries."""
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                           "-o", HOST_LIB, os.path.join(_HERE, "gen_host.c")])
    subprocess.check_call(["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, "-o", DEV_LIB,
                           os.path.join(_HERE, "gen_dev.hip")])


_host = None
_dev = None


def host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise ImportError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        _host = ctypes.CDLL(HOST_LIB)
        u64, i32, P = ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p
        _host.gen_hash.restype = u64
        _host.gen_hash.argtypes = [u64, u64, u64]
        _host.gen_host_ints.argtypes = [u64, u64, u64, u64, i32, i32, P]
        _host.gen_host_fp4.argtypes = [u64, u64, u64, u64, P]
        _host.gen_host_pow2_scales.argtypes = [u64, u64, u64, u64, i32, i32, P]
        i64 = ctypes.c_int64
        _host.gen_host_ints_runs.argtypes = [u64, u64, P, i64, i64, i32, i32, P]
        _host.gen_host_fp4_runs.argtypes = [u64, u64, P, i64, i64, P]
        _host.gen_host_pow2_scales_runs.argtypes = [u64, u64, P, i64, i64, i32, i32, P]
    return _host


def dev():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise ImportError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        _dev = ctypes.CDLL(DEV_LIB)
        u64, i32, P = ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p
        for name in ("gen_dev_ints", "gen_dev_fp4", "gen_dev_pow2_scales"):
            getattr(_dev, name).restype = ctypes.c_int
        _dev.gen_dev_ints.argtypes = [u64, u64, u64, u64, i32, i32, P, P]
        _dev.gen_dev_fp4.argtypes = [u64, u64, u64, u64, P, P]
        _dev.gen_dev_pow2_scales.argtypes = [u64, u64, u64, u64, i32, i32, P, P]
    return _dev


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- host side

def host_ints(seed, tensor, start, count, lo=-8, hi=8):
    out = np.empty(int(count), np.float32)
    host().gen_host_ints(seed, tensor, int(start), int(count), lo, hi, _ptr(out))
    return out


def host_fp4(seed, tensor, start, count):
    out = np.empty(int(count), np.uint8)
    host().gen_host_fp4(seed, tensor, int(start), int(count), _ptr(out))
    return out


def host_pow2_scales(seed, tensor, start, count, kmin=-4, kmax=4):
    out = np.empty(int(count), np.uint8)
    host().gen_host_pow2_scales(seed, tensor, int(start), int(count), kmin, kmax, _ptr(out))
    return out


def _starts(starts):
    return np.ascontiguousarray(starts, dtype=np.int64)


def host_ints_runs(seed, tensor, starts, run, lo=-8, hi=8):
    """host_ints for runs of `run` elements starting at each of `starts`,
    concatenated."""
    st = _starts(starts)
    out = np.empty(st.size * int(run), np.float32)
    host().gen_host_ints_runs(seed, tensor, _ptr(st), st.size, int(run), lo, hi, _ptr(out))
    return out


def host_fp4_runs(seed, tensor, starts, run):
    st = _starts(starts)
    out = np.empty(st.size * int(run), np.uint8)
    host().gen_host_fp4_runs(seed, tensor, _ptr(st), st.size, int(run), _ptr(out))
    return out


def host_pow2_scales_runs(seed, tensor, starts, run, kmin=-4, kmax=4):
    st = _starts(starts)
    out = np.empty(st.size * int(run), np.uint8)
    host().gen_host_pow2_scales_runs(seed, tensor, _ptr(st), st.size, int(run), kmin, kmax,
                                     _ptr(out))
    return out


def normal_f32(seed, tensor, shape):
    return np.random.default_rng([seed, tensor]).standard_normal(shape, dtype=np.float32)


def kv_rows_f32(seed, tensor, rows, D, log2_lo=-30.0, log2_hi=14.0):
    """fp32 main-KV rows [rows, D] before quantisation: N(0,1) values, each run
    of 16 channels multiplied by its own 2^u with u uniform in
    [log2_lo, log2_hi), so that the groups span tiny, ordinary and huge
    magnitudes."""
    rng = np.random.default_rng([seed, tensor])
    g = rows * D // 16
    mag = np.exp2(rng.uniform(log2_lo, log2_hi, size=(g, 1))).astype(np.float32)
    x = rng.standard_normal((g, 16), dtype=np.float32) * mag
    return x.reshape(rows, D)


def e4m3_bytes(x):
    """Round fp32 values to E4M3FN bytes (torch CPU cast, nearest-even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# -------------------------------------------------------------- device side

def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what}: hip error {rc}")


def dev_ints(t, seed, tensor, start=0, lo=-8, hi=8, stream=0):
    """Fill the contiguous float32 device tensor t."""
    _check(dev().gen_dev_ints(seed, tensor, int(start), t.numel(), lo, hi,
                              ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(stream)),
           "gen_dev_ints")


def dev_fp4(t, seed, tensor, start=0, stream=0):
    _check(dev().gen_dev_fp4(seed, tensor, int(start), t.numel(), ctypes.c_void_p(t.data_ptr()),
                             ctypes.c_void_p(stream)), "gen_dev_fp4")


def dev_pow2_scales(t, seed, tensor, start=0, kmin=-4, kmax=4, stream=0):
    _check(dev().gen_dev_pow2_scales(seed, tensor, int(start), t.numel(), kmin, kmax,
                                     ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(stream)),
           "gen_dev_pow2_scales")
