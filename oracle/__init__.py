"""CPU oracle for the CSA2 sparse-attention hot path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the benchmark's CPU-baseline leg, never by the product package.  The
arithmetic lives in ``oracle.c`` (plain C, double precision); this module only
marshals numpy arrays.  See ``oracle.c`` for the definitions and the passages
of the source pages each function follows.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build():
    """Compile liboracle.so with gcc (always rebuilds)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", LIB_PATH, os.path.join(_HERE, "oracle.c"), "-lm"]
    subprocess.check_call(cmd)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        _lib.oracle_e2m1.restype = ctypes.c_double
        _lib.oracle_e2m1.argtypes = [i32]
        _lib.oracle_e4m3.restype = ctypes.c_double
        _lib.oracle_e4m3.argtypes = [i32]
        _lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        _lib.oracle_e4m3_encode.argtypes = [f32]
        _lib.oracle_swa_append.argtypes = [P, P, P, i32, i32, i32, P, P]
        _lib.oracle_dequant_row.argtypes = [P, P, i32, P]
        _lib.oracle_fp4_quantize_row.argtypes = [P, i32, P, P]
        _lib.oracle_index_full.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, P, i32, i32, P]
        _lib.oracle_reindex.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, P]
        _lib.oracle_reindex_e4m3.argtypes = _lib.oracle_reindex.argtypes
        _lib.oracle_scores_e4m3.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P]
        _lib.oracle_index_full_ex.argtypes = [P, P, i32, P, P, P, i32, i32, i32, i32, i32, P, i32,
                                              i32, P, i32]
        _lib.oracle_attn_decode.argtypes = [P, P, P, P, P, i32, P, P, P, i32, i32, i32, i32, f32,
                                            P, P]
        _lib.oracle_attn_prefill.argtypes = [P, i64, P, P, P, i32, P, P, i32, i32, i32, i32, f32,
                                             P, P]
        _lib.oracle_scores.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P]
        _lib.oracle_set_threads.argtypes = [i32]
        _lib.oracle_max_threads.restype = i32
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def e2m1(code):
    return lib().oracle_e2m1(int(code))


def e4m3(byte):
    return lib().oracle_e4m3(int(byte))


def dequant_row(codes, scales, D):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    out = np.empty(D, np.float64)
    lib().oracle_dequant_row(_p(codes), _p(scales), D, _p(out))
    return out


def fp4_quantize_rows(x):
    """fp32 rows [R, D] -> (codes [R, D/2] u8, scales [R, D/16] u8)."""
    x = _c(x, np.float32)
    R, D = x.shape
    codes = np.zeros((R, D // 2), np.uint8)
    scales = np.zeros((R, D // 16), np.uint8)
    for r in range(R):
        lib().oracle_fp4_quantize_row(_p(x[r]), D, _p(codes[r]), _p(scales[r]))
    return codes, scales


def e4m3_encode(x):
    """fp32 values (any shape) -> E4M3FN bytes, element by element."""
    x = np.asarray(x, np.float32)
    f = lib().oracle_e4m3_encode
    return np.array([f(float(v)) for v in x.reshape(-1)], np.uint8).reshape(x.shape)


def swa_append(k_new, v_new, pos, swa_k, swa_v):
    """In place: token b's K/V rows [B, D] go to slot pos[b] mod W of the
    rings swa_k / swa_v [B, W, D] (u8, modified)."""
    k_new, v_new = _c(k_new, np.float32), _c(v_new, np.float32)
    pos = _c(pos, np.int64)
    assert swa_k.flags["C_CONTIGUOUS"] and swa_v.flags["C_CONTIGUOUS"]
    B, W, D = swa_k.shape
    lib().oracle_swa_append(_p(k_new), _p(v_new), _p(pos), B, D, W, _p(swa_k), _p(swa_v))


def set_threads(n):
    lib().oracle_set_threads(int(n))


def max_threads():
    return int(lib().oracle_max_threads())


def scores(qI, kI, seq_row_off, q_seq, q_nvis, q, Hi, Hk, Di):
    """Scores of query q; kI is an fp32 key cache or (uint8) E4M3FN key bytes."""
    qI = _c(qI, np.float32)
    kI, e4m3 = _keys(kI)
    seq_row_off, q_seq, q_nvis = _c(seq_row_off, np.int64), _c(q_seq, np.int32), _c(q_nvis, np.int32)
    out = np.empty(int(q_nvis[q]), np.float64)
    f = lib().oracle_scores_e4m3 if e4m3 else lib().oracle_scores
    f(_p(qI), _p(kI), _p(seq_row_off), _p(q_seq), _p(q_nvis), q, Hi, Hk, Di, _p(out))
    return out


def _keys(kI):
    """(pointer-ready array, e4m3?) for an fp32 key cache or a uint8 E4M3FN one."""
    if np.asarray(kI).dtype == np.uint8:
        return _c(kI, np.uint8), True
    return _c(kI, np.float32), False


def index_full(qI, kI, seq_row_off, q_seq, q_nvis, Hi, Hk, Di, topk, pool_blocks=0,
               block_size=8, block_rule="max"):
    """Returns (topk_idx [Q,topk] int32, pool [Q,pool_blocks] int32 or None).
    kI is an fp32 key cache or, as uint8, the compact E4M3FN key cache;
    block_rule "max" (the reading used) or "sum" (a variant) scores blocks."""
    qI = _c(qI, np.float32)
    kI, e4m3 = _keys(kI)
    seq_row_off, q_seq, q_nvis = _c(seq_row_off, np.int64), _c(q_seq, np.int32), _c(q_nvis, np.int32)
    Q = int(q_nvis.shape[0])
    idx = np.empty((Q, topk), np.int32)
    pool = np.empty((Q, pool_blocks), np.int32) if pool_blocks > 0 else None
    rule = {"max": 0, "sum": 1}[block_rule]
    rc = lib().oracle_index_full_ex(_p(qI), _p(kI), 1 if e4m3 else 0, _p(seq_row_off), _p(q_seq),
                                    _p(q_nvis), Q, Hi, Hk, Di, topk, _p(idx), pool_blocks,
                                    block_size, _p(pool), rule)
    if rc != 0:
        raise ValueError("oracle_index_full: bad argument")
    return idx, pool


def reindex(qI, kI, seq_row_off, q_seq, q_nvis, pool, block_size, Hi, Hk, Di, topk):
    """kI is an fp32 key cache or, as uint8, the compact E4M3FN key cache."""
    qI = _c(qI, np.float32)
    kI, e4m3 = _keys(kI)
    seq_row_off, q_seq, q_nvis = _c(seq_row_off, np.int64), _c(q_seq, np.int32), _c(q_nvis, np.int32)
    pool = _c(pool, np.int32)
    Q, P = pool.shape
    idx = np.empty((Q, topk), np.int32)
    f = lib().oracle_reindex_e4m3 if e4m3 else lib().oracle_reindex
    rc = f(_p(qI), _p(kI), _p(seq_row_off), _p(q_seq), _p(q_nvis), _p(pool), P, block_size, Q, Hi,
           Hk, Di, topk, _p(idx))
    if rc != 0:
        raise ValueError("oracle_reindex: bad argument")
    return idx


def attn_decode(q, kv_codes, kv_scales, seq_row_off, topk_idx, swa_k, swa_v, swa_len, scale,
                want_lse=True):
    """q [B,H,D] f32; topk_idx [B,topk]; swa_k/v [B,W,D] u8 -> (out [B,H,D], lse [B,H])."""
    q = _c(q, np.float32)
    kv_codes, kv_scales = _c(kv_codes, np.uint8), _c(kv_scales, np.uint8)
    seq_row_off, topk_idx = _c(seq_row_off, np.int64), _c(topk_idx, np.int32)
    swa_k, swa_v, swa_len = _c(swa_k, np.uint8), _c(swa_v, np.uint8), _c(swa_len, np.int32)
    B, H, D = q.shape
    topk = topk_idx.shape[1] if topk_idx.ndim == 2 else 0
    W = swa_k.shape[1]
    out = np.empty((B, H, D), np.float32)
    lse = np.empty((B, H), np.float32) if want_lse else None
    rc = lib().oracle_attn_decode(_p(q), _p(kv_codes), _p(kv_scales), _p(seq_row_off),
                                  _p(topk_idx), topk, _p(swa_k), _p(swa_v), _p(swa_len), W, B, H,
                                  D, float(scale), _p(out), _p(lse))
    if rc != 0:
        raise ValueError("oracle_attn_decode: bad argument")
    return out, lse


def attn_prefill(q, p0, kv_codes, kv_scales, topk_idx, swa_k, swa_v, W, scale, want_lse=True):
    """q [Qn,H,D]; topk_idx [Qn,topk]; swa_k/v [Qn+W-1,D] -> (out [Qn,H,D], lse [Qn,H])."""
    q = _c(q, np.float32)
    kv_codes, kv_scales = _c(kv_codes, np.uint8), _c(kv_scales, np.uint8)
    topk_idx = _c(topk_idx, np.int32)
    swa_k, swa_v = _c(swa_k, np.uint8), _c(swa_v, np.uint8)
    Qn, H, D = q.shape
    topk = topk_idx.shape[1]
    out = np.empty((Qn, H, D), np.float32)
    lse = np.empty((Qn, H), np.float32) if want_lse else None
    rc = lib().oracle_attn_prefill(_p(q), int(p0), _p(kv_codes), _p(kv_scales), _p(topk_idx), topk,
                                   _p(swa_k), _p(swa_v), W, Qn, H, D, float(scale), _p(out),
                                   _p(lse))
    if rc != 0:
        raise ValueError("oracle_attn_prefill: bad argument")
    return out, lse
