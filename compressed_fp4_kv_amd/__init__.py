"""Python binding of the CSA2 hot-path library (libcsa2.so, include/csa2.h).

Argument marshalling only: every function takes torch device tensors (or
None), checks dtype / contiguity / device, passes raw pointers, the sizes and
the current HIP stream to the C entry point of the same name, and raises
``CSA2Error`` on a non-zero status.  All computation happens in the HIP
kernels of the library; there is no fallback path.  Importing this package
fails loudly when the library has not been built.
"""
import ctypes
import os

__all__ = [
    "CSA2Error", "lib", "csa2_index_full", "csa2_index_full_workspace_bytes", "csa2_reindex",
    "csa2_index_full_e4m3", "csa2_reindex_e4m3", "csa2_index_full_ex",
    "csa2_index_prefill_workspace_bytes", "csa2_index_prefill_workspace_bytes_ex",
    "csa2_sparse_attn_decode_layers", "csa2_decode_layers_workspace_bytes",
    "csa2_reindex_workspace_bytes", "csa2_sparse_attn_decode", "csa2_decode_workspace_bytes",
    "csa2_reindex_noalloc", "NOALLOC_MAX_CAND",
    "csa2_sparse_attn_prefill_chunk", "csa2_prefill_workspace_bytes", "csa2_kv_quantize_fp4",
    "csa2_swa_append", "profile_enable",
    "profile_read", "profile_reset", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

EXPORTED_SYMBOLS = [
    "csa2_status_str", "csa2_last_hip_error",
    "csa2_index_full_workspace_bytes", "csa2_index_prefill_workspace_bytes", "csa2_index_full",
    "csa2_reindex_workspace_bytes", "csa2_reindex",
    "csa2_decode_workspace_bytes", "csa2_sparse_attn_decode",
    "csa2_prefill_workspace_bytes", "csa2_sparse_attn_prefill_chunk",
    "csa2_profile_enable", "csa2_profile_read", "csa2_profile_reset",
    "csa2_debug_decode_tables",
    "csa2_debug_dequant_tables",
    "csa2_kv_quantize_fp4",
    "csa2_swa_append",
    "csa2_index_full_e4m3", "csa2_reindex_e4m3", "csa2_index_full_ex",
    "csa2_index_prefill_workspace_bytes_ex",
    "csa2_sparse_attn_decode_layers", "csa2_decode_layers_workspace_bytes",
    "csa2_reindex_noalloc",
]

NOALLOC_MAX_CAND = 2097152   # CSA2_NOALLOC_MAX_CAND

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(hipcc, gfx950); there is no non-HIP implementation")

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float

lib = ctypes.CDLL(LIB_PATH)
lib.csa2_status_str.restype = ctypes.c_char_p
lib.csa2_status_str.argtypes = [ctypes.c_int]
lib.csa2_last_hip_error.restype = ctypes.c_int
lib.csa2_index_full_workspace_bytes.restype = _SZ
lib.csa2_index_full_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32]
lib.csa2_index_full.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _I32,
                                _I32, _P, _P, _SZ, _P]
lib.csa2_index_full_e4m3.argtypes = lib.csa2_index_full.argtypes
lib.csa2_index_prefill_workspace_bytes.restype = _SZ
lib.csa2_index_prefill_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32]
lib.csa2_index_prefill_workspace_bytes_ex.restype = _SZ
lib.csa2_index_prefill_workspace_bytes_ex.argtypes = [_I32, _I32, _I32, _I32, _I32, _I32, _I32]
lib.csa2_index_full_ex.argtypes = [_P, _P, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                   _P, _I32, _I32, _P, _I32, _P, _SZ, _P]
lib.csa2_reindex_workspace_bytes.restype = _SZ
lib.csa2_reindex_workspace_bytes.argtypes = [_I32, _I32, _I32]
lib.csa2_reindex.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P,
                             _P, _SZ, _P]
lib.csa2_reindex_e4m3.argtypes = lib.csa2_reindex.argtypes
lib.csa2_reindex_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                     _I32, _P, _P]
lib.csa2_decode_workspace_bytes.restype = _SZ
lib.csa2_decode_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32]
lib.csa2_sparse_attn_decode.argtypes = [_P, _P, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32, _I32,
                                        _I32, _F32, _P, _P, _P, _SZ, _P]
lib.csa2_decode_layers_workspace_bytes.restype = _SZ
lib.csa2_decode_layers_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32, _I32]
lib.csa2_sparse_attn_decode_layers.argtypes = [_I32, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _I32,
                                               _I32, _I32, _I32, _F32, _P, _P, _P, _SZ, _P]
lib.csa2_prefill_workspace_bytes.restype = _SZ
lib.csa2_prefill_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32]
lib.csa2_sparse_attn_prefill_chunk.argtypes = [_P, _I64, _P, _P, _P, _I32, _P, _P, _I32, _I32,
                                               _I32, _I32, _F32, _P, _P, _P, _SZ, _P]
lib.csa2_profile_enable.argtypes = [ctypes.c_int]
lib.csa2_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                  ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)]
lib.csa2_debug_decode_tables.argtypes = [_P, _P, _P, _P, _P]
lib.csa2_debug_dequant_tables.argtypes = [_P, _P, _P]
lib.csa2_kv_quantize_fp4.argtypes = [_P, _I64, _I32, _P, _P, _P]
lib.csa2_swa_append.argtypes = [_P, _P, _P, _I32, _I32, _I32, _P, _P, _P]


class CSA2Error(RuntimeError):
    def __init__(self, status, where):
        msg = lib.csa2_status_str(status).decode()
        if status == 5:
            msg += f" (hipError {lib.csa2_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


def _check(status, where):
    if status != 0:
        raise CSA2Error(status, where)


def _ptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous tensor (None -> NULL)."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t, shape, name):
    """Raises ValueError unless tensor t (skipped when None) has `shape`; an
    entry of None matches any extent.  The kernels trust these extents, so a
    mismatch is refused here rather than read or written out of bounds."""
    if t is None:
        return
    got = tuple(t.shape)
    if len(got) != len(shape) or any(w is not None and g != w for g, w in zip(got, shape)):
        want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
        raise ValueError(f"{name}: expected shape {want}, got {list(got)}")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws, name="ws"), ws.numel() * ws.element_size()


def _dt():
    import torch
    return torch.float32, torch.int32, torch.int64, torch.uint8


# ------------------------------------------------------------------ indexer

def csa2_index_full_workspace_bytes(Q, max_nvis, topk, pool_blocks=0, block_size=8):
    return int(lib.csa2_index_full_workspace_bytes(Q, max_nvis, topk, pool_blocks, block_size))


def csa2_index_prefill_workspace_bytes(Q, max_nvis, topk, Hk, Di):
    return int(lib.csa2_index_prefill_workspace_bytes(Q, max_nvis, topk, Hk, Di))


def csa2_index_prefill_workspace_bytes_ex(Q, max_nvis, topk, pool_blocks, block_size, Hk, Di):
    return int(lib.csa2_index_prefill_workspace_bytes_ex(Q, max_nvis, topk, pool_blocks,
                                                         block_size, Hk, Di))


def _index_shapes(qI, kI, seq_row_off, q_seq, q_nvis, topk, topk_idx, pool_blocks,
                  pool_block_idx):
    Q, _, Di = qI.shape
    _expect(kI, (None, None, Di), "kI")
    _expect(seq_row_off, (None,), "seq_row_off")
    _expect(q_seq, (Q,), "q_seq")
    _expect(q_nvis, (Q,), "q_nvis")
    _expect(topk_idx, (Q, topk), "topk_idx")
    if pool_blocks > 0:
        _expect(pool_block_idx, (Q, pool_blocks), "pool_block_idx")


def _index_full(fn, kdt, qI, kI, seq_row_off, q_seq, q_nvis, max_nvis, topk, topk_idx,
                pool_blocks, block_size, pool_block_idx, ws, stream):
    f32, i32, i64, _ = _dt()
    Q, Hi, Di = qI.shape
    Hk = kI.shape[1]
    name = fn.__name__
    _index_shapes(qI, kI, seq_row_off, q_seq, q_nvis, topk, topk_idx, pool_blocks,
                  pool_block_idx)
    wp, wn = _ws(ws)
    _check(fn(
        _ptr(qI, f32, "qI"), _ptr(kI, kdt, "kI"), _ptr(seq_row_off, i64, "seq_row_off"),
        _ptr(q_seq, i32, "q_seq"), _ptr(q_nvis, i32, "q_nvis"), Q, Hi, Hk, Di, max_nvis, topk,
        _ptr(topk_idx, i32, "topk_idx"), pool_blocks, block_size,
        _ptr(pool_block_idx, i32, "pool_block_idx"), wp, wn, _stream(stream)), name)


def csa2_index_full(qI, kI, seq_row_off, q_seq, q_nvis, max_nvis, topk, topk_idx,
                    pool_blocks=0, block_size=8, pool_block_idx=None, ws=None, stream=None):
    """qI [Q,Hi,Di] f32; kI [rows,Hk,Di] f32; seq_row_off [S] i64; q_seq [Q] i32 or None;
    q_nvis [Q] i32; topk_idx [Q,topk] i32 out; pool_block_idx [Q,pool_blocks] i32 out."""
    _index_full(lib.csa2_index_full, _dt()[0], qI, kI, seq_row_off, q_seq, q_nvis, max_nvis,
                topk, topk_idx, pool_blocks, block_size, pool_block_idx, ws, stream)


def csa2_index_full_e4m3(qI, kI, seq_row_off, q_seq, q_nvis, max_nvis, topk, topk_idx,
                         pool_blocks=0, block_size=8, pool_block_idx=None, ws=None, stream=None):
    """As csa2_index_full with kI [rows,Hk,Di] u8 holding E4M3FN key bytes."""
    _index_full(lib.csa2_index_full_e4m3, _dt()[3], qI, kI, seq_row_off, q_seq, q_nvis,
                max_nvis, topk, topk_idx, pool_blocks, block_size, pool_block_idx, ws, stream)


BLOCK_RULES = {"max": 0, "sum": 1}


def csa2_index_full_ex(qI, kI, seq_row_off, q_seq, q_nvis, max_nvis, topk, topk_idx,
                       pool_blocks=0, block_size=8, pool_block_idx=None, block_rule="max",
                       ws=None, stream=None):
    """General Full-mode indexer: kI [rows,Hk,Di] f32 (CSA2_KEYS_F32) or u8 E4M3FN bytes
    (CSA2_KEYS_E4M3), the key format following kI's dtype; block_rule "max" or "sum"."""
    f32, i32, i64, u8 = _dt()
    if kI.dtype == f32:
        fmt = 0
    elif kI.dtype == u8:
        fmt = 1
    else:
        raise TypeError(f"kI: expected {f32} or {u8}, got {kI.dtype}")
    if block_rule not in BLOCK_RULES:
        raise ValueError(f"block_rule: {block_rule!r} is not one of {sorted(BLOCK_RULES)}")
    Q, Hi, Di = qI.shape
    Hk = kI.shape[1]
    _index_shapes(qI, kI, seq_row_off, q_seq, q_nvis, topk, topk_idx, pool_blocks,
                  pool_block_idx)
    wp, wn = _ws(ws)
    _check(lib.csa2_index_full_ex(
        _ptr(qI, f32, "qI"), _ptr(kI, kI.dtype, "kI"), fmt, _ptr(seq_row_off, i64, "seq_row_off"),
        _ptr(q_seq, i32, "q_seq"), _ptr(q_nvis, i32, "q_nvis"), Q, Hi, Hk, Di, max_nvis, topk,
        _ptr(topk_idx, i32, "topk_idx"), pool_blocks, block_size,
        _ptr(pool_block_idx, i32, "pool_block_idx"), BLOCK_RULES[block_rule], wp, wn,
        _stream(stream)), "csa2_index_full_ex")


def csa2_reindex_workspace_bytes(Q, pool_blocks, block_size):
    return int(lib.csa2_reindex_workspace_bytes(Q, pool_blocks, block_size))


def _reindex(fn, kdt, qI, kI, seq_row_off, q_seq, q_nvis, pool_block_idx, block_size, topk,
             topk_idx, ws, stream):
    f32, i32, i64, _ = _dt()
    Q, Hi, Di = qI.shape
    Hk = kI.shape[1]
    P = pool_block_idx.shape[1]
    _expect(kI, (None, None, Di), "kI")
    _expect(seq_row_off, (None,), "seq_row_off")
    _expect(q_seq, (Q,), "q_seq")
    _expect(q_nvis, (Q,), "q_nvis")
    _expect(pool_block_idx, (Q, P), "pool_block_idx")
    _expect(topk_idx, (Q, topk), "topk_idx")
    wp, wn = _ws(ws)
    _check(fn(
        _ptr(qI, f32, "qI"), _ptr(kI, kdt, "kI"), _ptr(seq_row_off, i64, "seq_row_off"),
        _ptr(q_seq, i32, "q_seq"), _ptr(q_nvis, i32, "q_nvis"),
        _ptr(pool_block_idx, i32, "pool_block_idx"), P, block_size, Q, Hi, Hk, Di, topk,
        _ptr(topk_idx, i32, "topk_idx"), wp, wn, _stream(stream)), fn.__name__)


def csa2_reindex(qI, kI, seq_row_off, q_seq, q_nvis, pool_block_idx, block_size, topk, topk_idx,
                 ws=None, stream=None):
    _reindex(lib.csa2_reindex, _dt()[0], qI, kI, seq_row_off, q_seq, q_nvis, pool_block_idx,
             block_size, topk, topk_idx, ws, stream)


def csa2_reindex_e4m3(qI, kI, seq_row_off, q_seq, q_nvis, pool_block_idx, block_size, topk,
                      topk_idx, ws=None, stream=None):
    """As csa2_reindex with kI [rows,Hk,Di] u8 holding E4M3FN key bytes."""
    _reindex(lib.csa2_reindex_e4m3, _dt()[3], qI, kI, seq_row_off, q_seq, q_nvis,
             pool_block_idx, block_size, topk, topk_idx, ws, stream)


# ---------------------------------------------------------------- attention

def csa2_reindex_noalloc(qI, kI, seq_row_off, q_seq, q_nvis, pool_block_idx, block_size, topk,
                         topk_idx, stream=None):
    """csa2_reindex without a workspace argument: the library's static
    per-device scratch (at most NOALLOC_MAX_CAND candidates per call) is used
    and nothing is allocated.  Calls that overlap on one GPU race."""
    f32, i32, i64, _ = _dt()
    Q, Hi, Di = qI.shape
    Hk = kI.shape[1]
    P = pool_block_idx.shape[1]
    _expect(kI, (None, None, Di), "kI")
    _expect(seq_row_off, (None,), "seq_row_off")
    _expect(q_seq, (Q,), "q_seq")
    _expect(q_nvis, (Q,), "q_nvis")
    _expect(pool_block_idx, (Q, P), "pool_block_idx")
    _expect(topk_idx, (Q, topk), "topk_idx")
    _check(lib.csa2_reindex_noalloc(
        _ptr(qI, f32, "qI"), _ptr(kI, f32, "kI"), _ptr(seq_row_off, i64, "seq_row_off"),
        _ptr(q_seq, i32, "q_seq"), _ptr(q_nvis, i32, "q_nvis"),
        _ptr(pool_block_idx, i32, "pool_block_idx"), P, block_size, Q, Hi, Hk, Di, topk,
        _ptr(topk_idx, i32, "topk_idx"), _stream(stream)), "csa2_reindex_noalloc")


def csa2_decode_workspace_bytes(B, H, D, topk, W):
    return int(lib.csa2_decode_workspace_bytes(B, H, D, topk, W))


def csa2_sparse_attn_decode(q, kv_codes, kv_scales, seq_row_off, topk_idx, swa_k, swa_v, swa_len,
                            softmax_scale, out, lse=None, ws=None, stream=None):
    """q [B,H,D] f32; kv_codes [rows,D/2] u8; kv_scales [rows,D/16] u8; topk_idx [B,topk] i32;
    swa_k/swa_v [B,W,D] u8; swa_len [B] i32; out [B,H,D] f32; lse [B,H] f32 or None."""
    f32, i32, i64, u8 = _dt()
    B, H, D = q.shape
    topk = topk_idx.shape[1] if topk_idx is not None else 0
    W = swa_k.shape[1]
    _attn_kv_shapes(kv_codes, kv_scales, D)
    _expect(seq_row_off, (B,), "seq_row_off")
    _expect(topk_idx, (B, topk), "topk_idx")
    _expect(swa_k, (B, W, D), "swa_k")
    _expect(swa_v, (B, W, D), "swa_v")
    _expect(swa_len, (B,), "swa_len")
    _expect(out, (B, H, D), "out")
    _expect(lse, (B, H), "lse")
    wp, wn = _ws(ws)
    _check(lib.csa2_sparse_attn_decode(
        _ptr(q, f32, "q"), _ptr(kv_codes, u8, "kv_codes"), _ptr(kv_scales, u8, "kv_scales"),
        _ptr(seq_row_off, i64, "seq_row_off"), _ptr(topk_idx, i32, "topk_idx"), topk,
        _ptr(swa_k, u8, "swa_k"), _ptr(swa_v, u8, "swa_v"), _ptr(swa_len, i32, "swa_len"), W, B,
        H, D, float(softmax_scale), _ptr(out, f32, "out"), _ptr(lse, f32, "lse"), wp, wn,
        _stream(stream)), "csa2_sparse_attn_decode")


def _attn_kv_shapes(kv_codes, kv_scales, D):
    _expect(kv_codes, (None, D // 2), "kv_codes")
    if kv_codes is not None:
        _expect(kv_scales, (kv_codes.shape[0], D // 16), "kv_scales")


def csa2_decode_layers_workspace_bytes(L, B, H, D, topk, W):
    return int(lib.csa2_decode_layers_workspace_bytes(L, B, H, D, topk, W))


def _ptr_array(tensors, dtype, name):
    """Host array of device pointers (ctypes) for a list of tensors or Nones."""
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        p = _ptr(t, dtype, f"{name}[{i}]")
        arr[i] = p.value if p is not None else None
    return arr


def csa2_sparse_attn_decode_layers(qs, kv_codes, kv_scales, seq_row_off, topk_idx, swa_ks, swa_vs,
                                   swa_len, softmax_scale, outs, lses=None, ws=None, stream=None):
    """A layer group sharing topk_idx and the main KV: qs / swa_ks / swa_vs / outs / lses are
    lists of L tensors, each as for csa2_sparse_attn_decode (lses may be None)."""
    f32, i32, i64, u8 = _dt()
    L = len(qs)
    B, H, D = qs[0].shape
    topk = topk_idx.shape[1] if topk_idx is not None else 0
    W = swa_ks[0].shape[1]
    for name, lst in (("swa_k", swa_ks), ("swa_v", swa_vs), ("out", outs)) + (
            (("lse", lses),) if lses is not None else ()):
        if len(lst) != L:
            raise ValueError(f"{name}: {len(lst)} tensors for {L} layers")
    for i in range(L):
        _expect(qs[i], (B, H, D), f"q[{i}]")
        _expect(swa_ks[i], (B, W, D), f"swa_k[{i}]")
        _expect(swa_vs[i], (B, W, D), f"swa_v[{i}]")
        _expect(outs[i], (B, H, D), f"out[{i}]")
        if lses is not None:
            _expect(lses[i], (B, H), f"lse[{i}]")
    _attn_kv_shapes(kv_codes, kv_scales, D)
    _expect(seq_row_off, (B,), "seq_row_off")
    _expect(topk_idx, (B, topk), "topk_idx")
    _expect(swa_len, (B,), "swa_len")
    wp, wn = _ws(ws)
    _check(lib.csa2_sparse_attn_decode_layers(
        L, _ptr_array(qs, f32, "q"), _ptr(kv_codes, u8, "kv_codes"),
        _ptr(kv_scales, u8, "kv_scales"), _ptr(seq_row_off, i64, "seq_row_off"),
        _ptr(topk_idx, i32, "topk_idx"), topk, _ptr_array(swa_ks, u8, "swa_k"),
        _ptr_array(swa_vs, u8, "swa_v"), _ptr(swa_len, i32, "swa_len"), W, B, H, D,
        float(softmax_scale), _ptr_array(outs, f32, "out"),
        _ptr_array(lses, f32, "lse") if lses is not None else None, wp, wn, _stream(stream)),
        "csa2_sparse_attn_decode_layers")


def csa2_prefill_workspace_bytes(Qn, H, D, topk, W):
    return int(lib.csa2_prefill_workspace_bytes(Qn, H, D, topk, W))


def csa2_sparse_attn_prefill_chunk(q, p0, kv_codes, kv_scales, topk_idx, swa_k, swa_v, W,
                                   softmax_scale, out, lse=None, ws=None, stream=None):
    """q [Qn,H,D] f32; topk_idx [Qn,topk] i32; swa_k/swa_v [Qn+W-1,D] u8; out [Qn,H,D]."""
    f32, i32, i64, u8 = _dt()
    Qn, H, D = q.shape
    topk = topk_idx.shape[1] if topk_idx is not None else 0
    _attn_kv_shapes(kv_codes, kv_scales, D)
    _expect(topk_idx, (Qn, topk), "topk_idx")
    if W > 0:
        _expect(swa_k, (Qn + W - 1, D), "swa_k")
        _expect(swa_v, (Qn + W - 1, D), "swa_v")
    _expect(out, (Qn, H, D), "out")
    _expect(lse, (Qn, H), "lse")
    wp, wn = _ws(ws)
    _check(lib.csa2_sparse_attn_prefill_chunk(
        _ptr(q, f32, "q"), int(p0), _ptr(kv_codes, u8, "kv_codes"),
        _ptr(kv_scales, u8, "kv_scales"), _ptr(topk_idx, i32, "topk_idx"), topk,
        _ptr(swa_k, u8, "swa_k"), _ptr(swa_v, u8, "swa_v"), W, Qn, H, D, float(softmax_scale),
        _ptr(out, f32, "out"), _ptr(lse, f32, "lse"), wp, wn, _stream(stream)),
        "csa2_sparse_attn_prefill_chunk")


# ---------------------------------------------------------------- KV writer

def csa2_kv_quantize_fp4(x, codes, scales, stream=None):
    """x [rows, D] f32 (D % 16 == 0) -> codes [rows, D/2] u8 (even channel in
    the low nibble), scales [rows, D/16] u8 (E4M3)."""
    f32, _, _, u8 = _dt()
    rows, D = x.shape
    if tuple(codes.shape) != (rows, D // 2) or tuple(scales.shape) != (rows, D // 16):
        raise ValueError(f"codes {tuple(codes.shape)} / scales {tuple(scales.shape)} do not "
                         f"match x {tuple(x.shape)}")
    _check(lib.csa2_kv_quantize_fp4(_ptr(x, f32, "x"), rows, D, _ptr(codes, u8, "codes"),
                                    _ptr(scales, u8, "scales"), _stream(stream)),
           "csa2_kv_quantize_fp4")


def csa2_swa_append(k_new, v_new, pos, swa_k, swa_v, stream=None):
    """k_new, v_new [B, D] f32; pos [B] i64; swa_k, swa_v [B, W, D] u8 rings:
    token b goes to slot pos[b] mod W as E4M3FN bytes."""
    f32, _, i64, u8 = _dt()
    B, D = k_new.shape
    W = swa_k.shape[1]
    if (tuple(v_new.shape) != (B, D) or tuple(pos.shape) != (B,)
            or tuple(swa_k.shape) != (B, W, D) or tuple(swa_v.shape) != (B, W, D)):
        raise ValueError("csa2_swa_append: shapes of k_new, v_new, pos, swa_k, swa_v disagree")
    _check(lib.csa2_swa_append(_ptr(k_new, f32, "k_new"), _ptr(v_new, f32, "v_new"),
                               _ptr(pos, i64, "pos"), B, D, W, _ptr(swa_k, u8, "swa_k"),
                               _ptr(swa_v, u8, "swa_v"), _stream(stream)), "csa2_swa_append")


# ----------------------------------------------------------------- profiling

def profile_enable(on=True):
    _check(lib.csa2_profile_enable(1 if on else 0), "csa2_profile_enable")


def profile_reset():
    _check(lib.csa2_profile_reset(), "csa2_profile_reset")


def profile_read():
    """{kernel name: (launches, total_ms)} of the launches since the last reset."""
    res = {}
    i = 0
    while True:
        name, n, ms = ctypes.c_char_p(), ctypes.c_int(), ctypes.c_double()
        if lib.csa2_profile_read(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)) != 0:
            break
        res[name.value.decode()] = (n.value, ms.value)
        i += 1
    return res


def debug_decode_tables(stream=None):
    """Device decodes of all 256 FP4 byte pairs and FP8 bytes (hardware and
    definition paths), for the codec tests."""
    import torch
    dev = torch.device("cuda")
    fp4_hw = torch.empty(512, dtype=torch.float32, device=dev)
    fp4_ref = torch.empty(512, dtype=torch.float32, device=dev)
    fp8_hw = torch.empty(256, dtype=torch.float32, device=dev)
    fp8_ref = torch.empty(256, dtype=torch.float32, device=dev)
    _check(lib.csa2_debug_decode_tables(_ptr(fp4_hw), _ptr(fp4_ref), _ptr(fp8_hw), _ptr(fp8_ref),
                                        _stream(stream)), "csa2_debug_decode_tables")
    return fp4_hw, fp4_ref, fp8_hw, fp8_ref


def debug_dequant_tables(stream=None):
    """The attention kernels' fp16 dequantisation of every (E2M1 code, E4M3
    scale byte) pair, [256, 16, 8] (scale byte, code, nibble position), and of
    every E4M3 byte, [256, 8] (byte, position in a window chunk)."""
    import torch
    dev = torch.device("cuda")
    main = torch.empty((256, 16, 8), dtype=torch.float32, device=dev)
    win = torch.empty((256, 8), dtype=torch.float32, device=dev)
    _check(lib.csa2_debug_dequant_tables(_ptr(main), _ptr(win), _stream(stream)),
           "csa2_debug_dequant_tables")
    return main, win
