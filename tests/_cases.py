"""Helpers of the GPU parity tests: run the library's calls on a workload's
device tensors, and run the oracle on host copies of the same seeded inputs
(regenerated on the host from the generator, never read back from the GPU)."""
import numpy as np
import torch

import compressed_fp4_kv_amd as csa2
import oracle
from gen.workloads import (T_QI_FULL, T_QI_REINDEX, host_kI_rows, host_kv_rows, host_q, host_qI,
                           host_swa)

ATOL = 2e-3      # max-abs error bound on attention outputs
RL2 = 1e-3       # relative L2 error bound on attention outputs


def poison_i32(shape):
    return torch.full(shape, -7, dtype=torch.int32, device="cuda")


def poison_f32(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def ws(nbytes):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")


# ------------------------------------------------------------------ GPU side

def gpu_index_full(w, t, qI=None, topk=None, pool_blocks=0, prefill=None):
    qI = t["qI_full"] if qI is None else qI
    topk = w.topk if topk is None else topk
    prefill = (w.kind == "prefill") if prefill is None else prefill
    Q = qI.shape[0]
    max_nvis = int(w.q_nvis().max()) if Q else 0
    idx = poison_i32((Q, topk))
    pool = poison_i32((Q, pool_blocks)) if pool_blocks else None
    if prefill:
        buf = ws(csa2.csa2_index_prefill_workspace_bytes(Q, max_nvis, topk, w.Hk, w.Di))
    else:
        buf = ws(csa2.csa2_index_full_workspace_bytes(Q, max_nvis, topk, pool_blocks, w.block_size))
    csa2.csa2_index_full(qI, t["kI"], t["seq_row_off"], None if prefill else t["q_seq"],
                         t["q_nvis"], max_nvis, topk, idx, pool_blocks, w.block_size, pool, buf)
    torch.cuda.synchronize()
    return idx, pool


def gpu_reindex(w, t, pool, qI=None, topk=None):
    qI = t["qI_reindex"] if qI is None else qI
    topk = w.topk if topk is None else topk
    Q = qI.shape[0]
    idx = poison_i32((Q, topk))
    buf = ws(csa2.csa2_reindex_workspace_bytes(Q, pool.shape[1], w.block_size))
    csa2.csa2_reindex(qI, t["kI"], t["seq_row_off"], t["q_seq"], t["q_nvis"], pool, w.block_size,
                      topk, idx, buf)
    torch.cuda.synchronize()
    return idx


def gpu_attn(w, t, layer, idx, swa_len=None):
    q = t["q"][layer]
    out = poison_f32(tuple(q.shape))
    lse = poison_f32(tuple(q.shape[:2]))
    topk = idx.shape[1]
    if w.kind == "prefill":
        buf = ws(csa2.csa2_prefill_workspace_bytes(w.Qn, w.H, w.D, topk, w.W))
        csa2.csa2_sparse_attn_prefill_chunk(q, w.p0, t["kv_codes"], t["kv_scales"], idx,
                                            t["swa_k"][layer], t["swa_v"][layer], w.W, w.scale,
                                            out, lse, buf)
    else:
        sl = t["swa_len"] if swa_len is None else swa_len
        buf = ws(csa2.csa2_decode_workspace_bytes(w.B, w.H, w.D, topk, w.W))
        csa2.csa2_sparse_attn_decode(q, t["kv_codes"], t["kv_scales"], t["seq_row_off"], idx,
                                     t["swa_k"][layer], t["swa_v"][layer], sl, w.scale, out, lse,
                                     buf)
    torch.cuda.synchronize()
    return out, lse


# --------------------------------------------------------------- oracle side

def oracle_index_query(w, b, tensor=T_QI_FULL, topk=None, pool_blocks=0, nvis=None):
    """Oracle Top-K (and pool) of decode query b, on its own sequence's rows."""
    topk = w.topk if topk is None else topk
    n = int(w.ctx[b]) if nvis is None else int(nvis)
    off = int(w.seq_row_off[b])
    kI = host_kI_rows(w, off, int(w.ctx[b]))
    qI = host_qI(w, tensor)[b:b + 1]
    return oracle.index_full(qI, kI, [0], [0], [n], w.Hi, w.Hk, w.Di, topk, pool_blocks,
                             w.block_size)


def oracle_reindex_query(w, b, pool_row, tensor=T_QI_REINDEX, topk=None):
    topk = w.topk if topk is None else topk
    off = int(w.seq_row_off[b])
    kI = host_kI_rows(w, off, int(w.ctx[b]))
    qI = host_qI(w, tensor)[b:b + 1]
    return oracle.reindex(qI, kI, [0], [0], [int(w.ctx[b])], np.asarray(pool_row)[None], w.block_size,
                          w.Hi, w.Hk, w.Di, topk)


def oracle_attn_query(w, b, layer, idx_row, swa_len=None):
    """Oracle decode attention of query b (all heads) with index row idx_row."""
    off = int(w.seq_row_off[b])
    codes, scales = host_kv_rows(w, off, int(w.ctx[b]))
    q = host_q(w, layer)[b:b + 1]
    sk, sv = host_swa(w, layer)
    sl = int(w.swa_len()[b]) if swa_len is None else int(swa_len)
    return oracle.attn_decode(q, codes, scales, [0], np.asarray(idx_row, np.int32)[None],
                              sk[b:b + 1], sv[b:b + 1], [sl], w.scale)


def oracle_prefill_rows(w, layer, idx_rows, rows):
    """Oracle prefill attention of the chunk queries `rows` (list of i)."""
    codes, scales = host_kv_rows(w, 0, int(w.ctx[0]))
    q = host_q(w, layer)
    sk, sv = host_swa(w, layer)
    outs, lses = [], []
    for i in rows:
        # query i alone: its W window rows start at row i of the chunk's window
        o, l = oracle.attn_prefill(q[i:i + 1], w.p0 + i, codes, scales, idx_rows[i:i + 1],
                                   sk[i:i + w.W], sv[i:i + w.W], w.W, w.scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


# ------------------------------------------------------------------ checks

def assert_attn_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref).max() if got.size else 0.0
    rl2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err <= ATOL, f"{what}: max-abs {err:.3e} > {ATOL}"
    assert rl2 <= RL2, f"{what}: rel-L2 {rl2:.3e} > {RL2}"
    return err, rl2


def assert_lse_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: lse finiteness differs"
    if fin.any():
        err = np.abs(got[fin] - ref[fin]).max()
        assert err <= 1e-4 * max(1.0, np.abs(ref[fin]).max()), f"{what}: lse err {err:.3e}"
