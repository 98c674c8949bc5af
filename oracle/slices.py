"""The oracle on single decode queries, fed with only the rows their calls
read, regenerated on the host from the seeded generator.

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and the benchmark's CPU-baseline
leg, never by the product package.  No arithmetic of the method lives here:
these helpers slice and relabel inputs, and the oracle functions in
``oracle.c`` compute every result.

* Reindex over a pool reads only the pool's blocks (at most 2,048 x 8 key
  rows of a sequence of up to 1,048,576).  ``reindex_query`` packs those
  blocks back to back, relabels pool block i as block i and cuts the visible
  count at the same place, so that compact entry i*bs + j stands for entry
  pool[i]*bs + j.  The relabelling keeps the blocks' order, so the order of
  entries -- and with it the rule that ties go to the lower entry -- is
  unchanged, and the compact answer maps back entry by entry.
* Attention reads only the FP4 rows its index row selects.  ``attn_decode``
  packs each query's selected rows and renumbers the index row's entries in
  place (padding -1 kept), so every query attends over the same rows in the
  same order as over its whole sequence.
"""
import numpy as np

from gen import e4m3_bytes
from gen.workloads import T_QI_REINDEX, host_kI_row_runs, host_kv_rows_at, host_qI

from . import attn_decode as _attn_decode
from . import reindex as _reindex


def pool_slice(w, b, pool_row, keys="f32"):
    """(compact key rows, compact pool row [1, P], compact visible count,
    the pool's valid blocks) of decode query b."""
    pool_row = np.asarray(pool_row, np.int64).reshape(-1)
    bs = w.block_size
    nvis = int(w.q_nvis()[b])
    blocks = pool_row[pool_row >= 0]
    if np.any(np.diff(blocks) <= 0):
        raise ValueError("pool blocks must be distinct and ascending")
    blocks = blocks[blocks * bs < nvis]     # a block past the visible entries has no candidate
    P = int(blocks.size)
    kI = host_kI_row_runs(w, int(w.seq_row_off[b]) + blocks * bs, bs)
    if keys == "e4m3":
        kI = e4m3_bytes(kI)
    cnvis = (P - 1) * bs + min(bs, nvis - int(blocks[-1]) * bs) if P else 0
    cpool = np.full((1, pool_row.size), -1, np.int32)
    cpool[0, :P] = np.arange(P, dtype=np.int32)
    return kI, cpool, cnvis, blocks


def reindex_query(w, b, pool_row, qI=None, tensor=T_QI_REINDEX, topk=None, keys="f32"):
    """The oracle's Reindex Top-K row of decode query b over pool_row."""
    topk = w.topk if topk is None else topk
    qI = host_qI(w, tensor) if qI is None else qI
    kI, cpool, cnvis, blocks = pool_slice(w, b, pool_row, keys)
    r = _reindex(qI[b:b + 1], kI, [0], [0], [cnvis], cpool, w.block_size, w.Hi, w.Hk, w.Di,
                 topk)[0]
    out = r.copy()
    v = out >= 0
    bs = w.block_size
    out[v] = (blocks[out[v] // bs] * bs + out[v] % bs).astype(np.int32)
    return out


def pool_batch(w, pool, queries, keys="f32"):
    """The packed pools of `queries` as one batch for a single oracle call
    (one packed sequence per query): (kI, seq_row_off, q_seq, q_nvis, pool,
    blocks per query)."""
    parts = [pool_slice(w, b, pool[b], keys) for b in queries]
    kI = np.concatenate([p[0] for p in parts]) if parts else np.zeros((0, w.Hk, w.Di), np.float32)
    sizes = [p[0].shape[0] for p in parts]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
    cpool = np.concatenate([p[1] for p in parts]) if parts else np.zeros((0, pool.shape[1]), np.int32)
    nvis = np.asarray([p[2] for p in parts], np.int32)
    return kI, offs, np.arange(len(queries), dtype=np.int32), nvis, cpool, [p[3] for p in parts]


def reindex_batch(w, qI, batch, topk=None):
    """The oracle's Reindex of every query of a pool_batch (one call, the
    oracle's threads across queries), mapped back to entry indices."""
    topk = w.topk if topk is None else topk
    kI, offs, qseq, nvis, cpool, blocks = batch
    r = _reindex(qI, kI, offs, qseq, nvis, cpool, w.block_size, w.Hi, w.Hk, w.Di, topk)
    bs = w.block_size
    for j, bl in enumerate(blocks):
        v = r[j] >= 0
        r[j, v] = (bl[r[j, v] // bs] * bs + r[j, v] % bs).astype(np.int32)
    return r


def selected_rows(w, idx, queries):
    """Packed FP4 rows of the selected entries of `queries` and the index rows
    renumbered to them: (codes, scales, seq_row_off, idx [len(queries), K])."""
    idx = np.asarray(idx, np.int32)
    offs = w.seq_row_off
    rows, cidx, starts, n = [], np.full((len(queries), idx.shape[1]), -1, np.int32), [], 0
    for j, b in enumerate(queries):
        sel = idx[b] >= 0
        k = int(sel.sum())
        rows.append(int(offs[b]) + idx[b][sel].astype(np.int64))
        cidx[j, sel] = np.arange(k, dtype=np.int32)
        starts.append(n)
        n += k
    all_rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    codes, scales = host_kv_rows_at(w, all_rows)
    return codes, scales, np.asarray(starts, np.int64), cidx


def attn_decode(w, idx, q, swa_k, swa_v, queries=None, swa_len=None, want_lse=True):
    """The oracle's decode attention of `queries` (default: all) with index
    rows idx [B, K]; q [B, H, D] and swa_k/v [B, W, D] are the layer's whole
    tensors.  Returns (out [n, H, D], lse [n, H]) in the order of `queries`."""
    queries = list(range(w.B)) if queries is None else list(queries)
    codes, scales, starts, cidx = selected_rows(w, idx, queries)
    sl = w.swa_len() if swa_len is None else np.asarray(swa_len)
    qs = np.asarray(queries, np.int64)
    return _attn_decode(q[qs], codes, scales, starts, cidx, swa_k[qs], swa_v[qs], sl[qs],
                        w.scale, want_lse=want_lse)
