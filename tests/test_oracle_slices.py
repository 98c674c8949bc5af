"""The oracle fed with only the rows a query reads (oracle/slices.py) gives
exactly what it gives on the query's whole sequence: Reindex over a packed,
relabelled pool and attention over the packed selected rows."""
import numpy as np

import oracle
from oracle import slices
from gen.workloads import (T_QI_REINDEX, host_kI_rows, host_kv_rows, host_q, host_qI, host_swa,
                           workload)


def _whole_reindex(w, b, pool_row, keys="f32"):
    kI = host_kI_rows(w, int(w.seq_row_off[b]), int(w.ctx[b]))
    if keys == "e4m3":
        from gen import e4m3_bytes
        kI = e4m3_bytes(kI)
    qI = host_qI(w, T_QI_REINDEX)[b:b + 1]
    return oracle.reindex(qI, kI, [0], [0], [int(w.ctx[b])], np.asarray(pool_row)[None],
                          w.block_size, w.Hi, w.Hk, w.Di, w.topk)[0]


def test_reindex_on_packed_pool_equals_whole_sequence():
    w = workload(4, small=True)   # 6 mixed-length sequences, partial last blocks
    for b in range(w.B):
        got = slices.reindex_query(w, b, w.pool[b])
        assert np.array_equal(got, _whole_reindex(w, b, w.pool[b])), f"query {b}"
    b = 1
    assert np.array_equal(slices.reindex_query(w, b, w.pool[b], keys="e4m3"),
                          _whole_reindex(w, b, w.pool[b], keys="e4m3"))


def test_reindex_on_packed_pool_cut_visibility_and_short_pools():
    w = workload(4, small=True)
    rng = np.random.default_rng(7)
    for b in range(w.B):
        n = int(w.ctx[b])
        nb = (n + 7) // 8
        for take in (1, 3, min(nb, 40)):
            row = np.full(w.pool_blocks, -1, np.int32)
            blk = np.sort(rng.choice(nb, size=take, replace=False))
            if take > 1:
                blk[-1] = nb - 1          # the partial last block, when there is one
                blk = np.unique(blk)
            row[:blk.size] = blk
            assert np.array_equal(slices.reindex_query(w, b, row), _whole_reindex(w, b, row))


def test_attention_on_packed_rows_equals_whole_sequence():
    w = workload(4, small=True)
    rng = np.random.default_rng(3)
    idx = np.full((w.B, w.topk), -1, np.int32)
    for b in range(w.B):
        k = min(w.topk, int(w.ctx[b]))
        sel = np.sort(rng.choice(int(w.ctx[b]), size=k - (b % 3), replace=False))
        idx[b, :sel.size] = sel
    q = host_q(w, 2)
    sk, sv = host_swa(w, 2)
    out, lse = slices.attn_decode(w, idx, q, sk, sv)
    for b in range(w.B):
        off = int(w.seq_row_off[b])
        codes, scales = host_kv_rows(w, off, int(w.ctx[b]))
        ro, rl = oracle.attn_decode(q[b:b + 1], codes, scales, [0], idx[b:b + 1], sk[b:b + 1],
                                    sv[b:b + 1], w.swa_len()[b:b + 1], w.scale)
        assert np.array_equal(out[b], ro[0]) and np.array_equal(lse[b], rl[0]), f"query {b}"
    sub, _ = slices.attn_decode(w, idx, q, sk, sv, queries=[4, 1])
    assert np.array_equal(sub[0], out[4]) and np.array_equal(sub[1], out[1])


def test_reindex_batch_equals_single_queries():
    w = workload(4, small=True)
    qs = [5, 0, 2]
    qI = host_qI(w, T_QI_REINDEX)[qs]
    got = slices.reindex_batch(w, qI, slices.pool_batch(w, w.pool, qs))
    for j, b in enumerate(qs):
        assert np.array_equal(got[j], slices.reindex_query(w, b, w.pool[b]))
