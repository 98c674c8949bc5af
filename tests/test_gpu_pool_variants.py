"""GPU parity of the candidate-pool variants through csa2_index_full_ex:
blocks scored by the sum of their entries' scores (the variant) or by their
maximum (the reading used by csa2_index_full), over fp32 and E4M3 key caches,
for block sizes 1-8 and ragged sequences; pools, Top-K and the Reindex picks
over the variant pools bit-exact against the oracle."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gen.workloads import (T_QI_FULL, T_QI_REINDEX, Workload, build_device,  # noqa: E402
                           host_kI_rows, host_kI_rows_e4m3, host_qI, workload)

import _cases as C  # noqa: E402


@pytest.fixture(scope="module")
def csa2():
    assert torch.cuda.is_available(), "needs an MI355X"
    import compressed_fp4_kv_amd as m
    oracle.set_threads(16)
    return m


def teardown_module(module):
    torch.cuda.empty_cache()


def _say(*a):
    print(*a, flush=True)


def _gpu(csa2, w, t, keys, rule, P, bs):
    Q = w.Q
    maxn = int(w.q_nvis().max())
    idx, pool = C.poison_i32((Q, w.topk)), C.poison_i32((Q, P))
    buf = C.ws(csa2.csa2_index_full_workspace_bytes(Q, maxn, w.topk, P, bs))
    csa2.csa2_index_full_ex(t["qI_full"], t["kI8" if keys == "e4m3" else "kI"], t["seq_row_off"],
                            t["q_seq"], t["q_nvis"], maxn, w.topk, idx, P, bs, pool,
                            block_rule=rule, ws=buf)
    re = C.poison_i32((Q, w.topk))
    rbuf = C.ws(csa2.csa2_reindex_workspace_bytes(Q, P, bs))
    fn = csa2.csa2_reindex_e4m3 if keys == "e4m3" else csa2.csa2_reindex
    fn(t["qI_reindex"], t["kI8" if keys == "e4m3" else "kI"], t["seq_row_off"], t["q_seq"],
       t["q_nvis"], pool, bs, w.topk, re, rbuf)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), pool.cpu().numpy(), re.cpu().numpy()


def _check(w, keys, rule, P, bs, idx, pool, re, queries):
    rows = host_kI_rows_e4m3 if keys == "e4m3" else host_kI_rows
    for b in queries:
        kI = rows(w, int(w.seq_row_off[b]), int(w.ctx[b]))
        n = int(w.q_nvis()[b])
        r, p = oracle.index_full(host_qI(w, T_QI_FULL)[b:b + 1], kI, [0], [0], [n], w.Hi, w.Hk,
                                 w.Di, w.topk, P, bs, block_rule=rule)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b}"
        assert np.array_equal(pool[b], p[0]), f"{rule} pool of query {b}"
        rr = oracle.reindex(host_qI(w, T_QI_REINDEX)[b:b + 1], kI, [0], [0], [n], p, bs, w.Hi,
                            w.Hk, w.Di, w.topk)
        assert np.array_equal(re[b], rr[0]), f"Reindex over the {rule} pool, query {b}"


@pytest.mark.parametrize("keys", ["f32", "e4m3"])
def test_sum_rule_pool_and_reindex(csa2, keys):
    w = workload(3, small=True)
    _say(f"[{w.name} {keys} sum] ctx={w.ctx}")
    t = build_device(w, with_kv=False, layers=0, keys=keys)
    idx, pool, re = _gpu(csa2, w, t, keys, "sum", w.pool_blocks, w.block_size)
    _check(w, keys, "sum", w.pool_blocks, w.block_size, idx, pool, re, range(w.B))
    # the same call with the max rule is csa2_index_full's pool
    i2, p2, _ = _gpu(csa2, w, t, keys, "max", w.pool_blocks, w.block_size)
    ref_i, ref_p = C.gpu_index_full(w, t, pool_blocks=w.pool_blocks) if keys == "f32" else (None, None)
    if keys == "f32":
        assert np.array_equal(i2, ref_i.cpu().numpy()) and np.array_equal(p2, ref_p.cpu().numpy())
    assert not np.array_equal(pool, p2)            # the rules differ on these inputs


@pytest.mark.parametrize("keys", ["f32", "e4m3"])
@pytest.mark.parametrize("bs,P", [(1, 700), (2, 1000), (4, 2048), (8, 333)])
def test_pool_rules_block_sizes_ragged(csa2, keys, bs, P):
    ctx = [3001, 300, 20005, 2048]
    w = Workload(f"pool_bs{bs}", 31 + bs, "decode_hier", ctx, H=16, topk=256, layers=0,
                 pool_blocks=P, block_size=bs)
    t = build_device(w, with_kv=False, layers=0, keys=keys)
    for rule in ("sum", "max"):
        idx, pool, re = _gpu(csa2, w, t, keys, rule, P, bs)
        _check(w, keys, rule, P, bs, idx, pool, re, range(w.B))


def test_sum_rule_full_size_1m(csa2):
    w = workload(3)
    _say(f"[{w.name} e4m3 sum] building {w.rows} key rows")
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    idx, pool, re = _gpu(csa2, w, t, "e4m3", "sum", w.pool_blocks, w.block_size)
    _check(w, "e4m3", "sum", w.pool_blocks, w.block_size, idx, pool, re, (0, 7))
    del t
    torch.cuda.empty_cache()



def _prefill_pool(csa2, w, t, keys, rule, P, bs):
    Q = w.Qn
    maxn = int(w.q_nvis().max())
    kI = t["kI8" if keys == "e4m3" else "kI"]
    idx, pool = C.poison_i32((Q, w.topk)), C.poison_i32((Q, P))
    buf = C.ws(csa2.csa2_index_prefill_workspace_bytes_ex(Q, maxn, w.topk, P, bs, w.Hk, w.Di))
    csa2.csa2_index_full_ex(t["qI_full"], kI, t["seq_row_off"], None, t["q_nvis"], maxn, w.topk,
                            idx, P, bs, pool, block_rule=rule, ws=buf)
    qR = torch.from_numpy(host_qI(w, T_QI_REINDEX)).cuda()
    re = C.poison_i32((Q, w.topk))
    rbuf = C.ws(csa2.csa2_reindex_workspace_bytes(Q, P, bs))
    fn = csa2.csa2_reindex_e4m3 if keys == "e4m3" else csa2.csa2_reindex
    fn(qR, kI, t["seq_row_off"], None, t["q_nvis"], pool, bs, w.topk, re, rbuf)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), pool.cpu().numpy(), re.cpu().numpy()


def _check_prefill(w, keys, rule, P, bs, idx, pool, re, rows):
    kI = (host_kI_rows_e4m3 if keys == "e4m3" else host_kI_rows)(w, 0, int(w.ctx[0]))
    nv = w.q_nvis()
    qF, qR = host_qI(w, T_QI_FULL), host_qI(w, T_QI_REINDEX)
    for i in rows:
        r, p = oracle.index_full(qF[i:i + 1], kI, [0], [0], [nv[i]], w.Hi, w.Hk, w.Di, w.topk, P,
                                 bs, block_rule=rule)
        assert np.array_equal(idx[i], r[0]), f"Top-K of prefill query {i}"
        assert np.array_equal(pool[i], p[0]), f"{rule} pool of prefill query {i}"
        rr = oracle.reindex(qR[i:i + 1], kI, [0], [0], [nv[i]], p, bs, w.Hi, w.Hk, w.Di, w.topk)
        assert np.array_equal(re[i], rr[0]), f"Reindex of prefill query {i}"


@pytest.mark.parametrize("keys", ["f32", "e4m3"])
@pytest.mark.parametrize("rule,P,bs", [("max", 256, 8), ("sum", 256, 8), ("max", 2048, 2),
                                       ("sum", 100, 4)])
def test_prefill_chunk_pool_and_reindex(csa2, keys, rule, P, bs):
    # the encoder-side hierarchical indexer: a pool per prefill query, then
    # Reindex over it for the chunk (q_seq NULL)
    w = workload(2, small=True)
    _say(f"[{w.name} prefill pool {keys} {rule} {P}x{bs}] Qn={w.Qn}")
    t = build_device(w, with_kv=False, layers=0, keys=keys)
    idx, pool, re = _prefill_pool(csa2, w, t, keys, rule, P, bs)
    _check_prefill(w, keys, rule, P, bs, idx, pool, re, range(w.Qn))


def test_prefill_chunk_pool_full_size(csa2):
    w = workload(2)
    _say(f"[{w.name} prefill pool e4m3 max 2048x8] Qn={w.Qn} entries={w.ctx[0]}")
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    idx, pool, re = _prefill_pool(csa2, w, t, "e4m3", "max", 2048, 8)
    _check_prefill(w, "e4m3", "max", 2048, 8, idx, pool, re, (0, 1, 2047, 4095))
    del t
    torch.cuda.empty_cache()
