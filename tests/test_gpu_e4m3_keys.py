"""GPU parity of the compact indexer-key cache (E4M3FN key bytes) through
csa2_index_full_e4m3 and csa2_reindex_e4m3: Top-K, candidate pools and
Reindex picks bit-exact against the oracle run on the same key bytes, on the
decode, hierarchical, mixed-length and prefill workloads (reduced and full
size), on every supported key-row width, and on general (non-integer) key
values within the fp32 rounding of the K-th score."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gen.workloads import (T_QI_FULL, T_QI_REINDEX, Workload, build_device,  # noqa: E402
                           host_kI_rows_e4m3, host_qI, workload)

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


def _index8(csa2, w, t, qI=None, topk=None, pool_blocks=0, prefill=False):
    qI = t["qI_full"] if qI is None else qI
    topk = w.topk if topk is None else topk
    Q = qI.shape[0]
    max_nvis = int(w.q_nvis().max()) if Q else 0
    idx = C.poison_i32((Q, topk))
    pool = C.poison_i32((Q, pool_blocks)) if pool_blocks else None
    if prefill:
        buf = C.ws(csa2.csa2_index_prefill_workspace_bytes(Q, max_nvis, topk, w.Hk, w.Di))
    else:
        buf = C.ws(csa2.csa2_index_full_workspace_bytes(Q, max_nvis, topk, pool_blocks,
                                                        w.block_size))
    csa2.csa2_index_full_e4m3(qI, t["kI8"], t["seq_row_off"], None if prefill else t["q_seq"],
                              t["q_nvis"], max_nvis, topk, idx, pool_blocks, w.block_size, pool,
                              buf)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (pool.cpu().numpy() if pool is not None else None)


def _reindex8(csa2, w, t, pool, qI=None):
    qI = t["qI_reindex"] if qI is None else qI
    Q = qI.shape[0]
    idx = C.poison_i32((Q, w.topk))
    buf = C.ws(csa2.csa2_reindex_workspace_bytes(Q, pool.shape[1], w.block_size))
    csa2.csa2_reindex_e4m3(qI, t["kI8"], t["seq_row_off"], t["q_seq"], t["q_nvis"],
                           torch.as_tensor(pool).cuda(), w.block_size, w.topk, idx, buf)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def _oracle_index(w, b, pool_blocks=0, tensor=T_QI_FULL):
    k8 = host_kI_rows_e4m3(w, int(w.seq_row_off[b]), int(w.ctx[b]))
    qI = host_qI(w, tensor)[b:b + 1]
    return oracle.index_full(qI, k8, [0], [0], [int(w.q_nvis()[b])], w.Hi, w.Hk, w.Di, w.topk,
                             pool_blocks, w.block_size)


def _oracle_reindex(w, b, pool_row, tensor=T_QI_REINDEX):
    k8 = host_kI_rows_e4m3(w, int(w.seq_row_off[b]), int(w.ctx[b]))
    qI = host_qI(w, tensor)[b:b + 1]
    return oracle.reindex(qI, k8, [0], [0], [int(w.ctx[b])], np.asarray(pool_row)[None],
                          w.block_size, w.Hi, w.Hk, w.Di, w.topk)[0]


# ------------------------------------------------------------ reduced size

def test_e4m3_keys_decode_full(csa2):
    w = workload(1, small=True)
    _say(f"[{w.name} e4m3] B={w.B} ctx={w.ctx[0]}")
    t = build_device(w, with_kv=False, layers=0, keys="both")
    idx, _ = _index8(csa2, w, t)
    f32_idx, _ = C.gpu_index_full(w, t)
    assert np.array_equal(idx, f32_idx.cpu().numpy()), "E4M3 keys select differently from fp32"
    for b in range(w.B):
        r, _ = _oracle_index(w, b)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b}"


def test_e4m3_keys_pool_and_reindex(csa2):
    w = workload(3, small=True)
    _say(f"[{w.name} e4m3] ctx={w.ctx}")
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    idx, pool = _index8(csa2, w, t, pool_blocks=w.pool_blocks)
    re = _reindex8(csa2, w, t, pool)
    for b in range(w.B):
        r, p = _oracle_index(w, b, pool_blocks=w.pool_blocks)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b}"
        assert np.array_equal(pool[b], p[0]), f"pool of query {b}"
        assert np.array_equal(re[b], _oracle_reindex(w, b, p[0])), f"Reindex of query {b}"


def test_e4m3_keys_mixed_length_reindex(csa2):
    w = workload(4, small=True)
    _say(f"[{w.name} e4m3] ctx={w.ctx}")
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    re = _reindex8(csa2, w, t, w.pool)
    for b in range(w.B):
        assert np.array_equal(re[b], _oracle_reindex(w, b, w.pool[b])), f"Reindex of query {b}"


@pytest.mark.parametrize("Hi,Hk,Di", [(4, 4, 64), (4, 4, 256), (4, 1, 512), (2, 1, 256)])
def test_e4m3_keys_row_widths_and_ragged(csa2, Hi, Hk, Di):
    # key rows of 256, 1,024 and 512 bytes, a shared key head, ragged
    # sequences (one shorter than K, one ending mid-tile), pool of 8-blocks
    ctx = [3001, 300, 20000, 2048]
    w = Workload(f"rows_{Hi}x{Hk}x{Di}", 21, "decode_hier", ctx, H=16, Hi=Hi, Hk=Hk, Di=Di,
                 topk=512, layers=0, pool_blocks=600)
    _say(f"[{w.name}] ctx={ctx}")
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    idx, pool = _index8(csa2, w, t, pool_blocks=w.pool_blocks)
    re = _reindex8(csa2, w, t, pool)
    for b in range(w.B):
        r, p = _oracle_index(w, b, pool_blocks=w.pool_blocks)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b}"
        assert np.array_equal(pool[b], p[0]), f"pool of query {b}"
        assert np.array_equal(re[b], _oracle_reindex(w, b, p[0])), f"Reindex of query {b}"


def test_e4m3_keys_prefill_chunk(csa2):
    w = workload(2, small=True)
    _say(f"[{w.name} e4m3] Qn={w.Qn} p0={w.p0}")
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    idx, _ = _index8(csa2, w, t, prefill=True)
    k8 = host_kI_rows_e4m3(w, 0, int(w.ctx[0]))
    ref, _ = oracle.index_full(host_qI(w, T_QI_FULL), k8, [0], np.zeros(w.Qn, np.int32),
                               w.q_nvis(), w.Hi, w.Hk, w.Di, w.topk)
    assert np.array_equal(idx, ref)


def test_e4m3_keys_general_values(csa2):
    # every finite E4M3 value as a key, N(0,1) queries: the fp32 sums may
    # order near-ties differently from the oracle's double sums, so outside
    # the oracle's set only entries within the fp32 rounding of the K-th
    # score may appear (and vice versa)
    ctx = [5000, 777, 12000]
    w = Workload("e4m3_general", 22, "decode_hier", ctx, H=16, topk=256, layers=0,
                 pool_blocks=400)
    t = build_device(w, with_kI=False, with_kv=False, layers=0)
    rng = np.random.default_rng(22)
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    k8 = rng.choice(finite, size=(w.rows, w.Hk, w.Di)).astype(np.uint8)
    qI = rng.standard_normal((w.B, w.Hi, w.Di)).astype(np.float32)
    qR = rng.standard_normal((w.B, w.Hi, w.Di)).astype(np.float32)
    t["kI8"] = torch.from_numpy(k8).cuda()
    idx, pool = _index8(csa2, w, t, qI=torch.from_numpy(qI).cuda(), pool_blocks=w.pool_blocks)
    nv = w.q_nvis()
    off = w.seq_row_off
    seqs = np.arange(w.B, dtype=np.int32)
    ref, _ = oracle.index_full(qI, k8, off, seqs, nv, w.Hi, w.Hk, w.Di, w.topk)
    for b in range(w.B):
        s = oracle.scores(qI, k8, off, seqs, nv, b, w.Hi, w.Hk, w.Di)
        g = idx[b]
        assert np.all(np.diff(g[g >= 0]) > 0) and np.all(g[:min(w.topk, nv[b])] >= 0)
        kth = np.sort(s)[::-1][min(w.topk, nv[b]) - 1]
        eps = 1e-5 * np.abs(s).max()
        gsel, rsel = set(g[g >= 0].tolist()), set(ref[b][ref[b] >= 0].tolist())
        assert len(gsel ^ rsel) <= 4, f"query {b}: {len(gsel ^ rsel)} entries differ"
        assert all(s[j] >= kth - eps for j in gsel - rsel), f"query {b}"
        assert all(s[j] <= kth + eps for j in rsel - gsel), f"query {b}"
    # Reindex over the GPU's pools with another query
    re = _reindex8(csa2, w, t, pool, qI=torch.from_numpy(qR).cuda())
    rre = oracle.reindex(qR, k8, off, seqs, nv, pool, w.block_size, w.Hi, w.Hk, w.Di, w.topk)
    for b in range(w.B):
        s = oracle.scores(qR, k8, off, seqs, nv, b, w.Hi, w.Hk, w.Di)
        cand = (pool[b][pool[b] >= 0][:, None] * w.block_size + np.arange(w.block_size)).ravel()
        cand = cand[cand < nv[b]]
        cs = np.sort(s[cand])[::-1]
        kth = cs[min(w.topk, len(cand)) - 1]
        eps = 1e-5 * np.abs(s).max()
        g, r = set(re[b][re[b] >= 0].tolist()), set(rre[b][rre[b] >= 0].tolist())
        assert g <= set(cand.tolist())
        assert len(g ^ r) <= 4, f"reindex query {b}"
        assert all(s[j] >= kth - eps for j in g - r) and all(s[j] <= kth + eps for j in r - g)


# --------------------------------------------------------------- full size

def test_e4m3_keys_full_size_decode(csa2):
    w = workload(1)
    _say(f"[{w.name} e4m3] building {w.rows} key rows")
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    idx, _ = _index8(csa2, w, t)
    for b in (0, 13, 31):
        r, _ = _oracle_index(w, b)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b}"
    assert np.all(np.diff(idx, axis=1) > 0)
    del t
    torch.cuda.empty_cache()


def test_e4m3_keys_full_size_hierarchical_1m(csa2):
    w = workload(3)
    _say(f"[{w.name} e4m3] building {w.rows} key rows")
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    idx, pool = _index8(csa2, w, t, pool_blocks=w.pool_blocks)
    re = _reindex8(csa2, w, t, pool)
    for b in (0, 5):
        r, p = _oracle_index(w, b, pool_blocks=w.pool_blocks)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b}"
        assert np.array_equal(pool[b], p[0]), f"pool of query {b}"
        assert np.array_equal(re[b], _oracle_reindex(w, b, p[0])), f"Reindex of query {b}"
    del t
    torch.cuda.empty_cache()


def test_e4m3_keys_full_size_mixed_length_reindex(csa2):
    # 64 sequences of 8,192 .. 1,048,576 entries (7 GB of E4M3 keys): Reindex
    # over the inherited pools, sampled at the shortest, the longest and two
    # other sequences
    w = workload(4)
    _say(f"[{w.name} e4m3] building {w.rows} key rows")
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    re = _reindex8(csa2, w, t, w.pool)
    ctx = np.asarray(w.ctx)
    for b in sorted({0, int(ctx.argmin()), int(ctx.argmax()), 40}):
        assert np.array_equal(re[b], _oracle_reindex(w, b, w.pool[b])), \
            f"Reindex of query {b} (ctx {ctx[b]})"
        _say(f"[c4 e4m3] query {b} (ctx {ctx[b]}) ok")
    del t
    torch.cuda.empty_cache()


def test_e4m3_keys_full_size_prefill_chunk(csa2):
    # 4,096 prefill queries over 65,536 E4M3 key rows (the bf16 MFMA score
    # GEMM and the row select), sampled at both ends and in the middle
    w = workload(2)
    _say(f"[{w.name} e4m3] Qn={w.Qn} p0={w.p0}")
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    idx, _ = _index8(csa2, w, t, prefill=True)
    rows = [0, 1, 1000, 2047, 4094, 4095]
    k8 = host_kI_rows_e4m3(w, 0, int(w.ctx[0]))
    ref, _ = oracle.index_full(host_qI(w, T_QI_FULL)[rows], k8, [0],
                               np.zeros(len(rows), np.int32), w.q_nvis()[rows], w.Hi, w.Hk,
                               w.Di, w.topk)
    for j, i in enumerate(rows):
        assert np.array_equal(idx[i], ref[j]), f"prefill Top-K of query {i}"
    assert np.all((idx >= 0) & (idx < w.q_nvis()[:, None]))
    assert np.all(np.diff(idx, axis=1) > 0)
    del t
    torch.cuda.empty_cache()


@pytest.mark.parametrize("ctx,topk", [([10, 64, 65, 3000, 0, 1], 64), ([2049, 0, 4097], 2048)])
def test_e4m3_keys_ragged_empty_and_short(csa2, ctx, topk):
    # empty sequences, a single entry, K above the context, K = 2,048
    w = Workload("e4m3_ragged", 23, "decode_hier", ctx, H=16, topk=topk, layers=0,
                 pool_blocks=min(topk, 600))
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    idx, pool = _index8(csa2, w, t, pool_blocks=w.pool_blocks)
    for b in range(w.B):
        if w.ctx[b] == 0:
            assert np.all(idx[b] == -1) and np.all(pool[b] == -1)
            continue
        r, p = _oracle_index(w, b, pool_blocks=w.pool_blocks)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b} ctx {w.ctx[b]}"
        assert np.array_equal(pool[b], p[0]), f"pool of query {b} ctx {w.ctx[b]}"


def test_e4m3_keys_all_ties_and_long_rows(csa2):
    # qI = 0: every score is 0 (the lowest indices and block ids win); rows
    # past 65,536 keys take the filter + finalize selection
    w = Workload("e4m3_ties", 24, "decode_hier", [20000, 70000], H=16, topk=512, layers=0,
                 pool_blocks=2048)
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    idx, pool = _index8(csa2, w, t, qI=torch.zeros_like(t["qI_full"]), pool_blocks=2048)
    for b in range(2):
        assert np.array_equal(idx[b], np.arange(512))
        assert np.array_equal(pool[b], np.arange(2048))
    idx, pool = _index8(csa2, w, t, pool_blocks=2048)
    for b in range(2):
        r, p = _oracle_index(w, b, pool_blocks=2048)
        assert np.array_equal(idx[b], r[0]) and np.array_equal(pool[b], p[0]), f"query {b}"


@pytest.mark.parametrize("Hi,Hk,Di", [(4, 1, 512), (4, 4, 256)])
def test_e4m3_keys_prefill_row_widths(csa2, Hi, Hk, Di):
    # the prefill form over E4M3 keys with a shared key head (512-byte rows)
    # and with 1,024-byte rows
    w = Workload(f"e4m3_prefill_{Hi}x{Hk}x{Di}", 25, "prefill", [3000], Hi=Hi, Hk=Hk, Di=Di,
                 topk=128, layers=0, p0=5900, Qn=70, m=2)
    t = build_device(w, with_kv=False, layers=0, keys="e4m3")
    idx, _ = _index8(csa2, w, t, prefill=True)
    k8 = host_kI_rows_e4m3(w, 0, int(w.ctx[0]))
    ref, _ = oracle.index_full(host_qI(w, T_QI_FULL), k8, [0], np.zeros(w.Qn, np.int32),
                               w.q_nvis(), w.Hi, w.Hk, w.Di, w.topk)
    assert np.array_equal(idx, ref)
