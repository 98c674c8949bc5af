"""Seeded randomized sweep of small shapes, GPU against the oracle: contexts
shorter than K and ragged last blocks, pools below 2,048 blocks with block
sizes 1-8, windows shorter than 128 (and empty), topk 1 / 64 / 512, 16 or 64
heads, fp32 or E4M3 keys, a shared key head, and layer groups of 1-4 layers.
Indices and pools bit-exact; attention within max-abs 2e-3 / rel-L2 1e-3;
every case run twice, the second run bitwise equal to the first."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gen.workloads import (T_QI_FULL, T_QI_REINDEX, Workload, build_device,  # noqa: E402
                           host_kI_rows, host_kI_rows_e4m3, host_qI)

import _cases as C  # noqa: E402


@pytest.fixture(scope="module")
def csa2():
    assert torch.cuda.is_available(), "needs an MI355X"
    import compressed_fp4_kv_amd as m
    oracle.set_threads(16)
    return m


def teardown_module(module):
    torch.cuda.empty_cache()


def _case(seed):
    rng = np.random.default_rng([7, seed])
    B = int(rng.integers(1, 7))
    ctx = [int(x) for x in rng.integers(1, 3000, size=B)]
    if rng.random() < 0.3:
        ctx[int(rng.integers(B))] = int(rng.integers(1, 12))          # shorter than most K
    topk = int(rng.choice([1, 64, 512]))
    bs = int(rng.choice([1, 2, 4, 8]))
    P = int(rng.integers(1, min(2048, 16384 // bs) + 1))
    H = int(rng.choice([16, 64]))
    Hi, Hk, Di = [(4, 4, 64), (4, 1, 256), (2, 2, 128), (4, 4, 128)][int(rng.integers(4))]
    keys = str(rng.choice(["f32", "e4m3"]))
    L = int(rng.choice([1, 2, 4]))
    rule = str(rng.choice(["max", "sum"]))
    w = Workload(f"sweep{seed}", 100 + seed, "decode_hier", ctx, H=H, Hi=Hi, Hk=Hk, Di=Di,
                 topk=topk, layers=L, pool_blocks=P, block_size=bs)
    swa_len = np.minimum(rng.integers(0, 129, size=B), 128).astype(np.int32)
    return w, keys, rule, swa_len


@pytest.mark.parametrize("seed", range(16))
def test_random_small_shapes(csa2, seed):
    w, keys, rule, swa_len = _case(seed)
    print(f"[sweep {seed}] ctx={w.ctx} topk={w.topk} pool={w.pool_blocks}x{w.block_size} "
          f"H={w.H} idx={w.Hi}x{w.Hk}x{w.Di} keys={keys} rule={rule} L={w.layers}", flush=True)
    t = build_device(w, keys=keys)
    kI = t["kI8" if keys == "e4m3" else "kI"]
    Q, maxn = w.B, int(max(w.ctx))
    sl = torch.from_numpy(swa_len).cuda()

    def run():
        idx, pool = C.poison_i32((Q, w.topk)), C.poison_i32((Q, w.pool_blocks))
        buf = C.ws(csa2.csa2_index_full_workspace_bytes(Q, maxn, w.topk, w.pool_blocks,
                                                        w.block_size))
        csa2.csa2_index_full_ex(t["qI_full"], kI, t["seq_row_off"], t["q_seq"], t["q_nvis"], maxn,
                                w.topk, idx, w.pool_blocks, w.block_size, pool, block_rule=rule,
                                ws=buf)
        re = C.poison_i32((Q, w.topk))
        rbuf = C.ws(csa2.csa2_reindex_workspace_bytes(Q, w.pool_blocks, w.block_size))
        (csa2.csa2_reindex_e4m3 if keys == "e4m3" else csa2.csa2_reindex)(
            t["qI_reindex"], kI, t["seq_row_off"], t["q_seq"], t["q_nvis"], pool, w.block_size,
            w.topk, re, rbuf)
        outs = [C.poison_f32((w.B, w.H, w.D)) for _ in range(w.layers)]
        lses = [C.poison_f32((w.B, w.H)) for _ in range(w.layers)]
        abuf = C.ws(csa2.csa2_decode_layers_workspace_bytes(w.layers, Q, w.H, w.D, w.topk, w.W))
        csa2.csa2_sparse_attn_decode_layers(t["q"], t["kv_codes"], t["kv_scales"],
                                            t["seq_row_off"], re, t["swa_k"], t["swa_v"], sl,
                                            w.scale, outs, lses, ws=abuf)
        torch.cuda.synchronize()
        return (idx.cpu().numpy(), pool.cpu().numpy(), re.cpu().numpy(),
                [o.cpu().numpy() for o in outs], [x.cpu().numpy() for x in lses])

    idx, pool, re, outs, lses = run()
    # a second run into freshly poisoned outputs is bitwise identical
    again = run()
    for a, b in zip((idx, pool, re) + tuple(outs) + tuple(lses),
                    again[:3] + tuple(again[3]) + tuple(again[4])):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), "rerun differs"
    rows = host_kI_rows_e4m3 if keys == "e4m3" else host_kI_rows
    for b in range(w.B):
        kh = rows(w, int(w.seq_row_off[b]), int(w.ctx[b]))
        n = int(w.ctx[b])
        r, p = oracle.index_full(host_qI(w, T_QI_FULL)[b:b + 1], kh, [0], [0], [n], w.Hi, w.Hk,
                                 w.Di, w.topk, w.pool_blocks, w.block_size, block_rule=rule)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b}"
        assert np.array_equal(pool[b], p[0]), f"pool of query {b}"
        rr = oracle.reindex(host_qI(w, T_QI_REINDEX)[b:b + 1], kh, [0], [0], [n], p,
                            w.block_size, w.Hi, w.Hk, w.Di, w.topk)
        assert np.array_equal(re[b], rr[0]), f"Reindex of query {b}"
        for layer in range(w.layers):
            ro, rl = C.oracle_attn_query(w, b, layer, rr[0], swa_len=int(swa_len[b]))
            C.assert_attn_close(outs[layer][b], ro[0], f"layer {layer} query {b}")
            C.assert_lse_close(lses[layer][b], rl[0], f"layer {layer} query {b}")
