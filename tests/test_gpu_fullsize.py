"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the layer group in one csa2_sparse_attn_decode_layers
call): every query of the decode workloads is compared with the oracle --
Top-K, pool and Reindex bit-exactly, every attention layer within max-abs
2e-3 / rel-L2 1e-3 -- and 256 rows of the prefill chunk (16 runs of 16
consecutive queries spread over the chunk) on all six layers.  The oracle
reads regenerated host copies of only the rows each call reads (a query's
whole sequence for a Full layer, its pool blocks for Reindex, its selected
FP4 rows for attention)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import compressed_fp4_kv_amd as csa2  # noqa: E402
import oracle  # noqa: E402
from oracle import slices  # noqa: E402
from gen.workloads import (FULL_LAYER, T_QI_FULL, T_QI_REINDEX, build_device,  # noqa: E402
                           host_kI_rows, host_kv_rows, host_q, host_qI, host_swa, workload)

import _cases as C  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _threads():
    oracle.set_threads(16)
    yield
    torch.cuda.empty_cache()


def _say(*a):
    print(*a, flush=True)


def _group(w, t, idx):
    """The layer group of the workload in one call (as the benchmark runs it)."""
    L = w.layers
    outs = [C.poison_f32((w.B, w.H, w.D)) for _ in range(L)]
    lses = [C.poison_f32((w.B, w.H)) for _ in range(L)]
    buf = C.ws(csa2.csa2_decode_layers_workspace_bytes(L, w.B, w.H, w.D, idx.shape[1], w.W))
    csa2.csa2_sparse_attn_decode_layers(t["q"], t["kv_codes"], t["kv_scales"], t["seq_row_off"],
                                        idx, t["swa_k"], t["swa_v"], t["swa_len"], w.scale, outs,
                                        lses, ws=buf)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs], [x.cpu().numpy() for x in lses]


def _check_layer(w, out, lse, idx, q, swa, what):
    ro, rl = slices.attn_decode(w, idx, q, swa[0], swa[1])
    for b in range(w.B):
        C.assert_attn_close(out[b], ro[b], f"{what} query {b}")
        C.assert_lse_close(lse[b], rl[b], f"{what} query {b}")


def _check_group(w, outs, lses, idx):
    for layer in range(w.layers):
        _check_layer(w, outs[layer], lses[layer], idx, host_q(w, layer), host_swa(w, layer),
                     f"{w.name} layer {layer}")
        _say(f"[{w.name}] layer {layer}: all {w.B} queries within bounds")


def _oracle_full(w, queries, pool_blocks=0):
    """The oracle's Full-layer Top-K (and pool) of decode `queries`, each on
    its whole sequence of keys, in one call."""
    n = [int(w.ctx[b]) for b in queries]
    offs = np.concatenate([[0], np.cumsum(n)[:-1]]).astype(np.int64)
    kI = np.empty((sum(n), w.Hk, w.Di), np.float32)
    for j, b in enumerate(queries):
        kI[offs[j]:offs[j] + n[j]] = host_kI_rows(w, int(w.seq_row_off[b]), n[j])
    qI = host_qI(w, T_QI_FULL)[list(queries)]
    return oracle.index_full(qI, kI, offs, np.arange(len(queries), dtype=np.int32), n, w.Hi, w.Hk,
                             w.Di, w.topk, pool_blocks, w.block_size)


def test_full_size_decode_full_plus_reuse():
    w = workload(1)
    _say(f"[{w.name}] building {w.rows} rows")
    t = build_device(w)
    idx, _ = C.gpu_index_full(w, t)
    idx = idx.cpu().numpy()
    ref, _ = _oracle_full(w, range(w.B))
    for b in range(w.B):
        assert np.array_equal(idx[b], ref[b]), f"Top-K of query {b}"
    _say(f"[{w.name}] Top-512 of all {w.B} queries bit-exact")
    outs, lses = _group(w, t, torch.from_numpy(idx).cuda())
    del t
    torch.cuda.empty_cache()
    _check_group(w, outs, lses, idx)


def test_full_size_hierarchical_1m():
    w = workload(3)
    _say(f"[{w.name}] building {w.rows} rows")
    t = build_device(w)
    idx, pool = C.gpu_index_full(w, t, pool_blocks=w.pool_blocks)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    re = C.gpu_reindex(w, t, torch.from_numpy(pool).cuda())
    # the Full layer's own attention over its Top-K (one layer, as the benchmark runs it)
    out_f = C.poison_f32((w.B, w.H, w.D))
    lse_f = C.poison_f32((w.B, w.H))
    csa2.csa2_sparse_attn_decode(t["q_full"], t["kv_codes"], t["kv_scales"], t["seq_row_off"],
                                 torch.from_numpy(idx).cuda(), t["swa_k_full"], t["swa_v_full"],
                                 t["swa_len"], w.scale, out_f, lse_f,
                                 ws=C.ws(csa2.csa2_decode_workspace_bytes(w.B, w.H, w.D, w.topk,
                                                                          w.W)))
    outs, lses = _group(w, t, re)
    re = re.cpu().numpy()
    out_f, lse_f = out_f.cpu().numpy(), lse_f.cpu().numpy()
    del t
    torch.cuda.empty_cache()
    for q0 in range(0, w.B, 4):      # four 1M-entry sequences (8 GB of keys) per oracle call
        qs = list(range(q0, min(w.B, q0 + 4)))
        r, p = _oracle_full(w, qs, w.pool_blocks)
        for j, b in enumerate(qs):
            assert np.array_equal(idx[b], r[j]), f"Top-K of query {b}"
            assert np.array_equal(pool[b], p[j]), f"pool of query {b}"
        del r, p
    _say(f"[{w.name}] Top-512 and 2,048-block pools of all {w.B} queries bit-exact")
    rr = slices.reindex_batch(w, host_qI(w, T_QI_REINDEX), slices.pool_batch(w, pool,
                                                                            range(w.B)))
    assert np.array_equal(re, rr), "Reindex Top-512"
    _say(f"[{w.name}] Reindex of all {w.B} queries bit-exact")
    _check_layer(w, out_f, lse_f, idx, host_q(w, FULL_LAYER), host_swa(w, FULL_LAYER),
                 f"{w.name} Full layer")
    _check_group(w, outs, lses, re)


def test_full_size_mixed_length_reindex():
    w = workload(4)
    _say(f"[{w.name}] building {w.rows} rows")
    t = build_device(w)
    re = C.gpu_reindex(w, t, t["pool"])
    outs, lses = _group(w, t, re)
    re = re.cpu().numpy()
    del t
    torch.cuda.empty_cache()
    rr = slices.reindex_batch(w, host_qI(w, T_QI_REINDEX), slices.pool_batch(w, w.pool,
                                                                            range(w.B)))
    for b in range(w.B):
        assert np.array_equal(re[b], rr[b]), f"Reindex of query {b} (ctx {w.ctx[b]})"
    _say(f"[{w.name}] Reindex of all {w.B} queries bit-exact")
    _check_group(w, outs, lses, re)


def test_full_size_prefill_chunk():
    w = workload(2)
    _say(f"[{w.name}] Qn={w.Qn} p0={w.p0}")
    t = build_device(w)
    idx, _ = C.gpu_index_full(w, t)
    idx = idx.cpu().numpy()
    outs = []
    for layer in range(w.layers):
        out, lse = C.gpu_attn(w, t, layer, torch.from_numpy(idx).cuda())
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    del t
    torch.cuda.empty_cache()
    # 16 runs of 16 consecutive queries, one every 256 (first and last query included)
    starts = list(range(0, w.Qn - 16, 256)) + [w.Qn - 16]
    rows = np.concatenate([np.arange(s, s + 16) for s in starts])
    assert rows.size >= 256
    kI = host_kI_rows(w, 0, w.ctx[0])
    qI = host_qI(w, T_QI_FULL)[rows]
    ref, _ = oracle.index_full(qI, kI, [0], np.zeros(rows.size, np.int32), w.q_nvis()[rows],
                               w.Hi, w.Hk, w.Di, w.topk)
    for j, i in enumerate(rows):
        assert np.array_equal(idx[i], ref[j]), f"prefill Top-K of query {i}"
    _say(f"[{w.name}] Top-512 of {rows.size} chunk queries bit-exact")
    del kI
    codes, scales = host_kv_rows(w, 0, int(w.ctx[0]))
    for layer in range(w.layers):
        q = host_q(w, layer)
        sk, sv = host_swa(w, layer)
        out, lse = outs[layer]
        for s in starts:
            ro, rl = oracle.attn_prefill(q[s:s + 16], w.p0 + s, codes, scales, idx[s:s + 16],
                                         sk[s:s + 16 + w.W - 1], sv[s:s + 16 + w.W - 1], w.W,
                                         w.scale)
            for j in range(16):
                C.assert_attn_close(out[s + j], ro[j], f"c2 layer {layer} query {s + j}")
                C.assert_lse_close(lse[s + j], rl[j], f"c2 layer {layer} query {s + j}")
        _say(f"[{w.name}] layer {layer}: {rows.size} queries within bounds")
