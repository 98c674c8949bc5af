"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: the GPU runs every query; the oracle recomputes a sample of
queries (each one on its whole sequence) and the two must agree bit-exactly
on indices and within the attention bounds on outputs."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gen.workloads import T_QI_FULL, build_device, host_kI_rows, host_qI, workload  # noqa: E402

import _cases as C  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _threads():
    oracle.set_threads(16)
    yield
    torch.cuda.empty_cache()


def _say(*a):
    print(*a, flush=True)


def test_full_size_decode_full_plus_reuse():
    w = workload(1)
    _say(f"[{w.name}] building {w.rows} rows")
    t = build_device(w)
    idx, _ = C.gpu_index_full(w, t)
    idx = idx.cpu().numpy()
    for b in range(w.B):
        r, _ = C.oracle_index_query(w, b)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b}"
    _say("[c1] Top-512 of all 32 queries bit-exact")
    idx_d = torch.from_numpy(idx).cuda()
    for layer in range(w.layers):
        out, lse = C.gpu_attn(w, t, layer, idx_d)
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        for b in (0, 13, 31):
            ro, rl = C.oracle_attn_query(w, b, layer, idx[b])
            C.assert_attn_close(out[b], ro[0], f"c1 layer {layer} query {b}")
            C.assert_lse_close(lse[b], rl[0], f"c1 layer {layer} query {b}")
    del t
    torch.cuda.empty_cache()


def test_full_size_hierarchical_1m():
    w = workload(3)
    _say(f"[{w.name}] building {w.rows} rows")
    t = build_device(w)
    idx, pool = C.gpu_index_full(w, t, pool_blocks=w.pool_blocks)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    re = C.gpu_reindex(w, t, torch.from_numpy(pool).cuda()).cpu().numpy()
    for b in (0, 5):
        r, p = C.oracle_index_query(w, b, pool_blocks=w.pool_blocks)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b}"
        assert np.array_equal(pool[b], p[0]), f"pool of query {b}"
        rr = C.oracle_reindex_query(w, b, p[0])
        assert np.array_equal(re[b], rr[0]), f"reindex of query {b}"
        _say(f"[c3] query {b}: Top-512, pool and reindex bit-exact")
        out, lse = C.gpu_attn(w, t, 0, torch.from_numpy(re).cuda())
        ro, rl = C.oracle_attn_query(w, b, 0, rr[0])
        C.assert_attn_close(out.cpu().numpy()[b], ro[0], f"c3 query {b}")
        C.assert_lse_close(lse.cpu().numpy()[b], rl[0], f"c3 query {b}")
    del t
    torch.cuda.empty_cache()


def test_full_size_mixed_length_reindex():
    w = workload(4)
    _say(f"[{w.name}] building {w.rows} rows")
    t = build_device(w)
    re = C.gpu_reindex(w, t, t["pool"]).cpu().numpy()
    ctx = np.asarray(w.ctx)
    sample = sorted({0, int(ctx.argmin()), int(ctx.argmax()), 40})
    re_d = torch.from_numpy(re).cuda()
    outs = [C.gpu_attn(w, t, layer, re_d) for layer in (0, 3)]
    for b in sample:
        rr = C.oracle_reindex_query(w, b, w.pool[b])
        assert np.array_equal(re[b], rr[0]), f"reindex of query {b} (ctx {ctx[b]})"
        for (out, lse), layer in zip(outs, (0, 3)):
            ro, rl = C.oracle_attn_query(w, b, layer, rr[0])
            C.assert_attn_close(out.cpu().numpy()[b], ro[0], f"c4 layer {layer} query {b}")
            C.assert_lse_close(lse.cpu().numpy()[b], rl[0], f"c4 layer {layer} query {b}")
        _say(f"[c4] query {b} (ctx {ctx[b]}) ok")
    del t
    torch.cuda.empty_cache()


def test_full_size_prefill_chunk():
    w = workload(2)
    _say(f"[{w.name}] Qn={w.Qn} p0={w.p0}")
    t = build_device(w)
    idx, _ = C.gpu_index_full(w, t)
    idx = idx.cpu().numpy()
    rows = [0, 1, 1000, 2047, 4094, 4095]
    kI = host_kI_rows(w, 0, w.ctx[0])
    qI = host_qI(w, T_QI_FULL)[rows]
    nv = w.q_nvis()[rows]
    ref, _ = oracle.index_full(qI, kI, [0], np.zeros(len(rows), np.int32), nv, w.Hi, w.Hk, w.Di,
                               w.topk)
    for j, i in enumerate(rows):
        assert np.array_equal(idx[i], ref[j]), f"prefill Top-K of query {i}"
    _say("[c2] sampled prefill Top-512 bit-exact")
    idx_d = torch.from_numpy(idx).cuda()
    full_ref = np.full((w.Qn, w.topk), -1, np.int32)
    full_ref[rows] = ref
    for layer in (0, 5):
        out, lse = C.gpu_attn(w, t, layer, idx_d)
        ro, rl = C.oracle_prefill_rows(w, layer, full_ref, rows)
        C.assert_attn_close(out.cpu().numpy()[rows], ro, f"c2 layer {layer}")
        C.assert_lse_close(lse.cpu().numpy()[rows], rl, f"c2 layer {layer}")
    del t
    torch.cuda.empty_cache()
