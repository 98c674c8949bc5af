"""GPU parity of the HIP path against the CPU oracle, through the C ABI, on
the five workloads at reduced context (several tiles and ragged tails) and on
edge cases.  Indices: bit-exact.  Attention: max-abs 2e-3 and rel-L2 1e-3."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gen import host_ints  # noqa: E402
from gen.workloads import (T_QI_FULL, T_QI_REINDEX, Workload, build_device, host_kI_rows,  # noqa: E402
                           host_kv_rows, host_qI, host_swa, workload)

import _cases as C  # noqa: E402


@pytest.fixture(scope="module")
def csa2():
    assert torch.cuda.is_available(), "needs an MI355X"
    import compressed_fp4_kv_amd as m
    return m


def teardown_module(module):
    torch.cuda.empty_cache()


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ codecs

def test_device_codecs_match_oracle_tables(csa2):
    fp4_hw, fp4_ref, fp8_hw, fp8_ref = [x.cpu().numpy() for x in csa2.debug_decode_tables()]
    torch.cuda.synchronize()
    exp4 = np.array([oracle.e2m1(b & 15) if j == 0 else oracle.e2m1(b >> 4)
                     for b in range(256) for j in range(2)])
    exp8 = np.array([oracle.e4m3(b) for b in range(256)])
    assert np.array_equal(fp4_ref, exp4)
    assert np.array_equal(fp4_hw, exp4), "gfx950 FP4 conversion disagrees with E2M1"
    nan = np.isnan(exp8)
    assert np.array_equal(np.isnan(fp8_ref), nan) and np.array_equal(fp8_ref[~nan], exp8[~nan])
    assert np.array_equal(np.isnan(fp8_hw), nan), "gfx950 FP8 NaN codes differ from E4M3FN"
    assert np.array_equal(fp8_hw[~nan], exp8[~nan]), "gfx950 FP8 conversion differs from E4M3FN"


def test_attention_dequant_is_exact(csa2):
    """Every E2M1 code times every E4M3 scale byte, at every nibble position,
    and every E4M3 byte at every byte position, as the attention kernels
    dequantise them, against the oracle's codec tables."""
    main, win = [x.cpu().numpy() for x in csa2.debug_dequant_tables()]
    torch.cuda.synchronize()
    e2 = np.array([oracle.e2m1(c) for c in range(16)])
    e8 = np.array([oracle.e4m3(b) for b in range(256)])
    exp_main = np.broadcast_to((e8[:, None] * e2[None, :])[:, :, None], main.shape)
    nan = np.isnan(exp_main)
    assert np.array_equal(np.isnan(main), nan)
    assert np.array_equal(main[~nan], exp_main[~nan]), "FP4 x E4M3 dequantisation is not exact"
    exp_win = np.broadcast_to(e8[:, None], win.shape)
    nan = np.isnan(exp_win)
    assert np.array_equal(np.isnan(win), nan)
    assert np.array_equal(win[~nan], exp_win[~nan]), "E4M3 window conversion is not exact"


# ----------------------------------------------------------- decode groups

def _check_decode_group(csa2, w, t, idx_gpu, idx_ref_rows, layers, queries):
    for layer in range(layers):
        out, lse = C.gpu_attn(w, t, layer, idx_gpu)
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        for b in queries:
            ro, rl = C.oracle_attn_query(w, b, layer, idx_ref_rows[b])
            C.assert_attn_close(out[b], ro[0], f"{w.name} layer {layer} query {b}")
            C.assert_lse_close(lse[b], rl[0], f"{w.name} layer {layer} query {b}")


@pytest.mark.parametrize("wid", [0, 1])
def test_full_then_reuse_group(csa2, wid):
    w = workload(wid, small=True)
    _say(f"[{w.name}] B={w.B} ctx={w.ctx[0]} topk={w.topk}")
    t = build_device(w)
    idx, _ = C.gpu_index_full(w, t)
    idx = idx.cpu().numpy()
    ref = {}
    for b in range(w.B):
        r, _ = C.oracle_index_query(w, b)
        assert np.array_equal(idx[b], r[0]), f"{w.name}: Top-K of query {b} differs"
        ref[b] = r[0]
    # Full layer + Reuse layers: same indices, same KV, own q and window
    _check_decode_group(csa2, w, t, torch.from_numpy(idx).cuda(), ref, w.layers, range(w.B))


def test_hierarchical_pool_reindex_group(csa2):
    w = workload(3, small=True)
    _say(f"[{w.name}] ctx={w.ctx}")
    t = build_device(w)
    idx, pool = C.gpu_index_full(w, t, pool_blocks=w.pool_blocks)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    ref_re = {}
    for b in range(w.B):
        r, p = C.oracle_index_query(w, b, pool_blocks=w.pool_blocks)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b}"
        assert np.array_equal(pool[b], p[0]), f"pool of query {b}"
        ref_re[b] = C.oracle_reindex_query(w, b, p[0])[0]
    re = C.gpu_reindex(w, t, torch.from_numpy(pool).cuda()).cpu().numpy()
    for b in range(w.B):
        assert np.array_equal(re[b], ref_re[b]), f"reindex of query {b}"
    _check_decode_group(csa2, w, t, torch.from_numpy(re).cuda(), ref_re, w.layers, range(w.B))


def test_mixed_length_reindex_group(csa2):
    w = workload(4, small=True)
    _say(f"[{w.name}] ctx={w.ctx}")
    t = build_device(w, with_kI=True)
    re = C.gpu_reindex(w, t, t["pool"]).cpu().numpy()
    ref = {}
    for b in range(w.B):
        ref[b] = C.oracle_reindex_query(w, b, w.pool[b])[0]
        assert np.array_equal(re[b], ref[b]), f"reindex of query {b} (ctx {w.ctx[b]})"
    _check_decode_group(csa2, w, t, torch.from_numpy(re).cuda(), ref, w.layers, range(w.B))


def test_prefill_chunk(csa2):
    w = workload(2, small=True)
    _say(f"[{w.name}] Qn={w.Qn} p0={w.p0}")
    t = build_device(w)
    idx, _ = C.gpu_index_full(w, t)
    idx = idx.cpu().numpy()
    kI = host_kI_rows(w, 0, w.ctx[0])
    qI = host_qI(w, T_QI_FULL)
    ref, _ = oracle.index_full(qI, kI, [0], np.zeros(w.Qn, np.int32), w.q_nvis(), w.Hi, w.Hk, w.Di,
                               w.topk)
    assert np.array_equal(idx, ref)
    idx_d = torch.from_numpy(idx).cuda()
    rows = list(range(w.Qn))
    for layer in range(w.layers):
        out, lse = C.gpu_attn(w, t, layer, idx_d)
        ro, rl = C.oracle_prefill_rows(w, layer, ref, rows)
        C.assert_attn_close(out.cpu().numpy(), ro, f"prefill layer {layer}")
        C.assert_lse_close(lse.cpu().numpy(), rl, f"prefill layer {layer}")


# ------------------------------------------------------------- edge cases

def _edge(ctx, **kw):
    w = Workload("edge", 9, "decode_full", list(ctx), **kw)
    return w


@pytest.mark.parametrize("ctx,topk", [([10, 64, 65, 3000, 0, 1], 64),
                                      ([1, 2, 7, 5000], 512),
                                      ([2049, 2047, 4097], 2048)])
def test_index_ragged_and_short(csa2, ctx, topk):
    w = _edge(ctx, topk=topk)
    t = build_device(w, layers=0, with_kv=False)
    idx, _ = C.gpu_index_full(w, t)
    idx = idx.cpu().numpy()
    for b in range(w.B):
        if w.ctx[b] == 0:
            assert np.all(idx[b] == -1)
            continue
        r, _ = C.oracle_index_query(w, b)
        assert np.array_equal(idx[b], r[0]), f"query {b} ctx {w.ctx[b]}"


def test_index_all_ties_takes_lowest_indices(csa2):
    # qI = 0: every score is 0; more candidates than one workgroup holds, so
    # the whole-row exact select runs
    w = _edge([20000, 70000], topk=512)
    t = build_device(w, layers=0, with_kv=False)
    zero = torch.zeros_like(t["qI_full"])
    idx, pool = C.gpu_index_full(w, t, qI=zero, pool_blocks=2048)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    for b in range(2):
        assert np.array_equal(idx[b], np.arange(512))
        assert np.array_equal(pool[b], np.arange(2048))


def test_index_heavy_ties_narrow_values(csa2):
    # indexer values in [-1, 1]: scores take few distinct values
    w = _edge([30000, 12345], topk=512)
    t = build_device(w, layers=0, with_kv=False)
    n = sum(w.ctx) * w.row_width
    kI = torch.from_numpy(host_ints(77, 1, 0, n, -1, 1).reshape(-1, w.Hk, w.Di)).cuda()
    qI = torch.from_numpy(host_ints(77, 2, 0, w.B * w.Hi * w.Di, -1, 1).reshape(w.B, w.Hi, w.Di)).cuda()
    t["kI"] = kI
    idx, pool = C.gpu_index_full(w, t, qI=qI, pool_blocks=2048)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    kh, qh = kI.cpu().numpy(), qI.cpu().numpy()
    for b in range(w.B):
        off = int(w.seq_row_off[b])
        r, p = oracle.index_full(qh[b:b + 1], kh[off:off + w.ctx[b]], [0], [0], [w.ctx[b]], w.Hi,
                                 w.Hk, w.Di, 512, 2048, 8)
        assert np.array_equal(idx[b], r[0]) and np.array_equal(pool[b], p[0])


@pytest.mark.parametrize("bs", [1, 2, 4])
def test_pool_block_sizes(csa2, bs):
    w = _edge([9000, 3001], topk=64, pool_blocks=300, block_size=bs)
    t = build_device(w, layers=0, with_kv=False)
    idx, pool = C.gpu_index_full(w, t, pool_blocks=300)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    for b in range(w.B):
        r, p = C.oracle_index_query(w, b, pool_blocks=300)
        assert np.array_equal(idx[b], r[0]) and np.array_equal(pool[b], p[0])
    re = C.gpu_reindex(w, t, torch.from_numpy(pool).cuda(), qI=t["qI_full"], topk=64).cpu().numpy()
    for b in range(w.B):
        r = C.oracle_reindex_query(w, b, pool[b], tensor=T_QI_FULL, topk=64)
        assert np.array_equal(re[b], r[0])


def test_shared_key_head_and_narrow_rows(csa2):
    # Hk = 1 with Di = 256 (one key row shared by the 4 indexer heads), and
    # Hi x Di = 4 x 64 rows of 1 KB
    for kw in (dict(Hi=4, Hk=1, Di=256), dict(Hi=4, Hk=4, Di=64)):
        w = _edge([5000, 777], topk=128, **kw)
        t = build_device(w, layers=0, with_kv=False)
        idx, _ = C.gpu_index_full(w, t)
        idx = idx.cpu().numpy()
        for b in range(w.B):
            r, _ = C.oracle_index_query(w, b)
            assert np.array_equal(idx[b], r[0]), f"{kw} query {b}"


def test_index_is_deterministic(csa2):
    w = workload(3, small=True)
    t = build_device(w, layers=0, with_kv=False)
    a = [x.cpu() for x in C.gpu_index_full(w, t, pool_blocks=2048)]
    b = [x.cpu() for x in C.gpu_index_full(w, t, pool_blocks=2048)]
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("H", [16, 32, 48, 64, 80, 128])
def test_attention_heads_padding_and_short_windows(csa2, H):
    w = _edge([300, 50, 1000], H=H, topk=96, W=128)
    t = build_device(w, layers=1, with_kI=False)
    rng = np.random.default_rng(H)
    idx = np.full((w.B, w.topk), -1, np.int32)
    idx[0, :90] = np.sort(rng.choice(300, 90, replace=False))      # ragged tail of -1
    idx[1, :40] = np.arange(40)                                     # short sequence
    idx[2] = np.sort(rng.choice(1000, 96, replace=False))
    sl = torch.tensor([128, 50, 7], dtype=torch.int32, device="cuda")
    out, lse = C.gpu_attn(w, t, 0, torch.from_numpy(idx).cuda(), swa_len=sl)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b, s in zip(range(3), [128, 50, 7]):
        ro, rl = C.oracle_attn_query(w, b, 0, idx[b], swa_len=s)
        C.assert_attn_close(out[b], ro[0], f"H={H} query {b}")
        C.assert_lse_close(lse[b], rl[0], f"H={H} query {b}")


def test_attention_window_only_main_only_and_empty(csa2):
    w = _edge([400, 400], H=64, topk=32, W=128)
    t = build_device(w, layers=1, with_kI=False)
    none = torch.full((2, 32), -1, dtype=torch.int32, device="cuda")
    some = torch.from_numpy(np.tile(np.arange(0, 320, 10, dtype=np.int32), (2, 1))).cuda()
    cases = [(none, [128, 0], "window only / nothing"), (some, [0, 0], "main only")]
    for idx, sl, what in cases:
        out, lse = C.gpu_attn(w, t, 0, idx, swa_len=torch.tensor(sl, dtype=torch.int32, device="cuda"))
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        for b in range(2):
            ro, rl = C.oracle_attn_query(w, b, 0, idx[b].cpu().numpy(), swa_len=sl[b])
            C.assert_attn_close(out[b], ro[0], what)
            C.assert_lse_close(lse[b], rl[0], what)
    # no key at all: zeros and -inf
    out, lse = C.gpu_attn(w, t, 0, none, swa_len=torch.zeros(2, dtype=torch.int32, device="cuda"))
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_attention_is_deterministic(csa2):
    w = workload(1, small=True)
    t = build_device(w, layers=1, with_kI=False)
    rng = np.random.default_rng(5)
    idx = torch.from_numpy(np.stack([np.sort(rng.choice(w.ctx[0], 512, replace=False))
                                     for _ in range(w.B)]).astype(np.int32)).cuda()
    a = C.gpu_attn(w, t, 0, idx)
    b = C.gpu_attn(w, t, 0, idx)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_prefill_window_before_position_zero(csa2):
    w = Workload("edge_prefill", 9, "prefill", [40], H=16, topk=8, W=128, layers=1, p0=3, Qn=20,
                 m=2)
    t = build_device(w)
    idx, _ = C.gpu_index_full(w, t)
    idx_h = idx.cpu().numpy()
    kI = host_kI_rows(w, 0, w.ctx[0])
    ref, _ = oracle.index_full(host_qI(w, T_QI_FULL), kI, [0], np.zeros(w.Qn, np.int32),
                               w.q_nvis(), w.Hi, w.Hk, w.Di, w.topk)
    assert np.array_equal(idx_h, ref)
    out, lse = C.gpu_attn(w, t, 0, idx)
    ro, rl = C.oracle_prefill_rows(w, 0, ref, list(range(w.Qn)))
    C.assert_attn_close(out.cpu().numpy(), ro, "prefill near position 0")
    C.assert_lse_close(lse.cpu().numpy(), rl, "prefill near position 0")


def test_index_long_rows_filter_paths(csa2):
    # rows longer than one selecting workgroup reads: the multi-workgroup
    # filter + finalize, with heavy ties (values in [-1, 1]) and with all-equal
    # scores (the whole-row fallback)
    w = _edge([150000, 140001], topk=512)
    t = build_device(w, layers=0, with_kv=False)
    n = sum(w.ctx) * w.row_width
    kI = torch.from_numpy(host_ints(78, 1, 0, n, -1, 1).reshape(-1, w.Hk, w.Di)).cuda()
    qI = torch.from_numpy(host_ints(78, 2, 0, w.B * w.Hi * w.Di, -1, 1).reshape(w.B, w.Hi, w.Di)).cuda()
    t["kI"] = kI
    idx, pool = C.gpu_index_full(w, t, qI=qI, pool_blocks=2048)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    kh, qh = kI.cpu().numpy(), qI.cpu().numpy()
    for b in range(w.B):
        off = int(w.seq_row_off[b])
        r, p = oracle.index_full(qh[b:b + 1], kh[off:off + w.ctx[b]], [0], [0], [w.ctx[b]], w.Hi,
                                 w.Hk, w.Di, 512, 2048, 8)
        assert np.array_equal(idx[b], r[0]) and np.array_equal(pool[b], p[0]), f"query {b}"
    zero = torch.zeros_like(qI)
    idx, pool = C.gpu_index_full(w, t, qI=zero, pool_blocks=2048)
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(512), (2, 1)))
    assert np.array_equal(pool.cpu().numpy(), np.tile(np.arange(2048), (2, 1)))


def test_index_candidate_radix_paths(csa2):
    # integer scores in a narrow range put several hundred to a thousand keys
    # into the K-th key's histogram bin: the candidates are then picked by the
    # radix select (from global memory after the multi-workgroup filter for
    # the two long rows, from LDS in the one-workgroup select for the short
    # row and the block rows), and Top-2048 lists are ordered by the bitonic
    # sort
    w = _edge([200000, 70000, 60000], topk=2048)
    t = build_device(w, layers=0, with_kv=False)
    n = sum(w.ctx) * w.row_width
    kI = torch.from_numpy(host_ints(80, 1, 0, n, -2, 2).reshape(-1, w.Hk, w.Di)).cuda()
    qI = torch.from_numpy(host_ints(80, 2, 0, w.B * w.Hi * w.Di, -2, 2).reshape(w.B, w.Hi, w.Di)).cuda()
    t["kI"] = kI
    idx, pool = C.gpu_index_full(w, t, qI=qI, pool_blocks=2048)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    kh, qh = kI.cpu().numpy(), qI.cpu().numpy()
    for b in range(w.B):
        off = int(w.seq_row_off[b])
        r, p = oracle.index_full(qh[b:b + 1], kh[off:off + w.ctx[b]], [0], [0], [w.ctx[b]], w.Hi,
                                 w.Hk, w.Di, 2048, 2048, 8)
        assert np.array_equal(idx[b], r[0]), f"Top-K of query {b}"
        assert np.array_equal(pool[b], p[0]), f"pool of query {b}"


@pytest.mark.parametrize("order", ["random", "ascending", "holes"])
@pytest.mark.parametrize("case", ["top2048", "narrow", "ties", "signs"])
def test_reindex_select_paths(csa2, case, order):
    # Paths of the Reindex select beyond the common one (the K-th key's
    # histogram bin holding a few hundred keys, ranked directly): Top-2,048
    # (the long-list output sort); keys in [0, 2] against a 0/1 query (about
    # 2,300 keys in the K-th key's bin: radix pick in LDS); 0/1 keys against
    # an all-ones query (thousands tied: the radix select over all keys); key
    # rows turned so that all but about 2 % of the scores are negative or zero
    # (the K-th key far below the top one, across the sign).  Pools are
    # random distinct blocks, a short sequence's pool padded with -1, in
    # random order, in ascending order (the Full layer's order: the select
    # then writes the winners from a bitmap in candidate order when at most
    # 512 keys share the K-th key's bin), or ascending with empty slots
    # between valid ones (which must not take that path).
    w = _edge([140000, 30000, 9000, 700], topk=2048 if case == "top2048" else 512,
              pool_blocks=2048, block_size=8)
    topk = w.topk
    t = build_device(w, layers=0, with_kv=False)
    n = w.rows * w.row_width
    rng = np.random.default_rng([31, len(case)])
    if case == "ties":
        kh = host_ints(82, 1, 0, n, 0, 1).reshape(-1, w.Hk, w.Di)
        qh = np.ones((w.B, w.Hi, w.Di), np.float32)
    elif case == "narrow":
        kh = host_ints(82, 1, 0, n, 0, 2).reshape(-1, w.Hk, w.Di)
        qh = host_ints(82, 2, 0, w.B * w.Hi * w.Di, 0, 1).reshape(w.B, w.Hi, w.Di)
    else:
        kh = host_ints(82, 1, 0, n, -8, 8).reshape(-1, w.Hk, w.Di)
        qh = host_ints(82, 2, 0, w.B * w.Hi * w.Di, -8, 8).reshape(w.B, w.Hi, w.Di)
    if case == "signs":
        for b in range(w.B):
            off, nb = int(w.seq_row_off[b]), int(w.ctx[b])
            s = np.einsum("rd,d->r", kh[off:off + nb].reshape(nb, -1).astype(np.float64),
                          qh[b].reshape(-1).astype(np.float64))
            flip = (s > 0) & (rng.random(nb) >= 0.02)
            kh[off:off + nb][flip] *= -1.0
    pool = np.full((w.B, w.pool_blocks), -1, np.int32)
    for b in range(w.B):
        nblk = (int(w.ctx[b]) + w.block_size - 1) // w.block_size
        m = min(nblk, w.pool_blocks)
        row = rng.choice(nblk, m, replace=False)
        if order != "random":
            row = np.sort(row)
        pool[b, :m] = row
        if order == "holes" and m > 8:
            pool[b, rng.choice(m - 1, 4, replace=False)] = -1
    t["kI"] = torch.from_numpy(kh).cuda()
    re = C.gpu_reindex(w, t, torch.from_numpy(pool).cuda(), qI=torch.from_numpy(qh).cuda(),
                       topk=topk).cpu().numpy()
    for b in range(w.B):
        off = int(w.seq_row_off[b])
        r = oracle.reindex(qh[b:b + 1], kh[off:off + w.ctx[b]], [0], [0], [w.ctx[b]],
                           pool[b:b + 1], w.block_size, w.Hi, w.Hk, w.Di, topk)
        assert np.array_equal(re[b], r[0]), f"{case}, {order} pool: query {b} (ctx {w.ctx[b]})"


@pytest.mark.parametrize("bs", [3, 5, 16])
def test_reindex_other_block_sizes(csa2, bs):
    # Reindex accepts any positive block size (the Full layer's pools use 1,
    # 2, 4 or 8): candidate c is position c mod bs of pool block c / bs, here
    # for sizes that are not powers of two and for one above 8, with random
    # pools in random order, a short sequence's pool padded with -1.
    P = 16384 // bs if bs > 8 else 1000
    w = _edge([60000, 9000, 500], topk=512, pool_blocks=P, block_size=bs)
    t = build_device(w, layers=0, with_kv=False)
    rng = np.random.default_rng([41, bs])
    pool = np.full((w.B, P), -1, np.int32)
    for b in range(w.B):
        nblk = (int(w.ctx[b]) + bs - 1) // bs
        m = min(nblk, P)
        pool[b, :m] = rng.choice(nblk, m, replace=False)
    qh = host_qI(w, T_QI_FULL)
    re = C.gpu_reindex(w, t, torch.from_numpy(pool).cuda(), qI=t["qI_full"], topk=512).cpu().numpy()
    for b in range(w.B):
        off = int(w.seq_row_off[b])
        kh = host_kI_rows(w, off, int(w.ctx[b]))
        r = oracle.reindex(qh[b:b + 1], kh, [0], [0], [int(w.ctx[b])], pool[b:b + 1], bs, w.Hi,
                           w.Hk, w.Di, 512)
        assert np.array_equal(re[b], r[0]), f"block size {bs}: query {b} (ctx {w.ctx[b]})"


@pytest.mark.parametrize("split", ["both", "queries", "keys"])
@pytest.mark.parametrize("ctx,p0", [(3000, 4000), (12000, 20000)])
def test_prefill_indexer_general_fp32_inputs(csa2, split, ctx, p0):
    # values that are not exact in bf16 (on both sides, or on one side with
    # integers on the other) take the hi/lo split passes of the score GEMM.
    # Each score is within 2^-14 * sum_i |q_i k_i| of the exact one (the
    # dropped lo*lo term and the split's residual, each at most 2^-18 of a
    # product, and fp32 accumulation: at most 3 x 32 roundings of 16-product
    # MFMA steps, 96 * 2^-24 < 2^-17), so an entry the GPU picks
    # in place of the oracle's is within the sum of the two entries' bounds
    # of the K-th exact score.  The longer context puts the queries' visible
    # entries past the candidate lists' capacity, so the sampled thresholds
    # decide the lists.
    w = Workload("prefill_fp32", 11, "prefill", [ctx], topk=64, layers=0, p0=p0, Qn=40, m=2)
    t = build_device(w, with_kv=False, layers=0)
    kI = host_ints(79, 1, 0, w.rows * w.row_width).astype(np.float32).reshape(-1, w.Hk, w.Di)
    qI = host_ints(79, 2, 0, w.Qn * w.Hi * w.Di).astype(np.float32).reshape(w.Qn, w.Hi, w.Di)
    if split in ("both", "keys"):
        kI = (kI / 3.0).astype(np.float32)
    if split in ("both", "queries"):
        qI = (qI / 7.0).astype(np.float32)
    t["kI"] = torch.from_numpy(kI).cuda()
    idx, _ = C.gpu_index_full(w, t, qI=torch.from_numpy(qI).cuda())
    idx = idx.cpu().numpy()
    nv = w.q_nvis()
    assert nv.max() <= ctx
    ref, _ = oracle.index_full(qI, kI, [0], np.zeros(w.Qn, np.int32), nv, w.Hi, w.Hk, w.Di, w.topk)
    ka = np.abs(kI.astype(np.float64))
    for i in range(w.Qn):
        s = oracle.scores(qI, kI, [0], np.zeros(w.Qn, np.int32), nv, i, w.Hi, w.Hk, w.Di)
        n = int(nv[i])
        bound = 2.0 ** -14 * np.einsum("hd,nhd->n", np.abs(qI[i].astype(np.float64)), ka[:n])
        g = idx[i]
        k = min(w.topk, n)
        assert np.all(np.diff(g[g >= 0]) > 0) and np.all(g[:k] >= 0) and np.all(g[k:] == -1)
        kth = np.sort(s)[::-1][k - 1]
        gsel, rsel = set(g[g >= 0].tolist()), set(ref[i][ref[i] >= 0].tolist())
        bmax = bound.max()
        assert all(s[j] >= kth - bound[j] - bmax for j in gsel - rsel), f"query {i}"
        assert all(s[j] <= kth + bound[j] + bmax for j in rsel - gsel), f"query {i}"


def test_prefill_row_select_paths(csa2):
    # prefill rows are selected one workgroup per query: rows of up to 65,536
    # keys are read once and filtered against a sampled threshold, longer
    # rows (and rows whose threshold keeps too many keys) take the histogram
    # passes; integer scores with heavy ties and all-equal scores take the
    # fallbacks
    w = Workload("prefill_rows", 12, "prefill", [65600], topk=512, layers=0, p0=131059, Qn=34, m=2)
    nv = w.q_nvis()
    assert nv.min() < 65536 < nv.max()
    t = build_device(w, with_kv=False, layers=0)
    kI = t["kI"].cpu().numpy()
    for label, lo, hi in (("uniform [-8, 8]", -8, 8), ("ties [-1, 1]", -1, 1)):
        if lo == -8:
            qI = host_qI(w, T_QI_FULL)
        else:
            kI = host_ints(81, 1, 0, w.rows * w.row_width, lo, hi).reshape(-1, w.Hk, w.Di)
            qI = host_ints(81, 2, 0, w.Qn * w.Hi * w.Di, lo, hi).reshape(w.Qn, w.Hi, w.Di)
            t["kI"] = torch.from_numpy(kI).cuda()
        _say(f"[{w.name}] {label}")
        idx, _ = C.gpu_index_full(w, t, qI=torch.from_numpy(qI).cuda())
        ref, _ = oracle.index_full(qI, kI, [0], np.zeros(w.Qn, np.int32), nv, w.Hi, w.Hk, w.Di,
                                   w.topk)
        assert np.array_equal(idx.cpu().numpy(), ref), label
    zero = torch.zeros((w.Qn, w.Hi, w.Di), dtype=torch.float32, device="cuda")
    idx, _ = C.gpu_index_full(w, t, qI=zero)
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(512), (w.Qn, 1)))


@pytest.mark.parametrize("ctx,p0,m,zero_rows", [(4100, 7900, 2, (5, 299)),
                                                 (40300, 40000, 1, (130, 131, 299))])
def test_prefill_candidate_lists_and_exact_fallback(csa2, ctx, p0, m, zero_rows):
    # 300 queries (three query tiles, the last ragged).  A query with more
    # than 4,096 visible entries keeps a candidate list of the entries at or
    # above a threshold from sampled key tiles; a query whose scores all tie
    # (qI = 0) overflows its list and sends its query tile to the full-row
    # select, while the other tiles keep their lists
    w = Workload("prefill_cand", 14, "prefill", [ctx], topk=512, layers=0, p0=p0, Qn=300, m=m)
    nv = w.q_nvis()
    assert nv.max() <= ctx
    t = build_device(w, with_kv=False, layers=0)
    qI = host_qI(w, T_QI_FULL).copy()
    qI[list(zero_rows)] = 0.0
    idx, _ = C.gpu_index_full(w, t, qI=torch.from_numpy(qI).cuda())
    idx = idx.cpu().numpy()
    kI = host_kI_rows(w, 0, ctx)
    ref, _ = oracle.index_full(qI, kI, [0], np.zeros(w.Qn, np.int32), nv, w.Hi, w.Hk, w.Di, w.topk)
    for i in range(w.Qn):
        assert np.array_equal(idx[i], ref[i]), f"query {i} (nvis {nv[i]})"
    for i in zero_rows:
        assert np.array_equal(idx[i], np.arange(512)), f"all-tie query {i}"


def test_attention_largest_topk_and_window(csa2):
    # the largest Top-K list (2,048 entries, 64 main-KV tiles split across
    # workgroups) and the largest window (1,024 tokens), with a ragged tail
    w = _edge([5000, 2100], H=32, topk=2048, W=1024)
    t = build_device(w, layers=1, with_kI=False)
    rng = np.random.default_rng(11)
    idx = np.full((w.B, w.topk), -1, np.int32)
    idx[0] = np.sort(rng.choice(5000, 2048, replace=False))
    idx[1, :2000] = np.sort(rng.choice(2100, 2000, replace=False))
    sl = torch.tensor([1024, 700], dtype=torch.int32, device="cuda")
    out, lse = C.gpu_attn(w, t, 0, torch.from_numpy(idx).cuda(), swa_len=sl)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b, s in zip(range(2), [1024, 700]):
        ro, rl = C.oracle_attn_query(w, b, 0, idx[b], swa_len=s)
        C.assert_attn_close(out[b], ro[0], f"query {b}")
        C.assert_lse_close(lse[b], rl[0], f"query {b}")


def test_prefill_chunk_two_head_groups(csa2):
    # 128 heads (two 64-head groups per query) in the prefill form
    w = Workload("prefill_h128", 13, "prefill", [600], H=128, topk=64, W=128, layers=1, p0=1000,
                 Qn=24, m=2)
    t = build_device(w)
    idx, _ = C.gpu_index_full(w, t)
    ref, _ = oracle.index_full(host_qI(w, T_QI_FULL), host_kI_rows(w, 0, w.ctx[0]), [0],
                               np.zeros(w.Qn, np.int32), w.q_nvis(), w.Hi, w.Hk, w.Di, w.topk)
    assert np.array_equal(idx.cpu().numpy(), ref)
    out, lse = C.gpu_attn(w, t, 0, idx)
    ro, rl = C.oracle_prefill_rows(w, 0, ref, list(range(w.Qn)))
    C.assert_attn_close(out.cpu().numpy(), ro, "prefill, 128 heads")
    C.assert_lse_close(lse.cpu().numpy(), rl, "prefill, 128 heads")


@pytest.mark.parametrize("order", ["rising", "falling"])
def test_attention_rising_falling_and_peaky_logits(csa2, order):
    # Every head of a query sees the same key order: q[h] = c_h u with c_h > 0,
    # so sorting the Top-K row by u . k puts the logits of every head in rising
    # (or falling) order along the tiles and the key-range splits.  Rising
    # logits move the running maximum tile after tile (the deferred rescale
    # and the split merge with far-apart maxima); falling ones put the largest
    # logit first so that later probabilities underflow.  c_h spans 0.02 .. 4
    # (logits up to ~300): near-uniform to one-hot softmaxes in one launch.
    w = _edge([3000, 1500], topk=512, W=128)
    t = build_device(w, layers=1, with_kI=False)
    rng = np.random.default_rng(5)
    u = rng.standard_normal(w.D).astype(np.float32)
    c = np.geomspace(0.02, 4.0, w.H).astype(np.float32)
    q = np.broadcast_to(c[None, :, None] * u[None, None, :], (w.B, w.H, w.D)).copy()
    idx = np.full((w.B, w.topk), -1, np.int32)
    for b in range(w.B):
        off, n = int(w.seq_row_off[b]), int(w.ctx[b])
        codes, scales = host_kv_rows(w, off, n)
        logit = np.array([float(u.astype(np.float64) @ oracle.dequant_row(codes[r], scales[r], w.D))
                          for r in range(n)])
        pick = rng.choice(n, w.topk, replace=False)
        pick = pick[np.argsort(logit[pick], kind="stable")]
        idx[b] = pick if order == "rising" else pick[::-1]
        # premise: at the largest scale the top key outweighs the median one by e^20
        assert c[-1] * w.scale * (logit[pick[-1]] - logit[pick[w.topk // 2]]) > 20
    qd = torch.from_numpy(q).cuda()
    out = C.poison_f32((w.B, w.H, w.D))
    lse = C.poison_f32((w.B, w.H))
    buf = C.ws(csa2.csa2_decode_workspace_bytes(w.B, w.H, w.D, w.topk, w.W))
    csa2.csa2_sparse_attn_decode(qd, t["kv_codes"], t["kv_scales"], t["seq_row_off"],
                                 torch.from_numpy(idx).cuda(), t["swa_k"][0], t["swa_v"][0],
                                 t["swa_len"], w.scale, out, lse, buf)
    torch.cuda.synchronize()
    codes, scales = host_kv_rows(w, 0, w.rows)
    sk, sv = host_swa(w, 0)
    ro, rl = oracle.attn_decode(q, codes, scales, w.seq_row_off, idx, sk, sv, w.swa_len(), w.scale)
    C.assert_attn_close(out.cpu().numpy(), ro, f"{order} logits")
    C.assert_lse_close(lse.cpu().numpy(), rl, f"{order} logits")
