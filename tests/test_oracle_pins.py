"""Pins of the CPU oracle against what the pages, the format standards and
the mathematics fix (CPU only).

Each test checks the oracle against something other than itself: values from
the OCP format standards (golden files), torch's FP8 decoder, an int64
recomputation of the scores, the defining invariants of an exact Top-K
selection, closed forms of softmax attention in special cases, and a float64
textbook attention built from torch's softmax.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from gen import host_fp4, host_ints, host_pow2_scales

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


# --------------------------------------------------------------- codecs

def test_e2m1_all_codes_match_ocp_table():
    for code, val in _golden("e2m1_values.txt"):
        got = oracle.e2m1(int(code))
        assert got == float(val)
        assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_e4m3_spot_values_match_ocp_table():
    for byte, val in _golden("e4m3fn_spot.txt"):
        got = oracle.e4m3(int(byte, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_e4m3_all_256_match_torch_decoder():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert nan.sum() == 2  # 0x7F and 0xFF only


def test_scale_codes_are_powers_of_two():
    for k in range(-4, 5):
        assert oracle.e4m3((k + 7) << 3) == 2.0 ** k
    s = host_pow2_scales(7, 5, 0, 10000)
    vals = {oracle.e4m3(int(b)) for b in np.unique(s)}
    assert vals == {2.0 ** k for k in range(-4, 5)}


def test_fp4_generator_never_draws_negative_zero_and_covers_15_codes():
    b = host_fp4(3, 4, 0, 50000)
    nib = np.concatenate([b & 15, b >> 4])
    assert set(np.unique(nib).tolist()) == set(range(16)) - {8}


def test_row_bytes_fp4_vs_fp8():
    # 512 channels: 256 B of codes + 32 B of scales vs 512 B at FP8; the
    # review's "3) FP4 main KV" section says FP4 nearly halves the storage.
    D = 512
    fp4 = D // 2 + D // 16
    assert fp4 == 288 and 0.5 < fp4 / D < 0.6


def test_dequant_nibble_order_and_group_scale():
    D = 32
    codes = np.zeros(D // 2, np.uint8)
    codes[0] = 0x72          # channel 0 -> code 2 (1.0), channel 1 -> code 7 (6.0)
    codes[9] = 0xD5          # channel 18 -> code 5 (3.0), channel 19 -> code 13 (-3.0)
    scales = np.array([(1 + 7) << 3, (-2 + 7) << 3], np.uint8)   # 2, 0.25
    out = oracle.dequant_row(codes, scales, D)
    assert out[0] == 1.0 * 2 and out[1] == 6.0 * 2
    assert out[18] == 3.0 * 0.25 and out[19] == -3.0 * 0.25
    assert np.count_nonzero(out) == 4


# --------------------------------------------------------------- scores

@pytest.mark.parametrize("Hk", [4, 1])
def test_scores_equal_int64_recomputation(Hk):
    Hi, Di, n = 4, 64, 300
    kI = host_ints(11, 1, 0, n * Hk * Di).reshape(n, Hk, Di)
    qI = host_ints(11, 2, 0, Hi * Di).reshape(1, Hi, Di)
    s = oracle.scores(qI, kI, [0], [0], [n], 0, Hi, Hk, Di)
    ki = kI.astype(np.int64)
    qi = qI[0].astype(np.int64)
    ref = np.zeros(n, np.int64)
    for h in range(Hi):
        ref += ki[:, h % Hk, :] @ qi[h]
    assert np.array_equal(s, ref.astype(np.float64))
    assert np.abs(ref).max() <= Hi * Di * 64


# ------------------------------------------------------------ selection

def _check_topk_invariants(score, sel, k):
    """sel (ascending, -1 padded) is the unique top-k under (score desc, index asc)."""
    n = len(score)
    take = min(k, n)
    assert len(sel) == k
    chosen = sel[:take]
    assert np.all(sel[take:] == -1)
    assert np.all(chosen >= 0) and np.all(chosen < n)
    assert np.all(np.diff(chosen) > 0)  # ascending, no duplicates
    mask = np.zeros(n, bool)
    mask[chosen] = True
    if take < n:
        # weakest selected must beat strongest unselected
        s_sel, i_sel = score[mask], np.nonzero(mask)[0]
        s_un, i_un = score[~mask], np.nonzero(~mask)[0]
        worst = np.lexsort((-i_sel, s_sel))[0]          # lowest score, then highest index
        best = np.lexsort((i_un, -s_un))[0]             # highest score, then lowest index
        ws, wi, bs, bi = s_sel[worst], i_sel[worst], s_un[best], i_un[best]
        assert ws > bs or (ws == bs and wi < bi)


def _rand_full(seed, n, Hi=2, Hk=2, Di=8, lo=-2, hi=2):
    kI = host_ints(seed, 1, 0, n * Hk * Di, lo, hi).reshape(n, Hk, Di)
    qI = host_ints(seed, 2, 0, Hi * Di, lo, hi).reshape(1, Hi, Di)
    return qI, kI


@pytest.mark.parametrize("n,k", [(1, 4), (5, 4), (64, 4), (300, 17), (4096, 64), (2000, 2000)])
def test_topk_is_exact_selection(n, k):
    qI, kI = _rand_full(n + k, n)      # narrow value range: heavy ties
    idx, _ = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, k)
    s = oracle.scores(qI, kI, [0], [0], [n], 0, 2, 2, 8)
    _check_topk_invariants(s, idx[0], k)


def test_topk_brute_force_tiny():
    # every subset of size k of 7 entries: the oracle's pick is the unique one
    # whose members all outrank every non-member
    import itertools
    qI, kI = _rand_full(5, 7, lo=-1, hi=1)
    s = oracle.scores(qI, kI, [0], [0], [7], 0, 2, 2, 8)
    for k in range(1, 8):
        idx, _ = oracle.index_full(qI, kI, [0], [0], [7], 2, 2, 8, k)
        good = []
        for sub in itertools.combinations(range(7), k):
            rest = [t for t in range(7) if t not in sub]
            if all(s[a] > s[b] or (s[a] == s[b] and a < b) for a in sub for b in rest):
                good.append(sub)
        assert len(good) == 1
        assert tuple(idx[0]) == good[0]


def test_topk_all_ties_picks_lowest_indices():
    n, k = 1000, 64
    qI = np.zeros((1, 2, 8), np.float32)
    kI = host_ints(1, 1, 0, n * 16).reshape(n, 2, 8)
    idx, _ = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, k)
    assert np.array_equal(idx[0], np.arange(k))


def test_topk_respects_visibility_and_sequences():
    # two sequences packed back to back; query 1 sees only its first 50 rows
    qI, kI = _rand_full(9, 300)
    qI = np.concatenate([qI, qI])
    idx, _ = oracle.index_full(qI, kI, [0, 100], [0, 1], [100, 50], 2, 2, 8, 10)
    s1 = oracle.scores(qI, kI, [0, 100], [0, 1], [100, 50], 1, 2, 2, 8)
    _check_topk_invariants(s1, idx[1], 10)
    assert idx[1].max() < 50


def test_toy_example_modes():
    g = {r[0]: [int(x) for x in r[1:]] for r in _golden("toy_example.txt")}
    kI = np.array(g["keys"], np.float32).reshape(8, 1, 2)
    qf = np.array(g["full_query"], np.float32).reshape(1, 1, 2)
    qr = np.array(g["reindex_query"], np.float32).reshape(1, 1, 2)
    full, pool = oracle.index_full(qf, kI, [0], [0], [8], 1, 1, 2, 2, pool_blocks=8, block_size=1)
    assert full[0].tolist() == g["full_top2"]
    re = oracle.reindex(qr, kI, [0], [0], [8], pool, 1, 1, 1, 2, 2)
    assert re[0].tolist() == g["reindex_top2"]


# ----------------------------------------------------------------- pool

def test_pool_is_exact_block_selection():
    n, bs, P = 1003, 8, 20              # ragged last block
    qI, kI = _rand_full(21, n)
    idx, pool = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, 16, pool_blocks=P, block_size=bs)
    s = oracle.scores(qI, kI, [0], [0], [n], 0, 2, 2, 8)
    nb = (n + bs - 1) // bs
    bscore = np.maximum.reduceat(s, np.arange(0, n, bs))
    assert len(bscore) == nb
    _check_topk_invariants(bscore, pool[0], P)


def test_pool_with_unit_blocks_equals_topk():
    n = 500
    qI, kI = _rand_full(22, n)
    idx, pool = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, 37, pool_blocks=37, block_size=1)
    assert np.array_equal(idx, pool)


def test_pool_shorter_than_requested_is_padded():
    n = 50
    qI, kI = _rand_full(23, n)
    _, pool = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, 4, pool_blocks=2048, block_size=8)
    assert np.array_equal(pool[0, :7], np.arange(7)) and np.all(pool[0, 7:] == -1)


# -------------------------------------------------------------- reindex

def test_reindex_equals_full_topk_when_pool_holds_every_block():
    n, bs = 5000, 8
    qI, kI = _rand_full(31, n, lo=-8, hi=8)
    nb = (n + bs - 1) // bs
    full, pool = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, 512, pool_blocks=nb, block_size=bs)
    assert np.array_equal(pool[0], np.arange(nb))
    re = oracle.reindex(qI, kI, [0], [0], [n], pool, bs, 2, 2, 8, 512)
    assert np.array_equal(re, full)


def test_reindex_picks_only_pool_positions_and_bound():
    n, bs, P = 40000, 8, 2048
    qI, kI = _rand_full(32, n, lo=-8, hi=8)
    _, pool = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, 1, pool_blocks=P, block_size=bs)
    q2 = host_ints(32, 3, 0, 16, -8, 8).reshape(1, 2, 8)
    re = oracle.reindex(q2, kI, [0], [0], [n], pool, bs, 2, 2, 8, 512)
    cand = (pool[0][:, None] * bs + np.arange(bs)[None, :]).ravel()
    cand = cand[(cand >= 0) & (cand < n)]
    assert len(cand) <= 16384                       # 2,048 blocks x 8 positions
    assert set(re[0].tolist()) <= set(cand.tolist())
    s = oracle.scores(q2, kI, [0], [0], [n], 0, 2, 2, 8)
    sel = np.full(512, -1, np.int64)
    # invariants over the candidate set, with entry indices as tie-breakers
    order = np.argsort(cand)
    cs, ci = s[cand[order]], cand[order]
    pos = np.searchsorted(ci, re[0])
    assert np.array_equal(ci[pos], re[0])
    sel[:] = pos
    _check_topk_invariants(cs, sel.astype(np.int32), 512)


def test_reindex_skips_padding_and_invisible_tail():
    n, bs = 21, 8                                    # blocks 0,1 full, block 2 has 5 rows
    qI, kI = _rand_full(33, n)
    pool = np.array([[2, -1, -1]], np.int32)
    re = oracle.reindex(qI, kI, [0], [0], [n], pool, bs, 2, 2, 8, 8)
    assert np.array_equal(re[0], np.array([16, 17, 18, 19, 20, -1, -1, -1]))


# ------------------------------------------------------------ attention

def _kv(seed, rows, D):
    c = host_fp4(seed, 4, 0, rows * D // 2).reshape(rows, D // 2)
    s = host_pow2_scales(seed, 5, 0, rows * D // 16).reshape(rows, D // 16)
    return c, s


_E2M1 = np.array([float(v) for _, v in _golden("e2m1_values.txt")])


def _dequant_indep(codes, scales, D):
    """Dequantisation built from the golden E2M1 table and torch's FP8 decoder."""
    lo, hi = codes & 15, codes >> 4
    nib = np.stack([lo, hi], -1).reshape(codes.shape[0], D)
    sc = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return _E2M1[nib] * np.repeat(sc, 16, axis=1)


def _fp8(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _textbook(q, keys, vals, scale):
    """torch float64 softmax attention: q [H,D], keys/vals [n,D]."""
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(keys)
    vt = torch.from_numpy(vals)
    z = scale * (qt @ kt.T)
    p = torch.softmax(z, dim=-1)
    return (p @ vt).numpy(), torch.logsumexp(z, dim=-1).numpy()


def _swa(seed, B, W, D, layer=0):
    from gen import e4m3_bytes, normal_f32
    k = e4m3_bytes(normal_f32(seed, 32 + layer, (B, W, D)))
    v = e4m3_bytes(normal_f32(seed, 48 + layer, (B, W, D)))
    return k, v


@pytest.mark.parametrize("topk,swa_len", [(8, 5), (16, 0), (0, 7), (12, 12)])
def test_decode_attention_matches_textbook(topk, swa_len):
    B, H, D, W, rows = 2, 3, 64, 12, 40
    codes, scales = _kv(41, rows * B, D)
    q = np.random.default_rng(1).standard_normal((B, H, D)).astype(np.float32)
    rng = np.random.default_rng(2)
    idx = np.stack([np.sort(rng.choice(rows, topk, replace=False)) for _ in range(B)]).astype(np.int32)
    if topk:
        idx[1, -2:] = -1                                     # padding is skipped
    sk, sv = _swa(41, B, W, D)
    sl = np.array([swa_len, max(0, swa_len - 2)], np.int32)
    off = np.array([0, rows], np.int64)
    scale = 1 / math.sqrt(D)
    out, lse = oracle.attn_decode(q, codes, scales, off, idx.reshape(B, topk), sk, sv, sl, scale)
    for b in range(B):
        sel = [off[b] + t for t in idx[b] if t >= 0]
        main = _dequant_indep(codes[sel], scales[sel], D) if sel else np.zeros((0, D))
        keys = np.concatenate([main, _fp8(sk[b, :sl[b]])])
        vals = np.concatenate([main, _fp8(sv[b, :sl[b]])])
        if len(keys) == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        ref, rlse = _textbook(q[b], keys, vals, scale)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-5)
        np.testing.assert_allclose(lse[b], rlse, rtol=1e-6, atol=1e-5)


def _one_seq_case(topk=6, D=32, rows=20, W=4, H=2, seed=50):
    codes, scales = _kv(seed, rows, D)
    sk, sv = _swa(seed, 1, W, D)
    return codes, scales, sk, sv


def test_attention_single_key_returns_its_value_row():
    D = 32
    codes, scales, sk, sv = _one_seq_case(D=D)
    q = np.random.default_rng(3).standard_normal((1, 2, D)).astype(np.float32)
    out, lse = oracle.attn_decode(q, codes, scales, [0], np.array([[5, -1, -1]], np.int32),
                                  sk, sv, [0], 0.1)
    row = _dequant_indep(codes[5:6], scales[5:6], D)[0]
    assert np.array_equal(out[0, 0], row.astype(np.float32))
    assert np.array_equal(out[0, 1], row.astype(np.float32))
    # window-only single key: its V row
    out, _ = oracle.attn_decode(q, codes, scales, [0], np.zeros((1, 0), np.int32), sk, sv, [1], 0.1)
    assert np.array_equal(out[0, 0], _fp8(sv[0, 0]).astype(np.float32))


def test_attention_zero_query_is_mean_of_values():
    D = 32
    codes, scales, sk, sv = _one_seq_case(D=D)
    q = np.zeros((1, 1, D), np.float32)
    idx = np.array([[1, 4, 9]], np.int32)
    out, lse = oracle.attn_decode(q, codes, scales, [0], idx, sk, sv, [4], 0.5)
    vals = np.concatenate([_dequant_indep(codes[[1, 4, 9]], scales[[1, 4, 9]], D), _fp8(sv[0, :4])])
    np.testing.assert_allclose(out[0, 0], vals.mean(0), rtol=0, atol=1e-6)
    assert abs(lse[0, 0] - math.log(7)) < 1e-6


def test_attention_is_invariant_to_index_order():
    D = 64
    codes, scales, sk, sv = _one_seq_case(D=D, rows=30)
    q = np.random.default_rng(4).standard_normal((1, 4, D)).astype(np.float32)
    idx = np.array([[3, 7, 11, 20, 29, -1]], np.int32)
    a, _ = oracle.attn_decode(q, codes, scales, [0], idx, sk, sv, [3], 0.125)
    b, _ = oracle.attn_decode(q, codes, scales, [0], idx[:, [5, 4, 0, 2, 1, 3]], sk, sv, [3], 0.125)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-6)


def test_attention_large_logit_gap_is_one_hot():
    D = 32
    codes, scales, sk, sv = _one_seq_case(D=D)
    rows = _dequant_indep(codes, scales, D)
    q = (rows[7] * 50).astype(np.float32).reshape(1, 1, D)   # aligns with row 7 only
    idx = np.array([[2, 7, 13]], np.int32)
    z = rows[[2, 7, 13]] @ q[0, 0].astype(np.float64)
    assert z[1] - max(z[0], z[2]) > 200
    out, _ = oracle.attn_decode(q, codes, scales, [0], idx, sk, sv, [0], 1.0)
    np.testing.assert_allclose(out[0, 0], rows[7], rtol=0, atol=1e-12)


def test_reuse_layer_attends_over_the_full_layers_selection():
    # a Reuse layer = attention with the Full layer's indices and KV as they
    # are, plus its own query and window; it equals textbook attention over
    # exactly the Full layer's set
    n, D, H, W = 600, 64, 2, 6
    qI, kI = _rand_full(60, n, lo=-8, hi=8)
    full, _ = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, 16)
    codes, scales = _kv(60, n, D)
    sk, sv = _swa(60, 1, W, D, layer=2)
    q = np.random.default_rng(61).standard_normal((1, H, D)).astype(np.float32)
    out, _ = oracle.attn_decode(q, codes, scales, [0], full, sk, sv, [W], 0.125)
    main = _dequant_indep(codes[full[0]], scales[full[0]], D)
    ref, _ = _textbook(q[0], np.concatenate([main, _fp8(sk[0])]),
                       np.concatenate([main, _fp8(sv[0])]), 0.125)
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-5)


# -------------------------------------------------------------- prefill

@pytest.mark.parametrize("p0", [0, 3, 50])
def test_prefill_row_equals_decode_with_window_ending_at_p(p0):
    Qn, H, D, W, n, topk = 7, 2, 32, 5, 40, 4
    codes, scales = _kv(70, n, D)
    rng = np.random.default_rng(71)
    q = rng.standard_normal((Qn, H, D)).astype(np.float32)
    idx = np.stack([np.sort(rng.choice(n, topk, replace=False)) for _ in range(Qn)]).astype(np.int32)
    from gen import e4m3_bytes
    sk = e4m3_bytes(rng.standard_normal((Qn + W - 1, D)).astype(np.float32))
    sv = e4m3_bytes(rng.standard_normal((Qn + W - 1, D)).astype(np.float32))
    out, lse = oracle.attn_prefill(q, p0, codes, scales, idx, sk, sv, W, 0.2)
    for i in range(Qn):
        p = p0 + i
        # window rows i..i+W-1 hold positions p-W+1..p; keep positions >= 0
        rows = [r for r in range(i, i + W) if p0 - W + 1 + r >= 0]
        assert len(rows) == min(W, p + 1)
        o, l = oracle.attn_decode(q[i:i + 1], codes, scales, [0], idx[i:i + 1],
                                  sk[rows][None], sv[rows][None], [len(rows)], 0.2)
        np.testing.assert_array_equal(out[i], o[0])
        np.testing.assert_array_equal(lse[i], l[0])


def test_prefill_visibility_rule_m2():
    # entry j covers tokens 2j, 2j+1 and is visible at position p iff 2j+1 <= p
    from gen.workloads import workload
    w = workload(2, small=True)
    nv = w.q_nvis()
    p = w.p0 + np.arange(w.Qn)
    for pi, n in zip(p, nv):
        assert 2 * (n - 1) + 1 <= pi and not (2 * n + 1 <= pi)


# ------------------------------------------------------ FP4 main-KV writer

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _dequant_rows(codes, scales):
    return np.stack([oracle.dequant_row(codes[r], scales[r], codes.shape[1] * 2)
                     for r in range(codes.shape[0])])


def test_fp4_writer_round_trips_every_grid_row():
    # rows that are exactly representable (each group holds a +-6 value, so
    # its scale is recovered) come back with the same codes and scales
    rng = np.random.default_rng(31)
    R, D = 64, 512
    nonneg0 = np.array([c for c in range(16) if c != 8], np.uint8)
    nib = rng.choice(nonneg0, size=(R, D))
    nib[:, ::16] = rng.choice([7, 15], size=(R, D // 16))   # one +-6 per group
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(1, 127, size=(R, D // 16)).astype(np.uint8)
    x = _dequant_rows(codes, scales).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), _dequant_rows(codes, scales))   # exact in fp32
    c2, s2 = oracle.fp4_quantize_rows(x)
    assert np.array_equal(s2, scales)
    assert np.array_equal(c2, codes)


def test_fp4_writer_scale_is_the_smallest_that_covers_the_group():
    rng = np.random.default_rng(32)
    R, D = 96, 256
    mags = 10.0 ** rng.uniform(-4, 4, size=(R, 1))
    x = (rng.standard_normal((R, D)) * mags).astype(np.float32)
    x[0] = 0.0                    # all-zero row
    x[1, :16] = 1e5               # saturating group
    _, s = oracle.fp4_quantize_rows(x)
    e4 = np.array([oracle.e4m3(b) for b in range(127)])
    for r in range(R):
        for g in range(D // 16):
            amax = np.abs(x[r, 16 * g:16 * g + 16].astype(np.float64)).max()
            b = int(s[r, g])
            if amax == 0.0:
                assert b == 0
            elif amax > 6 * 448:
                assert b == 0x7E
            else:
                assert 1 <= b <= 0x7E and 6 * e4[b] >= amax and (b == 1 or 6 * e4[b - 1] < amax)


def test_fp4_writer_picks_the_nearest_grid_value():
    # brute force: the decoded value is a nearest point of the group's grid
    # {+-m * s}; a tie goes to the even magnitude code
    rng = np.random.default_rng(33)
    R, D = 128, 256
    x = (rng.standard_normal((R, D)) * 10.0 ** rng.uniform(-3, 3, size=(R, 1))).astype(np.float32)
    codes, scales = oracle.fp4_quantize_rows(x)
    y = _dequant_rows(codes, scales)
    for r in range(R):
        for g in range(D // 16):
            s = oracle.e4m3(int(scales[r, g]))
            xs = x[r, 16 * g:16 * g + 16].astype(np.float64)
            d = np.abs(np.abs(xs)[:, None] - E2M1_MAG[None, :] * s)
            best = d.min(axis=1)
            got = np.abs(np.abs(y[r, 16 * g:16 * g + 16]) - np.abs(xs))
            assert np.array_equal(got, best)
            assert np.all(np.sign(y[r, 16 * g:16 * g + 16]) * np.sign(xs) >= 0)


def test_fp4_writer_ties_go_to_the_even_code_and_no_negative_zero():
    # a group with scale 1 (one value 6): the other 15 sit on midpoints
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    even_choice = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]   # the even neighbour of each midpoint
    row = np.zeros(16, np.float32)
    row[0] = 6.0
    for i, m in enumerate(mids):
        row[1 + 2 * i] = m
        row[2 + 2 * i] = -m
    row[15] = -1e-9                                    # rounds to 0: code 0, not -0
    codes, scales = oracle.fp4_quantize_rows(row[None])
    assert oracle.e4m3(int(scales[0, 0])) == 1.0
    y = _dequant_rows(codes, scales)[0]
    for i, m in enumerate(mids):
        assert y[1 + 2 * i] == even_choice[i] and y[2 + 2 * i] == -even_choice[i]
    assert (codes[0, 7] >> 4) == 0


# ------------------------------------------------- FP8 window ring writer

def _e4m3_values():
    return _fp8(np.arange(256, dtype=np.uint8))


def test_e4m3_encode_matches_torch_cast_in_range():
    # torch's CPU cast to float8_e4m3fn rounds to nearest even; within the
    # finite rounding range (|x| < 464) the oracle must agree with it exactly
    rng = np.random.default_rng(61)
    x = (rng.standard_normal(6000) * np.exp2(rng.uniform(-14, 9, 6000))).astype(np.float32)
    vals = _e4m3_values()[:127]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)     # exact in fp32
    edges = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                            np.nextafter(mids, np.float32(1e9)), vals.astype(np.float32)])
    x = np.concatenate([x, edges, -edges, [0.0, -0.0, 1e-30, -1e-30, 463.99, -463.99]])
    x = x[np.abs(x) < 464].astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), want)


def test_e4m3_encode_saturates_and_keeps_sign():
    x = np.array([464, 480, 1e6, 3.4e38, -464, -1e30, 448, -448], np.float32)
    assert oracle.e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7E, 0xFE]
    # a negative value that rounds to zero keeps its sign; ties between 0 and
    # the smallest subnormal 2^-9 go to 0 (even)
    x = np.array([-1e-6, 1e-6, 2 ** -10, -(2 ** -10), 3 * 2 ** -11], np.float32)
    assert oracle.e4m3_encode(x).tolist() == [0x80, 0x00, 0x00, 0x80, 0x01]


def test_e4m3_encode_is_a_nearest_value():
    # brute force independent of the oracle's loop: the decoded byte is at a
    # minimal distance from x among all finite E4M3 values
    rng = np.random.default_rng(62)
    x = (rng.standard_normal(3000) * np.exp2(rng.uniform(-12, 8, 3000))).astype(np.float32)
    got = _fp8(oracle.e4m3_encode(x))
    vals = _e4m3_values()
    fin = vals[np.isfinite(vals)]
    dist = np.abs(np.abs(x.astype(np.float64))[:, None] - np.abs(fin)[None, :]).min(axis=1)
    assert np.array_equal(np.abs(np.abs(got) - np.abs(x.astype(np.float64))), dist)
    assert np.all((got == 0) | (np.sign(got) == np.sign(x)))


def test_swa_ring_holds_the_last_w_tokens():
    B, W, D, T = 2, 5, 32, 13
    rng = np.random.default_rng(63)
    k = rng.standard_normal((T, B, D)).astype(np.float32)
    v = rng.standard_normal((T, B, D)).astype(np.float32)
    sk = np.zeros((B, W, D), np.uint8)
    sv = np.zeros((B, W, D), np.uint8)
    start = np.array([0, 3], np.int64)            # sequence 1 starts at position 3
    for t in range(T):
        oracle.swa_append(k[t], v[t], start + t, sk, sv)
        for b in range(B):
            n = min(W, t + 1)
            held = sorted(sk[b, (start[b] + t - j) % W].tobytes() for j in range(n))
            want = sorted(oracle.e4m3_encode(k[t - j, b]).tobytes() for j in range(n))
            assert held == want
            assert np.array_equal(sv[b, (start[b] + t) % W], oracle.e4m3_encode(v[t, b]))


def test_swa_ring_negative_position_appends_nothing():
    # a sequence with no token at this step (negative position) keeps its ring
    B, W, D = 3, 4, 16
    rng = np.random.default_rng(64)
    sk = rng.integers(0, 256, (B, W, D)).astype(np.uint8)
    sv = rng.integers(0, 256, (B, W, D)).astype(np.uint8)
    k0, v0 = sk.copy(), sv.copy()
    k = rng.standard_normal((B, D)).astype(np.float32)
    v = rng.standard_normal((B, D)).astype(np.float32)
    oracle.swa_append(k, v, np.array([-1, 6, -5], np.int64), sk, sv)
    for b in (0, 2):
        assert np.array_equal(sk[b], k0[b]) and np.array_equal(sv[b], v0[b])
    assert np.array_equal(sk[1, 2], oracle.e4m3_encode(k[1]))
    assert np.array_equal(sk[1, [0, 1, 3]], k0[1, [0, 1, 3]])


def test_attention_over_the_ring_equals_the_window_in_position_order():
    # a window-only (K = 0) layer over the ring after 11 appends with W = 4
    # equals the same layer with the last 4 tokens laid out in position order
    B, H, W, D, T = 1, 3, 4, 32, 11
    rng = np.random.default_rng(64)
    k = rng.standard_normal((T, 1, D)).astype(np.float32)
    v = rng.standard_normal((T, 1, D)).astype(np.float32)
    sk = np.zeros((B, W, D), np.uint8)
    sv = np.zeros((B, W, D), np.uint8)
    for t in range(T):
        oracle.swa_append(k[t], v[t], np.array([t], np.int64), sk, sv)
    lin_k = np.stack([oracle.e4m3_encode(k[t, 0]) for t in range(T - W, T)])[None]
    lin_v = np.stack([oracle.e4m3_encode(v[t, 0]) for t in range(T - W, T)])[None]
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    codes = np.zeros((1, D // 2), np.uint8)
    scales = np.zeros((1, D // 16), np.uint8)
    none = np.zeros((B, 0), np.int32)
    off = np.zeros(1, np.int64)
    sl = np.array([W], np.int32)
    o1, l1 = oracle.attn_decode(q, codes, scales, off, none, sk, sv, sl, 0.2)
    o2, l2 = oracle.attn_decode(q, codes, scales, off, none, lin_k, lin_v, sl, 0.2)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)
    ref, rl = _textbook(q[0], _fp8(lin_k[0]), _fp8(lin_v[0]), 0.2)
    np.testing.assert_allclose(o1[0], ref, rtol=0, atol=1e-5)


# ------------------------------------------------- compact (E4M3) indexer keys

def _e4m3_bytes_of(x):
    """fp32 values -> E4M3FN bytes with torch's cast (exact for the integers used here)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_decode_torch(b):
    return torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def test_integer_keys_are_exact_in_e4m3():
    v = np.arange(-16, 17, dtype=np.float32)
    assert np.array_equal(_e4m3_decode_torch(_e4m3_bytes_of(v)), v.astype(np.float64))


@pytest.mark.parametrize("Hk", [4, 1])
def test_e4m3_key_scores_equal_int64_recomputation(Hk):
    Hi, Di, n = 4, 64, 300
    kI = host_ints(12, 1, 0, n * Hk * Di).reshape(n, Hk, Di)
    qI = host_ints(12, 2, 0, Hi * Di).reshape(1, Hi, Di)
    k8 = _e4m3_bytes_of(kI)
    assert k8.dtype == np.uint8 and k8.shape == (n, Hk, Di)
    s = oracle.scores(qI, k8, [0], [0], [n], 0, Hi, Hk, Di)
    ki, qi = kI.astype(np.int64), qI[0].astype(np.int64)
    ref = np.zeros(n, np.int64)
    for h in range(Hi):
        ref += ki[:, h % Hk, :] @ qi[h]
    assert np.array_equal(s, ref.astype(np.float64))


def test_e4m3_key_scores_over_every_finite_value():
    # random bytes over all 254 finite E4M3FN values (subnormals, 448, both
    # zeros) against general fp32 queries: a float64 sum of torch's decodes
    rng = np.random.default_rng(5)
    Hi, Hk, Di, n = 2, 2, 128, 64
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    k8 = rng.choice(finite, size=(n, Hk, Di)).astype(np.uint8)
    k8[0, 0, :] = finite[:128]
    k8[0, 1, :] = finite[126:]
    qI = rng.standard_normal((1, Hi, Di)).astype(np.float32)
    s = oracle.scores(qI, k8, [0], [0], [n], 0, Hi, Hk, Di)
    kd = _e4m3_decode_torch(k8)
    ref = np.einsum("nhd,hd->n", kd, qI[0].astype(np.float64))
    assert np.allclose(s, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


def test_e4m3_keys_select_as_the_fp32_keys_they_encode():
    # packed sequences, partial visibility, Top-K, pool and Reindex
    Hi, Hk, Di = 4, 4, 64
    ctx = [3000, 1500, 777]
    off = np.concatenate([[0], np.cumsum(ctx)[:-1]]).astype(np.int64)
    rows = int(np.sum(ctx))
    kI = host_ints(13, 1, 0, rows * Hk * Di).reshape(rows, Hk, Di)
    qI = host_ints(13, 2, 0, 3 * Hi * Di).reshape(3, Hi, Di)
    k8 = _e4m3_bytes_of(kI)
    nvis = [3000, 1200, 777]
    a = oracle.index_full(qI, kI, off, [0, 1, 2], nvis, Hi, Hk, Di, 64, pool_blocks=40,
                          block_size=8)
    b = oracle.index_full(qI, k8, off, [0, 1, 2], nvis, Hi, Hk, Di, 64, pool_blocks=40,
                          block_size=8)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    q2 = host_ints(13, 3, 0, 3 * Hi * Di).reshape(3, Hi, Di)
    ra = oracle.reindex(q2, kI, off, [0, 1, 2], nvis, a[1], 8, Hi, Hk, Di, 64)
    rb = oracle.reindex(q2, k8, off, [0, 1, 2], nvis, a[1], 8, Hi, Hk, Di, 64)
    assert np.array_equal(ra, rb)
    for q in range(3):
        s = oracle.scores(qI, k8, off, [0, 1, 2], nvis, q, Hi, Hk, Di)
        _check_topk_invariants(s, b[0][q], 64)


def test_e4m3_key_topk_invariants_on_general_values():
    rng = np.random.default_rng(6)
    Hi, Hk, Di, n, k = 4, 1, 64, 2000, 100
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    k8 = rng.choice(finite, size=(n, Hk, Di)).astype(np.uint8)
    qI = rng.standard_normal((1, Hi, Di)).astype(np.float32)
    idx, _ = oracle.index_full(qI, k8, [0], [0], [n], Hi, Hk, Di, k)
    kd = _e4m3_decode_torch(k8)[:, 0, :]
    s = kd @ qI[0].astype(np.float64).sum(axis=0)
    _check_topk_invariants(s, idx[0], k)


# ------------------------------------------------------------ pool variants

def test_pool_sum_rule_is_exact_block_selection():
    # variant block score: the sum of the block's visible entries (ragged
    # last block sums fewer entries)
    n, bs, P = 1003, 8, 20
    qI, kI = _rand_full(24, n)
    _, pool = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, 16, pool_blocks=P, block_size=bs,
                                block_rule="sum")
    s = oracle.scores(qI, kI, [0], [0], [n], 0, 2, 2, 8)
    bsum = np.add.reduceat(s, np.arange(0, n, bs))
    _check_topk_invariants(bsum, pool[0], P)
    _, pmax = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, 16, pool_blocks=P, block_size=bs)
    assert not np.array_equal(pool, pmax)          # the two rules differ on these inputs


def test_pool_sum_rule_with_unit_blocks_equals_topk():
    n = 500
    qI, kI = _rand_full(25, n)
    idx, pool = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, 37, pool_blocks=37,
                                  block_size=1, block_rule="sum")
    assert np.array_equal(idx, pool)


@pytest.mark.parametrize("bs,lo,hi", [(8, -1, 1), (8, -8, 8), (4, -2, 2), (2, -1, 1)])
def test_pool_of_widened_top_entries_equals_max_rule(bs, lo, hi):
    # the other reading of "blocks x positions": walk the entries in rank
    # order (score desc, index asc) and take the block of each until P
    # distinct blocks are held.  A block enters at its best entry, so this is
    # the max rule with ties to the lower block id, heavy ties included
    n, P = 777, 40
    qI, kI = _rand_full(26 + bs, n, lo=lo, hi=hi)
    s = oracle.scores(qI, kI, [0], [0], [n], 0, 2, 2, 8)
    order = np.lexsort((np.arange(n), -s))
    held = []
    for t in order:
        b = t // bs
        if b not in held:
            held.append(b)
        if len(held) == P:
            break
    _, pool = oracle.index_full(qI, kI, [0], [0], [n], 2, 2, 8, 1, pool_blocks=P, block_size=bs)
    assert pool[0].tolist() == sorted(held)
