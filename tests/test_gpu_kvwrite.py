"""GPU parity of the KV writers with the oracle.

FP4 main-KV writer (csa2_kv_quantize_fp4): E2M1 codes and E4M3 scale bytes
bit-exact, on random rows spanning every scale byte, on rows built around the
rounding boundaries, at the prefill context's size and at 1M rows (sampled).
FP8 window ring (csa2_swa_append): ring bytes bit-exact, and a window-only
layer over the ring within the attention tolerance."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gen import kv_rows_f32  # noqa: E402

T_KV_F32 = 9001   # generator stream of the writer's fp32 rows


@pytest.fixture(scope="module")
def csa2():
    assert torch.cuda.is_available(), "needs an MI355X"
    import compressed_fp4_kv_amd as m
    return m


def _say(*a):
    print(*a, flush=True)


def _run(csa2, x):
    R, D = x.shape
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    codes = torch.full((R, D // 2), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((R, D // 16), 0xAB, dtype=torch.uint8, device="cuda")
    csa2.csa2_kv_quantize_fp4(xd, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _check(csa2, x, what):
    codes, scales = _run(csa2, x)
    ec, es = oracle.fp4_quantize_rows(x)
    bad_s = np.argwhere(scales != es)
    assert bad_s.size == 0, f"{what}: scale bytes differ at {bad_s[:5].tolist()}"
    bad_c = np.argwhere(codes != ec)
    assert bad_c.size == 0, f"{what}: code bytes differ at {bad_c[:5].tolist()}"
    return codes, scales


@pytest.mark.parametrize("rows,D", [(1, 16), (3, 48), (257, 128), (3001, 512)])
def test_kv_writer_matches_oracle(csa2, rows, D):
    _say(f"kv writer rows={rows} D={D}")
    x = kv_rows_f32(11, T_KV_F32, rows, D)
    _, scales = _check(csa2, x, f"rows={rows} D={D}")
    if rows * D >= 1 << 20:
        # the draw reaches the subnormal scales, ordinary ones and saturation
        assert scales.min() <= 7 and scales.max() == 0x7E


def _e4m3(b):
    return np.float32(oracle.e4m3(b))


def test_kv_writer_boundaries(csa2):
    """Groups at the decisions' edges: every midpoint between E2M1 values for
    several scales (ties), one ulp either side of them, largest magnitudes at
    and one ulp above 6 x scale, all-zero and negative-zero groups, fp32
    subnormal inputs and saturation beyond 6 x 448."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    groups = []
    for b in (1, 2, 7, 8, 9, 0x30, 0x38, 0x3B, 0x55, 0x7D, 0x7E):
        s = _e4m3(b)
        six = np.float32(6) * s
        for k in range(7):
            m = mids[k] * s
            for v in (m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(np.inf))):
                g = np.zeros(16, np.float32)
                g[0] = six
                g[1], g[2], g[3] = v, -v, v
                g[4:11] = mids * s
                g[11:] = -mids[:5] * s
                groups.append(g)
        up = np.full(16, np.nextafter(six, np.float32(np.inf)), np.float32)
        up[1::2] *= -1
        groups.append(up)
        groups.append(np.linspace(-six, six, 16).astype(np.float32))
    groups.append(np.zeros(16, np.float32))
    groups.append(np.full(16, -0.0, np.float32))
    tiny = np.array([2 ** -149, -2 ** -149, 2 ** -140, 0, 1e-40, -3e-39, 2 ** -127, 0] * 2,
                    np.float32)
    groups.append(tiny)
    big = np.array([2688, -2688, 2689, 3000, 1e6, -1e30, 3.4e38, 448, -5, 0.1] + [0] * 6,
                   np.float32)
    groups.append(big)
    x = np.stack(groups).reshape(-1, 32) if len(groups) % 2 == 0 else \
        np.concatenate([np.stack(groups), np.zeros((1, 16), np.float32)]).reshape(-1, 32)
    _say(f"kv writer boundary groups={len(groups)}")
    _check(csa2, x, "boundaries")


def test_kv_writer_round_trip(csa2):
    """Rows whose every group holds a +-6 x s element and other E2M1 grid
    values times s decode back to themselves exactly."""
    rng = np.random.default_rng([5, 77])
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    R, D = 64, 512
    g = R * D // 16
    sb = rng.integers(1, 127, size=g)
    s = np.array([_e4m3(b) for b in sb], np.float32)
    vals = grid[rng.integers(0, 8, size=(g, 16))] * np.where(rng.random((g, 16)) < 0.5, -1, 1)
    vals[np.arange(g), rng.integers(0, 16, size=g)] = 6 * np.where(rng.random(g) < 0.5, -1, 1)
    x = (vals.astype(np.float32) * s[:, None]).reshape(R, D)
    codes, scales = _check(csa2, x, "grid rows")
    assert np.array_equal(scales.reshape(-1), sb.astype(np.uint8))
    e2 = np.array([oracle.e2m1(c) for c in range(16)], np.float64)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(R, D)
    dec = e2[nib] * np.repeat(s.reshape(R, D // 16), 16, axis=1)
    assert np.array_equal(dec, x.astype(np.float64))


def test_kv_writer_prefill_context(csa2):
    """The prefill context's main KV at once: 65,536 rows x 512 channels."""
    _say("kv writer rows=65536 D=512")
    x = kv_rows_f32(2, T_KV_F32, 65536, 512)
    _check(csa2, x, "65,536 rows")


def test_kv_writer_argument_checks(csa2):
    dev = "cuda"
    codes = torch.empty((4, 12), dtype=torch.uint8, device=dev)
    scales = torch.empty((4, 1), dtype=torch.uint8, device=dev)
    with pytest.raises(csa2.CSA2Error):        # D not a multiple of 16
        csa2.csa2_kv_quantize_fp4(torch.zeros((4, 24), device=dev), codes, scales)
    flat = torch.zeros(4 * 32 + 1, device=dev)
    c32 = torch.empty((4, 16), dtype=torch.uint8, device=dev)
    s32 = torch.empty((4, 2), dtype=torch.uint8, device=dev)
    with pytest.raises(csa2.CSA2Error):        # x not 16-byte aligned
        csa2.csa2_kv_quantize_fp4(flat[1:].view(4, 32), c32, s32)
    e = torch.empty((0, 32), device=dev)
    csa2.csa2_kv_quantize_fp4(e, c32[:0], s32[:0])   # no rows: nothing to do
    torch.cuda.synchronize()


def test_kv_writer_random_bit_patterns(csa2):
    """Groups led by a random finite fp32 bit pattern (any exponent), the
    other 15 values uniform multiples of it."""
    rng = np.random.default_rng([6, 11])
    n = 1 << 17
    lead = rng.integers(1, 0x7F7FFFFF, size=n, dtype=np.uint32).view(np.float32)
    x = np.empty((n, 16), np.float32)
    x[:, 0] = lead * np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32)
    x[:, 1:] = lead[:, None] * rng.uniform(-1, 1, size=(n, 15)).astype(np.float32)
    _say(f"kv writer random bit patterns groups={n}")
    _check(csa2, x.reshape(-1, 512), "random bit patterns")


def test_kv_writer_million_rows_sampled(csa2):
    """1,048,576 rows x 512 channels in one launch (the size the writer's
    bandwidth is measured at), checked on the first, the last and 4,096
    random rows."""
    rows, D = 1 << 20, 512
    _say(f"kv writer rows={rows} D={D} (sampled)")
    base = torch.from_numpy(kv_rows_f32(3, T_KV_F32, 65536, D)).cuda()
    x = base.repeat(rows // 65536, 1)
    codes = torch.full((rows, D // 2), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, D // 16), 0xAB, dtype=torch.uint8, device="cuda")
    csa2.csa2_kv_quantize_fp4(x, codes, scales)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    pick = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 4096)]))
    sel = torch.from_numpy(pick).cuda()
    xs = x[sel].cpu().numpy()
    ec, es = oracle.fp4_quantize_rows(xs)
    assert np.array_equal(scales[sel].cpu().numpy(), es)
    assert np.array_equal(codes[sel].cpu().numpy(), ec)


# ------------------------------------------------------------ window ring

def _fp8_edges():
    """E4M3 values, midpoints between neighbours and one ulp either side,
    saturation, tiny values and signed zeros, all as fp32."""
    vals = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    e = np.concatenate([vals.astype(np.float32), mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1e9)),
                        np.array([448, 460, 464, 465, 480, 1e6, 3.4e38, 1e-30, 2 ** -10,
                                  2 ** -149, 0.0], np.float32)])
    return np.concatenate([e, -e]).astype(np.float32)


def test_swa_append_matches_oracle(csa2):
    """One token per sequence into rings that already hold bytes: only slot
    pos mod W changes, with the oracle's E4M3 bytes; a negative position
    changes nothing."""
    B, W, D = 37, 128, 512
    rng = np.random.default_rng([7, 1])
    k = (rng.standard_normal((B, D)) * np.exp2(rng.uniform(-14, 10, (B, 1)))).astype(np.float32)
    v = (rng.standard_normal((B, D)) * np.exp2(rng.uniform(-14, 10, (B, 1)))).astype(np.float32)
    edges = _fp8_edges()
    k[:3].reshape(-1)[:edges.size] = edges
    v[3:6].reshape(-1)[:edges.size] = edges[::-1]
    pos = rng.integers(0, 5000, size=B).astype(np.int64)
    pos[4], pos[5], pos[6] = 0, W - 1, -3
    sk = rng.integers(0, 256, size=(B, W, D), dtype=np.uint8)
    sv = rng.integers(0, 256, size=(B, W, D), dtype=np.uint8)
    gk, gv = torch.from_numpy(sk.copy()).cuda(), torch.from_numpy(sv.copy()).cuda()
    _say(f"swa append B={B} W={W} D={D}")
    csa2.csa2_swa_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                         torch.from_numpy(pos).cuda(), gk, gv)
    torch.cuda.synchronize()
    keep = pos >= 0
    ek, ev = sk.copy(), sv.copy()
    for b in range(B):
        if pos[b] >= 0:
            ek[b, pos[b] % W] = oracle.e4m3_encode(k[b])
            ev[b, pos[b] % W] = oracle.e4m3_encode(v[b])
    # the same through the oracle's own ring update (negative positions
    # append nothing there too)
    rk, rv = sk.copy(), sv.copy()
    oracle.swa_append(k, v, pos, rk, rv)
    assert np.array_equal(rk, ek) and np.array_equal(rv, ev)
    assert np.array_equal(rk[~keep], sk[~keep]) and np.array_equal(rv[~keep], sv[~keep])
    assert np.array_equal(gk.cpu().numpy(), ek), "window K ring differs"
    assert np.array_equal(gv.cpu().numpy(), ev), "window V ring differs"


def test_swa_ring_feeds_a_window_only_layer(csa2):
    """300 appends per sequence (W = 128) through the ring, sequences
    starting at different positions, then a window-only layer (K = 0) on
    each sequence's ring at several points: rings bit-exact against the
    oracle's, attention within max-abs 2e-3 / rel-L2 1e-3 of the oracle's."""
    import _cases as C
    B, W, D, H, T = 4, 128, 512, 64, 300
    start = np.array([0, 5, 127, 1000], np.int64)
    rng = np.random.default_rng([7, 2])
    ks = rng.standard_normal((T, B, D)).astype(np.float32)
    vs = rng.standard_normal((T, B, D)).astype(np.float32)
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    gk = torch.zeros((B, W, D), dtype=torch.uint8, device="cuda")
    gv = torch.zeros((B, W, D), dtype=torch.uint8, device="cuda")
    ok_, ov_ = np.zeros((B, W, D), np.uint8), np.zeros((B, W, D), np.uint8)
    dk, dv = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    qd = torch.from_numpy(q).cuda()
    codes = torch.zeros((1, D // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((1, D // 16), dtype=torch.uint8, device="cuda")
    off = torch.zeros(B, dtype=torch.int64, device="cuda")
    scale = 1.0 / np.sqrt(D)
    _say(f"swa ring B={B} W={W} T={T}")
    for t in range(T):
        p = start + t
        csa2.csa2_swa_append(dk[t], dv[t], torch.from_numpy(p).cuda(), gk, gv)
        oracle.swa_append(ks[t], vs[t], p, ok_, ov_)
        if t in (0, 60, 127, 128, 299):
            n = np.minimum(W, start + t + 1).astype(np.int32)
            out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
            lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
            nb = csa2.csa2_decode_workspace_bytes(B, H, D, 0, W)
            ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
            csa2.csa2_sparse_attn_decode(qd, codes, scales, off, None, gk, gv,
                                         torch.from_numpy(n).cuda(), scale, out, lse, ws=ws)
            torch.cuda.synchronize()
            assert np.array_equal(gk.cpu().numpy(), ok_) and np.array_equal(gv.cpu().numpy(), ov_)
            ro, rl = oracle.attn_decode(q, codes.cpu().numpy(), scales.cpu().numpy(),
                                        np.zeros(B, np.int64), np.zeros((B, 0), np.int32),
                                        ok_, ov_, n, scale)
            C.assert_attn_close(out.cpu().numpy(), ro, f"window-only layer after {t + 1} appends")
            C.assert_lse_close(lse.cpu().numpy(), rl, f"window-only lse after {t + 1} appends")


def test_swa_append_argument_checks(csa2):
    dev = "cuda"
    k = torch.zeros((2, 12), device=dev)
    pos = torch.zeros(2, dtype=torch.int64, device=dev)
    ring = torch.zeros((2, 4, 12), dtype=torch.uint8, device=dev)
    with pytest.raises(csa2.CSA2Error):        # D not a multiple of 8
        csa2.csa2_swa_append(k, k, pos, ring, ring.clone())
    with pytest.raises(ValueError):            # ring shape disagrees
        csa2.csa2_swa_append(torch.zeros((2, 16), device=dev), torch.zeros((2, 16), device=dev),
                             pos, ring, ring.clone())
