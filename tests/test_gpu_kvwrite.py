"""GPU parity of the FP4 main-KV writer (csa2_kv_quantize_fp4) with the
oracle's quantiser: E2M1 codes and E4M3 scale bytes bit-exact, on random rows
spanning every scale byte, on rows built around the rounding boundaries, at
the prefill context's size, and on the argument checks."""
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
