"""Seeded input generator (CPU side): published hash values and workload shapes."""
import numpy as np

import gen
from gen.workloads import workload


def test_hash_is_splitmix64():
    # SplitMix64 started from state 0 first returns 0xE220A8397B1DCDAF
    # (Steele, Lea, Flood 2014; the reference output widely quoted for it).
    assert gen.host().gen_hash(0, 0, 0) == 0xE220A8397B1DCDAF


def test_ints_range_and_determinism():
    a = gen.host_ints(3, 1, 100, 20000)
    b = gen.host_ints(3, 1, 0, 20100)[100:]
    assert np.array_equal(a, b)
    assert a.min() == -8 and a.max() == 8
    assert np.all(a == np.round(a))
    counts = np.bincount((a + 8).astype(int), minlength=17)
    assert counts.min() > 0.8 * 20000 / 17


def test_workload_shapes():
    w1 = workload(1)
    assert w1.B == 32 and w1.rows == 32 * 65536 and w1.row_width == 512
    w2 = workload(2)
    nv = w2.q_nvis()
    assert nv[0] == 63488 and nv[-1] == 65536 and w2.swa_rows() == 4223
    w3 = workload(3)
    assert w3.rows == 8 << 20 and w3.pool_blocks * w3.block_size == 16384
    w4 = workload(4)
    assert w4.B == 64 and min(w4.ctx) >= 8192 and max(w4.ctx) <= 1 << 20
    assert w4.rows * w4.row_width * 4 < 60e9
    for b, n in enumerate(w4.ctx):
        p = w4.pool[b]
        v = p[p >= 0]
        assert len(v) == min(2048, (n + 7) // 8) and np.all(np.diff(v) > 0)


def test_runs_equal_slices_of_the_contiguous_tensors():
    starts = np.array([5, 0, 4096, 77, 123456789], np.int64)
    run = 40
    ints = gen.host_ints_runs(4, 1, starts, run)
    fp4 = gen.host_fp4_runs(4, 4, starts, run)
    sc = gen.host_pow2_scales_runs(4, 5, starts, run)
    for r, s in enumerate(starts):
        sl = slice(r * run, (r + 1) * run)
        assert np.array_equal(ints[sl], gen.host_ints(4, 1, s, run))
        assert np.array_equal(fp4[sl], gen.host_fp4(4, 4, s, run))
        assert np.array_equal(sc[sl], gen.host_pow2_scales(4, 5, s, run))
    assert gen.host_ints_runs(4, 1, np.zeros(0, np.int64), run).size == 0
