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
