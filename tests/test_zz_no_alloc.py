"""The allocation-free Reindex (csa2_reindex_noalloc: the library's static
per-device scratch instead of a caller workspace) against csa2_reindex on the
same inputs, bit for bit: two calls in a row, the second smaller, so the
second finds the first one's keys in the shared scratch.  Also against the
oracle, and the host-side refusal of a call larger than the scratch."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import compressed_fp4_kv_amd as csa2  # noqa: E402
from gen.workloads import Workload, build_device, workload  # noqa: E402
from oracle import slices  # noqa: E402

import _cases as C  # noqa: E402


def _noalloc(w, t, pool, qI=None, topk=None):
    qI = t["qI_reindex"] if qI is None else qI
    topk = w.topk if topk is None else topk
    Q = qI.shape[0]
    idx = C.poison_i32((Q, topk))
    csa2.csa2_reindex_noalloc(qI, t["kI"], t["seq_row_off"], t["q_seq"][:Q], t["q_nvis"][:Q],
                              pool, w.block_size, topk, idx)
    torch.cuda.synchronize()
    return idx


def test_noalloc_reindex_equals_reindex_on_two_calls():
    w = workload(4, small=True)    # 6 mixed-length sequences, pools up to 2,048 blocks
    t = build_device(w, layers=1, with_kv=False)
    print(f"[noalloc] call 1: Q={w.B} pool={w.pool_blocks}x{w.block_size}", flush=True)
    got1 = _noalloc(w, t, t["pool"]).cpu().numpy()
    ref1 = C.gpu_reindex(w, t, t["pool"]).cpu().numpy()
    assert np.array_equal(got1, ref1)
    for b in range(w.B):
        assert np.array_equal(got1[b], slices.reindex_query(w, b, w.pool[b])), f"query {b}"
    # second call: fewer queries, a shorter pool and a shorter Top-K
    Q2, P2, K2 = 3, 300, 100
    pool2 = t["pool"][:Q2, :P2].contiguous()
    print(f"[noalloc] call 2: Q={Q2} pool={P2}x{w.block_size} topk={K2}", flush=True)
    got2 = _noalloc(w, t, pool2, qI=t["qI_reindex"][:Q2].contiguous(), topk=K2).cpu().numpy()
    idx = C.poison_i32((Q2, K2))
    buf = C.ws(csa2.csa2_reindex_workspace_bytes(Q2, P2, w.block_size))
    csa2.csa2_reindex(t["qI_reindex"][:Q2].contiguous(), t["kI"], t["seq_row_off"],
                      t["q_seq"][:Q2], t["q_nvis"][:Q2], pool2, w.block_size, K2, idx, buf)
    torch.cuda.synchronize()
    assert np.array_equal(got2, idx.cpu().numpy())
    assert np.all((got2 >= -1) & (got2 < np.asarray(w.ctx[:Q2])[:, None]))


def test_noalloc_reindex_at_the_scratch_limit_and_beyond():
    # 128 queries of 2,048 x 8 candidates fill the scratch exactly; one more is refused
    w = Workload("noalloc_limit", 21, "decode_reindex", [20000] * 128, layers=1,
                 pool_blocks=2048)
    rng = np.random.default_rng(5)
    w.pool = np.stack([np.sort(rng.choice(2500, 2048, replace=False)) for _ in range(128)]
                      ).astype(np.int32)
    assert w.B * w.pool_blocks * w.block_size == csa2.NOALLOC_MAX_CAND
    t = build_device(w, layers=1, with_kv=False)
    print(f"[noalloc] limit: Q={w.B} pool={w.pool_blocks}x{w.block_size}", flush=True)
    got = _noalloc(w, t, t["pool"]).cpu().numpy()
    ref = C.gpu_reindex(w, t, t["pool"]).cpu().numpy()
    assert np.array_equal(got, ref)
    for b in (0, 77, 127):
        assert np.array_equal(got[b], slices.reindex_query(w, b, w.pool[b])), f"query {b}"
    big = torch.cat([t["pool"], t["pool"][:1]])
    qI = torch.cat([t["qI_reindex"], t["qI_reindex"][:1]])
    seq = torch.cat([t["q_seq"], t["q_seq"][:1]])
    nv = torch.cat([t["q_nvis"], t["q_nvis"][:1]])
    idx = C.poison_i32((129, w.topk))
    with pytest.raises(csa2.CSA2Error):
        csa2.csa2_reindex_noalloc(qI, t["kI"], t["seq_row_off"], seq, nv, big, w.block_size,
                                  w.topk, idx)
    torch.cuda.synchronize()
    assert int(idx.min()) == -7 and int(idx.max()) == -7   # nothing was written
