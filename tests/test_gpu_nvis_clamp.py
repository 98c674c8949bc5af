"""A visible count above the call's max_nvis is read as max_nvis: the score
stream, the selects and the prefill row select never read past the rows
they scored.  Each case runs a query with q_nvis in (max_nvis, max_nvis + 64]
beside ordinary ones and must equal the oracle at q_nvis = max_nvis."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import compressed_fp4_kv_amd as csa2  # noqa: E402
import oracle  # noqa: E402
from gen.workloads import T_QI_FULL, Workload, build_device, host_kI_rows, host_qI  # noqa: E402

import _cases as C  # noqa: E402


def _say(*a):
    print(*a, flush=True)


def _run(w, t, nvis, max_nvis, topk, pool_blocks, prefill):
    q_nvis = torch.from_numpy(np.asarray(nvis, np.int32)).cuda()
    Q = len(nvis)
    idx = C.poison_i32((Q, topk))
    pool = C.poison_i32((Q, pool_blocks)) if pool_blocks else None
    if prefill:
        nb = csa2.csa2_index_prefill_workspace_bytes_ex(Q, max_nvis, topk, pool_blocks,
                                                        w.block_size, w.Hk, w.Di)
    else:
        nb = csa2.csa2_index_full_workspace_bytes(Q, max_nvis, topk, pool_blocks, w.block_size)
    csa2.csa2_index_full(t["qI_full"][:Q], t["kI"], t["seq_row_off"],
                         None if prefill else t["q_seq"][:Q], q_nvis, max_nvis, topk, idx,
                         pool_blocks, w.block_size, pool, C.ws(nb))
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (pool.cpu().numpy() if pool_blocks else None)


def _expect(w, nvis_eff, topk, pool_blocks, prefill):
    kI = host_kI_rows(w, 0, w.rows)
    qI = host_qI(w, T_QI_FULL)[:len(nvis_eff)]
    qs = np.zeros(len(nvis_eff), np.int32) if prefill else np.arange(len(nvis_eff), dtype=np.int32)
    return oracle.index_full(qI, kI, w.seq_row_off, qs, np.asarray(nvis_eff, np.int32), w.Hi,
                             w.Hk, w.Di, topk, pool_blocks, w.block_size)


@pytest.mark.parametrize("ctx,max_nvis,over", [
    ([6000, 6000, 6000, 6000], 5000, [5000, 5001, 5064, 4000]),       # one-workgroup select
    ([70000, 70000], 66000, [66001, 66040]),                          # filter + finalize
])
def test_decode_index_clamps_visible_count(ctx, max_nvis, over):
    w = Workload("nvis_clamp", 11, "decode_full", ctx, layers=1, pool_blocks=64)
    t = build_device(w, layers=1, with_kv=False)
    _say(f"[nvis clamp] ctx={ctx} max_nvis={max_nvis} q_nvis={over}")
    idx, pool = _run(w, t, over, max_nvis, w.topk, w.pool_blocks, prefill=False)
    eff = np.minimum(over, max_nvis)
    ridx, rpool = _expect(w, eff, w.topk, w.pool_blocks, prefill=False)
    assert np.array_equal(idx, ridx)
    assert np.array_equal(pool, rpool)
    assert idx.max() < max_nvis and pool.max() < (max_nvis + 7) // 8


def test_prefill_index_clamps_visible_count():
    w = Workload("nvis_clamp_prefill", 12, "prefill", [4096], layers=1, p0=0, Qn=64, m=1,
                 pool_blocks=32)
    t = build_device(w, layers=1, with_kv=False)
    max_nvis = 3000
    nvis = np.minimum(2950 + np.arange(64), 3063).astype(np.int32)   # some above max_nvis
    _say(f"[nvis clamp] prefill max_nvis={max_nvis} q_nvis={int(nvis.min())}..{int(nvis.max())}")
    idx, pool = _run(w, t, nvis, max_nvis, w.topk, w.pool_blocks, prefill=True)
    eff = np.minimum(nvis, max_nvis)
    ridx, rpool = _expect(w, eff, w.topk, w.pool_blocks, prefill=True)
    assert np.array_equal(idx, ridx)
    assert np.array_equal(pool, rpool)
