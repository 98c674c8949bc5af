"""GPU parity of csa2_sparse_attn_decode_layers: a Full (or Reindex) layer and
its Reuse layers in one call, sharing the index list and the main KV, each
with its own query and window.  Every layer's output and log-sum-exp within
max-abs 2e-3 / rel-L2 1e-3 of the oracle; one layer reproduces the per-layer
call bit for bit.  (The groups of the decode workloads at full size, every
query, are in test_gpu_fullsize.py.)"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gen.workloads import build_device, workload  # noqa: E402

import _cases as C  # noqa: E402


@pytest.fixture(scope="module")
def csa2():
    assert torch.cuda.is_available(), "needs an MI355X"
    import compressed_fp4_kv_amd as m
    oracle.set_threads(16)
    return m


def teardown_module(module):
    torch.cuda.empty_cache()


def _say(*a):
    print(*a, flush=True)


def _group(csa2, w, t, idx, layers=None, with_lse=True):
    L = w.layers if layers is None else layers
    outs = [C.poison_f32((w.B, w.H, w.D)) for _ in range(L)]
    lses = [C.poison_f32((w.B, w.H)) for _ in range(L)] if with_lse else None
    buf = C.ws(csa2.csa2_decode_layers_workspace_bytes(L, w.B, w.H, w.D, idx.shape[1], w.W))
    csa2.csa2_sparse_attn_decode_layers(t["q"][:L], t["kv_codes"], t["kv_scales"],
                                        t["seq_row_off"], idx, t["swa_k"][:L], t["swa_v"][:L],
                                        t["swa_len"], w.scale, outs, lses, ws=buf)
    torch.cuda.synchronize()
    return ([o.cpu().numpy() for o in outs],
            [x.cpu().numpy() for x in lses] if with_lse else None)


def _indices(w, t):
    if w.kind == "decode_full":
        idx, _ = C.gpu_index_full(w, t)
        return idx
    if w.kind == "decode_hier":
        _, pool = C.gpu_index_full(w, t, pool_blocks=w.pool_blocks)
        return C.gpu_reindex(w, t, pool)
    return C.gpu_reindex(w, t, t["pool"])


@pytest.mark.parametrize("wid", [0, 1, 3, 4])
def test_layer_group_matches_oracle(csa2, wid):
    w = workload(wid, small=True)
    _say(f"[{w.name} layer group] B={w.B} layers={w.layers}")
    t = build_device(w)
    idx = _indices(w, t)
    outs, lses = _group(csa2, w, t, idx)
    ih = idx.cpu().numpy()
    for layer in range(w.layers):
        for b in range(w.B):
            ro, rl = C.oracle_attn_query(w, b, layer, ih[b])
            C.assert_attn_close(outs[layer][b], ro[0], f"{w.name} layer {layer} query {b}")
            C.assert_lse_close(lses[layer][b], rl[0], f"{w.name} layer {layer} query {b}")


def test_one_layer_equals_per_layer_call(csa2):
    w = workload(1, small=True)
    t = build_device(w)
    idx = _indices(w, t)
    for layer in range(w.layers):
        outs, lses = _group(csa2, w, {**t, "q": t["q"][layer:], "swa_k": t["swa_k"][layer:],
                                      "swa_v": t["swa_v"][layer:]}, idx, layers=1)
        ref_o, ref_l = C.gpu_attn(w, t, layer, idx)
        assert np.array_equal(outs[0], ref_o.cpu().numpy())
        assert np.array_equal(lses[0], ref_l.cpu().numpy())


def test_layer_group_without_lse_and_eight_layers(csa2):
    # lse omitted; the largest group (8 layers: the same four twice, so each
    # pair of layers must agree exactly)
    w = workload(4, small=True)
    t = build_device(w)
    idx = _indices(w, t)
    t8 = {**t, "q": t["q"] * 2, "swa_k": t["swa_k"] * 2, "swa_v": t["swa_v"] * 2}
    outs, _ = _group(csa2, w, t8, idx, layers=8, with_lse=False)
    for layer in range(4):
        assert np.array_equal(outs[layer], outs[layer + 4])
    ih = idx.cpu().numpy()
    for layer in range(4):
        for b in range(w.B):
            ro, _ = C.oracle_attn_query(w, b, layer, ih[b])
            C.assert_attn_close(outs[layer][b], ro[0], f"8-layer group layer {layer} query {b}")


def test_layer_group_at_the_limits(csa2):
    # 8 layers (the most one call takes), the largest Top-K list (2,048: 64
    # main-KV tiles) and window (1,024 tokens: 32 tiles), 32 heads (half a
    # head group), a ragged index tail and short windows
    from gen.workloads import Workload
    w = Workload("limits", 19, "decode_full", [5000, 2100], H=32, topk=2048, W=1024, layers=8)
    t = build_device(w, with_kI=False)
    rng = np.random.default_rng(12)
    idx = np.full((w.B, w.topk), -1, np.int32)
    idx[0] = np.sort(rng.choice(5000, 2048, replace=False))
    idx[1, :1999] = np.sort(rng.choice(2100, 1999, replace=False))
    sl = np.array([1024, 333], np.int32)
    t["swa_len"] = torch.from_numpy(sl).cuda()
    outs, lses = _group(csa2, w, t, torch.from_numpy(idx).cuda())
    for layer in (0, 3, 7):
        for b in range(w.B):
            ro, rl = C.oracle_attn_query(w, b, layer, idx[b], swa_len=int(sl[b]))
            C.assert_attn_close(outs[layer][b], ro[0], f"layer {layer} query {b}")
            C.assert_lse_close(lses[layer][b], rl[0], f"layer {layer} query {b}")
