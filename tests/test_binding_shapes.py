"""The Python binding refuses tensors whose extents disagree with the call's
sizes before any pointer reaches a kernel (CPU only: the shape checks run
before the device checks, so CPU tensors exercise them)."""
import pytest
import torch

csa2 = pytest.importorskip("compressed_fp4_kv_amd")

f32, i32, i64, u8 = torch.float32, torch.int32, torch.int64, torch.uint8
B, H, D, W, TOPK = 3, 64, 512, 128, 16


def _decode_args(**over):
    a = dict(q=torch.zeros(B, H, D, dtype=f32),
             kv_codes=torch.zeros(100, D // 2, dtype=u8),
             kv_scales=torch.zeros(100, D // 16, dtype=u8),
             seq_row_off=torch.zeros(B, dtype=i64),
             topk_idx=torch.zeros(B, TOPK, dtype=i32),
             swa_k=torch.zeros(B, W, D, dtype=u8), swa_v=torch.zeros(B, W, D, dtype=u8),
             swa_len=torch.zeros(B, dtype=i32), softmax_scale=0.04,
             out=torch.zeros(B, H, D, dtype=f32), lse=torch.zeros(B, H, dtype=f32))
    a.update(over)
    return a


def test_decode_accepts_matching_shapes_up_to_the_device_check():
    with pytest.raises(ValueError, match="must be a device tensor"):
        csa2.csa2_sparse_attn_decode(**_decode_args())


@pytest.mark.parametrize("name,bad", [
    ("out", torch.zeros(B, H, D - 16, dtype=f32)),
    ("out", torch.zeros(B - 1, H, D, dtype=f32)),
    ("lse", torch.zeros(B, H // 2, dtype=f32)),
    ("swa_v", torch.zeros(B, W, D // 2, dtype=u8)),
    ("swa_len", torch.zeros(B + 1, dtype=i32)),
    ("seq_row_off", torch.zeros(B - 1, dtype=i64)),
    ("topk_idx", torch.zeros(B - 1, TOPK, dtype=i32)),
    ("kv_codes", torch.zeros(100, D // 4, dtype=u8)),
    ("kv_scales", torch.zeros(99, D // 16, dtype=u8)),
])
def test_decode_refuses_mismatched_extents(name, bad):
    with pytest.raises(ValueError, match=rf"{name}: expected shape"):
        csa2.csa2_sparse_attn_decode(**_decode_args(**{name: bad}))


def test_decode_layers_refuses_mismatched_lists_and_extents():
    a = _decode_args()
    common = dict(kv_codes=a["kv_codes"], kv_scales=a["kv_scales"],
                  seq_row_off=a["seq_row_off"], topk_idx=a["topk_idx"], swa_len=a["swa_len"],
                  softmax_scale=0.04)
    qs = [a["q"], a["q"].clone()]
    ks = [a["swa_k"], a["swa_k"].clone()]
    outs = [a["out"], a["out"].clone()]
    with pytest.raises(ValueError, match="out: 1 tensors for 2 layers"):
        csa2.csa2_sparse_attn_decode_layers(qs, swa_ks=ks, swa_vs=ks, outs=outs[:1], **common)
    with pytest.raises(ValueError, match=r"q\[1\]: expected shape"):
        csa2.csa2_sparse_attn_decode_layers([qs[0], qs[1][:, :32]], swa_ks=ks, swa_vs=ks,
                                            outs=outs, **common)
    with pytest.raises(ValueError, match=r"swa_v\[1\]: expected shape"):
        csa2.csa2_sparse_attn_decode_layers(qs, swa_ks=ks, swa_vs=[ks[0], ks[1][:2]],
                                            outs=outs, **common)
    with pytest.raises(ValueError, match="must be a device tensor"):
        csa2.csa2_sparse_attn_decode_layers(qs, swa_ks=ks, swa_vs=ks, outs=outs, **common)


def test_prefill_refuses_a_window_of_the_wrong_length():
    Qn = 5
    args = dict(q=torch.zeros(Qn, H, D, dtype=f32), p0=40,
                kv_codes=torch.zeros(64, D // 2, dtype=u8),
                kv_scales=torch.zeros(64, D // 16, dtype=u8),
                topk_idx=torch.zeros(Qn, TOPK, dtype=i32),
                swa_k=torch.zeros(Qn + W - 1, D, dtype=u8),
                swa_v=torch.zeros(Qn + W - 1, D, dtype=u8), W=W, softmax_scale=0.04,
                out=torch.zeros(Qn, H, D, dtype=f32))
    with pytest.raises(ValueError, match="must be a device tensor"):
        csa2.csa2_sparse_attn_prefill_chunk(**args)
    args["swa_k"] = torch.zeros(Qn + W - 2, D, dtype=u8)
    with pytest.raises(ValueError, match="swa_k: expected shape"):
        csa2.csa2_sparse_attn_prefill_chunk(**args)


def _index_args(**over):
    Q, Hi, Hk, Di = 4, 64, 4, 128
    a = dict(qI=torch.zeros(Q, Hi, Di, dtype=f32), kI=torch.zeros(1000, Hk, Di, dtype=f32),
             seq_row_off=torch.zeros(2, dtype=i64), q_seq=torch.zeros(Q, dtype=i32),
             q_nvis=torch.zeros(Q, dtype=i32), max_nvis=500, topk=TOPK,
             topk_idx=torch.zeros(Q, TOPK, dtype=i32))
    a.update(over)
    return a


@pytest.mark.parametrize("fn", ["csa2_index_full", "csa2_index_full_ex"])
def test_index_full_refuses_mismatched_extents(fn):
    call = getattr(csa2, fn)
    with pytest.raises(ValueError, match="must be a device tensor"):
        call(**_index_args())
    with pytest.raises(ValueError, match="kI: expected shape"):
        call(**_index_args(kI=torch.zeros(1000, 4, 64, dtype=f32)))
    with pytest.raises(ValueError, match="topk_idx: expected shape"):
        call(**_index_args(topk_idx=torch.zeros(4, TOPK + 1, dtype=i32)))
    with pytest.raises(ValueError, match="q_nvis: expected shape"):
        call(**_index_args(q_nvis=torch.zeros(3, dtype=i32)))
    with pytest.raises(ValueError, match="pool_block_idx: expected shape"):
        call(**_index_args(pool_blocks=8, pool_block_idx=torch.zeros(4, 7, dtype=i32)))


def test_reindex_refuses_mismatched_extents():
    a = _index_args()
    del a["max_nvis"]
    a.update(pool_block_idx=torch.zeros(4, 32, dtype=i32), block_size=8)
    with pytest.raises(ValueError, match="must be a device tensor"):
        csa2.csa2_reindex(**a)
    a["topk_idx"] = torch.zeros(5, TOPK, dtype=i32)
    with pytest.raises(ValueError, match="topk_idx: expected shape"):
        csa2.csa2_reindex(**a)
