"""The five synthetic CSA2 workloads (shapes, distributions, seeds).

Each workload is described by a ``Workload`` record; ``host_*`` helpers
regenerate any slice of its tensors on the host (for the oracle), and
``build_device`` materialises the whole workload in device memory (for the
GPU library).  Seed = workload number.  Tensor ids: 1 indexer keys (shared by
Full and Reindex layers), 2 Full-layer indexer query, 3 Reindex-layer indexer
query, 4 main-KV FP4 code bytes, 5 main-KV E4M3 scale bytes, 16+l attention
query of layer l, 32+l window K of layer l, 48+l window V of layer l.  In the
hierarchical workload the Full layer that builds the pool attends too, with
the query and window of tensor ids of layer FULL_LAYER (its Reindex group's
layers are 0..3).

Distributions: indexer inputs are integers uniform on [-8, 8] stored as fp32;
FP4 codes are uniform over the 15 codes other than negative zero; scales are
2^k with k uniform on [-4, 4]; queries and window sources are N(0, 1); window
K/V are those normals rounded to E4M3FN.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from . import (dev_fp4, dev_ints, dev_pow2_scales, e4m3_bytes, host_fp4, host_fp4_runs,
               host_ints, host_ints_runs, host_pow2_scales, host_pow2_scales_runs, normal_f32)

T_KI, T_QI_FULL, T_QI_REINDEX, T_CODES, T_SCALES = 1, 2, 3, 4, 5


FULL_LAYER = 8   # hierarchical workload: tensor ids of the Full layer's own attention


def T_Q(layer):
    return 16 + layer


def T_SWA_K(layer):
    return 32 + layer


def T_SWA_V(layer):
    return 48 + layer


@dataclass
class Workload:
    name: str
    seed: int
    kind: str                 # "decode_full", "decode_hier", "decode_reindex", "prefill"
    ctx: List[int]            # entries per sequence (main-KV rows)
    H: int = 64               # attention heads
    D: int = 512              # channels of main KV / window / query heads
    Hi: int = 4               # indexer heads
    Hk: int = 4               # indexer key heads (Hi or 1)
    Di: int = 128             # indexer dims per head
    topk: int = 512
    W: int = 128              # window tokens
    layers: int = 4           # attention layers in the group (first is Full/Reindex)
    pool_blocks: int = 0      # candidate pool blocks (0: none)
    block_size: int = 8
    # prefill only
    p0: int = 0
    Qn: int = 0
    m: int = 1                # tokens per compressed entry
    pool: Optional[np.ndarray] = field(default=None, repr=False)   # inherited pool (reindex)

    @property
    def B(self):
        return len(self.ctx)

    @property
    def row_width(self):
        return self.Hk * self.Di

    @property
    def seq_row_off(self):
        return np.concatenate([[0], np.cumsum(self.ctx)[:-1]]).astype(np.int64)

    @property
    def rows(self):
        return int(np.sum(self.ctx))

    @property
    def scale(self):
        return float(1.0 / np.sqrt(self.D))

    # decode: one query per sequence; prefill: Qn queries of sequence 0
    @property
    def Q(self):
        return self.Qn if self.kind == "prefill" else self.B

    def q_nvis(self):
        if self.kind == "prefill":
            p = self.p0 + np.arange(self.Qn, dtype=np.int64)
            return ((p + 1) // self.m).astype(np.int32)
        return np.asarray(self.ctx, np.int32)

    def q_seq(self):
        if self.kind == "prefill":
            return np.zeros(self.Qn, np.int32)
        return np.arange(self.B, dtype=np.int32)

    def swa_len(self):
        return np.minimum(np.asarray(self.ctx, np.int64), self.W).astype(np.int32)

    def swa_rows(self):
        """Window rows per layer: [B, W] for decode, Qn + W - 1 for prefill."""
        return self.Qn + self.W - 1 if self.kind == "prefill" else self.W


def _ctx_mixed(seed, n=64, lo=8192, hi=1 << 20):
    rng = np.random.default_rng(seed)
    return np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi), n))).astype(np.int64).tolist()


def _pool_mixed(seed, ctx, pool_blocks=2048, bs=8):
    rng = np.random.default_rng([seed, 99])
    pool = np.full((len(ctx), pool_blocks), -1, np.int32)
    for b, n in enumerate(ctx):
        nb = (n + bs - 1) // bs
        take = min(pool_blocks, nb)
        pool[b, :take] = np.sort(rng.choice(nb, size=take, replace=False))
    return pool


def workload(i, small=False):
    """Workload i (0..4).  small=True keeps the shapes and structure but shrinks
    the context so that the oracle finishes in seconds."""
    if i == 0:
        return Workload("c0_tiny_full", 0, "decode_full", [4096], H=16, Di=64, topk=64, layers=1)
    if i == 1:
        ctx = [8192] * 4 if small else [65536] * 32
        return Workload("c1_full_reuse3", 1, "decode_full", ctx, layers=4)
    if i == 2:
        if small:
            return Workload("c2_prefill_m2", 2, "prefill", [4096], layers=6, p0=8192 - 96,
                            Qn=96, m=2)
        return Workload("c2_prefill_m2", 2, "prefill", [65536], layers=6, p0=126976, Qn=4096,
                        m=2)
    if i == 3:
        ctx = [40000, 24000] if small else [1 << 20] * 8
        return Workload("c3_hier_1m", 3, "decode_hier", ctx, layers=4, pool_blocks=2048)
    if i == 4:
        ctx = _ctx_mixed(4)
        if small:
            ctx = [max(1, c // 64) for c in ctx[:6]]
        w = Workload("c4_mixed_reindex", 4, "decode_reindex", ctx, layers=4, pool_blocks=2048)
        w.pool = _pool_mixed(4, ctx, w.pool_blocks, w.block_size)
        return w
    raise ValueError(i)


# ------------------------------------------------------------- host slices

def host_kI_rows(w, row0, nrows):
    rw = w.row_width
    return host_ints(w.seed, T_KI, row0 * rw, nrows * rw).reshape(nrows, w.Hk, w.Di)


def host_kI_rows_e4m3(w, row0, nrows):
    """The same key rows as E4M3FN bytes (torch's cast; the integers drawn
    are exact in E4M3), the compact key cache's input."""
    return e4m3_bytes(host_kI_rows(w, row0, nrows))


def host_kI_row_runs(w, row_starts, run_rows):
    """Key rows [len(row_starts) * run_rows, Hk, Di]: run_rows consecutive
    rows from each absolute row in row_starts, runs back to back."""
    rw = w.row_width
    st = np.asarray(row_starts, np.int64) * rw
    return host_ints_runs(w.seed, T_KI, st, run_rows * rw).reshape(-1, w.Hk, w.Di)


def host_kv_rows_at(w, rows):
    """FP4 code rows [n, D/2] and scale rows [n, D/16] at the absolute rows
    `rows` (in that order)."""
    r = np.asarray(rows, np.int64)
    codes = host_fp4_runs(w.seed, T_CODES, r * (w.D // 2), w.D // 2)
    scales = host_pow2_scales_runs(w.seed, T_SCALES, r * (w.D // 16), w.D // 16)
    return codes.reshape(-1, w.D // 2), scales.reshape(-1, w.D // 16)


def host_qI(w, tensor):
    return host_ints(w.seed, tensor, 0, w.Q * w.Hi * w.Di).reshape(w.Q, w.Hi, w.Di)


def host_kv_rows(w, row0, nrows):
    codes = host_fp4(w.seed, T_CODES, row0 * (w.D // 2), nrows * (w.D // 2))
    scales = host_pow2_scales(w.seed, T_SCALES, row0 * (w.D // 16), nrows * (w.D // 16))
    return codes.reshape(nrows, w.D // 2), scales.reshape(nrows, w.D // 16)


def host_q(w, layer):
    return normal_f32(w.seed, T_Q(layer), (w.Q, w.H, w.D))


def host_swa(w, layer):
    if w.kind == "prefill":
        shape = (w.swa_rows(), w.D)
    else:
        shape = (w.B, w.W, w.D)
    k = e4m3_bytes(normal_f32(w.seed, T_SWA_K(layer), shape))
    v = e4m3_bytes(normal_f32(w.seed, T_SWA_V(layer), shape))
    return k, v


# ----------------------------------------------------------- device build

def dev_kI_e4m3(w, device="cuda", chunk_rows=1 << 18):
    """The key cache of workload w as E4M3FN bytes [rows, Hk, Di] on the
    device: generated as fp32 integers chunk by chunk and cast by torch (the
    values are exact in E4M3), so the fp32 copy never exists whole."""
    import torch
    dev = torch.device(device)
    out = torch.empty((w.rows, w.Hk, w.Di), dtype=torch.uint8, device=dev)
    rw = w.row_width
    tmp = torch.empty((min(chunk_rows, max(w.rows, 1)), w.Hk, w.Di), dtype=torch.float32,
                      device=dev)
    for r0 in range(0, w.rows, chunk_rows):
        n = min(chunk_rows, w.rows - r0)
        dev_ints(tmp[:n], w.seed, T_KI, start=r0 * rw)
        out[r0:r0 + n] = tmp[:n].to(torch.float8_e4m3fn).view(torch.uint8)
    torch.cuda.synchronize(dev)
    return out


def build_device(w, device="cuda", layers=None, with_kI=True, with_kv=True, keys="f32"):
    """All inputs of workload w as device tensors (dict of torch tensors).
    keys: "f32" (t["kI"] fp32), "e4m3" (t["kI8"] E4M3 bytes) or "both"."""
    import torch
    dev = torch.device(device)
    L = w.layers if layers is None else layers
    t = {}
    if with_kI and keys in ("f32", "both"):
        t["kI"] = torch.empty((w.rows, w.Hk, w.Di), dtype=torch.float32, device=dev)
        dev_ints(t["kI"], w.seed, T_KI)
    if with_kI and keys in ("e4m3", "both"):
        t["kI8"] = dev_kI_e4m3(w, device)
    if with_kv:
        t["kv_codes"] = torch.empty((w.rows, w.D // 2), dtype=torch.uint8, device=dev)
        t["kv_scales"] = torch.empty((w.rows, w.D // 16), dtype=torch.uint8, device=dev)
        dev_fp4(t["kv_codes"], w.seed, T_CODES)
        dev_pow2_scales(t["kv_scales"], w.seed, T_SCALES)
    t["seq_row_off"] = torch.from_numpy(w.seq_row_off).to(dev)
    t["q_seq"] = torch.from_numpy(w.q_seq()).to(dev)
    t["q_nvis"] = torch.from_numpy(w.q_nvis()).to(dev)
    t["swa_len"] = torch.from_numpy(w.swa_len()).to(dev)
    t["qI_full"] = torch.from_numpy(host_qI(w, T_QI_FULL)).to(dev)
    if w.kind in ("decode_hier", "decode_reindex"):
        t["qI_reindex"] = torch.from_numpy(host_qI(w, T_QI_REINDEX)).to(dev)
    if w.pool is not None:
        t["pool"] = torch.from_numpy(w.pool).to(dev)
    if w.kind == "decode_hier":
        t["q_full"] = torch.from_numpy(host_q(w, FULL_LAYER)).to(dev)
        k, v = host_swa(w, FULL_LAYER)
        t["swa_k_full"] = torch.from_numpy(k).to(dev)
        t["swa_v_full"] = torch.from_numpy(v).to(dev)
    t["q"] = [torch.from_numpy(host_q(w, l)).to(dev) for l in range(L)]
    swa = [host_swa(w, l) for l in range(L)]
    t["swa_k"] = [torch.from_numpy(k).to(dev) for k, _ in swa]
    t["swa_v"] = [torch.from_numpy(v).to(dev) for _, v in swa]
    torch.cuda.synchronize(dev)
    return t
