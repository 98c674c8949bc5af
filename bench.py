"""CSA2 decode benchmark on one MI355X.

Default: one JSON line whose `value` is the mixed-length serving decode
workload, the largest of the five that runs on one GPU: 64 decode queries
over sequences of 8,192 .. 1,048,576 entries (log-uniform, seeded; 13.7 M
entries, 28 GB of fp32 indexer keys).  One step = the Reindex layer over
each sequence's inherited candidate pool (2,048 blocks x 8 positions, fewer
for short sequences; exact Top-512) and the sparse attention of the Reindex
layer and its 3 Reuse layers (64 heads x 512 channels over the 512 selected
FP4 rows + a 128-token FP8 window, one layer-group launch).  value = 64
queries / the median step time.

The same line carries the other workloads, each timed the same way, under
"other_workloads": the 32 x 65,536 decode (Full layer + 3 Reuse), the
8 x 1,048,576 hierarchical decode (Full layer: score stream, Top-512, pool
and its own attention; then Reindex + 3 Reuse) and the 4,096-query prefill
chunk (Full + 5 Reuse layers, with its matrix-core utilisation); and the
headline step over the compact E4M3 key cache under "e4m3_keys".

Timing: W warm-up steps, then K timed steps, each between its own pair of
HIP events on the launch stream, with a read pass over 1 GiB between steps
(outside the events) so that no step finds the previous step's data in the
256 MB last-level cache.  ms_per_step is the median of the K steps.  The
same K steps are also timed after a read-modify-write pass over the 1 GiB
instead ("rmw_touch"): that pass leaves the last-level cache full of dirty
lines, and the step then also pays for writing them back.  A second pass
with per-launch events gives each kernel's average duration, from which the
dominant kernel's roofline is computed.

cpu_baseline: the oracle (plain C, double precision) on the host cores, on
the headline workload: all queries with every core, and a labelled sample
single-threaded, with the CPU model.  Input generation is not timed.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --workload N [--keys f32|e4m3]  (one workload alone)
       python bench.py --kv-writer   (the FP4 main-KV writer alone, its own line)

--keys e4m3 runs the same step over the compact indexer-key cache (one
E4M3FN byte per key value instead of fp32), through csa2_index_full_e4m3 and
csa2_reindex_e4m3.  For the hierarchical workload (--workload 3) the
candidate pool is a parameter: --pool-blocks P --block-size S (P x S <=
16,384) and --block-rule max|sum (the block score; max is the reading used).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFS = 2500.0   # dense fp16 / bf16 matrix-core peak of an MI355X
HEADLINE = 4                 # the mixed-length serving decode workload
FLUSH_BYTES = 1 << 30        # touched between timed steps (the last-level cache is 256 MB)

WORKLOAD_NAMES = {
    "c0_tiny_full": "decode Full layer: 1 sequence x 4,096 entries, indexer 4x64, Top-64, 16 heads",
    "c1_full_reuse3": "decode Full + 3 Reuse layers: 32 sequences x 65,536 entries, indexer 4x128 "
                      "fp32, Top-512, 64 heads x 512 ch, FP4 main KV, 128-token FP8 window",
    "c2_prefill_m2": "prefill chunk, m=2: 4,096 queries over 65,536 entries, Full + 5 Reuse layers",
    "c3_hier_1m": "decode, 8 sequences x 1,048,576 entries: Full layer (score stream, Top-512, "
                  "2,048x8 pool, its attention), then Reindex + 3 Reuse layers",
    "c4_mixed_reindex": "decode, 64 sequences of 8,192..1,048,576 entries (log-uniform): Reindex "
                        "over inherited 2,048x8 pools (Top-512, fp32 indexer keys 4x128) + 3 "
                        "Reuse layers, 64 heads x 512 ch, FP4 main KV, 128-token FP8 window",
}

# committed rocprofv3 counter summaries of each workload's dominant kernel
TRAFFIC_PROFILES = {
    ("c1_full_reuse3", "f32"): "score_stream_c1_traffic.md",
    ("c1_full_reuse3", "e4m3"): "score_stream_e4m3_c1_traffic.md",
    ("c3_hier_1m", "f32"): "score_stream_c3_traffic.md",
    ("c4_mixed_reindex", "f32"): "reindex_c4_traffic.md",
    ("c4_mixed_reindex", "e4m3"): "reindex_c4_traffic.md",
    ("c2_prefill_m2", "f32"): "prefill_c2_traffic.md",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(profile, kernel=None):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a plain-copy calibration),
    or None if the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    try:
        for line in open(path):
            if line.startswith("traffic_record:"):
                rec = json.loads(line.split(":", 1)[1])
                if kernel is not None and rec.get("kernel") != kernel:
                    continue
                h = hashlib.sha256()
                for src in rec["sources"]:
                    h.update(open(os.path.join(ROOT, src), "rb").read())
                if h.hexdigest()[:16] == rec["sources_sha256_16"]:
                    return rec["traffic_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        pass
    return None


def make_step(csa2, w, t, torch, keys="f32", block_rule="max"):
    """One pass of the workload's call sequence (all of its layers)."""
    e4m3 = keys == "e4m3"
    kI = t["kI8"] if e4m3 else t["kI"]
    index_full = csa2.csa2_index_full_e4m3 if e4m3 else csa2.csa2_index_full
    reindex = csa2.csa2_reindex_e4m3 if e4m3 else csa2.csa2_reindex
    Q = w.Q
    max_nvis = int(w.q_nvis().max())
    dev = "cuda"
    idx = torch.empty((Q, w.topk), dtype=torch.int32, device=dev)
    ridx = torch.empty((Q, w.topk), dtype=torch.int32, device=dev)
    pool = t.get("pool")
    if w.kind == "decode_hier":
        pool = torch.empty((Q, w.pool_blocks), dtype=torch.int32, device=dev)
    P = w.pool_blocks if w.kind == "decode_hier" else 0
    if w.kind == "prefill":
        nb_i = csa2.csa2_index_prefill_workspace_bytes(Q, max_nvis, w.topk, w.Hk, w.Di)
    else:
        nb_i = csa2.csa2_index_full_workspace_bytes(Q, max_nvis, w.topk, P, w.block_size)
    ws_i = torch.empty(max(256, nb_i), dtype=torch.uint8, device=dev)
    ws_r = torch.empty(max(256, csa2.csa2_reindex_workspace_bytes(Q, w.pool_blocks, w.block_size)),
                       dtype=torch.uint8, device=dev)
    if w.kind == "prefill":
        nb = csa2.csa2_prefill_workspace_bytes(Q, w.H, w.D, w.topk, w.W)
    else:
        # the decode layers of a group share the indices and the KV: one call
        nb = max(csa2.csa2_decode_layers_workspace_bytes(w.layers, Q, w.H, w.D, w.topk, w.W),
                 csa2.csa2_decode_workspace_bytes(Q, w.H, w.D, w.topk, w.W))
    ws_a = torch.empty(max(256, nb), dtype=torch.uint8, device=dev)
    outs = [torch.empty((Q, w.H, w.D), dtype=torch.float32, device=dev) for _ in range(w.layers)]
    lses = [torch.empty((Q, w.H), dtype=torch.float32, device=dev) for _ in range(w.layers)]
    if w.kind == "decode_hier":
        out_f = torch.empty((Q, w.H, w.D), dtype=torch.float32, device=dev)
        lse_f = torch.empty((Q, w.H), dtype=torch.float32, device=dev)

    def attn_layers(ix):
        if w.kind == "prefill":
            for layer in range(w.layers):
                csa2.csa2_sparse_attn_prefill_chunk(t["q"][layer], w.p0, t["kv_codes"],
                                                    t["kv_scales"], ix, t["swa_k"][layer],
                                                    t["swa_v"][layer], w.W, w.scale, outs[layer],
                                                    lses[layer], ws=ws_a)
        else:
            csa2.csa2_sparse_attn_decode_layers(t["q"], t["kv_codes"], t["kv_scales"],
                                                t["seq_row_off"], ix, t["swa_k"], t["swa_v"],
                                                t["swa_len"], w.scale, outs, lses, ws=ws_a)

    def step():
        if w.kind in ("decode_full", "prefill"):
            # Full layer: indexer, then Full + Reuse layers on the same indices and KV
            index_full(t["qI_full"], kI, t["seq_row_off"],
                       None if w.kind == "prefill" else t["q_seq"], t["q_nvis"], max_nvis, w.topk,
                       idx, ws=ws_i)
            attn_layers(idx)
            return
        if w.kind == "decode_hier":
            # the Full layer's indexer builds Top-K and the candidate pool; the
            # Full layer attends over its Top-K with its own query and window
            csa2.csa2_index_full_ex(t["qI_full"], kI, t["seq_row_off"], t["q_seq"], t["q_nvis"],
                                    max_nvis, w.topk, idx, P, w.block_size, pool,
                                    block_rule=block_rule, ws=ws_i)
            csa2.csa2_sparse_attn_decode(t["q_full"], t["kv_codes"], t["kv_scales"],
                                         t["seq_row_off"], idx, t["swa_k_full"], t["swa_v_full"],
                                         t["swa_len"], w.scale, out_f, lse_f, ws=ws_a)
        # Reindex layer over the pool, then Reindex + Reuse layers' attention
        reindex(t["qI_reindex"], kI, t["seq_row_off"], t["q_seq"], t["q_nvis"], pool,
                w.block_size, w.topk, ridx, ws=ws_r)
        attn_layers(ridx)
    return step, idx


def candidate_rows(w):
    """Key rows a Reindex layer gathers: each sequence's valid pool blocks,
    cut at its visible entries."""
    import numpy as np
    if w.pool is not None:
        return sum(min(int(np.sum(w.pool[b] >= 0)) * w.block_size, int(w.ctx[b]))
                   for b in range(w.B))
    return sum(min(w.pool_blocks * w.block_size, int(w.ctx[b])) for b in range(w.B))


def dominant_roofline(w, kern, keys="f32"):
    """Roofline record of the workload's dominant kernel: algorithmic work per
    launch / its measured average launch duration.  Key bytes per value: 4
    (fp32) or 1 (E4M3 key cache)."""
    sfx, vb = ("_e4m3", 1) if keys == "e4m3" else ("", 4)
    stream, rscore = "score_stream" + sfx, "reindex_score" + sfx
    prof = TRAFFIC_PROFILES.get((w.name, keys))
    if w.kind in ("decode_full", "decode_hier") and stream in kern:
        alg = float(w.rows) * w.row_width * vb + float(w.Q) * w.Hi * w.Di * 4
        ach = alg / (kern[stream]["avg_us"] * 1e-6) / 1e9
        return {"bound": "hbm", "kernel": stream, "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "algorithmic_bytes": alg,
                "traffic": measured_traffic(prof, stream) if prof else None}
    if w.kind == "decode_reindex" and rscore in kern:
        alg = float(candidate_rows(w)) * w.row_width * vb + float(w.Q) * w.Hi * w.Di * 4
        ach = alg / (kern[rscore]["avg_us"] * 1e-6) / 1e9
        return {"bound": "hbm", "kernel": rscore, "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "algorithmic_bytes": alg,
                "traffic": measured_traffic(prof, rscore) if prof else None}
    if "attn" in kern:
        return mfma_utilisation(w, kern)["attn"] | {
            "traffic": measured_traffic(prof, "attn") if prof else None}
    return None


def step_hbm(w, ms_step, keys="f32"):
    """Algorithmic HBM bytes of one whole step (every call of the workload's
    sequence) and the rate they imply at the measured step time: the key rows
    streamed by a Full layer, the key rows a Reindex layer gathers, and per
    attention layer the query, the output, the selected FP4 rows (288 B), the
    window K and V (E4M3) and the index row.  Workspace traffic (score keys,
    split partials) is not algorithmic and not counted."""
    import numpy as np
    vb = 1 if keys == "e4m3" else 4
    rb = w.row_width * vb                           # bytes of one key row
    qb = w.Hi * w.Di * 4                            # one indexer query
    total = 0.0
    if w.kind in ("decode_full", "decode_hier", "prefill"):
        total += float(np.sum(w.ctx)) * rb + w.Q * qb          # Full-layer stream (prefill: once)
    if w.kind in ("decode_hier", "decode_reindex"):
        total += float(candidate_rows(w)) * rb + w.Q * qb
    sel = np.minimum(w.q_nvis(), w.topk).astype(np.float64)
    win = float(w.swa_rows() if w.kind == "prefill" else w.B * w.W)
    per_layer = (2.0 * w.Q * w.H * w.D * 4 + float(np.sum(sel)) * (w.D // 2 + w.D // 16)
                 + win * 2 * w.D + w.Q * w.topk * 4)
    if w.kind == "prefill":
        # every query's selected rows come from one 65,536-entry sequence:
        # the unique rows bound the compulsory bytes
        per_layer = (2.0 * w.Q * w.H * w.D * 4 + min(float(np.sum(sel)), float(w.ctx[0]))
                     * (w.D // 2 + w.D // 16) + win * 2 * w.D + w.Q * w.topk * 4)
    layers = w.layers + (1 if w.kind == "decode_hier" else 0)   # + the Full layer's attention
    total += layers * per_layer
    ach = total / (ms_step * 1e-3) / 1e9
    return {"algorithmic_bytes": total, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBS}


def mfma_utilisation(w, kern):
    """Algorithmic flops per launch / measured launch time of the matrix-core
    kernels, against the dense fp16/bf16 peak.  The attention's two-part fp16
    splits of the query and the probabilities execute twice the algorithmic
    flops (issued / algorithmic = 2); the score GEMM's hi/lo bf16 parts
    execute 1x (integer-valued inputs: the lo parts are zero and skipped)."""
    res = {}
    if "attn" in kern:
        # QK^T and PV, 2 flops per MAC; a decode launch covers the group's layers
        flops = 4.0 * w.H * (w.topk + w.W) * w.D * w.Q * (1 if w.kind == "prefill" else w.layers)
        ach = flops / (kern["attn"]["avg_us"] * 1e-6) / 1e12
        res["attn"] = {"bound": "mfma", "kernel": "attn (fp16 MFMA)", "achieved": ach,
                       "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
                       "frac": ach / MFMA_F16_PEAK_TFS, "issued_per_algorithmic": 2.0}
    if "prefill_scores" in kern:
        import numpy as np
        flops = 2.0 * float(np.sum(w.q_nvis())) * w.Hi * w.Di   # visible (query, entry) dots
        ach = flops / (kern["prefill_scores"]["avg_us"] * 1e-6) / 1e12
        res["prefill_scores"] = {"bound": "mfma", "kernel": "prefill_scores (bf16 MFMA)",
                                 "achieved": ach, "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
                                 "frac": ach / MFMA_F16_PEAK_TFS, "issued_per_algorithmic": 1.0}
    return res


# ------------------------------------------------------------------ timing

class Touch:
    """The pass over FLUSH_BYTES of device memory between timed steps: a read
    (every cache level then holds clean lines of this buffer only), or a
    read-modify-write (the same, but the last-level cache is left full of
    dirty lines that the next step has to write back)."""

    def __init__(self, torch):
        self.buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.float32, device="cuda")
        self.kind = "read"

    def __call__(self):
        if self.kind == "read":
            self.sink.add_(self.buf.sum())
        else:
            self.buf.add_(1.0)


def time_steps(torch, step, steps, warmup, touch):
    """Per-step times (ms) of `steps` steps, each between its own events,
    with the touch pass between steps."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        touch()
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def kernel_times(csa2, torch, step, steps, touch):
    """Average duration of each kernel over `steps` steps (per-launch events
    on the launch stream), touch pass between steps."""
    csa2.profile_reset()
    csa2.profile_enable(True)
    for _ in range(steps):
        touch()
        step()
    torch.cuda.synchronize()
    prof = csa2.profile_read()
    csa2.profile_enable(False)
    return {k: {"launches": n, "avg_us": 1000.0 * ms / n} for k, (n, ms) in prof.items()}


def summarize(times):
    import numpy as np
    a = np.asarray(times)
    return {"median_ms": float(np.median(a)), "mean_ms": float(a.mean()),
            "min_ms": float(a.min()), "max_ms": float(a.max()), "n": int(a.size)}


def run_workload(csa2, torch, w, args, touch, keys="f32", block_rule="max", tag=""):
    """Builds workload w on the device, times it, and returns its record."""
    log(f"[{w.name}{tag}] building inputs: B={w.B} Q={w.Q} max ctx={max(w.ctx)}")
    from gen.workloads import build_device
    t = build_device(w, keys=keys)
    step, _ = make_step(csa2, w, t, torch, keys, block_rule)
    touch.kind = "read"
    times = time_steps(torch, step, args.steps, args.warmup, touch)
    touch.kind = "rmw"
    st_rmw = summarize(time_steps(torch, step, args.steps, 0, touch))
    touch.kind = "read"
    st = summarize(times)
    ms = st["median_ms"]
    log(f"[{w.name}{tag}] median {ms:.4f} ms/step (min {st['min_ms']:.4f}, max "
        f"{st['max_ms']:.4f}); after a read-modify-write touch {st_rmw['median_ms']:.4f}")
    kern = kernel_times(csa2, torch, step, args.steps, touch)
    log(f"[{w.name}{tag}] kernels: " + json.dumps(kern))
    rec = {"value": w.Q / (ms * 1e-3), "unit": "queries/s", "ms_per_step": ms, "step_times": st,
           "rmw_touch": {"ms_per_step": st_rmw["median_ms"], "step_times": st_rmw,
                         "value": w.Q / (st_rmw["median_ms"] * 1e-3)},
           "workload": WORKLOAD_NAMES.get(w.name, w.name), "global_batch": w.Q,
           "kernels": kern, "roofline": dominant_roofline(w, kern, keys),
           "step_hbm": step_hbm(w, ms, keys)}
    if w.kind == "prefill":
        rec["mfma_utilisation"] = mfma_utilisation(w, kern)
    del t, step
    torch.cuda.empty_cache()
    return rec


# -------------------------------------------------------------- CPU baseline

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads(limit):
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, limit))


def _oracle_step(w, queries, inputs):
    """The oracle's whole step on `queries` (indices into the workload's
    queries); returns seconds spent in oracle calls (input generation and
    the packing of selected rows are not timed)."""
    import numpy as np

    import oracle
    from oracle import slices
    spent = 0.0
    qs = np.asarray(queries, np.int64)
    if w.kind == "decode_reindex":
        t0 = time.perf_counter()
        ridx = slices.reindex_batch(w, inputs["qI_reindex"][qs], inputs["pool_batch"])
        spent += time.perf_counter() - t0
        full = np.full((w.B, w.topk), -1, np.int32)
        full[qs] = ridx
        rows = slices.selected_rows(w, full, list(queries))
        for layer in range(w.layers):
            sk, sv = inputs["swa"][layer]
            t0 = time.perf_counter()
            oracle.attn_decode(inputs["q"][layer][qs], rows[0], rows[1], rows[2], rows[3],
                               sk[qs], sv[qs], w.swa_len()[qs], w.scale)
            spent += time.perf_counter() - t0
        return spent
    if w.kind in ("decode_full", "decode_hier"):
        kI, offs = inputs["kI"], inputs["offs"]
        nv = w.q_nvis()[qs]
        P = w.pool_blocks if w.kind == "decode_hier" else 0
        t0 = time.perf_counter()
        idx, pool = oracle.index_full(inputs["qI_full"][qs], kI, offs,
                                      np.arange(len(qs), dtype=np.int32), nv, w.Hi, w.Hk, w.Di,
                                      w.topk, P, w.block_size)
        spent += time.perf_counter() - t0
        full = np.full((w.B, w.topk), -1, np.int32)
        full[qs] = idx
        groups = []
        if w.kind == "decode_hier":
            groups.append((full, [inputs["q_full"]], [inputs["swa_full"]]))
            # Reindex over each query's pool (its rows regenerated and packed)
            pb = slices.pool_batch(w, _scatter_rows(w, qs, pool), list(queries))
            t0 = time.perf_counter()
            ridx = slices.reindex_batch(w, inputs["qI_reindex"][qs], pb)
            spent += time.perf_counter() - t0
            full = np.full((w.B, w.topk), -1, np.int32)
            full[qs] = ridx
        groups.append((full, inputs["q"], inputs["swa"]))
        for ix, qlist, swalist in groups:
            rows = slices.selected_rows(w, ix, list(queries))
            for ql, (sk, sv) in zip(qlist, swalist):
                t0 = time.perf_counter()
                oracle.attn_decode(ql[qs], rows[0], rows[1], rows[2], rows[3], sk[qs], sv[qs],
                                   w.swa_len()[qs], w.scale)
                spent += time.perf_counter() - t0
        return spent
    if w.kind == "prefill":
        # a contiguous run of chunk queries: one oracle call per layer
        i0, n = int(queries[0]), len(queries)
        nv = w.q_nvis()[i0:i0 + n]
        t0 = time.perf_counter()
        idx, _ = oracle.index_full(inputs["qI_full"][i0:i0 + n], inputs["kI"], [0],
                                   np.zeros(n, np.int32), nv, w.Hi, w.Hk, w.Di, w.topk)
        spent += time.perf_counter() - t0
        codes, scales = inputs["kv"]
        for layer in range(w.layers):
            sk, sv = inputs["swa"][layer]
            t0 = time.perf_counter()
            oracle.attn_prefill(inputs["q"][layer][i0:i0 + n], w.p0 + i0, codes, scales, idx,
                                sk[i0:i0 + n + w.W - 1], sv[i0:i0 + n + w.W - 1], w.W, w.scale)
            spent += time.perf_counter() - t0
        return spent
    raise ValueError(w.kind)


def _scatter_rows(w, qs, rows):
    """A [B, ...] array holding rows[j] at query qs[j] (others -1)."""
    import numpy as np
    out = np.full((w.B,) + rows.shape[1:], -1, rows.dtype)
    out[qs] = rows
    return out


def _oracle_inputs(w, queries):
    """Host inputs of `queries` for the oracle (generation, not timed)."""
    import numpy as np

    from gen.workloads import (FULL_LAYER, T_QI_FULL, T_QI_REINDEX, host_kI_rows, host_kv_rows,
                               host_q, host_qI, host_swa)
    from oracle import slices
    inp = {"q": [host_q(w, l) for l in range(w.layers)],
           "swa": [host_swa(w, l) for l in range(w.layers)]}
    if w.kind == "decode_reindex":
        inp["qI_reindex"] = host_qI(w, T_QI_REINDEX)
        inp["pool_batch"] = slices.pool_batch(w, w.pool, list(queries))
        return inp
    inp["qI_full"] = host_qI(w, T_QI_FULL)
    if w.kind == "prefill":
        inp["kI"] = host_kI_rows(w, 0, int(w.ctx[0]))
        inp["kv"] = host_kv_rows(w, 0, int(w.ctx[0]))
        return inp
    # decode Full layer: each query's whole sequence of keys, packed
    n = [int(w.ctx[b]) for b in queries]
    inp["offs"] = np.concatenate([[0], np.cumsum(n)[:-1]]).astype(np.int64)
    inp["kI"] = np.empty((sum(n), w.Hk, w.Di), np.float32)
    for j, b in enumerate(queries):
        o = int(inp["offs"][j])
        inp["kI"][o:o + n[j]] = host_kI_rows(w, int(w.seq_row_off[b]), n[j])
    if w.kind == "decode_hier":
        inp["qI_reindex"] = host_qI(w, T_QI_REINDEX)
        inp["q_full"] = host_q(w, FULL_LAYER)
        inp["swa_full"] = host_swa(w, FULL_LAYER)
    return inp


# queries of each workload the oracle runs: (all-core set, single-thread sample)
def baseline_queries(w):
    if w.kind == "prefill":
        mid = w.Qn // 2 - 128
        return list(range(mid, mid + 256)), list(range(mid, mid + 8))
    if w.kind == "decode_hier":
        return list(range(w.B)), [0]
    if w.kind == "decode_full":
        return list(range(w.B)), list(range(0, w.B, max(1, w.B // 4)))[:4]
    return list(range(w.B)), list(range(0, w.B, 4))


def cpu_baseline(w, max_threads):
    """The oracle, as it stands, on the host cores: every query of the
    workload (a labelled 256-query run of the prefill chunk) with all the
    threads the oracle can use, and a labelled sample on one thread."""
    import oracle
    allq, oneq = baseline_queries(w)
    threads = host_threads(max_threads)
    res = {"kind": "oracle", "unit": "queries/s", "cpu_model": cpu_model()}
    inp = _oracle_inputs(w, allq)
    used = min(threads, len(allq))
    oracle.set_threads(used)
    dt = _oracle_step(w, allq, inp)
    what = (f"chunk queries {allq[0]}..{allq[-1]} (positions {w.p0 + allq[0]}..{w.p0 + allq[-1]})"
            if w.kind == "prefill" else f"all {len(allq)} queries")
    res.update({"value": len(allq) / dt, "cores": used,
                "sample": f"{what}, whole step (every layer), {dt:.2f} s of oracle time"})
    oracle.set_threads(1)
    if w.kind != "prefill":
        del inp
        inp = _oracle_inputs(w, oneq)
    dt1 = _oracle_step(w, oneq, inp)
    res["single_thread"] = {"value": len(oneq) / dt1, "unit": "queries/s", "cores": 1,
                            "sample": f"queries {oneq}, whole step, {dt1:.2f} s"}
    oracle.set_threads(threads)
    return res


def kv_writer_bench(args, torch, csa2):
    """The KV writers.  FP4 main-KV writer: fp32 rows -> E2M1 codes + E4M3 scale per 16
    channels, on a 1M-entry context's main KV (1,048,576 entries x 512
    channels: 65,536 generated rows tiled 16 times, 2 GiB of fp32, more than
    the last-level cache holds), on the 65,536-entry prefill context and on
    one prefill chunk's append (4,096 queries, m = 2: 2,048 entries).  One
    step = one writer launch over all rows.  Also the FP8 window ring append
    (one token per sequence, W = 128) for 32, 4,096 and 65,536 sequences, in
    "swa_append"."""
    import oracle
    from gen import kv_rows_f32

    D = 512
    res_sizes = {}
    base = torch.from_numpy(kv_rows_f32(2, 9001, 65536, D)).cuda()
    for name, rows in (("context_1m", 1 << 20), ("context_64k", 65536), ("chunk_append", 2048)):
        x = base.repeat(rows // 65536, 1) if rows > 65536 else base[:rows].contiguous()
        codes = torch.empty((rows, D // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((rows, D // 16), dtype=torch.uint8, device="cuda")
        for _ in range(args.warmup):
            csa2.csa2_kv_quantize_fp4(x, codes, scales)
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            csa2.csa2_kv_quantize_fp4(x, codes, scales)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        csa2.profile_reset()
        csa2.profile_enable(True)
        for _ in range(args.steps):
            csa2.csa2_kv_quantize_fp4(x, codes, scales)
        torch.cuda.synchronize()
        n, kms = csa2.profile_read()["kv_quantize_fp4"]
        csa2.profile_enable(False)
        avg_us = 1000.0 * kms / n
        alg = rows * (4 * D + D // 2 + D // 16)     # fp32 read, codes + scale bytes written
        ach = alg / (avg_us * 1e-6) / 1e9
        res_sizes[name] = {"rows": rows, "ms_per_step": ms, "avg_us": avg_us,
                           "achieved_gbs": ach, "frac": ach / HBM_PEAK_GBS}
        log(f"kv writer {name}: rows={rows} {ms * 1e3:.1f} us/step, kernel {avg_us:.1f} us, "
            f"{ach:.0f} GB/s")
        del x, codes, scales
    del base
    # FP8 window ring append: one token per sequence, 512 channels of K and V
    swa = {}
    for B in (32, 4096, 65536):
        W = 128
        k = torch.randn((B, D), device="cuda")
        v = torch.randn((B, D), device="cuda")
        pos = torch.arange(B, dtype=torch.int64, device="cuda") * 7 + 1000
        rk = torch.zeros((B, W, D), dtype=torch.uint8, device="cuda")
        rv = torch.zeros_like(rk)
        for _ in range(args.warmup):
            csa2.csa2_swa_append(k, v, pos, rk, rv)
        csa2.profile_reset()
        csa2.profile_enable(True)
        for _ in range(args.steps):
            csa2.csa2_swa_append(k, v, pos, rk, rv)
        torch.cuda.synchronize()
        n, kms = csa2.profile_read()["swa_append"]
        csa2.profile_enable(False)
        avg_us = 1000.0 * kms / n
        alg = B * (2 * 4 * D + 2 * D)      # K and V: fp32 read, E4M3 bytes written
        ach = alg / (avg_us * 1e-6) / 1e9
        swa[f"B{B}"] = {"sequences": B, "avg_us": avg_us, "achieved_gbs": ach,
                        "frac": ach / HBM_PEAK_GBS}
        log(f"swa append B={B}: kernel {avg_us:.2f} us, {ach:.0f} GB/s")
        del k, v, pos, rk, rv
    big = res_sizes["context_1m"]
    res = {
        "metric": "FP4 main-KV writer rows/s (fp32 -> E2M1 + E4M3 per 16 channels) at 1 MI355X",
        "value": big["rows"] / (big["ms_per_step"] * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": big["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (N(0,1) rows, each 16-channel group scaled by 2^U[-30,14))",
        "config": {"workload": "FP4 main-KV writer: 1,048,576 entries x 512 channels",
                   "rows": big["rows"], "D": D, "parallelism": "single GPU"},
        "sizes": res_sizes,
        "swa_append": swa,
        "roofline": {"bound": "hbm", "kernel": "kv_quantize_fp4", "achieved": big["achieved_gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": big["frac"],
                     "traffic": measured_traffic("kv_writer_1m_rows.md")},
    }
    if not args.no_cpu_baseline:
        rows = 16384
        xs = kv_rows_f32(2, 9001, rows, D)
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.fp4_quantize_rows(xs)
            reps += 1
            if time.perf_counter() - t0 > 5.0:
                break
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": reps * rows / dt, "unit": "rows/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{reps} x {rows} rows x {D} channels, {dt:.2f} s"}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=None,
                    help="run one workload alone (0-4); default: the mixed-length serving "
                         "decode workload as the line's value, the others as extra keys")
    ap.add_argument("--cpu-threads", type=int, default=16)
    ap.add_argument("--keys", choices=("f32", "e4m3"), default="f32",
                    help="indexer-key cache: fp32 (the workloads as stated) or E4M3 bytes")
    ap.add_argument("--no-extras", action="store_true",
                    help="default line: skip the other workloads and the E4M3 key-cache figure")
    ap.add_argument("--pool-blocks", type=int, default=None,
                    help="hierarchical workload: blocks in the candidate pool (default 2,048)")
    ap.add_argument("--block-size", type=int, default=None,
                    help="hierarchical workload: positions per block (default 8)")
    ap.add_argument("--block-rule", choices=("max", "sum"), default="max",
                    help="hierarchical workload: block score of the candidate pool")
    ap.add_argument("--kv-writer", action="store_true",
                    help="measure the FP4 main-KV writer alone (its own JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (reference "
                         "kernel of known traffic for the hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the path is single-GPU "
              "and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": src.numel() * 4,
                          "calibrate_copy_bytes_written": dst.numel() * 4, "launches": 3}))
        return
    import compressed_fp4_kv_amd as csa2
    from gen.workloads import workload
    if args.kv_writer:
        kv_writer_bench(args, torch, csa2)
        return

    wid = HEADLINE if args.workload is None else args.workload
    w = workload(wid)
    pool_variant = (args.pool_blocks, args.block_size, args.block_rule) != (None, None, "max")
    if pool_variant:
        if w.kind != "decode_hier":
            print("--pool-blocks / --block-size / --block-rule apply to --workload 3 only",
                  file=sys.stderr)
            sys.exit(2)
        w.pool_blocks = args.pool_blocks or w.pool_blocks
        w.block_size = args.block_size or w.block_size
    touch = Touch(torch)
    torch.cuda.synchronize()
    head = run_workload(csa2, torch, w, args, touch, args.keys, args.block_rule)
    res = {
        "metric": "CSA2 decode queries/sec and achieved HBM GB/s (% of peak) at 1 MI355X",
        "value": head["value"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded integer indexer inputs, FP4 E2M1/E4M3 KV, N(0,1) queries, "
                "FP8 window)",
        "config": {"workload": head["workload"] + (
                       "; indexer keys stored as E4M3FN bytes" if args.keys == "e4m3" else "") + (
                       f"; pool {w.pool_blocks} blocks x {w.block_size}, block score "
                       f"{args.block_rule}" if pool_variant else ""),
                   "global_batch": w.Q, "seq_len": int(max(w.ctx)), "total_entries": w.rows,
                   "parallelism": "single GPU"},
        "timing": "median of the timed steps, each between its own HIP events, 1 GiB read "
                  "between steps; rmw_touch: the same steps after a read-modify-write of the "
                  "1 GiB",
        "step_times": head["step_times"],
        "rmw_touch": head["rmw_touch"],
        "kernels": head["kernels"],
        "roofline": head["roofline"],
        "step_hbm": head["step_hbm"],
    }
    if "mfma_utilisation" in head:
        res["mfma_utilisation"] = head["mfma_utilisation"]
    if args.workload is None and not args.no_extras:
        if args.keys == "f32":
            # the same step over the compact indexer-key cache (E4M3 bytes), a
            # storage variant reported beside the fp32 figure, never as `value`
            r8 = run_workload(csa2, torch, workload(wid), args, touch, "e4m3", tag=" e4m3 keys")
            res["e4m3_keys"] = {k: r8[k] for k in ("value", "unit", "ms_per_step", "step_times",
                                                   "rmw_touch", "kernels", "roofline",
                                                   "step_hbm")}
            res["e4m3_keys"]["config"] = "same step, indexer keys stored as E4M3FN bytes"
        other = {}
        for oid in (1, 3, 2):
            ow = workload(oid)
            other[ow.name] = run_workload(csa2, torch, ow, args, touch)
        res["other_workloads"] = other
    del touch
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline and "other_workloads" in res:
        for name, rec in res["other_workloads"].items():
            ow = workload({"c1_full_reuse3": 1, "c3_hier_1m": 3, "c2_prefill_m2": 2}[name])
            log(f"[{name}] cpu baseline (oracle) ...")
            rec["cpu_baseline"] = cpu_baseline(ow, args.cpu_threads)
    if not args.no_cpu_baseline:
        log(f"[{w.name}] cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_threads)
        log(f"[{w.name}] cpu baseline: {json.dumps(res['cpu_baseline'])}")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
