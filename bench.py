"""CSA2 decode benchmark on one MI355X.

One step = one CSA2 decoder layer group on the decode workload of 32
sequences x 65,536 entries: the Full layer's indexer (score stream over
32 x 65,536 fp32 key rows of 4 heads x 128 dims, exact Top-512), then
sparse attention for the Full layer and its 3 Reuse layers (64 heads x 512
channels over the 512 selected FP4 rows + a 128-token FP8 window, each layer
with its own query and window; the four layers share the indices and the
KV and go in one csa2_sparse_attn_decode_layers call).  Inputs are seeded synthetic tensors already
resident in HBM.  Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N] [--keys f32|e4m3]
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

WORKLOAD_NAMES = {
    "c0_tiny_full": "decode Full layer: 1 sequence x 4,096 entries, indexer 4x64, Top-64, 16 heads",
    "c1_full_reuse3": "decode Full + 3 Reuse layers: 32 sequences x 65,536 entries, indexer 4x128 "
                      "fp32, Top-512, 64 heads x 512 ch, FP4 main KV, 128-token FP8 window",
    "c2_prefill_m2": "prefill chunk, m=2: 4,096 queries over 65,536 entries, Full + 5 Reuse layers",
    "c3_hier_1m": "decode, 8 sequences x 1,048,576 entries: Full indexer + 2,048x8 pool, Reindex "
                  "+ 3 Reuse layers",
    "c4_mixed_reindex": "decode, 64 sequences of 8K..1M entries: Reindex over inherited pools + "
                        "3 Reuse layers",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(profile="score_stream_c1_traffic.md"):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a plain-copy calibration),
    or None if the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    try:
        for line in open(path):
            if line.startswith("traffic_record:"):
                rec = json.loads(line.split(":", 1)[1])
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
        nb = csa2.csa2_decode_layers_workspace_bytes(w.layers, Q, w.H, w.D, w.topk, w.W)
    ws_a = torch.empty(max(256, nb), dtype=torch.uint8, device=dev)
    outs = [torch.empty((Q, w.H, w.D), dtype=torch.float32, device=dev) for _ in range(w.layers)]
    lses = [torch.empty((Q, w.H), dtype=torch.float32, device=dev) for _ in range(w.layers)]

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
            # the Full layer's indexer builds Top-K and the candidate pool
            csa2.csa2_index_full_ex(t["qI_full"], kI, t["seq_row_off"], t["q_seq"], t["q_nvis"],
                                    max_nvis, w.topk, idx, P, w.block_size, pool,
                                    block_rule=block_rule, ws=ws_i)
        # Reindex layer over the pool, then Reindex + Reuse layers' attention
        reindex(t["qI_reindex"], kI, t["seq_row_off"], t["q_seq"], t["q_nvis"], pool,
                w.block_size, w.topk, ridx, ws=ws_r)
        attn_layers(ridx)
    return step, idx


def dominant_roofline(w, kern, keys="f32"):
    """Roofline record of the workload's dominant kernel (algorithmic work per
    launch / measured average launch time).  Key bytes per value: 4 (fp32) or
    1 (E4M3 key cache)."""
    sfx, vb = ("_e4m3", 1) if keys == "e4m3" else ("", 4)
    stream, rscore = "score_stream" + sfx, "reindex_score" + sfx
    if w.kind in ("decode_full", "decode_hier") and stream in kern:
        alg = float(w.rows) * w.row_width * vb + float(w.Q) * w.Hi * w.Di * 4
        ach = alg / (kern[stream]["avg_us"] * 1e-6) / 1e9
        traffic = None
        if w.name.startswith("c1"):
            traffic = measured_traffic("score_stream_e4m3_c1_traffic.md" if sfx
                                       else "score_stream_c1_traffic.md")
        return {"bound": "hbm", "kernel": stream, "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": traffic}
    if w.kind == "decode_reindex" and rscore in kern:
        import numpy as np
        rows = sum(min(int(np.sum(w.pool[b] >= 0)) * w.block_size, w.ctx[b]) for b in range(w.B))
        alg = float(rows) * w.row_width * vb
        ach = alg / (kern[rscore]["avg_us"] * 1e-6) / 1e9
        return {"bound": "hbm", "kernel": rscore, "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": None}
    if "attn" in kern:
        return mfma_utilisation(w, kern)["attn"] | {"traffic": None}
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
        if w.pool is not None:
            cand = sum(min(int(np.sum(w.pool[b] >= 0)) * w.block_size, w.ctx[b])
                       for b in range(w.B))
        else:
            cand = sum(min(w.pool_blocks * w.block_size, w.ctx[b]) for b in range(w.B))
        total += float(cand) * rb + w.Q * qb
    sel = np.minimum(w.q_nvis(), w.topk).astype(np.float64)
    win = float(w.swa_rows() if w.kind == "prefill" else w.B * w.W)
    per_layer = (2.0 * w.Q * w.H * w.D * 4 + float(np.sum(sel)) * (w.D // 2 + w.D // 16)
                 + win * 2 * w.D + w.Q * w.topk * 4)
    if w.kind == "prefill":
        # every query's selected rows come from one 65,536-entry sequence:
        # the unique rows bound the compulsory bytes
        per_layer = (2.0 * w.Q * w.H * w.D * 4 + min(float(np.sum(sel)), float(w.ctx[0]))
                     * (w.D // 2 + w.D // 16) + win * 2 * w.D + w.Q * w.topk * 4)
    total += w.layers * per_layer
    ach = total / (ms_step * 1e-3) / 1e9
    return {"algorithmic_bytes": total, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBS}


def mfma_utilisation(w, kern):
    """Algorithmic flops per launch / measured launch time of the matrix-core
    kernels, against the dense fp16/bf16 peak (the two-part fp16 splits of
    the attention execute twice the algorithmic flops; they are not counted)."""
    res = {}
    if "attn" in kern:
        # QK^T and PV, 2 flops per MAC; a decode launch covers the group's layers
        flops = 4.0 * w.H * (w.topk + w.W) * w.D * w.Q * (1 if w.kind == "prefill" else w.layers)
        ach = flops / (kern["attn"]["avg_us"] * 1e-6) / 1e12
        res["attn"] = {"bound": "mfma", "kernel": "attn (fp16 MFMA)", "achieved": ach,
                       "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
                       "frac": ach / MFMA_F16_PEAK_TFS}
    if "prefill_scores" in kern:
        import numpy as np
        flops = 2.0 * float(np.sum(w.q_nvis())) * w.Hi * w.Di   # visible (query, entry) dots
        ach = flops / (kern["prefill_scores"]["avg_us"] * 1e-6) / 1e12
        res["prefill_scores"] = {"bound": "mfma", "kernel": "prefill_scores (bf16 MFMA)",
                                 "achieved": ach, "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
                                 "frac": ach / MFMA_F16_PEAK_TFS}
    return res


def cpu_baseline(w, max_threads, keys="f32"):
    """The oracle on the host cores, on the same workload (whole batch)."""
    import oracle
    from gen.workloads import (T_QI_FULL, host_kI_rows, host_kI_rows_e4m3, host_kv_rows, host_q,
                               host_qI, host_swa)

    threads = max(1, min(max_threads, w.B))
    oracle.set_threads(threads)
    kI = (host_kI_rows_e4m3 if keys == "e4m3" else host_kI_rows)(w, 0, w.rows)
    qI = host_qI(w, T_QI_FULL)
    codes, scales = host_kv_rows(w, 0, w.rows)
    qs = [host_q(w, l) for l in range(w.layers)]
    swa = [host_swa(w, l) for l in range(w.layers)]
    t0 = time.perf_counter()
    idx, _ = oracle.index_full(qI, kI, w.seq_row_off, w.q_seq(), w.q_nvis(), w.Hi, w.Hk, w.Di,
                               w.topk)
    for l in range(w.layers):
        oracle.attn_decode(qs[l], codes, scales, w.seq_row_off, idx, swa[l][0], swa[l][1],
                           w.swa_len(), w.scale, want_lse=True)
    dt = time.perf_counter() - t0
    del kI
    return {"value": w.B / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"whole step on all {w.B} queries (index_full + {w.layers} attention layers), "
                      f"{dt:.2f} s"}


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
    ap.add_argument("--workload", type=int, default=1,
                    help="workload number (1 = the decode workload the metric is quoted on)")
    ap.add_argument("--cpu-threads", type=int, default=16)
    ap.add_argument("--keys", choices=("f32", "e4m3"), default="f32",
                    help="indexer-key cache: fp32 (the workloads as stated) or E4M3 bytes")
    ap.add_argument("--no-e4m3-line", action="store_true",
                    help="decode workload: skip the E4M3 key-cache figure added to the line")
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
    from gen.workloads import build_device, workload
    if args.kv_writer:
        kv_writer_bench(args, torch, csa2)
        return

    w = workload(args.workload)
    pool_variant = (args.pool_blocks, args.block_size, args.block_rule) != (None, None, "max")
    if pool_variant:
        if w.kind != "decode_hier":
            print("--pool-blocks / --block-size / --block-rule apply to --workload 3 only",
                  file=sys.stderr)
            sys.exit(2)
        w.pool_blocks = args.pool_blocks or w.pool_blocks
        w.block_size = args.block_size or w.block_size
    log(f"building inputs: {w.name} B={w.B} ctx={w.ctx[0]} H={w.H} topk={w.topk}")
    t = build_device(w, keys=args.keys)
    step, idx = make_step(csa2, w, t, torch, args.keys, args.block_rule)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"timed: {ms_step:.3f} ms/step")

    # kernel breakdown: same steps again with per-launch events on the launch stream
    csa2.profile_reset()
    csa2.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = csa2.profile_read()
    csa2.profile_enable(False)
    kern = {k: {"launches": n, "avg_us": 1000.0 * ms / n} for k, (n, ms) in prof.items()}
    log("kernels:", json.dumps(kern))

    res = {
        "metric": "CSA2 decode queries/sec and achieved HBM GB/s (% of peak) at 1 MI355X",
        "value": w.Q / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded integer indexer inputs, FP4 E2M1/E4M3 KV, N(0,1) queries, "
                "FP8 window)",
        "config": {"workload": WORKLOAD_NAMES.get(w.name, w.name) + (
                       "; indexer keys stored as E4M3FN bytes" if args.keys == "e4m3" else "") + (
                       f"; pool {w.pool_blocks} blocks x {w.block_size}, block score "
                       f"{args.block_rule}" if pool_variant else ""),
                   "global_batch": w.Q, "seq_len": int(max(w.ctx)), "parallelism": "single GPU"},
        "kernels": kern,
        "roofline": dominant_roofline(w, kern, args.keys),
        "step_hbm": step_hbm(w, ms_step, args.keys),
    }
    if w.kind == "prefill":
        res["mfma_utilisation"] = mfma_utilisation(w, kern)
    if args.workload == 1 and args.keys == "f32" and not args.no_e4m3_line:
        # the same step over the compact indexer-key cache (E4M3 bytes), a
        # storage variant reported beside the fp32 figure, never as `value`
        from gen.workloads import dev_kI_e4m3
        del t["kI"]
        torch.cuda.empty_cache()
        t["kI8"] = dev_kI_e4m3(w)
        step8, _ = make_step(csa2, w, t, torch, "e4m3")
        for _ in range(args.warmup):
            step8()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            step8()
        e1.record(stream)
        torch.cuda.synchronize()
        ms8 = e0.elapsed_time(e1) / args.steps
        csa2.profile_reset()
        csa2.profile_enable(True)
        for _ in range(args.steps):
            step8()
        torch.cuda.synchronize()
        prof8 = csa2.profile_read()
        csa2.profile_enable(False)
        kern8 = {k: {"launches": n, "avg_us": 1000.0 * ms / n} for k, (n, ms) in prof8.items()}
        res["e4m3_keys"] = {"value": w.Q / (ms8 * 1e-3), "unit": "queries/s", "ms_per_step": ms8,
                            "config": "same step, indexer keys stored as E4M3FN bytes (512 B "
                                      "rows instead of 2 KB)",
                            "kernels": kern8, "roofline": dominant_roofline(w, kern8, "e4m3"),
                            "step_hbm": step_hbm(w, ms8, "e4m3")}
        log(f"e4m3 keys: {ms8:.3f} ms/step")
    del t
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline and args.workload == 1:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_threads, args.keys)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
