"""CSA2 decode benchmark on one MI355X.

One step = one CSA2 decoder layer group on the decode workload of 32
sequences x 65,536 entries: the Full layer's indexer (score stream over
32 x 65,536 fp32 key rows of 4 heads x 128 dims, exact Top-512), then
sparse attention for the Full layer and its 3 Reuse layers (64 heads x 512
channels over the 512 selected FP4 rows + a 128-token FP8 window, each layer
with its own query and window).  Inputs are seeded synthetic tensors already
resident in HBM.  Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic():
    """HBM bytes per score-stream launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a plain-copy calibration),
    or None if the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "score_stream_c1_traffic.md")
    try:
        for line in open(path):
            if line.startswith("traffic_record:"):
                rec = json.loads(line.split(":", 1)[1])
                src = open(os.path.join(ROOT, rec["source"]), "rb").read()
                if hashlib.sha256(src).hexdigest()[:16] == rec["source_sha256_16"]:
                    return rec["traffic_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        pass
    return None


def make_step(csa2, w, t, torch):
    Q = w.B
    max_nvis = int(max(w.ctx))
    idx = torch.empty((Q, w.topk), dtype=torch.int32, device="cuda")
    ws_i = torch.empty(csa2.csa2_index_full_workspace_bytes(Q, max_nvis, w.topk, 0, 8),
                       dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(256, csa2.csa2_decode_workspace_bytes(Q, w.H, w.D, w.topk, w.W)),
                       dtype=torch.uint8, device="cuda")
    outs = [torch.empty((Q, w.H, w.D), dtype=torch.float32, device="cuda") for _ in range(w.layers)]
    lses = [torch.empty((Q, w.H), dtype=torch.float32, device="cuda") for _ in range(w.layers)]

    def step():
        csa2.csa2_index_full(t["qI_full"], t["kI"], t["seq_row_off"], t["q_seq"], t["q_nvis"],
                             max_nvis, w.topk, idx, ws=ws_i)
        for layer in range(w.layers):   # Full layer, then Reuse layers: same idx and KV
            csa2.csa2_sparse_attn_decode(t["q"][layer], t["kv_codes"], t["kv_scales"],
                                         t["seq_row_off"], idx, t["swa_k"][layer],
                                         t["swa_v"][layer], t["swa_len"], w.scale, outs[layer],
                                         lses[layer], ws=ws_a)
    return step, idx


def cpu_baseline(w, max_threads):
    """The oracle on the host cores, on the same workload (whole batch)."""
    import numpy as np
    import oracle
    from gen.workloads import T_QI_FULL, host_kI_rows, host_kv_rows, host_q, host_qI, host_swa

    threads = max(1, min(max_threads, w.B))
    oracle.set_threads(threads)
    kI = host_kI_rows(w, 0, w.rows)
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=16)
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

    w = workload(1)
    log(f"building inputs: {w.name} B={w.B} ctx={w.ctx[0]} H={w.H} topk={w.topk}")
    t = build_device(w)
    step, idx = make_step(csa2, w, t, torch)
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

    key_bytes = float(w.rows) * w.row_width * 4
    q_bytes = float(w.B) * w.Hi * w.Di * 4
    alg = key_bytes + q_bytes
    ss = kern.get("score_stream")
    ach = alg / (ss["avg_us"] * 1e-6) / 1e9 if ss else None

    res = {
        "metric": "CSA2 decode queries/sec and achieved HBM GB/s (% of peak) at 1 MI355X",
        "value": w.B / (ms_step * 1e-3),
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
        "config": {"workload": "decode Full + 3 Reuse layers: 32 sequences x 65,536 entries, "
                               "indexer 4x128 fp32, Top-512, 64 heads x 512 ch, FP4 main KV, "
                               "128-token FP8 window",
                   "global_batch": w.B, "seq_len": int(w.ctx[0]), "parallelism": "single GPU"},
        "step_hbm_gbs": (alg + w.layers * w.B * (512 * 288 + 2 * 128 * 512 + 2 * w.H * w.D * 4))
                        / (ms_step * 1e-3) / 1e9,
        "kernels": kern,
        "roofline": {"bound": "hbm", "kernel": "score_stream", "achieved": ach,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": (ach / HBM_PEAK_GBS) if ach else None,
                     "traffic": measured_traffic()},
    }
    del t
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_threads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
