"""Benchmark of the speculative-sampling verify step on one MI355X.

One step = one chain verify (row statistics, accept/reject, residual or bonus
draw, emit) over one batch of the chain_t1_128k workload: B=64 sequences,
K=5 drafts, V=128256, bf16 logits, T=1 (180,584,448 logit bytes).  Inputs are
resident in HBM before timing; several input sets rotate so that the 256 MB
Infinity Cache cannot hold the working set between steps.

Prints one JSON line.  `roofline` covers the streaming statistics kernel (the
dominant one), timed alone with HIP events on the launch stream;
`cpu_baseline` times the fp64 oracle on a bounded sample on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "verify steps/s (B×(K+1)×V logits) + achieved HBM GB/s vs peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chain_stats_chain_t1_128k_traffic.json")
STATS_KERNEL_SRC = [os.path.join(ROOT, "speculative_decoding_verification_08_amd", "csrc", f)
                    for f in ("chain.hip", "device.hpp", "plan.hpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in STATS_KERNEL_SRC:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def to_dev(a, device):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def measured_traffic(algo_bytes: float):
    """HBM bytes per launch from the committed PMC summary, if it was taken on this kernel."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    t = json.load(open(TRAFFIC_FILE))
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(inp, budget_s: float, gpu_out):
    """The oracle as it stands, single-threaded, on whole steps of the same workload."""
    import oracle
    from oracle import parity
    t0 = time.perf_counter()
    steps = 0
    while True:
        oracle.verify_chain(inp["target"], inp["draft"], inp["tokens"], inp["u_accept"],
                            inp["u_sample"], inp["T"])
        steps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    counts = parity.check_chain(inp, *gpu_out)
    return {"value": steps / dt, "unit": "verify steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} whole steps of input set 0 (B=64, K=5, V=128256), fp64, one thread, "
                      f"{dt:.1f} s", "parity_on_sample": dict(counts)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--rotate", type=int, default=3, help="input sets cycled through")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verify step runs independently per "
              "sequence batch and this build has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import speculative_decoding_verification_08_amd as sv
    import workloads as W

    w = W.WORKLOADS["chain_t1_128k"]
    B, K, V = w.B, w.K, w.V
    device = torch.device("cuda:0")
    print(f"[bench] generating {args.rotate} input sets of {w.name}", file=sys.stderr, flush=True)
    host_sets = [W.chain_inputs(w, s) for s in range(args.rotate)]
    sets = [{k: to_dev(v, device) for k, v in h.items() if isinstance(v, np.ndarray)} for h in host_sets]
    ws = sv.workspace(sv.SPEC_MODE_CHAIN, B, K, V, sv.SPEC_DTYPE_BF16, device)
    out_t = torch.empty((B, K + 1), dtype=torch.int32, device=device)
    out_a = torch.empty((B,), dtype=torch.int32, device=device)
    stream = torch.cuda.current_stream(device)

    def step(i):
        s = sets[i % len(sets)]
        sv.spec_verify_chain(s["target"], s["draft"], s["tokens"], s["u_accept"], s["u_sample"],
                             w.T, out_tokens=out_t, out_accepted=out_a, workspace_buf=ws,
                             stream=stream)

    def stats_only(i):
        s = sets[i % len(sets)]
        sv.spec_verify_chain_stats(s["target"], s["draft"], w.T, ws, stream=stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # whole steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # the streaming statistics kernel alone, back to back on the same stream
    for i in range(args.warmup):
        stats_only(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        stats_only(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_stats = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {ms_step * 1e3:.2f} us/step, stats kernel {ms_stats * 1e3:.2f} us", file=sys.stderr,
          flush=True)

    # outputs of set 0 for the oracle comparison and the emitted-token rate
    step(0)
    diag = torch.empty((B, K + 1, 4), dtype=torch.float32, device=device)
    s0 = sets[0]
    tok, acc, _ = sv.spec_verify_chain(s0["target"], s0["draft"], s0["tokens"], s0["u_accept"],
                                       s0["u_sample"], w.T, out_diag=diag)
    torch.cuda.synchronize()
    gpu_out = (tok.cpu().numpy(), acc.cpu().numpy(), diag.cpu().numpy())

    algo_bytes = B * (2 * K + 1) * V * 2                        # every logit read once
    io_bytes = 4 * B * K + 4 * B * (K + 1) + 4 * B * (K + 2)   # tokens, uniforms, outputs
    steps_per_s = 1e3 / ms_step
    achieved_step = (algo_bytes + io_bytes) / (ms_step * 1e-3) / 1e9
    achieved_stats = algo_bytes / (ms_stats * 1e-3) / 1e9
    traffic = measured_traffic(algo_bytes)
    line = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "verify steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "mode": "chain", "B": B, "K": K, "V": V, "T": w.T,
                   "logits": "bf16", "input_sets_rotated": args.rotate,
                   "logit_bytes_per_step": algo_bytes},
        "achieved_GBps": achieved_step,
        "frac_of_hbm_peak": achieved_step / HBM_PEAK_GBPS,
        "tokens_verified_per_s": steps_per_s * B * K,
        "tokens_emitted_per_s": steps_per_s * float((gpu_out[1] + 1).sum()),
        "roofline": {"kernel": "k_chain_stats", "bound": "hbm", "achieved": achieved_stats,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved_stats / HBM_PEAK_GBPS,
                     "traffic": traffic, "avg_launch_us": ms_stats * 1e3,
                     "algorithmic_bytes_per_launch": algo_bytes},
    }
    if not args.no_cpu_baseline:
        print("[bench] oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(host_sets[0], args.cpu_seconds, gpu_out)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
