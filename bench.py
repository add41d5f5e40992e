"""Benchmark of the speculative-sampling verify step on one MI355X.

One step = one chain verify (row statistics, accept/reject, residual or bonus
draw, emit) over one batch of the chain_t1_128k workload: B=64 sequences,
K=5 drafts, V=128256, bf16 logits, T=1 (180,584,448 logit bytes).  Inputs are
resident in HBM before timing; enough logit sets rotate (3 here, 542 MB) that
the 256 MB Infinity Cache cannot hold the working set between steps, and every
timed step draws with uniforms of its own.  `--workload` measures the other
workloads the same way.

Prints one JSON line.  A chain step is one kernel (k_chain_fused: the
statistics pass over every logit, the accept test, the residual or bonus draw
and the emission), so `roofline` covers that kernel, i.e. the whole step,
timed back to back with HIP events on the launch stream; the statistics pass
alone (the two-phase entry point's first kernel) is reported beside it.
`cpu_baseline` times the fp64 oracle on a bounded sample on the host, on one
thread and on the host threads the process may use.
"""
from __future__ import annotations

import argparse
import functools
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "verify steps/s (B×(K+1)×V logits) + achieved HBM GB/s vs peak"
CHAIN_KERNEL_SRC = [os.path.join(ROOT, "speculative_decoding_verification_08_amd", "csrc", f)
                    for f in ("chain.hip", "device.hpp", "handover.hpp", "plan.hpp", "fastdiv.hpp",
                              "grid_order.hpp", "planning.hpp", "abi.hip")]


def code_tokens(text: str) -> str:
    """Source text with comments removed and whitespace collapsed, so that a
    comment-only edit does not count as a change of the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the chain kernel's code (comments and layout ignored): the HBM
    traffic figures under profiles/ hold for the code they were taken on."""
    h = hashlib.sha256()
    for p in CHAIN_KERNEL_SRC:
        h.update(code_tokens(open(p).read()).encode())
    return h.hexdigest()[:16]


def to_dev(a, device):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def measured_traffic(workload: str):
    """HBM bytes per launch of the chain kernel from the committed PMC summary,
    if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"k_chain_fused_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def kv_bytes(w, count) -> int:
    """KV commit: every committed row read from the scratch and written to
    the cache, in every plane."""
    return 2 * int(np.asarray(count).sum()) * w.planes * w.row_bytes


def kv_cache_pattern(w, device):
    """The initial cache on the device: byte j of the flat array is
    (7 j + 3) mod 251 (filled a plane at a time)."""
    import torch
    shape = (w.planes, w.B, w.slots, w.row_bytes)
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    per = w.B * w.slots * w.row_bytes
    for l in range(w.planes):
        j = torch.arange(l * per, (l + 1) * per, dtype=torch.int64, device=device)
        out[l] = ((j * 7 + 3) % 251).to(torch.uint8).view(shape[1:])
    return out


@functools.lru_cache(maxsize=2)
def kv_scratch_host(w):
    """The KV commit's scratch rows on the host, generated once per workload."""
    import workloads as W
    return W.kv_scratch(w, 0)


def kv_sample(w, inp):
    """The CPU leg's sample of a KV commit step: plane 0 of every sequence."""
    per = w.B * w.slots * w.row_bytes
    cache0 = ((np.arange(per, dtype=np.int64) * 7 + 3) % 251).astype(np.uint8)
    return dict(scratch=kv_scratch_host(w)[:1], cache=cache0.reshape(1, w.B, w.slots, w.row_bytes),
                **{k: inp[k] for k in ("path", "count", "cache_len")})


def set_bytes(w, inputs=None) -> int:
    """Logit bytes one step reads (every row once).  Per-sequence trees read
    only their trees' rows: their node counts when `inputs` are given, else
    the bound of Nmax rows per sequence."""
    esize = 2 if w.dtype == "bf16" else 4
    if w.mode == "chain":
        rows = w.B * (2 * w.K + 1)
    elif w.mode == "greedy":
        rows = w.B * (w.K + 1)
    elif w.mode == "tree_dyn":
        rows = int(inputs["node_count"].sum()) if inputs is not None else w.B * w.K
    elif w.mode == "topk":
        rows = w.B
    elif w.mode == "kv":
        return kv_bytes(w, inputs["count"]) if inputs is not None else 2 * w.B * 4 * w.planes * w.row_bytes
    elif w.mode == "mask":   # parents and counts read, mask words and depths written
        return w.B * w.K * 4 + w.B * 4 + w.B * w.K * ((w.K + 31) // 32) * 4 + w.B * w.K * 4
    else:
        rows = w.B * (1 + sum(int(np.prod(w.branching[:i + 1])) for i in range(len(w.branching))))
    return rows * w.V * esize


def oracle_step(w, inp):
    import oracle
    if w.mode == "chain":
        return oracle.verify_chain(inp["target"], inp["draft"], inp["tokens"], inp["u_accept"],
                                   inp["u_sample"], inp["T"])
    if w.mode == "greedy":
        return oracle.verify_greedy(inp["target"], inp["tokens"])
    if w.mode == "tree_dyn":
        return oracle.verify_tree_greedy_dyn(inp["node_logits"], inp["node_tokens"], inp["parents"],
                                             inp["node_count"])
    if w.mode == "topk":
        return oracle.topk(inp["logits"], w.K)
    if w.mode == "kv":
        return oracle.kv_commit(inp["scratch"], inp["cache"], inp["path"], inp["count"],
                                inp["cache_len"])
    if w.mode == "mask":
        return oracle.tree_mask(inp["parents"], inp["node_count"])
    return oracle.verify_tree_greedy(inp["node_logits"], inp["node_tokens"], inp["parents"])


def check(w, inp, gpu_out):
    from oracle import parity
    if w.mode == "chain":
        return parity.check_chain(inp, *gpu_out)
    if w.mode == "greedy":
        return parity.check_greedy(inp, *gpu_out)
    if w.mode == "tree_dyn":
        return parity.check_tree_dyn(inp, *gpu_out)
    if w.mode == "topk":
        return parity.check_topk(inp, *gpu_out)
    if w.mode == "mask":
        want_m, want_d = oracle_step(w, inp)
        assert np.array_equal(gpu_out[0], want_m) and np.array_equal(gpu_out[1], want_d), \
            "tree mask differs from the oracle's"
        return {"sequences": int(w.B), "exact": int(w.B)}
    if w.mode == "kv":   # plane 0 of every sequence, and every new length
        want_c, want_l = oracle_step(w, inp)
        got_c0, got_l = gpu_out
        assert np.array_equal(got_l, want_l), "KV commit lengths differ from the oracle's"
        assert np.array_equal(got_c0, want_c[0]), "KV commit plane 0 differs from the oracle's"
        return {"sequences": int(w.B), "exact": int(w.B)}
    return parity.check_tree(inp, *gpu_out)


def cpu_baseline(w, inp, budget_s: float, gpu_out):
    """The oracle as it stands on whole steps of the same workload (for the KV
    commit, on one plane of the step, scaled), timed twice: on one thread, and
    with its sequences spread over the host threads this process may use
    (OMP_NUM_THREADS when set, else its CPU affinity).  Each leg takes about
    half of `budget_s`.  The oracle's results do not depend on the thread
    count."""
    import oracle
    scale, what = 1.0, "whole steps"
    if w.mode == "kv":
        inp = kv_sample(w, inp)
        scale, what = 1.0 / w.planes, f"steps on plane 0 of {w.planes} (rate scaled by 1/{w.planes})"
    host = host_cpu()

    def leg(threads):
        used = oracle.set_threads(threads)
        oracle_step(w, inp)                     # untimed: first-touch and thread start-up
        t0 = time.perf_counter()
        steps = 0
        while True:
            oracle_step(w, inp)
            steps += 1
            if time.perf_counter() - t0 >= budget_s / 2:
                break
        dt = time.perf_counter() - t0
        return {"value": steps / dt * scale, "cores": used,
                "sample": f"{steps} {what} of input set 0 of {w.name}, {used} thread(s), {dt:.1f} s"}
    one = leg(1)
    many = leg(host["threads_usable"])
    oracle.set_threads(1)
    counts = check(w, inp, gpu_out)
    unit = {"topk": "top-k steps/s", "kv": "KV commit steps/s",
            "mask": "tree mask steps/s"}.get(w.mode, "verify steps/s")
    return {"value": many["value"], "unit": unit, "cores": many["cores"], "kind": "oracle",
            "sample": many["sample"], "single_thread": one, "host": host,
            "parity_on_sample": dict(counts)}


def host_cpu() -> dict:
    """The host the CPU leg ran on: CPU model, the processors the OS shows
    (nproc), and the threads this process may use."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    omp = os.environ.get("OMP_NUM_THREADS", "")
    usable = int(omp) if omp.isdigit() and int(omp) > 0 else affinity
    return {"cpu": model, "nproc": os.cpu_count(), "affinity": affinity,
            "OMP_NUM_THREADS": omp or None, "threads_usable": min(usable, affinity)}


def graph_replay(make, sets, stream, G: int, steps: int) -> dict:
    """Per-step time of G consecutive steps (input sets in turn) captured in
    one HIP graph and replayed back to back: what a serving loop that records
    its steps pays, without the per-launch host cost.  The last captured
    step's outputs are checked, bit for bit, against an eager call on the same
    input set."""
    import torch
    cap = torch.cuda.Stream()
    prepared = [make(s, cap) for s in sets]   # launches bound to the capture stream
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):               # one eager pass on the capture stream first
        for p in prepared:
            p[0]()
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for i in range(G):
            prepared[i % len(sets)][0]()
    reps = max(1, -(-steps // G))
    with torch.cuda.stream(stream):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * G)
    last = prepared[(G - 1) % len(sets)]
    replayed = [o.clone() for o in last[1]]
    with torch.cuda.stream(cap):
        last[0]()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(replayed, last[1]))
    if not same:
        raise SystemExit("bench.py: a replayed graph's outputs differ from an eager call's")
    print(f"[bench] graph of {G} steps: {us:.2f} us/step over {reps} replays", file=sys.stderr, flush=True)
    return {"steps_per_graph": G, "replays": reps, "us_per_step": us, "steps_per_s": 1e6 / us,
            "outputs_equal_eager": same}


def main():
    import workloads as W
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: enough for about "
                         "0.3 s, at least 100, so that clocks have settled)")
    ap.add_argument("--workload", default="chain_t1_128k", choices=sorted(W.WORKLOADS))
    ap.add_argument("--rotate", type=int, default=0,
                    help="input sets cycled through (default: enough to exceed 512 MB)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph-steps", type=int, default=20,
                    help="also time this many consecutive steps captured in one HIP graph and "
                         "replayed (0: skip)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run device-to-device copies of this many MB (to scale HBM "
                         "traffic counters against a copy of known size)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verify step runs independently per "
              "sequence batch and this build has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import speculative_decoding_verification_08_amd as sv

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": max(args.steps, 1)}), flush=True)
        return

    w = W.WORKLOADS[args.workload]
    B, V = w.B, w.V
    nbytes = set_bytes(w)
    # Per-sequence trees hold 5/8 of Nmax nodes on average (counts uniform in
    # [Nmax/4, Nmax]).
    est = nbytes * 5 // 8 if w.mode == "tree_dyn" else nbytes
    nsets = args.rotate or max(1, -(-512_000_000 // est))
    if w.mode == "mask":   # 64 KB per step lives in L2 whatever rotates; a few sets suffice
        nsets = args.rotate or 4
    device = torch.device("cuda:0")
    print(f"[bench] generating {nsets} input sets of {w.name}", file=sys.stderr, flush=True)
    host_sets = [W.make_inputs(w, s) for s in range(nsets)]
    if w.mode in ("tree_dyn", "kv"):  # the mean over the rotated sets, each timed equally often
        nbytes = int(round(np.mean([set_bytes(w, h) for h in host_sets])))
    sets = [{k: to_dev(v, device) for k, v in h.items() if isinstance(v, np.ndarray)}
            for h in host_sets]
    stream = torch.cuda.current_stream(device)
    dt_code = sv.SPEC_DTYPE_BF16 if w.dtype == "bf16" else sv.SPEC_DTYPE_F32
    step_launches = None   # per-step launches, where inputs change every step

    if w.mode == "chain":
        K = w.K
        ws = sv.workspace(sv.SPEC_MODE_CHAIN, B, K, V, dt_code, device)
        out_t = torch.empty((B, K + 1), dtype=torch.int32, device=device)
        out_a = torch.empty((B,), dtype=torch.int32, device=device)

        def make(s, st):
            return (sv.prepare_chain(s["target"], s["draft"], s["tokens"], s["u_accept"],
                                     s["u_sample"], w.T, out_t, out_a, ws, stream=st), (out_t, out_a))

        stats_launches = [sv.spec_verify_chain_stats(s["target"], s["draft"], s["tokens"], w.T, ws,
                                                     stream=stream, prepare=True) for s in sets]

        def stats_phase(i):
            stats_launches[i % nsets]()

        def outputs():
            diag = torch.empty((B, K + 1, 4), dtype=torch.float32, device=device)
            s = sets[0]
            tok, acc, _ = sv.spec_verify_chain(s["target"], s["draft"], s["tokens"], s["u_accept"],
                                               s["u_sample"], w.T, out_diag=diag)
            torch.cuda.synchronize()
            return tok.cpu().numpy(), acc.cpu().numpy(), diag.cpu().numpy()
        dominant_name = "k_chain_fused (whole step)"
        io_bytes = 4 * B * K + 4 * B * (K + 1) + 4 * B * (K + 2)
        verified = B * K
        # Fresh uniforms for every timed step: step i draws with the uniforms
        # of workload step i, on logit set i mod nsets (all resident before
        # timing starts).
        nu = max(args.steps, 1)
        uni = [W.chain_uniforms(w, i) for i in range(nu)]
        ua_all = torch.from_numpy(np.stack([u[0] for u in uni])).to(device)
        us_all = torch.from_numpy(np.stack([u[1] for u in uni])).to(device)
        step_launches = [sv.prepare_chain(sets[i % nsets]["target"], sets[i % nsets]["draft"],
                                          sets[i % nsets]["tokens"], ua_all[i], us_all[i], w.T, out_t,
                                          out_a, ws, stream=stream) for i in range(nu)]
    elif w.mode == "greedy":
        K = w.K
        ws = sv.workspace(sv.SPEC_MODE_GREEDY, B, K, V, dt_code, device)
        out_t = torch.empty((B, K + 1), dtype=torch.int32, device=device)
        out_a = torch.empty((B,), dtype=torch.int32, device=device)

        def make(s, st):
            return sv.spec_verify_greedy(s["target"], s["tokens"], out_tokens=out_t, out_accepted=out_a,
                                         workspace_buf=ws, stream=st, prepare=True)
        stats_phase = None

        def outputs():
            tok, acc = sv.spec_verify_greedy(sets[0]["target"], sets[0]["tokens"])
            torch.cuda.synchronize()
            return tok.cpu().numpy(), acc.cpu().numpy()
        dominant_name = "k_greedy (whole step)"
        io_bytes = 4 * B * K + 4 * B * (K + 2)
        verified = B * K
    elif w.mode == "tree_dyn":
        Nmax = w.K
        ws = sv.workspace(sv.SPEC_MODE_TREE_DYN, B, Nmax, V, dt_code, device)
        out_t = torch.empty((B, Nmax), dtype=torch.int32, device=device)
        out_p = torch.empty((B, Nmax), dtype=torch.int32, device=device)
        out_d = torch.empty((B,), dtype=torch.int32, device=device)

        def make(s, st):
            return sv.spec_verify_tree_greedy_dyn(s["node_logits"], s["node_tokens"], s["parents"],
                                                  s["node_count"], out_tokens=out_t, out_path=out_p,
                                                  out_depth=out_d, workspace_buf=ws, stream=st,
                                                  prepare=True)
        stats_phase = None

        def outputs():
            s = sets[0]
            tok, path, depth = sv.spec_verify_tree_greedy_dyn(s["node_logits"], s["node_tokens"],
                                                              s["parents"], s["node_count"])
            torch.cuda.synchronize()
            return tok.cpu().numpy(), path.cpu().numpy(), depth.cpu().numpy()
        dominant_name = "k_tree_dyn (whole step)"
        io_bytes = 4 * B * Nmax * 2 + 4 * B + 4 * B * (2 * Nmax + 1)
        verified = float(np.mean([(h["node_count"] - 1).sum() for h in host_sets]))
    elif w.mode == "kv":
        scratch = to_dev(kv_scratch_host(w), device)
        cache = kv_cache_pattern(w, device)
        new_len = torch.empty((B,), dtype=torch.int32, device=device)
        def make(s, st):
            launch, nl = sv.spec_kv_commit(scratch, cache, s["count"], s["cache_len"], path=s["path"],
                                           new_len=new_len, stream=st, prepare=True)
            return launch, (nl, cache[0, 0])
        stats_phase = None

        def outputs():
            c = kv_cache_pattern(w, device)
            s = sets[0]
            nl = sv.spec_kv_commit(scratch, c, s["count"], s["cache_len"], path=s["path"])
            torch.cuda.synchronize()
            return c[0].cpu().numpy(), nl.cpu().numpy()
        dominant_name = "k_kv_commit (whole step)"
        io_bytes = 4 * B * (w.K + 3)
        verified = 0
    elif w.mode == "mask":
        def make(s, st):
            return sv.spec_tree_mask(s["parents"], s["node_count"], stream=st, prepare=True)
        stats_phase = None

        def outputs():
            m, d = sv.spec_tree_mask(sets[0]["parents"], sets[0]["node_count"])
            torch.cuda.synchronize()
            return m.cpu().numpy().view(np.uint32), d.cpu().numpy()
        dominant_name = "k_tree_mask (whole step)"
        io_bytes = 0
        verified = 0
    elif w.mode == "topk":
        k = w.K
        ws = sv.workspace(sv.SPEC_MODE_TOPK, B, k, V, dt_code, device)
        out_i = torch.empty((B, k), dtype=torch.int32, device=device)
        out_v = torch.empty((B, k), dtype=torch.float32, device=device)

        def make(s, st):
            return sv.spec_draft_topk(s["logits"], k, out_idx=out_i, out_val=out_v, workspace_buf=ws,
                                      stream=st, prepare=True)
        stats_phase = None

        def outputs():
            idx, val = sv.spec_draft_topk(sets[0]["logits"], k)
            torch.cuda.synchronize()
            return idx.cpu().numpy(), val.cpu().numpy()
        dominant_name = "k_topk (whole step)"
        io_bytes = 8 * B * k
        verified = 0
    else:
        par = host_sets[0]["parents"]
        N = len(par)
        D = sv.tree_max_depth(par)
        ws = sv.workspace(sv.SPEC_MODE_TREE, B, N, V, dt_code, device)
        out_t = torch.empty((B, D + 1), dtype=torch.int32, device=device)
        out_p = torch.empty((B, D + 1), dtype=torch.int32, device=device)
        out_d = torch.empty((B,), dtype=torch.int32, device=device)

        def make(s, st):
            return sv.spec_verify_tree_greedy(s["node_logits"], s["node_tokens"], par, out_tokens=out_t,
                                              out_path=out_p, out_depth=out_d, workspace_buf=ws,
                                              stream=st, prepare=True)
        stats_phase = None

        def outputs():
            tok, path, depth = sv.spec_verify_tree_greedy(sets[0]["node_logits"],
                                                          sets[0]["node_tokens"], par)
            torch.cuda.synchronize()
            return tok.cpu().numpy(), path.cpu().numpy(), depth.cpu().numpy()
        dominant_name = "k_tree (whole step)"
        io_bytes = 4 * B * N + 4 * B * (2 * D + 3)
        verified = B * (N - 1)

    launches = step_launches or [make(s, stream)[0] for s in sets]

    def step(i):
        launches[i % len(launches)]()

    done = 0
    if args.warmup is None:
        # The clocks ramp up over about a tenth of a second of load: size the
        # warm-up from a short trial (counted in it; its first steps carry
        # one-time costs, so only the second half is timed) so that the timed
        # steps run settled.
        for done in range(1, 21):
            step(done - 1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for done in range(21, 41):
            step(done - 1)
        torch.cuda.synchronize()
        per = (time.perf_counter() - t0) / 20
        args.warmup = max(100, int(0.3 / max(per, 1e-7)))
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(done, args.warmup):
        step(i)
    torch.cuda.synchronize()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # Every step is reported whole (a chain step is one kernel).  For the
    # chain, the statistics pass alone (the first kernel of the two-phase
    # entry points), back to back on the launch stream, for reference.
    ms_dom = ms_step
    ms_stats = None
    if stats_phase is not None:
        for i in range(args.warmup):
            stats_phase(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            stats_phase(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_stats = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {ms_step * 1e3:.2f} us/step"
          + (f", statistics pass alone {ms_stats * 1e3:.2f} us" if ms_stats else ""),
          file=sys.stderr, flush=True)

    graph = graph_replay(make, sets, stream, args.graph_steps, args.steps) if args.graph_steps else None

    step(0)
    gpu_out = outputs()
    steps_per_s = 1e3 / ms_step
    achieved_step = (nbytes + io_bytes) / (ms_step * 1e-3) / 1e9
    achieved_dom = nbytes / (ms_dom * 1e-3) / 1e9
    is_tree = w.mode in ("tree", "tree_dyn")
    acceptance = None
    if w.mode not in ("topk", "kv", "mask"):
        emitted = (gpu_out[2] + 1).sum() if is_tree else (gpu_out[1] + 1).sum()
        # Acceptance on the timed batch (input set 0): mean accepted drafts per
        # sequence, and for chains the per-token acceptance rate alpha = accepted
        # / tested (a sequence tests positions up to its first rejection).
        acc = gpu_out[2] if is_tree else gpu_out[1]
        acceptance = {"mean_accepted": float(np.mean(acc)), "mean_emitted": float(np.mean(acc) + 1)}
        if not is_tree:
            tested = acc + (acc < w.K)
            alpha = float(acc.sum() / max(int(tested.sum()), 1))
            acceptance["alpha"] = alpha
            # Tokens per step if every position were accepted with probability alpha
            # independently: (1 - alpha^(K+1)) / (1 - alpha).
            acceptance["expected_emitted_at_alpha"] = (
                float((1 - alpha ** (w.K + 1)) / (1 - alpha)) if alpha < 1 else float(w.K + 1))
    config = {"workload": w.name, "mode": w.mode, "B": B, "V": V, "logits": w.dtype,
              "input_sets_rotated": nsets, "logit_bytes_per_step": nbytes}
    if w.mode == "chain":
        config.update(K=w.K, T=w.T, uniforms=f"fresh each timed step ({len(launches)} sets)",
                      arithmetic="fp32 exponentials and ratios, fp64 sums")
    elif w.mode == "greedy":
        config.update(K=w.K)
    elif w.mode == "tree_dyn":
        config.update(Nmax=w.K, mean_nodes=float(np.mean([h["node_count"].mean() for h in host_sets])))
    elif w.mode == "topk":
        config.update(rows=B, k=w.K)
    elif w.mode == "mask":
        config.update(Nmax=w.K, mean_nodes=float(np.mean([h["node_count"].mean() for h in host_sets])))
        for key in ("logit_bytes_per_step", "V", "logits"):
            config.pop(key, None)
        config["bytes_per_step"] = nbytes
    elif w.mode == "kv":
        config.update(planes=w.planes, row_bytes=w.row_bytes, scratch_rows=w.K, cache_slots=w.slots,
                      mean_committed=float(np.mean([h["count"].mean() for h in host_sets])))
        for key in ("logit_bytes_per_step", "V", "logits"):
            config.pop(key, None)
        config["bytes_per_step"] = nbytes
    else:
        config.update(branching=list(w.branching))
    line = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": {"topk": "top-k steps/s", "kv": "KV commit steps/s",
                 "mask": "tree mask steps/s"}.get(w.mode, "verify steps/s"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"kv": "u8", "mask": "int32"}.get(w.mode, w.dtype),
        "data": "synthetic",
        "config": config,
        "achieved_GBps": achieved_step,
        "frac_of_hbm_peak": achieved_step / HBM_PEAK_GBPS,
        "tokens_verified_per_s": steps_per_s * verified,
        "tokens_emitted_per_s": steps_per_s * float(emitted) if acceptance else None,
        "acceptance": acceptance,
        "roofline": {"kernel": dominant_name, "bound": "hbm", "achieved": achieved_dom,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved_dom / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(w.name) if w.mode == "chain" else None,
                     "avg_launch_us": ms_dom * 1e3, "algorithmic_bytes_per_launch": nbytes},
    }
    if ms_stats is not None:
        line["statistics_pass_alone"] = {
            "kernel": "k_chain_stats", "avg_launch_us": ms_stats * 1e3,
            "achieved": nbytes / (ms_stats * 1e-3) / 1e9, "unit": "GB/s",
            "frac": nbytes / (ms_stats * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    if graph is not None:
        line["graph_replay"] = graph
    if not args.no_cpu_baseline:
        print("[bench] oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, host_sets[0], args.cpu_seconds, gpu_out)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
