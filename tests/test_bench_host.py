"""Host-side checks of bench.py (no GPU): the one-GPU contract, the
algorithmic bytes behind every roofline figure, and the rules that tie a
committed traffic measurement to the kernel source it was taken on."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(args, env):
    """The step runs on one GPU: a request for more exits with status 2 and says so."""
    r = _run_bench(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_per_step():
    """Every logit of a step once, from each workload's shape: (B(K+1) + BK) V
    esize for a chain, B(K+1) V esize greedy, B N V esize for a static tree,
    rows V esize for top-k."""
    ws = W.WORKLOADS
    assert bench.set_bytes(ws["chain_t1_128k"]) == (64 * 6 + 64 * 5) * 128256 * 2 == 180_584_448
    assert bench.set_bytes(ws["chain_t07_152k"]) == (256 * 9 + 256 * 8) * 151936 * 4 == 2_644_901_888
    assert bench.set_bytes(ws["chain_t1_small"]) == (8 * 5 + 8 * 4) * 1024 * 4
    assert bench.set_bytes(ws["greedy_32k"]) == 64 * 6 * 32000 * 2 == 24_576_000
    # branching 4, 2, 2, 1: 1 + 4 + 8 + 16 + 16 = 45 nodes
    assert bench.set_bytes(ws["tree_128k"]) == 32 * 45 * 128256 * 2 == 369_377_280
    assert bench.set_bytes(ws["topk_128k"]) == 512 * 128256 * 2 == 131_334_144


def test_algorithmic_bytes_follow_the_inputs():
    """Per-sequence trees read only their trees' rows; the KV commit moves each
    committed row once in and once out of every plane; the mask step reads
    parents and counts and writes mask words and depths."""
    w = W.WORKLOADS["tree_dyn_128k"].with_sizes(B=5, K=12, V=300)
    d = W.tree_dyn_inputs(w, 0)
    assert bench.set_bytes(w, d) == int(d["node_count"].sum()) * 300 * 2
    assert bench.set_bytes(w) == 5 * 12 * 300 * 2
    kv = W.WORKLOADS["kv_commit_b64"]
    count = np.array([1, 3, 8, 0], np.int32)
    assert bench.kv_bytes(kv, count) == 2 * 12 * kv.planes * kv.row_bytes
    m = W.WORKLOADS["tree_mask_b64"]
    B, N = m.B, m.K
    assert bench.set_bytes(m) == 4 * B * N + 4 * B + 4 * B * N * ((N + 31) // 32) + 4 * B * N == 65_792


def test_comment_edits_do_not_change_the_kernel_hash():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* note */ }\n"
    b = "int f(int x) {\n    /* a longer\n       note */ return 2 * x; }"
    c = "int f(int x) { return 3 * x; }"
    assert bench.code_tokens(a) == bench.code_tokens(b)
    assert bench.code_tokens(a) != bench.code_tokens(c)


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(monkeypatch):
    path = os.path.join(ROOT, "profiles", "k_chain_fused_chain_t1_128k_traffic.json")
    t = json.load(open(path))
    assert t["bytes_per_launch"] == t["bytes_fetched_per_launch"] + t["bytes_written_per_launch"]
    assert t["algorithmic_bytes_per_launch"] == 180_584_448
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: t["kernel_source_hash"])
    assert bench.measured_traffic("chain_t1_128k") == t["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic("chain_t1_128k") is None
    assert bench.measured_traffic("greedy_32k") is None
