"""GPU parity at full size and step count, at the edges of temperature and
logit magnitude, and the workspace's hand-over semantics.

Every workload is compared with the fp64 oracle on every sequence:
chain_t1_small on all of its 1,000 steps, greedy_32k on 20 steps and
chain_t07_152k on two steps.  Tolerances are those of oracle.parity (exact
indices; 1e-5 relative on probabilities; the accept and CDF bands).
"""
from collections import Counter

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle                                     # noqa: E402
import workloads as W                             # noqa: E402
from oracle import parity                         # noqa: E402

DEV = "cuda:0"


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_decoding_verification_08_amd as m
    return m


def dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def case(msg):
    print(f"[case] {msg}", flush=True)


def run_chain(sv, d, ws=None):
    """One chain verify with per-position diagnostics, and the same call
    without them (for K >= 2 the position-major order that skips rows after a
    rejection): the two must agree bit for bit."""
    args = (dev(d["target"]), dev(d["draft"]), dev(d["tokens"]), dev(d["u_accept"]),
            dev(d["u_sample"]), d["T"])
    tok, acc, diag = sv.spec_verify_chain(*args, diag=True, workspace_buf=ws)
    tok2, acc2, _ = sv.spec_verify_chain(*args, workspace_buf=ws)
    torch.cuda.synchronize()
    got = tok.cpu().numpy(), acc.cpu().numpy(), diag.cpu().numpy()
    assert np.array_equal(tok2.cpu().numpy(), got[0]) and np.array_equal(acc2.cpu().numpy(), got[1])
    return got


def chain_case(name, B, K, V, dtype, T, recipe="peaked", sigma=0.7, step=0, target_sd=2.0):
    w = W.Workload(name, 94, "chain", B=B, K=K, V=V, dtype=dtype, T=T, recipe=recipe,
                   sigma=sigma, target_sd=target_sd)
    return W.chain_inputs(w, step)


# ------------------------------------------------------------------ full configurations

def test_chain_t1_small_every_step(sv):
    """The small chain workload on each of its 1,000 steps."""
    w = W.WORKLOADS["chain_t1_small"]
    ws = sv.workspace(sv.SPEC_MODE_CHAIN, w.B, w.K, w.V, sv.SPEC_DTYPE_F32, DEV)
    total = Counter()
    for step in range(w.steps):
        if step % 100 == 0:
            case(f"chain_t1_small steps {step}..{step + 99}")
        d = W.chain_inputs(w, step)
        total += parity.check_chain(d, *run_chain(sv, d, ws))
    assert total["sequences"] == w.B * w.steps
    assert sv.workspace_failures(ws) == 0
    print("chain_t1_small", dict(total))


def test_greedy_32k_twenty_steps(sv):
    w = W.WORKLOADS["greedy_32k"]
    for step in range(20):
        case(f"greedy_32k full size step {step}")
        d = W.greedy_inputs(w, step)
        tok, acc = sv.spec_verify_greedy(dev(d["target"]), dev(d["tokens"]))
        torch.cuda.synchronize()
        parity.check_greedy(d, tok.cpu().numpy(), acc.cpu().numpy())


@pytest.mark.timeout(900)
@pytest.mark.parametrize("step", [0, 1])
def test_chain_t07_152k_every_sequence(sv, step):
    """The batched-serving workload (B = 256, K = 8, V = 151936, fp32, T = 0.7):
    every sequence of a step."""
    w = W.WORKLOADS["chain_t07_152k"]
    case(f"chain_t07_152k step {step}: inputs")
    d = W.chain_inputs(w, step)
    case(f"chain_t07_152k step {step}: GPU")
    g = run_chain(sv, d)
    case(f"chain_t07_152k step {step}: oracle on all {w.B} sequences")
    oracle.set_threads(0)
    n = parity.check_chain(d, *g)
    assert n["sequences"] == w.B
    print("chain_t07_152k", step, dict(n), "mean accepted", g[1].mean())


# ------------------------------------------------------------------ edges

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.05, 5.0])
def test_chain_extreme_temperatures(sv, dtype, T):
    """c = log2(e)/T amplifies (T = 0.05) or flattens (T = 5) the exponents."""
    case(f"chain T={T} {dtype}")
    d = chain_case(f"temp{T}", 16, 5, 20011, dtype, T)
    n = parity.check_chain(d, *run_chain(sv, d))
    print("T", T, dtype, dict(n))


@pytest.mark.parametrize("shift", [1e4, -1e4])
def test_chain_logits_shifted_by_large_constants(sv, shift):
    """fp32 logits around +-1e4: softmax is shift-invariant, and every
    exponential of a row is taken against one rounded reference m*c."""
    case(f"chain logits shifted by {shift}")
    d = chain_case("shift", 12, 4, 30001, "f32", 1.0)
    d = dict(d, target=(d["target"] + np.float32(shift)).astype(np.float32),
             draft=(d["draft"] + np.float32(shift)).astype(np.float32))
    n = parity.check_chain(d, *run_chain(sv, d))
    print("shift", shift, dict(n))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_zero_draft_probability(sv, dtype):
    """A drafted token whose draft logit is -inf (q = 0): accepted when the
    target gives it mass, rejected when the target's logit is -inf too."""
    d = chain_case("qzero", 10, 4, 3001, dtype, 1.0)
    tgt = W.as_f32(d["target"]).copy()
    dft = W.as_f32(d["draft"]).copy()
    B, K = d["tokens"].shape
    bi, ki = np.meshgrid(np.arange(B), np.arange(K), indexing="ij")
    dft[bi, ki, d["tokens"]] = -np.inf                     # q(x_k) = 0 at every position
    store = (lambda a: W.bf16_bits(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    d1 = dict(d, target=store(tgt), draft=store(dft))
    case(f"chain q = 0 at every drafted token, {dtype}")
    g = run_chain(sv, d1)
    assert np.all(g[1] == K), g[1]                          # all accepted, then the bonus draw
    assert np.all(np.isinf(g[2][:, :K, 2])) and np.all(g[2][:, :K, 1] == 0)
    parity.check_chain(d1, *g)
    tgt[np.arange(B), 1, d["tokens"][:, 1]] = -np.inf      # p(x_1) = 0 as well
    d2 = dict(d1, target=store(tgt))
    case(f"chain q = p = 0 at position 1, {dtype}")
    g = run_chain(sv, d2)
    assert np.all(g[1] == 1), g[1]
    assert np.all(g[0][:, 1] != d["tokens"][:, 1])
    parity.check_chain(d2, *g)


# ------------------------------------------------------------------ the workspace

def test_sample_without_statistics_reports_failure(sv):
    """The sample phase on a fresh workspace (no statistics phase): every
    sequence reads -1 and the workspace counts one failure per sequence; no
    kernel waits for words that never come."""
    d = chain_case("nostats", 9, 3, 5000, "bf16", 1.0)
    B, K, V = 9, 3, 5000
    ws = sv.workspace(sv.SPEC_MODE_CHAIN, B, K, V, sv.SPEC_DTYPE_BF16, DEV)
    case("chain sample without statistics")
    tok, acc = sv.spec_verify_chain_sample(dev(d["target"]), dev(d["draft"]), dev(d["tokens"]),
                                           dev(d["u_accept"]), dev(d["u_sample"]), 1.0, ws)
    torch.cuda.synchronize()
    assert np.all(acc.cpu().numpy() == -1) and np.all(tok.cpu().numpy() == -1)
    assert sv.workspace_failures(ws, reset=True) == B
    assert sv.workspace_failures(ws) == 0


def test_two_phase_pairs_on_one_workspace(sv):
    """Two statistics + sample pairs with different inputs on one workspace:
    each sample reads its own pair's statistics, and each pair equals the
    one-call verify bit for bit (and the oracle)."""
    B, K, V = 11, 5, 20000
    ws = sv.workspace(sv.SPEC_MODE_CHAIN, B, K, V, sv.SPEC_DTYPE_BF16, DEV)
    for step in range(3):
        d = chain_case("pairs", B, K, V, "bf16", 1.0, step=step)
        case(f"chain stats + sample pair {step}")
        t, dr, x = dev(d["target"]), dev(d["draft"]), dev(d["tokens"])
        diag = torch.empty((B, K + 1, 4), dtype=torch.float32, device=DEV)
        sv.spec_verify_chain_stats(t, dr, x, 1.0, ws)
        tok, acc = sv.spec_verify_chain_sample(t, dr, x, dev(d["u_accept"]), dev(d["u_sample"]), 1.0,
                                               ws, out_diag=diag)
        torch.cuda.synchronize()
        got = (tok.cpu().numpy(), acc.cpu().numpy(), diag.cpu().numpy())
        one = run_chain(sv, d)
        assert all(np.array_equal(a, b) for a, b in zip(got, one))
        parity.check_chain(d, *got)
    assert sv.workspace_failures(ws) == 0


def test_sample_after_stale_statistics_reports_failure(sv):
    """Statistics, then a one-call verify on the same workspace (which leaves
    its own statistics), then the sample phase: the sample finds words of
    another call, and reports every sequence failed instead of drawing from
    them."""
    B, K, V = 7, 4, 9000
    ws = sv.workspace(sv.SPEC_MODE_CHAIN, B, K, V, sv.SPEC_DTYPE_F32, DEV)
    d = chain_case("stale", B, K, V, "f32", 1.0)
    t, dr, x = dev(d["target"]), dev(d["draft"]), dev(d["tokens"])
    ua, us = dev(d["u_accept"]), dev(d["u_sample"])
    case("chain stats, one call, then sample")
    sv.spec_verify_chain_stats(t, dr, x, 1.0, ws)
    sv.spec_verify_chain(t, dr, x, ua, us, 1.0, workspace_buf=ws)
    tok, acc = sv.spec_verify_chain_sample(t, dr, x, ua, us, 1.0, ws)
    torch.cuda.synchronize()
    assert np.all(acc.cpu().numpy() == -1) and np.all(tok.cpu().numpy() == -1)
    assert sv.workspace_failures(ws) == B


# ------------------------------------------------------------------ position-major order

@pytest.mark.parametrize("B,K,V,dtype", [(103, 8, 20000, "f32"), (128, 6, 32768, "bf16"),
                                         (128, 5, 32768, "bf16"), (1024, 64, 2048, "bf16"),
                                         (128, 3, 65536, "f32"), (256, 2, 65536, "bf16")])
def test_chain_position_major_order(sv, B, K, V, dtype):
    """Shapes whose one-call verify runs position by position (one position's
    items fill the chip; rows after a rejection are skipped from position 2,
    or from position 1 when a position's rows are 64 MB or more, as in the
    last two shapes): the tokens equal the sequence-major order's (the call
    with diagnostics) bit for bit, and the oracle's, at low and high
    acceptance."""
    for sigma, step in ((0.7, 0), (2.5, 1)):
        case(f"chain position-major B={B} K={K} V={V} {dtype} sigma={sigma}")
        d = chain_case(f"pm{B}_{K}", B, K, V, dtype, 1.0, sigma=sigma, step=step)
        tok, acc, diag = run_chain(sv, d)
        n = parity.check_chain(d, tok, acc, diag)
        assert n["sequences"] == B
        print("position-major", B, K, V, dtype, sigma, dict(n), "mean accepted", acc.mean())


# ------------------------------------------------------------------ documented size limits

@pytest.mark.parametrize("dtype,B,K", [("bf16", 8, 3), ("f32", 8, 3), ("bf16", 1, 64)])
def test_chain_at_the_vocabulary_limit(sv, dtype, B, K):
    """The largest vocabulary the chain verify takes in each logit type: 128
    statistics chunks and 128 draw chunks per row, so the wavefront that
    gathers a row's chunk masses holds two per lane.  With B = 8 the call
    without diagnostics runs position by position; with K = 64 the longest
    draft, sequence by sequence."""
    V = sv.MAX_CHAIN_V_BF16 if dtype == "bf16" else sv.MAX_CHAIN_V_F32
    for sigma, step in ((0.7, 0), (2.5, 1)):
        case(f"chain at the vocabulary limit B={B} K={K} V={V} {dtype} sigma={sigma}")
        d = chain_case(f"vlimit{K}", B, K, V, dtype, 1.0, sigma=sigma, step=step)
        tok, acc, diag = run_chain(sv, d)
        n = parity.check_chain(d, tok, acc, diag)
        assert n["sequences"] == B


@pytest.mark.parametrize("dtype,K", [("bf16", 2), ("f32", 1)])
def test_greedy_at_the_vocabulary_limit(sv, dtype, K):
    """Greedy verify at the largest vocabulary it takes (2^26 entries per row,
    thousands of argmax chunks per row for the resolve to merge)."""
    case(f"greedy at the vocabulary limit V={sv.MAX_V} {dtype} K={K}")
    w = W.Workload("glimit", 95, "greedy", B=1, K=K, V=sv.MAX_V, dtype=dtype, target_sd=3.0)
    d = W.greedy_inputs(w, 0)
    tok, acc = sv.spec_verify_greedy(dev(d["target"]), dev(d["tokens"]))
    torch.cuda.synchronize()
    n = parity.check_greedy(d, tok.cpu().numpy(), acc.cpu().numpy())
    assert n["sequences"] == 1


def test_tree_at_the_vocabulary_limit(sv):
    """Static-tree greedy verify at the largest vocabulary (four nodes: a root
    with two children, one of which has a child)."""
    case(f"tree at the vocabulary limit V={sv.MAX_V} bf16")
    w = W.Workload("tlimit", 96, "tree", B=1, V=sv.MAX_V, dtype="bf16", recipe="peaked")
    d = W.tree_inputs(w, 0, parents=[-1, 0, 0, 1], p_match=0.9)
    tok, path, depth = sv.spec_verify_tree_greedy(dev(d["node_logits"]), dev(d["node_tokens"]),
                                                  d["parents"])
    torch.cuda.synchronize()
    n = parity.check_tree(d, tok.cpu().numpy(), path.cpu().numpy(), depth.cpu().numpy())
    assert n["sequences"] == 1


@pytest.mark.parametrize("B,K,V,dtype", [(8192, 2, 2048, "bf16"), (70000, 2, 64, "f32")])
def test_chain_position_major_grid_limits(sv, B, K, V, dtype):
    """The position-major order puts the sequence in the grid's y dimension:
    8192 sequences run in it; past 65535 the call without diagnostics falls
    back to the sequence-major order.  Both agree with the call with
    diagnostics bit for bit, and with the oracle."""
    case(f"chain position-major grid limits B={B} K={K} V={V} {dtype}")
    d = chain_case(f"pmlim{B}", B, K, V, dtype, 1.0, sigma=0.7)
    tok, acc, diag = run_chain(sv, d)
    n = parity.check_chain(d, tok, acc, diag)
    assert n["sequences"] == B
