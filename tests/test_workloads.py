"""CPU tests of the seeded input generators and of the statistics each workload implies."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle_pins import expected_tokens


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200_000).astype(np.float32) * 50,
                        np.array([0.0, -0.0, np.inf, -np.inf, 1.00390625, 1.01171875], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.bf16_bits(x), ref)
    assert np.array_equal(W.bf16_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_seeded_and_deterministic():
    w = W.WORKLOADS["chain_t1_small"]
    a, b = W.chain_inputs(w, 3), W.chain_inputs(w, 3)
    for k in ("target", "draft", "tokens", "u_accept", "u_sample"):
        assert np.array_equal(a[k], b[k])
    c = W.chain_inputs(w, 4)
    assert not np.array_equal(a["target"], c["target"])
    assert a["u_accept"].dtype == np.float32 and a["u_accept"].max() < 1 and a["u_accept"].min() >= 0


def test_shapes_of_every_workload_at_small_sizes():
    for name, w in W.WORKLOADS.items():
        small = w.with_sizes(B=2, V=300)
        d = W.make_inputs(small, 0)
        if w.mode == "chain":
            assert d["target"].shape == (2, w.K + 1, 300) and d["draft"].shape == (2, w.K, 300)
            assert d["tokens"].shape == (2, w.K) and d["u_sample"].shape == (2,)
        elif w.mode == "greedy":
            assert d["target"].shape == (2, w.K + 1, 300) and d["tokens"].shape == (2, w.K)
        elif w.mode == "tree":
            assert d["node_logits"].shape == (2, 45, 300) and d["parents"].shape == (45,)
        elif w.mode == "topk":
            assert d["logits"].shape == (2, 300) and d["k"] == w.K
        elif w.mode == "mask":
            assert d["parents"].shape == (2, w.K) and d["node_count"].shape == (2,)
            for b in range(2):
                n = d["node_count"][b]
                assert w.K // 4 <= n <= w.K and d["parents"][b, 0] == -1
                assert all(0 <= d["parents"][b, v] < v for v in range(1, n))
            continue
        elif w.mode == "kv":
            assert d["path"].shape == (2, w.K) and d["count"].shape == (2,)
            assert np.all(d["path"][:, 0] == 0) and np.all((1 <= d["count"]) & (d["count"] <= 8))
            assert np.all(d["cache_len"] + d["count"] <= w.slots)
            for b in range(2):
                c = d["count"][b]
                assert np.all(np.diff(d["path"][b, :c]) > 0) and np.all(d["path"][b, :c] < w.K)
            continue
        else:
            assert d["node_logits"].shape == (2, w.K, 300) and d["parents"].shape == (2, w.K)
            assert d["node_tokens"].shape == (2, w.K) and d["node_count"].shape == (2,)
            for b in range(2):
                n = d["node_count"][b]
                assert w.K // 4 <= n <= w.K and d["parents"][b, 0] == -1
                assert all(0 <= d["parents"][b, v] < v for v in range(1, n))
        arr = d.get("target", d.get("node_logits", d.get("logits")))
        assert arr.dtype == (np.uint16 if w.dtype == "bf16" else np.float32)


def test_tree_parents_breadth_first():
    par = W.tree_parents((4, 2, 2, 1))
    assert len(par) == 45 and par[0] == -1
    assert all(0 <= par[v] < v for v in range(1, 45))
    assert list(par[1:5]) == [0, 0, 0, 0] and list(par[5:7]) == [1, 1]
    assert oracle.tree_max_depth(par) == 4


def test_gumbel_draft_tokens_follow_q():
    """Drafted tokens are draws from softmax(draft / T)."""
    from scipy.stats import chisquare
    w = W.WORKLOADS["chain_t1_small"].with_sizes(B=1, K=1, V=6)
    rng = np.random.default_rng(1)
    row = np.array([0.5, -1.0, 2.0, 0.0, 1.0, -0.25])
    T = 0.7
    rows = np.tile(row.astype(np.float32), (40_000, 1))
    toks = W._gumbel_draw(rows, T, rng)
    q = np.exp(row / T) / np.exp(row / T).sum()
    assert chisquare(np.bincount(toks, minlength=6), q * len(toks)).pvalue > 0.05


def test_greedy_match_rate_and_expected_emitted():
    """greedy_32k: drafts equal the argmax with probability 0.8, so the mean
    emitted count is (1 - 0.8^6)/(1 - 0.8) = 3.689 (closed form of the French
    lesson's "Accélération attendue")."""
    w = W.WORKLOADS["greedy_32k"].with_sizes(B=20_000, V=64)
    d = W.greedy_inputs(w, 0)
    _, acc = oracle.verify_greedy(d["target"], d["tokens"])
    want = expected_tokens(0.8, w.K)
    se = np.std(acc + 1) / np.sqrt(w.B)
    assert abs(float(np.mean(acc + 1)) - want) < 4 * se, (np.mean(acc + 1), want)


def _tree_depth_law(branching, p):
    """P(depth >= L): g(d, l) = 1 - (1 - p g(d+1, l-1))^b_d, g(., 0) = 1."""
    D = len(branching)

    def g(d, l):
        if l == 0:
            return 1.0
        if d >= D:
            return 0.0
        return 1.0 - (1.0 - p * g(d + 1, l - 1)) ** branching[d]
    return [g(0, L) for L in range(1, D + 1)]


def test_tree_expected_depth():
    """tree_128k: each child matches with probability 0.6 independently; the
    expected accepted depth is the sum of P(depth >= L) = 3.645."""
    law = _tree_depth_law((4, 2, 2, 1), 0.6)
    assert abs(law[0] - 0.9744) < 1e-12 and abs(sum(law) - 3.6452) < 1e-3
    w = W.WORKLOADS["tree_128k"].with_sizes(B=3000, V=48)
    d = W.tree_inputs(w, 0)
    _, _, depth = oracle.verify_tree_greedy(d["node_logits"], d["node_tokens"], d["parents"])
    se = np.std(depth) / np.sqrt(w.B)
    assert abs(float(depth.mean()) - sum(law)) < 4 * se, (depth.mean(), sum(law))
    for L in range(1, 5):
        assert abs(float((depth >= L).mean()) - law[L - 1]) < 0.03


def test_chain_small_mean_emitted_matches_closed_form():
    """chain_t1_small over its 1,000 steps: mean emitted tokens equals the
    closed form at the measured mean acceptance rate sum_i min(p_i, q_i)."""
    w = W.WORKLOADS["chain_t1_small"]
    em, alphas = [], []
    for step in range(w.steps):
        d = W.chain_inputs(w, step)
        _, acc, _ = oracle.verify_chain(d["target"], d["draft"], d["tokens"], d["u_accept"],
                                        d["u_sample"], w.T)
        em.append(acc + 1)
        if step % 10 == 0:
            alphas += [oracle.acceptance_rate(d["target"][b, k], d["draft"][b, k], w.T)
                       for b in range(w.B) for k in range(w.K)]
    em = np.concatenate(em)
    alpha = float(np.mean(alphas))
    want = expected_tokens(alpha, w.K)
    se = np.std(em) / np.sqrt(len(em))
    assert 0.78 < alpha < 0.84
    assert abs(em.mean() - want) < 4 * se + 0.01, (em.mean(), want, alpha)


@pytest.mark.slow
def test_chain_128k_acceptance_is_calibrated():
    """chain_t1_128k: sigma is chosen so that the mean acceptance rate is 0.75."""
    w = W.WORKLOADS["chain_t1_128k"]
    d = W.chain_inputs(w, 1)
    a = [oracle.acceptance_rate(d["target"][b, k], d["draft"][b, k], w.T)
         for b in range(w.B) for k in range(w.K)]
    assert abs(np.mean(a) - 0.75) < 0.01, np.mean(a)
