"""Pins of the CPU oracle against facts the pages and mathematics fix.

Each pin takes a loaded oracle library so that the mutation test can run the
same pins on copies of the oracle with a planted mistake and show that they
fail.  No pin reuses the oracle's code: expected values come from exact
enumeration of the output law, closed forms printed on the pages, numpy's
argmax, brute-force tree paths, and hand-derived fixtures under tests/golden/.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
from workloads import bf16_bits, bf16_to_f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def np_softmax(logits, T):
    """Textbook softmax(l / T) in float64 with numpy (the definition of p and q)."""
    l = np.asarray(logits, np.float64)
    m = np.max(l[np.isfinite(l)])
    e = np.exp((l - m) / T)
    return e / e.sum()


def widen(a):
    return bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


# ------------------------------------------------------------- exact law

def _boundaries(pred, n, iters=64):
    """Per-lane boundary of a predicate that is True for u < boundary, on [0, 1)."""
    lo, hi = np.zeros(n), np.ones(n)
    at_zero = np.asarray(pred(lo.copy()), bool)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        r = np.asarray(pred(mid), bool)
        lo, hi = np.where(r, mid, lo), np.where(r, hi, mid)
    return np.where(at_zero, hi, 0.0)


def exact_law(lib, target, draft, T):
    """Law of the emitted tokens of one sequence, found by bisecting the
    oracle's decisions over the uniforms (double-precision entry point).

    Returns (out, reach): out[k][y] = P(position k is emitted and equals y),
    reach[k] = P(position k is emitted).  The drafted token at position k is
    weighted by q_k (numpy softmax of draft row k), as a draft sampler would.
    """
    K1, V = target.shape
    K = K1 - 1
    q = [np_softmax(widen(draft[k]), T) for k in range(K)]

    def call(tok_rows, ua_rows, us):
        n = len(tok_rows)
        t, a, _ = oracle.verify_chain(
            np.repeat(target[None], n, 0), np.repeat(draft[None], n, 0),
            np.asarray(tok_rows, np.int32).reshape(n, K),
            np.asarray(ua_rows, np.float64).reshape(n, K),
            np.asarray(us, np.float64).reshape(n), T, lib=lib)
        return t, a

    def partition(toks, ua, pos):
        """Measure of u_s leading to each token at position pos (monotone inverse CDF)."""
        if V == 1:
            return np.ones(1)

        def pred(u):
            t, a = call([toks] * (V - 1), [ua] * (V - 1), u)
            assert np.all(a == pos)
            return t[:, pos] < np.arange(1, V)
        b = np.concatenate([[0.0], _boundaries(pred, V - 1), [1.0]])
        return np.diff(b)

    out = np.zeros((K + 1, V))
    reach = np.zeros(K + 1)
    prefixes = [((), 1.0)]
    for k in range(K + 1):
        nxt = []
        for pre, mass in prefixes:
            reach[k] += mass
            pad = [0] * (K - k - 1)
            if k == K:
                out[K] += mass * partition(list(pre), [0.0] * K, K)
                continue
            xs = [x for x in range(V) if q[k][x] > 0]

            def acc(u, pre=pre, xs=xs, pad=pad):
                rows = [list(pre) + [x] + pad for x in xs]
                ua = [[0.0] * k + [u[i]] + [0.0] * len(pad) for i in range(len(xs))]
                _, a = call(rows, ua, [0.5] * len(xs))
                return a > k
            thr = _boundaries(acc, len(xs))
            for i, x in enumerate(xs):
                a = thr[i]
                if a > 0:
                    nxt.append((pre + (x,), mass * q[k][x] * a))
                    out[k][x] += mass * q[k][x] * a
                if a < 1:
                    ua = [0.0] * k + [0.5 * (1.0 + a)] + [0.0] * len(pad)
                    out[k] += mass * q[k][x] * (1.0 - a) * partition(list(pre) + [x] + pad, ua, k)
        prefixes = nxt
    return out, reach


def _law_case(rng, V, K, T, dtype, zeros):
    """Random target/draft distributions p, q (with some zero entries) as logits T ln p."""
    def dist():
        d = rng.dirichlet(np.ones(V))
        if zeros and V > 2:
            d[rng.integers(0, V)] = 0.0
        return d / d.sum()
    p = [dist() for _ in range(K + 1)]
    q = [dist() for _ in range(K)]
    with np.errstate(divide="ignore"):
        tl = np.array([T * np.log(x) for x in p], np.float32)
        dl = np.array([T * np.log(x) for x in q], np.float32)
    if dtype == "bf16":
        tl, dl = bf16_bits(tl), bf16_bits(dl)
    return tl, dl, p


LAW_CASES = [  # (V, K, T, dtype, zero entries)
    (2, 1, 1.0, "f32", False),
    (3, 2, 1.0, "f32", True),
    (5, 1, 0.7, "f32", True),
    (8, 1, 1.0, "bf16", True),
    (8, 2, 1.3, "f32", False),
    (4, 2, 0.7, "bf16", True),
]


def pin_exact_law(lib, cases=LAW_CASES, seed=5):
    """The output law equals the target's: at every emitted position k the
    token is distributed as p_k, and position k+1 is reached with probability
    sum_i min(p_k,i, q_k,i) (forum post §3, the proof that the output law is p;
    French lesson, "La règle de l'exactitude")."""
    rng = np.random.default_rng(seed)
    for V, K, T, dtype, zeros in cases:
        tl, dl, p_chosen = _law_case(rng, V, K, T, dtype, zeros)
        out, reach = exact_law(lib, tl, dl, T)
        assert abs(reach[0] - 1.0) < 1e-12
        assert abs(out[0].sum() - 1.0) < 1e-12, f"mass {out[0].sum()}"
        for k in range(K + 1):
            p = np_softmax(widen(tl[k]), T)
            got = out[k] / reach[k]
            assert np.max(np.abs(got - p)) < 1e-12, (V, K, T, dtype, k, got, p)
            if dtype == "f32":  # logits T ln p rounded to fp32 only
                assert np.max(np.abs(got - p_chosen[k])) < 1e-6
            if k < K:
                qk = np_softmax(widen(dl[k]), T)
                alpha = np.minimum(p, qk).sum()
                assert abs(reach[k + 1] - reach[k] * alpha) < 1e-12, (k, reach, alpha)


# ------------------------------------------------------------- expected tokens

def expected_tokens(alpha, K):
    """Expected tokens per target pass (French lesson, "Accélération attendue";
    forum post §4): (1 - alpha^(K+1)) / (1 - alpha)."""
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


def pin_expected_tokens(lib, B=100_000, seed=7):
    """Monte Carlo on constant-alpha pairs (V = 2): mean emitted tokens within
    1% of the closed form; the French lesson prints 3.36 at alpha=0.8, K=4."""
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    printed = {(f["alpha"], f["K"]): f["printed"] for f in facts["expected_tokens"]}
    assert round(expected_tokens(0.8, 4), 2) == printed[(0.8, 4)]
    rng = np.random.default_rng(seed)
    for p, q, K in [((0.6, 0.4), (0.4, 0.6), 4), ((0.75, 0.25), (0.5, 0.5), 5)]:
        alpha = float(np.minimum(p, q).sum())
        tl = np.tile(np.log(np.array(p, np.float32)), (B, K + 1, 1)).astype(np.float32)
        dl = np.tile(np.log(np.array(q, np.float32)), (B, K, 1)).astype(np.float32)
        tokens = (rng.random((B, K)) >= q[0]).astype(np.int32)     # token 1 w.p. q[1]
        ua = rng.random((B, K), dtype=np.float32)
        us = rng.random((B,), dtype=np.float32)
        _, acc, _ = oracle.verify_chain(tl, dl, tokens, ua, us, 1.0, lib=lib)
        mean = float((acc + 1).mean())
        want = expected_tokens(alpha, K)
        assert abs(mean - want) / want < 0.01, (p, q, K, mean, want)


# ------------------------------------------------------------- page facts

def pin_page_counts(lib):
    """K+1 tokens when every draft is accepted, one when the first is rejected
    (French lesson, "Le concept"); five accepted drafts plus the bonus give six
    tokens (Arabic lesson, end of step 3)."""
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    rng = np.random.default_rng(3)
    for f in facts["emitted_counts"]:
        K, V, B = f["K"], 16, 64
        tl = rng.standard_normal((B, K + 1, V)).astype(np.float32)
        if f["case"] == "all_accepted":      # draft == target: ratio 1 > u
            dl = tl[:, :K].copy()
            tokens = rng.integers(0, V, (B, K)).astype(np.int32)
        else:                                # first drafted token has p = 0
            dl = rng.standard_normal((B, K, V)).astype(np.float32)
            tokens = rng.integers(0, V, (B, K)).astype(np.int32)
            tl[np.arange(B), 0, tokens[:, 0]] = -np.inf
        ua = rng.random((B, K), dtype=np.float32)
        us = rng.random((B,), dtype=np.float32)
        out, acc, _ = oracle.verify_chain(tl, dl, tokens, ua, us, 1.0, lib=lib)
        emitted = (out >= 0).sum(axis=1)
        assert np.all(emitted == f["tokens"]), (f, emitted)
        assert np.all(emitted == acc + 1)


def pin_strict_acceptance(lib):
    """Both lessons' code accepts on a strict comparison of the uniform with
    p(x)/q(x) (French lesson, "La règle de l'exactitude"; Arabic lesson,
    step 1), so u equal to the ratio rejects, and a token the target gives zero
    mass is rejected even at u = 0 (it can never be emitted, since the output
    law is p)."""
    V = 4
    tl = np.zeros((1, 2, V), np.float32)                      # p = 1/4 each
    dl = np.array([[[0.0, 0.0, -np.inf, -np.inf]]], np.float32)   # q = (1/2, 1/2, 0, 0)
    for u, accepted in [(0.5, 0), (np.nextafter(np.float32(0.5), np.float32(0)), 1), (0.0, 1)]:
        _, acc, d = oracle.verify_chain(tl, dl, [[1]], np.array([[u]], np.float32),
                                        np.array([0.5], np.float32), 1.0, diag=True, lib=lib)
        assert d[0, 0, 2] == 0.5 and acc[0] == accepted, (u, acc, d[0, 0])
    tl[0, 0, 1] = -np.inf                                     # p(1) = 0
    out, acc, _ = oracle.verify_chain(tl, dl, [[1]], np.array([[0.0]], np.float32),
                                      np.array([0.0], np.float32), 1.0, lib=lib)
    assert acc[0] == 0 and out[0, 0] != 1


def pin_zero_draft_probability(lib):
    """A drafted token the draft gives zero probability (Arabic lesson "Speculative
    decoding: draft, verify, repeat", "Build it" step 1: a zero draft probability
    makes the ratio infinite, so the token is accepted whatever u is) -- unless the
    target gives it zero probability too, when it is rejected: a token the target
    cannot emit never is (the output law is p).  Reachable through -inf draft
    logits.  The replacement after such a rejection never is the drafted token."""
    V, B = 5, 6
    ninf = np.float32(-np.inf)
    rng = np.random.default_rng(37)
    tl = rng.standard_normal((B, 2, V)).astype(np.float32)
    dl = rng.standard_normal((B, 1, V)).astype(np.float32)
    tokens = np.full((B, 1), 2, np.int32)
    dl[:, 0, 2] = ninf                                     # q(x) = 0
    ua = np.array([[0.0], [0.5], [0.99999994], [0.25], [0.75], [0.9]], np.float32)
    us = rng.random((B,), dtype=np.float32)
    out, acc, d = oracle.verify_chain(tl, dl, tokens, ua, us, 1.0, diag=True, lib=lib)
    assert np.all(acc == 1) and np.all(out[:, 0] == 2), (acc, out)
    assert np.all(d[:, 0, 1] == 0.0) and np.all(d[:, 0, 0] > 0.0) and np.all(np.isinf(d[:, 0, 2]))
    tl[:, 0, 2] = ninf                                     # p(x) = 0 as well
    out, acc, d = oracle.verify_chain(tl, dl, tokens, ua, us, 1.0, diag=True, lib=lib)
    assert np.all(acc == 0) and np.all(out[:, 0] != 2) and np.all(out[:, 0] >= 0), (acc, out)
    assert np.all(d[:, 0, :3] == 0.0)


# ------------------------------------------------------------- softmax values

def pin_softmax_values(lib):
    """A constant row gives p = 1/V exactly; a two-level row has the closed
    form 1 / (n_a + n_b exp((b - a) / T))."""
    B, K, V = 1, 1, 7
    tl = np.full((B, K + 1, V), 0.375, np.float32)
    dl = np.full((B, K, V), -1.25, np.float32)
    _, _, d = oracle.verify_chain(tl, dl, [[3]], np.array([[0.5]], np.float32),
                                  np.array([0.5], np.float32), 0.8, diag=True, lib=lib)
    assert d[0, 0, 0] == 1.0 / V and d[0, 0, 1] == 1.0 / V and d[0, 0, 2] == 1.0
    for T in (1.0, 0.7, 2.5):
        a, b, na, nb = 1.5, -0.5, 3, 9
        row = np.array([a] * na + [b] * nb, np.float32)
        tl = np.stack([row, row])[None]
        dl = np.full((1, 1, na + nb), 0.0, np.float32)
        _, _, d = oracle.verify_chain(tl, dl, [[1]], np.array([[0.0]], np.float32),
                                      np.array([0.0], np.float32), T, diag=True, lib=lib)
        want = 1.0 / (na + nb * np.exp((b - a) / T))
        assert abs(d[0, 0, 0] - want) <= 1e-14 * want, (T, d[0, 0, 0], want)
        assert abs(d[0, 0, 1] - 1.0 / (na + nb)) <= 1e-15


def pin_row_helpers(lib):
    """The single-row helpers: softmax_row is p = softmax(l / T) (constant row ->
    1/V exactly; two-level row -> closed form; -inf entries -> 0) and row_argmax is
    numpy's argmax over the widened values (first index among ties, -0.0 ties +0.0)."""
    for T in (1.0, 0.7, 2.5):
        p = oracle.softmax_row(np.full(9, -0.625, np.float32), T, lib=lib)
        assert np.all(p == 1.0 / 9)
        a, b, na, nb = 1.5, -0.5, 3, 9
        row = np.array([a] * na + [b] * nb + [-np.inf], np.float32)
        p = oracle.softmax_row(row, T, lib=lib)
        pa = 1.0 / (na + nb * np.exp((b - a) / T))
        assert np.all(np.abs(p[:na] - pa) <= 1e-15 * pa) and p[-1] == 0.0
        assert np.all(np.abs(p[na:na + nb] - pa * np.exp((b - a) / T)) <= 1e-15)
        pb = oracle.softmax_row(bf16_bits(row), T, lib=lib)          # bf16 widened exactly
        assert np.array_equal(pb, p)
    rng = np.random.default_rng(47)
    for dtype in ("f32", "bf16"):
        for _ in range(20):
            v = rng.integers(-3, 4, 50).astype(np.float32)          # many ties
            v[rng.random(50) < 0.1] = -0.0
            r = bf16_bits(v) if dtype == "bf16" else v
            assert oracle.row_argmax(r, lib=lib) == int(np.argmax(widen(r)))
    assert oracle.row_argmax(np.array([-0.0, 0.0, -1.0], np.float32), lib=lib) == 0


def pin_helper_closed_forms(lib):
    """The two oracle helpers the tests lean on, against closed forms.

    acceptance_rate is sum_i min(p_i, q_i), the probability that a drafted
    token is accepted (forum post, section 3): 1 for identical rows, 0 for
    disjoint supports, and 0.8 for p = (0.6, 0.4), q = (0.4, 0.6).
    draw_weights is max(0, p - q) after a rejection and p for the bonus draw
    (French lesson, "La règle de l'exactitude"): checked entry by entry on a
    two-level target row against a constant draft row (q = 1/V)."""
    row = np.array([0.3, -1.2, 2.0, 0.0, 0.7], np.float32)
    assert abs(oracle.acceptance_rate(row, row, 0.9, lib=lib) - 1.0) <= 1e-15
    ninf = np.float32(-np.inf)
    assert oracle.acceptance_rate(np.array([0.0, ninf], np.float32),
                                  np.array([ninf, 0.0], np.float32), 1.0, lib=lib) == 0.0
    for T in (1.0, 0.5):
        t = (T * np.log(np.array([0.6, 0.4]))).astype(np.float32)
        d = (T * np.log(np.array([0.4, 0.6]))).astype(np.float32)
        assert abs(oracle.acceptance_rate(t, d, T, lib=lib) - 0.8) <= 1e-6, T
    for T in (1.0, 0.7):
        a, b, na, nb = 1.5, -0.5, 3, 9
        V = na + nb
        t = np.array([a] * na + [b] * nb, np.float32)
        d = np.zeros(V, np.float32)
        pa = 1.0 / (na + nb * np.exp((b - a) / T))
        p = np.array([pa] * na + [pa * np.exp((b - a) / T)] * nb)
        w, S = oracle.draw_weights(t, d, T, lib=lib)
        want = np.maximum(p - 1.0 / V, 0.0)
        assert np.all(np.abs(w - want) <= 1e-14), (T, w, want)
        assert abs(S - want.sum()) <= 1e-14 and want[na:].sum() == 0.0
        w, S = oracle.draw_weights(t, None, T, lib=lib)
        assert np.all(np.abs(w - p) <= 1e-15) and abs(S - 1.0) <= 1e-14


# ------------------------------------------------------------- inverse CDF

def pin_inverse_cdf(lib):
    """Sampling is the inverse CDF with a strict comparison: with power-of-two
    masses u*S lands exactly on a running sum and the next token is taken; a
    zero-mass token is never drawn; an all-zero residual falls back to p."""
    V, K = 4, 1
    tl = np.zeros((1, K + 1, V), np.float32)       # bonus row uniform: C = .25 .5 .75 1
    dl = tl[:, :K].copy()
    for us, want in [(0.0, 0), (0.24999999, 0), (0.25, 1), (0.5, 2), (0.75, 3), (0.99999994, 3)]:
        out, acc, _ = oracle.verify_chain(tl, dl, [[2]], np.array([[0.5]], np.float32),
                                          np.array([us], np.float32), 1.0, lib=lib)
        assert acc[0] == 1 and out[0, 1] == want, (us, out)
    tl[0, 1] = [0.0, -np.inf, 0.0, -np.inf]       # p = (.5, 0, .5, 0)
    for us, want in [(0.0, 0), (0.5, 2), (0.99999994, 2)]:
        out, acc, _ = oracle.verify_chain(tl, dl, [[2]], np.array([[0.5]], np.float32),
                                          np.array([us], np.float32), 1.0, lib=lib)
        assert out[0, 1] == want, (us, out)
    p = np.array([0.25, 0.25, 0.5])
    tok, S = oracle.residual_draw(p, p, 0.3, lib=lib)
    assert tok == 1 and S == 1.0
    tok, S = oracle.residual_draw(p, np.array([0.5, 0.25, 0.25]), 0.5, lib=lib)
    assert tok == 2 and S == 0.25                  # residual (0, 0, .25)


# ------------------------------------------------------------- greedy

def _greedy_expect(vals, tokens):
    amax = np.argmax(vals, axis=-1)                # numpy: first maximum
    B, K = tokens.shape
    out = np.full((B, K + 1), -1, np.int64)
    acc = np.zeros(B, np.int64)
    for b in range(B):
        j = next((k for k in range(K) if tokens[b, k] != amax[b, k]), K)
        acc[b] = j
        out[b, :j + 1] = amax[b, :j + 1]
    return out, acc, amax


def pin_greedy(lib, seed=11):
    """Greedy chain (French lesson, "La règle de l'exactitude", greedy case)
    equals argmax decoding up to the first mismatch, with numpy's argmax
    (lowest index on ties; -0.0 ties +0.0)."""
    rng = np.random.default_rng(seed)
    for dtype in ("f32", "bf16"):
        B, K, V = 400, 4, 37
        vals = (rng.integers(-3, 4, size=(B, K + 1, V)) * 0.5).astype(np.float32)
        vals[rng.random(vals.shape) < 0.05] = -np.inf
        neg0 = (vals == 0) & (rng.random(vals.shape) < 0.5)
        vals[neg0] = -0.0
        logits = bf16_bits(vals) if dtype == "bf16" else vals
        amax = np.argmax(widen(logits), axis=-1)
        tokens = np.where(rng.random((B, K)) < 0.7, amax[:, :K],
                          rng.integers(0, V, (B, K))).astype(np.int32)
        out, acc = oracle.verify_greedy(logits, tokens, lib=lib)
        e_out, e_acc, _ = _greedy_expect(widen(logits), tokens)
        assert np.array_equal(acc, e_acc) and np.array_equal(out, e_out), dtype
        # all drafts equal to the argmax: plain greedy decoding of K+1 tokens
        out, acc = oracle.verify_greedy(logits, amax[:, :K].astype(np.int32), lib=lib)
        assert np.all(acc == K) and np.array_equal(out, amax)
    zero_rows = np.array([[[-0.0, 0.0, -1.0], [0.0, -0.0, -0.0]]], np.float32)
    out, acc = oracle.verify_greedy(zero_rows, [[0]], lib=lib)
    assert acc[0] == 1 and list(out[0]) == [0, 0]


# ------------------------------------------------------------- tree

def tree_bruteforce(vals, tokens, parents):
    """Deepest root path whose every node matches its parent's argmax; lowest
    node index among equally deep ones.  Enumerates every root path."""
    N = len(parents)
    amax = np.argmax(vals, axis=-1)
    best, best_path = 0, [0]
    for v in range(N):
        path = [v]
        while path[-1] != 0:
            path.append(parents[path[-1]])
        path = path[::-1]
        if all(tokens[c] == amax[u] for u, c in zip(path[:-1], path[1:])):
            if len(path) > len(best_path):
                best, best_path = v, path
    return best_path, [int(tokens[c]) for c in best_path[1:]] + [int(amax[best])]


def pin_tree_bruteforce(lib, seed=13):
    rng = np.random.default_rng(seed)
    for trial in range(80):
        N = int(rng.integers(1, 24))
        parents = [-1] + [int(rng.integers(0, v)) for v in range(1, N)]
        B, V = 4, 6
        dtype = "bf16" if trial % 2 else "f32"
        vals = (rng.integers(-2, 3, size=(B, N, V)) * 0.5).astype(np.float32)
        logits = bf16_bits(vals) if dtype == "bf16" else vals
        amax = np.argmax(widen(logits), axis=-1)
        tokens = np.zeros((B, N), np.int32)
        for b in range(B):
            for v in range(1, N):
                tokens[b, v] = amax[b, parents[v]] if rng.random() < 0.7 else rng.integers(0, V)
        out_t, out_p, out_d = oracle.verify_tree_greedy(logits, tokens, parents, lib=lib)
        for b in range(B):
            path, toks = tree_bruteforce(widen(logits[b]), tokens[b], parents)
            d = len(path) - 1
            assert out_d[b] == d, (trial, b, out_d[b], path)
            assert list(out_p[b, :d + 1]) == path and np.all(out_p[b, d + 1:] == -1)
            assert list(out_t[b, :d + 1]) == toks and np.all(out_t[b, d + 1:] == -1)


def pin_tree_chain(lib, seed=17):
    """A tree with branching 1,1,...,1 is a chain: its greedy tree verify
    equals the greedy chain verify."""
    rng = np.random.default_rng(seed)
    B, K, V = 200, 4, 29
    vals = (rng.integers(-3, 4, size=(B, K + 1, V)) * 0.5).astype(np.float32)
    amax = np.argmax(vals, axis=-1)
    x = np.where(rng.random((B, K)) < 0.75, amax[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    parents = [-1] + list(range(K))
    node_tokens = np.concatenate([np.zeros((B, 1), np.int32), x], axis=1)
    t_t, _, t_d = oracle.verify_tree_greedy(vals, node_tokens, parents, lib=lib)
    g_t, g_a = oracle.verify_greedy(vals, x, lib=lib)
    assert np.array_equal(t_d, g_a) and np.array_equal(t_t, g_t)


def pin_tree_figure(lib):
    """Hand-derived cases on the French lesson's root/a/b/c/d/e/f tree."""
    fx = json.load(open(os.path.join(GOLDEN, "tree_p1_figure.json")))
    parents = fx["parents"]
    for case in fx["cases"]:
        rows = np.array(case["rows"], np.float32)[None]
        toks = np.array(case["tokens"], np.int32)[None]
        out_t, out_p, out_d = oracle.verify_tree_greedy(rows, toks, parents, lib=lib)
        d = case["depth"]
        assert out_d[0] == d, case["name"]
        assert list(out_p[0, :d + 1]) == case["path"], case["name"]
        assert list(out_t[0, :d + 1]) == case["emitted"], case["name"]


def _dyn_case(rng, B, Nmax, V, dtype, p_match=0.7):
    """Per-sequence random trees (parents[b][v] uniform below v), ragged node
    counts, small-integer logits (ties likely), padding rows and tokens filled
    with noise that must not be read."""
    counts = rng.integers(1, Nmax + 1, size=B).astype(np.int32)
    parents = np.full((B, Nmax), 7, np.int32)
    for b in range(B):
        parents[b, 0] = -1
        for v in range(1, counts[b]):
            parents[b, v] = rng.integers(0, v)
    vals = (rng.integers(-2, 3, size=(B, Nmax, V)) * 0.5).astype(np.float32)
    logits = bf16_bits(vals) if dtype == "bf16" else vals
    amax = np.argmax(widen(logits), axis=-1)
    tokens = rng.integers(0, V, size=(B, Nmax)).astype(np.int32)
    for b in range(B):
        for v in range(1, counts[b]):
            if rng.random() < p_match:
                tokens[b, v] = amax[b, parents[b, v]]
    return logits, tokens, parents, counts


def pin_tree_dyn_bruteforce(lib, seed=23):
    """Per-sequence trees against the brute-force path enumeration of each
    sequence's own tree; outputs padded with -1 to Nmax."""
    rng = np.random.default_rng(seed)
    for trial in range(60):
        Nmax, B, V = int(rng.integers(1, 20)), 5, 6
        dtype = "bf16" if trial % 2 else "f32"
        logits, tokens, parents, counts = _dyn_case(rng, B, Nmax, V, dtype)
        out_t, out_p, out_d = oracle.verify_tree_greedy_dyn(logits, tokens, parents, counts, lib=lib)
        for b in range(B):
            n = counts[b]
            path, toks = tree_bruteforce(widen(logits[b, :n]), tokens[b, :n], list(parents[b, :n]))
            d = len(path) - 1
            assert out_d[b] == d, (trial, b, out_d[b], path)
            assert list(out_p[b, :d + 1]) == path and np.all(out_p[b, d + 1:] == -1)
            assert list(out_t[b, :d + 1]) == toks and np.all(out_t[b, d + 1:] == -1)


def pin_tree_dyn_padding(lib, seed=29):
    """Rows, tokens and parents past a sequence's node count are never read:
    rewriting them leaves every output unchanged."""
    rng = np.random.default_rng(seed)
    for trial in range(20):
        Nmax, B, V = 12, 6, 5
        logits, tokens, parents, counts = _dyn_case(rng, B, Nmax, V, "f32")
        ref = oracle.verify_tree_greedy_dyn(logits, tokens, parents, counts, lib=lib)
        l2, t2, p2 = logits.copy(), tokens.copy(), parents.copy()
        for b in range(B):
            n = counts[b]
            l2[b, n:] = rng.integers(-9, 9, size=l2[b, n:].shape)
            t2[b, n:] = rng.integers(0, V, size=Nmax - n)
            p2[b, n:] = rng.integers(-5, 50, size=Nmax - n)
        out = oracle.verify_tree_greedy_dyn(l2, t2, p2, counts, lib=lib)
        assert all(np.array_equal(x, y) for x, y in zip(ref, out)), trial


def pin_tree_dyn_chain(lib, seed=31):
    """A per-sequence chain of n nodes (parents v - 1) is the greedy chain with
    K = n - 1 drafts over that sequence's first n rows."""
    rng = np.random.default_rng(seed)
    Nmax, V = 7, 11
    for trial in range(40):
        n = int(rng.integers(1, Nmax + 1))
        vals = (rng.integers(-3, 4, size=(1, Nmax, V)) * 0.5).astype(np.float32)
        amax = np.argmax(vals, axis=-1)
        x = np.where(rng.random(n - 1) < 0.75, amax[0, :n - 1], rng.integers(0, V, n - 1)).astype(np.int32)
        parents = np.full((1, Nmax), 0, np.int32)
        parents[0, :n] = [-1] + list(range(n - 1))
        tokens = np.zeros((1, Nmax), np.int32)
        tokens[0, 1:n] = x
        t_t, _, t_d = oracle.verify_tree_greedy_dyn(vals, tokens, parents, np.array([n], np.int32), lib=lib)
        g_t, g_a = oracle.verify_greedy(vals[:, :n], x[None], lib=lib)
        assert t_d[0] == g_a[0] and np.array_equal(t_t[0, :n], g_t[0]) and np.all(t_t[0, n:] == -1)


# ------------------------------------------------------------- top-k

def pin_topk_sort(lib, seed=41):
    """Against a stable sort by (value descending, index ascending) of the
    widened values (numpy's lexsort), on rows full of ties, with -0.0 and
    +0.0 mixed and -inf entries."""
    rng = np.random.default_rng(seed)
    for trial in range(60):
        V = int(rng.integers(1, 40))
        k = int(rng.integers(1, min(8, V) + 1))
        vals = (rng.integers(-3, 4, size=(7, V)) * 0.5).astype(np.float32)
        vals[rng.random((7, V)) < 0.2] = -0.0
        vals[rng.random((7, V)) < 0.1] = -np.inf
        dtype = "bf16" if trial % 2 else "f32"
        logits = bf16_bits(vals) if dtype == "bf16" else vals
        w = widen(logits)
        idx, val = oracle.topk(logits, k, lib=lib)
        for r in range(w.shape[0]):
            order = np.lexsort((np.arange(V), -w[r].astype(np.float64)))[:k]
            assert list(idx[r]) == list(order), (trial, r, list(idx[r]), list(order))
            assert np.array_equal(val[r], w[r][order])


def pin_topk_argmax(lib, seed=43):
    """k = 1 is the row argmax; the values come back in descending order."""
    rng = np.random.default_rng(seed)
    vals = rng.standard_normal((50, 300)).astype(np.float32)
    idx, val = oracle.topk(vals, 1, lib=lib)
    assert np.array_equal(idx[:, 0], np.argmax(vals, axis=1))
    idx8, val8 = oracle.topk(vals, 8, lib=lib)
    assert np.all(np.diff(val8, axis=1) <= 0) and np.array_equal(idx8[:, 0], idx[:, 0])


# ------------------------------------------------------------- KV commit

def _kv_of(tokens, planes, row, salt=0):
    """Synthetic key/value rows: a fixed byte pattern per (plane, token), so a
    cache's contents can be predicted from the token sequence alone."""
    t = np.asarray(tokens, np.int64)
    out = np.empty((planes, len(t), row), np.uint8)
    for l in range(planes):
        for j, tok in enumerate(t):
            out[l, j] = ((tok * 131 + l * 17 + salt + np.arange(row) * 7) % 251).astype(np.uint8)
    return out


def pin_kv_rollback_exercise(lib):
    """The Arabic lesson's rollback exercise (tests/golden/kv_rollback_exercise.json):
    10 cached tokens, 5 drafts pushed to the scratch buffer, a rejection at the
    third; the cache must read the prefix and then the first two drafts, with
    length 12 and nothing past it written."""
    g = json.load(open(os.path.join(GOLDEN, "kv_rollback_exercise.json")))
    planes, row, S = 4, 24, 16
    prefix = np.arange(100, 100 + g["prefix_tokens"])
    drafts = np.arange(500, 500 + g["drafts_pushed"])
    cache = np.full((planes, 1, S, row), 0xEE, np.uint8)
    cache[:, 0, :len(prefix)] = _kv_of(prefix, planes, row)
    scratch = _kv_of(drafts, planes, row)[:, None]
    accepted = g["rejected_draft"] - 1
    assert accepted == g["accepted_drafts"]
    out, new_len = oracle.kv_commit(scratch, cache, None, [accepted], [len(prefix)], lib=lib)
    assert new_len[0] == g["cache_length_after"]
    want = _kv_of(np.concatenate([prefix, drafts[:accepted]]), planes, row)
    assert np.array_equal(out[:, 0, :new_len[0]], want)
    assert np.all(out[:, 0, new_len[0]:] == 0xEE)


def pin_kv_commit_tree_path(lib, seed=53):
    """After a greedy tree verify, committing the accepted path (root included)
    leaves the cache reading the prefix, the root token and the accepted
    tokens, in order; predicted from the token sequence alone."""
    rng = np.random.default_rng(seed)
    planes, row = 3, 16
    for trial in range(40):
        N, V, B = int(rng.integers(1, 16)), 6, 3
        parents = [-1] + [int(rng.integers(0, v)) for v in range(1, N)]
        logits = (rng.integers(-3, 4, size=(B, N, V)) * 0.5).astype(np.float32)
        tokens = rng.integers(0, V, size=(B, N)).astype(np.int32)
        amax = np.argmax(logits, axis=-1)
        for b in range(B):   # make acceptance likely: a child often carries its parent's argmax
            for v in range(1, N):
                if rng.random() < 0.7:
                    tokens[b, v] = amax[b, parents[v]]
        root_tok = rng.integers(0, V, size=B)
        tokens[:, 0] = root_tok
        out_t, out_p, out_d = oracle.verify_tree_greedy(logits, tokens, parents, lib=lib)
        S = 12 + N
        lens = rng.integers(0, 12, size=B).astype(np.int32)
        prefixes = [rng.integers(0, V, size=int(lens[b])) for b in range(B)]
        cache = np.zeros((planes, B, S, row), np.uint8)
        scratch = np.zeros((planes, B, N, row), np.uint8)
        for b in range(B):
            cache[:, b, :lens[b]] = _kv_of(prefixes[b], planes, row)
            scratch[:, b] = _kv_of(tokens[b], planes, row)
        count = (out_d + 1).astype(np.int32)
        out, new_len = oracle.kv_commit(scratch, cache, out_p, count, lens, lib=lib)
        for b in range(B):
            d = int(out_d[b])
            seq = np.concatenate([prefixes[b], [root_tok[b]], out_t[b, :d]])
            assert new_len[b] == lens[b] + d + 1
            assert np.array_equal(out[:, b, :new_len[b]], _kv_of(seq, planes, row)), (trial, b)
            assert not out[:, b, new_len[b]:].any()


def pin_kv_commit_invariants(lib, seed=59):
    """Random commits: slots outside [len, len + count) never change; a
    sequence whose count, length or path is out of range is left whole and
    keeps its length; two commits in a row equal one commit of both parts."""
    rng = np.random.default_rng(seed)
    for trial in range(60):
        planes, B, N, S, row = int(rng.integers(1, 4)), 5, int(rng.integers(1, 9)), 14, 8
        scratch = rng.integers(0, 256, size=(planes, B, N, row)).astype(np.uint8)
        cache = rng.integers(0, 256, size=(planes, B, S, row)).astype(np.uint8)
        P = N + 1
        path = rng.integers(0, N, size=(B, P)).astype(np.int32)
        count = rng.integers(0, N + 1, size=B).astype(np.int32)
        lens = rng.integers(0, S + 1, size=B).astype(np.int32)
        bad = rng.random(B) < 0.4
        for b in np.nonzero(bad)[0]:
            kind = int(rng.integers(0, 4))
            if kind == 0:
                count[b] = P + 1
            elif kind == 1:
                count[b] = max(count[b], 1)
                path[b, int(rng.integers(0, count[b]))] = int(rng.choice([-1, N]))
            elif kind == 2:
                lens[b] = S - count[b] + 1
            else:
                count[b] = -1
        out, new_len = oracle.kv_commit(scratch, cache, path, count, lens, lib=lib)
        for b in range(B):
            valid = (0 <= count[b] <= P and lens[b] >= 0 and lens[b] + count[b] <= S
                     and np.all((path[b, :max(count[b], 0)] >= 0) & (path[b, :max(count[b], 0)] < N)))
            if not valid:
                assert new_len[b] == lens[b] and np.array_equal(out[:, b], cache[:, b]), (trial, b)
                continue
            c, L = int(count[b]), int(lens[b])
            assert new_len[b] == L + c
            assert np.array_equal(out[:, b, :L], cache[:, b, :L])
            assert np.array_equal(out[:, b, L + c:], cache[:, b, L + c:])
            for i in range(c):
                assert np.array_equal(out[:, b, L + i], scratch[:, b, path[b, i]]), (trial, b, i)
        # two commits equal one: split each valid sequence's count in two
        ok = np.array([0 <= count[b] <= P and 0 <= lens[b] and lens[b] + count[b] <= S
                       and np.all((path[b, :max(count[b], 0)] >= 0) & (path[b, :max(count[b], 0)] < N))
                       for b in range(B)])
        c1 = np.where(ok, count // 2, 0).astype(np.int32)
        c2 = np.where(ok, count - c1, 0).astype(np.int32)
        mid, l1 = oracle.kv_commit(scratch, cache, path, c1, lens, lib=lib)
        path2 = np.zeros_like(path)
        for b in range(B):
            path2[b, :P - c1[b]] = path[b, c1[b]:]
        two, l2 = oracle.kv_commit(scratch, mid, path2, c2, l1, lib=lib)
        one, l12 = oracle.kv_commit(scratch, cache, path, np.where(ok, count, 0).astype(np.int32),
                                    lens, lib=lib)
        assert np.array_equal(two, one) and np.array_equal(l2, l12), trial


# ------------------------------------------------------------- tree attention mask

def _mask_bits(mask_rows, N):
    """Boolean [.., N, N] from packed ancestor words [.., N, ceil(N/32)]."""
    w = np.asarray(mask_rows, np.uint32)
    j = np.arange(N)
    return ((w[..., j // 32] >> (j % 32).astype(np.uint32)) & 1).astype(bool)


def pin_tree_mask_figure(lib):
    """The French lesson's drawn tree: each node attends to itself and its
    ancestors only (tests/golden/tree_mask_p1_figure.json, written by hand)."""
    g = json.load(open(os.path.join(GOLDEN, "tree_mask_p1_figure.json")))
    mask, depth = oracle.tree_mask(g["parents"], lib=lib)
    assert np.array_equal(_mask_bits(mask[0], 7), np.array(g["mask"], bool))
    assert list(depth[0]) == g["depth"]


def _subtrees(par, n):
    """Descendant sets by walking children lists top-down from each node,
    over the attached nodes below n (an independent construction)."""
    children = [[] for _ in range(n)]
    attached = [False] * n
    attached[0] = True
    for v in range(1, n):
        p = par[v]
        if 0 <= p < v and attached[p]:
            attached[v] = True
            children[p].append(v)
    sub = []
    for j in range(n):
        seen, stack = set(), [j] if attached[j] else []
        while stack:
            u = stack.pop()
            seen.add(u)
            stack.extend(children[u])
        sub.append(seen)
    return attached, sub


def pin_tree_mask_descendants(lib, seed=61):
    """Random per-sequence trees with padding and out-of-range parent
    entries: mask[i][j] holds iff i lies in j's subtree (children lists
    walked top-down), and depth is the number of strict ancestors."""
    rng = np.random.default_rng(seed)
    for trial in range(60):
        N, B = int(rng.integers(1, 80)), 4
        par = np.zeros((B, N), np.int32)
        counts = rng.integers(0, N + 3, size=B).astype(np.int32)   # clamped to [1, N]
        for b in range(B):
            par[b, 0] = -1
            for v in range(1, N):
                par[b, v] = rng.integers(0, v) if rng.random() > 0.05 else rng.choice([-1, v, v + 5])
        mask, depth = oracle.tree_mask(par, counts, lib=lib)
        bits = _mask_bits(mask, N)
        for b in range(B):
            n = int(min(max(counts[b], 1), N))
            attached, sub = _subtrees(par[b], n)
            want = np.zeros((N, N), bool)
            for j in range(n):
                for i in sub[j]:
                    want[i, j] = True
            assert np.array_equal(bits[b], want), (trial, b)
            for v in range(N):
                d = int(want[v].sum()) - 1 if v < n and attached[v] else -1
                assert depth[b, v] == d, (trial, b, v)


def pin_tree_mask_chain(lib):
    """A chain (parents v - 1) is plain causal attention: a lower-triangular
    mask, and depth v."""
    for N in (1, 5, 32, 33, 100):
        par = np.arange(-1, N - 1, dtype=np.int32)
        mask, depth = oracle.tree_mask(par, lib=lib)
        assert np.array_equal(_mask_bits(mask[0], N), np.tril(np.ones((N, N), bool)))
        assert list(depth[0]) == list(range(N))


# ------------------------------------------------------------- chi-square

def pin_chi_square(lib, n=50_000, seed=19):
    """The emitted token passes a chi-square test against p at the 0.05 level
    over 50,000 draws (Arabic lesson, exercises), at the first position and at
    the bonus position."""
    from scipy.stats import chisquare
    rng = np.random.default_rng(seed)
    V, K, T = 8, 1, 1.0
    p = [rng.dirichlet(np.ones(V) * 2) for _ in range(K + 1)]
    q = rng.dirichlet(np.ones(V) * 2)
    tl = np.tile(np.log(np.array(p, np.float32)), (n, 1, 1)).astype(np.float32)
    dl = np.tile(np.log(q.astype(np.float32)), (n, 1, 1)).astype(np.float32)
    tokens = rng.choice(V, size=(n, 1), p=q).astype(np.int32)
    ua = rng.random((n, 1), dtype=np.float32)
    us = rng.random((n,), dtype=np.float32)
    out, acc, _ = oracle.verify_chain(tl, dl, tokens, ua, us, T, lib=lib)
    p0 = np_softmax(np.log(np.array(p[0], np.float32)), 1.0)
    h0 = np.bincount(out[:, 0], minlength=V)
    assert chisquare(h0, p0 * n).pvalue > 0.05
    sel = acc == K
    p1 = np_softmax(np.log(np.array(p[1], np.float32)), 1.0)
    h1 = np.bincount(out[sel, 1], minlength=V)
    assert chisquare(h1, p1 * sel.sum()).pvalue > 0.05


ALL_PINS = [pin_exact_law, pin_expected_tokens, pin_page_counts, pin_strict_acceptance,
            pin_zero_draft_probability, pin_softmax_values, pin_row_helpers, pin_helper_closed_forms,
            pin_inverse_cdf, pin_greedy, pin_tree_bruteforce, pin_tree_chain,
            pin_tree_figure, pin_tree_dyn_bruteforce, pin_tree_dyn_padding, pin_tree_dyn_chain,
            pin_topk_sort, pin_topk_argmax, pin_kv_rollback_exercise, pin_kv_commit_tree_path,
            pin_kv_commit_invariants, pin_tree_mask_figure, pin_tree_mask_descendants,
            pin_tree_mask_chain, pin_chi_square]
