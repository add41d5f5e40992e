"""CPU tests: the fp64 oracle against what the pages and mathematics fix."""
import os
import re
import tempfile

import numpy as np
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_oracle_rejects_bad_arguments(lib):
    t = np.zeros((1, 2, 4), np.float32)
    d = np.zeros((1, 1, 4), np.float32)
    u = np.array([[0.5]], np.float32)
    s = np.array([0.5], np.float32)
    with pytest.raises(ValueError):
        oracle.verify_chain(t, d, [[4]], u, s, 1.0, lib=lib)        # token out of range
    with pytest.raises(ValueError):
        oracle.verify_chain(t, d, [[1]], u, s, 0.0, lib=lib)        # T must be > 0
    for bad in ([0, 0, 1], [-1, 1, 0], [-1, 0, 2], [-1, -1, 0]):
        with pytest.raises(ValueError):
            oracle.verify_tree_greedy(np.zeros((1, 3, 4), np.float32),
                                      np.zeros((1, 3), np.int32), bad, lib=lib)


def test_empty_and_degenerate(lib):
    # B = 0: nothing to do
    t, a, _ = oracle.verify_chain(np.zeros((0, 3, 5), np.float32), np.zeros((0, 2, 5), np.float32),
                                  np.zeros((0, 2), np.int32), np.zeros((0, 2), np.float32),
                                  np.zeros((0,), np.float32), 1.0, lib=lib)
    assert t.shape == (0, 3) and a.shape == (0,)
    # K = 0: the step is a plain draw from p_0 (and greedy is plain argmax)
    tl = np.log(np.array([[[0.25, 0.25, 0.5]]], np.float32))
    t, a, _ = oracle.verify_chain(tl, np.zeros((1, 0, 3), np.float32), np.zeros((1, 0), np.int32),
                                  np.zeros((1, 0), np.float32), np.array([0.6], np.float32), 1.0,
                                  lib=lib)
    assert a[0] == 0 and t[0, 0] == 2
    t, a = oracle.verify_greedy(tl, np.zeros((1, 0), np.int32), lib=lib)
    assert a[0] == 0 and t[0, 0] == 2
    # V = 1: every draw is token 0 and every draft is accepted
    t, a, _ = oracle.verify_chain(np.zeros((2, 3, 1), np.float32), np.zeros((2, 2, 1), np.float32),
                                  np.zeros((2, 2), np.int32), np.full((2, 2), 0.9, np.float32),
                                  np.full((2,), 0.9, np.float32), 1.0, lib=lib)
    assert np.all(a == 2) and np.all(t == 0)
    # tree with the root only: emit the root's argmax
    tt, tp, td = oracle.verify_tree_greedy(np.array([[[0, 3, 1]]], np.float32),
                                           np.zeros((1, 1), np.int32), [-1], lib=lib)
    assert td[0] == 0 and tt[0, 0] == 1 and tp[0, 0] == 0


# ---------------------------------------------------------------- mutations

MUTANTS = [
    # (name, pattern in spec_oracle.c, replacement, which occurrence)
    ("residual sign swapped", "double d = p[i] - q[i];", "double d = q[i] - p[i];", 0),
    ("residual positive part dropped", "w[i] = d > 0.0 ? d : 0.0;", "w[i] = d;", 0),
    ("acceptance ratio inverted", "return u < P / Q;", "return u < Q / P;", 0),
    ("non-strict acceptance", "return u < P / Q;", "return u <= P / Q;", 0),
    ("zero draft probability always rejects", "    return P > 0.0;\n}", "    return 0;\n}", 0),
    ("zero draft probability accepts whatever p", "    return P > 0.0;\n}", "    return 1;\n}", 0),
    ("single-row softmax ignores the temperature", "    softmax_T(l, V, T, out_p);", "    softmax_T(l, V, 1.0, out_p);", 0),
    ("temperature ignored", "p[i] = exp((l[i] - m) / T);", "p[i] = exp(l[i] - m);", 0),
    ("bonus from row K-1", "seq * (size_t)(K + 1) + (size_t)K, V, l);",
     "seq * (size_t)(K + 1) + (size_t)(K > 0 ? K - 1 : 0), V, l);", 0),
    ("draft row off by one", "load_row(draft, dtype, seq * (size_t)K + (size_t)k, V, l);",
     "load_row(draft, dtype, seq * (size_t)K + (size_t)(k + 1 < K ? k + 1 : k), V, l);", 0),
    ("non-strict inverse CDF", "if (C > tau)", "if (C >= tau)", 0),
    ("residual from q at rejection", "tokens[k] = residual_draw(p, q, V, us, w, &S);",
     "tokens[k] = residual_draw(q, p, V, us, w, &S);", 0),
    ("argmax ties to the highest index", "if (v > bv) {", "if (v >= bv) {", 0),
    ("greedy emits the draft at a mismatch", "                out[k] = a;\n                j = k;",
     "                out[k] = x[(size_t)b * K + k];\n                j = k;", 0),
    ("tree compares with the node's own argmax", "== amax[parents[v]];", "== amax[v];", 0),
    ("tree ties to the highest index", "if (ok[v] && depth[v] > depth[best])",
     "if (ok[v] && depth[v] >= depth[best])", 0),
    ("tree ignores ancestors", "ok[v] = ok[parents[v]] &&", "ok[v] = 1 &&", 0),
    ("per-sequence tree compares with the node's own argmax", "tok[v] == am[par[v]];",
     "tok[v] == am[v];", 0),
    ("per-sequence tree ties to the highest index", "if (acc[v] && dep[v] > dep[top])",
     "if (acc[v] && dep[v] >= dep[top])", 0),
    ("per-sequence tree ignores ancestors", "acc[v] = acc[par[v]] &&", "acc[v] = 1 &&", 0),
    ("top-k ties to the highest index", "if (best < 0 || v > bv) {", "if (best < 0 || v >= bv) {", 0),
    ("top-k takes an entry twice", "used |= taken[t] == i;", "used |= 0;", 0),
    ("per-sequence tree rows strided by the node count",
     "row_argmax(node_logits, dtype, (size_t)b * Nmax + (size_t)v, V);",
     "row_argmax(node_logits, dtype, (size_t)b * n + (size_t)v, V);", 0),
    ("acceptance rate takes the larger mass", "a += p[i] < q[i] ? p[i] : q[i];",
     "a += p[i] < q[i] ? q[i] : p[i];", 0),
    ("draw weights keep the negative part", "            out_w[i] = d > 0.0 ? d : 0.0;",
     "            out_w[i] = d;", 0),
    ("KV commit writes from slot 0, ignoring the length", "* S + L + i) * (size_t)row_bytes;",
     "* S + i) * (size_t)row_bytes;", 0),
    ("KV commit ignores the path", "                int r = path ? path[(size_t)b * P + i] : i;",
     "                int r = i;", 0),
    ("KV commit keeps the old length", "        new_len[b] = L + c;", "        new_len[b] = L;", 0),
    ("KV commit swaps plane and sequence strides", "size_t from = (((size_t)l * B + b) * N + r)",
     "size_t from = (((size_t)b * planes + l) * N + r)", 0),
    ("tree mask leaves out the node itself", "            row[cur / 32] |= 1u << (cur % 32);\n            while",
     "            while", 0),
    ("tree mask depth counts the node itself", "            depth[(size_t)b * N + v] = steps;",
     "            depth[(size_t)b * N + v] = steps + 1;", 0),
    ("tree mask keeps padding rows", "            if (v >= n)\n                continue;\n            int cur",
     "            int cur", 0),
    ("tree mask keeps unattached rows", "            if (!attached) {\n                for (int w = 0; w < W; ++w)\n                    row[w] = 0;\n                continue;",
     "            if (!attached) {\n                continue;", 0),
]

QUICK_PINS = [P.pin_exact_law, P.pin_expected_tokens, P.pin_page_counts, P.pin_strict_acceptance,
              P.pin_zero_draft_probability, P.pin_softmax_values, P.pin_row_helpers,
              P.pin_helper_closed_forms,
              P.pin_inverse_cdf, P.pin_greedy, P.pin_tree_bruteforce, P.pin_tree_figure,
              P.pin_tree_dyn_bruteforce, P.pin_tree_dyn_padding, P.pin_topk_sort,
              P.pin_kv_rollback_exercise, P.pin_kv_commit_tree_path, P.pin_kv_commit_invariants,
              P.pin_tree_mask_figure, P.pin_tree_mask_descendants, P.pin_chi_square]


def _mutant_lib(tmpdir, pattern, repl, which):
    src = open(oracle._SRC).read()
    starts = [m.start() for m in re.finditer(re.escape(pattern), src)]
    assert len(starts) > which, f"pattern not found: {pattern!r}"
    s = starts[which]
    mutated = src[:s] + repl + src[s + len(pattern):]
    path = os.path.join(tmpdir, "mutant.c")
    open(path, "w").write(mutated)
    so = os.path.join(tmpdir, "libmutant.so")
    oracle.build(so, path, extra_flags=("-w",))
    return oracle.load(so)


@pytest.mark.slow
@pytest.mark.parametrize("name,pattern,repl,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(name, pattern, repl, which):
    """Each plausible mistake planted in a copy of the oracle fails at least one pin."""
    with tempfile.TemporaryDirectory() as d:
        lib = _mutant_lib(d, pattern, repl, which)
        failed = []
        for pin in QUICK_PINS:
            try:
                pin(lib)
            except (AssertionError, ValueError, IndexError):
                failed.append(pin.__name__)
        assert failed, f"mutant '{name}' passed every pin"
