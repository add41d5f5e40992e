"""CPU tests: the oracle's results do not depend on how many threads it uses.

Sequences are independent and each one's arithmetic is the single-threaded
one, so every output (probabilities included) must match bit for bit."""
import numpy as np
import pytest

import oracle
import workloads as W


@pytest.fixture
def threads():
    yield
    oracle.set_threads(0)


def _both(fn):
    oracle.set_threads(1)
    one = fn()
    n = oracle.set_threads(0)
    many = fn()
    return one, many, n


def _same(a, b):
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        x, y = np.asarray(x), np.asarray(y)
        assert x.dtype == y.dtype and np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_bitwise_at_any_thread_count(threads, dtype):
    w = W.Workload("threads", 91, "chain", B=24, K=5, V=3001, dtype=dtype, T=0.9, recipe="peaked",
                   sigma=0.7)
    d = W.chain_inputs(w, 0)
    one, many, n = _both(lambda: oracle.verify_chain(d["target"], d["draft"], d["tokens"], d["u_accept"],
                                                     d["u_sample"], d["T"], diag=True))
    _same(one, many)


def test_greedy_trees_topk_bitwise_at_any_thread_count(threads):
    d = W.greedy_inputs(W.WORKLOADS["greedy_32k"].with_sizes(B=24, V=2001), 0)
    _same(*_both(lambda: oracle.verify_greedy(d["target"], d["tokens"]))[:2])
    t = W.tree_inputs(W.WORKLOADS["tree_128k"].with_sizes(B=12, V=1001), 0)
    _same(*_both(lambda: oracle.verify_tree_greedy(t["node_logits"], t["node_tokens"], t["parents"]))[:2])
    td = W.tree_dyn_inputs(W.WORKLOADS["tree_dyn_128k"].with_sizes(B=12, K=20, V=999), 0)
    _same(*_both(lambda: oracle.verify_tree_greedy_dyn(td["node_logits"], td["node_tokens"],
                                                       td["parents"], td["node_count"]))[:2])
    x = W.topk_inputs(W.WORKLOADS["topk_128k"].with_sizes(B=40, V=3000), 0)["logits"]
    _same(*_both(lambda: oracle.topk(x, 8))[:2])
