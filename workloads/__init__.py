"""Seeded synthetic inputs for the speculative-sampling verify step.

This module only *makes inputs*: logits with the shapes and value
distributions of the workloads below, drafted tokens, and the uniforms the
verify step consumes.  It holds none of the verify step's arithmetic (no
softmax, no acceptance test, no residual, no inverse CDF), and both the GPU
tests and the CPU oracle take their inputs from here.

Workloads (sizes and distributions as specified for this verify step):

  chain_t1_small   chain verify, T=1, B=8, K=4, V=1024, fp32; target iid N(0, 2^2);
                   draft = target + N(0, 0.5^2); drafted tokens sampled from q.
  greedy_32k       greedy chain verify, B=64, K=5, V=32000, bf16; target iid N(0, 3^2);
                   drafted token = target argmax with probability 0.8, else a
                   uniformly random other token.
  chain_t1_128k    chain verify, T=1, B=64, K=5, V=128256, bf16; target iid
                   N(0, 2.5^2) with 16 distinct random peak tokens per row raised
                   by +8; draft = target + N(0, sigma^2), sigma = C3_SIGMA so
                   that the mean acceptance rate is 0.75; drafted tokens from q.
  chain_t07_152k   chain verify, T=0.7, B=256, K=8, V=151936, fp32; target row
                   logit of the token at rank r (random permutation per row) is
                   -1.1 ln r plus N(0, 0.3^2); draft = target + N(0, 0.8^2);
                   drafted tokens from q.
  tree_128k        greedy static-tree verify, B=32, V=128256, bf16, branching
                   (4, 2, 2, 1) in breadth-first order (N = 45 nodes); rows as in
                   chain_t1_128k's target; the k-th child of node u carries u's
                   argmax with probability 0.6, else u's (k+1)-th ranked token.
  tree_dyn_128k    greedy verify on per-sequence trees, B=32, at most 64 nodes,
                   V=128256, bf16; each sequence's tree has a node count uniform
                   in [16, 64] and is grown breadth-first with 1 to 4 children
                   per node (a stand-in for trees shaped by the draft's
                   confidence); rows and node tokens as in tree_128k.
  topk_128k        top-k of draft rows for tree expansion, 512 rows (64
                   sequences x 8 frontier nodes), V=128256, bf16, k=8; rows are
                   chain_t1_128k's draft rows (peaked target + N(0, C3_SIGMA^2)).
  kv_commit_b64    KV commit after a tree verify, B=64 sequences, 64 planes (32
                   layers x keys and values), 2048-byte rows (8 KV heads x head
                   dim 128 x bf16), N=64 scratch rows (the tree's nodes), S=512
                   cache slots; per sequence a cache length uniform in [0, 440]
                   and an accepted path of 1 to 8 entries (root, then strictly
                   increasing node ids, as along a breadth-first tree's root
                   path).  Scratch and cache contents are random bytes.
  tree_mask_b64    tree attention mask for 64 sequences' trees of at most 64
                   nodes, shaped as in tree_dyn_128k (counts uniform in
                   [16, 64], 1 to 4 children per node, breadth-first).

Drafted tokens are "sampled from q" with the Gumbel-max construction
(argmax_i of d_i / T + G_i with G_i standard Gumbel), which draws exactly from
softmax(d / T) without computing it; it stands in for the draft model's own
sampling and uses the *rounded* draft logits the verifier sees.

Random streams: ``np.random.default_rng([workload_id, stream, step])`` with
streams 0 target logits, 1 draft noise, 2 peaks / permutations, 3 drafted-token
randomness, 4 verify uniforms.  bf16 values are made from float32 by
round-to-nearest-even.  Uniforms are float32 drawn directly in [0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

# sigma of the chain_t1_128k draft noise; calibrated so that the mean over rows
# of sum_i min(p_i, q_i) is 0.75 (checked by tests/test_workloads.py).
C3_SIGMA = 0.66


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # seed component
    mode: str                # "chain" | "greedy" | "tree" | "tree_dyn" | "topk" | "kv" | "mask"
    B: int
    V: int
    dtype: str               # "f32" | "bf16"
    K: int = 0               # chain / greedy draft length; tree_dyn: most nodes per tree; topk: k;
                             # kv: scratch rows per sequence
    T: float = 0.0           # chain temperature
    branching: tuple = field(default_factory=tuple)   # tree only
    recipe: str = "normal"   # target rows: "normal" | "peaked" | "zipf"
    target_sd: float = 2.0   # sd of the "normal" recipe
    sigma: float = 0.0       # sd of the draft noise (chain)
    steps: int = 1000
    planes: int = 0          # kv: planes (layers x keys/values)
    row_bytes: int = 0       # kv: bytes per row of a plane
    slots: int = 0           # kv: cache slots per sequence

    def with_sizes(self, **kw) -> "Workload":
        """Same recipe at other sizes (for small parity cases)."""
        return replace(self, **kw)


WORKLOADS = {
    "chain_t1_small": Workload("chain_t1_small", 1, "chain", B=8, K=4, V=1024, dtype="f32",
                               T=1.0, recipe="normal", target_sd=2.0, sigma=0.5),
    "greedy_32k": Workload("greedy_32k", 2, "greedy", B=64, K=5, V=32000, dtype="bf16",
                           recipe="normal", target_sd=3.0),
    "chain_t1_128k": Workload("chain_t1_128k", 3, "chain", B=64, K=5, V=128256, dtype="bf16",
                              T=1.0, recipe="peaked", sigma=C3_SIGMA),
    "chain_t07_152k": Workload("chain_t07_152k", 4, "chain", B=256, K=8, V=151936, dtype="f32",
                               T=0.7, recipe="zipf", sigma=0.8, steps=100),
    "tree_128k": Workload("tree_128k", 5, "tree", B=32, V=128256, dtype="bf16",
                          branching=(4, 2, 2, 1), recipe="peaked"),
    "tree_dyn_128k": Workload("tree_dyn_128k", 6, "tree_dyn", B=32, V=128256, dtype="bf16",
                              K=64, recipe="peaked"),
    "topk_128k": Workload("topk_128k", 7, "topk", B=512, V=128256, dtype="bf16", K=8,
                          recipe="peaked", sigma=C3_SIGMA),
    "kv_commit_b64": Workload("kv_commit_b64", 8, "kv", B=64, V=0, dtype="u8", K=64, planes=64,
                              row_bytes=2048, slots=512),
    "tree_mask_b64": Workload("tree_mask_b64", 9, "mask", B=64, V=0, dtype="i32", K=64),
}

TARGET, DRAFT_NOISE, STRUCTURE, DRAFT_TOKENS, UNIFORMS = range(5)


def rng_for(w: Workload, stream: int, step: int) -> np.random.Generator:
    return np.random.default_rng([w.wid, stream, step])


# ---------------------------------------------------------------- bf16 helpers

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    src = np.ascontiguousarray(x, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(src.shape, np.uint16)
    blk = 1 << 20
    u = np.empty(min(blk, src.size), np.uint32)
    lsb = np.empty_like(u)
    for s in range(0, src.size, blk):
        n = min(blk, src.size - s)
        np.right_shift(src[s:s + n], np.uint32(16), out=lsb[:n])
        np.bitwise_and(lsb[:n], np.uint32(1), out=lsb[:n])
        np.add(src[s:s + n], np.uint32(0x7FFF), out=u[:n])
        np.add(u[:n], lsb[:n], out=u[:n])
        np.right_shift(u[:n], np.uint32(16), out=u[:n])
        out[s:s + n] = u[:n]
    return out.reshape(np.shape(x))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(a: np.ndarray) -> np.ndarray:
    """Logit array (float32 or bf16 bits) as float32 values."""
    return bf16_to_f32(a) if a.dtype == np.uint16 else a


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


# ---------------------------------------------------------------- row recipes

def _normal(rng, shape, scale):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)


def _peaked_rows(w: Workload, rows: int, rng0, rng2) -> np.ndarray:
    """N(0, 2.5^2) rows with 16 distinct random peak tokens raised by +8."""
    x = _normal(rng0, (rows, w.V), 2.5)
    npk = min(16, w.V)
    for r in range(rows):
        idx = rng2.choice(w.V, size=npk, replace=False)
        x[r, idx] += np.float32(8.0)
    return x


def _zipf_rows(w: Workload, rows: int, rng0, rng2) -> np.ndarray:
    """Row logit of the token at rank r is -1.1 ln r (random rank order per row) + N(0, 0.3^2)."""
    base = (-1.1 * np.log(np.arange(1, w.V + 1, dtype=np.float64))).astype(np.float32)
    x = _normal(rng0, (rows, w.V), 0.3)
    for r in range(rows):
        perm = rng2.permutation(w.V)
        x[r, perm] += base
    return x


def _target_rows(w: Workload, rows: int, rng0, rng2) -> np.ndarray:
    if w.recipe == "peaked":
        return _peaked_rows(w, rows, rng0, rng2)
    if w.recipe == "zipf":
        return _zipf_rows(w, rows, rng0, rng2)
    return _normal(rng0, (rows, w.V), w.target_sd)


def _gumbel_draw(rows_f32: np.ndarray, T: float, rng) -> np.ndarray:
    """One token per row drawn from softmax(row / T) by the Gumbel-max construction."""
    out = np.empty(rows_f32.shape[0], np.int32)
    for r in range(rows_f32.shape[0]):
        u = rng.random(rows_f32.shape[1])
        g = -np.log(-np.log(u))
        out[r] = int(np.argmax(rows_f32[r].astype(np.float64) / T + g))
    return out


def _uniforms(w: Workload, step: int, B: int, K: int):
    rng = rng_for(w, UNIFORMS, step)
    ua = rng.random((B, K), dtype=np.float32)
    us = rng.random((B,), dtype=np.float32)
    return ua, us


# ---------------------------------------------------------------- public makers

def chain_uniforms(w: Workload, step: int):
    """The uniforms of chain step `step` alone (u_accept [B][K], u_sample [B]):
    the same values chain_inputs(w, step) holds, without its logits."""
    return _uniforms(w, step, w.B, w.K)


def chain_inputs(w: Workload, step: int = 0) -> dict:
    """Inputs of one chain verify step: target [B][K+1][V], draft [B][K][V],
    tokens [B][K] int32, u_accept [B][K] f32, u_sample [B] f32, T, dtype."""
    assert w.mode == "chain"
    B, K, V = w.B, w.K, w.V
    rng0, rng1 = rng_for(w, TARGET, step), rng_for(w, DRAFT_NOISE, step)
    rng2, rng3 = rng_for(w, STRUCTURE, step), rng_for(w, DRAFT_TOKENS, step)
    tgt = _store(_target_rows(w, B * (K + 1), rng0, rng2), w.dtype).reshape(B, K + 1, V)
    tgt_vals = as_f32(tgt)
    dft = tgt_vals[:, :K, :] + _normal(rng1, (B, K, V), w.sigma)
    dft = _store(dft, w.dtype).reshape(B, K, V)
    tokens = _gumbel_draw(as_f32(dft).reshape(B * K, V), w.T, rng3).reshape(B, K)
    ua, us = _uniforms(w, step, B, K)
    return dict(target=tgt, draft=dft, tokens=tokens, u_accept=ua, u_sample=us,
                T=w.T, dtype=w.dtype)


def greedy_inputs(w: Workload, step: int = 0, p_match: float = 0.8) -> dict:
    """Inputs of one greedy chain step: target [B][K+1][V], tokens [B][K]."""
    assert w.mode == "greedy"
    B, K, V = w.B, w.K, w.V
    tgt = _store(_target_rows(w, B * (K + 1), rng_for(w, TARGET, step), rng_for(w, STRUCTURE, step)),
                 w.dtype)
    tgt = tgt.reshape(B, K + 1, V)
    vals = as_f32(tgt)[:, :K, :]
    top = np.argmax(vals, axis=-1)                       # first maximum
    rng3 = rng_for(w, DRAFT_TOKENS, step)
    keep = rng3.random((B, K)) < p_match
    other = rng3.integers(0, max(V - 1, 1), size=(B, K))
    other = np.where(other >= top, other + 1, other) if V > 1 else top
    tokens = np.where(keep, top, other).astype(np.int32)
    return dict(target=tgt, tokens=tokens, dtype=w.dtype)


def tree_parents(branching) -> np.ndarray:
    """Breadth-first parent array of a tree with the given per-depth branching."""
    parents = [-1]
    level = [0]
    for b in branching:
        nxt = []
        for u in level:
            for _ in range(b):
                parents.append(u)
                nxt.append(len(parents) - 1)
        level = nxt
    return np.asarray(parents, np.int32)


def _ranked(row: np.ndarray, n: int) -> np.ndarray:
    """Indices of the n largest entries, by value descending then index ascending."""
    n = min(n, row.shape[0])
    kth = np.partition(row, row.shape[0] - n)[row.shape[0] - n]
    cand = np.nonzero(row >= kth)[0]
    order = np.lexsort((cand, -row[cand].astype(np.float64)))
    return cand[order][:n]


def _node_tokens(vals_b: np.ndarray, par: np.ndarray, n: int, rng3, p_match: float) -> np.ndarray:
    """Tokens of nodes 1..n-1 of one tree: the k-th child of node u carries u's
    argmax with probability p_match, else u's (k+1)-th ranked token."""
    ordinal = np.zeros(n, np.int64)  # 1-based place of each node among its parent's children
    seen = {}
    for v in range(1, n):
        seen[par[v]] = seen.get(par[v], 0) + 1
        ordinal[v] = seen[par[v]]
    nrank = int(ordinal.max()) + 1 if n > 1 else 1
    tokens = np.zeros(n, np.int32)
    ranks = {}
    for v in range(1, n):
        u = int(par[v])
        if u not in ranks:
            ranks[u] = _ranked(vals_b[u], nrank)
        r = ranks[u]
        k = int(ordinal[v])
        take_top = rng3.random() < p_match
        tokens[v] = r[0] if take_top or k >= len(r) else r[k]
    return tokens


def tree_inputs(w: Workload, step: int = 0, p_match: float = 0.6, parents=None) -> dict:
    """Inputs of one greedy tree step: node_logits [B][N][V], node_tokens [B][N], parents [N]."""
    assert w.mode == "tree"
    par = tree_parents(w.branching) if parents is None else np.asarray(parents, np.int32)
    N, B, V = len(par), w.B, w.V
    rng0, rng2, rng3 = rng_for(w, TARGET, step), rng_for(w, STRUCTURE, step), rng_for(w, DRAFT_TOKENS, step)
    logits = _store(_target_rows(w, B * N, rng0, rng2), w.dtype).reshape(B, N, V)
    vals = as_f32(logits)
    tokens = np.stack([_node_tokens(vals[b], par, N, rng3, p_match) for b in range(B)])
    return dict(node_logits=logits, node_tokens=tokens, parents=par, dtype=w.dtype)


def dyn_tree(rng, nmax: int, nmin: int = 1, max_children: int = 4) -> np.ndarray:
    """One tree of n nodes (n uniform in [nmin, nmax]) grown breadth-first,
    each node taking 1..max_children children until n nodes exist: parents in
    topological order (parents[0] = -1, parents[v] < v)."""
    n = int(rng.integers(nmin, nmax + 1))
    parents, queue = [-1], [0]
    while len(parents) < n:
        u = queue.pop(0)
        for _ in range(int(rng.integers(1, max_children + 1))):
            if len(parents) == n:
                break
            parents.append(u)
            queue.append(len(parents) - 1)
    return np.asarray(parents, np.int32)


def tree_dyn_inputs(w: Workload, step: int = 0, p_match: float = 0.6, nmin: int | None = None) -> dict:
    """Inputs of one greedy step on per-sequence trees: node_logits [B][Nmax][V],
    node_tokens [B][Nmax], parents [B][Nmax], node_count [B].  Padding (nodes
    past a tree's count) has logits like any row, token 0 and parent 0."""
    assert w.mode == "tree_dyn"
    B, Nmax, V = w.B, w.K, w.V
    rng0, rng2, rng3 = rng_for(w, TARGET, step), rng_for(w, STRUCTURE, step), rng_for(w, DRAFT_TOKENS, step)
    nmin = max(1, Nmax // 4) if nmin is None else nmin
    trees = [dyn_tree(rng2, Nmax, nmin) for _ in range(B)]
    logits = _store(_target_rows(w, B * Nmax, rng0, rng2), w.dtype).reshape(B, Nmax, V)
    vals = as_f32(logits)
    parents = np.zeros((B, Nmax), np.int32)
    tokens = np.zeros((B, Nmax), np.int32)
    counts = np.zeros(B, np.int32)
    for b, par in enumerate(trees):
        n = len(par)
        counts[b] = n
        parents[b, :n] = par
        tokens[b, :n] = _node_tokens(vals[b], par, n, rng3, p_match)
    return dict(node_logits=logits, node_tokens=tokens, parents=parents, node_count=counts,
                dtype=w.dtype)


def topk_inputs(w: Workload, step: int = 0) -> dict:
    """Draft rows [B][V] for a top-k expansion step: the target recipe plus
    N(0, sigma^2) draft noise (sigma 0 leaves the target rows)."""
    assert w.mode == "topk"
    rng0, rng1, rng2 = rng_for(w, TARGET, step), rng_for(w, DRAFT_NOISE, step), rng_for(w, STRUCTURE, step)
    x = _target_rows(w, w.B, rng0, rng2)
    if w.sigma > 0:
        x += _normal(rng1, x.shape, w.sigma)
    return dict(logits=_store(x, w.dtype), k=w.K, dtype=w.dtype)


def kv_paths(w: Workload, step: int = 0, max_count: int = 8) -> dict:
    """The per-step part of a KV commit: path [B][N] (root, then strictly
    increasing node ids; entries past the count are 0), count [B] uniform in
    [1, max_count], cache_len [B] uniform in [0, S - max_count]."""
    assert w.mode == "kv"
    rng = rng_for(w, STRUCTURE, step)
    B, N, S = w.B, w.K, w.slots
    mc = max(1, min(max_count, N))
    count = rng.integers(1, mc + 1, size=B).astype(np.int32)
    path = np.zeros((B, N), np.int32)
    for b in range(B):
        c = int(count[b])
        if c > 1:
            path[b, 1:c] = np.sort(rng.choice(np.arange(1, N), size=c - 1, replace=False))
    cache_len = rng.integers(0, max(S - mc, 0) + 1, size=B).astype(np.int32)
    return dict(path=path, count=count, cache_len=cache_len)


def kv_scratch(w: Workload, step: int = 0) -> np.ndarray:
    """Scratch rows [planes][B][N][row_bytes] of random bytes."""
    rng = rng_for(w, TARGET, step)
    return rng.integers(0, 256, size=(w.planes, w.B, w.K, w.row_bytes), dtype=np.uint8)


def kv_cache_init(w: Workload, step: int = 0) -> np.ndarray:
    """Initial cache [planes][B][S][row_bytes] of random bytes (small sizes only)."""
    rng = rng_for(w, DRAFT_NOISE, step)
    return rng.integers(0, 256, size=(w.planes, w.B, w.slots, w.row_bytes), dtype=np.uint8)


def tree_mask_inputs(w: Workload, step: int = 0, nmin: int | None = None) -> dict:
    """Per-sequence trees for the attention mask: parents [B][Nmax] (padding
    parent 0) and node_count [B]."""
    assert w.mode == "mask"
    rng = rng_for(w, STRUCTURE, step)
    B, Nmax = w.B, w.K
    nmin = max(1, Nmax // 4) if nmin is None else nmin
    parents = np.zeros((B, Nmax), np.int32)
    counts = np.zeros(B, np.int32)
    for b in range(B):
        par = dyn_tree(rng, Nmax, nmin)
        counts[b] = len(par)
        parents[b, :len(par)] = par
    return dict(parents=parents, node_count=counts)


def make_inputs(w: Workload, step: int = 0) -> dict:
    if w.mode == "chain":
        return chain_inputs(w, step)
    if w.mode == "greedy":
        return greedy_inputs(w, step)
    if w.mode == "tree_dyn":
        return tree_dyn_inputs(w, step)
    if w.mode == "topk":
        return topk_inputs(w, step)
    if w.mode == "kv":
        return kv_paths(w, step)
    if w.mode == "mask":
        return tree_mask_inputs(w, step)
    return tree_inputs(w, step)
