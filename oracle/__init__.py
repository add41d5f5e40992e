"""Plain fp64 CPU oracle of the speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library never imports, links or
runs anything here, and nothing here comes from the GPU library.

The arithmetic lives in ``spec_oracle.c`` (double precision, scalar loops in
index order); this module builds it with gcc and marshals numpy arrays into it.
p is the target distribution and q the draft distribution, as on the French
lesson "Décodage spéculatif et Eagle" and the forum post "Speculative Decoding:
от идеи до SOTA".

Every function has at least one pin in ``tests/test_oracle_*.py`` that does not
reuse the oracle's own formula (exact enumeration of the output law, closed
forms, library argmax, brute-force tree paths, hand-derived fixtures).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def build(out_path: str = _LIB, src_path: str = _SRC, extra_flags=()) -> str:
    """Compile the oracle with gcc: plain IEEE double arithmetic, no FMA contraction."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra", *extra_flags, "-o", out_path + ".tmp",
           src_path, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def _bind(lib):
    vp, i32p = ctypes.c_void_p, ctypes.c_void_p
    d, i = ctypes.c_double, ctypes.c_int
    lib.oracle_verify_chain.argtypes = [vp, vp, i, i32p, vp, vp, i, i, i, d, vp, vp, vp]
    lib.oracle_verify_chain.restype = i
    lib.oracle_verify_chain_f64u.argtypes = [vp, vp, i, i32p, vp, vp, i, i, i, d, vp, vp, vp]
    lib.oracle_verify_chain_f64u.restype = i
    lib.oracle_draw_weights.argtypes = [vp, vp, i, i, d, vp]
    lib.oracle_draw_weights.restype = d
    lib.oracle_softmax_row.argtypes = [vp, i, i, d, vp]
    lib.oracle_softmax_row.restype = i
    lib.oracle_residual_draw.argtypes = [vp, vp, i, d, vp]
    lib.oracle_residual_draw.restype = i
    lib.oracle_acceptance_rate.argtypes = [vp, vp, i, i, d]
    lib.oracle_acceptance_rate.restype = d
    lib.oracle_row_argmax.argtypes = [vp, i, i]
    lib.oracle_row_argmax.restype = i
    lib.oracle_verify_greedy.argtypes = [vp, i, i32p, i, i, i, vp, vp]
    lib.oracle_verify_greedy.restype = i
    lib.oracle_verify_tree_greedy.argtypes = [vp, i, i32p, i32p, i, i, i, vp, vp, vp]
    lib.oracle_verify_tree_greedy.restype = i
    lib.oracle_verify_tree_greedy_dyn.argtypes = [vp, i, i32p, i32p, i32p, i, i, i, vp, vp, vp]
    lib.oracle_verify_tree_greedy_dyn.restype = i
    lib.oracle_topk.argtypes = [vp, i, i, i, i, vp, vp]
    lib.oracle_topk.restype = i
    lib.oracle_kv_commit.argtypes = [vp, vp, i, i, i, i, ctypes.c_int64, vp, i, vp, vp, vp]
    lib.oracle_kv_commit.restype = i
    lib.oracle_tree_mask.argtypes = [vp, vp, i, i, vp, vp]
    lib.oracle_tree_mask.restype = i
    lib.oracle_set_threads.argtypes = [i]
    lib.oracle_set_threads.restype = None
    lib.oracle_get_threads.argtypes = []
    lib.oracle_get_threads.restype = i
    return lib


def set_threads(n: int, *, lib=None) -> int:
    """Threads the oracle spreads sequences over (n <= 0: every processor).
    Returns the count now in force.  Results do not depend on it."""
    lib = lib or load()
    lib.oracle_set_threads(int(n))
    return lib.oracle_get_threads()


def load(path: str | None = None):
    """Load the oracle library, building it first if it is not there."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits(a):
    """Logit arrays are float32 (fp32) or uint16 (bf16 bit patterns)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def verify_chain(target, draft, tokens, u_accept, u_sample, temperature, *, diag=False,
                 lib=None):
    """Chain verify at T > 0.

    target [B][K+1][V], draft [B][K][V] (float32 or bf16 bits), tokens [B][K],
    u_accept [B][K] and u_sample [B] (float32 in [0,1), or float64 to use the
    double-precision entry).  Returns (tokens [B][K+1], accepted [B], diag or None)
    with diag [B][K+1][4] = (P, Q, ratio, S).
    """
    lib = lib or load()
    t, dt = _logits(target)
    d, dd = _logits(draft)
    assert dt == dd, "target and draft must share a dtype"
    B, K1, V = t.shape
    K = K1 - 1
    x = _i32(tokens).reshape(B, K)
    out_t = np.empty((B, K + 1), np.int32)
    out_a = np.empty((B,), np.int32)
    out_d = np.empty((B, K + 1, 4), np.float64) if diag else None
    ua = np.ascontiguousarray(u_accept).reshape(B, K)
    us = np.ascontiguousarray(u_sample).reshape(B)
    if ua.dtype == np.float64:
        fn = lib.oracle_verify_chain_f64u
        us = us.astype(np.float64)
    else:
        fn = lib.oracle_verify_chain
        ua = ua.astype(np.float32)
        us = us.astype(np.float32)
    rc = fn(_ptr(t), _ptr(d), dt, _ptr(x), _ptr(ua), _ptr(us), B, K, V,
            float(temperature), _ptr(out_t), _ptr(out_a), _ptr(out_d))
    if rc != 0:
        raise ValueError(f"oracle_verify_chain rejected its arguments (code {rc})")
    return out_t, out_a, out_d


def draw_weights(target_row, draft_row, temperature, *, lib=None):
    """Weights of the final draw: max(0, p - q) with a draft row, p without.  Returns (w, S)."""
    lib = lib or load()
    t, dt = _logits(target_row)
    V = t.shape[-1]
    d = None
    if draft_row is not None:
        d, dd = _logits(draft_row)
        assert dd == dt
    w = np.empty((V,), np.float64)
    S = lib.oracle_draw_weights(_ptr(t), _ptr(d), dt, V, float(temperature), _ptr(w))
    if S < 0:
        raise ValueError("oracle_draw_weights rejected its arguments")
    return w, S


def softmax_row(row, temperature, *, lib=None):
    lib = lib or load()
    r, dt = _logits(row)
    V = r.shape[-1]
    p = np.empty((V,), np.float64)
    if lib.oracle_softmax_row(_ptr(r), dt, V, float(temperature), _ptr(p)) != 0:
        raise ValueError("oracle_softmax_row rejected its arguments")
    return p


def residual_draw(p, q, u, *, lib=None):
    """Residual draw on given double distributions; returns (token, S)."""
    lib = lib or load()
    p = np.ascontiguousarray(p, np.float64)
    q = np.ascontiguousarray(q, np.float64)
    S = ctypes.c_double(0.0)
    tok = lib.oracle_residual_draw(_ptr(p), _ptr(q), p.shape[0], float(u), ctypes.byref(S))
    return tok, S.value


def acceptance_rate(target_row, draft_row, temperature, *, lib=None):
    """sum_i min(p_i, q_i) for one row pair."""
    lib = lib or load()
    t, dt = _logits(target_row)
    d, _ = _logits(draft_row)
    return lib.oracle_acceptance_rate(_ptr(t), _ptr(d), dt, t.shape[-1], float(temperature))


def row_argmax(row, *, lib=None):
    lib = lib or load()
    r, dt = _logits(row)
    return lib.oracle_row_argmax(_ptr(r), dt, r.shape[-1])


def verify_greedy(target, tokens, *, lib=None):
    """Greedy chain verify: target [B][K+1][V], tokens [B][K] -> (tokens [B][K+1], accepted [B])."""
    lib = lib or load()
    t, dt = _logits(target)
    B, K1, V = t.shape
    K = K1 - 1
    x = _i32(tokens).reshape(B, K)
    out_t = np.empty((B, K + 1), np.int32)
    out_a = np.empty((B,), np.int32)
    rc = lib.oracle_verify_greedy(_ptr(t), dt, _ptr(x), B, K, V, _ptr(out_t), _ptr(out_a))
    if rc != 0:
        raise ValueError(f"oracle_verify_greedy rejected its arguments (code {rc})")
    return out_t, out_a


def tree_max_depth(parents):
    parents = np.asarray(parents)
    depth = np.zeros(len(parents), np.int64)
    for v in range(1, len(parents)):
        depth[v] = depth[parents[v]] + 1
    return int(depth.max())


def verify_tree_greedy(node_logits, node_tokens, parents, *, lib=None):
    """Greedy static-tree verify -> (tokens [B][D+1], path [B][D+1], depth [B])."""
    lib = lib or load()
    t, dt = _logits(node_logits)
    B, N, V = t.shape
    par = _i32(parents).reshape(N)
    tok = _i32(node_tokens).reshape(B, N)
    D = tree_max_depth(par) if N > 1 else 0
    out_t = np.empty((B, D + 1), np.int32)
    out_p = np.empty((B, D + 1), np.int32)
    out_d = np.empty((B,), np.int32)
    rc = lib.oracle_verify_tree_greedy(_ptr(t), dt, _ptr(tok), _ptr(par), B, N, V,
                                       _ptr(out_t), _ptr(out_p), _ptr(out_d))
    if rc != 0:
        raise ValueError(f"oracle_verify_tree_greedy rejected its arguments (code {rc})")
    return out_t, out_p, out_d


def verify_tree_greedy_dyn(node_logits, node_tokens, parents, node_count, *, lib=None):
    """Greedy verify on per-sequence trees -> (tokens [B][Nmax], path [B][Nmax], depth [B])."""
    lib = lib or load()
    t, dt = _logits(node_logits)
    B, Nmax, V = t.shape
    tok = _i32(node_tokens).reshape(B, Nmax)
    par = _i32(parents).reshape(B, Nmax)
    cnt = _i32(node_count).reshape(B)
    out_t = np.empty((B, Nmax), np.int32)
    out_p = np.empty((B, Nmax), np.int32)
    out_d = np.empty((B,), np.int32)
    rc = lib.oracle_verify_tree_greedy_dyn(_ptr(t), dt, _ptr(tok), _ptr(par), _ptr(cnt), B, Nmax, V,
                                           _ptr(out_t), _ptr(out_p), _ptr(out_d))
    if rc != 0:
        raise ValueError(f"oracle_verify_tree_greedy_dyn rejected its arguments (code {rc})")
    return out_t, out_p, out_d


def topk(logits, k, *, lib=None):
    """Top-k of each row: (indices [rows][k], values [rows][k] float32), by value
    descending then index ascending."""
    lib = lib or load()
    t, dt = _logits(logits)
    V = t.shape[-1]
    t2 = t.reshape(-1, V)
    rows = t2.shape[0]
    out_i = np.empty((rows, k), np.int32)
    out_v = np.empty((rows, k), np.float32)
    rc = lib.oracle_topk(_ptr(t2), dt, rows, V, k, _ptr(out_i), _ptr(out_v))
    if rc != 0:
        raise ValueError(f"oracle_topk rejected its arguments (code {rc})")
    return out_i.reshape(t.shape[:-1] + (k,)), out_v.reshape(t.shape[:-1] + (k,))


def kv_commit(scratch, cache, path, count, length, *, lib=None):
    """KV commit: a copy of `cache` [planes][B][S][row] (uint8) with each
    sequence's accepted scratch rows (`scratch` [planes][B][N][row]) written at
    its slots length[b] .. length[b] + count[b] - 1, and the new lengths.
    `path` [B][P] int32 or None (row i).  Sequences whose arguments are out of
    range are left as they were."""
    lib = lib or load()
    scratch = np.ascontiguousarray(scratch, dtype=np.uint8)
    out = np.array(cache, dtype=np.uint8, copy=True, order="C")
    planes, B, N, row = scratch.shape
    assert out.shape[:2] == (planes, B) and out.shape[3] == row, "scratch and cache disagree"
    S = out.shape[2]
    count = np.ascontiguousarray(count, dtype=np.int32)
    length = np.ascontiguousarray(length, dtype=np.int32)
    new_len = np.empty(B, np.int32)
    if path is not None:
        path = np.ascontiguousarray(path, dtype=np.int32)
        P = path.shape[1]
    else:
        P = 0
    rc = lib.oracle_kv_commit(_ptr(scratch), _ptr(out), planes, B, N, S, row,
                              None if path is None else _ptr(path), P, _ptr(count), _ptr(length),
                              _ptr(new_len))
    if rc != 0:
        raise ValueError(f"oracle_kv_commit rejected its arguments (code {rc})")
    return out, new_len


def tree_mask(parents, node_count=None, *, lib=None):
    """Tree attention mask: (mask [B][N][ceil(N/32)] uint32 ancestor bits,
    depth [B][N] int32), per sequence from parents [B][N] (or one tree [N])
    and node_count [B] or None."""
    lib = lib or load()
    par = np.ascontiguousarray(parents, dtype=np.int32)
    if par.ndim == 1:
        par = par[None]
    B, N = par.shape
    W = (N + 31) // 32
    mask = np.empty((B, N, W), np.uint32)
    depth = np.empty((B, N), np.int32)
    cnt = None if node_count is None else np.ascontiguousarray(node_count, dtype=np.int32)
    rc = lib.oracle_tree_mask(_ptr(par), None if cnt is None else _ptr(cnt), B, N, _ptr(mask),
                              _ptr(depth))
    if rc != 0:
        raise ValueError(f"oracle_tree_mask rejected its arguments (code {rc})")
    return mask, depth
