"""Parity rules between the GPU library's outputs and the fp64 oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU-baseline leg).

Chain verify (T > 0):
  - accepted lengths and emitted tokens match exactly, with two allowances:
    * an accept decision at position k may differ only if the oracle's
      |u_k - p_k(x_k)/q_k(x_k)| <= 1e-6; the rest of that sequence is then not
      compared;
    * a drawn token may differ only if the oracle's threshold u*S lies within
      1e-5*S of the running sums that separate the two tokens (the end of the
      lower token's interval and the start of the higher one's), and the GPU's
      token has positive weight;
  - p_k(x_k) and q_k(x_k) agree to 1e-5 relative, plus an absolute floor of
    2^-126 (about 1.2e-38), the smallest normal fp32 number: below it the
    GPU's fp32 probabilities are subnormal or flushed to zero, so no relative
    match is possible there;
  - the drawn mass S (a diagnostic) agrees to 1e-5 relative plus 2^-18 times
    M, the mass of p and q on the residual's support (sum of p_i + q_i over
    i with p_i > q_i, at most 2).  Each fp32 weight p_i (and q_i) carries a
    relative error of about eps (ln2 |a_i| + 3), a_i its exponent argument
    (eps = 2^-24), so S = sum max(0, p_i - q_i) is off by up to that much of
    M, however small S is: 2^-18 = 64 eps covers |a_i| up to about 88 (every
    weight above 2^-88).  When p and q nearly coincide (S << M) this bound,
    not the relative one, is the binding one.
Greedy chain and tree verify: every output matches exactly.
"""
from __future__ import annotations

from collections import Counter

import numpy as np

from . import (draw_weights, softmax_row, topk, verify_chain, verify_greedy, verify_tree_greedy,
               verify_tree_greedy_dyn)

REL = 1e-5
RATIO_BAND = 1e-6
CDF_BAND = 1e-5
ABS_FLOOR = float(np.finfo(np.float32).tiny)   # 2^-126
S_MASS_REL = 2.0 ** -18


def _close(g, o, rel=REL):
    return abs(float(g) - float(o)) <= rel * abs(float(o)) + ABS_FLOOR


def check_chain(inp: dict, gpu_tokens, gpu_accepted, gpu_diag=None, seqs=None) -> Counter:
    """Compare one chain verify step on sequences `seqs` (all by default).

    inp: the numpy inputs (target, draft, tokens, u_accept, u_sample, T).
    Raises AssertionError listing every violation; returns counts of exact
    sequences and of each allowance used."""
    B = inp["target"].shape[0]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    t, d = inp["target"][seqs], inp["draft"][seqs]
    x, ua, us = inp["tokens"][seqs], inp["u_accept"][seqs], inp["u_sample"][seqs]
    T = inp["T"]
    o_tok, o_acc, o_diag = verify_chain(t, d, x, ua, us, T, diag=True)
    g_tok, g_acc = np.asarray(gpu_tokens)[seqs], np.asarray(gpu_accepted)[seqs]
    g_diag = None if gpu_diag is None else np.asarray(gpu_diag)[seqs]
    K = x.shape[1]
    bad, n = [], Counter()
    for i, b in enumerate(seqs):
        if g_diag is not None:
            for k in range(K):
                for c, name in ((0, "P"), (1, "Q")):
                    if not _close(g_diag[i, k, c], o_diag[i, k, c]):
                        bad.append(f"seq {b} pos {k}: {name} gpu {g_diag[i, k, c]!r} oracle {o_diag[i, k, c]!r}")
        jg, jo = int(g_acc[i]), int(o_acc[i])
        if jg != jo:
            k = min(jg, jo)
            gap = abs(float(ua[i, k]) - float(o_diag[i, k, 2]))
            if gap <= RATIO_BAND:
                n["accept_band"] += 1
            else:
                bad.append(f"seq {b}: accepted gpu {jg} oracle {jo}, |u - ratio| = {gap:.3g}")
            continue
        j = jo
        if not np.array_equal(g_tok[i, :j], o_tok[i, :j]) or np.any(g_tok[i, j + 1:] != -1):
            bad.append(f"seq {b}: tokens gpu {g_tok[i].tolist()} oracle {o_tok[i].tolist()}")
            continue
        S_o = o_diag[i, j, 3]
        if g_diag is not None and not _close(g_diag[i, j, 3], S_o):
            M = _support_mass(t[i, j], d[i, j] if j < K else None, T)
            if abs(float(g_diag[i, j, 3]) - float(S_o)) > REL * abs(float(S_o)) + S_MASS_REL * M + ABS_FLOOR:
                bad.append(f"seq {b}: S gpu {g_diag[i, j, 3]!r} oracle {S_o!r} (support mass {M:.4g})")
            else:
                n["S_mass_band"] += 1
        tg, to = int(g_tok[i, j]), int(o_tok[i, j])
        if tg == to:
            n["exact"] += 1
            continue
        w, S = draw_weights(t[i, j], d[i, j] if j < K else None, T)
        if S == 0.0:          # the oracle fell back to p_j
            w, S = draw_weights(t[i, j], None, T)
        C = np.cumsum(w)
        tau = float(us[i]) * S
        lo, hi = min(tg, to), max(tg, to)
        ok = (0 <= tg < len(w) and w[tg] > 0 and abs(tau - C[lo]) <= CDF_BAND * S
              and abs(tau - C[hi - 1]) <= CDF_BAND * S)
        if ok:
            n["cdf_band"] += 1
        else:
            bad.append(f"seq {b}: drawn token gpu {tg} oracle {to}, tau {tau!r}, "
                       f"C[lo] {C[lo]!r}, C[hi-1] {C[hi - 1]!r}, S {S!r}")
    n["sequences"] = len(seqs)
    assert not bad, "chain parity violations:\n" + "\n".join(bad[:20])
    return n


def _support_mass(target_row, draft_row, T) -> float:
    """M of the S rule: the mass of p and q where p > q (of p alone for the
    bonus draw, where S sums p)."""
    p = softmax_row(target_row, T)
    if draft_row is None:
        return float(p.sum())
    q = softmax_row(draft_row, T)
    return float((p + q)[p > q].sum())


def check_greedy(inp: dict, gpu_tokens, gpu_accepted, seqs=None) -> Counter:
    B = inp["target"].shape[0]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    o_tok, o_acc = verify_greedy(inp["target"][seqs], inp["tokens"][seqs])
    g_tok, g_acc = np.asarray(gpu_tokens)[seqs], np.asarray(gpu_accepted)[seqs]
    bad = [f"seq {b}: gpu {g_tok[i].tolist()} / {g_acc[i]} oracle {o_tok[i].tolist()} / {o_acc[i]}"
           for i, b in enumerate(seqs)
           if g_acc[i] != o_acc[i] or not np.array_equal(g_tok[i], o_tok[i])]
    assert not bad, "greedy parity violations:\n" + "\n".join(bad[:20])
    return Counter(sequences=len(seqs), exact=len(seqs))


def check_tree(inp: dict, gpu_tokens, gpu_path, gpu_depth, seqs=None) -> Counter:
    B = inp["node_logits"].shape[0]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    o_tok, o_path, o_depth = verify_tree_greedy(inp["node_logits"][seqs], inp["node_tokens"][seqs],
                                                inp["parents"])
    g_tok, g_depth = np.asarray(gpu_tokens)[seqs], np.asarray(gpu_depth)[seqs]
    g_path = None if gpu_path is None else np.asarray(gpu_path)[seqs]
    bad = []
    for i, b in enumerate(seqs):
        same = g_depth[i] == o_depth[i] and np.array_equal(g_tok[i], o_tok[i])
        if g_path is not None:
            same = same and np.array_equal(g_path[i], o_path[i])
        if not same:
            bad.append(f"seq {b}: gpu {g_tok[i].tolist()} depth {g_depth[i]} "
                       f"oracle {o_tok[i].tolist()} depth {o_depth[i]}")
    assert not bad, "tree parity violations:\n" + "\n".join(bad[:20])
    return Counter(sequences=len(seqs), exact=len(seqs))


def check_tree_dyn(inp: dict, gpu_tokens, gpu_path, gpu_depth, seqs=None) -> Counter:
    """Per-sequence trees: depth, tokens and path exactly equal to the oracle's
    (argmax ties go to the lowest index, so the result is unique)."""
    B = inp["node_logits"].shape[0]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    o_tok, o_path, o_depth = verify_tree_greedy_dyn(inp["node_logits"][seqs], inp["node_tokens"][seqs],
                                                    inp["parents"][seqs], inp["node_count"][seqs])
    g_tok, g_depth = np.asarray(gpu_tokens)[seqs], np.asarray(gpu_depth)[seqs]
    g_path = None if gpu_path is None else np.asarray(gpu_path)[seqs]
    bad = []
    for i, b in enumerate(seqs):
        same = g_depth[i] == o_depth[i] and np.array_equal(g_tok[i], o_tok[i])
        if g_path is not None:
            same = same and np.array_equal(g_path[i], o_path[i])
        if not same:
            bad.append(f"seq {b}: gpu {g_tok[i].tolist()} depth {g_depth[i]} "
                       f"oracle {o_tok[i].tolist()} depth {o_depth[i]}")
    assert not bad, "per-sequence tree parity violations:\n" + "\n".join(bad[:20])
    return Counter(sequences=len(seqs), exact=len(seqs))


def check_topk(inp: dict, gpu_idx, gpu_val=None, rows=None) -> Counter:
    """Top-k: indices exactly equal to the oracle's (the order by value, then
    index, is total, so the result is unique) and values equal to the logits
    at those indices, bit for bit as float32."""
    x = inp["logits"]
    V = x.shape[-1]
    x2 = x.reshape(-1, V)
    gi = np.asarray(gpu_idx).reshape(x2.shape[0], -1)
    k = gi.shape[1]
    rows = np.arange(x2.shape[0]) if rows is None else np.asarray(rows)
    o_idx, o_val = topk(x2[rows], k)
    bad = [f"row {r}: gpu {gi[r].tolist()} oracle {o_idx[i].tolist()}"
           for i, r in enumerate(rows) if not np.array_equal(gi[r], o_idx[i])]
    assert not bad, "top-k index parity violations:\n" + "\n".join(bad[:20])
    if gpu_val is not None:
        gv = np.asarray(gpu_val, np.float32).reshape(x2.shape[0], -1)[rows]
        assert np.array_equal(gv.view(np.uint32), o_val.view(np.uint32)), \
            "top-k values differ from the oracle's"
    return Counter(rows=len(rows), exact=len(rows))
