"""Speculative-sampling verify step on MI355X (gfx950): Python binding.

Thin ctypes binding of ``libspecverify.so`` (declared in include/spec_verify.h)
with the same entry-point names.  It only marshals torch tensors into device
pointers and the current HIP stream; every step of the verify runs in the
library's HIP kernels.  PyTorch supplies device memory and streams.

The library must be built first (``__graft_entry__.build()``); importing this
package without it raises ImportError.  There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "spec_verify.h")

SPEC_DTYPE_F32, SPEC_DTYPE_BF16 = 0, 1
SPEC_MODE_CHAIN, SPEC_MODE_GREEDY, SPEC_MODE_TREE, SPEC_MODE_TREE_DYN, SPEC_MODE_TOPK = 0, 1, 2, 3, 4
SPEC_OK, SPEC_ERR_INVALID_ARG, SPEC_ERR_WORKSPACE, SPEC_ERR_LAUNCH = 0, 1, 2, 3
SPEC_ERR_SCRATCH_LIMIT = 4
NOALLOC_SCRATCH_BYTES = 8 << 20
MAX_K, MAX_TREE_NODES, MAX_V = 64, 256, 1 << 26
MAX_CHAIN_V_BF16, MAX_CHAIN_V_F32 = 1 << 19, 1 << 18
TOPK_MAX_K, TOPK_MAX_V = 8, 1 << 19


class SpecVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        text = _lib.spec_verify_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status} ({text})")


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.spec_verify_status_string.argtypes = [ctypes.c_int]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    lib.spec_verify_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32, ctypes.c_int,
                                                ctypes.POINTER(sz)]
    lib.spec_verify_chain.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, i32, i32, i32, f32,
                                      vp, vp, vp, vp, sz, vp]
    lib.spec_verify_chain_stats.argtypes = [vp, vp, ctypes.c_int, vp, i32, i32, i32, f32, vp, sz,
                                            vp]
    lib.spec_verify_chain_sample.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, i32, i32, i32,
                                             f32, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_greedy.argtypes = [vp, ctypes.c_int, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.spec_verify_tree_greedy.argtypes = [vp, ctypes.c_int, vp, vp, i32, i32, i32, vp, vp, vp,
                                            vp, sz, vp]
    lib.spec_verify_tree_greedy_dyn.argtypes = [vp, ctypes.c_int, vp, vp, vp, i32, i32, i32, vp, vp,
                                                vp, vp, sz, vp]
    lib.spec_draft_topk.argtypes = [vp, ctypes.c_int, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.spec_kv_commit.argtypes = [vp, vp, i32, i32, i32, i32, ctypes.c_int64, vp, i32, vp, vp, vp,
                                   vp]
    lib.spec_tree_mask.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    lib.spec_verify_workspace_failures.argtypes = [vp, sz, i32, ctypes.POINTER(ctypes.c_uint32), vp]
    lib.spec_verify_chain_noalloc.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, i32, i32, i32, f32,
                                              vp, vp, vp, vp]
    for fn in ("spec_verify_workspace_bytes", "spec_verify_chain", "spec_verify_chain_stats",
               "spec_verify_chain_sample", "spec_verify_greedy", "spec_verify_tree_greedy",
               "spec_verify_tree_greedy_dyn", "spec_draft_topk", "spec_kv_commit",
               "spec_tree_mask", "spec_verify_workspace_failures", "spec_verify_chain_noalloc"):
        getattr(lib, fn).restype = ctypes.c_int
    return lib


_lib = _load()


def header_symbols(path: str = HEADER_PATH) -> list[str]:
    """Entry points declared in the public header."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\S.*?\b(spec_(?:verify|draft|kv|tree)_\w+)\s*\(", text, flags=re.M)))


def library():
    return _lib


# ------------------------------------------------------------------ marshalling

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPEC_DTYPE_BF16
    if t.dtype == torch.float32:
        return SPEC_DTYPE_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _check_dev(name, t, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(device, stream):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _call(fn, *args):
    st = getattr(_lib, fn)(*args)
    if st != SPEC_OK:
        raise SpecVerifyError(fn, st)


def _enqueue(prepare, keep, fn, *args):
    """Calls entry point `fn` now, or with `prepare` returns a function that
    enqueues the same call again with no Python-side checks (for serving
    loops and graph capture).  The function holds the tensors in `keep` (every
    tensor of the call), so their storage outlives it; their contents may be
    rewritten in place between launches."""
    f = getattr(_lib, fn)

    def launch():
        st = f(*args)
        if st != SPEC_OK:
            raise SpecVerifyError(fn, st)
    launch.keep = keep
    if prepare:
        return launch
    launch()
    return None


def spec_verify_workspace_bytes(mode: int, B: int, K_or_N: int, V: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    _call("spec_verify_workspace_bytes", mode, B, K_or_N, V, dtype, ctypes.byref(out))
    return out.value


def workspace(mode: int, B: int, K_or_N: int, V: int, dtype: int, device) -> torch.Tensor:
    """A zero-filled device byte buffer large enough for one call.  Zeroed
    once, it can be reused for any later calls (their hand-over words carry
    per-call tags); a buffer with other prior contents must be zeroed first."""
    n = spec_verify_workspace_bytes(mode, B, K_or_N, V, dtype)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def workspace_failures(workspace_buf, *, reset=False, stream=None) -> int:
    """Bounded waits that ran out (and chain samples without statistics) since
    the workspace was zeroed or last reset; 0 means every output written
    through it is valid.  Synchronises the stream."""
    _check_dev("workspace_buf", workspace_buf, torch.uint8)
    out = ctypes.c_uint32(0)
    _call("spec_verify_workspace_failures", _ptr(workspace_buf), workspace_buf.numel(), int(bool(reset)),
          ctypes.byref(out), _stream(workspace_buf.device, stream))
    return out.value


def check_workspace(workspace_buf, *, stream=None) -> None:
    """Raises SpecVerifyError if any bounded wait ran out on this workspace."""
    n = workspace_failures(workspace_buf, stream=stream)
    if n:
        raise SpecVerifyError(f"workspace reports {n} failed wait(s);", SPEC_ERR_LAUNCH)


def _chain_check(target, draft, draft_tokens, u_accept, u_sample):
    _check_dev("target_logits", target)
    dt = _dtype_code(target)
    if target.dim() != 3:
        raise ValueError("target_logits must be [B][K+1][V]")
    B, K1, V = target.shape
    K = K1 - 1
    _check_dev("draft_logits", draft, target.dtype, (B, K, V))
    if draft_tokens is not None:
        _check_dev("draft_tokens", draft_tokens, torch.int32, (B, K))
        _check_dev("u_accept", u_accept, torch.float32, (B, K))
        _check_dev("u_sample", u_sample, torch.float32, (B,))
    return dt, B, K, V


def spec_verify_chain(target_logits, draft_logits, draft_tokens, u_accept, u_sample,
                      temperature: float, *, out_tokens=None, out_accepted=None, diag=False,
                      out_diag=None, workspace_buf=None, stream=None):
    """Chain verify at T > 0.  Returns (tokens [B][K+1], accepted [B], diag [B][K+1][4] or None)."""
    dt, B, K, V = _chain_check(target_logits, draft_logits, draft_tokens, u_accept, u_sample)
    dev = target_logits.device
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if out_accepted is None:
        out_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_diag is None and diag:
        out_diag = torch.empty((B, K + 1, 4), dtype=torch.float32, device=dev)
    if workspace_buf is None:
        workspace_buf = workspace(SPEC_MODE_CHAIN, B, K, V, dt, dev)
    _call("spec_verify_chain", _ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens),
          _ptr(u_accept), _ptr(u_sample), B, K, V, float(temperature), _ptr(out_tokens),
          _ptr(out_accepted), _ptr(out_diag), _ptr(workspace_buf), workspace_buf.numel(),
          _stream(dev, stream))
    return out_tokens, out_accepted, out_diag


def spec_verify_chain_noalloc(target_logits, draft_logits, draft_tokens, u_accept, u_sample,
                              temperature: float, *, out_tokens=None, out_accepted=None,
                              diag=False, out_diag=None, stream=None):
    """spec_verify_chain on the library's fixed device array instead of a
    workspace (the outputs are the caller's tensors, allocated here when not
    given).  Returns (tokens [B][K+1], accepted [B], diag or None)."""
    dt, B, K, V = _chain_check(target_logits, draft_logits, draft_tokens, u_accept, u_sample)
    dev = target_logits.device
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if out_accepted is None:
        out_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_diag is None and diag:
        out_diag = torch.empty((B, K + 1, 4), dtype=torch.float32, device=dev)
    _call("spec_verify_chain_noalloc", _ptr(target_logits), _ptr(draft_logits), dt,
          _ptr(draft_tokens), _ptr(u_accept), _ptr(u_sample), B, K, V, float(temperature),
          _ptr(out_tokens), _ptr(out_accepted), _ptr(out_diag), _stream(dev, stream))
    return out_tokens, out_accepted, out_diag


def spec_verify_chain_stats(target_logits, draft_logits, draft_tokens, temperature: float,
                            workspace_buf, *, stream=None, prepare=False):
    """First phase of the chain verify (softmax statistics of every row into the
    workspace).  With `prepare`, returns a function that enqueues the call again."""
    dt, B, K, V = _chain_check(target_logits, draft_logits, None, None, None)
    _check_dev("draft_tokens", draft_tokens, torch.int32, (B, K))
    dev = target_logits.device
    return _enqueue(prepare, (target_logits, draft_logits, draft_tokens, workspace_buf),
                    "spec_verify_chain_stats", _ptr(target_logits), _ptr(draft_logits), dt,
                    _ptr(draft_tokens), B, K, V, ctypes.c_float(float(temperature)),
                    _ptr(workspace_buf), ctypes.c_size_t(workspace_buf.numel()), _stream(dev, stream))


def spec_verify_chain_sample(target_logits, draft_logits, draft_tokens, u_accept, u_sample,
                             temperature: float, workspace_buf, *, out_tokens=None,
                             out_accepted=None, out_diag=None, stream=None):
    """Second phase of the chain verify; follows spec_verify_chain_stats on the same workspace."""
    dt, B, K, V = _chain_check(target_logits, draft_logits, draft_tokens, u_accept, u_sample)
    dev = target_logits.device
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if out_accepted is None:
        out_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    _call("spec_verify_chain_sample", _ptr(target_logits), _ptr(draft_logits), dt,
          _ptr(draft_tokens), _ptr(u_accept), _ptr(u_sample), B, K, V, float(temperature),
          _ptr(out_tokens), _ptr(out_accepted), _ptr(out_diag), _ptr(workspace_buf),
          workspace_buf.numel(), _stream(dev, stream))
    return out_tokens, out_accepted


def prepare_chain(target_logits, draft_logits, draft_tokens, u_accept, u_sample,
                  temperature: float, out_tokens, out_accepted, workspace_buf, *, out_diag=None,
                  stream=None):
    """Checks and marshals the arguments of one spec_verify_chain call once and
    returns a function that enqueues it again with no Python-side work (for
    serving loops and graph capture).  The function holds every tensor of the
    call; their contents may be rewritten in place between launches."""
    dt, B, K, V = _chain_check(target_logits, draft_logits, draft_tokens, u_accept, u_sample)
    dev = target_logits.device
    _check_dev("out_tokens", out_tokens, torch.int32, (B, K + 1))
    _check_dev("out_accepted", out_accepted, torch.int32, (B,))
    if out_diag is not None:
        _check_dev("out_diag", out_diag, torch.float32, (B, K + 1, 4))
    need = spec_verify_workspace_bytes(SPEC_MODE_CHAIN, B, K, V, dt)
    if workspace_buf.numel() < need:
        raise SpecVerifyError("spec_verify_chain", SPEC_ERR_WORKSPACE)
    fn = _lib.spec_verify_chain
    args = (_ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens), _ptr(u_accept),
            _ptr(u_sample), B, K, V, ctypes.c_float(float(temperature)), _ptr(out_tokens),
            _ptr(out_accepted), _ptr(out_diag), _ptr(workspace_buf),
            ctypes.c_size_t(workspace_buf.numel()), _stream(dev, stream))

    def launch():
        st = fn(*args)
        if st != SPEC_OK:
            raise SpecVerifyError("spec_verify_chain", st)
    launch.keep = (target_logits, draft_logits, draft_tokens, u_accept, u_sample, out_tokens,
                   out_accepted, out_diag, workspace_buf)
    return launch


def spec_verify_greedy(target_logits, draft_tokens, *, out_tokens=None, out_accepted=None,
                       workspace_buf=None, stream=None, prepare=False):
    """Greedy chain verify (T = 0).  Returns (tokens [B][K+1], accepted [B]);
    with `prepare`, (launch, (tokens, accepted)) and nothing is enqueued."""
    _check_dev("target_logits", target_logits)
    dt = _dtype_code(target_logits)
    B, K1, V = target_logits.shape
    K = K1 - 1
    _check_dev("draft_tokens", draft_tokens, torch.int32, (B, K))
    dev = target_logits.device
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if out_accepted is None:
        out_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if workspace_buf is None:
        workspace_buf = workspace(SPEC_MODE_GREEDY, B, K, V, dt, dev)
    launch = _enqueue(prepare, (target_logits, draft_tokens, out_tokens, out_accepted, workspace_buf),
                      "spec_verify_greedy",
                      _ptr(target_logits), dt, _ptr(draft_tokens), B, K, V, _ptr(out_tokens),
                      _ptr(out_accepted), _ptr(workspace_buf), workspace_buf.numel(),
                      _stream(dev, stream))
    return (launch, (out_tokens, out_accepted)) if prepare else (out_tokens, out_accepted)


def tree_max_depth(parents) -> int:
    depth = [0] * len(parents)
    for v in range(1, len(parents)):
        depth[v] = depth[int(parents[v])] + 1
    return max(depth)


def spec_verify_tree_greedy(node_logits, node_tokens, parents, *, with_path=True,
                            out_tokens=None, out_path=None, out_depth=None, workspace_buf=None,
                            stream=None, prepare=False):
    """Greedy static-tree verify (T = 0).  `parents` is a host sequence of N ints.
    Returns (tokens [B][D+1], path [B][D+1] or None, depth [B]); with
    `prepare`, (launch, outputs) and nothing is enqueued."""
    _check_dev("node_logits", node_logits)
    dt = _dtype_code(node_logits)
    B, N, V = node_logits.shape
    _check_dev("node_tokens", node_tokens, torch.int32, (B, N))
    if len(parents) != N:
        raise ValueError("parents must have N entries")
    par = (ctypes.c_int32 * N)(*[int(p) for p in parents])
    D = tree_max_depth(parents) if N > 1 else 0
    dev = node_logits.device
    if out_tokens is None:
        out_tokens = torch.empty((B, D + 1), dtype=torch.int32, device=dev)
    if out_path is None and with_path:
        out_path = torch.empty((B, D + 1), dtype=torch.int32, device=dev)
    if out_depth is None:
        out_depth = torch.empty((B,), dtype=torch.int32, device=dev)
    if workspace_buf is None:
        workspace_buf = workspace(SPEC_MODE_TREE, B, N, V, dt, dev)
    launch = _enqueue(prepare, (node_logits, node_tokens, out_tokens, out_path, out_depth,
                                workspace_buf), "spec_verify_tree_greedy", _ptr(node_logits), dt, _ptr(node_tokens),
                      par, B, N, V, _ptr(out_tokens), _ptr(out_path), _ptr(out_depth),
                      _ptr(workspace_buf), workspace_buf.numel(), _stream(dev, stream))
    outs = (out_tokens, out_path, out_depth)
    return (launch, outs) if prepare else outs


def spec_verify_tree_greedy_dyn(node_logits, node_tokens, parents, node_count, *, with_path=True,
                                out_tokens=None, out_path=None, out_depth=None, workspace_buf=None,
                                stream=None, prepare=False):
    """Greedy verify on per-sequence trees (T = 0).  `parents` [B][Nmax] and
    `node_count` [B] are int32 device tensors.  Returns (tokens [B][Nmax],
    path [B][Nmax] or None, depth [B]), rows padded with -1; with `prepare`,
    (launch, outputs) and nothing is enqueued."""
    _check_dev("node_logits", node_logits)
    dt = _dtype_code(node_logits)
    B, Nmax, V = node_logits.shape
    _check_dev("node_tokens", node_tokens, torch.int32, (B, Nmax))
    _check_dev("parents", parents, torch.int32, (B, Nmax))
    _check_dev("node_count", node_count, torch.int32, (B,))
    dev = node_logits.device
    if out_tokens is None:
        out_tokens = torch.empty((B, Nmax), dtype=torch.int32, device=dev)
    if out_path is None and with_path:
        out_path = torch.empty((B, Nmax), dtype=torch.int32, device=dev)
    if out_depth is None:
        out_depth = torch.empty((B,), dtype=torch.int32, device=dev)
    if workspace_buf is None:
        workspace_buf = workspace(SPEC_MODE_TREE_DYN, B, Nmax, V, dt, dev)
    launch = _enqueue(prepare, (node_logits, node_tokens, parents, node_count, out_tokens, out_path,
                                out_depth, workspace_buf), "spec_verify_tree_greedy_dyn", _ptr(node_logits), dt,
                      _ptr(node_tokens), _ptr(parents), _ptr(node_count), B, Nmax, V,
                      _ptr(out_tokens), _ptr(out_path), _ptr(out_depth), _ptr(workspace_buf),
                      workspace_buf.numel(), _stream(dev, stream))
    outs = (out_tokens, out_path, out_depth)
    return (launch, outs) if prepare else outs


def spec_draft_topk(logits, k, *, with_values=True, out_idx=None, out_val=None, workspace_buf=None,
                    stream=None, prepare=False):
    """Per-row top-k of draft logits [..., V] (bf16 or fp32): the k largest by
    value descending, equal values by index ascending.  Returns (idx [..., k]
    int32, values [..., k] float32 or None); with `prepare`, (launch,
    outputs) and nothing is enqueued."""
    _check_dev("logits", logits)
    dt = _dtype_code(logits)
    if logits.dim() < 1:
        raise ValueError("logits must have a vocabulary dimension")
    lead, V = tuple(logits.shape[:-1]), logits.shape[-1]
    rows = 1
    for d in lead:
        rows *= d
    dev = logits.device
    if out_idx is None:
        out_idx = torch.empty(lead + (k,), dtype=torch.int32, device=dev)
    else:
        _check_dev("out_idx", out_idx, torch.int32, lead + (k,))
    if out_val is None and with_values:
        out_val = torch.empty(lead + (k,), dtype=torch.float32, device=dev)
    elif out_val is not None:
        _check_dev("out_val", out_val, torch.float32, lead + (k,))
    if workspace_buf is None:
        workspace_buf = workspace(SPEC_MODE_TOPK, rows, k, V, dt, dev)
    launch = _enqueue(prepare, (logits, out_idx, out_val, workspace_buf), "spec_draft_topk", _ptr(logits),
                      dt, rows, V, k, _ptr(out_idx), _ptr(out_val), _ptr(workspace_buf),
                      workspace_buf.numel(), _stream(dev, stream))
    return (launch, (out_idx, out_val)) if prepare else (out_idx, out_val)


def spec_kv_commit(scratch, cache, count, cache_len, *, path=None, new_len=None, stream=None,
                   prepare=False):
    """KV commit after verify: for each sequence b, scratch rows path[b][i]
    (row i when `path` is None), i < count[b], are copied to cache slots
    cache_len[b] + i of every plane.  `scratch` is [planes][B][N][...] and
    `cache` [planes][B][S][...], same dtype and row shape, contiguous device
    tensors; `path` int32 [B][P] or None; `count` and `cache_len` int32 [B].
    Returns new_len (int32 [B]); with `prepare`, (launch, new_len) and nothing
    is enqueued."""
    _check_dev("scratch", scratch)
    _check_dev("cache", cache, scratch.dtype)
    if scratch.dim() < 4 or cache.dim() != scratch.dim():
        raise ValueError("scratch and cache must be [planes][B][rows][...] with the same row shape")
    planes, B, N = scratch.shape[:3]
    S = cache.shape[2]
    if tuple(cache.shape[:2]) != (planes, B) or tuple(cache.shape[3:]) != tuple(scratch.shape[3:]):
        raise ValueError(f"cache {tuple(cache.shape)} does not match scratch {tuple(scratch.shape)}")
    row_bytes = scratch.element_size()
    for d in scratch.shape[3:]:
        row_bytes *= d
    _check_dev("count", count, torch.int32, (B,))
    _check_dev("cache_len", cache_len, torch.int32, (B,))
    P = N
    if path is not None:
        _check_dev("path", path, torch.int32)
        if path.dim() != 2 or path.shape[0] != B:
            raise ValueError("path must be [B][P]")
        P = path.shape[1]
    dev = scratch.device
    if new_len is None:
        new_len = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        _check_dev("new_len", new_len, torch.int32, (B,))
    launch = _enqueue(prepare, (scratch, cache, path, count, cache_len, new_len), "spec_kv_commit",
                      _ptr(scratch), _ptr(cache), planes, B, N, S, row_bytes, _ptr(path), P,
                      _ptr(count), _ptr(cache_len), _ptr(new_len), _stream(dev, stream))
    return (launch, new_len) if prepare else new_len


def spec_tree_mask(parents, node_count=None, *, mask=None, depth=None, stream=None, prepare=False):
    """Tree attention mask: parents int32 [B][N] (device), node_count int32
    [B] or None.  Returns (mask uint32-as-int32 [B][N][ceil(N/32)], depth
    int32 [B][N]); bit j % 32 of word j / 32 of row v is set iff node v
    attends to node j.  With `prepare`, (launch, outputs)."""
    _check_dev("parents", parents, torch.int32)
    if parents.dim() != 2:
        raise ValueError("parents must be [B][N]")
    B, N = parents.shape
    W = (N + 31) // 32
    if node_count is not None:
        _check_dev("node_count", node_count, torch.int32, (B,))
    dev = parents.device
    if mask is None:
        mask = torch.empty((B, N, W), dtype=torch.int32, device=dev)   # uint32 bits
    else:
        _check_dev("mask", mask, torch.int32, (B, N, W))
    if depth is None:
        depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    else:
        _check_dev("depth", depth, torch.int32, (B, N))
    launch = _enqueue(prepare, (parents, node_count, mask, depth), "spec_tree_mask", _ptr(parents),
                      _ptr(node_count), B, N, _ptr(mask), _ptr(depth), _stream(dev, stream))
    return (launch, (mask, depth)) if prepare else (mask, depth)
