"""CPU oracle of the CSA2 sparse-attention step (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
imports nothing from the HIP library: both sides read the same seeded bytes
from ``top_kv_selection_amd.workloads`` and nothing else.

The arithmetic lives in ``csa2_oracle.c`` (plain C, exact integers for the
selection, fp64 for attention).  This file only marshals numpy arrays, threads
the C loops over independent query ranges (ctypes releases the GIL), and applies
the layer-mode rules of the "CSA2 with cross-layer reuse" mode table on the
DeepSeek V4.1 Flash page (k-a.in): Full and Reindex layers compute fresh
indices with their own indexer query, Reuse layers take the indices of the most
recent Full/Reindex layer, and every layer has its own Q and window K/V.  A
token-only Reindex layer (the page's Reindex "recomputes only the Top-K"
reading) keeps the pool of the most recent index set and reselects the tokens
with its own indexer query.
Sliding-window-only layers (the page's first two encoder layers) attend to the
window alone.  With a compression ratio r (the page's CSA2(ratio, mode), whose
ratio it leaves undefined) the main-KV and indexer caches hold one entry per r
tokens, a query sees the entries complete at its token position, and its
window stays per token (``orc_visible_entries`` states the rule).  These sequencing rules are pinned by tests that recompute every
layer of small multi-layer workloads from scratch (selection by enumeration,
attention by fp64 SDPA over the gathered rows).
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        L.orc_round_half_even_div.restype = ctypes.c_int64
        L.orc_round_half_even_div.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.orc_block_key.restype = None
        L.orc_block_key.argtypes = [P, i32, i32, i32, i32, P]
        L.orc_select_one.restype = i32
        L.orc_select_one.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32, P, P, P, P]
        L.orc_select_batch.restype = i32
        L.orc_select_batch.argtypes = [i32, i32, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                       i32, P, P, P, P]
        L.orc_topk_batch.restype = i32
        L.orc_topk_batch.argtypes = [i32, i32, P, P, P, P, i32, i32, i32, i32, i32, i32, P, P, P, P]
        L.orc_visible_entries.restype = i32
        L.orc_visible_entries.argtypes = [i32, i32]
        L.orc_attend_batch.restype = i32
        L.orc_attend_batch.argtypes = [i32, i32, P, P, P, P, P, i32, i32, P, P, i32, i32,
                                       P, P, i32, i32, i32, i32, i32, ctypes.c_double, P, P]
        _lib = L
    return _lib


@contextlib.contextmanager
def using(path):
    """Temporarily load another build of the oracle (mutation tests build
    copies with a planted mistake and check that the pins catch it)."""
    global _lib, _LIB_PATH
    saved = (_lib, _LIB_PATH)
    _lib, _LIB_PATH = None, path
    try:
        yield lib()
    finally:
        _lib, _LIB_PATH = saved


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _elem_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"attention inputs must be float32 or uint16 (bf16 bits), got {a.dtype}")


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return os.cpu_count() or 1


def _parallel(n, threads, fn):
    """Run fn(begin, end) over [0, n) split into contiguous ranges; sum results."""
    threads = max(1, min(threads, n))
    if threads == 1:
        return fn(0, n)
    bounds = np.linspace(0, n, threads + 1).astype(int)
    with ThreadPoolExecutor(threads) as ex:
        return sum(ex.map(lambda ab: fn(*ab), zip(bounds[:-1], bounds[1:])))


# --------------------------------------------------------------------------
# Step 1: block keys (exposed for the pins)
# --------------------------------------------------------------------------
def round_half_even_div(total: int, n: int) -> int:
    return int(lib().orc_round_half_even_div(int(total), int(n)))


def block_key(k_seq: np.ndarray, B: int, j: int, t: int) -> np.ndarray:
    """Key of block j seen from position t (rounded mean of its visible rows)."""
    k_seq = np.ascontiguousarray(k_seq, dtype=np.int8)
    d = k_seq.shape[1]
    out = np.zeros(d, dtype=np.int8)
    lib().orc_block_key(_ptr(k_seq), d, B, j, t, _ptr(out))
    return out


# --------------------------------------------------------------------------
# Steps 2-5: block pool and token Top-K
# --------------------------------------------------------------------------
TAIL_VISIBLE, TAIL_EXCLUDE, TAIL_WHOLE = 0, 1, 2


def visible_entries(t: int, ratio: int) -> int:
    """Main-KV entries a query at token t sees when each entry compresses
    ``ratio`` consecutive tokens (complete entries only)."""
    return int(lib().orc_visible_entries(int(t), int(ratio)))


def select(q_idx, q_seq, q_pos, k_idx, B, P, K, threads=None, tail=TAIL_VISIBLE, ratio=1):
    """Per query: pooled blocks and Top-K positions (ascending, -1 padded).
    q_idx int8 [n_q][d]; k_idx int8 [S][T][d].  ``tail`` picks the reading of
    the query's partial own block (visible rows / excluded / whole block).
    ``ratio``: tokens per main-KV entry; q_pos holds token positions, k_idx
    one row per entry, and the ids returned are entry ids.
    Returns (blk_ids [n_q][P], blk_cnt [n_q], topk [n_q][K], topk_cnt [n_q])."""
    q_idx = np.ascontiguousarray(q_idx, dtype=np.int8)
    k_idx = np.ascontiguousarray(k_idx, dtype=np.int8)
    q_seq = np.ascontiguousarray(q_seq, dtype=np.int32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    n_q, d = q_idx.shape
    S, T, d2 = k_idx.shape
    assert d == d2
    blk_ids = np.empty((n_q, P), np.int32)
    blk_cnt = np.empty(n_q, np.int32)
    topk = np.empty((n_q, max(K, 1)), np.int32)[:, :K].copy()
    topk_cnt = np.empty(n_q, np.int32)
    L = lib()

    def run(a, b):
        return L.orc_select_batch(int(a), int(b), _ptr(q_idx), _ptr(q_seq), _ptr(q_pos),
                                  _ptr(k_idx), S, T, d, B, P, K, int(tail), int(ratio), _ptr(blk_ids), _ptr(blk_cnt),
                                  _ptr(topk), _ptr(topk_cnt))

    bad = _parallel(n_q, threads or default_threads(), run)
    if bad:
        raise ValueError(f"oracle select rejected {bad} queries")
    return blk_ids, blk_cnt, topk, topk_cnt


def topk_given_pool(q_idx, q_seq, q_pos, k_idx, B, K, blk_ids, blk_cnt, threads=None, ratio=1):
    """Step 5 alone over given pools: the Reindex variant that keeps the pool
    of the shared index set and reselects only the tokens with its own
    q_idx.  blk_ids [n_q][P] ascending, -1 padded; blk_cnt [n_q].
    Returns (topk [n_q][K], topk_cnt [n_q])."""
    q_idx = np.ascontiguousarray(q_idx, dtype=np.int8)
    k_idx = np.ascontiguousarray(k_idx, dtype=np.int8)
    q_seq = np.ascontiguousarray(q_seq, dtype=np.int32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    blk_ids = np.ascontiguousarray(blk_ids, dtype=np.int32)
    blk_cnt = np.ascontiguousarray(blk_cnt, dtype=np.int32)
    n_q, d = q_idx.shape
    S, T, d2 = k_idx.shape
    assert d == d2 and blk_ids.shape[0] == n_q
    P = blk_ids.shape[1]
    topk = np.empty((n_q, max(K, 1)), np.int32)[:, :K].copy()
    topk_cnt = np.empty(n_q, np.int32)
    L = lib()

    def run(a, b):
        return L.orc_topk_batch(int(a), int(b), _ptr(q_idx), _ptr(q_seq), _ptr(q_pos), _ptr(k_idx),
                                T, d, B, P, K, int(ratio), _ptr(blk_ids), _ptr(blk_cnt), _ptr(topk),
                                _ptr(topk_cnt))

    bad = _parallel(n_q, threads or default_threads(), run)
    if bad:
        raise ValueError(f"oracle token Top-K rejected {bad} queries")
    return topk, topk_cnt


# --------------------------------------------------------------------------
# Steps 6-7: window + attention
# --------------------------------------------------------------------------
def attend(q, q_seq, q_pos, k_main, v_main, k_swa, v_swa, swa_first, topk, topk_cnt,
           W, scale=None, threads=None):
    """One layer.  q [n_q][H][D]; k_main/v_main [S][T][D]; k_swa/v_swa
    [S][swa_len][D] (row r = position swa_first + r); topk [n_q][K] or None for a
    window-only layer.  Inputs are float32 or uint16 bf16 bits.
    Returns (out fp64 [n_q][H][D], lse fp64 [n_q][H])."""
    elem = _elem_of(q)
    for a in (k_main, v_main, k_swa, v_swa):
        assert _elem_of(a) == elem
    q, k_main, v_main, k_swa, v_swa = (np.ascontiguousarray(a) for a in (q, k_main, v_main, k_swa, v_swa))
    q_seq = np.ascontiguousarray(q_seq, dtype=np.int32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    n_q, H, D = q.shape
    S, T, _ = k_main.shape
    swa_len = k_swa.shape[1]
    if topk is not None:
        topk = np.ascontiguousarray(topk, dtype=np.int32)
        topk_cnt = np.ascontiguousarray(topk_cnt, dtype=np.int32)
        K_stride = topk.shape[1]
    else:
        K_stride = 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((n_q, H, D), np.float64)
    lse = np.empty((n_q, H), np.float64)
    L = lib()

    def run(a, b):
        return L.orc_attend_batch(int(a), int(b), _ptr(q), _ptr(q_seq), _ptr(q_pos), _ptr(k_main),
                                  _ptr(v_main), S, T, _ptr(k_swa), _ptr(v_swa), int(swa_first),
                                  swa_len, _ptr(topk), _ptr(topk_cnt), K_stride, W, H, D, elem,
                                  float(scale), _ptr(out), _ptr(lse))

    bad = _parallel(n_q, threads or default_threads(), run)
    if bad:
        raise ValueError(f"oracle attend rejected {bad} queries")
    return out, lse


# --------------------------------------------------------------------------
# Layer modes
# --------------------------------------------------------------------------
def run_layers(wl, rows=None, threads=None):
    """Run every layer of a workload in model order with the mode rules above.
    ``rows`` optionally restricts the computation to a subset of query rows
    (used to sample full-size workloads).  Returns a dict with per-layer
    ``out``/``lse`` (fp64) and per indexing layer ``blk_ids``/``blk_cnt``/
    ``topk``/``topk_cnt``."""
    cfg = wl.cfg
    idx = np.arange(cfg.n_q) if rows is None else np.asarray(rows)
    q_seq, q_pos = wl.q_seq[idx], wl.q_pos[idx]
    res = {"rows": idx, "index": {}, "out": [], "lse": []}
    current = None
    # every Full layer has its own main-KV and indexer cache, which the
    # layers after it share until the next Full layer (mode table of "CSA2
    # with cross-layer reuse": a Full layer computes its own keys, Reuse and
    # Reindex layers share them)
    n_full = 0
    for layer, mode in enumerate(cfg.layers):
        if mode == "full":
            n_full += 1
        k_idx, k_main, v_main = wl.cache(max(n_full - 1, 0))
        if mode in ("full", "reindex"):
            sel = select(wl.q_idx[layer][idx], q_seq, q_pos, k_idx, cfg.block, cfg.pool,
                         cfg.top_k, threads, cfg.tail, cfg.ratio)
            res["index"][layer] = dict(zip(("blk_ids", "blk_cnt", "topk", "topk_cnt"), sel))
            current = sel
        elif mode == "reindex_tokens":
            if current is None:
                raise ValueError("a token-only Reindex layer needs an earlier Full/Reindex layer")
            topk, cnt = topk_given_pool(wl.q_idx[layer][idx], q_seq, q_pos, k_idx, cfg.block,
                                        cfg.top_k, current[0], current[1], threads, cfg.ratio)
            sel = (current[0], current[1], topk, cnt)
            res["index"][layer] = dict(zip(("blk_ids", "blk_cnt", "topk", "topk_cnt"), sel))
            current = sel
        if mode == "swa":
            topk, cnt = None, None
        else:
            if current is None:
                raise ValueError("a Reuse layer needs an earlier Full/Reindex layer")
            topk, cnt = current[2], current[3]
        o, l = attend(wl.q[layer][idx], q_seq, q_pos, k_main, v_main, wl.k_swa[layer],
                      wl.v_swa[layer], cfg.swa_first, topk, cnt, cfg.window, None, threads)
        res["out"].append(o)
        res["lse"].append(l)
    return res
