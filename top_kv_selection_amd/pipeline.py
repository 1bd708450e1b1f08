"""Runs a workload's CSA2 layers on the GPU through the C ABI.

Host-side plumbing only: device buffers come from torch, and each layer group
(an indexing or window-only layer plus the Reuse layers that share its indices)
is one ``csa2_layer_group`` call, issued in model order on the current stream.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import binding as B
from .workloads import Config, Workload, query_rows


def _dev(a: np.ndarray, device, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def _real(a: np.ndarray, cfg: Config, device):
    return _dev(a, device, torch.bfloat16 if cfg.dtype == "bf16" else None)


@dataclass
class Group:
    mode: str
    layers: list
    q: torch.Tensor                 # [L][n_q][H][D]
    k_swa: torch.Tensor             # [L][S][swa_len][D]
    v_swa: torch.Tensor
    out: torch.Tensor               # [L][n_q][H][D]
    lse: torch.Tensor               # [L][n_q][H]
    q_idx: torch.Tensor = None      # [n_q][d] for full/reindex/reindex_tokens
    index_of: int = -1              # group whose indices a reuse group takes
    pool_of: int = -1               # group whose pool a token-only Reindex group reads
    cache: int = 0                  # main-KV + indexer cache (one per Full layer)


@dataclass
class DeviceWorkload:
    cfg: Config
    lcfg: B.Cfg
    q_seq: torch.Tensor
    q_pos: torch.Tensor
    k_idx: torch.Tensor
    k_blk: torch.Tensor
    k_main: torch.Tensor
    v_main: torch.Tensor
    groups: list
    # caches of the second, third, ... Full layer: (k_idx, k_blk, k_main, v_main)
    extra: list = field(default_factory=list)
    # one index set per indexing group
    blk_ids: dict = field(default_factory=dict)
    blk_cnt: dict = field(default_factory=dict)
    topk: dict = field(default_factory=dict)
    topk_cnt: dict = field(default_factory=dict)
    ws: torch.Tensor = None


def whole_prefix_pools(cfg: Config) -> bool:
    """Every query's pool is all of its eligible blocks (the longest context
    has at most P blocks): the library then needs no stored pool ids."""
    return (cfg.main_len - 1) // cfg.block + 1 <= cfg.pool


def group_caches(cfg: Config) -> list:
    """Cache of each layer group: a Full layer opens its own main-KV and
    indexer cache, and the groups after it share that cache until the next
    Full layer (groups before the first Full layer use cache 0)."""
    out, n_full = [], 0
    for mode, _ in cfg.groups():
        n_full += mode == "full"
        out.append(max(n_full - 1, 0))
    return out


def cache(dw: DeviceWorkload, c: int):
    """(k_idx, k_blk, k_main, v_main) of cache c (0: the first Full layer's)."""
    return (dw.k_idx, dw.k_blk, dw.k_main, dw.v_main) if c == 0 else dw.extra[c - 1]


def upload(wl: Workload, device="cuda", q_idx=None, q=None) -> DeviceWorkload:
    """Copies a workload to the GPU, grouping per-layer tensors by layer group.
    ``q_idx``/``q`` optionally replace the workload's queries (fresh replicas)."""
    cfg = wl.cfg
    q_idx = wl.q_idx if q_idx is None else q_idx
    q = wl.q if q is None else q
    lcfg = B.cfg_of(cfg)
    S, T, d = wl.k_idx.shape
    k_idx = _dev(wl.k_idx, device)
    dw = DeviceWorkload(cfg, lcfg, _dev(wl.q_seq, device), _dev(wl.q_pos, device), k_idx,
                        torch.zeros((S, T // cfg.block, d), dtype=torch.int8, device=device),
                        _real(wl.k_main, cfg, device), _real(wl.v_main, cfg, device), [])
    for c in range(1, cfg.n_caches):
        ki, km, vm = wl.cache(c)
        dw.extra.append((_dev(ki, device), torch.zeros((S, T // cfg.block, d), dtype=torch.int8, device=device),
                         _real(km, cfg, device), _real(vm, cfg, device)))
    tdt = lcfg.torch_dtype
    caches = group_caches(cfg)
    for mode, layers in cfg.groups():
        grp = Group(mode, layers,
                    _real(np.stack([q[l] for l in layers]), cfg, device),
                    _real(np.stack([wl.k_swa[l] for l in layers]), cfg, device),
                    _real(np.stack([wl.v_swa[l] for l in layers]), cfg, device),
                    torch.empty((len(layers), cfg.n_q, cfg.n_heads, cfg.head_dim), dtype=tdt, device=device),
                    torch.empty((len(layers), cfg.n_q, cfg.n_heads), dtype=torch.float32, device=device))
        grp.cache = caches[len(dw.groups)]
        if mode in ("full", "reindex", "reindex_tokens"):
            grp.q_idx = _dev(q_idx[layers[0]], device)
            g = len(dw.groups)
            if mode != "reindex_tokens":   # a token-only Reindex group reads the shared pool
                # when every pool is the whole prefix the count describes it
                # and no ids are stored
                dw.blk_ids[g] = None if whole_prefix_pools(cfg) else \
                    torch.empty((cfg.n_q, cfg.pool), dtype=torch.int32, device=device)
                dw.blk_cnt[g] = torch.empty(cfg.n_q, dtype=torch.int32, device=device)
            dw.topk[g] = torch.empty((cfg.n_q, cfg.top_k), dtype=torch.int32, device=device)
            dw.topk_cnt[g] = torch.empty(cfg.n_q, dtype=torch.int32, device=device)
        dw.groups.append(grp)
    last = -1
    for g, grp in enumerate(dw.groups):
        if grp.mode == "reindex_tokens":
            if last < 0:
                raise ValueError("a token-only Reindex layer needs an earlier Full/Reindex layer")
            # the pool of the most recent index set (a token-only group passes its own on)
            grp.pool_of = last if dw.groups[last].mode != "reindex_tokens" else dw.groups[last].pool_of
        if grp.mode in ("full", "reindex", "reindex_tokens"):
            last = g
        grp.index_of = last if grp.mode != "swa" else -1
    max_layers = max(len(g.layers) for g in dw.groups)
    dw.ws = B.new_workspace(lcfg, cfg.n_q, T, max_layers, device)
    return dw


def build_cache(dw: DeviceWorkload, upto_block=None):
    """Block keys of every complete block of every cache (the state of the
    caches before a step)."""
    T = dw.k_idx.shape[1]
    end = T // dw.cfg.block if upto_block is None else upto_block
    for c in range(dw.cfg.n_caches):
        k_idx, k_blk, _, _ = cache(dw, c)
        B.csa2_build_block_keys(dw.lcfg, k_idx, k_blk, 0, end)


def step_update_begin(dw: DeviceWorkload) -> int:
    """First block a Full layer rebuilds in bulk inside a step.  None in
    decode (earlier steps left every other block's key current, and the block
    pass stores the block the newest token completes) and in prompts whose
    every position is a query and whose pools are whole prefixes (the block
    pass then reads no block key, and stores the key of every block a query
    completes, i.e. every complete block).  Otherwise every block, before the
    block pass reads them."""
    T = dw.k_idx.shape[1]
    cfg = dw.cfg
    if cfg.decode or (cfg.replay == 0 and whole_prefix_pools(cfg)):
        return T // cfg.block
    return 0


def run(dw: DeviceWorkload, single: bool = False):
    """One pass of every layer group, in model order.  ``single``: Full and
    Reindex groups go through csa2_layer_group_single (one launch each)."""
    begin = step_update_begin(dw)
    for g, grp in enumerate(dw.groups):
        src = grp.index_of
        idx = src if src >= 0 else None
        pool = grp.pool_of if grp.mode == "reindex_tokens" else idx
        k_idx, k_blk, k_main, v_main = cache(dw, grp.cache)
        B.csa2_layer_group(
            dw.lcfg, grp.mode, grp.q_idx, dw.q_seq, dw.q_pos, k_idx, k_blk, begin, grp.q,
            k_main, v_main, grp.k_swa, grp.v_swa, dw.cfg.swa_first,
            dw.blk_ids.get(pool), dw.blk_cnt.get(pool), dw.topk.get(idx), dw.topk_cnt.get(idx),
            grp.out, grp.lse, dw.ws, single=single and grp.mode in ("full", "reindex"))


def outputs(dw: DeviceWorkload):
    """Host copies: per layer (out fp32, lse) and per indexing layer the index set."""
    n_layers = dw.cfg.n_layers
    out, lse = [None] * n_layers, [None] * n_layers
    index = {}
    for g, grp in enumerate(dw.groups):
        o = grp.out.float().cpu().numpy()
        l = grp.lse.cpu().numpy()
        for j, layer in enumerate(grp.layers):
            out[layer], lse[layer] = o[j], l[j]
        if g in dw.topk:
            pg = grp.pool_of if grp.mode == "reindex_tokens" else g
            cnt = dw.blk_cnt[pg].cpu().numpy()
            if dw.blk_ids[pg] is None:     # unstored: pool slot r holds block r
                slots = np.arange(dw.cfg.pool, dtype=np.int32)
                ids = np.where(slots[None, :] < cnt[:, None], slots[None, :], -1).astype(np.int32)
            else:
                ids = dw.blk_ids[pg].cpu().numpy()
            index[grp.layers[0]] = {
                "blk_ids": ids, "blk_cnt": cnt,
                "topk": dw.topk[g].cpu().numpy(), "topk_cnt": dw.topk_cnt[g].cpu().numpy()}
    return {"out": out, "lse": lse, "index": index}


def replicate(dw: DeviceWorkload, q_idx=None, q=None) -> DeviceWorkload:
    """A copy of ``dw`` with its own device caches (cloned on the GPU) and,
    optionally, fresh queries from the host.  Rotating over several replicas
    keeps one step's working set from being served by the last-level cache."""
    cfg = dw.cfg
    dev = dw.k_idx.device
    new = DeviceWorkload(cfg, dw.lcfg, dw.q_seq.clone(), dw.q_pos.clone(), dw.k_idx.clone(),
                         dw.k_blk.clone(), dw.k_main.clone(), dw.v_main.clone(), [])
    new.extra = [tuple(x.clone() for x in c) for c in dw.extra]
    for g, grp in enumerate(dw.groups):
        ng = Group(grp.mode, list(grp.layers),
                   grp.q.clone() if q is None else _real(np.stack([q[l] for l in grp.layers]), cfg, dev),
                   grp.k_swa.clone(), grp.v_swa.clone(), torch.empty_like(grp.out), torch.empty_like(grp.lse),
                   None, grp.index_of, grp.pool_of, grp.cache)
        if grp.q_idx is not None:
            ng.q_idx = grp.q_idx.clone() if q_idx is None else _dev(q_idx[grp.layers[0]], dev)
            if g in dw.blk_ids:
                new.blk_ids[g] = None if dw.blk_ids[g] is None else torch.empty_like(dw.blk_ids[g])
                new.blk_cnt[g] = torch.empty_like(dw.blk_cnt[g])
            new.topk[g] = torch.empty_like(dw.topk[g])
            new.topk_cnt[g] = torch.empty_like(dw.topk_cnt[g])
        new.groups.append(ng)
    new.ws = torch.zeros_like(dw.ws)
    return new


def algorithmic_bytes(cfg: Config) -> dict:
    """Bytes each kernel launch of one decode step must move at minimum (every
    input read once, every output written once; every query at t = T-1).
    Returns kernel -> list of per-launch byte counts, in launch order."""
    S, T, d, B, P, K, W_, H, D = (cfg.n_seq, cfg.ctx, cfg.d_idx, cfg.block, cfg.pool, cfg.top_k,
                                  cfg.window, cfg.n_heads, cfg.head_dim)
    esz = 4 if cfg.dtype == "f32" else 2
    n_q = cfg.n_q
    t = T - 1                                       # token position (window)
    tm = (t + 1) // cfg.ratio - 1                   # last visible main-KV entry (selection)
    n_elig = tm // B + 1
    own = tm - (n_elig - 1) * B + 1                 # visible rows of the query's own block
    pool = min(P, n_elig)
    n_cand = pool * B - (B - own)                   # the own block is pooled at most once
    sel = min(K, n_cand)
    per_layer = min(W_, t + 1) * 2 * D * esz + 2 * H * D * esz + H * 4
    out = {"index_blocks": [], "topk_tokens": [], "attend": []}
    for mode, layers in cfg.groups():
        if mode in ("full", "reindex"):
            store = n_q * d if (mode == "full" and own == B) else 0   # completed block key written back
            if n_elig > P:
                out["index_blocks"].append(n_q * ((n_elig - 1) * d + own * d + d + P * 4 + 4) + store)
            else:
                out["index_blocks"].append(n_q * (own * d + P * 4 + 4) + store)
            out["topk_tokens"].append(n_q * (d + pool * 4 + 4 + n_cand * d + K * 4 + 4))
        elif mode == "reindex_tokens":
            out["topk_tokens"].append(n_q * (d + pool * 4 + 4 + n_cand * d + K * 4 + 4))
        main = 0 if mode == "swa" else K * 4 + 4 + sel * 2 * D * esz
        out["attend"].append(n_q * (main + len(layers) * per_layer))
    return out


def algorithmic_ops(cfg: Config) -> dict:
    """Arithmetic each call of one step must do at minimum, for the MFMA
    roofline of prefill: int8 multiply-adds of the block and token scoring
    (2 ops each) and the bf16 flops of attention (QK and PV, 2 each), every
    query at its own position t.  Returns call -> list per launch."""
    S, T, d, B, P, K, W_, H, D = (cfg.n_seq, cfg.ctx, cfg.d_idx, cfg.block, cfg.pool, cfg.top_k,
                                  cfg.window, cfg.n_heads, cfg.head_dim)
    _, q_pos = query_rows(cfg)
    t = q_pos.astype(np.int64)                               # token positions (window)
    tm = (t + 1) // cfg.ratio - 1                            # last visible main-KV entry (-1: none)
    n_elig = np.where(tm >= 0, tm // B + 1, 0)
    pool = np.minimum(P, n_elig)
    block_ops = np.where(n_elig > P, n_elig * d * 2, 0)      # no scoring when the pool is the prefix
    own = np.where(tm >= 0, tm - (n_elig - 1) * B + 1, B)
    n_cand = np.maximum(pool * B - (B - own), 0)
    sel = np.minimum(K, n_cand)
    win = np.minimum(W_, t + 1)
    out = {"index_blocks": [], "topk_tokens": [], "attend": []}
    for mode, layers in cfg.groups():
        if mode in ("full", "reindex"):
            out["index_blocks"].append(int(block_ops.sum()))
        if mode in ("full", "reindex", "reindex_tokens"):
            out["topk_tokens"].append(int((n_cand * d * 2).sum()))
        keys = win + (0 if mode == "swa" else sel)
        out["attend"].append(int(len(layers) * (keys * H * D * 4).sum()))
    return out


def kernel_work(cfg: Config) -> dict:
    """Algorithmic work of one step per kernel of the library, for the
    rooflines of bench.py: kernel name -> (unit, amount per step), where unit
    is "bytes" (decode: every input read once and every output written once,
    as the kernel that moves it) or "int8_ops" / "bf16_flops" (prompts: the
    indexer scoring and the attention, 2 ops per multiply-add).  Covers the
    kernels of the decode layer group (block scoring; pool selection and token
    scoring; token Top-K and attention with the merge of its chunk records)
    and of prompts whose pools are whole prefixes (dense token Top-K, row
    attention, window attention)."""
    S, T, d, B, P, K, W_, H, D = (cfg.n_seq, cfg.ctx, cfg.d_idx, cfg.block, cfg.pool, cfg.top_k,
                                  cfg.window, cfg.n_heads, cfg.head_dim)
    esz = 4 if cfg.dtype == "f32" else 2
    work = {}

    def add(kernel, unit, amount):
        u, a = work.get(kernel, (unit, 0))
        work[kernel] = (unit, a + int(amount))

    if cfg.decode:
        n_q = cfg.n_q
        t = T - 1                                   # token position (window)
        tm = (t + 1) // cfg.ratio - 1               # last visible main-KV entry (selection)
        n_elig = tm // B + 1
        own = tm - (n_elig - 1) * B + 1
        pool = min(P, n_elig)
        n_cand = pool * B - (B - own)
        sel = min(K, n_cand)
        per_layer = min(W_, t + 1) * 2 * D * esz + 2 * H * D * esz + H * 4
        for mode, layers in cfg.groups():
            if mode in ("full", "reindex"):
                store = n_q * d if (mode == "full" and own == B) else 0
                add("k_index_blocks", "bytes", n_q * (d + (n_elig - 1) * d + own * d) + store)
                add("k_pool_tokens", "bytes", n_q * (d + P * 4 + 4 + n_cand * d))
                add("k_attend_chunks", "bytes",
                    n_q * (P * 4 + 4 + K * 4 + 4 + sel * 2 * D * esz + len(layers) * per_layer))
        return work
    # prompts: the attention kernel follows the number of (query, layer, head
    # group) items of a call (fewer than 256: key-list chunks; 256: one
    # workgroup per item; more: one wave per item, or the shared-window kernel
    # for window-only layers of 1,024 items or more), and the token Top-K is the dense MFMA kernel
    # when every pool is the whole prefix and the call has enough queries
    ops = algorithmic_ops(cfg)
    hg = max(1, H // 16)
    for (mode, layers), flops in zip(cfg.groups(), ops["attend"]):
        items = cfg.n_q * len(layers) * hg
        if items < 256:
            kernel = "k_attend_chunks"
        elif items == 256:
            kernel = "k_attend_mfma"
        elif mode == "swa" and items >= 1024:
            kernel = "k_attend_window"
        else:
            kernel = "k_attend_rows"
        add(kernel, "bf16_flops", flops)
    dense = whole_prefix_pools(cfg) and cfg.main_len <= 16384 and cfg.n_q >= 256
    for n in ops["topk_tokens"]:
        add("k_topk_dense" if dense else "k_topk_tokens", "int8_ops", n)
    return work
