"""ctypes binding of libcsa2.so (the C ABI in include/csa2.h).

Argument marshalling only: every function checks that torch tensors have the
dtype, device and contiguity the C call expects, passes their data pointers and
the current HIP stream, and turns a non-zero status into an exception.  All
arithmetic runs in the library's HIP kernels; there is no CPU fallback, and the
module raises on import if the library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

FULL, REINDEX, REUSE, SWA, REINDEX_TOKENS = 0, 1, 2, 3, 4
MODES = {"full": FULL, "reindex": REINDEX, "reuse": REUSE, "swa": SWA, "reindex_tokens": REINDEX_TOKENS}
F32, BF16 = 0, 1
TAIL_VISIBLE, TAIL_EXCLUDE, TAIL_WHOLE = 0, 1, 2
ABI_VERSION = 3          # csa2_cfg layout of include/csa2.h

STATUS = {0: "CSA2_OK", 1: "CSA2_E_NULL", 2: "CSA2_E_SHAPE", 3: "CSA2_E_DTYPE",
          4: "CSA2_E_UNSUPPORTED", 5: "CSA2_E_ALIGN", 6: "CSA2_E_WORKSPACE", 7: "CSA2_E_HIP",
          8: "CSA2_E_MODE"}

EXPORTS = ["csa2_abi_version", "csa2_status_str", "csa2_profile_begin", "csa2_profile_end", "csa2_profile_record",
           "csa2_workspace_bytes", "csa2_workspace_init", "csa2_build_block_keys", "csa2_append_tokens",
           "csa2_index_blocks", "csa2_topk_tokens", "csa2_attend_group", "csa2_attend", "csa2_layer_group",
           "csa2_layer_group_single", "csa2_layer_group_static"]


class Csa2Error(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


class _CCfg(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("pool", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("window", ctypes.c_int32), ("d_idx", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("tail", ctypes.c_int32), ("ratio", ctypes.c_int32)]


@dataclass(frozen=True)
class Cfg:
    block: int = 8
    pool: int = 2048
    top_k: int = 512
    window: int = 128
    d_idx: int = 64
    n_heads: int = 16
    head_dim: int = 128
    dtype: int = BF16
    scale: float = 0.0
    tail: int = 0           # TAIL_VISIBLE / TAIL_EXCLUDE / TAIL_WHOLE
    ratio: int = 1          # tokens per main-KV entry (compressed main-KV and indexer caches)

    def c(self) -> _CCfg:
        return _CCfg(self.block, self.pool, self.top_k, self.window, self.d_idx, self.n_heads,
                     self.head_dim, self.dtype, float(self.scale), int(self.tail), int(self.ratio))

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == F32 else torch.bfloat16


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -m top_kv_selection_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    C = ctypes.POINTER(_CCfg)
    sig = {
        "csa2_abi_version": (I, []),
        "csa2_status_str": (ctypes.c_char_p, [I]),
        "csa2_profile_begin": (I, [ctypes.c_char_p, I]),
        "csa2_profile_end": (I, [ctypes.POINTER(I)]),
        "csa2_profile_record": (I, [I, ctypes.c_char_p, I, ctypes.POINTER(ctypes.c_float)]),
        "csa2_workspace_bytes": (I, [C, I, I, I, ctypes.POINTER(ctypes.c_size_t)]),
        "csa2_workspace_init": (I, [P, Z, P]),
        "csa2_build_block_keys": (I, [C, P, I, I, I, I, P, P]),
        "csa2_append_tokens": (I, [C, I, P, P, P, P, P, P, P, P, P, I, I, P]),
        "csa2_index_blocks": (I, [C, I, P, P, P, P, P, I, I, P, P, P, Z, P]),
        "csa2_topk_tokens": (I, [C, I, P, P, P, P, I, I, P, P, P, P, P, Z, P]),
        "csa2_attend_group": (I, [C, I, I, P, P, P, P, P, I, I, P, P, I, I, P, P, P, P, P, Z, P]),
        "csa2_attend": (I, [C, I, P, P, P, P, P, I, I, P, P, I, I, P, P, P, P, P, Z, P]),
        "csa2_layer_group": (I, [C, I, I, I, P, P, P, P, P, I, I, I, P, P, P, P, P, I, I, P, P, P, P,
                                 P, P, P, Z, P]),
        "csa2_layer_group_single": (I, [C, I, I, I, P, P, P, P, P, I, I, I, P, P, P, P, P, I, I, P, P, P, P,
                                        P, P, P, Z, P]),
        "csa2_layer_group_static": (I, [C, I, I, I, P, P, P, P, P, I, I, I, P, P, P, P, P, I, I, P, P, P, P,
                                        P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    if lib.csa2_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.csa2_abi_version()}, this binding speaks "
                          f"{ABI_VERSION}: rebuild it (python -m top_kv_selection_amd.build)")
    return lib


_lib = _load()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn, status):
    if status != 0:
        raise Csa2Error(fn, status, _lib.csa2_status_str(status).decode())


def _need(t, name, dtype, ndim=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def csa2_abi_version() -> int:
    return int(_lib.csa2_abi_version())


def csa2_profile_begin(kernel_filter: str = "", max_launches: int = 4096):
    """Arms the library's per-kernel timing: the next max_launches kernel
    launches whose name contains kernel_filter carry HIP start/stop events."""
    _check("csa2_profile_begin", _lib.csa2_profile_begin(kernel_filter.encode(), int(max_launches)))


def csa2_profile_end():
    """Disarms the timing and returns [(kernel name, milliseconds)] of every
    timed launch, in launch order."""
    n = ctypes.c_int32(0)
    _check("csa2_profile_end", _lib.csa2_profile_end(ctypes.byref(n)))
    out = []
    buf = ctypes.create_string_buffer(64)
    ms = ctypes.c_float(0.0)
    for i in range(n.value):
        _check("csa2_profile_record", _lib.csa2_profile_record(i, buf, 64, ctypes.byref(ms)))
        out.append((buf.value.decode(), float(ms.value)))
    return out


def csa2_workspace_bytes(cfg: Cfg, n_q: int, T: int, n_layers: int = 1) -> int:
    out = ctypes.c_size_t(0)
    _check("csa2_workspace_bytes", _lib.csa2_workspace_bytes(ctypes.byref(cfg.c()), n_q, T, n_layers,
                                                             ctypes.byref(out)))
    return int(out.value)


def csa2_workspace_init(ws: torch.Tensor):
    _need(ws, "ws", torch.uint8)
    _check("csa2_workspace_init", _lib.csa2_workspace_init(_p(ws), ws.numel(), _stream(ws.device)))


def new_workspace(cfg: Cfg, n_q: int, T: int, n_layers: int = 1, device="cuda") -> torch.Tensor:
    """Allocates and zero-fills a workspace for calls up to (n_q, T, n_layers)."""
    n = max(256, csa2_workspace_bytes(cfg, n_q, T, n_layers))
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    csa2_workspace_init(ws)
    return ws


def csa2_build_block_keys(cfg: Cfg, k_idx, k_blk, blk_begin=0, blk_end=None):
    _need(k_idx, "k_idx", torch.int8, 3)
    _need(k_blk, "k_blk", torch.int8, 3)
    S, T, _ = k_idx.shape
    if blk_end is None:
        blk_end = T // cfg.block
    _check("csa2_build_block_keys", _lib.csa2_build_block_keys(
        ctypes.byref(cfg.c()), _p(k_idx), S, T, blk_begin, blk_end, _p(k_blk), _stream(k_idx.device)))


def csa2_append_tokens(cfg: Cfg, seq, pos, new_k_idx, new_k, new_v, k_idx, k_main, v_main, k_blk=None):
    """Writes n_new tokens' rows into the caches; with k_blk, also the key of
    every block a new token completes."""
    for t, n, d in ((seq, "seq", torch.int32), (pos, "pos", torch.int32), (new_k_idx, "new_k_idx", torch.int8),
                    (k_idx, "k_idx", torch.int8)):
        _need(t, n, d)
    for t, n in ((new_k, "new_k"), (new_v, "new_v"), (k_main, "k_main"), (v_main, "v_main")):
        _need(t, n, cfg.torch_dtype)
    if k_blk is not None:
        _need(k_blk, "k_blk", torch.int8, 3)
    S, T, _ = k_idx.shape
    n_new = seq.shape[0]
    if not (pos.shape[0] == new_k_idx.shape[0] == new_k.shape[0] == new_v.shape[0] == n_new):
        raise ValueError("seq, pos, new_k_idx, new_k and new_v need one row per new token")
    if (tuple(new_k_idx.shape[1:]) != (cfg.d_idx,) or tuple(new_k.shape[1:]) != (cfg.head_dim,)
            or tuple(new_v.shape[1:]) != (cfg.head_dim,) or k_idx.shape[2] != cfg.d_idx
            or tuple(k_main.shape) != (S, T, cfg.head_dim) or tuple(v_main.shape) != (S, T, cfg.head_dim)
            or (k_blk is not None and tuple(k_blk.shape) != (S, T // cfg.block, cfg.d_idx))):
        raise ValueError("cache or row shapes disagree with the config")
    _check("csa2_append_tokens", _lib.csa2_append_tokens(
        ctypes.byref(cfg.c()), n_new, _p(seq), _p(pos), _p(new_k_idx), _p(new_k), _p(new_v), _p(k_idx),
        _p(k_main), _p(v_main), _p(k_blk), S, T, _stream(k_idx.device)))


def csa2_index_blocks(cfg: Cfg, q_idx, q_seq, q_pos, k_idx, k_blk, blk_ids, blk_cnt, ws):
    for t, n, d in ((q_idx, "q_idx", torch.int8), (k_idx, "k_idx", torch.int8), (k_blk, "k_blk", torch.int8),
                    (q_seq, "q_seq", torch.int32), (q_pos, "q_pos", torch.int32),
                    (blk_ids, "blk_ids", torch.int32), (blk_cnt, "blk_cnt", torch.int32), (ws, "ws", torch.uint8)):
        _need(t, n, d)
    S, T, _ = k_idx.shape
    _check("csa2_index_blocks", _lib.csa2_index_blocks(
        ctypes.byref(cfg.c()), q_idx.shape[0], _p(q_idx), _p(q_seq), _p(q_pos), _p(k_idx), _p(k_blk), S, T,
        _p(blk_ids), _p(blk_cnt), _p(ws), 0 if ws is None else ws.numel(), _stream(k_idx.device)))


def csa2_topk_tokens(cfg: Cfg, q_idx, q_seq, q_pos, k_idx, blk_ids, blk_cnt, topk, topk_cnt, ws):
    for t, n, d in ((q_idx, "q_idx", torch.int8), (k_idx, "k_idx", torch.int8),
                    (q_seq, "q_seq", torch.int32), (q_pos, "q_pos", torch.int32),
                    (blk_ids, "blk_ids", torch.int32), (blk_cnt, "blk_cnt", torch.int32),
                    (topk, "topk", torch.int32), (topk_cnt, "topk_cnt", torch.int32), (ws, "ws", torch.uint8)):
        _need(t, n, d)
    S, T, _ = k_idx.shape
    _check("csa2_topk_tokens", _lib.csa2_topk_tokens(
        ctypes.byref(cfg.c()), q_idx.shape[0], _p(q_idx), _p(q_seq), _p(q_pos), _p(k_idx), S, T, _p(blk_ids),
        _p(blk_cnt), _p(topk), _p(topk_cnt), _p(ws), 0 if ws is None else ws.numel(), _stream(k_idx.device)))


def _attend_checks(cfg, q, k_main, v_main, k_swa, v_swa, out, lse, q_seq, q_pos, topk, topk_cnt, ws):
    dt = cfg.torch_dtype
    for t, n in ((q, "q"), (k_main, "k_main"), (v_main, "v_main"), (k_swa, "k_swa"), (v_swa, "v_swa"),
                 (out, "out")):
        _need(t, n, dt)
    for t, n in ((q_seq, "q_seq"), (q_pos, "q_pos"), (topk, "topk"), (topk_cnt, "topk_cnt")):
        _need(t, n, torch.int32)
    _need(lse, "lse", torch.float32)
    _need(ws, "ws", torch.uint8)


def csa2_attend_group(cfg: Cfg, q, q_seq, q_pos, k_main, v_main, k_swa, v_swa, swa_first, topk,
                      topk_cnt, out, lse=None, ws=None):
    """q [L][n_q][H][D]; k_swa/v_swa [L][S][swa_len][D]; out like q."""
    _attend_checks(cfg, q, k_main, v_main, k_swa, v_swa, out, lse, q_seq, q_pos, topk, topk_cnt, ws)
    L, n_q = q.shape[0], q.shape[1]
    S, T = k_main.shape[0], k_main.shape[1]
    swa_len = k_swa.shape[2] if k_swa is not None else 0
    _check("csa2_attend_group", _lib.csa2_attend_group(
        ctypes.byref(cfg.c()), L, n_q, _p(q), _p(q_seq), _p(q_pos), _p(k_main), _p(v_main), S, T, _p(k_swa),
        _p(v_swa), int(swa_first), swa_len, _p(topk), _p(topk_cnt), _p(out), _p(lse), _p(ws),
        0 if ws is None else ws.numel(), _stream(q.device)))


def csa2_attend(cfg: Cfg, q, q_seq, q_pos, k_main, v_main, k_swa, v_swa, swa_first, topk, topk_cnt,
                out, lse=None, ws=None):
    """q [n_q][H][D]; k_swa/v_swa [S][swa_len][D]; out like q."""
    _attend_checks(cfg, q, k_main, v_main, k_swa, v_swa, out, lse, q_seq, q_pos, topk, topk_cnt, ws)
    n_q = q.shape[0]
    S, T = k_main.shape[0], k_main.shape[1]
    swa_len = k_swa.shape[1] if k_swa is not None else 0
    _check("csa2_attend", _lib.csa2_attend(
        ctypes.byref(cfg.c()), n_q, _p(q), _p(q_seq), _p(q_pos), _p(k_main), _p(v_main), S, T, _p(k_swa),
        _p(v_swa), int(swa_first), swa_len, _p(topk), _p(topk_cnt), _p(out), _p(lse), _p(ws),
        0 if ws is None else ws.numel(), _stream(q.device)))


def csa2_layer_group(cfg: Cfg, mode, q_idx, q_seq, q_pos, k_idx, k_blk, blk_update_begin, q, k_main,
                     v_main, k_swa, v_swa, swa_first, blk_ids, blk_cnt, topk, topk_cnt, out, lse=None,
                     ws=None, single=False):
    """One CSA2 layer group: the first layer's mode (full/reindex/reuse/swa/
    reindex_tokens) picks the selection work; all layers of q [L][n_q][H][D]
    attend with the shared indices.  ``single`` calls csa2_layer_group_single
    (the fused decode group as one launch)."""
    fn = "csa2_layer_group_single" if single else "csa2_layer_group"
    mode = MODES[mode] if isinstance(mode, str) else int(mode)
    _attend_checks(cfg, q, k_main, v_main, k_swa, v_swa, out, lse, q_seq, q_pos, topk, topk_cnt, ws)
    for t, n, d in ((q_idx, "q_idx", torch.int8), (k_idx, "k_idx", torch.int8), (k_blk, "k_blk", torch.int8),
                    (blk_ids, "blk_ids", torch.int32), (blk_cnt, "blk_cnt", torch.int32)):
        _need(t, n, d)
    L, n_q = q.shape[0], q.shape[1]
    S, T = k_main.shape[0], k_main.shape[1]
    swa_len = k_swa.shape[2] if k_swa is not None else 0
    _check(fn, getattr(_lib, fn)(
        ctypes.byref(cfg.c()), mode, L, n_q, _p(q_idx), _p(q_seq), _p(q_pos), _p(k_idx), _p(k_blk),
        int(blk_update_begin), S, T, _p(q), _p(k_main), _p(v_main), _p(k_swa), _p(v_swa), int(swa_first),
        swa_len, _p(blk_ids), _p(blk_cnt), _p(topk), _p(topk_cnt), _p(out), _p(lse), _p(ws),
        0 if ws is None else ws.numel(), _stream(q.device)))


def csa2_layer_group_static(cfg: Cfg, mode, q_idx, q_seq, q_pos, k_idx, k_blk, blk_update_begin, q, k_main,
                            v_main, k_swa, v_swa, swa_first, blk_ids, blk_cnt, topk, topk_cnt, out, lse=None):
    """csa2_layer_group with the library's own fixed device scratch instead of
    a workspace (allocates nothing); calls on one GPU must not overlap."""
    mode = MODES[mode] if isinstance(mode, str) else int(mode)
    _attend_checks(cfg, q, k_main, v_main, k_swa, v_swa, out, lse, q_seq, q_pos, topk, topk_cnt, None)
    for t, n, d in ((q_idx, "q_idx", torch.int8), (k_idx, "k_idx", torch.int8), (k_blk, "k_blk", torch.int8),
                    (blk_ids, "blk_ids", torch.int32), (blk_cnt, "blk_cnt", torch.int32)):
        _need(t, n, d)
    L, n_q = q.shape[0], q.shape[1]
    S, T = k_main.shape[0], k_main.shape[1]
    swa_len = k_swa.shape[2] if k_swa is not None else 0
    _check("csa2_layer_group_static", _lib.csa2_layer_group_static(
        ctypes.byref(cfg.c()), mode, L, n_q, _p(q_idx), _p(q_seq), _p(q_pos), _p(k_idx), _p(k_blk),
        int(blk_update_begin), S, T, _p(q), _p(k_main), _p(v_main), _p(k_swa), _p(v_swa), int(swa_first),
        swa_len, _p(blk_ids), _p(blk_cnt), _p(topk), _p(topk_cnt), _p(out), _p(lse), _stream(q.device)))


def cfg_of(wcfg) -> Cfg:
    """Library config from a workload description (top_kv_selection_amd.workloads.Config)."""
    return Cfg(wcfg.block, wcfg.pool, wcfg.top_k, wcfg.window, wcfg.d_idx, wcfg.n_heads, wcfg.head_dim,
               F32 if wcfg.dtype == "f32" else BF16, 0.0, wcfg.tail, wcfg.ratio)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
