"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, sizes workspaces, and rejects bad arguments with the documented
status before anything is launched (no GPU needed: no test here reaches a
launch)."""
import ctypes
import dataclasses
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


@pytest.fixture(scope="module")
def B():
    from top_kv_selection_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|const char \*|size_t)\s*\*?\s*(csa2_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("csa2_index_blocks", "csa2_topk_tokens", "csa2_attend", "csa2_attend_group",
              "csa2_layer_group", "csa2_build_block_keys", "csa2_append_tokens", "csa2_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(B):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (csa2_\w+)$", out, re.M))
    missing = set(declared_functions()) - exported
    assert not missing, missing
    assert set(B.EXPORTS) == set(declared_functions())


def test_abi_version_and_status_strings(B):
    assert B.csa2_abi_version() == B.ABI_VERSION == 3
    for s in range(9):
        assert B._lib.csa2_status_str(s).decode()
    assert B._lib.csa2_status_str(99).decode() == "unknown status"


def _ws(B, cfg, n_q, T, L=1):
    return B.csa2_workspace_bytes(cfg, n_q, T, L)


def test_workspace_bytes_follow_the_work_split(B):
    cfg = B.Cfg()                       # P=2048, B=8, K=512, W=128, H=16, D=128, bf16
    # decode at 128K: block scores + candidate scores through the workspace
    n128 = _ws(B, cfg, 8, 131072, 6)
    assert n128 >= 8 * 16384 * 4
    # prefill of 8K: every query fits its own workgroup's LDS; the pool is the whole prefix
    assert _ws(B, cfg, 8192, 8192, 1) < 8192 * 16384 * 4
    # fp32 small heads: the generic attention kernel needs no partials
    small = B.Cfg(pool=8, top_k=32, window=16, d_idx=32, n_heads=4, head_dim=64, dtype=B.F32)
    assert _ws(B, small, 256, 256) < 1 << 20


def test_workspace_bytes_grow_with_every_size(B):
    """A workspace sized for (n_q, T, n_layers) must hold the head and scratch
    of every smaller call, so the size never shrinks as a size grows."""
    for cfg in (B.Cfg(), B.Cfg(pool=64, top_k=100, window=37), B.Cfg(n_heads=32),
                B.Cfg(pool=8, top_k=32, window=16, d_idx=32, n_heads=4, head_dim=64, dtype=B.F32)):
        for T in (300, 5003, 32768, 131072, 262144):
            prev = 0
            for n_q in (1, 7, 8, 64, 255, 256, 511, 512, 2048, 8192):
                cur = _ws(B, cfg, n_q, T, 6)
                assert cur >= prev, (cfg, T, n_q)
                assert _ws(B, cfg, n_q, T, 1) <= cur
                assert T < 300 or _ws(B, cfg, n_q, T // 2, 6) <= cur
                prev = cur


@pytest.mark.parametrize("field,value,status", [
    ("d_idx", 48, 4), ("head_dim", 96, 4), ("block", 0, 2), ("block", 17, 2), ("pool", 0, 2),
    ("top_k", -1, 2), ("window", 2000, 2), ("dtype", 7, 3), ("n_heads", 0, 2),
    ("scale", float("nan"), 2), ("scale", -1.0, 2), ("tail", 3, 2), ("tail", -1, 2),
    ("ratio", -1, 2), ("ratio", 257, 2),
])
def test_bad_config_is_rejected(B, field, value, status):
    c = dataclasses.asdict(B.Cfg())
    c[field] = value
    cfg = B.Cfg(**c)
    out = ctypes.c_size_t(0)
    assert B._lib.csa2_workspace_bytes(ctypes.byref(cfg.c()), 8, 1024, 1, ctypes.byref(out)) == status


def test_pool_times_block_cap_and_empty_selection(B):
    out = ctypes.c_size_t(0)
    f = lambda cfg: B._lib.csa2_workspace_bytes(ctypes.byref(cfg.c()), 1, 64, 1, ctypes.byref(out))
    assert f(B.Cfg(pool=2049, block=8)) == 2          # more than 16,384 candidates
    assert f(B.Cfg(pool=2048, block=8, top_k=16385)) == 2
    assert f(B.Cfg(top_k=0, window=0)) == 2            # nothing to attend
    assert f(B.Cfg(ratio=4, window=0)) == 2            # a query before the first entry would see nothing
    assert f(B.Cfg(ratio=4, window=1)) == 0
    assert f(B.Cfg(top_k=0, window=128)) == 0          # window only is fine
    assert B._lib.csa2_workspace_bytes(None, 1, 64, 1, ctypes.byref(out)) == 1


FAKE = 1 << 20      # a 16-byte aligned address that is never dereferenced


def _index_call(B, cfg, **kw):
    a = dict(n_q=4, q_idx=FAKE, q_seq=FAKE, q_pos=FAKE, k_idx=FAKE, k_blk=FAKE, n_seq=1, T=4096,
             blk_ids=FAKE, blk_cnt=FAKE, ws=FAKE, ws_bytes=0)
    a.update(kw)
    P = ctypes.c_void_p
    return B._lib.csa2_index_blocks(ctypes.byref(cfg.c()), a["n_q"], P(a["q_idx"]), P(a["q_seq"]), P(a["q_pos"]),
                                    P(a["k_idx"]), P(a["k_blk"]), a["n_seq"], a["T"], P(a["blk_ids"]),
                                    P(a["blk_cnt"]), P(a["ws"]), a["ws_bytes"], None)


def test_index_blocks_argument_errors(B):
    cfg = B.Cfg(pool=64)
    assert _index_call(B, cfg, q_idx=None) == 1
    assert _index_call(B, cfg, k_blk=None) == 1
    assert _index_call(B, cfg, k_idx=FAKE + 4) == 5      # not 16-byte aligned
    assert _index_call(B, cfg, q_seq=FAKE + 2) == 5      # int32 array not 4-byte aligned
    assert _index_call(B, cfg, ws=None) == 6             # the block pass needs a workspace
    assert _index_call(B, cfg, ws_bytes=1024) == 6       # too small
    assert _index_call(B, cfg, T=0) == 2
    assert _index_call(B, cfg, n_q=-1) == 2
    assert _index_call(B, cfg, n_q=0) == 0               # nothing to do, nothing launched
    # a cache shorter than one block has no block key: k_blk may be NULL
    # (checked with a misaligned q_seq, which fails right after the pointer
    # checks, so nothing is launched)
    assert _index_call(B, cfg, k_blk=None, T=7, q_seq=FAKE + 2) == 5
    assert _index_call(B, cfg, k_blk=None, T=8, q_seq=FAKE + 2) == 1


def test_block_keys_of_a_cache_without_a_complete_block(B):
    P = ctypes.c_void_p
    f = lambda T, k_blk: B._lib.csa2_build_block_keys(ctypes.byref(B.Cfg().c()), P(FAKE), 1, T, 0, 1 << 20,
                                                      P(k_blk), None)
    assert f(7, None) == 0          # T < B: nothing to write, nothing launched
    assert f(8, None) == 1


def test_layer_group_checks_every_stage_before_launching(B):
    """A Full layer group whose attention arguments are bad must fail before
    the block-key update is launched (no launch can happen on this CPU)."""
    cfg = B.Cfg(pool=64)
    P = ctypes.c_void_p
    need = B.csa2_workspace_bytes(cfg, 4, 4096, 1)
    args = lambda mode, out, ws_bytes: B._lib.csa2_layer_group(
        ctypes.byref(cfg.c()), mode, 1, 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 0, 1, 4096,
        P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 4096 - 128, 128, P(FAKE), P(FAKE), P(FAKE), P(FAKE),
        P(out), None, P(FAKE), ws_bytes, None)
    assert args(0, None, need) == 1          # missing output
    assert args(0, FAKE, 16) == 6            # workspace too small for the block pass
    assert args(9, FAKE, need) == 8          # unknown mode
    assert args(2, None, need) == 1          # reuse with no output
    assert args(4, None, need) == 1          # token-only reindex with no output


def test_token_only_reindex_needs_the_shared_pool(B):
    """CSA2_REINDEX_TOKENS reads blk_ids/blk_cnt: without them it fails before
    any launch."""
    cfg = B.Cfg(pool=64)
    P = ctypes.c_void_p
    need = B.csa2_workspace_bytes(cfg, 4, 4096, 1)
    call = lambda blk: B._lib.csa2_layer_group(
        ctypes.byref(cfg.c()), 4, 1, 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 0, 1, 4096,
        P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 4096 - 128, 128, P(blk), P(blk), P(FAKE), P(FAKE),
        P(FAKE), None, P(FAKE), need, None)
    assert call(None) == 1
    assert B.MODES["reindex_tokens"] == 4


def test_reuse_and_attend_argument_errors(B):
    cfg = B.Cfg()
    P = ctypes.c_void_p
    f = lambda **kw: B._lib.csa2_attend_group(
        ctypes.byref(cfg.c()), kw.get("L", 1), 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 1, 4096,
        P(kw.get("k_swa", FAKE)), P(FAKE), kw.get("swa_first", 0), kw.get("swa_len", 4096),
        P(kw.get("topk", FAKE)), P(kw.get("topk_cnt", FAKE)), P(kw.get("out", FAKE)), None, P(FAKE),
        1 << 20, None)
    assert f(L=0) == 2
    assert f(topk=None) == 1                 # topk and topk_cnt go together
    assert f(k_swa=None) == 1                # a window needs window rows
    assert f(swa_first=-1) == 2
    assert f(swa_len=0) == 2
    assert f(out=FAKE + 8) == 5


def test_append_argument_errors(B):
    """Token append: missing or misaligned arrays and bad sizes fail before any
    launch; an empty call succeeds whatever its pointers."""
    cfg = B.Cfg()
    P = ctypes.c_void_p
    names = ("seq", "pos", "new_k_idx", "new_k", "new_v", "k_idx", "k_main", "v_main", "k_blk")
    def f(n=4, S=2, T=64, **kw):
        ptrs = [P(kw.get(k, FAKE)) for k in names]
        return B._lib.csa2_append_tokens(ctypes.byref(cfg.c()), n, *ptrs, S, T, None)
    assert f(seq=None) == 1
    assert f(v_main=None) == 1
    assert f(new_k=FAKE + 8) == 5
    assert f(pos=FAKE + 2) == 5
    assert f(k_blk=FAKE + 4) == 5
    assert f(n=-1) == 2
    assert f(T=0) == 2
    assert f(S=0) == 2
    assert f(n=0) == 0
    assert f(n=0, seq=None, k_idx=None) == 0
    bad = dataclasses.replace(cfg, d_idx=48)
    assert B._lib.csa2_append_tokens(ctypes.byref(bad.c()), 4, *[P(FAKE)] * 9, 2, 64, None) == 4
