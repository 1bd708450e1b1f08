"""Token append through the C ABI: rows land at their cache positions and the
key of every block a new token completes matches the oracle's block key;
everything else is left as it was.  All comparisons are bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from top_kv_selection_amd import binding as B

pytestmark = pytest.mark.gpu


def _case(cfg, S, T, new, seed, with_blk=True):
    """new: list of (sequence, position) of the tokens appended in one call."""
    rng = np.random.default_rng(seed)
    dt = np.float32
    nblk = T // cfg.block
    k_idx = rng.integers(-127, 128, size=(S, T, cfg.d_idx), dtype=np.int8)
    k_main = rng.standard_normal((S, T, cfg.head_dim)).astype(dt)
    v_main = rng.standard_normal((S, T, cfg.head_dim)).astype(dt)
    k_blk = rng.integers(-127, 128, size=(S, nblk, cfg.d_idx), dtype=np.int8)
    n = len(new)
    seq = np.array([s for s, _ in new], dtype=np.int32)
    pos = np.array([t for _, t in new], dtype=np.int32)
    nk_idx = rng.integers(-127, 128, size=(n, cfg.d_idx), dtype=np.int8)
    nk = rng.standard_normal((n, cfg.head_dim)).astype(dt)
    nv = rng.standard_normal((n, cfg.head_dim)).astype(dt)

    tdt = cfg.torch_dtype
    dev = lambda a, d=None: torch.from_numpy(a).to("cuda", dtype=d) if d is not None else torch.from_numpy(a).cuda()
    g = dict(k_idx=dev(k_idx), k_main=dev(k_main, tdt), v_main=dev(v_main, tdt), k_blk=dev(k_blk))
    B.csa2_append_tokens(cfg, dev(seq), dev(pos), dev(nk_idx), dev(nk, tdt), dev(nv, tdt), g["k_idx"],
                         g["k_main"], g["v_main"], g["k_blk"] if with_blk else None)
    torch.cuda.synchronize()

    # expected: the rows copied (values as the device dtype holds them), then
    # the oracle's key of each completed block
    as_dev = lambda a: torch.from_numpy(a).to(tdt).float().numpy()
    e_idx, e_k, e_v = k_idx.copy(), as_dev(k_main), as_dev(v_main)
    nk_d, nv_d = as_dev(nk), as_dev(nv)
    for i, (s, t) in enumerate(new):
        e_idx[s, t], e_k[s, t], e_v[s, t] = nk_idx[i], nk_d[i], nv_d[i]
    e_blk = k_blk.copy()
    completed = set()
    if with_blk:
        for s, t in new:
            if (t + 1) % cfg.block == 0:
                j = t // cfg.block
                e_blk[s, j] = oracle.block_key(e_idx[s], cfg.block, j, t)
                completed.add((s, j))
    assert np.array_equal(g["k_idx"].cpu().numpy(), e_idx)
    assert np.array_equal(g["k_main"].float().cpu().numpy(), e_k)
    assert np.array_equal(g["v_main"].float().cpu().numpy(), e_v)
    assert np.array_equal(g["k_blk"].cpu().numpy(), e_blk)
    return completed


def test_append_decode_tokens_and_completed_blocks():
    """One token per sequence, as in decode: two complete their block (one at
    the last position of the cache), one does not."""
    cfg = B.Cfg()
    done = _case(cfg, S=3, T=200, new=[(0, 7), (1, 100), (2, 199)], seed=1)
    assert done == {(0, 0), (2, 24)}


def test_append_whole_blocks_in_one_call():
    """Several rows of one block in one call: the block key sees all of them,
    including rows written by other workgroups of the same call."""
    cfg = B.Cfg()
    new = [(0, p) for p in range(8, 16)] + [(2, p) for p in (3, 0, 7, 5, 1, 6, 2, 4)] + [(1, 20), (0, 199)]
    done = _case(cfg, S=3, T=200, new=new, seed=2)
    assert done == {(0, 1), (2, 0), (0, 24)}


def test_append_fp32_small_index_and_block_of_two():
    cfg = B.Cfg(block=2, pool=64, top_k=32, window=16, d_idx=32, n_heads=4, head_dim=64, dtype=B.F32)
    new = [(0, 1), (0, 2), (1, 5), (1, 4), (0, 63)]
    done = _case(cfg, S=2, T=64, new=new, seed=3)
    assert done == {(0, 0), (1, 2), (0, 31)}


def test_append_without_block_keys():
    cfg = B.Cfg()
    assert _case(cfg, S=2, T=64, new=[(0, 7), (1, 15), (1, 3)], seed=4, with_blk=False) == set()


def test_append_nothing():
    cfg = B.Cfg()
    assert _case(cfg, S=1, T=16, new=[], seed=5) == set()
