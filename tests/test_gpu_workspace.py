"""One workspace shared by calls of different kinds and sizes (GPU).

A workspace sized by csa2_workspace_bytes for (n_q, T, n_layers) serves every
call with no more queries, positions and layers, in any order: each call keeps
its zero-between-calls state (selection histograms, attention merge counters)
at the head and its scratch at the tail end, and no call's scratch reaches
another call's head.  Here a fused decode layer group (8 queries) runs before
and after split selections of 64 queries on the same workspace, and every
result is compared with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import assert_index_equal, compare_run
from top_kv_selection_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from top_kv_selection_amd import binding, pipeline
    return binding, pipeline


def test_fused_group_and_larger_split_selection_share_one_workspace(lib):
    B, pipeline = lib
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=8, ctx=32768, layers=("full", "reuse"))
    wl = W.generate(cfg, seed=41)
    n_big = 64
    rng = np.random.default_rng(42)
    q_idx_big = rng.integers(-127, 128, size=(n_big, cfg.d_idx), dtype=np.int8)
    q_seq_big = (np.arange(n_big) % cfg.n_seq).astype(np.int32)
    q_pos_big = rng.integers(cfg.pool * cfg.block, cfg.ctx, size=n_big).astype(np.int32)
    print(f"case fused n_q={cfg.n_q} then split n_q={n_big}, T={cfg.ctx}", flush=True)

    dw = pipeline.upload(wl)
    pipeline.build_cache(dw)
    lc = dw.lcfg
    # one workspace for every call below: sized for the largest query count
    dw.ws = B.new_workspace(lc, n_big, cfg.ctx, len(cfg.layers))
    ref = oracle.run_layers(wl)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    qi, qs, qp = dev(q_idx_big), dev(q_seq_big), dev(q_pos_big)
    blk = torch.empty((n_big, cfg.pool), dtype=torch.int32, device="cuda")
    bc = torch.empty(n_big, dtype=torch.int32, device="cuda")
    tk = torch.empty((n_big, cfg.top_k), dtype=torch.int32, device="cuda")
    tc = torch.empty(n_big, dtype=torch.int32, device="cuda")
    want = dict(zip(("blk_ids", "blk_cnt", "topk", "topk_cnt"),
                    oracle.select(q_idx_big, q_seq_big, q_pos_big, wl.k_idx, cfg.block, cfg.pool, cfg.top_k)))
    for rnd in range(2):
        pipeline.run(dw)                                  # fused layer group, 8 queries
        torch.cuda.synchronize()
        compare_run(pipeline.outputs(dw), ref, cfg, what=f"fused group, round {rnd}")
        blk.fill_(-7)
        tk.fill_(-7)
        B.csa2_index_blocks(lc, qi, qs, qp, dw.k_idx, dw.k_blk, blk, bc, dw.ws)    # split, 64 queries
        B.csa2_topk_tokens(lc, qi, qs, qp, dw.k_idx, blk, bc, tk, tc, dw.ws)
        torch.cuda.synchronize()
        got = {"blk_ids": blk.cpu().numpy(), "blk_cnt": bc.cpu().numpy(), "topk": tk.cpu().numpy(),
               "topk_cnt": tc.cpu().numpy()}
        assert_index_equal(got, want, what=f"split selection after the fused group, round {rnd}")
