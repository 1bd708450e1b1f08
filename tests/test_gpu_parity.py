"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Indices must be identical and outputs within 2e-2 + 1e-2*|ref|.  Cases cover
the five workload shapes (full size where the oracle can take every query,
sampled rows for the 8K prefill), scaled versions that span several tiles with
ragged tails, tie-heavy draws, and the edge cases of the method: the pool
covering every block, fewer candidates than K, the query's own partial block,
no window, window-only layers, several head groups, fp32 and bf16, d_idx 32.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from parity import assert_close, assert_index_equal, compare_run
from top_kv_selection_amd import workloads as W

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "toy16.json")


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from top_kv_selection_amd import binding, pipeline
    return binding, pipeline


def run_gpu(pipeline, wl):
    dw = pipeline.upload(wl)
    pipeline.build_cache(dw)
    pipeline.run(dw)
    torch.cuda.synchronize()
    return pipeline.outputs(dw)


def check(lib, cfg, seed=None, rows=None, int_range=(-127, 127)):
    _, pipeline = lib
    print(f"case {cfg.name} S={cfg.n_seq} T={cfg.ctx} P={cfg.pool} K={cfg.top_k} W={cfg.window} "
          f"layers={cfg.layers} seed={seed} rows={'all' if rows is None else len(rows)}", flush=True)
    wl = W.generate(cfg, seed=seed, int_range=int_range)
    got = run_gpu(pipeline, wl)
    ref = oracle.run_layers(wl, rows=rows)
    return compare_run(got, ref, cfg, rows=rows, what=cfg.name)


# ------------------------------------------------------------------ the five workloads
def test_tiny_full_fp32_all_queries(lib):
    check(lib, W.CONFIGS["tiny_full_fp32"])


def test_decode_full_32k(lib):
    check(lib, W.CONFIGS["decode_full_32k"])


def test_decode_group_128k(lib):
    check(lib, W.CONFIGS["decode_group_128k"])


def test_decoder_pattern_64k(lib):
    check(lib, W.CONFIGS["decoder_pattern_64k"])


def test_prefill_8k_all_rows(lib):
    check(lib, W.CONFIGS["prefill_8k"])


# ------------------------------------------------------------------ scaled cases
def test_decode_scaled_ragged_context(lib):
    """Context not a multiple of the block: the own block is partial; several
    workgroups per query, pool smaller than the eligible blocks."""
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=5, ctx=5003, pool=96, top_k=100, window=37)
    check(lib, cfg, seed=21)


def test_decode_queries_not_in_sequence_order(lib):
    """Query i of a decode batch reads sequence n_seq - 1 - i: the block pass
    cannot take its first batch from the sequence numbered like the query and
    loads it again."""
    _, pipeline = lib
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=5, ctx=9001, pool=128, top_k=200, window=64,
                   layers=("full", "reuse"))
    wl = W.generate(cfg, seed=27)
    wl.q_seq = np.ascontiguousarray(wl.q_seq[::-1])
    print(f"case {cfg.name} reversed q_seq {wl.q_seq.tolist()}", flush=True)
    got = run_gpu(pipeline, wl)
    ref = oracle.run_layers(wl)
    compare_run(got, ref, cfg, what="reversed q_seq")


def test_decode_scaled_tie_heavy(lib):
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=3, ctx=8192, pool=128, top_k=200, window=64,
                   layers=("full", "reuse", "reuse"))
    check(lib, cfg, seed=22, int_range=(-2, 2))


def test_decode_pool_covers_everything(lib):
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=4, ctx=1000, pool=2048)
    check(lib, cfg, seed=23)


def test_decode_fewer_candidates_than_k(lib):
    # 300 visible tokens < K = 512 <= P*B: every candidate is selected
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=4, ctx=300, pool=64, top_k=512)
    check(lib, cfg, seed=24)


def test_prefill_scaled_all_rows(lib):
    """Every position of a 700-token prompt: own partial blocks, pool active
    past 8*64 tokens, K larger than the prefix for early rows; the window-only
    layer's 700 items take the row kernel (too few for the shared-window one)."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=700, pool=64, top_k=96, window=40,
                   layers=("full", "reuse", "swa"))
    check(lib, cfg, seed=25)


def test_prefill_scaled_tie_heavy_d32(lib):
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=600, d_idx=32, pool=24, top_k=50, window=16,
                   layers=("full", "reindex"))
    check(lib, cfg, seed=26, int_range=(-1, 1))


def test_prefill_row_kernel_long_lists(lib):
    """Many queries take the wave-per-item attention kernel: key lists longer
    than one staged chunk of row codes (K + W up to 1,000), a window-only
    layer, and an item count that leaves the last workgroups part-filled."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=1501, pool=128, top_k=900, window=100,
                   layers=("full", "reuse", "swa"))
    check(lib, cfg, seed=29)


def test_prefill_row_kernel_blocks_in_rounds(lib):
    """More (query, layer, head group) items than one round of the row kernel
    takes (four per wave over the chip's workgroups): the items go in blocks
    of 16 consecutive ones per workgroup, run in rounds, the last block
    part-filled (3,001 queries x 3 layers = 9,003 items)."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=3001, layers=("full", "reuse", "reuse"))
    check(lib, cfg, seed=31)


def test_prefill_row_kernel_two_head_groups(lib):
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=1100, pool=64, top_k=200, window=128, n_heads=32,
                   layers=("full", "swa"))
    check(lib, cfg, seed=30)


# ------------------------------------------------------------------ encoder-decoder flow
def test_encoder_pattern_scaled_all_rows(lib):
    """Window, [Full + Reuse...] with three Full layers, each with its own
    main-KV and indexer cache, at every position of a prompt."""
    cfg = W.scaled(W.CONFIGS["encoder_prefill_8k"], ctx=600, pool=32, top_k=64, window=24,
                   layers=("swa", "full", "reuse", "reuse", "full", "reuse", "full"))
    check(lib, cfg, seed=50)


def test_encoder_prefill_8k_all_rows(lib):
    check(lib, W.CONFIGS["encoder_prefill_8k"])


def test_one_round_of_attention_workgroups(lib):
    """256 (query, layer) items, one round of one attention workgroup per
    item (the MFMA kernel): 64 replayed prompt positions through Full + 3
    Reuse.  One item more takes the row kernel (the replay test below)."""
    cfg = W.scaled(W.CONFIGS["decoder_replay_8k"], replay=64, layers=("full", "reuse", "reuse", "reuse"))
    check(lib, cfg, seed=62)


def test_decoder_replay_8k(lib):
    """The last 128 prompt positions through the 20-layer decoder pattern."""
    check(lib, W.CONFIGS["decoder_replay_8k"])


# ------------------------------------------------------------------ selection variants
@pytest.mark.parametrize("tail", [W.TAIL_EXCLUDE, W.TAIL_WHOLE])
def test_tail_reading_prefill_block_pass(lib, tail):
    """Every position of a prompt under the other two readings of a partial
    own block: block pass with one workgroup per query (pool smaller than the
    eligible blocks), per-query token Top-K; with the tail excluded the first
    B-1 queries select nothing and attend to their window alone."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=700, pool=64, top_k=96, window=40,
                   layers=("full", "reuse"), tail=tail)
    check(lib, cfg, seed=40 + tail)


@pytest.mark.parametrize("tail", [W.TAIL_EXCLUDE, W.TAIL_WHOLE])
def test_tail_reading_prefill_whole_prefix_pools(lib, tail):
    """Pools that hold every eligible block: the pool-all kernel and the dense
    (MFMA tile) token Top-K under the other two tail readings."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=1200, pool=2048, top_k=96, window=16, layers=("full",),
                   tail=tail)
    check(lib, cfg, seed=42 + tail)


def test_tail_excluded_decode_split_pass_and_layer_group(lib):
    """Decode with a partial own block excluded: block pass split over many
    workgroups per query, fused layer group with two Reuse layers."""
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=4, ctx=20003, pool=256, top_k=300, window=64,
                   layers=("full", "reuse", "reuse"), tail=W.TAIL_EXCLUDE)
    check(lib, cfg, seed=44)


def test_flat_topk_blocks_of_one_token_decode(lib):
    """Flat Top-K: blocks of one token and a pool of K blocks select the K
    best tokens of a 40,000-token prefix (more blocks than one workgroup holds
    in registers)."""
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=3, ctx=40000, block=1, pool=512, top_k=512)
    check(lib, cfg, seed=45)


def test_flat_topk_blocks_of_one_token_prefill(lib):
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=600, block=1, pool=64, top_k=64, window=32,
                   layers=("full", "reuse"))
    check(lib, cfg, seed=46)


@pytest.mark.parametrize("B", [3, 5, 7, 12])
def test_decode_block_sizes_not_a_power_of_two(lib, B):
    """Blocks of 3 to 12 tokens in the decode layer group: each pool/token
    scoring workgroup takes a whole number of pool slots, so its candidate
    range is not a power of two; the query's own block is partial for most B."""
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=3, ctx=9001, block=B, pool=300, top_k=256, window=64,
                   layers=("full", "reuse", "reuse"))
    check(lib, cfg, seed=60 + B)


def test_prefill_block_size_not_a_power_of_two(lib):
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=700, block=5, pool=40, top_k=64, window=32,
                   layers=("full", "reuse"))
    check(lib, cfg, seed=59)


def test_prefill_dense_topk_two_sequences(lib):
    """Pool covering every block: the MFMA tile Top-K, with a workgroup tile
    that holds queries of both sequences (1,000 is not a multiple of 16)."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], n_seq=2, ctx=1000, pool=256, top_k=200, window=64,
                   layers=("full", "reuse"))
    check(lib, cfg, seed=31)


def test_prefill_dense_topk_tie_heavy_d32(lib):
    """Indexer values in {-1, 0, 1} at d_idx 32: thousands of equal scores, so
    most queries take their last entries from a long run of ties."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=2000, d_idx=32, pool=256, top_k=300, window=32,
                   layers=("full",))
    check(lib, cfg, seed=32, int_range=(-1, 1))


def test_prefill_dense_topk_longest_context(lib):
    """16,384 tokens with a pool of 2,048 blocks: the longest context the
    tile Top-K takes; sampled rows."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=16384, layers=("full",))
    rng = np.random.default_rng(33)
    edges = [0, 1, 15, 16, 17, 511, 512, 513, 4095, 8191, 12000, 16367, 16368, 16383]
    rows = np.unique(np.concatenate([edges, rng.choice(cfg.n_q, 40, replace=False)]))
    check(lib, cfg, seed=33, rows=rows)


def test_decode_more_blocks_than_one_workgroup_holds(lib):
    """Blocks of 2 at a 40,000-token context: 20,000 eligible blocks, more than
    16,384 keys per selection workgroup, so the layer group keeps 32 block keys
    per thread of its pool selection."""
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=2, ctx=40000, block=2, pool=4096, top_k=512)
    check(lib, cfg, seed=34)


def test_decode_group_256k_batch_8(lib):
    """The 128K layer group's shapes (batch 8, Full + 5 Reuse, blocks of 8,
    pool 2,048, Top-512, window 128) at a 262,144-token context: 32,768
    eligible blocks per query, the most the fused layer group takes."""
    check(lib, W.CONFIGS["decode_group_256k"])


def test_decode_past_the_fused_limit(lib):
    """280,000 tokens in blocks of 8 (35,000 eligible blocks, past the fused
    layer group's 32,768): the block pass, pool selection, token Top-K and
    attention run as separate launches, and the pool is chosen by the
    streaming two-pass path over the workspace keys."""
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=2, ctx=280000, layers=("full", "reuse"))
    check(lib, cfg, seed=35)


def test_prefill_window_layer_chunks_and_mixed_tiles(lib):
    """Window-only layers take the shared-window kernel: a 300-token window is
    wider than one staged chunk of rows, and with two prompts of 1,003 tokens
    some 8-query tiles hold queries of both sequences."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], n_seq=2, ctx=1003, pool=128, top_k=200, window=300,
                   layers=("full", "swa"))
    check(lib, cfg, seed=35)


def test_prefill_window_runs_of_tiles(lib):
    """Enough window-layer tiles that each workgroup walks a run of them: a
    tile continuing the previous one adds only its new rows to the ring; runs
    cross the two head groups and the edges of three 1,501-token prompts,
    where tiles mix sequences and the next tile is staged whole."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], n_seq=3, ctx=1501, pool=128, top_k=200, window=128, n_heads=32,
                   layers=("full", "swa"))
    check(lib, cfg, seed=38)


def test_prefill_window_long_runs(lib):
    """Two 9,001-token prompts: nine tiles per workgroup, more than one load of
    query positions covers, so the run reloads them midway."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], n_seq=2, ctx=9001, pool=256, top_k=128, window=64,
                   layers=("full", "swa"))
    check(lib, cfg, seed=39)


def test_token_only_reindex_decode(lib):
    """A token-only Reindex group reads the Full group's pool and writes its
    own Top-K; the Reuse layer after it takes those indices."""
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=3, ctx=9000, pool=256,
                   layers=("full", "reuse", "reindex_tokens", "reuse"))
    check(lib, cfg, seed=36)


def test_token_only_reindex_prefill_whole_prefix_pools(lib):
    """In prefill with every pool the whole prefix, the token-only Reindex runs
    the MFMA tile Top-K with its own indexer query."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=1200, pool=256, top_k=128, window=64,
                   layers=("full", "reindex_tokens", "swa"))
    check(lib, cfg, seed=37)


def test_no_window(lib):
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=3, ctx=4096, pool=64, top_k=128, window=0)
    check(lib, cfg, seed=27)


def test_two_head_groups_and_generic_kernels(lib):
    # H = 32: two 16-head groups on the MFMA path
    check(lib, W.scaled(W.CONFIGS["decode_full_32k"], n_seq=2, ctx=3000, pool=64, top_k=128, n_heads=32), seed=28)
    # D = 64 bf16 and H = 8: the generic kernel
    check(lib, W.scaled(W.CONFIGS["decode_full_32k"], n_seq=2, ctx=3000, pool=64, top_k=128, n_heads=8,
                        head_dim=64), seed=29)


def test_decoder_pattern_scaled(lib):
    cfg = W.scaled(W.CONFIGS["decoder_pattern_64k"], n_seq=2, ctx=6000, pool=200)
    check(lib, cfg, seed=30)


def test_fp32_decode_long(lib):
    cfg = W.scaled(W.CONFIGS["tiny_full_fp32"], n_seq=2, ctx=20000, decode=True, pool=300, top_k=128, window=64)
    check(lib, cfg, seed=31)


# ------------------------------------------------------------------ single calls
def test_block_keys_bit_exact(lib):
    B, _ = lib
    rng = np.random.default_rng(32)
    for blk, d in ((8, 64), (2, 32), (16, 64), (5, 32)):
        k = rng.integers(-128, 128, size=(3, 203, d), dtype=np.int8)
        T = k.shape[1]
        cfg = B.Cfg(block=blk, pool=4, top_k=8, window=4, d_idx=d)
        kd = torch.from_numpy(k).cuda()
        kb = torch.full((3, T // blk, d), 77, dtype=torch.int8, device="cuda")
        B.csa2_build_block_keys(cfg, kd, kb, 1, T // blk - 1)
        got = kb.cpu().numpy()
        for s in range(3):
            for j in range(T // blk):
                want = oracle.block_key(k[s], blk, j, T - 1) if 1 <= j < T // blk - 1 else np.full(d, 77, np.int8)
                assert np.array_equal(got[s, j], want), (blk, d, s, j)


def test_golden_toy_selection(lib):
    B, _ = lib
    g = json.load(open(GOLDEN))
    k = np.zeros((1, g["T"], 32), np.int8)
    k[0, :, 0] = g["k_idx"]
    kd = torch.from_numpy(k).cuda()
    for case in g["cases"]:
        P = case.get("pool_override", g["pool"])
        cfg = B.Cfg(block=g["block"], pool=P, top_k=g["top_k"], window=g["window"], d_idx=32)
        q = np.zeros((1, 32), np.int8)
        q[0, 0] = case["q_idx"]
        qd = torch.from_numpy(q).cuda()
        seq = torch.zeros(1, dtype=torch.int32, device="cuda")
        pos = torch.full((1,), case["t"], dtype=torch.int32, device="cuda")
        kb = torch.zeros((1, g["T"] // g["block"], 32), dtype=torch.int8, device="cuda")
        B.csa2_build_block_keys(cfg, kd, kb)
        ids = torch.empty((1, P), dtype=torch.int32, device="cuda")
        cnt = torch.empty(1, dtype=torch.int32, device="cuda")
        tk = torch.empty((1, g["top_k"]), dtype=torch.int32, device="cuda")
        tc = torch.empty(1, dtype=torch.int32, device="cuda")
        ws = B.new_workspace(cfg, 1, g["T"])
        B.csa2_index_blocks(cfg, qd, seq, pos, kd, kb, ids, cnt, ws)
        B.csa2_topk_tokens(cfg, qd, seq, pos, kd, ids, cnt, tk, tc, ws)
        torch.cuda.synchronize()
        assert ids[0, :cnt.item()].tolist() == case["pool"], case["name"]
        assert tk[0, :tc.item()].tolist() == case["topk"], case["name"]


def test_reuse_equals_attend_with_full_indices(lib):
    """The layer group's Reuse layers equal single attend calls that take the
    Full layer's indices (and the group call equals per-layer calls)."""
    B, pipeline = lib
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=4, ctx=9000, pool=256)
    wl = W.generate(cfg, seed=33)
    dw = pipeline.upload(wl)
    pipeline.build_cache(dw)
    pipeline.run(dw)
    grp = dw.groups[0]
    for j in range(len(grp.layers)):
        out = torch.empty_like(grp.out[j])
        lse = torch.empty_like(grp.lse[j])
        B.csa2_attend(dw.lcfg, grp.q[j].contiguous(), dw.q_seq, dw.q_pos, dw.k_main, dw.v_main,
                      grp.k_swa[j].contiguous(), grp.v_swa[j].contiguous(), cfg.swa_first, dw.topk[0],
                      dw.topk_cnt[0], out, lse, dw.ws)
        torch.cuda.synchronize()
        assert torch.equal(out, grp.out[j]), j
        assert torch.equal(lse, grp.lse[j]), j


def test_deterministic_bitwise(lib):
    B, pipeline = lib
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=3, ctx=20000, pool=512)
    wl = W.generate(cfg, seed=34)
    dw = pipeline.upload(wl)
    pipeline.build_cache(dw)
    outs = []
    for _ in range(3):
        pipeline.run(dw)
        torch.cuda.synchronize()
        outs.append((dw.groups[0].out.clone(), dw.topk[0].clone(), dw.blk_ids[0].clone()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


def test_empty_query_batch_is_a_no_op(lib):
    B, _ = lib
    cfg = B.Cfg(pool=64)
    e8 = torch.empty((0, 64), dtype=torch.int8, device="cuda")
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    k = torch.zeros((1, 1024, 64), dtype=torch.int8, device="cuda")
    kb = torch.zeros((1, 128, 64), dtype=torch.int8, device="cuda")
    ids = torch.empty((0, 64), dtype=torch.int32, device="cuda")
    B.csa2_index_blocks(cfg, e8, e32, e32, k, kb, ids, e32, None)
    torch.cuda.synchronize()


def test_full_mode_stores_the_block_a_query_completes(lib):
    """A decode step in Full mode writes the key of the block its newest token
    completes (and only that block), so the next step finds k_blk current."""
    B, pipeline = lib
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=3, ctx=4096, pool=64, top_k=128)
    wl = W.generate(cfg, seed=35)
    dw = pipeline.upload(wl)
    nblk = cfg.ctx // cfg.block
    pipeline.build_cache(dw, upto_block=nblk - 1)      # the last block's key is still zero
    before = dw.k_blk.clone()
    pipeline.run(dw)
    torch.cuda.synchronize()
    after = dw.k_blk.cpu().numpy()
    for s in range(cfg.n_seq):
        want = oracle.block_key(wl.k_idx[s], cfg.block, nblk - 1, cfg.ctx - 1)
        assert np.array_equal(after[s, nblk - 1], want)
    assert torch.equal(dw.k_blk[:, :nblk - 1], before[:, :nblk - 1])
    # and the selection of that step already used the right key
    ref = oracle.run_layers(wl)
    got = pipeline.outputs(dw)
    assert_index_equal(got["index"][0], ref["index"][0], what="completed block")


@pytest.mark.parametrize("name,kw", [
    ("decode_group_128k", dict(n_seq=4, ctx=40000, layers=("full", "reuse", "reuse"))),
    ("decode_full_32k", dict(n_seq=3, ctx=5001, pool=300, top_k=700, window=100)),
    ("decode_full_32k", dict(n_seq=2, ctx=900, pool=2048)),            # pool covers every block
    ("decode_group_128k", dict(n_seq=3, ctx=12000, pool=256, layers=("reindex", "reuse"))),
    # 42 queries x 6 layers = 252 items: the most the chunked attention of
    # the fused layer group takes
    ("decode_group_128k", dict(n_seq=42, ctx=3000, pool=128)),
])
def test_fused_layer_group_equals_separate_calls(lib, name, kw):
    """The layer-group call (fused decode launches) and the separate calls
    (block pass, token Top-K, attention) give identical indices and outputs."""
    B, pipeline = lib
    cfg = W.scaled(W.CONFIGS[name], **kw)
    wl = W.generate(cfg, seed=36)
    dw = pipeline.upload(wl)
    pipeline.build_cache(dw)
    pipeline.run(dw)                    # csa2_layer_group
    torch.cuda.synchronize()
    grp = dw.groups[0]
    lc = dw.lcfg
    ids = torch.empty((cfg.n_q, cfg.pool), dtype=torch.int32, device="cuda"); cnt = torch.empty_like(dw.blk_cnt[0])
    tk = torch.empty_like(dw.topk[0]); tc = torch.empty_like(dw.topk_cnt[0])
    out = torch.empty_like(grp.out); lse = torch.empty_like(grp.lse)
    B.csa2_index_blocks(lc, grp.q_idx, dw.q_seq, dw.q_pos, dw.k_idx, dw.k_blk, ids, cnt, dw.ws)
    B.csa2_topk_tokens(lc, grp.q_idx, dw.q_seq, dw.q_pos, dw.k_idx, ids, cnt, tk, tc, dw.ws)
    B.csa2_attend_group(lc, grp.q, dw.q_seq, dw.q_pos, dw.k_main, dw.v_main, grp.k_swa, grp.v_swa,
                        cfg.swa_first, tk, tc, out, lse, dw.ws)
    torch.cuda.synchronize()
    assert torch.equal(cnt, dw.blk_cnt[0])
    if dw.blk_ids[0] is not None:
        assert torch.equal(ids, dw.blk_ids[0])
    else:   # the layer group stored no ids: the standalone pass writes blocks 0 .. cnt-1
        slots = torch.arange(cfg.pool, device="cuda", dtype=torch.int32)[None, :]
        assert torch.equal(ids, torch.where(slots < cnt[:, None], slots, torch.full_like(slots, -1)))
    assert torch.equal(tc, dw.topk_cnt[0]) and torch.equal(tk, dw.topk[0])
    assert torch.equal(out, grp.out) and torch.equal(lse, grp.lse)
    ref = oracle.run_layers(wl)
    compare_run(pipeline.outputs(dw), ref, cfg, what="fused")


@pytest.mark.parametrize("decode", [False, True])
def test_unstored_pool_ids_give_the_same_selection(lib, decode):
    """Every pool is the whole prefix: a layer group that stores the pool ids
    and one that stores none (blk_cnt describes the pool) select the same
    tokens and attend identically; the stored ids are blocks 0 .. cnt-1."""
    B, pipeline = lib
    base = W.CONFIGS["decode_full_32k" if decode else "prefill_8k"]
    kw = dict(n_seq=5, ctx=1500, pool=200, top_k=300, window=50) if decode else \
        dict(ctx=1500, pool=200, top_k=300, window=50, layers=("full", "reuse"))
    cfg = W.scaled(base, **kw)
    print(f"case unstored pool ids decode={decode} n_q={cfg.n_q}", flush=True)
    wl = W.generate(cfg, seed=37)
    dw = pipeline.upload(wl)
    pipeline.build_cache(dw)
    assert dw.blk_ids[0] is None                    # the pipeline stores none here
    pipeline.run(dw)
    torch.cuda.synchronize()
    grp = dw.groups[0]
    ids = torch.full((cfg.n_q, cfg.pool), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty_like(dw.blk_cnt[0])
    tk = torch.empty_like(dw.topk[0]); tc = torch.empty_like(dw.topk_cnt[0])
    out = torch.empty_like(grp.out); lse = torch.empty_like(grp.lse)
    B.csa2_layer_group(dw.lcfg, "full", grp.q_idx, dw.q_seq, dw.q_pos, dw.k_idx, dw.k_blk,
                       pipeline.step_update_begin(dw), grp.q, dw.k_main, dw.v_main, grp.k_swa, grp.v_swa,
                       cfg.swa_first, ids, cnt, tk, tc, out, lse, dw.ws)
    torch.cuda.synchronize()
    assert torch.equal(cnt, dw.blk_cnt[0])
    assert torch.equal(tk, dw.topk[0]) and torch.equal(tc, dw.topk_cnt[0])
    assert torch.equal(out, grp.out) and torch.equal(lse, grp.lse)
    slots = torch.arange(cfg.pool, device="cuda", dtype=torch.int32)[None, :]
    assert torch.equal(ids, torch.where(slots < cnt[:, None], slots, torch.full_like(slots, -1)))
    compare_run(pipeline.outputs(dw), oracle.run_layers(wl), cfg, what="unstored pool ids")


@pytest.mark.parametrize("decode", [False, True])
def test_layer_group_leaves_every_completed_block_key(lib, decode):
    """After a Full layer group whose queries complete blocks (every position
    of a prompt, or the newest token of decode), k_blk holds the key of every
    complete block, bit-exact, without a bulk block-key launch; a prompt's
    layer group starts from zeroed block keys."""
    B, pipeline = lib
    if decode:
        cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=3, ctx=4096, pool=64, top_k=128)
    else:
        cfg = W.scaled(W.CONFIGS["prefill_8k"], n_seq=2, ctx=1003, pool=200, top_k=100, window=40,
                       layers=("full", "reuse"))
    print(f"case completed block keys decode={decode} S={cfg.n_seq} T={cfg.ctx}", flush=True)
    wl = W.generate(cfg, seed=38)
    dw = pipeline.upload(wl)
    nblk = cfg.ctx // cfg.block
    if decode:
        pipeline.build_cache(dw, upto_block=nblk - 1)   # the newest token completes the last block
    assert pipeline.step_update_begin(dw) == nblk     # no bulk rebuild inside the step
    pipeline.run(dw)
    torch.cuda.synchronize()
    got = dw.k_blk.cpu().numpy()
    for s in range(cfg.n_seq):
        for j in range(nblk):
            want = oracle.block_key(wl.k_idx[s], cfg.block, j, cfg.ctx - 1)
            assert np.array_equal(got[s, j], want), (s, j)
    compare_run(pipeline.outputs(dw), oracle.run_layers(wl), cfg, what="completed block keys")


def test_prefill_dense_topk_extreme_scores(lib):
    """int8 values of -128 (the ABI accepts them): a block of rows and
    queries of all -128 scores exactly 2^20, the one score in the top bin of
    the dense Top-K's first pass; the rest of the prompt draws in [-127, 127]
    and ties are broken by position."""
    _, pipeline = lib
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=1000, pool=200, top_k=96, window=16, layers=("full",))
    wl = W.generate(cfg, seed=39)
    wl.k_idx[0, 100:400] = -128
    wl.q_idx[0][500:] = -128
    print(f"case dense Top-K with scores of 2^20: n_q={cfg.n_q}", flush=True)
    got = run_gpu(pipeline, wl)
    compare_run(got, oracle.run_layers(wl), cfg, what="extreme scores")


@pytest.mark.parametrize("top_k", [700, 1100])
def test_prefill_dense_topk_wide_k(lib, top_k):
    """Whole-prefix pools with a Top-K longer than the dense kernel's 512-slot
    output stage: every query's entries are written in several rounds."""
    _, pipeline = lib
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=2000, pool=256, top_k=top_k, window=64, layers=("full",))
    wl = W.generate(cfg, seed=41)
    print(f"case dense Top-K K={top_k}: n_q={cfg.n_q} T={cfg.ctx}", flush=True)
    got = run_gpu(pipeline, wl)
    compare_run(got, oracle.run_layers(wl), cfg, what=f"dense Top-K K={top_k}")


@pytest.mark.parametrize("kind", ["equal_scores", "zero_strided_rows"])
def test_prefill_dense_topk_adversarial(lib, kind):
    """Prompts far from random scores: every key row equal (every query's
    scores tie, so the K-th key's bin holds far more keys than a per-query
    list, and the ties are taken lowest position first), and zero rows in
    every fourth run of 64 positions (a strided sample of the prefix would
    put the K-th key near score 0, while the prefix's K best lie far above
    it)."""
    _, pipeline = lib
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=3000, layers=("full",))
    wl = W.generate(cfg, seed=40)
    if kind == "equal_scores":
        wl.k_idx[0, :] = wl.k_idx[0, 7]
    else:
        pos = np.arange(cfg.ctx)
        wl.k_idx[0, (pos // 64) % 4 == 0] = 0
    print(f"case dense Top-K adversarial ({kind}): n_q={cfg.n_q} T={cfg.ctx}", flush=True)
    got = run_gpu(pipeline, wl)
    compare_run(got, oracle.run_layers(wl), cfg, what=f"adversarial ({kind})")


# ------------------------------------------------------------------ compressed main-KV
# CSA2(ratio, mode): the main-KV and indexer caches hold one entry per `ratio`
# tokens (entry j = tokens j*ratio .. j*ratio + ratio - 1), a query at token t
# selects among the entries complete at t, and its window stays per token.
def test_compressed_decode_layer_group_128k(lib):
    """The 128K layer group at ratio 4: 32,768 entries, 4,096 eligible blocks
    per query through the fused layer group."""
    check(lib, W.CONFIGS["decode_group_128k_c4"])


def test_compressed_decode_ragged_context(lib):
    """A context that is no multiple of the ratio (the newest tokens form an
    incomplete entry that only the window holds) nor of the block; ratio 3,
    pool below the eligible blocks, several workgroups per query."""
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=5, ctx=20002, pool=96, top_k=100, window=37, ratio=3)
    check(lib, cfg, seed=51)


def test_compressed_decode_past_the_fused_limit(lib):
    """Ratio 2 at 600,000 tokens: 300,000 entries in blocks of 8 (37,500
    eligible blocks) take the separate launches."""
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=2, ctx=600000, layers=("full", "reuse"), ratio=2)
    check(lib, cfg, seed=52)


def test_compressed_reindex_and_token_only_reindex_decode(lib):
    """Reindex and token-only Reindex layers over compressed caches (ratio
    3): fresh pool and Top-K, and a fresh Top-K over the shared pool, each
    followed by a Reuse layer, in the fused layer group."""
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=3, ctx=24002, pool=256, top_k=300, window=64,
                   layers=("full", "reuse", "reindex", "reuse", "reindex_tokens", "reuse"), ratio=3)
    check(lib, cfg, seed=60)


def test_compressed_reindex_and_token_only_reindex_prefill(lib):
    """The same layer kinds over a compressed 1,201-token prompt (ratio 2,
    pool below the eligible blocks): separate block pass, pool selection and
    token Top-K launches."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=1201, pool=40, top_k=96, window=48,
                   layers=("full", "reindex", "reuse", "reindex_tokens", "reuse"), ratio=2)
    check(lib, cfg, seed=61)


@pytest.mark.parametrize("tail", [W.TAIL_VISIBLE, W.TAIL_EXCLUDE, W.TAIL_WHOLE])
def test_compressed_prefill_block_pass(lib, tail):
    """Every token of a 1,501-token prompt at ratio 3 (500 entries) with a pool
    below the eligible blocks: block pass, pool selection and per-query token
    Top-K over entries; the first two tokens see no entry and attend to their
    window alone."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=1501, pool=24, top_k=64, window=40,
                   layers=("full", "reuse", "swa"), ratio=3, tail=tail)
    check(lib, cfg, seed=53 + tail)


@pytest.mark.parametrize("tail", [W.TAIL_VISIBLE, W.TAIL_EXCLUDE, W.TAIL_WHOLE])
def test_compressed_prefill_whole_prefix_pools(lib, tail):
    """A 3,001-token prompt at ratio 4 (750 entries): whole-prefix pools, the
    dense token Top-K over entries and the row attention, four queries per
    entry."""
    cfg = W.scaled(W.CONFIGS["prefill_8k_c4"], ctx=3001, tail=tail, layers=("full", "reuse", "swa"))
    check(lib, cfg, seed=56 + tail)


def test_compressed_prefill_8k_all_rows(lib):
    check(lib, W.CONFIGS["prefill_8k_c4"])


@pytest.mark.parametrize("decode", [False, True])
def test_compressed_layer_group_leaves_every_completed_block_key(lib, decode):
    """With compressed caches a Full layer group stores the key of every entry
    block its queries complete (a block is complete once its last entry is),
    bit-exact, and leaves the others alone."""
    B, pipeline = lib
    if decode:
        cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=3, ctx=4096, pool=64, top_k=128, ratio=4)
    else:
        cfg = W.scaled(W.CONFIGS["prefill_8k"], n_seq=2, ctx=1003, pool=200, top_k=100, window=40,
                       layers=("full", "reuse"), ratio=3)
    print(f"case compressed block keys decode={decode} S={cfg.n_seq} T={cfg.ctx} r={cfg.ratio}", flush=True)
    wl = W.generate(cfg, seed=59)
    dw = pipeline.upload(wl)
    n = cfg.main_len
    nblk = n // cfg.block
    if decode:
        pipeline.build_cache(dw, upto_block=nblk - 1)   # the newest entry completes the last block
    assert pipeline.step_update_begin(dw) == nblk
    pipeline.run(dw)
    torch.cuda.synchronize()
    got = dw.k_blk.cpu().numpy()
    for s in range(cfg.n_seq):
        for j in range(nblk):
            want = oracle.block_key(wl.k_idx[s], cfg.block, j, n - 1)
            assert np.array_equal(got[s, j], want), (s, j)
    compare_run(pipeline.outputs(dw), oracle.run_layers(wl), cfg, what="compressed block keys")
