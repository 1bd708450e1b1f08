"""Pins of the CPU oracle against things other than itself.

* rounding: Python's exact ``round(Fraction)`` (ties to even) and hand ties;
* block keys: closed forms (constant blocks), numpy's round-half-even on exact
  means, and the partial-block rule on a hand case;
* pool and Top-K: exhaustive enumeration on tiny inputs (``brute.py``), the
  flat special case against ``numpy.lexsort``, the hand toy in
  ``golden/toy16.json``, and invariants on random data;
* attention: textbook dense causal attention and sliding-window attention from
  ``torch.nn.functional.scaled_dot_product_attention`` (fp64, CPU), dense
  attention over the concatenated key set, Q = 0 giving the mean of the
  attended values, one-hot values recovering the attended set, and the toy's
  470/7;
* modes: Reuse equals attention with the Full layer's indices; Reindex with the
  Full layer's indexer query reproduces its indices; and the layer sequencing
  of ``run_layers`` (a Reuse layer after a Reindex or token-only Reindex layer
  takes that layer's fresh indices, window-only layers attend to their window
  alone wherever they sit, each Full layer opens its own cache) against each
  layer recomputed from scratch by enumeration and fp64 SDPA.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from brute import block_key_exact, dot, select_brute, top_n_by_enumeration
from top_kv_selection_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "toy16.json")


# ---------------------------------------------------------------- rounding
def test_round_half_even_matches_exact_fraction_rounding():
    for n in range(1, 17):
        for s in range(-128 * n, 127 * n + 1):
            assert oracle.round_half_even_div(s, n) == round(Fraction(s, n)), (s, n)


@pytest.mark.parametrize("s,n,want", [
    (4, 8, 0), (-4, 8, 0), (12, 8, 2), (-12, 8, -2), (20, 8, 2), (-20, 8, -2),
    (3, 2, 2), (-3, 2, -2), (1, 2, 0), (-1, 2, 0), (3, 6, 0), (9, 6, 2), (-9, 6, -2),
    (5, 8, 1), (-5, 8, -1), (3, 8, 0), (-3, 8, 0), (127 * 8, 8, 127), (-127 * 8, 8, -127),
])
def test_round_half_even_hand_cases(s, n, want):
    assert oracle.round_half_even_div(s, n) == want


# ---------------------------------------------------------------- block keys
def test_block_key_constant_block_is_that_constant():
    rng = np.random.default_rng(0)
    for B in (2, 4, 8, 16):
        for _ in range(20):
            row = rng.integers(-127, 128, size=32, dtype=np.int8)
            k = np.tile(row, (B * 3, 1))
            for j in range(3):
                assert (oracle.block_key(k, B, j, 3 * B - 1) == row).all()


def test_block_key_matches_numpy_round_of_exact_mean():
    rng = np.random.default_rng(1)
    for B in (2, 4, 8, 16):
        k = rng.integers(-127, 128, size=(B * 8, 64), dtype=np.int8)
        t = B * 8 - 1
        for j in range(8):
            mean = k[j * B:(j + 1) * B].astype(np.float64).mean(axis=0)
            assert (oracle.block_key(k, B, j, t) == np.round(mean).astype(np.int8)).all()


def test_block_key_partial_block_uses_visible_rows_only():
    rng = np.random.default_rng(2)
    k = rng.integers(-127, 128, size=(40, 8), dtype=np.int8)
    for B in (2, 8, 16):
        for t in range(40):
            j = t // B
            got = oracle.block_key(k, B, j, t)
            assert list(got) == block_key_exact(k, B, j, t)
            # a future row must not change the key
            k2 = k.copy()
            if t + 1 < 40:
                k2[t + 1] = -k2[t + 1] // 2 + 7
                assert (oracle.block_key(k2, B, j, t) == got).all()


def test_block_key_ties_to_even_per_dimension():
    # sums over 8 rows of +4, -4, +12, -12 -> means 0.5, -0.5, 1.5, -1.5 -> 0, 0, 2, -2
    k = np.zeros((8, 4), np.int8)
    k[0] = [4, -4, 12, -12]
    assert list(oracle.block_key(k, 8, 0, 7)) == [0, 0, 2, -2]


# ---------------------------------------------------------------- selection
def _tiny_cases(seed, n, lo=-2, hi=2):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        B = int(rng.choice([2, 4]))
        T = int(rng.integers(2, 19))
        d = int(rng.integers(1, 4))
        P = int(rng.integers(1, 5))
        K = int(rng.integers(1, 4))
        k = rng.integers(lo, hi + 1, size=(T, d), dtype=np.int8)
        q = rng.integers(lo, hi + 1, size=d, dtype=np.int8)
        t = int(rng.integers(0, T))
        yield B, T, d, P, K, k, q, t


def test_select_matches_enumeration_on_tiny_tie_heavy_inputs():
    for B, T, d, P, K, k, q, t in _tiny_cases(3, 300):
        blk, bc, tk, tc = oracle.select(q[None], [0], [t], k[None], B, P, K)
        pool, top = select_brute(q, k, t, B, P, K)
        assert list(blk[0, :bc[0]]) == pool
        assert (blk[0, bc[0]:] == -1).all()
        assert list(tk[0, :tc[0]]) == top
        assert (tk[0, tc[0]:] == -1).all()


def test_select_matches_enumeration_wide_value_range():
    for B, T, d, P, K, k, q, t in _tiny_cases(4, 150, -127, 127):
        blk, bc, tk, tc = oracle.select(q[None], [0], [t], k[None], B, P, K)
        pool, top = select_brute(q, k, t, B, P, K)
        assert list(blk[0, :bc[0]]) == pool
        assert list(tk[0, :tc[0]]) == top


@pytest.mark.parametrize("tail", [oracle.TAIL_EXCLUDE, oracle.TAIL_WHOLE])
def test_tail_block_readings_match_enumeration(tail):
    """The two other readings of a partial own block (not eligible; keyed by
    the whole block including rows after t) against enumeration."""
    for B, T, d, P, K, k, q, t in _tiny_cases(11 + tail, 250):
        blk, bc, tk, tc = oracle.select(q[None], [0], [t], k[None], B, P, K, tail=tail)
        pool, top = select_brute(q, k, t, B, P, K, tail)
        assert list(blk[0, :bc[0]]) == pool, (B, T, t)
        assert (blk[0, bc[0]:] == -1).all()
        assert list(tk[0, :tc[0]]) == top, (B, T, t)
        assert (tk[0, tc[0]:] == -1).all()


def test_tail_readings_agree_when_the_own_block_is_complete():
    rng = np.random.default_rng(17)
    for _ in range(200):
        B = int(rng.choice([2, 4, 8]))
        T = B * int(rng.integers(1, 6))
        k = rng.integers(-4, 5, size=(T, 3), dtype=np.int8)
        q = rng.integers(-4, 5, size=3, dtype=np.int8)
        t = B * int(rng.integers(1, T // B + 1)) - 1          # last position of a block
        P, K = int(rng.integers(1, 4)), int(rng.integers(1, 6))
        base = oracle.select(q[None], [0], [t], k[None], B, P, K)
        for tail in (oracle.TAIL_EXCLUDE, oracle.TAIL_WHOLE):
            got = oracle.select(q[None], [0], [t], k[None], B, P, K, tail=tail)
            for a, b in zip(base, got):
                assert (a == b).all(), (B, T, t, tail)


def test_excluding_the_partial_block_is_selecting_at_its_last_complete_position():
    """Without the partial own block the eligible blocks, their keys and the
    candidates are those of a query at the last position of the previous
    block (same indexer query)."""
    rng = np.random.default_rng(18)
    for _ in range(300):
        B = int(rng.choice([2, 4, 8]))
        T = int(rng.integers(B + 1, 6 * B))
        k = rng.integers(-3, 4, size=(T, 2), dtype=np.int8)
        q = rng.integers(-3, 4, size=2, dtype=np.int8)
        t = int(rng.integers(B, T))
        if (t + 1) % B == 0:
            continue
        t_prev = (t + 1) // B * B - 1
        P, K = int(rng.integers(1, 4)), int(rng.integers(1, 6))
        got = oracle.select(q[None], [0], [t], k[None], B, P, K, tail=oracle.TAIL_EXCLUDE)
        want = oracle.select(q[None], [0], [t_prev], k[None], B, P, K)
        for a, b in zip(got, want):
            assert (a == b).all(), (B, T, t)


def test_block_size_one_with_pool_k_is_the_flat_topk():
    """Blocks of one token with a pool of K blocks select the K best tokens
    of the whole prefix directly (the flat Top-K variant): numpy.lexsort on
    (position, -score) over every visible token."""
    rng = np.random.default_rng(19)
    for _ in range(30):
        T = int(rng.integers(40, 3000))
        d = int(rng.choice([8, 32]))
        K = int(rng.integers(1, 64))
        k = rng.integers(-4, 5, size=(T, d), dtype=np.int8)   # narrow range: many ties
        q = rng.integers(-4, 5, size=d, dtype=np.int8)
        t = int(rng.integers(0, T))
        blk, bc, tk, tc = oracle.select(q[None], [0], [t], k[None], 1, K, K)
        scores = k[: t + 1].astype(np.int64) @ q.astype(np.int64)
        order = np.lexsort((np.arange(t + 1), -scores))
        want = np.sort(order[:K])
        assert list(tk[0, :tc[0]]) == list(want)
        assert list(blk[0, :bc[0]]) == list(want)


def test_token_topk_over_a_given_pool_matches_enumeration():
    """The token step alone, over arbitrary pools (any ascending subset of the
    eligible blocks, not only the hierarchical one)."""
    rng = np.random.default_rng(14)
    for B, T, d, P, K, k, q, t in _tiny_cases(5, 200):
        n_elig = t // B + 1
        n_pool = int(rng.integers(0, min(n_elig, P) + 1))
        pool = np.sort(rng.choice(n_elig, n_pool, replace=False)).astype(np.int32)
        blk = np.full((1, P), -1, np.int32)
        blk[0, :n_pool] = pool
        tk, tc = oracle.topk_given_pool(q[None], [0], [t], k[None], B, K, blk, [n_pool])
        cands = [(dot(q, k[p]), p) for j in pool for p in range(j * B, j * B + B) if p <= t]
        want = top_n_by_enumeration(cands, K) if cands else []
        assert list(tk[0, :tc[0]]) == want
        assert (tk[0, tc[0]:] == -1).all()


def test_token_only_reindex_keeps_the_pool_and_reselects_tokens():
    """A token-only Reindex layer shares the pool of the index set before it;
    with the Full layer's own query it reproduces the Full indices, and with
    its own query it takes the flat Top-K of the pool's candidates."""
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=3, ctx=2048, pool=32, top_k=40, window=16,
                   layers=("full", "reuse", "reindex_tokens", "reuse"))
    wl = W.generate(cfg, seed=15)
    res = oracle.run_layers(wl)
    full, tok = res["index"][0], res["index"][2]
    assert (tok["blk_ids"] == full["blk_ids"]).all() and (tok["blk_cnt"] == full["blk_cnt"]).all()
    for i in range(cfg.n_q):
        t = wl.q_pos[i]
        pool = full["blk_ids"][i, :full["blk_cnt"][i]]
        pos = np.array([p for j in pool for p in range(j * 8, j * 8 + 8) if p <= t])
        s = wl.k_idx[wl.q_seq[i], pos].astype(np.int64) @ wl.q_idx[2][i].astype(np.int64)
        want = np.sort(pos[np.lexsort((pos, -s))[:cfg.top_k]])
        assert (tok["topk"][i, :tok["topk_cnt"][i]] == want).all()
    same = W.generate(cfg, seed=15)
    same.q_idx[2] = same.q_idx[0].copy()
    res2 = oracle.run_layers(same)
    for key in ("topk", "topk_cnt"):
        assert (res2["index"][2][key] == res2["index"][0][key]).all()


def test_flat_case_is_lexsort_topk():
    """With the pool covering every eligible block the selection is a plain
    Top-K over the causal prefix: numpy.lexsort by (-score, position)."""
    rng = np.random.default_rng(5)
    T, d, B, K = 200, 16, 8, 20
    k = rng.integers(-3, 4, size=(1, T, d), dtype=np.int8)
    q = rng.integers(-3, 4, size=(T, d), dtype=np.int8)
    pos = np.arange(T, dtype=np.int32)
    blk, bc, tk, tc = oracle.select(q, np.zeros(T, np.int32), pos, k, B, T // B + 1, K)
    for t in range(T):
        s = (k[0, :t + 1].astype(np.int64) @ q[t].astype(np.int64))
        order = np.lexsort((np.arange(t + 1), -s))
        want = np.sort(order[:K])
        assert tc[t] == min(K, t + 1)
        assert (tk[t, :tc[t]] == want).all()
        assert bc[t] == t // B + 1


def test_golden_toy():
    g = json.load(open(GOLDEN))
    k = np.array(g["k_idx"], np.int8).reshape(1, g["T"], 1)
    assert [int(oracle.block_key(k[0], g["block"], j, 15)[0]) for j in range(8)] == g["block_keys_t15"]
    for case in g["cases"]:
        P = case.get("pool_override", g["pool"])
        q = np.array([[case["q_idx"]]], np.int8)
        blk, bc, tk, tc = oracle.select(q, [0], [case["t"]], k, g["block"], P, g["top_k"])
        assert list(blk[0, :bc[0]]) == case["pool"], case["name"]
        assert list(tk[0, :tc[0]]) == case["topk"], case["name"]
        if "block_scores" in case:
            t = case["t"]
            bs = [int(case["q_idx"]) * int(oracle.block_key(k[0], g["block"], j, t)[0])
                  for j in range(t // g["block"] + 1)]
            assert bs == case["block_scores"]
        # zero-padding the indexer dimension leaves every selection unchanged
        k32 = np.zeros((1, g["T"], 32), np.int8)
        k32[..., :1] = k
        q32 = np.zeros((1, 32), np.int8)
        q32[0, 0] = case["q_idx"]
        blk2, bc2, tk2, tc2 = oracle.select(q32, [0], [case["t"]], k32, g["block"], P, g["top_k"])
        assert (blk2 == blk).all() and (tk2 == tk).all()


def test_golden_toy_attention():
    g = json.load(open(GOLDEN))
    a = g["attention"]
    D = 1
    T = g["T"]
    q = np.zeros((1, 1, D), np.float32)
    v_main = np.arange(T, dtype=np.float32).reshape(1, T, D)
    v_swa = (100 + np.arange(T, dtype=np.float32)).reshape(1, T, D)
    k_main = np.ones((1, T, D), np.float32)
    k_swa = np.ones((1, T, D), np.float32)
    topk = np.array([[2, 6, 8]], np.int32)
    out, lse = oracle.attend(q, [0], [15], k_main, v_main, k_swa, v_swa, 0, topk, [3], g["window"])
    assert out[0, 0, 0] == pytest.approx(a["out"], rel=1e-14)
    assert lse[0, 0] == pytest.approx(a["lse"], rel=1e-14)


def test_selection_invariants_random():
    cfg = W.scaled(W.CONFIGS["tiny_full_fp32"], ctx=300)
    wl = W.generate(cfg, seed=77)
    blk, bc, tk, tc = oracle.select(wl.q_idx[0], wl.q_seq, wl.q_pos, wl.k_idx, cfg.block,
                                    cfg.pool, cfg.top_k)
    k = wl.k_idx[0].astype(np.int64)
    for i in range(cfg.n_q):
        t = int(wl.q_pos[i])
        pool = blk[i, :bc[i]]
        sel = tk[i, :tc[i]]
        n_cand = sum(min(cfg.block, t - j * cfg.block + 1) for j in pool)
        assert bc[i] == min(cfg.pool, t // cfg.block + 1)
        assert tc[i] == min(cfg.top_k, n_cand)
        assert (np.diff(pool) > 0).all() and (np.diff(sel) > 0).all()
        assert (sel <= t).all() and (sel >= 0).all()
        assert set((sel // cfg.block).tolist()) <= set(pool.tolist())
        # every kept candidate beats every dropped one
        cands = [p for j in pool for p in range(j * cfg.block, min(j * cfg.block + cfg.block, t + 1))]
        s = {p: int(k[p] @ wl.q_idx[0][i].astype(np.int64)) for p in cands}
        kept = set(sel.tolist())
        dropped = [p for p in cands if p not in kept]
        if dropped:
            worst_kept = min(kept, key=lambda p: (s[p], -p))
            best_dropped = max(dropped, key=lambda p: (s[p], -p))
            assert (s[worst_kept], -worst_kept) > (s[best_dropped], -best_dropped)


# ---------------------------------------------------------------- attention
def _f64(a):
    return torch.from_numpy(np.asarray(a, np.float64))


def _rand_attn(seed, S=2, T=40, H=3, D=16, dtype="f32"):
    rng = np.random.default_rng(seed)
    mk = lambda *s: rng.standard_normal(s).astype(np.float32)
    arrs = [mk(S * T, H, D), mk(S, T, D), mk(S, T, D), mk(S, T, D), mk(S, T, D)]
    if dtype == "bf16":
        arrs = [W.f32_to_bf16_bits(a) for a in arrs]
    return arrs


def test_attend_dense_causal_equals_sdpa():
    """Top-K covering the prefix and no window: dense causal attention."""
    S, T, H, D = 2, 40, 3, 16
    q, km, vm, ks, vs = _rand_attn(6, S, T, H, D)
    q_seq = np.repeat(np.arange(S), T).astype(np.int32)
    q_pos = np.tile(np.arange(T), S).astype(np.int32)
    topk = np.full((S * T, T), -1, np.int32)
    cnt = np.zeros(S * T, np.int32)
    for i in range(S * T):
        t = q_pos[i]
        topk[i, :t + 1] = np.arange(t + 1)
        cnt[i] = t + 1
    out, lse = oracle.attend(q, q_seq, q_pos, km, vm, ks, vs, 0, topk, cnt, 0)
    for s in range(S):
        Q = _f64(q[s * T:(s + 1) * T]).permute(1, 0, 2)        # [H][T][D]
        K = _f64(km[s])[None].expand(H, T, D)
        V = _f64(vm[s])[None].expand(H, T, D)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
        np.testing.assert_allclose(out[s * T:(s + 1) * T], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
        logits = (Q @ K.transpose(1, 2)) / math.sqrt(D)
        logits = logits.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
        np.testing.assert_allclose(lse[s * T:(s + 1) * T], torch.logsumexp(logits, -1).T.numpy(), rtol=1e-12)


def test_attend_window_only_equals_banded_sdpa():
    """K = 0: textbook sliding-window attention over the layer's own K/V."""
    S, T, H, D, Wn = 1, 50, 2, 8, 7
    q, km, vm, ks, vs = _rand_attn(7, S, T, H, D)
    q_pos = np.arange(T, dtype=np.int32)
    out, _ = oracle.attend(q, np.zeros(T, np.int32), q_pos, km, vm, ks, vs, 0, None, None, Wn)
    i = torch.arange(T)
    allowed = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - Wn)
    Q = _f64(q).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q, _f64(ks[0])[None].expand(H, T, D), _f64(vs[0])[None].expand(H, T, D), attn_mask=allowed)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_attend_full_cover_plus_window_equals_concatenated_sdpa():
    S, T, H, D, Wn = 1, 30, 2, 8, 5
    q, km, vm, ks, vs = _rand_attn(8, S, T, H, D, "bf16")
    q_pos = np.arange(T, dtype=np.int32)
    topk = np.array([[p if p <= t else -1 for p in range(T)] for t in range(T)], np.int32)
    cnt = q_pos + 1
    out, _ = oracle.attend(q, np.zeros(T, np.int32), q_pos, km, vm, ks, vs, 0, topk, cnt, Wn)
    f = lambda a: _f64(W.bf16_bits_to_f32(a))
    Kc = torch.cat([f(km[0]), f(ks[0])], 0)             # [2T][D]
    Vc = torch.cat([f(vm[0]), f(vs[0])], 0)
    i = torch.arange(T)
    main_ok = i[None, :] <= i[:, None]
    win_ok = main_ok & (i[None, :] > i[:, None] - Wn)
    mask = torch.cat([main_ok, win_ok], 1)
    Q = f(q).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q, Kc[None].expand(H, 2 * T, D), Vc[None].expand(H, 2 * T, D), attn_mask=mask)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_attend_zero_query_is_mean_of_attended_values():
    S, T, H, D, Wn = 1, 64, 2, 4, 6
    _, km, vm, ks, vs = _rand_attn(9, S, T, H, D)
    q = np.zeros((1, H, D), np.float32)
    t = 50
    sel = np.array([[3, 17, 18, 40, 50]], np.int32)
    out, lse = oracle.attend(q, [0], [t], km, vm, ks, vs, 0, sel, [5], Wn)
    want = (vm[0, sel[0]].astype(np.float64).sum(0) + vs[0, t - Wn + 1:t + 1].astype(np.float64).sum(0)) / (5 + Wn)
    for h in range(H):
        np.testing.assert_allclose(out[0, h], want, rtol=1e-13)
        assert lse[0, h] == pytest.approx(math.log(5 + Wn), rel=1e-14)


def test_attend_one_hot_values_recover_the_attended_set():
    T, H, Wn = 24, 1, 4
    D = 2 * T
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    km = rng.standard_normal((1, T, D)).astype(np.float32)
    ks = rng.standard_normal((1, T, D)).astype(np.float32)
    vm = np.eye(T, D, dtype=np.float32)[None]            # main value p -> e_p
    vs = np.eye(T, D, k=T, dtype=np.float32)[None]       # window value p -> e_{T+p}
    t = 20
    sel = np.array([[1, 5, 9, 19]], np.int32)
    out, _ = oracle.attend(q, [0], [t], km, vm, ks, vs, 0, sel, [4], Wn)
    nz = set(np.nonzero(out[0, 0] > 0)[0].tolist())
    assert nz == {1, 5, 9, 19} | {T + p for p in range(t - Wn + 1, t + 1)}
    assert out[0, 0].sum() == pytest.approx(1.0, rel=1e-13)


def test_attend_rejects_window_not_covered():
    _, km, vm, ks, vs = _rand_attn(11, 1, 16, 1, 4)
    q = np.zeros((1, 1, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.attend(q, [0], [15], km, vm, ks[:, 10:], vs[:, 10:], 10, None, None, 8)


# ---------------------------------------------------------------- modes
def test_reuse_equals_attention_with_full_indices_and_reindex_same_query_same_indices():
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=3, ctx=2048, pool=64, top_k=40, window=16,
                   layers=("full", "reuse", "reindex", "reuse"))
    wl = W.generate(cfg, seed=12)
    wl.q_idx[2] = wl.q_idx[0].copy()
    res = oracle.run_layers(wl)
    full = res["index"][0]
    for key in ("blk_ids", "blk_cnt", "topk", "topk_cnt"):
        assert (res["index"][2][key] == full[key]).all()
    o, l = oracle.attend(wl.q[1], wl.q_seq, wl.q_pos, wl.k_main, wl.v_main, wl.k_swa[1],
                         wl.v_swa[1], cfg.swa_first, full["topk"], full["topk_cnt"], cfg.window)
    np.testing.assert_array_equal(o, res["out"][1])
    np.testing.assert_array_equal(l, res["lse"][1])


def test_hierarchy_changes_selection_only_through_the_pool():
    """Candidates outside the pool are never selected, and with the pool
    covering the prefix the result equals the flat Top-K."""
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=2, ctx=1024, pool=16, top_k=24)
    wl = W.generate(cfg, seed=13)
    blk, bc, tk, tc = oracle.select(wl.q_idx[0], wl.q_seq, wl.q_pos, wl.k_idx, 8, 16, 24)
    blk_f, bc_f, tk_f, tc_f = oracle.select(wl.q_idx[0], wl.q_seq, wl.q_pos, wl.k_idx, 8, 128, 24)
    for i in range(2):
        assert set((tk[i, :tc[i]] // 8).tolist()) <= set(blk[i, :bc[i]].tolist())
        assert bc_f[i] == 128
        t = wl.q_pos[i]
        s = wl.k_idx[i, :t + 1].astype(np.int64) @ wl.q_idx[0][i].astype(np.int64)
        want = np.sort(np.lexsort((np.arange(t + 1), -s))[:24])
        assert (tk_f[i, :tc_f[i]] == want).all()


# ---------------------------------------------------------------- layer-mode rules
# The mode table of "CSA2 with cross-layer reuse" (page "DeepSeek V4.1
# Flash"): a Full layer selects with its own indexer query over its own keys
# and opens its own main-KV/indexer cache, a Reindex layer selects afresh with
# its own query over the shared keys, a Reuse layer takes the indices of the
# most recent Full/Reindex layer, and every layer attends with its own Q and
# window K/V; window-only layers attend to the window alone.  These pins
# compute each layer's expected result from scratch (selection by enumeration,
# attention by torch's fp64 SDPA over the gathered rows) and compare
# run_layers with it, so a slip in the mode sequencing fails here.
def _mode_workload(layers, seed):
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=2, ctx=16, n_heads=2, head_dim=8, d_idx=32,
                   block=2, pool=4, top_k=3, window=4, layers=layers)
    return cfg, W.generate(cfg, seed=seed)


def _brute_sets(wl, layer, c):
    """(pool, Top-K) of indexing layer `layer` over cache c, per query, by enumeration."""
    cfg = wl.cfg
    k_idx = wl.cache(c)[0]
    return [select_brute(wl.q_idx[layer][i], k_idx[wl.q_seq[i]], int(wl.q_pos[i]), cfg.block, cfg.pool,
                         cfg.top_k, cfg.tail) for i in range(cfg.n_q)]


def _sdpa_layer(wl, layer, c, sets):
    """Output of layer `layer`: softmax attention of its Q over the main rows
    sets[i][1] of cache c (none when sets is None) and its own window rows."""
    cfg = wl.cfg
    f = (lambda a: _f64(W.bf16_bits_to_f32(a))) if cfg.dtype == "bf16" else _f64
    _, k_main, v_main = wl.cache(c)
    out = np.empty((cfg.n_q, cfg.n_heads, cfg.head_dim))
    for i in range(cfg.n_q):
        s, t = int(wl.q_seq[i]), int(wl.q_pos[i])
        rows = [] if sets is None else list(sets[i][1])
        win = [p - cfg.swa_first for p in range(max(0, t - cfg.window + 1), t + 1)]
        K = torch.cat([f(k_main[s])[rows], f(wl.k_swa[layer][s])[win]], 0)
        V = torch.cat([f(v_main[s])[rows], f(wl.v_swa[layer][s])[win]], 0)
        Q = f(wl.q[layer][i])[:, None, :]                                 # [H][1][D]
        H = cfg.n_heads
        o = torch.nn.functional.scaled_dot_product_attention(Q, K[None].expand(H, -1, -1),
                                                             V[None].expand(H, -1, -1))
        out[i] = o[:, 0, :].numpy()
    return out


def _assert_index(got, sets):
    for i, (pool, top) in enumerate(sets):
        assert got["blk_ids"][i, :got["blk_cnt"][i]].tolist() == pool
        assert got["topk"][i, :got["topk_cnt"][i]].tolist() == top
        assert (got["topk"][i, got["topk_cnt"][i]:] == -1).all()


def test_reuse_after_reindex_takes_the_reindex_indices():
    """Full, Reuse, Reindex, Reuse with a Reindex indexer query of its own:
    the second Reuse layer attends over the Reindex layer's fresh selection,
    not the Full layer's."""
    cfg, wl = _mode_workload(("full", "reuse", "reindex", "reuse"), seed=31)
    res = oracle.run_layers(wl)
    full, reidx = _brute_sets(wl, 0, 0), _brute_sets(wl, 2, 0)
    assert any(f[1] != r[1] for f, r in zip(full, reidx)), "the two index sets must differ"
    _assert_index(res["index"][0], full)
    _assert_index(res["index"][2], reidx)
    for layer, sets in ((0, full), (1, full), (2, reidx), (3, reidx)):
        np.testing.assert_allclose(res["out"][layer], _sdpa_layer(wl, layer, 0, sets), rtol=1e-12, atol=1e-12)
    assert not np.allclose(res["out"][3], _sdpa_layer(wl, 3, 0, full))


def test_window_only_layers_attend_to_their_window_alone():
    """Window-only layers before the first Full layer (the encoder's first two
    layers) and after a Full layer attend to their own window only, whatever
    index set is current."""
    cfg, wl = _mode_workload(("swa", "full", "reuse", "swa"), seed=32)
    res = oracle.run_layers(wl)
    full = _brute_sets(wl, 1, 0)
    _assert_index(res["index"][1], full)
    for layer, sets in ((0, None), (1, full), (2, full), (3, None)):
        np.testing.assert_allclose(res["out"][layer], _sdpa_layer(wl, layer, 0, sets), rtol=1e-12, atol=1e-12)
    assert not np.allclose(res["out"][3], _sdpa_layer(wl, 3, 0, full))


def test_each_full_layer_opens_its_own_cache():
    """Full, Reuse, Full, Reuse: the second Full layer selects over its own
    indexer keys and both it and the Reuse layer after it read its own main
    K/V, while the first pair keeps reading the first cache."""
    cfg, wl = _mode_workload(("full", "reuse", "full", "reuse"), seed=33)
    assert cfg.n_caches == 2
    res = oracle.run_layers(wl)
    first, second = _brute_sets(wl, 0, 0), _brute_sets(wl, 2, 1)
    _assert_index(res["index"][0], first)
    _assert_index(res["index"][2], second)
    for layer, c, sets in ((0, 0, first), (1, 0, first), (2, 1, second), (3, 1, second)):
        np.testing.assert_allclose(res["out"][layer], _sdpa_layer(wl, layer, c, sets), rtol=1e-12, atol=1e-12)
    assert not np.allclose(res["out"][3], _sdpa_layer(wl, 3, 0, second))


def test_reuse_after_token_only_reindex_takes_its_fresh_topk():
    """Full, Reuse, token-only Reindex, Reuse: the token-only Reindex layer
    keeps the Full layer's pool, reselects the tokens with its own indexer
    query, and the Reuse layer after it attends over that new selection."""
    cfg, wl = _mode_workload(("full", "reuse", "reindex_tokens", "reuse"), seed=34)
    res = oracle.run_layers(wl)
    full = _brute_sets(wl, 0, 0)
    tok = []
    for i, (pool, _) in enumerate(full):
        t, s = int(wl.q_pos[i]), int(wl.q_seq[i])
        cands = [(dot(wl.q_idx[2][i], wl.k_idx[s][p]), p) for j in pool
                 for p in range(j * cfg.block, j * cfg.block + cfg.block) if p <= t]
        tok.append((pool, top_n_by_enumeration(cands, cfg.top_k)))
    assert any(f[1] != r[1] for f, r in zip(full, tok)), "the two selections must differ"
    _assert_index(res["index"][0], full)
    _assert_index(res["index"][2], tok)
    for layer, sets in ((0, full), (1, full), (2, tok), (3, tok)):
        np.testing.assert_allclose(res["out"][layer], _sdpa_layer(wl, layer, 0, sets), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- compressed main-KV
# The figure caption of the "DeepSeek V4.1 Flash" page names CSA2(ratio,
# mode) and leaves the compression undefined.  Reading: main-KV entry j
# stands for tokens j*r .. j*r + r - 1 and exists once its last token has
# arrived; selection runs over entries, the window stays per token.  The
# brute force below finds the visible entries by testing each entry's last
# token against t, not by the division the oracle uses.
def _select_compressed_brute(q, k_entries, t, r, B, P, K, tail=0):
    vis = [j for j in range(len(k_entries)) if j * r + r - 1 <= t]
    if not vis:
        return [], []
    assert vis == list(range(len(vis)))
    return select_brute(q, k_entries, vis[-1], B, P, K, tail)


def test_visible_entries_by_definition():
    for r in range(1, 7):
        for t in range(0, 40):
            want = sum(1 for j in range(64) if j * r + r - 1 <= t)
            assert oracle.visible_entries(t, r) == want, (r, t)
    # the largest int32 position (reachable only with compression: T <= 2^24
    # entries): entries j with (j + 1) * r <= 2^31
    t = 2**31 - 1
    for r in (2, 3, 256):
        assert oracle.visible_entries(t, r) == 2**31 // r, r


def test_compressed_selection_matches_enumeration():
    rng = np.random.default_rng(41)
    for _ in range(300):
        r = int(rng.integers(2, 5))
        B = int(rng.choice([2, 4]))
        n = int(rng.integers(1, 9))            # entries in the cache
        d = int(rng.integers(1, 4))
        P = int(rng.integers(1, 5))
        K = int(rng.integers(1, 4))
        tail = int(rng.integers(0, 3))
        k = rng.integers(-3, 4, size=(n, d), dtype=np.int8)
        q = rng.integers(-3, 4, size=d, dtype=np.int8)
        t = int(rng.integers(0, n * r + r - 1))  # up to the token before entry n completes
        blk, bc, tk, tc = oracle.select(q[None], [0], [t], k[None], B, P, K, tail=tail, ratio=r)
        pool, top = _select_compressed_brute(q, k, t, r, B, P, K, tail)
        assert list(blk[0, :bc[0]]) == pool, (r, B, n, t, tail)
        assert (blk[0, bc[0]:] == -1).all()
        assert list(tk[0, :tc[0]]) == top, (r, B, n, t, tail)
        assert (tk[0, tc[0]:] == -1).all()


def test_compressed_selection_hand_case():
    """Ratio 4, blocks of 2 entries, pool 1, Top-2; entry scores 1, 2, 5, 4
    (d = 1, q = 1).  Worked by hand:
      t = 2 : no entry complete                       -> nothing selected
      t = 3 : entry 0 (tokens 0..3)                    -> pool [0], Top-K [0]
      t = 7 : entries 0, 1; block 0 key round(1.5) = 2 -> pool [0], Top-K [0, 1]
      t = 11: entries 0..2; block 1 holds entry 2 only, key 5 beats 2
                                                      -> pool [1], Top-K [2]
      t = 14: still entries 0..2 (entry 3 ends at 15)  -> pool [1], Top-K [2]
      t = 15: entries 0..3; block 1 key round(4.5) = 4 -> pool [1], Top-K [2, 3]"""
    k = np.array([[1], [2], [5], [4]], dtype=np.int8)
    q = np.array([1], dtype=np.int8)
    want = {2: ([], []), 3: ([0], [0]), 7: ([0], [0, 1]), 11: ([1], [2]), 14: ([1], [2]),
            15: ([1], [2, 3])}
    for t, (pool, top) in want.items():
        blk, bc, tk, tc = oracle.select(q[None], [0], [t], k[None], 2, 1, 2, ratio=4)
        assert list(blk[0, :bc[0]]) == pool, t
        assert list(tk[0, :tc[0]]) == top, t


def test_compressed_layers_against_scratch():
    """A compressed prompt (ratio 2, every token a query) through Full, Reuse,
    window-only: each layer recomputed from scratch (entries by enumeration,
    fp64 SDPA over the selected entries plus the per-token window).  The
    first token sees no entry and attends to its window alone."""
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=21, n_heads=2, head_dim=8, d_idx=32, block=2, pool=3,
                   top_k=3, window=4, layers=("full", "reuse", "swa"), ratio=2)
    wl = W.generate(cfg, seed=43)
    assert wl.k_idx.shape[1] == 10 and wl.k_swa[0].shape[1] == 21
    res = oracle.run_layers(wl)
    sets = [_select_compressed_brute(wl.q_idx[0][i], wl.k_idx[0], int(wl.q_pos[i]), 2, cfg.block,
                                     cfg.pool, cfg.top_k, cfg.tail) for i in range(cfg.n_q)]
    assert sets[0] == ([], []) and sets[1][1] == [0]
    _assert_index(res["index"][0], sets)
    for layer, s in ((0, sets), (1, sets), (2, None)):
        np.testing.assert_allclose(res["out"][layer], _sdpa_layer(wl, layer, 0, s), rtol=1e-12, atol=1e-12)
