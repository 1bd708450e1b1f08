"""Workload structure (CPU): the encoder and decoder halves of the causal
encoder-decoder flow of the V4.1 Flash page ("Asymmetric encoder-decoder
(CED)" and the mode table's layer patterns), and the cache each layer group
reads."""
import numpy as np

from top_kv_selection_amd import pipeline
from top_kv_selection_amd import workloads as W


def test_encoder_pattern_and_its_caches():
    cfg = W.CONFIGS["encoder_prefill_8k"]
    assert cfg.layers == ("swa", "swa") + ("full",) + ("reuse",) * 5 + ("full",) + ("reuse",) * 5 \
        + ("full",) + ("reuse",) * 5
    assert cfg.n_layers == 20 and cfg.n_caches == 3 and cfg.n_q == 8192
    # groups: window, window, then three Full + 5 Reuse groups with caches 0, 1, 2
    assert [m for m, _ in cfg.groups()] == ["swa", "swa", "full", "full", "full"]
    assert pipeline.group_caches(cfg) == [0, 0, 0, 1, 2]


def test_decoder_replay_queries_are_the_last_128_positions():
    cfg = W.CONFIGS["decoder_replay_8k"]
    q_seq, q_pos = W.query_rows(cfg)
    assert cfg.n_q == 128 and cfg.n_layers == 20 and cfg.n_caches == 1
    assert (q_seq == 0).all() and (q_pos == np.arange(8064, 8192)).all()
    assert cfg.swa_first == 0 and cfg.swa_len == cfg.ctx


def test_every_full_layer_draws_its_own_cache():
    cfg = W.scaled(W.CONFIGS["encoder_prefill_8k"], ctx=64, n_heads=16, layers=("swa", "full", "reuse", "full"))
    wl = W.generate(cfg)
    assert cfg.n_caches == 2 and len(wl.extra_caches) == 1
    k0, m0, v0 = wl.cache(0)
    k1, m1, v1 = wl.cache(1)
    assert k1.shape == k0.shape and m1.shape == m0.shape and v1.shape == v0.shape
    assert not np.array_equal(k0, k1) and not np.array_equal(m0, m1)
    assert pipeline.group_caches(cfg) == [0, 0, 1]


def test_single_cache_workloads_draw_nothing_extra():
    for name in ("tiny_full_fp32", "prefill_8k", "decoder_pattern_64k"):
        assert W.CONFIGS[name].n_caches == 1
    wl = W.generate(W.CONFIGS["tiny_full_fp32"])
    assert wl.extra_caches == []
