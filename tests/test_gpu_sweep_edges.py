"""Seeded sweep of boundary configurations, each through the C ABI and
compared with the oracle (indices exact, outputs within the tolerance of
parity.py).  Where the random sweep draws sizes uniformly, this one draws
them from the edges of what the library accepts: caches of one entry, just
under, at and just over one block; blocks of 1, 2, 3 and 16; pools of one
block, of two, and of the full 16,384-candidate cap; Top-K of 1 and of every
candidate of the pool; windows of 1 and of 1,024 rows, also longer than the
context; 128 heads (8 head groups); one to 16 decode sequences; the three
tail readings; and compression ratios up to 8 with an incomplete group of
tokens at the end of the context."""
import numpy as np
import pytest
import torch

import oracle
from parity import compare_run
from top_kv_selection_amd import workloads as W

pytestmark = pytest.mark.gpu

PATTERNS = [
    ("full",),
    ("full", "reuse"),
    ("full", "reindex", "reuse"),
    ("full", "reuse", "reindex_tokens", "reuse"),
    ("swa", "full", "reuse"),
]

N_CASES = 40


def edge_cfg(k: int):
    rng = np.random.default_rng(7000 + k)
    decode = bool(rng.integers(0, 2))
    B = int(rng.choice([1, 2, 3, 16]))
    ratio = int(rng.choice([1, 1, 2, 8]))
    fp32 = rng.random() < 0.2
    H = 16 if fp32 else int(rng.choice([16, 32, 128]))
    # main-KV entries around one block, a few blocks, or many
    near = [1, 2, max(B - 1, 1), B, B + 1]
    n_main = int(rng.choice(near + ([37, 2000, 40000 // ratio] if decode else [37, 300 // ratio + 1])))
    ctx = n_main * ratio + int(rng.integers(0, ratio))     # tokens; the last group may be incomplete
    P = int(rng.choice([1, 2, 64, 16384 // B]))
    K = int(rng.choice([1, P * B, int(rng.integers(1, P * B + 1))]))
    Wn = int(rng.choice([1, 2, 127, 1024]))
    # bounds that keep the oracle's fp64 attention to seconds
    K = min(K, 2048 if decode else 512)
    if not decode and H > 32:
        K, Wn = min(K, 256), min(Wn, 128)
    n_seq = int(rng.choice([1, 3, 16])) if decode else int(rng.integers(1, 3))
    layers = PATTERNS[int(rng.integers(0, len(PATTERNS)))]
    return W.scaled(W.CONFIGS["decode_full_32k" if decode else "prefill_8k"],
                    name=f"edge{k}", n_seq=n_seq, ctx=ctx, block=B, pool=P, top_k=K, window=Wn,
                    d_idx=int(rng.choice([32, 64])), n_heads=H, head_dim=64 if fp32 else 128,
                    dtype="f32" if fp32 else "bf16", layers=layers, tail=int(rng.integers(0, 3)),
                    ratio=ratio)


@pytest.fixture(scope="module")
def pipeline():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from top_kv_selection_amd import pipeline as pl
    return pl


@pytest.mark.parametrize("k", range(N_CASES))
def test_boundary_configuration_matches_the_oracle(pipeline, k):
    cfg = edge_cfg(k)
    ties = k % 3 == 2                      # narrow int8 draws: long runs of equal scores
    print(f"case {cfg.name}: decode={cfg.decode} S={cfg.n_seq} T={cfg.ctx} entries={cfg.main_len} "
          f"B={cfg.block} P={cfg.pool} K={cfg.top_k} W={cfg.window} d={cfg.d_idx} H={cfg.n_heads} "
          f"D={cfg.head_dim} {cfg.dtype} tail={cfg.tail} ratio={cfg.ratio} layers={cfg.layers} "
          f"ties={ties}", flush=True)
    wl = W.generate(cfg, seed=7000 + k, int_range=(-2, 2) if ties else (-127, 127))
    dw = pipeline.upload(wl)
    pipeline.build_cache(dw)
    pipeline.run(dw)
    torch.cuda.synchronize()
    got = pipeline.outputs(dw)
    ref = oracle.run_layers(wl)
    compare_run(got, ref, cfg, what=cfg.name)
