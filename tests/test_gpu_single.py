"""The fused decode layer group as one launch (csa2_layer_group_single)
against the four-launch csa2_layer_group (bitwise: the same kernel bodies
on the same inputs) and against the oracle, on the decode shapes where the
fused path applies, with each case called twice in a row (the per-query
counters in the workspace head must be left zero); and the calls it refuses."""
import numpy as np
import pytest
import torch

import oracle
from parity import compare_run
from top_kv_selection_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from top_kv_selection_amd import binding, pipeline
    return binding, pipeline


CASES = [
    ("decode_group_128k", {}),                      # batch 8 at 128K, Full + 5 Reuse
    ("decode_full_32k", {}),                        # batch 16 at 32K, one Full layer
    ("decode_group_256k", dict(n_seq=2)),           # 32,768 eligible blocks: 32 block keys per thread
    ("decode_group_128k", dict(n_seq=3, ctx=20003, pool=256, top_k=300, window=64,
                               layers=("full", "reuse", "reindex", "reuse"))),
    ("decode_group_128k_c4", dict(n_seq=3, ctx=131074, layers=("full", "reuse"))),   # 32,768 entries
    ("decode_full_32k", dict(n_seq=4, ctx=9001, pool=256, d_idx=32, tail=W.TAIL_EXCLUDE)),
]


def _flat(res):
    arrays = [a for a in res["out"]] + [a for a in res["lse"]]
    for layer in sorted(res["index"]):
        arrays += [res["index"][layer][k] for k in ("blk_ids", "blk_cnt", "topk", "topk_cnt")]
    return arrays


@pytest.mark.parametrize("name,kw", CASES)
def test_single_launch_equals_the_layer_group(lib, name, kw):
    B, pipeline = lib
    cfg = W.scaled(W.CONFIGS[name], **kw) if kw else W.CONFIGS[name]
    print(f"case single launch {name} S={cfg.n_seq} T={cfg.ctx} P={cfg.pool} K={cfg.top_k} W={cfg.window} "
          f"d={cfg.d_idx} tail={cfg.tail} ratio={cfg.ratio} layers={cfg.layers}", flush=True)
    wl = W.generate(cfg, seed=70)
    ref_dw = pipeline.upload(wl)
    pipeline.build_cache(ref_dw)
    pipeline.run(ref_dw)
    torch.cuda.synchronize()
    ref = _flat(pipeline.outputs(ref_dw))
    del ref_dw
    dw = pipeline.upload(wl)
    pipeline.build_cache(dw)
    for call in range(2):
        pipeline.run(dw, single=True)
        torch.cuda.synchronize()
        got = pipeline.outputs(dw)
        for a, b in zip(_flat(got), ref):
            assert np.array_equal(a, b), f"call {call}: single launch differs from the layer group"
    compare_run(got, oracle.run_layers(wl), cfg, what="single launch")


def test_single_launch_refuses_other_regimes(lib):
    """A prompt's layer group (many queries) has no single-launch form."""
    B, pipeline = lib
    cfg = W.scaled(W.CONFIGS["prefill_8k"], ctx=600, layers=("full",))
    print("case single launch refused: prefill", flush=True)
    dw = pipeline.upload(W.generate(cfg, seed=71))
    pipeline.build_cache(dw)
    with pytest.raises(B.Csa2Error) as e:
        pipeline.run(dw, single=True)
    assert e.value.status == 4


def test_single_launch_in_a_graph(lib):
    """Captured in a graph (an ordinary launch of the single kernel), replayed
    three times with eager work and synchronisation between the replays:
    every replay equals the eager call bitwise, so the counters are left zero
    by every replay too."""
    B, pipeline = lib
    cfg = W.scaled(W.CONFIGS["decode_group_128k"], n_seq=4, ctx=40000, layers=("full", "reuse", "reuse"))
    print(f"case single launch in a graph S={cfg.n_seq} T={cfg.ctx}", flush=True)
    wl = W.generate(cfg, seed=72)
    dw = pipeline.upload(wl)
    pipeline.build_cache(dw)
    pipeline.run(dw, single=True)
    torch.cuda.synchronize()
    eager = _flat(pipeline.outputs(dw))
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        pipeline.run(dw, single=True)
    for rep in range(3):
        for grp in dw.groups:            # eager work between replays: clobber the outputs
            grp.out.zero_()
            grp.lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(_flat(pipeline.outputs(dw)), eager):
            assert np.array_equal(a, b), f"replay {rep} differs from the eager call"
