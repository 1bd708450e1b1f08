"""Layer groups captured in a HIP graph, as the step is replayed when it is
timed: each case is captured once on a side stream and replayed three times,
with eager work (the outputs and index sets overwritten) and a
synchronisation between replays; every replay must equal the eager call
bitwise, and the eager call must match the oracle.  Covers the fused decode
group (four launches), the separate decode launches past the fused limit, a
prompt through the dense Top-K with row and window attention, and a Reindex
group reading the Full group's indices."""
import numpy as np
import pytest
import torch

import oracle
from parity import compare_run
from top_kv_selection_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pipeline():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from top_kv_selection_amd import pipeline as pl
    return pl


CASES = [
    ("decode_group_128k", dict(n_seq=4, ctx=40000, layers=("full", "reuse", "reuse"))),
    ("decode_group_128k", dict(n_seq=2, ctx=280003, layers=("full", "reuse"))),   # 35,000 blocks: separate launches
    ("prefill_8k", dict(ctx=1500, layers=("full", "reuse", "swa"))),
    ("decoder_replay_8k", dict(replay=40, layers=("full", "reuse", "reindex", "reuse"))),
]


def _flat(res):
    arrays = [a for a in res["out"]] + [a for a in res["lse"]]
    for layer in sorted(res["index"]):
        arrays += [res["index"][layer][k] for k in ("blk_ids", "blk_cnt", "topk", "topk_cnt")]
    return arrays


def _clobber(dw):
    for grp in dw.groups:
        grp.out.zero_()
        grp.lse.zero_()
    for d in (dw.topk, dw.topk_cnt, dw.blk_cnt):
        for t in d.values():
            if t is not None:
                t.fill_(-7)


@pytest.mark.parametrize("name,kw", CASES)
def test_graph_replays_equal_the_eager_call(pipeline, name, kw):
    cfg = W.scaled(W.CONFIGS[name], **kw)
    print(f"case graph {name} S={cfg.n_seq} T={cfg.ctx} P={cfg.pool} layers={cfg.layers}", flush=True)
    wl = W.generate(cfg, seed=80)
    dw = pipeline.upload(wl)
    pipeline.build_cache(dw)
    pipeline.run(dw)
    torch.cuda.synchronize()
    eager = pipeline.outputs(dw)
    compare_run(eager, oracle.run_layers(wl), cfg, what=f"{name} eager")
    ref = _flat(eager)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        pipeline.run(dw)
    for rep in range(3):
        _clobber(dw)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(_flat(pipeline.outputs(dw)), ref):
            assert np.array_equal(a, b), f"replay {rep} differs from the eager call"
