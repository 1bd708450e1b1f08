"""The allocation-free layer group (csa2_layer_group_static) against
csa2_layer_group with a workspace (GPU, through the C ABI).

Two calls in a row on the library's fixed scratch, the second with a smaller
input (so it runs on the first call's leftovers): indices must be identical
and outputs must match the workspace call (same kernels, so bitwise), and
both must match the oracle.  A call too large for the fixed scratch is
refused with CSA2_E_WORKSPACE and leaves its outputs untouched.
"""
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


def _run_static(B, pipeline, dw):
    begin = pipeline.step_update_begin(dw)
    for g, grp in enumerate(dw.groups):
        idx = grp.index_of if grp.index_of >= 0 else None
        k_idx, k_blk, k_main, v_main = pipeline.cache(dw, grp.cache)
        B.csa2_layer_group_static(dw.lcfg, grp.mode, grp.q_idx, dw.q_seq, dw.q_pos, k_idx, k_blk, begin, grp.q,
                                  k_main, v_main, grp.k_swa, grp.v_swa, dw.cfg.swa_first, dw.blk_ids.get(idx),
                                  dw.blk_cnt.get(idx), dw.topk.get(idx), dw.topk_cnt.get(idx), grp.out, grp.lse)


@pytest.mark.parametrize("first,second", [
    (dict(name="decode_group_128k"), dict(name="decode_group_128k", n_seq=3, ctx=20000, pool=640)),
    (dict(name="decoder_pattern_64k", n_seq=4, ctx=20011), dict(name="decode_full_32k", n_seq=2, ctx=9001, pool=300)),
])
def test_static_scratch_matches_the_workspace_call(lib, first, second):
    B, pipeline = lib
    for k, spec in enumerate((first, second)):
        spec = dict(spec)
        cfg = W.CONFIGS[spec.pop("name")]
        if spec:
            cfg = W.scaled(cfg, **spec)
        print(f"case static call {k}: {cfg.name} S={cfg.n_seq} T={cfg.ctx} P={cfg.pool} layers={len(cfg.layers)}",
              flush=True)
        wl = W.generate(cfg, seed=50 + k)
        dw_ws = pipeline.upload(wl)
        pipeline.build_cache(dw_ws)
        pipeline.run(dw_ws)
        torch.cuda.synchronize()
        want = pipeline.outputs(dw_ws)
        dw = pipeline.upload(wl)
        pipeline.build_cache(dw)
        for grp in dw.groups:
            grp.out.fill_(float("nan"))
        _run_static(B, pipeline, dw)
        torch.cuda.synchronize()
        got = pipeline.outputs(dw)
        for layer in range(cfg.n_layers):
            assert np.array_equal(got["out"][layer], want["out"][layer]), f"layer {layer} out"
            assert np.array_equal(got["lse"][layer], want["lse"][layer]), f"layer {layer} lse"
        for layer, idx in want["index"].items():
            for key, v in idx.items():
                assert np.array_equal(got["index"][layer][key], v), f"layer {layer} {key}"
        compare_run(got, oracle.run_layers(wl), cfg, what=f"static call {k}")


def test_static_scratch_refuses_a_call_it_cannot_hold(lib):
    B, pipeline = lib
    cfg = W.scaled(W.CONFIGS["decode_full_32k"], n_seq=400, ctx=20000, pool=2048)   # 400 x 2,500 blocks of keys
    print(f"case static refusal: S={cfg.n_seq} T={cfg.ctx}", flush=True)
    wl = W.generate(cfg, seed=52)
    dw = pipeline.upload(wl)
    pipeline.build_cache(dw)
    grp = dw.groups[0]
    grp.out.fill_(7.0)
    torch.cuda.synchronize()
    with pytest.raises(B.Csa2Error) as err:
        _run_static(B, pipeline, dw)
    assert err.value.status == 6          # CSA2_E_WORKSPACE
    torch.cuda.synchronize()
    assert bool((grp.out == 7.0).all())
