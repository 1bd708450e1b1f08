"""Comparison helpers for the GPU parity tests.

Indices (pooled blocks, Top-K positions, counts) must be identical.  Outputs
pass when |gpu - oracle| <= 2e-2 + 1e-2 * |oracle| elementwise (bf16 output
of an fp32-accumulated kernel against the fp64 oracle); the log-sum-exp uses
the same gate.
"""
import numpy as np

ATOL, RTOL = 2e-2, 1e-2


def assert_index_equal(gpu: dict, ref: dict, rows=None, what=""):
    for key in ("blk_cnt", "blk_ids", "topk_cnt", "topk"):
        g = gpu[key] if rows is None else gpu[key][rows]
        r = ref[key]
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{what} {key}: {len(bad)} mismatches, first at {bad[:5].tolist()}")


def assert_close(gpu: np.ndarray, ref: np.ndarray, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    ok = err <= ATOL + RTOL * np.abs(ref)
    if not ok.all():
        i = np.unravel_index(np.argmax(err - (ATOL + RTOL * np.abs(ref))), err.shape)
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} out of tolerance; worst at {i}: "
                             f"gpu {gpu[i]!r} oracle {ref[i]!r}")
    return float(err.max())


def compare_run(gpu_res: dict, ref_res: dict, cfg, rows=None, what=""):
    """gpu_res from pipeline.outputs, ref_res from oracle.run_layers(rows=rows)."""
    worst = 0.0
    for layer in range(cfg.n_layers):
        g_out = gpu_res["out"][layer] if rows is None else gpu_res["out"][layer][rows]
        g_lse = gpu_res["lse"][layer] if rows is None else gpu_res["lse"][layer][rows]
        worst = max(worst, assert_close(g_out, ref_res["out"][layer], f"{what} layer {layer} out"))
        assert_close(g_lse, ref_res["lse"][layer], f"{what} layer {layer} lse")
    for layer, idx in ref_res["index"].items():
        assert_index_equal(gpu_res["index"][layer], idx, rows, f"{what} layer {layer}")
    return worst
