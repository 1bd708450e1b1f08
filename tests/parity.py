"""Comparison helpers for the GPU parity tests.

Indices (pooled blocks, Top-K positions, counts) must be identical.  Outputs
pass when |gpu - oracle| <= ATOL + RTOL * |oracle| elementwise against the
fp64 oracle, the log-sum-exp under the same gate:
* bf16 workloads: 2e-2 + 1e-2 * |oracle| (bf16 inputs and a bf16 output of an
  fp32-accumulated kernel: the output rounding alone is up to 2^-9 relative);
* fp32 workloads: 1e-4 + 1e-4 * |oracle| (fp32 inputs, fp32 accumulation and an
  fp32 output: each output is a convex combination of at most K + W values of
  magnitude ~1, so fp32 rounding over a few hundred terms stays near 1e-6).
"""
import numpy as np

ATOL, RTOL = 2e-2, 1e-2
ATOL_F32, RTOL_F32 = 1e-4, 1e-4


def tolerance(cfg):
    return (ATOL_F32, RTOL_F32) if cfg.dtype == "f32" else (ATOL, RTOL)


def assert_index_equal(gpu: dict, ref: dict, rows=None, what=""):
    for key in ("blk_cnt", "blk_ids", "topk_cnt", "topk"):
        g = gpu[key] if rows is None else gpu[key][rows]
        r = ref[key]
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{what} {key}: {len(bad)} mismatches, first at {bad[:5].tolist()}")


def assert_close(gpu: np.ndarray, ref: np.ndarray, what="", atol=ATOL, rtol=RTOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    ok = err <= atol + rtol * np.abs(ref)
    if not ok.all():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} out of tolerance; worst at {i}: "
                             f"gpu {gpu[i]!r} oracle {ref[i]!r}")
    return float(err.max())


def compare_run(gpu_res: dict, ref_res: dict, cfg, rows=None, what=""):
    """gpu_res from pipeline.outputs, ref_res from oracle.run_layers(rows=rows)."""
    worst = 0.0
    atol, rtol = tolerance(cfg)
    for layer in range(cfg.n_layers):
        g_out = gpu_res["out"][layer] if rows is None else gpu_res["out"][layer][rows]
        g_lse = gpu_res["lse"][layer] if rows is None else gpu_res["lse"][layer][rows]
        worst = max(worst, assert_close(g_out, ref_res["out"][layer], f"{what} layer {layer} out", atol, rtol))
        assert_close(g_lse, ref_res["lse"][layer], f"{what} layer {layer} lse", atol, rtol)
    for layer, idx in ref_res["index"].items():
        assert_index_equal(gpu_res["index"][layer], idx, rows, f"{what} layer {layer}")
    return worst
