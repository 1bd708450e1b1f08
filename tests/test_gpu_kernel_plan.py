"""Which kernels a layer-group call launches, per regime, with a workspace
sized by csa2_workspace_bytes: a decode group must take the fused four-launch
path, a prompt the dense Top-K with row and window attention, and the
attention kernel must follow the item count (fewer than 256 items: key-list
chunks and their merge; 256: one workgroup per item; more: the row kernel;
window-only layers of 1,024 items or more: the shared-window kernel).  A
silent fall back to another path would keep every parity test green while
changing the timed work, so the launch sequence is checked here by the
library's own launch hook."""
import pytest
import torch

from top_kv_selection_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from top_kv_selection_amd import binding, pipeline
    return binding, pipeline


def launches(lib, cfg):
    B, pipeline = lib
    dw = pipeline.upload(W.generate(cfg, seed=90))
    pipeline.build_cache(dw)
    torch.cuda.synchronize()
    B.csa2_profile_begin("", 4096)
    pipeline.run(dw)
    torch.cuda.synchronize()
    return [name for name, _ in B.csa2_profile_end()]


CASES = [
    (W.CONFIGS["decode_group_128k"],
     ["k_index_blocks", "k_pool_tokens", "k_attend_chunks", "k_attend_combine"]),
    (W.scaled(W.CONFIGS["decode_group_128k"], n_seq=42, ctx=3000, pool=128),      # 252 items
     ["k_index_blocks", "k_pool_tokens", "k_attend_chunks", "k_attend_combine"]),
    (W.CONFIGS["prefill_8k"],
     ["k_topk_dense", "k_attend_rows", "k_attend_window", "k_attend_window"]),
    (W.scaled(W.CONFIGS["prefill_8k"], ctx=700, layers=("full", "swa")),           # 700 window-only items
     ["k_topk_dense", "k_attend_rows", "k_attend_rows"]),
]


@pytest.mark.parametrize("k", range(len(CASES)))
def test_launch_sequence(lib, k):
    cfg, expected = CASES[k]
    print(f"case kernel plan {cfg.name} S={cfg.n_seq} T={cfg.ctx} layers={cfg.layers}", flush=True)
    got = launches(lib, cfg)
    assert got == expected, f"{cfg.name}: launched {got}"


def test_attention_kernel_follows_the_item_count(lib):
    """Replayed prompt positions through Full + 3 Reuse: 64 positions are 256
    (query, layer) items (one round of one workgroup per item), 65 are 260."""
    for replay, kernel in ((64, "k_attend_mfma"), (65, "k_attend_rows")):
        cfg = W.scaled(W.CONFIGS["decoder_replay_8k"], replay=replay, layers=("full", "reuse", "reuse", "reuse"))
        print(f"case kernel plan replay={replay}", flush=True)
        got = launches(lib, cfg)
        assert got.count(kernel) == 1 and not any(n.startswith("k_attend") and n != kernel for n in got), got
