"""Seeded synthetic workloads for the CSA2 sparse-attention step.

This module only draws random inputs and describes their shapes.  It holds none
of the method's arithmetic (no scores, no selection, no attention), so both the
CPU oracle and the HIP path can consume the very same bytes.

Shapes follow the sparse-attention facts on the DeepSeek V4.1 Flash page
(k-a.in, "Sparse attention": a Top-512 main-KV selection plus a 128-token
window; "Hierarchical indexer": at most 16,384 candidates) and the layer
patterns of its "CSA2 with cross-layer reuse" section.  Five workloads:

* ``tiny_full_fp32``      one sequence of 256 tokens, every position a query, fp32
* ``decode_full_32k``     batch 16, 32K context, one Full layer, bf16
* ``decode_group_128k``   batch 8, 128K context, Full + 5 Reuse sharing one index set
* ``prefill_8k``          causal prefill of 8,192 tokens + 2 pure sliding-window layers
* ``decoder_pattern_64k`` batch 8, 64K context, Full + 3 Reuse, [Reindex + 3 Reuse] x 4

and the two halves of the causal encoder-decoder flow of the V4.1 Flash page
("Asymmetric encoder-decoder (CED)": prompt tokens go through the 20 encoder
layers only, plus a 128-token decoder replay; the mode table's encoder and
decoder patterns):

* ``encoder_prefill_8k``  an 8,192-token prompt through window, window,
  [Full + 5 Reuse] x 3 (every Full layer with its own main-KV and indexer cache)
* ``decoder_replay_8k``   the last 128 prompt positions through the decoder
  pattern Full + 3 Reuse, [Reindex + 3 Reuse] x 4

and the 128K layer group's shapes at twice the context ("Hierarchical
indexer": the candidate cap holds whatever the context length):

* ``decode_group_256k``   batch 8, 256K context, Full + 5 Reuse

and two workloads with compressed main-KV and indexer caches (the page's
CSA2(ratio, mode); the ratio is not given there, 4 is an illustration):

* ``decode_group_128k_c4`` the 128K layer group with one entry per 4 tokens
  (32,768 entries per sequence; the window stays 128 tokens)
* ``prefill_8k_c4``        the 8K prefill with one entry per 4 tokens

Recipe (both sides read identical bytes):
* ``numpy.random.Generator(PCG64(1000 + config_number))``;
* draw order: ``k_idx``, each indexing layer's ``q_idx`` (model order), main K,
  main V, then per layer (model order) Q, sliding-window K, sliding-window V,
  then for every Full layer after the first its own ``k_idx``, main K, main V;
* main-KV and indexer caches hold ``ctx // ratio`` entries per sequence, the
  window caches one row per token;
* int8 values are uniform integers in [-127, 127];
* real values are standard normal drawn in fp32 and, for bf16 workloads,
  rounded to bf16 with round-to-nearest-even (stored as uint16 bit patterns).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

FULL, REINDEX, REUSE, SWA_ONLY = "full", "reindex", "reuse", "swa"
REINDEX_TOKENS = "reindex_tokens"   # own q_idx over the shared pool: token Top-K only
# Readings of a query's partial own block in the block pass: keyed by its
# visible rows (default), not eligible, or keyed by all of its rows.
TAIL_VISIBLE, TAIL_EXCLUDE, TAIL_WHOLE = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    number: int              # 1-based; seed = 1000 + number
    dtype: str               # "f32" | "bf16"
    n_seq: int               # S
    ctx: int                 # T: cache length per sequence (positions 0..T-1)
    decode: bool             # decode: one query per sequence at t = T-1
    n_heads: int             # H
    head_dim: int            # D
    d_idx: int               # indexer dimension
    block: int               # B
    pool: int                # P (blocks kept by the hierarchical pass)
    top_k: int               # K
    window: int              # W
    layers: tuple            # per-layer mode, model order
    tail: int = TAIL_VISIBLE  # reading of a partial own block (see TAIL_*)
    replay: int = 0          # (not decode) queries are only the last `replay` positions
    ratio: int = 1           # tokens per main-KV entry (compressed main-KV and indexer caches)

    @property
    def seed(self) -> int:
        return 1000 + self.number

    @property
    def n_q(self) -> int:
        if self.decode:
            return self.n_seq
        return self.n_seq * (self.replay if self.replay > 0 else self.ctx)

    @property
    def main_len(self) -> int:
        """Entries of the main-KV and indexer caches per sequence: one per
        ``ratio`` tokens, complete groups only."""
        return self.ctx // self.ratio

    @property
    def n_caches(self) -> int:
        """Main-KV + indexer caches: one per Full layer (at least one)."""
        return max(1, sum(1 for m in self.layers if m == FULL))

    @property
    def n_layers(self) -> int:
        return len(self.layers)

    @property
    def index_layers(self) -> List[int]:
        return [i for i, m in enumerate(self.layers) if m in (FULL, REINDEX, REINDEX_TOKENS)]

    @property
    def swa_first(self) -> int:
        """First position held by the per-layer sliding-window K/V rows (decode:
        the last `window` positions, or every position of a shorter context)."""
        return max(self.ctx - self.window, 0) if self.decode else 0

    @property
    def swa_len(self) -> int:
        return min(self.window, self.ctx) if self.decode else self.ctx

    def groups(self):
        """Split the layer list into (mode, [layers]) groups: an indexing or
        sliding-window layer followed by the Reuse layers that share its indices."""
        out = []
        for i, m in enumerate(self.layers):
            if m == REUSE:
                if not out or out[-1][0] == SWA_ONLY:
                    raise ValueError("a Reuse layer needs an earlier Full/Reindex layer")
                out[-1][1].append(i)
            else:
                out.append((m, [i]))
        return out


def _encoder_pattern():
    pat = [SWA_ONLY, SWA_ONLY]
    for _ in range(3):
        pat += [FULL] + [REUSE] * 5
    return tuple(pat)


def _decoder_pattern():
    pat = [FULL, REUSE, REUSE, REUSE]
    for _ in range(4):
        pat += [REINDEX, REUSE, REUSE, REUSE]
    return tuple(pat)


CONFIGS = {
    c.name: c
    for c in [
        Config("tiny_full_fp32", 1, "f32", 1, 256, False, 4, 64, 32, 8, 8, 32, 16, (FULL,)),
        Config("decode_full_32k", 2, "bf16", 16, 32768, True, 16, 128, 64, 8, 2048, 512, 128, (FULL,)),
        Config("decode_group_128k", 3, "bf16", 8, 131072, True, 16, 128, 64, 8, 2048, 512, 128,
               (FULL,) + (REUSE,) * 5),
        Config("prefill_8k", 4, "bf16", 1, 8192, False, 16, 128, 64, 8, 2048, 512, 128,
               (FULL, SWA_ONLY, SWA_ONLY)),
        Config("decoder_pattern_64k", 5, "bf16", 8, 65536, True, 16, 128, 64, 8, 2048, 512, 128,
               _decoder_pattern()),
        Config("encoder_prefill_8k", 6, "bf16", 1, 8192, False, 16, 128, 64, 8, 2048, 512, 128,
               _encoder_pattern()),
        Config("decoder_replay_8k", 7, "bf16", 1, 8192, False, 16, 128, 64, 8, 2048, 512, 128,
               _decoder_pattern(), replay=128),
        Config("decode_group_256k", 8, "bf16", 8, 262144, True, 16, 128, 64, 8, 2048, 512, 128,
               (FULL,) + (REUSE,) * 5),
        Config("decode_group_128k_c4", 9, "bf16", 8, 131072, True, 16, 128, 64, 8, 2048, 512, 128,
               (FULL,) + (REUSE,) * 5, ratio=4),
        Config("prefill_8k_c4", 10, "bf16", 1, 8192, False, 16, 128, 64, 8, 2048, 512, 128,
               (FULL, SWA_ONLY, SWA_ONLY), ratio=4),
    ]
}


def scaled(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields replaced (used for smaller parity cases)."""
    return dataclasses.replace(cfg, **kw)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns.
    Inputs here are finite normal draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    cfg: Config
    k_idx: np.ndarray          # int8 [S][main_len][d]
    q_idx: dict                # layer -> int8 [n_q][d]  (indexing layers only)
    k_main: np.ndarray         # [S][main_len][D]  float32 or uint16 (bf16 bits)
    v_main: np.ndarray
    q: list                    # per layer [n_q][H][D]
    k_swa: list                # per layer [S][swa_len][D]
    v_swa: list
    q_seq: np.ndarray          # int32 [n_q]
    q_pos: np.ndarray          # int32 [n_q]
    extra_caches: list = dataclasses.field(default_factory=list)   # (k_idx, k_main, v_main) of Full layers 2, 3, ...

    def cache(self, c: int):
        """(k_idx, k_main, v_main) of cache c (c = 0: the first Full layer's)."""
        return (self.k_idx, self.k_main, self.v_main) if c == 0 else self.extra_caches[c - 1]


def _real(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def _ints(rng, shape, lo=-127, hi=127):
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int8)


def query_rows(cfg: Config):
    if cfg.decode:
        q_seq = np.arange(cfg.n_seq, dtype=np.int32)
        q_pos = np.full(cfg.n_seq, cfg.ctx - 1, dtype=np.int32)
    elif cfg.replay > 0:
        q_seq = np.repeat(np.arange(cfg.n_seq, dtype=np.int32), cfg.replay)
        q_pos = np.tile(np.arange(cfg.ctx - cfg.replay, cfg.ctx, dtype=np.int32), cfg.n_seq)
    else:
        q_seq = np.repeat(np.arange(cfg.n_seq, dtype=np.int32), cfg.ctx)
        q_pos = np.tile(np.arange(cfg.ctx, dtype=np.int32), cfg.n_seq)
    return q_seq, q_pos


def generate(cfg: Config, seed: Optional[int] = None, int_range=(-127, 127)) -> Workload:
    """Draw one workload in the fixed order stated in the module docstring.
    ``int_range`` narrows the int8 draws (e.g. (-2, 2)) to force many score ties."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    S, T, d, H, D = cfg.n_seq, cfg.main_len, cfg.d_idx, cfg.n_heads, cfg.head_dim
    lo, hi = int_range
    k_idx = _ints(rng, (S, T, d), lo, hi)
    q_idx = {i: _ints(rng, (cfg.n_q, d), lo, hi) for i in cfg.index_layers}
    k_main = _real(rng, (S, T, D), cfg.dtype)
    v_main = _real(rng, (S, T, D), cfg.dtype)
    q, k_swa, v_swa = [], [], []
    for _ in cfg.layers:
        q.append(_real(rng, (cfg.n_q, H, D), cfg.dtype))
        k_swa.append(_real(rng, (S, cfg.swa_len, D), cfg.dtype))
        v_swa.append(_real(rng, (S, cfg.swa_len, D), cfg.dtype))
    extra = []
    for _ in range(cfg.n_caches - 1):
        extra.append((_ints(rng, (S, T, d), lo, hi), _real(rng, (S, T, D), cfg.dtype),
                      _real(rng, (S, T, D), cfg.dtype)))
    q_seq, q_pos = query_rows(cfg)
    return Workload(cfg, k_idx, q_idx, k_main, v_main, q, k_swa, v_swa, q_seq, q_pos, extra)


def fresh_queries(cfg: Config, seed: int):
    """New indexer queries and attention queries over the same caches (used to
    build rotating replicas): returns (q_idx dict, q list)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q_idx = {i: _ints(rng, (cfg.n_q, cfg.d_idx)) for i in cfg.index_layers}
    q = [_real(rng, (cfg.n_q, cfg.n_heads, cfg.head_dim), cfg.dtype) for _ in cfg.layers]
    return q_idx, q
