"""Model and run shapes for the DFlash draft+verify step.

The shapes follow the Qwen-class pairs that the DFlash pages run (mirror-sd
README, "Results" and "Supported Models"; dflash-mlx note, "Benchmarks"):
a target decoder plus a small block-diffusion drafter of the same width that
shares the target's embedding and lm-head (mlx-dspark v0.0.3 notes,
"Highlights").  Weights are random-init (no checkpoints exist here), drawn by
``synth.py``.

Everything in this file is plain data: no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple

# weight storage formats (must match include/dflash.h)
FMT_F32 = 0        # fp32 weights, fp32 activations
FMT_BF16 = 1       # bf16 weights, bf16 activations
FMT_W8A16 = 2      # int8 codes, one fp16 scale per output channel, bf16 activations
FMT_W4A16 = 3      # int4 codes, one fp16 scale per 64-wide K group, bf16 activations

FMT_NAMES = {FMT_F32: "f32", FMT_BF16: "bf16", FMT_W8A16: "w8a16", FMT_W4A16: "w4a16"}

LAYER_ATTN = 0
LAYER_GDN = 1


@dataclass(frozen=True)
class ModelShape:
    """One decoder stack (target or drafter)."""
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_layers: int
    fmt: int
    layer_kinds: Tuple[int, ...] = ()          # empty -> all attention
    gdn_heads: int = 16
    gdn_dk: int = 128
    gdn_dv: int = 128
    eps: float = 1e-6
    rope_base: float = 1e6

    def kinds(self) -> Tuple[int, ...]:
        return self.layer_kinds if self.layer_kinds else (LAYER_ATTN,) * self.n_layers

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def gdn_rows(self) -> int:
        # fused projection rows: q, k, v (gdn_heads x dk/dk/dv) then a, b (gdn_heads each)
        return self.gdn_heads * (2 * self.gdn_dk + self.gdn_dv) + 2 * self.gdn_heads


@dataclass(frozen=True)
class PairConfig:
    """A target/drafter pair and the run shape of one workload."""
    name: str
    target: ModelShape
    drafter: ModelShape
    sel_layers: Tuple[int, ...]     # target layers whose outputs condition the drafter
    block: int                      # B: anchor + B-1 mask slots
    contexts: Tuple[int, ...]       # committed context lengths the workload runs at
    new_tokens: int = 64            # tiny end-to-end generation length
    # injected acceptance: k = min(K, B-1), K geometric on {0,1,..} with this mean
    # (None = the real method, no injection)
    inject_geo_mean: Optional[float] = None
    seed: int = 0

    @property
    def mask_token(self) -> int:
        # reserved mask id for the drafter's noise slots: the last vocab id
        return self.target.vocab - 1

    def reduced(self, target_layers: int, drafter_layers: int = 1) -> "PairConfig":
        """Same widths, fewer layers (for oracle-checkable parity at real widths)."""
        kinds = self.target.kinds()[:target_layers]
        t = replace(self.target, n_layers=target_layers,
                    layer_kinds=kinds if self.target.layer_kinds else ())
        d = replace(self.drafter, n_layers=drafter_layers)
        # keep up to two conditioning layers: the first layers of the reduced stack
        sel = tuple(range(min(2, len(self.sel_layers), target_layers)))
        return replace(self, name=f"{self.name}-L{target_layers}d{drafter_layers}",
                       target=t, drafter=d, sel_layers=sel)


def _evenly_spaced_sel(n_layers: int, k: int = 5) -> Tuple[int, ...]:
    # conditioning layers spread over [1, L-3]
    lo, hi = 1, n_layers - 3
    return tuple(int(round(lo + i * (hi - lo) / (k - 1))) for i in range(k))


def tiny() -> PairConfig:
    t = ModelShape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=768,
                   vocab=1024, n_layers=2, fmt=FMT_F32)
    d = replace(t, n_layers=1)
    return PairConfig("tiny", t, d, sel_layers=(0, 1), block=16, contexts=(64,),
                      new_tokens=64)


def qwen4b() -> PairConfig:
    t = ModelShape(hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=9728,
                   vocab=151936, n_layers=36, fmt=FMT_BF16)
    d = replace(t, n_layers=5)
    return PairConfig("4b", t, d, sel_layers=_evenly_spaced_sel(36), block=16,
                      contexts=(512, 2048), inject_geo_mean=6.0)


def qwen8b() -> PairConfig:
    t = ModelShape(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=12288,
                   vocab=151936, n_layers=36, fmt=FMT_W4A16)
    d = replace(t, n_layers=5, fmt=FMT_W8A16)
    return PairConfig("8b", t, d, sel_layers=_evenly_spaced_sel(36), block=32,
                      contexts=(64, 2048, 4096), inject_geo_mean=23.125)


def qwen27b() -> PairConfig:
    t = ModelShape(hidden=5120, n_q_heads=40, n_kv_heads=8, head_dim=128, ffn=17408,
                   vocab=151936, n_layers=64, fmt=FMT_W4A16)
    d = replace(t, n_layers=5, fmt=FMT_W8A16)
    return PairConfig("27b", t, d, sel_layers=_evenly_spaced_sel(64), block=32,
                      contexts=(64, 2048, 4096), inject_geo_mean=23.125)


def hybrid() -> PairConfig:
    kinds = tuple(LAYER_ATTN if l % 4 == 3 else LAYER_GDN for l in range(36))
    t = ModelShape(hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=9728,
                   vocab=151936, n_layers=36, fmt=FMT_BF16, layer_kinds=kinds)
    d = ModelShape(hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=9728,
                   vocab=151936, n_layers=5, fmt=FMT_BF16)
    return PairConfig("hybrid", t, d, sel_layers=_evenly_spaced_sel(36), block=16,
                      contexts=(2048,), inject_geo_mean=6.0)


CONFIGS = {"tiny": tiny, "4b": qwen4b, "8b": qwen8b, "27b": qwen27b, "hybrid": hybrid}


def get(name: str) -> PairConfig:
    return CONFIGS[name]()
