"""Seeded synthetic inputs: random-init weights, prompts, acceptance schedules.

This module is shared by the CPU oracle tests and the HIP path.  It holds no
arithmetic of the draft+verify step: it only draws numbers and writes the
"checkpoint" that both sides then read.

* Linear and embedding weights are N(0, 0.02); every norm gain is 1.
  GatedDeltaNet gate rows (a, b) are N(0, 1/H) so that the gate
  pre-activations are about N(0, 1) on unit-RMS input.
* bf16 checkpoints hold bf16-representable values (fp32 -> bf16 by
  round-to-nearest-even, done by torch's dtype conversion).
* Quantised checkpoints (symmetric, scale only):
  - int8, one fp16 scale per output row:  s = fp16(max|W_n| / 127),
    q = clip(rint(W / s), -127, 127)
  - int4, one fp16 scale per 64-wide K group: s = fp16(max|W_g| / 7),
    q = clip(rint(W / s), -8, 7)
  (mirror-sd README, "The Story" and "How It Works": int8 projection weights
  with per-channel fp16 scales; the 4-bit target of "Results".)
  A zero scale gives zero codes.

Two generators exist: ``HostSynth`` (numpy PCG64, used wherever the oracle
must see the same model) and ``DeviceSynth`` (torch's Philox on the GPU, used
for full-size benchmark models that would take minutes to draw on the host).
They draw different numbers from the same seeds; each is deterministic.
"""
from __future__ import annotations

import os
import zlib
from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

from .configs import (FMT_BF16, FMT_F32, FMT_W4A16, FMT_W8A16, LAYER_ATTN,
                      LAYER_GDN, ModelShape, PairConfig)

GROUP = 64
STD = 0.02


def subseed(seed: int, name: str) -> int:
    return (seed * 1000003 + zlib.crc32(name.encode())) & 0x7FFFFFFF


@dataclass
class Weight:
    """A canonical (unpacked) weight matrix [N, K] in one storage format."""
    fmt: int
    n: int
    k: int
    values: Optional[np.ndarray] = None    # f32 / bf16 formats: float32 [N, K]
    codes: Optional[np.ndarray] = None     # quantised: int8 [N, K]
    scales: Optional[np.ndarray] = None    # quantised: float16 [N] or [N, K/64]


# ---------------------------------------------------------------- host (numpy)
def _to_bf16_values(x: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()


def quantize_host(w: np.ndarray, fmt: int) -> Weight:
    """Quantise a host fp32 matrix (torch CPU ops, several threads); returns
    numpy arrays.  Same recipe as quantize_device."""
    import torch
    q = quantize_device(torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)), fmt)
    cv = lambda t: None if t is None else t.numpy()
    return Weight(fmt, q.n, q.k, values=cv(q.values), codes=cv(q.codes), scales=cv(q.scales))


class HostSynth:
    """numpy generator: every tensor gets its own PCG64 stream from (seed, name)."""

    def __init__(self, seed: int = 0):
        self.seed = seed

    CHUNK = 1 << 20

    def normal(self, name: str, shape, std: float) -> np.ndarray:
        """N(0, std^2) in fp32; drawn in fixed 1 Mi-element chunks, chunk c from
        its own PCG64 stream (seed, name, c), so the result does not depend on
        how many threads draw it."""
        total = int(np.prod(shape))
        out = np.empty(total, dtype=np.float32)
        nch = (total + self.CHUNK - 1) // self.CHUNK

        def draw(c):
            lo, hi = c * self.CHUNK, min(total, (c + 1) * self.CHUNK)
            rng = np.random.Generator(np.random.PCG64(subseed(self.seed, f"{name}#{c}")))
            rng.standard_normal(out=out[lo:hi], dtype=np.float32)

        if nch == 1:
            draw(0)
        else:
            from concurrent.futures import ThreadPoolExecutor
            with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
                list(ex.map(draw, range(nch)))
        out *= np.float32(std)
        return out.reshape(shape)

    def weight(self, name: str, n: int, k: int, fmt: int, std: float = STD,
               row_std: Optional[np.ndarray] = None) -> Weight:
        w = self.normal(name, (n, k), 1.0)
        if row_std is None:
            w *= np.float32(std)
        else:
            w *= row_std.astype(np.float32)[:, None]
        return quantize_host(w, fmt)

    def act_values(self, name: str, shape, fmt: int, std: float = STD) -> np.ndarray:
        v = self.normal(name, shape, std)
        return v if fmt == FMT_F32 else _to_bf16_values(v)


def act_fmt(fmt: int) -> int:
    """Activation storage of a stack: fp32 for fp32 models, bf16 otherwise."""
    return FMT_F32 if fmt == FMT_F32 else FMT_BF16


def _layer_tensors(g, prefix: str, m: ModelShape, kind: int):
    H, F = m.hidden, m.ffn
    L = {"kind": kind,
         "in_norm": np.ones(H, np.float32),
         "post_norm": np.ones(H, np.float32)}
    if kind == LAYER_ATTN:
        L["q_norm"] = np.ones(m.head_dim, np.float32)
        L["k_norm"] = np.ones(m.head_dim, np.float32)
        L["w_qkv"] = g.weight(prefix + "w_qkv", m.qkv_rows, H, m.fmt)
        L["w_o"] = g.weight(prefix + "w_o", H, m.n_q_heads * m.head_dim, m.fmt)
    else:
        gh = m.gdn_heads
        rows = m.gdn_rows
        row_std = np.full(rows, STD, np.float32)
        row_std[gh * (2 * m.gdn_dk + m.gdn_dv):] = 1.0 / np.sqrt(H)
        L["w_qkv"] = g.weight(prefix + "w_qkvab", rows, H, m.fmt, row_std=row_std)
        L["w_o"] = g.weight(prefix + "w_o", H, gh * m.gdn_dv, m.fmt)
    L["w_gu"] = g.weight(prefix + "w_gu", 2 * F, H, m.fmt)
    L["w_down"] = g.weight(prefix + "w_down", H, F, m.fmt)
    return L


def make_pair(cfg: PairConfig, g=None) -> Dict:
    """The canonical checkpoint of a target/drafter pair.

    Returns {"target": {...}, "drafter": {...}} where each stack holds
    ``layers`` (list of dicts), ``final_norm``; the target also holds
    ``embed`` [V, H] and ``w_lm`` [V, H]; the drafter holds ``w_fc``
    [H, n_sel*H] and ``hidden_norm`` [H].
    """
    if g is None:
        g = HostSynth(cfg.seed)
    t, d = cfg.target, cfg.drafter
    tgt = {"layers": [_layer_tensors(g, f"t{l}.", t, k) for l, k in enumerate(t.kinds())],
           "final_norm": np.ones(t.hidden, np.float32),
           "embed": g.act_values("embed", (t.vocab, t.hidden), t.fmt),
           "w_lm": g.weight("w_lm", t.vocab, t.hidden, t.fmt)}
    drf = {"layers": [_layer_tensors(g, f"d{l}.", d, k) for l, k in enumerate(d.kinds())],
           "final_norm": np.ones(d.hidden, np.float32),
           "hidden_norm": np.ones(d.hidden, np.float32),
           "w_fc": g.weight("w_fc", d.hidden, len(cfg.sel_layers) * t.hidden, d.fmt)}
    return {"target": tgt, "drafter": drf}


# ------------------------------------------------------- prompts and schedules
def prompt(cfg: PairConfig, n: int, seed: int = 1) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, cfg.target.vocab, size=n, dtype=np.int64).astype(np.int32)


def accept_schedule(cfg: PairConfig, steps: int, seed: int = 2,
                    forced: Optional[List[int]] = None) -> np.ndarray:
    """k_s = min(K, B-1), K geometric on {0,1,...} with mean cfg.inject_geo_mean."""
    mean = cfg.inject_geo_mean if cfg.inject_geo_mean is not None else 6.0
    rng = np.random.Generator(np.random.PCG64(seed))
    p = 1.0 / (1.0 + mean)                      # success prob; numpy's geometric is on {1,2,..}
    k = rng.geometric(p, size=steps) - 1
    k = np.minimum(k, cfg.block - 1).astype(np.int32)
    if forced:
        k[: len(forced)] = np.asarray(forced, np.int32)
    return k


def filler_tokens(cfg: PairConfig, steps: int, seed: int = 3) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, cfg.target.vocab, size=(steps, cfg.block),
                        dtype=np.int64).astype(np.int32)


# -------------------------------------------------------------- device (torch)
class DeviceSynth:
    """torch generator on a device; same names and sub-seeds as HostSynth,
    different numbers.  Returns canonical tensors as torch tensors."""

    def __init__(self, seed: int = 0, device: str = "cuda"):
        self.seed = seed
        self.device = device

    def _gen(self, name: str):
        import torch
        g = torch.Generator(device=self.device)
        g.manual_seed(subseed(self.seed, name))
        return g

    def normal(self, name: str, shape, std: float):
        import torch
        return torch.randn(*shape, generator=self._gen(name), device=self.device,
                           dtype=torch.float32) * std

    def weight(self, name: str, n: int, k: int, fmt: int, std: float = STD,
               row_std: Optional[np.ndarray] = None):
        import torch
        w = self.normal(name, (n, k), 1.0)
        if row_std is None:
            w *= std
        else:
            w *= torch.from_numpy(row_std).to(w.device)[:, None]
        out = quantize_device(w, fmt)
        del w
        return out

    def act_values(self, name: str, shape, fmt: int, std: float = STD):
        import torch
        v = self.normal(name, shape, std)
        return v if fmt == FMT_F32 else v.to(torch.bfloat16).to(torch.float32)


def quantize_device(w, fmt: int) -> Weight:
    """Same recipe as quantize_host, with torch ops (used only to synthesise
    full-size checkpoints on the device)."""
    import torch
    n, k = w.shape
    if fmt == FMT_W8A16:
        s16 = (w.abs().amax(dim=1) / 127.0).to(torch.float16)
        s = s16.to(torch.float32)[:, None]
        q = torch.where(s > 0, torch.round(w / torch.where(s > 0, s, torch.ones_like(s))),
                        torch.zeros_like(w))
        return Weight(fmt, n, k, codes=q.clamp_(-127, 127).to(torch.int8), scales=s16)
    if fmt == FMT_W4A16:
        wg = w.view(n, k // GROUP, GROUP)
        s16 = (wg.abs().amax(dim=2) / 7.0).to(torch.float16)
        s = s16.to(torch.float32)[:, :, None]
        q = torch.where(s > 0, torch.round(wg / torch.where(s > 0, s, torch.ones_like(s))),
                        torch.zeros_like(wg))
        return Weight(fmt, n, k, codes=q.clamp_(-8, 7).to(torch.int8).view(n, k), scales=s16)
    if fmt == FMT_BF16:
        return Weight(fmt, n, k, values=w.to(torch.bfloat16).to(torch.float32))
    return Weight(fmt, n, k, values=w)
