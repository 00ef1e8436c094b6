"""Oracle forward passes: decoder layers, target stack, drafter stack.

Notation: H hidden, hq/hkv query/KV heads, d head dim, F FFN width, V vocab,
B block, n committed (target-processed) tokens.  ``R`` is the stack's
materialisation rounding (bf16, or none for fp32 models); everything between
two roundings is float64.  bf16 is materialised at: embedding rows, every
RMSNorm output, every GEMM output except the logits, q/k after QK-norm+RoPE,
the KV cache, the attention output, each residual add and the SiLU*mul
output.

Layer (Qwen3-shaped decoder, which the DFlash pairs on the pages use; the
per-head Q/K norm and neox RoPE are the two details mirror-sd's README,
"The Story", had to get right):

  u = RMSNorm(x; g_in);  q,k,v = u W_qkv^T;  q,k <- per-head RMSNorm over d,
  then neox RoPE at their positions;  o = softmax(q k^T / sqrt(d) + mask) v;
  x += o W_o^T;  u2 = RMSNorm(x; g_post);  x += (silu(u2 W_g^T) * u2 W_u^T) W_d^T

GQA: query head i reads KV head floor(i * hkv / hq).
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from .numerics import F64, dequant, linear, rounder

LAYER_ATTN = 0
LAYER_GDN = 1


# ------------------------------------------------------------------ pieces
def rmsnorm(z, g, eps):
    """z * (mean(z^2) + eps)^-1/2 * g over the last axis."""
    z = np.asarray(z, F64)
    r = 1.0 / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)
    return z * r * np.asarray(g, F64)


def head_rmsnorm(z, g, eps):
    """RMSNorm of every head separately: z is [..., heads, d], g is [d].
    Normalising across all channels at once instead is the bug mirror-sd's
    README ("The Story") reports (cosine ~0.5 against the reference)."""
    return rmsnorm(z, g, eps)


def rope_table(n_pos: int, d: int, base: float):
    """cos/sin of pos * base^(-2i/d), i < d/2: angles in float64, table in fp32."""
    i = np.arange(d // 2, dtype=F64)
    inv_freq = base ** (-2.0 * i / d)
    ang = np.arange(n_pos, dtype=F64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_neox(x, pos, cos, sin):
    """Split-half rotation: pairs (i, i + d/2) (mirror-sd README, "The Story":
    neox convention, mx.fast.rope(traditional=False)).  x is [T, heads, d]."""
    x = np.asarray(x, F64)
    d = x.shape[-1]
    h = d // 2
    c = cos[pos].astype(F64)[:, None, :]
    s = sin[pos].astype(F64)[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q, k, v, visible):
    """q [Tq, hq, d], k/v [Tk, hkv, d], visible [Tq, Tk] bool -> [Tq, hq, d]."""
    q, k, v = (np.asarray(a, F64) for a in (q, k, v))
    tq, hq, d = q.shape
    hkv = k.shape[1]
    out = np.empty((tq, hq, d), F64)
    for i in range(hq):
        j = (i * hkv) // hq
        s = q[:, i, :] @ k[:, j, :].T / np.sqrt(d)
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        p /= p.sum(axis=1, keepdims=True)
        out[:, i, :] = p @ v[:, j, :]
    return out


def silu(z):
    z = np.asarray(z, F64)
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    z = np.asarray(z, F64)
    return 1.0 / (1.0 + np.exp(-z))


def softplus(z):
    z = np.asarray(z, F64)
    return np.logaddexp(0.0, z)


def argmax_first(logits):
    """Row-wise argmax, lowest index on ties."""
    return np.argmax(np.asarray(logits), axis=-1)


def top2_margin(logits):
    part = np.sort(np.asarray(logits, F64), axis=-1)
    return part[..., -1] - part[..., -2]


# ------------------------------------------------------------ stack state
class Shape:
    """Plain view of a ModelShape (oracle takes duck-typed configs)."""

    def __init__(self, m):
        self.H, self.hq, self.hkv, self.d = m.hidden, m.n_q_heads, m.n_kv_heads, m.head_dim
        self.F, self.V, self.L = m.ffn, m.vocab, m.n_layers
        self.kinds = list(m.kinds())
        self.gh, self.dk, self.dv = m.gdn_heads, m.gdn_dk, m.gdn_dv
        self.eps, self.base = m.eps, m.rope_base
        self.act = "f32" if m.fmt == 0 else "bf16"


def ffn_block(L, x, s: Shape, R):
    u2 = R(rmsnorm(x, L["post_norm"], s.eps))
    gu = R(linear(u2, L["w_gu"]))
    g, up = gu[:, : s.F], gu[:, s.F:]
    act = R(silu(g) * up)
    return R(x + R(linear(act, L["w_down"])))


def qkv_heads(L, u, s: Shape, R):
    qkv = R(linear(u, L["w_qkv"]))
    t = qkv.shape[0]
    nq = s.hq * s.d
    nk = s.hkv * s.d
    return (qkv[:, :nq].reshape(t, s.hq, s.d),
            qkv[:, nq:nq + nk].reshape(t, s.hkv, s.d),
            qkv[:, nq + nk:].reshape(t, s.hkv, s.d))


def norm_rope(z, g, pos, s: Shape, cos, sin, R):
    return R(rope_neox(head_rmsnorm(z, g, s.eps), pos, cos, sin))
