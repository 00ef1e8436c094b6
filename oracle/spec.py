"""Oracle of the whole loop: prefill, draft, verify, accept, commit, generate.

One draft+verify step (mirror-sd README, "How It Works"; dflash-mlx note,
"How it works"; agentlens summary, "How it works"):

1. draft: the drafter denoises a block [anchor, m, ..., m] of B slots at
   positions n..n+B-1 in ONE parallel pass (mlx-dspark v0.0.3, "Highlights");
   slot j (1 <= j < B) predicts the token at position n+j; its keys/values are
   the committed context features (projected target hidden states, one row
   per committed position) plus the B block slots, all visible to every slot.
2. verify: the target runs [anchor, d_1..d_{B-1}] in one forward at positions
   n..n+B-1 over its committed KV cache, causal inside the block; y_i is the
   argmax of row i.
3. accept: a = the largest k <= B-1 with d_j == y_{j-1} for all j <= k; emit
   d_1..d_a and the correction y_a (B tokens when every draft matches).
4. commit: keep the KV of positions n..n+a, drop the rest; n <- n+a+1; the
   target hidden states of those a+1 rows become new drafter context rows;
   GatedDeltaNet layers replay their tape for the a+1 tokens.

Draft cap (mlx-dspark v0.0.3, "Highlights" and "API", --max-draft; its
head-to-head table compares a cap of 2 with the full 16-block): with N > 0
only the first min(N, B-1) drafts are verified -- the target forward runs the
anchor and those drafts and a <= N; 0 verifies the whole block.  The drafter
still drafts the whole block.

Temperature T > 0 (mlx-dspark v0.0.3, "Highlights"): drafts are sampled
from the drafter's tempered distributions and accepted by the speculative
sampling rule of oracle/sampling.py; T = 0 is the greedy loop above.

Greedy speculative output equals plain greedy decoding of the target
(mlx-dspark v0.0.3 intro; agentlens summary, "Highlights") -- the invariant
tests check on this oracle.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from .gdn import gdn_layer, recurrence
from .model import (F64, LAYER_ATTN, Shape, argmax_first, attention, ffn_block,
                    norm_rope, qkv_heads, rmsnorm, rope_table, top2_margin)
from .numerics import linear, rounder
from .sampling import STREAM_FIRST, categorical, draft_samples, spec_accept, tempered, uniform


class OracleTarget:
    def __init__(self, shape, ckpt: Dict, sel_layers, cap: int):
        self.s = s = Shape(shape)
        self.R = rounder(s.act)
        self.ck = ckpt
        self.sel = list(sel_layers)
        self.cap = cap
        self.cos, self.sin = rope_table(cap, s.d, s.base)
        self.K, self.V, self.S = {}, {}, {}
        for l, kind in enumerate(s.kinds):
            if kind == LAYER_ATTN:
                self.K[l] = np.zeros((cap, s.hkv, s.d), F64)
                self.V[l] = np.zeros((cap, s.hkv, s.d), F64)
            else:
                self.S[l] = np.zeros((s.gh, s.dv, s.dk), F64)
        self.n = 0

    def embed(self, tokens):
        return self.R(np.asarray(self.ck["embed"], F64)[np.asarray(tokens)])

    def forward(self, tokens, layers: Optional[int] = None) -> Dict:
        """Target forward of T tokens at positions n..n+T-1, causal.

        Returns logits [T, V] (float64, not rounded), hidden [T, n_sel*H]
        (layer outputs of the conditioning layers), per-layer block K/V or GDN
        traces for commit.
        """
        s, R = self.s, self.R
        T = len(tokens)
        n = self.n
        pos = n + np.arange(T)
        x = self.embed(tokens)
        visible = np.arange(n + T)[None, :] <= (n + np.arange(T))[:, None]
        hidden, blk = [], {}
        nl = s.L if layers is None else layers
        for l in range(nl):
            L = self.ck["layers"][l]
            if s.kinds[l] == LAYER_ATTN:
                u = R(rmsnorm(x, L["in_norm"], s.eps))
                q, k, v = qkv_heads(L, u, s, R)
                q = norm_rope(q, L["q_norm"], pos, s, self.cos, self.sin, R)
                k = norm_rope(k, L["k_norm"], pos, s, self.cos, self.sin, R)
                keys = np.concatenate([self.K[l][:n], k])
                vals = np.concatenate([self.V[l][:n], v])
                o = R(attention(q, keys, vals, visible)).reshape(T, -1)
                x = R(x + R(linear(o, L["w_o"])))
                x = ffn_block(L, x, s, R)
                blk[l] = (k, v)
            else:
                x, tape, states = gdn_layer(L, x, self.S[l], s, R)
                blk[l] = (tape, states)
            if l in self.sel:
                hidden.append(x)
        out = {"blk": blk, "x": x,
               "hidden": np.concatenate(hidden, axis=1) if hidden else None}
        if layers is None:
            xf = R(rmsnorm(x, self.ck["final_norm"], s.eps))
            out["logits"] = linear(xf, self.ck["w_lm"])
        return out

    def commit(self, fwd: Dict, a: int):
        """Keep block rows 0..a: KV written at n..n+a, GDN state = S after token a."""
        n = self.n
        for l, b in fwd["blk"].items():
            if self.s.kinds[l] == LAYER_ATTN:
                k, v = b
                self.K[l][n:n + a + 1] = k[:a + 1]
                self.V[l][n:n + a + 1] = v[:a + 1]
            else:
                self.S[l] = b[1][a].copy()
        self.n = n + a + 1


class OracleDrafter:
    def __init__(self, shape, ckpt: Dict, target_ckpt: Dict, mask_token: int,
                 block: int, cap: int):
        self.s = s = Shape(shape)
        self.R = rounder(s.act)
        self.ck = ckpt
        self.embed_w = target_ckpt["embed"]
        self.w_lm = target_ckpt["w_lm"]
        self.mask = mask_token
        self.B = block
        self.cos, self.sin = rope_table(cap, s.d, s.base)
        self.K = [np.zeros((cap, s.hkv, s.d), F64) for _ in range(s.L)]
        self.V = [np.zeros((cap, s.hkv, s.d), F64) for _ in range(s.L)]
        self.n_ctx = 0

    def ctx_features(self, hidden_rows):
        """c = RMSNorm(fc(concat of the conditioning layers' outputs))."""
        s, R = self.s, self.R
        return R(rmsnorm(R(linear(hidden_rows, self.ck["w_fc"])),
                         self.ck["hidden_norm"], s.eps))

    def ctx_append(self, hidden_rows, pos):
        """Append K/V of new context rows at their own positions (every layer
        projects them with its own k/v weights, QK-norm and RoPE)."""
        s, R = self.s, self.R
        pos = np.asarray(pos)
        c = self.ctx_features(hidden_rows)
        lo = s.hq * s.d
        nk = s.hkv * s.d
        for l in range(s.L):
            L = self.ck["layers"][l]
            kv = R(linear(c, L["w_qkv"], rows=(lo, lo + 2 * nk)))
            t = kv.shape[0]
            k = kv[:, :nk].reshape(t, s.hkv, s.d)
            v = kv[:, nk:].reshape(t, s.hkv, s.d)
            self.K[l][pos] = norm_rope(k, L["k_norm"], pos, s, self.cos, self.sin, R)
            self.V[l][pos] = v
        self.n_ctx = int(pos[-1]) + 1

    def draft(self, anchor: int, n: int):
        """One parallel denoising pass over [anchor, m x (B-1)] -> (drafts, logits)."""
        s, R, B = self.s, self.R, self.B
        tokens = np.array([anchor] + [self.mask] * (B - 1))
        pos = n + np.arange(B)
        x = R(np.asarray(self.embed_w, F64)[tokens])
        visible = np.ones((B, n + B), dtype=bool)
        for l in range(s.L):
            L = self.ck["layers"][l]
            u = R(rmsnorm(x, L["in_norm"], s.eps))
            q, k, v = qkv_heads(L, u, s, R)
            q = norm_rope(q, L["q_norm"], pos, s, self.cos, self.sin, R)
            k = norm_rope(k, L["k_norm"], pos, s, self.cos, self.sin, R)
            keys = np.concatenate([self.K[l][:n], k])
            vals = np.concatenate([self.V[l][:n], v])
            o = R(attention(q, keys, vals, visible)).reshape(B, -1)
            x = R(x + R(linear(o, L["w_o"])))
            x = ffn_block(L, x, s, R)
        xf = R(rmsnorm(x, self.ck["final_norm"], s.eps))
        logits = linear(xf[1:], self.w_lm)
        return argmax_first(logits).astype(np.int64), logits


def accept_length(drafts, y) -> int:
    """a = max{k <= B-1 : d_j == y_{j-1} for all j <= k} (drafts are d_1..d_{B-1})."""
    a = 0
    for j in range(1, len(drafts) + 1):
        if int(drafts[j - 1]) != int(y[j - 1]):
            break
        a = j
    return a


def inject_drafts(drafts, n: int, k: int, ref, filler_row, vocab: int):
    """Benchmark harness: make the first k drafts the reference stream's tokens
    and the (k+1)-th a token that differs from it; later ones are filler."""
    out = np.array(drafts, copy=True)
    for j in range(1, len(out) + 1):
        p = n + j
        if j <= k and p < len(ref):
            out[j - 1] = ref[p]
        else:
            f = int(filler_row[j])
            if j == k + 1 and p < len(ref) and f == int(ref[p]):
                f = (f + 1) % vocab
            out[j - 1] = f
    return out


class OraclePair:
    def __init__(self, cfg, ckpt: Dict, cap: int, max_draft: int = 0, temperature: float = 0.0,
                 seed: int = 0):
        self.cfg = cfg
        self.T, self.seed = float(temperature), int(seed)
        self.B = cfg.block
        # drafts verified per step
        self.N = self.B - 1 if max_draft == 0 else min(int(max_draft), self.B - 1)
        self.t = OracleTarget(cfg.target, ckpt["target"], cfg.sel_layers, cap)
        self.d = OracleDrafter(cfg.drafter, ckpt["drafter"], ckpt["target"],
                               cfg.mask_token, cfg.block, cap)
        self.seq: List[int] = []
        self.anchor = None
        self.steps: List[Dict] = []

    def prefill(self, prompt) -> int:
        prompt = [int(t) for t in prompt]
        fwd = self.t.forward(prompt)
        P = len(prompt)
        self.t.commit(fwd, P - 1)
        self.d.ctx_append(fwd["hidden"], np.arange(P))
        self.anchor = int(argmax_first(fwd["logits"][-1]))
        if self.T > 0:
            self.anchor = categorical(tempered(fwd["logits"][-1], self.T),
                                      uniform(self.seed, P, 0, STREAM_FIRST))
        self.prefill_margin = float(top2_margin(fwd["logits"][-1]))
        self.prefill_logits = fwd["logits"][-1]
        self.seq = prompt + [self.anchor]
        return self.anchor

    def step(self, inject=None) -> Dict:
        """One draft+verify+accept+commit step.  ``inject(drafts, n)`` may
        overwrite the drafts (benchmark acceptance schedule)."""
        n = self.t.n
        drafts, dlogits = self.d.draft(self.anchor, n)
        if self.T > 0:
            drafts = np.array(draft_samples(dlogits, self.T, self.seed, n), dtype=np.int64)
        raw = drafts.copy()
        if inject is not None:
            drafts = inject(drafts, n)
        block = [self.anchor] + [int(t) for t in drafts[:self.N]]
        fwd = self.t.forward(block)
        y = argmax_first(fwd["logits"]).astype(np.int64)
        sample_info = None
        if self.T > 0:
            a, nxt, sample_info = spec_accept(drafts[:self.N], dlogits[:self.N], fwd["logits"], self.T,
                                              self.seed, n)
        else:
            a = accept_length(drafts[:self.N], y)
            nxt = int(y[a])
        self.t.commit(fwd, a)
        self.d.ctx_append(fwd["hidden"][: a + 1], n + np.arange(a + 1))
        emitted = [int(t) for t in drafts[:a]] + [int(nxt)]
        self.anchor = int(nxt)
        self.seq += emitted
        rec = {"n": n, "block": block, "raw_drafts": raw, "drafts": drafts, "y": y,
               "a": a, "emitted": emitted, "draft_logits": dlogits,
               "logits": fwd["logits"], "hidden": fwd["hidden"],
               "draft_margin": top2_margin(dlogits),
               "verify_margin": top2_margin(fwd["logits"]), "fwd": fwd, "sample": sample_info}
        self.steps.append(rec)
        return rec

    def generate(self, prompt, max_new: int, inject=None) -> List[int]:
        self.prefill(prompt)
        out = [self.anchor]
        while len(out) < max_new:
            out += self.step(inject)["emitted"]
        return out[:max_new]


def greedy(cfg, ckpt: Dict, prompt, max_new: int, cap: int) -> List[int]:
    """Plain greedy decoding of the target, one token per forward."""
    t = OracleTarget(cfg.target, ckpt["target"], cfg.sel_layers, cap)
    prompt = [int(x) for x in prompt]
    fwd = t.forward(prompt)
    t.commit(fwd, len(prompt) - 1)
    tok = int(argmax_first(fwd["logits"][-1]))
    out = [tok]
    while len(out) < max_new:
        fwd = t.forward([tok])
        t.commit(fwd, 0)
        tok = int(argmax_first(fwd["logits"][-1]))
        out.append(tok)
    return out
