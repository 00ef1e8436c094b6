"""Pins of how the oracle assembles its pieces into layers and stacks.

The piece pins (RMSNorm, QK norm, RoPE, attention, dequantisation, the delta
rule) do not fix how the pieces are wired: which half of the fused gate/up
gets the SiLU, where the residuals go, which keys a drafter slot sees, how the
target's hidden states reach the drafter, or how the GatedDeltaNet layer forms
its gates and its scaled query.  Each case here uses constructed weights that
collapse the layer to a closed form derived by hand (the derivations are in
tests/golden/assembly_derivations.md), evaluated with scalar math on the
constructed values -- never with the oracle's own functions -- or an exact
invariant that a wiring mistake breaks:

* decoder layer (mirror-sd README, "The Story": a Qwen3-shaped decoder with
  per-head Q/K norm; SwiGLU FFN): one token, where attention over its single
  key returns its value;
* target stack, causal verify and the hidden side-write (mirror-sd README,
  "How It Works": the target verifies the block in one forward and hands its
  intermediate hidden states to the drafter): W_q = 0 makes every visible
  key equally weighted, so each row's attention output is the mean of the
  values it may see;
* drafter (mlx-dspark v0.0.3, "Highlights": one parallel pass over the whole
  block, reusing the target's embedding and lm-head; dflash-mlx note,
  "Technical challenges": conditioned on the target's hidden states): with
  W_q = 0 every slot must average the values of all committed context rows
  and all block slots;
* context keys (mirror-sd README, "The Story": per-head Q/K RMSNorm and
  neox RoPE): scaling W_k by 4 must leave the draft bit-identical (both
  block and context keys are per-head normalised), and shifting every
  position by a constant must leave it unchanged (context keys rotated at
  their own positions, like the block's);
* GatedDeltaNet layer (dflash-mlx note, "Technical challenges"; agentlens
  summary, "How it works"): two tokens with orthogonal keys, where the
  state, the outputs and the tape have closed forms in the gates and the
  1/sqrt(d_k) query scale.
"""
import copy
import math
from dataclasses import replace

import numpy as np
import pytest

from dflash_block_diffusion_amd import configs as C
from dflash_block_diffusion_amd import synth
from dflash_block_diffusion_amd.synth import Weight
from oracle.gdn import gdn_layer
from oracle.model import Shape
from oracle.numerics import rounder
from oracle.spec import OracleDrafter, OracleTarget

EPS = 1e-6


# ----------------------------------------------------- scalar helpers (test side)
def _rms_scale(v):
    """1 / sqrt(mean(v^2) + eps) for a short tuple, by plain scalar math."""
    return 1.0 / math.sqrt(sum(t * t for t in v) / len(v) + EPS)


def _norm(v, g=None):
    r = _rms_scale(v)
    g = g or (1.0,) * len(v)
    return tuple(t * r * gi for t, gi in zip(v, g))


def _silu(z):
    return z / (1.0 + math.exp(-z))


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def _add(a, b, c=1.0):
    return tuple(x + c * y for x, y in zip(a, b))


def _lm(v, rows):
    return [sum(vi * wi for vi, wi in zip(v, r)) for r in rows]


# -------------------------------------------------------- constructed weights
def _w(rows):
    a = np.asarray(rows, dtype=np.float32)
    return Weight(C.FMT_F32, a.shape[0], a.shape[1], values=a)


def _shape(L=1, kinds=(), gh=1):
    return C.ModelShape(hidden=2, n_q_heads=1, n_kv_heads=1, head_dim=2, ffn=1, vocab=4,
                        n_layers=L, fmt=C.FMT_F32, layer_kinds=kinds, gdn_heads=gh, gdn_dk=2,
                        gdn_dv=2)


def _attn_layer(wq, wk, wv, wo, wg=(0.0, 0.0), wu=(0.0, 0.0), wd=(0.0, 0.0)):
    """Attention layer of the H=2, one-head, d=2, F=1 shape.  w_gu stacks the
    gate row over the up row; w_down is [H][F]."""
    return {"kind": C.LAYER_ATTN, "in_norm": np.ones(2, np.float32), "post_norm": np.ones(2, np.float32),
            "q_norm": np.ones(2, np.float32), "k_norm": np.ones(2, np.float32),
            "w_qkv": _w(list(wq) + list(wk) + list(wv)), "w_o": _w(wo),
            "w_gu": _w([wg, wu]), "w_down": _w([[wd[0]], [wd[1]]])}


ZERO2 = [[0.0, 0.0], [0.0, 0.0]]
EYE2 = [[1.0, 0.0], [0.0, 1.0]]
W_LM = [[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [2.0, -1.0]]


def _target_ckpt(layers, embed):
    return {"layers": layers, "final_norm": np.ones(2, np.float32),
            "embed": np.asarray(embed, np.float32), "w_lm": _w(W_LM)}


# ---------------------------------------------------------------- decoder layer
def test_decoder_layer_wiring_hand_case():
    """x = (3, 4), one token: o = v = (u0, 2 u1); x1 = x + W_o o with W_o the
    swap; the FFN's gate row reads u2_0, its up row u2_1, and SiLU goes on
    the gate: x2 = x1 + (silu(u2_0) * u2_1, 0)."""
    layer = _attn_layer(ZERO2, ZERO2, [[1.0, 0.0], [0.0, 2.0]], [[0.0, 1.0], [1.0, 0.0]],
                        wg=(1.0, 0.0), wu=(0.0, 1.0), wd=(1.0, 0.0))
    ck = _target_ckpt([layer], [[3.0, 4.0], [0.0, 0.0], [0.0, 0.0], [1.0, 1.0]])
    t = OracleTarget(_shape(), ck, sel_layers=(0,), cap=8)
    out = t.forward([0])

    x0 = (3.0, 4.0)
    u = _norm(x0)
    x1 = _add(x0, (2.0 * u[1], u[0]))
    u2 = _norm(x1)
    x2 = (x1[0] + _silu(u2[0]) * u2[1], x1[1])
    assert np.allclose(out["hidden"][0], x2, rtol=0, atol=1e-12)
    assert np.allclose(out["logits"][0], _lm(_norm(x2), W_LM), rtol=0, atol=1e-12)
    # what the common wiring mistake would give: SiLU on the up half instead
    wrong = x1[0] + _silu(u2[1]) * u2[0]
    assert abs(out["hidden"][0][0] - wrong) > 1e-3


def test_verify_causal_mask_residuals_and_side_write_hand_case():
    """Two layers, two tokens, W_q = 0 so a row's attention output is the mean
    of the values it may see: row 0 sees key 0, row 1 keys 0 and 1.  Layer l
    adds c_l times that mean (c = 1, 2) to the residual; the FFN is zero.  The
    side-write of a conditioning layer is that layer's output residual."""
    l0 = _attn_layer(ZERO2, EYE2, EYE2, EYE2)
    l1 = _attn_layer(ZERO2, EYE2, EYE2, [[2.0, 0.0], [0.0, 2.0]])
    embed = [[3.0, 4.0], [0.0, 0.0], [0.0, 0.0], [2.0, -1.0]]
    t = OracleTarget(_shape(L=2), _target_ckpt([l0, l1], embed), sel_layers=(0, 1), cap=8)
    out = t.forward([0, 3])

    xa, xb = (3.0, 4.0), (2.0, -1.0)
    ua, ub = _norm(xa), _norm(xb)
    ya = _add(xa, ua)
    yb = _add(xb, tuple((p + q) / 2 for p, q in zip(ua, ub)))
    va, vb = _norm(ya), _norm(yb)
    za = _add(ya, va, 2.0)
    zb = _add(yb, tuple((p + q) / 2 for p, q in zip(va, vb)), 2.0)
    assert np.allclose(out["hidden"], [ya + za, yb + zb], rtol=0, atol=1e-12)
    assert np.allclose(out["logits"], [_lm(_norm(za), W_LM), _lm(_norm(zb), W_LM)], rtol=0, atol=1e-12)
    # the committed keys are the block rows' (k-normed, rotated) keys and
    # values; a later forward sees them as context
    t.commit(out, 1)
    assert t.n == 2


# ---------------------------------------------------------------------- drafter
def _drafter_case():
    """Target: embedding and lm-head only.  Drafter: one layer with W_q = 0,
    W_k = W_v = W_o = I and a zero FFN; fc picks the second conditioning
    layer's hidden state; its own final norm has gain (2, 0.5)."""
    embed = [[3.0, 4.0], [0.0, 0.0], [0.0, 0.0], [2.0, -1.0]]
    tck = _target_ckpt([], embed)
    dck = {"layers": [_attn_layer(ZERO2, EYE2, EYE2, EYE2)],
           "final_norm": np.array([2.0, 0.5], np.float32),
           "hidden_norm": np.ones(2, np.float32),
           "w_fc": _w([[0.0, 0.0, 1.0, 0.0], [0.0, 0.0, 0.0, 1.0]])}
    return tck, dck


def test_drafter_sees_whole_context_and_whole_block_closed_form():
    """Block [anchor=0, m, m] (m = 3) at positions 2..4 after two context
    rows.  Every slot attends uniformly to all 2 + 3 keys, so each gets the
    same o = (c_0 + c_1 + u_0 + u_1 + u_2) / 5, where c_p = RMSNorm(fc(h_p))
    are the context features and u_j = RMSNorm(E[block_j]) the block's own
    values.  Logits of slots 1, 2 = RMSNorm(E[m] + o) * (2, 0.5) times the
    target's lm-head."""
    tck, dck = _drafter_case()
    d = OracleDrafter(_shape(), dck, tck, mask_token=3, block=3, cap=8)
    hidden = np.array([[9.0, 9.0, 1.0, 0.0], [7.0, -7.0, 0.0, 2.0]])   # concat(h_layer0, h_layer1)
    d.ctx_append(hidden, np.arange(2))
    drafts, logits = d.draft(anchor=0, n=2)

    c0, c1 = _norm((1.0, 0.0)), _norm((0.0, 2.0))
    u0, um = _norm((3.0, 4.0)), _norm((2.0, -1.0))
    o = tuple((a + b + p + 2.0 * q) / 5.0 for a, b, p, q in zip(c0, c1, u0, um))
    xf = _norm(_add((2.0, -1.0), o), (2.0, 0.5))
    want = _lm(xf, W_LM)
    assert logits.shape == (2, 4)
    assert np.allclose(logits, [want, want], rtol=0, atol=1e-12)
    assert drafts.tolist() == [int(np.argmax(want))] * 2
    # a causal mask inside the block would give slot 1 only four keys
    o_causal = tuple((a + b + p + q) / 4.0 for a, b, p, q in zip(c0, c1, u0, um))
    assert np.max(np.abs(np.array(_lm(_norm(_add((2.0, -1.0), o_causal), (2.0, 0.5)), W_LM)) - want)) > 1e-3


@pytest.fixture(scope="module")
def tiny_eps0():
    cfg = C.tiny()
    cfg = replace(cfg, drafter=replace(cfg.drafter, eps=0.0))
    ck = synth.make_pair(cfg)
    rng = np.random.default_rng(11)
    hidden = rng.standard_normal((40, len(cfg.sel_layers) * cfg.target.hidden))
    return cfg, ck, hidden


def _draft_logits(cfg, ck, hidden, shift=0):
    d = OracleDrafter(cfg.drafter, ck["drafter"], ck["target"], cfg.mask_token, cfg.block, 256)
    if shift:
        d.cos, d.sin = d.cos[shift:], d.sin[shift:]
    n = hidden.shape[0]
    d.ctx_append(hidden, np.arange(n))
    return d.draft(anchor=5, n=n)[1]


def test_drafter_keys_are_per_head_normalised_including_context_keys(tiny_eps0):
    """With eps = 0, RMSNorm(4 z) equals RMSNorm(z) bit for bit, so scaling
    the key rows (or the query rows) of every drafter W_qkv by 4 must leave
    the draft logits bit-identical.  A context key stored without its
    per-head norm would be 4x larger and change every score it enters."""
    cfg, ck, hidden = tiny_eps0
    base = _draft_logits(cfg, ck, hidden)
    s = Shape(cfg.drafter)
    nq, nk = s.hq * s.d, s.hkv * s.d
    for lo, hi in ((nq, nq + nk), (0, nq)):
        ck2 = copy.deepcopy(ck)
        for L in ck2["drafter"]["layers"]:
            L["w_qkv"].values[lo:hi] *= np.float32(4.0)
        assert np.array_equal(_draft_logits(cfg, ck2, hidden), base)
    # and the value rows are not normalised: scaling them changes the draft
    ck3 = copy.deepcopy(ck)
    for L in ck3["drafter"]["layers"]:
        L["w_qkv"].values[nq + nk:] *= np.float32(4.0)
    assert not np.allclose(_draft_logits(cfg, ck3, hidden), base, atol=1e-3)


def test_drafter_depends_on_relative_positions_only(tiny_eps0):
    """RoPE enters attention through position differences alone when the
    context keys are rotated at their own positions and the block's at
    n..n+B-1: shifting every position by 37 leaves the draft unchanged up
    to the fp32 precision of the cos/sin table."""
    cfg, ck, hidden = tiny_eps0
    base = _draft_logits(cfg, ck, hidden)
    shifted = _draft_logits(cfg, ck, hidden, shift=37)
    assert np.allclose(shifted, base, rtol=1e-5, atol=1e-6)


# --------------------------------------------------------------- GatedDeltaNet
def test_gdn_layer_two_token_closed_form():
    """One head, d_k = d_v = 2, x = [(3, 0), (0, 5)], zero initial state.
    Projections: q = (u0 + u1, 0), k = v = u, a = u0 + u1, b = u0 / 2.
    With p = 3/sqrt(4.5+eps), s = 5/sqrt(12.5+eps), kappa1 = p/sqrt(p^2+1e-6),
    kappa2 = s/sqrt(s^2+1e-6):  khat_1 = (kappa1, 0), khat_2 = (0, kappa2),
    qhat_1 = (kappa1, 0)/sqrt 2, qhat_2 = (kappa2, 0)/sqrt 2,
    alpha_t = sigmoid(-a_t), beta_t = sigmoid(b_t).
    Token 1: S_1 = beta_1 v_1 khat_1^T, o_1 = S_1 qhat_1 = (beta_1 p kappa1^2/sqrt 2, 0).
    Token 2: S_1 khat_2 = 0, so u_2 = beta_2 v_2 and
    S_2 = alpha_2 S_1 + beta_2 v_2 khat_2^T, o_2 = (alpha_2 beta_1 p kappa1 kappa2/sqrt 2, 0).
    W_o = I and a zero FFN give x_out = x + o."""
    shp = _shape(kinds=(C.LAYER_GDN,), gh=1)
    L = {"kind": C.LAYER_GDN, "in_norm": np.ones(2, np.float32), "post_norm": np.ones(2, np.float32),
         # rows: q (2), k (2), v (2), a (1), b (1)
         "w_qkv": _w([[1.0, 1.0], [0.0, 0.0], [1.0, 0.0], [0.0, 1.0], [1.0, 0.0], [0.0, 1.0],
                      [1.0, 1.0], [0.5, 0.0]]),
         "w_o": _w(EYE2), "w_gu": _w(ZERO2), "w_down": _w([[0.0], [0.0]])}
    s = Shape(shp)
    x = np.array([[3.0, 0.0], [0.0, 5.0]])
    out, tape, states = gdn_layer(L, x, np.zeros((1, 2, 2)), s, rounder("f32"))

    p = 3.0 / math.sqrt(4.5 + EPS)
    sq = 5.0 / math.sqrt(12.5 + EPS)
    k1 = p / math.sqrt(p * p + 1e-6)
    k2 = sq / math.sqrt(sq * sq + 1e-6)
    a1, a2, b1, b2 = p, sq, 0.5 * p, 0.0
    al1, al2, be1, be2 = _sig(-a1), _sig(-a2), _sig(b1), _sig(b2)
    r2 = math.sqrt(2.0)
    o1 = (be1 * p * k1 * k1 / r2, 0.0)
    o2 = (al2 * be1 * p * k1 * k2 / r2, 0.0)
    assert np.allclose(out, [[3.0 + o1[0], 0.0], [o2[0], 5.0]], rtol=0, atol=1e-12)
    S2 = [[al2 * be1 * p * k1, 0.0], [0.0, be2 * sq * k2]]
    assert np.allclose(states[1][0], S2, rtol=0, atol=1e-12)
    assert np.allclose(tape["k"][:, 0], [[k1, 0.0], [0.0, k2]], atol=1e-7)
    assert np.allclose(tape["v"][:, 0], [[p, 0.0], [0.0, sq]], atol=1e-7)
    assert np.allclose(tape["alpha"][:, 0], [al1, al2], atol=1e-7)
    assert np.allclose(tape["beta"][:, 0], [be1, be2], atol=1e-7)
    # the unscaled query would give o_1 larger by sqrt 2
    assert abs(out[0, 0] - (3.0 + be1 * p * k1 * k1)) > 1e-2
