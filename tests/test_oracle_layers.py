"""Pins of the oracle's layer pieces: RMSNorm, per-head QK norm, neox RoPE,
attention masks and GQA, activations, argmax."""
import numpy as np
import pytest

from oracle.model import (argmax_first, attention, head_rmsnorm, rmsnorm, rope_neox,
                          rope_table, sigmoid, silu, softplus)


def test_rmsnorm_hand_case(hand_cases):
    c = hand_cases["rmsnorm"]
    assert np.allclose(rmsnorm(np.array(c["x"]), np.array(c["g"]), c["eps"]), c["y"], atol=1e-7)


def test_qk_norm_is_per_head(hand_cases):
    c = hand_cases["qk_norm_per_head"]
    z = np.array(c["heads"])[None]                     # [T=1, heads=2, d=2]
    out = head_rmsnorm(z, np.ones(2), c["eps"])[0]
    assert np.allclose(out, c["per_head"], atol=1e-7)
    # the bug signature: one norm across all channels
    glob = rmsnorm(z.reshape(1, 4), np.ones(4), c["eps"])[0]
    assert np.allclose(glob, c["global_bug"], atol=1e-7)
    assert not np.allclose(out.reshape(-1), glob, atol=1e-2)


def test_rope_hand_cases(hand_cases):
    c = hand_cases["rope_neox"]
    cos, sin = rope_table(4, c["d"], c["base"])
    assert np.allclose(cos[1], [np.cos(1.0), np.cos(1e-3)], atol=1e-7)
    for case in c["cases"]:
        x = np.array(case["x"])[None, None]
        y = rope_neox(x, np.array([c["pos"]]), cos, sin)[0, 0]
        assert np.allclose(y, case["y"], atol=1e-6)
        if "interleaved_would_give" in case:
            assert not np.allclose(y, case["interleaved_would_give"], atol=1e-3)
    # position 0 is the identity
    x = np.random.default_rng(0).standard_normal((1, 1, 4))
    assert np.allclose(rope_neox(x, np.array([0]), cos, sin), x, atol=0)


def test_rope_relative_position_invariance():
    d = 64
    cos, sin = rope_table(64, d, 1e6)
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))

    def dot(m, n):
        return float((rope_neox(q, np.array([m]), cos, sin) * rope_neox(k, np.array([n]), cos, sin)).sum())
    assert dot(9, 4) == pytest.approx(dot(40, 35), rel=1e-6)
    assert dot(9, 4) != pytest.approx(dot(9, 5), rel=1e-3)
    # a rotation keeps the norm
    r = rope_neox(q, np.array([17]), cos, sin)
    assert np.linalg.norm(r) == pytest.approx(np.linalg.norm(q), rel=1e-6)


def _brute_attention(q, k, v, visible):
    tq, hq, d = q.shape
    hkv = k.shape[1]
    out = np.zeros_like(q)
    for t in range(tq):
        for h in range(hq):
            j = h // (hq // hkv)
            ws = []
            for s in range(k.shape[0]):
                if visible[t, s]:
                    ws.append((s, np.exp(sum(q[t, h, c] * k[s, j, c] for c in range(d)) / np.sqrt(d))))
            tot = sum(w for _, w in ws)
            for s, w in ws:
                out[t, h] += w / tot * v[s, j]
    return out


def test_attention_against_brute_force_softmax():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((3, 4, 8))
    k = rng.standard_normal((5, 2, 8))
    v = rng.standard_normal((5, 2, 8))
    vis = np.arange(5)[None, :] <= (2 + np.arange(3))[:, None]
    assert np.allclose(attention(q, k, v, vis), _brute_attention(q, k, v, vis), atol=1e-12)


def test_gqa_head_mapping():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 4, 8))
    k = rng.standard_normal((6, 2, 8))
    v = rng.standard_normal((6, 2, 8))
    vis = np.ones((2, 6), bool)
    base = attention(q, k, v, vis)
    v2 = v.copy()
    v2[:, 1] += 1.0                       # touch KV head 1 only
    out = attention(q, k, v2, vis)
    assert np.allclose(out[:, :2], base[:, :2])          # q heads 0,1 read KV head 0
    assert not np.allclose(out[:, 2:], base[:, 2:])      # q heads 2,3 read KV head 1


def test_draft_mask_bidirectional_verify_mask_causal():
    rng = np.random.default_rng(4)
    n, B = 5, 4
    q = rng.standard_normal((B, 2, 8))
    k = rng.standard_normal((n + B, 1, 8))
    v = rng.standard_normal((n + B, 1, 8))
    k2 = k.copy()
    k2[n + B - 1] += 3.0                  # change the last block slot's key
    v2 = v.copy()
    v2[n + B - 1] += 3.0
    draft = np.ones((B, n + B), bool)
    verify = np.arange(n + B)[None, :] <= (n + np.arange(B))[:, None]
    d0, d1 = attention(q, k, v, draft), attention(q, k2, v2, draft)
    assert not np.allclose(d0[0], d1[0])                 # earlier slots see later ones
    c0, c1 = attention(q, k, v, verify), attention(q, k2, v2, verify)
    assert np.array_equal(c0[:B - 1], c1[:B - 1])        # causal: earlier rows untouched
    assert not np.allclose(c0[B - 1], c1[B - 1])


def test_activation_closed_forms():
    assert silu(0.0) == 0.0
    assert silu(30.0) == pytest.approx(30.0, rel=1e-12)
    assert sigmoid(0.0) == 0.5
    assert softplus(0.0) == pytest.approx(np.log(2.0), rel=1e-15)
    a = np.linspace(-6, 6, 13)
    assert np.allclose(np.exp(-softplus(a)), sigmoid(-a), rtol=1e-14)


def test_argmax_lowest_index_on_ties():
    assert argmax_first(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert argmax_first(np.array([[0.0, 0.0], [2.0, 5.0]])).tolist() == [0, 1]
