"""Pins of the GatedDeltaNet recurrence and its tape-replay rollback."""
import numpy as np
import pytest

from oracle.gdn import gates, halving_sum, l2norm, recurrence, recurrence_chunked, replay_pinned
from oracle.model import sigmoid


def _tape(rng, T, gh=2, dk=16, dv=16):
    k = l2norm(rng.standard_normal((T, gh, dk)))
    q = l2norm(rng.standard_normal((T, gh, dk))) / np.sqrt(dk)
    v = rng.standard_normal((T, gh, dv))
    alpha, beta = gates(rng.standard_normal((T, gh)), rng.standard_normal((T, gh)))
    return q, k, v, alpha, beta


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(0)
    q, k, v, alpha, _ = _tape(rng, 5)
    S0 = rng.standard_normal((2, 16, 16))
    _, st = recurrence(S0, q, k, v, alpha, np.zeros_like(alpha))
    expect = S0 * np.prod(alpha, axis=0)[:, None, None]
    assert np.allclose(st[-1], expect, rtol=1e-13)
    # pinned fp32: beta = 0 gives exactly alpha * S (u = 0 exactly)
    S32 = S0.astype(np.float32)
    out = replay_pinned(S32, k[:1].astype(np.float32), v[:1].astype(np.float32),
                        alpha[:1].astype(np.float32), np.zeros((1, 2), np.float32))
    assert np.array_equal(out, alpha[0].astype(np.float32)[:, None, None] * S32)


def test_unit_gates_write_value_exactly():
    # alpha = beta = 1 and |k| = 1: the delta rule stores v at key k, S_t k = v
    rng = np.random.default_rng(1)
    q, _, v, _, _ = _tape(rng, 1)
    raw = rng.standard_normal((1, 2, 16))
    k = raw / np.linalg.norm(raw, axis=-1, keepdims=True)      # exactly unit length
    S0 = rng.standard_normal((2, 16, 16))
    one = np.ones((1, 2))
    _, st = recurrence(S0, q, k, v, one, one)
    assert np.allclose(np.einsum("hij,hj->hi", st[0], k[0]), v[0], atol=1e-12)


def test_gate_identity():
    a = np.linspace(-8, 8, 33)
    alpha, beta = gates(a, a)
    assert np.allclose(alpha, sigmoid(-a), rtol=1e-14)
    assert np.allclose(beta, sigmoid(a), rtol=1e-14)


def test_recurrence_matches_matrix_form():
    # S_t = alpha S (I - beta k k^T) + beta v k^T, written as a matrix product
    rng = np.random.default_rng(2)
    q, k, v, alpha, beta = _tape(rng, 4)
    S0 = rng.standard_normal((2, 16, 16))
    _, st = recurrence(S0, q, k, v, alpha, beta)
    S = S0.copy()
    for t in range(4):
        for h in range(2):
            kk = np.outer(k[t, h], k[t, h])
            S[h] = alpha[t, h] * S[h] @ (np.eye(16) - beta[t, h] * kk) + beta[t, h] * np.outer(v[t, h], k[t, h])
    assert np.allclose(st[-1], S, rtol=1e-12, atol=1e-12)


def test_halving_sum_order(hand_cases):
    c = hand_cases["halving_sum_order"]
    x = np.array(c["x_f32"], np.float32)
    assert halving_sum(x) == np.float32(c["halving_tree"])
    acc = np.float32(0)
    for e in x:
        acc = np.float32(acc + e)
    assert acc == np.float32(c["left_to_right"])
    # integer-valued inputs: exact sum in any order
    y = np.arange(128, dtype=np.float32)
    assert halving_sum(y) == np.float32(127 * 128 // 2)


def test_pinned_replay_close_to_float64():
    rng = np.random.default_rng(3)
    q, k, v, alpha, beta = _tape(rng, 12, gh=3, dk=32, dv=32)
    S0 = rng.standard_normal((3, 32, 32)) * 0.1
    _, st = recurrence(S0, q, k, v, alpha, beta)
    S = replay_pinned(S0.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                      alpha.astype(np.float32), beta.astype(np.float32))
    assert np.allclose(S, st[-1], rtol=1e-5, atol=1e-5)


def test_pinned_replay_split_is_bitwise():
    rng = np.random.default_rng(4)
    _, k, v, alpha, beta = _tape(rng, 10)
    f = lambda a: np.asarray(a, np.float32)
    S0 = f(rng.standard_normal((2, 16, 16)))
    full = replay_pinned(S0, f(k), f(v), f(alpha), f(beta))
    part = replay_pinned(S0, f(k[:4]), f(v[:4]), f(alpha[:4]), f(beta[:4]))
    part = replay_pinned(part, f(k[4:]), f(v[4:]), f(alpha[4:]), f(beta[4:]))
    assert np.array_equal(full, part)


def test_commit_state_equals_tape_replay():
    # rollback: the state after accepting a+1 of T tokens equals replaying the
    # first a+1 tape entries from the committed state; later tokens leave no trace
    rng = np.random.default_rng(5)
    q, k, v, alpha, beta = _tape(rng, 8)
    S0 = rng.standard_normal((2, 16, 16))
    _, st = recurrence(S0, q, k, v, alpha, beta)
    for a in (0, 3, 7):
        _, st2 = recurrence(S0, q[:a + 1], k[:a + 1], v[:a + 1], alpha[:a + 1], beta[:a + 1])
        assert np.array_equal(st2[-1], st[a])


def test_chunked_form_equals_sequential():
    # the UT / WY chunk form is an exact rewriting of the sequential rule
    rng = np.random.default_rng(6)
    q, k, v, alpha, beta = _tape(rng, 16, gh=3, dk=32, dv=32)
    S0 = rng.standard_normal((3, 32, 32))
    o_seq, st = recurrence(S0, q, k, v, alpha, beta)
    o_ch, S_end = recurrence_chunked(S0, q, k, v, alpha, beta)
    assert np.allclose(o_ch, o_seq, rtol=1e-10, atol=1e-10)
    assert np.allclose(S_end, st[-1], rtol=1e-10, atol=1e-10)


def test_chunked_form_special_cases():
    rng = np.random.default_rng(7)
    q, k, v, alpha, beta = _tape(rng, 6)
    S0 = rng.standard_normal((2, 16, 16))
    # beta = 0: pure decay, o_t = gamma_t S0 q_t
    o, S_end = recurrence_chunked(S0, q, k, v, alpha, np.zeros_like(beta))
    gam = np.cumprod(alpha, axis=0)
    assert np.allclose(o, gam[:, :, None] * np.einsum("hij,thj->thi", S0, q), rtol=1e-12, atol=1e-13)
    assert np.allclose(S_end, gam[-1][:, None, None] * S0, rtol=1e-12)
    # one token: one step of the rule
    o1, S1 = recurrence_chunked(S0, q[:1], k[:1], v[:1], alpha[:1], beta[:1])
    r = v[0] - alpha[0][:, None] * np.einsum("hij,hj->hi", S0, k[0])
    Sx = alpha[0][:, None, None] * S0 + (beta[0][:, None] * r)[:, :, None] * k[0][:, None, :]
    assert np.allclose(S1, Sx, rtol=1e-13, atol=1e-13)
    assert np.allclose(o1[0], np.einsum("hij,hj->hi", Sx, q[0]), rtol=1e-13, atol=1e-13)


def test_chunks_chain():
    # two chunks chained through the end state equal one chunk of both
    rng = np.random.default_rng(8)
    q, k, v, alpha, beta = _tape(rng, 12)
    S0 = rng.standard_normal((2, 16, 16))
    o, S_end = recurrence_chunked(S0, q, k, v, alpha, beta)
    oa, Sa = recurrence_chunked(S0, q[:5], k[:5], v[:5], alpha[:5], beta[:5])
    ob, Sb = recurrence_chunked(Sa, q[5:], k[5:], v[5:], alpha[5:], beta[5:])
    assert np.allclose(np.concatenate([oa, ob]), o, rtol=1e-11, atol=1e-11)
    assert np.allclose(Sb, S_end, rtol=1e-11, atol=1e-11)
