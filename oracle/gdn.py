"""GatedDeltaNet layer of the hybrid target, and its tape-replay rollback.

The dflash-mlx note ("Technical challenges") and the agentlens summary of
bstnxbt/dflash-mlx ("How it works") say that for hybrid GatedDeltaNet +
attention targets the recurrent state is rolled back by replaying a tape
recorded during verify, instead of snapshotting the whole state.  They give
no formula; the layer below is the gated delta rule in its plain sequential
form, per head, with state S of shape [dv, dk]:

    r_t = v_t - alpha_t * S_{t-1} k_t
    u_t = beta_t * r_t
    S_t = alpha_t * S_{t-1} + u_t k_t^T        (= alpha S (I - beta k k^T) + beta v k^T)
    o_t = S_t q_t

with q, k L2-normalised (z / sqrt(sum z^2 + 1e-6)), q additionally scaled by
1/sqrt(dk), alpha_t = exp(-softplus(a_t)) and beta_t = sigmoid(b_t).  No
short convolution, no output gate (the pages name neither).

The tape of one token and head is (k_t, v_t, alpha_t, beta_t) in fp32.
Committing a+1 tokens replays the tape of those tokens from the committed
state; rejected tokens leave no trace.

The verify runs the B tokens of a block in the chunked (UT / WY) form of the
same rule (``recurrence_chunked``), which the tests pin against the
sequential definition above.

Bit-exact replay.  ``replay_pinned`` fixes the fp32 operation order so that
two implementations can agree to the bit: per token, per head, per value row
i,

    prod_j = S[i, j] * k[j]                      (rounded fp32 products)
    acc    = halving-tree sum of prod over j:  at each level the first half
             of the vector is added elementwise to the second half, until one
             element is left (dk must be a power of two)
    p = alpha * acc;  r = v[i] - p;  u = beta * r
    S[i, j] = (alpha * S[i, j]) + (u * k[j])     (three rounded ops)

all round-to-nearest-even, no fused multiply-add, no flush of subnormals.
"""
from __future__ import annotations

import numpy as np

from .model import F64, Shape, ffn_block, rmsnorm, sigmoid, softplus
from .numerics import linear


def l2norm(z, eps=1e-6):
    z = np.asarray(z, F64)
    return z / np.sqrt(np.sum(z * z, axis=-1, keepdims=True) + eps)


def gates(a, b):
    """alpha = exp(-softplus(a)) (equal to sigmoid(-a)), beta = sigmoid(b)."""
    return np.exp(-softplus(a)), sigmoid(b)


def split_proj(proj, s: Shape):
    t = proj.shape[0]
    gh, dk, dv = s.gh, s.dk, s.dv
    o = 0
    q = proj[:, o:o + gh * dk].reshape(t, gh, dk); o += gh * dk
    k = proj[:, o:o + gh * dk].reshape(t, gh, dk); o += gh * dk
    v = proj[:, o:o + gh * dv].reshape(t, gh, dv); o += gh * dv
    a = proj[:, o:o + gh]; o += gh
    b = proj[:, o:o + gh]
    return q, k, v, a, b


def recurrence(S0, qh, kh, v, alpha, beta):
    """Sequential gated delta rule in float64.

    S0 [gh, dv, dk]; qh, kh [T, gh, dk]; v [T, gh, dv]; alpha, beta [T, gh].
    Returns (o [T, gh, dv], states [T, gh, dv, dk]) where states[t] is S_t.
    """
    S = np.array(S0, dtype=F64, copy=True)
    T = kh.shape[0]
    o = np.empty(v.shape, F64)
    states = np.empty((T,) + S.shape, F64)
    for t in range(T):
        sk = np.einsum("hij,hj->hi", S, kh[t])
        r = v[t] - alpha[t][:, None] * sk
        u = beta[t][:, None] * r
        S = alpha[t][:, None, None] * S + u[:, :, None] * kh[t][:, None, :]
        o[t] = np.einsum("hij,hj->hi", S, qh[t])
        states[t] = S
    return o, states


def recurrence_chunked(S0, qh, kh, v, alpha, beta):
    """The same gated delta rule over one chunk of T tokens in its UT / WY
    (chunked) form, in float64.  With gamma_t = alpha_1 ... alpha_t (gamma_0 = 1)
    the recurrence unrolls to

        S_t = gamma_t S0 + sum_{s<=t} (gamma_t / gamma_s) u_s k_s^T
        u_s = beta_s v_s - beta_s gamma_s S0 k_s
              - beta_s sum_{r<s} (gamma_s / gamma_r) (k_r . k_s) u_r

    i.e. (I + A) U = diag(beta) (V - diag(gamma) K S0^T) with A strictly lower
    triangular, A[s, r] = beta_s (gamma_s / gamma_r) k_s . k_r, solved by forward
    substitution (the unit lower-triangular inverse is the UT transform), and

        O   = diag(gamma) Q S0^T + (M o Q K^T) U,  M[t, s] = gamma_t / gamma_s (s <= t)
        S_T = gamma_T S0 + U^T diag(gamma_T / gamma) K.

    Decay ratios are exp(log gamma_t - log gamma_s), never a division by a small
    gamma.  Returns (o [T, gh, dv], S_T [gh, dv, dk]).
    """
    S0 = np.asarray(S0, F64)
    qh, kh, v = (np.asarray(a, F64) for a in (qh, kh, v))
    alpha, beta = np.asarray(alpha, F64), np.asarray(beta, F64)
    T, gh = kh.shape[0], kh.shape[1]
    lg = np.cumsum(np.log(alpha), axis=0)               # log gamma_t, [T, gh]
    o = np.empty(v.shape, F64)
    S_end = np.empty(S0.shape, F64)
    for h in range(gh):
        K, Q, V, b, g = kh[:, h], qh[:, h], v[:, h], beta[:, h], lg[:, h]
        S = S0[h]
        ratio = np.exp(g[:, None] - g[None, :])           # gamma_t / gamma_s
        A = np.tril(b[:, None] * ratio * (K @ K.T), -1)
        rhs = b[:, None] * (V - np.exp(g)[:, None] * (K @ S.T))
        U = np.empty_like(rhs)
        for t in range(T):                                # forward substitution
            U[t] = rhs[t] - A[t, :t] @ U[:t]
        o[:, h] = np.exp(g)[:, None] * (Q @ S.T) + (np.tril(ratio) * (Q @ K.T)) @ U
        S_end[h] = np.exp(g[-1]) * S + (U * np.exp(g[-1] - g)[:, None]).T @ K
    return o, S_end


def gdn_layer(L, x, S0, s: Shape, R):
    """One hybrid GDN decoder layer over T tokens from committed state S0.

    Returns (x_out, tape, states): tape = dict(k, v, alpha, beta) as fp32
    arrays [T, gh, ...]; states [T, gh, dv, dk] float64.
    """
    u = R(rmsnorm(x, L["in_norm"], s.eps))
    proj = R(linear(u, L["w_qkv"]))
    q, k, v, a, b = split_proj(proj, s)
    qh = l2norm(q) / np.sqrt(s.dk)
    kh = l2norm(k)
    alpha, beta = gates(a, b)
    o, states = recurrence(S0, qh, kh, v, alpha, beta)
    t = x.shape[0]
    o = R(o.reshape(t, s.gh * s.dv))
    x = R(x + R(linear(o, L["w_o"])))
    x = ffn_block(L, x, s, R)
    tape = {"k": kh.astype(np.float32), "v": v.astype(np.float32),
            "alpha": alpha.astype(np.float32), "beta": beta.astype(np.float32)}
    return x, tape, states


# ------------------------------------------------------------ pinned replay
def halving_sum(prod):
    """Sum over the last axis by the halving tree (first half + second half)."""
    w = prod.shape[-1]
    assert w & (w - 1) == 0, "halving tree needs a power-of-two length"
    while w > 1:
        w //= 2
        prod = prod[..., :w] + prod[..., w:2 * w]
    return prod[..., 0]


def replay_pinned(S, k, v, alpha, beta):
    """Apply tape tokens to state S in the pinned fp32 order (module docstring).

    S [gh, dv, dk] float32 (not modified); k [T, gh, dk], v [T, gh, dv],
    alpha/beta [T, gh], all float32.  Returns the new float32 state.
    """
    f32 = np.float32
    S = np.array(S, dtype=f32, copy=True)
    k, v = np.asarray(k, f32), np.asarray(v, f32)
    alpha, beta = np.asarray(alpha, f32), np.asarray(beta, f32)
    for t in range(k.shape[0]):
        kt = k[t][:, None, :]                        # [gh, 1, dk]
        acc = halving_sum(S * kt)                    # [gh, dv]
        p = alpha[t][:, None] * acc
        r = v[t] - p
        u = beta[t][:, None] * r
        S = (alpha[t][:, None, None] * S) + (u[:, :, None] * kt)
    return S
