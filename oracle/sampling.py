"""Temperature sampling in the speculative loop (oracle; test infrastructure --
only tests/, smoke() and bench.py's CPU baseline use this package).

The mlx-dspark v0.0.3 release notes ("Highlights") state that sampling at a
temperature T > 0 stays lossless: the output is an exact sample from the
target at T, through the same acceptance rule as its DSpark path.  The pages
do not spell that rule out; the reading taken here is the standard
speculative-sampling rule, the one whose output distribution is exactly the
target's:

* draft: slot j draws d_j ~ q_j = softmax(z_j / T) from the drafter's logits;
* verify: p_i = softmax(y_i / T) from the target's logits of row i, which
  predicts the token after position n+i (so d_j is judged by p_{j-1});
* accept d_j (j = 1, 2, ...) while u_j < p_{j-1}(d_j) / q_j(d_j); at the
  first rejection j = a+1 the correction is drawn from the residual
  max(0, p_a - q_{a+1}) (renormalised); if all N verified drafts pass, a
  bonus token is drawn from p_N;
* emit d_1..d_a and the correction (or bonus) token.

Random numbers come from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC 2011), a counter-based generator the
GPU path implements independently from the same definition.  Counter
(n, row, stream, 0), key (seed low, seed high): n is the committed length at
the start of the step, row the slot or row index, stream 0 for draft
samples, 1 for acceptance tests, 2 for the correction/bonus sample, 3 for
the first token after the prompt (counter (P, 0, 3, 0), P the prompt length).  The
first output word x gives u = (floor(x / 2^8) + 1/2) * 2^-24, in (0, 1).

A categorical draw from weights w (not necessarily normalised) takes the
smallest index v whose running sum w_0 + ... + w_v exceeds u * sum(w) (the
inverse of the cumulative distribution, summed here in index order in
float64).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

F64 = np.float64
MASK32 = 0xFFFFFFFF
# Philox4x32 multipliers and Weyl key increments (the published constants)
PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85

STREAM_DRAFT, STREAM_ACCEPT, STREAM_CORRECT, STREAM_FIRST = 0, 1, 2, 3


def philox4x32(ctr: Sequence[int], key: Sequence[int], rounds: int = 10) -> Tuple[int, int, int, int]:
    """Philox4x32-R: each round multiplies words 0 and 2 by the two
    multipliers, splits the 64-bit products into high and low halves and
    mixes them with words 1 and 3 and the key; the key advances by the Weyl
    increments between rounds."""
    c0, c1, c2, c3 = (int(v) & MASK32 for v in ctr)
    k0, k1 = (int(v) & MASK32 for v in key)
    for _ in range(rounds):
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & MASK32, p1 & MASK32, ((p0 >> 32) ^ c3 ^ k1) & MASK32, p0 & MASK32
        k0 = (k0 + PHILOX_W0) & MASK32
        k1 = (k1 + PHILOX_W1) & MASK32
    return c0, c1, c2, c3


def uniform(seed: int, n: int, row: int, stream: int) -> float:
    """u in (0, 1) from the first Philox word of counter (n, row, stream, 0)."""
    x = philox4x32((n, row, stream, 0), (seed & MASK32, (seed >> 32) & MASK32))[0]
    return ((x >> 8) + 0.5) * 2.0 ** -24


def tempered(logits_row, T: float) -> np.ndarray:
    """softmax(logits / T) in float64."""
    z = np.asarray(logits_row, F64) / F64(T)
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def categorical(weights, u: float) -> int:
    """Smallest v with w_0 + ... + w_v > u * sum(w) (index-order sums)."""
    w = np.asarray(weights, F64)
    c = np.cumsum(w)
    target = u * c[-1]
    v = int(np.searchsorted(c, target, side="right"))
    if v >= len(w):                         # u * sum rounded up to the total
        v = int(np.flatnonzero(w > 0)[-1])
    return v


def categorical_margin(weights, u: float) -> float:
    """How far u * sum(w) lies from the nearest running-sum boundary of the
    chosen index, as a fraction of sum(w): a draw whose margin is below the
    error of the weights cannot be decided by a different evaluation."""
    w = np.asarray(weights, F64)
    c = np.cumsum(w)
    S = c[-1]
    v = categorical(w, u)
    lo = c[v - 1] if v > 0 else 0.0
    return float(min(c[v] - u * S, u * S - lo) / S)


def draft_samples(dlogits, T: float, seed: int, n: int) -> List[int]:
    """d_j for slots j = 1..len(dlogits) (dlogits row j-1 is slot j)."""
    return [categorical(tempered(dlogits[j - 1], T), uniform(seed, n, j, STREAM_DRAFT))
            for j in range(1, len(dlogits) + 1)]


def spec_accept(drafts, dlogits, vlogits, T: float, seed: int, n: int) -> Tuple[int, int, dict]:
    """Accept over the N = len(vlogits) - 1 verified drafts.

    drafts[j-1] = d_j, dlogits[j-1] = drafter logits of slot j, vlogits[i] =
    target logits of row i (i = 0..N).  Returns (a, correction token, info)."""
    N = len(vlogits) - 1
    info = {"ratio": [], "u": []}
    a = 0
    for j in range(1, N + 1):
        d = int(drafts[j - 1])
        if not 0 <= d < len(vlogits[j - 1]):
            break                               # not a token: rejected
        p = tempered(vlogits[j - 1], T)[d]
        q = tempered(dlogits[j - 1], T)[d]
        u = uniform(seed, n, j, STREAM_ACCEPT)
        info["ratio"].append(p / q)
        info["u"].append(u)
        if not u < p / q:
            break
        a = j
    u = uniform(seed, n, a, STREAM_CORRECT)
    p = tempered(vlogits[a], T)
    if a < N:
        r = np.maximum(p - tempered(dlogits[a], T), 0.0)
        w = r if np.sum(r) > 0 else p
    else:
        w = p
    info["weights"] = w
    info["u_correct"] = u
    return a, categorical(w, u), info


def first_token_law(p, q) -> np.ndarray:
    """Probability of each token being the first one emitted, when one draft
    d ~ q is judged against p (accept with min(1, p/q), else residual):
    min(p, q) + (1 - sum min(p, q)) * (p - q)+ / sum (p - q)+."""
    p = np.asarray(p, F64)
    q = np.asarray(q, F64)
    acc = np.minimum(p, q)
    r = np.maximum(p - q, 0.0)
    rej = 1.0 - np.sum(acc)
    return acc + (rej * r / np.sum(r) if np.sum(r) > 0 else 0.0)
