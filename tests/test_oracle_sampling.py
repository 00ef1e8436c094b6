"""Pins of the oracle's temperature sampling (oracle/sampling.py).

* Philox4x32-10 against the published known-answer vectors of the generator
  (Random123 distribution, kat_vectors: philox4x32 with 10 rounds);
* the categorical draw against a brute-force running-sum loop;
* the speculative rule: the closed-form law of the first emitted token equals
  the target distribution, and a Monte-Carlo run of the oracle's own
  accept/resample step (Philox uniforms) matches it (chi-square);
* T -> 0 turns the sampled loop into greedy decoding.
"""
import numpy as np
import pytest

from dflash_block_diffusion_amd import configs as C
from dflash_block_diffusion_amd import synth
from oracle import sampling as S
from oracle.spec import OraclePair, greedy

# counter (4 words), key (2 words) -> output, philox4x32 10 rounds
KAT = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
       ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
       ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
        (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    assert S.philox4x32(ctr, key) == want


def test_uniform_range_and_streams():
    us = [S.uniform(7, n, r, s) for n in range(40) for r in range(4) for s in range(4)]
    assert all(0.0 < u < 1.0 for u in us)
    assert len(set(us)) == len(us)              # distinct counters give distinct draws here
    assert S.uniform(2 ** 40 + 5, 3, 1, 0) != S.uniform(5, 3, 1, 0)     # the key's high word counts


def test_categorical_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(300):
        w = rng.random(rng.integers(1, 40)) * (rng.random() < 0.5 and rng.random(1) or 1.0)
        w[rng.random(len(w)) < 0.3] = 0.0
        if w.sum() == 0:
            w[0] = 1.0
        u = rng.random()
        tot = sum(float(x) for x in w)
        run, pick = 0.0, None
        for v, x in enumerate(w):
            run += float(x)
            if run > u * tot:
                pick = v
                break
        if pick is None:
            pick = max(v for v, x in enumerate(w) if x > 0)
        assert S.categorical(w, u) == pick


def test_first_token_law_is_the_target():
    rng = np.random.default_rng(1)
    for _ in range(200):
        V = int(rng.integers(2, 30))
        p = rng.dirichlet(np.ones(V) * rng.uniform(0.1, 3))
        q = rng.dirichlet(np.ones(V) * rng.uniform(0.1, 3))
        assert np.allclose(S.first_token_law(p, q), p, rtol=0, atol=1e-12)
    p = np.array([0.2, 0.3, 0.5])
    assert np.allclose(S.first_token_law(p, p), p)        # identical: always accepted


def test_spec_step_samples_the_target_montecarlo():
    # one verified draft (N = 1): the first emitted token must follow p_0
    rng = np.random.default_rng(2)
    V, T, seed, trials = 6, 0.7, 11, 12000
    vlog = rng.normal(size=(2, V)) * 1.5
    dlog = rng.normal(size=(1, V)) * 1.5
    p0 = S.tempered(vlog[0], T)
    counts = np.zeros(V)
    acc = 0
    for n in range(trials):
        d = S.draft_samples(dlog, T, seed, n)
        a, nxt, _ = S.spec_accept(d, dlog, vlog, T, seed, n)
        counts[d[0] if a == 1 else nxt] += 1
        acc += a
    expected = p0 * trials
    chi2 = float(np.sum((counts - expected) ** 2 / expected))
    # 5 degrees of freedom: P(chi2 > 25.7) = 1e-4
    assert chi2 < 25.7, (counts, expected)
    # acceptance rate equals sum min(p, q)
    q = S.tempered(dlog[0], T)
    assert abs(acc / trials - np.minimum(p0, q).sum()) < 4 * np.sqrt(0.25 / trials)


def test_low_temperature_is_greedy():
    cfg = C.tiny()
    ck = synth.make_pair(cfg)
    pr = synth.prompt(cfg, 64)
    ref = greedy(cfg, ck, pr, 40, cap=256)
    op = OraclePair(cfg, ck, cap=256, temperature=1e-4, seed=3)
    assert op.generate(pr, 40) == ref


def test_sampled_loop_is_deterministic_in_the_seed():
    cfg = C.tiny()
    ck = synth.make_pair(cfg)
    pr = synth.prompt(cfg, 64)
    a = OraclePair(cfg, ck, cap=256, temperature=0.9, seed=5).generate(pr, 40)
    b = OraclePair(cfg, ck, cap=256, temperature=0.9, seed=5).generate(pr, 40)
    c = OraclePair(cfg, ck, cap=256, temperature=0.9, seed=6).generate(pr, 40)
    assert a == b
    assert a != c
