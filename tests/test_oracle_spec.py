"""Pins of the oracle's loop: acceptance rule, verify == sequential decode,
losslessness (speculative greedy == plain greedy), commit bookkeeping."""
import itertools
from dataclasses import replace

import numpy as np
import pytest

from dflash_block_diffusion_amd import configs as C
from dflash_block_diffusion_amd import synth
from oracle.spec import OraclePair, OracleTarget, accept_length, greedy, inject_drafts

from conftest import tiny_hybrid_config


@pytest.mark.parametrize("B", [2, 5, 8])
def test_accept_exhaustive(B):
    # every pattern of draft/target agreement: a is the index of the first mismatch
    for pattern in itertools.product([0, 1], repeat=B - 1):
        y = np.arange(B) + 100
        d = np.array([y[j] if pattern[j] else -1 for j in range(B - 1)])
        a = accept_length(d, y)
        first_miss = next((j for j, p in enumerate(pattern) if not p), B - 1)
        assert a == first_miss
        assert 1 <= a + 1 <= B                     # tokens emitted per step


@pytest.fixture(scope="module")
def tiny():
    cfg = C.tiny()
    return cfg, synth.make_pair(cfg), synth.prompt(cfg, 64)


def test_verify_equals_sequential_decode(tiny):
    cfg, ck, pr = tiny
    a = OracleTarget(cfg.target, ck["target"], cfg.sel_layers, 256)
    b = OracleTarget(cfg.target, ck["target"], cfg.sel_layers, 256)
    f = a.forward(pr[:48]); a.commit(f, 47)
    f = b.forward(pr[:48]); b.commit(f, 47)
    block = pr[48:64]
    batched = a.forward(block)
    seq = []
    for t in block:
        fw = b.forward([t]); b.commit(fw, 0)
        seq.append(fw["logits"][0])
    assert np.allclose(batched["logits"], np.array(seq), rtol=1e-10, atol=1e-12)


def test_forward_depends_on_relative_positions_only(tiny):
    # RoPE enters attention only through position differences, so running the
    # same tokens at positions 37.. instead of 0.. (empty cache) changes nothing
    cfg, ck, pr = tiny
    a = OracleTarget(cfg.target, ck["target"], cfg.sel_layers, 256)
    b = OracleTarget(cfg.target, ck["target"], cfg.sel_layers, 256)
    b.cos, b.sin = a.cos[37:], a.sin[37:]
    fa, fb = a.forward(pr[:16]), b.forward(pr[:16])
    # the cos/sin table is fp32, so the invariance holds to fp32 table precision
    assert np.allclose(fa["logits"], fb["logits"], rtol=1e-5, atol=1e-6)


def test_speculative_equals_greedy_tiny(tiny):
    cfg, ck, pr = tiny
    ref = greedy(cfg, ck, pr, cfg.new_tokens, cap=256)
    op = OraclePair(cfg, ck, cap=256)
    out = op.generate(pr, cfg.new_tokens)
    assert out == ref


@pytest.mark.parametrize("forced", [[0, 15, 7, 3], [15, 15, 15], None])
def test_speculative_with_injection_is_lossless_and_accepts_k(tiny, forced):
    cfg, ck, pr = tiny
    ref_tail = greedy(cfg, ck, pr, 200, cap=512)
    ref = list(pr) + ref_tail                        # token at every absolute position
    ks = synth.accept_schedule(cfg, 64, forced=forced)
    fill = synth.filler_tokens(cfg, 64)
    op = OraclePair(cfg, ck, cap=512)
    op.prefill(pr)
    out = [op.anchor]
    s = 0
    while len(out) < 128:
        k = int(ks[s])
        rec = op.step(lambda d, n: inject_drafts(d, n, k, ref, fill[s], cfg.target.vocab))
        assert rec["a"] == k
        out += rec["emitted"]
        s += 1
    assert out[:128] == ref_tail[:128]


def test_commit_bookkeeping(tiny):
    cfg, ck, pr = tiny
    op = OraclePair(cfg, ck, cap=256)
    op.prefill(pr)
    K0 = {l: v[:64].copy() for l, v in op.t.K.items()}
    n0 = op.t.n
    rec = op.step()
    a = rec["a"]
    assert op.t.n == n0 + a + 1
    for l, (k, v) in rec["fwd"]["blk"].items():
        assert np.array_equal(op.t.K[l][:64], K0[l])                  # committed rows kept
        assert np.array_equal(op.t.K[l][n0:n0 + a + 1], k[:a + 1])     # kept block rows
        assert not np.any(op.t.K[l][n0 + a + 1:n0 + cfg.block])        # dropped rows absent
    assert op.d.n_ctx == op.t.n
    assert op.seq[-(a + 1):] == rec["emitted"]


def test_rollback_replays_same_tokens(tiny):
    cfg, ck, pr = tiny
    a = OraclePair(cfg, ck, cap=256)
    out1 = a.generate(pr, 40)
    b = OraclePair(cfg, ck, cap=256)
    out2 = b.generate(pr, 40)
    assert out1 == out2


def test_speculative_equals_greedy_tiny_hybrid():
    cfg = tiny_hybrid_config()
    ck = synth.make_pair(cfg)
    pr = synth.prompt(cfg, 40)
    ref = greedy(cfg, ck, pr, 48, cap=256)
    ref_full = list(pr) + greedy(cfg, ck, pr, 160, cap=512)
    ks = synth.accept_schedule(cfg, 64, forced=[0, 15, 5])
    fill = synth.filler_tokens(cfg, 64)
    op = OraclePair(cfg, ck, cap=512)
    op.prefill(pr)
    out = [op.anchor]
    s = 0
    while len(out) < 48:
        k = int(ks[s])
        rec = op.step(lambda d, n: inject_drafts(d, n, k, ref_full, fill[s], cfg.target.vocab))
        assert rec["a"] == k
        out += rec["emitted"]
        s += 1
    assert out[:48] == ref


def test_bf16_stack_rounds_activations():
    cfg = C.qwen4b().reduced(1, 1)
    cfg = replace(cfg, target=replace(cfg.target, hidden=256, n_q_heads=4, n_kv_heads=2,
                                      head_dim=64, ffn=512, vocab=512),
                  drafter=replace(cfg.drafter, hidden=256, n_q_heads=4, n_kv_heads=2,
                                  head_dim=64, ffn=512, vocab=512), sel_layers=(0,))
    ck = synth.make_pair(cfg)
    t = OracleTarget(cfg.target, ck["target"], cfg.sel_layers, 64)
    f = t.forward(list(range(8)))
    from oracle.numerics import round_bf16
    assert np.array_equal(round_bf16(f["hidden"]), f["hidden"])
    assert np.array_equal(round_bf16(t.K[0]), t.K[0])


@pytest.mark.parametrize("max_draft", [1, 2, 6, 0])
def test_draft_cap_is_lossless_and_bounds_acceptance(tiny, max_draft):
    # a cap on the drafts verified per step changes how many tokens a step
    # emits, never which tokens: the output stays plain greedy decoding
    cfg, ck, pr = tiny
    ref = greedy(cfg, ck, pr, cfg.new_tokens, cap=256)
    op = OraclePair(cfg, ck, cap=256, max_draft=max_draft)
    out = op.generate(pr, cfg.new_tokens)
    assert out == ref
    N = cfg.block - 1 if max_draft == 0 else max_draft
    for rec in op.steps:
        assert len(rec["block"]) == N + 1            # anchor + verified drafts
        assert rec["logits"].shape[0] == N + 1
        assert 0 <= rec["a"] <= N
        assert len(rec["emitted"]) == rec["a"] + 1


@pytest.mark.parametrize("max_draft", [3, 9])
def test_draft_cap_realises_min_of_forced_and_cap(tiny, max_draft):
    cfg, ck, pr = tiny
    ref_tail = greedy(cfg, ck, pr, 200, cap=512)
    ref = list(pr) + ref_tail
    ks = synth.accept_schedule(cfg, 64, forced=[0, 15, 2, 7, 12])
    fill = synth.filler_tokens(cfg, 64)
    op = OraclePair(cfg, ck, cap=512, max_draft=max_draft)
    op.prefill(pr)
    out = [op.anchor]
    s = 0
    while len(out) < 96:
        k = int(ks[s])
        rec = op.step(lambda d, n: inject_drafts(d, n, k, ref, fill[s], cfg.target.vocab))
        assert rec["a"] == min(k, max_draft)
        out += rec["emitted"]
        s += 1
    assert out[:96] == ref_tail[:96]


def test_draft_cap_lossless_tiny_hybrid():
    cfg = tiny_hybrid_config()
    ck = synth.make_pair(cfg)
    pr = synth.prompt(cfg, 40)
    ref = greedy(cfg, ck, pr, 40, cap=256)
    op = OraclePair(cfg, ck, cap=256, max_draft=4)
    assert op.generate(pr, 40) == ref
    assert all(rec["a"] <= 4 for rec in op.steps)
