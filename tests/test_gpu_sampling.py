"""GPU parity of temperature sampling (csrc/sample.hip) against the oracle
(oracle/sampling.py), through the C ABI.

Both sides draw from the same Philox4x32-10 uniforms, so on the same logits
they must make the same draws and the same acceptance decisions.  A draw is
compared when the oracle's u * sum lies farther than 1e-4 of the total mass
from the nearest running-sum boundary (fp32 sums on the GPU against float64
in the oracle); an acceptance test is compared when u differs from the
ratio p/q by more than 1e-4 relative; a residual draw additionally needs a
residual mass above 1e-2 (p - q is a difference of nearly equal numbers
below that).  Excluded decisions are counted.
"""
import numpy as np
import pytest
import torch

from dflash_block_diffusion_amd import binding as bn
from dflash_block_diffusion_amd import configs as C
from dflash_block_diffusion_amd import synth
from dflash_block_diffusion_amd.runtime import Pair, stream_handle
from oracle import sampling as S
from oracle.gdn import replay_pinned
from oracle.spec import OraclePair

from conftest import tiny_hybrid_config

pytestmark = pytest.mark.gpu
MARGIN = 1e-4


def peaked_logits(rng, rows, V, scale):
    x = rng.standard_normal((rows, V)) * scale
    return x.astype(np.float32)


def logsumexp(z):
    m = np.max(z)
    return m + np.log(np.sum(np.exp(z - m)))


@pytest.mark.parametrize("V", [1024, 151936])
def test_sample_logits_matches_oracle(V):
    L = bn.lib()
    rng = np.random.default_rng(1)
    rows = 8
    logits = peaked_logits(rng, rows, V, 5.0)
    logits[3] = (rng.standard_normal(V) * 0.5).astype(np.float32)       # a flat row
    logits[5, 17] += 40.0                                                  # one token carries the mass
    d = torch.from_numpy(logits).cuda()
    tok = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    lse = torch.zeros(rows, dtype=torch.float32, device="cuda")
    compared = 0
    for T in (0.6, 1.3):
        for seed, n, row0, stream in [(1, 100, 1, 0), (2 ** 40 + 3, 7, 0, 3), (99, 5000, 2, 2)]:
            bn.check(L.dflash_sample_logits(d.data_ptr(), V, rows, V, T, seed, n, row0, stream, tok.data_ptr(),
                                            lse.data_ptr(), stream_handle()))
            torch.cuda.synchronize()
            got, got_lse = tok.cpu().numpy(), lse.cpu().numpy()
            for r in range(rows):
                z = logits[r].astype(np.float64)
                w = S.tempered(z, T)
                u = S.uniform(seed, n, row0 + r, stream)
                ref_lse = logsumexp(z / T)
                assert abs(got_lse[r] - ref_lse) <= 2e-5 * max(1.0, abs(ref_lse))
                if S.categorical_margin(w, u) > MARGIN:
                    assert got[r] == S.categorical(w, u), (T, seed, r)
                    compared += 1
    assert compared >= 30


@pytest.mark.parametrize("V,N,block", [(1024, 7, 16), (151936, 15, 32)])
def test_accept_logits_matches_oracle(V, N, block):
    L = bn.lib()
    rng = np.random.default_rng(2)
    stats = {"a": 0, "tok": 0, "excluded": 0, "accepted": 0}
    lse = torch.zeros(2 * block, dtype=torch.float32, device="cuda")
    acc = torch.zeros(1, dtype=torch.int32, device="cuda")
    emit = torch.zeros(block, dtype=torch.int32, device="cuda")
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    for trial in range(16):
        T = [0.7, 1.0, 1.6][trial % 3]
        seed, n = 1000 + trial, 50 * trial + 3
        dl = peaked_logits(rng, N, V, 4.0)
        if trial % 2 == 0:      # a target close to the drafter: long acceptances
            vl = np.concatenate([dl + rng.standard_normal((N, V)).astype(np.float32) * 0.05,
                                 peaked_logits(rng, 1, V, 4.0)])
        else:
            vl = peaked_logits(rng, N + 1, V, 4.0)
        drafts = S.draft_samples(dl, T, seed, n)
        blk = np.full(block, 0, np.int32)
        blk[0] = 5
        blk[1:N + 1] = drafts
        # device copies held in names: a temporary's memory could be reused by the next one
        dblk = torch.from_numpy(blk).cuda()
        ddl = torch.from_numpy(dl).cuda()
        dvl = torch.from_numpy(vl).cuda()
        bn.check(L.dflash_accept_logits(dblk.data_ptr(), ddl.data_ptr(), dvl.data_ptr(), V, N, block, T, seed, n,
                                        lse.data_ptr(), acc.data_ptr(), emit.data_ptr(), nxt.data_ptr(),
                                        stream_handle()))
        torch.cuda.synchronize()
        a = int(acc.item())
        e = emit.cpu().numpy()
        a_o, tok_o, info = S.spec_accept(drafts, dl.astype(np.float64), vl.astype(np.float64), T, seed, n)
        decisive = all(abs(u - r) > MARGIN * max(1.0, r)
                       for u, r in zip(info["u"][:min(a_o, N - 1) + 1], info["ratio"][:min(a_o, N - 1) + 1]))
        # the emitted list is always well formed
        assert 0 <= a <= N and list(e[:a]) == list(drafts[:a]) and all(e[a + 1:] == -1)
        assert int(nxt.item()) == e[a] and 0 <= e[a] < V
        if not decisive:
            stats["excluded"] += 1
            continue
        assert a == a_o, (trial, a, a_o)
        stats["a"] += 1
        stats["accepted"] += a
        w = info["weights"]
        if S.categorical_margin(w, info["u_correct"]) > MARGIN and (a == N or np.sum(w) > 1e-2):
            assert e[a] == tok_o, (trial, e[a], tok_o)
            stats["tok"] += 1
        else:
            stats["excluded"] += 1
    print(stats)
    assert stats["a"] >= 10 and stats["tok"] >= 6 and stats["accepted"] > 0


def sampled_lockstep(cfg, P, steps, T, seed, max_draft=0, gdn_exact=False):
    """GPU and oracle in lockstep at temperature T; the oracle judges the
    GPU's drafts with its own logits and follows the GPU's accepted count."""
    B, V = cfg.block, cfg.target.vocab
    ck = synth.make_pair(cfg)
    prompt = synth.prompt(cfg, P)
    cap = P + (steps + 4) * B + 64
    pair = Pair(cfg, ck, max_ctx=cap)
    pair.set_sampling(T, seed)
    if max_draft:
        pair.set_max_draft(max_draft)
    op = OraclePair(cfg, ck, cap=cap + 2 * B, max_draft=max_draft, temperature=T, seed=seed)
    first = pair.prefill(prompt)
    op.prefill(prompt)
    stats = {"compared": 0, "excluded": 0}
    w0 = S.tempered(op.prefill_logits, T)
    u0 = S.uniform(seed, P, 0, S.STREAM_FIRST)
    if S.categorical_margin(w0, u0) > MARGIN:
        assert first == op.anchor
    op.anchor = first
    N = op.N
    tapes = []
    if gdn_exact:
        tapes.append(pair.gdn_tape().cpu().numpy()[:, :P])
    dlog = torch.empty(B - 1, V, device="cuda")
    vlog = torch.empty(B, V, device="cuda")
    for s in range(steps):
        n = op.t.n
        assert pair.query()["n"] == n
        pair.draft(dlog)
        gd = pair.block[1:B].cpu().numpy()
        _, dl_o = op.d.draft(op.anchor, n)
        assert np.max(np.abs(dlog.cpu().numpy() - dl_o)) <= 1e-4
        for j in range(1, B):
            w = S.tempered(dl_o[j - 1], T)
            u = S.uniform(seed, n, j, S.STREAM_DRAFT)
            if S.categorical_margin(w, u) > MARGIN:
                assert gd[j - 1] == S.categorical(w, u), (s, j)
                stats["compared"] += 1
            else:
                stats["excluded"] += 1
        block = pair.block[:N + 1].cpu().numpy()
        pair.verify(vlog)
        fwd = op.t.forward([int(t) for t in block])
        assert np.max(np.abs(vlog[:N + 1].cpu().numpy() - fwd["logits"])) <= 1e-4
        pair.accept()
        a = int(pair.acc.item())
        emit = pair.emit[:a + 1].cpu().numpy()
        a_o, tok_o, info = S.spec_accept(block[1:], dl_o[:N], fwd["logits"], T, seed, n)
        k = min(a_o, N - 1) + 1
        if all(abs(u - r) > MARGIN * max(1.0, r) for u, r in zip(info["u"][:k], info["ratio"][:k])):
            assert a == a_o, (s, a, a_o)
            stats["compared"] += 1
            w = info["weights"]
            if S.categorical_margin(w, info["u_correct"]) > MARGIN and (a == N or np.sum(w) > 1e-2):
                assert emit[a] == tok_o
                stats["compared"] += 1
        else:
            stats["excluded"] += 1
        assert list(emit[:a]) == [int(t) for t in block[1:a + 1]]
        pair.commit()
        if gdn_exact:
            tapes.append(pair.gdn_tape().cpu().numpy()[:, :a + 1])
        op.t.commit(fwd, a)
        op.d.ctx_append(fwd["hidden"][:a + 1], n + np.arange(a + 1))
        op.anchor = int(emit[a])
    assert pair.query()["n"] == op.t.n
    return pair, op, stats, tapes


def test_tiny_sampled_lockstep():
    _, _, stats, _ = sampled_lockstep(C.tiny(), 64, 10, 0.8, 9)
    print(stats)
    assert stats["compared"] >= 10 * 10


def test_tiny_sampled_lockstep_draft_cap():
    _, _, stats, _ = sampled_lockstep(C.tiny(), 40, 8, 1.1, 21, max_draft=4)
    assert stats["compared"] >= 8 * 8


def test_tiny_hybrid_sampled_lockstep_replays_bitexact():
    cfg = tiny_hybrid_config()
    pair, op, stats, tapes = sampled_lockstep(cfg, 16, 8, 0.9, 4, gdn_exact=True)
    S_gpu = pair.gdn_state().cpu().numpy()
    cat = np.concatenate(tapes, axis=1)
    dk, dv = cfg.target.gdn_dk, cfg.target.gdn_dv
    for l in range(S_gpu.shape[0]):
        t = cat[l]
        R = replay_pinned(np.zeros(S_gpu.shape[1:], np.float32), t[:, :, :dk], t[:, :, dk:dk + dv],
                          t[:, :, dk + dv], t[:, :, dk + dv + 1])
        assert np.array_equal(R, S_gpu[l])
    assert stats["compared"] > 0


def test_sampled_generation_is_seeded_and_well_formed():
    cfg = C.tiny()
    ck = synth.make_pair(cfg)
    pr = synth.prompt(cfg, 64)
    outs = []
    for seed in (3, 3, 4):
        pair = Pair(cfg, ck, max_ctx=256)
        pair.set_sampling(1.0, seed)
        outs.append(pair.generate(pr, 48))
        acc = pair.acc_log().cpu().numpy()[:pair.query()["steps"]]
        assert acc.max() <= cfg.block - 1
    assert outs[0] == outs[1]
    assert outs[0] != outs[2]
    assert all(0 <= t < cfg.target.vocab for t in outs[0])


@pytest.mark.parametrize("P", [700, 1025, 33])
def test_prompt_chunk_first_draw_at_low_temperature_is_the_greedy_token(P):
    # the dense prompt pass keeps the last prompt row's logits for the first
    # draw (the lm-head over that row's 16-row group): at T = 1e-4 the draw
    # is the argmax, so it equals the greedy first token of the same prompt
    from dataclasses import replace
    cfg = C.get("8b").reduced(2, 1)
    cfg = replace(cfg, target=replace(cfg.target, vocab=32768), drafter=replace(cfg.drafter, vocab=32768))
    ck = synth.make_pair(cfg)
    prompt = synth.prompt(cfg, P)
    greedy = Pair(cfg, ck, max_ctx=P + 256)
    first0 = greedy.prefill(prompt)
    del greedy
    samp = Pair(cfg, ck, max_ctx=P + 256)
    samp.set_sampling(1e-4, 5)
    first1 = samp.prefill(prompt)
    assert 0 <= first0 < cfg.target.vocab
    assert first1 == first0
