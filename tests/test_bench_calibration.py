"""The benchmark's injected-acceptance reference (bench.calibrate_reference)
on a host stand-in for the step: a verify whose argmax depends causally on
the block and also on where the block starts (as the chunk-form GatedDeltaNet
verify does), the injection, acceptance and commit rules of the C ABI.  After
calibration every step, replayed from the same start, accepts exactly its
schedule entry."""
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

V = 97


def _y(ctx_tokens, block, n):
    """Argmax of every verify row: a hash of the committed tokens, the block
    up to that row and the block's start (placement-dependent rounding)."""
    out = []
    h = (sum((i + 1) * t for i, t in enumerate(ctx_tokens[-8:])) + 131 * (n % 5)) % 1000003
    for j, t in enumerate(block):
        h = (h * 31 + int(t) + 7 * j) % 1000003
        out.append(h % V)
    return out


class StandInPair:
    def __init__(self, B, prompt):
        self.B = B
        self.tokens = list(prompt)          # committed tokens; tokens[n] is the anchor
        self.n = len(prompt) - 1
        self.steps = 0
        self.block = torch.zeros(B, dtype=torch.int32)
        self.block[0] = self.tokens[self.n]
        self.y = torch.zeros(B, dtype=torch.int32)
        self.acc = torch.zeros(1, dtype=torch.int32)
        self.emit = []
        self.verifies = 0

    def query(self):
        return {"n": self.n, "steps": self.steps}

    def draft(self):
        self.block[1:] = torch.arange(1, self.B, dtype=torch.int32) % V

    def inject(self, ref, sched, filler):
        k = int(sched[self.steps % sched.numel()])
        for j in range(1, self.B):
            p = self.n + j
            if j <= k and p < ref.numel():
                tok = int(ref[p])
            else:
                tok = int(filler[self.steps % sched.numel(), j])
                if j == k + 1 and p < ref.numel() and tok == int(ref[p]):
                    tok = (tok + 1) % V
            self.block[j] = tok

    def verify(self):
        self.verifies += 1
        self.y[:] = torch.as_tensor(_y(self.tokens[:self.n], self.block.tolist(), self.n), dtype=torch.int32)

    def accept(self):
        b, y = self.block.tolist(), self.y.tolist()
        a = 0
        while a + 1 < self.B and b[a + 1] == y[a]:
            a += 1
        self.acc[0] = a

    def commit(self):
        a = int(self.acc[0])
        b, y = self.block.tolist(), self.y.tolist()
        self.tokens = self.tokens[:self.n + 1] + b[1:a + 1] + [y[a]]
        self.n += a + 1
        self.steps += 1
        self.block[0] = self.tokens[self.n]


def test_calibrated_reference_realises_the_schedule_exactly():
    B, K = 16, 12
    rng = np.random.default_rng(0)
    prompt = rng.integers(0, V, 20).tolist()
    sched = torch.as_tensor(rng.integers(0, B, K), dtype=torch.int32)
    filler = torch.as_tensor(rng.integers(0, V, (K, B)), dtype=torch.int32)
    ref = torch.zeros(len(prompt) + (K + 2) * B + 1, dtype=torch.int32)   # no first guess at all
    ref[:len(prompt)] = torch.as_tensor(prompt, dtype=torch.int32)
    pair = StandInPair(B, prompt)
    fixes = bench.calibrate_reference(pair, ref, sched, filler, K, B - 1)
    assert fixes > 0
    # a verify per forced draft at most, plus the one that confirms
    assert pair.verifies <= int(sched.sum()) + 2 * K
    replay = StandInPair(B, prompt)
    for s in range(K):
        replay.draft()
        replay.inject(ref, sched, filler)
        replay.verify()
        replay.accept()
        assert int(replay.acc[0]) == int(sched[s])
        replay.commit()
    assert replay.tokens == pair.tokens


def test_calibration_respects_the_draft_cap():
    B, K, N = 16, 8, 5
    rng = np.random.default_rng(1)
    prompt = rng.integers(0, V, 10).tolist()
    sched = torch.as_tensor(rng.integers(0, B, K), dtype=torch.int32)
    filler = torch.as_tensor(rng.integers(0, V, (K, B)), dtype=torch.int32)
    ref = torch.zeros(len(prompt) + (K + 2) * B + 1, dtype=torch.int32)
    pair = StandInPair(B, prompt)

    capped_accept = pair.accept

    def accept():
        capped_accept()
        pair.acc[0] = min(int(pair.acc[0]), N)
    pair.accept = accept
    bench.calibrate_reference(pair, ref, sched, filler, K, N)
