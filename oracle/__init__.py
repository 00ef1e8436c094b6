"""CPU oracle of the DFlash draft+verify step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything here.  The HIP
path never calls it, and this package imports nothing from the HIP path
(``dflash_block_diffusion_amd``): the only thing both sides share is the
seeded checkpoint/prompt generator, which holds none of the step's
arithmetic.

It is deliberately plain and slow: NumPy, float64 arithmetic between the
points where the method materialises a bf16 tensor, every step written in
the order the pages describe it:

* the step: drafter proposes a whole block in one parallel pass, the target
  verifies it in one forward, the longest prefix of drafts that equals the
  target's argmax is accepted and the target's next token is appended
  (mirror-sd README, "How It Works"; dflash-mlx note, "What It Does" and
  "How it works"; agentlens dflash-mlx summary, "How it works");
* drafter conditioned on target intermediate hidden states, reusing the
  target's embedding and lm-head (dflash-mlx note, "Technical challenges";
  mlx-dspark v0.0.3, "Highlights");
* per-head Q/K RMSNorm and neox split-half RoPE (mirror-sd README, "The
  Story");
* int8 per-channel / int4 group-64 weights (mirror-sd README, "The Story",
  "Results");
* GatedDeltaNet layers and their tape-replay rollback (dflash-mlx note,
  "Technical challenges"; agentlens summary, "How it works").

Pinned against the pages and the mathematics by ``tests/test_oracle_*.py``.

The way the pieces are assembled -- decoder-layer wiring, the causal verify
and its hidden side-write, the drafter's view of the whole context and the
whole block, context keys normed and rotated at their own positions, the
GatedDeltaNet gates and query scale -- is pinned by constructed-weight closed
forms and exact invariants (tests/test_oracle_assembly.py).  The choices that
remain readings (mask token id, which slot predicts which position, that the
projected hidden states enter each drafter layer as extra keys/values) are
pinned to their stated definition, not to a worked example on the pages,
which give none.
"""
