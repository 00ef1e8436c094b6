"""Pins of the oracle's number formats: bf16 rounding and int8/int4 dequant."""
import itertools

import numpy as np
import pytest
import torch

from dflash_block_diffusion_amd import configs as C
from dflash_block_diffusion_amd import synth
from oracle.numerics import dequant, linear, round_bf16


def test_round_bf16_matches_torch_conversion():
    # library routine: torch's fp32 -> bf16 conversion (round to nearest even)
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 20000),
                        np.array([0.0, -0.0, 1.0, -3.5, 65504.0, 1e-30], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(x), ref)


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even neighbour is 1
    assert round_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7


def _brute_dequant(w):
    n, k = w.codes.shape
    out = [[0.0] * k for _ in range(n)]
    for i in range(n):
        for j in range(k):
            s = w.scales[i] if w.scales.ndim == 1 else w.scales[i, j // 64]
            out[i][j] = float(s) * int(w.codes[i, j])
    return np.array(out)


@pytest.mark.parametrize("fmt", [C.FMT_W8A16, C.FMT_W4A16])
def test_dequant_bitwise_against_brute_force(fmt):
    g = synth.HostSynth(7)
    w = g.weight("dq", 5, 128, fmt)
    assert np.array_equal(dequant(w), _brute_dequant(w))


def test_quantiser_worked_example(hand_cases):
    ex = hand_cases["quant_example"]
    w = np.zeros((1, 64), np.float32)
    w[0, :4] = ex["w"]
    w4 = synth.quantize_host(w, C.FMT_W4A16)
    assert float(w4.scales[0, 0]) == pytest.approx(ex["int4"]["scale"], rel=1e-7)
    assert w4.codes[0, :4].tolist() == ex["int4"]["codes"]
    w8 = synth.quantize_host(w, C.FMT_W8A16)
    assert float(w8.scales[0]) == pytest.approx(ex["int8"]["scale"], rel=1e-7)
    assert w8.codes[0, :4].tolist() == ex["int8"]["codes"]


def test_quantiser_ranges_and_error():
    g = synth.HostSynth(3)
    raw = g.normal("qr", (16, 256), 0.02)
    for fmt, lim in ((C.FMT_W8A16, 127), (C.FMT_W4A16, 8)):
        w = synth.quantize_host(raw, fmt)
        assert w.codes.min() >= -lim and w.codes.max() <= (127 if lim == 127 else 7)
        deq = dequant(w)
        s = (w.scales.astype(np.float64)[:, None] if w.scales.ndim == 1
             else np.repeat(w.scales.astype(np.float64), 64, axis=1))
        assert np.all(np.abs(deq - raw) <= s * 0.5 + 1e-12 + np.abs(raw) * 1e-3)


def test_zero_group_gives_zero_codes():
    w = np.zeros((2, 128), np.float32)
    w[1, 64:] = 0.5
    q = synth.quantize_host(w, C.FMT_W4A16)
    assert np.all(q.codes[0] == 0) and np.all(q.codes[1, :64] == 0)
    assert np.all(q.codes[1, 64:] == 7)


def test_quantised_linear_is_fp64_product():
    g = synth.HostSynth(11)
    w = g.weight("ql", 48, 192, C.FMT_W4A16)
    x = g.normal("qx", (3, 192), 1.0).astype(np.float64)
    y = linear(x, w, chunk_rows=16)
    deq = _brute_dequant(w)
    brute = np.array([[sum(x[t, j] * deq[i, j] for j in range(192)) for i in range(48)]
                      for t in range(3)])
    assert np.allclose(y, brute, rtol=1e-12, atol=1e-13)
    # a row range equals the same rows of the full product
    assert np.array_equal(linear(x, w, rows=(16, 40), chunk_rows=8)[:, 3], y[:, 19])
