"""GPU parity of the packed skinny GEMM (dflash_linear) against the oracle's
float64 dequant-GEMM, on the same seeded weights and activations.

Tolerance: fp32 accumulation of K products in a different order than the
oracle; |err| <= 2e-6 * sum_k |x_k w_k| + 1e-7 per output (about 30x the
unit roundoff: the sums below use K <= 20480).
"""
import numpy as np
import pytest
import torch
from ctypes import c_size_t, byref

from dflash_block_diffusion_amd import binding as bn
from dflash_block_diffusion_amd import configs as C
from dflash_block_diffusion_amd import synth
from dflash_block_diffusion_amd.runtime import pack_weight, stream_handle, tile_activations
from oracle.model import top2_margin
from oracle.numerics import linear

pytestmark = pytest.mark.gpu


def x_values(rng, m, k, fmt):
    x = rng.standard_normal((m, k)).astype(np.float32)
    if fmt != C.FMT_F32:
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    return x


def x_device(x, fmt, pad=0):
    """fp32: row-major [m][k + pad]; 16-bit formats: the tiled GEMM-input layout."""
    if fmt == C.FMT_F32:
        return torch.from_numpy(np.pad(x, ((0, 0), (0, pad)))).cuda().contiguous()
    t = torch.from_numpy(x).cuda()
    t = t.to(torch.bfloat16) if fmt == C.FMT_BF16 else t.to(torch.float16)   # fp16: exact for bf16 values
    return tile_activations(t)


def run_linear(w, x, fmt, epilogue=0, want_logits=True, pad=64):
    L = bn.lib()
    m = x.shape[0]
    dst, dsts = pack_weight(w)
    ws_bytes = L.dflash_linear_workspace_bytes(fmt, w.n, w.k, m)
    assert ws_bytes > 0
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    xd = x_device(x, fmt, pad)
    out = torch.full((m, w.n), float("nan"), device="cuda") if (epilogue == 0 or want_logits) else None
    am = torch.full((m,), -1, dtype=torch.int32, device="cuda")
    bn.check(L.dflash_linear(fmt, w.n, w.k, dst.data_ptr(), None if dsts is None else dsts.data_ptr(),
                             xd.data_ptr(), w.k + pad, m, epilogue, None if out is None else out.data_ptr(),
                             am.data_ptr(), ws.data_ptr(), ws_bytes, stream_handle()))
    torch.cuda.synchronize()
    return (None if out is None else out.cpu().numpy().astype(np.float64)), am.cpu().numpy(), ws


def bound(x, w, rows=None):
    """2e-6 * sum_k |x_k w_k| + 1e-7, computed in row chunks."""
    aw = synth.Weight(w.fmt, w.n, w.k,
                      values=None if w.values is None else np.abs(w.values),
                      codes=None if w.codes is None else np.abs(w.codes),
                      scales=None if w.scales is None else np.abs(w.scales))
    return linear(np.abs(x.astype(np.float64)), aw, rows=rows) * 2e-6 + 1e-7


FMTS = [C.FMT_F32, C.FMT_BF16, C.FMT_W8A16, C.FMT_W4A16]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k,m", [(48, 256, 16), (80, 384, 17), (1040, 512, 32), (272, 4096, 33),
                                   (1024, 4096, 64), (64, 1024, 1), (6128, 4096, 32)])
def test_linear_parity_small(fmt, n, k, m):
    # spans several row tiles, ragged row blocks (N/16 not a multiple of the
    # tile group), ragged token blocks (m not a multiple of 16) and split-K
    g = synth.HostSynth(100 + fmt)
    w = g.weight(f"lin{n}x{k}", n, k, fmt)
    x = x_values(np.random.default_rng(n + k + m), m, k, fmt)
    y, _, ws = run_linear(w, x, fmt)
    ref = linear(x, w)
    assert np.all(np.isfinite(y))
    assert np.all(np.abs(y - ref) <= bound(x, w))


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_unpadded_rows(fmt):
    # fp32 inputs take a row stride; exact k works too
    g = synth.HostSynth(5)
    w = g.weight("unpad", 272, 512, fmt)
    x = x_values(np.random.default_rng(6), 20, 512, fmt)
    y, _, _ = run_linear(w, x, fmt, pad=0)
    assert np.all(np.abs(y - linear(x, w)) <= bound(x, w))


@pytest.mark.parametrize("fmt", [C.FMT_BF16, C.FMT_W4A16])
def test_linear_repeat_is_bitwise_and_counters_reset(fmt):
    # split-K partials are summed in a fixed order: two calls agree to the bit,
    # and the arrival counters are zero again after every call
    g = synth.HostSynth(7)
    w = g.weight("rep", 512, 4096, fmt)
    x = x_values(np.random.default_rng(3), 32, 4096, fmt)
    y1, _, ws1 = run_linear(w, x, fmt)
    y2, _, _ = run_linear(w, x, fmt)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_argmax_small(fmt):
    g = synth.HostSynth(9)
    w = g.weight("am", 1024, 256, fmt)
    x = x_values(np.random.default_rng(4), 16, 256, fmt)
    logits, am, _ = run_linear(w, x, fmt, epilogue=1)
    ref = linear(x, w)
    assert np.all(np.abs(logits - ref) <= bound(x, w))
    marg = top2_margin(ref)
    ok = marg >= 1e-2
    assert np.array_equal(am[ok], np.argmax(ref, axis=1)[ok])


def test_linear_argmax_ties_take_lowest_index():
    # identical rows 5 and 700 of W: equal logits, the lower index must win
    w = synth.HostSynth(2).weight("tie", 1024, 256, C.FMT_BF16)
    w.values[700] = w.values[5]
    w.values[5] *= 0
    w.values[5] += 0.5                         # make both rows the clear maximum
    w.values[700] = w.values[5]
    x = np.abs(x_values(np.random.default_rng(5), 4, 256, C.FMT_BF16))
    _, am, _ = run_linear(w, x, C.FMT_BF16, epilogue=1, want_logits=False)
    assert am.tolist() == [5, 5, 5, 5]


# ------------------------------------------------------------ full sizes
FULL = [  # (name, fmt, N, K, m): the weight-streaming GEMMs of the 8B / 27B block-32 step
    ("8b_qkv_w4", C.FMT_W4A16, 6144, 4096, 32),
    ("8b_gateup_w4", C.FMT_W4A16, 24576, 4096, 32),
    ("8b_down_w4", C.FMT_W4A16, 4096, 12288, 32),
    ("8b_drafter_qkv_w8", C.FMT_W8A16, 6144, 4096, 64),
    ("8b_fc_w8", C.FMT_W8A16, 4096, 20480, 32),
    ("27b_gateup_w4", C.FMT_W4A16, 34816, 5120, 32),
    ("4b_gateup_bf16", C.FMT_BF16, 19456, 2560, 16),
]


@pytest.mark.parametrize("name,fmt,n,k,m", FULL)
def test_linear_parity_full_size_sampled(name, fmt, n, k, m):
    g = synth.HostSynth(11)
    w = g.weight(name, n, k, fmt)
    x = x_values(np.random.default_rng(12), m, k, fmt)
    y, _, _ = run_linear(w, x, fmt)
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(13)
    for r0 in list(rng.integers(0, n // 16, 6) * 16) + [n - 16]:
        ref = linear(x, w, rows=(int(r0), int(r0) + 16))
        got = y[:, r0:r0 + 16]
        assert np.all(np.abs(got - ref) <= bound(x, w, rows=(int(r0), int(r0) + 16))), (name, r0)


@pytest.mark.parametrize("m", [8, 32])
def test_lm_head_argmax_full_size(m):
    # 8B-class lm-head: 151936 x 4096 int4, every row's argmax (near ties
    # excluded); 32 rows is the verify of a 32-token block (the launch shape
    # of the step: two 16-row token blocks on 512 work-groups)
    g = synth.HostSynth(21)
    w = g.weight("lm_full", 151936, 4096, C.FMT_W4A16)
    x = x_values(np.random.default_rng(22), m, 4096, C.FMT_W4A16)
    logits, am, _ = run_linear(w, x, C.FMT_W4A16, epilogue=1)
    ref = linear(x, w)
    assert np.max(np.abs(logits - ref) / (bound(x, w))) <= 1.0
    ok = top2_margin(ref) >= 1e-2
    assert np.array_equal(am[ok], np.argmax(ref, axis=1)[ok])


# ------------------------------------------------------------ prompt chunks
# m > 64 (multiples of 16) takes the dense W4 kernel of prefill: activations
# staged in LDS and shared by 256 weight rows, K split for the partial sums.
# Past 512 rows, N >= 16384 or K >= 8192 take the 8-token-block work-group.
@pytest.mark.parametrize("n,k,m", [(48, 256, 80), (1040, 1024, 128), (272, 4096, 1024), (4128, 512, 96),
                                   (784, 2048, 512), (256, 128, 208), (16400, 256, 784), (272, 8192, 1008),
                                   (16384, 128, 528)])
def test_linear_dense_w4_parity(n, k, m):
    # ragged row-tile groups (N/16 not a multiple of 16), ragged token groups
    # (m/16 not a multiple of 4), one K tile, splits of uneven length
    g = synth.HostSynth(300)
    w = g.weight(f"dense{n}x{k}", n, k, C.FMT_W4A16)
    x = x_values(np.random.default_rng(n + k + m), m, k, C.FMT_W4A16)
    y, _, _ = run_linear(w, x, C.FMT_W4A16)
    ref = linear(x, w)
    assert np.all(np.isfinite(y))
    assert np.all(np.abs(y - ref) <= bound(x, w))


@pytest.mark.parametrize("n,k,m", [(48, 256, 80), (1040, 1024, 128), (272, 4096, 512), (4096, 20480, 96),
                                   (272, 4096, 784), (4096, 20480, 1024)])
def test_linear_dense_w8_parity(n, k, m):
    # the int8 dense path (the drafter's context pass of a prompt chunk):
    # the row scale on the finished sum; past 512 rows the 128-row shape
    g = synth.HostSynth(303)
    w = g.weight(f"dense8_{n}x{k}", n, k, C.FMT_W8A16)
    x = x_values(np.random.default_rng(n + k + m + 1), m, k, C.FMT_W8A16)
    y, _, _ = run_linear(w, x, C.FMT_W8A16)
    if n * k > 4096 * 4096:                    # full-size drafter fc: sampled rows
        for r0 in (0, 2048, n - 16):
            ref = linear(x, w, rows=(r0, r0 + 16))
            assert np.all(np.abs(y[:, r0:r0 + 16] - ref) <= bound(x, w, rows=(r0, r0 + 16)))
        return
    ref = linear(x, w)
    assert np.all(np.isfinite(y))
    assert np.all(np.abs(y - ref) <= bound(x, w))


@pytest.mark.parametrize("n,k,m", [(48, 256, 80), (1040, 1024, 128), (272, 2560, 1024), (2560, 12800, 96),
                                   (19456, 2560, 528)])
def test_linear_dense_bf16_parity(n, k, m):
    # the bf16 dense path (4B-class targets and drafters): bf16 MFMA on the
    # stored weights; the last shapes are the 4B drafter fc (sampled rows)
    # and gate/up
    g = synth.HostSynth(304)
    w = g.weight(f"dense16_{n}x{k}", n, k, C.FMT_BF16)
    x = x_values(np.random.default_rng(n + k + m + 2), m, k, C.FMT_BF16)
    y, _, _ = run_linear(w, x, C.FMT_BF16)
    assert np.all(np.isfinite(y))
    if n * k > 4096 * 4096:
        for r0 in (0, n // 2, n - 16):
            ref = linear(x, w, rows=(r0, r0 + 16))
            assert np.all(np.abs(y[:, r0:r0 + 16] - ref) <= bound(x, w, rows=(r0, r0 + 16)))
        return
    ref = linear(x, w)
    assert np.all(np.abs(y - ref) <= bound(x, w))


def test_linear_dense_w4_repeat_is_bitwise():
    g = synth.HostSynth(301)
    w = g.weight("dense_rep", 1024, 4096, C.FMT_W4A16)
    x = x_values(np.random.default_rng(8), 256, 4096, C.FMT_W4A16)
    y1, _, _ = run_linear(w, x, C.FMT_W4A16)
    y2, _, _ = run_linear(w, x, C.FMT_W4A16)
    assert np.array_equal(y1, y2)


DENSE_FULL = [  # the target projections of an 8B / 27B prompt chunk
    ("8b_qkv_dense", 6144, 4096, 512),
    ("8b_down_dense", 4096, 12288, 512),
    ("8b_o_dense", 4096, 4096, 1024),
    ("8b_down_dense_1024", 4096, 12288, 1024),
    ("8b_gateup_dense_1024", 24576, 4096, 1024),
    ("27b_gateup_dense", 34816, 5120, 512),
]


@pytest.mark.parametrize("name,n,k,m", DENSE_FULL)
def test_linear_dense_w4_full_size_sampled(name, n, k, m):
    g = synth.HostSynth(302)
    w = g.weight(name, n, k, C.FMT_W4A16)
    x = x_values(np.random.default_rng(14), m, k, C.FMT_W4A16)
    y, _, _ = run_linear(w, x, C.FMT_W4A16)
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(15)
    for r0 in list(rng.integers(0, n // 16, 4) * 16) + [n - 16]:
        ref = linear(x, w, rows=(int(r0), int(r0) + 16))
        got = y[:, r0:r0 + 16]
        assert np.all(np.abs(got - ref) <= bound(x, w, rows=(int(r0), int(r0) + 16))), (name, r0)



def test_bf16_rounding_hardware_equals_integer_rne():
    """The packed hardware bf16 conversion the norm and attention kernels use
    rounds every fp32 bit pattern (both halves of the pair) exactly as the
    integer round-to-nearest-even the other kernels use; NaN inputs too."""
    from ctypes import c_uint64
    L = bn.lib()
    d = torch.zeros(2, dtype=torch.int64, device="cuda")
    h = (c_uint64 * 2)(7, 7)
    bn.check(L.dflash_check_bf16_rounding(d.data_ptr(), stream_handle(), h))
    assert (h[0], h[1]) == (0, 0)
