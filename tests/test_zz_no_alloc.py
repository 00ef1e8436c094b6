"""The allocation-free linear (dflash_linear_noalloc): the same GEMM as
dflash_linear with its workspace in the library's static per-device scratch
array.  Its outputs must equal dflash_linear's bit for bit (same kernels,
same split plan) on consecutive calls -- the second with a smaller input, so
that it runs over what the first left in the shared array -- and a call
needing more workspace than the array holds is refused before any launch."""
import numpy as np
import pytest
import torch

from dflash_block_diffusion_amd import binding as bn
from dflash_block_diffusion_amd import configs as C
from dflash_block_diffusion_amd import synth
from dflash_block_diffusion_amd.runtime import pack_weight, stream_handle, tile_activations

pytestmark = pytest.mark.gpu


def _x(fmt, m, k, seed):
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal((m, k)).astype(np.float32))
    if fmt == C.FMT_F32:
        return x.cuda().contiguous()
    x = x.to(torch.bfloat16)
    return tile_activations((x if fmt == C.FMT_BF16 else x.float().to(torch.float16)).cuda())


def _both(w, packed, m, epilogue, seed):
    """(dflash_linear result, dflash_linear_noalloc result) for one input."""
    L = bn.lib()
    dst, dsts = packed
    x = _x(w.fmt, m, w.k, seed)
    ws_bytes = L.dflash_linear_workspace_bytes(w.fmt, w.n, w.k, m)
    assert 0 < ws_bytes <= L.dflash_linear_noalloc_scratch_bytes()
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    outs = []
    for noalloc in (False, True):
        out = torch.full((m, w.n), float("nan"), device="cuda")
        am = torch.full((m,), -1, dtype=torch.int32, device="cuda")
        args = (w.fmt, w.n, w.k, dst.data_ptr(), None if dsts is None else dsts.data_ptr(), x.data_ptr(),
                w.k, m, epilogue, out.data_ptr(), am.data_ptr())
        if noalloc:
            bn.check(L.dflash_linear_noalloc(*args, stream_handle()))
        else:
            bn.check(L.dflash_linear(*args, ws.data_ptr(), ws_bytes, stream_handle()))
        outs.append((out, am))
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("fmt", [C.FMT_W4A16, C.FMT_W8A16, C.FMT_BF16, C.FMT_F32])
@pytest.mark.parametrize("epilogue", [0, 1])
def test_noalloc_linear_equals_linear_on_consecutive_calls(fmt, epilogue):
    g = synth.HostSynth(31)
    big = g.weight("noalloc_big", 6144, 4096, fmt)
    small = g.weight("noalloc_small", 1024, 1024, fmt)
    for w, m, seed in ((big, 32, 1), (small, 7, 2)):        # the second call is smaller
        (ref, ref_am), (got, got_am) = _both(w, pack_weight(w), m, epilogue, seed)
        assert torch.isfinite(ref).all()
        assert torch.equal(ref, got)
        if epilogue == 1:
            assert torch.equal(ref_am, got_am) and int(ref_am.min()) >= 0


def test_noalloc_linear_prompt_chunk_equals_linear():
    # a dense prompt-chunk shape (m > 64) through the same static scratch
    w = synth.HostSynth(33).weight("noalloc_dense", 2048, 1024, C.FMT_W4A16)
    (ref, _), (got, _) = _both(w, pack_weight(w), 256, 0, 3)
    assert torch.isfinite(ref).all() and torch.equal(ref, got)


def test_noalloc_linear_refuses_oversized_workspace():
    L = bn.lib()
    cap = L.dflash_linear_noalloc_scratch_bytes()
    assert cap == 64 << 20
    n, k, m = 24576, 4096, 1024                      # fp32 partial sums alone exceed 64 MiB
    assert L.dflash_linear_workspace_bytes(C.FMT_W4A16, n, k, m) > cap
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = torch.zeros(16, device="cuda")
    rc = L.dflash_linear_noalloc(C.FMT_W4A16, n, k, dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(), k, m, 0,
                                 out.data_ptr(), None, stream_handle())
    assert rc == -3 and b"static scratch" in L.dflash_last_error()
