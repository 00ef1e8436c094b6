"""The C ABI library: it loads, exports every function include/dflash.h
declares, and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re
from ctypes import byref, c_int, c_size_t, c_void_p

import pytest

from dflash_block_diffusion_amd import binding as bn

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dflash.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_step_calls():
    names = declared_functions()
    for n in ("dflash_draft_block", "dflash_verify_block", "dflash_accept", "dflash_kv_commit",
              "dflash_kv_rollback", "dflash_prefill", "dflash_pack_weight", "dflash_linear"):
        assert n in names


def test_library_exports_every_declared_function():
    L = ctypes.CDLL(bn.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_binding_covers_every_declared_function():
    assert set(declared_functions()) == set(bn.SIGNATURES)


def test_packed_sizes():
    L = bn.lib()
    wb, sb = c_size_t(), c_size_t()
    assert L.dflash_packed_bytes(bn.FMT_W4A16, 4096, 4096, byref(wb), byref(sb)) == 0
    assert wb.value == 4096 * 4096 // 2 and sb.value == 4096 * 64 * 2
    assert L.dflash_packed_bytes(bn.FMT_W8A16, 6144, 4096, byref(wb), byref(sb)) == 0
    assert wb.value == 6144 * 4096 and sb.value == 6144 * 2
    assert L.dflash_packed_bytes(bn.FMT_BF16, 512, 256, byref(wb), byref(sb)) == 0
    assert wb.value == 512 * 256 * 2 and sb.value == 0


@pytest.mark.parametrize("fmt,n,k,code", [(9, 16, 128, -1), (bn.FMT_W4A16, 24, 128, -2),
                                          (bn.FMT_W4A16, 32, 96, -2), (bn.FMT_W8A16, 32, 32, -2)])
def test_bad_shapes_rejected(fmt, n, k, code):
    wb, sb = c_size_t(), c_size_t()
    assert bn.lib().dflash_packed_bytes(fmt, n, k, byref(wb), byref(sb)) == code
    assert bn.lib().dflash_last_error()


def test_null_arguments_rejected_without_device():
    L = bn.lib()
    assert L.dflash_accept(None, None, 16, None, None, None, None) == -1
    assert L.dflash_draft_block(None, None, None, None) == -1
    assert L.dflash_verify_block(None, None, None, None, None) == -1
    assert L.dflash_kv_commit(None, None, None, None) == -1
    assert L.dflash_prefill(None, None, 0, None, None) == -1
    assert L.dflash_model_create(None, None) == -1
    assert L.dflash_linear_workspace_bytes(bn.FMT_W4A16, 4096, 4096, 65) == 0
    fake = c_void_p(0x1000)
    assert L.dflash_accept(fake, fake, 1, fake, fake, None, None) == -2


def _fake_desc(drafter=False, n_layers=2, head_dim=64):
    layers = (bn.LayerDesc * n_layers)()
    for l in range(n_layers):
        d = layers[l]
        d.kind = bn.LAYER_ATTN
        for f in ("in_norm", "post_norm", "q_norm", "k_norm", "w_qkv", "w_o", "w_gu", "w_down"):
            setattr(d, f, 0x1000)
    m = bn.ModelDesc()
    m.hidden, m.n_q_heads, m.n_kv_heads, m.head_dim, m.ffn, m.vocab = 256, 4, 2, head_dim, 768, 1024
    m.n_layers, m.eps, m.rope_base, m.fmt = n_layers, 1e-6, 1e6, bn.FMT_F32
    m.final_norm = 0x1000
    if drafter:
        m.w_fc, m.hidden_norm, m.n_sel, m.mask_token = 0x1000, 0x1000, 2, 1023
        m.sel_layers[0], m.sel_layers[1] = 0, 1
    else:
        m.embed, m.w_lm = 0x1000, 0x1000
    m.layers = layers
    return m, layers


def test_model_create_bind_and_state_size_on_host():
    # creating models, binding and sizing a state never touch the device
    L = bn.lib()
    td, tl = _fake_desc()
    dd, dl = _fake_desc(drafter=True, n_layers=1)
    t, d = c_void_p(), c_void_p()
    assert L.dflash_model_create(byref(td), byref(t)) == 0
    assert L.dflash_model_create(byref(dd), byref(d)) == 0
    assert L.dflash_state_bytes(t, d, 256, 16) == 0          # not bound yet
    assert L.dflash_drafter_bind(t, d) == -1                 # arguments swapped
    assert L.dflash_drafter_bind(d, t) == 0
    small = L.dflash_state_bytes(t, d, 256, 16)
    big = L.dflash_state_bytes(t, d, 4096, 16)
    assert 0 < small < big
    assert L.dflash_state_bytes(t, d, 256, 24) == 0          # unsupported block
    L.dflash_model_destroy(d)
    L.dflash_model_destroy(t)


def test_model_create_rejects_bad_head_dim_and_sel():
    L = bn.lib()
    md, ml = _fake_desc(head_dim=96)
    h = c_void_p()
    assert L.dflash_model_create(byref(md), byref(h)) == -2
    td, tl = _fake_desc()
    dd, dl = _fake_desc(drafter=True, n_layers=1)
    dd.sel_layers[1] = 5                                     # past the target's 2 layers
    t, d = c_void_p(), c_void_p()
    assert L.dflash_model_create(byref(td), byref(t)) == 0
    assert L.dflash_model_create(byref(dd), byref(d)) == 0
    assert L.dflash_drafter_bind(d, t) == -2
    L.dflash_model_destroy(d)
    L.dflash_model_destroy(t)


def test_linear_rows_beyond_the_limits_are_refused():
    # prompt chunks: BF16, W8A16 and W4A16, multiples of 16 up to 1024 rows
    from dflash_block_diffusion_amd import configs as C
    L = bn.lib()
    assert L.dflash_linear_workspace_bytes(C.FMT_W4A16, 256, 512, 72) == 0      # not a multiple of 16
    assert L.dflash_linear_workspace_bytes(C.FMT_W4A16, 256, 512, 1040) == 0    # above 1024
    assert L.dflash_linear_workspace_bytes(C.FMT_F32, 256, 512, 128) == 0       # no fp32 dense path
    assert L.dflash_linear_workspace_bytes(C.FMT_BF16, 256, 480, 128) == 0      # dense needs K % 128
    assert L.dflash_linear_workspace_bytes(C.FMT_BF16, 256, 512, 128) > 0
    assert L.dflash_linear_workspace_bytes(C.FMT_W8A16, 256, 448, 128) == 0     # W8 dense needs K % 128
    assert L.dflash_linear_workspace_bytes(C.FMT_W8A16, 256, 512, 128) > 0
    assert L.dflash_linear_workspace_bytes(C.FMT_W4A16, 256, 512, 128) > 0
    assert L.dflash_linear_workspace_bytes(C.FMT_W4A16, 256, 512, 64) > 0


def test_fp16_encoding_bound_of_bf16_activations():
    """The quantised GEMMs read their bf16 activations as fp16 encodings.
    Over every finite bf16 value: magnitudes up to 65280 (the largest bf16
    value below the fp16 limit 65504) encode exactly down to 2^-17, with an
    absolute error of at most 2^-25 below that, and 65536 and up become inf
    -- the values the status bit DFLASH_STATUS_ACT_RANGE (|v| > 65504 or
    NaN) reports."""
    import numpy as np
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v)]
    h = torch.from_numpy(v).to(torch.float16).float().numpy()
    a = np.abs(v)
    ok = a <= 65504.0
    assert a[ok].max() == 65280.0 and a[~ok].min() == 65536.0
    assert np.all(np.isinf(h[~ok]))
    exact = ok & (a >= 2.0 ** -17)
    assert np.array_equal(h[exact], v[exact])
    assert np.max(np.abs(h[ok & ~exact] - v[ok & ~exact])) <= 2.0 ** -25
    assert bn.STATUS_ACT_RANGE == 4
