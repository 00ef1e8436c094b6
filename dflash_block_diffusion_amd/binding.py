"""ctypes binding of libdflash (include/dflash.h): argument marshalling only.

Every function of the header is exposed under its own name on ``lib()``.
The shared library must have been built (``python -m
dflash_block_diffusion_amd.build`` or ``__graft_entry__.build()``); loading
fails loudly otherwise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import (POINTER, Structure, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_uint64,
                    c_size_t, c_void_p)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libdflash.so")

DFLASH_OK = 0
ERRORS = {-1: "INVALID", -2: "SHAPE", -3: "CAPACITY", -4: "DEVICE", -5: "UNSUPPORTED"}
FMT_F32, FMT_BF16, FMT_W8A16, FMT_W4A16 = 0, 1, 2, 3
LAYER_ATTN, LAYER_GDN = 0, 1
STATUS_CAPACITY, STATUS_TOKEN_RANGE, STATUS_ACT_RANGE = 1, 2, 4


class LayerDesc(Structure):
    _fields_ = [("kind", c_int), ("in_norm", c_void_p), ("post_norm", c_void_p),
                ("q_norm", c_void_p), ("k_norm", c_void_p),
                ("w_qkv", c_void_p), ("s_qkv", c_void_p), ("w_o", c_void_p), ("s_o", c_void_p),
                ("w_gu", c_void_p), ("s_gu", c_void_p), ("w_down", c_void_p), ("s_down", c_void_p)]


class ModelDesc(Structure):
    _fields_ = [("hidden", c_int), ("n_q_heads", c_int), ("n_kv_heads", c_int), ("head_dim", c_int),
                ("ffn", c_int), ("vocab", c_int), ("n_layers", c_int),
                ("gdn_heads", c_int), ("gdn_dk", c_int), ("gdn_dv", c_int),
                ("eps", c_float), ("rope_base", c_double), ("fmt", c_int),
                ("embed", c_void_p), ("w_lm", c_void_p), ("s_lm", c_void_p), ("final_norm", c_void_p),
                ("n_sel", c_int), ("sel_layers", c_int * 8), ("mask_token", c_int),
                ("w_fc", c_void_p), ("s_fc", c_void_p), ("hidden_norm", c_void_p),
                ("layers", POINTER(LayerDesc))]


class StateView(Structure):
    _fields_ = [("tokens", c_void_p), ("acc_log", c_void_p), ("acc_log_len", c_int),
                ("side", c_void_p), ("ctx_feat", c_void_p), ("gdn_state", c_void_p),
                ("gdn_tape", c_void_p), ("tape_stride", c_int), ("n_gdn", c_int), ("capacity", c_int)]


# name -> (restype, argtypes); mirrors include/dflash.h
SIGNATURES = {
    "dflash_last_error": (c_char_p, []),
    "dflash_device_count": (c_int, [POINTER(c_int)]),
    "dflash_packed_bytes": (c_int, [c_int, c_int, c_int, POINTER(c_size_t), POINTER(c_size_t)]),
    "dflash_pack_weight": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dflash_linear_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
    "dflash_linear": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                              c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dflash_linear_noalloc_scratch_bytes": (c_size_t, []),
    "dflash_linear_noalloc": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                                      c_void_p, c_void_p, c_void_p]),
    "dflash_model_create": (c_int, [POINTER(ModelDesc), POINTER(c_void_p)]),
    "dflash_model_destroy": (None, [c_void_p]),
    "dflash_drafter_bind": (c_int, [c_void_p, c_void_p]),
    "dflash_state_bytes": (c_size_t, [c_void_p, c_void_p, c_int, c_int]),
    "dflash_state_init": (c_int, [POINTER(c_void_p), c_void_p, c_void_p, c_void_p, c_size_t, c_int, c_int]),
    "dflash_state_destroy": (None, [c_void_p]),
    "dflash_prefill": (c_int, [c_void_p, c_void_p, c_int, c_void_p, c_void_p]),
    "dflash_draft_block": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p]),
    "dflash_verify_block": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dflash_accept": (c_int, [c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dflash_set_max_draft": (c_int, [c_void_p, c_int, POINTER(c_int), POINTER(c_int)]),
    "dflash_set_overlap": (c_int, [c_void_p, c_int]),
    "dflash_set_sampling": (c_int, [c_void_p, c_float, c_uint64]),
    "dflash_accept_sampled": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dflash_sample_logits": (c_int, [c_void_p, c_int, c_int, c_int, c_float, c_uint64, c_int, c_int, c_int,
                                     c_void_p, c_void_p, c_void_p]),
    "dflash_accept_logits": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_float, c_uint64, c_int,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dflash_kv_commit": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p]),
    "dflash_kv_rollback": (c_int, [c_void_p, c_int, c_void_p, c_void_p]),
    "dflash_gdn_snapshot": (c_int, [c_void_p, c_void_p]),
    "dflash_inject": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_int, c_void_p, c_void_p]),
    "dflash_state_query": (c_int, [c_void_p, POINTER(c_int32), c_void_p]),
    "dflash_state_buffers": (c_int, [c_void_p, POINTER(StateView)]),
    "dflash_prof_enable": (c_int, [c_void_p, c_int]),
    "dflash_prof_replay": (c_int, [c_void_p, c_char_p, c_int, c_void_p, POINTER(c_double), POINTER(c_int64)]),
    "dflash_read_floor": (c_int, [c_void_p, c_size_t, c_int, c_int, c_int, c_void_p, c_void_p, POINTER(c_double)]),
    "dflash_check_bf16_rounding": (c_int, [c_void_p, c_void_p, POINTER(c_uint64)]),
    "dflash_prof_read": (c_int, [c_void_p, POINTER(c_char_p), POINTER(c_int64), POINTER(c_double),
                                 POINTER(c_double), POINTER(c_double), c_int, POINTER(c_int)]),
}

_LIB = None


class DflashError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


def lib():
    """Load libdflash.so once (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m dflash_block_diffusion_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def check(rc: int):
    if rc != DFLASH_OK:
        raise DflashError(rc, lib().dflash_last_error().decode(errors="replace"))
    return rc


def ptr(t) -> int:
    """Device address of a torch tensor (None -> NULL)."""
    return None if t is None else t.data_ptr()
