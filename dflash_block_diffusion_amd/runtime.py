"""Device-side models and the draft/verify loop, driven through libdflash.

PyTorch allocates device memory (packed weights, the state arena, I/O
buffers) and provides the stream; every step of the method runs in the HIP
kernels behind the C ABI.  Nothing here computes a step on the host.
"""
from __future__ import annotations

import ctypes
from ctypes import byref, c_char_p, c_double, c_int, c_int32, c_int64, c_size_t, c_void_p
from typing import Dict, List, Optional

import numpy as np
import torch

from . import binding as bn
from .binding import LayerDesc, ModelDesc, StateView, check, lib, ptr
from .configs import FMT_BF16, FMT_F32, FMT_W4A16, FMT_W8A16, LAYER_ATTN, PairConfig


def stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def tile_activations(x: torch.Tensor) -> torch.Tensor:
    """Row-major [m, k] -> the library's tiled GEMM-input layout (16-bit
    formats): 16-row blocks, each 32-column step one 512-element fragment in
    lane order (lane = row%16 + 16*((col%32)//8), 8 columns per lane)."""
    m, k = x.shape
    mb = (m + 15) // 16
    xp = torch.zeros(mb * 16, k, dtype=x.dtype, device=x.device)
    xp[:m] = x
    return xp.view(mb, 16, k // 32, 4, 8).permute(0, 2, 3, 1, 4).contiguous().view(-1)


def untile_activations(flat: torch.Tensor, m: int, k: int) -> torch.Tensor:
    """Inverse of tile_activations (first m rows)."""
    mb = (m + 15) // 16
    return flat[: mb * 16 * k].view(mb, k // 32, 4, 16, 8).permute(0, 3, 1, 2, 4).reshape(mb * 16, k)[:m]


def _dev(a, dtype, device):
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=dtype).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype).contiguous()


def canonical_on_device(w, device):
    """(codes/values tensor, scales tensor or None) in the encoding
    dflash_pack_weight reads: fp32, bf16 bits, or int8 codes + fp16 scales."""
    if w.fmt == FMT_F32:
        return _dev(w.values, torch.float32, device), None
    if w.fmt == FMT_BF16:
        return _dev(w.values, torch.float32, device).to(torch.bfloat16), None
    return _dev(w.codes, torch.int8, device), _dev(w.scales, torch.float16, device)


def pack_weight(w, gate_up: int = 0, device="cuda"):
    """Pack one canonical weight into the library's tile layout (on device)."""
    wb, sb = c_size_t(), c_size_t()
    check(lib().dflash_packed_bytes(w.fmt, w.n, w.k, byref(wb), byref(sb)))
    dst = torch.empty(wb.value, dtype=torch.uint8, device=device)
    dsts = torch.empty(sb.value, dtype=torch.uint8, device=device) if sb.value else None
    src, srcs = canonical_on_device(w, device)
    check(lib().dflash_pack_weight(w.fmt, w.n, w.k, gate_up, ptr(src), ptr(srcs), ptr(dst),
                                   ptr(dsts), stream_handle()))
    return dst, dsts


class DeviceStack:
    """One decoder stack (target or drafter) resident on the device."""

    def __init__(self, shape, ck: Dict, cfg: PairConfig, role: str, device="cuda"):
        self.shape, self.role, self.device = shape, role, device
        self.keep: List[torch.Tensor] = []
        nl = shape.n_layers
        self.layer_descs = (LayerDesc * nl)()
        for l, L in enumerate(ck["layers"]):
            d = self.layer_descs[l]
            d.kind = L["kind"]
            d.in_norm = self._f32(L["in_norm"])
            d.post_norm = self._f32(L["post_norm"])
            if L["kind"] == LAYER_ATTN:
                d.q_norm = self._f32(L["q_norm"])
                d.k_norm = self._f32(L["k_norm"])
            d.w_qkv, d.s_qkv = self._pack(L["w_qkv"])
            d.w_o, d.s_o = self._pack(L["w_o"])
            d.w_gu, d.s_gu = self._pack(L["w_gu"], gate_up=1)
            d.w_down, d.s_down = self._pack(L["w_down"])
        desc = ModelDesc()
        desc.hidden, desc.n_q_heads, desc.n_kv_heads = shape.hidden, shape.n_q_heads, shape.n_kv_heads
        desc.head_dim, desc.ffn, desc.vocab, desc.n_layers = shape.head_dim, shape.ffn, shape.vocab, nl
        desc.gdn_heads, desc.gdn_dk, desc.gdn_dv = shape.gdn_heads, shape.gdn_dk, shape.gdn_dv
        desc.eps, desc.rope_base, desc.fmt = shape.eps, shape.rope_base, shape.fmt
        desc.final_norm = self._f32(ck["final_norm"])
        if role == "target":
            etype = torch.float32 if shape.fmt == FMT_F32 else torch.bfloat16
            emb = _dev(ck["embed"], torch.float32, device).to(etype)
            self.keep.append(emb)
            self.embed = emb
            desc.embed = emb.data_ptr()
            desc.w_lm, desc.s_lm = self._pack(ck["w_lm"])
        else:
            desc.n_sel = len(cfg.sel_layers)
            for i, s in enumerate(cfg.sel_layers):
                desc.sel_layers[i] = s
            desc.mask_token = cfg.mask_token
            desc.w_fc, desc.s_fc = self._pack(ck["w_fc"])
            desc.hidden_norm = self._f32(ck["hidden_norm"])
        desc.layers = self.layer_descs
        self.desc = desc
        h = c_void_p()
        check(lib().dflash_model_create(byref(desc), byref(h)))
        self.h = h

    def _f32(self, a) -> int:
        t = _dev(a, torch.float32, self.device)
        self.keep.append(t)
        return t.data_ptr()

    def _pack(self, w, gate_up: int = 0):
        dst, dsts = pack_weight(w, gate_up, self.device)
        self.keep.append(dst)
        if dsts is not None:
            self.keep.append(dsts)
        return dst.data_ptr(), (dsts.data_ptr() if dsts is not None else None)

    def weight_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.keep)

    def __del__(self):
        try:
            if getattr(self, "h", None):
                lib().dflash_model_destroy(self.h)
                self.h = None
        except Exception:
            pass


class Pair:
    """Target + bound drafter + one sequence state (arena) on the device."""

    def __init__(self, cfg: PairConfig, ck: Dict, max_ctx: int, device: str = "cuda"):
        self.cfg, self.B, self.device = cfg, cfg.block, device
        self.t = DeviceStack(cfg.target, ck["target"], cfg, "target", device)
        self.d = DeviceStack(cfg.drafter, ck["drafter"], cfg, "drafter", device)
        check(lib().dflash_drafter_bind(self.d.h, self.t.h))
        nbytes = lib().dflash_state_bytes(self.t.h, self.d.h, max_ctx, self.B)
        if nbytes == 0:
            raise bn.DflashError(-1, lib().dflash_last_error().decode())
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=device)
        torch.cuda.synchronize()
        st = c_void_p()
        check(lib().dflash_state_init(byref(st), self.t.h, self.d.h, self.arena.data_ptr(), nbytes,
                                      max_ctx, self.B))
        self.st = st
        z = lambda n: torch.zeros(n, dtype=torch.int32, device=device)
        self.block, self.y, self.acc, self.emit, self.first = z(64), z(64), z(1), z(64), z(1)
        self.view = StateView()
        check(lib().dflash_state_buffers(self.st, byref(self.view)))
        self.prompt_len = 0
        self.vrows, self.accept_block = self.B, self.B
        self.temperature = 0.0

    # ------------------------------------------------------------- views
    def _arena_slice(self, addr: int, nbytes: int, dtype) -> torch.Tensor:
        off = addr - self.arena.data_ptr()
        return self.arena[off:off + nbytes].view(dtype)

    def tokens(self, count: int) -> torch.Tensor:
        return self._arena_slice(self.view.tokens, 4 * count, torch.int32)

    def acc_log(self) -> torch.Tensor:
        return self._arena_slice(self.view.acc_log, 4 * self.view.acc_log_len, torch.int32)

    def gdn_state(self) -> torch.Tensor:
        t = self.cfg.target
        n = self.view.n_gdn * t.gdn_heads * t.gdn_dv * t.gdn_dk
        return self._arena_slice(self.view.gdn_state, 4 * n, torch.float32).view(
            self.view.n_gdn, t.gdn_heads, t.gdn_dv, t.gdn_dk)

    def gdn_tape(self) -> torch.Tensor:
        t = self.cfg.target
        n = self.view.n_gdn * self.B * t.gdn_heads * self.view.tape_stride
        return self._arena_slice(self.view.gdn_tape, 4 * n, torch.float32).view(
            self.view.n_gdn, self.B, t.gdn_heads, self.view.tape_stride)

    def side(self) -> torch.Tensor:
        """Conditioning-layer outputs of the last verify [B, n_sel*H] as float32."""
        H = self.cfg.target.hidden
        w = len(self.cfg.sel_layers) * H
        if self.cfg.drafter.fmt == FMT_F32:
            return self._arena_slice(self.view.side, 4 * self.B * w, torch.float32).view(self.B, w)
        dt = torch.bfloat16 if self.cfg.drafter.fmt == FMT_BF16 else torch.float16
        flat = self._arena_slice(self.view.side, 2 * self.B * w, dt)
        return untile_activations(flat, self.B, w).float()

    # ------------------------------------------------------------- calls
    def prefill(self, prompt) -> int:
        tok = torch.as_tensor(np.asarray(prompt, dtype=np.int32), device=self.device)
        self.prompt_len = int(tok.numel())
        check(lib().dflash_prefill(self.st, ptr(tok), self.prompt_len, ptr(self.first), stream_handle()))
        self.block[0:1].copy_(self.first)
        torch.cuda.current_stream().synchronize()
        return int(self.first.item())

    def draft(self, logits: Optional[torch.Tensor] = None):
        check(lib().dflash_draft_block(self.st, ptr(self.block), ptr(logits), stream_handle()))

    def verify(self, logits: Optional[torch.Tensor] = None):
        check(lib().dflash_verify_block(self.st, ptr(self.block), ptr(self.y), ptr(logits), stream_handle()))

    def set_max_draft(self, max_draft: int) -> int:
        """Verify only the first min(max_draft, B-1) drafts (0 = the whole
        block); returns the number of rows a verify now runs."""
        v, a = c_int(), c_int()
        check(lib().dflash_set_max_draft(self.st, int(max_draft), byref(v), byref(a)))
        self.vrows, self.accept_block = v.value, a.value
        return self.vrows

    def set_overlap(self, on: bool):
        """Run the next draft's context rows on a second stream while each
        verify finishes (dflash_set_overlap)."""
        check(lib().dflash_set_overlap(self.st, 1 if on else 0))

    def set_sampling(self, temperature: float, seed: int = 0):
        """Speculative sampling at `temperature` (0 = greedy) with Philox seed `seed`."""
        check(lib().dflash_set_sampling(self.st, float(temperature), int(seed) & (2 ** 64 - 1)))
        self.temperature = float(temperature)

    def accept(self):
        if self.temperature > 0:
            check(lib().dflash_accept_sampled(self.st, ptr(self.block), ptr(self.acc), ptr(self.emit),
                                              ptr(self.block), stream_handle()))
            return
        check(lib().dflash_accept(ptr(self.block), ptr(self.y), self.accept_block, ptr(self.acc), ptr(self.emit),
                                  ptr(self.block), stream_handle()))

    def commit(self):
        check(lib().dflash_kv_commit(self.st, ptr(self.acc), ptr(self.emit), stream_handle()))

    def inject(self, ref: torch.Tensor, sched: torch.Tensor, filler: torch.Tensor):
        check(lib().dflash_inject(self.st, ptr(self.block), ptr(ref), int(ref.numel()), ptr(sched),
                                  int(sched.numel()), ptr(filler), stream_handle()))

    def step(self, inject=None):
        self.draft()
        if inject is not None:
            self.inject(*inject)
        self.verify()
        self.accept()
        self.commit()

    def rollback(self, new_len: int):
        check(lib().dflash_kv_rollback(self.st, new_len, ptr(self.block), stream_handle()))

    def snapshot(self):
        check(lib().dflash_gdn_snapshot(self.st, stream_handle()))

    def query(self) -> Dict[str, int]:
        out = (c_int32 * 4)()
        check(lib().dflash_state_query(self.st, out, stream_handle()))
        return {"n": out[0], "steps": out[1], "status": out[2], "pending": out[3]}

    def generate(self, prompt, max_new: int, inject=None) -> List[int]:
        self.prefill(prompt)
        P = self.prompt_len
        while self.query()["n"] + 1 - P < max_new:
            self.step(inject)
        return self.tokens(P + max_new)[P:].cpu().tolist()

    def prof(self, on: bool):
        check(lib().dflash_prof_enable(self.st, 1 if on else 0))

    def prof_read(self):
        cap = 64
        names = (c_char_p * cap)()
        launches = (c_int64 * cap)()
        ms = (c_double * cap)()
        by = (c_double * cap)()
        io = (c_double * cap)()
        n = c_int()
        check(lib().dflash_prof_read(self.st, names, launches, ms, by, io, cap, byref(n)))
        return [{"kernel": names[i].decode(), "launches": launches[i], "ms": ms[i], "bytes": by[i],
                 "io_bytes": io[i]} for i in range(min(n.value, cap))]

    def prof_replay(self, variant: str, reps: int = 1):
        """Kernel-only time of one GEMM variant's recorded launches, replayed
        back to back: (total ms, launches).  Clobbers the per-step buffers."""
        ms, n = c_double(), c_int64()
        check(lib().dflash_prof_replay(self.st, variant.encode(), reps, stream_handle(), byref(ms), byref(n)))
        return ms.value, n.value

    def __del__(self):
        try:
            if getattr(self, "st", None):
                lib().dflash_state_destroy(self.st)
                self.st = None
        except Exception:
            pass
