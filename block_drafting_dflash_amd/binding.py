"""Thin Python binding of libdflash.so (include/dflash.h): argument marshalling only.

Every step of the round runs in the library's HIP kernels; PyTorch only provides device
memory (weights, ring, workspace, inputs and outputs) and the stream. If the library is
not built this module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash.so")

DFLASH_F32, DFLASH_BF16, DFLASH_Q4G64 = 0, 1, 2
_DTYPE = {"f32": DFLASH_F32, "bf16": DFLASH_BF16, "q4": DFLASH_Q4G64}

EXPORTS = ("dflash_query_sizes", "dflash_create", "dflash_destroy", "dflash_cache_append", "dflash_cache_trim",
           "dflash_draft_block", "dflash_lm_head_argmax", "dflash_lm_head_argmax_noalloc", "dflash_time_next_argmax",
           "dflash_time_next_chain",
           "dflash_verify_greedy", "dflash_hbm_read_probe", "dflash_width_ctl_create", "dflash_width_ctl_width",
           "dflash_width_ctl_record", "dflash_width_ctl_state", "dflash_width_ctl_destroy",
           "dflash_target_query_sizes", "dflash_target_create", "dflash_target_destroy", "dflash_target_forward",
           "dflash_target_trim", "dflash_target_state", "dflash_target_cache_read", "dflash_target_last_error",
           "dflash_cache_state",
           "dflash_cache_read", "dflash_last_error", "dflash_status_string",
           "dflash_batch_query_sizes", "dflash_batch_create", "dflash_batch_destroy", "dflash_batch_append",
           "dflash_batch_trim", "dflash_batch_draft", "dflash_batch_lm_head_argmax", "dflash_batch_verify_greedy",
           "dflash_batch_state", "dflash_batch_cache_read", "dflash_batch_last_error")


class dflash_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "layers", "q_heads", "kv_heads", "head_dim", "intermediate", "vocab",
        "target_streams", "target_width", "window", "max_block", "mask_token_id", "ring_phase")] + [
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("weight_dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
        ("variant", ctypes.c_int32), ("rope_traditional", ctypes.c_int32), ("markov_rank", ctypes.c_int32)]


VARIANT = {"dflash": 0, "dspark": 1}


class dflash_linear(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class dflash_layer(ctypes.Structure):
    _fields_ = [(n, dflash_linear) for n in ("q", "k", "v", "o", "gate", "up", "down")] + [
        (n, ctypes.c_void_p) for n in ("in_norm", "post_norm", "q_norm", "k_norm")]


class dflash_target_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "layers", "q_heads", "kv_heads", "head_dim", "intermediate", "vocab",
        "window", "max_context", "max_block")] + [
        ("full_mask", ctypes.c_uint64), ("n_capture", ctypes.c_int32), ("capture_layers", ctypes.c_int32 * 8),
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("weight_dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32)]


class dflash_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", dflash_linear), ("fc", dflash_linear),
                ("enc_norm", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(dflash_layer)),
                ("markov_w1", ctypes.c_void_p), ("markov_w2", ctypes.c_void_p)]


class dflash_target_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", dflash_linear), ("final_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(dflash_layer))]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "dflash_query_sizes": (i32, [P(dflash_config), P(sz), P(sz), P(sz)]),
        "dflash_create": (i32, [P(dflash_config), P(dflash_weights), vp, sz, vp, sz, vp, sz, vp, P(vp)]),
        "dflash_destroy": (None, [vp]),
        "dflash_cache_append": (i32, [vp, vp, i32, i32, vp]),
        "dflash_cache_trim": (i32, [vp, i32]),
        "dflash_draft_block": (i32, [vp, i32, i32, vp, vp, vp]),
        "dflash_lm_head_argmax": (i32, [vp, vp, i32, vp, vp]),
        "dflash_lm_head_argmax_noalloc": (i32, [vp, vp, i32, vp, vp]),
        "dflash_time_next_argmax": (i32, [vp, vp, vp]),
        "dflash_time_next_chain": (i32, [vp, vp, vp]),
        "dflash_hbm_read_probe": (i32, [vp, sz, vp, i32, vp]),
        "dflash_width_ctl_create": (i32, [i32, i32, i32, i32, P(vp)]),
        "dflash_width_ctl_width": (i32, [vp]),
        "dflash_width_ctl_record": (i32, [vp, i32, i32, ctypes.c_double]),
        "dflash_width_ctl_state": (i32, [vp, P(i32), P(i32), P(i32), P(ctypes.c_double), P(ctypes.c_double),
                                         P(i64), P(i64)]),
        "dflash_width_ctl_destroy": (None, [vp]),
        "dflash_target_query_sizes": (i32, [P(dflash_target_config), P(sz), P(sz), P(sz)]),
        "dflash_target_create": (i32, [P(dflash_target_config), P(dflash_target_weights), vp, sz, vp, sz, vp, sz, vp,
                                       P(vp)]),
        "dflash_target_destroy": (None, [vp]),
        "dflash_target_forward": (i32, [vp, i32, vp, i32, vp, vp, vp]),
        "dflash_target_trim": (i32, [vp, i32]),
        "dflash_target_state": (i32, [vp, P(i64), P(i32), P(i32)]),
        "dflash_target_cache_read": (i32, [vp, i32, vp, vp, P(i32), vp]),
        "dflash_target_last_error": (ctypes.c_char_p, [vp]),
        "dflash_verify_greedy": (i32, [vp, vp, vp, i32, vp, vp]),
        "dflash_cache_state": (i32, [vp, P(i64), P(i32), P(i32), P(i32)]),
        "dflash_cache_read": (i32, [vp, i32, vp, vp, P(i32), vp]),
        "dflash_last_error": (ctypes.c_char_p, [vp]),
        "dflash_status_string": (ctypes.c_char_p, [i32]),
        "dflash_batch_query_sizes": (i32, [P(dflash_config), i32, P(sz), P(sz), P(sz)]),
        "dflash_batch_create": (i32, [P(dflash_config), i32, P(dflash_weights), vp, sz, vp, sz, vp, sz, vp, P(vp)]),
        "dflash_batch_destroy": (None, [vp]),
        "dflash_batch_append": (i32, [vp, vp, P(i32), i32, vp]),
        "dflash_batch_trim": (i32, [vp, P(i32)]),
        "dflash_batch_draft": (i32, [vp, P(i32), i32, vp, vp, vp]),
        "dflash_batch_lm_head_argmax": (i32, [vp, vp, i32, vp, vp]),
        "dflash_batch_verify_greedy": (i32, [vp, vp, vp, i32, vp, vp]),
        "dflash_batch_state": (i32, [vp, i32, P(i64), P(i32)]),
        "dflash_batch_cache_read": (i32, [vp, i32, i32, vp, vp, P(i32), vp]),
        "dflash_batch_last_error": (ctypes.c_char_p, [vp]),
    }
    for name, (res, args) in sig.items():  # every symbol include/dflash.h declares
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


class DFlashError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


def _check(status: int, ctx) -> None:
    if status != 0:
        L = lib()
        msg = L.dflash_last_error(ctx).decode() or L.dflash_status_string(status).decode()
        raise DFlashError(status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_config(shape, max_block: int, phase: int = 0) -> dflash_config:
    return dflash_config(
        hidden=shape.hidden, layers=shape.layers, q_heads=shape.q_heads, kv_heads=shape.kv_heads,
        head_dim=shape.head_dim, intermediate=shape.intermediate, vocab=shape.vocab,
        target_streams=shape.target_streams, target_width=shape.target_width, window=shape.window,
        max_block=max_block, mask_token_id=shape.mask_id, ring_phase=phase, rms_eps=shape.rms_eps,
        rope_theta=shape.rope_theta, weight_dtype=_DTYPE[shape.weight_dtype], act_dtype=_DTYPE[shape.act_dtype],
        variant=VARIANT[getattr(shape, "variant", "dflash")],
        rope_traditional=int(getattr(shape, "rope_style", "neox") == "traditional"),
        markov_rank=getattr(shape, "markov_rank", 0))


def act_torch_dtype(shape) -> torch.dtype:
    return torch.float32 if shape.act_dtype == "f32" else torch.bfloat16


def to_device(shape, weights: Dict[str, object], device="cuda") -> Dict[str, object]:
    """Storage-form numpy weights -> device tensors (bf16-exact values become bfloat16)."""
    dt = act_torch_dtype(shape)
    out: Dict[str, object] = {}
    for name, w in weights.items():
        if hasattr(w, "packed"):
            out[name] = (torch.from_numpy(w.packed.view(np.int32)).to(device),
                         torch.from_numpy(w.scales).to(torch.bfloat16).to(device),
                         torch.from_numpy(w.biases).to(torch.bfloat16).to(device))
        else:
            out[name] = torch.from_numpy(np.ascontiguousarray(w)).to(dt).to(device)
    return out


def query_sizes(cfg: dflash_config) -> Tuple[int, int, int]:
    rb, wb, pb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().dflash_query_sizes(ctypes.byref(cfg), ctypes.byref(rb), ctypes.byref(wb), ctypes.byref(pb)), None)
    return rb.value, wb.value, pb.value


class Drafter:
    """One dflash_ctx: the drafter bound to device weights, its ring and its workspace."""

    def __init__(self, shape, dev_weights: Dict[str, object], max_block: int, phase: int = 0,
                 device="cuda", stream=None):
        L = lib()
        self.shape = shape
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.cfg = make_config(shape, max_block, phase)
        self._w = dev_weights  # keeps every weight alive while the context is

        def lin(name):
            t = dev_weights[name]
            if isinstance(t, tuple):
                return dflash_linear(_ptr(t[0]), _ptr(t[1]), _ptr(t[2]))
            return dflash_linear(_ptr(t), None, None)

        layers = (dflash_layer * shape.layers)()
        for l in range(shape.layers):
            p = f"layers.{l}."
            layers[l] = dflash_layer(*[lin(p + n) for n in ("q", "k", "v", "o", "gate", "up", "down")],
                                     *[_ptr(dev_weights[p + n]) for n in ("in_norm", "post_norm", "q_norm", "k_norm")])
        self._layers = layers
        self.weights = dflash_weights(_ptr(dev_weights["embed"]), lin("lm_head"), lin("fc"),
                                      _ptr(dev_weights["enc_norm"]), _ptr(dev_weights["final_norm"]),
                                      ctypes.cast(layers, ctypes.POINTER(dflash_layer)),
                                      _ptr(dev_weights.get("markov_w1")), _ptr(dev_weights.get("markov_w2")))
        self.dspark = getattr(shape, "variant", "dflash") == "dspark"
        ring_b, ws_b, pk_b = query_sizes(self.cfg)
        self.ring = torch.empty(max(ring_b, 256), dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(max(ws_b, 256), dtype=torch.uint8, device=self.device)
        self.packed = torch.empty(max(pk_b, 256), dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        _check(L.dflash_create(ctypes.byref(self.cfg), ctypes.byref(self.weights), _ptr(self.ring), ring_b,
                               _ptr(self.workspace), ws_b, _ptr(self.packed), pk_b, _stream(stream),
                               ctypes.byref(h)), None)
        self.ctx = h
        self.act_dtype = act_torch_dtype(shape)

    def __del__(self):
        ctx = getattr(self, "ctx", None)
        if ctx and _lib is not None:
            _lib.dflash_destroy(ctx)
            self.ctx = None

    # ---- the C-ABI calls, same names --------------------------------------------------
    def cache_append(self, resid: torch.Tensor, commit: bool = False, stream=None) -> None:
        self._dev(resid, self.act_dtype)
        if resid.dim() != 2 or resid.shape[1] != self.shape.fc_in:
            raise ValueError("residual rows must be [n, target_streams*target_width]")
        _check(lib().dflash_cache_append(self.ctx, _ptr(resid), resid.shape[0], int(bool(commit)), _stream(stream)),
               self.ctx)

    def cache_trim(self, m: int) -> None:
        _check(lib().dflash_cache_trim(self.ctx, int(m)), self.ctx)

    def draft_block(self, anchor: int, block: int, tokens: Optional[torch.Tensor] = None,
                    hidden: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        if tokens is None:
            tokens = torch.empty(block, dtype=torch.int32, device=self.device)
        self._dev(tokens, torch.int32)
        if hidden is not None:
            self._dev(hidden, torch.float32)
            rows = block if self.dspark else block + 1  # DSpark blocks have gamma rows
            if hidden.numel() < rows * self.shape.hidden:
                raise ValueError("hidden output too small")
        if tokens.numel() < block:
            raise ValueError("token output too small")
        _check(lib().dflash_draft_block(self.ctx, int(anchor), int(block), _ptr(tokens), _ptr(hidden),
                                        _stream(stream)), self.ctx)
        return tokens

    def lm_head_argmax(self, rows: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        self._dev(rows, self.act_dtype)
        if rows.dim() != 2 or rows.shape[1] != self.shape.hidden:
            raise ValueError("rows must be [n, hidden]")
        n = rows.shape[0]
        if out is None:
            out = torch.empty(n, dtype=torch.int32, device=self.device)
        self._dev(out, torch.int32)
        _check(lib().dflash_lm_head_argmax(self.ctx, _ptr(rows), n, _ptr(out), _stream(stream)), self.ctx)
        return out

    def lm_head_argmax_noalloc(self, rows: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
        """lm_head_argmax whose scratch is the library's fixed per-GPU array (no allocation:
        the caller provides the output too)."""
        self._dev(rows, self.act_dtype)
        if rows.dim() != 2 or rows.shape[1] != self.shape.hidden:
            raise ValueError("rows must be [n, hidden]")
        self._dev(out, torch.int32)
        if out.numel() < rows.shape[0]:
            raise ValueError("output too small")
        _check(lib().dflash_lm_head_argmax_noalloc(self.ctx, _ptr(rows), rows.shape[0], _ptr(out), _stream(stream)),
               self.ctx)
        return out

    def time_next_argmax(self, start: "torch.cuda.Event", end: "torch.cuda.Event") -> None:
        """Have the next lm_head_argmax call record `start` and `end` (timing-enabled
        torch.cuda.Event) right around its argmax kernel, so start.elapsed_time(end) is that
        kernel's duration."""
        handles = []
        for ev in (start, end):
            if not ev.cuda_event:
                ev.record()  # torch creates the underlying event on its first record
            handles.append(ctypes.c_void_p(ev.cuda_event))
        _check(lib().dflash_time_next_argmax(self.ctx, *handles), self.ctx)

    def time_next_chain(self, start: "torch.cuda.Event", end: "torch.cuda.Event") -> None:
        """Have the next draft_block of a DSpark context record `start` and `end` right around
        its Markov chain (gamma step launches)."""
        handles = []
        for ev in (start, end):
            if not ev.cuda_event:
                ev.record()
            handles.append(ctypes.c_void_p(ev.cuda_event))
        _check(lib().dflash_time_next_chain(self.ctx, *handles), self.ctx)

    def verify_greedy(self, draft: torch.Tensor, target: torch.Tensor, block: int,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        self._dev(draft, torch.int32)
        self._dev(target, torch.int32)
        if draft.numel() < block or target.numel() < block + 1:
            raise ValueError("draft needs block rows and target block + 1")
        if out is None:
            out = torch.empty(3, dtype=torch.int32, device=self.device)
        if out.device.type == "cpu":
            # pinned host memory: the verify kernel writes the result there itself, readable
            # once the stream has passed the call (no device->host copy)
            if not (out.is_pinned() and out.dtype == torch.int32 and out.is_contiguous() and out.numel() >= 3):
                raise ValueError("a host output must be a pinned, contiguous int32 tensor of 3 elements")
        else:
            self._dev(out, torch.int32)
        _check(lib().dflash_verify_greedy(self.ctx, _ptr(draft), _ptr(target), int(block), _ptr(out),
                                          _stream(stream)), self.ctx)
        return out

    def cache_state(self) -> Tuple[int, int, int, int]:
        e, pend, s, c = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().dflash_cache_state(self.ctx, ctypes.byref(e), ctypes.byref(pend), ctypes.byref(s),
                                        ctypes.byref(c)), self.ctx)
        return e.value, pend.value, s.value, c.value

    def cache_read(self, layer: int, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
        e, _, _, _ = self.cache_state()
        n_max = min(e, self.shape.window)
        sh = (self.shape.kv_heads, max(n_max, 1), self.shape.head_dim)
        k = torch.empty(sh, dtype=self.act_dtype, device=self.device)
        v = torch.empty(sh, dtype=self.act_dtype, device=self.device)
        n = ctypes.c_int32()
        _check(lib().dflash_cache_read(self.ctx, int(layer), _ptr(k), _ptr(v), ctypes.byref(n), _stream(stream)),
               self.ctx)
        return k[:, :n.value], v[:, :n.value]

    def _dev(self, t: torch.Tensor, dtype: torch.dtype) -> None:
        if t.device != self.device or t.dtype != dtype or not t.is_contiguous():
            raise ValueError(f"expected a contiguous {dtype} tensor on {self.device}, got {t.dtype} on {t.device}")


def hbm_read_probe(src: torch.Tensor, sink: torch.Tensor, groups: int, stream=None) -> None:
    """dflash_hbm_read_probe over the bytes of src (sink: int32 [groups] on the same device)."""
    if not (src.is_cuda and src.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32 and
            sink.numel() >= groups):
        raise ValueError("src and sink must be contiguous device tensors, sink int32 [groups]")
    _check(lib().dflash_hbm_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink), int(groups),
                                       _stream(stream)), None)


class WidthController:
    """dflash_width_ctl: the adaptive verify width of the round loop (host code in the library)."""

    def __init__(self, depth: int, ceiling: int, window: int, challenge_every: int):
        h = ctypes.c_void_p()
        _check(lib().dflash_width_ctl_create(depth, ceiling, window, challenge_every, ctypes.byref(h)), None)
        self.h = h

    def __del__(self):
        h = getattr(self, "h", None)
        if h and _lib is not None:
            _lib.dflash_width_ctl_destroy(h)
            self.h = None

    def width(self) -> int:
        return lib().dflash_width_ctl_width(self.h)

    def record(self, block: int, committed: int, ms: float) -> None:
        st = lib().dflash_width_ctl_record(self.h, int(block), int(committed), float(ms))
        if st != 0:
            raise DFlashError(st, lib().dflash_status_string(st).decode())

    def state(self) -> dict:
        i, c, ch = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        ir, cr = ctypes.c_double(), ctypes.c_double()
        n, a = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().dflash_width_ctl_state(self.h, *(ctypes.byref(x) for x in (i, c, ch, ir, cr, n, a))), None)
        return {"incumbent": i.value, "challenger": c.value, "challenging": bool(ch.value),
                "incumbent_rate": ir.value, "challenge_rate": cr.value, "challenges": n.value, "adoptions": a.value}


def make_target_config(t, max_block: int) -> dflash_target_config:
    cfg = dflash_target_config(
        hidden=t.hidden, layers=t.layers, q_heads=t.q_heads, kv_heads=t.kv_heads, head_dim=t.head_dim,
        intermediate=t.intermediate, vocab=t.vocab, window=t.window, max_context=t.max_context, max_block=max_block,
        full_mask=sum(1 << l for l in t.full_layers), n_capture=len(t.capture_layers),
        rms_eps=t.rms_eps, rope_theta=t.rope_theta, weight_dtype=_DTYPE[t.weight_dtype], act_dtype=_DTYPE[t.act_dtype])
    for i, l in enumerate(t.capture_layers):
        cfg.capture_layers[i] = l
    return cfg


def _check_target(status: int, t) -> None:
    if status != 0:
        L = lib()
        msg = L.dflash_target_last_error(t).decode() or L.dflash_status_string(status).decode()
        raise DFlashError(status, msg)


class Target:
    """One dflash_target: the round's target (verify forward, caches, trim) bound to device
    weights; `dev_weights` holds its layers, final_norm, and the embedding table and lm_head
    it shares with the drafter."""

    def __init__(self, tshape, dev_weights: Dict[str, object], max_block: int, device="cuda", stream=None):
        L = lib()
        self.shape = tshape
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.cfg = make_target_config(tshape, max_block)
        self._w = dev_weights

        def lin(name):
            t = dev_weights[name]
            if isinstance(t, tuple):
                return dflash_linear(_ptr(t[0]), _ptr(t[1]), _ptr(t[2]))
            return dflash_linear(_ptr(t), None, None)

        layers = (dflash_layer * tshape.layers)()
        for l in range(tshape.layers):
            p = f"layers.{l}."
            layers[l] = dflash_layer(*[lin(p + n) for n in ("q", "k", "v", "o", "gate", "up", "down")],
                                     *[_ptr(dev_weights[p + n]) for n in ("in_norm", "post_norm", "q_norm", "k_norm")])
        self._layers = layers
        self.weights = dflash_target_weights(_ptr(dev_weights["embed"]), lin("lm_head"), _ptr(dev_weights["final_norm"]),
                                             ctypes.cast(layers, ctypes.POINTER(dflash_layer)))
        cb, wb, pb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        _check(L.dflash_target_query_sizes(ctypes.byref(self.cfg), ctypes.byref(cb), ctypes.byref(wb), ctypes.byref(pb)),
               None)
        self.cache = torch.empty(max(cb.value, 256), dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(max(wb.value, 256), dtype=torch.uint8, device=self.device)
        self.packed = torch.empty(max(pb.value, 256), dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        _check(L.dflash_target_create(ctypes.byref(self.cfg), ctypes.byref(self.weights), _ptr(self.cache), cb.value,
                                      _ptr(self.workspace), wb.value, _ptr(self.packed), pb.value, _stream(stream),
                                      ctypes.byref(h)), None)
        self.t = h
        self.act_dtype = torch.float32 if tshape.act_dtype == "f32" else torch.bfloat16
        self.rows_max = max(max_block + 1, 32)

    def __del__(self):
        t = getattr(self, "t", None)
        if t and _lib is not None:
            _lib.dflash_target_destroy(t)
            self.t = None

    def forward(self, anchor: int, tokens: Optional[torch.Tensor], n: int, argmax: Optional[torch.Tensor] = None,
                capture: Optional[torch.Tensor] = None, stream=None):
        """Rows [anchor, tokens[0..n-2]]: returns (argmax int32 [n], capture or None)."""
        if argmax is None:
            argmax = torch.empty(n, dtype=torch.int32, device=self.device)
        for t_, dt in ((tokens, torch.int32), (argmax, torch.int32), (capture, self.act_dtype)):
            if t_ is not None and (t_.device != self.device or t_.dtype != dt or not t_.is_contiguous()):
                raise ValueError(f"expected a contiguous {dt} tensor on {self.device}")
        if tokens is not None and tokens.numel() < n - 1:
            raise ValueError("tokens too short")
        if capture is not None and capture.numel() < n * len(self.shape.capture_layers) * self.shape.hidden:
            raise ValueError("capture output too small")
        _check_target(lib().dflash_target_forward(self.t, int(anchor), _ptr(tokens), int(n), _ptr(argmax),
                                                  _ptr(capture), _stream(stream)), self.t)
        return argmax, capture

    def trim(self, m: int) -> None:
        _check_target(lib().dflash_target_trim(self.t, int(m)), self.t)

    def state(self) -> Tuple[int, int, int]:
        e, p, s = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check_target(lib().dflash_target_state(self.t, ctypes.byref(e), ctypes.byref(p), ctypes.byref(s)), self.t)
        return e.value, p.value, s.value

    def cache_read(self, layer: int, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
        """The committed keys and values the next query sees on `layer`: [kv_heads, n, head_dim]
        each (the library writes them packed; n <= e)."""
        e = self.state()[0]
        kv, hd = self.shape.kv_heads, self.shape.head_dim
        k = torch.empty(max(1, e) * kv * hd, dtype=self.act_dtype, device=self.device)
        v = torch.empty_like(k)
        n = ctypes.c_int32()
        _check_target(lib().dflash_target_cache_read(self.t, int(layer), _ptr(k), _ptr(v), ctypes.byref(n),
                                                     _stream(stream)), self.t)
        m = n.value
        return k[:kv * m * hd].view(kv, m, hd), v[:kv * m * hd].view(kv, m, hd)



def _check_batch(status: int, b) -> None:
    if status != 0:
        L = lib()
        msg = L.dflash_batch_last_error(b).decode() or L.dflash_status_string(status).decode()
        raise DFlashError(status, msg)


def _i32_array(vals) -> "ctypes.Array":
    vals = [int(v) for v in vals]
    return (ctypes.c_int32 * len(vals))(*vals)


class Batch:
    """One dflash_batch: n_seq independent sequences of one drafter, drafted together."""

    def __init__(self, shape, dev_weights: Dict[str, object], n_seq: int, max_block: int, phase: int = 0,
                 device="cuda", stream=None):
        L = lib()
        self.shape, self.n_seq = shape, n_seq
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.cfg = make_config(shape, max_block, phase)
        self._w = dev_weights

        def lin(name):
            t = dev_weights[name]
            if isinstance(t, tuple):
                return dflash_linear(_ptr(t[0]), _ptr(t[1]), _ptr(t[2]))
            return dflash_linear(_ptr(t), None, None)

        layers = (dflash_layer * shape.layers)()
        for l in range(shape.layers):
            p = f"layers.{l}."
            layers[l] = dflash_layer(*[lin(p + n) for n in ("q", "k", "v", "o", "gate", "up", "down")],
                                     *[_ptr(dev_weights[p + n]) for n in ("in_norm", "post_norm", "q_norm", "k_norm")])
        self._layers = layers
        self.weights = dflash_weights(_ptr(dev_weights["embed"]), lin("lm_head"), lin("fc"),
                                      _ptr(dev_weights["enc_norm"]), _ptr(dev_weights["final_norm"]),
                                      ctypes.cast(layers, ctypes.POINTER(dflash_layer)), None, None)
        rb, wb, pb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        _check(L.dflash_batch_query_sizes(ctypes.byref(self.cfg), n_seq, ctypes.byref(rb), ctypes.byref(wb),
                                          ctypes.byref(pb)), None)
        self.ring = torch.empty(max(rb.value, 256), dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(max(wb.value, 256), dtype=torch.uint8, device=self.device)
        self.packed = torch.empty(max(pb.value, 256), dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        _check(L.dflash_batch_create(ctypes.byref(self.cfg), n_seq, ctypes.byref(self.weights), _ptr(self.ring),
                                     rb.value, _ptr(self.workspace), wb.value, _ptr(self.packed), pb.value,
                                     _stream(stream), ctypes.byref(h)), None)
        self.b = h
        self.act_dtype = act_torch_dtype(shape)

    def __del__(self):
        b = getattr(self, "b", None)
        if b and _lib is not None:
            _lib.dflash_batch_destroy(b)
            self.b = None

    def append(self, resid: torch.Tensor, counts, commit: bool = False, stream=None) -> None:
        """resid: [sum(counts), fc_in], sequence 0's rows first."""
        self._dev(resid, self.act_dtype)
        if len(counts) != self.n_seq or resid.dim() != 2 or resid.shape[0] != sum(counts) or \
                resid.shape[1] != self.shape.fc_in:
            raise ValueError("residual rows must be [sum(counts), target_streams*target_width], one count per sequence")
        _check_batch(lib().dflash_batch_append(self.b, _ptr(resid), _i32_array(counts), int(bool(commit)),
                                               _stream(stream)), self.b)

    def trim(self, m) -> None:
        if len(m) != self.n_seq:
            raise ValueError("one rewind count per sequence")
        _check_batch(lib().dflash_batch_trim(self.b, _i32_array(m)), self.b)

    def draft(self, anchors, block: int, tokens: Optional[torch.Tensor] = None,
              hidden: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        if len(anchors) != self.n_seq:
            raise ValueError("one anchor per sequence")
        if tokens is None:
            tokens = torch.empty((self.n_seq, block), dtype=torch.int32, device=self.device)
        self._dev(tokens, torch.int32)
        if tokens.numel() < self.n_seq * block:
            raise ValueError("token output too small")
        if hidden is not None:
            self._dev(hidden, torch.float32)
            if hidden.numel() < self.n_seq * (block + 1) * self.shape.hidden:
                raise ValueError("hidden output too small")
        _check_batch(lib().dflash_batch_draft(self.b, _i32_array(anchors), int(block), _ptr(tokens), _ptr(hidden),
                                              _stream(stream)), self.b)
        return tokens

    def lm_head_argmax(self, rows: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        self._dev(rows, self.act_dtype)
        if rows.dim() != 2 or rows.shape[1] != self.shape.hidden:
            raise ValueError("rows must be [n, hidden]")
        if out is None:
            out = torch.empty(rows.shape[0], dtype=torch.int32, device=self.device)
        self._dev(out, torch.int32)
        _check_batch(lib().dflash_batch_lm_head_argmax(self.b, _ptr(rows), rows.shape[0], _ptr(out), _stream(stream)),
                     self.b)
        return out

    def verify_greedy(self, draft: torch.Tensor, target: torch.Tensor, block: int,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        self._dev(draft, torch.int32)
        self._dev(target, torch.int32)
        if draft.numel() < self.n_seq * block or target.numel() < self.n_seq * (block + 1):
            raise ValueError("draft needs [n_seq, block] and target [n_seq, block + 1]")
        if out is None:
            out = torch.empty((self.n_seq, 3), dtype=torch.int32, device=self.device)
        if out.device.type == "cpu":
            if not (out.is_pinned() and out.dtype == torch.int32 and out.is_contiguous() and
                    out.numel() >= 3 * self.n_seq):
                raise ValueError("a host output must be a pinned, contiguous int32 tensor of 3 * n_seq elements")
        else:
            self._dev(out, torch.int32)
        _check_batch(lib().dflash_batch_verify_greedy(self.b, _ptr(draft), _ptr(target), int(block), _ptr(out),
                                                      _stream(stream)), self.b)
        return out

    def state(self, seq: int) -> Tuple[int, int]:
        e, pend = ctypes.c_int64(), ctypes.c_int32()
        _check_batch(lib().dflash_batch_state(self.b, int(seq), ctypes.byref(e), ctypes.byref(pend)), self.b)
        return e.value, pend.value

    def cache_read(self, seq: int, layer: int, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
        e, _ = self.state(seq)
        n_max = min(e, self.shape.window)
        sh = (self.shape.kv_heads, max(n_max, 1), self.shape.head_dim)
        k = torch.empty(sh, dtype=self.act_dtype, device=self.device)
        v = torch.empty(sh, dtype=self.act_dtype, device=self.device)
        n = ctypes.c_int32()
        _check_batch(lib().dflash_batch_cache_read(self.b, int(seq), int(layer), _ptr(k), _ptr(v), ctypes.byref(n),
                                                   _stream(stream)), self.b)
        return k[:, :n.value], v[:, :n.value]

    def _dev(self, t: torch.Tensor, dtype: torch.dtype) -> None:
        if t.device != self.device or t.dtype != dtype or not t.is_contiguous():
            raise ValueError(f"expected a contiguous {dtype} tensor on {self.device}, got {t.dtype} on {t.device}")
