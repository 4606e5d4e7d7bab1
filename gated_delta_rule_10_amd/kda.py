"""Python binding of libkda (include/kda.h): argument marshalling only.

Every step of the operator runs in the HIP kernels of libkda.so. PyTorch is
used for device memory and streams. If the library is not built, or a tensor
is not on a GPU, the functions raise; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)
KDA_F32, KDA_BF16 = 0, 1
KDA_ACT_NONE, KDA_ACT_SIGMOID = 0, 1
CHUNK_SIZE = 64


class KdaOptions(ctypes.Structure):
    """kda_options_t of include/kda.h (field order and C types as declared there)."""
    _fields_ = [("num_k_heads", ctypes.c_int32),
                ("gate_x", ctypes.c_void_p),
                ("beta_y", ctypes.c_void_p),
                ("gate_scale", ctypes.c_float),
                ("norm", ctypes.c_int32),
                ("norm_eps", ctypes.c_float),
                ("norm_weight", ctypes.c_void_p),
                ("out_gate", ctypes.c_void_p),
                ("out_gate_act", ctypes.c_int),
                ("state_slots", ctypes.c_void_p),
                ("num_slots", ctypes.c_int32)]

_lib = None


class KDAError(RuntimeError):
    """A libkda entry point returned a status other than KDA_OK."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kda_status_string(status)}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so and declare its C signatures (no HIP call is made)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m gated_delta_rule_10_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    lib.kda_chunk_fwd_workspace_size.restype = sz
    lib.kda_chunk_fwd.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_int,
                                  ctypes.c_int, f32, P, P, P, i32, P, sz, P]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                    ctypes.c_int, ctypes.c_int, f32, P]
    lib.kda_decode_step.restype = ctypes.c_int
    opt = ctypes.POINTER(KdaOptions)
    lib.kda_chunk_fwd_ex.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_int,
                                     ctypes.c_int, f32, P, P, P, i32, P, sz, opt, P]
    lib.kda_chunk_fwd_ex.restype = ctypes.c_int
    lib.kda_chunk_fwd_ex_noalloc.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_int,
                                             ctypes.c_int, f32, P, P, P, i32, opt, P]
    lib.kda_chunk_fwd_ex_noalloc.restype = ctypes.c_int
    lib.kda_decode_step_ex.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                       ctypes.c_int, ctypes.c_int, f32, opt, P]
    lib.kda_decode_step_ex.restype = ctypes.c_int
    _lib = lib
    return lib


def kda_abi_version() -> int:
    return int(load_library().kda_abi_version())


def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def _code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return KDA_F32
    if dt == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out(o: Optional[torch.Tensor], shape, dtype: torch.dtype, device) -> torch.Tensor:
    """The output tensor: a new one, or the caller's after checking its shape and dtype
    (the kernels write every element of that shape)."""
    if o is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(o.shape) != tuple(shape) or o.dtype != dtype:
        raise ValueError(f"o must be {dtype} {tuple(shape)}")
    return _dev(o, "o")


def _workspace(lib, workspace: Optional[torch.Tensor], N, T, H, d_k, d_v, in_dtype, device):
    """(workspace, bytes): the caller's (on the GPU; the library checks its size) or a new
    one of the size the library asks for (none when it asks for 0 bytes)."""
    if workspace is None:
        need = int(lib.kda_chunk_fwd_workspace_size(N, T, H, d_k, d_v, _code(in_dtype)))
        if not need:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _dev(workspace, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def _one_device(device, *tensors) -> None:
    """Every tensor given (None skipped) on `device`: the call runs there."""
    for t in tensors:
        if t is not None and t.device != device:
            raise ValueError(f"all tensors must be on {device} (found one on {t.device})")


def _stream(stream, device) -> ctypes.c_void_p:
    """The stream to enqueue on: the given one (of `device`), else the current one of `device`."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    if s.device != device:
        raise ValueError(f"stream is on {s.device}, the tensors on {device}")
    return ctypes.c_void_p(s.cuda_stream)


def kda_chunk_fwd_workspace_size(N: int, T_total: int, H: int, d_k: int, d_v: int,
                                 in_dtype: torch.dtype) -> int:
    return int(load_library().kda_chunk_fwd_workspace_size(N, T_total, H, d_k, d_v,
                                                           _code(in_dtype)))


def kda_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  log_alpha: torch.Tensor, beta: torch.Tensor, cu_seqlens: torch.Tensor,
                  *, scale: float = 1.0, initial_state: Optional[torch.Tensor] = None,
                  output_final_state: bool = True, final_state: Optional[torch.Tensor] = None,
                  out_dtype: Optional[torch.dtype] = None, o: Optional[torch.Tensor] = None,
                  chunk_size: int = CHUNK_SIZE, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunk prefill over packed sequences (see kda_chunk_fwd in include/kda.h).

    q, k, log_alpha: [T, H, d_k]; v: [T, H, d_v]; beta: [T, H];
    cu_seqlens: int32 [N+1] on the GPU; initial_state: fp32 [N, H, d_k, d_v] or None.
    Returns (o [T, H, d_v], final_state [N, H, d_k, d_v] or None).
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta),
                    ("cu_seqlens", cu_seqlens)):
        _dev(t, name)
    T, H, d_k = q.shape
    d_v = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape[:2] != (T, H) \
            or beta.shape != (T, H) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("inconsistent q/k/v/log_alpha/beta shapes or dtypes")
    if log_alpha.dtype != torch.float32 or beta.dtype != torch.float32 \
            or cu_seqlens.dtype != torch.int32:
        raise ValueError("log_alpha and beta must be float32, cu_seqlens int32")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o = _out(o, (T, H, d_v), out_dtype, q.device)
    if initial_state is not None:
        _dev(initial_state, "initial_state")
        if initial_state.shape != (N, H, d_k, d_v) or initial_state.dtype != torch.float32:
            raise ValueError("initial_state must be float32 [N, H, d_k, d_v]")
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, d_k, d_v), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _dev(final_state, "final_state")
        if final_state.shape != (N, H, d_k, d_v) or final_state.dtype != torch.float32:
            raise ValueError("final_state must be float32 [N, H, d_k, d_v]")
    workspace, ws_bytes = _workspace(lib, workspace, N, T, H, d_k, d_v, q.dtype, q.device)
    _one_device(q.device, k, v, log_alpha, beta, cu_seqlens, initial_state, final_state, o, workspace)
    with torch.cuda.device(q.device):
        st = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                               _ptr(cu_seqlens), N, T, H, d_k, d_v, _code(q.dtype),
                               _code(out_dtype), float(scale), _ptr(initial_state),
                               _ptr(final_state), _ptr(o), int(chunk_size), _ptr(workspace),
                               ws_bytes, _stream(stream, q.device))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd")
    return o, final_state


def kda_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    log_alpha: torch.Tensor, beta: torch.Tensor, state_cache: torch.Tensor,
                    slot_idx: Optional[torch.Tensor] = None, *, scale: float = 1.0,
                    out_dtype: Optional[torch.dtype] = None, o: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """One decode step, updating state_cache [slots, H, d_k, d_v] fp32 in place.

    q, k, log_alpha: [B, H, d_k]; v: [B, H, d_v]; beta: [B, H];
    slot_idx: int32 [B] on the GPU or None. Returns o [B, H, d_v].
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta),
                    ("state_cache", state_cache)):
        _dev(t, name)
    B, H, d_k = q.shape
    d_v = v.shape[2]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape[:2] != (B, H) \
            or beta.shape != (B, H) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("inconsistent q/k/v/log_alpha/beta shapes or dtypes")
    if state_cache.dtype != torch.float32 or state_cache.shape[1:] != (H, d_k, d_v):
        raise ValueError("state_cache must be float32 [slots, H, d_k, d_v]")
    if slot_idx is not None:
        _dev(slot_idx, "slot_idx")
        if slot_idx.dtype != torch.int32 or slot_idx.shape != (B,):
            raise ValueError("slot_idx must be int32 [B]")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o = _out(o, (B, H, d_v), out_dtype, q.device)
    _one_device(q.device, k, v, log_alpha, beta, state_cache, slot_idx, o)
    with torch.cuda.device(q.device):
        st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                 _ptr(state_cache), _ptr(slot_idx), _ptr(o), B, H, d_k, d_v,
                                 state_cache.shape[0], _code(q.dtype), _code(out_dtype),
                                 float(scale), _stream(stream, q.device))
    if st != KDA_OK:
        raise KDAError(st, "kda_decode_step")
    return o


def _act_code(act) -> int:
    if act in (None, "none", KDA_ACT_NONE):
        return KDA_ACT_NONE
    if act in ("sigmoid", KDA_ACT_SIGMOID):
        return KDA_ACT_SIGMOID
    raise ValueError(f"unknown output gate activation {act!r}")


def _options(H, num_k_heads=None, gate_x=None, beta_y=None, gate_scale=1.0, norm=False,
             norm_eps=1e-6, norm_weight=None, out_gate=None, out_gate_act="none",
             state_slots=None, num_slots=0) -> KdaOptions:
    op = KdaOptions()
    op.num_k_heads = int(num_k_heads or H)
    for name, t in (("gate_x", gate_x), ("beta_y", beta_y), ("norm_weight", norm_weight),
                    ("out_gate", out_gate), ("state_slots", state_slots)):
        if t is not None:
            _dev(t, name)
    op.gate_x = None if gate_x is None else gate_x.data_ptr()
    op.beta_y = None if beta_y is None else beta_y.data_ptr()
    op.gate_scale = float(gate_scale)
    op.norm = int(bool(norm))
    op.norm_eps = float(norm_eps)
    op.norm_weight = None if norm_weight is None else norm_weight.data_ptr()
    op.out_gate = None if out_gate is None else out_gate.data_ptr()
    op.out_gate_act = _act_code(out_gate_act)
    op.state_slots = None if state_slots is None else state_slots.data_ptr()
    op.num_slots = int(num_slots)
    return op


def kda_chunk_fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, *,
                     workspace: Optional[torch.Tensor] = None, **kw) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_chunk_fwd_ex of include/kda.h (arguments as for _chunk_fwd_ex below; the
    workspace is the caller's or, when None, a new one of the size the library asks for)."""
    return _chunk_fwd_ex(q, k, v, cu_seqlens, noalloc=False, workspace=workspace, **kw)


def kda_chunk_fwd_ex_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                             **kw) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_chunk_fwd_ex_noalloc of include/kda.h: no workspace; the library works in its
    static scratch. Pass o (and final_state, or output_final_state=False) to have the
    binding allocate nothing either."""
    return _chunk_fwd_ex(q, k, v, cu_seqlens, noalloc=True, workspace=None, **kw)


def _chunk_fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, *,
                  noalloc: bool, log_alpha: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
                  gate_x: Optional[torch.Tensor] = None, beta_y: Optional[torch.Tensor] = None,
                  gate_scale: float = 1.0, norm: bool = False, norm_eps: float = 1e-6,
                  norm_weight: Optional[torch.Tensor] = None, out_gate: Optional[torch.Tensor] = None,
                  out_gate_act="none", state_slots: Optional[torch.Tensor] = None,
                  scale: float = 1.0, initial_state: Optional[torch.Tensor] = None,
                  output_final_state: bool = True, final_state: Optional[torch.Tensor] = None,
                  out_dtype: Optional[torch.dtype] = None, o: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_chunk_fwd_ex (noalloc: kda_chunk_fwd_ex_noalloc) of include/kda.h.

    q, k: [T, Hk, d_k]; v: [T, H, d_v] with H a multiple of Hk (value head h uses key
    head h // (H // Hk)); gates either log_alpha [T, H, d_k] fp32 and beta [T, H] fp32,
    or gate_x [T, H, d_k] / beta_y [T, H] in the input dtype (log_alpha =
    -gate_scale * softplus(gate_x), beta = sigmoid(beta_y)). Epilogue: norm (RMS over
    d_v, times norm_weight [d_v] fp32), then out_gate [T, H, d_v] (act "none" or
    "sigmoid"). With state_slots [N] int32, initial_state is a cache [slots, H, d_k, d_v]
    and final_state defaults to that same cache (updated in place).
    Returns (o [T, H, d_v], final_state).
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("cu_seqlens", cu_seqlens)):
        _dev(t, name)
    T, Hk, d_k = q.shape
    H, d_v = v.shape[1], v.shape[2]
    N = cu_seqlens.shape[0] - 1
    if k.shape != q.shape or v.shape[0] != T or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("inconsistent q/k/v shapes or dtypes")
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    for name, t, shape, dt in (("log_alpha", log_alpha, (T, H, d_k), torch.float32),
                               ("beta", beta, (T, H), torch.float32),
                               ("gate_x", gate_x, (T, H, d_k), q.dtype),
                               ("beta_y", beta_y, (T, H), q.dtype),
                               ("out_gate", out_gate, (T, H, d_v), q.dtype),
                               ("norm_weight", norm_weight, (d_v,), torch.float32)):
        if t is not None:
            _dev(t, name)
            if tuple(t.shape) != shape or t.dtype != dt:
                raise ValueError(f"{name} must be {dt} {shape}")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o = _out(o, (T, H, d_v), out_dtype, q.device)
    num_slots = 0
    if state_slots is not None:
        _dev(state_slots, "state_slots")
        if state_slots.dtype != torch.int32 or state_slots.shape != (N,):
            raise ValueError("state_slots must be int32 [N]")
        if initial_state is None:
            raise ValueError("state_slots needs the state cache as initial_state")
        num_slots = initial_state.shape[0]
        if final_state is None and output_final_state:
            final_state = initial_state
    else:
        if final_state is None and output_final_state:
            final_state = torch.empty((N, H, d_k, d_v), dtype=torch.float32, device=q.device)
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None:
            _dev(t, name)
            if t.dtype != torch.float32 or tuple(t.shape[1:]) != (H, d_k, d_v) or \
                    (state_slots is None and t.shape[0] != N):
                raise ValueError(f"{name} must be float32 [{'slots' if state_slots is not None else 'N'}, H, d_k, d_v]")
    op = _options(H, Hk, gate_x, beta_y, gate_scale, norm, norm_eps, norm_weight, out_gate, out_gate_act,
                  state_slots, num_slots)
    if noalloc:
        _one_device(q.device, k, v, cu_seqlens, log_alpha, beta, gate_x, beta_y, norm_weight, out_gate,
                    state_slots, initial_state, final_state, o)
        with torch.cuda.device(q.device):
            st = lib.kda_chunk_fwd_ex_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                              _ptr(cu_seqlens), N, T, H, d_k, d_v, _code(q.dtype),
                                              _code(out_dtype), float(scale), _ptr(initial_state),
                                              _ptr(final_state), _ptr(o), CHUNK_SIZE, ctypes.byref(op),
                                              _stream(stream, q.device))
        if st != KDA_OK:
            raise KDAError(st, "kda_chunk_fwd_ex_noalloc")
        return o, final_state
    workspace, ws_bytes = _workspace(lib, workspace, N, T, H, d_k, d_v, q.dtype, q.device)
    _one_device(q.device, k, v, cu_seqlens, log_alpha, beta, gate_x, beta_y, norm_weight, out_gate, state_slots,
                initial_state, final_state, o, workspace)
    with torch.cuda.device(q.device):
        st = lib.kda_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(cu_seqlens),
                                  N, T, H, d_k, d_v, _code(q.dtype), _code(out_dtype), float(scale),
                                  _ptr(initial_state), _ptr(final_state), _ptr(o), CHUNK_SIZE,
                                  _ptr(workspace), ws_bytes, ctypes.byref(op), _stream(stream, q.device))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_ex")
    return o, final_state


def kda_decode_step_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state_cache: torch.Tensor,
                       slot_idx: Optional[torch.Tensor] = None, *,
                       log_alpha: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
                       gate_x: Optional[torch.Tensor] = None, beta_y: Optional[torch.Tensor] = None,
                       gate_scale: float = 1.0, norm: bool = False, norm_eps: float = 1e-6,
                       norm_weight: Optional[torch.Tensor] = None, out_gate: Optional[torch.Tensor] = None,
                       out_gate_act="none", scale: float = 1.0, out_dtype: Optional[torch.dtype] = None,
                       o: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kda_decode_step_ex of include/kda.h: q, k [B, Hk, d_k]; v [B, H, d_v]; the other
    options as for kda_chunk_fwd_ex. Returns o [B, H, d_v]."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("state_cache", state_cache)):
        _dev(t, name)
    B, Hk, d_k = q.shape
    H, d_v = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != B or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("inconsistent q/k/v shapes or dtypes")
    if state_cache.dtype != torch.float32 or tuple(state_cache.shape[1:]) != (H, d_k, d_v):
        raise ValueError("state_cache must be float32 [slots, H, d_k, d_v]")
    for name, t, shape, dt in (("log_alpha", log_alpha, (B, H, d_k), torch.float32),
                               ("beta", beta, (B, H), torch.float32),
                               ("gate_x", gate_x, (B, H, d_k), q.dtype),
                               ("beta_y", beta_y, (B, H), q.dtype),
                               ("out_gate", out_gate, (B, H, d_v), q.dtype),
                               ("norm_weight", norm_weight, (d_v,), torch.float32)):
        if t is not None:
            _dev(t, name)
            if tuple(t.shape) != shape or t.dtype != dt:
                raise ValueError(f"{name} must be {dt} {shape}")
    if slot_idx is not None:
        _dev(slot_idx, "slot_idx")
        if slot_idx.dtype != torch.int32 or slot_idx.shape != (B,):
            raise ValueError("slot_idx must be int32 [B]")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o = _out(o, (B, H, d_v), out_dtype, q.device)
    op = _options(H, Hk, gate_x, beta_y, gate_scale, norm, norm_eps, norm_weight, out_gate, out_gate_act)
    _one_device(q.device, k, v, state_cache, slot_idx, log_alpha, beta, gate_x, beta_y, norm_weight, out_gate, o)
    with torch.cuda.device(q.device):
        st = lib.kda_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(state_cache),
                                    _ptr(slot_idx), _ptr(o), B, H, d_k, d_v, state_cache.shape[0],
                                    _code(q.dtype), _code(out_dtype), float(scale), ctypes.byref(op),
                                    _stream(stream, q.device))
    if st != KDA_OK:
        raise KDAError(st, "kda_decode_step_ex")
    return o
