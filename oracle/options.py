"""Options of the extended entry points, in fp64 -- TEST INFRASTRUCTURE.

Plain numpy definitions around the token-loop oracle (``oracle.prefill`` /
``oracle.decode``) for the steps just before and just after the operator and
for the serving layout of the states. Only the test-suite may import this
module; the GPU library never does.

Sources:
  - The 2025 attention/MoE review (lanjinlin.com.cn), section
    "GatedDeltaNet解读": the gates g and beta are produced from two inputs
    (a, b) before the recurrence; the query/key heads are shared by groups of
    value heads (broadcast of q_t to the value heads); after the loop the
    read-out is RMS-normalised and multiplied by an output gate z. Its
    MiniMax section fuses the group RMS norm, the sigmoid gate and the
    product into one kernel, hence the sigmoid option for z.
  - "线性注意力机制Kimi Linear架构解析与优化实践" (coreui.cn), section 3.2: the
    recurrent states live in one contiguous cache indexed per sequence.

Readings (the pages do not fix these; the same choices are stated in
include/kda.h): log alpha = -gate_scale * softplus(gate_x) and beta =
sigmoid(beta_y), the form the synthetic inputs are drawn with; the RMS norm
is taken over the d_v outputs of one token and head, o / sqrt(mean o^2 + eps),
then times a per-channel weight; a negative state slot is padding (zero
initial state, final state not written). The gates are evaluated in fp64
and handed to the token loop at fp32, the input type of its gate arguments.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import decode, prefill


def softplus(x):
    """ln(1 + e^x), evaluated without overflow."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def sigmoid(y):
    """1 / (1 + e^-y); for y < 0 written e^y / (1 + e^y), so that only e^-|y| is
    formed (no overflow) and small values keep their relative precision."""
    y = np.asarray(y, dtype=np.float64)
    e = np.exp(-np.abs(y))
    return np.where(y >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gate_log_alpha(x, gate_scale: float):
    return -float(gate_scale) * softplus(x)


def rms_norm(o, eps: float, weight=None):
    """o / sqrt(mean over the last axis of o^2 + eps), times weight (per last-axis channel)."""
    o = np.asarray(o, dtype=np.float64)
    out = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    if weight is not None:
        out = out * np.asarray(weight, dtype=np.float64)
    return out


def output_gate(o, z, act: str = "none"):
    z = np.asarray(z, dtype=np.float64)
    return o * (sigmoid(z) if act == "sigmoid" else z)


def expand_heads(x, H: int):
    """Key/query heads [.., Hk, d] broadcast to H value heads: value head h uses key head h // (H // Hk)."""
    Hk = x.shape[1]
    if H % Hk:
        raise ValueError("value heads must be a multiple of key heads")
    return np.repeat(np.asarray(x), H // Hk, axis=1)


def _gates(log_alpha, beta, gate_x, beta_y, gate_scale):
    if (log_alpha is None) == (gate_x is None) or (beta is None) == (beta_y is None):
        raise ValueError("give exactly one form of each gate")
    g = log_alpha if gate_x is None else gate_log_alpha(gate_x, gate_scale).astype(np.float32)
    b = beta if beta_y is None else sigmoid(beta_y).astype(np.float32)
    return g, b


def _epilogue(o, norm, norm_eps, norm_weight, out_gate, out_gate_act):
    if norm:
        o = rms_norm(o, norm_eps, norm_weight)
    if out_gate is not None:
        o = output_gate(o, out_gate, out_gate_act)
    return o


def prefill_ex(q, k, v, cu_seqlens, *, log_alpha=None, beta=None, gate_x=None, beta_y=None,
               gate_scale: float = 1.0, norm: bool = False, norm_eps: float = 1e-6, norm_weight=None,
               out_gate=None, out_gate_act: str = "none", state_slots: Optional[np.ndarray] = None,
               scale: float = 1.0, initial_state=None, nthreads: int = 0):
    """Prefill with the options of kda_chunk_fwd_ex. q, k [T, Hk, d_k]; v [T, H, d_v].

    Without state_slots: returns (o [T, H, d_v], final_state [N, H, d_k, d_v]).
    With state_slots: initial_state is a cache [slots, H, d_k, d_v]; returns
    (o, the cache after the call), where slot state_slots[n] >= 0 holds the
    final state of sequence n and every other slot is unchanged.
    """
    H = v.shape[1]
    qe, ke = expand_heads(q, H), expand_heads(k, H)
    g, b = _gates(log_alpha, beta, gate_x, beta_y, gate_scale)
    N = len(cu_seqlens) - 1
    s0 = initial_state
    if state_slots is not None:
        cache = np.asarray(initial_state, dtype=np.float64)
        s0 = np.zeros((N,) + cache.shape[1:], dtype=np.float64)
        for n, sl in enumerate(np.asarray(state_slots)):
            if sl >= 0:
                s0[n] = cache[sl]
    o, sf = prefill(qe, ke, v, g, b, cu_seqlens, scale, s0, nthreads=nthreads)
    o = _epilogue(o, norm, norm_eps, norm_weight, out_gate, out_gate_act)
    if state_slots is None:
        return o, sf
    out_cache = np.array(initial_state, dtype=np.float64)
    for n, sl in enumerate(np.asarray(state_slots)):
        if sl >= 0:
            out_cache[sl] = sf[n]
    return o, out_cache


def decode_ex(q, k, v, state: np.ndarray, slot_idx=None, *, log_alpha=None, beta=None, gate_x=None,
              beta_y=None, gate_scale: float = 1.0, norm: bool = False, norm_eps: float = 1e-6,
              norm_weight=None, out_gate=None, out_gate_act: str = "none", scale: float = 1.0,
              nthreads: int = 0):
    """One decode step with the options of kda_decode_step_ex; `state` (float64
    [slots, H, d_k, d_v]) is updated in place. Returns o [B, H, d_v]."""
    H = v.shape[1]
    g, b = _gates(log_alpha, beta, gate_x, beta_y, gate_scale)
    o = decode(expand_heads(q, H), expand_heads(k, H), v, g, b, state, slot_idx, scale, nthreads=nthreads)
    return _epilogue(o, norm, norm_eps, norm_weight, out_gate, out_gate_act)
