"""Seeded synthetic inputs for the KDA operator.

This module only draws random tensors with the distributions of the
workloads and lays them out as the library expects. It holds no part of the
operator's arithmetic, so both the HIP path and the fp64 oracle may use it.

Layouts (packed variable-length, tokens of all sequences back to back):
    q, k, log_alpha : [T_total, H, d_k]     v : [T_total, H, d_v]
    beta            : [T_total, H]          cu_seqlens : [N + 1] int32
    initial_state   : [N, H, d_k, d_v] fp32, or None for zeros

Recipe (one ``numpy.random.default_rng(seed)`` stream per workload, float32
normal draws in this fixed order: sequence lengths (variable-length case
only), q, k, v, x, y, initial state):
    q, k       ~ N(0, 1), L2-normalised over d_k per (token, head) in fp32,
               then rounded to bf16 (round-to-nearest-even) for bf16 inputs
    v          ~ N(0, 1), rounded to bf16 for bf16 inputs
    log_alpha  = -softplus(x) * decay_scale, fp32 (so alpha is in (0, 1))
    beta       = sigmoid(y), fp32, one value per (token, head)
    state      ~ 0.02 * N(0, 1) fp32 where the workload asks for one

bf16 values are carried in float32 containers (exact) plus their raw 16-bit
patterns, so the oracle reads exactly the numbers the GPU receives.

Two generators follow this recipe: a numpy one (PCG64, for small cases built
on the host) and a torch one that draws directly on the target device
(`device_*`, for the 128K-token and larger workloads, where host generation
takes minutes). A given seed gives different numbers on the two, so every
comparison feeds the same drawn tensors to both sides.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits",
    "PrefillInputs",
    "DecodeInputs",
    "prefill_inputs",
    "decode_inputs",
    "varlen_lengths",
    "WORKLOADS",
    "workload_inputs",
    "device_prefill_inputs",
    "device_decode_inputs",
    "device_workload_inputs",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of float32 values that are bf16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _sigmoid(y: np.ndarray) -> np.ndarray:
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-y))).astype(np.float32)


@dataclasses.dataclass
class PrefillInputs:
    q: np.ndarray  # [T, H, K] float32 container
    k: np.ndarray  # [T, H, K]
    v: np.ndarray  # [T, H, V]
    log_alpha: np.ndarray  # [T, H, K] float32
    beta: np.ndarray  # [T, H] float32
    cu_seqlens: np.ndarray  # [N+1] int32
    initial_state: Optional[np.ndarray]  # [N, H, K, V] float32 or None
    in_dtype: str  # "f32" or "bf16"

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def K(self) -> int:
        return int(self.q.shape[2])

    @property
    def V(self) -> int:
        return int(self.v.shape[2])


@dataclasses.dataclass
class DecodeInputs:
    q: np.ndarray  # [steps, B, H, K]
    k: np.ndarray  # [steps, B, H, K]
    v: np.ndarray  # [steps, B, H, V]
    log_alpha: np.ndarray  # [steps, B, H, K]
    beta: np.ndarray  # [steps, B, H]
    state: np.ndarray  # [slots, H, K, V] float32 initial cache
    in_dtype: str


def varlen_lengths(rng: np.random.Generator, n: int, lo: int, hi: int,
                   total: int) -> np.ndarray:
    """n lengths drawn log-uniform in [lo, hi], rescaled to sum to `total`.

    The rescaled reals are rounded by largest remainder so the sum is exact;
    the rescaled lengths are not clamped back into [lo, hi].
    """
    x = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n))
    scaled = x * (total / x.sum())
    base = np.floor(scaled).astype(np.int64)
    short = total - int(base.sum())
    order = np.argsort(-(scaled - base), kind="stable")
    base[order[:short]] += 1
    return base.astype(np.int64)


def prefill_inputs(seed: int, lengths: Sequence[int], H: int, K: int, V: int,
                   in_dtype: str = "bf16", decay_scale: float = 0.1,
                   init: str = "zero",
                   rng: Optional[np.random.Generator] = None) -> PrefillInputs:
    """Draw one packed prefill batch.

    init: "zero" (no initial state), "random" (every sequence ~0.02 N(0,1)),
          "odd_zero" (random for even sequence index, zero for odd).
    """
    if in_dtype not in ("f32", "bf16"):
        raise ValueError(in_dtype)
    rng = np.random.default_rng(seed) if rng is None else rng
    lengths = [int(x) for x in lengths]
    N, T = len(lengths), int(sum(lengths))
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    q = _l2_normalise(_normal(rng, (T, H, K)))
    k = _l2_normalise(_normal(rng, (T, H, K)))
    v = _normal(rng, (T, H, V))
    if in_dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    x = _normal(rng, (T, H, K))
    log_alpha = (-_softplus(x) * np.float32(decay_scale)).astype(np.float32)
    del x
    beta = _sigmoid(_normal(rng, (T, H)))
    s0 = None
    if init != "zero":
        s0 = (np.float32(0.02) * _normal(rng, (N, H, K, V))).astype(np.float32)
        if init == "odd_zero":
            s0[1::2] = 0.0
        elif init != "random":
            raise ValueError(init)
    return PrefillInputs(q, k, v, log_alpha, beta, cu, s0, in_dtype)


def option_inputs(seed: int, T: int, Hk: int, H: int, K: int, V: int, in_dtype: str = "bf16") -> dict:
    """Inputs of the extended entry points for T tokens (or T decode sequences):
    q, k [T, Hk, K] (unit rows), v [T, H, V], gate pre-activations gate_x
    [T, H, K] and beta_y [T, H], output gate out_gate [T, H, V], all ~N(0, 1)
    and rounded to in_dtype, and an fp32 norm weight [V] ~ 1 + 0.1 N(0, 1)."""
    rng = np.random.default_rng(seed)
    rnd = bf16_round if in_dtype == "bf16" else (lambda x: x)
    q = rnd(_l2_normalise(_normal(rng, (T, Hk, K))))
    k = rnd(_l2_normalise(_normal(rng, (T, Hk, K))))
    v = rnd(_normal(rng, (T, H, V)))
    gate_x = rnd(_normal(rng, (T, H, K)))
    beta_y = rnd(_normal(rng, (T, H)))
    out_gate = rnd(_normal(rng, (T, H, V)))
    norm_weight = (np.float32(1.0) + np.float32(0.1) * _normal(rng, (V,))).astype(np.float32)
    return dict(q=q, k=k, v=v, gate_x=gate_x, beta_y=beta_y, out_gate=out_gate, norm_weight=norm_weight)


def decode_inputs(seed: int, steps: int, B: int, H: int, K: int, V: int,
                  slots: Optional[int] = None, in_dtype: str = "bf16",
                  decay_scale: float = 0.1) -> DecodeInputs:
    """Draw `steps` single-token batches and an initial fp32 state cache."""
    rng = np.random.default_rng(seed)
    slots = B if slots is None else slots
    q = _l2_normalise(_normal(rng, (steps, B, H, K)))
    k = _l2_normalise(_normal(rng, (steps, B, H, K)))
    v = _normal(rng, (steps, B, H, V))
    if in_dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    x = _normal(rng, (steps, B, H, K))
    log_alpha = (-_softplus(x) * np.float32(decay_scale)).astype(np.float32)
    del x
    beta = _sigmoid(_normal(rng, (steps, B, H)))
    state = (np.float32(0.02) * _normal(rng, (slots, H, K, V))).astype(np.float32)
    return DecodeInputs(q, k, v, log_alpha, beta, state, in_dtype)


# The five workloads: the tiny fp32 case, a mid-size batch, one 128K-token
# sequence, a 64 x 32-head decode batch, and a 16-sequence packed batch of
# 524,288 tokens with log-uniform lengths in [1K, 64K].
WORKLOADS = {
    "tiny_f32": dict(kind="prefill", seed=0, lengths=[256], H=2, K=64, V=64,
                     in_dtype="f32", decay_scale=0.1, init="zero"),
    "mid_4x4k": dict(kind="prefill", seed=1, lengths=[4096] * 4, H=16, K=128,
                     V=128, in_dtype="bf16", decay_scale=0.1, init="zero"),
    "long_128k": dict(kind="prefill", seed=2, lengths=[131072], H=32, K=128,
                      V=128, in_dtype="bf16", decay_scale=0.05, init="random"),
    "decode_b64": dict(kind="decode", seed=3, steps=1000, B=64, H=32, K=128,
                       V=128, in_dtype="bf16", decay_scale=0.1),
    "varlen_512k": dict(kind="prefill", seed=4, lengths=None, H=32, K=128,
                        V=128, in_dtype="bf16", decay_scale=0.1,
                        init="odd_zero", n_seqs=16, len_lo=1024,
                        len_hi=65536, total=524288),
    # the 1M-token point of the pages' long-context figures (timed only)
    "long_1m": dict(kind="prefill", seed=5, lengths=[1048576], H=32, K=128,
                    V=128, in_dtype="bf16", decay_scale=0.05, init="random"),
}


def workload_inputs(name: str, steps: Optional[int] = None):
    """Inputs of one named workload (decode: optionally fewer steps)."""
    w = dict(WORKLOADS[name])
    if w.pop("kind") == "decode":
        if steps is not None:
            w["steps"] = steps
        return decode_inputs(**w)
    rng = np.random.default_rng(w.pop("seed"))
    lengths = w.pop("lengths")
    n_seqs = w.pop("n_seqs", None)
    lo, hi, total = w.pop("len_lo", None), w.pop("len_hi", None), w.pop("total", None)
    if lengths is None:
        lengths = varlen_lengths(rng, n_seqs, lo, hi, total)
    return prefill_inputs(seed=-1, lengths=lengths, rng=rng, **w)


# --- torch generator drawing on the target device ------------------------


def _torch():
    import torch
    return torch


def device_prefill_inputs(seed: int, lengths: Sequence[int], H: int, K: int, V: int,
                          in_dtype: str = "bf16", decay_scale: float = 0.1,
                          init: str = "zero", device="cuda") -> dict:
    """The prefill recipe drawn with torch on `device`.

    Returns a dict of tensors: q, k, v (bf16 or fp32), log_alpha, beta (fp32),
    cu_seqlens (int32), initial_state (fp32 or None).
    """
    torch = _torch()
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    lengths = [int(x) for x in lengths]
    N, T = len(lengths), int(sum(lengths))
    dt = torch.bfloat16 if in_dtype == "bf16" else torch.float32

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    def unit(x):
        return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)

    q = unit(normal(T, H, K)).to(dt)
    k = unit(normal(T, H, K)).to(dt)
    v = normal(T, H, V).to(dt)
    x = normal(T, H, K)
    log_alpha = -torch.logaddexp(x, torch.zeros((), device=device)) * decay_scale
    del x
    beta = torch.sigmoid(normal(T, H))
    s0 = None
    if init != "zero":
        s0 = 0.02 * normal(N, H, K, V)
        if init == "odd_zero":
            s0[1::2] = 0.0
    cu = torch.zeros(N + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return dict(q=q, k=k, v=v, log_alpha=log_alpha.contiguous(), beta=beta,
                cu_seqlens=cu.to(device), initial_state=s0)


def device_decode_inputs(seed: int, steps: int, B: int, H: int, K: int, V: int,
                         slots: Optional[int] = None, in_dtype: str = "bf16",
                         decay_scale: float = 0.1, device="cuda") -> dict:
    """The decode recipe drawn with torch on `device`: per-step tensors with a
    leading `steps` axis, plus the initial fp32 state cache."""
    torch = _torch()
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    slots = B if slots is None else slots
    dt = torch.bfloat16 if in_dtype == "bf16" else torch.float32

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    def unit(x):
        return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)

    q = unit(normal(steps, B, H, K)).to(dt)
    k = unit(normal(steps, B, H, K)).to(dt)
    v = normal(steps, B, H, V).to(dt)
    x = normal(steps, B, H, K)
    log_alpha = (-torch.logaddexp(x, torch.zeros((), device=device)) * decay_scale).contiguous()
    del x
    beta = torch.sigmoid(normal(steps, B, H))
    state = 0.02 * normal(slots, H, K, V)
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, state=state)


def device_workload_inputs(name: str, device="cuda", steps: Optional[int] = None) -> dict:
    """A named workload drawn on `device` (variable lengths still from numpy)."""
    w = dict(WORKLOADS[name])
    if w.pop("kind") == "decode":
        if steps is not None:
            w["steps"] = steps
        return device_decode_inputs(device=device, **w)
    lengths = w.pop("lengths")
    n_seqs = w.pop("n_seqs", None)
    lo, hi, total = w.pop("len_lo", None), w.pop("len_hi", None), w.pop("total", None)
    if lengths is None:
        lengths = varlen_lengths(np.random.default_rng(w["seed"]), n_seqs, lo, hi, total)
    return device_prefill_inputs(lengths=lengths, device=device, **w)
