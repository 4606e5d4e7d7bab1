"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
running the library through its binding, running the oracle on the same
bytes, and the comparison metric."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from gated_delta_rule_10_amd import inputs, kda

# Tolerances, as max-abs error over RMS of the reference, per tensor:
# fp32 inputs 1e-4; bf16 inputs 2e-2, applied to the error beyond the final
# bf16 rounding of o (which alone can reach 2-3% of RMS(o) on the largest
# outputs), and directly to fp32 outputs and fp32 states.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def to_device(inp: inputs.PrefillInputs, device="cuda") -> dict:
    def t(x, bf16):
        if bf16:
            return torch.from_numpy(inputs.bf16_bits(x)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)

    bf = inp.in_dtype == "bf16"
    return dict(q=t(inp.q, bf), k=t(inp.k, bf), v=t(inp.v, bf),
                log_alpha=t(inp.log_alpha, False), beta=t(inp.beta, False),
                cu_seqlens=torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device),
                initial_state=None if inp.initial_state is None
                else t(inp.initial_state, False))


def host(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy()


def run_prefill(d: dict, out_dtype=None, **kw):
    o, sT = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                              d["cu_seqlens"], initial_state=d.get("initial_state"),
                              out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return o, sT


def oracle_prefill(d: dict, heads=None, seqs=None, nthreads=0):
    """Oracle on the device tensors' exact values, for a subset of heads and
    sequences. Returns (o [T_sub, H_sub, V], sT [N_sub, H_sub, K, V], token
    index array of the subset)."""
    cu = d["cu_seqlens"].cpu().numpy().astype(np.int64)
    N = len(cu) - 1
    seqs = list(range(N)) if seqs is None else list(seqs)
    H = d["q"].shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    tok = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs]).astype(np.int64)
    tok_t = torch.from_numpy(tok).to(d["q"].device)
    hd = torch.tensor(heads, device=d["q"].device)

    def sub(x):
        return host(x.index_select(0, tok_t).index_select(1, hd))

    lens = [cu[n + 1] - cu[n] for n in seqs]
    cu_sub = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    s0 = d.get("initial_state")
    s0_sub = None if s0 is None else host(
        s0.index_select(0, torch.tensor(seqs, device=s0.device)).index_select(1, hd))
    o, sT = oracle.prefill(sub(d["q"]), sub(d["k"]), sub(d["v"]), sub(d["log_alpha"]),
                           sub(d["beta"]), cu_sub, 1.0, s0_sub, nthreads=nthreads)
    return o, sT, tok


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8.0), 0.0)


def err_over_rms(got, ref, bf16_rounded: bool = False) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = np.abs(got - ref)
    if bf16_rounded:
        d = np.maximum(d - half_ulp_bf16(np.maximum(np.abs(ref), np.abs(got))), 0.0)
    return float(d.max()) / max(rms, 1e-300)  # a floor only for an all-zero reference


def norm_epilogue_bound(pre, tol, norm_eps, weight=None, gate=None):
    """Per-element error bound of the RMS-norm epilogue's output, propagated from
    the bar on the operator's own output o (every element of o within
    e = tol * RMS(o)). With s = sqrt(mean over the row of o^2 + eps) and
    y_i = w_i o_i / s, a change d in o moves y_i by
    w_i (d_i / s - o_i (sum_j o_j d_j / d_v) / s^3), and |sum_j o_j d_j / d_v| <= e s,
    so |dy_i| <= e |w_i| (1 / s + |o_i| / s^2); an output gate multiplies it by
    |act(z_i)|. `pre` is the oracle's output before the epilogue, `gate` the
    values act(z)."""
    pre = np.asarray(pre, np.float64)
    if pre.size == 0:
        return pre
    e = tol * float(np.sqrt(np.mean(pre * pre)))
    s = np.sqrt(np.mean(pre * pre, axis=-1, keepdims=True) + norm_eps)
    w = 1.0 if weight is None else np.abs(np.asarray(weight, np.float64))
    bound = e * w * (1.0 / s + np.abs(pre) / (s * s))
    if gate is not None:
        bound = bound * np.abs(np.asarray(gate, np.float64))
    return bound


def gate_epilogue_bound(pre, tol, gate):
    """Per-element error bound of an output gated without the norm, y_i = o_i act(z_i),
    from the bar on o (every element within e = tol * RMS(o)): |dy_i| <= e |act(z_i)|.
    The plain bar on y itself would instead be tol * RMS(y), about tol * RMS(o) * RMS(act(z)),
    which an element with |act(z_i)| several times RMS(act(z)) exceeds whenever its o carries
    an error near the bar. `pre` is the oracle's output before the gate, `gate` act(z)."""
    pre = np.asarray(pre, np.float64)
    if pre.size == 0:
        return pre
    e = tol * float(np.sqrt(np.mean(pre * pre)))
    return e * np.abs(np.asarray(gate, np.float64))


def assert_within_bound(name, got, ref, bound, bf16_rounded=False):
    """Every element within its own bound (after half a bf16 ulp for bf16 outputs)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if ref.size == 0:
        return 0.0
    d = np.abs(got - ref)
    if bf16_rounded:
        d = np.maximum(d - half_ulp_bf16(np.maximum(np.abs(ref), np.abs(got))), 0.0)
    r = float(np.max(d / np.maximum(bound, 1e-300)))
    print(f"  {name}: max error / propagated bound = {r:.3f} (err/RMS = {err_over_rms(got, ref, bf16_rounded):.3e})",
          flush=True)
    assert r <= 1.0, f"{name}: error {r:.3f} x its propagated bound"
    return r


def assert_close(name, got, ref, tol, bf16_rounded=False):
    e = err_over_rms(got, ref, bf16_rounded)
    print(f"  {name}: err/RMS = {e:.3e} (tol {tol:.0e})", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert e <= tol, f"{name}: max-abs error {e:.3e} x RMS exceeds {tol:.0e}"
    return e
