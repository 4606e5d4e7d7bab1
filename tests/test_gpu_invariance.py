"""GPU invariances between the library's own entry points, independent of the
oracle: a packed variable-length batch equals its sequences run one call at a
time, T decode steps equal one prefill over the same T tokens, and repeated
calls give the same bits (a missing wait between the copies into LDS and their
reads would show up as a changed result).
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_10_amd import inputs, kda
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu


def _slice_seq(d, n):
    cu = d["cu_seqlens"].cpu().tolist()
    a, b = cu[n], cu[n + 1]
    s0 = d["initial_state"]
    # copies: the ABI wants every array 16-byte aligned, which a slice need not be
    return dict(q=d["q"][a:b].clone(), k=d["k"][a:b].clone(), v=d["v"][a:b].clone(),
                log_alpha=d["log_alpha"][a:b].clone(), beta=d["beta"][a:b].clone(),
                cu_seqlens=torch.tensor([0, b - a], dtype=torch.int32, device="cuda"),
                initial_state=None if s0 is None else s0[n:n + 1].clone())


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("seg", ["3", None])
def test_packed_batch_equals_separate_calls(dt, seg, monkeypatch):
    """Sequences never interact: each one's outputs and final state are the same
    packed or alone. With a fixed segment length the work of a sequence is cut
    the same way in both calls, so they agree bit for bit; with the default
    segment length (which depends on the whole batch) they agree to the parity
    tolerance."""
    if seg is not None:
        monkeypatch.setenv("KDA_SEG_CHUNKS", seg)
    lens = [300, 0, 129, 64, 1000, 1]
    d = gc.to_device(inputs.prefill_inputs(61, lens, 2, 128, 128, dt, 0.1, "random"))
    od = torch.float32
    o, sT = gc.run_prefill(d, out_dtype=od)
    cu = d["cu_seqlens"].cpu().tolist()
    tol = gc.TOL_BF16 if dt == "bf16" else gc.TOL_F32
    for n in range(len(lens)):
        dn = _slice_seq(d, n)
        on, sn = gc.run_prefill(dn, out_dtype=od)
        got_o, got_s = o[cu[n]:cu[n + 1]], sT[n:n + 1]
        print(f"  sequence {n} ({lens[n]} tokens)", flush=True)
        if seg is not None:
            assert torch.equal(on, got_o), f"sequence {n}: outputs differ from the packed call"
            assert torch.equal(sn, got_s), f"sequence {n}: final state differs from the packed call"
        else:
            if lens[n]:
                gc.assert_close(f"o[{n}]", gc.host(on), gc.host(got_o).astype(np.float64), tol)
            gc.assert_close(f"state[{n}]", gc.host(sn), gc.host(got_s).astype(np.float64), tol)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_steps_equal_prefill(dt):
    """B sequences of T tokens each: T decode steps over a state cache that
    starts at the initial states give the prefill's outputs and final states
    (prefill in fp32 output, compared at the parity tolerance of its path)."""
    B, T, H = 4, 70, 3
    inp = inputs.prefill_inputs(62, [T] * B, H, 128, 128, dt, 0.1, "random")
    d = gc.to_device(inp)
    o, sT = gc.run_prefill(d, out_dtype=torch.float32)
    state = d["initial_state"].clone()
    tok = torch.arange(B, device="cuda") * T
    outs = []
    for t in range(T):
        idx = tok + t
        outs.append(kda.kda_decode_step(d["q"][idx], d["k"][idx], d["v"][idx], d["log_alpha"][idx],
                                        d["beta"][idx], state, out_dtype=torch.float32))
    torch.cuda.synchronize()
    od = torch.stack(outs, 1).reshape(B * T, H, 128)  # [B, T, H, V] -> token order
    tol = gc.TOL_BF16 if dt == "bf16" else gc.TOL_F32
    gc.assert_close("o (decode vs prefill)", gc.host(od), gc.host(o).astype(np.float64), tol)
    gc.assert_close("state (decode vs prefill)", gc.host(state), gc.host(sT).astype(np.float64), tol)


@pytest.mark.parametrize("name,seg,reps,epi", [
    ("long_128k", None, 6, False),
    ("mid_4x4k", "2", 16, False),
    ("mid_4x4k", "3", 16, False),
    ("mid_4x4k", "2", 8, True),
])
def test_repeated_calls_are_bitwise_identical(name, seg, reps, epi, monkeypatch):
    if seg is None:
        monkeypatch.delenv("KDA_SEG_CHUNKS", raising=False)
    else:
        monkeypatch.setenv("KDA_SEG_CHUNKS", seg)
    d = inputs.device_workload_inputs(name)
    ex = {}
    if epi:
        T, H, V = d["v"].shape
        gen = torch.Generator(device="cuda")
        gen.manual_seed(61)
        ex = dict(norm=True, norm_eps=1e-6, norm_weight=1 + 0.1 * torch.randn((V,), generator=gen, device="cuda"),
                  out_gate=torch.randn((T, H, V), generator=gen, device="cuda").to(torch.bfloat16),
                  out_gate_act="sigmoid")

    def call():
        return kda.kda_chunk_fwd_ex(d["q"], d["k"], d["v"], d["cu_seqlens"], log_alpha=d["log_alpha"],
                                    beta=d["beta"], initial_state=d["initial_state"], **ex)

    o0, s0 = call()
    for _ in range(reps - 1):
        o, s = call()
        assert torch.equal(o, o0) and torch.equal(s, s0)
