"""kda_chunk_fwd_ex_noalloc, which works in the library's static scratch instead
of a caller workspace, against kda_chunk_fwd_ex on the same inputs: two calls in
a row, the second with a smaller input (and options), bit for bit, and both
against the fp64 oracle at the parity bar."""

import numpy as np
import pytest
import torch

from gated_delta_rule_10_amd import inputs, kda
from oracle import options as oo
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu


def _run(d, noalloc, out_dtype, **kw):
    T, H, V = d["v"].shape
    K = d["q"].shape[2]
    N = d["cu_seqlens"].numel() - 1
    slots = kw.get("state_slots")
    o = torch.full((T, H, V), float("nan"), dtype=out_dtype, device="cuda")
    if slots is None:
        fin = torch.full((N, H, K, V), float("nan"), dtype=torch.float32, device="cuda")
        s0 = d["initial_state"]
    else:  # the cache is read and written in place: a copy per call
        s0 = fin = d["initial_state"].clone()
    fn = kda.kda_chunk_fwd_ex_noalloc if noalloc else kda.kda_chunk_fwd_ex
    fn(d["q"], d["k"], d["v"], d["cu_seqlens"], log_alpha=d.get("log_alpha"), beta=d.get("beta"),
       initial_state=s0, final_state=fin, o=o, **kw)
    torch.cuda.synchronize()
    return o, fin


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_matches_the_workspace_entry(dt, monkeypatch):
    # segments of 3 chunks: offsets, initial-state copies, map pass, prefix and
    # output pass all keep their data in the scratch
    monkeypatch.setenv("KDA_SEG_CHUNKS", "3")
    bf = dt == "bf16"
    od = torch.bfloat16 if bf else torch.float32
    tol = gc.TOL_BF16 if bf else gc.TOL_F32

    # first call: 3 sequences, H = 4, d = 128, plain gates
    big = inputs.prefill_inputs(51, [700, 64, 300], 4, 128, 128, dt, 0.1, "random")
    d = gc.to_device(big)
    ref = _run(d, False, od)
    got = _run(d, True, od)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), "first call differs"
    ro, rs, _ = gc.oracle_prefill(d)
    gc.assert_close("o (first call)", gc.host(got[0]), ro, tol, bf16_rounded=bf)
    gc.assert_close("final_state (first call)", gc.host(got[1]), rs, tol)

    # second, smaller call: 2 sequences, H = 2 over one key head, d_v = 64, gate
    # pre-activations and slot-indexed states (one padding slot)
    lens = [130, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = inputs.option_inputs(52, int(sum(lens)), 1, 2, 128, 64, dt)
    cache = (0.02 * np.random.default_rng(52).standard_normal((3, 2, 128, 64))).astype(np.float32)
    slots = np.array([2, -1], np.int32)

    def t(a, keep_dtype):
        if keep_dtype and bf:
            return torch.from_numpy(inputs.bf16_bits(a)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()

    d2 = dict(q=t(x["q"], True), k=t(x["k"], True), v=t(x["v"], True), cu_seqlens=torch.from_numpy(cu).cuda(),
              initial_state=t(cache, False))
    kw = dict(gate_x=t(x["gate_x"], True), beta_y=t(x["beta_y"], True), gate_scale=0.1,
              state_slots=torch.from_numpy(slots).cuda())
    ref = _run(d2, False, od, **kw)
    got = _run(d2, True, od, **kw)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), "second call differs"
    ro, rs = oo.prefill_ex(x["q"], x["k"], x["v"], cu, gate_x=x["gate_x"], beta_y=x["beta_y"], gate_scale=0.1,
                           state_slots=slots, initial_state=cache)
    gc.assert_close("o (second call)", gc.host(got[0]), ro, tol, bf16_rounded=bf)
    gc.assert_close("state cache (second call)", gc.host(got[1]), rs, tol)
