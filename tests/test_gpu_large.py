"""GPU parity where element offsets pass 2^31: every index into q, k, v, the
gates, the outputs and the state cache must be computed in 64 bits. Heads and
slots at both ends of the arrays are checked against the fp64 oracle.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_10_amd import inputs, kda
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seg", [None, "100"])
def test_prefill_beyond_2_31_elements(seg, monkeypatch):
    """Two sequences (40,000 and 30,001 tokens), H = 256, d = 128, bf16: q holds
    70,001 * 256 * 128 = 2.29e9 elements. Heads 0 and 255 against the oracle.
    With seg, segments of 100 chunks (map pass and prefix)."""
    if seg is not None:
        monkeypatch.setenv("KDA_SEG_CHUNKS", seg)
    d = inputs.device_prefill_inputs(71, [40000, 30001], 256, 128, 128, "bf16", 0.1, "random")
    assert d["q"].numel() > 2 ** 31
    o, sT = gc.run_prefill(d)
    heads = [0, 255]
    ref_o, ref_s, _ = gc.oracle_prefill(d, heads=heads, nthreads=0)
    hd = torch.tensor(heads, device="cuda")
    gc.assert_close("o", gc.host(o.index_select(1, hd)), ref_o, gc.TOL_BF16, bf16_rounded=True)
    gc.assert_close("final_state", gc.host(sT.index_select(1, hd)), ref_s, gc.TOL_BF16)


def test_decode_beyond_2_31_elements():
    """A 1024-slot x 256-head fp32 cache (4.3e9 elements, 17 GB); three sequences
    write slots 1023, 0 and 700. Those slots (heads 0 and 255) and their outputs
    against the oracle; an untouched slot keeps its state."""
    slots, H, K, V = 1024, 256, 128, 128
    slot_idx = np.array([1023, 0, 700], np.int32)
    x = inputs.device_decode_inputs(72, 1, 3, H, K, V)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(72)
    state = torch.empty((slots, H, K, V), dtype=torch.float32, device="cuda")
    for s in range(0, slots, 128):  # drawn in pieces to bound the temporary
        state[s:s + 128] = 0.02 * torch.randn((128, H, K, V), generator=gen, device="cuda")
    assert state.numel() > 2 ** 31
    heads = torch.tensor([0, 255], device="cuda")
    si = torch.from_numpy(slot_idx).long().cuda()
    before = gc.host(state.index_select(0, si).index_select(1, heads)).astype(np.float64)
    untouched = state[5, 255].clone()
    o = kda.kda_decode_step(x["q"][0], x["k"][0], x["v"][0], x["log_alpha"][0], x["beta"][0], state,
                            torch.from_numpy(slot_idx).cuda())
    torch.cuda.synchronize()

    def sub(t):
        return gc.host(t[0].index_select(1, heads))

    ref_state = before.copy()  # slots in slot_idx order, heads 0 and 255
    ref_o = gc.oracle.decode(sub(x["q"]), sub(x["k"]), sub(x["v"]), sub(x["log_alpha"]),
                             gc.host(x["beta"][0].index_select(1, heads)), ref_state,
                             np.arange(3, dtype=np.int32))
    gc.assert_close("o", gc.host(o.index_select(1, heads)), ref_o, gc.TOL_BF16, bf16_rounded=True)
    gc.assert_close("state", gc.host(state.index_select(0, si).index_select(1, heads)), ref_state, gc.TOL_BF16)
    assert torch.equal(state[5, 255], untouched)
