"""The kernels against the hand-derived worked example under tests/golden/,
without the oracle: the 2-channel example embedded in d_k = d_v = 64 (zero q
and k in the other key channels, zero v and initial state in the other value
channels, which therefore contribute nothing and stay zero), at read-out
scales 1 and 1/2, through prefill on both input paths and through decode."""

import numpy as np
import pytest
import torch

from gated_delta_rule_10_amd import inputs, kda
from tests import gpu_common as gc
from tests import pins

pytestmark = pytest.mark.gpu

D = 64


def _embedded():
    q, k, v, g, b, s0, o_ref, s_ref, sc, o_sc = pins.load_worked_example(scaled=True)
    T = q.shape[0]

    def pad(x, last):
        out = np.zeros(x.shape[:-1] + (last,), np.float64)
        out[..., :x.shape[-1]] = x
        return out

    e = dict(q=pad(q, D), k=pad(k, D), v=pad(v, D), g=pad(g, D), b=b, s0=np.zeros((1, 1, D, D)),
             o=pad(o_ref, D), o_half=pad(o_sc, D), sT=np.zeros((1, 1, D, D)), scale_half=sc, T=T)
    e["s0"][..., :2, :2] = s0
    e["sT"][..., :2, :2] = s_ref
    return e


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_prefill_reproduces_the_worked_example(dt):
    e = _embedded()
    bf = dt == "bf16"

    def t(x, low):
        x = np.ascontiguousarray(x, np.float32)
        if low:  # every input of the example is dyadic, so exact in bf16
            return torch.from_numpy(inputs.bf16_bits(x)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    cu = torch.tensor([0, e["T"]], dtype=torch.int32, device="cuda")
    tol = gc.TOL_BF16 if bf else gc.TOL_F32
    for scale, o_exp in ((1.0, e["o"]), (e["scale_half"], e["o_half"])):
        o, sT = kda.kda_chunk_fwd(t(e["q"], bf), t(e["k"], bf), t(e["v"], bf), t(e["g"], False), t(e["b"], False),
                                  cu, scale=scale, initial_state=t(e["s0"], False), out_dtype=torch.float32)
        torch.cuda.synchronize()
        gc.assert_close(f"o (scale {scale})", gc.host(o), o_exp, tol)
        gc.assert_close(f"final state (scale {scale})", gc.host(sT), e["sT"], tol)


def test_decode_reproduces_the_worked_example():
    e = _embedded()
    for scale, o_exp in ((1.0, e["o"]), (e["scale_half"], e["o_half"])):
        state = torch.from_numpy(np.ascontiguousarray(e["s0"][0][None], np.float32)).cuda()
        for s in range(e["T"]):
            def t(x):
                return torch.from_numpy(np.ascontiguousarray(x[s:s + 1], np.float32)).cuda()
            o = kda.kda_decode_step(t(e["q"]), t(e["k"]), t(e["v"]), t(e["g"]), t(e["b"]), state, scale=scale,
                                    out_dtype=torch.float32)
            torch.cuda.synchronize()
            gc.assert_close(f"o step {s} (scale {scale})", gc.host(o), o_exp[s:s + 1], gc.TOL_F32)
        gc.assert_close(f"state (scale {scale})", gc.host(state), e["sT"][0], gc.TOL_F32)
