"""The Python binding's own checks (host side, before anything is enqueued): a
caller's output of the wrong shape or dtype, or a workspace that is not on the
GPU, is refused with ValueError, and a correct caller's buffer is used as given."""

import pytest
import torch

from gated_delta_rule_10_amd import inputs, kda
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pre():
    return gc.to_device(inputs.prefill_inputs(71, [100, 30], 2, 128, 64, "bf16", 0.1, "random"))


def _fwd(d, **kw):
    return kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"],
                             initial_state=d["initial_state"], **kw)


def _fwd_ex(d, **kw):
    return kda.kda_chunk_fwd_ex(d["q"], d["k"], d["v"], d["cu_seqlens"], log_alpha=d["log_alpha"], beta=d["beta"],
                                initial_state=d["initial_state"], **kw)


@pytest.mark.parametrize("call", [_fwd, _fwd_ex])
def test_prefill_output_and_workspace_checks(pre, call):
    T, H, V = pre["v"].shape
    for bad in (torch.empty((T, H, V + 1), dtype=torch.bfloat16, device="cuda"),
                torch.empty((T, H, V), dtype=torch.float16, device="cuda"),
                torch.empty((T - 1, H, V), dtype=torch.bfloat16, device="cuda")):
        with pytest.raises(ValueError):
            call(pre, o=bad)
    with pytest.raises(ValueError):
        call(pre, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    o = torch.empty((T, H, V), dtype=torch.bfloat16, device="cuda")
    got, _ = call(pre, o=o)
    ref, _ = call(pre)
    torch.cuda.synchronize()
    assert got.data_ptr() == o.data_ptr() and torch.equal(o, ref)


def test_decode_output_checks():
    x = inputs.device_decode_inputs(72, 1, 3, 2, 128, 128)
    q, k, v, g, b = (x[n][0].clone() for n in ("q", "k", "v", "log_alpha", "beta"))
    st = x["state"].clone()
    for bad in (torch.empty((3, 2, 64), dtype=torch.bfloat16, device="cuda"),
                torch.empty((3, 2, 128), dtype=torch.float16, device="cuda")):
        with pytest.raises(ValueError):
            kda.kda_decode_step(q, k, v, g, b, st, o=bad)
        with pytest.raises(ValueError):
            kda.kda_decode_step_ex(q, k, v, st, log_alpha=g, beta=b, o=bad)
    torch.cuda.synchronize()
    assert torch.equal(st, x["state"]), "a refused call changed the state"
