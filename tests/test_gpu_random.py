"""GPU parity on seeded random configurations through the C ABI: sequence count
and lengths (empty, single-token, partial and several chunks), key-head
grouping, head sizes, input type, gate form, output epilogue, slot caches and
segment length (so that the map pass, the prefix and the output pass all take
part), each against the fp64 oracle with the same options."""

import numpy as np
import pytest

from tests.test_gpu_options import _prefill_case

pytestmark = pytest.mark.gpu

CASES = 64


def _config(i):
    r = np.random.default_rng(1000 + i)
    N = int(r.integers(1, 5))
    lens = [int(r.choice([0, 1, 63, 64, 65, int(r.integers(1, 400))])) for _ in range(N)]
    if sum(lens) == 0:
        lens[0] = 130
    Hk = int(r.choice([1, 2]))
    H = Hk * int(r.choice([1, 2]))
    K, V = int(r.choice([64, 128])), int(r.choice([64, 128]))
    dt = str(r.choice(["bf16", "f32"]))
    gates = str(r.choice(["pre", "plain"]))
    norm = bool(r.integers(0, 2))
    z_act = [None, "none", "sigmoid"][int(r.integers(0, 3))]
    slots = None
    if r.integers(0, 2):
        slots = [int(x) for x in r.permutation(N + 2)[:N]]
        if N > 1 and r.integers(0, 2):
            slots[int(r.integers(0, N))] = -1
    seg = [None, "1", "2", "3"][int(r.integers(0, 4))]
    return dict(lens=lens, Hk=Hk, H=H, K=K, V=V, dt=dt, gates=gates, norm=norm, z_act=z_act, slots=slots, seg=seg)


@pytest.mark.parametrize("i", range(CASES))
def test_random_configuration(i, monkeypatch):
    c = _config(i)
    print(f"  case {i}: {c}", flush=True)
    if c["seg"] is not None:
        monkeypatch.setenv("KDA_SEG_CHUNKS", c["seg"])
    _prefill_case(2000 + i, c["lens"], c["Hk"], c["H"], c["K"], c["V"], c["dt"], gates=c["gates"], norm=c["norm"],
                  z_act=c["z_act"], slots=c["slots"])


def _large_config(i):
    r = np.random.default_rng(95000 + i)
    N = int(r.integers(1, 9))
    lens = [int(np.exp(r.uniform(0, np.log(20000)))) if r.random() > 0.1 else 0 for _ in range(N)]
    if sum(lens) == 0:
        lens[0] = 5000
    H = int(r.choice([4, 8, 16, 32]))
    Hk = int(r.choice([d for d in (1, 2, 4) if H % d == 0]))
    K, V = int(r.choice([64, 128])), int(r.choice([64, 128]))
    gates = str(r.choice(["pre", "plain"]))
    norm = bool(r.integers(0, 2))
    z_act = [None, "none", "sigmoid"][int(r.integers(0, 3))]
    slots = None
    if r.integers(0, 2):
        slots = [int(x) for x in r.permutation(N + 2)[:N]]
    decay = float(r.choice([0.05, 0.1, 0.3]))
    return dict(lens=lens, Hk=Hk, H=H, K=K, V=V, gates=gates, norm=norm, z_act=z_act, slots=slots, decay=decay)


@pytest.mark.parametrize("i", range(8))
def test_random_large_configuration(i, monkeypatch):
    """Up to 8 sequences of up to 20K tokens, H up to 32, bf16, with the library's
    own segment length; bf16 outputs, and fp32 outputs held to the bar directly."""
    monkeypatch.delenv("KDA_SEG_CHUNKS", raising=False)
    c = _large_config(i)
    print(f"  large case {i}: T={sum(c['lens'])} {c}", flush=True)
    _prefill_case(8000 + i, c["lens"], c["Hk"], c["H"], c["K"], c["V"], "bf16", gates=c["gates"], norm=c["norm"],
                  z_act=c["z_act"], slots=c["slots"], decay=c["decay"])


def _decode_config(i):
    r = np.random.default_rng(3000 + i)
    B = int(r.integers(1, 17))
    Hk = int(r.choice([1, 2]))
    H = Hk * int(r.choice([1, 2, 4]))
    K, V = int(r.choice([64, 128])), int(r.choice([64, 128]))
    dt = str(r.choice(["bf16", "f32"]))
    nslots = B + int(r.integers(0, 5))
    use_slots = bool(r.integers(0, 2)) or nslots > B
    gates = str(r.choice(["pre", "plain"]))
    norm = bool(r.integers(0, 2))
    z_act = [None, "none", "sigmoid"][int(r.integers(0, 3))]
    return dict(B=B, Hk=Hk, H=H, K=K, V=V, dt=dt, nslots=nslots, use_slots=use_slots, gates=gates, norm=norm,
                z_act=z_act)


@pytest.mark.parametrize("i", range(12))
def test_random_decode_configuration(i):
    import torch
    from gated_delta_rule_10_amd import inputs, kda
    from oracle import options as oo
    from tests import gpu_common as gc
    from tests.test_gpu_options import _t
    c = _decode_config(i)
    print(f"  decode case {i}: {c}", flush=True)
    bf = c["dt"] == "bf16"
    B, Hk, H, K, V = c["B"], c["Hk"], c["H"], c["K"], c["V"]
    rng = np.random.default_rng(4000 + i)
    state = (0.02 * rng.standard_normal((c["nslots"], H, K, V))).astype(np.float32)
    si = rng.permutation(c["nslots"])[:B].astype(np.int32) if c["use_slots"] else None
    dstate = torch.from_numpy(state).cuda()
    ref_state = state.astype(np.float64)
    tol = gc.TOL_BF16 if bf else gc.TOL_F32
    for step in range(2):
        x = inputs.option_inputs(5000 + 10 * i + step, B, Hk, H, K, V, c["dt"])
        kw_o, kw_g = {}, {}
        if c["gates"] == "pre":
            kw_o.update(gate_x=x["gate_x"], beta_y=x["beta_y"], gate_scale=0.1)
            kw_g.update(gate_x=_t(x["gate_x"], bf), beta_y=_t(x["beta_y"], bf), gate_scale=0.1)
        else:
            g = (-0.1 * oo.softplus(x["gate_x"])).astype(np.float32)
            b = oo.sigmoid(x["beta_y"]).astype(np.float32)
            kw_o.update(log_alpha=g, beta=b)
            kw_g.update(log_alpha=_t(g, False), beta=_t(b, False))
        if c["norm"]:
            kw_o.update(norm=True, norm_eps=1e-5, norm_weight=x["norm_weight"])
            kw_g.update(norm=True, norm_eps=1e-5, norm_weight=_t(x["norm_weight"], False))
        if c["z_act"] is not None:
            kw_o.update(out_gate=x["out_gate"], out_gate_act=c["z_act"])
            kw_g.update(out_gate=_t(x["out_gate"], bf), out_gate_act=c["z_act"])
        ref_o = oo.decode_ex(x["q"], x["k"], x["v"], ref_state, si, **kw_o)
        o = kda.kda_decode_step_ex(_t(x["q"], bf), _t(x["k"], bf), _t(x["v"], bf), dstate,
                                   None if si is None else torch.from_numpy(si).cuda(), **kw_g)
        torch.cuda.synchronize()
        gc.assert_close(f"o step {step}", gc.host(o), ref_o, tol, bf16_rounded=bf)
    gc.assert_close("state", gc.host(dstate), ref_state, tol)
