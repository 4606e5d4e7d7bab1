"""GPU parity of the extended entry points (kda_chunk_fwd_ex, kda_decode_step_ex)
against the fp64 oracle with the same options (oracle/options.py): grouped
key heads, gate pre-activations, the RMS-norm / output-gate epilogue and
slot-indexed states, alone and together, on both input types."""

import numpy as np
import pytest
import torch

from gated_delta_rule_10_amd import inputs, kda
from oracle import options as oo
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu


def _t(x, bf):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if bf:
        t = torch.from_numpy(inputs.bf16_bits(x)).view(torch.bfloat16)
    return t.cuda()


def _prefill_case(seed, lens, Hk, H, K, V, dt, *, gates="pre", norm=False, z_act=None,
                  slots=None, out_dtypes=None, decay=0.1):
    bf = dt == "bf16"
    T = int(sum(lens))
    x = inputs.option_inputs(seed, T, Hk, H, K, V, dt)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = len(lens)
    rng = np.random.default_rng(seed + 1000)
    kw_o, kw_g = {}, {}
    if gates == "pre":
        kw_o.update(gate_x=x["gate_x"], beta_y=x["beta_y"], gate_scale=decay)
        kw_g.update(gate_x=_t(x["gate_x"], bf), beta_y=_t(x["beta_y"], bf), gate_scale=decay)
    else:
        g = (-decay * oo.softplus(x["gate_x"])).astype(np.float32)
        b = oo.sigmoid(x["beta_y"]).astype(np.float32)
        kw_o.update(log_alpha=g, beta=b)
        kw_g.update(log_alpha=_t(g, False), beta=_t(b, False))
    if norm:
        kw_o.update(norm=True, norm_eps=1e-5, norm_weight=x["norm_weight"])
        kw_g.update(norm=True, norm_eps=1e-5, norm_weight=_t(x["norm_weight"], False))
    if z_act is not None:
        kw_o.update(out_gate=x["out_gate"], out_gate_act=z_act)
        kw_g.update(out_gate=_t(x["out_gate"], bf), out_gate_act=z_act)
    if slots is not None:
        nslots = max(max(slots) + 2, N)
        cache = (0.02 * rng.standard_normal((nslots, H, K, V))).astype(np.float32)
        s_np = np.asarray(slots, np.int32)
        ref_o, ref_s = oo.prefill_ex(x["q"], x["k"], x["v"], cu, state_slots=s_np, initial_state=cache,
                                     **kw_o)
    else:
        s0 = (0.02 * rng.standard_normal((N, H, K, V))).astype(np.float32)
        ref_o, ref_s = oo.prefill_ex(x["q"], x["k"], x["v"], cu, initial_state=s0, **kw_o)
    tol = gc.TOL_BF16 if bf else gc.TOL_F32
    bound = None
    if norm or z_act is not None:  # the bar on the operator's o, carried through the epilogue
        kw_pre = {k: v for k, v in kw_o.items() if k not in ("norm", "norm_eps", "norm_weight", "out_gate",
                                                              "out_gate_act")}
        init = cache if slots is not None else s0
        extra = dict(state_slots=s_np) if slots is not None else {}
        pre, _ = oo.prefill_ex(x["q"], x["k"], x["v"], cu, initial_state=init, **extra, **kw_pre)
        gate = None if z_act is None else oo.output_gate(np.ones_like(pre), x["out_gate"], z_act)
        if norm:
            bound = gc.norm_epilogue_bound(pre, tol, 1e-5, x["norm_weight"], gate)
        else:
            bound = gc.gate_epilogue_bound(pre, tol, gate)
    for od in (out_dtypes or ([torch.bfloat16, torch.float32] if bf else [torch.float32])):
        if slots is not None:
            st = torch.from_numpy(cache).cuda()
            o, sT = kda.kda_chunk_fwd_ex(_t(x["q"], bf), _t(x["k"], bf), _t(x["v"], bf), torch.from_numpy(cu).cuda(),
                                         state_slots=torch.from_numpy(s_np).cuda(), initial_state=st,
                                         out_dtype=od, **kw_g)
        else:
            o, sT = kda.kda_chunk_fwd_ex(_t(x["q"], bf), _t(x["k"], bf), _t(x["v"], bf), torch.from_numpy(cu).cuda(),
                                         initial_state=torch.from_numpy(s0).cuda(), out_dtype=od, **kw_g)
        torch.cuda.synchronize()
        if bound is None:
            gc.assert_close(f"o[{od}]", gc.host(o), ref_o, tol, bf16_rounded=od == torch.bfloat16)
        else:
            gc.assert_within_bound(f"o[{od}]", gc.host(o), ref_o, bound, bf16_rounded=od == torch.bfloat16)
        gc.assert_close("final_state", gc.host(sT), ref_s, tol)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("Hk", [1, 2])
def test_grouped_key_heads(dt, Hk):
    _prefill_case(21, [150, 70], Hk, 4, 128, 128, dt, gates="plain")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gate_preactivations(dt):
    _prefill_case(22, [200, 129], 3, 3, 128, 128, dt, gates="pre")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("norm,z_act", [(True, None), (False, "sigmoid"), (True, "none"), (True, "sigmoid")])
def test_output_epilogue(dt, norm, z_act):
    _prefill_case(23, [190, 64, 1], 2, 2, 128, 128, dt, gates="plain", norm=norm, z_act=z_act)


@pytest.mark.parametrize("case", [
    dict(seed=7051, lens=[129, 129, 2, 128, 129, 127], Hk=3, H=6, K=64, V=128, z_act=None,
         slots=[3, -1, 8, 5, 4, 6], seg="1"),
    dict(seed=7114, lens=[1, 129], Hk=1, H=3, K=128, V=64, z_act="none", slots=[-1, 1], seg="3"),
])
def test_output_norm_strong_decay(case, monkeypatch):
    """Strong decay (log alpha = -0.5 softplus(x)) and the RMS norm: rows whose
    output is small before the norm (here down to 7 % of RMS(o)) are scaled up
    by it, and their error with them, so o is held to the propagated bound."""
    monkeypatch.setenv("KDA_SEG_CHUNKS", case["seg"])
    _prefill_case(case["seed"], case["lens"], case["Hk"], case["H"], case["K"], case["V"], "bf16", gates="pre",
                  norm=True, z_act=case["z_act"], slots=case["slots"], decay=0.5)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("seg", ["2", "16"])
def test_state_slots(dt, seg, monkeypatch):
    monkeypatch.setenv("KDA_SEG_CHUNKS", seg)
    # shuffled slots, a padding sequence and an empty one; several segments per sequence
    _prefill_case(24, [300, 0, 77, 260], 2, 2, 128, 128, dt, gates="plain", slots=[5, 2, -1, 0])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_no_tokens_with_slots_and_epilogue(dt):
    # T = 0: the cache passes through (slot 2 and 0 keep their states, the padding
    # sequence writes nothing) and there are no output rows to normalise or gate
    _prefill_case(26, [0, 0, 0], 2, 4, 128, 128, dt, gates="pre", norm=True, z_act="sigmoid", slots=[2, -1, 0])


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_all_options_together(dk, dv, monkeypatch):
    monkeypatch.setenv("KDA_SEG_CHUNKS", "2")
    _prefill_case(25, [333, 5, 180], 2, 4, dk, dv, "bf16", gates="pre", norm=True, z_act="sigmoid",
                  slots=[1, 3, 0])


def test_all_options_fp32():
    _prefill_case(26, [140, 70], 1, 2, 64, 64, "f32", gates="pre", norm=True, z_act="sigmoid", slots=[2, 0])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_options(dt):
    bf = dt == "bf16"
    B, Hk, H, K, V, slots_n = 8, 2, 4, 128, 128, 12
    rng = np.random.default_rng(27)
    state = (0.02 * rng.standard_normal((slots_n, H, K, V))).astype(np.float32)
    si = rng.permutation(slots_n)[:B].astype(np.int32)
    dstate = torch.from_numpy(state).cuda()
    ref_state = state.astype(np.float64)
    tol = gc.TOL_BF16 if bf else gc.TOL_F32
    for step in range(3):
        x = inputs.option_inputs(270 + step, B, Hk, H, K, V, dt)
        ref_o = oo.decode_ex(x["q"], x["k"], x["v"], ref_state, si, gate_x=x["gate_x"], beta_y=x["beta_y"],
                             gate_scale=0.1, norm=True, norm_eps=1e-5, norm_weight=x["norm_weight"],
                             out_gate=x["out_gate"], out_gate_act="sigmoid")
        o = kda.kda_decode_step_ex(_t(x["q"], bf), _t(x["k"], bf), _t(x["v"], bf), dstate,
                                   torch.from_numpy(si).cuda(), gate_x=_t(x["gate_x"], bf),
                                   beta_y=_t(x["beta_y"], bf), gate_scale=0.1, norm=True, norm_eps=1e-5,
                                   norm_weight=_t(x["norm_weight"], False), out_gate=_t(x["out_gate"], bf),
                                   out_gate_act="sigmoid")
        torch.cuda.synchronize()
        gc.assert_close(f"o step {step}", gc.host(o), ref_o, tol, bf16_rounded=bf)
    gc.assert_close("state", gc.host(dstate), ref_state, tol)


def test_extended_entry_points_without_options_match_the_plain_ones():
    inp = inputs.prefill_inputs(28, [130, 61], 2, 128, 128, "bf16", 0.1, "random")
    d = gc.to_device(inp)
    o1, s1 = gc.run_prefill(d)
    o2, s2 = kda.kda_chunk_fwd_ex(d["q"], d["k"], d["v"], d["cu_seqlens"], log_alpha=d["log_alpha"],
                                  beta=d["beta"], initial_state=d["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_decode_steps_replayed_from_a_hip_graph_match_eager():
    """Decode steps (plain and extended) captured once in a HIP graph and replayed
    three times, with eager work and synchronisation between the replays, give
    bitwise the eager outputs and states."""
    B, H, K, V, steps = 8, 4, 128, 128, 3
    rng = np.random.default_rng(29)
    state0 = torch.from_numpy((0.02 * rng.standard_normal((B, H, K, V))).astype(np.float32)).cuda()
    xs = [inputs.option_inputs(290 + s, B, 2, H, K, V, "bf16") for s in range(steps)]
    dev = [{n: _t(x[n], n != "norm_weight") for n in x} for x in xs]
    la = [torch.from_numpy((-0.1 * oo.softplus(x["gate_x"])).astype(np.float32)).cuda() for x in xs]
    be = [torch.from_numpy(oo.sigmoid(x["beta_y"]).astype(np.float32)).cuda() for x in xs]
    outs = [torch.empty((B, H, V), dtype=torch.bfloat16, device="cuda") for _ in range(2 * steps)]
    state = state0.clone()

    def run():
        for s in range(steps):
            d = dev[s]
            kda.kda_decode_step_ex(d["q"], d["k"], d["v"], state, log_alpha=la[s], beta=be[s], o=outs[2 * s])
            kda.kda_decode_step_ex(d["q"], d["k"], d["v"], state, gate_x=d["gate_x"], beta_y=d["beta_y"],
                                   gate_scale=0.1, norm=True, norm_weight=d["norm_weight"], out_gate=d["out_gate"],
                                   out_gate_act="sigmoid", o=outs[2 * s + 1])

    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    ref_state = state.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the capture stream first, as torch graph capture expects
        state.copy_(state0)
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    state.copy_(state0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        state.copy_(state0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {rep}: output differs from eager"
        assert torch.equal(state, ref_state), f"replay {rep}: state differs from eager"
        _ = (state * 2).sum().item()   # eager work between replays


def test_prefill_replayed_from_a_hip_graph_matches_eager(monkeypatch):
    """Prefill (plain and extended, several segments per sequence, so every kernel
    of the call runs) captured once in a HIP graph with caller-provided outputs and
    workspace, replayed three times with eager work and synchronisation between
    the replays: outputs and final states equal the eager ones bitwise."""
    monkeypatch.setenv("KDA_SEG_CHUNKS", "2")
    lens = [300, 77, 500]
    Hk, H, K, V = 2, 4, 128, 128
    T, N = sum(lens), len(lens)
    x = inputs.option_inputs(31, T, Hk, H, K, V, "bf16")
    d = {n: _t(x[n], n != "norm_weight") for n in x}
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    rng = np.random.default_rng(31)
    s0 = torch.from_numpy((0.02 * rng.standard_normal((N, H, K, V))).astype(np.float32)).cuda()
    la = torch.from_numpy((-0.1 * oo.softplus(x["gate_x"])).astype(np.float32)).cuda()
    be = torch.from_numpy(oo.sigmoid(x["beta_y"]).astype(np.float32)).cuda()
    o = [torch.empty((T, H, V), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    fin = [torch.empty((N, H, K, V), dtype=torch.float32, device="cuda") for _ in range(2)]
    ws = torch.empty(kda.kda_chunk_fwd_workspace_size(N, T, H, K, V, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")

    def run():
        kda.kda_chunk_fwd_ex(d["q"], d["k"], d["v"], cu, log_alpha=la, beta=be, initial_state=s0,
                             final_state=fin[0], o=o[0], workspace=ws)
        kda.kda_chunk_fwd_ex(d["q"], d["k"], d["v"], cu, gate_x=d["gate_x"], beta_y=d["beta_y"], gate_scale=0.1,
                             norm=True, norm_weight=d["norm_weight"], out_gate=d["out_gate"],
                             out_gate_act="sigmoid", initial_state=s0, final_state=fin[1], o=o[1], workspace=ws)

    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in o + fin]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the capture stream first, as torch graph capture expects
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for t in o + fin:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(o + fin, ref):
            assert torch.equal(t, r), f"replay {rep}: differs from eager"
        _ = (s0 * 2).sum().item()   # eager work between replays


def _row_err(got, ref):
    """max over output rows (one token or sequence, one head) of max |got - ref| / RMS(ref) of the row"""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    return float(np.max(np.abs(got - ref) / np.maximum(rms, 1e-300)))


def _epilogue_ref(raw, x, norm, z_act):
    ref = np.asarray(raw, np.float64)
    if norm:
        ref = oo.rms_norm(ref, 1e-5, x["norm_weight"])
    if z_act is not None:
        ref = oo.output_gate(ref, x["out_gate"], z_act)
    return ref


def _epilogue_kw(x, bf, norm, z_act):
    kw = {}
    if norm:
        kw.update(norm=True, norm_eps=1e-5, norm_weight=_t(x["norm_weight"], False))
    if z_act is not None:
        kw.update(out_gate=_t(x["out_gate"], bf), out_gate_act=z_act)
    return kw


EPI_CASES = [(True, None), (False, "sigmoid"), (True, "none"), (True, "sigmoid")]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("norm,z_act", EPI_CASES)
def test_epilogue_arithmetic_prefill(dt, norm, z_act, monkeypatch):
    """The fused RMS-norm / output-gate epilogue of the prefill against the oracle's
    rms_norm and output_gate applied in fp64 to the same kernels' fp32 output
    without the epilogue, from the same inputs (identical up to the epilogue): only
    the epilogue's own fp32 arithmetic separates the two, held to 1e-5 of each
    row's RMS. The parity tests above hold the whole path to the oracle."""
    monkeypatch.setenv("KDA_SEG_CHUNKS", "2")
    bf = dt == "bf16"
    lens = [190, 64, 1, 333]
    T, Hk, H, K, V = int(sum(lens)), 2, 4, 128, 128
    x = inputs.option_inputs(31, T, Hk, H, K, V, dt)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    g = (-0.1 * oo.softplus(x["gate_x"])).astype(np.float32)
    b = oo.sigmoid(x["beta_y"]).astype(np.float32)
    s0 = (0.02 * np.random.default_rng(32).standard_normal((len(lens), H, K, V))).astype(np.float32)
    q, k, v = _t(x["q"], bf), _t(x["k"], bf), _t(x["v"], bf)
    common = dict(log_alpha=_t(g, False), beta=_t(b, False), initial_state=_t(s0, False), out_dtype=torch.float32)
    raw, _ = kda.kda_chunk_fwd_ex(q, k, v, cu, **common)
    epi, _ = kda.kda_chunk_fwd_ex(q, k, v, cu, **common, **_epilogue_kw(x, bf, norm, z_act))
    torch.cuda.synchronize()
    err = _row_err(gc.host(epi), _epilogue_ref(gc.host(raw), x, norm, z_act))
    print(f"prefill epilogue {dt} norm={norm} z={z_act}: max err / row RMS {err:.2e}")
    assert err <= 1e-5


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("norm,z_act", EPI_CASES)
def test_epilogue_arithmetic_decode(dt, norm, z_act):
    """As above for one decode step (each call on its own copy of the state cache).
    With the norm the decode kernel keeps whole rows in one workgroup, so its column
    sums over d_k are grouped differently from the call without it: a difference of
    the order of the fp32 rounding of those sums, far below the 1e-5 bar."""
    bf = dt == "bf16"
    B, Hk, H, K, V = 16, 2, 4, 128, 128
    x = inputs.option_inputs(33, B, Hk, H, K, V, dt)
    g = (-0.1 * oo.softplus(x["gate_x"])).astype(np.float32)
    b = oo.sigmoid(x["beta_y"]).astype(np.float32)
    state = torch.from_numpy((0.02 * np.random.default_rng(34).standard_normal((B, H, K, V))).astype(np.float32)).cuda()
    q, k, v = _t(x["q"], bf), _t(x["k"], bf), _t(x["v"], bf)
    common = dict(log_alpha=_t(g, False), beta=_t(b, False), out_dtype=torch.float32)
    raw = kda.kda_decode_step_ex(q, k, v, state.clone(), **common)
    epi = kda.kda_decode_step_ex(q, k, v, state.clone(), **common, **_epilogue_kw(x, bf, norm, z_act))
    torch.cuda.synchronize()
    err = _row_err(gc.host(epi), _epilogue_ref(gc.host(raw), x, norm, z_act))
    print(f"decode epilogue {dt} norm={norm} z={z_act}: max err / row RMS {err:.2e}")
    assert err <= 1e-5
