"""Pins of oracle/options.py (the extended entry points' definitions) against
closed forms, invariants and reductions to the plain token-loop oracle."""

import numpy as np
import pytest

import oracle
from oracle import options as op


def _rng(seed):
    return np.random.default_rng(seed)


def test_softplus_closed_forms():
    x = np.concatenate([_rng(0).standard_normal(200) * 10, [0.0, 40.0, -40.0, 700.0, -700.0]])
    sp = op.softplus(x)
    assert op.softplus(0.0) == pytest.approx(np.log(2.0), rel=1e-15)
    np.testing.assert_allclose(sp - op.softplus(-x), x, rtol=0, atol=1e-12)   # softplus(x) - softplus(-x) = x
    assert np.all(sp > 0)
    assert op.softplus(700.0) == 700.0
    assert op.softplus(-40.0) == pytest.approx(np.exp(-40.0), rel=1e-12)     # ln(1 + e^x) ~ e^x
    np.testing.assert_allclose(op.gate_log_alpha(0.0, 0.3), -0.3 * np.log(2.0), rtol=1e-15)
    assert np.all(op.gate_log_alpha(x, 0.1) < 0)


def test_sigmoid_closed_forms():
    y = np.concatenate([_rng(1).standard_normal(200) * 8, [0.0, 800.0, -800.0]])
    s = op.sigmoid(y)
    assert op.sigmoid(0.0) == 0.5
    np.testing.assert_allclose(s + op.sigmoid(-y), 1.0, rtol=0, atol=1e-15)
    m = np.abs(y) < 30
    np.testing.assert_allclose(s[m], np.exp(y[m]) / (1 + np.exp(y[m])), rtol=1e-13)
    assert op.sigmoid(800.0) == 1.0 and op.sigmoid(-800.0) == 0.0


def test_rms_norm_and_output_gate():
    r = _rng(2)
    o = r.standard_normal((5, 3, 64))
    n = op.rms_norm(o, 0.0)
    np.testing.assert_allclose(np.mean(n * n, axis=-1), 1.0, rtol=1e-13)      # unit mean square
    np.testing.assert_allclose(op.rms_norm(7.5 * o, 0.0), n, rtol=1e-13)       # scale invariance
    np.testing.assert_allclose(np.sign(n), np.sign(o))
    c = np.full((1, 1, 64), -3.0)
    np.testing.assert_allclose(op.rms_norm(c, 0.5), -3.0 / np.sqrt(9.5), rtol=1e-15)
    w = r.standard_normal(64)
    np.testing.assert_allclose(op.rms_norm(o, 1e-3, w), op.rms_norm(o, 1e-3) * w, rtol=1e-15)
    np.testing.assert_allclose(op.output_gate(o, np.ones_like(o)), o)
    np.testing.assert_allclose(op.output_gate(o, np.zeros_like(o), "sigmoid"), o / 2)
    assert np.all(op.output_gate(o, np.full_like(o, -800.0), "sigmoid") == 0)


def _inputs(seed, lens, Hk, H, K=16, V=8, s0=True):
    r = _rng(seed)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)

    def unit(x):
        return x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = unit(r.standard_normal((T, Hk, K))).astype(np.float32)
    k = unit(r.standard_normal((T, Hk, K))).astype(np.float32)
    v = r.standard_normal((T, H, V)).astype(np.float32)
    gx = r.standard_normal((T, H, K)).astype(np.float32)
    by = r.standard_normal((T, H)).astype(np.float32)
    # states exactly representable in fp32 (the token loop reads them at fp32)
    st = (0.1 * r.standard_normal((len(lens), H, K, V))).astype(np.float32).astype(np.float64) if s0 else None
    return q, k, v, gx, by, cu, st


def test_grouped_heads_reduce_to_plain_and_to_single_heads():
    q, k, v, gx, by, cu, st = _inputs(3, [9, 14], Hk=2, H=6)
    g = op.gate_log_alpha(gx, 0.1).astype(np.float32)
    b = op.sigmoid(by).astype(np.float32)
    o, sf = op.prefill_ex(q, k, v, cu, log_alpha=g, beta=b, initial_state=st)
    # every value head equals a plain one-head run with its key head's q and k
    for h in range(6):
        hk = h // 3
        oh, sh = oracle.prefill(q[:, hk:hk + 1], k[:, hk:hk + 1], v[:, h:h + 1], g[:, h:h + 1],
                                b[:, h:h + 1], cu, 1.0, st[:, h:h + 1])
        np.testing.assert_array_equal(o[:, h:h + 1], oh)
        np.testing.assert_array_equal(sf[:, h:h + 1], sh)
    # Hk = H is the plain operator
    q2, k2, v2, _, _, cu2, st2 = _inputs(4, [11], Hk=3, H=3)
    g2 = np.full((11, 3, 16), -0.05, np.float32)
    b2 = np.full((11, 3), 0.5, np.float32)
    a = op.prefill_ex(q2, k2, v2, cu2, log_alpha=g2, beta=b2, initial_state=st2)
    p = oracle.prefill(q2, k2, v2, g2, b2, cu2, 1.0, st2)
    np.testing.assert_array_equal(a[0], p[0])
    np.testing.assert_array_equal(a[1], p[1])


def test_gate_preactivation_limits():
    q, k, v, gx, by, cu, st = _inputs(5, [12], Hk=2, H=2)
    # beta -> 0 (beta_y -> -inf): nothing is written; alpha -> 1 (gate_x -> -inf): no decay,
    # so o_t = S_0^T q_t and the state is unchanged
    o, sf = op.prefill_ex(q, k, v, cu, gate_x=np.full_like(gx, -200.0), beta_y=np.full_like(by, -800.0),
                          gate_scale=0.1, initial_state=st)
    s32 = st.astype(np.float32).astype(np.float64)  # the token loop reads states at fp32
    np.testing.assert_allclose(sf, s32, rtol=0, atol=1e-15)
    ref = np.einsum("thk,hkv->thv", q.astype(np.float64), s32[0])
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-14)
    # gate_x = 0: log alpha = -s ln 2 exactly as the plain operator with that gate
    o1, s1 = op.prefill_ex(q, k, v, cu, gate_x=np.zeros_like(gx), beta_y=by, gate_scale=0.2, initial_state=st)
    g = np.full_like(gx, np.float32(-0.2 * np.log(2.0)))
    o2, s2 = oracle.prefill(q, k, v, g, op.sigmoid(by).astype(np.float32), cu, 1.0, st)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_state_slots():
    q, k, v, gx, by, cu, st = _inputs(6, [7, 0, 10], Hk=2, H=2)
    g = op.gate_log_alpha(gx, 0.1).astype(np.float32)
    b = op.sigmoid(by).astype(np.float32)
    cache = (0.1 * _rng(7).standard_normal((5, 2, 16, 8))).astype(np.float32).astype(np.float64)
    slots = np.array([3, 0, 4], np.int32)
    o, out = op.prefill_ex(q, k, v, cu, log_alpha=g, beta=b, state_slots=slots, initial_state=cache)
    o_ref, sf_ref = oracle.prefill(q, k, v, g, b, cu, 1.0, cache[slots])
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(out[slots], sf_ref)
    np.testing.assert_array_equal(out[[1, 2]], cache[[1, 2]])   # other slots untouched
    np.testing.assert_array_equal(out[0], cache[0])             # the empty sequence hands its state through
    # padding: sequence 2 starts from zeros and writes nothing
    pad = np.array([3, 0, -1], np.int32)
    o_p, out_p = op.prefill_ex(q, k, v, cu, log_alpha=g, beta=b, state_slots=pad, initial_state=cache)
    s0 = cache[[3, 0, 0]].copy()
    s0[2] = 0
    o_z, sf_z = oracle.prefill(q, k, v, g, b, cu, 1.0, s0)
    np.testing.assert_array_equal(o_p, o_z)
    np.testing.assert_array_equal(out_p[4], cache[4])
    np.testing.assert_array_equal(out_p[3], sf_z[0])


def test_decode_options():
    r = _rng(8)
    B, Hk, H, K, V = 4, 2, 4, 16, 8
    q = r.standard_normal((B, Hk, K)).astype(np.float32)
    k = (r.standard_normal((B, Hk, K)) / 4).astype(np.float32)
    v = r.standard_normal((B, H, V)).astype(np.float32)
    gx = r.standard_normal((B, H, K)).astype(np.float32)
    by = r.standard_normal((B, H)).astype(np.float32)
    z = r.standard_normal((B, H, V)).astype(np.float32)
    w = r.standard_normal(V)
    state = (0.1 * r.standard_normal((6, H, K, V))).astype(np.float32).astype(np.float64)
    slots = np.array([5, 1, 0, 3], np.int32)
    s_a = state.copy()
    o = op.decode_ex(q, k, v, s_a, slots, gate_x=gx, beta_y=by, gate_scale=0.1, norm=True, norm_eps=1e-5,
                     norm_weight=w, out_gate=z, out_gate_act="sigmoid")
    s_b = state.copy()
    g = op.gate_log_alpha(gx, 0.1).astype(np.float32)
    b = op.sigmoid(by).astype(np.float32)
    o_b = oracle.decode(op.expand_heads(q, H), op.expand_heads(k, H), v, g, b, s_b, slots)
    np.testing.assert_array_equal(s_a, s_b)
    np.testing.assert_allclose(o, op.rms_norm(o_b, 1e-5, w) * op.sigmoid(z), rtol=1e-13)
