"""CPU tests of the seeded input generators."""

import hashlib

import numpy as np

from gated_delta_rule_10_amd import inputs


def _digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_bf16_round_is_rne():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-39, 65504.0], np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    want = np.array([1.0, 1.0, 1.015625, -2.5, 3.0e-39, 65536.0], np.float32)
    got = inputs.bf16_round(x)
    assert np.array_equal(got[[0, 1, 2, 3, 5]], want[[0, 1, 2, 3, 5]])
    assert np.array_equal(inputs.bf16_round(got), got)
    assert np.array_equal(inputs.bf16_bits(np.array([1.0], np.float32)),
                          np.array([0x3F80], np.uint16))


def test_generator_is_deterministic_and_distributed():
    a = inputs.prefill_inputs(7, [100, 28], 2, 64, 32, "bf16", 0.1, "odd_zero")
    b = inputs.prefill_inputs(7, [100, 28], 2, 64, 32, "bf16", 0.1, "odd_zero")
    assert _digest(a.q, a.k, a.v, a.log_alpha, a.beta, a.initial_state) == \
        _digest(b.q, b.k, b.v, b.log_alpha, b.beta, b.initial_state)
    assert list(a.cu_seqlens) == [0, 100, 128]
    assert np.array_equal(inputs.bf16_round(a.q), a.q)
    nq = np.linalg.norm(a.q.astype(np.float64), axis=-1)
    assert np.all(np.abs(nq - 1) < 1e-2)  # unit norm before the bf16 cast
    alpha = np.exp(a.log_alpha.astype(np.float64))
    assert np.all(alpha > 0) and np.all(alpha < 1)
    assert 0.85 < alpha.mean() < 0.97
    assert np.all(a.beta > 0) and np.all(a.beta < 1)
    assert np.all(a.initial_state[1] == 0) and np.any(a.initial_state[0] != 0)
    assert abs(a.initial_state[0].std() - 0.02) < 0.002


def test_varlen_lengths_sum_exactly():
    rng = np.random.default_rng(4)
    lens = inputs.varlen_lengths(rng, 16, 1024, 65536, 524288)
    assert lens.sum() == 524288 and len(lens) == 16 and lens.min() > 0


def test_workload_table():
    w = inputs.WORKLOADS
    assert w["long_128k"]["lengths"] == [131072] and w["long_128k"]["H"] == 32
    assert w["decode_b64"]["B"] == 64 and w["decode_b64"]["steps"] == 1000
    t = inputs.workload_inputs("tiny_f32")
    assert t.q.shape == (256, 2, 64) and t.in_dtype == "f32" and t.initial_state is None
    d = inputs.workload_inputs("decode_b64", steps=2)
    assert d.q.shape == (2, 64, 32, 128) and d.state.shape == (64, 32, 128, 128)
