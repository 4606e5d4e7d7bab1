"""CPU tests of the fp64 oracle: its pins, the chunk algebra, and mutants.

Runs without a GPU.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module", autouse=True)
def _built_oracle():
    oracle.build(force=False)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


# --- the chunkwise form the GPU kernels implement ------------------------


def chunk_form(q, k, v, g, b, C, s0=None):
    """Chunkwise-parallel KDA for one (sequence, head), fp64 numpy.

    Within a chunk of n tokens with cumulative log-decay G_r = sum_{s<=r} g_s:
        A = strict_lower(Diag(b) [sum_i k_r[i] k_s[i] e^{G_r[i]-G_s[i]}])
        P = lower_incl([sum_i q_r[i] k_s[i] e^{G_r[i]-G_s[i]}])
        U' = (I + A)^{-1} Diag(b) (V - (K . e^G) S)      (WY / UT transform)
        O  = (Q . e^G) S + P U'
        S  <- Diag(e^{G_n}) S + (K . e^{G_n - G})^T U'
    ("Kimi Linear爆发背后的秘密" page, section "硬件效率的深度优化": chunk-parallel
    inside a chunk, recurrent across chunks, WY representation, UT transform.)
    """
    T, K = q.shape
    V = v.shape[1]
    S = np.zeros((K, V)) if s0 is None else s0.astype(np.float64).copy()
    O = np.zeros((T, V))
    for a in range(0, T, C):
        e = min(a + C, T)
        qc, kc, vc, gc, bc = (x[a:e].astype(np.float64) for x in (q, k, v, g, b))
        n = e - a
        G = np.cumsum(gc, axis=0)
        D = G[:, None, :] - G[None, :, :]  # [r, s, i] = G_r - G_s
        low = np.tril(np.ones((n, n), bool))
        D = np.where(low[:, :, None], D, -np.inf)  # only s <= r is ever used
        E = np.exp(D)
        A = np.tril(bc[:, None] * np.einsum("ri,si,rsi->rs", kc, kc, E), -1)
        P = np.einsum("ri,si,rsi->rs", qc, kc, E)
        X = bc[:, None] * (vc - (kc * np.exp(G)) @ S)
        Up = np.linalg.solve(np.eye(n) + A, X)
        O[a:e] = (qc * np.exp(G)) @ S + P @ Up
        S = np.exp(G[-1])[:, None] * S + (kc * np.exp(G[-1] - G)).T @ Up
    return O, S


@pytest.mark.parametrize("C", [1, 7, 16, 64, 200])
def test_chunk_form_matches_oracle(C):
    T, H, K, V = 150, 2, 16, 12
    q, k, v, g, b, s0 = pins.random_problem(40, T, H, K, V)
    o, sf = oracle.prefill(q, k, v, g, b, [0, T], 1.0, s0)
    for h in range(H):
        O, S = chunk_form(q[:, h], k[:, h], v[:, h], g[:, h], b[:, h], C, s0[0, h])
        assert pins.rel_err(O, o[:, h]) < 1e-12
        assert pins.rel_err(S, sf[0, h]) < 1e-12


# --- mutants: plant a mistake in a copy of the oracle, expect a pin to fail --

MUTANTS = {
    "no_decay": ("s[i] = alpha[i] * s[i];", "s[i] = s[i];"),
    "gate_sign": ("alpha[i] = exp((double)g[bk + i]);",
                  "alpha[i] = exp(-(double)g[bk + i]);"),
    "delta_sign": ("const double u = b * ((double)v[bv + j0 + j] - r);",
                   "const double u = b * ((double)v[bv + j0 + j] + r);"),
    "no_beta": ("const double u = b * ((double)v[bv + j0 + j] - r);",
                "const double u = 1.0 * ((double)v[bv + j0 + j] - r);"),
    "delta_on_undecayed": ("r += s[i] * kk[i];", "r += s[i] / alpha[i] * kk[i];"),
    "read_with_k": ("acc += s[i] * qq[i];", "acc += s[i] * kk[i];"),
    "predict_with_q": ("r += s[i] * kk[i];", "r += s[i] * qq[i];"),
    "no_write": ("s[i] = s[i] + kk[i] * u;", "s[i] = s[i] + 0.0 * u;"),
    "write_with_q": ("s[i] = s[i] + kk[i] * u;", "s[i] = s[i] + qq[i] * u;"),
    "no_scale": ("o[bv + j0 + j] = scale * acc;", "o[bv + j0 + j] = acc;"),
    "state_transposed": ("(double)s0[(size_t)i * V + j0 + j]",
                         "(double)s0[(size_t)(j0 + j) * K + i]"),
    "read_before_write": (
        "            /* S = S' + k_t u^T */\n"
        "            for (int i = 0; i < K; ++i)\n"
        "                s[i] = s[i] + kk[i] * u;\n"
        "            /* o_t[j] = scale * (S^T q_t)_j */\n"
        "            double acc = 0.0;\n"
        "            for (int i = 0; i < K; ++i)\n"
        "                acc += s[i] * qq[i];\n",
        "            double acc = 0.0;\n"
        "            for (int i = 0; i < K; ++i)\n"
        "                acc += s[i] * qq[i];\n"
        "            for (int i = 0; i < K; ++i)\n"
        "                s[i] = s[i] + kk[i] * u;\n"),
    "decode_delta_sign": ("const double u = bt * ((double)v[bv + j] - r);",
                          "const double u = bt * ((double)v[bv + j] + r);"),
    "decode_no_decay": ("const double sd = alpha[i] * S[(size_t)i * V + j];",
                        "const double sd = S[(size_t)i * V + j];"),
    "decode_read_with_k": ("acc += sn * (double)q[bk + i];",
                           "acc += sn * (double)k[bk + i];"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmut.so")
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                           "-o", lib, str(path), "-lm"])
    bad = oracle.load_variant(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(bad)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin detects mutant {name}"


def test_oracle_rejects_bad_arguments():
    q = np.zeros((4, 1, 2), np.float32)
    v = np.zeros((4, 1, 3), np.float32)
    b = np.zeros((4, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.prefill(q, q, v, q, b, [0, 3, 2, 4])  # decreasing offsets
    with pytest.raises(ValueError):
        oracle.prefill(q, q, v, q, b, [0, 5])  # total != T
    st = np.zeros((2, 1, 2, 3))
    with pytest.raises(ValueError):
        oracle.decode(q[:1], q[:1], v[:1], q[:1], b[:1], st, np.array([2], np.int32))
