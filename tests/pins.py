"""Pins of the fp64 oracle: checks against facts the mathematics fixes.

Every check here is computed by a route that does not share the oracle's
arithmetic (a closed form, a different formulation, a brute-force product of
explicit transition matrices, or an invariant of the recurrence), so that a
plausible mistake in the oracle -- a dropped term, a wrong sign or index, a
transposed operand -- fails at least one of them. The functions raise
AssertionError and take the oracle module as an argument, so the mutation
test can run them against deliberately broken builds of the oracle.

The recurrence (row i of S is key channel i):
    S_t = (I - b_t k_t k_t^T) Diag(alpha_t) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t
("Kimi Linear爆发背后的秘密" page, section "Kimi Delta Attention的技术内核"; the
read-out o_t = S_t^T q_t from the 2025 attention review page, section "KLA").
"""

from __future__ import annotations

import numpy as np

TIGHT = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _unit_rows(rng, shape):
    x = rng.standard_normal(shape)
    return _f32(x / np.linalg.norm(x, axis=-1, keepdims=True))


def rel_err(a, b):
    scale = max(float(np.sqrt(np.mean(np.asarray(b, np.float64) ** 2))), 1e-300)
    return float(np.max(np.abs(np.asarray(a, np.float64) - b))) / scale


def random_problem(seed, T, H, K, V, init=True, decay=0.3):
    rng = _rng(seed)
    q = _unit_rows(rng, (T, H, K))
    k = _unit_rows(rng, (T, H, K))
    v = _f32(rng.standard_normal((T, H, V)))
    g = _f32(-decay * np.log1p(np.exp(rng.standard_normal((T, H, K)))))
    b = _f32(1.0 / (1.0 + np.exp(-rng.standard_normal((T, H)))))
    s0 = _f32(0.5 * rng.standard_normal((1, H, K, V))) if init else None
    return q, k, v, g, b, s0


# --- closed forms -------------------------------------------------------


def pin_single_token_zero_state(oracle):
    """T = 1 from S_0 = 0: S_1 = b k v^T, so o = b (q . k) v."""
    rng = _rng(11)
    for K, V in ((1, 1), (3, 5), (16, 8), (64, 64)):
        q = _f32(rng.standard_normal((1, 2, K)))
        k = _f32(rng.standard_normal((1, 2, K)))
        v = _f32(rng.standard_normal((1, 2, V)))
        g = _f32(-np.abs(rng.standard_normal((1, 2, K))))
        b = _f32(rng.uniform(0.1, 1.9, (1, 2)))
        o, sf = oracle.prefill(q, k, v, g, b, [0, 1])
        q64, k64, v64, b64 = (x.astype(np.float64) for x in (q, k, v, b))
        for h in range(2):
            want_o = b64[0, h] * np.dot(q64[0, h], k64[0, h]) * v64[0, h]
            want_s = b64[0, h] * np.outer(k64[0, h], v64[0, h])
            assert rel_err(o[0, h], want_o) < TIGHT, (K, V, h)
            assert rel_err(sf[0, h], want_s) < TIGHT, (K, V, h)


def pin_scale(oracle):
    """The output scale multiplies o only, never the state."""
    q, k, v, g, b, s0 = random_problem(12, 9, 2, 8, 6)
    o1, s1 = oracle.prefill(q, k, v, g, b, [0, 9], 1.0, s0)
    o2, s2 = oracle.prefill(q, k, v, g, b, [0, 9], 0.375, s0)
    assert rel_err(o2, 0.375 * o1) < TIGHT
    assert np.array_equal(s1, s2)


def pin_zero_write(oracle):
    """alpha = 1, beta = 0, S_0 = 0: nothing is ever written, o = 0."""
    q, k, v, g, b, _ = random_problem(13, 17, 2, 8, 8)
    o, sf = oracle.prefill(q, k, v, np.zeros_like(g), np.zeros_like(b), [0, 17])
    assert np.all(o == 0.0) and np.all(sf == 0.0)


def pin_pure_decay(oracle):
    """beta = 0: S_t = Diag(exp(G_t)) S_0 with G_t = sum_{s<=t} g_s, o_t = S_t^T q_t."""
    T, H, K, V = 13, 2, 8, 8  # K == V so a transposed state read fails too
    q, k, v, g, b, s0 = random_problem(14, T, H, K, V)
    o, sf = oracle.prefill(q, k, v, g, np.zeros_like(b), [0, T], 1.0, s0)
    G = np.cumsum(g.astype(np.float64), axis=0)  # [T, H, K]
    S0 = s0[0].astype(np.float64)
    for h in range(H):
        for t in range(T):
            St = np.exp(G[t, h])[:, None] * S0[h]
            assert rel_err(o[t, h], St.T @ q[t, h].astype(np.float64)) < TIGHT
        assert rel_err(sf[0, h], np.exp(G[-1, h])[:, None] * S0[h]) < TIGHT


# --- delta-rule memory --------------------------------------------------


def _retrieval_problem(rng, n, K, V, repeat_last=False):
    """Write n orthonormal keys with alpha = 1, beta = 1, then query them."""
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    keys = _f32(Qm[:, :n].T)  # rows are (float32-rounded) orthonormal keys
    vals = _f32(rng.standard_normal((n, V)))
    wk, wv = list(keys), list(vals)
    if repeat_last:
        newer = _f32(rng.standard_normal(V))
        wk.append(keys[0])
        wv.append(newer)
        vals = vals.copy()
        vals[0] = newer
    W = len(wk)
    T = W + n
    q = np.zeros((T, 1, K), np.float32)
    k = np.zeros((T, 1, K), np.float32)
    v = np.zeros((T, 1, V), np.float32)
    b = np.zeros((T, 1), np.float32)
    k[:W, 0] = wk
    v[:W, 0] = wv
    b[:W, 0] = 1.0
    q[W:, 0] = keys  # query tokens: beta = 0, so they read without writing
    k[W:, 0] = keys
    return q, k, v, np.zeros((T, 1, K), np.float32), b, W, vals


def pin_exact_retrieval(oracle):
    """alpha = 1, beta = 1, orthonormal keys: querying k_i returns v_i."""
    rng = _rng(15)
    for n, K, V in ((1, 4, 3), (5, 8, 6), (16, 16, 16), (40, 64, 32)):
        q, k, v, g, b, W, vals = _retrieval_problem(rng, n, K, V)
        o, _ = oracle.prefill(q, k, v, g, b, [0, q.shape[0]])
        assert rel_err(o[W:, 0], vals) < 1e-5, (n, K, V)


def pin_overwrite(oracle):
    """Writing an already stored key again replaces its value (the delta rule)."""
    rng = _rng(16)
    q, k, v, g, b, W, vals = _retrieval_problem(rng, 6, 8, 5, repeat_last=True)
    o, _ = oracle.prefill(q, k, v, g, b, [0, q.shape[0]])
    assert rel_err(o[W:, 0], vals) < 1e-5


# --- brute force and other formulations ---------------------------------


def pin_dense_transition_products(oracle):
    """S_t = (prod_{s<=t} A_s) S_0 + sum_{s<=t} (prod_{s<r<=t} A_r) b_s k_s v_s^T,
    with A_s = (I - b_s k_s k_s^T) Diag(alpha_s) built as explicit K x K matrices."""
    T, H, K, V = 7, 2, 5, 3
    q, k, v, g, b, s0 = random_problem(17, T, H, K, V, decay=0.8)
    q64, k64, v64, g64, b64 = (x.astype(np.float64) for x in (q, k, v, g, b))
    o, sf = oracle.prefill(q, k, v, g, b, [0, T], 1.0, s0)
    for h in range(H):
        A = [(np.eye(K) - b64[s, h] * np.outer(k64[s, h], k64[s, h]))
             @ np.diag(np.exp(g64[s, h])) for s in range(T)]
        for t in range(T):
            P = np.eye(K)
            for s in range(t + 1):
                P = A[s] @ P
            St = P @ s0[0, h].astype(np.float64)
            for s in range(t + 1):
                M = np.eye(K)
                for r in range(s + 1, t + 1):
                    M = A[r] @ M
                St = St + M @ (b64[s, h] * np.outer(k64[s, h], v64[s, h]))
            assert rel_err(o[t, h], St.T @ q64[t, h]) < 1e-11, (h, t)
        assert rel_err(sf[0, h], St) < 1e-11


def pin_gated_deltanet_orientation(oracle):
    """A channel-constant gate reduces KDA to Gated DeltaNet. Written in the
    value-by-key orientation S~_t = S~_{t-1} (a_t (I - b_t k_t k_t^T)) + b_t v_t k_t^T,
    o_t = S~_t q_t (2025 attention review page, section "GatedDeltaNet解读"),
    S~ must be the transpose of the oracle's state. a = 1 is DeltaNet."""
    T, H, K, V = 11, 3, 6, 4
    q, k, v, g, b, s0 = random_problem(18, T, H, K, V)
    for gate in ("scalar", "one"):
        if gate == "scalar":
            gs = _f32(-np.abs(np.random.default_rng(19).standard_normal((T, H, 1))) * 0.4)
            gg = np.repeat(gs, K, axis=2)
        else:
            gg = np.zeros((T, H, K), np.float32)
        o, sf = oracle.prefill(q, k, v, gg, b, [0, T], 1.0, s0)
        for h in range(H):
            St = s0[0, h].astype(np.float64).T  # V x K
            for t in range(T):
                a = np.exp(np.float64(gg[t, h, 0]))
                kt, vt, qt = (x[t, h].astype(np.float64) for x in (k, v, q))
                St = St @ (a * (np.eye(K) - b[t, h] * np.outer(kt, kt))) \
                    + b[t, h] * np.outer(vt, kt)
                assert rel_err(o[t, h], St @ qt) < 1e-12, (gate, h, t)
            assert rel_err(sf[0, h], St.T) < 1e-12


def pin_scalar_key(oracle):
    """K = 1: s_t = (1 - b_t k_t^2) alpha_t s_{t-1} + b_t k_t v_t (a row vector), o_t = q_t s_t."""
    T, V = 20, 5
    rng = _rng(20)
    q = _f32(rng.standard_normal((T, 1, 1)))
    k = _f32(rng.uniform(-1, 1, (T, 1, 1)))
    v = _f32(rng.standard_normal((T, 1, V)))
    g = _f32(-rng.uniform(0, 0.5, (T, 1, 1)))
    b = _f32(rng.uniform(0, 1, (T, 1)))
    s0 = _f32(rng.standard_normal((1, 1, 1, V)))
    o, sf = oracle.prefill(q, k, v, g, b, [0, T], 1.0, s0)
    s = s0[0, 0, 0].astype(np.float64)
    for t in range(T):
        kt, bt = np.float64(k[t, 0, 0]), np.float64(b[t, 0])
        s = (1.0 - bt * kt * kt) * np.exp(np.float64(g[t, 0, 0])) * s + bt * kt * v[t, 0]
        assert rel_err(o[t, 0], np.float64(q[t, 0, 0]) * s) < 1e-12
    assert rel_err(sf[0, 0, 0], s) < 1e-12


# --- invariants ---------------------------------------------------------


def pin_linearity(oracle):
    """(o, S_T) is linear in (v, S_0) jointly for fixed (q, k, alpha, beta)."""
    T, H, K, V = 15, 2, 8, 7
    q, k, v1, g, b, s01 = random_problem(21, T, H, K, V)
    _, _, v2, _, _, s02 = random_problem(22, T, H, K, V)
    # dyadic values with few significant bits, so v1 + v2 and S01 + S02 are
    # exact in the float32 containers the oracle reads
    v1, v2, s01, s02 = (_f32(np.round(x * 64.0) / 64.0) for x in (v1, v2, s01, s02))
    o1, f1 = oracle.prefill(q, k, v1, g, b, [0, T], 1.0, s01)
    o2, f2 = oracle.prefill(q, k, v2, g, b, [0, T], 1.0, s02)
    o3, f3 = oracle.prefill(q, k, v1 + v2, g, b, [0, T], 1.0, s01 + s02)
    assert rel_err(o3, o1 + o2) < TIGHT and rel_err(f3, f1 + f2) < TIGHT
    o4, f4 = oracle.prefill(q, k, 2 * v1, g, b, [0, T], 1.0, 2 * s01)
    assert rel_err(o4, 2 * o1) < TIGHT and rel_err(f4, 2 * f1) < TIGHT


def pin_state_split(oracle):
    """Running [0, T) equals [0, t) followed by [t, T) from the saved state."""
    T, H, K, V = 23, 2, 8, 8
    q, k, v, g, b, s0 = random_problem(23, T, H, K, V)
    o, sf = oracle.prefill(q, k, v, g, b, [0, T], 1.0, s0)
    for t in (1, 9, 22):
        oa, sa = oracle.prefill(q[:t], k[:t], v[:t], g[:t], b[:t], [0, t], 1.0, s0)
        # the intermediate state is handed over through float32 containers,
        # so the second half agrees to float32 rounding of that state
        ob, sb = oracle.prefill(q[t:], k[t:], v[t:], g[t:], b[t:], [0, T - t], 1.0,
                                sa.astype(np.float32))
        assert rel_err(oa, o[:t]) < TIGHT
        assert rel_err(ob, o[t:]) < 1e-6 and rel_err(sb, sf) < 1e-6


def pin_varlen_equals_separate(oracle):
    """Packed sequences are independent: equal to one call per sequence."""
    H, K, V = 2, 8, 4
    lens = [5, 0, 12, 1, 7]
    T = sum(lens)
    q, k, v, g, b, _ = random_problem(24, T, H, K, V)
    s0 = _f32(np.random.default_rng(25).standard_normal((len(lens), H, K, V)))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, sf = oracle.prefill(q, k, v, g, b, cu, 1.0, s0)
    for n, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        on, sn = oracle.prefill(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], [0, e - a],
                                1.0, s0[n:n + 1])
        assert np.array_equal(on, o[a:e]) and np.array_equal(sn[0], sf[n])
    assert np.array_equal(sf[1], s0[1].astype(np.float64))  # empty sequence


def pin_decode_equals_prefill(oracle):
    """T decode steps on a state cache equal one prefill of T tokens, per slot."""
    T, B, H, K, V = 6, 3, 2, 8, 5
    rng = _rng(26)
    q, k, v, g, b, _ = random_problem(27, T * B, H, K, V)
    q, k, v, g = (x.reshape(T, B, H, -1) for x in (q, k, v, g))
    b = b.reshape(T, B, H)
    slots = np.array([4, 0, 2], np.int32)
    s0 = _f32(rng.standard_normal((5, H, K, V)))
    state = s0.astype(np.float64)
    outs = np.stack([oracle.decode(q[t], k[t], v[t], g[t], b[t], state, slots)
                     for t in range(T)])
    for i, s in enumerate(slots):
        o, sf = oracle.prefill(q[:, i], k[:, i], v[:, i], g[:, i], b[:, i], [0, T],
                               1.0, s0[s:s + 1])
        assert rel_err(outs[:, i], o) < TIGHT
        assert rel_err(state[s], sf[0]) < TIGHT
    for s in (1, 3):  # untouched slots
        assert np.array_equal(state[s], s0[s].astype(np.float64))


def pin_decode_closed_forms(oracle):
    """Decode from a zero slot: o = b (q . k) v and S = b k v^T. Decode with
    b = 0: S = Diag(alpha) S_0 and o = S^T q."""
    B, H, K, V = 2, 3, 8, 6
    rng = _rng(29)
    q, k, v, g, b, _ = random_problem(30, B, H, K, V)
    state = np.zeros((B, H, K, V))
    o = oracle.decode(q, k, v, g, b, state)
    q64, k64, v64, b64, g64 = (x.astype(np.float64) for x in (q, k, v, b, g))
    for i in range(B):
        for h in range(H):
            assert rel_err(o[i, h], b64[i, h] * (q64[i, h] @ k64[i, h]) * v64[i, h]) < TIGHT
            assert rel_err(state[i, h], b64[i, h] * np.outer(k64[i, h], v64[i, h])) < TIGHT
    s0 = rng.standard_normal((B, H, K, V))
    state = s0.copy()
    o = oracle.decode(q, k, v, g, np.zeros_like(b), state)
    want = np.exp(g64)[..., None] * s0
    assert rel_err(state, want) < TIGHT
    assert rel_err(o, np.einsum("bhkv,bhk->bhv", want, q64)) < TIGHT


def pin_contraction_bound(oracle):
    """|k| = 1, beta in [0,1], alpha in (0,1]: A_t is a contraction, so
    ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||."""
    T, K, V = 40, 8, 6
    q, k, v, g, b, s0 = random_problem(28, T, 1, K, V)
    prev = float(np.linalg.norm(s0[0, 0]))
    for t in range(T):
        _, sf = oracle.prefill(q[:t + 1], k[:t + 1], v[:t + 1], g[:t + 1], b[:t + 1],
                               [0, t + 1], 1.0, s0)
        cur = float(np.linalg.norm(sf[0, 0]))
        assert cur <= prev + float(b[t, 0]) * float(np.linalg.norm(v[t, 0])) + 1e-9
        prev = cur


def load_worked_example(name="worked_3tok_dk2.json", scaled=False):
    """A hand-derived example under tests/golden/ (exact fractions), as arrays:
    q, k, v, log_alpha [T, 1, dim], beta [T, 1], initial state [1, 1, K, V],
    expected o [T, 1, V] and final state [1, 1, K, V]; with `scaled`, also the
    read-out scale and the expected o at that scale (appended)."""
    import json
    import os
    from fractions import Fraction
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    with open(path, encoding="utf-8") as f:
        ex = json.load(f)
    num = lambda x: float(Fraction(x))
    toks = ex["tokens"]
    arr = lambda key: np.array([[num(x) for x in t[key]] for t in toks])[:, None, :]
    beta = np.array([[num(t["beta"])] for t in toks])
    s0 = np.array([[num(x) for x in row] for row in ex["initial_state"]])[None, None]
    o = np.array([[num(x) for x in row] for row in ex["expected"]["o"]])[:, None, :]
    sT = np.array([[num(x) for x in row] for row in ex["expected"]["final_state"]])[None, None]
    out = (arr("q"), arr("k"), arr("v"), np.log(arr("alpha")), beta, s0, o, sT)
    if scaled:
        o_s = np.array([[num(x) for x in row] for row in ex["scaled"]["o"]])[:, None, :]
        out = out + (num(ex["scaled"]["scale"]), o_s)
    return out


def pin_worked_example(oracle):
    """Prefill and decode reproduce the hand-derived worked example, at scale 1
    and at its read-out scale 1/2 (the gates reach the oracle as fp32 log alpha:
    compared to a few fp32 ulps)."""
    q, k, v, g, b, s0, o_ref, s_ref, sc, o_sc = load_worked_example(scaled=True)
    T = q.shape[0]
    for scale, o_exp in ((1.0, o_ref), (sc, o_sc)):
        o, sT = oracle.prefill(q, k, v, g, b, [0, T], scale, s0)
        assert np.abs(o - o_exp).max() < 1e-6 and np.abs(sT - s_ref).max() < 1e-6
        state = np.array(s0[0][None], dtype=np.float64)  # a copy: decode updates it in place
        for t in range(T):
            od = oracle.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], state, scale=scale)
            assert np.abs(od[0] - o_exp[t]).max() < 1e-6
        assert np.abs(state - s_ref).max() < 1e-6


ALL_PINS = [
    pin_single_token_zero_state, pin_scale, pin_zero_write, pin_pure_decay,
    pin_exact_retrieval, pin_overwrite, pin_dense_transition_products,
    pin_gated_deltanet_orientation, pin_scalar_key, pin_linearity,
    pin_state_split, pin_varlen_equals_separate, pin_decode_equals_prefill,
    pin_decode_closed_forms, pin_contraction_bound, pin_worked_example,
]
