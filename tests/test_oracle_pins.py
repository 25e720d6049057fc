"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU. None re-types the oracle's formula: each
checks the oracle against a value derived by hand, a different algebraic form
(exact rational arithmetic of the DPLR transition), a special case with a
known answer, an invariant of the method, or a library routine.
Page references are to the Doubleword page "You Could Have Come Up with Kimi
Delta Attention" (sections 2-6) and the FlashKDA pages.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "two_token_example.md")
RNG = np.random.default_rng(12345)


def _golden():
    text = open(GOLDEN).read()
    body = text.split("```json")[1].split("```")[0]
    return json.loads(body)


def _f(x):
    return float(x) if not isinstance(x, str) else float(x.replace("inf", "inf"))


def _rel(a, b):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(np.asarray(b))), 1e-300)


# ---------------------------------------------------------------- P1 sigmoid
def test_sigmoid_special_values_and_library():
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.sigmoid(math.inf) == 1.0
    assert oracle.sigmoid(-math.inf) == 0.0
    assert oracle.sigmoid(-800.0) == 0.0 and oracle.sigmoid(800.0) == 1.0
    xs = np.linspace(-40, 40, 801)
    ours = np.array([oracle.sigmoid(x) for x in xs])
    assert np.max(np.abs(ours - scipy.special.expit(xs)) / scipy.special.expit(xs)) < 1e-14
    assert np.max(np.abs(ours + np.array([oracle.sigmoid(-x) for x in xs]) - 1.0)) < 1e-15
    assert np.max(np.abs(chunked.sigmoid(xs) - scipy.special.expit(xs)) / scipy.special.expit(xs)) < 1e-14


# ---------------------------------------------------------------- hand-worked example
def test_golden_core_example():
    gd = _golden()
    o, S = oracle.core(gd["q"], gd["k"], gd["v"], gd["alpha"], gd["beta"], gd["S0"], gd["scale"])
    assert np.allclose(o, gd["o"], rtol=0, atol=1e-14)
    assert np.allclose(S, gd["S_T"], rtol=0, atol=1e-14)


def test_golden_full_example_through_activations():
    gd = _golden()
    raw = gd["raw"]
    conv = lambda a: np.array([[float(x) for x in row] for row in a])  # noqa: E731
    q = conv(raw["q"])[:, None, :]
    k = conv(raw["k"])[:, None, :]
    v = np.array(gd["v"])[:, None, :]
    g = conv(raw["g_raw"])[:, None, :]
    b = np.array([float(x) for x in raw["beta_raw"]])[:, None]
    S0 = np.array(gd["S0"], dtype=float)[None, None]
    o, S = oracle.token_forward(q, k, v, g, b, [0, 2], S0, lower_bound=raw["lower_bound"],
                                scale=gd["scale"], eps=0.0)
    assert np.allclose(o[:, 0], gd["o"], rtol=0, atol=1e-14)
    assert np.allclose(S[0, 0], gd["S_T"], rtol=0, atol=1e-14)
    # the chunked form reproduces the same example
    oc, Sc, _ = chunked.forward(q, k, v, g, b, [0, 2], S0, lower_bound=raw["lower_bound"],
                                scale=gd["scale"], eps=0.0)
    assert np.allclose(oc[:, 0], gd["o"], rtol=0, atol=1e-14)
    assert np.allclose(Sc[0, 0], gd["S_T"], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- P2: exact DPLR transition form
def _frac_mat(a):
    return [[Fraction(x) for x in row] for row in a]


def test_exact_rational_dplr_form():
    """Section 4.1: S_t = S_{t-1} A_t + beta_t v_t k_t^T with A_t = D_t - beta_t D_t k_t k_t^T,
    o_t = S_t (s q_t), evaluated in exact rational arithmetic."""
    rng = np.random.default_rng(7)
    T, dk, dv = 5, 3, 2
    rat = lambda *sh: rng.integers(-8, 9, size=sh) / 8.0  # noqa: E731  (exact in binary)
    q, k, v = rat(T, dk), rat(T, dk), rat(T, dv)
    alpha = rng.integers(1, 9, size=(T, dk)) / 8.0
    beta = rng.integers(0, 9, size=T) / 8.0
    S0 = rat(dv, dk)
    s = 0.25
    S = _frac_mat(S0)
    o_exact = []
    for t in range(T):
        kt = [Fraction(x) for x in k[t]]
        at = [Fraction(x) for x in alpha[t]]
        bt = Fraction(beta[t])
        A = [[(at[i] if i == j else 0) - bt * at[i] * kt[i] * kt[j] for j in range(dk)] for i in range(dk)]
        S = [[sum(S[r][m] * A[m][c] for m in range(dk)) + bt * Fraction(v[t][r]) * kt[c] for c in range(dk)]
             for r in range(dv)]
        o_exact.append([sum(S[r][c] * Fraction(s) * Fraction(q[t][c]) for c in range(dk)) for r in range(dv)])
    o, Sf = oracle.core(q, k, v, alpha, beta, S0, s)
    assert np.allclose(o, np.array(o_exact, dtype=float), rtol=0, atol=1e-13)
    assert np.allclose(Sf, np.array(S, dtype=float), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P3, P4: read-back and locality
def _unit(x):
    return x / np.linalg.norm(x)


def test_readback_identity():
    """Section 2.1: after a write at unit key k, S_t k = (1-beta) S~ k + beta v."""
    for _ in range(5):
        dv, dk = 6, 9
        S0 = RNG.standard_normal((dv, dk))
        k = _unit(RNG.standard_normal(dk))
        q = RNG.standard_normal(dk)
        v = RNG.standard_normal(dv)
        a = RNG.uniform(0.05, 1.0, dk)
        b = RNG.uniform(0, 1)
        _, S1 = oracle.core(q[None], k[None], v[None], a[None], [b], S0, 1.0)
        Stilde = S0 * a[None, :]
        assert np.allclose(S1 @ k, (1 - b) * (Stilde @ k) + b * v, rtol=0, atol=1e-13)


def test_write_is_local_in_key_space():
    """Section 2.1: directions orthogonal to the written key are read as before the write."""
    dv, dk = 5, 7
    S0 = RNG.standard_normal((dv, dk))
    k = _unit(RNG.standard_normal(dk))
    x = RNG.standard_normal(dk)
    x -= (x @ k) * k
    a = RNG.uniform(0.1, 1.0, dk)
    _, S1 = oracle.core(np.zeros((1, dk)), k[None], RNG.standard_normal((1, dv)), a[None], [0.7], S0, 1.0)
    assert np.allclose(S1 @ x, (S0 * a[None, :]) @ x, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P5: beta = 0
def test_beta_zero_is_pure_decay():
    """beta = 0: nothing is written, the state only decays channel-wise and
    o_t = s S_0 D_{0:t} qhat_t (section 4 with e = 0)."""
    T, H, D = 12, 2, 16
    q, k, v, g = (RNG.standard_normal((T, H, D)) for _ in range(4))
    b = np.full((T, H), -np.inf)
    S0 = RNG.standard_normal((1, H, D, D))
    lb, s = -5.0, D ** -0.5
    o, S = oracle.token_forward(q, k, v, g, b, [0, T], S0, lower_bound=lb, scale=s, eps=0.0)
    alpha = np.exp(lb * scipy.special.expit(g))  # [T,H,D]
    cum = np.cumprod(alpha, axis=0)
    qhat = q / np.linalg.norm(q, axis=-1, keepdims=True)
    for h in range(H):
        for t in range(T):
            assert np.allclose(o[t, h], s * S0[0, h] @ (cum[t, h] * qhat[t, h]), rtol=1e-12, atol=1e-14)
        assert np.allclose(S[0, h], S0[0, h] * cum[-1, h][None, :], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- P6: exact retrieval
def test_orthonormal_keys_exact_retrieval():
    """alpha = 1, beta = 1, orthonormal keys: every written pair is retrieved exactly,
    S k_i = v_i (sections 2.1, 2.3)."""
    dk, dv = 8, 5
    Q, _ = np.linalg.qr(RNG.standard_normal((dk, dk)))
    keys = Q.T  # rows orthonormal
    vals = RNG.standard_normal((dk, dv))
    S0 = RNG.standard_normal((dv, dk))
    _, S = oracle.core(RNG.standard_normal((dk, dk)), keys, vals, np.ones((dk, dk)), np.ones(dk), S0, 1.0)
    for i in range(dk):
        assert np.allclose(S @ keys[i], vals[i], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P7: DeltaNet and Gated DeltaNet
def test_reduces_to_deltanet_and_gated_deltanet():
    """alpha = 1 is DeltaNet, S_t = S_{t-1}(I - b k k^T) + b v k^T (section 2.3);
    alpha equal across channels is Gated DeltaNet, S_t = a S_{t-1}(I - b k k^T) + b v k^T
    (section 3, expanded form)."""
    T, dk, dv = 20, 6, 4
    keys = np.stack([_unit(RNG.standard_normal(dk)) for _ in range(T)])
    q = RNG.standard_normal((T, dk))
    v = RNG.standard_normal((T, dv))
    b = RNG.uniform(0, 1, T)
    a = RNG.uniform(0.3, 1.0, T)
    S0 = RNG.standard_normal((dv, dk))
    for gated in (False, True):
        alpha = (a[:, None] if gated else np.ones((T, 1))) * np.ones((T, dk))
        o, S = oracle.core(q, keys, v, alpha, b, S0, 0.5)
        R = S0.copy()
        for t in range(T):
            P = np.eye(dk) - b[t] * np.outer(keys[t], keys[t])
            R = (a[t] if gated else 1.0) * R @ P + b[t] * np.outer(v[t], keys[t])
            assert np.allclose(o[t], R @ (0.5 * q[t]), rtol=0, atol=1e-12)
        assert np.allclose(S, R, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P8: chunked == token
def _random_inputs(T, H, D, seed, g_mean=0.0, b_mean=0.0):
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((T, H, D)) for _ in range(3))
    g = r.standard_normal((T, H, D)) + g_mean
    b = r.standard_normal((T, H)) + b_mean
    return q, k, v, g, b


@pytest.mark.parametrize("T", [1, 15, 16, 17, 33, 64])
def test_chunked_equals_token(T):
    """Section 6: the chunkwise form gives exactly the token recurrence's states and outputs."""
    H, D = 2, 128
    q, k, v, g, b = _random_inputs(T, H, D, seed=T)
    S0 = np.random.default_rng(99).standard_normal((1, H, D, D)) * 0.1
    ot, St = oracle.token_forward(q, k, v, g, b, [0, T], S0)
    oc, Sc, _ = chunked.forward(q, k, v, g, b, [0, T], S0)
    assert _rel(oc, ot) < 1e-12
    assert _rel(Sc, St) < 1e-12


def test_chunked_equals_token_varlen_with_empty_sequence():
    lens = [5, 0, 40, 16]
    T = sum(lens)
    offs = np.concatenate([[0], np.cumsum(lens)])
    H, D = 2, 128
    q, k, v, g, b = _random_inputs(T, H, D, seed=5, g_mean=-1.0, b_mean=1.0)
    S0 = np.random.default_rng(3).standard_normal((len(lens), H, D, D)) * 0.02
    ot, St = oracle.token_forward(q, k, v, g, b, offs, S0)
    oc, Sc, _ = chunked.forward(q, k, v, g, b, offs, S0)
    assert _rel(oc, ot) < 1e-12 and _rel(Sc, St) < 1e-12
    assert np.array_equal(St[1], S0[1])  # empty sequence: final = initial


# ---------------------------------------------------------------- P9, P10: streaming, varlen
def test_streaming_split_invariance():
    """Recurrent state passing (instagit FlashKDA summary, streaming example):
    run(T) == run(T1) then run(T - T1) from its final state."""
    T, T1, H, D = 70, 23, 2, 128
    q, k, v, g, b = _random_inputs(T, H, D, seed=11)
    S0 = np.random.default_rng(4).standard_normal((1, H, D, D)) * 0.02
    o, S = oracle.token_forward(q, k, v, g, b, [0, T], S0)
    o1, S1 = oracle.token_forward(q[:T1], k[:T1], v[:T1], g[:T1], b[:T1], [0, T1], S0)
    o2, S2 = oracle.token_forward(q[T1:], k[T1:], v[T1:], g[T1:], b[T1:], [0, T - T1], S1)
    assert _rel(np.concatenate([o1, o2]), o) < 1e-13 and _rel(S2, S) < 1e-13


def test_varlen_equals_independent_sequences():
    """Packed sequences (DocSearch FlashKDA digest, varlen batching) are independent."""
    lens = [7, 30, 1]
    offs = np.concatenate([[0], np.cumsum(lens)])
    H, D = 3, 128
    q, k, v, g, b = _random_inputs(int(offs[-1]), H, D, seed=21)
    o, S = oracle.token_forward(q, k, v, g, b, offs)
    for n, L in enumerate(lens):
        a, e = offs[n], offs[n + 1]
        on, Sn = oracle.token_forward(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], [0, L])
        assert np.array_equal(o[a:e], on) and np.array_equal(S[n], Sn[0])


# ---------------------------------------------------------------- P11: Neumann inverse
def _strict_lower(n, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return np.tril(r.standard_normal((n, n)) * scale, -1)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_neumann_series_is_exact_inverse(seed):
    """FlashKDA deep-dive section 1: the 16x16 inverse by a Neumann series.
    R strictly lower => R^16 = 0 exactly; series, forward substitution
    (section 6.3) and LAPACK agree; so does the doubling product
    (I - R)(I + R^2)(I + R^4)(I + R^8)."""
    R = _strict_lower(16, seed, scale=0.5)
    assert np.count_nonzero(np.linalg.matrix_power(R, 16)) == 0
    ref = np.linalg.inv(np.eye(16) + R)
    neu = chunked.unit_lower_inverse_neumann(R)
    sub = chunked.unit_lower_inverse_substitution(R)
    R2 = R @ R
    R4 = R2 @ R2
    prod = (np.eye(16) - R) @ (np.eye(16) + R2) @ (np.eye(16) + R4) @ (np.eye(16) + R4 @ R4)
    for X in (neu, sub, prod):
        assert _rel(X, ref) < 1e-12


# ---------------------------------------------------------------- P12, P13: linearity, invariances
def test_linear_in_values_and_initial_state():
    T, H, D = 40, 2, 128
    q, k, v, g, b = _random_inputs(T, H, D, seed=31)
    S0 = np.random.default_rng(8).standard_normal((1, H, D, D)) * 0.05
    o, S = oracle.token_forward(q, k, v, g, b, [0, T], S0)
    o3, S3 = oracle.token_forward(q, k, 3.0 * v, g, b, [0, T], 3.0 * S0)
    assert _rel(o3, 3.0 * o) < 1e-13 and _rel(S3, 3.0 * S) < 1e-13
    # superposition in (v, S0)
    v2 = np.random.default_rng(9).standard_normal(v.shape)
    oa, Sa = oracle.token_forward(q, k, v2, g, b, [0, T], np.zeros_like(S0))
    ob, Sb = oracle.token_forward(q, k, v + v2, g, b, [0, T], S0)
    assert _rel(ob, o + oa) < 1e-12 and _rel(Sb, S + Sa) < 1e-12


def test_qk_scale_invariance_and_head_independence():
    T, H, D = 33, 3, 128
    q, k, v, g, b = _random_inputs(T, H, D, seed=41)
    o, S = oracle.token_forward(q, k, v, g, b, [0, T], eps=0.0)
    o2, S2 = oracle.token_forward(4.0 * q, 0.25 * k, v, g, b, [0, T], eps=0.0)
    assert _rel(o2, o) < 1e-13 and _rel(S2, S) < 1e-13
    perm = [2, 0, 1]
    op, Sp = oracle.token_forward(q[:, perm], k[:, perm], v[:, perm], g[:, perm], b[:, perm], [0, T], eps=0.0)
    assert np.array_equal(op, o[:, perm]) and np.array_equal(Sp, S[:, perm])


# ---------------------------------------------------------------- readings of section 6.6 and pages' claims
def test_wy_factor_reading():
    """Reading of section 6.6's WY form: E = U - W S_c^T with U = A^kk Diag(beta) V,
    W = A^kk Diag(beta) K_b, against the literal substitution of section 6.3."""
    T, H, D = 48, 1, 128
    q, k, v, g, b = _random_inputs(T, H, D, seed=51)
    S0 = np.random.default_rng(2).standard_normal((1, H, D, D)) * 0.1
    _, _, inter = chunked.forward(q, k, v, g, b, [0, T], S0, keep=True)
    for it in inter[(0, 0)]:
        assert _rel(it["U"] - it["W"] @ it["S_in"].T, it["E"]) < 1e-11


def test_inverse_entries_bounded_on_workload_distribution():
    """The FlashKDA pages state the entries of (I + R)^-1 lie in [-1, 1]
    (deep-dive section 3). Checked here as a property of seeded inputs drawn like
    the benchmark workloads (not assumed by any kernel)."""
    T, H, D = 512, 2, 128
    worst = 0.0
    for seed, gm, bm in [(61, 0.0, 0.0), (62, -1.0, 0.0), (63, 0.0, 1.0)]:
        q, k, v, g, b = _random_inputs(T, H, D, seed=seed, g_mean=gm, b_mean=bm)
        _, _, inter = chunked.forward(q, k, v, g, b, [0, T], keep=True)
        for lst in inter.values():
            for it in lst:
                worst = max(worst, float(np.max(np.abs(it["Akk"]))))
    assert worst <= 1.0 + 1e-12
