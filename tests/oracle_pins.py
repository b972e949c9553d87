"""Pins of the CPU oracle: checks against what the page and the mathematics fix.

Each pin takes the oracle module and raises AssertionError if it disagrees. The pins
never re-type the oracle's own formula: they use closed forms, invariants, hand-worked
golden values, finite differences and a pure-Python brute force. tests/test_oracle_pins.py
runs them on the oracle; tests/test_oracle_mutants.py plants plausible mistakes in the
oracle and checks that at least one pin fails for each.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _read_golden(name):
    fields = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            rows = [[float(Fraction(t)) for t in r.split()] for r in val.split(";")]
            fields[key.strip()] = np.array(rows if len(rows) > 1 else rows[0])
    return fields


def _tables(seed, T, H=1):
    r = _rng(seed)
    alpha = 0.5 * r.standard_normal((H, T))
    alpha[:, 0] = 4.0
    rho = -0.5 * np.log1p(np.arange(T))[None, :] + 0.1 * r.standard_normal((H, T))
    return alpha, rho


# ---------------------------------------------------------------- frozen pattern, Eq. (3)

def pin_frozen_rows_and_causality(orc):
    """Rows of P-hat sum to 1 and every weight with j > i is exactly 0 (Eq. (3))."""
    alpha, rho = _tables(1, 96)
    P, _ = orc.frozen_probs(alpha[0], rho[0])
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-14
    assert np.all(P[np.triu_indices(96, 1)] == 0.0)
    assert np.all(P[np.tril_indices(96)] > 0.0)


def pin_frozen_golden_T3(orc):
    """Hand-worked 3x3 pattern (tests/golden/frozen_T3.txt)."""
    g = _read_golden("frozen_T3.txt")
    P, logZ = orc.frozen_probs(np.log(g["exp_alpha"]), np.log(g["exp_rho"]))
    assert np.max(np.abs(P - g["P"])) < 1e-15
    assert np.max(np.abs(logZ - np.log(g["Z"]))) < 1e-15


def pin_frozen_uniform(orc):
    """alpha = rho = 0: P(i,j) = 1/(i+1) ('1/i' 1-indexed), O = prefix mean, dV by reverse cumsum."""
    B, H, T, D = 2, 2, 40, 5
    r = _rng(2)
    v, do = r.standard_normal((B, H, T, D)), r.standard_normal((B, H, T, D))
    z = np.zeros((H, T))
    frozen = np.ones(H, np.uint8)
    O, lse = orc.attn_fwd(None, None, v, frozen, z, z, 0.5)
    cnt = np.arange(1, T + 1)[None, None, :, None]
    assert np.max(np.abs(O - np.cumsum(v, axis=2) / cnt)) < 1e-13
    assert np.max(np.abs(lse - np.log(np.arange(1, T + 1))[None, None])) < 1e-13
    _, _, dv = orc.attn_bwd(None, None, v, do, frozen, z, z, 0.5)
    ref = np.cumsum((do / cnt)[:, :, ::-1], axis=2)[:, :, ::-1]
    assert np.max(np.abs(dv - ref)) < 1e-13


def pin_frozen_rho_zero(orc):
    """rho = 0: O = cumsum(e^alpha V) / cumsum(e^alpha)."""
    T, D = 33, 3
    r = _rng(3)
    alpha = r.standard_normal((1, T))
    v = r.standard_normal((1, 1, T, D))
    O, _ = orc.attn_fwd(None, None, v, np.ones(1, np.uint8), alpha, np.zeros((1, T)), 1.0)
    ea = np.exp(alpha[0])[:, None]
    ref = np.cumsum(ea * v[0, 0], axis=0) / np.cumsum(ea, axis=0)
    assert np.max(np.abs(O[0, 0] - ref)) < 1e-13


def pin_frozen_identity(orc):
    """rho(0) = 0, rho(d >= 1) = -inf: P = I, so O = V and dV = dO."""
    T, D = 20, 4
    r = _rng(4)
    alpha = r.standard_normal((1, T))
    rho = np.full((1, T), -np.inf)
    rho[0, 0] = 0.0
    v, do = r.standard_normal((1, 1, T, D)), r.standard_normal((1, 1, T, D))
    f = np.ones(1, np.uint8)
    O, lse = orc.attn_fwd(None, None, v, f, alpha, rho, 1.0)
    _, _, dv = orc.attn_bwd(None, None, v, do, f, alpha, rho, 1.0)
    assert np.max(np.abs(O - v)) < 1e-15 and np.max(np.abs(dv - do)) < 1e-15
    assert np.max(np.abs(lse[0, 0] - alpha[0])) < 1e-15


def pin_frozen_shift_invariance(orc):
    """alpha + c1 and rho + c2 leave P-hat unchanged (c = +80 overflows a naive float32 exp)."""
    alpha, rho = _tables(5, 64)
    P0, lz0 = orc.frozen_probs(alpha[0], rho[0])
    P1, lz1 = orc.frozen_probs(alpha[0] + 80.0, rho[0] + 80.0)
    assert np.max(np.abs(P1 - P0)) < 1e-13
    assert np.max(np.abs(lz1 - lz0 - 160.0)) < 1e-11


def pin_frozen_equals_dynamic(orc):
    """Affine rho(d) = -lam d makes Eq. (3) an ordinary softmax head with rank-1 q, k:
    q_i = e0 / scale, k_j = (alpha(j) + lam j) e0 gives S_ij = alpha(j) + lam j, which differs
    from alpha(j) + rho(i-j) by the row constant -lam i."""
    T, D, lam = 48, 4, 0.37
    scale = 1.0 / math.sqrt(D)
    r = _rng(6)
    alpha = r.standard_normal((1, T))
    rho = -lam * np.arange(T)[None, :]
    q = np.zeros((1, 1, T, D)); q[..., 0] = 1.0 / scale
    k = np.zeros((1, 1, T, D)); k[0, 0, :, 0] = alpha[0] + lam * np.arange(T)
    v, do = r.standard_normal((1, 1, T, D)), r.standard_normal((1, 1, T, D))
    Of, lf = orc.attn_fwd(q, k, v, np.ones(1, np.uint8), alpha, rho, scale)
    Od, ld = orc.attn_fwd(q, k, v, np.zeros(1, np.uint8), alpha, rho, scale)
    assert np.max(np.abs(Of - Od)) < 1e-12
    assert np.max(np.abs((ld - lf) - (-lam) * -np.arange(T))) < 1e-10
    _, _, dvf = orc.attn_bwd(q, k, v, do, np.ones(1, np.uint8), alpha, rho, scale)
    _, _, dvd = orc.attn_bwd(q, k, v, do, np.zeros(1, np.uint8), alpha, rho, scale)
    assert np.max(np.abs(dvf - dvd)) < 1e-12


# ---------------------------------------------------------------- ordinary head

def pin_dynamic_golden_T3(orc):
    """Hand-worked 3x3 softmax (tests/golden/dynamic_T3.txt)."""
    g = _read_golden("dynamic_T3.txt")
    q = np.ones((3, 1))
    k = np.log(g["exp_k"])[:, None]
    A, lse = orc.dynamic_probs(q, k, 1.0)
    assert np.max(np.abs(A - g["A"])) < 1e-15
    assert np.max(np.abs(lse - np.log(g["sum_exp"]))) < 1e-15


def pin_dynamic_q_zero(orc):
    """Q = 0: uniform causal weights, O = prefix mean, lse = log(i+1)."""
    B, H, T, D = 1, 2, 30, 6
    r = _rng(7)
    k, v = r.standard_normal((B, H, T, D)), r.standard_normal((B, H, T, D))
    O, lse = orc.attn_fwd(np.zeros_like(k), k, v, np.zeros(H, np.uint8), None, None, 0.4)
    assert np.max(np.abs(O - np.cumsum(v, 2) / np.arange(1, T + 1)[None, None, :, None])) < 1e-13
    assert np.max(np.abs(lse - np.log(np.arange(1, T + 1)))) < 1e-13


def pin_brute_force(orc):
    """Vectorised oracle equals the pure-Python loops (oracle/brute.py) at T <= 16."""
    from oracle import brute
    r = _rng(8)
    for T in (1, 5, 16):
        D, H = 3, 2
        q, k, v = (r.standard_normal((1, H, T, D)) for _ in range(3))
        alpha, rho = r.standard_normal((H, T)), r.standard_normal((H, T))
        frozen = np.array([0, 1], np.uint8)
        O, lse = orc.attn_fwd(q, k, v, frozen, alpha, rho, 0.7)
        bo, bl = brute.dynamic_head(q[0, 0], k[0, 0], v[0, 0], 0.7)
        assert np.max(np.abs(O[0, 0] - np.array(bo))) < 1e-13
        assert np.max(np.abs(lse[0, 0] - np.array(bl))) < 1e-13
        fo, fl, _ = brute.frozen_head(alpha[1], rho[1], v[0, 1])
        assert np.max(np.abs(O[0, 1] - np.array(fo))) < 1e-13
        assert np.max(np.abs(lse[0, 1] - np.array(fl))) < 1e-13


def _fd_grad(f, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + eps
        fp = f()
        x[idx] = old - eps
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * eps)
    return g


def pin_gradients_finite_difference(orc):
    """dQ, dK, dV of <dO, O> against central differences (T=8, D=4), relative error <= 1e-7;
    frozen heads: dV only, dQ and dK are not produced."""
    B, H, T, D = 1, 2, 8, 4
    scale = 1.0 / math.sqrt(D)
    r = _rng(9)
    q, k, v, do = (r.standard_normal((B, H, T, D)) for _ in range(4))
    alpha, rho = r.standard_normal((H, T)), r.standard_normal((H, T))
    frozen = np.array([0, 1], np.uint8)

    def loss():
        return float((orc.attn_fwd(q, k, v, frozen, alpha, rho, scale)[0] * do).sum())

    dq, dk, dv = orc.attn_bwd(q, k, v, do, frozen, alpha, rho, scale)
    for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
        num = _fd_grad(loss, x)
        heads = [0] if name != "dv" else [0, 1]
        for h in heads:
            err = np.max(np.abs(g[:, h] - num[:, h])) / np.max(np.abs(num[:, h]))
            assert err < 1e-7, (name, h, err)
    assert np.all(np.isnan(dq[:, 1])) and np.all(np.isnan(dk[:, 1]))
    # a frozen head's output does not depend on its q, k at all
    num_q = _fd_grad(loss, q)
    assert np.max(np.abs(num_q[:, 1])) == 0.0


def pin_gqa_equals_repeated_heads(orc):
    """Grouped-query attention (shared K/V, part 二.4) is ordinary attention on K and V
    repeated for each query head of a group; the shared K and V receive the sum of the
    repeated copies' gradients (dK only from ordinary heads, NaN for a group of frozen heads
    only)."""
    B, T, D = 2, 9, 4
    scale = 0.5
    r = _rng(21)
    for H, H_kv, frozen in ((4, 2, [0, 1, 1, 1]), (6, 2, [1, 0, 0, 1, 0, 1]), (3, 1, [0, 1, 0])):
        G = H // H_kv
        frozen = np.array(frozen, np.uint8)
        q, do = r.standard_normal((B, H, T, D)), r.standard_normal((B, H, T, D))
        k, v = r.standard_normal((B, H_kv, T, D)), r.standard_normal((B, H_kv, T, D))
        alpha, rho = r.standard_normal((H, T)), r.standard_normal((H, T))
        kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
        O, lse = orc.attn_fwd(q, k, v, frozen, alpha, rho, scale)
        O_r, lse_r = orc.attn_fwd(q, kr, vr, frozen, alpha, rho, scale)
        assert np.max(np.abs(O - O_r)) < 1e-13 and np.max(np.abs(lse - lse_r)) < 1e-13
        dq, dk, dv = orc.attn_bwd(q, k, v, do, frozen, alpha, rho, scale)
        dq_r, dk_r, dv_r = orc.attn_bwd(q, kr, vr, do, frozen, alpha, rho, scale)
        assert np.array_equal(np.isnan(dq), np.isnan(dq_r))
        assert np.nanmax(np.abs(dq - dq_r)) < 1e-13
        for g in range(H_kv):
            heads = range(g * G, (g + 1) * G)
            want_v = sum(dv_r[:, h] for h in heads)
            assert np.max(np.abs(dv[:, g] - want_v)) < 1e-12
            ordinary = [h for h in heads if not frozen[h]]
            if ordinary:
                want_k = sum(dk_r[:, h] for h in ordinary)
                assert np.max(np.abs(dk[:, g] - want_k)) < 1e-12
            else:
                assert np.all(np.isnan(dk[:, g]))


def pin_gqa_gradients_finite_difference(orc):
    """dK and dV of shared key/value heads against central differences of <dO, O>
    (H = 4 query heads over 2 shared heads, one frozen head in each group)."""
    B, H, H_kv, T, D = 1, 4, 2, 6, 3
    scale = 0.7
    r = _rng(22)
    q, do = r.standard_normal((B, H, T, D)), r.standard_normal((B, H, T, D))
    k, v = r.standard_normal((B, H_kv, T, D)), r.standard_normal((B, H_kv, T, D))
    alpha, rho = r.standard_normal((H, T)), r.standard_normal((H, T))
    frozen = np.array([0, 1, 1, 0], np.uint8)

    def loss():
        return float((orc.attn_fwd(q, k, v, frozen, alpha, rho, scale)[0] * do).sum())

    dq, dk, dv = orc.attn_bwd(q, k, v, do, frozen, alpha, rho, scale)
    for name, x, g in (("dk", k, dk), ("dv", v, dv), ("dq", q, dq)):
        num = _fd_grad(loss, x)
        sel = (slice(None), [0, 3]) if name == "dq" else (slice(None),)
        err = np.max(np.abs(g[sel] - num[sel])) / np.max(np.abs(num[sel]))
        assert err < 1e-7, (name, err)


# ---------------------------------------------------------------- calibration, Eq. (1)

def pin_var_identical_inputs(orc):
    """N identical sequences: A-hat equals every A^(n) and s_var = 0 (up to fp64 rounding)."""
    r = _rng(10)
    N, H, T, D = 5, 2, 24, 4
    q1, k1 = r.standard_normal((1, H, T, D)), r.standard_normal((1, H, T, D))
    q, k = np.repeat(q1, N, 0), np.repeat(k1, N, 0)
    A_hat, s_var, _ = orc.var_score(q, k, 0.5)
    assert np.max(s_var) < 1e-30
    for h in range(H):
        A, _ = orc.dynamic_probs(q1[0, h], k1[0, h], 0.5)
        assert np.max(np.abs(A_hat[h] - A)) < 1e-15


def pin_var_q_zero(orc):
    """Q = 0: every A^(n) is uniform causal, so A-hat(i,j) = 1/(i+1) and s_var = 0."""
    r = _rng(11)
    N, H, T, D = 4, 1, 17, 3
    k = r.standard_normal((N, H, T, D))
    A_hat, s_var, _ = orc.var_score(np.zeros_like(k), k, 1.0)
    ref = np.tril(np.ones((T, T))) / np.arange(1, T + 1)[:, None]
    assert np.max(np.abs(A_hat[0] - ref)) < 1e-15 and s_var[0] < 1e-30


def pin_var_T2_closed_form(orc):
    """T = 2: row 0 is [1, 0]; row 1 is [a_n, 1 - a_n] with a_n = sigmoid(scale q1 (k0 - k1)),
    so Eq. (1) reduces to s_var = (sample variance of a_n) / 2."""
    r = _rng(12)
    N, D, scale = 9, 3, 0.8
    q, k = r.standard_normal((N, 1, 2, D)), r.standard_normal((N, 1, 2, D))
    _, s_var, _ = orc.var_score(q, k, scale)
    a = 1.0 / (1.0 + np.exp(-scale * np.einsum("nd,nd->n", q[:, 0, 1], k[:, 0, 0] - k[:, 0, 1])))
    assert abs(s_var[0] - np.var(a, ddof=1) / 2) < 1e-15


def pin_kl_score_closed_forms(orc):
    """s^KL: 0 for identical inputs; the T = 2 closed form (row 0 is always [1]; row 1 is
    (a_n, 1 - a_n) against the mean (a, 1 - a)) written with math.log; scipy's rel_entr on a
    random stack; non-negative (Jensen)."""
    from scipy.special import rel_entr
    r = _rng(31)
    N, T = 5, 2
    a = r.uniform(0.05, 0.95, N)
    stack = np.zeros((N, T, T))
    stack[:, 0, 0] = 1.0
    stack[:, 1, 0], stack[:, 1, 1] = a, 1 - a
    s_kl, _ = orc.kl_score_of(stack)
    ab = sum(a) / N
    want = sum(x * math.log(x / ab) + (1 - x) * math.log((1 - x) / (1 - ab)) for x in a) / (N * T)
    assert abs(s_kl - want) < 1e-15
    same, _ = orc.kl_score_of(np.repeat(stack[:1], 4, axis=0))
    assert same == 0.0
    N, T = 6, 11
    E = np.tril(r.uniform(0.0, 1.0, (N, T, T)))
    E[:, 3, 1] = 0.0   # a zero weight in every sequence
    A = E / E.sum(axis=2, keepdims=True)
    s_kl, A_hat = orc.kl_score_of(A)
    ref = sum(rel_entr(A[n], A_hat).sum() for n in range(N)) / (N * T)
    assert abs(s_kl - ref) < 1e-14 and s_kl > 0


def pin_kl_score_through_qk(orc):
    """The wrapper kl_score(q, k, scale) (part 二.1, the s^KL selector): at T = 5 with three
    sequences and two heads, every attention row is formed in pure Python (math.exp over
    scale * q_i . k_j for j <= i), averaged into A-hat, and the score summed as
    (1/(N T)) sum_n sum_i sum_j A log(A / A-hat) with math.log. The scale is not 1 and q, k
    differ, so a dropped scale or swapped operands change the result; the heads' temperatures
    differ so the ranking is not the head order; the T = 1 case (one key per row) scores 0."""
    r = _rng(33)
    N, H, T, D, scale = 3, 3, 5, 4, 0.7
    q = r.standard_normal((N, H, T, D)) * np.array([2.5, 0.3, 1.2])[None, :, None, None]
    k = r.standard_normal((N, H, T, D))
    A_hat, s_kl, rank = orc.kl_score(q, k, scale)
    want = []
    for h in range(H):
        rows = []
        for n in range(N):
            A = [[0.0] * T for _ in range(T)]
            for i in range(T):
                logits = [scale * sum(q[n, h, i, c] * k[n, h, j, c] for c in range(D)) for j in range(i + 1)]
                mx = max(logits)
                w = [math.exp(x - mx) for x in logits]
                for j in range(i + 1):
                    A[i][j] = w[j] / sum(w)
            rows.append(A)
        mean = [[sum(rows[n][i][j] for n in range(N)) / N for j in range(T)] for i in range(T)]
        tot = 0.0
        for n in range(N):
            for i in range(T):
                for j in range(i + 1):
                    tot += rows[n][i][j] * math.log(rows[n][i][j] / mean[i][j])
        want.append(tot / (N * T))
        for i in range(T):
            for j in range(T):
                assert abs(A_hat[h, i, j] - mean[i][j]) < 1e-14
    for h in range(H):
        assert abs(s_kl[h] - want[h]) <= 1e-13 * want[h] + 1e-16, (h, s_kl[h], want[h])
    order = sorted(range(H), key=lambda h: (want[h], h))
    assert list(rank) == order and order != list(range(H))
    _, s1, _ = orc.kl_score(q[:, :, :1], k[:, :, :1], scale)
    assert np.all(s1 == 0.0)


def pin_sharp_mean(orc):
    """Sharp mean (part 二.2): one sequence gives that sequence's attention; the logits are
    averaged before the softmax (pure-Python evaluation at T = 4 with two sequences); it
    differs from the probability mean A-hat when the sequences differ."""
    r = _rng(32)
    N, H, T, D = 2, 2, 4, 3
    q, k = r.standard_normal((N, H, T, D)), r.standard_normal((N, H, T, D))
    scale = 0.6
    P = orc.sharp_mean(q, k, scale)
    for h in range(H):
        for i in range(T):
            logits = [sum(scale * sum(q[n, h, i, d] * k[n, h, j, d] for d in range(D)) for n in range(N)) / N
                      for j in range(i + 1)]
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            for j in range(T):
                want = w[j] / sum(w) if j <= i else 0.0
                assert abs(P[h, i, j] - want) < 1e-14
    one = orc.sharp_mean(q[:1], k[:1], scale)
    for h in range(H):
        A, _ = orc.dynamic_probs(q[0, h], k[0, h], scale)
        assert np.max(np.abs(one[h] - A)) < 1e-15
    A_hat, _, _ = orc.var_score(q, k, scale)
    assert np.max(np.abs(A_hat - P)) > 1e-3


def pin_mean_optimality(orc):
    """Appendix B.1: R_N(P) = R_N(A-hat) + ||P - A-hat||_F^2 / T^2 for any fixed P, and the
    minimum R_N(A-hat) equals (N-1)/N s_var."""
    r = _rng(13)
    N, T, D = 6, 12, 4
    q, k = r.standard_normal((N, 1, T, D)), r.standard_normal((N, 1, T, D))
    A_hat, s_var, _ = orc.var_score(q, k, 1.0)
    A_stack = np.stack([orc.dynamic_probs(q[n, 0], k[n, 0], 1.0)[0] for n in range(N)])
    base = orc.reconstruction_risk(A_stack, A_hat[0])
    for s in range(5):
        W = np.tril(_rng(100 + s).random((T, T)))
        P = W / W.sum(axis=1, keepdims=True)
        lhs = orc.reconstruction_risk(A_stack, P)
        rhs = base + ((P - A_hat[0]) ** 2).sum() / T ** 2
        assert abs(lhs - rhs) <= 1e-12 * lhs
    assert abs(base - (N - 1) / N * s_var[0]) <= 1e-12 * base


def pin_ranking_and_count(orc):
    """Ascending s_var order with ties to the lower index; k = round(r L H) (golden counts)."""
    s = np.array([3.0, 1.0, 2.0, 1.0, 0.5])
    assert list(orc.rank_heads(s)) == [4, 1, 3, 2, 0]
    with open(os.path.join(GOLDEN, "head_count.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for rr, L, H, kk in rows:
        assert orc.n_selected(float(rr), int(L) * int(H)) == int(kk)
    sel = orc.select_heads(np.arange(144)[::-1].astype(float), 0.25)
    assert len(sel) == 36 and set(sel) == set(range(108, 144))


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
