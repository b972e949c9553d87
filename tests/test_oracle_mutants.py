"""Plants plausible mistakes in the CPU oracle and checks that the pins catch each one.

The mistakes are planted in the oracle module for the duration of one test (monkeypatch),
on the CPU only: a dropped term, a wrong index or sign, a transposed operand, a wrong
denominator. A mutant that no pin rejects would mean the pins leave that part unchecked.
"""
import numpy as np
import pytest

from oracle import saf_oracle as so
from tests.oracle_pins import PINS


def _frozen_alpha_by_query(alpha, rho):
    alpha, rho = np.asarray(alpha, float), np.asarray(rho, float)
    T = alpha.shape[0]
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    c = j <= i
    E = np.where(c, np.exp(alpha[i] + rho[np.where(c, i - j, 0)]), 0.0)
    Z = E.sum(1)
    return E / Z[:, None], np.log(Z)


def _frozen_no_alpha(alpha, rho):
    return so.__dict__["_orig_frozen"](np.zeros_like(np.asarray(alpha, float)), rho)


def _frozen_rho_by_key(alpha, rho):
    alpha, rho = np.asarray(alpha, float), np.asarray(rho, float)
    T = alpha.shape[0]
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    c = j <= i
    E = np.where(c, np.exp(alpha[j] + rho[np.broadcast_to(j, (T, T))]), 0.0)
    Z = E.sum(1)
    return E / Z[:, None], np.log(Z)


def _frozen_strict(alpha, rho):
    alpha, rho = np.asarray(alpha, float), np.asarray(rho, float)
    T = alpha.shape[0]
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    c = (j < i) | ((i == 0) & (j == 0))
    E = np.where(c, np.exp(alpha[j] + rho[np.where(c, i - j, 0)]), 0.0)
    Z = E.sum(1)
    return E / Z[:, None], np.log(Z)


def _dynamic_no_scale(q, k, scale):
    return so.__dict__["_orig_dynamic"](q, k, 1.0)


def _dynamic_swapped(q, k, scale):
    return so.__dict__["_orig_dynamic"](k, q, scale)


def _dynamic_lse_no_max(q, k, scale):
    A, lse = so.__dict__["_orig_dynamic"](q, k, scale)
    S = scale * np.asarray(q, float) @ np.asarray(k, float).T
    m = np.where(so.causal_mask(S.shape[0]), S, -np.inf).max(1)
    return A, lse - m


def _bwd_factory(kind):
    def attn_bwd(q, k, v, do, frozen, alpha, rho, scale):
        v, do = np.asarray(v, float), np.asarray(do, float)
        B, H, T, D = v.shape
        dq = np.full(v.shape, np.nan); dk = np.full(v.shape, np.nan); dv = np.empty(v.shape)
        for h in range(H):
            for b in range(B):
                if frozen[h]:
                    P, _ = so.frozen_probs(alpha[h, :T], rho[h, :T])
                    dv[b, h] = (P if kind == "frozen_no_T" else P.T) @ do[b, h]
                    continue
                qb, kb = np.asarray(q[b, h], float), np.asarray(k[b, h], float)
                A, _ = so.dynamic_probs(qb, kb, scale)
                dv[b, h] = A.T @ do[b, h]
                dA = do[b, h] @ v[b, h].T
                if kind == "no_rowterm":
                    dS = A * dA
                else:
                    dS = A * (dA - (A * dA).sum(1, keepdims=True))
                dq[b, h] = scale * (dS @ kb)
                dk[b, h] = scale * ((dS if kind == "dk_untransposed" else dS.T) @ qb)
                if kind == "dq_no_scale":
                    dq[b, h] = dS @ kb
        return dq, dk, dv
    return attn_bwd


def _gqa_factory(kind):
    def attn_bwd(q, k, v, do, frozen, alpha, rho, scale):
        v, do = np.asarray(v, float), np.asarray(do, float)
        B, H_kv, T, D = v.shape
        H = len(frozen)
        G = H // H_kv
        dq = np.full((B, H, T, D), np.nan); dk = np.zeros(v.shape); dv = np.zeros(v.shape)
        for h in range(H):
            g = h % H_kv if kind == "interleaved" else h // G
            for b in range(B):
                if frozen[h]:
                    if kind != "frozen_dv_dropped":
                        P, _ = so.frozen_probs(alpha[h, :T], rho[h, :T])
                        dv[b, g] += P.T @ do[b, h]
                    continue
                qb, kb = np.asarray(q[b, h], float), np.asarray(k[b, g], float)
                A, _ = so.dynamic_probs(qb, kb, scale)
                dv[b, g] += A.T @ do[b, h]
                dA = do[b, h] @ v[b, g].T
                dS = A * (dA - (A * dA).sum(1, keepdims=True))
                dq[b, h] = scale * (dS @ kb)
                contrib = scale * (dS.T @ qb)
                dk[b, g] = contrib if kind == "dk_overwritten" else dk[b, g] + contrib
        for g in range(H_kv):
            if all(frozen[h] for h in range(g * G, (g + 1) * G)):
                dk[:, g] = np.nan
        return dq, dk, dv
    return attn_bwd


def _gqa_fwd_interleaved(q, k, v, frozen, alpha, rho, scale):
    v = np.asarray(v, float)
    B, H_kv, T, D = v.shape
    H = len(frozen)
    O = np.empty((B, H, T, D)); lse = np.empty((B, H, T))
    for h in range(H):
        g = h % H_kv
        for b in range(B):
            if frozen[h]:
                P, lz = so.frozen_probs(alpha[h, :T], rho[h, :T])
            else:
                P, lz = so.dynamic_probs(q[b, h], k[b, g], scale)
            O[b, h] = P @ v[b, g]
            lse[b, h] = lz
    return O, lse


def _var_div_n(A_stack):
    A_stack = np.asarray(A_stack, float)
    N, T, _ = A_stack.shape
    A_hat = A_stack.mean(0)
    return float(((A_stack - A_hat) ** 2).sum() / (N * T * T)), A_hat


def _var_div_pairs(A_stack):
    A_stack = np.asarray(A_stack, float)
    N, T, _ = A_stack.shape
    A_hat = A_stack.mean(0)
    return float(((A_stack - A_hat) ** 2).sum() / ((N - 1) * T * (T + 1) / 2)), A_hat


def _kl_reverse(A_stack):
    A_stack = np.asarray(A_stack, float)
    N, T, _ = A_stack.shape
    A_hat = A_stack.mean(0)
    pos = A_hat > 0
    terms = [np.where(pos, A_hat * np.log(np.where(pos, A_hat, 1) / np.where(pos, A_stack[n], 1)), 0)
             for n in range(N)]
    return float(np.sum(terms) / (N * T)), A_hat


def _kl_by_t2(A_stack):
    val, A_hat = so.__dict__["_orig_kl"](A_stack)
    return val / np.shape(A_stack)[1], A_hat


def _kl_wrapper_factory(kind):
    """Mistakes in the q, k -> s^KL wrapper itself (kl_score_of left intact)."""
    def kl_score(q, k, scale):
        N, H, T, _ = np.shape(q)
        A_hat = np.empty((H, T, T))
        s = np.empty(H)
        for h in range(H):
            if kind == "no_scale":
                stack = [so.dynamic_probs(q[n, h], k[n, h], 1.0)[0] for n in range(N)]
            elif kind == "swapped":
                stack = [so.dynamic_probs(k[n, h], q[n, h], scale)[0] for n in range(N)]
            else:   # "first_head": every head scored on head 0's inputs
                stack = [so.dynamic_probs(q[n, 0], k[n, 0], scale)[0] for n in range(N)]
            s[h], A_hat[h] = so.kl_score_of(np.stack(stack))
        return A_hat, s, so.rank_heads(s)
    return kl_score


def _sharp_prob_mean(q, k, scale):
    return so.var_score(q, k, scale)[0]


def _rank_desc(s):
    return np.argsort(-np.asarray(s), kind="stable").astype(np.int32)


MUTANTS = {
    "frozen: alpha indexed by query": ("frozen_probs", _frozen_alpha_by_query),
    "frozen: alpha dropped": ("frozen_probs", _frozen_no_alpha),
    "frozen: rho indexed by key, not distance": ("frozen_probs", _frozen_rho_by_key),
    "frozen: diagonal excluded": ("frozen_probs", _frozen_strict),
    "dynamic: 1/sqrt(d) scale dropped": ("dynamic_probs", _dynamic_no_scale),
    "dynamic: q and k swapped": ("dynamic_probs", _dynamic_swapped),
    "dynamic: lse without the max": ("dynamic_probs", _dynamic_lse_no_max),
    "bwd: softmax row term dropped": ("attn_bwd", _bwd_factory("no_rowterm")),
    "bwd: dK operand not transposed": ("attn_bwd", _bwd_factory("dk_untransposed")),
    "bwd: dQ scale dropped": ("attn_bwd", _bwd_factory("dq_no_scale")),
    "bwd: frozen dV with P instead of P^T": ("attn_bwd", _bwd_factory("frozen_no_T")),
    "gqa fwd: query head h reads shared head h mod H_kv": ("attn_fwd", _gqa_fwd_interleaved),
    "gqa bwd: query head h reads shared head h mod H_kv": ("attn_bwd", _gqa_factory("interleaved")),
    "gqa bwd: frozen heads left out of the shared dV": ("attn_bwd", _gqa_factory("frozen_dv_dropped")),
    "gqa bwd: shared dK overwritten, not summed": ("attn_bwd", _gqa_factory("dk_overwritten")),
    "var: divides by N": ("variance_score", _var_div_n),
    "var: divides by causal pairs": ("variance_score", _var_div_pairs),
    "rank: descending": ("rank_heads", _rank_desc),
    "kl: reverse direction KL(A-hat || A)": ("kl_score_of", _kl_reverse),
    "kl: divides by N T^2": ("kl_score_of", _kl_by_t2),
    "kl wrapper: 1/sqrt(d) scale dropped": ("kl_score", _kl_wrapper_factory("no_scale")),
    "kl wrapper: q and k swapped": ("kl_score", _kl_wrapper_factory("swapped")),
    "kl wrapper: every head scored on head 0": ("kl_score", _kl_wrapper_factory("first_head")),
    "sharp mean: probabilities averaged instead of logits": ("sharp_mean", _sharp_prob_mean),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_reject_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(so.__dict__, "_orig_frozen", so.frozen_probs)
    monkeypatch.setitem(so.__dict__, "_orig_dynamic", so.dynamic_probs)
    monkeypatch.setitem(so.__dict__, "_orig_kl", so.kl_score_of)
    monkeypatch.setattr(so, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin(so)
        except Exception:  # an assertion, or the mutant breaking the pin outright
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the mutant '{name}'"
