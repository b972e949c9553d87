"""CPU oracle for Selective Attention Freezing (SAF): hybrid causal attention and the
calibration variance score.

TEST INFRASTRUCTURE ONLY. Nothing outside tests/, __graft_entry__.smoke() and the CPU
baseline leg of bench.py may import or call this module. The product path (the HIP
library and its Python binding) never reaches it.

Everything here is plain numpy in float64 and materialises the dense T x T matrices,
one (batch, head) at a time, so that each line can be checked against the page by eye.
Inputs are the same (bf16- or fp32-exact) values the GPU receives, upcast exactly.

Citations refer to the web page "When Can Attention Heads Be Statically Defined?:
中文精读笔记" (reading notes on the SAF paper):
  * part 一 (motivation): causal softmax attention A = softmax_causal(Q K^T / sqrt(d_h)),
    Z = A V, for an ordinary head;
  * part 二.1: the mean attention A-hat over N calibration sequences and the variance
    score s_var of Eq. (1); heads sorted by s_var ascending, k = round(r L H) chosen;
  * part 二.2: the mean-optimality identity of Appendix B.1;
  * part 二.3, Eq. (3): the compact static pattern P-hat(i,j) = exp(alpha(j) + rho(i-j)) / Z(i),
    zero for j > i;
  * part 二.4 (Algorithm 1, section 3.3 / Appendix D.2, Fig. 2): alpha, rho are fixed
    buffers without gradient; a frozen head still multiplies the current V, and its
    attention backward is only dV = P-hat^T dZ.

Readings taken where the page is silent:
  * positions are 0-indexed: query i, key j, distance d = i - j in [0, T); the page's
    1-indexed sum k = 1..i becomes j = 0..i, and the diagonal j = i is included;
  * frozen logits alpha + rho are not scaled by 1/sqrt(d_h); dynamic logits are;
  * the log-normaliser returned for a frozen head is log Z(i); for a dynamic head it is
    log sum_j exp(S_ij), the usual saved statistic of a flash-style backward;
  * the dynamic-head backward is the textbook softmax-attention gradient.

Parity: every function here is pinned by the -m "not gpu" tests in tests/ (closed
forms, invariants, finite differences and a pure-Python brute force).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def causal_mask(T: int) -> np.ndarray:
    """Boolean [T,T]: True where key j <= query i."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return j <= i


def dynamic_probs(q, k, scale: float):
    """Causal softmax attention of one ordinary head (part 一).

    q, k: [T, D]. Returns A [T,T] (exact zeros above the diagonal) and
    lse [T] = log sum_{j<=i} exp(S_ij) with S = scale * q k^T.
    """
    q, k = _f64(q), _f64(k)
    T = q.shape[0]
    S = scale * (q @ k.T)
    S = np.where(causal_mask(T), S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    A = E / l
    lse = m[:, 0] + np.log(l[:, 0])
    return A, lse


def frozen_probs(alpha, rho):
    """Compact static pattern of one frozen head, Eq. (3) (part 二.3).

    alpha, rho: [T]. Returns P [T,T] with P(i,j) = exp(alpha(j) + rho(i-j)) / Z(i) for
    j <= i and 0 for j > i, and logZ [T] = log Z(i), Z(i) = sum_{j<=i} exp(alpha(j) + rho(i-j)).
    """
    alpha, rho = _f64(alpha), _f64(rho)
    T = alpha.shape[0]
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    causal = j <= i
    dist = np.where(causal, i - j, 0)
    E = np.where(causal, np.exp(alpha[j] + rho[dist]), 0.0)
    Z = E.sum(axis=1)
    P = E / Z[:, None]
    return P, np.log(Z)


def _kv_group(frozen, v):
    """Head counts of a layer: H query heads (len(frozen)), H_kv key/value heads (v.shape[1]),
    and the group size G = H / H_kv. H_kv = H is ordinary multi-head attention; H_kv < H is
    grouped-query attention (part 二.4, the GQA path of section 3.3 / Appendix D.2): query head
    h reads the keys and values of head h // G, so a frozen head still mixes the current V of
    its group and drops only its query."""
    H, H_kv = len(frozen), np.shape(v)[1]
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"{H} query heads cannot share {H_kv} key/value heads evenly")
    return H, H_kv, H // H_kv


def attn_fwd(q, k, v, frozen, alpha, rho, scale: float):
    """Hybrid causal attention forward. q: [B,H,T,D]; k, v: [B,H_kv,T,D] (H_kv = H, or a
    divisor of H for grouped-query attention, see _kv_group).

    Ordinary heads: O = A V (part 一). Frozen heads (frozen[h] != 0): O = P-hat V with the
    current V (part 二.4, Fig. 2); their q (and, in MHA, k) are never used.
    Returns O [B,H,T,D] and lse [B,H,T] (log-normaliser of each row, see module notes).
    """
    v = _f64(v)
    B, _, T, D = v.shape
    H, _, G = _kv_group(frozen, v)
    O = np.empty((B, H, T, D))
    lse = np.empty((B, H, T))
    for h in range(H):
        g = h // G
        if frozen[h]:
            P, logZ = frozen_probs(alpha[h, :T], rho[h, :T])
            for b in range(B):
                O[b, h] = P @ v[b, g]
                lse[b, h] = logZ
        else:
            for b in range(B):
                A, l = dynamic_probs(q[b, h], k[b, g], scale)
                O[b, h] = A @ v[b, g]
                lse[b, h] = l
    return O, lse


def attn_bwd(q, k, v, do, frozen, alpha, rho, scale: float):
    """Hybrid causal attention backward for upstream gradient dO = dL/dO, [B,H,T,D].

    Ordinary heads (textbook softmax-attention gradient):
        dV = A^T dO;  dA = dO V^T;  dS_ij = A_ij (dA_ij - sum_k A_ik dA_ik);
        dQ = scale * dS K;  dK = scale * dS^T Q.
    Frozen heads (part 二.4): dV = P-hat^T dO only; alpha and rho are fixed buffers, and
    no query or key exists, so dQ of a frozen head is NaN here (never produced).
    With shared key/value heads (grouped-query attention) the gradient of a shared K or V is
    the sum over the query heads that read it: dK of head g sums the ordinary heads of its
    group (NaN, never produced, when the group has none) and dV of head g sums all of them.
    Returns dQ [B,H,T,D], dK, dV [B,H_kv,T,D].
    """
    v, do = _f64(v), _f64(do)
    B, H_kv, T, D = v.shape
    H, _, G = _kv_group(frozen, v)
    dq = np.full((B, H, T, D), np.nan)
    dk = np.zeros((B, H_kv, T, D))
    dv = np.zeros((B, H_kv, T, D))
    for h in range(H):
        g = h // G
        if frozen[h]:
            P, _ = frozen_probs(alpha[h, :T], rho[h, :T])
            for b in range(B):
                dv[b, g] += P.T @ do[b, h]
            continue
        for b in range(B):
            qb, kb = _f64(q[b, h]), _f64(k[b, g])
            A, _ = dynamic_probs(qb, kb, scale)
            dv[b, g] += A.T @ do[b, h]
            dA = do[b, h] @ v[b, g].T
            dS = A * (dA - (A * dA).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (dS @ kb)
            dk[b, g] += scale * (dS.T @ qb)
    for g in range(H_kv):
        if all(frozen[h] for h in range(g * G, (g + 1) * G)):
            dk[:, g] = np.nan   # no query head reads this K: no gradient is produced
    return dq, dk, dv


def mean_attention(A_stack):
    """A-hat = (1/N) sum_n A^(n) (part 二.1). A_stack: [N,T,T]."""
    return _f64(A_stack).mean(axis=0)


def variance_score(A_stack):
    """Eq. (1): s_var = sum_n ||A^(n) - A-hat||_F^2 / ((N - 1) T^2). A_stack: [N,T,T]."""
    A_stack = _f64(A_stack)
    N, T, _ = A_stack.shape
    A_hat = mean_attention(A_stack)
    return float(((A_stack - A_hat[None]) ** 2).sum() / ((N - 1) * T * T)), A_hat


def var_score(q, k, scale: float):
    """Calibration score of every head of one layer (part 二.1, Eq. (1)).

    q, k: [N,H,T,D] for N calibration sequences. Returns
      A_hat [H,T,T] (mean causal attention, zeros above the diagonal),
      s_var [H]    (Eq. (1) per head),
      rank [H]     (head indices by ascending s_var; ties keep the lower index first).
    """
    N, H, T, _ = np.shape(q)
    if N < 2:
        raise ValueError("Eq. (1) needs N >= 2 calibration sequences")
    A_hat = np.empty((H, T, T))
    s_var = np.empty(H)
    for h in range(H):
        A_stack = np.stack([dynamic_probs(q[n, h], k[n, h], scale)[0] for n in range(N)])
        s_var[h], A_hat[h] = variance_score(A_stack)
    return A_hat, s_var, rank_heads(s_var)


def kl_score_of(A_stack):
    """Row-wise forward-KL score of one head (part 二.1 names it s^KL as the alternative
    selector and prints no formula; read as the mean over sequences n and rows i of
    KL(A^(n)_i || A-hat_i)): (1/(N T)) sum_n sum_i sum_{j<=i} A^(n)(i,j) log(A^(n)(i,j) / A-hat(i,j)),
    with 0 log 0 = 0. A_stack: [N,T,T]. Returns s_kl and A-hat."""
    A_stack = _f64(A_stack)
    N, T, _ = A_stack.shape
    A_hat = mean_attention(A_stack)
    pos = A_stack > 0
    ratio = np.where(pos, A_stack, 1.0) / np.where(pos, A_hat[None], 1.0)
    terms = np.where(pos, A_stack * np.log(ratio), 0.0)
    return float(terms.sum() / (N * T)), A_hat


def kl_score(q, k, scale: float):
    """The forward-KL selector for every head of one layer, like var_score: returns
    A_hat [H,T,T], s_kl [H] and rank [H] (ascending s_kl, ties to the lower index)."""
    N, H, T, _ = np.shape(q)
    if N < 2:
        raise ValueError("the score compares N >= 2 calibration sequences")
    A_hat = np.empty((H, T, T))
    s_kl = np.empty(H)
    for h in range(H):
        A_stack = np.stack([dynamic_probs(q[n, h], k[n, h], scale)[0] for n in range(N)])
        s_kl[h], A_hat[h] = kl_score_of(A_stack)
    return A_hat, s_kl, rank_heads(s_kl)


def sharp_mean(q, k, scale: float):
    """The "sharp mean" candidate pattern of part 二.2: average the logits over the N
    calibration sequences first, then take the causal softmax,
        P_sharp = softmax_causal((1/N) sum_n scale Q_n K_n^T),
    for every head. q, k: [N,H,T,D]. Returns P_sharp [H,T,T] (zeros above the diagonal)."""
    q, k = _f64(q), _f64(k)
    N, H, T, _ = q.shape
    out = np.empty((H, T, T))
    for h in range(H):
        S = sum(scale * (q[n, h] @ k[n, h].T) for n in range(N)) / N
        S = np.where(causal_mask(T), S, -np.inf)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        out[h] = E / E.sum(axis=1, keepdims=True)
    return out


def rank_heads(s_var):
    """Head indices sorted by ascending s_var, stable (lower index first on ties)."""
    return np.argsort(np.asarray(s_var), kind="stable").astype(np.int32)


def n_selected(r: float, n_heads_total: int) -> int:
    """k = round(r L H) (part 二.1); halves round up."""
    return int(np.floor(r * n_heads_total + 0.5))


def select_heads(s_var_all, r: float):
    """Global selection over all L*H heads: the k lowest-s_var head indices (part 二.1)."""
    s = np.asarray(s_var_all).reshape(-1)
    return rank_heads(s)[: n_selected(r, s.size)]


def reconstruction_risk(A_stack, P):
    """Empirical R_N(P) = (1/N) sum_n ||A^(n) - P||_F^2 / T^2 (Appendix B.1, part 二.2)."""
    A_stack = _f64(A_stack)
    N, T, _ = A_stack.shape
    return float(((A_stack - _f64(P)[None]) ** 2).sum() / (N * T * T))
