"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle on the same
seeded inputs, element by element, plus the pages' closed forms and the ABI's read/write
contract. Run on an MI355X with `pytest -m gpu`."""
import math

import numpy as np
import pytest
import torch

from hybrid_static_pattern_amd import inputs
from oracle import saf_oracle
from tests import golden_calibration
from tests.gpu_util import check, dev, down, layer_on_device, oracle_head, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    from hybrid_static_pattern_amd import saf
    saf.load()
    return saf


def run(S, L, bwd=True, sentinel=float("nan")):
    g = layer_on_device(L)
    fz = L["frozen"]
    allf = bool(fz.all())
    q = None if allf else g["q"]
    k = None if allf else g["k"]
    o, lse = S.attn_fwd(q, k, g["v"], fz, g["alpha"], g["rho"])
    res = dict(o=o, lse=lse)
    if bwd:
        dq = torch.full(tuple(g["do"].shape), sentinel, dtype=torch.float32, device=dev())
        dk = torch.full(tuple(g["v"].shape), sentinel, dtype=torch.float32, device=dev())
        dq, dk, dv = S.attn_bwd(q, k, g["v"], o, g["do"], lse, fz, g["alpha"], g["rho"], dq=dq, dk=dk)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {key: down(val) for key, val in res.items()}


def compare_layer(L, out, bwd=True):
    """Every output of a layer without shared key/value heads against the oracle."""
    assert L["v"].shape[1] == L["H"], "shared key/value heads: use compare_shared"
    scale = 1.0 / math.sqrt(L["D"])
    dt = L["dtype"]
    O, lse = saf_oracle.attn_fwd(L["q"], L["k"], L["v"], L["frozen"], L["alpha"], L["rho"], scale)
    check(out["o"], O, dt, "O")
    check(out["lse"], lse, dt, "lse", lse=True)
    if not bwd:
        return
    dq, dk, dv = saf_oracle.attn_bwd(L["q"], L["k"], L["v"], L["do"], L["frozen"], L["alpha"], L["rho"], scale)
    dyn = L["frozen"] == 0
    if dyn.any():
        check(out["dq"][:, dyn], dq[:, dyn], dt, "dQ")
        check(out["dk"][:, dyn], dk[:, dyn], dt, "dK")
    check(out["dv"], dv, dt, "dV")
    # dQ and dK of frozen heads are never written (NaN sentinels survive)
    assert np.all(np.isnan(out["dq"][:, ~dyn])) and np.all(np.isnan(out["dk"][:, ~dyn]))


def repeat_kv(L):
    """The same layer with every shared key/value head repeated once per query head that reads
    it (H_kv = H): ordinary multi-head attention whose per-head dK, dV are the summands of the
    shared heads' gradients."""
    G = L["H"] // L["v"].shape[1]
    R = dict(L)
    R["k"] = np.repeat(L["k"], G, axis=1)
    R["v"] = np.repeat(L["v"], G, axis=1)
    R["H_kv"] = L["H"]
    return R


def sum_close(got, want, name):
    """Float32 sums of the same per-head gradients in another order: normwise 1e-5."""
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    scale = max(np.abs(want).max(), 1e-30)
    rel = np.abs(got - want).max() / scale
    assert rel <= 1e-5, f"{name}: normwise rel err {rel:.3e} against the sum of the per-head gradients"


def compare_shared(S, L, out, groups=None, oracle_heads=None):
    """A layer with shared key/value heads (G = H / H_kv query heads per key/value head).

    O, lse and dQ are per query head and held to the bar against the oracle directly. The
    gradient of a shared K or V is a sum over its group; each summand is held to the bar:
    the same inputs run with K, V repeated per query head (repeat_kv) give the per-head
    gradients, which must meet the bar against the oracle, and the shared gradient must equal
    their float32 sum (dK over the group's ordinary heads, dV over all of them). `groups`
    limits the checks to some key/value heads (full-size shapes, where the oracle runs on a
    sample)."""
    scale = 1.0 / math.sqrt(L["D"])
    dt = L["dtype"]
    H, H_kv = L["H"], L["v"].shape[1]
    G = H // H_kv
    fz = L["frozen"]
    groups = range(H_kv) if groups is None else groups
    R = repeat_kv(L)
    rep = run(S, R)
    for g in groups:
        hs = slice(g * G, (g + 1) * G)
        O, lse = saf_oracle.attn_fwd(L["q"][:, hs], L["k"][:, g:g + 1], L["v"][:, g:g + 1], fz[hs],
                                     L["alpha"][hs], L["rho"][hs], scale)
        check(out["o"][:, hs], O, dt, f"O group {g}")
        check(out["lse"][:, hs], lse, dt, f"lse group {g}", lse=True)
        dq, dk_h, dv_h = saf_oracle.attn_bwd(R["q"][:, hs], R["k"][:, hs], R["v"][:, hs], R["do"][:, hs],
                                             fz[hs], R["alpha"][hs], R["rho"][hs], scale)
        dyn = fz[hs] == 0
        # the summands: per-query-head gradients of the repeated layer, each at the bar
        check(rep["dv"][:, hs], dv_h, dt, f"dV summands of group {g}")
        if dyn.any():
            check(out["dq"][:, hs][:, dyn], dq[:, dyn], dt, f"dQ group {g}")
            check(rep["dk"][:, hs][:, dyn], dk_h[:, dyn], dt, f"dK summands of group {g}")
            sum_close(out["dk"][:, g], rep["dk"][:, hs][:, dyn].sum(axis=1), f"dK group {g}")
        else:
            # no ordinary head reads this K: its gradient is never written
            assert np.all(np.isnan(out["dk"][:, g])), f"dK group {g} written"
        sum_close(out["dv"][:, g], rep["dv"][:, hs].sum(axis=1), f"dV group {g}")
        assert np.all(np.isnan(out["dq"][:, hs][:, ~dyn]))


def compare(S, L, out):
    if L["v"].shape[1] == L["H"]:
        compare_layer(L, out)
    else:
        compare_shared(S, L, out)


# ---------------------------------------------------------------- small layers

def test_tiny_fp32_forward(S):
    """The tiny float32 workload: B=1, H=4 (head 3 frozen), T=256, d_h=64."""
    L = inputs.make_layer(**inputs.WORKLOADS["tiny_fwd_fp32"])
    compare_layer(L, run(S, L, bwd=False), bwd=False)


@pytest.mark.parametrize("B,H,T,D,frozen", [
    (1, 3, 150, 128, [2]), (2, 2, 70, 64, [0]), (1, 2, 1, 64, [1]), (2, 2, 33, 64, [0, 1]),
])
def test_fp32_forward_backward(S, B, H, T, D, frozen):
    L = inputs.make_layer(B, H, T, D, dtype="fp32", seed=11, frozen_heads=frozen)
    compare_layer(L, run(S, L))


BF16_CASES = [
    (2, 4, 300, 64, [1, 3]),      # several tiles, ragged tail
    (1, 3, 257, 128, [0]),        # ragged; folded columns 128 < 256
    (3, 2, 130, 128, [1]),        # folded columns 384: three forward items of 128, two dV items of 256
    (8, 2, 129, 64, [0]),         # folded columns 512: four 128-column items (D = 64 takes at most 128)
    (1, 2, 1, 64, [1]),           # T = 1
    (2, 3, 64, 64, []),           # all ordinary (r = 0)
    (2, 2, 200, 128, [0, 1]),     # all frozen: q, k are NULL
    (1, 2, 513, 128, [1]),        # crosses the 512-key boundary of the dK/dV tiles
    (1, 2, 700, 64, [0]),         # folded columns 64 (the narrowest frozen item), ragged
    (3, 2, 150, 64, [1]),         # folded columns 192 (two 128-column forward items at T <= 512)
    (3, 2, 600, 64, [1]),         # folded columns 192 at T > 512: a full and a partial 128-column item
    (5, 2, 520, 128, [0]),        # folded columns 640: three 256-column items, the last partial
    (3, 4, 300, 128, [2]),        # a quarter frozen, folded columns 384: three 128-column items
    (8, 4, 600, 64, [1]),         # a quarter frozen, folded columns 512: four 128-column items
]


@pytest.mark.parametrize("B,H,T,D,frozen", BF16_CASES)
def test_bf16_forward_backward(S, B, H, T, D, frozen):
    L = inputs.make_layer(B, H, T, D, dtype="bf16", seed=7, frozen_heads=frozen)
    compare_layer(L, run(S, L))


# Shared key/value heads (grouped-query attention): B, H, H_kv, T, D, frozen heads, dtype
GQA_CASES = [
    (2, 4, 2, 300, 64, [1, 2], "bf16"),        # one frozen head in each group
    (1, 6, 2, 257, 128, [0, 1, 2], "bf16"),    # group 0 all frozen: its dK is never written
    (3, 4, 1, 130, 64, [3], "bf16"),           # one shared head (multi-query)
    (1, 8, 2, 513, 64, [0, 5, 6, 7], "bf16"),  # crosses the 512-key dK/dV tile; folded 64 columns
    (2, 4, 2, 70, 64, [1, 2], "fp32"),
    (1, 4, 1, 33, 128, [0], "fp32"),
    (2, 6, 3, 40, 64, [2, 3], "fp32"),         # group 1 all frozen
    # 16 ordinary heads (a multiple of 8): the ordinary head list is dealt out so that each
    # group's heads share an XCD, which must not change any result
    (1, 16, 4, 200, 64, [], "bf16"),
    (2, 24, 6, 130, 128, [0, 3, 7, 8, 12, 13, 17, 23], "bf16"),
]


@pytest.mark.parametrize("B,H,H_kv,T,D,frozen,dt", GQA_CASES)
def test_gqa_forward_backward(S, B, H, H_kv, T, D, frozen, dt):
    L = inputs.make_layer(B, H, T, D, dtype=dt, seed=17, frozen_heads=frozen, kv_heads=H_kv)
    compare(S, L, run(S, L))


def _random_cases(n, seed=123):
    """Seeded random layer shapes: ragged lengths, both widths, shared key/value heads, any
    frozen subset (all, none or some), both storage types."""
    r = np.random.default_rng(seed)
    cases = []
    for x in range(n):
        H = int(r.integers(1, 9))
        divisors = [d for d in range(1, H + 1) if H % d == 0]
        H_kv = int(r.choice(divisors))
        T = int(r.choice([int(r.integers(1, 64)), int(r.integers(64, 300)), int(r.integers(300, 700))]))
        D = int(r.choice([64, 128]))
        B = int(r.integers(1, 4))
        frozen = [h for h in range(H) if r.random() < 0.4]
        dt = "fp32" if r.random() < 0.3 else "bf16"
        cases.append((B, H, H_kv, T, D, frozen, dt, 1000 + x))
    return cases


@pytest.mark.parametrize("B,H,H_kv,T,D,frozen,dt,seed", _random_cases(16))
def test_random_layers(S, B, H, H_kv, T, D, frozen, dt, seed):
    L = inputs.make_layer(B, H, T, D, dtype=dt, seed=seed, frozen_heads=frozen, kv_heads=H_kv)
    compare(S, L, run(S, L))


def test_max_head_count(S):
    """H = 256, the most heads a layer may have (the head lists are 8-bit), a quarter frozen,
    with and without shared key/value heads."""
    fz = [h for h in range(256) if h % 4 == 1]
    L = inputs.make_layer(1, 256, 65, 64, dtype="bf16", seed=19, frozen_heads=fz)
    compare_layer(L, run(S, L))
    L = inputs.make_layer(1, 256, 40, 64, dtype="bf16", seed=20, frozen_heads=fz, kv_heads=32)
    compare_shared(S, L, run(S, L))


def test_gqa_frozen_query_never_read(S):
    """A frozen head of a shared group reads V of its group but never its own query."""
    L = inputs.make_layer(1, 4, 100, 64, dtype="bf16", seed=18, frozen_heads=[1, 3], kv_heads=2)
    ref = run(S, L)
    L2 = dict(L)
    L2["q"] = L["q"].copy()
    L2["q"][:, [1, 3]] = np.nan
    out = run(S, L2)
    for key in ("o", "lse", "dv"):
        assert np.array_equal(out[key], ref[key]), key


# ---------------------------------------------------------------- closed forms on the GPU

def _frozen_layer(B, T, D, dtype, alpha, rho, seed=3):
    L = inputs.make_layer(B, 1, T, D, dtype=dtype, seed=seed, frozen_heads=[0])
    L["alpha"] = np.asarray(alpha, np.float32).reshape(1, T)
    L["rho"] = np.asarray(rho, np.float32).reshape(1, T)
    return L


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_identity_pattern(S, dtype):
    """rho(0) = 0, rho(d >= 1) = -inf: P = I, so O = V and dV = dO."""
    T = 190
    rho = np.full(T, -np.inf)
    rho[0] = 0.0
    L = _frozen_layer(2, T, 64, dtype, np.random.default_rng(1).standard_normal(T), rho)
    out = run(S, L)
    tol = 1e-6 if dtype == "fp32" else 1e-2
    assert np.max(np.abs(out["o"] - L["v"])) <= tol
    assert np.max(np.abs(out["dv"] - L["do"])) <= tol


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_uniform_pattern_is_prefix_mean(S, dtype):
    """alpha = rho = 0: P(i, j) = 1/(i+1), O = prefix mean, dV = reverse cumsum of dO/(i+1)."""
    T = 333
    L = _frozen_layer(1, T, 128, dtype, np.zeros(T), np.zeros(T))
    out = run(S, L)
    cnt = np.arange(1, T + 1)[None, None, :, None]
    check(out["o"], np.cumsum(L["v"].astype(np.float64), 2) / cnt, dtype, "O")
    ref = np.cumsum((L["do"].astype(np.float64) / cnt)[:, :, ::-1], 2)[:, :, ::-1]
    check(out["dv"], ref, dtype, "dV")


def test_alpha_rho_shift_invariance(S):
    """alpha + 80 and rho + 80 leave the pattern unchanged (a naive float32 exp overflows)."""
    L = inputs.make_layer(2, 3, 260, 64, dtype="bf16", seed=5, frozen_heads=[0, 2])
    base = run(S, L)
    L2 = dict(L)
    L2["alpha"] = (L["alpha"] + 80.0).astype(np.float32)
    L2["rho"] = (L["rho"] + 80.0).astype(np.float32)
    shifted = run(S, L2)
    for key in ("o", "dv"):
        assert np.max(np.abs(shifted[key] - base[key])) <= 2e-2
    assert np.max(np.abs(shifted["lse"][:, [0, 2]] - base["lse"][:, [0, 2]] - 160.0)) <= 1e-3
    compare_layer(L2, shifted)


@pytest.mark.parametrize("k", [20, -20, 60, -60])
def test_frozen_dv_power_of_two_scaling(S, k):
    """The frozen-head dV product takes dO in fp16 after scaling each (batch, frozen head) slice
    by a power of two chosen from its largest magnitude, and scales dV back: dO times 2^k
    (exact in bf16) must give the frozen heads' dV times 2^k exactly, far outside fp16's range
    too; ordinary heads' gradients scale the same way within their float32 rounding."""
    L = inputs.make_layer(2, 3, 300, 128, dtype="bf16", seed=31, frozen_heads=[0, 2])
    base = run(S, L)
    L2 = dict(L)
    L2["do"] = (L["do"] * 2.0 ** k).astype(np.float32)
    out = run(S, L2)
    assert np.array_equal(out["dv"][:, [0, 2]], base["dv"][:, [0, 2]] * 2.0 ** k)
    compare_layer(L, base)


def test_frozen_dv_wide_dynamic_range(S):
    """dO rows spread over 2^-20 .. 2^10 (beyond fp16's range at both ends): the frozen heads'
    dV against the oracle within 2e-3 of sum_i P(i, j) |dO_i| per entry (fp16 keeps 11
    significant bits of P; dO converts exactly within 2^28 of the slice's largest value)."""
    L = inputs.make_layer(2, 2, 257, 64, dtype="bf16", seed=32, frozen_heads=[1])
    r = np.random.default_rng(33)
    row_scale = 2.0 ** r.integers(-20, 11, size=(2, 2, 257, 1))
    L["do"] = inputs.round_to_bf16((L["do"] * row_scale).astype(np.float32))
    out = run(S, L)
    P, _ = saf_oracle.frozen_probs(L["alpha"][1], L["rho"][1])
    for b in range(2):
        ref = P.T @ L["do"][b, 1].astype(np.float64)
        bound = P.T @ np.abs(L["do"][b, 1].astype(np.float64))
        err = np.abs(out["dv"][b, 1] - ref)
        assert np.all(err <= 2e-3 * bound + 1e-30), (b, float((err / (bound + 1e-30)).max()))


def test_frozen_equals_dynamic_rank1(S):
    """Affine rho(d) = -lam d: the frozen head equals an ordinary head with q_i = e0/scale,
    k_j = (alpha(j) + lam j) e0 (float32 path)."""
    T, D, lam = 300, 64, 0.05
    scale = 1.0 / math.sqrt(D)
    r = np.random.default_rng(9)
    alpha = (0.5 * r.standard_normal(T)).astype(np.float32)
    q = np.zeros((1, 2, T, D), np.float32)
    q[..., 0] = 1.0 / scale
    k = np.zeros((1, 2, T, D), np.float32)
    k[:, :, :, 0] = alpha + lam * np.arange(T)
    v = r.standard_normal((1, 2, T, D)).astype(np.float32)
    v[:, 1] = v[:, 0]
    tabs = np.stack([alpha, alpha]).astype(np.float32)
    rho = np.stack([-lam * np.arange(T)] * 2).astype(np.float32)
    o, lse = S.attn_fwd(up(q, "fp32"), up(k, "fp32"), up(v, "fp32"), [0, 1],
                        torch.from_numpy(tabs).to(dev()), torch.from_numpy(rho).to(dev()))
    o = down(o)
    rel = np.max(np.abs(o[:, 0] - o[:, 1])) / np.max(np.abs(o[:, 0]))
    assert rel <= 1e-5


# ---------------------------------------------------------------- read/write contract

def test_frozen_qk_never_read(S):
    """NaN in the q, k slices of frozen heads changes nothing."""
    L = inputs.make_layer(2, 3, 150, 64, dtype="bf16", seed=13, frozen_heads=[1])
    a = run(S, L)
    L2 = dict(L)
    for key in ("q", "k"):
        x = L[key].copy()
        x[:, 1] = np.nan
        L2[key] = x
    b = run(S, L2)
    for key in ("o", "lse", "dv"):
        assert np.array_equal(a[key], b[key]), key
    dyn = [0, 2]
    for key in ("dq", "dk"):
        assert np.array_equal(a[key][:, dyn], b[key][:, dyn]), key


def test_frozen_grads_untouched_and_deterministic(S):
    L = inputs.make_layer(1, 4, 200, 128, dtype="bf16", seed=17, frozen_heads=[0, 3])
    a = run(S, L, sentinel=12345.0)
    assert np.all(a["dq"][:, [0, 3]] == 12345.0) and np.all(a["dk"][:, [0, 3]] == 12345.0)
    b = run(S, L, sentinel=12345.0)
    for key in a:
        assert np.array_equal(a[key], b[key]), key  # no atomics: bit-identical reruns


def test_bad_workspace_is_rejected(S):
    L = inputs.make_layer(1, 2, 64, 64, dtype="bf16", seed=1, frozen_heads=[1])
    g = layer_on_device(L)
    o, lse = S.attn_fwd(g["q"], g["k"], g["v"], L["frozen"], g["alpha"], g["rho"])
    ws = torch.empty(16, dtype=torch.uint8, device=dev())
    with pytest.raises(S.SafError) as e:
        S.attn_bwd(g["q"], g["k"], g["v"], o, g["do"], lse, L["frozen"], g["alpha"], g["rho"], workspace=ws)
    assert e.value.status == S.SAF_EWORKSPACE


# ---------------------------------------------------------------- calibration score

def _check_var(S, C, heads=None):
    scale = 1.0 / math.sqrt(C["D"])
    a_hat, s_var, rank = S.var_score(up(C["q"], "bf16"), up(C["k"], "bf16"))
    torch.cuda.synchronize()
    a_hat, s_var, rank = a_hat.cpu().numpy(), s_var.cpu().numpy(), rank.cpu().numpy()
    H = C["H"]
    heads = range(H) if heads is None else heads
    ref_s = {}
    for h in heads:
        A_hat, sv, _ = saf_oracle.var_score(C["q"][:, h:h + 1], C["k"][:, h:h + 1], scale)
        assert np.max(np.abs(a_hat[h] - A_hat[0])) <= 1e-5, h
        assert abs(s_var[h] - sv[0]) <= 1e-3 * sv[0], (h, s_var[h], sv[0])
        ref_s[h] = sv[0]
    # the ranking is the stable ascending order of the scores
    assert list(rank) == list(np.argsort(s_var, kind="stable"))
    return ref_s, s_var, rank


def test_var_score_small(S):
    C = inputs.make_calibration(6, 4, 200, 64, seed=21)
    ref, s_var, rank = _check_var(S, C)
    assert list(rank) == list(saf_oracle.rank_heads([ref[h] for h in range(4)]))


def test_var_score_d64_ragged_several_tiles(S):
    """Ragged T over several Welford tiles: zero tiles above the diagonal, diagonal tiles
    that some waves skip, and keys past T in the last tile."""
    C = inputs.make_calibration(3, 2, 333, 64, seed=24)
    _check_var(S, C)


def test_var_score_d128_ragged(S):
    C = inputs.make_calibration(3, 2, 67, 128, seed=22)
    _check_var(S, C)


def test_var_score_identical_sequences(S):
    C = inputs.make_calibration(2, 3, 96, 64, seed=23)
    for key in ("q", "k"):
        C[key] = np.repeat(C[key][:1], 4, axis=0)
    C["N"] = 4
    a_hat, s_var, rank = S.var_score(up(C["q"], "bf16"), up(C["k"], "bf16"))
    assert np.all(s_var.cpu().numpy() < 1e-12)


def _check_kl(S, C, heads=None):
    """Forward-KL selector: A_hat as for Eq. (1); s^KL within 1e-3 relative + 2e-5 absolute.
    The kernel forms s^KL per entry as (1/N) sum_n A log A - A_hat log A_hat, two float32
    sums of size ~T·H(row) per head whose difference is the score; their rounding bounds
    the absolute part."""
    scale = 1.0 / math.sqrt(C["D"])
    a_hat, s_kl, rank = S.kl_score(up(C["q"], "bf16"), up(C["k"], "bf16"))
    torch.cuda.synchronize()
    a_hat, s_kl, rank = a_hat.cpu().numpy(), s_kl.cpu().numpy(), rank.cpu().numpy()
    heads = range(C["H"]) if heads is None else heads
    ref = {}
    for h in heads:
        A_hat, sk, _ = saf_oracle.kl_score(C["q"][:, h:h + 1], C["k"][:, h:h + 1], scale)
        assert np.max(np.abs(a_hat[h] - A_hat[0])) <= 1e-5, h
        assert abs(s_kl[h] - sk[0]) <= 1e-3 * sk[0] + 2e-5, (h, s_kl[h], sk[0])
        ref[h] = sk[0]
    assert list(rank) == list(np.argsort(s_kl, kind="stable"))
    return ref, s_kl, rank


def test_kl_score_small(S):
    C = inputs.make_calibration(6, 4, 200, 64, seed=24)
    ref, s_kl, rank = _check_kl(S, C)
    gaps = np.diff(sorted(ref.values()))
    if np.all(gaps > 4e-5):   # well separated: the ranking must match the oracle's
        assert list(rank) == list(saf_oracle.rank_heads([ref[h] for h in range(4)]))


def test_kl_score_d128_ragged(S):
    C = inputs.make_calibration(3, 2, 67, 128, seed=25)
    _check_kl(S, C)


def test_kl_score_identical_sequences(S):
    C = inputs.make_calibration(2, 3, 96, 64, seed=26)
    for key in ("q", "k"):
        C[key] = np.repeat(C[key][:1], 4, axis=0)
    C["N"] = 4
    a_hat, s_kl, rank = S.kl_score(up(C["q"], "bf16"), up(C["k"], "bf16"))
    assert np.all(np.abs(s_kl.cpu().numpy()) < 2e-5)


def _check_sharp(S, C, heads=None):
    """Sharp mean: the mean logits accumulate N D bf16 products in float32 (relative rounding
    ~1e-6 of the logits), so the pattern is held to 2e-5 absolute per entry."""
    scale = 1.0 / math.sqrt(C["D"])
    P = S.sharp_mean(up(C["q"], "bf16"), up(C["k"], "bf16"))
    torch.cuda.synchronize()
    P = P.cpu().numpy()
    for h in (range(C["H"]) if heads is None else heads):
        ref = saf_oracle.sharp_mean(C["q"][:, h:h + 1], C["k"][:, h:h + 1], scale)[0]
        err = np.abs(P[h] - ref).max()
        assert err <= 2e-5, (h, err)


def test_sharp_mean_small(S):
    _check_sharp(S, inputs.make_calibration(6, 4, 200, 64, seed=27))


def test_sharp_mean_d128_ragged(S):
    _check_sharp(S, inputs.make_calibration(3, 2, 67, 128, seed=28))


@pytest.mark.parametrize("N,D", [(2, 64), (3, 64), (2, 128)])
def test_calibration_fewer_sequences_than_stages(S, N, D):
    """N at or below the depth of the kernels' sequence pipeline (the loads run ahead of the
    sequence in use, and those past the last sequence re-read it): all three scores."""
    C = inputs.make_calibration(N, 2, 130, D, seed=40 + N + D)
    _check_var(S, C)
    _check_kl(S, C)
    _check_sharp(S, C)


def test_full_calibration_sharp_sampled(S):
    C = inputs.make_calibration(**inputs.CALIBRATION)
    _check_sharp(S, C, heads=[int(np.argmin(C["tau"])), int(np.argmax(C["tau"]))])


# ---------------------------------------------------------------- full-size workloads, sampled

def _full(S, name, heads, bwd=True, n_frozen=None):
    spec = dict(inputs.WORKLOADS[name])
    if n_frozen is not None:
        spec["n_frozen"] = n_frozen
    L = inputs.make_layer(**spec)
    out = run(S, L, bwd=bwd)
    scale = 1.0 / math.sqrt(L["D"])
    dt = L["dtype"]
    for b, hsel in heads:
        h = hsel(L["frozen"])
        O, lse, dq, dk, dv = oracle_head(L, b, h, scale)
        check(out["o"][b, h], O, dt, f"O[{b},{h}]")
        check(out["lse"][b, h], lse, dt, f"lse[{b},{h}]", lse=True)
        if bwd:
            check(out["dv"][b, h], dv, dt, f"dV[{b},{h}]")
            if not L["frozen"][h]:
                check(out["dq"][b, h], dq, dt, f"dQ[{b},{h}]")
                check(out["dk"][b, h], dk, dt, f"dK[{b},{h}]")


def first_frozen(fz):
    return int(np.flatnonzero(fz)[0])


def last_dynamic(fz):
    return int(np.flatnonzero(fz == 0)[-1])


def test_full_124m_forward(S):
    _full(S, "l124m_fwd", [(7, first_frozen), (3, last_dynamic)], bwd=False)


def test_full_124m_forward_backward(S):
    _full(S, "l124m_fwdbwd", [(0, first_frozen), (5, last_dynamic)])


def test_full_124m_all_dynamic(S):
    _full(S, "l124m_fwdbwd", [(2, last_dynamic)], n_frozen=0)


def test_full_1b_forward_backward(S):
    _full(S, "l1b_fwdbwd", [(1, first_frozen), (0, last_dynamic)])


def test_full_1b_half_frozen(S):
    _full(S, "l1b_fwdbwd", [(0, first_frozen)], n_frozen=8)


def test_full_1b_all_frozen(S):
    """Every head frozen (the frozen path the bench times alone): no ordinary item at all."""
    _full(S, "l1b_fwdbwd", [(1, first_frozen), (0, lambda fz: 15)], n_frozen=16)


def test_full_1b_all_dynamic(S):
    _full(S, "l1b_fwdbwd", [(1, last_dynamic)], n_frozen=0)


def test_full_prefill_t512(S):
    _full(S, "prefill_t512", [(63, first_frozen), (0, last_dynamic)], bwd=False)


def test_full_prefill_single_sequence(S):
    _full(S, "prefill_b1_t4096", [(0, first_frozen), (0, last_dynamic)])


def test_full_gqa_4b_sampled(S):
    """The shared-key/value shape (B=1, H=32 over 8 key/value heads, T=4096, D=128, r=25%):
    two whole groups (four query heads each) against the oracle, the shared dK, dV through
    their per-head summands."""
    L = inputs.make_layer(**dict(inputs.WORKLOADS["gqa_4b"]))
    out = run(S, L)
    G = L["H"] // L["H_kv"]
    fz = L["frozen"]
    groups = sorted({int(np.flatnonzero(fz)[0]) // G, int(np.flatnonzero(fz == 0)[-1]) // G})
    compare_shared(S, L, out, groups=groups)


@pytest.mark.parametrize("n_frozen", [0, 16])
def test_full_gqa_4b_other_ratios(S, n_frozen):
    """The shared-key/value shape at the bench's other ratios, r = 0 and r = 50%: two whole
    groups against the oracle (the first and the last; at r = 50% the groups of the first
    frozen and the last ordinary head)."""
    spec = dict(inputs.WORKLOADS["gqa_4b"])
    spec["n_frozen"] = n_frozen
    L = inputs.make_layer(**spec)
    out = run(S, L)
    G = L["H"] // L["H_kv"]
    fz = L["frozen"]
    if fz.any():
        groups = sorted({int(np.flatnonzero(fz)[0]) // G, int(np.flatnonzero(fz == 0)[-1]) // G})
    else:
        groups = [0, L["H_kv"] - 1]
    compare_shared(S, L, out, groups=groups)


def test_full_prefill_t2048_half_frozen(S):
    _full(S, "prefill_t2048", [(31, first_frozen), (5, last_dynamic)], bwd=False)


def test_full_prefill_t16384_sampled(S):
    """The longest prefill the bench times (B=64, H=12, T=16384, D=64, 3 of 12 heads frozen):
    Q, K, V drawn on the device by the seeded generator (a host draw of this size takes
    minutes), two whole heads, a frozen one in the last batch entry and an ordinary one in
    the first, copied back and checked against the oracle."""
    B, H, T, D = 64, 12, 16384, 64
    q, k, v = inputs.randn_bf16_device(torch, [(B, H, T, D)] * 3, seed=16)
    rng = np.random.default_rng(16)
    alpha, rho = inputs.make_tables(rng, H, T)
    fz = inputs.choose_frozen(rng, H, 3)
    heads = ((B - 1, first_frozen(fz)), (0, last_dynamic(fz)))
    # the sampled heads' inputs are copied to the host before the kernel runs
    host = {(b, h): [down(t[b:b + 1, h:h + 1]) for t in (q, k, v)] for b, h in heads}
    o, lse = S.attn_fwd(q, k, v, fz, torch.from_numpy(alpha).to(dev()), torch.from_numpy(rho).to(dev()))
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(D)
    for b, h in heads:
        O, ls = saf_oracle.attn_fwd(*host[b, h], fz[h:h + 1], alpha[h:h + 1], rho[h:h + 1], scale)
        check(down(o[b, h]), O[0, 0], "bf16", f"O[{b},{h}]")
        check(down(lse[b, h]), ls[0, 0], "bf16", f"lse[{b},{h}]", lse=True)
    del q, k, v, o, lse


def test_full_calibration_sampled(S):
    """The calibration workload: A-hat of three sampled heads entry by entry against the oracle,
    and every head's s_var (1e-3 relative), the sum of its A-hat squared and the full ranking
    against the oracle's stored values (tests/golden/calibration_N64_H12_T1024.txt)."""
    C = inputs.make_calibration(**inputs.CALIBRATION)
    tau = C["tau"]
    heads = [int(np.argmin(tau)), int(np.argmax(tau)), 5]
    _, s_var, rank = _check_var(S, C, heads=heads)
    g = golden_calibration.load()
    for h in range(C["H"]):
        assert abs(s_var[h] - g["s_var"][h]) <= 1e-3 * g["s_var"][h], (h, s_var[h], g["s_var"][h])
    assert list(rank) == g["rank_var"]
    a_hat, _, _ = S.var_score(up(C["q"], "bf16"), up(C["k"], "bf16"))
    torch.cuda.synchronize()
    sq = (a_hat.cpu().numpy().astype(np.float64) ** 2).sum(axis=(1, 2))
    # each entry within 1e-5 of the oracle's and the rows summing to 1 bound the change of the
    # sum of squares by 2e-5 T (+ T^2 1e-10)
    T = C["T"]
    assert np.all(np.abs(sq - g["a_hat_sq"]) <= 2e-5 * T + 1e-10 * T * T), (sq, g["a_hat_sq"])


def test_full_calibration_kl_sampled(S):
    """s^KL on the calibration workload: A-hat of two sampled heads against the oracle, every
    head's score and the full ranking against the oracle's stored values."""
    C = inputs.make_calibration(**inputs.CALIBRATION)
    tau = C["tau"]
    _, s_kl, rank = _check_kl(S, C, heads=[int(np.argmin(tau)), int(np.argmax(tau))])
    g = golden_calibration.load()
    for h in range(C["H"]):
        assert abs(s_kl[h] - g["s_kl"][h]) <= 1e-3 * g["s_kl"][h] + 2e-5, (h, s_kl[h], g["s_kl"][h])
    assert list(rank) == g["rank_kl"]
