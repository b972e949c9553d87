"""The C ABI on the CPU: the library loads, exports every declared symbol, and rejects bad
arguments before touching a device. No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

from hybrid_static_pattern_amd import saf
from oracle import saf_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(saf.LIB_PATH):
        from hybrid_static_pattern_amd import build_lib
        build_lib.build()
    return saf.load()


def declared_symbols():
    with open(os.path.join(ROOT, "include", "saf.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(saf_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = declared_symbols()
    assert set(declared) == set(saf.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in range(5):
        assert lib.saf_status_string(st).decode().startswith("SAF_")


def _desc(B=1, H=2, T=16, D=64, io=saf.SAF_BF16, grad=saf.SAF_FP32, scale=0.125, stride=16, mask=None, kv=0):
    mask = np.zeros(H, np.uint8) if mask is None else mask
    d = saf.AttnDesc(B, H, T, D, io, grad, scale, mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), stride, kv)
    return d, mask


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), saf.SAF_EINVAL), (dict(T=0), saf.SAF_EINVAL), (dict(D=96), saf.SAF_EUNSUPPORTED),
    (dict(H=300, stride=16), saf.SAF_EUNSUPPORTED), (dict(grad=saf.SAF_BF16), saf.SAF_EUNSUPPORTED),
    (dict(scale=0.0), saf.SAF_EINVAL), (dict(io=7), saf.SAF_EINVAL),
    (dict(H=6, kv=4), saf.SAF_EINVAL), (dict(H=2, kv=3), saf.SAF_EINVAL), (dict(kv=-1), saf.SAF_EINVAL),
])
def test_fwd_rejects_bad_descriptor(lib, kw, status):
    d, mask = _desc(**kw)
    st = lib.saf_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None)
    assert st == status, lib.saf_last_error()
    assert lib.saf_last_error().decode()


def test_fwd_rejects_null_and_misaligned(lib):
    d, mask = _desc()
    assert lib.saf_attn_fwd(None, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None) == saf.SAF_EINVAL
    assert lib.saf_attn_fwd(ctypes.byref(d), None, FAKE, FAKE, None, None, FAKE, FAKE, None) == saf.SAF_EINVAL
    bad = ctypes.c_void_p(0x10004)
    assert lib.saf_attn_fwd(ctypes.byref(d), FAKE, FAKE, bad, None, None, FAKE, FAKE, None) == saf.SAF_EINVAL
    assert b"aligned" in lib.saf_last_error()
    # a frozen head needs alpha/rho and a table stride >= T
    d2, m2 = _desc(mask=np.array([0, 1], np.uint8), stride=8)
    assert lib.saf_attn_fwd(ctypes.byref(d2), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == saf.SAF_EINVAL
    d3, m3 = _desc(mask=np.array([0, 1], np.uint8))
    assert lib.saf_attn_fwd(ctypes.byref(d3), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == saf.SAF_EINVAL


def test_bwd_workspace_contract(lib):
    d, mask = _desc(B=2, H=3, T=100)
    need = lib.saf_attn_workspace_size(ctypes.byref(d))
    assert need >= 2 * 3 * 100 * 4 and need % 256 == 0
    st = lib.saf_attn_bwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                          FAKE, FAKE, FAKE, FAKE, need - 1, None)
    assert st == saf.SAF_EWORKSPACE
    assert lib.saf_attn_workspace_size(None) == 0


def test_noalloc_bounds(lib):
    """saf_attn_bwd_noalloc: a layer whose workspace exceeds the library's array is rejected
    with SAF_EWORKSPACE before anything is touched (B * H * T = 16M here); a bad descriptor
    gets saf_attn_bwd's own error; the array's size is the header's."""
    d, mask = _desc(B=64, H=4, T=65536, stride=65536)
    assert lib.saf_attn_workspace_size(ctypes.byref(d)) > saf.NOALLOC_SCRATCH_BYTES
    st = lib.saf_attn_bwd_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                  FAKE, FAKE, FAKE, None)
    assert st == saf.SAF_EWORKSPACE and b"scratch" in lib.saf_last_error()
    d, mask = _desc(B=0)
    assert lib.saf_attn_bwd_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                    FAKE, FAKE, FAKE, None) == saf.SAF_EINVAL
    with open(os.path.join(ROOT, "include", "saf.h")) as f:
        m = re.search(r"#define SAF_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == saf.NOALLOC_SCRATCH_BYTES


def test_gqa_workspace_contract(lib):
    """Shared key/value heads need two more [B, H, T, D] float32 arrays (per-query-head dK, dV)."""
    d1, m1 = _desc(B=2, H=8, T=100, kv=8)
    d2, m2 = _desc(B=2, H=8, T=100, kv=2)
    n1, n2 = lib.saf_attn_workspace_size(ctypes.byref(d1)), lib.saf_attn_workspace_size(ctypes.byref(d2))
    assert n2 - n1 >= 2 * 2 * 8 * 100 * 64 * 4
    d0, m0 = _desc(B=2, H=8, T=100, kv=0)
    assert lib.saf_attn_workspace_size(ctypes.byref(d0)) == n1


def test_var_contract(lib):
    d = saf.VarDesc(1, 2, 16, 64, saf.SAF_BF16, 0.125)
    assert lib.saf_var_score(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == saf.SAF_EINVAL
    d = saf.VarDesc(4, 2, 16, 64, saf.SAF_FP32, 0.125)
    assert lib.saf_var_workspace_size(ctypes.byref(d)) == 0
    d = saf.VarDesc(4, 2, 16, 64, saf.SAF_BF16, 0.125)
    need = lib.saf_var_workspace_size(ctypes.byref(d))
    assert need > 0
    assert lib.saf_var_score(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == saf.SAF_EWORKSPACE


def test_select_heads_matches_oracle(lib):
    r = np.random.default_rng(0)
    s = r.random(144)
    s[10] = s[20]  # a tie: lower index first
    for frac in (0.0, 0.1, 0.25, 0.5, 1.0):
        assert list(saf.select_heads(s, frac)) == list(saf_oracle.select_heads(s, frac))
    assert len(saf.select_heads(s, 0.25)) == 36


def test_fit_contract(lib):
    assert lib.saf_pattern_stats(0, 16, FAKE, FAKE, FAKE, FAKE, None) == saf.SAF_EINVAL
    assert lib.saf_pattern_stats(2, 16, None, FAKE, FAKE, FAKE, None) == saf.SAF_EINVAL
    assert lib.saf_compact_marginals(70000, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None) == saf.SAF_EUNSUPPORTED
    assert lib.saf_compact_marginals(2, 16, FAKE, ctypes.c_void_p(0x10008), FAKE, FAKE, FAKE, None) == saf.SAF_EINVAL
    good = saf.FitDesc(3, 100, 400, 0.1, 0.9, 0.999, 1e-8)
    need = lib.saf_fit_workspace_size(ctypes.byref(good))
    assert need >= 7 * 3 * 100 * 4 and need % 256 == 0
    assert lib.saf_compact_fit(ctypes.byref(good), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                               None) == saf.SAF_EWORKSPACE
    for bad in (saf.FitDesc(3, 100, -1, 0.1, 0.9, 0.999, 1e-8), saf.FitDesc(3, 100, 400, 0.0, 0.9, 0.999, 1e-8),
                saf.FitDesc(3, 100, 400, 0.1, 1.0, 0.999, 1e-8), saf.FitDesc(3, 100, 400, 0.1, 0.9, 0.999, -1.0),
                saf.FitDesc(3, 0, 400, 0.1, 0.9, 0.999, 1e-8)):
        assert lib.saf_fit_workspace_size(ctypes.byref(bad)) == 0
        assert lib.saf_compact_fit(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                   None) == saf.SAF_EINVAL
    assert lib.saf_compact_fit(ctypes.byref(good), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, need,
                               None) == saf.SAF_EINVAL
    # schedules: unknown values are rejected, the per-head one needs T <= 2048
    for sched in (-1, 3):
        bad = saf.FitDesc(3, 100, 400, 0.1, 0.9, 0.999, 1e-8, sched)
        assert lib.saf_fit_workspace_size(ctypes.byref(bad)) == 0
        assert lib.saf_compact_fit(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                   None) == saf.SAF_EINVAL
    long_t = saf.FitDesc(3, 2049, 400, 0.1, 0.9, 0.999, 1e-8, saf.SAF_FIT_PER_HEAD)
    assert lib.saf_compact_fit(ctypes.byref(long_t), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                               None) == saf.SAF_EUNSUPPORTED
    assert lib.saf_fit_workspace_size(ctypes.byref(saf.FitDesc(3, 2049, 400, 0.1, 0.9, 0.999, 1e-8,
                                                               saf.SAF_FIT_PER_STEP))) > 0


def test_select_fitted_matches_oracle(lib):
    from oracle import compact_fit
    r = np.random.default_rng(1)
    s = r.random(144)
    s[3] = s[77]  # a tie: lower index first
    kl = r.random(144).astype(np.float32) * 0.4
    for frac in (0.0, 0.1, 0.25, 0.5, 1.0):
        for thr in (0.2, 0.05, 1.0):
            assert list(saf.select_fitted(s, kl, frac, thr)) == list(compact_fit.select_fitted(s, kl, frac, thr))
    assert lib.saf_select_fitted(None, None, 4, 0.5, 0.2, None) == -1
