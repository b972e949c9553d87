"""Python binding of libsaf (include/saf.h): argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI. torch supplies device
memory and the current stream; the functions below check shapes, dtypes and devices,
allocate outputs when none are given, and pass raw pointers through ctypes. If
libsaf.so has not been built they raise SafError; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsaf.so")

SAF_OK, SAF_EINVAL, SAF_EUNSUPPORTED, SAF_EWORKSPACE, SAF_EHIP = range(5)
SAF_FP32, SAF_BF16 = 0, 1

# Every symbol include/saf.h declares.
EXPORTS = (
    "saf_attn_fwd", "saf_attn_workspace_size", "saf_attn_bwd", "saf_var_workspace_size",
    "saf_var_score", "saf_select_heads", "saf_status_string", "saf_last_error",
    "saf_prof_enable", "saf_prof_read", "saf_pattern_stats", "saf_compact_marginals",
    "saf_fit_workspace_size", "saf_compact_fit", "saf_select_fitted", "saf_kl_score", "saf_sharp_mean",
    "saf_attn_bwd_noalloc",
)

# Bytes of the library's own device array behind saf_attn_bwd_noalloc (SAF_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


class SafError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32),
        ("io_dtype", ctypes.c_int), ("grad_dtype", ctypes.c_int), ("scale", ctypes.c_float),
        ("frozen_mask", ctypes.POINTER(ctypes.c_uint8)), ("tab_stride", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
    ]


class VarDesc(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32),
        ("io_dtype", ctypes.c_int), ("scale", ctypes.c_float),
    ]


class FitDesc(ctypes.Structure):
    _fields_ = [
        ("H", ctypes.c_int32), ("T", ctypes.c_int32), ("steps", ctypes.c_int32),
        ("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
        ("schedule", ctypes.c_int32),
    ]


# Fit settings: 400 Adam steps (the page); lr, betas and eps are a reading (the page names
# only the optimiser); acceptance at a mean row KL of 0.2 nat (the page).
FIT_STEPS, FIT_LR, FIT_BETA1, FIT_BETA2, FIT_EPS, FIT_MAX_KL = 400, 0.1, 0.9, 0.999, 1e-8, 0.2
# saf_fit_schedule
SAF_FIT_AUTO, SAF_FIT_PER_STEP, SAF_FIT_PER_HEAD = 0, 1, 2

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libsaf.so once and declares the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise SafError(SAF_EHIP, f"{path} is missing: build it with hybrid_static_pattern_amd.build_lib")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    pd, pv = ctypes.POINTER(AttnDesc), ctypes.POINTER(VarDesc)
    lib.saf_attn_fwd.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.saf_attn_workspace_size.argtypes = [pd]
    lib.saf_attn_workspace_size.restype = sz
    lib.saf_attn_bwd.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.saf_attn_bwd_noalloc.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.saf_var_workspace_size.argtypes = [pv]
    lib.saf_var_workspace_size.restype = sz
    lib.saf_var_score.argtypes = [pv, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.saf_kl_score.argtypes = [pv, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.saf_sharp_mean.argtypes = [pv, vp, vp, vp, vp]
    lib.saf_select_heads.argtypes = [ctypes.POINTER(ctypes.c_double), i32, ctypes.c_double, ctypes.POINTER(i32)]
    lib.saf_select_heads.restype = i32
    lib.saf_status_string.argtypes = [ctypes.c_int]
    lib.saf_status_string.restype = ctypes.c_char_p
    lib.saf_last_error.restype = ctypes.c_char_p
    lib.saf_prof_enable.argtypes = [ctypes.c_int]
    lib.saf_prof_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), i32]
    lib.saf_prof_read.restype = i32
    pf = ctypes.POINTER(FitDesc)
    lib.saf_pattern_stats.argtypes = [i32, i32, vp, vp, vp, vp, vp]
    lib.saf_compact_marginals.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp]
    lib.saf_fit_workspace_size.argtypes = [pf]
    lib.saf_fit_workspace_size.restype = sz
    lib.saf_compact_fit.argtypes = [pf, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.saf_select_fitted.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_float), i32,
                                      ctypes.c_double, ctypes.c_float, ctypes.POINTER(i32)]
    lib.saf_select_fitted.restype = i32
    for fn in ("saf_attn_fwd", "saf_attn_bwd", "saf_attn_bwd_noalloc", "saf_var_score", "saf_kl_score", "saf_sharp_mean",
               "saf_prof_enable", "saf_pattern_stats",
               "saf_compact_marginals", "saf_compact_fit"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != SAF_OK:
        lib = load()
        raise SafError(status, f"{lib.saf_status_string(status).decode()}: {lib.saf_last_error().decode()}")


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SAF_BF16
    if t.dtype == torch.float32:
        return SAF_FP32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _need(t, name, shape=None, dtype=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _mask(frozen, H):
    m = np.ascontiguousarray(np.asarray(frozen, dtype=np.uint8).reshape(-1))
    if m.size != H:
        raise ValueError(f"frozen mask has {m.size} entries, expected H={H}")
    return m


def _heads(v, frozen):
    """(B, H, H_kv, T, D): H query heads from the frozen mask, H_kv key/value heads from v."""
    B, H_kv, T, D = v.shape
    H = int(np.asarray(frozen).reshape(-1).size)
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"v has {H_kv} heads, which must divide the {H} query heads of the frozen mask")
    return B, H, H_kv, T, D


def _attn_desc(v, frozen, alpha, scale):
    B, H, H_kv, T, D = _heads(v, frozen)
    mask = _mask(frozen, H)
    tab = alpha.shape[-1] if alpha is not None else T
    desc = AttnDesc(B, H, T, D, _io_dtype(v), SAF_FP32,
                    float(scale if scale is not None else 1.0 / math.sqrt(D)),
                    mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), tab, H_kv)
    return desc, mask


def _tables(alpha, rho, H, T, dev):
    for name, t in (("alpha", alpha), ("rho", rho)):
        if t is None:
            continue
        _need(t, name, dtype=torch.float32, device=dev)
        if t.dim() != 2 or t.shape[0] != H or t.shape[1] < T:
            raise ValueError(f"{name} must be [H, >=T] float32, got {tuple(t.shape)}")
    if (alpha is None) != (rho is None) or (alpha is not None and alpha.shape != rho.shape):
        raise ValueError("alpha and rho must both be given with the same shape")


def attn_fwd(q, k, v, frozen, alpha=None, rho=None, scale=None, o=None, lse=None):
    """Hybrid forward (saf_attn_fwd). q: [B,H,T,D], k, v: [B,H_kv,T,D] (H_kv = H, or a divisor
    of H for grouped-query attention), bf16 or fp32 device tensors (q, k may be None if every
    head is frozen); frozen: host sequence of H flags; alpha, rho: [H, >=T] float32.
    Returns (o [B,H,T,D] in v's dtype, lse [B,H,T] float32)."""
    lib = load()
    B, H, H_kv, T, D = _heads(v, frozen)
    for name, t, hh in (("q", q, H), ("k", k, H_kv), ("v", v, H_kv), ("o", o, H)):
        _need(t, name, shape=(B, hh, T, D), dtype=v.dtype, device=v.device)
    _need(lse, "lse", shape=(B, H, T), dtype=torch.float32, device=v.device)
    _tables(alpha, rho, H, T, v.device)
    desc, mask = _attn_desc(v, frozen, alpha, scale)
    if o is None:
        o = torch.empty((B, H, T, D), dtype=v.dtype, device=v.device)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=v.device)
    _check(lib.saf_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(rho),
                            _ptr(o), _ptr(lse), _stream(v)))
    return o, lse


def attn_workspace_size(v, frozen, alpha=None, scale=None) -> int:
    desc, mask = _attn_desc(v, frozen, alpha, scale)
    return int(load().saf_attn_workspace_size(ctypes.byref(desc)))


def attn_bwd(q, k, v, o, do, lse, frozen, alpha=None, rho=None, scale=None,
             dq=None, dk=None, dv=None, workspace=None):
    """Hybrid backward (saf_attn_bwd). Returns (dq [B,H,T,D], dk, dv [B,H_kv,T,D]), float32.
    dq of frozen heads and dk of key/value heads read by frozen heads only are never written
    (they keep whatever the given buffers, or zeros, hold)."""
    lib = load()
    B, H, H_kv, T, D = _heads(v, frozen)
    for name, t, hh in (("q", q, H), ("k", k, H_kv), ("v", v, H_kv), ("o", o, H), ("do", do, H)):
        _need(t, name, shape=(B, hh, T, D), dtype=v.dtype, device=v.device)
    _need(lse, "lse", shape=(B, H, T), dtype=torch.float32, device=v.device)
    for name, t, hh in (("dq", dq, H), ("dk", dk, H_kv), ("dv", dv, H_kv)):
        _need(t, name, shape=(B, hh, T, D), dtype=torch.float32, device=v.device)
    _tables(alpha, rho, H, T, v.device)
    desc, mask = _attn_desc(v, frozen, alpha, scale)
    need = int(lib.saf_attn_workspace_size(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=v.device)
    _need(workspace, "workspace", device=v.device)
    if dq is None:
        dq = torch.zeros((B, H, T, D), dtype=torch.float32, device=v.device)
    if dk is None:
        dk = torch.zeros((B, H_kv, T, D), dtype=torch.float32, device=v.device)
    if dv is None:
        dv = torch.empty((B, H_kv, T, D), dtype=torch.float32, device=v.device)
    _check(lib.saf_attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                            _ptr(alpha), _ptr(rho), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(v)))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, do, lse, frozen, dq, dk, dv, alpha=None, rho=None, scale=None):
    """Hybrid backward without a workspace (saf_attn_bwd_noalloc): the library's own device
    array stands in for it, so nothing is allocated here either; the caller passes dq, dk, dv.
    Results as attn_bwd. Calls that overlap in time on one GPU share that array and race."""
    lib = load()
    B, H, H_kv, T, D = _heads(v, frozen)
    for name, t, hh in (("q", q, H), ("k", k, H_kv), ("v", v, H_kv), ("o", o, H), ("do", do, H)):
        _need(t, name, shape=(B, hh, T, D), dtype=v.dtype, device=v.device)
    _need(lse, "lse", shape=(B, H, T), dtype=torch.float32, device=v.device)
    for name, t, hh in (("dq", dq, H), ("dk", dk, H_kv), ("dv", dv, H_kv)):
        if t is None:
            raise ValueError(f"{name} is required (this entry point allocates nothing)")
        _need(t, name, shape=(B, hh, T, D), dtype=torch.float32, device=v.device)
    _tables(alpha, rho, H, T, v.device)
    desc, mask = _attn_desc(v, frozen, alpha, scale)
    _check(lib.saf_attn_bwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                                    _ptr(lse), _ptr(alpha), _ptr(rho), _ptr(dq), _ptr(dk), _ptr(dv), _stream(v)))
    return dq, dk, dv


def var_workspace_size(N, H, T, D, scale=None) -> int:
    desc = VarDesc(N, H, T, D, SAF_BF16, float(scale if scale is not None else 1.0 / math.sqrt(D)))
    return int(load().saf_var_workspace_size(ctypes.byref(desc)))


def var_score(q, k, scale=None, a_hat=None, s_var=None, rank=None, workspace=None):
    """Calibration score (saf_var_score). q, k: [N,H,T,D] bf16 device tensors. Returns
    (a_hat [H,T,T] float32, s_var [H] float64, rank [H] int32), all on the device."""
    return _score(load().saf_var_score, q, k, scale, a_hat, s_var, rank, workspace)


def kl_score(q, k, scale=None, a_hat=None, s_kl=None, rank=None, workspace=None):
    """Forward-KL selector (saf_kl_score), arguments as var_score. Returns (a_hat, s_kl [H]
    float64, rank [H] int32 by ascending s_kl)."""
    return _score(load().saf_kl_score, q, k, scale, a_hat, s_kl, rank, workspace)


def sharp_mean(q, k, scale=None, out=None):
    """Sharp-mean pattern (saf_sharp_mean). q, k: [N,H,T,D] bf16 device tensors. Returns
    p_sharp [H,T,T] float32 on the device."""
    lib = load()
    N, H, T, D = q.shape
    _need(q, "q", dtype=torch.bfloat16)
    _need(k, "k", shape=(N, H, T, D), dtype=q.dtype, device=q.device)
    _need(out, "out", shape=(H, T, T), dtype=torch.float32, device=q.device)
    if out is None:
        out = torch.empty((H, T, T), dtype=torch.float32, device=q.device)
    desc = VarDesc(N, H, T, D, _io_dtype(q), float(scale if scale is not None else 1.0 / math.sqrt(D)))
    _check(lib.saf_sharp_mean(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(out), _stream(q)))
    return out


def _score(entry, q, k, scale, a_hat, s_var, rank, workspace):
    lib = load()
    N, H, T, D = q.shape
    _need(q, "q", dtype=q.dtype)
    _need(k, "k", shape=(N, H, T, D), dtype=q.dtype, device=q.device)
    _need(a_hat, "a_hat", shape=(H, T, T), dtype=torch.float32, device=q.device)
    _need(s_var, "s_var", shape=(H,), dtype=torch.float64, device=q.device)
    _need(rank, "rank", shape=(H,), dtype=torch.int32, device=q.device)
    desc = VarDesc(N, H, T, D, _io_dtype(q), float(scale if scale is not None else 1.0 / math.sqrt(D)))
    need = int(lib.saf_var_workspace_size(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if a_hat is None:
        a_hat = torch.empty((H, T, T), dtype=torch.float32, device=q.device)
    if s_var is None:
        s_var = torch.empty((H,), dtype=torch.float64, device=q.device)
    if rank is None:
        rank = torch.empty((H,), dtype=torch.int32, device=q.device)
    _check(entry(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(a_hat), _ptr(s_var), _ptr(rank),
                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q)))
    return a_hat, s_var, rank


def select_heads(s_var_all, r: float) -> np.ndarray:
    """Indices of the k = round(r * n) lowest-scoring heads over all layers (host only)."""
    s = np.ascontiguousarray(np.asarray(s_var_all, dtype=np.float64).reshape(-1))
    out = np.zeros(s.size, dtype=np.int32)
    kk = load().saf_select_heads(s.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), s.size, float(r),
                                 out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if kk < 0:
        _check(SAF_EINVAL)
    return out[:kk].copy()


def pattern_stats(a, col=None, dist=None, ent=None):
    """Eq. (4) statistics of targets a [H,T,T] float32 (saf_pattern_stats). Returns
    (col, dist, ent), each [H,T] float32 on a's device."""
    lib = load()
    _need(a, "a", dtype=torch.float32)
    if a.dim() != 3 or a.shape[1] != a.shape[2]:
        raise ValueError(f"a must be [H, T, T], got {tuple(a.shape)}")
    H, T = a.shape[0], a.shape[1]
    outs = []
    for name, t in (("col", col), ("dist", dist), ("ent", ent)):
        _need(t, name, shape=(H, T), dtype=torch.float32, device=a.device)
        outs.append(t if t is not None else torch.empty((H, T), dtype=torch.float32, device=a.device))
    _check(lib.saf_pattern_stats(H, T, _ptr(a), *(_ptr(t) for t in outs), _stream(a)))
    return tuple(outs)


def compact_marginals(alpha, rho, logz=None, col=None, dist=None):
    """log Z and the two marginals of the compact pattern (saf_compact_marginals). alpha, rho:
    [H,T] float32. Returns (logz, col, dist), each [H,T] float32."""
    lib = load()
    _need(alpha, "alpha", dtype=torch.float32)
    if alpha.dim() != 2:
        raise ValueError(f"alpha must be [H, T], got {tuple(alpha.shape)}")
    H, T = alpha.shape
    _need(rho, "rho", shape=(H, T), dtype=torch.float32, device=alpha.device)
    outs = []
    for name, t in (("logz", logz), ("col", col), ("dist", dist)):
        _need(t, name, shape=(H, T), dtype=torch.float32, device=alpha.device)
        outs.append(t if t is not None else torch.empty((H, T), dtype=torch.float32, device=alpha.device))
    _check(lib.saf_compact_marginals(H, T, _ptr(alpha), _ptr(rho), *(_ptr(t) for t in outs), _stream(alpha)))
    return tuple(outs)


def _fit_desc(H, T, steps, lr, beta1, beta2, eps, schedule=SAF_FIT_AUTO):
    return FitDesc(H, T, int(steps), float(lr), float(beta1), float(beta2), float(eps), int(schedule))


def fit_workspace_size(H, T, steps=FIT_STEPS, lr=FIT_LR, beta1=FIT_BETA1, beta2=FIT_BETA2, eps=FIT_EPS,
                       schedule=SAF_FIT_AUTO) -> int:
    d = _fit_desc(H, T, steps, lr, beta1, beta2, eps, schedule)
    return int(load().saf_fit_workspace_size(ctypes.byref(d)))


def compact_fit(col, dist, ent, alpha=None, rho=None, kl=None, steps=FIT_STEPS, lr=FIT_LR,
                beta1=FIT_BETA1, beta2=FIT_BETA2, eps=FIT_EPS, workspace=None, schedule=SAF_FIT_AUTO):
    """Fits alpha, rho [H,T] to targets with statistics (col, dist, ent) (saf_compact_fit).
    alpha, rho: the starting point, updated in place (zeros, the uniform pattern, when None).
    schedule: SAF_FIT_AUTO, SAF_FIT_PER_STEP or SAF_FIT_PER_HEAD.
    Returns (alpha, rho, kl [H] float32: mean row KL of each fitted pattern)."""
    lib = load()
    _need(col, "col", dtype=torch.float32)
    if col.dim() != 2:
        raise ValueError(f"col must be [H, T], got {tuple(col.shape)}")
    H, T = col.shape
    dev = col.device
    for name, t in (("dist", dist), ("ent", ent), ("alpha", alpha), ("rho", rho)):
        _need(t, name, shape=(H, T), dtype=torch.float32, device=dev)
    _need(kl, "kl", shape=(H,), dtype=torch.float32, device=dev)
    if dist is None or ent is None:
        raise ValueError("dist and ent are required")
    d = _fit_desc(H, T, steps, lr, beta1, beta2, eps, schedule)
    need = int(lib.saf_fit_workspace_size(ctypes.byref(d)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", device=dev)
    if alpha is None:
        alpha = torch.zeros((H, T), dtype=torch.float32, device=dev)
    if rho is None:
        rho = torch.zeros((H, T), dtype=torch.float32, device=dev)
    if kl is None:
        kl = torch.empty((H,), dtype=torch.float32, device=dev)
    _check(lib.saf_compact_fit(ctypes.byref(d), _ptr(col), _ptr(dist), _ptr(ent), _ptr(alpha), _ptr(rho),
                               _ptr(kl), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(col)))
    return alpha, rho, kl


def select_fitted(s_var_all, kl_all, r: float, max_kl: float = FIT_MAX_KL) -> np.ndarray:
    """Walks all heads by ascending s_var and keeps those whose fit passes (mean row KL <=
    max_kl) until round(r * n) are kept (host only). Returns the kept indices in walk order."""
    s = np.ascontiguousarray(np.asarray(s_var_all, dtype=np.float64).reshape(-1))
    kl = np.ascontiguousarray(np.asarray(kl_all, dtype=np.float32).reshape(-1))
    if kl.size != s.size:
        raise ValueError("s_var_all and kl_all differ in length")
    out = np.zeros(s.size, dtype=np.int32)
    kk = load().saf_select_fitted(s.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                  kl.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), s.size, float(r),
                                  float(max_kl), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if kk < 0:
        _check(SAF_EINVAL)
    return out[:kk].copy()


def prof_enable(on: bool = True) -> None:
    _check(load().saf_prof_enable(1 if on else 0))


def prof_read(cap: int = 4096):
    """(kernel name, milliseconds) for each library launch since the last read; synchronises."""
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    n = load().saf_prof_read(names, ms, cap)
    return [(names[x].decode(), float(ms[x])) for x in range(n)]
