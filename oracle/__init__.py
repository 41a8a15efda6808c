"""ctypes front end of the fp64 CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU-baseline leg
import this package. It shares no code with the GPU library and never loads it.

Arrays cross as numpy buffers: bf16 tensors are uint16 arrays of raw bits, fp32 tensors are
float32 arrays, fp64 tensors are float64 arrays. Results are float64.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc -O2 (no fast-math) into liboracle.so and return its path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        i64, dbl, ci, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_void_p
        L.oracle_bf16_rne.argtypes = [dbl]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_round_bf16_array.argtypes = [i64, vp, vp]
        L.oracle_rmsnorm_rows.argtypes = [i64, i64, dbl, ci, vp, i64, ci, vp, vp, i64]
        L.oracle_partial_sumsq.argtypes = [i64, i64, ci, vp, i64, vp]
        L.oracle_apply_with_stats.argtypes = [i64, i64, i64, dbl, ci, vp, i64, ci, vp, ci, vp,
                                              i64, ci, vp, i64, vp, i64]
        L.oracle_fold_weight.argtypes = [i64, i64, ci, vp, i64, ci, vp, vp, i64]
        L.oracle_normproj.argtypes = [i64, i64, i64, dbl, ci, vp, i64, ci, vp, i64, vp, i64]
        L.oracle_normproj_unfused.argtypes = [i64, i64, i64, dbl, ci, vp, i64, ci, vp, ci, vp,
                                              i64, vp, i64]
        L.oracle_matmul.argtypes = [i64, i64, i64, ci, vp, i64, ci, vp, i64, vp, i64]
        L.oracle_qk_chain.argtypes = [i64, i64, i64, i64, dbl, dbl, ci, vp, i64, ci, vp, ci, vp,
                                      i64, vp, i64, ci, vp, vp, vp, vp, vp]
        L.oracle_qk_eliminated.argtypes = [i64, i64, i64, i64, dbl, dbl, ci, ci, vp, i64, ci, vp,
                                           i64, vp, i64, ci, vp, vp, vp, vp, vp]
        L.oracle_layernorm_rows.argtypes = [i64, i64, dbl, ci, vp, i64, ci, vp, ci, vp, vp, i64]
        L.oracle_colsum.argtypes = [i64, i64, ci, vp, i64, vp]
        L.oracle_normproj_layernorm.argtypes = [i64, i64, i64, dbl, ci, vp, i64, ci, vp, i64, ci,
                                                vp, ci, vp, vp, i64]
        L.oracle_layernorm_proj_unfused.argtypes = [i64, i64, i64, dbl, ci, vp, i64, ci, vp, ci,
                                                    vp, ci, vp, i64, vp, i64]
        for f in ("oracle_round_bf16_array", "oracle_rmsnorm_rows", "oracle_partial_sumsq",
                  "oracle_apply_with_stats", "oracle_fold_weight", "oracle_normproj",
                  "oracle_normproj_unfused", "oracle_matmul", "oracle_qk_chain",
                  "oracle_qk_eliminated", "oracle_layernorm_rows", "oracle_colsum",
                  "oracle_normproj_layernorm", "oracle_layernorm_proj_unfused"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle: unsupported storage {a.dtype}")


def _c(a):
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _rows(x: np.ndarray, d: int | None):
    """x is [T, ld]; the row width used is d (<= ld)."""
    x = _c(x)
    T, ld = x.shape
    return x, T, ld, (ld if d is None else d)


def bf16_rne(v: float) -> int:
    return int(lib().oracle_bf16_rne(float(v)))


def round_bf16(a: np.ndarray) -> np.ndarray:
    a = _c(np.asarray(a, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_round_bf16_array(a.size, _ptr(a), _ptr(out))
    return out


def rmsnorm_rows(x, gamma, eps: float, d: int | None = None) -> np.ndarray:
    x, T, ld, d = _rows(x, d)
    g = None if gamma is None else _c(gamma)
    y = np.empty((T, d), dtype=np.float64)
    lib().oracle_rmsnorm_rows(T, d, float(eps), _code(x), _ptr(x), ld,
                              _code(g) if g is not None else 0, _ptr(g), _ptr(y), d)
    return y


def partial_sumsq(x, d_local: int | None = None) -> np.ndarray:
    x, T, ld, d = _rows(x, d_local)
    s = np.empty((T,), dtype=np.float64)
    lib().oracle_partial_sumsq(T, d, _code(x), _ptr(x), ld, _ptr(s))
    return s


def apply_with_stats(x, gamma, s_own, s_ext, d_full: int, eps: float,
                     d_local: int | None = None) -> np.ndarray:
    """s_own: [T] f32/f64; s_ext: [n_ext, T] f32/f64 or None."""
    x, T, ld, d = _rows(x, d_local)
    g = None if gamma is None else _c(gamma)
    so = _c(s_own)
    if s_ext is None or s_ext.shape[0] == 0:
        se, n_ext, ld_ext, edt = np.zeros((1, 1), np.float64), 0, 0, F64
    else:
        se = _c(s_ext)
        n_ext, ld_ext, edt = se.shape[0], se.shape[1], _code(se)
    y = np.empty((T, d), dtype=np.float64)
    lib().oracle_apply_with_stats(T, d, int(d_full), float(eps), _code(x), _ptr(x), ld,
                                  _code(g) if g is not None else 0, _ptr(g), _code(so), _ptr(so),
                                  n_ext, edt, _ptr(se), ld_ext, _ptr(y), d)
    return y


def fold_weight(w, gamma) -> np.ndarray:
    """W' = diag(gamma) W in fp64; w is [K, N]."""
    w = _c(w)
    K, N = w.shape
    g = None if gamma is None else _c(gamma)
    wf = np.empty((K, N), dtype=np.float64)
    lib().oracle_fold_weight(K, N, _code(w), _ptr(w), N, _code(g) if g is not None else 0,
                             _ptr(g), _ptr(wf), N)
    return wf


def normproj(x, wf, eps: float) -> np.ndarray:
    """y = (x @ W') * r(x); x [T, K], wf [K, N]."""
    x, wf = _c(x), _c(wf)
    T, K = x.shape
    K2, N = wf.shape
    assert K == K2
    y = np.empty((T, N), dtype=np.float64)
    lib().oracle_normproj(T, K, N, float(eps), _code(x), _ptr(x), K, _code(wf), _ptr(wf), N,
                          _ptr(y), N)
    return y


def normproj_unfused(x, gamma, w, eps: float) -> np.ndarray:
    x, w = _c(x), _c(w)
    g = None if gamma is None else _c(gamma)
    T, K = x.shape
    K2, N = w.shape
    assert K == K2
    y = np.empty((T, N), dtype=np.float64)
    lib().oracle_normproj_unfused(T, K, N, float(eps), _code(x), _ptr(x), K,
                                  _code(g) if g is not None else 0, _ptr(g), _code(w), _ptr(w),
                                  N, _ptr(y), N)
    return y


def matmul(a, b) -> np.ndarray:
    a, b = _c(a), _c(b)
    T, K = a.shape
    K2, N = b.shape
    assert K == K2
    y = np.empty((T, N), dtype=np.float64)
    lib().oracle_matmul(T, K, N, _code(a), _ptr(a), K, _code(b), _ptr(b), N, _ptr(y), N)
    return y


def _opt(a):
    """(storage code, contiguous array or None) of an optional vector."""
    if a is None:
        return 0, None
    a = _c(a)
    return _code(a), a


def qk_chain(x, gamma_pre, wq, wk, gamma_q, gamma_k, eps_pre: float, eps_qk: float):
    """Pre-attention RMSNorm, Q and K projections (wq [K, nq], wk [K, nk]), then layerwise
    QK-Norm of each. Returns (yq [T, nq], yk [T, nk])."""
    x, wq, wk = _c(x), _c(wq), _c(wk)
    T, K = x.shape
    nq, nk = wq.shape[1], wk.shape[1]
    assert wq.shape[0] == K and wk.shape[0] == K and _code(wq) == _code(wk)
    g1dt, g1 = _opt(gamma_pre)
    gq, gk = _c(gamma_q), _c(gamma_k)
    assert _code(gq) == _code(gk)
    work = np.empty(K + nq + nk, dtype=np.float64)
    yq = np.empty((T, nq), dtype=np.float64)
    yk = np.empty((T, nk), dtype=np.float64)
    lib().oracle_qk_chain(T, K, nq, nk, float(eps_pre), float(eps_qk), _code(x), _ptr(x), K,
                          g1dt, _ptr(g1), _code(wq), _ptr(wq), nq, _ptr(wk), nk, _code(gq),
                          _ptr(gq), _ptr(gk), _ptr(work), _ptr(yq), _ptr(yk))
    return yq, yk


def qk_eliminated(x, wqf, wkf, gamma_q, gamma_k, eps_qk: float, eps_pre: float = 0.0,
                  exact: bool = False):
    """Projection with the pre-norm weight folded in and no pre-norm (wqf [K, nq], wkf
    [K, nk]), then layerwise QK-Norm; exact=True uses eps_qk * (mean(x^2) + eps_pre)."""
    x, wqf, wkf = _c(x), _c(wqf), _c(wkf)
    T, K = x.shape
    nq, nk = wqf.shape[1], wkf.shape[1]
    assert wqf.shape[0] == K and wkf.shape[0] == K and _code(wqf) == _code(wkf)
    gq, gk = _c(gamma_q), _c(gamma_k)
    assert _code(gq) == _code(gk)
    work = np.empty(nq + nk, dtype=np.float64)
    yq = np.empty((T, nq), dtype=np.float64)
    yk = np.empty((T, nk), dtype=np.float64)
    lib().oracle_qk_eliminated(T, K, nq, nk, float(eps_qk), float(eps_pre), int(bool(exact)),
                               _code(x), _ptr(x), K, _code(wqf), _ptr(wqf), nq, _ptr(wkf), nk,
                               _code(gq), _ptr(gq), _ptr(gk), _ptr(work), _ptr(yq), _ptr(yk))
    return yq, yk


def layernorm_rows(x, gamma, beta, eps: float, d: int | None = None) -> np.ndarray:
    x, T, ld, d = _rows(x, d)
    gdt, g = _opt(gamma)
    bdt, b = _opt(beta)
    y = np.empty((T, d), dtype=np.float64)
    lib().oracle_layernorm_rows(T, d, float(eps), _code(x), _ptr(x), ld, gdt, _ptr(g), bdt,
                                _ptr(b), _ptr(y), d)
    return y


def colsum(w) -> np.ndarray:
    """c[n] = sum_k w[k][n] for w [K, N]."""
    w = _c(w)
    K, N = w.shape
    c = np.empty((N,), dtype=np.float64)
    lib().oracle_colsum(K, N, _code(w), _ptr(w), N, _ptr(c))
    return c


def normproj_layernorm(x, wf, csum, bias, eps: float) -> np.ndarray:
    """y = r * (x @ W' - mu * colsum) + bias; x [T, K], wf [K, N], colsum / bias [N]."""
    x, wf, cs = _c(x), _c(wf), _c(csum)
    T, K = x.shape
    K2, N = wf.shape
    assert K == K2 and cs.shape == (N,)
    bdt, b = _opt(bias)
    y = np.empty((T, N), dtype=np.float64)
    lib().oracle_normproj_layernorm(T, K, N, float(eps), _code(x), _ptr(x), K, _code(wf),
                                    _ptr(wf), N, _code(cs), _ptr(cs), bdt, _ptr(b), _ptr(y), N)
    return y


def layernorm_proj_unfused(x, gamma, beta, w, eps: float) -> np.ndarray:
    x, w = _c(x), _c(w)
    T, K = x.shape
    K2, N = w.shape
    assert K == K2
    gdt, g = _opt(gamma)
    bdt, b = _opt(beta)
    y = np.empty((T, N), dtype=np.float64)
    lib().oracle_layernorm_proj_unfused(T, K, N, float(eps), _code(x), _ptr(x), K, gdt, _ptr(g),
                                        bdt, _ptr(b), _code(w), _ptr(w), N, _ptr(y), N)
    return y
