"""ctypes binding of libqknorm.so: argument marshalling only.

Every function here takes torch tensors (device memory) and forwards raw pointers, sizes,
strides and the current HIP stream to the C entry point of the same name; all computation
happens in the library's gfx950 kernels. There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# QKN_LIBRARY selects another build of the same C ABI (for instance a host-only build under the
# sanitizers); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("QKN_LIBRARY") or os.path.join(PKG, "libqknorm.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "qknorm.h")

QKN_F32, QKN_BF16 = 0, 1
STATUS = {0: "QKN_OK", 1: "QKN_ERR_NULL", 2: "QKN_ERR_SHAPE", 3: "QKN_ERR_DTYPE",
          4: "QKN_ERR_EPS", 5: "QKN_ERR_ALIAS", 6: "QKN_ERR_ALIGN", 7: "QKN_ERR_HIP",
          8: "QKN_ERR_SCRATCH"}


class QknError(RuntimeError):
    def __init__(self, func: str, status: int, lib):
        msg = lib.qkn_status_string(status).decode()
        extra = f" (hipError {lib.qkn_last_hip_error()})" if status == 7 else ""
        super().__init__(f"{func}: {STATUS.get(status, status)}: {msg}{extra}")
        self.status = status


_lib = None
_i64, _f32, _int, _vp = ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_void_p
_PROTOS = {
    "qknorm_fused": [_i64, _f32, _int, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                     _i64, _vp, _i64, _vp],
    "qknorm_partial_sumsq": [_i64, _int, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp],
    "qknorm_apply_with_stats": [_i64, _f32, _int, _int, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                _i64, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64,
                                _vp, _vp, _i64, _vp],
    "normproj_fold_weight": [_i64, _i64, _int, _int, _vp, _i64, _vp, _vp, _i64, _vp],
    "normproj_deferred": [_i64, _i64, _i64, _f32, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp],
    "normproj_unfused": [_i64, _i64, _i64, _f32, _int, _int, _vp, _i64, _vp, _vp, _i64, _vp,
                         _i64, _vp, _i64, _vp],
    "normproj_fold_layernorm": [_i64, _i64, _int, _int, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp,
                                _vp],
    "normproj_deferred_layernorm": [_i64, _i64, _i64, _f32, _int, _vp, _i64, _vp, _i64, _vp, _vp,
                                    _vp, _i64, _vp, _vp],
    "normproj_deferred_layernorm_noalloc": [_i64, _i64, _i64, _f32, _int, _vp, _i64, _vp, _i64,
                                            _vp, _vp, _vp, _i64, _vp],
    "normproj_layernorm_unfused": [_i64, _i64, _i64, _f32, _int, _int, _vp, _i64, _vp, _vp, _vp,
                                   _i64, _vp, _i64, _vp, _i64, _vp],
    "qknorm_project_eliminated": [_i64, _i64, _i64, _i64, _f32, _f32, _int, _int, _vp, _i64, _vp,
                                  _i64, _vp, _vp, _vp, _i64, _vp],
    "qknorm_project_unfused": [_i64, _i64, _i64, _i64, _f32, _f32, _int, _vp, _i64, _vp, _vp,
                               _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp],
    "qkn_device_copy": [_vp, _vp, _i64, _vp],
    "qknorm_shard_fused": [_i64, _f32, _int, _int, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64,
                           _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _i64,
                           ctypes.c_uint32, _int, _i64, _vp, _vp],
    "qknorm_shard_publish": [_i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                             ctypes.c_uint32, _vp],
    "qkn_status_string": [_int],
    "qkn_last_hip_error": [],
}


def lib() -> ctypes.CDLL:
    """Load libqknorm.so (built in-tree by layerwise_qk_norm_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m layerwise_qk_norm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _PROTOS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name == "qkn_status_string" else ctypes.c_int
        _lib = L
    return _lib


def header_entry_points() -> list[str]:
    """Names of the functions include/qknorm.h declares with QKN_API."""
    text = open(HEADER).read()
    return re.findall(r"QKN_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def _check(name: str, status: int):
    if status != 0:
        raise QknError(name, status, lib())


# ----------------------------------------------------------------------------- marshalling
def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return QKN_BF16
    if t.dtype == torch.float32:
        return QKN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _ld(t) -> int:
    """Row stride of a 2-D tensor whose rows are contiguous (an empty tensor's strides are
    arbitrary, so it gets its width)."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor with unit column stride")
    if t.numel() == 0:
        return max(t.shape[1], 1)
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    ld = t.stride(0)
    return ld if t.shape[0] > 1 else max(ld, t.shape[1])


def _vec(t, n: int, what: str):
    """A 1-D operand passed as a bare pointer (gamma, column sums, per-row partials): it must be
    contiguous and hold at least n elements, or be None."""
    if t is not None and (not t.is_contiguous() or t.numel() < n):
        raise ValueError(f"{what} must be a contiguous tensor of at least {n} elements")


def _mat(t, rows: int, cols: int, what: str):
    """A 2-D operand the kernels address as rows x cols from its pointer and row stride: it
    must be at least that large (an undersized buffer would be read or written past its end)."""
    if t is not None and (t.dim() != 2 or t.shape[0] < rows or t.shape[1] < cols):
        raise ValueError(f"{what} must be a 2-D tensor of at least [{rows}, {cols}], "
                         f"got {list(t.shape)}")


def _dtypes(dtype, what: str, *ts):
    """Companion tensors share the one dtype code the C call receives for them."""
    for t in ts:
        if t is not None and t.dtype != dtype:
            raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")


def _stream(t):
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


# ----------------------------------------------------------------------------- entry points
def qknorm_fused(q, gamma_q, k=None, gamma_k=None, eps: float = 1e-6, q_out=None, k_out=None,
                 dq: int | None = None, dk: int | None = None):
    """RMSNorm of each row of q (and k) over its full width, in one launch.
    Returns (q_out, k_out); outputs may be the inputs themselves (in place)."""
    torch = _torch()
    _check_device(q, k, gamma_q, gamma_k)
    T = q.shape[0]
    dq = q.shape[1] if dq is None else dq
    if q_out is None:
        q_out = torch.empty((T, dq), dtype=q.dtype, device=q.device)
    if k is not None:
        dk = k.shape[1] if dk is None else dk
        if k_out is None:
            k_out = torch.empty((T, dk), dtype=k.dtype, device=k.device)
    _vec(gamma_q, dq, "gamma_q")
    if k is not None:
        _vec(gamma_k, dk, "gamma_k")
    gdt = _dtype_code(gamma_q)
    _dtypes(q.dtype, "k, q_out and k_out must match q", k, q_out, k_out)
    _dtypes(gamma_q.dtype, "gamma_k must match gamma_q", gamma_k)
    _mat(q, T, dq, "q")
    _mat(q_out, T, dq, "q_out")
    if k is not None:
        _mat(k, T, dk, "k")
        _mat(k_out, T, dk, "k_out")
    _check("qknorm_fused", lib().qknorm_fused(
        T, float(eps), _dtype_code(q), gdt,
        _ptr(q), _ld(q), _ptr(q_out), _ld(q_out), _ptr(gamma_q), dq,
        _ptr(k), _ld(k) if k is not None else 0, _ptr(k_out),
        _ld(k_out) if k is not None else 0, _ptr(gamma_k), dk if k is not None else 0,
        _stream(q)))
    return q_out, k_out


def qknorm_partial_sumsq(q, k=None, psq_q=None, psq_k=None, dq_local: int | None = None,
                         dk_local: int | None = None):
    """Per-row fp32 sums of squares of the slices; returns (psq_q, psq_k)."""
    torch = _torch()
    _check_device(q, k)
    T = q.shape[0]
    dq_local = q.shape[1] if dq_local is None else dq_local
    if psq_q is None:
        psq_q = torch.empty((T,), dtype=torch.float32, device=q.device)
    if k is not None:
        dk_local = k.shape[1] if dk_local is None else dk_local
        if psq_k is None:
            psq_k = torch.empty((T,), dtype=torch.float32, device=q.device)
    _vec(psq_q, T, "psq_q")
    _vec(psq_k, T, "psq_k")
    _dtypes(q.dtype, "k must match q", k)
    _dtypes(torch.float32, "psq_q / psq_k", psq_q, psq_k)
    _mat(q, T, dq_local, "q")
    if k is not None:
        _mat(k, T, dk_local, "k")
    _check("qknorm_partial_sumsq", lib().qknorm_partial_sumsq(
        T, _dtype_code(q), _ptr(q), _ld(q), dq_local, _ptr(psq_q),
        _ptr(k), _ld(k) if k is not None else 0, dk_local if k is not None else 0,
        _ptr(psq_k), _stream(q)))
    return psq_q, psq_k


def qknorm_apply_with_stats(q, gamma_q, psq_q, ext_q, dq_full: int, k=None, gamma_k=None,
                            psq_k=None, ext_k=None, dk_full: int | None = None,
                            eps: float = 1e-6, q_out=None, k_out=None,
                            dq_local: int | None = None, dk_local: int | None = None):
    """Aggregate own + peers' partials ([n_ext, T] fp32, or None) and scale the slices."""
    torch = _torch()
    _check_device(q, k, gamma_q, gamma_k, psq_q, psq_k, ext_q, ext_k)
    T = q.shape[0]
    dq_local = q.shape[1] if dq_local is None else dq_local
    n_ext = 0 if ext_q is None else ext_q.shape[0]
    if q_out is None:
        q_out = torch.empty((T, dq_local), dtype=q.dtype, device=q.device)
    if k is not None:
        dk_local = k.shape[1] if dk_local is None else dk_local
        if k_out is None:
            k_out = torch.empty((T, dk_local), dtype=k.dtype, device=k.device)
        n_ext_k = 0 if ext_k is None else ext_k.shape[0]
        if n_ext_k != n_ext:
            raise ValueError("ext_q and ext_k must hold the same number of peers")
    _vec(gamma_q, dq_local, "gamma_q")
    _vec(psq_q, T, "psq_q")
    if k is not None:
        _vec(gamma_k, dk_local, "gamma_k")
        _vec(psq_k, T, "psq_k")
    gdt = _dtype_code(gamma_q)
    _dtypes(q.dtype, "k, q_out and k_out must match q", k, q_out, k_out)
    _dtypes(gamma_q.dtype, "gamma_k must match gamma_q", gamma_k)
    _dtypes(torch.float32, "psq_* / ext_*", psq_q, psq_k, ext_q, ext_k)
    _mat(q, T, dq_local, "q")
    _mat(q_out, T, dq_local, "q_out")
    _mat(ext_q, n_ext, T, "ext_q")
    if k is not None:
        _mat(k, T, dk_local, "k")
        _mat(k_out, T, dk_local, "k_out")
        _mat(ext_k, n_ext, T, "ext_k")
    _check("qknorm_apply_with_stats", lib().qknorm_apply_with_stats(
        T, float(eps), _dtype_code(q), gdt, n_ext,
        _ptr(q), _ld(q), _ptr(q_out), _ld(q_out), _ptr(gamma_q), dq_local, dq_full,
        _ptr(psq_q), _ptr(ext_q), _ld(ext_q) if n_ext else 0,
        _ptr(k), _ld(k) if k is not None else 0, _ptr(k_out),
        _ld(k_out) if k is not None else 0, _ptr(gamma_k), dk_local if k is not None else 0,
        dk_full if k is not None else 0, _ptr(psq_k), _ptr(ext_k) if k is not None else None,
        _ld(ext_k) if (k is not None and n_ext) else 0, _stream(q)))
    return q_out, k_out


def mailbox_words(n_ext: int, T: int, device="cuda"):
    """A zeroed shard mailbox: [n_ext, T] 64-bit words (int64 storage of the uint64 words)."""
    return _torch().zeros((n_ext, T), dtype=_torch().int64, device=device)


def mailbox_values(words):
    """fp32 values held in mailbox words (their low 32 bits), as a float32 tensor view."""
    torch = _torch()
    return words.view(torch.int32)[..., 0::2].view(torch.float32)


def mailbox_epochs(words):
    """Epoch tags of mailbox words (their high 32 bits)."""
    return (words >> 32) & 0xFFFFFFFF


def qknorm_shard_fused(q, gamma_q, mail_q, dq_full: int, k=None, gamma_k=None, mail_k=None,
                       dk_full: int | None = None, eps: float = 1e-6, q_out=None, k_out=None,
                       psq_q=None, psq_k=None, epoch: int = 1, max_spin: int = 1 << 22,
                       timed_out=None, publish: bool = True, persistent: bool = True):
    """One-pass shard stage. mail_* [n_ext, T] int64 mailbox words filled by the peers
    (qknorm_shard_publish); psq_* [T] int64 words receive this rank's own partials (not
    written when publish is False). epoch == 0: the mailbox is complete, no waiting.
    persistent=True leaves a quarter of each CU to a producer on the same device;
    persistent=False reserves nothing (producers on other devices only).
    Returns (q_out, k_out, psq_q, psq_k)."""
    torch = _torch()
    _check_device(q, k, gamma_q, gamma_k, mail_q, mail_k, timed_out)
    T, dq_local = q.shape
    n_ext = 0 if mail_q is None else mail_q.shape[0]
    if q_out is None:
        q_out = torch.empty_like(q)
    if psq_q is None and publish:
        psq_q = torch.empty((T,), dtype=torch.int64, device=q.device)
    dk_local = 0
    if k is not None:
        dk_local = k.shape[1]
        if k_out is None:
            k_out = torch.empty_like(k)
        if psq_k is None and publish:
            psq_k = torch.empty((T,), dtype=torch.int64, device=q.device)
    if not publish:
        psq_q = psq_k = None
    if timed_out is None and epoch != 0:
        timed_out = torch.zeros((1,), dtype=torch.int32, device=q.device)
    _vec(gamma_q, dq_local, "gamma_q")
    _vec(gamma_k, dk_local, "gamma_k")
    _vec(psq_q, T, "psq_q")
    _vec(psq_k, T, "psq_k")
    _vec(timed_out, 1, "timed_out")
    _dtypes(q.dtype, "k, q_out and k_out must match q", k, q_out, k_out)
    _dtypes(gamma_q.dtype, "gamma_k must match gamma_q", gamma_k)
    _dtypes(torch.int64, "mailbox and psq words", mail_q, mail_k, psq_q, psq_k)
    _dtypes(torch.int32, "timed_out", timed_out)
    _mat(q_out, T, dq_local, "q_out")
    _mat(mail_q, n_ext, T, "mail_q")
    if k is not None:
        _mat(k, T, 1, "k")
        _mat(k_out, T, dk_local, "k_out")
        _mat(mail_k, n_ext, T, "mail_k")
    _check("qknorm_shard_fused", lib().qknorm_shard_fused(
        T, float(eps), _dtype_code(q), _dtype_code(gamma_q), n_ext,
        _ptr(q), _ld(q), _ptr(q_out), _ld(q_out), _ptr(gamma_q), dq_local, dq_full,
        _ptr(psq_q), _ptr(mail_q), _ld(mail_q) if n_ext else 0,
        _ptr(k), _ld(k) if k is not None else 0, _ptr(k_out), _ld(k_out) if k is not None else 0,
        _ptr(gamma_k), dk_local, dk_full if k is not None else 0, _ptr(psq_k),
        _ptr(mail_k) if k is not None else None, _ld(mail_k) if (k is not None and n_ext) else 0,
        int(epoch), int(bool(persistent)), int(max_spin), _ptr(timed_out), _stream(q)))
    return q_out, k_out, psq_q, psq_k


def qknorm_shard_publish(part_q, mail_q, epoch: int, part_k=None, mail_k=None):
    """Write peers' partials part_* [n_ext, T] fp32 into the mailboxes mail_* as words tagged
    with epoch."""
    _check_device(part_q, mail_q, part_k, mail_k)
    n_ext, T = part_q.shape
    _dtypes(_torch().float32, "part_q / part_k", part_q, part_k)
    _dtypes(_torch().int64, "mailbox words", mail_q, mail_k)
    _mat(mail_q, n_ext, T, "mail_q")
    if part_k is not None:
        _mat(part_k, n_ext, T, "part_k")
        _mat(mail_k, n_ext, T, "mail_k")
    _check("qknorm_shard_publish", lib().qknorm_shard_publish(
        T, n_ext, _ptr(part_q), _ld(part_q), _ptr(mail_q), _ld(mail_q),
        _ptr(part_k), _ld(part_k) if part_k is not None else 0, _ptr(mail_k),
        _ld(mail_k) if mail_k is not None else 0, int(epoch), _stream(part_q)))


def normproj_fold_weight(w, gamma=None, w_fold=None):
    """W [K, N] bf16 -> W' = diag(gamma) W, [K, N] bf16 (the layout of W; w_fold may be w
    itself for an in-place fold)."""
    torch = _torch()
    _check_device(w, gamma)
    K, N = w.shape
    if w_fold is None:
        w_fold = torch.empty((K, N), dtype=torch.bfloat16, device=w.device)
    _vec(gamma, K, "gamma")
    _dtypes(torch.bfloat16, "w_fold", w_fold)
    _mat(w_fold, K, N, "w_fold")
    _check("normproj_fold_weight", lib().normproj_fold_weight(
        K, N, _dtype_code(w), _dtype_code(gamma) if gamma is not None else QKN_BF16,
        _ptr(w), _ld(w), _ptr(gamma), _ptr(w_fold), _ld(w_fold), _stream(w)))
    return w_fold


def normproj_deferred(x, w_fold, eps: float = 1e-6, y=None):
    """y [T, N] = (x @ W') * (1/rms(x)) with w_fold = W' [K, N] (normproj_fold_weight)."""
    torch = _torch()
    _check_device(x, w_fold)
    T, K = x.shape
    N = w_fold.shape[1]
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _dtypes(torch.bfloat16, "w_fold and y", w_fold, y)
    _mat(w_fold, K, N, "w_fold")
    _mat(y, T, N, "y")
    _check("normproj_deferred", lib().normproj_deferred(
        T, K, N, float(eps), _dtype_code(x), _ptr(x), _ld(x), _ptr(w_fold), _ld(w_fold),
        _ptr(y), _ld(y), _stream(x)))
    return y


def normproj_unfused(x, gamma, w, eps: float = 1e-6, xn=None, y=None):
    """RMSNorm launch into xn, then a plain product with the unfolded weight w [K, N]."""
    torch = _torch()
    _check_device(x, gamma, w)
    T, K = x.shape
    N = w.shape[1]
    if xn is None:
        xn = torch.empty((T, K), dtype=torch.bfloat16, device=x.device)
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _vec(gamma, K, "gamma")
    _dtypes(torch.bfloat16, "w, xn and y", w, xn, y)
    _mat(w, K, N, "w")
    _mat(xn, T, K, "xn")
    _mat(y, T, N, "y")
    _check("normproj_unfused", lib().normproj_unfused(
        T, K, N, float(eps), _dtype_code(x), _dtype_code(gamma), _ptr(x), _ld(x), _ptr(gamma),
        _ptr(w), _ld(w), _ptr(xn), _ld(xn), _ptr(y), _ld(y), _stream(x)))
    return xn, y


def normproj_fold_layernorm(w, gamma=None, beta=None, w_fold=None, colsum=None, bias=None):
    """W [K, N] bf16 -> (W' = diag(gamma) W [K, N] bf16, colsum [N] fp32 of the
    stored W', bias = beta W [N] fp32 or None when beta is None)."""
    torch = _torch()
    _check_device(w, gamma, beta)
    K, N = w.shape
    if w_fold is None:
        w_fold = torch.empty((K, N), dtype=torch.bfloat16, device=w.device)
    if colsum is None:
        colsum = torch.empty((N,), dtype=torch.float32, device=w.device)
    if bias is None and beta is not None:
        bias = torch.empty((N,), dtype=torch.float32, device=w.device)
    _vec(gamma, K, "gamma")
    _vec(beta, K, "beta")
    _vec(colsum, N, "colsum")
    _vec(bias, N, "bias")
    gdt = _dtype_code(gamma) if gamma is not None else (
        _dtype_code(beta) if beta is not None else QKN_BF16)
    _dtypes(torch.bfloat16, "w_fold", w_fold)
    _dtypes(torch.float32, "colsum and bias", colsum, bias)
    if gamma is not None:
        _dtypes(gamma.dtype, "beta must match gamma", beta)
    _mat(w_fold, K, N, "w_fold")
    _check("normproj_fold_layernorm", lib().normproj_fold_layernorm(
        K, N, _dtype_code(w), gdt, _ptr(w), _ld(w), _ptr(gamma), _ptr(beta), _ptr(w_fold),
        _ld(w_fold), _ptr(colsum), _ptr(bias), _stream(w)))
    return w_fold, colsum, bias


def normproj_deferred_layernorm(x, w_fold, colsum, bias=None, eps: float = 1e-5, y=None,
                                row_stats="auto"):
    """y [T, N] = r * (x @ W' - mu * colsum) + bias (LayerNorm then project, deferred).

    row_stats: the [T, 2] fp32 workspace for (mu, r) of each row; "auto" allocates one, None
    passes none (the statistics are then accumulated inside the product)."""
    torch = _torch()
    _check_device(x, w_fold, colsum, bias)
    T, K = x.shape
    N = w_fold.shape[1]
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    if isinstance(row_stats, str):
        if row_stats != "auto":
            raise ValueError("row_stats must be 'auto', None or a [T, 2] float32 tensor")
        row_stats = torch.empty((T, 2), dtype=torch.float32, device=x.device)
    if row_stats is not None:
        _check_device(row_stats)
        if tuple(row_stats.shape) != (T, 2) or row_stats.dtype != torch.float32 \
                or not row_stats.is_contiguous():
            raise ValueError("row_stats must be a contiguous [T, 2] float32 tensor")
    _vec(colsum, N, "colsum")
    _vec(bias, N, "bias")
    _dtypes(torch.bfloat16, "w_fold and y", w_fold, y)
    _dtypes(torch.float32, "colsum and bias", colsum, bias)
    _mat(w_fold, K, N, "w_fold")
    _mat(y, T, N, "y")
    _check("normproj_deferred_layernorm", lib().normproj_deferred_layernorm(
        T, K, N, float(eps), _dtype_code(x), _ptr(x), _ld(x), _ptr(w_fold), _ld(w_fold),
        _ptr(colsum), _ptr(bias), _ptr(y), _ld(y), _ptr(row_stats), _stream(x)))
    return y


def normproj_deferred_layernorm_noalloc(x, w_fold, colsum, bias=None, eps: float = 1e-5, y=None):
    """normproj_deferred_layernorm with the row statistics in the library's own static device
    workspace (at most 131072 rows); the C call allocates nothing. Pass y to allocate nothing
    here either."""
    torch = _torch()
    _check_device(x, w_fold, colsum, bias, y)
    T, K = x.shape
    N = w_fold.shape[1]
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _vec(colsum, N, "colsum")
    _vec(bias, N, "bias")
    _dtypes(torch.bfloat16, "w_fold and y", w_fold, y)
    _dtypes(torch.float32, "colsum and bias", colsum, bias)
    _mat(w_fold, K, N, "w_fold")
    _mat(y, T, N, "y")
    _check("normproj_deferred_layernorm_noalloc", lib().normproj_deferred_layernorm_noalloc(
        T, K, N, float(eps), _dtype_code(x), _ptr(x), _ld(x), _ptr(w_fold), _ld(w_fold),
        _ptr(colsum), _ptr(bias), _ptr(y), _ld(y), _stream(x)))
    return y


def normproj_layernorm_unfused(x, gamma, beta, w, eps: float = 1e-5, xn=None, y=None):
    """LayerNorm launch into xn, then a plain product with the unfolded weight w [K, N]."""
    torch = _torch()
    _check_device(x, gamma, beta, w)
    T, K = x.shape
    N = w.shape[1]
    if xn is None:
        xn = torch.empty((T, K), dtype=torch.bfloat16, device=x.device)
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    g = gamma if gamma is not None else beta
    _vec(gamma, K, "gamma")
    _vec(beta, K, "beta")
    _dtypes(torch.bfloat16, "w, xn and y", w, xn, y)
    if gamma is not None:
        _dtypes(gamma.dtype, "beta must match gamma", beta)
    _mat(w, K, N, "w")
    _mat(xn, T, K, "xn")
    _mat(y, T, N, "y")
    _check("normproj_layernorm_unfused", lib().normproj_layernorm_unfused(
        T, K, N, float(eps), _dtype_code(x), _dtype_code(g) if g is not None else QKN_BF16,
        _ptr(x), _ld(x), _ptr(gamma), _ptr(beta), _ptr(w), _ld(w), _ptr(xn),
        _ld(xn), _ptr(y), _ld(y), _stream(x)))
    return xn, y


def qknorm_project_eliminated(x, w_qk, nq: int, gamma_q, gamma_k=None, eps_qk: float = 1e-6,
                              eps_pre: float = 1e-6, exact: bool = False, y=None):
    """y [T, nq + nk] = layerwise QK-Norm of x @ W' (pre-norm eliminated; exact=True keeps
    its deferred scale). w_qk [K, nq + nk] is the stacked weight [Wq | Wk] with the pre-norm
    gamma folded in (normproj_fold_weight)."""
    torch = _torch()
    _check_device(x, w_qk, gamma_q, gamma_k)
    T, K = x.shape
    N = w_qk.shape[1]
    nk = N - nq
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _vec(gamma_q, nq, "gamma_q")
    _vec(gamma_k, nk, "gamma_k")
    _dtypes(torch.bfloat16, "w_qk and y", w_qk, y)
    _dtypes(gamma_q.dtype, "gamma_k must match gamma_q", gamma_k)
    _mat(w_qk, K, N, "w_qk")
    _mat(y, T, N, "y")
    _check("qknorm_project_eliminated", lib().qknorm_project_eliminated(
        T, K, nq, nk, float(eps_qk), float(eps_pre), int(bool(exact)), _dtype_code(gamma_q),
        _ptr(x), _ld(x), _ptr(w_qk), _ld(w_qk), _ptr(gamma_q), _ptr(gamma_k), _ptr(y), _ld(y),
        _stream(x)))
    return y


def qknorm_project_unfused(x, gamma_pre, w, nq: int, gamma_q, gamma_k=None,
                           eps_qk: float = 1e-6, eps_pre: float = 1e-6, xn=None, y=None):
    """The unsimplified chain: RMSNorm launch into xn, plain product with the unfolded stacked
    weight w [K, nq + nk] into y, layerwise QK-Norm of y's Q and K blocks in place. Returns
    (xn, y)."""
    torch = _torch()
    _check_device(x, gamma_pre, w, gamma_q, gamma_k)
    T, K = x.shape
    N = w.shape[1]
    nk = N - nq
    if xn is None:
        xn = torch.empty((T, K), dtype=torch.bfloat16, device=x.device)
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _vec(gamma_pre, K, "gamma_pre")
    _vec(gamma_q, nq, "gamma_q")
    _vec(gamma_k, nk, "gamma_k")
    _dtypes(torch.bfloat16, "w, xn and y", w, xn, y)
    _dtypes(gamma_q.dtype, "gamma_pre and gamma_k must match gamma_q", gamma_pre, gamma_k)
    _mat(w, K, N, "w")
    _mat(xn, T, K, "xn")
    _mat(y, T, N, "y")
    _check("qknorm_project_unfused", lib().qknorm_project_unfused(
        T, K, nq, nk, float(eps_qk), float(eps_pre), _dtype_code(gamma_q), _ptr(x), _ld(x),
        _ptr(gamma_pre), _ptr(w), _ld(w), _ptr(gamma_q), _ptr(gamma_k), _ptr(xn),
        _ld(xn), _ptr(y), _ld(y), _stream(x)))
    return xn, y


def qkn_device_copy(dst, src, nbytes: int | None = None):
    """Copy nbytes (default: all of src) from src to dst, both contiguous device tensors that
    hold at least that many bytes."""
    _check_device(dst, src)
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    for t, what in ((dst, "dst"), (src, "src")):
        if not t.is_contiguous() or t.numel() * t.element_size() < n:
            raise ValueError(f"{what} must be a contiguous tensor of at least {n} bytes")
    _check("qkn_device_copy", lib().qkn_device_copy(_ptr(dst), _ptr(src), n, _stream(src)))
    return dst
