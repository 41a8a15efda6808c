"""Shared test utilities: host <-> device marshalling and the parity tolerances.

Tolerances (stated for the row operations and the projection):
  fp32 outputs    |got - ref| <= 1e-5 * |ref|
  bf16 outputs    |got - ref| <= 8e-3 * |ref|  and  <= 2 bf16 ulp of |ref|
  projection      |got - ref| <= 8e-3 * |ref| + 2^-13 * r_t * sum_k |x_tk W'_kn|
                  (the second term bounds fp32 accumulation over K terms that may cancel)
"""

from __future__ import annotations

import numpy as np

from layerwise_qk_norm_amd import inputs


def torch():
    import torch as _t

    return _t


def to_dev(a: np.ndarray, device="cuda"):
    """numpy (uint16 bf16 bits / float32) -> torch device tensor."""
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16)).view(t.bfloat16).to(device)
    return t.from_numpy(a).to(device)


def to_host(x) -> np.ndarray:
    """torch tensor -> numpy (bf16 as uint16 bits, fp32 as float32)."""
    t = torch()
    x = x.detach().cpu().contiguous()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).numpy().view(np.uint16)
    return x.numpy()


def widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return inputs.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def bf16_ulp(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.exp2(e - 7.0)


def check_rows(got: np.ndarray, ref: np.ndarray, what: str = "", exact_rate: float = 0.99):
    """Compare a kernel output (bf16 bits or fp32) with the oracle's fp64 values."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    g = widen(got)
    nan_ref, nan_got = np.isnan(ref), np.isnan(g)
    assert np.array_equal(nan_ref, nan_got), f"{what}: NaN positions differ"
    m = ~nan_ref
    g, r = g[m], ref[m]
    inf = np.isinf(r)
    assert np.array_equal(g[inf], r[inf]), f"{what}: infinities differ"
    g, r = g[~inf], r[~inf]
    err = np.abs(g - r)
    if got.dtype == np.uint16:
        bound = np.minimum(8e-3 * np.abs(r), 2.0 * bf16_ulp(r))
        bad = err > bound
        if bad.any():
            i = int(np.argmax(err - bound))
            raise AssertionError(f"{what}: {int(bad.sum())} of {r.size} bf16 outputs out of "
                                 f"tolerance; worst got {g[i]!r} ref {r[i]!r}")
        if exact_rate is not None and r.size:
            import oracle

            rate = float(np.mean(got[m][~inf] == oracle.round_bf16(r)))
            assert rate >= exact_rate, f"{what}: exact-match rate {rate:.5f} vs RNE(oracle)"
    else:
        bad = err > 1e-5 * np.abs(r)
        if bad.any():
            i = int(np.argmax(err / np.maximum(np.abs(r), 1e-300)))
            raise AssertionError(f"{what}: {int(bad.sum())} of {r.size} fp32 outputs out of "
                                 f"tolerance; worst got {g[i]!r} ref {r[i]!r}")


def check_projection(got: np.ndarray, ref: np.ndarray, absbound: np.ndarray, what: str = "",
                     abs_coeff: float = 2.0 ** -13):
    """got: bf16 bits [T, N]; ref: fp64 [T, N]; absbound: r_t * sum_k |x_tk W'_kn| (fp64)."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    g = widen(got)
    err = np.abs(g - ref)
    bound = 8e-3 * np.abs(ref) + abs_coeff * absbound
    bad = err > bound
    if bad.any():
        i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {ref.size} outputs out of tolerance; "
                             f"worst at {i}: got {g[i]!r} ref {ref[i]!r} bound {bound[i]!r}")
