"""Seeded synthetic inputs for the five QK-Norm workloads.

This module is the only code shared by the GPU path's callers and the CPU oracle's callers. It
draws random tensors and rounds them to the storage precision; it holds none of the method's
arithmetic (no sums of squares, no scaling, no folding, no products).

The workloads stand in for activations and weights of the models the pages measure on (OLMo
models in "SwiftQK: Fast and Communication-Efficient Tensor Parallelism for Query-Key
Normalization", abstract; SmolLM2-135M / Llama-7B scale in "FlashNorm: Fast Normalization for
Transformers", abstract), which are not available here. Shapes and distributions:

  tiny-fp32:          Q, K [T, 512] fp32, x ~ N(0, 1), gamma ~ N(1, 0.1), eps 1e-6, T = 64
  olmo2-7b:           Q, K [T, 4096] bf16 (32 heads x 128), x ~ N(0, 2), gamma ~ N(1, 0.05)
  gqa-olmo2-32b-like: Q [T, 5120] (40 x 128), K [T, 1024] (8 x 128) bf16, x ~ N(0, 1),
                      1% of the columns of each tensor multiplied by 20 (channel outliers),
                      independent gammas ~ N(1, 0.05)
  tp8-shard:          Q, K [T, 512] bf16 (one 4096/8 column slice), x ~ N(0, 1), the shard's
                      own gamma slices ~ N(1, 0.05), and 7 peers' partial sums of squares per
                      row and tensor, each a chi-square draw with 512 degrees of freedom (the
                      sum of 512 squared N(0, 1)), fp32, laid out [7, T] peer-major
  flashnorm-2048:     x [T, 2048] ~ N(0, 1), W [2048, 2048] ~ N(0, 0.02), gamma [2048]
                      ~ N(1, 0.05), all bf16

Two further workloads exercise the pre-norm elimination and the LayerNorm fold ("FlashNorm",
abstract), which the five above do not cover:

  elimination:      x [T, 4096] ~ N(0, 1) (the attention block's input), pre-norm gamma
                    ~ N(1, 0.05), Wq, Wk [4096, 4096] ~ N(0, 0.02) (OLMo-2-7B widths, 32 heads
                    x 128), QK-Norm gammas ~ N(1, 0.05), eps 1e-6 for both norms, all bf16
  layernorm:        as flashnorm-2048 plus beta [2048] ~ N(0, 0.05), eps 1e-5; x ~ N(mean, 1) with a
                    selectable per-workload mean (0 by default) to exercise the mean term

N(mu, s) names the standard deviation s. Every (workload, T, seed) gets its own PCG64 stream
(``numpy.random.default_rng(seed)``); draws happen in a fixed order (weights first, then
activations, then outlier columns or peer partials), so weights are identical across T within
a workload. Draws are float32 and are rounded to bf16 with round-to-nearest-even.
"""

from __future__ import annotations

import numpy as np

EPS_DEFAULT = 1e-6

# workload name -> shapes and the token counts it is defined for
WORKLOADS = {
    "tiny-fp32": dict(dq=512, dk=512, dtype="f32", Ts=(64,)),
    "olmo2-7b": dict(dq=4096, dk=4096, dtype="bf16", Ts=(1, 16, 256, 4096, 8192)),
    "gqa-olmo2-32b-like": dict(dq=5120, dk=1024, dtype="bf16", Ts=(1, 512, 8192)),
    "tp8-shard": dict(dq=512, dk=512, dq_full=4096, dk_full=4096, n_ext=7, dtype="bf16",
                      Ts=(131072,)),
    "flashnorm-2048": dict(K=2048, N=2048, dtype="bf16", Ts=(1, 2048, 16384)),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the raw uint16 bits.

    NaN stays NaN (quiet bit forced), infinities stay infinite, overflow rounds to infinity.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded[nan] = ((u[nan] >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040))
    return rounded.reshape(a.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).reshape(b.shape)


def _normal(rng: np.random.Generator, mu: float, sd: float, shape) -> np.ndarray:
    return rng.normal(mu, sd, size=shape).astype(np.float32)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, np.float32)


def make_case(workload: str, T: int, seed: int = 0) -> dict:
    """Return the tensors of ``workload`` (a key of WORKLOADS) at ``T`` tokens as host numpy
    arrays.

    bf16 tensors are uint16 arrays of raw bits; fp32 tensors are float32 arrays. Keys:
      tiny-fp32, olmo2-7b, gqa-olmo2-32b-like: q, k [T, d], gamma_q, gamma_k, eps, dtype,
                                               gamma_dtype
      tp8-shard:      the same plus ext_q, ext_k [7, T] fp32, dq_full, dk_full
      flashnorm-2048: x [T, K], w [K, N], gamma [K], eps
    """
    if workload not in WORKLOADS:
        raise ValueError(f"unknown workload {workload!r}")
    if T < 0:
        raise ValueError("T must be >= 0")
    c = WORKLOADS[workload]
    rng = np.random.default_rng(seed)
    out = dict(T=T, seed=seed, eps=EPS_DEFAULT, dtype=c["dtype"], name=workload)
    if workload == "tiny-fp32":
        gq = _normal(rng, 1.0, 0.1, (c["dq"],))
        gk = _normal(rng, 1.0, 0.1, (c["dk"],))
        xq = _normal(rng, 0.0, 1.0, (T, c["dq"]))
        xk = _normal(rng, 0.0, 1.0, (T, c["dk"]))
        out.update(q=xq, k=xk, gamma_q=gq, gamma_k=gk, gamma_dtype="f32")
    elif workload == "olmo2-7b":
        gq = _normal(rng, 1.0, 0.05, (c["dq"],))
        gk = _normal(rng, 1.0, 0.05, (c["dk"],))
        xq = _normal(rng, 0.0, 2.0, (T, c["dq"]))
        xk = _normal(rng, 0.0, 2.0, (T, c["dk"]))
        out.update(q=_store(xq, "bf16"), k=_store(xk, "bf16"), gamma_q=_store(gq, "bf16"),
                   gamma_k=_store(gk, "bf16"), gamma_dtype="bf16")
    elif workload == "gqa-olmo2-32b-like":
        gq = _normal(rng, 1.0, 0.05, (c["dq"],))
        gk = _normal(rng, 1.0, 0.05, (c["dk"],))
        xq = _normal(rng, 0.0, 1.0, (T, c["dq"]))
        xk = _normal(rng, 0.0, 1.0, (T, c["dk"]))
        cols_q = rng.choice(c["dq"], size=c["dq"] // 100, replace=False)
        cols_k = rng.choice(c["dk"], size=c["dk"] // 100, replace=False)
        xq[:, cols_q] *= np.float32(20.0)
        xk[:, cols_k] *= np.float32(20.0)
        out.update(q=_store(xq, "bf16"), k=_store(xk, "bf16"), gamma_q=_store(gq, "bf16"),
                   gamma_k=_store(gk, "bf16"), gamma_dtype="bf16",
                   outlier_cols_q=np.sort(cols_q), outlier_cols_k=np.sort(cols_k))
    elif workload == "tp8-shard":
        gq = _normal(rng, 1.0, 0.05, (c["dq"],))
        gk = _normal(rng, 1.0, 0.05, (c["dk"],))
        xq = _normal(rng, 0.0, 1.0, (T, c["dq"]))
        xk = _normal(rng, 0.0, 1.0, (T, c["dk"]))
        ext_q = rng.chisquare(512, size=(c["n_ext"], T)).astype(np.float32)
        ext_k = rng.chisquare(512, size=(c["n_ext"], T)).astype(np.float32)
        out.update(q=_store(xq, "bf16"), k=_store(xk, "bf16"), gamma_q=_store(gq, "bf16"),
                   gamma_k=_store(gk, "bf16"), gamma_dtype="bf16", ext_q=ext_q, ext_k=ext_k,
                   dq_full=c["dq_full"], dk_full=c["dk_full"], n_ext=c["n_ext"])
    else:
        K, N = c["K"], c["N"]
        w = _normal(rng, 0.0, 0.02, (K, N))
        g = _normal(rng, 1.0, 0.05, (K,))
        x = _normal(rng, 0.0, 1.0, (T, K))
        out.update(x=_store(x, "bf16"), w=_store(w, "bf16"), gamma=_store(g, "bf16"),
                   gamma_dtype="bf16", K=K, N=N)
    return out


ELIMINATION = dict(name="qk-proj-olmo2-7b-width", K=4096, nq=4096, nk=4096,
                   Ts=(16, 2048, 4096))
LAYERNORM = dict(name="flashnorm-layernorm-2048", K=2048, N=2048, Ts=(1, 2048, 16384))


def make_elimination_case(T: int, seed: int = 0, K: int = ELIMINATION["K"],
                          nq: int = ELIMINATION["nq"], nk: int = ELIMINATION["nk"]) -> dict:
    """Pre-norm -> Q/K projection -> QK-Norm workload. Keys: x [T, K]; gamma_pre [K];
    wq [K, nq], wk [K, nk] and their column-wise concatenation w [K, nq + nk]; gamma_q [nq],
    gamma_k [nk]; eps_pre, eps_qk (all bf16 bits except the epsilons)."""
    rng = np.random.default_rng(seed)
    g1 = _normal(rng, 1.0, 0.05, (K,))
    wq = _normal(rng, 0.0, 0.02, (K, nq))
    wk = _normal(rng, 0.0, 0.02, (K, nk))
    gq = _normal(rng, 1.0, 0.05, (nq,))
    gk = _normal(rng, 1.0, 0.05, (nk,))
    x = _normal(rng, 0.0, 1.0, (T, K))
    wq, wk = _store(wq, "bf16"), _store(wk, "bf16")
    return dict(T=T, seed=seed, name=ELIMINATION["name"], K=K, nq=nq, nk=nk, x=_store(x, "bf16"),
                gamma_pre=_store(g1, "bf16"), wq=wq, wk=wk,
                w=np.ascontiguousarray(np.concatenate([wq, wk], axis=1)),
                gamma_q=_store(gq, "bf16"), gamma_k=_store(gk, "bf16"), eps_pre=EPS_DEFAULT,
                eps_qk=EPS_DEFAULT)


def make_layernorm_case(T: int, seed: int = 0, K: int = LAYERNORM["K"], N: int = LAYERNORM["N"],
                        x_mean: float = 0.0) -> dict:
    """LayerNorm -> projection workload. Keys: x [T, K], w [K, N], gamma [K], beta [K] (bf16
    bits) and eps."""
    rng = np.random.default_rng(seed)
    w = _normal(rng, 0.0, 0.02, (K, N))
    g = _normal(rng, 1.0, 0.05, (K,))
    b = _normal(rng, 0.0, 0.05, (K,))
    x = _normal(rng, x_mean, 1.0, (T, K))
    return dict(T=T, seed=seed, name=LAYERNORM["name"], K=K, N=N, x=_store(x, "bf16"),
                w=_store(w, "bf16"), gamma=_store(g, "bf16"), beta=_store(b, "bf16"), eps=1e-5)


def random_rows(rng: np.random.Generator, T: int, d: int, dtype: str, scale: float = 1.0,
                ld: int | None = None) -> np.ndarray:
    """Seeded N(0, scale) rows for edge-case tests; with ``ld`` > d the array is [T, ld] and the
    padding columns hold a recognisable sentinel draw (N(0, 1000))."""
    ld = d if ld is None else ld
    a = rng.normal(0.0, 1000.0, size=(T, ld)).astype(np.float32)
    a[:, :d] = rng.normal(0.0, scale, size=(T, d)).astype(np.float32)
    return _store(a, dtype)


def random_gamma(rng: np.random.Generator, d: int, dtype: str, sd: float = 0.05) -> np.ndarray:
    return _store(_normal(rng, 1.0, sd, (d,)), dtype)
