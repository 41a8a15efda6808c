"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a hand-derived
worked example, a closed form, an invariant, brute force in exact rational arithmetic, or a
library routine that the definition reduces to. They are run as ordinary tests and, against
deliberately broken copies of the oracle, by the mutation test (every planted mistake must
trip at least one pin).
"""

from __future__ import annotations

import math
import os
from fractions import Fraction
from itertools import product

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------- fixtures
def _expr(s: str) -> float:
    return float(eval(s, {"__builtins__": {}}, {"sqrt": math.sqrt}))


def load_blocks(name: str) -> list[dict]:
    blocks, cur = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line:
                if cur:
                    blocks.append(cur)
                    cur = {}
                continue
            if line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            cur[key.strip()] = val.strip()
    if cur:
        blocks.append(cur)
    return blocks


def _vec(s: str) -> np.ndarray:
    return np.array([_expr(t) for t in s.split()], dtype=np.float64)


def _mat(s: str) -> np.ndarray:
    return np.array([[_expr(t) for t in row.split()] for row in s.split("|")], dtype=np.float64)


def _close(a, b, rtol=1e-14, atol=1e-300):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    ok = np.abs(a - b) <= rtol * np.abs(b) + atol
    assert ok.all(), f"max diff {np.max(np.abs(a - b))}: {a} vs {b}"


# --------------------------------------------------------------------------- worked examples
def pin_rmsnorm_worked(o):
    for b in load_blocks("rmsnorm_worked.txt"):
        x, g, eps, y = _vec(b["x"]), _vec(b["gamma"]), _expr(b["eps"]), _vec(b["y"])
        got = o.rmsnorm_rows(x[None, :], g, eps)[0]
        _close(got, y, atol=1e-15)


def pin_decomposition_worked(o):
    for b in load_blocks("decomposition_worked.txt"):
        x, g, eps, y = _vec(b["x"]), _vec(b["gamma"]), _expr(b["eps"]), _vec(b["y"])
        cuts = [0] + [int(c) for c in b["slices"].split()] + [x.size]
        parts = [o.partial_sumsq(x[None, cuts[i]:cuts[i + 1]].copy())[0]
                 for i in range(len(cuts) - 1)]
        _close(parts, _vec(b["partials"]), atol=0)
        d_full = x.size
        out = []
        for i in range(len(cuts) - 1):
            ext = np.array([[p] for j, p in enumerate(parts) if j != i], dtype=np.float64)
            out.append(o.apply_with_stats(x[None, cuts[i]:cuts[i + 1]].copy(),
                                          g[cuts[i]:cuts[i + 1]].copy(),
                                          np.array([parts[i]]), ext, d_full, eps)[0])
        _close(np.concatenate(out), y, atol=1e-15)
        _close(o.rmsnorm_rows(x[None, :], g, eps)[0], y, atol=1e-15)


def pin_flashnorm_worked(o):
    for b in load_blocks("flashnorm_worked.txt"):
        x, g, eps, y = _vec(b["x"]), _vec(b["gamma"]), _expr(b["eps"]), _vec(b["y"])
        w, wf = _mat(b["w"]), _mat(b["wfold"])
        _close(o.fold_weight(w, g), wf, atol=0)
        _close(o.normproj(x[None, :], wf, eps)[0], y, atol=1e-15)
        _close(o.normproj_unfused(x[None, :], g, w, eps)[0], y, atol=1e-15)


def pin_bf16_rounding(o):
    with open(os.path.join(GOLDEN, "bf16_rounding.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v, h = line.split()
            assert o.bf16_rne(float(v)) == int(h, 16), (v, h, hex(o.bf16_rne(float(v))))
            assert o.bf16_rne(-float(v)) == int(h, 16) ^ 0x8000, (v, "negated")


# --------------------------------------------------------------------------- closed forms
def pin_constant_vector(o):
    """c * 1 maps to gamma * c / sqrt(c^2 + eps); at eps = 0 that is gamma * sign(c)."""
    rng = np.random.default_rng(11)
    for d in (1, 2, 7, 64, 513):
        g = rng.normal(1.0, 0.3, d)
        for c in (-3.5, 0.25, 7.0, 1e-3):
            for eps in (0.0, 1e-6, 0.5):
                x = np.full((1, d), c)
                _close(o.rmsnorm_rows(x, g, eps)[0], g * c / math.sqrt(c * c + eps),
                       rtol=1e-13)


def pin_eps_small_rows(o):
    """x ~ 1e-3 so that mean(x^2) ~ eps: the closed-form ratio between eps = 1e-6 and eps = 0
    is sqrt(m / (m + eps)) per row."""
    rng = np.random.default_rng(12)
    x = rng.normal(0.0, 1e-3, (8, 256))
    g = rng.normal(1.0, 0.05, 256)
    y0 = o.rmsnorm_rows(x, g, 0.0)
    y1 = o.rmsnorm_rows(x, g, 1e-6)
    m = (x * x).mean(axis=1)
    _close(y1, y0 * np.sqrt(m / (m + 1e-6))[:, None], rtol=1e-12)


# --------------------------------------------------------------------------- invariants
def pin_invariants(o):
    rng = np.random.default_rng(13)
    T, d = 6, 333
    x = rng.normal(0.0, 2.0, (T, d))
    g = rng.normal(1.0, 0.5, d)
    # scale invariance at eps = 0: y(c x) = sign(c) y(x)
    y = o.rmsnorm_rows(x, g, 0.0)
    for c in (3.0, -0.125, 1e5):
        _close(o.rmsnorm_rows(c * x, g, 0.0), math.copysign(1.0, c) * y, rtol=1e-12)
    # sign(y) = sign(x) sign(gamma)
    assert np.array_equal(np.sign(y), np.sign(x) * np.sign(g))
    # y / (x gamma) is one constant per row, equal to r = 1/sqrt(mean(x^2) + eps)
    eps = 0.3
    y = o.rmsnorm_rows(x, g, eps)
    ratio = y / (x * g)
    _close(ratio, np.repeat(ratio[:, :1], d, axis=1), rtol=1e-13)
    # L2 relation: sum_i (y_i / gamma_i)^2 = d * m / (m + eps)
    m = np.array([math.fsum(v * v for v in row) / d for row in x])
    _close(((y / g) ** 2).sum(axis=1), d * m / (m + eps), rtol=1e-12)
    _close(((o.rmsnorm_rows(x, g, 0.0) / g) ** 2).sum(axis=1), np.full(T, float(d)), rtol=1e-12)
    # gamma enters linearly: gamma = 1 then multiplied by gamma equals the weighted norm
    _close(o.rmsnorm_rows(x, None, eps) * g, y, rtol=1e-14)


def pin_sumsq_exact(o):
    """Partial sums of squares of small integers are exact in fp64."""
    rng = np.random.default_rng(14)
    x = rng.integers(-50, 51, size=(5, 777)).astype(np.float64)
    s = o.partial_sumsq(x)
    assert np.array_equal(s, np.array([sum(int(v) ** 2 for v in row) for row in x],
                                      dtype=np.float64))


# --------------------------------------------------------------------------- brute force
def pin_brute_force_tiny(o):
    """For d in 1..4 and all integer x in {-3..3}^d (x != 0), eps = 0, gamma = 1:
    y_i^2 = x_i^2 d / sum x^2 exactly (rational arithmetic)."""
    for d in range(1, 5):
        xs = np.array([v for v in product(range(-3, 4), repeat=d) if any(v)], dtype=np.float64)
        y = o.rmsnorm_rows(xs, None, 0.0)
        for row, yr in zip(xs, y):
            ss = sum(Fraction(int(v)) ** 2 for v in row)
            for v, yv in zip(row, yr):
                exact = Fraction(int(v)) ** 2 * d / ss
                assert abs(yv * yv - float(exact)) <= 2e-15 * max(1.0, float(exact)), (row, d)
                assert math.copysign(1.0, yv) == math.copysign(1.0, v) or v == 0


# --------------------------------------------------------------------------- decomposition
def pin_decomposition_random(o):
    """Monolithic norm == partial sums over column slices + aggregation + scale, with the
    divisor being the full width (the factor depends on the full vector)."""
    rng = np.random.default_rng(15)
    T, d = 9, 520
    x = rng.normal(0.0, 1.0, (T, d))
    g = rng.normal(1.0, 0.1, d)
    eps = 1e-2
    ref = o.rmsnorm_rows(x, g, eps)
    for cuts in ([0, 65, 130, 195, 260, 325, 390, 455, 520], [0, 1, 519, 520], [0, 520]):
        parts = [o.partial_sumsq(x[:, a:b].copy()) for a, b in zip(cuts[:-1], cuts[1:])]
        for i, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
            others = [p for j, p in enumerate(parts) if j != i]
            ext = np.stack(others) if others else None
            y = o.apply_with_stats(x[:, a:b].copy(), g[a:b].copy(), parts[i], ext, d, eps)
            _close(y, ref[:, a:b], rtol=1e-13)
    # fp32 stored statistics are read exactly (widened), not re-rounded
    s32 = np.array([1.5, 2.25], dtype=np.float32)
    e32 = np.array([[0.25, 0.75]], dtype=np.float32)
    y = o.apply_with_stats(np.ones((2, 2)), None, s32, e32, 4, 0.0)
    _close(y, np.array([[1.0, 1.0], [1.0, 1.0]]) / np.sqrt(np.array([[0.4375], [0.75]])))


# --------------------------------------------------------------------------- library cases
def pin_torch_rms_norm(o):
    import torch

    rng = np.random.default_rng(16)
    for T, d, eps in ((4, 512, 1e-6), (3, 4096, 1e-5), (2, 5, 0.7)):
        x = rng.normal(0.0, 2.0, (T, d))
        g = rng.normal(1.0, 0.05, d)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (d,), torch.from_numpy(g),
                                           eps=eps).numpy()
        _close(o.rmsnorm_rows(x, g, eps), ref, rtol=1e-13)


def pin_normproj_library(o):
    """Deferred scaling equals the matrix product of the folded weight scaled per row, and the
    unfused order; checked against numpy's fp64 matmul with K != N (a transposed operand
    cannot pass)."""
    rng = np.random.default_rng(17)
    T, K, N = 5, 48, 40
    x = rng.normal(0.0, 1.0, (T, K))
    w = rng.normal(0.0, 0.02, (K, N))
    g = rng.normal(1.0, 0.05, K)
    eps = 1e-3
    wf = o.fold_weight(w, g)
    _close(wf, g[:, None] * w, rtol=0)
    r = 1.0 / np.sqrt((x * x).mean(axis=1) + eps)
    ref = (x @ (g[:, None] * w)) * r[:, None]
    _close(o.normproj(x, wf, eps), ref, rtol=1e-12, atol=1e-15)
    _close(o.normproj_unfused(x, g, w, eps), ref, rtol=1e-12, atol=1e-15)
    _close(o.matmul(x, w), x @ w, rtol=1e-12, atol=1e-15)
    # exactness of the reformulation, including eps, between the two oracle orders
    x2 = rng.normal(0.0, 1e-3, (T, K))
    _close(o.normproj(x2, wf, 1e-6), o.normproj_unfused(x2, g, w, 1e-6), rtol=1e-12,
           atol=1e-15)


def pin_bf16_widening(o):
    """bf16 storage is widened exactly; checked against torch's bf16 -> fp64 conversion."""
    import torch

    rng = np.random.default_rng(18)
    bits = rng.integers(0, 65536, size=(3, 4096), dtype=np.uint32).astype(np.uint16)
    bits[(bits & 0x7F80) == 0x7F80] = 0x3F80  # keep finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    y = o.rmsnorm_rows(bits, None, 0.0)
    yr = o.rmsnorm_rows(ref, None, 0.0)
    _close(y, yr, rtol=0, atol=0)
    s = o.partial_sumsq(bits)
    _close(s, np.array([math.fsum(v * v for v in row) for row in ref]), rtol=1e-13)


def pin_bf16_rne_library(o):
    """RNE into bf16 agrees with torch's float32 -> bfloat16 conversion on random values,
    including exact ties."""
    import torch

    rng = np.random.default_rng(19)
    v = rng.normal(0.0, 10.0, 20000).astype(np.float32)
    ties = ((rng.integers(0, 65536, 2000, dtype=np.uint32) << 16) | 0x8000).astype(np.uint32)
    ties = ties.view(np.float32)
    v = np.concatenate([v, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref), int(np.sum(got != ref))


# --------------------------------------------------------------------------- pre-norm elimination
ELIM_WQ = np.eye(2)
ELIM_WK = np.array([[1.0], [1.0]])


def pin_elimination_worked(o):
    for b in load_blocks("elimination_worked.txt"):
        x = _vec(b["x"])[None, :]
        e1, e2 = _expr(b["eps_pre"]), _expr(b["eps_qk"])
        ones_q, ones_k = np.ones(2), np.ones(1)
        yq, yk = o.qk_chain(x, None, ELIM_WQ, ELIM_WK, ones_q, ones_k, e1, e2)
        _close(yq[0], _vec(b["chain_q"]), rtol=1e-14)
        _close(yk[0], _vec(b["chain_k"]), rtol=1e-14)
        for mode in ("plain", "exact"):
            yq, yk = o.qk_eliminated(x, ELIM_WQ, ELIM_WK, ones_q, ones_k, e2, e1,
                                     exact=(mode == "exact"))
            _close(yq[0], _vec(b[mode + "_q"]), rtol=1e-14)
            _close(yk[0], _vec(b[mode + "_k"]), rtol=1e-14)


def _elim_case(seed, scale=1.0):
    rng = np.random.default_rng(seed)
    T, K, nq, nk = 5, 48, 40, 24
    x = rng.normal(0.0, scale, (T, K))
    g1 = rng.normal(1.0, 0.1, K)
    wq = rng.normal(0.0, 0.1, (K, nq))
    wk = rng.normal(0.0, 0.1, (K, nk))
    gq = rng.normal(1.0, 0.05, nq)
    gk = rng.normal(1.0, 0.05, nk)
    return x, g1, wq, wk, gq, gk


def pin_elimination_identities(o):
    """Scale invariance: with eps_qk = 0 the pre-norm cancels; the exact form equals the chain
    for any epsilons; the plain form equals the chain run with eps_qk / (mean(x^2) + eps_pre)
    per token; in the small-activation regime the plain form visibly differs."""
    x, g1, wq, wk, gq, gk = _elim_case(21)
    wqf, wkf = g1[:, None] * wq, g1[:, None] * wk
    for e1 in (0.0, 1e-2, 0.7):
        cq, ck = o.qk_chain(x, g1, wq, wk, gq, gk, e1, 0.0)
        for exact in (False, True):
            pq, pk = o.qk_eliminated(x, wqf, wkf, gq, gk, 0.0, e1, exact=exact)
            _close(pq, cq, rtol=1e-12)
            _close(pk, ck, rtol=1e-12)
    e1, e2 = 1e-2, 0.3
    cq, ck = o.qk_chain(x, g1, wq, wk, gq, gk, e1, e2)
    pq, pk = o.qk_eliminated(x, wqf, wkf, gq, gk, e2, e1, exact=True)
    _close(pq, cq, rtol=1e-12)
    _close(pk, ck, rtol=1e-12)
    pq, pk = o.qk_eliminated(x, wqf, wkf, gq, gk, e2, e1, exact=False)
    m1 = (x * x).mean(axis=1)
    for t in range(x.shape[0]):
        rq, rk = o.qk_chain(x[t:t + 1], g1, wq, wk, gq, gk, e1, e2 / (m1[t] + e1))
        _close(pq[t], rq[0], rtol=1e-12)
        _close(pk[t], rk[0], rtol=1e-12)
    xs = x * 1e-3
    cq, _ = o.qk_chain(xs, g1, wq, wk, gq, gk, 1e-6, 1e-6)
    pq, _ = o.qk_eliminated(xs, wqf, wkf, gq, gk, 1e-6, 1e-6, exact=False)
    assert np.max(np.abs(pq - cq) / np.abs(cq)) > 1e-2


def pin_elimination_library(o):
    """The chain and the eliminated form against torch's fp64 rms_norm and matmul."""
    import torch

    F = torch.nn.functional
    x, g1, wq, wk, gq, gk = _elim_case(22)
    X, G1, WQ, WK = (torch.from_numpy(a) for a in (x, g1, wq, wk))
    GQ, GK = torch.from_numpy(gq), torch.from_numpy(gk)
    e1, e2 = 1e-3, 0.05
    h = F.rms_norm(X, (x.shape[1],), G1, eps=e1)
    rq = F.rms_norm(h @ WQ, (wq.shape[1],), GQ, eps=e2).numpy()
    rk = F.rms_norm(h @ WK, (wk.shape[1],), GK, eps=e2).numpy()
    cq, ck = o.qk_chain(x, g1, wq, wk, gq, gk, e1, e2)
    _close(cq, rq, rtol=1e-12)
    _close(ck, rk, rtol=1e-12)
    wqf, wkf = g1[:, None] * wq, g1[:, None] * wk
    rq = F.rms_norm(X @ torch.from_numpy(wqf), (wq.shape[1],), GQ, eps=e2).numpy()
    rk = F.rms_norm(X @ torch.from_numpy(wkf), (wk.shape[1],), GK, eps=e2).numpy()
    pq, pk = o.qk_eliminated(x, wqf, wkf, gq, gk, e2, e1, exact=False)
    _close(pq, rq, rtol=1e-12)
    _close(pk, rk, rtol=1e-12)


# --------------------------------------------------------------------------- LayerNorm
def pin_layernorm_worked(o):
    for b in load_blocks("layernorm_worked.txt"):
        x, g, be, eps = _vec(b["x"]), _vec(b["gamma"]), _vec(b["beta"]), _expr(b["eps"])
        w, wf = _mat(b["w"]), _mat(b["wfold"])
        _close(o.layernorm_rows(x[None, :], g, be, eps)[0], _vec(b["ln"]), rtol=1e-14,
               atol=1e-15)
        _close(o.fold_weight(w, g), wf, atol=0)
        _close(o.colsum(wf), _vec(b["colsum"]), atol=0)
        _close(o.matmul(be[None, :], w)[0], _vec(b["bias"]), atol=0)
        y = _vec(b["y"])
        _close(o.normproj_layernorm(x[None, :], wf, _vec(b["colsum"]), _vec(b["bias"]), eps)[0],
               y, rtol=1e-14, atol=1e-15)
        _close(o.layernorm_proj_unfused(x[None, :], g, be, w, eps)[0], y, rtol=1e-14,
               atol=1e-15)


def pin_layernorm_library(o):
    """LayerNorm, LayerNorm-then-project and its deferred form against torch's fp64
    layer_norm and matmul, with K != N (a transposed operand cannot pass)."""
    import torch

    F = torch.nn.functional
    rng = np.random.default_rng(23)
    T, K, N = 6, 56, 40
    x = rng.normal(0.7, 2.0, (T, K))
    g = rng.normal(1.0, 0.1, K)
    be = rng.normal(0.0, 0.5, K)
    w = rng.normal(0.0, 0.05, (K, N))
    for eps in (0.0, 1e-5, 0.4):
        ln = F.layer_norm(torch.from_numpy(x), (K,), torch.from_numpy(g), torch.from_numpy(be),
                          eps=eps)
        _close(o.layernorm_rows(x, g, be, eps), ln.numpy(), rtol=1e-12, atol=1e-14)
        ref = (ln @ torch.from_numpy(w)).numpy()
        _close(o.layernorm_proj_unfused(x, g, be, w, eps), ref, rtol=1e-11, atol=1e-13)
        wf = o.fold_weight(w, g)
        y = o.normproj_layernorm(x, wf, o.colsum(wf), o.matmul(be[None, :], w)[0], eps)
        _close(y, ref, rtol=1e-11, atol=1e-13)
    _close(o.colsum(w), w.sum(axis=0), rtol=1e-13, atol=1e-15)
    # no beta: the bias is optional and means zero
    ln = F.layer_norm(torch.from_numpy(x), (K,), torch.from_numpy(g), None, eps=1e-5).numpy()
    _close(o.layernorm_rows(x, g, None, 1e-5), ln, rtol=1e-12, atol=1e-14)
    wf = o.fold_weight(w, g)
    _close(o.normproj_layernorm(x, wf, o.colsum(wf), None, 1e-5), ln @ w, rtol=1e-11,
           atol=1e-13)


def pin_layernorm_invariants(o):
    rng = np.random.default_rng(24)
    T, d = 5, 301
    x = rng.normal(0.0, 1.5, (T, d))
    g = rng.normal(1.0, 0.3, d)
    be = rng.normal(0.0, 1.0, d)
    eps = 0.2
    y = o.layernorm_rows(x, g, be, eps)
    # invariant to a per-row shift
    _close(o.layernorm_rows(x + 3.0, g, be, eps), y, rtol=1e-11, atol=1e-12)
    # scale invariance at eps = 0: LN(c x) - beta = sign(c) (LN(x) - beta)
    y0 = o.layernorm_rows(x, g, be, 0.0)
    for c in (4.0, -0.5):
        _close(o.layernorm_rows(c * x, g, be, 0.0) - be, math.copysign(1.0, c) * (y0 - be),
               rtol=1e-11, atol=1e-12)
    # normalised values have zero mean and mean square var / (var + eps)
    z = (y - be) / g
    assert np.all(np.abs(z.sum(axis=1)) <= 1e-11 * d)
    var = np.array([np.mean((row - row.mean()) ** 2) for row in x])
    _close((z * z).sum(axis=1), d * var / (var + eps), rtol=1e-12)
    # a constant row maps to beta
    _close(o.layernorm_rows(np.full((2, d), -2.5), g, be, 1e-3), np.tile(be, (2, 1)),
           rtol=1e-15, atol=1e-15)


def pin_layernorm_brute_force_tiny(o):
    """d in 2..4, integer rows in {-2..2}^d that are not constant, eps = 0, gamma = 1,
    beta = 0: y_i^2 = (x_i - mu)^2 d / sum (x - mu)^2 exactly (rational arithmetic)."""
    for d in range(2, 5):
        xs = np.array([v for v in product(range(-2, 3), repeat=d) if len(set(v)) > 1],
                      dtype=np.float64)
        y = o.layernorm_rows(xs, None, None, 0.0)
        for row, yr in zip(xs, y):
            mu = sum(Fraction(int(v)) for v in row) / d
            ss = sum((Fraction(int(v)) - mu) ** 2 for v in row)
            for v, yv in zip(row, yr):
                exact = (Fraction(int(v)) - mu) ** 2 * d / ss
                assert abs(yv * yv - float(exact)) <= 4e-15 * max(1.0, float(exact)), (row, d)


ALL_PINS = [pin_rmsnorm_worked, pin_decomposition_worked, pin_flashnorm_worked,
            pin_bf16_rounding, pin_constant_vector, pin_eps_small_rows, pin_invariants,
            pin_sumsq_exact, pin_brute_force_tiny, pin_decomposition_random,
            pin_torch_rms_norm, pin_normproj_library, pin_bf16_widening, pin_bf16_rne_library,
            pin_elimination_worked, pin_elimination_identities, pin_elimination_library,
            pin_layernorm_worked, pin_layernorm_library, pin_layernorm_invariants,
            pin_layernorm_brute_force_tiny]
