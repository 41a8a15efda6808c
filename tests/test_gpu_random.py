"""GPU parity on a seeded sweep of random configurations, against the fp64 oracle: breadth
beyond the hand-picked cases. Each case draws its own shapes, storage types, row strides,
pointer offsets (elements past a 16-byte boundary), in-place use, peer counts and epsilon from
a fixed seed, so every run checks the same configurations and a failure names its case.
QKN_RANDOM_SEED_BASE (default 0) shifts every seed, to sweep another set of configurations.

Operations: layerwise QK-Norm in one launch, its scalar-statistics split (partial sums, then
aggregation and scale) and the single-launch shard stage ("SwiftQK: Fast and
Communication-Efficient Tensor Parallelism for Query-Key Normalization", abstract), the
deferred norm-then-project products, RMSNorm and LayerNorm, and the projection with the
pre-norm eliminated ("FlashNorm: Fast Normalization for Transformers", abstract). Outputs'
padding around the written views must stay untouched."""

import os

import numpy as np
import pytest

import oracle
from helpers import check_projection, check_rows, to_host, widen
from layerwise_qk_norm_amd import inputs

pytestmark = pytest.mark.gpu

SENTINEL = 5.0
SEED_BASE = int(os.environ.get("QKN_RANDOM_SEED_BASE", "0"))


@pytest.fixture(scope="module")
def Q():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import layerwise_qk_norm_amd as Q

    Q.lib()
    return Q


def sync():
    import torch

    torch.cuda.synchronize()


def tdtype(dtype):
    import torch

    return torch.bfloat16 if dtype == "bf16" else torch.float32


def place(host, dtype, off, pad):
    """A device buffer [rows, off + cols + pad] filled with SENTINEL, host copied into columns
    off .. off + cols; returns (buffer, view). 1-D host arrays become 1-D views."""
    import torch

    h = np.ascontiguousarray(host)
    if h.ndim == 1:
        buf = torch.full((off + h.shape[0] + pad,), SENTINEL, dtype=tdtype(dtype), device="cuda")
        view = buf[off:off + h.shape[0]]
    else:
        rows, cols = h.shape
        buf = torch.full((rows, off + cols + pad), SENTINEL, dtype=tdtype(dtype), device="cuda")
        view = buf[:, off:off + cols]
    src = torch.from_numpy(h.view(np.int16) if h.dtype == np.uint16 else h)
    if h.dtype == np.uint16:
        src = src.view(tdtype("bf16"))
    view.copy_(src.to("cuda"))
    return buf, view


def padding_intact(buf, off, cols, what):
    b = widen(to_host(buf))
    if b.ndim == 1:
        rest = np.concatenate([b[:off], b[off + cols:]])
    else:
        rest = np.concatenate([b[:, :off].ravel(), b[:, off + cols:].ravel()])
    assert np.all(rest == SENTINEL), f"{what}: padding written"


def width(rng, dtype, hi):
    """Half the time a whole number of 16-byte vectors, otherwise any width."""
    epv = 8 if dtype == "bf16" else 4
    if rng.random() < 0.5:
        return int(rng.integers(1, max(2, hi // epv))) * epv
    return int(rng.integers(1, hi))


def layout(rng):
    """(offset, padding) of a row-major operand: aligned and tight, or shifted and padded."""
    if rng.random() < 0.4:
        return 0, int(rng.choice([0, 0, 8, 64]))
    return int(rng.choice([1, 2, 3, 5])), int(rng.choice([0, 1, 7, 13]))


# ----------------------------------------------------------------------------- fused Q + K
@pytest.mark.parametrize("case", range(80))
def test_random_fused(Q, case):
    rng = np.random.default_rng(SEED_BASE + 7000 + case)
    dtype = str(rng.choice(["bf16", "f32"]))
    gdtype = str(rng.choice(["bf16", "f32"]))
    T = int(rng.integers(1, 300))
    dq = width(rng, dtype, 9000)
    has_k = rng.random() < 0.7
    dk = width(rng, dtype, 5000) if has_k else 0
    eps = float(rng.choice([1e-6, 1e-5, 0.0]))
    inplace = rng.random() < 0.25
    what = (f"case {case} (seed base {SEED_BASE}): {dtype}/{gdtype} T={T} dq={dq} dk={dk} "
            f"eps={eps} inplace={inplace}")
    q = inputs.random_rows(rng, T, dq, dtype, scale=float(rng.uniform(0.1, 3.0)))
    gq = inputs.random_gamma(rng, dq, gdtype)
    (qo_off, qo_pad), (q_off, q_pad), g_off = layout(rng), layout(rng), int(rng.integers(0, 3))
    qbuf, qd = place(q, dtype, q_off, q_pad)
    _, gqd = place(gq, gdtype, g_off, 1)
    if inplace:
        qobuf, qod, qo_off = qbuf, qd, q_off
    else:
        qobuf, qod = place(np.zeros_like(q), dtype, qo_off, qo_pad)
    args = dict(eps=eps, q_out=qod)
    if has_k:
        k = inputs.random_rows(rng, T, dk, dtype, scale=float(rng.uniform(0.1, 3.0)))
        gk = inputs.random_gamma(rng, dk, gdtype)
        _, kd = place(k, dtype, *layout(rng))
        _, gkd = place(gk, gdtype, int(rng.integers(0, 3)), 0)
        kobuf, kod = place(np.zeros_like(k), dtype, 3, 2)
        args.update(k=kd, gamma_k=gkd, k_out=kod)
    Q.qknorm_fused(qd, gqd, **args)
    sync()
    check_rows(to_host(qod), oracle.rmsnorm_rows(q, gq, eps), what + " Q")
    padding_intact(qobuf, qo_off, dq, what + " Q")
    if has_k:
        check_rows(to_host(kod), oracle.rmsnorm_rows(k, gk, eps), what + " K")
        padding_intact(kobuf, 3, dk, what + " K")


# ----------------------------------------------------------------------------- split stage
@pytest.mark.parametrize("case", range(48))
def test_random_split(Q, case):
    """Partial sums of a slice, then aggregation with n_ext peers' fp32 partials (a row slice of
    a wider buffer) and the scale over the full width."""
    rng = np.random.default_rng(SEED_BASE + 8000 + case)
    dtype = str(rng.choice(["bf16", "f32"]))
    gdtype = str(rng.choice(["bf16", "f32"]))
    T = int(rng.integers(1, 400))
    dl = width(rng, dtype, 5000)
    n_ext = int(rng.integers(0, 24))
    eps = float(rng.choice([1e-6, 1e-5]))
    what = f"case {case} (seed base {SEED_BASE}): {dtype}/{gdtype} T={T} d_local={dl} n_ext={n_ext}"
    x = inputs.random_rows(rng, T, dl, dtype)
    g = inputs.random_gamma(rng, dl, gdtype)
    ext = rng.chisquare(dl, size=(n_ext, T)).astype(np.float32)
    d_full = dl * (n_ext + 1)
    _, xd = place(x, dtype, *layout(rng))
    _, gd = place(g, gdtype, int(rng.integers(0, 3)), 0)
    psq, _ = Q.qknorm_partial_sumsq(xd)
    sync()
    ref_psq = oracle.partial_sumsq(x)
    check_rows(to_host(psq), ref_psq, what + " partial sums")
    ext_d = place(ext, "f32", 0, int(rng.integers(0, 40)))[1] if n_ext else None
    obuf, od = place(np.zeros_like(x), dtype, 1, 3)
    Q.qknorm_apply_with_stats(xd, gd, psq, ext_d, d_full, eps=eps, q_out=od)
    sync()
    check_rows(to_host(od), oracle.apply_with_stats(x, g, ref_psq, ext if n_ext else None,
                                                     d_full, eps), what + " apply")
    padding_intact(obuf, 1, dl, what)


# ----------------------------------------------------------------------------- shard stage
@pytest.mark.parametrize("case", range(48))
def test_random_shard(Q, case):
    """The single-launch shard stage with a published mailbox, the mailbox checked or taken as
    complete, either residency policy, Q alone or Q and K."""
    import torch

    rng = np.random.default_rng(SEED_BASE + 9000 + case)
    dtype = str(rng.choice(["bf16", "f32"]))
    gdtype = str(rng.choice(["bf16", "f32"]))
    T = int(rng.integers(1, 700))
    dl = width(rng, dtype, 2048 if dtype == "bf16" else 1024)
    n_ext = int(rng.integers(0, 65))
    epoch = int(rng.choice([0, int(rng.integers(1, 1 << 31))]))
    persistent = bool(rng.random() < 0.5)
    has_k = rng.random() < 0.6
    what = (f"case {case} (seed base {SEED_BASE}): {dtype}/{gdtype} T={T} d_local={dl} "
            f"n_ext={n_ext} epoch={epoch} persistent={persistent} k={has_k}")
    x = inputs.random_rows(rng, T, dl, dtype)
    g = inputs.random_gamma(rng, dl, gdtype)
    ext = rng.chisquare(dl, size=(n_ext, T)).astype(np.float32)
    d_full = dl * (n_ext + 1)
    _, xd = place(x, dtype, *layout(rng))
    _, gd = place(g, gdtype, int(rng.integers(0, 3)), 0)
    mail = Q.mailbox_words(n_ext, T)
    pub = epoch if epoch else 3
    if n_ext:
        Q.qknorm_shard_publish(torch.from_numpy(ext).cuda(), mail, pub)
    obuf, od = place(np.zeros_like(x), dtype, 2, 5)
    args = dict(eps=1e-6, q_out=od, epoch=epoch, persistent=persistent)
    if has_k:
        dk = width(rng, dtype, 2048 if dtype == "bf16" else 1024)
        k = inputs.random_rows(rng, T, dk, dtype)
        gk = inputs.random_gamma(rng, dk, gdtype)
        extk = rng.chisquare(dk, size=(n_ext, T)).astype(np.float32)
        mailk = Q.mailbox_words(n_ext, T)
        if n_ext:
            Q.qknorm_shard_publish(torch.from_numpy(extk).cuda(), mailk, pub)
        _, kd = place(k, dtype, *layout(rng))
        kobuf, kod = place(np.zeros_like(k), dtype, 0, 9)
        args.update(k=kd, gamma_k=place(gk, gdtype, 1, 0)[1], mail_k=mailk,
                    dk_full=dk * (n_ext + 1), k_out=kod)
    if epoch:
        args["timed_out"] = torch.zeros((1,), dtype=torch.int32, device="cuda")
    _, _, psq, psq_k = Q.qknorm_shard_fused(xd, gd, mail, d_full, **args)
    sync()
    if epoch:
        assert int(args["timed_out"].item()) == 0, what
    ref_psq = oracle.partial_sumsq(x)
    check_rows(to_host(Q.mailbox_values(psq[None, :]))[0], ref_psq, what + " own partial")
    assert np.all(to_host(Q.mailbox_epochs(psq)) == epoch), what
    check_rows(to_host(od), oracle.apply_with_stats(x, g, ref_psq, ext if n_ext else None,
                                                     d_full, 1e-6), what + " Q")
    padding_intact(obuf, 2, dl, what + " Q")
    if has_k:
        ref_k = oracle.partial_sumsq(k)
        check_rows(to_host(kod), oracle.apply_with_stats(k, gk, ref_k, extk if n_ext else None,
                                                          dk * (n_ext + 1), 1e-6), what + " K")
        padding_intact(kobuf, 0, dk, what + " K")


# ----------------------------------------------------------------------------- products
def rms_bound(x_bits, wf_bits, eps):
    x, wf = widen(x_bits), widen(wf_bits)
    r = 1.0 / np.sqrt((x * x).mean(axis=1) + eps)
    return r[:, None] * (np.abs(x) @ np.abs(wf))


def ln_bound(x_bits, wf_bits, eps):
    x, wf = widen(x_bits), widen(wf_bits)
    mu = x.mean(axis=1)
    r = 1.0 / np.sqrt(((x - mu[:, None]) ** 2).mean(axis=1) + eps)
    return r[:, None] * (np.abs(x) @ np.abs(wf) + np.abs(mu)[:, None] * np.abs(wf).sum(axis=0))


def product_shape(rng):
    T = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 700)),
                        int(rng.integers(700, 2600))]))
    K = width(rng, "bf16", 3000)
    N = width(rng, "bf16", 2200)
    return T, K, N


def sample(T, rng, n=40):
    if T <= n:
        return np.arange(T)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, n, replace=False)]))


@pytest.mark.parametrize("case", range(48))
def test_random_deferred(Q, case):
    """The fold, then the deferred RMSNorm product: x, W' and y at random offsets and row
    strides; the matrix-vector, element-load and 128 x 128 kernels are each reached by some
    draw (the 256 x 256 ones need more tiles than these shapes give)."""
    rng = np.random.default_rng(SEED_BASE + 10000 + case)
    T, K, N = product_shape(rng)
    what = f"case {case} (seed base {SEED_BASE}): T={T} K={K} N={N}"
    x = inputs.random_rows(rng, T, K, "bf16")
    w = inputs.random_rows(rng, K, N, "bf16", scale=0.02)
    g = inputs.random_gamma(rng, K, "bf16")
    wf_ref = oracle.round_bf16(oracle.fold_weight(w, g))
    (w_off, w_pad), (wf_off, wf_pad) = layout(rng), layout(rng)
    _, wd = place(w, "bf16", w_off, w_pad)
    wfbuf, wfd = place(np.zeros_like(w), "bf16", wf_off, wf_pad)
    Q.normproj_fold_weight(wd, place(g, "bf16", int(rng.integers(0, 3)), 0)[1], w_fold=wfd)
    _, xd = place(x, "bf16", *layout(rng))
    y_off, y_pad = layout(rng)
    ybuf, yd = place(np.zeros((T, N), np.uint16), "bf16", y_off, y_pad)
    Q.normproj_deferred(xd, wfd, eps=1e-6, y=yd)
    sync()
    assert np.array_equal(to_host(wfd), wf_ref), what + " fold"
    padding_intact(wfbuf, wf_off, N, what + " fold")
    rows = sample(T, rng)
    xs = np.ascontiguousarray(x[rows])
    check_projection(to_host(yd)[rows], oracle.normproj(xs, wf_ref, 1e-6),
                     rms_bound(xs, wf_ref, 1e-6), what)
    padding_intact(ybuf, y_off, N, what + " y")


@pytest.mark.parametrize("case", range(32))
def test_random_deferred_layernorm(Q, case):
    """The LayerNorm fold and the deferred LayerNorm product with beta or without, x with a
    random mean, the statistics from the workspace pass or from inside the product."""
    rng = np.random.default_rng(SEED_BASE + 11000 + case)
    T, K, N = product_shape(rng)
    with_beta = rng.random() < 0.6
    stats = "auto" if rng.random() < 0.5 else None
    mean = float(rng.choice([0.0, 2.0, -3.0]))
    what = (f"case {case} (seed base {SEED_BASE}): T={T} K={K} N={N} beta={with_beta} "
            f"stats={stats} mean={mean}")
    x = inputs.f32_to_bf16_bits((widen(inputs.random_rows(rng, T, K, "bf16")) + mean)
                                .astype(np.float32))
    w = inputs.random_rows(rng, K, N, "bf16", scale=0.02)
    g = inputs.random_gamma(rng, K, "bf16")
    beta = inputs.random_rows(rng, 1, K, "bf16", scale=0.05)[0] if with_beta else None
    wf_ref = oracle.round_bf16(oracle.fold_weight(w, g))
    cs_ref = oracle.colsum(wf_ref)
    b_ref = oracle.matmul(beta[None, :], w)[0] if with_beta else None
    _, wd = place(w, "bf16", *layout(rng))
    wf, cs, b = Q.normproj_fold_layernorm(wd, place(g, "bf16", 1, 0)[1],
                                          place(beta, "bf16", 1, 0)[1] if with_beta else None)
    _, xd = place(x, "bf16", *layout(rng))
    y_off, y_pad = layout(rng)
    ybuf, yd = place(np.zeros((T, N), np.uint16), "bf16", y_off, y_pad)
    Q.normproj_deferred_layernorm(xd, wf, cs, b, eps=1e-5, y=yd, row_stats=stats)
    sync()
    rows = sample(T, rng)
    xs = np.ascontiguousarray(x[rows])
    check_projection(to_host(yd)[rows],
                     oracle.normproj_layernorm(xs, wf_ref, cs_ref, b_ref, 1e-5),
                     ln_bound(xs, wf_ref, 1e-5), what)
    padding_intact(ybuf, y_off, N, what + " y")


def elim_bound(x_bits, wf_bits, g_bits, eps_qk, eps_pre, exact):
    x, wf, g = widen(x_bits), widen(wf_bits), widen(g_bits)
    p = x @ wf
    eps = eps_qk * ((x * x).mean(axis=1) + eps_pre) if exact else np.full(len(x), eps_qk)
    s = 1.0 / np.sqrt((p * p).mean(axis=1) + eps)
    return s[:, None] * np.abs(g)[None, :] * (np.abs(x) @ np.abs(wf))


@pytest.mark.parametrize("case", range(20))
def test_random_eliminated(Q, case):
    """The stacked Q/K projection without the pre-norm, then layerwise QK-Norm of its two
    column blocks ("FlashNorm", abstract, scale invariance), plain or exact, Q alone or with K,
    at random widths and offsets."""
    rng = np.random.default_rng(SEED_BASE + 12000 + case)
    T = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 600))]))
    K = width(rng, "bf16", 1500)
    nq = width(rng, "bf16", 1500)
    nk = width(rng, "bf16", 700) if rng.random() < 0.8 else 0
    exact = bool(rng.random() < 0.5)
    eps_qk, eps_pre = float(rng.choice([1e-6, 1e-5])), float(rng.choice([1e-6, 1e-5]))
    what = f"case {case} (seed base {SEED_BASE}): T={T} K={K} nq={nq} nk={nk} exact={exact}"
    x = inputs.random_rows(rng, T, K, "bf16")
    w = inputs.random_rows(rng, K, nq + nk, "bf16", scale=0.02)
    gp = inputs.random_gamma(rng, K, "bf16")
    gq = inputs.random_gamma(rng, nq, "bf16")
    gk = inputs.random_gamma(rng, nk, "bf16") if nk else None
    wf_ref = oracle.round_bf16(oracle.fold_weight(w, gp))
    _, wd = place(w, "bf16", *layout(rng))
    wqk = Q.normproj_fold_weight(wd, place(gp, "bf16", 1, 0)[1])
    _, xd = place(x, "bf16", *layout(rng))
    y_off, y_pad = layout(rng)
    ybuf, yd = place(np.zeros((T, nq + nk), np.uint16), "bf16", y_off, y_pad)
    Q.qknorm_project_eliminated(xd, wqk, nq, place(gq, "bf16", 2, 0)[1],
                                place(gk, "bf16", 0, 1)[1] if nk else None, eps_qk=eps_qk,
                                eps_pre=eps_pre, exact=exact, y=yd)
    sync()
    rows = sample(T, rng, n=24)
    xs = np.ascontiguousarray(x[rows])
    wq_ref = np.ascontiguousarray(wf_ref[:, :nq])
    if nk:
        wk_ref, gk_h = np.ascontiguousarray(wf_ref[:, nq:]), gk
    else:  # Q only: a one-column K the oracle computes and the check ignores
        wk_ref, gk_h = np.zeros((K, 1), np.uint16), np.zeros(1, np.uint16) + 0x3F80
    rq, rk = oracle.qk_eliminated(xs, wq_ref, wk_ref, gq, gk_h, eps_qk, eps_pre, exact=exact)
    got = to_host(yd)[rows]
    args = (eps_qk, eps_pre, exact)
    check_projection(got[:, :nq], rq, elim_bound(xs, wq_ref, gq, *args), what + " Q")
    if nk:
        check_projection(got[:, nq:], rk, elim_bound(xs, wk_ref, gk, *args), what + " K")
    padding_intact(ybuf, y_off, nq + nk, what + " y")
