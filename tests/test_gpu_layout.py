"""GPU parity of the norm-then-project calls for the weight layout they take and for operands
at any alignment, against the fp64 oracle.

The folded weight W' = diag(gamma) W is row-major [K, N] like W ("FlashNorm: Fast
Normalization for Transformers", abstract, item (i): gamma is merged into the next linear
layer's weights; item (ii): the 1/RMS scale is applied after the product). Square weights that
are not symmetric catch a transposed read on every kernel (matrix-vector, 128 x 128 tiles,
256 x 256 tiles with k-tiles of 64 and 32). Odd K, odd row strides and pointers one element
past a 16-byte boundary run the element-load kernel."""

import numpy as np
import pytest

import oracle
from helpers import check_projection, check_rows, to_dev, to_host, widen
from layerwise_qk_norm_amd import inputs

pytestmark = pytest.mark.gpu


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


def sample_rows(T, n=192, seed=0):
    if T <= n + 2:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, n, replace=False)]))


def bound(x_bits, wf_bits, eps):
    x, wf = widen(x_bits), widen(wf_bits)
    r = 1.0 / np.sqrt((x * x).mean(axis=1) + eps)
    return r[:, None] * (np.abs(x) @ np.abs(wf))


def oracle_folded(w, g):
    """W' = diag(gamma) W in fp64 by the oracle, rounded once to bf16: [K, N] bits."""
    return oracle.round_bf16(oracle.fold_weight(w, g))


@pytest.mark.parametrize("T,K", [(8, 512), (300, 768), (2048, 1024), (8192, 1024),
                                 (4096, 4096), (4096, 4128)])
def test_square_weight_is_read_row_major(Q, T, K):
    """K == N with a W' built by the oracle and handed over directly (not through the library's
    fold): y must be x W' and not x W'^T. Shapes reach the matrix-vector kernel, the 128 x 128
    tiles with 4 stages and with 2, and the 256 x 256 tiles with k-tiles of 64 and of 32."""
    rng = np.random.default_rng(T + K)
    x = inputs.random_rows(rng, T, K, "bf16")
    w = inputs.random_rows(rng, K, K, "bf16", scale=0.02)
    g = inputs.random_gamma(rng, K, "bf16", sd=0.3)
    wf = oracle_folded(w, g)
    assert not np.array_equal(wf, wf.T)
    y = Q.normproj_deferred(to_dev(x), to_dev(wf), eps=1e-6)
    sync()
    rows = sample_rows(T, seed=T)
    xs = np.ascontiguousarray(x[rows])
    check_projection(to_host(y)[rows], oracle.normproj(xs, wf, 1e-6), bound(xs, wf, 1e-6),
                     f"square T={T} K=N={K}")


def test_fold_layout_in_place_and_strided(Q):
    """The fold writes [K, N] like W: bit-exact against the oracle's fp64 fold rounded once, with
    an odd output stride and an output one element past a 16-byte boundary, and in place."""
    import torch

    rng = np.random.default_rng(77)
    K, N = 300, 130
    w = inputs.random_rows(rng, K, N, "bf16", scale=0.02)
    for gdt in ("bf16", "f32"):
        g = inputs.random_gamma(rng, K, gdt)
        ref = oracle_folded(w, g)
        buf = torch.full((K, N + 3), 5.0, dtype=torch.bfloat16, device="cuda")
        Q.normproj_fold_weight(to_dev(w), to_dev(g), w_fold=buf[:, 1:N + 1])
        wd = to_dev(w)
        Q.normproj_fold_weight(wd, to_dev(g), w_fold=wd)
        sync()
        got = to_host(buf)
        assert np.array_equal(got[:, 1:N + 1], ref), gdt
        assert np.all(widen(got[:, :1]) == 5.0) and np.all(widen(got[:, N + 1:]) == 5.0)
        assert np.array_equal(to_host(wd), ref), f"in place {gdt}"


def misaligned(rng, rows, cols, scale=1.0, off=1, pad=3):
    """A [rows, cols] bf16 operand as a view starting `off` elements into a [rows, cols + pad]
    buffer: row stride cols + pad, base 2 * off bytes past a 16-byte boundary."""
    full = inputs.random_rows(rng, rows, cols + pad, "bf16", scale=scale)
    return full, to_dev(full)[:, off:off + cols], np.ascontiguousarray(full[:, off:off + cols])


@pytest.mark.parametrize("T,K,N", [(5, 1001, 130), (300, 1001, 264), (16, 1024, 520),
                                   (200, 1024, 520), (33, 8, 24), (130, 2051, 72)])
def test_deferred_any_alignment(Q, T, K, N):
    """x, W' and y one element past a 16-byte boundary with odd row strides, odd K: every
    shape runs (no alignment status) and matches the oracle; y's padding stays untouched."""
    import torch

    rng = np.random.default_rng(T * 7 + K + N)
    _, xd, x = misaligned(rng, T, K)
    w = inputs.random_rows(rng, K, N, "bf16", scale=0.02)
    g = inputs.random_gamma(rng, K, "bf16")
    wf = oracle_folded(w, g)
    wbuf = torch.zeros((K, N + 5), dtype=torch.bfloat16, device="cuda")
    wbuf[:, 1:N + 1] = to_dev(wf)
    ybuf = torch.full((T, N + 7), 3.0, dtype=torch.bfloat16, device="cuda")
    Q.normproj_deferred(xd, wbuf[:, 1:N + 1], eps=1e-6, y=ybuf[:, 1:N + 1])
    sync()
    yh = to_host(ybuf)
    assert np.all(widen(yh[:, :1]) == 3.0) and np.all(widen(yh[:, N + 1:]) == 3.0)
    rows = sample_rows(T, seed=K)
    xs = np.ascontiguousarray(x[rows])
    check_projection(np.ascontiguousarray(yh[rows, 1:N + 1]), oracle.normproj(xs, wf, 1e-6),
                     bound(xs, wf, 1e-6), f"misaligned T={T} K={K} N={N}")


@pytest.mark.parametrize("T,K,N", [(7, 1001, 130), (300, 1001, 264), (260, 1024, 512)])
def test_layernorm_and_unfused_any_alignment(Q, T, K, N):
    """The deferred LayerNorm (with and without the workspace), the unfused RMSNorm and
    LayerNorm baselines with misaligned x, odd K, and gamma / beta one element off."""
    import torch

    rng = np.random.default_rng(5 * T + K)
    _, xd, x = misaligned(rng, T, K, scale=1.0)
    w = inputs.random_rows(rng, K, N, "bf16", scale=0.02)
    gfull = inputs.random_gamma(rng, K + 1, "bf16")
    bfull = inputs.random_gamma(rng, K + 1, "bf16", sd=0.05)
    g, b = gfull[1:], bfull[1:]
    gd, bd = to_dev(gfull)[1:], to_dev(bfull)[1:]
    rows = sample_rows(T, seed=N)
    xs = np.ascontiguousarray(x[rows])

    # deferred LayerNorm: fold, then the product with and without the statistics workspace
    wf, cs, bias = Q.normproj_fold_layernorm(to_dev(w), gd, bd)
    wf_ref = oracle_folded(w, g)
    sync()
    assert np.array_equal(to_host(wf), wf_ref)
    cs_ref = oracle.colsum(wf_ref)
    b_ref = oracle.matmul(b[None, :], w)[0]
    ref = oracle.normproj_layernorm(xs, wf_ref, cs_ref, b_ref, 1e-5)
    xw = widen(xs)
    mu = xw.mean(axis=1)
    r = 1.0 / np.sqrt(((xw - mu[:, None]) ** 2).mean(axis=1) + 1e-5)
    lb = r[:, None] * (np.abs(xw) @ np.abs(widen(wf_ref)) +
                       np.abs(mu)[:, None] * np.abs(widen(wf_ref)).sum(0))
    for stats in ("auto", None):
        y = Q.normproj_deferred_layernorm(xd, wf, cs, bias, eps=1e-5, row_stats=stats)
        sync()
        check_projection(to_host(y)[rows], ref, lb, f"layernorm stats={stats}")

    # unfused RMSNorm baseline: RMSNorm launch into xn, plain product with W
    xn, y = Q.normproj_unfused(xd, gd, to_dev(w), eps=1e-6)
    sync()
    check_rows(to_host(xn), oracle.rmsnorm_rows(x, g, 1e-6), "unfused xn")
    xn_ref = oracle.round_bf16(oracle.rmsnorm_rows(xs, g, 1e-6))
    check_projection(to_host(y)[rows], oracle.matmul(xn_ref, w),
                     np.abs(widen(xn_ref)) @ np.abs(widen(w)), "unfused y", abs_coeff=2.0 ** -12)

    # unfused LayerNorm baseline (element path: gamma and beta are 2 bytes off)
    xn, y = Q.normproj_layernorm_unfused(xd, gd, bd, to_dev(w), eps=1e-5)
    sync()
    ln_ref = oracle.layernorm_rows(xs, g, b, 1e-5)
    # a LayerNorm output can sit near zero: the bound adds the fp32 rounding of the normalised
    # value (as in the aligned baseline's test)
    absb = (np.abs(xw) + np.abs(mu)[:, None]) * r[:, None] * np.abs(widen(g)) + np.abs(widen(b))
    check_projection(to_host(xn)[rows], ln_ref, absb, "ln unfused xn", abs_coeff=2.0 ** -16)
    xn_ref = oracle.round_bf16(ln_ref)
    check_projection(to_host(y)[rows], oracle.matmul(xn_ref, w),
                     np.abs(widen(xn_ref)) @ np.abs(widen(w)), "ln unfused y",
                     abs_coeff=2.0 ** -12)


def test_eliminated_any_alignment(Q):
    """The pre-norm elimination with odd K and x one element off (element-load product, then
    the in-place QK-Norm launch) against the oracle's eliminated form."""
    rng = np.random.default_rng(1234)
    T, K, nq, nk = 40, 1001, 256, 136
    c = inputs.make_elimination_case(T, seed=9, K=K, nq=nq, nk=nk)
    full = np.zeros((T, K + 2), dtype=np.uint16)
    full[:, 1:K + 1] = c["x"]
    xd = to_dev(full)[:, 1:K + 1]
    wqk = Q.normproj_fold_weight(to_dev(c["w"]), to_dev(c["gamma_pre"]))
    y = Q.qknorm_project_eliminated(xd, wqk, nq, to_dev(c["gamma_q"]), to_dev(c["gamma_k"]),
                                    eps_qk=c["eps_qk"], eps_pre=c["eps_pre"], exact=True)
    sync()
    wf = oracle_folded(c["w"], c["gamma_pre"])
    assert np.array_equal(to_host(wqk), wf)
    rq, rk = oracle.qk_eliminated(c["x"], np.ascontiguousarray(wf[:, :nq]),
                                  np.ascontiguousarray(wf[:, nq:]), c["gamma_q"], c["gamma_k"],
                                  c["eps_qk"], c["eps_pre"], exact=True)
    ref = np.concatenate([rq, rk], axis=1)
    x, wfw = widen(c["x"]), widen(wf)
    p = x @ wfw
    m1 = (x * x).mean(axis=1)
    e = c["eps_qk"] * (m1 + c["eps_pre"])
    sq = 1.0 / np.sqrt((p[:, :nq] ** 2).mean(axis=1) + e)
    sk = 1.0 / np.sqrt((p[:, nq:] ** 2).mean(axis=1) + e)
    gam = np.concatenate([widen(c["gamma_q"]), widen(c["gamma_k"])])
    s = np.concatenate([np.repeat(sq[:, None], nq, 1), np.repeat(sk[:, None], nk, 1)], 1)
    check_projection(to_host(y), ref, s * np.abs(gam)[None, :] * (np.abs(x) @ np.abs(wfw)),
                     "eliminated misaligned")


def strided_rows(x_host, ld):
    """A device tensor viewing x_host's rows at row stride ld (elements) inside one buffer of
    rows x ld; the columns past x_host's width are left unwritten."""
    import torch

    T, K = x_host.shape
    buf = torch.empty((T, ld), dtype=torch.bfloat16, device="cuda")
    view = buf[:, :K]
    view.copy_(to_dev(x_host))
    return buf, view


@pytest.mark.parametrize("T,K,N,ldx,ldw", [
    # 256 x 256 tiles: per-lane DMA offsets up to 255 * (2^23 - 8) * 2 bytes, past 2^31
    (512, 64, 32768, (1 << 23) - 8, None),
    # strides from 2^23 elements take the element-load kernel
    (300, 256, 264, 1 << 23, None),
    (300, 64, 264, None, 1 << 23),
    # the matrix-vector form: W' offsets up to 63 * (2^25 - 8) * 2 bytes; from 2^25 elements on,
    # the element kernel
    (16, 64, 264, None, (1 << 25) - 8),
    (16, 64, 264, None, 1 << 25),
    (16, 64, 264, (1 << 25) - 8, None),
])
def test_deferred_huge_row_strides(Q, T, K, N, ldx, ldw):
    """Row strides near and past the 32-bit offset range of the pipelined and matrix-vector
    kernels (buffers of up to 8.6 GB): the offsets stay unsigned, and larger strides route to
    the element kernel."""
    import torch

    rng = np.random.default_rng(K + N)
    x = inputs.random_rows(rng, T, K, "bf16")
    w = inputs.random_rows(rng, K, N, "bf16", scale=0.02)
    g = inputs.random_gamma(rng, K, "bf16")
    wf = oracle_folded(w, g)
    xbuf, xd = strided_rows(x, ldx) if ldx else (None, to_dev(x))
    wbuf, wd = strided_rows(wf, ldw) if ldw else (None, to_dev(wf))
    y = Q.normproj_deferred(xd, wd, eps=1e-6)
    sync()
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 254, 255, T - 2, T - 1],
                                     np.random.default_rng(1).choice(T, 24)]) % T)
    xs = np.ascontiguousarray(x[rows])
    check_projection(to_host(y)[rows], oracle.normproj(xs, wf, 1e-6), bound(xs, wf, 1e-6),
                     f"strides T={T} K={K} N={N} ldx={ldx} ldw={ldw}")
    del xbuf, wbuf, xd, wd, y
    torch.cuda.empty_cache()


def test_row_kernels_huge_row_strides(Q):
    """Row strides of 2^26 + 8 elements (5.4 GB buffers): row offsets past 2^32 bytes in the
    fused, partial-sum and single-launch shard kernels."""
    import torch

    rng = np.random.default_rng(5)
    T, d, ld = 40, 4096, (1 << 26) + 8
    q = inputs.random_rows(rng, T, d, "bf16")
    g = inputs.random_gamma(rng, d, "bf16")
    qbuf, qd = strided_rows(q, ld)
    obuf, od = strided_rows(np.zeros((T, d), np.uint16), ld)
    Q.qknorm_fused(qd, to_dev(g), q_out=od)
    psq, _ = Q.qknorm_partial_sumsq(qd)
    sync()
    check_rows(to_host(od), oracle.rmsnorm_rows(q, g, 1e-6), "fused, huge stride")
    ref_psq = oracle.partial_sumsq(q)
    assert np.all(np.abs(to_host(psq) - ref_psq) <= 1e-5 * ref_psq)
    # the shard stage takes slices of up to 2048 bf16 columns: the first half of each row
    ds = 2048
    qs, gs = np.ascontiguousarray(q[:, :ds]), g[:ds]
    ext = rng.chisquare(ds, size=(3, T)).astype(np.float32)
    mail = Q.mailbox_words(3, T)
    Q.qknorm_shard_publish(to_dev(ext), mail, 4)
    od.zero_()
    Q.qknorm_shard_fused(qd[:, :ds], to_dev(gs), mail, 4 * ds, eps=1e-6, epoch=4,
                         q_out=od[:, :ds])
    sync()
    check_rows(to_host(od[:, :ds]),
               oracle.apply_with_stats(qs, gs, oracle.partial_sumsq(qs), ext, 4 * ds, 1e-6),
               "shard, huge stride")
    del qbuf, obuf, qd, od
    torch.cuda.empty_cache()
