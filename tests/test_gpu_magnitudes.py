"""GPU parity at the edges of the fp32 statistics, against the fp64 oracle. Each case mixes
these rows: a zero row, rows whose squares underflow fp32 (eps alone then sets the scale, as it
does in fp64), eps-dominated rows, rows of unit scale, and rows of magnitude 1e15, whose sums of
squares (about 1e33) still fit fp32. They run through the row kernels (fused, the two-launch
split, the single-launch shard stage) and through every kernel of the deferred RMSNorm and
LayerNorm products.

Sums of squares accumulate in fp32 on the device. A row whose sum of squares passes the fp32
range (|x| above about 1e17 at d = 4096) gets 1/rms = 0 there, where the fp64 oracle stays
finite; such rows are outside what these kernels compute and are not exercised here."""

import numpy as np
import pytest

import oracle
from helpers import check_projection, check_rows, to_dev, to_host, widen
from layerwise_qk_norm_amd import inputs

pytestmark = pytest.mark.gpu

# row scales, placed on the first rows and repeated on the last ones
SCALES = (0.0, 1e-30, 3e-20, 1e-4, 1.0, 1e15)


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


def scaled_rows(rng, T, d, dtype):
    """N(0, 1) rows, the first and last len(SCALES) rows multiplied by SCALES; stored as the
    dtype's values (bf16 bits or fp32)."""
    x = widen(inputs.random_rows(rng, T, d, dtype))
    s = np.ones(T)
    n = len(SCALES)
    s[:n] = SCALES
    s[T - n:] = SCALES
    v = (x * s[:, None]).astype(np.float32)
    return inputs.f32_to_bf16_bits(v) if dtype == "bf16" else v


def special_rows(T):
    n = len(SCALES)
    return np.unique(np.concatenate([np.arange(n), np.arange(T - n, T)]))


def check_sumsq(got, ref, d, what):
    """fp32 partial sums of squares: within 1e-5 of the fp64 sum, plus, for squares below the
    fp32 range, the half of the smallest subnormal each of the d products may lose."""
    err = np.abs(got.astype(np.float64) - ref)
    bound = 1e-5 * np.abs(ref) + d * 2.0 ** -150
    assert np.all(err <= bound), f"{what}: worst {err.max()!r} at {int(np.argmax(err - bound))}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_row_magnitudes(Q, dtype):
    rng = np.random.default_rng(101)
    T = 300
    q, k = scaled_rows(rng, T, 4096, dtype), scaled_rows(rng, T, 512, dtype)
    gq, gk = inputs.random_gamma(rng, 4096, dtype), inputs.random_gamma(rng, 512, dtype)
    qo, ko = Q.qknorm_fused(to_dev(q), to_dev(gq), to_dev(k), to_dev(gk), eps=1e-6)
    sync()
    check_rows(to_host(qo), oracle.rmsnorm_rows(q, gq, 1e-6), f"fused Q {dtype}")
    check_rows(to_host(ko), oracle.rmsnorm_rows(k, gk, 1e-6), f"fused K {dtype}")
    assert not np.any(widen(to_host(qo))[0])  # the zero row stays zero


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_and_shard_magnitudes(Q, dtype):
    """TP-4: each row of a [T, 4 * 512] tensor is split into four slices; this rank holds slice
    0 and the peers' partial sums are the oracle's sums of slices 1..3 stored as fp32. Rows
    keep one scale across their slices."""
    rng = np.random.default_rng(102)
    T, dl, n_ext = 300, 512, 3
    full = scaled_rows(rng, T, dl * (n_ext + 1), dtype)
    x = np.ascontiguousarray(full[:, :dl])
    g = inputs.random_gamma(rng, dl, dtype)
    ext = np.stack([oracle.partial_sumsq(np.ascontiguousarray(full[:, (e + 1) * dl:(e + 2) * dl]))
                    for e in range(n_ext)]).astype(np.float32)
    d_full = dl * (n_ext + 1)
    xd = to_dev(x)

    psq, _ = Q.qknorm_partial_sumsq(xd)
    sync()
    ref_psq = oracle.partial_sumsq(x)
    check_sumsq(to_host(psq), ref_psq, dl, f"partial {dtype}")

    psq32 = ref_psq.astype(np.float32)
    yo, _ = Q.qknorm_apply_with_stats(xd, to_dev(g), to_dev(psq32), to_dev(ext), d_full, eps=1e-6)
    sync()
    check_rows(to_host(yo), oracle.apply_with_stats(x, g, psq32, ext, d_full, 1e-6),
               f"apply {dtype}")

    mail = Q.mailbox_words(n_ext, T)
    Q.qknorm_shard_publish(to_dev(ext), mail, 9)
    for persistent in (True, False):
        yo, _, own, _ = Q.qknorm_shard_fused(xd, to_dev(g), mail, d_full, eps=1e-6, epoch=9,
                                             persistent=persistent)
        sync()
        check_sumsq(to_host(Q.mailbox_values(own[None, :]))[0], ref_psq, dl,
                    f"shard own partial {dtype}")
        check_rows(to_host(yo), oracle.apply_with_stats(x, g, ref_psq, ext, d_full, 1e-6),
                   f"shard {dtype} persistent={persistent}")


def rms_bound(x_bits, wf_bits, eps):
    x, wf = widen(x_bits), widen(wf_bits)
    r = 1.0 / np.sqrt((x * x).mean(axis=1) + eps)
    return r[:, None] * (np.abs(x) @ np.abs(wf))


def ln_bound(x_bits, wf_bits, eps):
    x, wf = widen(x_bits), widen(wf_bits)
    mu = x.mean(axis=1)
    r = 1.0 / np.sqrt(((x - mu[:, None]) ** 2).mean(axis=1) + eps)
    return r[:, None] * (np.abs(x) @ np.abs(wf) + np.abs(mu)[:, None] * np.abs(wf).sum(axis=0))


# the matrix-vector form (T <= 16), the element-load tiles (K not a multiple of 32), the
# 128 x 128 pipelined tiles and the 256 x 256 ring
PRODUCT_SHAPES = [(14, 1024, 512), (300, 1000, 264), (300, 1024, 512), (8192, 1024, 2048)]


@pytest.mark.parametrize("T,K,N", PRODUCT_SHAPES)
def test_deferred_product_magnitudes(Q, T, K, N):
    rng = np.random.default_rng(T + K + N)
    x = scaled_rows(rng, T, K, "bf16")
    w = inputs.random_rows(rng, K, N, "bf16", scale=0.02)
    g = inputs.random_gamma(rng, K, "bf16")
    wf_ref = oracle.round_bf16(oracle.fold_weight(w, g))
    wf = Q.normproj_fold_weight(to_dev(w), to_dev(g))
    y = Q.normproj_deferred(to_dev(x), wf, eps=1e-6)
    sync()
    rows = special_rows(T)
    xs = np.ascontiguousarray(x[rows])
    got = to_host(y)[rows]
    check_projection(got, oracle.normproj(xs, wf_ref, 1e-6), rms_bound(xs, wf_ref, 1e-6),
                     f"deferred T={T} K={K} N={N}")
    assert not np.any(widen(got[0]))  # the zero row


@pytest.mark.parametrize("stats", ["auto", None])
@pytest.mark.parametrize("T,K,N", PRODUCT_SHAPES)
def test_deferred_layernorm_magnitudes(Q, T, K, N, stats):
    """LayerNorm rows with a mean of the row's own scale (x = s (z + 2)); a zero row gives the
    bias alone."""
    rng = np.random.default_rng(T * 3 + K + N)
    z = widen(inputs.random_rows(rng, T, K, "bf16")) + 2.0
    s = np.ones(T)
    n = len(SCALES)
    s[:n] = SCALES
    s[T - n:] = SCALES
    x = inputs.f32_to_bf16_bits((z * s[:, None]).astype(np.float32))
    w = inputs.random_rows(rng, K, N, "bf16", scale=0.02)
    g = inputs.random_gamma(rng, K, "bf16")
    beta = inputs.random_rows(rng, 1, K, "bf16", scale=0.1)[0]
    wf_ref = oracle.round_bf16(oracle.fold_weight(w, g))
    cs_ref = oracle.colsum(wf_ref)
    b_ref = oracle.matmul(beta[None, :], w)[0]
    wf, cs, b = Q.normproj_fold_layernorm(to_dev(w), to_dev(g), to_dev(beta))
    y = Q.normproj_deferred_layernorm(to_dev(x), wf, cs, b, eps=1e-5, row_stats=stats)
    sync()
    rows = special_rows(T)
    xs = np.ascontiguousarray(x[rows])
    ref = oracle.normproj_layernorm(xs, wf_ref, cs_ref, b_ref, 1e-5)
    check_projection(to_host(y)[rows], ref, ln_bound(xs, wf_ref, 1e-5),
                     f"LN T={T} K={K} N={N} stats={stats}")
