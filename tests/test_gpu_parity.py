"""GPU parity: every entry point of libqknorm.so against the fp64 CPU oracle on the same seeded
inputs (all five workloads at their full sizes, plus edge cases). Calls go through the C ABI
via the package's ctypes binding."""

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


# ----------------------------------------------------------------------------- fused Q + K
def run_fused(Q, c, check=True):
    q, k = to_dev(c["q"]), to_dev(c["k"])
    gq, gk = to_dev(c["gamma_q"]), to_dev(c["gamma_k"])
    qo, ko = Q.qknorm_fused(q, gq, k, gk, eps=c["eps"])
    sync()
    got_q, got_k = to_host(qo), to_host(ko)
    if check:
        check_rows(got_q, oracle.rmsnorm_rows(c["q"], c["gamma_q"], c["eps"]), "Q")
        check_rows(got_k, oracle.rmsnorm_rows(c["k"], c["gamma_k"], c["eps"]), "K")
    return got_q, got_k


def test_fused_tiny_fp32(Q):
    run_fused(Q, inputs.make_case("tiny-fp32", 64))


@pytest.mark.parametrize("T", inputs.WORKLOADS["olmo2-7b"]["Ts"])
def test_fused_olmo7b(Q, T):
    run_fused(Q, inputs.make_case("olmo2-7b", T))


@pytest.mark.parametrize("T", inputs.WORKLOADS["gqa-olmo2-32b-like"]["Ts"])
def test_fused_gqa_outliers(Q, T):
    run_fused(Q, inputs.make_case("gqa-olmo2-32b-like", T))


def test_fused_deterministic(Q):
    c = inputs.make_case("olmo2-7b", 1024, seed=5)
    a = run_fused(Q, c, check=False)
    b = run_fused(Q, c, check=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ----------------------------------------------------------------------------- shard stage
def test_shard_stage_tp8(Q):
    """K1 partial sums, then K2 aggregation + scale, at T = 131072 (one 512-column slice of
    4096-wide Q and K, seven peers' partials generated)."""
    c = inputs.make_case("tp8-shard", 131072)
    q, k = to_dev(c["q"]), to_dev(c["k"])
    gq, gk = to_dev(c["gamma_q"]), to_dev(c["gamma_k"])
    eq, ek = to_dev(c["ext_q"]), to_dev(c["ext_k"])
    pq, pk = Q.qknorm_partial_sumsq(q, k)
    sync()
    ref_pq, ref_pk = oracle.partial_sumsq(c["q"]), oracle.partial_sumsq(c["k"])
    check_rows(to_host(pq), ref_pq, "psq_q")
    check_rows(to_host(pk), ref_pk, "psq_k")

    # K2 alone, fed the oracle's own partials stored as fp32
    pq32, pk32 = ref_pq.astype(np.float32), ref_pk.astype(np.float32)
    qo, ko = Q.qknorm_apply_with_stats(q, gq, to_dev(pq32), eq, 4096, k, gk, to_dev(pk32), ek,
                                       4096, eps=c["eps"])
    sync()
    check_rows(to_host(qo), oracle.apply_with_stats(c["q"], c["gamma_q"], pq32, c["ext_q"], 4096,
                                                    c["eps"]), "K2 Q")
    check_rows(to_host(ko), oracle.apply_with_stats(c["k"], c["gamma_k"], pk32, c["ext_k"], 4096,
                                                    c["eps"]), "K2 K")

    # the hot path as chained on the GPU (K1 -> K2) against the oracle's chain in fp64
    qo, ko = Q.qknorm_apply_with_stats(q, gq, pq, eq, 4096, k, gk, pk, ek, 4096, eps=c["eps"])
    sync()
    check_rows(to_host(qo), oracle.apply_with_stats(c["q"], c["gamma_q"], ref_pq, c["ext_q"],
                                                    4096, c["eps"]), "K1->K2 Q")
    check_rows(to_host(ko), oracle.apply_with_stats(c["k"], c["gamma_k"], ref_pk, c["ext_k"],
                                                    4096, c["eps"]), "K1->K2 K")


def test_decomposition_matches_fused_on_gpu(Q):
    """Eight column slices of a 4096-wide row (views with ld = 4096): partials, aggregation
    with the other seven slices' partials, scale; equal to the fused launch within rounding."""
    torch = pytest.importorskip("torch")
    c = inputs.make_case("olmo2-7b", 777, seed=3)
    q, gq = to_dev(c["q"]), to_dev(c["gamma_q"])
    fused_q, _ = Q.qknorm_fused(q, gq, eps=c["eps"])
    parts = [Q.qknorm_partial_sumsq(q[:, 512 * s:512 * (s + 1)])[0] for s in range(8)]
    out = torch.empty_like(q)
    for s in range(8):
        ext = torch.stack([parts[j] for j in range(8) if j != s])
        Q.qknorm_apply_with_stats(q[:, 512 * s:512 * (s + 1)], gq[512 * s:512 * (s + 1)],
                                  parts[s], ext, 4096, eps=c["eps"],
                                  q_out=out[:, 512 * s:512 * (s + 1)])
    sync()
    ref = oracle.rmsnorm_rows(c["q"], c["gamma_q"], c["eps"])
    check_rows(to_host(out), ref, "split")
    a, b = widen(to_host(out)), widen(to_host(fused_q))
    assert np.all(np.abs(a - b) <= 2.0 ** -6 * np.abs(b) + 1e-30)


def test_apply_without_peers_is_local_norm(Q):
    c = inputs.make_case("tp8-shard", 300, seed=2)
    q, gq = to_dev(c["q"]), to_dev(c["gamma_q"])
    pq, _ = Q.qknorm_partial_sumsq(q)
    qo, _ = Q.qknorm_apply_with_stats(q, gq, pq, None, 512, eps=1e-6)
    sync()
    check_rows(to_host(qo), oracle.rmsnorm_rows(c["q"], c["gamma_q"], 1e-6), "n_ext=0")


# ----------------------------------------------------------------------------- norm-then-project
def folded_reference(c):
    """Oracle side of the fold: W' = diag(gamma) W in fp64, rounded once to bf16 ([K, N])."""
    return oracle.round_bf16(oracle.fold_weight(c["w"], c["gamma"]))


def sample_rows(T, n=512, seed=0):
    if T <= n + 2:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, n, replace=False)]))


def projection_bound(x_bits, wf_bits, eps):
    x, wf = widen(x_bits), widen(wf_bits)
    r = 1.0 / np.sqrt((x * x).mean(axis=1) + eps)
    return r[:, None] * (np.abs(x) @ np.abs(wf))


def test_fold_weight_bit_exact(Q):
    c = inputs.make_case("flashnorm-2048", 1)
    wf = Q.normproj_fold_weight(to_dev(c["w"]), to_dev(c["gamma"]))
    sync()
    assert np.array_equal(to_host(wf), folded_reference(c))


@pytest.mark.parametrize("T", inputs.WORKLOADS["flashnorm-2048"]["Ts"])
def test_normproj_deferred(Q, T):
    c = inputs.make_case("flashnorm-2048", T)
    wf_ref = folded_reference(c)
    wf = Q.normproj_fold_weight(to_dev(c["w"]), to_dev(c["gamma"]))
    y = Q.normproj_deferred(to_dev(c["x"]), wf, eps=c["eps"])
    sync()
    rows = sample_rows(T)
    xs = c["x"][rows]
    ref = oracle.normproj(xs, wf_ref, c["eps"])
    check_projection(to_host(y)[rows], ref, projection_bound(xs, wf_ref, c["eps"]),
                     f"deferred T={T}")


def test_normproj_unfused_baseline(Q):
    c = inputs.make_case("flashnorm-2048", 2048)
    x, g = to_dev(c["x"]), to_dev(c["gamma"])
    wp = Q.normproj_fold_weight(to_dev(c["w"]), None)
    sync()
    assert np.array_equal(to_host(wp), c["w"])  # gamma = 1: a plain copy
    xn, y = Q.normproj_unfused(x, g, wp, eps=c["eps"])
    sync()
    xn_h = to_host(xn)
    check_rows(xn_h, oracle.rmsnorm_rows(c["x"], c["gamma"], c["eps"]), "unfused norm")
    rows = sample_rows(2048)
    xn_ref = oracle.round_bf16(oracle.rmsnorm_rows(c["x"][rows], c["gamma"], c["eps"]))
    ref = oracle.matmul(xn_ref, c["w"])
    bound = np.abs(widen(xn_ref)) @ np.abs(widen(c["w"]))
    check_projection(to_host(y)[rows], ref, bound, "unfused", abs_coeff=2.0 ** -12)


@pytest.mark.parametrize("T,K,N", [(5, 256, 130), (16, 1032, 64), (17, 1024, 520),
                                   (300, 264, 200), (129, 2048, 2048), (8200, 1056, 4104),
                                   (8200, 1024, 4104), (4096, 64, 4096), (4096, 128, 4096),
                                   (4100, 192, 4104), (4096, 96, 4096),
                                   (4100, 512, 2056), (12, 512, 4104), (8, 1000, 4104),
                                   (1, 8, 24), (3, 64, 40), (16, 4096, 8200), (3, 520, 4104),
                                   (12, 264, 3000), (2, 2048, 2056), (2, 16, 1),
                                   (4, 16392, 520), (16, 8200, 4200), (4352, 64, 4096),
                                   (4352, 128, 4096), (8192, 128, 8192), (6000, 256, 6000)])
def test_normproj_ragged(Q, T, K, N):
    """Every kernel of the projection: the matrix-vector path (T <= 16), the generic tile
    kernel (K not a multiple of 32), and the pipelined tilings (128 x 128 with 4 stages when
    there is at most one tile per CU and 2 otherwise; 256 x 256 with k-tiles of 64 through the
    five-part ring, or of 32), with T and N not multiples of the tile and rings of one, two and
    three k-tiles, grids of one to four rounds of tiles per CU; large cases are checked on a
    sample of rows that meets every tile."""
    rng = np.random.default_rng(T + K + N)
    x = inputs.random_rows(rng, T, K, "bf16")
    w = inputs.random_rows(rng, K, N, "bf16", scale=0.02)
    g = inputs.random_gamma(rng, K, "bf16")
    c = dict(w=w, gamma=g)
    wf_ref = folded_reference(c)
    wf = Q.normproj_fold_weight(to_dev(w), to_dev(g))
    y = Q.normproj_deferred(to_dev(x), wf, eps=1e-6)
    sync()
    assert np.array_equal(to_host(wf), wf_ref)
    rows = sample_rows(T, n=256, seed=T)
    xs = np.ascontiguousarray(x[rows])
    check_projection(to_host(y)[rows], oracle.normproj(xs, wf_ref, 1e-6),
                     projection_bound(xs, wf_ref, 1e-6), f"T={T} K={K} N={N}")


@pytest.mark.parametrize("T,K,N", [(200, 512, 256), (4096, 256, 4096), (9, 520, 4104)])
def test_normproj_strided_rows(Q, T, K, N):
    """x and y with row strides above their widths (128 x 128 tiles, the 256 x 256 ring, and
    the matrix-vector form)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    xfull = inputs.random_rows(rng, T, K, "bf16", ld=K + 64)
    w = inputs.random_rows(rng, K, N, "bf16", scale=0.02)
    g = inputs.random_gamma(rng, K, "bf16")
    wf_ref = folded_reference(dict(w=w, gamma=g))
    wf = Q.normproj_fold_weight(to_dev(w), to_dev(g))
    ybuf = torch.full((T, N + 8), 7.0, dtype=torch.bfloat16, device="cuda")
    Q.normproj_deferred(to_dev(xfull)[:, :K], wf, eps=1e-6, y=ybuf[:, :N])
    sync()
    yh = to_host(ybuf)
    assert np.all(widen(yh[:, N:]) == 7.0)
    rows = sample_rows(T, n=256, seed=T)
    x = np.ascontiguousarray(xfull[rows, :K])
    check_projection(yh[rows, :N], oracle.normproj(x, wf_ref, 1e-6),
                     projection_bound(x, wf_ref, 1e-6), f"strided T={T}")
