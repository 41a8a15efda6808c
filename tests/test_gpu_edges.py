"""GPU edge cases of the row operations against the fp64 oracle: empty and ragged inputs, odd
and very wide rows, misaligned and strided tensors, in-place calls, special values, the
epsilon-dominated regime, mixed gamma storage and concurrent streams."""

import numpy as np
import pytest

import oracle
from helpers import check_rows, to_dev, to_host, widen
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


def test_empty_T_is_a_noop(Q):
    import torch

    q = torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(4096, dtype=torch.bfloat16, device="cuda")
    qo, ko = Q.qknorm_fused(q, g, q, g)
    pq, pk = Q.qknorm_partial_sumsq(q, q)
    ao, _ = Q.qknorm_apply_with_stats(q, g, pq, None, 4096)
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    y = Q.normproj_deferred(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), w)
    sync()
    assert qo.shape == (0, 4096) and pq.shape == (0,) and y.shape == (0, 64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dq,dk", [(1, 3), (520, 4104), (8, 16), (4096, 512), (12288, 64),
                                   (8192, 2048), (1024, 5120), (16384, 768), (20000, 16392)])
def test_odd_and_wide_widths(Q, dtype, dq, dk):
    """Widths that are not multiples of a wavefront's vector width, every team shape (1, 2 and 4
    wavefronts per row, 1-8 vectors per lane, with partly filled last vectors), K wider than Q,
    and rows wider than the register-resident kernel holds (two-pass path); T ragged."""
    rng = np.random.default_rng(dq * 7 + dk)
    T = 37
    q = inputs.random_rows(rng, T, dq, dtype, scale=1.5)
    k = inputs.random_rows(rng, T, dk, dtype, scale=0.5)
    gq, gk = inputs.random_gamma(rng, dq, dtype), inputs.random_gamma(rng, dk, dtype)
    qo, ko = Q.qknorm_fused(to_dev(q), to_dev(gq), to_dev(k), to_dev(gk), eps=1e-6)
    sync()
    check_rows(to_host(qo), oracle.rmsnorm_rows(q, gq, 1e-6), f"Q d={dq}")
    check_rows(to_host(ko), oracle.rmsnorm_rows(k, gk, 1e-6), f"K d={dk}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gdtype", ["bf16", "f32"])
@pytest.mark.parametrize("vectors", [64, 128, 256, 512, 768, 1024, 2048])
@pytest.mark.parametrize("T", [1, 37])
def test_fused_widths_that_fill_a_shape(Q, dtype, gdtype, vectors, T):
    """Q and K whose width fills a team shape exactly (64 .. 2048 vectors of 16 bytes), gamma
    stored either way: the unmasked kernels, with one row per workgroup (every row exists) or
    several (the last workgroup's extra rows skipped); T = 37 is ragged for every
    rows-per-workgroup count; T = 1, Q alone, leaves the one workgroup's other rows empty
    where it holds several."""
    rng = np.random.default_rng(vectors * 16 + (dtype == "f32") + 2 * (gdtype == "f32") + 4 * T)
    d = vectors * (8 if dtype == "bf16" else 4)
    q = inputs.random_rows(rng, T, d, dtype, scale=1.5)
    k = inputs.random_rows(rng, T, d, dtype, scale=0.5)
    gq, gk = inputs.random_gamma(rng, d, gdtype), inputs.random_gamma(rng, d, gdtype)
    if T == 1:
        qo, _ = Q.qknorm_fused(to_dev(q), to_dev(gq), eps=1e-6)
        sync()
        check_rows(to_host(qo), oracle.rmsnorm_rows(q, gq, 1e-6), f"Q alone d={d}")
        return
    qo, ko = Q.qknorm_fused(to_dev(q), to_dev(gq), to_dev(k), to_dev(gk), eps=1e-6)
    sync()
    check_rows(to_host(qo), oracle.rmsnorm_rows(q, gq, 1e-6), f"Q d={d}")
    check_rows(to_host(ko), oracle.rmsnorm_rows(k, gk, 1e-6), f"K d={d}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_misaligned_views_and_strides(Q, dtype):
    """Tensors starting one element past a 16-byte boundary, with odd row strides: the element
    path runs; padding columns of the output buffer stay untouched."""
    import torch

    rng = np.random.default_rng(21)
    T, d = 50, 1000
    xfull = inputs.random_rows(rng, T, d + 3, dtype, ld=d + 3)
    g = inputs.random_gamma(rng, d + 1, dtype)
    xd, gd = to_dev(xfull), to_dev(g)
    buf = torch.full((T, d + 3), 5.0, dtype=xd.dtype, device="cuda")
    Q.qknorm_fused(xd[:, 1:d + 1], gd[1:], q_out=buf[:, 2:d + 2], eps=1e-5)
    sync()
    got = to_host(buf)
    x = np.ascontiguousarray(xfull[:, 1:d + 1])
    check_rows(np.ascontiguousarray(got[:, 2:d + 2]), oracle.rmsnorm_rows(x, g[1:], 1e-5),
               "misaligned")
    assert np.all(widen(got[:, :2]) == 5.0) and np.all(widen(got[:, d + 2:]) == 5.0)


def test_row_stride_above_width_keeps_padding(Q):
    import torch

    rng = np.random.default_rng(22)
    T, d, ld = 33, 4096, 4096 + 256
    x = inputs.random_rows(rng, T, d, "bf16", scale=2.0, ld=ld)
    g = inputs.random_gamma(rng, d, "bf16")
    xd = to_dev(x)
    out = torch.full((T, ld), 3.0, dtype=torch.bfloat16, device="cuda")
    Q.qknorm_fused(xd[:, :d], to_dev(g), q_out=out[:, :d], eps=1e-6)
    sync()
    got = to_host(out)
    check_rows(np.ascontiguousarray(got[:, :d]),
               oracle.rmsnorm_rows(np.ascontiguousarray(x[:, :d]), g, 1e-6), "strided")
    assert np.all(widen(got[:, d:]) == 3.0)


def test_in_place(Q):
    c = inputs.make_case("olmo2-7b", 300, seed=4)
    q, k = to_dev(c["q"]), to_dev(c["k"])
    Q.qknorm_fused(q, to_dev(c["gamma_q"]), k, to_dev(c["gamma_k"]), eps=c["eps"], q_out=q,
                   k_out=k)
    sync()
    check_rows(to_host(q), oracle.rmsnorm_rows(c["q"], c["gamma_q"], c["eps"]), "in-place Q")
    check_rows(to_host(k), oracle.rmsnorm_rows(c["k"], c["gamma_k"], c["eps"]), "in-place K")
    # in-place shard stage
    c4 = inputs.make_case("tp8-shard", 200, seed=4)
    q4 = to_dev(c4["q"])
    pq, _ = Q.qknorm_partial_sumsq(q4)
    Q.qknorm_apply_with_stats(q4, to_dev(c4["gamma_q"]), pq, to_dev(c4["ext_q"]), 4096,
                              eps=c4["eps"], q_out=q4)
    sync()
    ref = oracle.apply_with_stats(c4["q"], c4["gamma_q"], oracle.partial_sumsq(c4["q"]),
                                  c4["ext_q"], 4096, c4["eps"])
    check_rows(to_host(q4), ref, "in-place apply")


def test_alias_rejected_on_device(Q):
    import torch

    q = torch.zeros((8, 4096), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(4096, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(Q.QknError) as e:
        Q.qknorm_fused(q[:4], g, q_out=q[1:5])
    assert e.value.status == 5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_special_values(Q, dtype):
    """NaN anywhere in a row makes the whole row NaN; +-inf does too (inf/inf); a zero row is
    zero for eps > 0 and NaN for eps = 0 (0 * inf), exactly as the oracle's IEEE arithmetic."""
    rng = np.random.default_rng(23)
    T, d = 8, 4096
    x = rng.normal(0.0, 1.0, (T, d)).astype(np.float32)
    x[1, 17] = np.nan
    x[2, 4000] = np.inf
    x[3, 5] = -np.inf
    x[4, :] = 0.0
    xs = inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x
    g = inputs.random_gamma(rng, d, dtype)
    for eps in (1e-6, 0.0):
        qo, _ = Q.qknorm_fused(to_dev(xs), to_dev(g), eps=eps)
        sync()
        check_rows(to_host(qo), oracle.rmsnorm_rows(xs, g, eps), f"special eps={eps}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_eps_dominated_rows(Q, dtype):
    """x ~ N(0, 1e-3): mean(x^2) ~ eps, so where eps sits changes y by about 1/sqrt(2)."""
    rng = np.random.default_rng(24)
    x = inputs.random_rows(rng, 64, 2048, dtype, scale=1e-3)
    g = inputs.random_gamma(rng, 2048, dtype)
    qo, _ = Q.qknorm_fused(to_dev(x), to_dev(g), eps=1e-6)
    sync()
    got = to_host(qo)
    check_rows(got, oracle.rmsnorm_rows(x, g, 1e-6), "eps regime")
    assert not np.allclose(widen(got), oracle.rmsnorm_rows(x, g, 0.0), rtol=0.05)


def test_mixed_gamma_storage(Q):
    rng = np.random.default_rng(25)
    xb = inputs.random_rows(rng, 40, 4096, "bf16")
    g32 = inputs.random_gamma(rng, 4096, "f32")
    qo, _ = Q.qknorm_fused(to_dev(xb), to_dev(g32), eps=1e-6)
    xf = inputs.random_rows(rng, 40, 512, "f32")
    gb = inputs.random_gamma(rng, 512, "bf16")
    fo, _ = Q.qknorm_fused(to_dev(xf), to_dev(gb), eps=1e-6)
    sync()
    check_rows(to_host(qo), oracle.rmsnorm_rows(xb, g32, 1e-6), "bf16 x, f32 gamma")
    check_rows(to_host(fo), oracle.rmsnorm_rows(xf, gb, 1e-6), "f32 x, bf16 gamma")


def test_partial_apply_edge_widths(Q):
    """Shard stage with slice widths 1, 3 and 700 (element path) and T not a multiple of the
    rows a wavefront batches."""
    rng = np.random.default_rng(26)
    T = 45
    for dl, df in ((1, 8), (3, 24), (700, 5600), (64, 512)):
        q = inputs.random_rows(rng, T, dl, "bf16")
        k = inputs.random_rows(rng, T, dl, "bf16")
        gq, gk = inputs.random_gamma(rng, dl, "bf16"), inputs.random_gamma(rng, dl, "bf16")
        ext = rng.chisquare(dl, size=(3, T)).astype(np.float32)
        pq, pk = Q.qknorm_partial_sumsq(to_dev(q), to_dev(k))
        sync()
        check_rows(to_host(pq), oracle.partial_sumsq(q), f"psq d={dl}")
        check_rows(to_host(pk), oracle.partial_sumsq(k), f"psk d={dl}")
        qo, ko = Q.qknorm_apply_with_stats(to_dev(q), to_dev(gq), pq, to_dev(ext), df,
                                           to_dev(k), to_dev(gk), pk, to_dev(ext), df, eps=1e-6)
        sync()
        check_rows(to_host(qo), oracle.apply_with_stats(q, gq, oracle.partial_sumsq(q), ext, df,
                                                        1e-6), f"apply Q d={dl}")
        check_rows(to_host(ko), oracle.apply_with_stats(k, gk, oracle.partial_sumsq(k), ext, df,
                                                        1e-6), f"apply K d={dl}")


def test_concurrent_streams(Q):
    import torch

    cases = [inputs.make_case("olmo2-7b", 2048, seed=s) for s in (31, 32)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    dev = [(to_dev(c["q"]), to_dev(c["gamma_q"]), to_dev(c["k"]), to_dev(c["gamma_k"]))
           for c in cases]
    sync()
    for (q, gq, k, gk), s in zip(dev, streams):
        with torch.cuda.stream(s):
            for _ in range(3):
                outs.append(Q.qknorm_fused(q, gq, k, gk, eps=1e-6))
    sync()
    for i, c in enumerate(cases):
        ref_q = oracle.rmsnorm_rows(c["q"], c["gamma_q"], 1e-6)
        for j in range(3):
            check_rows(to_host(outs[3 * i + j][0]), ref_q, f"stream {i} rep {j}")


def test_fused_column_blocks_in_place(Q):
    """Q and K as the two column blocks of one [T, nq + nk] matrix (a stacked projection's
    output), normalised in place: the validation accepts the interleaved blocks and each block
    is normalised over its own width."""
    rng = np.random.default_rng(31)
    T, nq, nk = 257, 640, 128
    y = inputs.random_rows(rng, T, nq + nk, "bf16")
    gq, gk = inputs.random_gamma(rng, nq, "bf16"), inputs.random_gamma(rng, nk, "bf16")
    yd = to_dev(y)
    Q.qknorm_fused(yd[:, :nq], to_dev(gq), yd[:, nq:], to_dev(gk), eps=1e-6, q_out=yd[:, :nq],
                   k_out=yd[:, nq:])
    sync()
    got = to_host(yd)
    check_rows(got[:, :nq], oracle.rmsnorm_rows(np.ascontiguousarray(y[:, :nq]), gq, 1e-6), "Q")
    check_rows(got[:, nq:], oracle.rmsnorm_rows(np.ascontiguousarray(y[:, nq:]), gk, 1e-6), "K")


@pytest.mark.parametrize("n,doff,soff", [(1, 0, 0), (15, 0, 0), (16, 0, 0), (17, 3, 0),
                                         (4097, 0, 5), ((1 << 20) + 3, 16, 32),
                                         ((1 << 28) + 4099, 0, 0), ((1 << 28) + 77, 1, 1)])
def test_device_copy(Q, n, doff, soff):
    """The reference copy the benchmark calibrates against: every byte lands, aligned (16-byte
    vectors plus a byte tail) or not (bytes), including sizes past the grid cap, where the
    threads stride; the bytes around the destination stay untouched."""
    import torch

    gen = torch.Generator(device="cuda").manual_seed(n)
    src = torch.randint(0, 256, (n + soff,), dtype=torch.uint8, device="cuda", generator=gen)
    dst = torch.full((n + doff + 64,), 0xAB, dtype=torch.uint8, device="cuda")
    Q.qkn_device_copy(dst[doff:doff + n], src[soff:], n)
    sync()
    assert torch.equal(dst[doff:doff + n], src[soff:soff + n])
    assert bool((dst[:doff] == 0xAB).all()) and bool((dst[doff + n:] == 0xAB).all())
