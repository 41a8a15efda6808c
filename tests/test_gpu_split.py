"""GPU parity of the two-launch scalar-statistics split (qknorm_partial_sumsq, then
qknorm_apply_with_stats) against the fp64 oracle, element by element, over the cases the
tensor-parallel degree and the model widths reach: every team shape of the row kernels and the
two-pass path beyond them, fp32 and bf16 storage with either gamma storage, Q and K slices of
different widths in one launch, peer counts past the first batch of preloaded peers (TP-16 to
TP-65), and peers' partials taken as row slices of a wider buffer (ld_ext > T).

Source of the split: "SwiftQK: Fast and Communication-Efficient Tensor Parallelism for Query-Key
Normalization", abstract (ranks exchange per-row scalar partial sums, aggregate them, then
scale their own slice)."""

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


def peers_buffer(rng, n_ext, T, d_local, pad):
    """Peers' partial sums as a [n_ext, T + pad] fp32 buffer (pad columns hold a sentinel that
    would show up in any row that read them): each is the sum of d_local squared N(0, 1), a
    chi-square draw with d_local degrees of freedom."""
    buf = np.full((n_ext, T + pad), 3.0e9, dtype=np.float32)
    buf[:, :T] = rng.chisquare(d_local, size=(n_ext, T)).astype(np.float32)
    return buf


def run_split(Q, rng, T, dq, dk, dtype, gdtype, n_ext, pad, what):
    """Partial sums of Q [T, dq] and K [T, dk] slices, then aggregation with n_ext peers and the
    scale over d_full = (n_ext + 1) * d_local; every output is checked against the oracle."""
    q = inputs.random_rows(rng, T, dq, dtype, scale=1.3)
    k = inputs.random_rows(rng, T, dk, dtype, scale=0.7)
    gq, gk = inputs.random_gamma(rng, dq, gdtype), inputs.random_gamma(rng, dk, gdtype)
    eq = peers_buffer(rng, n_ext, T, dq, pad) if n_ext else None
    ek = peers_buffer(rng, n_ext, T, dk, pad) if n_ext else None
    dqf, dkf = (n_ext + 1) * dq, (n_ext + 1) * dk
    qd, kd = to_dev(q), to_dev(k)

    pq, pk = Q.qknorm_partial_sumsq(qd, kd)
    sync()
    ref_pq, ref_pk = oracle.partial_sumsq(q), oracle.partial_sumsq(k)
    check_rows(to_host(pq), ref_pq, f"{what} psq_q")
    check_rows(to_host(pk), ref_pk, f"{what} psq_k")

    eqd = to_dev(eq)[:, :T] if n_ext else None   # row stride T + pad
    ekd = to_dev(ek)[:, :T] if n_ext else None
    if n_ext:
        assert eqd.stride(0) == T + pad
    eqh = np.ascontiguousarray(eq[:, :T]) if n_ext else None
    ekh = np.ascontiguousarray(ek[:, :T]) if n_ext else None
    # the aggregation alone, fed the oracle's partials stored as fp32
    pq32, pk32 = ref_pq.astype(np.float32), ref_pk.astype(np.float32)
    qo, ko = Q.qknorm_apply_with_stats(qd, to_dev(gq), to_dev(pq32), eqd, dqf, kd, to_dev(gk),
                                       to_dev(pk32), ekd, dkf, eps=1e-6)
    sync()
    check_rows(to_host(qo), oracle.apply_with_stats(q, gq, pq32, eqh, dqf, 1e-6),
               f"{what} apply Q")
    check_rows(to_host(ko), oracle.apply_with_stats(k, gk, pk32, ekh, dkf, 1e-6),
               f"{what} apply K")
    # the chain as it runs on the GPU: the device partials feed the aggregation
    qo, ko = Q.qknorm_apply_with_stats(qd, to_dev(gq), pq, eqd, dqf, kd, to_dev(gk), pk, ekd, dkf,
                                       eps=1e-6)
    sync()
    check_rows(to_host(qo), oracle.apply_with_stats(q, gq, ref_pq, eqh, dqf, 1e-6),
               f"{what} chain Q")
    check_rows(to_host(ko), oracle.apply_with_stats(k, gk, ref_pk, ekh, dkf, 1e-6),
               f"{what} chain K")


# Slice widths per storage: the smallest of each team-shape class (1, 2, 4 wavefronts per row;
# 1, 2, 3, 4, 8 vectors of 16 bytes per lane), a width with a partly filled wavefront, and one
# wider than 2048 vectors (the two-pass path). bf16 640 is one eighth of a 5120-wide GQA Q.
WIDTHS = {
    "bf16": [520, 640, 1024, 2048, 4096, 6144, 8192, 16384, 16400],
    "f32": [256, 320, 512, 1024, 2048, 3072, 4096, 8192, 8200],
}


@pytest.mark.parametrize("gdtype", ["bf16", "f32"])
@pytest.mark.parametrize("dtype,d", [(dt, d) for dt in ("bf16", "f32") for d in WIDTHS[dt]])
def test_split_team_shapes(Q, dtype, d, gdtype):
    """Every team shape of both split kernels (including the partial sums' cross-wavefront
    reduction through LDS), both storages of x and of gamma; T = 37 leaves a ragged last row
    block under every rows-per-workgroup count."""
    rng = np.random.default_rng(1000 + d + (7 if dtype == "f32" else 0) + (3 if gdtype == "f32" else 0))
    run_split(Q, rng, 37, d, d, dtype, gdtype, 7, 64, f"{dtype}/{gdtype} d={d}")


@pytest.mark.parametrize("n_ext", [0, 1, 8, 9, 15, 31, 63, 64])
@pytest.mark.parametrize("dtype,d", [("bf16", 512), ("bf16", 1024), ("f32", 2048)])
def test_split_peer_counts(Q, dtype, d, n_ext):
    """Peer counts of TP-1 to TP-65: no peers, within the first 8 preloaded with the rows, and
    past them (the remaining peers are added in order by a loop); peers' partials are row
    slices of a [n_ext, T + 64] buffer. T = 45 is odd, so the last two-row batch of the
    single-wavefront shape has one row."""
    rng = np.random.default_rng(2000 + 17 * n_ext + d)
    run_split(Q, rng, 45, d, d, dtype, "bf16" if dtype == "bf16" else "f32", n_ext, 64,
              f"{dtype} d={d} n_ext={n_ext}")


@pytest.mark.parametrize("dtype,dq,dk", [("bf16", 640, 128), ("bf16", 4096, 512),
                                         ("bf16", 2048, 16400), ("f32", 1280, 256)])
def test_split_q_k_widths_differ(Q, dtype, dq, dk):
    """Q and K slices of different widths in one launch (a GQA model's Q and K under TP-8, and
    a K slice that takes the two-pass path while Q does not): the split kernels run both with
    the wider tensor's shape."""
    rng = np.random.default_rng(3000 + dq + dk)
    run_split(Q, rng, 130, dq, dk, dtype, dtype, 7, 16, f"{dtype} dq={dq} dk={dk}")


def test_split_long_ragged_tp16(Q):
    """A longer ragged run (T = 4099) at a TP-16 GQA shard of OLMo-2-32B-like widths
    (Q 5120 / 16 = 320, K 1024 / 16 = 64 bf16 columns) with 15 peers."""
    rng = np.random.default_rng(4099)
    run_split(Q, rng, 4099, 320, 64, "bf16", "bf16", 15, 128, "tp16 gqa")


def test_split_equals_monolithic_over_slices(Q):
    """A 6144-wide fp32 row cut into 3 slices of 2048 (team shape 3): each slice's partials from
    the GPU, aggregated with the other two slices' and scaled, reproduce the monolithic norm."""
    import torch

    rng = np.random.default_rng(6144)
    T, d, P = 29, 6144, 3
    x = inputs.random_rows(rng, T, d, "f32")
    g = inputs.random_gamma(rng, d, "f32")
    xd, gd = to_dev(x), to_dev(g)
    w = d // P
    parts = [Q.qknorm_partial_sumsq(xd[:, w * s:w * (s + 1)])[0] for s in range(P)]
    out = torch.empty_like(xd)
    for s in range(P):
        ext = torch.stack([parts[j] for j in range(P) if j != s])
        Q.qknorm_apply_with_stats(xd[:, w * s:w * (s + 1)], gd[w * s:w * (s + 1)], parts[s], ext,
                                  d, eps=1e-6, q_out=out[:, w * s:w * (s + 1)])
    sync()
    got = to_host(out)
    check_rows(got, oracle.rmsnorm_rows(x, g, 1e-6), "3-slice fp32")
    assert np.isfinite(widen(got)).all()
