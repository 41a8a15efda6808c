"""The single-launch shard stage (partial sums, publication, wait on the peers' flags,
aggregation and scale in one pass) against the fp64 oracle's two-step definition, with the
mailbox protocol exercised in its normal, concurrent and timed-out forms. Timeouts are forced
from the host with a tiny spin limit and flags that are never set; every kernel still exits."""

import numpy as np
import pytest

import oracle
from helpers import check_rows, to_dev, to_host
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


def zeros_i32(*shape):
    import torch

    return torch.zeros(shape, dtype=torch.int32, device="cuda")


def reference(c, d_full, eps):
    pq, pk = oracle.partial_sumsq(c["q"]), oracle.partial_sumsq(c["k"])
    yq = oracle.apply_with_stats(c["q"], c["gamma_q"], pq, c["ext_q"], d_full, eps)
    yk = oracle.apply_with_stats(c["k"], c["gamma_k"], pk, c["ext_k"], d_full, eps)
    return pq, pk, yq, yk


def check_all(got, ref, what):
    qo, ko, pq, pk = got
    rpq, rpk, ryq, ryk = ref
    check_rows(to_host(pq), rpq, f"{what} psq_q")
    check_rows(to_host(pk), rpk, f"{what} psq_k")
    check_rows(to_host(qo), ryq, f"{what} Q")
    check_rows(to_host(ko), ryk, f"{what} K")


def test_shard_fused_prepublished_tp8(Q):
    """TP-8 shard at T = 131072: peers' partials published (same stream) before the pass."""
    import torch

    c = inputs.make_case(4, 131072)
    T, nfb = 131072, Q.shard_flag_blocks(131072)
    q, k, gq, gk = (to_dev(c[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    part_q, part_k = to_dev(c["ext_q"]), to_dev(c["ext_k"])
    mail_q, mail_k = torch.zeros_like(part_q), torch.zeros_like(part_k)
    peer, own, to = zeros_i32(7, 2, nfb), zeros_i32(2, nfb), zeros_i32(1)
    Q.qknorm_shard_publish(part_q, mail_q, peer, 1, part_k, mail_k)
    got = Q.qknorm_shard_fused(q, gq, mail_q, 4096, k, gk, mail_k, 4096, eps=c["eps"],
                               peer_ready=peer, own_ready=own, epoch=1, timed_out=to)
    sync()
    assert int(to.item()) == 0
    assert np.array_equal(to_host(mail_q), c["ext_q"]) and np.array_equal(to_host(mail_k), c["ext_k"])
    assert bool((own == 1).all()) and bool((peer == 1).all())
    check_all(got, reference(c, 4096, c["eps"]), "prepublished")


@pytest.mark.parametrize("dtype,dl", [("bf16", 512), ("bf16", 520), ("bf16", 2048), ("f32", 8),
                                      ("f32", 1024)])
def test_shard_fused_without_flags(Q, dtype, dl):
    """No flags: the mailboxes are already filled. Ragged T, 1, 2 and 4 vectors per lane."""
    rng = np.random.default_rng(dl)
    T, n_ext = 1001, 3
    c = dict(q=inputs.random_rows(rng, T, dl, dtype), k=inputs.random_rows(rng, T, dl, dtype),
             gamma_q=inputs.random_gamma(rng, dl, dtype), gamma_k=inputs.random_gamma(rng, dl, dtype),
             ext_q=rng.chisquare(dl, size=(n_ext, T)).astype(np.float32),
             ext_k=rng.chisquare(dl, size=(n_ext, T)).astype(np.float32))
    d_full = dl * (n_ext + 1)
    got = Q.qknorm_shard_fused(to_dev(c["q"]), to_dev(c["gamma_q"]), to_dev(c["ext_q"]), d_full,
                               to_dev(c["k"]), to_dev(c["gamma_k"]), to_dev(c["ext_k"]), d_full,
                               eps=1e-6)
    sync()
    check_all(got, reference(c, d_full, 1e-6), f"no flags d={dl}")


def test_shard_fused_concurrent_publisher(Q):
    """The pass starts first on one stream and waits; the simulated peers publish from another
    stream of the same GPU while it runs (the pass leaves a quarter of the device free)."""
    import torch

    c = inputs.make_case(4, 65536, seed=9)
    T, nfb = 65536, Q.shard_flag_blocks(65536)
    q, k, gq, gk = (to_dev(c[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    part_q, part_k = to_dev(c["ext_q"]), to_dev(c["ext_k"])
    mail_q, mail_k = torch.zeros_like(part_q), torch.zeros_like(part_k)
    peer, own, to = zeros_i32(7, 2, nfb), zeros_i32(2, nfb), zeros_i32(1)
    sync()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(sa):
        got = Q.qknorm_shard_fused(q, gq, mail_q, 4096, k, gk, mail_k, 4096, eps=c["eps"],
                                   peer_ready=peer, own_ready=own, epoch=3, timed_out=to)
    with torch.cuda.stream(sb):
        Q.qknorm_shard_publish(part_q, mail_q, peer, 3, part_k, mail_k)
    sync()
    assert int(to.item()) == 0, "the pass timed out waiting for the publisher"
    check_all(got, reference(c, 4096, c["eps"]), "concurrent")


@pytest.mark.parametrize("stale", [0, 4])
def test_shard_fused_times_out_without_flags(Q, stale):
    """Flags never reach the epoch (never set, or left at an older epoch): with a spin limit of
    8 polls the pass records the timeout and still finishes; its own partials are right."""
    c = inputs.make_case(4, 4096, seed=10)
    nfb = Q.shard_flag_blocks(4096)
    peer, to = zeros_i32(7, 2, nfb), zeros_i32(1)
    peer.fill_(stale)
    got = Q.qknorm_shard_fused(to_dev(c["q"]), to_dev(c["gamma_q"]), to_dev(c["ext_q"]), 4096,
                               to_dev(c["k"]), to_dev(c["gamma_k"]), to_dev(c["ext_k"]), 4096,
                               peer_ready=peer, epoch=5, max_spin=8, timed_out=to)
    sync()
    assert int(to.item()) == 1
    check_rows(to_host(got[2]), oracle.partial_sumsq(c["q"]), "psq_q after timeout")


def test_shard_fused_epochs_advance(Q):
    """Two passes over the same mailboxes with successive epochs."""
    import torch

    c = inputs.make_case(4, 2000, seed=11)
    nfb = Q.shard_flag_blocks(2000)
    q, k, gq, gk = (to_dev(c[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    part_q, part_k = to_dev(c["ext_q"]), to_dev(c["ext_k"])
    mail_q, mail_k = torch.zeros_like(part_q), torch.zeros_like(part_k)
    peer, own, to = zeros_i32(7, 2, nfb), zeros_i32(2, nfb), zeros_i32(1)
    ref = reference(c, 4096, c["eps"])
    for epoch in (1, 2):
        Q.qknorm_shard_publish(part_q, mail_q, peer, epoch, part_k, mail_k)
        got = Q.qknorm_shard_fused(q, gq, mail_q, 4096, k, gk, mail_k, 4096, eps=c["eps"],
                                   peer_ready=peer, own_ready=own, epoch=epoch, timed_out=to)
        sync()
        assert int(to.item()) == 0 and bool((own == epoch).all())
        check_all(got, ref, f"epoch {epoch}")
