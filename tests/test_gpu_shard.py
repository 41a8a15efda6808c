"""The single-launch shard stage (partial sums, publication, wait on the peers' mailbox words,
aggregation and scale in one pass) against the fp64 oracle's two-step definition, with the
mailbox exercised in its normal, concurrent and timed-out forms. Timeouts are forced from the
host with a tiny spin limit and words that never carry the epoch; every kernel still exits."""

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


def host_words(values: np.ndarray, epoch: int) -> np.ndarray:
    """Mailbox words built on the host: epoch in the upper 32 bits, fp32 bits in the lower."""
    bits = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((np.uint64(epoch) << np.uint64(32)) | bits).view(np.int64)


def words_split(words) -> tuple[np.ndarray, np.ndarray]:
    """(fp32 values, epochs) of device mailbox words."""
    w = to_host(words).view(np.uint64)
    return (w & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32), (w >> np.uint64(32))


def reference(c, d_full, eps):
    pq, pk = oracle.partial_sumsq(c["q"]), oracle.partial_sumsq(c["k"])
    yq = oracle.apply_with_stats(c["q"], c["gamma_q"], pq, c["ext_q"], d_full, eps)
    yk = oracle.apply_with_stats(c["k"], c["gamma_k"], pk, c["ext_k"], d_full, eps)
    return pq, pk, yq, yk


def check_all(got, ref, what, epoch):
    qo, ko, pq, pk = got
    rpq, rpk, ryq, ryk = ref
    for words, r, name in ((pq, rpq, "psq_q"), (pk, rpk, "psq_k")):
        vals, tags = words_split(words)
        assert np.all(tags == epoch), f"{what} {name}: own partials not tagged with the epoch"
        check_rows(vals, r, f"{what} {name}")
    check_rows(to_host(qo), ryq, f"{what} Q")
    check_rows(to_host(ko), ryk, f"{what} K")


@pytest.mark.parametrize("persistent", [True, False])
def test_shard_fused_prepublished_tp8(Q, persistent):
    """TP-8 shard at T = 131072: peers' partials published (same stream) before the pass, with
    and without the residency cap that leaves room for a same-device producer."""
    c = inputs.make_case("tp8-shard", 131072)
    q, k, gq, gk = (to_dev(c[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    part_q, part_k = to_dev(c["ext_q"]), to_dev(c["ext_k"])
    mail_q, mail_k = Q.mailbox_words(7, 131072), Q.mailbox_words(7, 131072)
    to = zeros_i32(1)
    Q.qknorm_shard_publish(part_q, mail_q, 1, part_k, mail_k)
    got = Q.qknorm_shard_fused(q, gq, mail_q, 4096, k, gk, mail_k, 4096, eps=c["eps"], epoch=1,
                               timed_out=to, persistent=persistent)
    sync()
    assert int(to.item()) == 0
    for mail, ext in ((mail_q, c["ext_q"]), (mail_k, c["ext_k"])):
        vals, tags = words_split(mail)
        assert np.array_equal(vals.view(np.uint32), ext.view(np.uint32)) and np.all(tags == 1)
    check_all(got, reference(c, 4096, c["eps"]), "prepublished", 1)


@pytest.mark.parametrize("dtype,dl", [("bf16", 512), ("bf16", 520), ("bf16", 2048), ("f32", 8),
                                      ("f32", 1024)])
def test_shard_fused_complete_mailbox(Q, dtype, dl):
    """epoch 0: the mailboxes were filled before the launch and their tags are not looked at
    (here they carry an unrelated tag). Ragged T, 1, 2 and 4 vectors per lane."""
    rng = np.random.default_rng(dl)
    T, n_ext = 1001, 3
    c = dict(q=inputs.random_rows(rng, T, dl, dtype), k=inputs.random_rows(rng, T, dl, dtype),
             gamma_q=inputs.random_gamma(rng, dl, dtype), gamma_k=inputs.random_gamma(rng, dl, dtype),
             ext_q=rng.chisquare(dl, size=(n_ext, T)).astype(np.float32),
             ext_k=rng.chisquare(dl, size=(n_ext, T)).astype(np.float32))
    d_full = dl * (n_ext + 1)
    got = Q.qknorm_shard_fused(to_dev(c["q"]), to_dev(c["gamma_q"]),
                               to_dev(host_words(c["ext_q"], 77)), d_full, to_dev(c["k"]),
                               to_dev(c["gamma_k"]), to_dev(host_words(c["ext_k"], 77)), d_full,
                               eps=1e-6, epoch=0)
    sync()
    check_all(got, reference(c, d_full, 1e-6), f"complete mailbox d={dl}", 0)


@pytest.mark.parametrize("persistent", [True, False])
@pytest.mark.parametrize("dtype,dl,n_ext", [("bf16", 520, 3), ("bf16", 2048, 17), ("f32", 1024, 3),
                                            ("f32", 8, 17), ("bf16", 512, 0)])
def test_shard_fused_widths_waiting(Q, dtype, dl, n_ext, persistent):
    """Slices of 1, 2 and 4 vectors per lane with the mailbox checked (epoch != 0), in both
    residency policies and with no peers, one and four 16-peer lane groups. With 4 vectors per
    lane one workgroup fits per CU, and the reservation that leaves room for a producer takes
    half the LDS (more than 64 KB of dynamic LDS, allowed explicitly)."""
    rng = np.random.default_rng(dl + n_ext)
    T = 1001
    c = dict(q=inputs.random_rows(rng, T, dl, dtype), k=inputs.random_rows(rng, T, dl, dtype),
             gamma_q=inputs.random_gamma(rng, dl, dtype), gamma_k=inputs.random_gamma(rng, dl, dtype),
             ext_q=rng.chisquare(dl, size=(n_ext, T)).astype(np.float32),
             ext_k=rng.chisquare(dl, size=(n_ext, T)).astype(np.float32))
    d_full = dl * (n_ext + 1)
    mail_q, mail_k = Q.mailbox_words(n_ext, T), Q.mailbox_words(n_ext, T)
    Q.qknorm_shard_publish(to_dev(c["ext_q"]), mail_q, 6, to_dev(c["ext_k"]), mail_k)
    to = zeros_i32(1)
    got = Q.qknorm_shard_fused(to_dev(c["q"]), to_dev(c["gamma_q"]), mail_q, d_full,
                               to_dev(c["k"]), to_dev(c["gamma_k"]), mail_k, d_full, eps=1e-6,
                               epoch=6, timed_out=to, persistent=persistent)
    sync()
    assert int(to.item()) == 0
    check_all(got, reference(c, d_full, 1e-6), f"{dtype} d={dl} n_ext={n_ext}", 6)


@pytest.mark.parametrize("persistent", [True, False])
@pytest.mark.parametrize("dtype,dl,off,pad", [("bf16", 500, 1, 3), ("bf16", 1030, 3, 5),
                                              ("bf16", 512, 1, 1), ("f32", 300, 1, 1),
                                              ("f32", 1021, 2, 3)])
def test_shard_fused_any_alignment(Q, dtype, dl, off, pad, persistent):
    """Slices off a 16-byte boundary (inputs, outputs and gamma one or more elements in), odd
    row strides and widths that are not a whole number of 16-byte vectors take the element
    accesses; the outputs' padding stays untouched."""
    import torch

    rng = np.random.default_rng(dl + 7 * off)
    T, n_ext = 777, 5
    qf = inputs.random_rows(rng, T, dl + pad, dtype)
    kf = inputs.random_rows(rng, T, dl + pad, dtype)
    gqf = inputs.random_gamma(rng, dl + off, dtype)
    gkf = inputs.random_gamma(rng, dl + off, dtype)
    c = dict(q=np.ascontiguousarray(qf[:, off:off + dl]), k=np.ascontiguousarray(kf[:, off:off + dl]),
             gamma_q=gqf[off:], gamma_k=gkf[off:],
             ext_q=rng.chisquare(dl, size=(n_ext, T)).astype(np.float32),
             ext_k=rng.chisquare(dl, size=(n_ext, T)).astype(np.float32))
    d_full = dl * (n_ext + 1)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qo_buf = torch.full((T, dl + pad), 7.0, dtype=tdt, device="cuda")
    ko_buf = torch.full((T, dl + pad), 7.0, dtype=tdt, device="cuda")
    mail_q, mail_k = Q.mailbox_words(n_ext, T), Q.mailbox_words(n_ext, T)
    Q.qknorm_shard_publish(to_dev(c["ext_q"]), mail_q, 3, to_dev(c["ext_k"]), mail_k)
    to = zeros_i32(1)
    got = Q.qknorm_shard_fused(to_dev(qf)[:, off:off + dl], to_dev(gqf)[off:], mail_q, d_full,
                               to_dev(kf)[:, off:off + dl], to_dev(gkf)[off:], mail_k, d_full,
                               eps=1e-6, q_out=qo_buf[:, off:off + dl],
                               k_out=ko_buf[:, off:off + dl], epoch=3, timed_out=to,
                               persistent=persistent)
    sync()
    assert int(to.item()) == 0
    check_all(got, reference(c, d_full, 1e-6), f"{dtype} d={dl} off={off}", 3)
    for buf in (qo_buf, ko_buf):
        h = buf.float().cpu().numpy()
        assert np.all(h[:, :off] == 7.0) and np.all(h[:, off + dl:] == 7.0), "padding written"


@pytest.mark.parametrize("n_ext", [1, 16, 17, 64])
def test_shard_fused_peer_counts(Q, n_ext):
    """Peer counts that fill one, several and all four 16-peer lane groups of the gather."""
    rng = np.random.default_rng(n_ext)
    T, dl = 333, 128
    c = dict(q=inputs.random_rows(rng, T, dl, "bf16"), k=inputs.random_rows(rng, T, dl, "bf16"),
             gamma_q=inputs.random_gamma(rng, dl, "bf16"), gamma_k=inputs.random_gamma(rng, dl, "bf16"),
             ext_q=rng.chisquare(dl, size=(n_ext, T)).astype(np.float32),
             ext_k=rng.chisquare(dl, size=(n_ext, T)).astype(np.float32))
    d_full = dl * (n_ext + 1)
    mail_q, mail_k = Q.mailbox_words(n_ext, T), Q.mailbox_words(n_ext, T)
    Q.qknorm_shard_publish(to_dev(c["ext_q"]), mail_q, 2, to_dev(c["ext_k"]), mail_k)
    to = zeros_i32(1)
    got = Q.qknorm_shard_fused(to_dev(c["q"]), to_dev(c["gamma_q"]), mail_q, d_full,
                               to_dev(c["k"]), to_dev(c["gamma_k"]), mail_k, d_full, eps=1e-6,
                               epoch=2, timed_out=to)
    sync()
    assert int(to.item()) == 0
    check_all(got, reference(c, d_full, 1e-6), f"n_ext={n_ext}", 2)


def test_shard_fused_concurrent_publisher(Q):
    """The simulated peers publish from another stream of the same GPU while the pass runs (the
    pass leaves a quarter of the device free). The publisher's work is submitted first, behind
    a spin of a few milliseconds on its stream: when the two streams run on different hardware
    queues the pass starts first and waits for the words; when HIP has put both streams on one
    queue, the queue runs the publisher first and the pass finds the words ready. Either way
    the pass must not time out."""
    import torch

    c = inputs.make_case("tp8-shard", 65536, seed=9)
    q, k, gq, gk = (to_dev(c[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    part_q, part_k = to_dev(c["ext_q"]), to_dev(c["ext_k"])
    mail_q, mail_k = Q.mailbox_words(7, 65536), Q.mailbox_words(7, 65536)
    to = zeros_i32(1)
    sync()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(sb):
        torch.cuda._sleep(5_000_000)
        Q.qknorm_shard_publish(part_q, mail_q, 3, part_k, mail_k)
    with torch.cuda.stream(sa):
        got = Q.qknorm_shard_fused(q, gq, mail_q, 4096, k, gk, mail_k, 4096, eps=c["eps"],
                                   epoch=3, timed_out=to)
    sync()
    assert int(to.item()) == 0, "the pass timed out waiting for the publisher"
    check_all(got, reference(c, 4096, c["eps"]), "concurrent", 3)


@pytest.mark.parametrize("persistent", [True, False])
@pytest.mark.parametrize("stale", [0, 4])
def test_shard_fused_times_out(Q, stale, persistent):
    """Mailbox words that never carry the epoch (never written, or left at an older epoch):
    with a spin limit of 8 polls the pass records the timeout and still finishes; its own
    partials are right."""
    c = inputs.make_case("tp8-shard", 4096, seed=10)
    mail_q = to_dev(host_words(c["ext_q"], stale))
    mail_k = to_dev(host_words(c["ext_k"], stale))
    to = zeros_i32(1)
    got = Q.qknorm_shard_fused(to_dev(c["q"]), to_dev(c["gamma_q"]), mail_q, 4096,
                               to_dev(c["k"]), to_dev(c["gamma_k"]), mail_k, 4096,
                               epoch=5, max_spin=8, timed_out=to, persistent=persistent)
    sync()
    assert int(to.item()) == 1
    vals, tags = words_split(got[2])
    assert np.all(tags == 5)
    check_rows(vals, oracle.partial_sumsq(c["q"]), "psq_q after timeout")


@pytest.mark.parametrize("persistent", [True, False])
def test_shard_fused_epochs_advance(Q, persistent):
    """Two passes over the same mailboxes with successive epochs."""
    c = inputs.make_case("tp8-shard", 2000, seed=11)
    q, k, gq, gk = (to_dev(c[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    part_q, part_k = to_dev(c["ext_q"]), to_dev(c["ext_k"])
    mail_q, mail_k = Q.mailbox_words(7, 2000), Q.mailbox_words(7, 2000)
    to = zeros_i32(1)
    ref = reference(c, 4096, c["eps"])
    for epoch in (1, 2):
        Q.qknorm_shard_publish(part_q, mail_q, epoch, part_k, mail_k)
        got = Q.qknorm_shard_fused(q, gq, mail_q, 4096, k, gk, mail_k, 4096, eps=c["eps"],
                                   epoch=epoch, timed_out=to, persistent=persistent)
        sync()
        assert int(to.item()) == 0
        check_all(got, ref, f"epoch {epoch}", epoch)
