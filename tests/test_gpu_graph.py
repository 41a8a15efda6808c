"""Entry points captured into a HIP graph: every replay (with eager work and synchronisations in
between) must reproduce the eager results bit for bit."""

import numpy as np
import pytest

from helpers import to_dev, to_host
from layerwise_qk_norm_amd import inputs

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import layerwise_qk_norm_amd as Q

    c2 = inputs.make_case("olmo2-7b", 512, seed=8)
    c4 = inputs.make_case("tp8-shard", 1000, seed=8)
    c5 = inputs.make_case("flashnorm-2048", 300, seed=8)
    q, k, gq, gk = (to_dev(c2[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    sq, sk, sgq, sgk = (to_dev(c4[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    eq, ek = to_dev(c4["ext_q"]), to_dev(c4["ext_k"])
    x = to_dev(c5["x"])
    wf = Q.normproj_fold_weight(to_dev(c5["w"]), to_dev(c5["gamma"]))
    # pre-norm elimination (matrix-core and matrix-vector paths) and its unfused chain,
    # deferred LayerNorm
    el = {T: inputs.make_elimination_case(T, seed=8, K=512, nq=384, nk=128) for T in (200, 12)}
    el_x = {T: to_dev(c["x"]) for T, c in el.items()}
    el_w = Q.normproj_fold_weight(to_dev(el[200]["w"]), to_dev(el[200]["gamma_pre"]))
    el_gq, el_gk = to_dev(el[200]["gamma_q"]), to_dev(el[200]["gamma_k"])
    el_g1, el_wp = to_dev(el[200]["gamma_pre"]), to_dev(el[200]["w"])
    ln = {T: inputs.make_layernorm_case(T, seed=8, K=512, N=256, x_mean=1.0) for T in (300, 5)}
    ln_x = {T: to_dev(c["x"]) for T, c in ln.items()}
    ln_w, ln_c, ln_b = Q.normproj_fold_layernorm(to_dev(ln[300]["w"]), to_dev(ln[300]["gamma"]),
                                                 to_dev(ln[300]["beta"]))
    # single-launch shard stage: peers published once, before capture
    mail_q, mail_k = Q.mailbox_words(7, 1000), Q.mailbox_words(7, 1000)
    tout = torch.zeros((1,), dtype=torch.int32, device="cuda")
    Q.qknorm_shard_publish(eq, mail_q, 1, ek, mail_k)

    def outputs():
        return dict(qo=torch.empty_like(q), ko=torch.empty_like(k),
                    pq=torch.empty(1000, device="cuda"), pk=torch.empty(1000, device="cuda"),
                    so=torch.empty_like(sq), sko=torch.empty_like(sk),
                    y=torch.empty((300, 2048), dtype=torch.bfloat16, device="cuda"),
                    fo=torch.empty_like(sq), fko=torch.empty_like(sk),
                    fpq=torch.empty(1000, dtype=torch.int64, device="cuda"),
                    fpk=torch.empty(1000, dtype=torch.int64, device="cuda"),
                    e200=torch.empty((200, 512), dtype=torch.bfloat16, device="cuda"),
                    x200=torch.empty((200, 512), dtype=torch.bfloat16, device="cuda"),
                    e12=torch.empty((12, 512), dtype=torch.bfloat16, device="cuda"),
                    u200=torch.empty((200, 512), dtype=torch.bfloat16, device="cuda"),
                    un200=torch.empty((200, 512), dtype=torch.bfloat16, device="cuda"),
                    l300=torch.empty((300, 256), dtype=torch.bfloat16, device="cuda"),
                    l5=torch.empty((5, 256), dtype=torch.bfloat16, device="cuda"))

    def run(o):
        Q.qknorm_fused(q, gq, k, gk, eps=1e-6, q_out=o["qo"], k_out=o["ko"])
        Q.qknorm_partial_sumsq(sq, sk, psq_q=o["pq"], psq_k=o["pk"])
        Q.qknorm_apply_with_stats(sq, sgq, o["pq"], eq, 4096, sk, sgk, o["pk"], ek, 4096,
                                  eps=1e-6, q_out=o["so"], k_out=o["sko"])
        Q.normproj_deferred(x, wf, eps=1e-6, y=o["y"])
        Q.qknorm_shard_fused(sq, sgq, mail_q, 4096, sk, sgk, mail_k, 4096, eps=1e-6,
                             q_out=o["fo"], k_out=o["fko"], psq_q=o["fpq"], psq_k=o["fpk"],
                             epoch=1, timed_out=tout)
        Q.qknorm_project_eliminated(el_x[200], el_w, 384, el_gq, el_gk, exact=False, y=o["e200"])
        Q.qknorm_project_eliminated(el_x[200], el_w, 384, el_gq, el_gk, exact=True, y=o["x200"])
        Q.qknorm_project_eliminated(el_x[12], el_w, 384, el_gq, el_gk, exact=True, y=o["e12"])
        Q.qknorm_project_unfused(el_x[200], el_g1, el_wp, 384, el_gq, el_gk, xn=o["un200"],
                                 y=o["u200"])
        Q.normproj_deferred_layernorm(ln_x[300], ln_w, ln_c, ln_b, eps=1e-5, y=o["l300"])
        Q.normproj_deferred_layernorm(ln_x[5], ln_w, ln_c, ln_b, eps=1e-5, y=o["l5"])

    eager = outputs()
    run(eager)
    torch.cuda.synchronize()
    ref = {n: to_host(t) for n, t in eager.items()}

    s = torch.cuda.Stream()
    got = outputs()
    with torch.cuda.stream(s):
        run(got)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(got)
    for rep in range(3):
        for t in got.values():
            t.zero_()
        run(eager)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in got.items():
            assert np.array_equal(to_host(t), ref[n]), f"replay {rep}: {n} differs"
    assert int(tout.item()) == 0
