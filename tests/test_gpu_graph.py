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

    c2 = inputs.make_case(2, 512, seed=8)
    c4 = inputs.make_case(4, 1000, seed=8)
    c5 = inputs.make_case(5, 300, seed=8)
    q, k, gq, gk = (to_dev(c2[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    sq, sk, sgq, sgk = (to_dev(c4[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    eq, ek = to_dev(c4["ext_q"]), to_dev(c4["ext_k"])
    x = to_dev(c5["x"])
    wf = Q.normproj_fold_weight(to_dev(c5["w"]), to_dev(c5["gamma"]))

    def outputs():
        return dict(qo=torch.empty_like(q), ko=torch.empty_like(k),
                    pq=torch.empty(1000, device="cuda"), pk=torch.empty(1000, device="cuda"),
                    so=torch.empty_like(sq), sko=torch.empty_like(sk),
                    y=torch.empty((300, 2048), dtype=torch.bfloat16, device="cuda"))

    def run(o):
        Q.qknorm_fused(q, gq, k, gk, eps=1e-6, q_out=o["qo"], k_out=o["ko"])
        Q.qknorm_partial_sumsq(sq, sk, psq_q=o["pq"], psq_k=o["pk"])
        Q.qknorm_apply_with_stats(sq, sgq, o["pq"], eq, 4096, sk, sgk, o["pk"], ek, 4096,
                                  eps=1e-6, q_out=o["so"], k_out=o["sko"])
        Q.normproj_deferred(x, wf, eps=1e-6, y=o["y"])

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
