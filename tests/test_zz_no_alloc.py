"""normproj_deferred_layernorm_noalloc (row statistics in the library's static per-GPU
workspace; the call allocates nothing) against normproj_deferred_layernorm with a caller-owned
workspace, through the C ABI: bit-identical outputs on consecutive calls whose sizes shrink, so
a stale workspace from the previous call would show, and the size limit."""

import numpy as np
import pytest

from helpers import to_dev, to_host
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


def test_noalloc_matches_workspace_entry_point(Q):
    import torch

    # the first two shapes run the statistics pass (pipelined product), the last the
    # in-product statistics (matrix-vector path), which uses no workspace at all
    for i, (T, K, N, mean) in enumerate([(4096, 1024, 768, 2.0), (1000, 512, 384, -1.0),
                                         (8, 512, 384, 0.5)]):
        c = inputs.make_layernorm_case(T, seed=40 + i, K=K, N=N, x_mean=mean)
        x = to_dev(c["x"])
        wf, cs, b = Q.normproj_fold_layernorm(to_dev(c["w"]), to_dev(c["gamma"]),
                                              to_dev(c["beta"]))
        ws = torch.empty((T, 2), dtype=torch.float32, device="cuda")
        y_ref = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        y = torch.full((T, N), 9.0, dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        Q.normproj_deferred_layernorm(x, wf, cs, b, eps=c["eps"], y=y_ref, row_stats=ws)
        Q.normproj_deferred_layernorm_noalloc(x, wf, cs, b, eps=c["eps"], y=y)
        torch.cuda.synchronize()
        got, ref = to_host(y), to_host(y_ref)
        assert np.array_equal(got, ref), f"call {i} (T={T}): outputs differ"


def test_noalloc_rejects_rows_beyond_the_workspace(Q):
    import torch

    T, K, N = 131073, 64, 64
    x = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda")
    wf = torch.zeros((K, N), dtype=torch.bfloat16, device="cuda")
    cs = torch.zeros((N,), dtype=torch.float32, device="cuda")
    y = torch.zeros((T, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(Q.QknError) as e:
        Q.normproj_deferred_layernorm_noalloc(x, wf, cs, None, y=y)
    assert e.value.status == 8
