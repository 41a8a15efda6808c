"""GPU parity of the pre-norm elimination ahead of QK-Norm and of the folded / deferred
LayerNorm-then-project, against the fp64 CPU oracle on the same seeded inputs.

Tolerance (as for the RMSNorm projection): |got - ref| <= 8e-3 |ref| + 2^-13 * A, where A
bounds the fp32 accumulation of the product in output units:
  elimination  A = |gamma_n| s_t sum_k |x_tk W'_kn|, s_t = 1/sqrt(mean(p_t^2) + eps_eff)
               (the intermediate p is stored in bf16, which the relative term covers)
  LayerNorm    A = r_t (sum_k |x_tk W'_kn| + |mu_t| sum_k |W'_kn|)
Large workloads are checked on a seeded sample of rows (rows are independent)."""

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


def sample_rows(T, n, seed=0):
    if T <= n + 2:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, n, replace=False)]))


# ----------------------------------------------------------------------------- elimination
def folded(w_bits, g_bits):
    """Oracle side of the fold: bf16(diag(gamma) W), [K, n]."""
    return oracle.round_bf16(oracle.fold_weight(w_bits, g_bits))


def elim_bound(x_bits, wf_bits, g_bits, eps_qk, eps_pre, exact):
    x, wf, g = widen(x_bits), widen(wf_bits), widen(g_bits)
    p = x @ wf
    eps = eps_qk * ((x * x).mean(axis=1) + eps_pre) if exact else np.full(len(x), eps_qk)
    s = 1.0 / np.sqrt((p * p).mean(axis=1) + eps)
    return s[:, None] * np.abs(g)[None, :] * (np.abs(x) @ np.abs(wf))


def run_elimination(Q, c, exact, rows, what, chain_rows=None):
    nq = c["nq"]
    wf_ref = folded(c["w"], c["gamma_pre"])              # [K, nq + nk]
    wqk = Q.normproj_fold_weight(to_dev(c["w"]), to_dev(c["gamma_pre"]))
    gk = to_dev(c["gamma_k"]) if c["nk"] > 0 else None
    y = Q.qknorm_project_eliminated(to_dev(c["x"]), wqk, nq, to_dev(c["gamma_q"]), gk,
                                    eps_qk=c["eps_qk"], eps_pre=c["eps_pre"], exact=exact)
    sync()
    assert np.array_equal(to_host(wqk), wf_ref)
    got = to_host(y)[rows]
    xs = np.ascontiguousarray(c["x"][rows])
    wq_ref = np.ascontiguousarray(wf_ref[:, :nq])
    if c["nk"] > 0:
        wk_ref, gk_h = np.ascontiguousarray(wf_ref[:, nq:]), c["gamma_k"]
    else:  # Q only: give the oracle a one-column K it can ignore
        wk_ref, gk_h = np.zeros((c["K"], 1), np.uint16), np.zeros(1, np.uint16) + 0x3F80
    rq, rk = oracle.qk_eliminated(xs, wq_ref, wk_ref, c["gamma_q"], gk_h, c["eps_qk"],
                                  c["eps_pre"], exact=exact)
    args = (c["eps_qk"], c["eps_pre"], exact)
    check_projection(got[:, :nq], rq, elim_bound(xs, wq_ref, c["gamma_q"], *args), what + " Q")
    if c["nk"] > 0:
        check_projection(got[:, nq:], rk, elim_bound(xs, wk_ref, c["gamma_k"], *args),
                         what + " K")
    if chain_rows is not None:
        # the unsimplified chain (pre-norm with the unfolded weights), which exact == 1 equals
        # for any epsilon and exact == 0 equals when eps_qk == 0
        sel = chain_rows
        cq, ck = oracle.qk_chain(np.ascontiguousarray(xs[sel]), c["gamma_pre"], c["wq"], c["wk"],
                                 c["gamma_q"], c["gamma_k"], c["eps_pre"], c["eps_qk"])
        xw = xs[sel]
        # the fold rounds gamma * W to bf16 once: the chain differs from the folded form by
        # at most that rounding, 2^-9 relative per weight, inside the same accumulation bound
        check_projection(got[sel, :nq], cq, elim_bound(xw, wq_ref, c["gamma_q"], *args),
                         what + " chain Q", abs_coeff=2.0 ** -8)
        check_projection(got[sel, nq:], ck, elim_bound(xw, wk_ref, c["gamma_k"], *args),
                         what + " chain K", abs_coeff=2.0 ** -8)
    return got


@pytest.mark.parametrize("exact", [False, True])
@pytest.mark.parametrize("T,K,nq,nk", [(300, 512, 384, 136), (300, 512, 384, 130),
                                       (16, 256, 256, 64), (37, 264, 200, 0),
                                       (129, 1024, 1024, 1024), (1, 520, 256, 264),
                                       (4096, 96, 4096, 4096), (2100, 256, 2048, 8),
                                       (4352, 64, 4096, 4096)])
def test_elimination_shapes(Q, T, K, nq, nk, exact):
    """Every product kernel (matrix-vector T <= 16, generic tiles for K % 32 != 0 or N % 8 != 0,
    pipelined tiles: 128 x 128 with 4 and with 2 stages, 256 x 256 with k-tiles of 64 and of 32,
    all with the ordinary output stores this entry point uses) followed by the row kernel on
    the two column blocks in place (16-byte team kernel, or the generic one when the K block is
    misaligned), Q only included."""
    c = inputs.make_elimination_case(T, seed=T + K + nq + nk, K=K, nq=nq, nk=nk)
    run_elimination(Q, c, exact, np.arange(T), f"T={T} K={K} nq={nq} nk={nk} exact={exact}")


@pytest.mark.parametrize("exact", [False, True])
@pytest.mark.parametrize("T", inputs.ELIMINATION["Ts"])
def test_elimination_full_width(Q, T, exact):
    """OLMo-2-7B widths (x [T, 4096], Wq, Wk [4096, 4096]); 32 sampled rows (all at T = 16),
    and the unsimplified chain on 6 of them."""
    c = inputs.make_elimination_case(T)
    rows = sample_rows(T, 32, seed=T)
    chain = np.arange(min(6, len(rows)))
    run_elimination(Q, c, exact, rows, f"T={T} exact={exact}", chain_rows=chain)


@pytest.mark.parametrize("T,K,nq,nk", [(300, 512, 384, 136), (16, 256, 256, 64),
                                       (37, 264, 200, 8), (129, 1024, 1024, 1024),
                                       (2048, 4096, 4096, 4096)])
def test_project_unfused_chain(Q, T, K, nq, nk):
    """The unsimplified chain in one call (RMSNorm launch, plain product with the unfolded
    weight, QK-Norm in place): xn against the oracle's RMSNorm, y against the oracle
    chain. The GPU rounds xn and p to bf16 on the way: the relative term covers p, and xn's
    rounding (2^-9 relative per element) enters the product's accumulation bound, hence the
    2^-8 absolute coefficient (as for the fold's rounding above)."""
    c = inputs.make_elimination_case(T, seed=T + K + nq + nk, K=K, nq=nq, nk=nk)
    wp = to_dev(c["w"])
    xn, y = Q.qknorm_project_unfused(to_dev(c["x"]), to_dev(c["gamma_pre"]), wp, nq,
                                     to_dev(c["gamma_q"]), to_dev(c["gamma_k"]),
                                     eps_qk=c["eps_qk"], eps_pre=c["eps_pre"])
    sync()
    rows = sample_rows(T, 64, seed=T)
    xs = np.ascontiguousarray(c["x"][rows])
    check_rows(to_host(xn)[rows], oracle.rmsnorm_rows(xs, c["gamma_pre"], c["eps_pre"]),
               f"unfused chain xn T={T}")
    cq, ck = oracle.qk_chain(xs, c["gamma_pre"], c["wq"], c["wk"], c["gamma_q"], c["gamma_k"],
                             c["eps_pre"], c["eps_qk"])
    wf_ref = folded(c["w"], c["gamma_pre"])
    got = to_host(y)[rows]
    args = (c["eps_qk"], c["eps_pre"], True)
    what = f"unfused chain T={T} K={K} nq={nq} nk={nk}"
    check_projection(got[:, :nq], cq, elim_bound(xs, wf_ref[:, :nq], c["gamma_q"], *args),
                     what + " Q", abs_coeff=2.0 ** -8)
    check_projection(got[:, nq:], ck, elim_bound(xs, wf_ref[:, nq:], c["gamma_k"], *args),
                     what + " K", abs_coeff=2.0 ** -8)


def test_elimination_eps_regime(Q):
    """Small activations (mean(x^2) ~ 1e-6 ~ eps): the plain form follows its own definition
    and visibly departs from the chain, the exact form still equals the chain."""
    c = inputs.make_elimination_case(64, seed=5, K=512, nq=256, nk=256)
    x = widen(c["x"]) * 1e-3
    c["x"] = inputs.f32_to_bf16_bits(x.astype(np.float32))
    c["eps_qk"] = 1e-3
    rows = np.arange(64)
    plain = run_elimination(Q, c, False, rows, "small-x plain")
    exact = run_elimination(Q, c, True, rows, "small-x exact", chain_rows=np.arange(8))
    assert np.max(np.abs(widen(plain) - widen(exact)) / np.abs(widen(exact))) > 0.05


# ----------------------------------------------------------------------------- LayerNorm
def ln_bound(x_bits, wf_bits, eps):
    x, wf = widen(x_bits), widen(wf_bits)
    mu = x.mean(axis=1)
    r = 1.0 / np.sqrt(((x - mu[:, None]) ** 2).mean(axis=1) + eps)
    return r[:, None] * (np.abs(x) @ np.abs(wf) + np.abs(mu)[:, None] * np.abs(wf).sum(axis=0))


def ln_reference_parts(c):
    wf_ref = folded(c["w"], c["gamma"])
    return wf_ref, oracle.colsum(wf_ref), oracle.matmul(c["beta"][None, :], c["w"])[0]


def test_fold_layernorm(Q):
    c = inputs.make_layernorm_case(1)
    wf_ref, cs_ref, b_ref = ln_reference_parts(c)
    wf, cs, b = Q.normproj_fold_layernorm(to_dev(c["w"]), to_dev(c["gamma"]), to_dev(c["beta"]))
    sync()
    assert np.array_equal(to_host(wf), wf_ref)
    # fp64 sums rounded once to fp32: within an fp32 rounding of the exact sum
    tol_c = 2.0 ** -23 * np.abs(cs_ref) + 2.0 ** -40 * np.abs(widen(wf_ref)).sum(axis=0)
    assert np.all(np.abs(to_host(cs).astype(np.float64) - cs_ref) <= tol_c)
    tol_b = 2.0 ** -23 * np.abs(b_ref) + 2.0 ** -40 * (np.abs(widen(c["beta"]))
                                                        @ np.abs(widen(c["w"])))
    assert np.all(np.abs(to_host(b).astype(np.float64) - b_ref) <= tol_b)
    # no beta: no bias
    _, cs2, b2 = Q.normproj_fold_layernorm(to_dev(c["w"]), to_dev(c["gamma"]), None)
    sync()
    assert b2 is None and np.array_equal(to_host(cs2), to_host(cs))


@pytest.mark.parametrize("stats", ["auto", None])
@pytest.mark.parametrize("T,x_mean", [(1, 0.0), (2048, 0.0), (16384, 0.0), (2048, 4.0),
                                      (16, 3.0)])
def test_deferred_layernorm(Q, T, x_mean, stats):
    """Both sources of the row statistics: a streaming pass into the workspace ("auto") and
    accumulation inside the product (None)."""
    c = inputs.make_layernorm_case(T, x_mean=x_mean)
    wf_ref, cs_ref, b_ref = ln_reference_parts(c)
    wf, cs, b = Q.normproj_fold_layernorm(to_dev(c["w"]), to_dev(c["gamma"]), to_dev(c["beta"]))
    y = Q.normproj_deferred_layernorm(to_dev(c["x"]), wf, cs, b, eps=c["eps"], row_stats=stats)
    sync()
    rows = sample_rows(T, 256, seed=T)
    xs = np.ascontiguousarray(c["x"][rows])
    ref = oracle.normproj_layernorm(xs, wf_ref, cs_ref, b_ref, c["eps"])
    check_projection(to_host(y)[rows], ref, ln_bound(xs, wf_ref, c["eps"]),
                     f"deferred LN T={T} mean={x_mean}")
    if T == 2048 and x_mean == 0.0:
        # the rewritten order is exact: the unfused LayerNorm-then-project in fp64 agrees too
        ref_u = oracle.layernorm_proj_unfused(xs[:16], c["gamma"], c["beta"], c["w"], c["eps"])
        check_projection(to_host(y)[rows[:16]], ref_u, ln_bound(xs[:16], wf_ref, c["eps"]),
                         "deferred LN vs unfused definition", abs_coeff=2.0 ** -8)


@pytest.mark.parametrize("stats", ["auto", None])
@pytest.mark.parametrize("T,K,N", [(5, 256, 130), (16, 1032, 64), (17, 1024, 520),
                                   (300, 264, 200), (129, 2048, 2048), (8200, 1056, 4104),
                                   (8200, 1024, 4104), (4096, 64, 4096), (4100, 192, 4104),
                                   (4100, 512, 2056), (12, 512, 4104), (8, 1000, 4104),
                                   (1, 8, 24), (3, 520, 4104), (4352, 128, 4096),
                                   (6000, 256, 6000)])
def test_deferred_layernorm_ragged(Q, T, K, N, stats):
    """All product kernels with the LayerNorm epilogue, ragged T and N, no beta, x with a mean
    of 2 (the mean term is exercised everywhere), statistics from the workspace pass or from
    inside the product."""
    rng = np.random.default_rng(T * 7 + K + N)
    x = inputs.f32_to_bf16_bits((widen(inputs.random_rows(rng, T, K, "bf16")) + 2.0)
                                .astype(np.float32))
    w = inputs.random_rows(rng, K, N, "bf16", scale=0.02)
    g = inputs.random_gamma(rng, K, "bf16")
    wf_ref = folded(w, g)
    cs_ref = oracle.colsum(wf_ref)
    wf, cs, b = Q.normproj_fold_layernorm(to_dev(w), to_dev(g), None)
    y = Q.normproj_deferred_layernorm(to_dev(x), wf, cs, None, eps=1e-5, row_stats=stats)
    sync()
    assert b is None
    rows = sample_rows(T, 128, seed=T)
    xs = np.ascontiguousarray(x[rows])
    check_projection(to_host(y)[rows], oracle.normproj_layernorm(xs, wf_ref, cs_ref, None, 1e-5),
                     ln_bound(xs, wf_ref, 1e-5), f"LN T={T} K={K} N={N}")


@pytest.mark.parametrize("T,K,N,pass_runs", [(4096, 2048, 2048, True), (300, 264, 200, False),
                                             (12, 2048, 2048, False)])
def test_deferred_layernorm_row_stats(Q, T, K, N, pass_runs):
    """The workspace holds (mean, 1/std) of every row when the streaming pass runs (matrix-core
    shapes) and is left untouched otherwise (K not a multiple of 64 and no 256-tile path; the
    matrix-vector path for T <= 16)."""
    import torch

    c = inputs.make_layernorm_case(T, seed=5, K=K, N=N, x_mean=3.0)
    wf, cs, b = Q.normproj_fold_layernorm(to_dev(c["w"]), to_dev(c["gamma"]), to_dev(c["beta"]))
    ws = torch.full((T, 2), float("nan"), dtype=torch.float32, device="cuda")
    Q.normproj_deferred_layernorm(to_dev(c["x"]), wf, cs, b, eps=c["eps"], row_stats=ws)
    sync()
    got = to_host(ws).astype(np.float64)
    if not pass_runs:
        assert np.all(np.isnan(got)), "row_stats written although the pass does not run"
        return
    xw = widen(c["x"])
    mu = xw.mean(axis=1)
    var = ((xw - mu[:, None]) ** 2).mean(axis=1)
    r = 1.0 / np.sqrt(var + c["eps"])
    # fp32 sums of x - x0 over K terms: the mean within 2^-16 of the mean |x - x0| (plus its own
    # rounding), r within 2^-14 relative; a dropped term or a wrong shift is off by far more
    spread = np.abs(xw - xw[:, :1]).mean(axis=1)
    assert np.all(np.abs(got[:, 0] - mu) <= 2.0 ** -16 * spread + 2.0 ** -22 * np.abs(mu)), \
        "row means"
    assert np.all(np.abs(got[:, 1] - r) <= 2.0 ** -14 * r), "row 1/std"


def test_layernorm_unfused_baseline(Q):
    c = inputs.make_layernorm_case(2048, seed=3, x_mean=1.0)
    wp = to_dev(c["w"])
    xn, y = Q.normproj_layernorm_unfused(to_dev(c["x"]), to_dev(c["gamma"]), to_dev(c["beta"]),
                                         wp, eps=c["eps"])
    sync()
    xn_h = to_host(xn)
    ln_ref = oracle.layernorm_rows(c["x"], c["gamma"], c["beta"], c["eps"])
    # a LayerNorm output can sit near zero (x near its mean, or beta cancelling): relative
    # error is unsound there, so the bound adds the fp32 rounding of the normalised value
    xw, g, be = widen(c["x"]), widen(c["gamma"]), widen(c["beta"])
    mu = xw.mean(axis=1, keepdims=True)
    r = 1.0 / np.sqrt(((xw - mu) ** 2).mean(axis=1, keepdims=True) + c["eps"])
    absb = (np.abs(xw) + np.abs(mu)) * r * np.abs(g) + np.abs(be)
    check_projection(xn_h, ln_ref, absb, "unfused LayerNorm rows", abs_coeff=2.0 ** -16)
    rows = sample_rows(2048, 256)
    xn_ref = oracle.round_bf16(ln_ref[rows])
    ref = oracle.matmul(xn_ref, c["w"])
    bound = np.abs(widen(xn_ref)) @ np.abs(widen(c["w"]))
    check_projection(to_host(y)[rows], ref, bound, "unfused LN projection",
                     abs_coeff=2.0 ** -12)
