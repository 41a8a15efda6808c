"""The seeded input generator: determinism, shapes and the stated distributions (CPU)."""

import numpy as np
import pytest

from layerwise_qk_norm_amd import inputs


def test_same_seed_same_bits():
    a = inputs.make_case("olmo2-7b", 16, seed=0)
    b = inputs.make_case("olmo2-7b", 16, seed=0)
    c = inputs.make_case("olmo2-7b", 16, seed=1)
    for key in ("q", "k", "gamma_q", "gamma_k"):
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["q"], c["q"])


def test_weights_identical_across_T():
    a = inputs.make_case("olmo2-7b", 1)
    b = inputs.make_case("olmo2-7b", 256)
    assert np.array_equal(a["gamma_q"], b["gamma_q"])
    assert np.array_equal(a["q"][0], b["q"][0])


@pytest.mark.parametrize("workload,T", [("tiny-fp32", 64), ("olmo2-7b", 256),
                                        ("gqa-olmo2-32b-like", 512), ("tp8-shard", 4096),
                                        ("flashnorm-2048", 64)])
def test_shapes_and_moments(workload, T):
    c = inputs.make_case(workload, T)
    if workload == "flashnorm-2048":
        assert c["x"].shape == (T, 2048) and c["w"].shape == (2048, 2048)
        x = inputs.bf16_bits_to_f32(c["x"])
        w = inputs.bf16_bits_to_f32(c["w"])
        assert abs(x.std() - 1.0) < 0.01 and abs(w.std() - 0.02) < 0.001
        return
    q = c["q"] if c["dtype"] == "f32" else inputs.bf16_bits_to_f32(c["q"])
    gq = c["gamma_q"] if c["gamma_dtype"] == "f32" else inputs.bf16_bits_to_f32(c["gamma_q"])
    spec = inputs.WORKLOADS[workload]
    assert q.shape == (T, spec["dq"])
    assert c["k"].shape == (T, spec["dk"])
    sd = {"tiny-fp32": 1.0, "olmo2-7b": 2.0, "gqa-olmo2-32b-like": None, "tp8-shard": 1.0}[workload]
    if sd is not None:
        assert abs(q.std() / sd - 1.0) < 0.02
    assert abs(gq.mean() - 1.0) < 0.02
    if workload == "tp8-shard":
        assert c["ext_q"].shape == (7, T) and c["ext_q"].dtype == np.float32
        assert abs(c["ext_q"].mean() / 512.0 - 1.0) < 0.01


def test_gqa_outlier_columns():
    c = inputs.make_case("gqa-olmo2-32b-like", 512)
    q = inputs.bf16_bits_to_f32(c["q"])
    cols = c["outlier_cols_q"]
    assert cols.size == 51 and c["outlier_cols_k"].size == 10
    rms = np.sqrt((q * q).mean(axis=0))
    assert np.all(rms[cols] > 10.0)
    mask = np.ones(q.shape[1], bool)
    mask[cols] = False
    assert np.all(rms[mask] < 2.0)


def test_bf16_rounding_matches_torch():
    import torch

    rng = np.random.default_rng(3)
    v = rng.normal(0.0, 3.0, 10000).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(inputs.f32_to_bf16_bits(v), ref)
    assert np.array_equal(inputs.bf16_bits_to_f32(ref), torch.from_numpy(v).to(
        torch.bfloat16).float().numpy())
