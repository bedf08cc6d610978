"""The seeded generators produce the shapes and routing structure each
workload states, deterministically."""
import numpy as np
import pytest

from workloads import CONFIGS, f32_from_bf16_bits, make_inputs, make_routing, make_tokens


@pytest.mark.parametrize("key", ["A", "B", "C", "E", "Ep"])
def test_shapes_and_ranges(key):
    cfg = CONFIGS[key]
    idx, w = make_routing(cfg)
    assert idx.shape == (cfg.N, cfg.T, cfg.K) and idx.dtype == np.int32
    assert w.shape == idx.shape and w.dtype == np.float32
    assert idx.min() >= 0 and idx.max() < cfg.E
    assert np.all(w > 0) and np.all(np.isfinite(w))
    # top-K ids of a token are distinct for every named workload
    srt = np.sort(idx, axis=-1)
    assert np.all(np.diff(srt, axis=-1) > 0)
    if cfg.routing in ("softmax_renorm", "zipf", "worst"):
        assert np.allclose(w.sum(-1), 1.0, atol=1e-6)


def test_determinism_and_per_rank_streams():
    cfg = CONFIGS["A"]
    a, b = make_inputs(cfg), make_inputs(cfg)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(make_tokens(cfg, 1), a["x"][1])
    i1, w1 = make_routing(cfg, ranks=[1])
    assert np.array_equal(i1[0], a["idx"][1]) and np.array_equal(w1[0], a["w"][1])


def test_token_values_are_bf16_normal():
    cfg = CONFIGS["B"]
    x = f32_from_bf16_bits(make_tokens(cfg, 0))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_zipf_skews_toward_rank0():
    cfg = CONFIGS["E"]
    idx, _ = make_routing(cfg)
    per_rank = np.bincount((idx // cfg.L).ravel(), minlength=cfg.N)
    assert per_rank[0] == per_rank.max() and per_rank[0] > 4 * per_rank.mean()


def test_worst_case_routes_all_of_rank0():
    cfg = CONFIGS["Ep"]
    idx, _ = make_routing(cfg)
    for row in idx.reshape(-1, cfg.K):
        assert set(range(cfg.L)) <= set(row.tolist())
