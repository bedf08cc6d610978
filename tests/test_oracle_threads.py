"""The oracle's threaded forms (each stage's outer loop split over ranks or
experts, one range per thread; used to time the oracle on several host
cores) give every buffer of the single-thread forms bit for bit."""
import numpy as np
import pytest

import oracle
from workloads import CONFIGS, make_inputs

CASES = [("A", None, 3), ("C", 16, 7), ("D", 4, 16), ("Ep", 8, 5), ("A", 0, 2)]


@pytest.mark.parametrize("key,T,threads", CASES)
def test_threaded_forms_equal_single_thread(key, T, threads):
    cfg = CONFIGS[key]
    if key == "D":
        cfg = cfg.with_(N=8, E=32)          # a small fp8 group of the same kind
    inp = make_inputs(cfg, T=T)
    fp8 = cfg.dtype == "fp8"
    d1 = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E, fp8=fp8)
    d2 = oracle.run_dispatch_threads(inp["x"], inp["idx"], cfg.E, threads, fp8=fp8)
    for k, v in d1.items():
        if v is None:
            assert d2[k] is None, k
        else:
            assert np.array_equal(np.asarray(v), np.asarray(d2[k])), k
    y = oracle.expert_standin(d1["expert_x"], d1["expert_scale"], d1["eoff"], cfg.H)
    c1 = oracle.run_combine(y, inp["w"], d1, cfg.H)
    c2 = oracle.run_combine_threads(y, inp["w"], d2, cfg.H, threads)
    for k in c1:
        assert np.array_equal(c1[k], c2[k]), k
    p1 = oracle.run_partial_combine(y, inp["w"], inp["idx"], d1, cfg.H)
    p2 = oracle.run_partial_combine_threads(y, inp["w"], inp["idx"], d2, cfg.H, threads)
    for k in ("pc", "owner_row", "token_row", "psend", "precv", "out"):
        assert np.array_equal(p1[k], p2[k]), k
    assert p1["P"] == p2["P"]


def test_threaded_dispatch_rejects_invalid_ids():
    cfg = CONFIGS["A"]
    inp = make_inputs(cfg)
    bad = inp["idx"].copy()
    bad[1, 2, 0] = cfg.E
    with pytest.raises(oracle.RoutingError):
        oracle.run_dispatch_threads(inp["x"], bad, cfg.E, 2)
