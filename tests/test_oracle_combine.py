"""Pins of the oracle's combine: identity experts with weights summing to one
return the input bit-exactly; workload A's stand-in expert gives a closed form;
the fp32 chain stays within the rounding bound of an exact double sum; one-hot
weights read back exactly the expert row each (t,k) went to."""
import numpy as np
import pytest

import oracle
from oracle.brute import brute_plan
from workloads import CONFIGS, f32_from_bf16_bits, make_inputs, renormalised

U = 2.0 ** -24


def _ulp_dist_bf16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in units of bf16 ulp on the monotone integer line of patterns."""
    def ordered(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


@pytest.mark.parametrize("key", ["A", "B", "C"])
def test_identity_experts_return_the_input(key):
    """y = expert input and renormalised weights: out == x bit-exactly
    (the fp32 sum is x*(1 +- K*2^-24), far inside half a bf16 ulp), except
    that an input -0 comes back as +0: the chain starts from +0.  The
    DeepSeek-R1 shape runs with 16 tokens per rank (the full batch is a GPU
    test) and some -0 inputs planted."""
    cfg = CONFIGS[key]
    if key == "C":
        cfg = cfg.with_(T=16)
    inp = make_inputs(cfg)
    if key == "C":
        inp["x"].reshape(-1)[::9973] = 0x8000
    w = renormalised(inp["w"])
    d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E)
    c = oracle.run_combine(d["expert_x"], w, d, cfg.H)
    expect = np.where(inp["x"] == 0x8000, np.uint16(0), inp["x"])
    assert np.array_equal(c["out"], expect)
    if key == "C":
        assert (inp["x"] == 0x8000).sum() > 0


def test_closed_form_workload_a():
    """Stand-in expert y = x*(e+1): out = x * sum_k w_k (e_k+1) up to the
    rounding of y to bf16 and of the result (<= 2 bf16 ulp)."""
    cfg = CONFIGS["A"]
    inp = make_inputs(cfg)
    d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E)
    y = oracle.expert_standin(d["expert_x"], None, d["eoff"], cfg.H)
    c = oracle.run_combine(y, inp["w"], d, cfg.H)
    x = f32_from_bf16_bits(inp["x"]).astype(np.float64)
    factor = (inp["w"].astype(np.float64) * (inp["idx"] + 1)).sum(axis=-1)
    expect = x * factor[..., None]
    got = f32_from_bf16_bits(c["out"]).astype(np.float64)
    tol = 2 * 2.0 ** -8 * np.abs(expect) + 1e-30
    assert np.all(np.abs(got - expect) <= tol)


@pytest.mark.parametrize("key", ["A", "B"])
def test_fp32_chain_within_bound_of_exact_sum(key):
    """|bf16(chain) - exact| <= gamma_K * sum|w y| + half a bf16 ulp of the
    rounded result, gamma_K = K u / (1 - K u), u = 2^-24."""
    cfg = CONFIGS[key]
    inp = make_inputs(cfg)
    d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E)
    y = oracle.expert_standin(d["expert_x"], None, d["eoff"], cfg.H)
    c = oracle.run_combine(y, inp["w"], d, cfg.H)
    exact, mag = oracle.combine_recv_f64(c["comb_recv"], d["pos"], inp["w"], cfg.H)
    got = f32_from_bf16_bits(c["out"]).astype(np.float64)
    K = cfg.K
    gamma = K * U / (1 - K * U)
    # bf16 keeps 8 significant bits: half an ulp is at most 2^-8 of the value
    half_ulp = np.maximum(np.abs(got), np.abs(exact)) * 2.0 ** -8 + 2.0 ** -133
    assert np.all(np.abs(got - exact) <= gamma * mag * (1 + 2.0 ** -7) + half_ulp)


def test_one_hot_weights_read_back_each_slot():
    """With w = e_k (one-hot) the output is exactly the expert row (s,t,k) was
    shuffled to, located independently by the brute-force layout."""
    cfg = CONFIGS["A"].with_(routing="uniform")      # duplicates inside tokens too
    inp = make_inputs(cfg)
    N, T, K, H, E = cfg.N, cfg.T, cfg.K, cfg.H, cfg.E
    d = oracle.run_dispatch(inp["x"], inp["idx"], E)
    b = brute_plan(inp["idx"].tolist(), E)
    R = cfg.rows
    y = np.zeros((R, H), dtype=np.uint16)
    g = np.random.default_rng(5)
    y[:] = g.integers(0, 0x7F00, size=(R, H)).astype(np.uint16)   # finite bf16 patterns
    comb_recv = oracle.combine_transfer(oracle.combine_send(y, d), d, T, K)
    where = {stk: r for r, stk in enumerate(b["expert_rows"])}
    for k in range(K):
        w = np.zeros((N, T, K), dtype=np.float32)
        w[:, :, k] = 1.0
        out = oracle.combine_recv(comb_recv, d["pos"], w, H)
        for s in range(N):
            for t in range(T):
                assert np.array_equal(out[s, t], y[where[(s, t, k)]])


def test_combine_token_matches_full_combine():
    cfg = CONFIGS["A"]
    inp = make_inputs(cfg)
    d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E)
    y = oracle.expert_standin(d["expert_x"], None, d["eoff"], cfg.H)
    c = oracle.run_combine(y, inp["w"], d, cfg.H)
    T, K = cfg.T, cfg.K
    for s, t in [(0, 0), (1, T - 1), (0, 7)]:
        rows = c["comb_recv"][s * T * K + d["pos"][s, t]]
        assert np.array_equal(oracle.combine_token(rows, inp["w"][s, t]), c["out"][s, t])


def test_ulp_distance_helper():
    a = np.array([0x3F80, 0x0000, 0x8000, 0x0001, 0x8001], dtype=np.uint16)
    b = np.array([0x3F81, 0x8000, 0x0001, 0x8001, 0x0001], dtype=np.uint16)
    assert _ulp_dist_bf16(a, b).tolist() == [1, 0, 1, 2, 2]


def test_hand_worked_combine():
    """The receiver-side combine of the hand-worked 2-rank example
    (tests/golden/tiny_hand_example.json, "combine"), derived on paper."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "tiny_hand_example.json")))
    idx = np.array(g["idx"], dtype=np.int32)
    N, T, K, E = g["N"], g["T"], g["K"], g["E"]
    H = 4
    pl = oracle.plan(idx, E)
    y = oracle.f32_to_bf16(np.repeat(np.arange(1, N * T * K + 1, dtype=np.float32)[:, None], H,
                                     axis=1))
    w = np.array(g["partial"]["w"], dtype=np.float32)
    out = oracle.run_combine(y, w, pl, H)["out"]
    got = (out.astype(np.uint32) << 16).view(np.float32)[:, :, 0]
    assert got.tolist() == g["combine"]["out"]


@pytest.mark.parametrize("key", ["A", "B"])
def test_combine_tokens_matches_full_combine(key):
    """The many-token form (returned rows indexed in the expert-order output
    y) gives every token of the whole-batch combine (pinned above)."""
    cfg = CONFIGS[key].with_(T=24)
    inp = make_inputs(cfg)
    d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E)
    y = oracle.expert_standin(d["expert_x"], None, d["eoff"], cfg.H)
    c = oracle.run_combine(y, inp["w"], d, cfg.H)
    rows = oracle.expert_rows(inp["idx"], d).reshape(-1, cfg.K)
    got = oracle.combine_tokens(y, rows, inp["w"].reshape(-1, cfg.K))
    assert np.array_equal(got, c["out"].reshape(-1, cfg.H))
