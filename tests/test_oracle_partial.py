"""Pins of the oracle's combine with sender-side partial sums (each expert
owner returns one pre-summed row per (token, destination rank)): layouts
against sorted brute-force lists, reduction to the receiver-side combine when
every expert of a token lives on one rank, one-hot weights reading back exact
rows, and the rounding bound against an exact double-precision sum."""
import numpy as np
import pytest

import oracle
from oracle.brute import brute_plan
from workloads import CONFIGS, Config, f32_from_bf16_bits, make_inputs, renormalised


def _dispatch(cfg, inp):
    d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E)
    y = oracle.expert_standin(d["expert_x"], None, d["eoff"], cfg.H)
    return d, y


@pytest.mark.parametrize("seed", range(6))
def test_partial_layout_matches_sorted_lists(seed):
    g = np.random.default_rng(300 + seed)
    N = int(g.choice([1, 2, 3, 4, 8]))
    L = int(g.integers(1, 5))
    E, K, T = N * L, int(g.integers(1, 9)), int(g.integers(0, 7))
    idx = g.integers(0, E, size=(N, T, K)).astype(np.int32)
    pp = oracle.partial_plan(idx, E)
    visits = sorted({(s, t, int(idx[s, t, k]) // L) for s in range(N) for t in range(T)
                     for k in range(K)})
    assert pp["P"] == len(visits)
    for s in range(N):
        for d in range(N):
            assert pp["pc"][s, d] == sum(1 for (a, _, b) in visits if a == s and b == d)
    owner_order = sorted(visits, key=lambda v: (v[2], v[0], v[1]))     # (d, s, t)
    token_order = sorted(visits, key=lambda v: (v[0], v[2], v[1]))
    for row, (s, t, d) in enumerate(owner_order):
        assert pp["owner_row"][s, t, d] == row
    for row, (s, t, d) in enumerate(token_order):
        assert pp["token_row"][s, t, d] == row
    unvisited = np.ones((N, T, N), dtype=bool)
    for (s, t, d) in visits:
        unvisited[s, t, d] = False
    assert np.all(pp["owner_row"][unvisited] == -1) and np.all(pp["token_row"][unvisited] == -1)


def test_single_rank_equals_receiver_combine():
    """With one rank every token has one partial, bf16(full chain), and the
    final sum of one bf16 value rounds back to itself: bit-identical to the
    receiver-side combine."""
    cfg = CONFIGS["A"].with_(N=1, E=8, K=4, routing="uniform")
    inp = make_inputs(cfg)
    d, y = _dispatch(cfg, inp)
    ref = oracle.run_combine(y, inp["w"], d, cfg.H)["out"]
    got = oracle.run_partial_combine(y, inp["w"], inp["idx"], d, cfg.H)["out"]
    assert np.array_equal(got, ref)


def test_identity_when_all_experts_of_a_token_share_a_rank():
    """Identity experts, weights summing to one, every expert of a token on
    one rank: the one partial is bf16(x * sum w) = x, so out == x (-0 -> +0)."""
    cfg = Config("P", "same-rank", 4, 16, 256, 16, 3, "bf16", "uniform", 9)
    inp = make_inputs(cfg)
    g = np.random.default_rng(9)
    L = cfg.L
    ranks = g.integers(0, cfg.N, size=(cfg.N, cfg.T))
    inp["idx"] = (ranks[..., None] * L + g.integers(0, L, size=(cfg.N, cfg.T, cfg.K))).astype(np.int32)
    w = renormalised(inp["w"])
    d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E)
    got = oracle.run_partial_combine(d["expert_x"], w, inp["idx"], d, cfg.H)["out"]
    assert np.array_equal(got, np.where(inp["x"] == 0x8000, np.uint16(0), inp["x"]))


def test_one_hot_weights_read_back_each_slot():
    cfg = CONFIGS["A"].with_(routing="uniform", K=3)
    inp = make_inputs(cfg)
    N, T, K, H, E = cfg.N, cfg.T, cfg.K, cfg.H, cfg.E
    d = oracle.run_dispatch(inp["x"], inp["idx"], E)
    b = brute_plan(inp["idx"].tolist(), E)
    where = {stk: r for r, stk in enumerate(b["expert_rows"])}
    y = np.random.default_rng(4).integers(0, 0x7F00, size=(cfg.rows, H)).astype(np.uint16)
    for k in range(K):
        w = np.zeros((N, T, K), dtype=np.float32)
        w[:, :, k] = 1.0
        out = oracle.run_partial_combine(y, w, inp["idx"], d, H)["out"]
        for s in range(N):
            for t in range(T):
                assert np.array_equal(out[s, t], y[where[(s, t, k)]])


@pytest.mark.parametrize("key", ["A", "B", "Ep"])
def test_partial_sums_within_rounding_bound(key):
    """|out - exact| <= sum over partials of (chain error + half a bf16 ulp)
    + the fp32 sum's error + half a bf16 ulp of the result."""
    cfg = CONFIGS[key]
    if key == "Ep":
        cfg = cfg.with_(N=8, E=48, T=16, H=512)        # same routing rule, small
    inp = make_inputs(cfg)
    d, y = _dispatch(cfg, inp)
    res = oracle.run_partial_combine(y, inp["w"], inp["idx"], d, cfg.H)
    rows = oracle.expert_rows(inp["idx"], d)
    yv = f32_from_bf16_bits(y).astype(np.float64)
    terms = inp["w"].astype(np.float64)[..., None] * yv[rows]          # [N][T][K][H]
    exact = terms.sum(axis=2)
    mag = np.abs(terms).sum(axis=2)
    got = f32_from_bf16_bits(res["out"]).astype(np.float64)
    u = 2.0 ** -24
    K, Nd = cfg.K, cfg.N
    bound = (K * u * 1.01 * mag                     # fp32 chains inside the partials
             + 2.0 ** -8 * mag * (1 + 2 * K * u)    # bf16 rounding of every partial
             + Nd * u * 1.01 * mag * (1 + 2.0 ** -7)   # fp32 sum of the partials
             + 2.0 ** -8 * np.abs(got) + 2.0 ** -133)  # final bf16 rounding
    assert np.all(np.abs(got - exact) <= bound)
    # the bytes saved: one row per (token, destination rank)
    assert res["P"] <= cfg.rows
    if key == "Ep":
        assert res["P"] < 0.5 * cfg.rows           # 6 of 8 experts share rank 0


@pytest.mark.parametrize("key", ["A", "B"])
def test_single_token_form_matches_the_batch(key):
    """The one-token form gives every token's output of the whole-batch
    form (pinned above)."""
    cfg = CONFIGS[key].with_(T=24)
    inp = make_inputs(cfg)
    d, y = _dispatch(cfg, inp)
    out = oracle.run_partial_combine(y, inp["w"], inp["idx"], d, cfg.H)["out"]
    rows = oracle.expert_rows(inp["idx"], d)
    for s in range(cfg.N):
        for t in range(cfg.T):
            got = oracle.partial_token(y[rows[s, t]], inp["w"][s, t], inp["idx"][s, t] // cfg.L)
            assert np.array_equal(got, out[s, t]), (s, t)


def test_single_token_form_reduces_to_receiver_combine_on_one_rank():
    """All items on one rank: one partial, rounded twice to the same bf16."""
    g = np.random.default_rng(8)
    rows = g.integers(0, 0x7F00, size=(5, 64)).astype(np.uint16)
    w = g.random(5).astype(np.float32)
    got = oracle.partial_token(rows, w, np.full(5, 3, dtype=np.int32))
    assert np.array_equal(got, oracle.combine_token(rows, w))


def test_hand_worked_partial_example():
    """The partial-row layouts, partial rows and outputs of the hand-worked
    2-rank example (tests/golden/tiny_hand_example.json, "partial"), derived
    on paper from the definitions."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "tiny_hand_example.json")))
    gp = g["partial"]
    idx = np.array(g["idx"], dtype=np.int32)
    N, T, K, E = g["N"], g["T"], g["K"], g["E"]
    H = 4
    pp = oracle.partial_plan(idx, E)
    assert pp["pc"].tolist() == gp["pc"]
    assert pp["P"] == gp["P"]
    assert pp["token_row"].tolist() == gp["token_row"]
    assert pp["owner_row"].tolist() == gp["owner_row"]
    pl = oracle.plan(idx, E)
    # expert row r holds r + 1 in every element (exact in bf16)
    R = N * T * K
    y = oracle.f32_to_bf16(np.repeat(np.arange(1, R + 1, dtype=np.float32)[:, None], H, axis=1))
    w = np.array(gp["w"], dtype=np.float32)
    res = oracle.run_partial_combine(y, w, idx, pl, H)
    f = lambda a: f32_from_bf16_bits(a)[:, 0].tolist()  # noqa: E731
    assert f(res["psend"]) == gp["owner_layout_values"]
    assert f(res["precv"]) == gp["token_layout_values"]
    assert f32_from_bf16_bits(res["out"])[:, :, 0].tolist() == gp["out"]


@pytest.mark.parametrize("key", ["A", "C"])
def test_partial_tokens_matches_the_batch(key):
    """The many-token form gives every token of the whole-batch partial
    combine (pinned above)."""
    cfg = CONFIGS[key].with_(T=12)
    inp = make_inputs(cfg)
    d, y = _dispatch(cfg, inp)
    out = oracle.run_partial_combine(y, inp["w"], inp["idx"], d, cfg.H)["out"]
    rows = oracle.expert_rows(inp["idx"], d).reshape(-1, cfg.K)
    got = oracle.partial_tokens(y, rows, inp["w"].reshape(-1, cfg.K),
                                (inp["idx"] // cfg.L).reshape(-1, cfg.K))
    assert np.array_equal(got, out.reshape(-1, cfg.H))
