"""Pins of the oracle's dispatch steps against things other than itself:
a hand-worked example, an independent sort-based brute force (including
exhaustive enumeration of every routing of a tiny group), the invariants the
pages fix, and property checks on the moved bytes."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle.brute import brute_plan
from workloads import CONFIGS, make_inputs, make_routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "tiny_hand_example.json")))
    idx = np.array(g["idx"], dtype=np.int32)
    N, T, K, E = g["N"], g["T"], g["K"], g["E"]
    pl = oracle.plan(idx, E)
    assert pl["cnt"].tolist() == g["cnt"]
    assert pl["soff"].tolist() == g["soff"]
    assert pl["pos"].tolist() == g["pos"]
    assert pl["roff"].tolist() == g["roff"]
    assert pl["G"].tolist() == g["G"]
    assert pl["eoff"].tolist() == g["eoff"]
    # rows carry their own (rank, token) identity so the moves can be read off
    H = 8
    x = np.zeros((N, T, H), dtype=np.uint16)
    for s in range(N):
        for t in range(T):
            x[s, t, :] = 100 * s + t
    d = oracle.run_dispatch(x, idx, E)
    assert d["send_meta"].tolist() == g["send_meta"]
    assert d["recv_meta"].tolist() == g["recv_meta"]
    assert d["expert_src_rank"].tolist() == g["expert_src_rank"]
    assert d["expert_src_slot"].tolist() == g["expert_src_slot"]
    y = np.repeat(np.arange(N * T * K, dtype=np.uint16)[:, None], H, axis=1)
    comb = oracle.combine_transfer(oracle.combine_send(y, pl), pl, T, K)
    assert comb[:, 0].tolist() == g["comb_recv_from_expert_row"]


def _check_against_brute(idx, E, H=4):
    N, T, K = idx.shape
    b = brute_plan(idx.tolist(), E)
    pl = oracle.plan(idx, E)
    assert pl["cnt"].tolist() == b["cnt"]
    assert pl["pos"].tolist() == b["pos"]
    assert pl["G"].tolist() == b["G"]
    assert pl["eoff"].tolist() == b["eoff"]
    # identity-carrying rows: word 0 = s, word 1 = t, word 2 = k
    x = np.zeros((N, T, H), dtype=np.uint16)
    for s in range(N):
        x[s, :, 0] = s
        x[s, :, 1] = np.arange(T)
    d = oracle.run_dispatch(x, idx, E)
    for rows_key, buf, meta in (("send_rows", d["send_x"], d["send_meta"]),
                                ("recv_rows", d["recv_x"], d["recv_meta"])):
        for r, (s, t, k) in enumerate(b[rows_key]):
            assert buf[r, 0] == s and buf[r, 1] == t and meta[r] == t * K + k, (rows_key, r)
    for r, (s, t, k) in enumerate(b["expert_rows"]):
        assert d["expert_x"][r, 0] == s and d["expert_x"][r, 1] == t
        assert d["expert_src_rank"][r] == s and d["expert_src_slot"][r] == t * K + k
    rows = oracle.expert_rows(idx, pl)
    for r, (s, t, k) in enumerate(b["expert_rows"]):
        assert rows[s, t, k] == r
    assert np.array_equal(oracle.send_meta(pl["pos"]), d["send_meta"])
    return pl


def test_exhaustive_tiny_routings():
    """Every routing of N=2, T=2, E=4 with K=1 (4^4 = 256 cases) and with K=2
    (16^4 = 65536 cases, duplicates included): oracle == brute force on the
    integer plan; the page's receive bound N*T*max(K, E/N) always holds, and
    its tight form N*T*min(K, E/N) holds when a token's ids are distinct."""
    N, T, E = 2, 2, 4
    L = E // N
    for K in (1, 2):
        choices = list(itertools.product(range(E), repeat=K))
        worst_any, worst_distinct = 0, 0
        for combo in itertools.product(choices, repeat=N * T):
            idx = np.array(combo, dtype=np.int32).reshape(N, T, K)
            b = brute_plan(idx.tolist(), E)
            pl = oracle.plan(idx, E)
            assert pl["pos"].tolist() == b["pos"]
            assert pl["G"].tolist() == b["G"]
            assert pl["eoff"].tolist() == b["eoff"]
            recv = np.diff(pl["G"])
            assert recv.max() <= N * T * max(K, L)
            worst_any = max(worst_any, int(recv.max()))
            if all(len(set(c)) == K for c in combo):
                assert recv.max() <= N * T * min(K, L)
                worst_distinct = max(worst_distinct, int(recv.max()))
        assert worst_any == N * T * K               # all copies to one rank
        assert worst_distinct == N * T * min(K, L)  # the tight bound is reached


@pytest.mark.parametrize("seed", range(12))
def test_random_small_groups_match_brute(seed):
    g = np.random.default_rng(100 + seed)
    N = int(g.choice([1, 2, 3, 4, 8]))
    L = int(g.integers(1, 5))
    E = N * L
    K = int(g.integers(1, 9))
    T = int(g.integers(0, 7))
    idx = g.integers(0, E, size=(N, T, K)).astype(np.int32)
    _check_against_brute(idx, E)


@pytest.mark.parametrize("key", ["A", "B", "C", "E", "Ep"])
def test_plan_invariants_on_workloads(key):
    cfg = CONFIGS[key]
    idx, _ = make_routing(cfg)
    N, T, K, E, L = cfg.N, cfg.T, cfg.K, cfg.E, cfg.L
    pl = oracle.plan(idx, E)
    # counts per sender sum to T*K
    assert np.all(pl["cnt"].sum(axis=1) == T * K)
    # positions are a bijection of each sender's T*K slots, grouped by expert
    for s in range(N):
        p = pl["pos"][s].ravel()
        assert np.array_equal(np.sort(p), np.arange(T * K))
        e = idx[s].ravel()
        assert np.all(p >= pl["soff"][s][e]) and np.all(p < pl["soff"][s][e + 1])
    # receive totals: sum to N*T*K, within the page's bound and the tight bound
    recv = np.diff(pl["G"])
    assert recv.sum() == N * T * K and pl["G"][N] == N * T * K
    assert recv.max() <= N * T * max(K, L)
    distinct = all(len(set(r)) == K for r in idx.reshape(-1, K).tolist())
    if distinct:
        assert recv.max() <= N * T * min(K, L)
    assert pl["eoff"][E] == N * T * K and np.all(np.diff(pl["eoff"]) >= 0)
    if key == "Ep":
        assert recv[0] == N * T * L           # every token sends L rows to rank 0


def test_pack_transfer_shuffle_move_every_pair_once():
    """Bytes of workload A through the whole dispatch: every expert row holds
    the token of its recorded (rank, slot), that (t,k) really routed to the
    row's expert, and the union over rows is every (s,t,k) exactly once."""
    cfg = CONFIGS["A"]
    inp = make_inputs(cfg)
    d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E)
    N, T, K, E = cfg.N, cfg.T, cfg.K, cfg.E
    seen = set()
    eoff = d["eoff"]
    for e in range(E):
        for r in range(eoff[e], eoff[e + 1]):
            s, slot = int(d["expert_src_rank"][r]), int(d["expert_src_slot"][r])
            t, k = divmod(slot, K)
            assert inp["idx"][s, t, k] == e
            assert np.array_equal(d["expert_x"][r], inp["x"][s, t])
            seen.add((s, t, k))
    assert len(seen) == N * T * K
    # the transfer moved each (s -> d) region unchanged
    L = cfg.L
    for s in range(N):
        for dd in range(N):
            a, b = d["soff"][s][dd * L], d["soff"][s][(dd + 1) * L]
            q = d["G"][dd] + d["roff"][dd][s]
            assert np.array_equal(d["recv_x"][q:q + b - a], d["send_x"][s * T * K + a:s * T * K + b])


def test_fp8_dispatch_rows_are_the_quantised_tokens():
    cfg = CONFIGS["A"].with_(dtype="fp8")
    inp = make_inputs(cfg)
    d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E, fp8=True)
    for r in range(cfg.rows):
        s, slot = int(d["expert_src_rank"][r]), int(d["expert_src_slot"][r])
        q, sc = oracle.quant_row_fp8(inp["x"][s, slot // cfg.K])
        assert np.array_equal(d["expert_x"][r], q)
        assert np.array_equal(d["expert_scale"][r], sc)


def test_invalid_expert_id_is_rejected():
    idx = np.array([[[0, 4]], [[1, 2]]], dtype=np.int32)
    with pytest.raises(oracle.RoutingError):
        oracle.route_count(idx, 4)
    with pytest.raises(oracle.RoutingError):
        oracle.route_count(np.array([[[-1]], [[0]]], dtype=np.int32), 2)


def test_empty_batch():
    cfg = CONFIGS["A"]
    inp = make_inputs(cfg, T=0)
    d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E)
    assert d["cnt"].sum() == 0 and d["G"].tolist() == [0] * (cfg.N + 1)
    assert d["expert_x"].shape[0] == 0
