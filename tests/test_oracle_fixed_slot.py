"""Pins of the oracle's fixed-slot receive layout (T_max slots per (source
rank, expert), slot index major and source minor within each expert's area):
slot rows against a brute-force walk of the routing, slot contents against
identity-carrying tokens, the dispatch result against the packed layout's
(pinned elsewhere), and the capacity rule."""
import numpy as np
import pytest

import oracle
from workloads import CONFIGS, Config, make_inputs


def _brute_slots(idx, E, T_max):
    """Walk the items of each sender in (t,k) order; the i-th item of (s, e)
    takes slot i of that pair: row s of slot plane i of expert e's area."""
    N, T, K = idx.shape
    seen = {}
    slot = np.zeros(idx.shape, dtype=np.int64)
    for s in range(N):
        for t in range(T):
            for k in range(K):
                e = int(idx[s, t, k])
                i = seen.get((s, e), 0)
                seen[(s, e)] = i + 1
                area = e * T_max * N                  # expert e's T_max planes of N rows
                slot[s, t, k] = area + i * N + s
    return slot, seen


def _random_group(seed, distinct=False):
    g = np.random.default_rng(seed)
    N = int(g.choice([1, 2, 3, 4, 8]))
    L = int(g.integers(1, 5))
    E = N * L
    K = int(g.integers(1, min(E, 6) + 1)) if distinct else int(g.integers(1, 7))
    T_max = int(g.integers(1, 9))
    T = int(g.integers(0, T_max + 1))
    if distinct:
        idx = np.stack([np.stack([g.permutation(E)[:K] for _ in range(T)]) if T else
                        np.zeros((0, K), dtype=np.int64) for _ in range(N)]).astype(np.int32)
    else:
        idx = g.integers(0, E, size=(N, T, K)).astype(np.int32)
    return idx.reshape(N, T, K), E, T_max


@pytest.mark.parametrize("seed", range(8))
def test_slot_rows_match_brute_force(seed):
    idx, E, T_max = _random_group(400 + seed, distinct=seed % 2 == 0)
    pl = oracle.plan(idx, E)
    brute, counts = _brute_slots(idx, E, T_max)
    fits = all(c <= T_max for c in counts.values())
    assert oracle.slot_capacity_ok(pl["cnt"], T_max) == fits
    if not fits:
        return
    got = oracle.slot_rows(idx, pl, T_max)
    assert np.array_equal(got, brute)
    N = idx.shape[0]
    flat = got.reshape(-1)
    assert len(set(flat.tolist())) == flat.size                  # one item per slot
    assert flat.size == 0 or (flat.min() >= 0 and flat.max() < N * E * T_max)


def test_capacity_rule():
    """Distinct ids per token always fit (a sender has at most T <= T_max
    rows for one expert); a token naming one expert twice can overflow."""
    for seed in range(20):
        idx, E, T_max = _random_group(500 + seed, distinct=True)
        assert oracle.slot_capacity_ok(oracle.plan(idx, E)["cnt"], T_max)
    idx = np.zeros((2, 3, 2), dtype=np.int32)                     # every item -> expert 0
    assert not oracle.slot_capacity_ok(oracle.plan(idx, 4)["cnt"], 3)
    assert oracle.slot_capacity_ok(oracle.plan(idx, 4)["cnt"], 6)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("seed", range(4))
def test_fixed_layout_gives_the_packed_dispatch_result(seed, fp8):
    idx, E, T_max = _random_group(600 + seed, distinct=True)
    N, T, K = idx.shape
    H = 256 if fp8 else 40
    cfg = Config("S", "slots", N, T, H, E, K, "fp8" if fp8 else "bf16", "uniform", 7 + seed)
    x = make_inputs(cfg)["x"]
    packed = oracle.run_dispatch(x, idx, E, fp8=fp8)
    fixed = oracle.run_dispatch_fixed(x, idx, E, T_max, fp8=fp8)
    assert fixed["capacity_ok"]
    for k in ["expert_x", "expert_src_rank", "expert_src_slot"] + (["expert_scale"] if fp8 else []):
        assert np.array_equal(fixed[k], packed[k]), k


def test_slot_contents_carry_their_tokens():
    """Identity-carrying tokens (element 0 = s, element 1 = t): the first cnt
    slots of (source s, expert e) -- row s of slot planes 0, 1, ... of e's
    area -- hold the tokens of sender s routed to e, t ascending, with their
    meta words; every other slot is empty, and receiver d's rows are the areas
    of its experts d*L .. d*L + L - 1."""
    cfg = CONFIGS["A"].with_(N=4, E=8, K=2, T=6, H=16, routing="uniform")
    T_max = 9
    inp = make_inputs(cfg)
    N, T, K, E, L = cfg.N, cfg.T, cfg.K, cfg.E, cfg.L
    x = np.zeros((N, T, cfg.H), dtype=np.uint16)
    x[:, :, 0] = np.arange(N)[:, None]
    x[:, :, 1] = np.arange(T)[None, :]
    res = oracle.run_dispatch_fixed(x, inp["idx"], E, T_max)
    meta = res["recv_meta"]
    filled = np.zeros(N * E * T_max, dtype=bool)
    for d in range(N):
        for s in range(N):
            for j in range(L):
                e = d * L + j
                items = [(t, k) for t in range(T) for k in range(K) if inp["idx"][s, t, k] == e]
                for i, (t, k) in enumerate(items):
                    q = d * L * T_max * N + (j * T_max + i) * N + s
                    row = res["recv_x"][q]
                    assert (row[0], row[1]) == (s, t)
                    assert meta[q] == t * K + k
                    filled[q] = True
    assert np.all(meta[~filled] == -1)


def test_hand_worked_slot_rows():
    """Slot rows of the hand-worked 2-rank example (tests/golden/
    tiny_hand_example.json, "fixed_slot"), derived on paper."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "tiny_hand_example.json")))
    idx = np.array(g["idx"], dtype=np.int32)
    pl = oracle.plan(idx, g["E"])
    slot = oracle.slot_rows(idx, pl, g["fixed_slot"]["T_max"])
    assert slot.tolist() == g["fixed_slot"]["slot_row"]
