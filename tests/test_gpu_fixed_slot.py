"""GPU parity of the fixed-slot receive layout (T_max slots per (source rank,
expert), each expert's area slot-major) against the oracle: the plan, the
receive planes read at the oracle's slot rows, the combine rows, the
dispatch outputs and the combined tokens, all bit-exact, both transports;
the capacity error when a sender has more rows for one expert than T_max."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import run_cycle, say, to_dev
from workloads import CONFIGS, Config, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402  (fails loudly if the library is missing)

FIXED = mep.MOE_LAYOUT_FIXED_SLOT
TRANSPORTS = [mep.MOE_TRANSPORT_STAGED, mep.MOE_TRANSPORT_DIRECT]


def _slots_in_receive_order(idx, pl, T_max):
    """Slot row of every packed receive row: the oracle's transfer of each
    send row's item number names the item at each receive row."""
    N, T, K = idx.shape
    slot = oracle.slot_rows(idx, pl, T_max)
    item = np.empty(N * T * K, dtype=np.int64)
    srow = (np.arange(N)[:, None, None] * (T * K) + pl["pos"]).reshape(-1)
    item[srow] = np.arange(N * T * K)
    recv_item = oracle.transfer(item, pl, T, K)
    return slot.reshape(-1)[recv_item]


def _check(cfg, inp, T_max, transport, combine_mode=0):
    fp8 = cfg.dtype == "fp8"
    idx = inp["idx"]
    d = oracle.run_dispatch(inp["x"], idx, cfg.E, fp8=fp8)
    assert oracle.slot_capacity_ok(d["cnt"], T_max)
    gather = _slots_in_receive_order(idx, d, T_max)
    gpu = run_cycle(torch, mep, cfg, inp, T_max=T_max, transport=transport,
                    combine_mode=combine_mode, layout=FIXED, recv_gather=gather)
    for k in ["cnt", "pos", "soff", "roff", "G", "eoff", "send_meta", "recv_meta",
              "expert_src_rank", "expert_src_slot"]:
        if k in gpu:
            assert np.array_equal(gpu[k], d[k]), k
    assert np.array_equal(gpu["expert_offsets"], d["eoff"])
    for k in ["send_x", "recv_x", "expert_x"] + (["send_scale", "recv_scale", "expert_scale"] if fp8 else []):
        if k not in gpu:
            continue
        g, o = gpu[k], d[k]
        if o.dtype == np.float32:
            g, o = g.view(np.uint32), o.view(np.uint32)
        assert np.array_equal(g, o), k
    y = oracle.expert_standin(d["expert_x"], d["expert_scale"] if fp8 else None, d["eoff"], cfg.H)
    assert np.array_equal(gpu["y"], y)
    if combine_mode == mep.MOE_COMBINE_PARTIAL:
        ref = oracle.run_partial_combine(y, inp["w"], idx, d, cfg.H)
        assert gpu["P"] == ref["P"]
        if "psend" in gpu:
            assert np.array_equal(gpu["psend"], ref["psend"])
        assert np.array_equal(gpu["precv"], ref["precv"])
    else:
        ref = oracle.run_combine(y, inp["w"], d, cfg.H)
        if "comb_send" in gpu:
            assert np.array_equal(gpu["comb_send"], ref["comb_send"])
        assert np.array_equal(gpu["comb_recv"], ref["comb_recv"])
    assert np.array_equal(gpu["out"], ref["out"])


@pytest.mark.parametrize("transport", TRANSPORTS)
@pytest.mark.parametrize("key", ["A", "B"])
def test_fixed_slot_small_workloads(key, transport):
    cfg = CONFIGS[key]
    say(f"[gpu] fixed-slot {cfg.describe()} transport={transport}")
    _check(cfg, make_inputs(cfg), cfg.T, transport)


@pytest.mark.parametrize("transport", TRANSPORTS)
@pytest.mark.parametrize("seed", range(4))
def test_fixed_slot_random_groups(seed, transport):
    """Random groups with T below T_max (slots partly filled), distinct ids per
    token, short and odd rows, e4m3 dispatch."""
    g = np.random.default_rng(3000 + seed)
    N = int(g.choice([1, 2, 3, 5, 8]))
    L = int(g.integers(1, 6))
    K = int(g.integers(1, min(N * L, 8) + 1))
    fp8 = seed % 2 == 1
    H = int(g.choice([128, 384])) if fp8 else int(g.choice([8, 64, 200, 1032]))
    T_max = int(g.integers(1, 40))
    T = int(g.integers(0, T_max + 1)) if seed != 0 else T_max
    cfg = Config("R", "random", N, T, H, N * L, K, "fp8" if fp8 else "bf16", "softmax", 90 + seed)
    say(f"[gpu] fixed-slot random {cfg.describe()} T_max={T_max} transport={transport}")
    _check(cfg, make_inputs(cfg), T_max, transport)


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_fixed_slot_partial_combine(transport):
    cfg = CONFIGS["B"].with_(T=100)
    say(f"[gpu] fixed-slot + partial {cfg.describe()} transport={transport}")
    _check(cfg, make_inputs(cfg), 128, transport, mep.MOE_COMBINE_PARTIAL)


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_fixed_slot_full_decode(transport):
    """The DeepSeek-R1 decode shape at full size: 32 x 256 x 128 = 1 048 576 slots."""
    cfg = CONFIGS["C"]
    say(f"[gpu] fixed-slot full {cfg.describe()} transport={transport}")
    _check(cfg, make_inputs(cfg), cfg.T, transport)


def test_fixed_slot_capacity_error_writes_nothing():
    """Every token names expert 1 twice, so sender 0 has 2T rows for it, more
    than its T_max = T slots: the cycle reports MOE_ERR_CAPACITY and writes
    none of the outputs."""
    cfg = CONFIGS["A"]
    say(f"[gpu] fixed-slot capacity {cfg.describe()}")
    inp = make_inputs(cfg)
    bad = inp["idx"].copy()
    bad[0, :, :] = 1
    g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16,
                             mep.MOE_TRANSPORT_STAGED, mep.MOE_COMBINE_RECEIVER, FIXED)
    try:
        R = cfg.rows
        x, idx, w = to_dev(torch, inp["x"]), to_dev(torch, bad), to_dev(torch, inp["w"])
        expert_x = torch.full((R * cfg.H,), -1, dtype=torch.int16, device="cuda")
        offs = torch.full((cfg.E + 1,), -7, dtype=torch.int32, device="cuda")
        y = torch.zeros((R, cfg.H), dtype=torch.bfloat16, device="cuda")
        out = torch.full((cfg.N, cfg.T, cfg.H), -1, dtype=torch.int16, device="cuda")
        mep.moe_dispatch_send(g, cfg.T, x, idx)
        mep.moe_dispatch_recv(g, expert_x, None, offs)
        mep.moe_combine_send(g, y)
        mep.moe_combine_recv(g, w, out)
        assert mep.moe_group_status(g) == mep.MOE_ERR_CAPACITY
        assert torch.all(expert_x == -1).item()
        assert torch.all(offs == -7).item()
        assert torch.all(out == -1).item()
        # usable again with routing that fits
        gather = _slots_in_receive_order(inp["idx"], oracle.plan(inp["idx"], cfg.E), cfg.T)
        gpu = run_cycle(torch, mep, cfg, inp, group=g, layout=FIXED, recv_gather=gather)
        d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E)
        assert np.array_equal(gpu["recv_x"], d["recv_x"])
        y = oracle.expert_standin(d["expert_x"], None, d["eoff"], cfg.H)
        assert np.array_equal(gpu["y"], y)
        assert np.array_equal(gpu["out"], oracle.run_combine(y, inp["w"], d, cfg.H)["out"])
    finally:
        mep.moe_group_destroy(g)


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_fixed_slot_senders_run_before_the_group_offsets(monkeypatch, transport):
    """Fixed slots with the receiver-side combine: dispatch_send's kernels
    address every row from its sender's own counts ([EPMC] "Portable
    kernels": a sender writes to an address it knows without synchronising
    with the other ranks), and the group offsets are formed at dispatch_recv.
    In debug mode the offset tables are filled with -1 before dispatch_send;
    after dispatch_send they still hold -1 (not yet computed) while every
    slot already holds its row and meta word (the oracle's slot layout);
    dispatch_recv then forms the offsets and the whole cycle equals the
    oracle."""
    from tests.gpu_util import d2h, d2h_rows
    monkeypatch.setenv("MOE_EP_DEBUG", "1")
    cfg = CONFIGS["B"]
    say(f"[gpu] fixed-slot senders before offsets {cfg.describe()} transport={transport}")
    inp = make_inputs(cfg)
    N, T, K, E, H = cfg.N, cfg.T, cfg.K, cfg.E, cfg.H
    g = mep.moe_group_create(N, E, K, H, T, mep.MOE_BF16, transport, mep.MOE_COMBINE_RECEIVER,
                             FIXED)
    try:
        x, idx, w = to_dev(torch, inp["x"]), to_dev(torch, inp["idx"]), to_dev(torch, inp["w"])
        mep.moe_dispatch_send(g, T, x, idx)
        torch.cuda.synchronize()
        v = mep.moe_group_view_get(g)
        assert np.all(d2h(v.recv_base, (N + 1,), np.int32) == -1)
        assert np.all(d2h(v.recv_off, (N, N + 1), np.int32) == -1)
        assert np.all(d2h(v.expert_off, (E + 1,), np.int32) == -1)
        ref = oracle.run_dispatch_fixed(inp["x"], inp["idx"], E, T)
        named = np.sort(ref["slot"].reshape(-1))
        got_x = d2h_rows(v.recv_x, named, (H,), np.uint16)
        assert np.array_equal(got_x, ref["recv_x"][named])
        got_m = d2h_rows(v.recv_meta, named, (), np.int32)
        assert np.array_equal(got_m, ref["recv_meta"][named])
        # the rest of the cycle
        R = cfg.rows
        expert_x = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
        offs = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
        mep.moe_dispatch_recv(g, expert_x, None, offs)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
        assert np.array_equal(d2h(v.recv_base, (N + 1,), np.int32), ref["G"])
        assert np.array_equal(offs.cpu().numpy(), ref["eoff"])
        ex = expert_x.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(ex, ref["expert_x"])
        y = oracle.expert_standin(ref["expert_x"], None, ref["eoff"], H)
        y_dev = to_dev(torch, y).view(torch.bfloat16)
        out = torch.empty((N, T, H), dtype=torch.bfloat16, device="cuda")
        mep.moe_combine_send(g, y_dev)
        mep.moe_combine_recv(g, w, out)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
        d = oracle.run_dispatch(inp["x"], inp["idx"], E)
        want = oracle.run_combine(y, inp["w"], d, H)["out"]
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), want)
    finally:
        mep.moe_group_destroy(g)
