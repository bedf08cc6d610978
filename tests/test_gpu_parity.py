"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
seeded inputs.  Integer and byte buffers must match bit-exactly; the combine
output must be within 1 bf16 ulp of the oracle's fp32 k-ascending fma chain
(the same chain on both sides, so 0 ulp is expected and checked separately)."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import d2h, run_cycle, say, ulp_dist_bf16
from workloads import CONFIGS, Config, make_inputs, make_routing, make_tokens, renormalised

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402  (fails loudly if the library is missing)


def _plus_zero(x):
    """The fma chain starts from +0, so an input -0 comes back as +0."""
    return np.where(x == 0x8000, np.uint16(0), x)


INT_KEYS = ["cnt", "pos", "soff", "roff", "G", "eoff", "send_meta", "recv_meta",
            "expert_src_rank", "expert_src_slot"]


def _compare_all(cfg, inp, gpu, *, identity=False):
    """Every buffer the run produced against the oracle (the send-side
    buffers exist only with the staged transport)."""
    fp8 = cfg.dtype == "fp8"
    d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E, fp8=fp8)
    for k in INT_KEYS:
        if k in gpu:
            assert np.array_equal(gpu[k], d[k]), k
    assert np.array_equal(gpu["expert_offsets"], d["eoff"])
    for k in ["send_x", "recv_x", "expert_x"] + (["send_scale", "recv_scale", "expert_scale"] if fp8 else []):
        if k not in gpu:
            continue
        g, o = gpu[k], d[k]
        if o.dtype == np.float32:
            g, o = g.view(np.uint32), o.view(np.uint32)
        bad = np.argwhere(g != o)
        assert bad.size == 0, (k, bad[:5])
    # combine from the oracle's stand-in expert output, which the GPU's (torch,
    # outside the path) must equal, given the equal expert rows above
    y = oracle.expert_standin(d["expert_x"], d["expert_scale"] if fp8 else None, d["eoff"], cfg.H)
    assert np.array_equal(gpu["y"], y)
    c = oracle.run_combine(y, inp["w"], d, cfg.H)
    if "comb_send" in gpu:
        assert np.array_equal(gpu["comb_send"], c["comb_send"])
    assert np.array_equal(gpu["comb_recv"], c["comb_recv"])
    dist = ulp_dist_bf16(gpu["out"], c["out"])
    assert dist.max(initial=0) <= 1, dist.max()
    assert dist.max(initial=0) == 0, "same fma chain on both sides should agree bit-exactly"
    if identity:
        assert np.array_equal(gpu["out"], _plus_zero(inp["x"]))


TRANSPORTS = [0, 1]     # staged, direct


@pytest.mark.parametrize("transport", TRANSPORTS)
@pytest.mark.parametrize("key", ["A", "B"])
def test_parity_small_workloads(key, transport):
    cfg = CONFIGS[key]
    say(f"[gpu] parity {cfg.describe()} transport={transport}")
    inp = make_inputs(cfg)
    _compare_all(cfg, inp, run_cycle(torch, mep, cfg, inp, transport=transport))


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_parity_tiny_fp8(transport):
    cfg = CONFIGS["A"].with_(dtype="fp8", H=512)
    say(f"[gpu] parity {cfg.describe()} transport={transport}")
    inp = make_inputs(cfg)
    _compare_all(cfg, inp, run_cycle(torch, mep, cfg, inp, transport=transport))


@pytest.mark.parametrize("transport", TRANSPORTS)
@pytest.mark.parametrize("seed", range(6))
def test_parity_random_groups(seed, transport):
    """Random group shapes: several ranks and experts per rank, K from 1 to 12
    (ids with duplicates), ragged T below the group's maximum, odd hidden sizes
    (short rows, rows not a multiple of a wave's vectors)."""
    g = np.random.default_rng(1000 + seed)
    N = int(g.choice([1, 2, 3, 5, 8, 16]))
    L = int(g.integers(1, 6))
    K = int(g.integers(1, 13))
    fp8 = seed % 3 == 2
    H = int(g.choice([128, 384, 1024])) if fp8 else int(g.choice([8, 64, 200, 520, 1032, 4104]))
    T_max = int(g.integers(1, 40))
    T = int(g.integers(0, T_max + 1)) if seed != 0 else T_max
    cfg = Config("R", "random", N, T, H, N * L, K, "fp8" if fp8 else "bf16", "uniform", 50 + seed)
    say(f"[gpu] parity random {cfg.describe()} T_max={T_max} transport={transport}")
    inp = make_inputs(cfg)
    _compare_all(cfg, inp, run_cycle(torch, mep, cfg, inp, T_max=T_max, transport=transport))


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_parity_edge_shapes(transport):
    """T=1, T=0 (empty cycle), one rank, one expert per rank, K=1."""
    cases = [
        CONFIGS["A"].with_(T=1),
        CONFIGS["A"].with_(N=1, E=4),
        CONFIGS["A"].with_(N=4, E=4, K=1, routing="uniform"),
        CONFIGS["B"].with_(T=3, H=64),
    ]
    for cfg in cases:
        say(f"[gpu] parity edge {cfg.describe()} transport={transport}")
        inp = make_inputs(cfg)
        _compare_all(cfg, inp, run_cycle(torch, mep, cfg, inp, T_max=cfg.T + 2,
                                         transport=transport))
    cfg = CONFIGS["A"]
    say(f"[gpu] parity empty cycle {cfg.describe()} T=0 transport={transport}")
    inp = make_inputs(cfg, T=0)
    gpu = run_cycle(torch, mep, cfg, inp, T_max=16, transport=transport)
    assert gpu["cnt"].sum() == 0 and gpu["G"].tolist() == [0] * (cfg.N + 1)
    assert gpu["expert_offsets"].tolist() == [0] * (cfg.E + 1)
    # an empty cycle after a full one on the same group: the offsets are
    # formed again (all zero), not left from the full cycle
    for layout in (mep.MOE_LAYOUT_PACKED, mep.MOE_LAYOUT_FIXED_SLOT):
        g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16, transport, 0,
                                 layout)
        try:
            full = make_inputs(cfg)
            if layout == mep.MOE_LAYOUT_PACKED:
                _compare_all(cfg, full, run_cycle(torch, mep, cfg, full, group=g,
                                                  transport=transport))
            else:
                run_cycle(torch, mep, cfg, full, group=g, transport=transport, layout=layout,
                          want_rows=False)
            gpu = run_cycle(torch, mep, cfg, inp, group=g, transport=transport, layout=layout)
            assert gpu["cnt"].sum() == 0 and gpu["G"].tolist() == [0] * (cfg.N + 1)
            assert gpu["expert_offsets"].tolist() == [0] * (cfg.E + 1)
            assert gpu["eoff"].tolist() == [0] * (cfg.E + 1)
        finally:
            mep.moe_group_destroy(g)


@pytest.mark.parametrize("key", ["A", "B", "C", "E", "Ep"])
def test_identity_experts_return_input(key):
    cfg = CONFIGS[key]
    say(f"[gpu] identity {cfg.describe()}")
    inp = make_inputs(cfg)
    inp["w"] = renormalised(inp["w"])
    gpu = run_cycle(torch, mep, cfg, inp, identity=True, want_rows=False)
    assert np.array_equal(gpu["out"], _plus_zero(inp["x"]))


@pytest.mark.parametrize("transport", TRANSPORTS)
@pytest.mark.parametrize("key", ["C", "E", "Ep"])
def test_parity_full_decode_workloads(key, transport):
    """The DeepSeek-R1 and Kimi-K2 decode shapes at full size, every buffer."""
    cfg = CONFIGS[key]
    say(f"[gpu] parity full {cfg.describe()} transport={transport}")
    inp = make_inputs(cfg)
    gpu = run_cycle(torch, mep, cfg, inp, transport=transport)
    _compare_all(cfg, inp, gpu)
    recv = np.diff(gpu["G"])
    assert recv.max() <= cfg.N * cfg.T * min(cfg.K, cfg.L)
    if key == "Ep":
        assert recv[0] == cfg.N * cfg.T * cfg.L


def test_repeat_cycles_are_deterministic():
    cfg = CONFIGS["B"]
    say(f"[gpu] determinism {cfg.describe()}")
    inp = make_inputs(cfg)
    g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16)
    try:
        a = run_cycle(torch, mep, cfg, inp, group=g)
        b = run_cycle(torch, mep, cfg, inp, group=g)
        for k in INT_KEYS + ["send_x", "recv_x", "expert_x", "comb_send", "comb_recv", "out"]:
            assert np.array_equal(a[k], b[k]), k
        # a smaller cycle on the same group after a larger one
        inp2 = make_inputs(cfg, T=37)
        c = run_cycle(torch, mep, cfg, inp2, group=g)
        _compare_all(cfg, inp2, c)
    finally:
        mep.moe_group_destroy(g)
