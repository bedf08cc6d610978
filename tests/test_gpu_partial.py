"""GPU parity of the combine with expert-side partial sums (one pre-summed bf16
row per (token, destination rank), summed again by the token's owner) against
the oracle's partial combine on the same seeded inputs.  Everything is
bit-exact: the partial-row plan, the owner-layout rows (staged transport), the
token-layout rows and the output (the same fp32 chains on both sides)."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import run_cycle, say
from workloads import CONFIGS, Config, make_inputs, renormalised

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402  (fails loudly if the library is missing)

PARTIAL = mep.MOE_COMBINE_PARTIAL
TRANSPORTS = [mep.MOE_TRANSPORT_STAGED, mep.MOE_TRANSPORT_DIRECT]


def _first_of_rank(d: np.ndarray) -> np.ndarray:
    """[N][T][K] bool: item k is the first of its token with its rank."""
    K = d.shape[-1]
    same = d[..., :, None] == d[..., None, :]                     # [.., k, j]
    earlier = np.tril(np.ones((K, K), dtype=bool), -1)            # j < k
    return ~np.any(same & earlier, axis=-1)


def _check(cfg, inp, gpu):
    fp8 = cfg.dtype == "fp8"
    idx = inp["idx"]
    N, T, K = idx.shape
    L = cfg.L
    d = oracle.run_dispatch(inp["x"], idx, cfg.E, fp8=fp8)
    for k in ("cnt", "pos", "soff", "roff", "G", "eoff"):
        assert np.array_equal(gpu[k], d[k]), k
    y = oracle.expert_standin(d["expert_x"], d["expert_scale"] if fp8 else None, d["eoff"], cfg.H)
    assert np.array_equal(gpu["y"], y)
    ref = oracle.run_partial_combine(y, inp["w"], idx, d, cfg.H)
    P = ref["P"]
    assert gpu["P"] == P
    # the plan: rank of every item, the partial row of every head item
    ranks = idx // L
    assert np.array_equal(gpu["part_dst"], ranks)
    head = _first_of_rank(ranks)
    s_i, t_i, _ = np.indices(idx.shape)
    expect_pos = np.full(idx.shape, -1, dtype=np.int64)
    expect_pos[head] = ref["token_row"][s_i[head], t_i[head], ranks[head]] - gpu["part_base"][s_i[head]]
    assert np.array_equal(gpu["part_pos"], expect_pos)
    pc = ref["pc"].astype(np.int64)
    psoff = np.zeros((N, N + 1), dtype=np.int64)
    psoff[:, 1:] = np.cumsum(pc, axis=1)
    assert np.array_equal(gpu["part_send_off"], psoff)
    assert gpu["part_base"].tolist() == [0] + np.cumsum(pc.sum(axis=1)).tolist()
    assert gpu["part_owner_base"].tolist() == [0] + np.cumsum(pc.sum(axis=0)).tolist()
    # the rows and the output
    if "psend" in gpu:
        assert np.array_equal(gpu["psend"], ref["psend"])
    assert np.array_equal(gpu["precv"], ref["precv"])
    bad = np.argwhere(gpu["out"] != ref["out"])
    assert bad.size == 0, bad[:5]
    return ref


@pytest.mark.parametrize("transport", TRANSPORTS)
@pytest.mark.parametrize("key", ["A", "B"])
def test_partial_small_workloads(key, transport):
    cfg = CONFIGS[key]
    say(f"[gpu] partial {cfg.describe()} transport={transport}")
    inp = make_inputs(cfg)
    _check(cfg, inp, run_cycle(torch, mep, cfg, inp, transport=transport, combine_mode=PARTIAL))


@pytest.mark.parametrize("transport", TRANSPORTS)
@pytest.mark.parametrize("seed", range(6))
def test_partial_random_groups(seed, transport):
    """Random groups: K from 1 to 12 (also K above N, and the K the kernels
    are not specialised for), ragged T, short and odd rows, e4m3 dispatch."""
    g = np.random.default_rng(2000 + seed)
    N = int(g.choice([1, 2, 3, 5, 8, 16]))
    L = int(g.integers(1, 6))
    K = int(g.integers(1, 13))
    fp8 = seed % 3 == 2
    H = int(g.choice([128, 384, 1024])) if fp8 else int(g.choice([8, 64, 200, 520, 1032, 4104]))
    T_max = int(g.integers(1, 40))
    T = int(g.integers(0, T_max + 1)) if seed != 0 else T_max
    cfg = Config("R", "random", N, T, H, N * L, K, "fp8" if fp8 else "bf16", "uniform", 70 + seed)
    say(f"[gpu] partial random {cfg.describe()} T_max={T_max} transport={transport}")
    inp = make_inputs(cfg)
    _check(cfg, inp, run_cycle(torch, mep, cfg, inp, T_max=T_max, transport=transport,
                               combine_mode=PARTIAL))


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_partial_edge_shapes(transport):
    """T=1, one rank (every token one partial), K=1 (partial = weighted row),
    K well above N (most items share a rank), a 3-chunk route plan, a route
    plan past its register-held chunks, and an empty cycle."""
    cases = [
        CONFIGS["A"].with_(T=1),
        CONFIGS["A"].with_(N=1, E=4),
        CONFIGS["A"].with_(N=4, E=4, K=1, routing="uniform"),
        CONFIGS["A"].with_(N=2, E=8, K=8, routing="uniform"),
        CONFIGS["A"].with_(N=3, E=6, K=5, T=300, H=64, routing="uniform"),
        # more items per rank than the route plan keeps in registers
        CONFIGS["A"].with_(N=2, E=8, K=8, T=2100, H=64, routing="uniform"),
    ]
    for cfg in cases:
        say(f"[gpu] partial edge {cfg.describe()} transport={transport}")
        inp = make_inputs(cfg)
        _check(cfg, inp, run_cycle(torch, mep, cfg, inp, T_max=cfg.T + 2, transport=transport,
                                   combine_mode=PARTIAL))
    cfg = CONFIGS["A"]
    say(f"[gpu] partial empty cycle {cfg.describe()} T=0 transport={transport}")
    inp = make_inputs(cfg, T=0)
    gpu = run_cycle(torch, mep, cfg, inp, T_max=16, transport=transport, combine_mode=PARTIAL)
    assert gpu["P"] == 0 and gpu["part_base"].tolist() == [0] * (cfg.N + 1)


# Each block of the send-row-order pack's partial records forms its sender's
# bases from (E + 2N + 2) * N terms of the senders' send offsets up to 65 536
# terms, else reads the route plan's group tables: 126 ranks x 252 experts
# (63 756 terms) and 128 x 256 (65 792), packed and fixed-slot layouts.
RECORD_SIDES = {"sums": (126, 252), "tables": (128, 256)}


@pytest.mark.parametrize("layout", ["packed", "fixed"])
@pytest.mark.parametrize("transport", TRANSPORTS)
@pytest.mark.parametrize("side", list(RECORD_SIDES))
def test_partial_record_bases(side, transport, layout):
    from tests.test_gpu_fixed_slot import _check as check_fixed
    N, E = RECORD_SIDES[side]
    cfg = Config("Q", f"records-{side}", N, 5, 136, E, 6, "bf16", "softmax", 23)
    say(f"[gpu] partial record bases {cfg.describe()} transport={transport} layout={layout}")
    inp = make_inputs(cfg)
    if layout == "fixed":
        check_fixed(cfg, inp, cfg.T, transport, PARTIAL)
    else:
        _check(cfg, inp, run_cycle(torch, mep, cfg, inp, transport=transport, combine_mode=PARTIAL))


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_partial_same_rank_identity(transport):
    """Identity experts, weights summing to one, every expert of a token on
    one rank: the single partial is x itself, so out == x (-0 -> +0)."""
    cfg = Config("P", "same-rank", 4, 16, 256, 16, 3, "bf16", "uniform", 9)
    inp = make_inputs(cfg)
    g = np.random.default_rng(9)
    ranks = g.integers(0, cfg.N, size=(cfg.N, cfg.T))
    inp["idx"] = (ranks[..., None] * cfg.L +
                  g.integers(0, cfg.L, size=(cfg.N, cfg.T, cfg.K))).astype(np.int32)
    inp["w"] = renormalised(inp["w"])
    say(f"[gpu] partial same-rank identity {cfg.describe()} transport={transport}")
    gpu = run_cycle(torch, mep, cfg, inp, identity=True, transport=transport, combine_mode=PARTIAL)
    assert np.array_equal(gpu["out"], np.where(inp["x"] == 0x8000, np.uint16(0), inp["x"]))


@pytest.mark.parametrize("transport", TRANSPORTS)
@pytest.mark.parametrize("key", ["C", "E", "Ep"])
def test_partial_full_decode_workloads(key, transport):
    """The DeepSeek-R1 and Kimi-K2 decode shapes at full size."""
    cfg = CONFIGS[key]
    say(f"[gpu] partial full {cfg.describe()} transport={transport}")
    inp = make_inputs(cfg)
    ref = _check(cfg, inp, run_cycle(torch, mep, cfg, inp, transport=transport,
                                     combine_mode=PARTIAL))
    assert ref["P"] < cfg.rows
    if key == "Ep":
        assert ref["P"] < 0.5 * cfg.rows


def test_partial_group_reuse_and_arguments():
    """A larger then a smaller cycle on one group; weights are required by
    dispatch_send and not by combine_recv."""
    cfg = CONFIGS["B"]
    say(f"[gpu] partial reuse {cfg.describe()}")
    g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16,
                             mep.MOE_TRANSPORT_STAGED, PARTIAL)
    try:
        inp = make_inputs(cfg)
        x = torch.zeros((cfg.N, cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
        idx = torch.zeros((cfg.N, cfg.T, cfg.K), dtype=torch.int32, device="cuda")
        with pytest.raises(mep.MoeError) as ei:
            mep.moe_dispatch_send(g, cfg.T, x, idx, None)
        assert ei.value.status == mep.MOE_ERR_INVALID
        a = run_cycle(torch, mep, cfg, inp, group=g, combine_mode=PARTIAL)
        _check(cfg, inp, a)
        inp2 = make_inputs(cfg, T=37)
        b = run_cycle(torch, mep, cfg, inp2, group=g, combine_mode=PARTIAL)
        _check(cfg, inp2, b)
    finally:
        mep.moe_group_destroy(g)
