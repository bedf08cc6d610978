"""moe_group_create_static through the C ABI: a group whose buffers live in
the library's static device scratch area (for callers that cannot allocate)
gives, cycle for cycle, the same outputs as a group from moe_group_create,
which the oracle checks in turn.  Two static groups in a row, the second
smaller (fewer ranks, tokens and hidden), each run twice, the second cycle
with fewer tokens; the area's limits and its one-group-per-device rule."""
import numpy as np
import pytest

from tests.gpu_util import run_cycle, say
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402
from tests.test_gpu_parity import _compare_all  # noqa: E402

KEYS = ["cnt", "pos", "soff", "roff", "G", "eoff", "expert_offsets", "send_meta", "recv_meta",
        "expert_src_rank", "expert_src_slot", "send_x", "recv_x", "expert_x", "y", "comb_send",
        "comb_recv", "out"]


def _same(a: dict, b: dict):
    for k in KEYS:
        assert (k in a) == (k in b), k
        if k in a:
            assert np.array_equal(a[k], b[k]), k


def test_static_group_matches_allocated_group():
    # Mixtral-8x7B decode (about 35 MB of group buffers), then a tiny group
    for cfg, T2 in ((CONFIGS["B"], 37), (CONFIGS["A"], 5)):
        fp8 = cfg.dtype == "fp8"
        args = (cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_FP8_E4M3 if fp8 else mep.MOE_BF16)
        say(f"[gpu] static-scratch group {cfg.describe()}")
        gs = mep.moe_group_create_static(*args)
        try:
            ga = mep.moe_group_create(*args)
            try:
                for T in (cfg.T, T2):
                    inp = make_inputs(cfg, T=T)
                    say(f"[gpu] static-scratch cycle T={T}")
                    a = run_cycle(torch, mep, cfg, inp, group=gs, T_max=cfg.T)
                    b = run_cycle(torch, mep, cfg, inp, group=ga, T_max=cfg.T)
                    _same(a, b)
                    _compare_all(cfg.with_(T=T), inp, a)
            finally:
                mep.moe_group_destroy(ga)
        finally:
            mep.moe_group_destroy(gs)


def test_static_group_limits():
    say("[gpu] static-scratch limits")
    # the DeepSeek-R1 decode shape needs ~1 GB: larger than the area
    cfg = CONFIGS["C"]
    with pytest.raises(mep.MoeError) as ei:
        mep.moe_group_create_static(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T)
    assert ei.value.status == mep.MOE_ERR_SCRATCH
    a = CONFIGS["A"]
    gs = mep.moe_group_create_static(a.N, a.E, a.K, a.H, a.T)
    try:
        # one static group per device at a time
        with pytest.raises(mep.MoeError) as ei:
            mep.moe_group_create_static(a.N, a.E, a.K, a.H, a.T)
        assert ei.value.status == mep.MOE_ERR_STATE
    finally:
        mep.moe_group_destroy(gs)
    # released: a new one may be made, and it runs
    gs = mep.moe_group_create_static(a.N, a.E, a.K, a.H, a.T, mep.MOE_BF16,
                                     mep.MOE_TRANSPORT_DIRECT, mep.MOE_COMBINE_PARTIAL)
    try:
        inp = make_inputs(a)
        run_cycle(torch, mep, a, inp, group=gs, want_rows=False, transport=1, combine_mode=1)
    finally:
        mep.moe_group_destroy(gs)
