"""Debug mode (MOE_EP_DEBUG=1 when the group is created): before each call's
kernels the library fills, with 0xFF bytes, every buffer that call must
rewrite -- the row pools and planes, the plan tables and row maps before
dispatch_send, the expert-order metadata and the caller's expert rows and
offsets before dispatch_recv, both row pools before combine_send, the
caller's output before combine_recv -- so a read of anything a call did not
write surfaces as bf16 NaN or an index of -1 (out of range, reported as an
internal error).  Full cycles in every transport x combine x layout mode,
repeated on one group with a smaller batch, must still equal the oracle."""
import numpy as np
import pytest

from tests.gpu_util import run_cycle, say
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402
from tests import test_gpu_fixed_slot as fixed_slot  # noqa: E402
from tests.test_gpu_parity import _compare_all  # noqa: E402
from tests.test_gpu_partial import _check as _check_partial  # noqa: E402


@pytest.fixture
def debug_env(monkeypatch):
    monkeypatch.setenv("MOE_EP_DEBUG", "1")


def _group(cfg, T_max, transport, combine_mode, layout=mep.MOE_LAYOUT_PACKED):
    return mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, T_max,
                                mep.MOE_FP8_E4M3 if cfg.dtype == "fp8" else mep.MOE_BF16,
                                transport, combine_mode, layout)


@pytest.mark.parametrize("combine_mode", [0, 1])
@pytest.mark.parametrize("transport", [0, 1])
@pytest.mark.parametrize("key", ["A", "Afp8", "B"])
def test_debug_mode_cycles_match_oracle(debug_env, key, transport, combine_mode):
    cfg = CONFIGS["A"].with_(dtype="fp8", H=512) if key == "Afp8" else CONFIGS[key]
    say(f"[gpu] debug mode {cfg.describe()} transport={transport} combine_mode={combine_mode}")
    g = _group(cfg, cfg.T, transport, combine_mode)
    try:
        for T in (cfg.T, max(1, cfg.T // 3)):
            inp = make_inputs(cfg, T=T)
            gpu = run_cycle(torch, mep, cfg, inp, group=g, T_max=cfg.T, transport=transport,
                            combine_mode=combine_mode)
            if combine_mode == mep.MOE_COMBINE_PARTIAL:
                _check_partial(cfg.with_(T=T), inp, gpu)
            else:
                _compare_all(cfg.with_(T=T), inp, gpu)
    finally:
        mep.moe_group_destroy(g)


@pytest.mark.parametrize("combine_mode", [0, 1])
@pytest.mark.parametrize("transport", [0, 1])
def test_debug_mode_fixed_slot(debug_env, transport, combine_mode):
    cfg = CONFIGS["B"]
    say(f"[gpu] debug mode fixed slots {cfg.describe()} transport={transport} "
        f"combine_mode={combine_mode}")
    fixed_slot._check(cfg, make_inputs(cfg), cfg.T, transport, combine_mode)


@pytest.mark.parametrize("transport", [0, 1])
def test_debug_mode_full_decode(debug_env, transport):
    cfg = CONFIGS["C"]
    say(f"[gpu] debug mode {cfg.describe()} transport={transport}")
    inp = make_inputs(cfg)
    _compare_all(cfg, inp, run_cycle(torch, mep, cfg, inp, transport=transport))


def test_debug_poison_is_visible(debug_env):
    """The poison is really written: in debug mode an expert-output row that
    the shuffle has not written yet (rows past this cycle's count) reads 0xFF."""
    cfg = CONFIGS["A"]
    say(f"[gpu] debug poison visible {cfg.describe()}")
    g = _group(cfg, cfg.T, 0, 0)
    try:
        inp = make_inputs(cfg, T=4)
        x = torch.from_numpy(inp["x"].view(np.int16)).cuda()
        idx = torch.from_numpy(inp["idx"]).cuda()
        R = cfg.N * 4 * cfg.K
        expert_x = torch.zeros((cfg.rows, cfg.H), dtype=torch.int16, device="cuda")
        offs = torch.zeros((cfg.E + 1,), dtype=torch.int32, device="cuda")
        mep.moe_dispatch_send(g, 4, x, idx)
        mep.moe_dispatch_recv(g, expert_x, None, offs)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
        v = mep.moe_group_view_get(g)
        from tests.gpu_util import d2h
        # the receive pool past this cycle's rows still holds the poison
        tail = d2h(v.recv_x + R * cfg.H * 2, (cfg.rows - R, cfg.H), np.uint16)
        assert np.all(tail == 0xFFFF)
        # the caller's rows past this cycle's count were not poisoned (only
        # the rows the call writes are)
        assert torch.all(expert_x[R:] == 0).item()
        y = torch.zeros((R, cfg.H), dtype=torch.bfloat16, device="cuda")
        out = torch.zeros((cfg.N, 4, cfg.H), dtype=torch.bfloat16, device="cuda")
        mep.moe_combine_send(g, y)
        mep.moe_combine_recv(g, torch.from_numpy(inp["w"]).cuda(), out)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
        assert torch.all(out == 0).item()
    finally:
        mep.moe_group_destroy(g)
