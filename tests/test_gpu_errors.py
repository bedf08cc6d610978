"""Error behaviour through the C ABI on the GPU: a routing error found on the
device writes none of the cycle's outputs and is reported by the status call;
out-of-order calls and bad arguments are rejected on the host and enqueue
nothing."""
import numpy as np
import pytest

from tests.gpu_util import run_cycle, say, to_dev
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402


@pytest.mark.parametrize("combine_mode", [0, 1])
def test_routing_error_writes_nothing_and_is_reported(combine_mode):
    cfg = CONFIGS["A"]
    say(f"[gpu] routing error {cfg.describe()} combine_mode={combine_mode}")
    partial = combine_mode == mep.MOE_COMBINE_PARTIAL
    inp = make_inputs(cfg)
    bad = inp["idx"].copy()
    bad[1, 3, 1] = cfg.E          # one id out of range
    bad[0, 0, 0] = -1
    g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16,
                             mep.MOE_TRANSPORT_STAGED, combine_mode)
    try:
        R = cfg.rows
        x, idx, w = to_dev(torch, inp["x"]), to_dev(torch, bad), to_dev(torch, inp["w"])
        expert_x = torch.full((R * cfg.H,), -1, dtype=torch.int16, device="cuda")
        offs = torch.full((cfg.E + 1,), -7, dtype=torch.int32, device="cuda")
        y = torch.zeros((R, cfg.H), dtype=torch.bfloat16, device="cuda")
        out = torch.full((cfg.N, cfg.T, cfg.H), -1, dtype=torch.int16, device="cuda")
        mep.moe_dispatch_send(g, cfg.T, x, idx, w if partial else None)
        mep.moe_dispatch_recv(g, expert_x, None, offs)
        mep.moe_combine_send(g, y)
        mep.moe_combine_recv(g, None if partial else w, out)
        assert mep.moe_group_status(g) == mep.MOE_ERR_ROUTING
        assert mep.moe_group_status(g) == mep.MOE_OK          # reading clears it
        assert torch.all(expert_x == -1).item()
        assert torch.all(offs == -7).item()
        assert torch.all(out == -1).item()
        # the group is usable again with valid routing
        gpu = run_cycle(torch, mep, cfg, inp, group=g, combine_mode=combine_mode)
        if partial:
            from tests.test_gpu_partial import _check
            _check(cfg, inp, gpu)
        else:
            from tests.test_gpu_parity import _compare_all
            _compare_all(cfg, inp, gpu)
    finally:
        mep.moe_group_destroy(g)


@pytest.mark.parametrize("combine_mode", [0, 1])
def test_routing_error_stops_only_its_own_cycle(combine_mode):
    """A cycle with an invalid expert id, then a valid cycle on the same group
    with no status read in between: the valid cycle runs in full (its outputs
    equal the oracle's), and the status call afterwards still reports the
    earlier cycle's routing error, once."""
    cfg = CONFIGS["A"]
    say(f"[gpu] routing error then a valid cycle {cfg.describe()} combine_mode={combine_mode}")
    partial = combine_mode == mep.MOE_COMBINE_PARTIAL
    inp = make_inputs(cfg)
    bad = inp["idx"].copy()
    bad[0, 5, 1] = cfg.E + 3
    g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16,
                             mep.MOE_TRANSPORT_STAGED, combine_mode)
    try:
        R = cfg.rows
        x, idx, w = to_dev(torch, inp["x"]), to_dev(torch, bad), to_dev(torch, inp["w"])
        expert_x = torch.empty((R * cfg.H,), dtype=torch.int16, device="cuda")
        offs = torch.empty((cfg.E + 1,), dtype=torch.int32, device="cuda")
        y = torch.zeros((R, cfg.H), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((cfg.N, cfg.T, cfg.H), dtype=torch.int16, device="cuda")
        mep.moe_dispatch_send(g, cfg.T, x, idx, w if partial else None)
        mep.moe_dispatch_recv(g, expert_x, None, offs)
        mep.moe_combine_send(g, y)
        mep.moe_combine_recv(g, None if partial else w, out)
        gpu = run_cycle(torch, mep, cfg, inp, group=g, combine_mode=combine_mode,
                        check_status=False)
        if partial:
            from tests.test_gpu_partial import _check
            _check(cfg, inp, gpu)
        else:
            from tests.test_gpu_parity import _compare_all
            _compare_all(cfg, inp, gpu)
        assert mep.moe_group_status(g) == mep.MOE_ERR_ROUTING
        assert mep.moe_group_status(g) == mep.MOE_OK
    finally:
        mep.moe_group_destroy(g)


@pytest.mark.parametrize("transport", [0, 1])
def test_routing_errors_in_alternate_cycles(transport):
    """The group alternates two cycle error words (each route plan clears the
    next cycle's): failing and valid cycles in the pattern bad, good, bad,
    bad, good, good on one group with no status read in between -- every
    valid cycle equals the oracle whichever word it got, every failing cycle
    leaves the caller's output untouched, and the status afterwards reports
    the routing error once."""
    cfg = CONFIGS["A"]
    say(f"[gpu] alternating routing errors {cfg.describe()} transport={transport}")
    inp = make_inputs(cfg)
    bad = inp["idx"].copy()
    bad[1, 3, 0] = -1
    g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16, transport, 0)
    from tests.test_gpu_parity import _compare_all
    try:
        R = cfg.rows
        x, idx, w = to_dev(torch, inp["x"]), to_dev(torch, bad), to_dev(torch, inp["w"])
        expert_x = torch.empty((R * cfg.H,), dtype=torch.int16, device="cuda")
        offs = torch.empty((cfg.E + 1,), dtype=torch.int32, device="cuda")
        y = torch.zeros((R, cfg.H), dtype=torch.bfloat16, device="cuda")
        for n, good in enumerate([False, True, False, False, True, True]):
            if good:
                gpu = run_cycle(torch, mep, cfg, inp, group=g, transport=transport,
                                check_status=False)
                _compare_all(cfg, inp, gpu)
                continue
            out = torch.full((cfg.N, cfg.T, cfg.H), 0x1234, dtype=torch.int16, device="cuda")
            mep.moe_dispatch_send(g, cfg.T, x, idx)
            mep.moe_dispatch_recv(g, expert_x, None, offs)
            mep.moe_combine_send(g, y)
            mep.moe_combine_recv(g, w, out)
            torch.cuda.synchronize()
            assert torch.all(out == 0x1234).item(), f"cycle {n} wrote its output"
        assert mep.moe_group_status(g) == mep.MOE_ERR_ROUTING
        assert mep.moe_group_status(g) == mep.MOE_OK
    finally:
        mep.moe_group_destroy(g)


def test_call_order_and_arguments():
    cfg = CONFIGS["A"]
    say(f"[gpu] call order {cfg.describe()}")
    inp = make_inputs(cfg)
    g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16)
    try:
        R = cfg.rows
        x, idx, w = to_dev(torch, inp["x"]), to_dev(torch, inp["idx"]), to_dev(torch, inp["w"])
        expert_x = torch.empty((R, cfg.H), dtype=torch.bfloat16, device="cuda")
        offs = torch.empty((cfg.E + 1,), dtype=torch.int32, device="cuda")
        out = torch.empty((cfg.N, cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")

        def status_of(fn, *a):
            try:
                fn(*a)
                return mep.MOE_OK
            except mep.MoeError as e:
                return e.status

        assert status_of(mep.moe_dispatch_recv, g, expert_x, None, offs) == mep.MOE_ERR_STATE
        assert status_of(mep.moe_combine_send, g, expert_x) == mep.MOE_ERR_STATE
        assert status_of(mep.moe_combine_recv, g, w, out) == mep.MOE_ERR_STATE
        assert status_of(mep.moe_dispatch_send, g, cfg.T + 1, x, idx) == mep.MOE_ERR_INVALID
        assert status_of(mep.moe_dispatch_send, g, -1, x, idx) == mep.MOE_ERR_INVALID
        assert status_of(mep.moe_dispatch_send, g, cfg.T, x.data_ptr() + 2, idx) == mep.MOE_ERR_INVALID
        assert status_of(mep.moe_dispatch_send, g, cfg.T, None, idx) == mep.MOE_ERR_INVALID
        mep.moe_dispatch_send(g, cfg.T, x, idx)
        assert status_of(mep.moe_dispatch_send, g, cfg.T, x, idx) == mep.MOE_ERR_STATE
        # bf16 groups take no scale pointer
        assert status_of(mep.moe_dispatch_recv, g, expert_x, offs, offs) == mep.MOE_ERR_INVALID
        mep.moe_dispatch_recv(g, expert_x, None, offs)
        assert status_of(mep.moe_dispatch_recv, g, expert_x, None, offs) == mep.MOE_ERR_STATE
        mep.moe_combine_send(g, expert_x)
        mep.moe_combine_recv(g, w, out)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
    finally:
        mep.moe_group_destroy(g)


def test_create_rejects_bad_descriptors():
    say("[gpu] create descriptors")
    for args in [(2, 7, 2, 256, 16, 0), (0, 8, 2, 256, 16, 0), (2, 8, 0, 256, 16, 0),
                 (2, 8, 2, 100, 16, 0), (2, 8, 2, 256, 16, 1 + 5), (2, 8, 2, 264, 16, 1),
                 (2, 2048, 2, 256, 16, 0), (2, 8, 2, 256, -1, 0)]:
        with pytest.raises(mep.MoeError) as ei:
            mep.moe_group_create(*args)
        assert ei.value.status == mep.MOE_ERR_INVALID, args


def test_group_larger_than_the_device_reports_oom():
    """The DeepSeek-R1 prefill shape with the fixed-slot layout needs
    64 x 256 x 2048 slots of 14 KiB (~480 GB, more than the device holds):
    create reports MOE_ERR_OOM, frees what it had allocated, and a group that
    fits is created and runs afterwards."""
    say("[gpu] oversized fixed-slot group")
    free, total = torch.cuda.mem_get_info()
    slots_bytes = 64 * 256 * 2048 * 7168 * 2
    assert slots_bytes > total
    with pytest.raises(mep.MoeError) as ei:
        mep.moe_group_create(64, 256, 8, 7168, 2048, mep.MOE_FP8_E4M3, mep.MOE_TRANSPORT_STAGED,
                             mep.MOE_COMBINE_RECEIVER, mep.MOE_LAYOUT_FIXED_SLOT)
    assert ei.value.status == mep.MOE_ERR_OOM
    free_after, _ = torch.cuda.mem_get_info()
    assert free_after >= free - (64 << 20)
    cfg = CONFIGS["A"]
    inp = make_inputs(cfg)
    g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16)
    try:
        run_cycle(torch, mep, cfg, inp, group=g, want_rows=False)
        assert mep.moe_group_status(g) == mep.MOE_OK
    finally:
        mep.moe_group_destroy(g)


def test_kernel_timing_mask():
    """Timing events attach only to the selected kernels; a cycle with every
    kernel selected reports one launch of each (T > 0)."""
    cfg = CONFIGS["A"]
    say(f"[gpu] timing mask {cfg.describe()}")
    inp = make_inputs(cfg)
    g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16)
    try:
        mep.moe_group_timing_enable(g, True)
        run_cycle(torch, mep, cfg, inp, group=g, want_rows=False)
        t = mep.moe_group_timing_read(g)
        # the staged receiver-side combine runs every kernel but the direct
        # combine push and the partial-combine kernels
        unused = {"combine_push", "partial_send", "partial_transfer", "partial_reduce"}
        assert all(n == 1 and ms > 0 for k, (ms, n) in t.items() if k not in unused), t
        assert all(t[k][1] == 0 for k in unused), t
        mep.moe_group_timing_enable(g, ["transfer", "combine_reduce"])
        run_cycle(torch, mep, cfg, inp, group=g, want_rows=False)
        t = mep.moe_group_timing_read(g)
        assert {k for k, (ms, n) in t.items() if n} == {"transfer", "combine_reduce"}, t
        mep.moe_group_timing_enable(g, False)
        with pytest.raises(mep.MoeError):
            mep.moe_group_timing_enable(g, 1 << 12)
    finally:
        mep.moe_group_destroy(g)
    # the partial combine: its three kernels replace the combine pack,
    # transfer back and reduce
    g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16,
                             mep.MOE_TRANSPORT_STAGED, mep.MOE_COMBINE_PARTIAL)
    try:
        mep.moe_group_timing_enable(g, True)
        run_cycle(torch, mep, cfg, inp, group=g, want_rows=False,
                  combine_mode=mep.MOE_COMBINE_PARTIAL)
        t = mep.moe_group_timing_read(g)
        ran = {k for k, (ms, n) in t.items() if n}
        assert ran == {"route_plan", "pack", "transfer", "shuffle", "partial_send",
                       "partial_transfer", "partial_reduce", "recv_map"}, t
    finally:
        mep.moe_group_destroy(g)


def test_binding_rejects_bad_tensors():
    """The Python binding checks torch tensors before passing their address:
    on the device, dense, the fixed dtypes (int32 ids and offsets, fp32
    weights and scales), and large enough for the call; a failed check raises
    MOE_ERR_INVALID and enqueues nothing, and the cycle then runs normally."""
    cfg = CONFIGS["A"]
    say(f"[gpu] binding tensor checks {cfg.describe()}")
    inp = make_inputs(cfg)
    g = mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16)
    try:
        R = cfg.rows
        x, idx, w = to_dev(torch, inp["x"]), to_dev(torch, inp["idx"]), to_dev(torch, inp["w"])

        def status_of(fn, *a):
            try:
                fn(*a)
                return mep.MOE_OK
            except mep.MoeError as e:
                return e.status

        assert status_of(mep.moe_dispatch_send, g, cfg.T, x.cpu(), idx) == mep.MOE_ERR_INVALID
        assert status_of(mep.moe_dispatch_send, g, cfg.T, x, idx.long()) == mep.MOE_ERR_INVALID
        assert status_of(mep.moe_dispatch_send, g, cfg.T, x[:, :cfg.T - 1], idx) == mep.MOE_ERR_INVALID
        xt = torch.empty((cfg.N, cfg.H, cfg.T), dtype=torch.int16, device="cuda").transpose(1, 2)
        assert status_of(mep.moe_dispatch_send, g, cfg.T, xt, idx) == mep.MOE_ERR_INVALID
        mep.moe_dispatch_send(g, cfg.T, x, idx)
        offs = torch.empty((cfg.E + 1,), dtype=torch.int32, device="cuda")
        small = torch.empty((R - 1, cfg.H), dtype=torch.bfloat16, device="cuda")
        assert status_of(mep.moe_dispatch_recv, g, small, None, offs) == mep.MOE_ERR_INVALID
        assert status_of(mep.moe_dispatch_recv, g, torch.empty((R, cfg.H), dtype=torch.bfloat16,
                                                                device="cuda"),
                         None, offs[:cfg.E]) == mep.MOE_ERR_INVALID
        expert_x = torch.empty((R, cfg.H), dtype=torch.bfloat16, device="cuda")
        mep.moe_dispatch_recv(g, expert_x, None, offs)
        assert status_of(mep.moe_combine_send, g, expert_x[:R - 1]) == mep.MOE_ERR_INVALID
        mep.moe_combine_send(g, expert_x)
        out = torch.empty((cfg.N, cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
        assert status_of(mep.moe_combine_recv, g, w.double(), out) == mep.MOE_ERR_INVALID
        assert status_of(mep.moe_combine_recv, g, w, out[:, 1:]) == mep.MOE_ERR_INVALID
        mep.moe_combine_recv(g, w, out)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
    finally:
        mep.moe_group_destroy(g)
