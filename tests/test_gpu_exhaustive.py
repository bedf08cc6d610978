"""Exhaustive tiny routings on the GPU: N=2 ranks, T=2 tokens, E=4 experts,
every routing with K=1 (4^4 = 256) and every routing with K=2, repeated ids
included (16^4 = 65 536, of which 20 736 name two distinct experts per
token), each run as one cycle of the same group, in every transport, combine
mode and receive layout.  Every case's counts, positions, receive bases,
expert rows and combined tokens are compared with the oracle's.  The cycles
are enqueued back to back (no host synchronisation per case: each cycle's
results are copied device-to-device into its own slot) and checked at the
end."""
import ctypes
import itertools

import numpy as np
import pytest

import oracle
from tests.gpu_util import hip, say
from workloads import Config, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402

N, T, E, H = 2, 2, 4, 8

MODES = [
    # transport, combine mode, layout
    (mep.MOE_TRANSPORT_STAGED, mep.MOE_COMBINE_RECEIVER, mep.MOE_LAYOUT_PACKED),
    (mep.MOE_TRANSPORT_DIRECT, mep.MOE_COMBINE_RECEIVER, mep.MOE_LAYOUT_PACKED),
    (mep.MOE_TRANSPORT_STAGED, mep.MOE_COMBINE_PARTIAL, mep.MOE_LAYOUT_PACKED),
    (mep.MOE_TRANSPORT_DIRECT, mep.MOE_COMBINE_PARTIAL, mep.MOE_LAYOUT_FIXED_SLOT),
    (mep.MOE_TRANSPORT_STAGED, mep.MOE_COMBINE_RECEIVER, mep.MOE_LAYOUT_FIXED_SLOT),
    (mep.MOE_TRANSPORT_DIRECT, mep.MOE_COMBINE_PARTIAL, mep.MOE_LAYOUT_PACKED),
    (mep.MOE_TRANSPORT_DIRECT, mep.MOE_COMBINE_RECEIVER, mep.MOE_LAYOUT_FIXED_SLOT),
    (mep.MOE_TRANSPORT_STAGED, mep.MOE_COMBINE_PARTIAL, mep.MOE_LAYOUT_FIXED_SLOT),
]
MODE_IDS = ["staged", "direct", "staged-partial", "direct-partial-fixed", "staged-fixed",
            "direct-partial", "direct-fixed", "staged-partial-fixed"]


def _cases(K):
    """Every routing of the N*T tokens (K ids each, repeats allowed)."""
    choices = list(itertools.product(range(E), repeat=K))
    return np.array(list(itertools.product(choices, repeat=N * T)), dtype=np.int32)


_EXPECT = {}


def _expected(K, partial, inp, cases):
    """The oracle's results for every case (shared by the modes: the
    dispatch outputs do not depend on transport or layout, and the combined
    tokens depend only on the combine mode)."""
    key = (K, partial)
    if key not in _EXPECT:
        outs, plans = [], []
        for idx in cases:
            d = oracle.run_dispatch(inp["x"], idx, E)
            y = oracle.expert_standin(d["expert_x"], None, d["eoff"], H)
            if partial:
                out = oracle.run_partial_combine(y, inp["w"], idx, d, H)["out"]
            else:
                out = oracle.run_combine(y, inp["w"], d, H)["out"]
            outs.append(out)
            plans.append((d["cnt"], d["pos"], d["G"], d["expert_x"]))
        _EXPECT[key] = (outs, plans)
    return _EXPECT[key]


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("K", [1, 2])
def test_every_tiny_routing(K, mode):
    transport, combine_mode, layout = mode
    partial = combine_mode == mep.MOE_COMBINE_PARTIAL
    fixed = layout == mep.MOE_LAYOUT_FIXED_SLOT
    cases = _cases(K).reshape(-1, N, T, K)
    C = cases.shape[0]
    R = N * T * K
    # with repeated ids a sender can have T*K rows for one expert: the
    # fixed-slot group gets that many slots, so no case overflows
    T_max = T * K if fixed else T
    say(f"[gpu] exhaustive N={N} T={T} E={E} K={K} T_max={T_max} mode={mode}: {C} routings")
    cfg = Config("X", "exhaustive", N, T, H, E, K, "bf16", "uniform", 31)
    inp = make_inputs(cfg)
    lib = hip()
    lib.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.hipMemcpyAsync.restype = ctypes.c_int
    dev = "cuda"
    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev)
    w = torch.from_numpy(inp["w"]).to(dev)
    idx_all = torch.from_numpy(cases).to(dev)
    expert_x = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    out = torch.empty((N, T, H), dtype=torch.bfloat16, device=dev)
    rows = torch.arange(R, device=dev, dtype=torch.int32)
    res_out = torch.empty((C, N, T, H), dtype=torch.bfloat16, device=dev)
    res_ex = torch.empty((C, R, H), dtype=torch.bfloat16, device=dev)
    res_cnt = torch.empty((C, N, E), dtype=torch.int32, device=dev)
    res_pos = torch.empty((C, N, T, K), dtype=torch.int32, device=dev)
    res_g = torch.empty((C, N + 1), dtype=torch.int32, device=dev)
    g = mep.moe_group_create(N, E, K, H, T_max, mep.MOE_BF16, transport, combine_mode, layout)
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream
    try:
        v = mep.moe_group_view_get(g)

        def d2d(dst, src, nbytes):
            assert lib.hipMemcpyAsync(dst, src, nbytes, 3, st) == 0

        for c in range(C):
            mep.moe_dispatch_send(g, T, x, idx_all[c], w if partial else None)
            mep.moe_dispatch_recv(g, expert_x, None, offs)
            e_of_row = torch.bucketize(rows, offs[1:], right=True)
            y = (expert_x.float() * (e_of_row + 1).float()[:, None]).to(torch.bfloat16)
            mep.moe_combine_send(g, y)
            mep.moe_combine_recv(g, None if partial else w, out)
            res_out[c].copy_(out)
            res_ex[c].copy_(expert_x)
            d2d(res_cnt[c].data_ptr(), v.cnt, N * E * 4)
            d2d(res_pos[c].data_ptr(), v.pos, N * T * K * 4)
            d2d(res_g[c].data_ptr(), v.recv_base, (N + 1) * 4)
            if c % 8192 == 8191:
                torch.cuda.synchronize()
                say(f"[gpu]   {c + 1} cycles run")
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
    finally:
        torch.cuda.synchronize()
        mep.moe_group_destroy(g)
    got_out = res_out.view(torch.int16).cpu().numpy().view(np.uint16)
    got_ex = res_ex.view(torch.int16).cpu().numpy().view(np.uint16)
    got_cnt, got_pos, got_g = res_cnt.cpu().numpy(), res_pos.cpu().numpy(), res_g.cpu().numpy()
    say("[gpu]   checking against the oracle")
    outs, plans = _expected(K, partial, inp, cases)
    for c in range(C):
        cnt, pos, G, ex = plans[c]
        assert np.array_equal(got_cnt[c], cnt), c
        assert np.array_equal(got_pos[c], pos), c
        assert np.array_equal(got_g[c], G), c
        assert np.array_equal(got_ex[c], ex), c
        assert np.array_equal(got_out[c], outs[c]), c
