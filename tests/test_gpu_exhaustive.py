"""Exhaustive tiny routings on the GPU: N=2 ranks, T=2 tokens, E=4 experts,
every routing with K=1 (256), every routing with K=2 and distinct ids per
token (20 736) and a seeded sample of K=2 routings with repeated ids, each
run as one cycle of the same group.  Every case's counts, positions,
receive bases, expert rows and combined tokens are compared with the
oracle's.  The cycles are enqueued back to back (no host synchronisation per
case: each cycle's results are copied device-to-device into its own slot)
and checked at the end."""
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


def _cases(K):
    choices = list(itertools.product(range(E), repeat=K))
    if K == 1:
        return np.array(list(itertools.product(choices, repeat=N * T)), dtype=np.int32)
    distinct = [c for c in choices if len(set(c)) == K]
    all_distinct = np.array(list(itertools.product(distinct, repeat=N * T)), dtype=np.int32)
    g = np.random.default_rng(77)
    repeated = g.integers(0, E, size=(2048, N * T, K)).astype(np.int32)
    return np.concatenate([all_distinct, repeated])


@pytest.mark.parametrize("K", [1, 2])
def test_every_tiny_routing(K):
    cases = _cases(K).reshape(-1, N, T, K)
    C = cases.shape[0]
    R = N * T * K
    say(f"[gpu] exhaustive N={N} T={T} E={E} K={K}: {C} routings")
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
    g = mep.moe_group_create(N, E, K, H, T, mep.MOE_BF16)
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream
    try:
        v = mep.moe_group_view_get(g)

        def d2d(dst, src, nbytes):
            assert lib.hipMemcpyAsync(dst, src, nbytes, 3, st) == 0

        for c in range(C):
            mep.moe_dispatch_send(g, T, x, idx_all[c])
            mep.moe_dispatch_recv(g, expert_x, None, offs)
            e_of_row = torch.bucketize(rows, offs[1:], right=True)
            y = (expert_x.float() * (e_of_row + 1).float()[:, None]).to(torch.bfloat16)
            mep.moe_combine_send(g, y)
            mep.moe_combine_recv(g, w, out)
            res_out[c].copy_(out)
            res_ex[c].copy_(expert_x)
            d2d(res_cnt[c].data_ptr(), v.cnt, N * E * 4)
            d2d(res_pos[c].data_ptr(), v.pos, N * T * K * 4)
            d2d(res_g[c].data_ptr(), v.recv_base, (N + 1) * 4)
            if c % 4096 == 4095:
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
    for c in range(C):
        idx = cases[c]
        d = oracle.run_dispatch(inp["x"], idx, E)
        assert np.array_equal(got_cnt[c], d["cnt"]), c
        assert np.array_equal(got_pos[c], d["pos"]), c
        assert np.array_equal(got_g[c], d["G"]), c
        assert np.array_equal(got_ex[c], d["expert_x"]), c
        y = oracle.expert_standin(d["expert_x"], None, d["eoff"], H)
        ref = oracle.run_combine(y, inp["w"], d, H)["out"]
        assert np.array_equal(got_out[c], ref), c
