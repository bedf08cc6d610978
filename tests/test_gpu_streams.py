"""The send/recv split on several streams: the halves run on different
streams ordered by events, with unrelated work (a GEMM standing in for the
shared expert) running concurrently on a third stream ([EPMC] "Portable
kernels": other work overlaps the transfer between the halves; [EFA] "MoE
all-to-all over EFA").  Results must equal the oracle's, as on one stream."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import d2h, say, to_dev
from workloads import CONFIGS, make_inputs
from workloads.expert import standin_expert

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402


@pytest.mark.parametrize("transport", [0, 1])
def test_halves_on_separate_streams_with_concurrent_gemm(transport):
    cfg = CONFIGS["C"]
    say(f"[gpu] streams {cfg.describe()} transport={transport}")
    inp = make_inputs(cfg)
    N, T, K, E, H = cfg.N, cfg.T, cfg.K, cfg.E, cfg.H
    R = cfg.rows
    send_s, recv_s, other_s = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    x, idx, w = to_dev(torch, inp["x"]), to_dev(torch, inp["idx"]), to_dev(torch, inp["w"])
    expert_x = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    offs = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    out = torch.empty((N, T, H), dtype=torch.bfloat16, device="cuda")
    a = torch.randn((N * T, H), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((H, 2048), dtype=torch.bfloat16, device="cuda")
    ref_gemm = torch.matmul(a, b)
    torch.cuda.synchronize()
    g = mep.moe_group_create(N, E, K, H, T, mep.MOE_BF16, transport)
    try:
        sent, received, combined = torch.cuda.Event(), torch.cuda.Event(), torch.cuda.Event()
        with torch.cuda.stream(other_s):
            gemm = torch.matmul(a, b)                       # runs beside the send half
        mep.moe_dispatch_send(g, T, x, idx, stream=send_s)
        sent.record(send_s)
        recv_s.wait_event(sent)
        mep.moe_dispatch_recv(g, expert_x, None, offs, stream=recv_s)
        with torch.cuda.stream(recv_s):
            y = standin_expert(torch, expert_x.view(torch.uint8), None, offs, E, H, False)
        received.record(recv_s)
        send_s.wait_event(received)
        with torch.cuda.stream(other_s):
            gemm2 = torch.matmul(a, b)                      # runs beside the combine send
        mep.moe_combine_send(g, y, stream=send_s)
        combined.record(send_s)
        recv_s.wait_event(combined)
        mep.moe_combine_recv(g, w, out, stream=recv_s)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
        d = oracle.run_dispatch(inp["x"], inp["idx"], E)
        assert np.array_equal(expert_x.view(torch.int16).cpu().numpy().view(np.uint16),
                              d["expert_x"])
        c = oracle.run_combine(y.view(torch.int16).cpu().numpy().view(np.uint16), inp["w"], d, H)
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), c["out"])
        assert torch.equal(gemm, ref_gemm) and torch.equal(gemm2, ref_gemm)
    finally:
        mep.moe_group_destroy(g)


def test_two_groups_concurrently_on_two_streams():
    """Two groups with different shapes and modes, their cycles interleaved
    call by call on two streams (each group has its own plan, error word and
    arrival counter): both match the oracle."""
    cfg_a = CONFIGS["B"]
    cfg_b = CONFIGS["A"].with_(N=4, E=16, K=3, T=40, H=512, routing="uniform")
    say(f"[gpu] two groups {cfg_a.describe()} | {cfg_b.describe()}")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    setups = []
    for cfg, transport, mode in ((cfg_a, 0, mep.MOE_COMBINE_RECEIVER),
                                 (cfg_b, 1, mep.MOE_COMBINE_PARTIAL)):
        inp = make_inputs(cfg)
        R = cfg.rows
        setups.append({
            "cfg": cfg, "inp": inp, "partial": mode == mep.MOE_COMBINE_PARTIAL,
            "g": mep.moe_group_create(cfg.N, cfg.E, cfg.K, cfg.H, cfg.T, mep.MOE_BF16, transport, mode),
            "x": to_dev(torch, inp["x"]), "idx": to_dev(torch, inp["idx"]), "w": to_dev(torch, inp["w"]),
            "ex": torch.empty((R, cfg.H), dtype=torch.bfloat16, device="cuda"),
            "offs": torch.empty((cfg.E + 1,), dtype=torch.int32, device="cuda"),
            "out": torch.empty((cfg.N, cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda"),
        })
    try:
        for _ in range(3):
            for st, su in zip(streams, setups):
                mep.moe_dispatch_send(su["g"], su["cfg"].T, su["x"], su["idx"],
                                      su["w"] if su["partial"] else None, stream=st)
            for st, su in zip(streams, setups):
                mep.moe_dispatch_recv(su["g"], su["ex"], None, su["offs"], stream=st)
            for st, su in zip(streams, setups):
                with torch.cuda.stream(st):
                    su["y"] = standin_expert(torch, su["ex"].view(torch.uint8), None, su["offs"],
                                             su["cfg"].E, su["cfg"].H, False)
                mep.moe_combine_send(su["g"], su["y"], stream=st)
            for st, su in zip(streams, setups):
                mep.moe_combine_recv(su["g"], None if su["partial"] else su["w"], su["out"], stream=st)
            torch.cuda.synchronize()
            for su in setups:
                cfg, inp = su["cfg"], su["inp"]
                assert mep.moe_group_status(su["g"]) == mep.MOE_OK
                d = oracle.run_dispatch(inp["x"], inp["idx"], cfg.E)
                y = oracle.expert_standin(d["expert_x"], None, d["eoff"], cfg.H)
                ref = (oracle.run_partial_combine(y, inp["w"], inp["idx"], d, cfg.H) if su["partial"]
                       else oracle.run_combine(y, inp["w"], d, cfg.H))["out"]
                got = su["out"].view(torch.int16).cpu().numpy().view(np.uint16)
                assert np.array_equal(got, ref), cfg.name
    finally:
        torch.cuda.synchronize()
        for su in setups:
            mep.moe_group_destroy(su["g"])
