"""One whole dispatch + combine cycle captured as a HIP graph (torch's CUDAGraph
wrapper over hipStreamBeginCapture) and replayed: the four calls enqueue only
kernels (no allocation, memset or host synchronisation), so the capture holds
the whole path, and the stand-in expert between the halves is computed from
the device offsets.  New tokens, routing and weights are copied into the
captured input buffers between replays, with eager work and synchronisations
in between, and every replay is compared with eager cycles on the same
inputs, bit-exactly."""
import numpy as np
import pytest

from tests.gpu_util import say
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402


def standin_on_device(expert_x, offs, R):
    """The stand-in expert y = bf16(x * (e+1)) from the device offsets alone
    (no host synchronisation, so it can sit inside the capture)."""
    rows = torch.arange(R, device=expert_x.device, dtype=torch.int32)
    e_of_row = torch.bucketize(rows, offs[1:], right=True)
    return (expert_x.float() * (e_of_row + 1).float()[:, None]).to(torch.bfloat16)


@pytest.mark.parametrize("transport,combine_mode", [(0, 0), (1, 0), (0, 1)])
def test_captured_cycle_replays_match_eager(transport, combine_mode):
    cfg = CONFIGS["B"]
    say(f"[gpu] graph {cfg.describe()} transport={transport} combine_mode={combine_mode}")
    N, T, K, E, H = cfg.N, cfg.T, cfg.K, cfg.E, cfg.H
    R = cfg.rows
    partial = combine_mode == mep.MOE_COMBINE_PARTIAL
    seeds = [cfg.seed + 100 * i for i in range(4)]
    inputs = [make_inputs(cfg.with_(seed=s)) for s in seeds]
    dev = "cuda"
    x = torch.empty((N, T, H), dtype=torch.int16, device=dev)
    idx = torch.empty((N, T, K), dtype=torch.int32, device=dev)
    w = torch.empty((N, T, K), dtype=torch.float32, device=dev)
    expert_x = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    out = torch.empty((N, T, H), dtype=torch.bfloat16, device=dev)

    def load(inp):
        x.copy_(torch.from_numpy(inp["x"].view(np.int16)))
        idx.copy_(torch.from_numpy(inp["idx"]))
        w.copy_(torch.from_numpy(inp["w"]))

    g = mep.moe_group_create(N, E, K, H, T, mep.MOE_BF16, transport, combine_mode)
    try:
        def cycle(stream):
            mep.moe_dispatch_send(g, T, x, idx, w if partial else None, stream=stream)
            mep.moe_dispatch_recv(g, expert_x, None, offs, stream=stream)
            with torch.cuda.stream(stream):
                y = standin_on_device(expert_x, offs, R)
            mep.moe_combine_send(g, y, stream=stream)
            mep.moe_combine_recv(g, None if partial else w, out, stream=stream)
            return y

        # eager reference outputs for every input set
        eager = []
        side = torch.cuda.Stream()
        for inp in inputs:
            load(inp)
            torch.cuda.synchronize()
            cycle(side)
            torch.cuda.synchronize()
            assert mep.moe_group_status(g) == mep.MOE_OK
            eager.append(out.clone())
        # capture one cycle on inputs[0]
        load(inputs[0])
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                cycle(cap)
        torch.cuda.synchronize()
        # replays on new tokens, routing and weights (same T): the whole plan
        # is recomputed on the device by the captured kernels
        for rep in range(3):
            load(inputs[(rep + 1) % len(inputs)])
            out.fill_(-1.0)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = out.clone()
            # eager run of the same inputs between replays
            cycle(side)
            torch.cuda.synchronize()
            assert mep.moe_group_status(g) == mep.MOE_OK
            assert torch.equal(got.view(torch.int16), out.view(torch.int16)), rep
            assert torch.equal(got.view(torch.int16), eager[(rep + 1) % len(inputs)].view(torch.int16))
        del graph
    finally:
        torch.cuda.synchronize()
        mep.moe_group_destroy(g)
