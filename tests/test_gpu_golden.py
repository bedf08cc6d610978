"""The hand-worked 2-rank example (tests/golden/tiny_hand_example.json,
derived on paper) through the C ABI on the GPU, in every transport, combine
mode and receive layout: the plan, the back-routing metadata and the combined
tokens are compared with the paper values directly, with no oracle between."""
import json
import os

import numpy as np
import pytest

from tests.gpu_util import d2h, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_hand_example.json")))
MODES = [(t, c, l) for t in (mep.MOE_TRANSPORT_STAGED, mep.MOE_TRANSPORT_DIRECT)
         for c in (mep.MOE_COMBINE_RECEIVER, mep.MOE_COMBINE_PARTIAL)
         for l in (mep.MOE_LAYOUT_PACKED, mep.MOE_LAYOUT_FIXED_SLOT)]


@pytest.mark.parametrize("mode", MODES, ids=[f"t{t}-c{c}-l{l}" for t, c, l in MODES])
def test_hand_worked_example_on_gpu(mode):
    transport, combine_mode, layout = mode
    partial = combine_mode == mep.MOE_COMBINE_PARTIAL
    N, T, K, E, H = G["N"], G["T"], G["K"], G["E"], 8
    R = N * T * K
    say(f"[gpu] hand-worked example mode={mode}")
    idx = torch.tensor(G["idx"], dtype=torch.int32, device="cuda")
    w = torch.tensor(G["partial"]["w"], dtype=torch.float32, device="cuda")
    # token rows carry their identity: element 0 = 100*s + t
    x = torch.zeros((N, T, H), dtype=torch.bfloat16, device="cuda")
    for s in range(N):
        for t in range(T):
            x[s, t, 0] = 100 * s + t
    expert_x = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    offs = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    out = torch.empty((N, T, H), dtype=torch.bfloat16, device="cuda")
    g = mep.moe_group_create(N, E, K, H, G["fixed_slot"]["T_max"], mep.MOE_BF16, transport,
                             combine_mode, layout)
    try:
        mep.moe_dispatch_send(g, T, x, idx, w if partial else None)
        mep.moe_dispatch_recv(g, expert_x, None, offs)
        # expert row r outputs r + 1 in every element
        y = (torch.arange(1, R + 1, dtype=torch.float32, device="cuda")[:, None]
             .expand(R, H).to(torch.bfloat16).contiguous())
        mep.moe_combine_send(g, y)
        mep.moe_combine_recv(g, None if partial else w, out)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
        v = mep.moe_group_view_get(g)
        assert d2h(v.cnt, (N, E), np.int32).tolist() == G["cnt"]
        assert d2h(v.pos, (N, T, K), np.int32).tolist() == G["pos"]
        assert d2h(v.recv_base, (N + 1,), np.int32).tolist() == G["G"]
        assert offs.cpu().tolist() == G["eoff"]
        assert d2h(v.expert_src_rank, (R,), np.int32).tolist() == G["expert_src_rank"]
        assert d2h(v.expert_src_slot, (R,), np.int32).tolist() == G["expert_src_slot"]
        # expert row r holds the token of (expert_src_rank[r], expert_src_slot[r] // K)
        tok = expert_x[:, 0].float().cpu().tolist()
        assert tok == [100 * s + q // K for s, q in zip(G["expert_src_rank"], G["expert_src_slot"])]
        if partial:
            assert d2h(v.part_dst, (N, T, K), np.int32).tolist() == [
                [[e // (E // N) for e in row] for row in s] for s in G["idx"]]
        want = G["partial"]["out"] if partial else G["combine"]["out"]
        assert out[:, :, 0].float().cpu().tolist() == want
        assert torch.equal(out, out[:, :, :1].expand(N, T, H))
    finally:
        torch.cuda.synchronize()
        mep.moe_group_destroy(g)
