"""The DeepSeek-R1 prefill shape with fp8 dispatch at full size (64 ranks x
2048 tokens x 7168, top-8 of 256 experts: 1 048 576 rows): the integer plan and
all metadata (and, for the combine with sender-side partial sums, the
partial-row plan) are compared in full with the oracle; payload rows, block
scales and combined tokens are compared on a seeded sample, each computed by
the oracle one at a time."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import d2h, e4m3_lut, say, ulp_dist_bf16
from workloads import CONFIGS, make_routing, make_tokens

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402


@pytest.mark.parametrize("combine_mode", [0, 1])
@pytest.mark.parametrize("transport", [0, 1])
def test_prefill_fp8_full_size_sampled(transport, combine_mode):
    cfg = CONFIGS["D"]
    partial = combine_mode == mep.MOE_COMBINE_PARTIAL
    N, T, K, E, H = cfg.N, cfg.T, cfg.K, cfg.E, cfg.H
    R = cfg.rows
    say(f"[gpu] prefill full size {cfg.describe()} rows={R} transport={transport} "
        f"combine_mode={combine_mode}")
    idx, w = make_routing(cfg)
    x = torch.empty((N, T, H), dtype=torch.int16, device="cuda")
    for s in range(N):
        x[s].copy_(torch.from_numpy(make_tokens(cfg, s).view(np.int16)))
    d_idx = torch.from_numpy(idx).cuda()
    d_w = torch.from_numpy(w).cuda()
    expert_x = torch.empty((R, H), dtype=torch.uint8, device="cuda")
    expert_scale = torch.empty((R, H // 128), dtype=torch.float32, device="cuda")
    offs = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    out = torch.empty((N, T, H), dtype=torch.bfloat16, device="cuda")
    g = mep.moe_group_create(N, E, K, H, T, mep.MOE_FP8_E4M3, transport, combine_mode)
    try:
        mep.moe_dispatch_send(g, T, x, d_idx, d_w if partial else None)
        mep.moe_dispatch_recv(g, expert_x, expert_scale, offs)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
        say("[gpu] prefill dispatch done; checking plan and metadata")
        v = mep.moe_group_view_get(g)
        pl = oracle.plan(idx, E)
        assert np.array_equal(d2h(v.cnt, (N, E), np.int32), pl["cnt"])
        assert np.array_equal(d2h(v.pos, (N, T, K), np.int32), pl["pos"])
        assert np.array_equal(d2h(v.send_off, (N, E + 1), np.int32), pl["soff"])
        assert np.array_equal(d2h(v.recv_off, (N, N + 1), np.int32), pl["roff"])
        assert np.array_equal(d2h(v.recv_base, (N + 1,), np.int32), pl["G"])
        assert np.array_equal(offs.cpu().numpy(), pl["eoff"])
        meta = oracle.send_meta(pl["pos"])
        if v.send_meta:
            assert np.array_equal(d2h(v.send_meta, (R,), np.int32), meta)
        recv_meta = oracle.transfer(meta, pl, T, K)
        assert np.array_equal(d2h(v.recv_meta, (R,), np.int32), recv_meta)
        _, _, src_rank, src_slot = oracle.shuffle(np.zeros((R, 0), np.uint8), None, recv_meta, pl, T, K)
        assert np.array_equal(d2h(v.expert_src_rank, (R,), np.int32), src_rank)
        assert np.array_equal(d2h(v.expert_src_slot, (R,), np.int32), src_slot)
        assert np.diff(pl["G"]).max() <= N * T * min(K, cfg.L)

        say("[gpu] prefill: sampled payload rows")
        gsm = np.random.default_rng(11)
        sample = gsm.choice(R, size=256, replace=False)
        by_rank = {}
        for r in sample:
            by_rank.setdefault(int(src_rank[r]), []).append(int(r))
        for s, rs in sorted(by_rank.items())[:16]:          # 16 source ranks
            xs = make_tokens(cfg, s)
            for r in rs:
                q, sc = oracle.quant_row_fp8(xs[int(src_slot[r]) // K])
                assert np.array_equal(expert_x[r].cpu().numpy(), q), r
                assert np.array_equal(expert_scale[r].cpu().numpy().view(np.uint32),
                                      sc.view(np.uint32)), r

        say("[gpu] prefill: combine")
        # stand-in expert (outside the path), in slices of rows:
        # y = bf16(e4m3 value * block scale * (e+1)), e = the row's expert
        y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
        lut = e4m3_lut(torch)
        for a in range(0, R, 1 << 14):
            b = min(R, a + (1 << 14))
            e_of_row = torch.bucketize(torch.arange(a, b, device="cuda", dtype=torch.int32),
                                       offs[1:].contiguous(), right=True)
            v8 = lut[expert_x[a:b].long()] * expert_scale[a:b].repeat_interleave(128, dim=1)
            y[a:b] = (v8 * (e_of_row + 1).float()[:, None]).to(torch.bfloat16)
        mep.moe_combine_send(g, y)
        mep.moe_combine_recv(g, None if partial else d_w, out)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
        if partial:
            say("[gpu] prefill: partial-row plan")
            v = mep.moe_group_view_get(g)
            pp = oracle.partial_plan(idx, E)
            ranks = idx // cfg.L
            assert np.array_equal(d2h(v.part_dst, (N, T, K), np.int32), ranks)
            base = d2h(v.part_base, (N + 1,), np.int32)
            assert base[N] == pp["P"] < R
            ppos = d2h(v.part_pos, (N, T, K), np.int32)
            head = ppos >= 0
            s_i, t_i, _ = np.indices(idx.shape)
            assert np.array_equal(base[s_i[head]] + ppos[head],
                                  pp["token_row"][s_i[head], t_i[head], ranks[head]])
            assert head.sum() == pp["P"]
        rows_of = oracle.expert_rows(idx, pl)
        for _ in range(64):
            s, t = int(gsm.integers(N)), int(gsm.integers(T))
            yk = y[torch.from_numpy(rows_of[s, t].astype(np.int64)).cuda()].view(torch.int16)
            yk = yk.cpu().numpy().view(np.uint16)
            if partial:
                ref = oracle.partial_token(yk, w[s, t], idx[s, t] // cfg.L)
            else:
                ref = oracle.combine_token(yk, w[s, t])
            got = out[s, t].view(torch.int16).cpu().numpy().view(np.uint16)
            assert ulp_dist_bf16(got, ref).max() == 0, (s, t)
    finally:
        mep.moe_group_destroy(g)
