"""The DeepSeek-R1 prefill shape with fp8 dispatch at full size (64 ranks x
2048 tokens x 7168, top-8 of 256 experts: 1 048 576 rows), compared with the
oracle in full, in all four transport x combine modes:

- the integer plan and every metadata plane (and, for the combine with
  sender-side partial sums, the partial-row plan);
- every expert row's e4m3 codes and block scales: the oracle quantises each
  of the 131 072 tokens once, and expert row r must hold the codes of the
  token its (source rank, slot) names;
- every combined token: the oracle's per-token combine (the fp32 chain, or
  the partial sums) over the GPU's own expert outputs, copied back.

The oracle runs on WORKERS threads over token ranges (its C functions release
the interpreter lock); the GPU's rows come back in slices, so host memory
stays at about the size of one expert-output array (15 GB).  The identity
pin (identity experts, weights summing to one) closes the module: every
output token must equal its own dequantised token."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from tests.fp8_checks import e4m3_values
from tests.gpu_util import d2h, e4m3_lut, say, ulp_dist_bf16
from workloads import CONFIGS, bf16_bits_from_f32, make_routing, make_tokens, renormalised

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402

WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))
SLICE = 1 << 16          # rows per device-to-host slice


def _par(fn, n: int, chunk: int):
    """fn(a, b) over [0, n) in chunks of `chunk`, on WORKERS threads."""
    with ThreadPoolExecutor(WORKERS) as ex:
        list(ex.map(lambda a: fn(a, min(n, a + chunk)), range(0, n, chunk)))


@pytest.fixture(scope="module")
def prefill():
    cfg = CONFIGS["D"]
    N, T, K, E, H = cfg.N, cfg.T, cfg.K, cfg.E, cfg.H
    say(f"[gpu] prefill {cfg.describe()}: tokens and routing ({WORKERS} threads)")
    x = np.empty((N * T, H), dtype=np.uint16)

    def tokens(a, b):
        for s in range(a, b):
            x[s * T:(s + 1) * T] = make_tokens(cfg, s)
    _par(tokens, N, 1)
    idx, w = make_routing(cfg)
    say("[gpu] prefill: oracle quantisation of every token")
    q = np.empty((N * T, H), dtype=np.uint8)
    sc = np.empty((N * T, H // 128), dtype=np.float32)
    _par(lambda a, b: oracle.quant_rows_fp8(x[a:b], q[a:b], sc[a:b]), N * T, 1024)
    say("[gpu] prefill: oracle plan and metadata")
    pl = oracle.plan(idx, E)
    meta = oracle.send_meta(pl["pos"])
    recv_meta = oracle.transfer(meta, pl, T, K)
    R = cfg.rows
    _, _, src_rank, src_slot = oracle.shuffle(np.zeros((R, 0), np.uint8), None, recv_meta, pl, T, K)
    tok_of_row = src_rank.astype(np.int64) * T + src_slot // K
    rows_of = oracle.expert_rows(idx, pl).reshape(-1, K).astype(np.int64)
    x_dev = torch.from_numpy(x.view(np.int16)).cuda().view(N, T, H)
    return dict(cfg=cfg, x=x, idx=idx, w=w, q=q, sc=sc, pl=pl, meta=meta, recv_meta=recv_meta,
                src_rank=src_rank, src_slot=src_slot, tok_of_row=tok_of_row, rows_of=rows_of,
                x_dev=x_dev)


def _standin(expert_x, expert_scale, offs, R, H, identity=False):
    """Outside the path: y = bf16(e4m3 value * block scale * (e+1)), or the
    dequantised row itself for identity experts; in slices of rows."""
    y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    lut = e4m3_lut(torch)
    for a in range(0, R, 1 << 14):
        b = min(R, a + (1 << 14))
        v8 = lut[expert_x[a:b].long()] * expert_scale[a:b].repeat_interleave(128, dim=1)
        if not identity:
            e_of_row = torch.bucketize(torch.arange(a, b, device="cuda", dtype=torch.int32),
                                       offs[1:].contiguous(), right=True)
            v8 = v8 * (e_of_row + 1).float()[:, None]
        y[a:b] = v8.to(torch.bfloat16)
    return y


def _dispatch_and_check(P, g, partial):
    cfg = P["cfg"]
    N, T, K, E, H = cfg.N, cfg.T, cfg.K, cfg.E, cfg.H
    R = cfg.rows
    d_idx = torch.from_numpy(P["idx"]).cuda()
    d_w = torch.from_numpy(P["w"]).cuda()
    expert_x = torch.empty((R, H), dtype=torch.uint8, device="cuda")
    expert_scale = torch.empty((R, H // 128), dtype=torch.float32, device="cuda")
    offs = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    mep.moe_dispatch_send(g, T, P["x_dev"], d_idx, d_w if partial else None)
    mep.moe_dispatch_recv(g, expert_x, expert_scale, offs)
    torch.cuda.synchronize()
    assert mep.moe_group_status(g) == mep.MOE_OK
    say("[gpu] prefill dispatch done; plan and metadata")
    v = mep.moe_group_view_get(g)
    pl = P["pl"]
    assert np.array_equal(d2h(v.cnt, (N, E), np.int32), pl["cnt"])
    assert np.array_equal(d2h(v.pos, (N, T, K), np.int32), pl["pos"])
    assert np.array_equal(d2h(v.send_off, (N, E + 1), np.int32), pl["soff"])
    assert np.array_equal(d2h(v.recv_off, (N, N + 1), np.int32), pl["roff"])
    assert np.array_equal(d2h(v.recv_base, (N + 1,), np.int32), pl["G"])
    assert np.array_equal(offs.cpu().numpy(), pl["eoff"])
    if v.send_meta:
        assert np.array_equal(d2h(v.send_meta, (R,), np.int32), P["meta"])
    assert np.array_equal(d2h(v.recv_meta, (R,), np.int32), P["recv_meta"])
    assert np.array_equal(d2h(v.expert_src_rank, (R,), np.int32), P["src_rank"])
    assert np.array_equal(d2h(v.expert_src_slot, (R,), np.int32), P["src_slot"])
    assert np.diff(pl["G"]).max() <= N * T * min(K, cfg.L)

    say("[gpu] prefill: every expert row's codes and scales")
    q, sc, tok = P["q"], P["sc"], P["tok_of_row"]
    for a in range(0, R, SLICE):
        b = min(R, a + SLICE)
        got_q = expert_x[a:b].cpu().numpy()
        want_q = q[tok[a:b]]
        if not np.array_equal(got_q, want_q):
            r = a + int(np.nonzero((got_q != want_q).any(axis=1))[0][0])
            raise AssertionError(f"expert row {r} (token {tok[r]}) codes differ")
        got_s = expert_scale[a:b].cpu().numpy().view(np.uint32)
        assert np.array_equal(got_s, sc[tok[a:b]].view(np.uint32)), (a, b)
    return expert_x, expert_scale, offs, d_w


@pytest.mark.parametrize("combine_mode", [0, 1])
@pytest.mark.parametrize("transport", [0, 1])
def test_prefill_fp8_full_size(prefill, transport, combine_mode):
    P = prefill
    cfg = P["cfg"]
    N, T, K, E, H = cfg.N, cfg.T, cfg.K, cfg.E, cfg.H
    R = cfg.rows
    partial = combine_mode == mep.MOE_COMBINE_PARTIAL
    say(f"[gpu] prefill full size {cfg.describe()} rows={R} transport={transport} "
        f"combine_mode={combine_mode}")
    g = mep.moe_group_create(N, E, K, H, T, mep.MOE_FP8_E4M3, transport, combine_mode)
    try:
        expert_x, expert_scale, offs, d_w = _dispatch_and_check(P, g, partial)
        say("[gpu] prefill: combine")
        y = _standin(expert_x, expert_scale, offs, R, H)
        del expert_x, expert_scale
        out = torch.empty((N, T, H), dtype=torch.bfloat16, device="cuda")
        mep.moe_combine_send(g, y)
        mep.moe_combine_recv(g, None if partial else d_w, out)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
        idx = P["idx"]
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
        say("[gpu] prefill: expert outputs to the host; the oracle combines every token")
        y_host = y.view(torch.int16).cpu().numpy().view(np.uint16)
        del y
        got = out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(N * T, H)
        want = np.empty((N * T, H), dtype=np.uint16)
        rows_of = P["rows_of"]
        w2 = P["w"].reshape(-1, K)
        rank2 = (idx // cfg.L).reshape(-1, K)

        def combine(a, b):
            if partial:
                want[a:b] = oracle.partial_tokens(y_host, rows_of[a:b], w2[a:b], rank2[a:b])
            else:
                want[a:b] = oracle.combine_tokens(y_host, rows_of[a:b], w2[a:b])
        _par(combine, N * T, 512)
        bad = np.nonzero((got != want).any(axis=1))[0]
        assert bad.size == 0, (bad[:5], ulp_dist_bf16(got[bad[0]], want[bad[0]]).max())
        say(f"[gpu] prefill: {N * T} tokens equal")
    finally:
        mep.moe_group_destroy(g)


def test_prefill_identity_experts_return_dequantised_tokens(prefill):
    """Identity experts (each expert returns its dequantised input row, in
    bf16) and router weights renormalised to sum to one: every output token is
    its own dequantised token, bf16(e4m3 value * block scale), from the
    oracle's codes and scales (the K equal rows summed with weights of sum one
    stay within half a bf16 ulp of the row)."""
    P = prefill
    cfg = P["cfg"]
    N, T, K, E, H = cfg.N, cfg.T, cfg.K, cfg.E, cfg.H
    R = cfg.rows
    say(f"[gpu] prefill identity {cfg.describe()}")
    g = mep.moe_group_create(N, E, K, H, T, mep.MOE_FP8_E4M3)
    try:
        d_idx = torch.from_numpy(P["idx"]).cuda()
        d_w = torch.from_numpy(renormalised(P["w"])).cuda()
        expert_x = torch.empty((R, H), dtype=torch.uint8, device="cuda")
        expert_scale = torch.empty((R, H // 128), dtype=torch.float32, device="cuda")
        offs = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
        mep.moe_dispatch_send(g, T, P["x_dev"], d_idx, None)
        mep.moe_dispatch_recv(g, expert_x, expert_scale, offs)
        y = _standin(expert_x, expert_scale, offs, R, H, identity=True)
        del expert_x, expert_scale
        out = torch.empty((N, T, H), dtype=torch.bfloat16, device="cuda")
        mep.moe_combine_send(g, y)
        mep.moe_combine_recv(g, d_w, out)
        torch.cuda.synchronize()
        assert mep.moe_group_status(g) == mep.MOE_OK
        got = out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(N * T, H)
        vals = e4m3_values().astype(np.float32)
        q, sc = P["q"], P["sc"]

        def check(a, b):
            v = vals[q[a:b]] * np.repeat(sc[a:b], 128, axis=1)
            want = bf16_bits_from_f32(v)
            want = np.where(want == 0x8000, 0, want)        # -0 comes back as +0
            assert np.array_equal(got[a:b], want), a
        _par(check, N * T, 2048)
    finally:
        mep.moe_group_destroy(g)
