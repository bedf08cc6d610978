"""Helpers for the GPU parity tests: run one dispatch/combine cycle through the
C ABI and copy every buffer back to the host.  torch provides device memory
and the stream; raw device buffers of the group are read with hipMemcpy."""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np

from workloads.expert import e4m3_lut, standin_expert  # noqa: F401


def hip():
    """The HIP runtime already loaded in this process (torch's, which the
    library also binds to), found by its soname without loading another."""
    mode = getattr(os, "RTLD_NOLOAD", 4) | os.RTLD_LAZY
    lib = None
    for name in ("libamdhip64.so.7", "libamdhip64.so"):
        try:
            lib = ctypes.CDLL(name, mode=mode)
            break
        except OSError:
            continue
    assert lib is not None, "HIP runtime not loaded"
    lib.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    lib.hipMemcpy.restype = ctypes.c_int
    return lib


_HIP = None


def d2h(ptr: int, shape, dtype) -> np.ndarray:
    """Copy a device buffer (raw address) into a new numpy array."""
    global _HIP
    if _HIP is None:
        _HIP = hip()
    out = np.empty(shape, dtype=dtype)
    if out.nbytes:
        rc = _HIP.hipMemcpy(out.ctypes.data, ptr, out.nbytes, 2)   # device -> host
        assert rc == 0, f"hipMemcpy failed: {rc}"
    return out


def d2h_rows(ptr: int, rows: np.ndarray, row_shape, dtype) -> np.ndarray:
    """Copy the listed rows of a device row buffer (raw address) to the host,
    one copy per run of consecutive rows."""
    global _HIP
    if _HIP is None:
        _HIP = hip()
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    out = np.empty((rows.size,) + tuple(row_shape), dtype=dtype)
    rb = out[0].nbytes if rows.size else 0
    i = 0
    while i < rows.size:
        j = i + 1
        while j < rows.size and rows[j] == rows[j - 1] + 1:
            j += 1
        rc = _HIP.hipMemcpy(out[i:j].ctypes.data, ptr + int(rows[i]) * rb, rb * (j - i), 2)
        assert rc == 0, f"hipMemcpy failed: {rc}"
        i = j
    return out


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(torch, a: np.ndarray):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16)
    return t.to("cuda")


def run_cycle(torch, mep, cfg, inp, *, T_max=None, identity=False, group=None, want_rows=True,
              transport=0, combine_mode=0, layout=0, recv_gather=None, check_status=True):
    """One full dispatch + stand-in expert + combine cycle on the GPU.
    Returns a dict of host copies of every buffer (rows only if want_rows;
    the send-side buffers only with the staged transport).  With the partial
    combine the weights go to dispatch_send, combine_recv gets none, and the
    partial-row plan and rows are returned too.  With the fixed-slot layout the
    receive-layout rows (receive planes, combine send rows) are read only at
    the slot rows listed in recv_gather, in that order.  With
    check_status=False the group's status is not read (nor cleared)."""
    N, T, K, E, H = cfg.N, inp["idx"].shape[1], cfg.K, cfg.E, cfg.H
    fp8 = cfg.dtype == "fp8"
    T_max = T if T_max is None else T_max
    own = group is None
    g = group if group is not None else mep.moe_group_create(
        N, E, K, H, T_max, mep.MOE_FP8_E4M3 if fp8 else mep.MOE_BF16, transport, combine_mode,
        layout)
    try:
        R = N * T * K
        x = to_dev(torch, inp["x"])
        idx = to_dev(torch, inp["idx"])
        w = to_dev(torch, inp["w"])
        payload = H if fp8 else 2 * H
        expert_x = torch.empty(max(R, 1) * payload, dtype=torch.uint8, device="cuda")
        expert_scale = torch.empty(max(R, 1) * (H // 128), dtype=torch.float32,
                                   device="cuda") if fp8 else None
        expert_offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
        out = torch.empty((N, max(T, 1), H), dtype=torch.bfloat16, device="cuda")
        partial = combine_mode == mep.MOE_COMBINE_PARTIAL
        mep.moe_dispatch_send(g, T, x, idx, w if partial else None)
        mep.moe_dispatch_recv(g, expert_x, expert_scale, expert_offsets)
        torch.cuda.synchronize()
        if check_status:
            assert mep.moe_group_status(g) == mep.MOE_OK
        res = {}
        v = mep.moe_group_view_get(g)
        res["cnt"] = d2h(v.cnt, (N, E), np.int32)
        res["pos"] = d2h(v.pos, (N, T, K), np.int32)
        res["soff"] = d2h(v.send_off, (N, E + 1), np.int32)
        res["roff"] = d2h(v.recv_off, (N, N + 1), np.int32)
        res["G"] = d2h(v.recv_base, (N + 1,), np.int32)
        res["eoff"] = d2h(v.expert_off, (E + 1,), np.int32)
        res["expert_offsets"] = expert_offsets.cpu().numpy()
        staged = bool(v.send_x)
        fixed = v.desc.layout == mep.MOE_LAYOUT_FIXED_SLOT

        def recv_plane(ptr, row_shape, dtype):
            if fixed:
                return None if recv_gather is None else d2h_rows(ptr, recv_gather, row_shape, dtype)
            return d2h(ptr, (R,) + tuple(row_shape), dtype)

        if staged:
            res["send_meta"] = d2h(v.send_meta, (R,), np.int32)
        res["recv_meta"] = recv_plane(v.recv_meta, (), np.int32)
        res["expert_src_rank"] = d2h(v.expert_src_rank, (R,), np.int32)
        res["expert_src_slot"] = d2h(v.expert_src_slot, (R,), np.int32)
        pdt = np.uint8 if fp8 else np.uint16
        if want_rows:
            if staged:
                res["send_x"] = d2h(v.send_x, (R, H), pdt)
            res["recv_x"] = recv_plane(v.recv_x, (H,), pdt)
            res["expert_x"] = expert_x[:R * payload].cpu().numpy().view(pdt).reshape(R, H)
            if fp8:
                nb = H // 128
                if staged:
                    res["send_scale"] = d2h(v.send_scale, (R, nb), np.float32)
                res["recv_scale"] = recv_plane(v.recv_scale, (nb,), np.float32)
                res["expert_scale"] = expert_scale[:R * nb].cpu().numpy().reshape(R, nb)
        if identity:
            y = expert_x[:R * payload].view(torch.bfloat16).reshape(R, H) if R else \
                torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
        else:
            y = standin_expert(torch, expert_x, expert_scale, expert_offsets, E, H, fp8) if R else \
                torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
        y = y.contiguous()
        mep.moe_combine_send(g, y)
        mep.moe_combine_recv(g, None if partial else w, out)
        torch.cuda.synchronize()
        if check_status:
            assert mep.moe_group_status(g) == mep.MOE_OK
        v = mep.moe_group_view_get(g)
        res["y"] = y.view(torch.int16).cpu().numpy().view(np.uint16)
        if partial:
            res["part_dst"] = d2h(v.part_dst, (N, T, K), np.int32)
            res["part_pos"] = d2h(v.part_pos, (N, T, K), np.int32)
            res["part_send_off"] = d2h(v.part_send_off, (N, N + 1), np.int32)
            res["part_base"] = d2h(v.part_base, (N + 1,), np.int32)
            res["part_owner_base"] = d2h(v.part_owner_base, (N + 1,), np.int32)
            P = int(res["part_base"][N])
            res["P"] = P
            if want_rows:
                if staged:
                    res["psend"] = d2h(v.comb_send, (P, H), np.uint16)
                res["precv"] = d2h(v.comb_recv, (P, H), np.uint16)
        elif want_rows:
            if staged:
                res["comb_send"] = recv_plane(v.comb_send, (H,), np.uint16)
            res["comb_recv"] = d2h(v.comb_recv, (R, H), np.uint16)
        res["y_dev"] = y
        res["out"] = out[:, :T].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return res
    finally:
        if own:
            mep.moe_group_destroy(g)


def ulp_dist_bf16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def ordered(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))
