"""CPU oracle for the MoE dispatch/combine path (test infrastructure only).

Only tests/, the smoke check in __graft_entry__ and the CPU-baseline leg of
bench.py may import this package.  It loads oracle/liboracle.so, built from
oracle/oracle.c with gcc (-O2 -ffp-contract=off), and wraps its functions for
numpy arrays.  It shares no code with the HIP library.

Each wrapper names the step of the pages it follows; the C source states the
definition.  `run_dispatch` / `run_combine` chain the steps in the pages' order
and return every intermediate buffer, in the same flat layouts the HIP path
exposes for checking (send rows of sender s at rows s*T*K.., receive rows of
rank d at rows G[d]..).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIBRARY selects another build of oracle.c (the sanitizer test's)
_OVERRIDE = os.environ.get("ORACLE_LIBRARY")
LIB_PATH = _OVERRIDE or os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

_lib = None


def build() -> str:
    """Compile liboracle.so with gcc."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
           "-o", LIB_PATH, SRC_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not _OVERRIDE and (not os.path.exists(LIB_PATH)
                              or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH)):
            build()
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t


def _declare(L):
    L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_bf16_to_f32.restype = ctypes.c_float
    L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    L.orc_f32_to_bf16.restype = ctypes.c_uint16
    L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_value.restype = ctypes.c_double
    L.orc_f32_to_e4m3.argtypes = [ctypes.c_float]
    L.orc_f32_to_e4m3.restype = ctypes.c_uint8
    L.orc_route_count.argtypes = [_I, _I, _I, _I, _P, _P]
    L.orc_route_count.restype = _I
    L.orc_send_offsets.argtypes = [_I, _I, _P, _P]
    L.orc_positions.argtypes = [_I, _I, _I, _I, _P, _P, _P]
    L.orc_recv_offsets.argtypes = [_I, _I, _P, _P, _P]
    L.orc_expert_offsets.argtypes = [_I, _I, _P, _P]
    L.orc_pack_bf16.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P]
    L.orc_quant_row_fp8.argtypes = [_I, _P, _P, _P]
    L.orc_pack_fp8.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P]
    L.orc_transfer.argtypes = [_I, _I, _I, _I, _Z, _P, _P, _P, _P, _P]
    L.orc_shuffle.argtypes = [_I, _I, _I, _I, _Z, _Z, _P, _P, _P, _P, _P,
                              _P, _P, _P, _P, _P, _P, _P]
    L.orc_expert_standin.argtypes = [_I, _I, _P, _P, _P, _I, _P]
    L.orc_combine_send.argtypes = [_I, _I, _Z, _P, _P, _P, _P, _P, _P, _P]
    L.orc_combine_transfer.argtypes = [_I, _I, _I, _I, _Z, _P, _P, _P, _P, _P]
    L.orc_combine_recv.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P]
    L.orc_combine_recv_f64.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P]
    L.orc_combine_token.argtypes = [_I, _I, _P, _P, _P]
    L.orc_partial_token.argtypes = [_I, _I, _P, _P, _P, _P]
    L.orc_combine_tokens.argtypes = [ctypes.c_int64, _I, _I, _P, _P, _P, _P]
    L.orc_partial_tokens.argtypes = [ctypes.c_int64, _I, _I, _P, _P, _P, _P, _P]
    L.orc_quant_rows_fp8.argtypes = [ctypes.c_int64, _I, _P, _P, _P]
    L.orc_f32_to_bf16_n.argtypes = [_Z, _P, _P]
    L.orc_send_meta.argtypes = [_I, _I, _I, _P, _P]
    L.orc_partial_counts.argtypes = [_I, _I, _I, _I, _P, _P]
    L.orc_partial_rows.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P]
    L.orc_partial_send.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
    L.orc_partial_transfer.argtypes = [_I, _I, _I, _P, _P, _P, _P]
    L.orc_partial_recv.argtypes = [_I, _I, _I, _P, _P, _P]
    L.orc_expert_rows.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
    L.orc_f32_to_e4m3_n.argtypes = [_Z, _P, _P]
    L.orc_slot_capacity_ok.argtypes = [_I, _I, _I, _P]
    L.orc_slot_capacity_ok.restype = _I
    L.orc_slot_rows.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P]
    L.orc_transfer_slots.argtypes = [_I, _I, _I, _Z, _P, _P, _P, _P]
    L.orc_shuffle_slots.argtypes = [_I, _I, _I, _Z, _Z, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    L.orc_transfer_range.argtypes = [_I, _I, _I, _I, _Z, _P, _P, _P, _P, _P, _I, _I]
    L.orc_shuffle_range.argtypes = [_I, _I, _I, _I, _Z, _Z, _P, _P, _P, _P, _P,
                                    _P, _P, _P, _P, _P, _P, _P, _I, _I]
    L.orc_combine_send_range.argtypes = [_I, _I, _Z, _P, _P, _P, _P, _P, _P, _P, _I, _I]
    L.orc_combine_transfer_range.argtypes = [_I, _I, _I, _I, _Z, _P, _P, _P, _P, _P, _I, _I]
    L.orc_expert_rows_range.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I]
    L.orc_partial_counts_range.argtypes = [_I, _I, _I, _I, _P, _P, _I, _I]
    L.orc_partial_rows_range.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _I, _I]
    L.orc_partial_send_range.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I]
    L.orc_partial_transfer_range.argtypes = [_I, _I, _I, _P, _P, _P, _P, _I, _I]
    L.orc_partial_recv_range.argtypes = [_I, _I, _I, _P, _P, _P, _I, _I]


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- codecs

def bf16_to_f32(b) -> float:
    """Value of one bf16 pattern."""
    return lib().orc_bf16_to_f32(int(b))


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 patterns (uint16), nearest even."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16_n(f.size, _p(f), _p(out))
    return out


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def f32_to_e4m3(f: np.ndarray) -> np.ndarray:
    """fp32 array -> e4m3 codes (uint8), nearest even, saturating at 448."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint8)
    lib().orc_f32_to_e4m3_n(f.size, _p(f), _p(out))
    return out


def quant_row_fp8(xrow: np.ndarray):
    """Block-scaled e4m3 quantisation of one bf16 row -> (codes uint8[H], scales fp32[H/128])."""
    xrow = np.ascontiguousarray(xrow, dtype=np.uint16)
    H = xrow.shape[-1]
    q = np.empty(H, dtype=np.uint8)
    sc = np.empty(H // 128, dtype=np.float32)
    lib().orc_quant_row_fp8(H, _p(xrow), _p(q), _p(sc))
    return q, sc


def quant_rows_fp8(x: np.ndarray, q: np.ndarray = None, sc: np.ndarray = None):
    """quant_row_fp8 of every row of x (uint16 [n][H]) -> (codes uint8 [n][H],
    scales fp32 [n][H/128]); q and sc may be given to be filled in place."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    n, H = x.shape
    q = np.empty((n, H), dtype=np.uint8) if q is None else q
    sc = np.empty((n, H // 128), dtype=np.float32) if sc is None else sc
    assert q.shape == (n, H) and sc.shape == (n, H // 128)
    lib().orc_quant_rows_fp8(n, H, _p(x), _p(q), _p(sc))
    return q, sc


# ------------------------------------------------------------- dispatch

class RoutingError(ValueError):
    pass


def route_count(idx: np.ndarray, E: int) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    N, T, K = idx.shape
    cnt = np.empty((N, E), dtype=np.int32)
    if lib().orc_route_count(N, T, K, E, _p(idx), _p(cnt)) != 0:
        raise RoutingError("expert id outside [0, E)")
    return cnt


def send_offsets(cnt: np.ndarray) -> np.ndarray:
    N, E = cnt.shape
    soff = np.empty((N, E + 1), dtype=np.int32)
    lib().orc_send_offsets(N, E, _p(cnt), _p(soff))
    return soff


def positions(idx: np.ndarray, soff: np.ndarray) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    N, T, K = idx.shape
    E = soff.shape[1] - 1
    pos = np.empty((N, T, K), dtype=np.int32)
    lib().orc_positions(N, T, K, E, _p(idx), _p(soff), _p(pos))
    return pos


def recv_offsets(soff: np.ndarray, N: int):
    E = soff.shape[1] - 1
    roff = np.empty((N, N + 1), dtype=np.int32)
    G = np.empty(N + 1, dtype=np.int32)
    lib().orc_recv_offsets(N, E, _p(soff), _p(roff), _p(G))
    return roff, G


def expert_offsets(cnt: np.ndarray) -> np.ndarray:
    N, E = cnt.shape
    eoff = np.empty(E + 1, dtype=np.int32)
    lib().orc_expert_offsets(N, E, _p(cnt), _p(eoff))
    return eoff


def plan(idx: np.ndarray, E: int) -> dict:
    """Counts, positions and every offset table (integer part of dispatch)."""
    N = idx.shape[0]
    cnt = route_count(idx, E)
    soff = send_offsets(cnt)
    pos = positions(idx, soff)
    roff, G = recv_offsets(soff, N)
    eoff = expert_offsets(cnt)
    return {"cnt": cnt, "soff": soff, "pos": pos, "roff": roff, "G": G, "eoff": eoff}


def send_meta(pos: np.ndarray) -> np.ndarray:
    """Meta word (t*K+k) of every send row, without moving any payload."""
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    N, T, K = pos.shape
    meta = np.zeros(N * T * K, dtype=np.int32)
    lib().orc_send_meta(N, T, K, _p(pos), _p(meta))
    return meta


def expert_rows(idx: np.ndarray, pl: dict) -> np.ndarray:
    """Expert-order row of every (s,t,k), int32 [N][T][K]."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    N, T, K = idx.shape
    E = pl["cnt"].shape[1]
    rows = np.zeros((N, T, K), dtype=np.int32)
    lib().orc_expert_rows(N, T, K, E, _p(idx), _p(pl["cnt"]), _p(pl["soff"]), _p(pl["pos"]),
                          _p(pl["eoff"]), _p(rows))
    return rows


def pack_bf16(x: np.ndarray, pos: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    N, T, H = x.shape
    K = pos.shape[2]
    send_x = np.zeros((N * T * K, H), dtype=np.uint16)
    send_meta = np.zeros(N * T * K, dtype=np.int32)
    lib().orc_pack_bf16(N, T, K, H, _p(x), _p(pos), _p(send_x), _p(send_meta))
    return send_x, send_meta


def pack_fp8(x: np.ndarray, pos: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    N, T, H = x.shape
    K = pos.shape[2]
    send_q = np.zeros((N * T * K, H), dtype=np.uint8)
    send_scale = np.zeros((N * T * K, H // 128), dtype=np.float32)
    send_meta = np.zeros(N * T * K, dtype=np.int32)
    lib().orc_pack_fp8(N, T, K, H, _p(x), _p(pos), _p(send_q), _p(send_scale), _p(send_meta))
    return send_q, send_scale, send_meta


def transfer(send: np.ndarray, pl: dict, T: int, K: int) -> np.ndarray:
    """Modelled network transfer of one row plane (any dtype, rows on axis 0)."""
    send = np.ascontiguousarray(send)
    N, E = pl["cnt"].shape
    recv = np.zeros_like(send)
    row_bytes = send.nbytes // max(send.shape[0], 1) if send.shape[0] else 0
    lib().orc_transfer(N, E, T, K, row_bytes, _p(pl["soff"]), _p(pl["roff"]), _p(pl["G"]),
                       _p(send), _p(recv))
    return recv


def shuffle(recv_x: np.ndarray, recv_scale, recv_meta: np.ndarray, pl: dict, T: int, K: int):
    recv_x = np.ascontiguousarray(recv_x)
    N, E = pl["cnt"].shape
    R = recv_x.shape[0]
    row_bytes = recv_x.nbytes // R if R else 0
    expert_x = np.zeros_like(recv_x)
    if recv_scale is not None:
        recv_scale = np.ascontiguousarray(recv_scale)
        expert_scale = np.zeros_like(recv_scale)
        scale_bytes = recv_scale.nbytes // R if R else 0
        rs, es = _p(recv_scale), _p(expert_scale)
    else:
        expert_scale, scale_bytes, rs, es = None, 0, None, None
    src_rank = np.zeros(R, dtype=np.int32)
    src_slot = np.zeros(R, dtype=np.int32)
    recv_meta = np.ascontiguousarray(recv_meta, dtype=np.int32)
    lib().orc_shuffle(N, E, T, K, row_bytes, scale_bytes, _p(pl["cnt"]), _p(pl["soff"]),
                      _p(pl["roff"]), _p(pl["G"]), _p(pl["eoff"]), _p(recv_x), rs,
                      _p(recv_meta), _p(expert_x), es, _p(src_rank), _p(src_slot))
    return expert_x, expert_scale, src_rank, src_slot


def expert_standin(expert_x: np.ndarray, expert_scale, eoff: np.ndarray, H: int) -> np.ndarray:
    """Outside the path: y[r] = bf16(value * (e+1)) for row r of expert e."""
    expert_x = np.ascontiguousarray(expert_x)
    R = expert_x.shape[0]
    E = eoff.shape[0] - 1
    y = np.zeros((R, H), dtype=np.uint16)
    fp8 = expert_scale is not None
    sc = _p(np.ascontiguousarray(expert_scale, dtype=np.float32)) if fp8 else None
    lib().orc_expert_standin(E, H, _p(eoff), _p(expert_x), sc, int(fp8), _p(y))
    return y


# ------------------------------------------------- fixed-slot receive layout

def slot_capacity_ok(cnt: np.ndarray, T_max: int) -> bool:
    """Every (sender, expert) count fits its T_max slots."""
    cnt = np.ascontiguousarray(cnt, dtype=np.int32)
    N, E = cnt.shape
    return bool(lib().orc_slot_capacity_ok(N, E, T_max, _p(cnt)))


def slot_rows(idx: np.ndarray, pl: dict, T_max: int) -> np.ndarray:
    """Slot row of every (s,t,k) in the fixed-slot receive layout, int64 [N][T][K]."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    N, T, K = idx.shape
    E = pl["cnt"].shape[1]
    slot = np.zeros((N, T, K), dtype=np.int64)
    lib().orc_slot_rows(N, T, K, E, T_max, _p(idx), _p(pl["soff"]), _p(pl["pos"]), _p(slot))
    return slot


def transfer_slots(send: np.ndarray, pl: dict, slot: np.ndarray, n_slots: int,
                   fill: int = 0) -> np.ndarray:
    """Transfer of one row plane into the fixed-slot receive layout (n_slots
    rows; slots no row names hold `fill`)."""
    send = np.ascontiguousarray(send)
    N, T, K = slot.shape
    recv = np.full((n_slots,) + send.shape[1:], fill, dtype=send.dtype)
    row_bytes = send.nbytes // send.shape[0] if send.shape[0] else 0
    lib().orc_transfer_slots(N, T, K, row_bytes, _p(np.ascontiguousarray(pl["pos"])),
                             _p(np.ascontiguousarray(slot)), _p(send), _p(recv))
    return recv


def shuffle_slots(recv_x: np.ndarray, recv_scale, recv_meta: np.ndarray, pl: dict, T_max: int,
                  R: int):
    """Receive shuffle out of the fixed-slot layout into R expert-order rows."""
    recv_x = np.ascontiguousarray(recv_x)
    N, E = pl["cnt"].shape
    row_bytes = recv_x.nbytes // recv_x.shape[0] if recv_x.shape[0] else 0
    expert_x = np.zeros((R,) + recv_x.shape[1:], dtype=recv_x.dtype)
    if recv_scale is not None:
        recv_scale = np.ascontiguousarray(recv_scale)
        expert_scale = np.zeros((R,) + recv_scale.shape[1:], dtype=recv_scale.dtype)
        scale_bytes = recv_scale.nbytes // recv_scale.shape[0]
        rs, es = _p(recv_scale), _p(expert_scale)
    else:
        expert_scale, scale_bytes, rs, es = None, 0, None, None
    src_rank = np.zeros(R, dtype=np.int32)
    src_slot = np.zeros(R, dtype=np.int32)
    lib().orc_shuffle_slots(N, E, T_max, row_bytes, scale_bytes, _p(pl["cnt"]), _p(pl["eoff"]),
                            _p(recv_x), rs, _p(np.ascontiguousarray(recv_meta, dtype=np.int32)),
                            _p(expert_x), es, _p(src_rank), _p(src_slot))
    return expert_x, expert_scale, src_rank, src_slot


def run_dispatch_fixed(x: np.ndarray, idx: np.ndarray, E: int, T_max: int,
                       fp8: bool = False) -> dict:
    """Every dispatch step with the fixed-slot receive layout: the receive
    planes have N*E*T_max rows (-1 meta words and zero payload where no row
    arrived)."""
    N, T, H = x.shape
    K = idx.shape[2]
    pl = plan(idx, E)
    out = dict(pl)
    out["capacity_ok"] = slot_capacity_ok(pl["cnt"], T_max)
    if not out["capacity_ok"]:
        return out
    if fp8:
        send_x, send_scale, send_meta = pack_fp8(x, pl["pos"])
    else:
        send_x, send_meta = pack_bf16(x, pl["pos"])
        send_scale = None
    slot = slot_rows(idx, pl, T_max)
    n_slots = N * E * T_max
    recv_x = transfer_slots(send_x, pl, slot, n_slots)
    recv_scale = transfer_slots(send_scale, pl, slot, n_slots) if fp8 else None
    recv_meta = transfer_slots(send_meta, pl, slot, n_slots, fill=-1)
    R = N * T * K
    expert_x, expert_scale, src_rank, src_slot = shuffle_slots(recv_x, recv_scale, recv_meta, pl,
                                                               T_max, R)
    out.update(slot=slot, send_x=send_x, send_scale=send_scale, send_meta=send_meta,
               recv_x=recv_x, recv_scale=recv_scale, recv_meta=recv_meta, expert_x=expert_x,
               expert_scale=expert_scale, expert_src_rank=src_rank, expert_src_slot=src_slot)
    return out


def _assert_finite_bf16(a: np.ndarray, what: str):
    """The inputs are finite: every bf16 pattern has an exponent below 0xFF."""
    assert not np.any((np.asarray(a, dtype=np.uint16) & 0x7F80) == 0x7F80), f"non-finite {what}"


def run_dispatch(x: np.ndarray, idx: np.ndarray, E: int, fp8: bool = False) -> dict:
    """Every dispatch step, in the pages' order; returns all buffers."""
    _assert_finite_bf16(x, "tokens")
    N, T, H = x.shape
    K = idx.shape[2]
    pl = plan(idx, E)
    out = dict(pl)
    if fp8:
        send_x, send_scale, send_meta = pack_fp8(x, pl["pos"])
    else:
        send_x, send_meta = pack_bf16(x, pl["pos"])
        send_scale = None
    recv_x = transfer(send_x, pl, T, K)
    recv_scale = transfer(send_scale, pl, T, K) if fp8 else None
    recv_meta = transfer(send_meta, pl, T, K)
    expert_x, expert_scale, src_rank, src_slot = shuffle(recv_x, recv_scale, recv_meta, pl, T, K)
    out.update(send_x=send_x, send_scale=send_scale, send_meta=send_meta, recv_x=recv_x,
               recv_scale=recv_scale, recv_meta=recv_meta, expert_x=expert_x,
               expert_scale=expert_scale, expert_src_rank=src_rank, expert_src_slot=src_slot)
    return out


def combine_send(y: np.ndarray, pl: dict) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.uint16)
    N, E = pl["cnt"].shape
    R = y.shape[0]
    comb_send = np.zeros_like(y)
    row_bytes = y.nbytes // R if R else 0
    lib().orc_combine_send(N, E, row_bytes, _p(pl["cnt"]), _p(pl["soff"]), _p(pl["roff"]),
                           _p(pl["G"]), _p(pl["eoff"]), _p(y), _p(comb_send))
    return comb_send


def combine_transfer(comb_send: np.ndarray, pl: dict, T: int, K: int) -> np.ndarray:
    comb_send = np.ascontiguousarray(comb_send)
    N, E = pl["cnt"].shape
    R = comb_send.shape[0]
    comb_recv = np.zeros_like(comb_send)
    row_bytes = comb_send.nbytes // R if R else 0
    lib().orc_combine_transfer(N, E, T, K, row_bytes, _p(pl["soff"]), _p(pl["roff"]),
                               _p(pl["G"]), _p(comb_send), _p(comb_recv))
    return comb_recv


def combine_recv(comb_recv: np.ndarray, pos: np.ndarray, w: np.ndarray, H: int) -> np.ndarray:
    N, T, K = pos.shape
    w = np.ascontiguousarray(w, dtype=np.float32)
    comb_recv = np.ascontiguousarray(comb_recv, dtype=np.uint16)
    out = np.zeros((N, T, H), dtype=np.uint16)
    lib().orc_combine_recv(N, T, K, H, _p(np.ascontiguousarray(pos)), _p(w), _p(comb_recv),
                           _p(out))
    return out


def combine_recv_f64(comb_recv: np.ndarray, pos: np.ndarray, w: np.ndarray, H: int):
    N, T, K = pos.shape
    w = np.ascontiguousarray(w, dtype=np.float32)
    comb_recv = np.ascontiguousarray(comb_recv, dtype=np.uint16)
    out = np.zeros((N, T, H), dtype=np.float64)
    mag = np.zeros((N, T, H), dtype=np.float64)
    lib().orc_combine_recv_f64(N, T, K, H, _p(np.ascontiguousarray(pos)), _p(w),
                               _p(comb_recv), _p(out), _p(mag))
    return out, mag


def combine_token(rows: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Weighted sum of one token's K returned rows (uint16 [K][H])."""
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    K, H = rows.shape
    w = np.ascontiguousarray(w, dtype=np.float32)
    ptrs = (ctypes.c_void_p * K)(*[rows[k].ctypes.data for k in range(K)])
    out = np.zeros(H, dtype=np.uint16)
    lib().orc_combine_token(K, H, ctypes.cast(ptrs, ctypes.c_void_p), _p(w), _p(out))
    return out


def partial_token(rows: np.ndarray, w: np.ndarray, rank: np.ndarray) -> np.ndarray:
    """One token of the combine with sender-side partial sums: its K returned
    rows (uint16 [K][H]), weights and destination ranks."""
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    K, H = rows.shape
    w = np.ascontiguousarray(w, dtype=np.float32)
    rank = np.ascontiguousarray(rank, dtype=np.int32)
    ptrs = (ctypes.c_void_p * K)(*[rows[k].ctypes.data for k in range(K)])
    out = np.zeros(H, dtype=np.uint16)
    lib().orc_partial_token(K, H, ctypes.cast(ptrs, ctypes.c_void_p), _p(w), _p(rank), _p(out))
    return out


def combine_tokens(y: np.ndarray, rows: np.ndarray, w: np.ndarray) -> np.ndarray:
    """combine_token of many tokens: rows int64 [n][K] index the returned rows
    in y (uint16 [*][H]), w fp32 [n][K] -> out uint16 [n][H]."""
    y = np.ascontiguousarray(y, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, K = rows.shape
    H = y.shape[1]
    assert w.shape == (n, K) and (n == 0 or (rows.min() >= 0 and rows.max() < y.shape[0]))
    out = np.empty((n, H), dtype=np.uint16)
    lib().orc_combine_tokens(n, K, H, _p(rows), _p(w), _p(y), _p(out))
    return out


def partial_tokens(y: np.ndarray, rows: np.ndarray, w: np.ndarray, rank: np.ndarray) -> np.ndarray:
    """partial_token of many tokens (rows int64 [n][K] into y, w fp32 [n][K],
    destination ranks int32 [n][K]) -> out uint16 [n][H]."""
    y = np.ascontiguousarray(y, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    w = np.ascontiguousarray(w, dtype=np.float32)
    rank = np.ascontiguousarray(rank, dtype=np.int32)
    n, K = rows.shape
    H = y.shape[1]
    assert w.shape == (n, K) and rank.shape == (n, K)
    assert n == 0 or (rows.min() >= 0 and rows.max() < y.shape[0])
    out = np.empty((n, H), dtype=np.uint16)
    lib().orc_partial_tokens(n, K, H, _p(rows), _p(w), _p(rank), _p(y), _p(out))
    return out


def run_combine(y: np.ndarray, w: np.ndarray, pl: dict, H: int) -> dict:
    """Every combine step, in order; y is the expert output in expert-row order."""
    _assert_finite_bf16(y, "expert outputs")
    assert np.all(np.isfinite(w)), "non-finite weights"
    N, T, K = pl["pos"].shape
    comb_send = combine_send(y, pl)
    comb_recv = combine_transfer(comb_send, pl, T, K)
    out = combine_recv(comb_recv, pl["pos"], w, H)
    return {"comb_send": comb_send, "comb_recv": comb_recv, "out": out}


# ------------------------------------------ combine with sender-side partial sums

def partial_plan(idx: np.ndarray, E: int) -> dict:
    """Partial-row counts pc[s][d] and the owner-side / token-owner-side row of
    every visited (s,t,d) ([N][T][N], -1 where token (s,t) has no expert on d)."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    N, T, K = idx.shape
    pc = np.zeros((N, N), dtype=np.int32)
    lib().orc_partial_counts(N, T, K, E, _p(idx), _p(pc))
    owner_row = np.zeros((N, T, N), dtype=np.int32)
    token_row = np.zeros((N, T, N), dtype=np.int32)
    lib().orc_partial_rows(N, T, K, E, _p(idx), _p(pc), _p(owner_row), _p(token_row))
    return {"pc": pc, "owner_row": owner_row, "token_row": token_row, "P": int(pc.sum())}


def run_partial_combine(y: np.ndarray, w: np.ndarray, idx: np.ndarray, pl: dict, H: int) -> dict:
    """Combine with sender-side partial sums; y in expert-row order, pl from plan()."""
    _assert_finite_bf16(y, "expert outputs")
    assert np.all(np.isfinite(w)), "non-finite weights"
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    N, T, K = idx.shape
    E = pl["cnt"].shape[1]
    pp = partial_plan(idx, E)
    rows = expert_rows(idx, pl)
    P = pp["P"]
    psend = np.zeros((P, H), dtype=np.uint16)
    precv = np.zeros((P, H), dtype=np.uint16)
    out = np.zeros((N, T, H), dtype=np.uint16)
    y = np.ascontiguousarray(y, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    lib().orc_partial_send(N, T, K, E, H, _p(idx), _p(w), _p(rows), _p(y), _p(pp["owner_row"]),
                           _p(psend))
    lib().orc_partial_transfer(N, T, H, _p(pp["owner_row"]), _p(pp["token_row"]), _p(psend),
                               _p(precv))
    lib().orc_partial_recv(N, T, H, _p(pp["token_row"]), _p(precv), _p(out))
    pp.update(psend=psend, precv=precv, out=out)
    return pp


# ------------------------------------------- threaded forms (P-thread timing)
#
# The same steps with each stage's outer loop (over sender ranks, receiver
# ranks or experts) split into `threads` contiguous ranges, one per thread,
# and a join between stages.  Stages whose loop runs over senders alone are
# called on row slices of their arrays; the cross-rank stages take the
# range of their outer loop.  The arithmetic is the functions' own, so the
# results equal the single-thread forms bit for bit (checked by the tests).
# Used to time the oracle on several host cores.

def _ranges(n: int, parts: int):
    parts = max(1, min(parts, n)) if n > 0 else 1
    step, extra = divmod(n, parts)
    out, a = [], 0
    for i in range(parts):
        b = a + step + (1 if i < extra else 0)
        out.append((a, b))
        a = b
    return out


def _par(pool, n: int, threads: int, fn):
    """fn(a, b) over a split of [0, n) into `threads` ranges; returns the results."""
    return list(pool.map(lambda ab: fn(*ab), _ranges(n, threads)))


def run_dispatch_threads(x: np.ndarray, idx: np.ndarray, E: int, threads: int,
                         fp8: bool = False, pool=None) -> dict:
    """run_dispatch with every stage split over `threads` threads."""
    from concurrent.futures import ThreadPoolExecutor
    own = pool is None
    pool = ThreadPoolExecutor(threads) if own else pool
    try:
        return _run_dispatch_threads(x, idx, E, threads, fp8, pool)
    finally:
        if own:
            pool.shutdown()


def _run_dispatch_threads(x, idx, E, P, fp8, pool):
    _assert_finite_bf16(x, "tokens")
    x = np.ascontiguousarray(x, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    N, T, H = x.shape
    K = idx.shape[2]
    TK = T * K
    L_ = lib()
    cnt = np.empty((N, E), dtype=np.int32)
    soff = np.empty((N, E + 1), dtype=np.int32)
    pos = np.empty((N, T, K), dtype=np.int32)
    bad = _par(pool, N, P, lambda a, b: L_.orc_route_count(b - a, T, K, E, _p(idx[a:b]),
                                                            _p(cnt[a:b])))
    if any(r != 0 for r in bad):
        raise RoutingError("expert id outside [0, E)")
    _par(pool, N, P, lambda a, b: L_.orc_send_offsets(b - a, E, _p(cnt[a:b]), _p(soff[a:b])))
    _par(pool, N, P, lambda a, b: L_.orc_positions(b - a, T, K, E, _p(idx[a:b]), _p(soff[a:b]),
                                                    _p(pos[a:b])))
    roff, G = recv_offsets(soff, N)
    eoff = expert_offsets(cnt)
    R = N * TK
    send_meta = np.zeros(R, dtype=np.int32)
    if fp8:
        send_x = np.zeros((R, H), dtype=np.uint8)
        send_scale = np.zeros((R, H // 128), dtype=np.float32)
        _par(pool, N, P, lambda a, b: L_.orc_pack_fp8(
            b - a, T, K, H, _p(x[a:b]), _p(pos[a:b]), _p(send_x[a * TK:b * TK]),
            _p(send_scale[a * TK:b * TK]), _p(send_meta[a * TK:b * TK])))
    else:
        send_x = np.zeros((R, H), dtype=np.uint16)
        send_scale = None
        _par(pool, N, P, lambda a, b: L_.orc_pack_bf16(
            b - a, T, K, H, _p(x[a:b]), _p(pos[a:b]), _p(send_x[a * TK:b * TK]),
            _p(send_meta[a * TK:b * TK])))

    def xfer(plane):
        recv = np.zeros_like(plane)
        rb = plane.nbytes // R if R else 0
        _par(pool, N, P, lambda a, b: L_.orc_transfer_range(
            N, E, T, K, rb, _p(soff), _p(roff), _p(G), _p(plane), _p(recv), a, b))
        return recv
    recv_x = xfer(send_x)
    recv_scale = xfer(send_scale) if fp8 else None
    recv_meta = xfer(send_meta)
    expert_x = np.zeros_like(recv_x)
    expert_scale = np.zeros_like(recv_scale) if fp8 else None
    src_rank = np.zeros(R, dtype=np.int32)
    src_slot = np.zeros(R, dtype=np.int32)
    rb = recv_x.nbytes // R if R else 0
    sb = recv_scale.nbytes // R if (fp8 and R) else 0
    _par(pool, E, P, lambda a, b: L_.orc_shuffle_range(
        N, E, T, K, rb, sb, _p(cnt), _p(soff), _p(roff), _p(G), _p(eoff), _p(recv_x),
        _p(recv_scale) if fp8 else None, _p(recv_meta), _p(expert_x),
        _p(expert_scale) if fp8 else None, _p(src_rank), _p(src_slot), a, b))
    return {"cnt": cnt, "soff": soff, "pos": pos, "roff": roff, "G": G, "eoff": eoff,
            "send_x": send_x, "send_scale": send_scale, "send_meta": send_meta,
            "recv_x": recv_x, "recv_scale": recv_scale, "recv_meta": recv_meta,
            "expert_x": expert_x, "expert_scale": expert_scale, "expert_src_rank": src_rank,
            "expert_src_slot": src_slot}


def run_combine_threads(y: np.ndarray, w: np.ndarray, pl: dict, H: int, threads: int,
                        pool=None) -> dict:
    """run_combine with every stage split over `threads` threads."""
    from concurrent.futures import ThreadPoolExecutor
    own = pool is None
    pool = ThreadPoolExecutor(threads) if own else pool
    try:
        _assert_finite_bf16(y, "expert outputs")
        assert np.all(np.isfinite(w)), "non-finite weights"
        P = threads
        L_ = lib()
        y = np.ascontiguousarray(y, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        N, T, K = pl["pos"].shape
        E = pl["cnt"].shape[1]
        TK = T * K
        R = y.shape[0]
        rb = y.nbytes // R if R else 0
        comb_send = np.zeros_like(y)
        _par(pool, E, P, lambda a, b: L_.orc_combine_send_range(
            N, E, rb, _p(pl["cnt"]), _p(pl["soff"]), _p(pl["roff"]), _p(pl["G"]),
            _p(pl["eoff"]), _p(y), _p(comb_send), a, b))
        comb_recv = np.zeros_like(y)
        _par(pool, N, P, lambda a, b: L_.orc_combine_transfer_range(
            N, E, T, K, rb, _p(pl["soff"]), _p(pl["roff"]), _p(pl["G"]), _p(comb_send),
            _p(comb_recv), a, b))
        out = np.zeros((N, T, H), dtype=np.uint16)
        pos = np.ascontiguousarray(pl["pos"])
        _par(pool, N, P, lambda a, b: L_.orc_combine_recv(
            b - a, T, K, H, _p(pos[a:b]), _p(w[a:b]), _p(comb_recv[a * TK:b * TK]),
            _p(out[a:b])))
        return {"comb_send": comb_send, "comb_recv": comb_recv, "out": out}
    finally:
        if own:
            pool.shutdown()


def run_partial_combine_threads(y: np.ndarray, w: np.ndarray, idx: np.ndarray, pl: dict, H: int,
                                threads: int, pool=None) -> dict:
    """run_partial_combine with every stage split over `threads` threads."""
    from concurrent.futures import ThreadPoolExecutor
    own = pool is None
    pool = ThreadPoolExecutor(threads) if own else pool
    try:
        _assert_finite_bf16(y, "expert outputs")
        assert np.all(np.isfinite(w)), "non-finite weights"
        P = threads
        L_ = lib()
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        y = np.ascontiguousarray(y, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        N, T, K = idx.shape
        E = pl["cnt"].shape[1]
        pc = np.zeros((N, N), dtype=np.int32)
        _par(pool, N, P, lambda a, b: L_.orc_partial_counts_range(N, T, K, E, _p(idx), _p(pc),
                                                                   a, b))
        owner_row = np.zeros((N, T, N), dtype=np.int32)
        token_row = np.zeros((N, T, N), dtype=np.int32)
        _par(pool, N, P, lambda a, b: L_.orc_partial_rows_range(
            N, T, K, E, _p(idx), _p(pc), _p(owner_row), _p(token_row), a, b))
        rows = np.zeros((N, T, K), dtype=np.int32)
        _par(pool, N, P, lambda a, b: L_.orc_expert_rows_range(
            N, T, K, E, _p(idx), _p(pl["cnt"]), _p(pl["soff"]), _p(pl["pos"]), _p(pl["eoff"]),
            _p(rows), a, b))
        Pn = int(pc.sum())
        psend = np.zeros((Pn, H), dtype=np.uint16)
        precv = np.zeros((Pn, H), dtype=np.uint16)
        out = np.zeros((N, T, H), dtype=np.uint16)
        _par(pool, N, P, lambda a, b: L_.orc_partial_send_range(
            N, T, K, E, H, _p(idx), _p(w), _p(rows), _p(y), _p(owner_row), _p(psend), a, b))
        _par(pool, N, P, lambda a, b: L_.orc_partial_transfer_range(
            N, T, H, _p(owner_row), _p(token_row), _p(psend), _p(precv), a, b))
        _par(pool, N, P, lambda a, b: L_.orc_partial_recv_range(
            N, T, H, _p(token_row), _p(precv), _p(out), a, b))
        return {"pc": pc, "owner_row": owner_row, "token_row": token_row, "P": Pn,
                "psend": psend, "precv": precv, "out": out}
    finally:
        if own:
            pool.shutdown()
