"""Python binding of libmoe_ep.so, the MI355X MoE dispatch/combine library.

Argument marshalling only: every call below forwards to the C function of the
same name in include/moe_ep.h (ctypes), passing device pointers and the HIP
stream.  Tensors may be torch tensors (their data_ptr() is passed) or raw
integer device addresses.  A non-zero status raises MoeError.  Torch tensors
are checked before their address is passed (on the group's device, dense,
the expected dtype where one is fixed, at least as many bytes as the call
reads or writes) and a failed check raises MoeError(MOE_ERR_INVALID); raw
addresses are passed unchecked.

The library is built in-tree by ``python combine_moe_dispatch_amd/_build.py``;
importing this package without it raises ImportError -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_EP_LIBRARY selects another build of the same library (same C ABI)
LIB_PATH = os.environ.get("MOE_EP_LIBRARY") or os.path.join(_PKG, "lib", "libmoe_ep.so")

MOE_OK = 0
MOE_ERR_INVALID = -1
MOE_ERR_HIP = -2
MOE_ERR_OOM = -3
MOE_ERR_STATE = -4
MOE_ERR_ROUTING = -5
MOE_ERR_CAPACITY = -6
MOE_ERR_INTERNAL = -7
MOE_ERR_SCRATCH = -8

MOE_SCRATCH_BYTES = 64 << 20

MOE_BF16 = 0
MOE_FP8_E4M3 = 1

MOE_TRANSPORT_STAGED = 0
MOE_TRANSPORT_DIRECT = 1

MOE_COMBINE_RECEIVER = 0
MOE_COMBINE_PARTIAL = 1

MOE_LAYOUT_PACKED = 0
MOE_LAYOUT_FIXED_SLOT = 1

MOE_PROBE_COPY = 0
MOE_PROBE_READ = 1
MOE_PROBE_WRITE = 2

KERNELS = ["route_plan", "pack", "transfer", "shuffle", "combine_pack", "transfer_back",
           "combine_reduce", "combine_push", "partial_send", "partial_transfer",
           "partial_reduce", "recv_map"]
MOE_KERNEL_COUNT = len(KERNELS)
MOE_KERNEL_ALL = (1 << MOE_KERNEL_COUNT) - 1


class moe_group_desc(ctypes.Structure):
    _fields_ = [("num_ranks", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("dispatch_dtype", ctypes.c_int32),
                ("transport", ctypes.c_int32), ("combine_mode", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class moe_group_view(ctypes.Structure):
    _fields_ = [("desc", moe_group_desc), ("num_tokens", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("payload_row_bytes", ctypes.c_int64),
                ("combine_row_bytes", ctypes.c_int64), ("scale_blocks", ctypes.c_int32)] + [
        (name, ctypes.c_void_p) for name in (
            "cnt", "pos", "send_off", "recv_off", "recv_base", "expert_off", "send_x",
            "send_scale", "send_meta", "recv_x", "recv_scale", "recv_meta",
            "expert_src_rank", "expert_src_slot", "comb_send", "comb_recv", "send_w", "recv_w",
            "part_dst", "part_pos", "part_send_off", "part_base", "part_owner_base")] + [
        ("recv_rows", ctypes.c_int64)]


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {strerror(status)} ({status})")


def _load():
    # torch ships its own HIP runtime (soname libamdhip64.so.7); importing it
    # first makes the library bind to that same runtime instead of loading a
    # second one from the ROCm install.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python combine_moe_dispatch_amd/_build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I32, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64
    sig = {
        "moe_group_create": ([ctypes.POINTER(moe_group_desc), ctypes.POINTER(P)], I),
        "moe_group_create_static": ([ctypes.POINTER(moe_group_desc), ctypes.POINTER(P)], I),
        "moe_group_destroy": ([P], I),
        "moe_dispatch_send": ([P, I32, P, P, P, P], I),
        "moe_dispatch_recv": ([P, P, P, P, P], I),
        "moe_combine_send": ([P, P, P], I),
        "moe_combine_recv": ([P, P, P, P], I),
        "moe_group_view_get": ([P, ctypes.POINTER(moe_group_view)], I),
        "moe_group_status": ([P, P], I),
        "moe_group_timing_enable": ([P, I], I),
        "moe_group_timing_read": ([P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)], I),
        "moe_strerror": ([I], ctypes.c_char_p),
        "moe_kernel_name": ([I], ctypes.c_char_p),
        "moe_hbm_probe": ([I, P, P, ctypes.c_size_t, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


# group handle -> (desc, device index), for checking tensor arguments
_groups: dict = {}
_DT_I32, _DT_F32 = "int32", "float32"


def _arg(a, call: str, name: str, nbytes: int, g: int, dtype: str = None):
    """The address of a tensor argument after checking it; raw addresses and
    None pass through."""
    if a is None or isinstance(a, int):
        return _ptr(a)
    info = _groups.get(g)
    bad = None
    if not a.is_cuda:
        bad = "not a device tensor"
    elif info is not None and a.device.index != info[1]:
        bad = f"on device {a.device.index}, the group is on device {info[1]}"
    elif not a.is_contiguous():
        bad = "not contiguous"
    elif dtype is not None and str(a.dtype).rsplit(".", 1)[-1] != dtype:
        bad = f"dtype {a.dtype}, expected {dtype}"
    elif a.numel() * a.element_size() < nbytes:
        bad = f"{a.numel() * a.element_size()} bytes, the call needs {nbytes}"
    if bad is not None:
        raise MoeError(MOE_ERR_INVALID, f"{call}: {name} {bad}")
    return a.data_ptr()


def _shape(g: int):
    """(N, E, K, H, payload bytes per row, scale blocks per row) of a group
    this binding created, else None."""
    info = _groups.get(g)
    if info is None:
        return None
    d = info[0]
    fp8 = d.dispatch_dtype == MOE_FP8_E4M3
    return (d.num_ranks, d.num_experts, d.top_k, d.hidden, d.hidden * (1 if fp8 else 2),
            d.hidden // 128 if fp8 else 0)


def _cur_tokens(g: int) -> int:
    return moe_group_view_get(g).num_tokens if g in _groups else 0


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, call: str):
    if status != MOE_OK:
        raise MoeError(status, call)


def strerror(status: int) -> str:
    return _lib.moe_strerror(status).decode()


def moe_group_create(num_ranks: int, num_experts: int, top_k: int, hidden: int,
                     max_tokens: int, dispatch_dtype: int = MOE_BF16,
                     transport: int = MOE_TRANSPORT_STAGED,
                     combine_mode: int = MOE_COMBINE_RECEIVER,
                     layout: int = MOE_LAYOUT_PACKED) -> int:
    desc = moe_group_desc(num_ranks, num_experts, top_k, hidden, max_tokens, dispatch_dtype,
                          transport, combine_mode, layout)
    h = ctypes.c_void_p()
    _check(_lib.moe_group_create(ctypes.byref(desc), ctypes.byref(h)), "moe_group_create")
    _groups[h.value] = (desc, _current_device())
    return h.value


def moe_group_create_static(num_ranks: int, num_experts: int, top_k: int, hidden: int,
                            max_tokens: int, dispatch_dtype: int = MOE_BF16,
                            transport: int = MOE_TRANSPORT_STAGED,
                            combine_mode: int = MOE_COMBINE_RECEIVER,
                            layout: int = MOE_LAYOUT_PACKED) -> int:
    """A group whose buffers live in the library's static device scratch area
    (no device allocation); one per device at a time."""
    desc = moe_group_desc(num_ranks, num_experts, top_k, hidden, max_tokens, dispatch_dtype,
                          transport, combine_mode, layout)
    h = ctypes.c_void_p()
    _check(_lib.moe_group_create_static(ctypes.byref(desc), ctypes.byref(h)),
           "moe_group_create_static")
    _groups[h.value] = (desc, _current_device())
    return h.value


def _current_device() -> int:
    import torch
    return torch.cuda.current_device()


def moe_group_destroy(g: int) -> None:
    _groups.pop(g, None)
    _check(_lib.moe_group_destroy(g), "moe_group_destroy")


def moe_dispatch_send(g: int, num_tokens: int, x, topk_idx, topk_weights=None,
                      stream=None) -> None:
    c = "moe_dispatch_send"
    sh = _shape(g)
    N, E, K, H = sh[:4] if sh else (0, 0, 0, 0)
    T = max(int(num_tokens), 0)
    px = _arg(x, c, "x", N * T * H * 2, g)
    pi = _arg(topk_idx, c, "topk_idx", N * T * K * 4, g, _DT_I32)
    pw = _arg(topk_weights, c, "topk_weights", N * T * K * 4, g, _DT_F32)
    _check(_lib.moe_dispatch_send(g, num_tokens, px, pi, pw, _stream(stream)), c)


def moe_dispatch_recv(g: int, expert_x, expert_scale, expert_offsets, stream=None) -> None:
    c = "moe_dispatch_recv"
    sh = _shape(g)
    N, E, K, H, pb, nb = sh if sh else (0, 0, 0, 0, 0, 0)
    R = N * _cur_tokens(g) * K
    px = _arg(expert_x, c, "expert_x", R * pb, g)
    ps = _arg(expert_scale, c, "expert_scale", R * nb * 4, g, _DT_F32)
    po = _arg(expert_offsets, c, "expert_offsets", (E + 1) * 4 if sh else 0, g, _DT_I32)
    _check(_lib.moe_dispatch_recv(g, px, ps, po, _stream(stream)), c)


def moe_combine_send(g: int, expert_y, stream=None) -> None:
    c = "moe_combine_send"
    sh = _shape(g)
    N, E, K, H = sh[:4] if sh else (0, 0, 0, 0)
    py = _arg(expert_y, c, "expert_y", N * _cur_tokens(g) * K * H * 2, g)
    _check(_lib.moe_combine_send(g, py, _stream(stream)), c)


def moe_combine_recv(g: int, topk_weights, out, stream=None) -> None:
    c = "moe_combine_recv"
    sh = _shape(g)
    N, E, K, H = sh[:4] if sh else (0, 0, 0, 0)
    T = _cur_tokens(g)
    pw = _arg(topk_weights, c, "topk_weights", N * T * K * 4, g, _DT_F32)
    po = _arg(out, c, "out", N * T * H * 2, g)
    _check(_lib.moe_combine_recv(g, pw, po, _stream(stream)), c)


def moe_group_view_get(g: int) -> moe_group_view:
    v = moe_group_view()
    _check(_lib.moe_group_view_get(g, ctypes.byref(v)), "moe_group_view_get")
    return v


def moe_group_status(g: int, stream=None) -> int:
    """Synchronise and return (not raise) the device-side status."""
    return _lib.moe_group_status(g, _stream(stream))


def moe_group_timing_enable(g: int, kernels=True) -> None:
    """kernels: True (all), False (none), an int bit mask, or kernel names."""
    if kernels is True:
        mask = MOE_KERNEL_ALL
    elif kernels is False or kernels is None:
        mask = 0
    elif isinstance(kernels, int):
        mask = kernels
    else:
        mask = 0
        for name in kernels:
            mask |= 1 << KERNELS.index(name)
    _check(_lib.moe_group_timing_enable(g, mask), "moe_group_timing_enable")


def moe_group_timing_read(g: int) -> dict:
    """{kernel: (total_ms, launches)} for the launches since the last read."""
    ms = (ctypes.c_double * MOE_KERNEL_COUNT)()
    n = (ctypes.c_int64 * MOE_KERNEL_COUNT)()
    _check(_lib.moe_group_timing_read(g, ms, n), "moe_group_timing_read")
    return {KERNELS[i]: (ms[i], n[i]) for i in range(MOE_KERNEL_COUNT)}


def moe_kernel_name(kernel_id: int) -> str:
    return _lib.moe_kernel_name(kernel_id).decode()


def moe_hbm_probe(kind: int, dst, src, nbytes: int, stream=None) -> None:
    """Measurement aid: one streaming copy / read / write kernel of nbytes."""
    _check(_lib.moe_hbm_probe(kind, _ptr(dst), _ptr(src), nbytes, _stream(stream)),
           "moe_hbm_probe")
