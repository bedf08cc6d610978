"""The C-ABI library loads and exports every function include/moe_ep.h
declares; host-side validation that needs no GPU answers as documented."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ep.h")
LIB = os.path.join(ROOT, "combine_moe_dispatch_amd", "lib", "libmoe_ep.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("moe_dispatch_send", "moe_dispatch_recv", "moe_combine_send", "moe_combine_recv",
              "moe_group_create", "moe_group_destroy"):
        assert n in names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built")
    return ctypes.CDLL(LIB)


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_strerror_and_kernel_names(lib):
    lib.moe_strerror.restype = ctypes.c_char_p
    lib.moe_kernel_name.restype = ctypes.c_char_p
    assert lib.moe_strerror(0) == b"ok"
    assert lib.moe_strerror(-5).startswith(b"expert id")
    assert lib.moe_strerror(12345) == b"unknown status"
    assert lib.moe_kernel_name(0) == b"route_plan_kernel"
    assert lib.moe_kernel_name(6) == b"combine_reduce_kernel"
    assert lib.moe_kernel_name(7) == b"combine_push_kernel"
    assert lib.moe_kernel_name(8) == b"partial_send_kernel"
    assert lib.moe_kernel_name(10) == b"partial_reduce_kernel"
    assert lib.moe_kernel_name(11) == b"recv_map_kernel"
    assert lib.moe_kernel_name(12) == b""


def test_host_validation_without_gpu(lib):
    import combine_moe_dispatch_amd as mep
    # descriptor checks happen before any HIP call
    for args in [(2, 7, 2, 256, 16, 0), (0, 8, 2, 256, 16, 0), (2, 8, 2, 100, 16, 0),
                 (2, 8, 2, 264, 16, 1), (2, 8, 65, 256, 16, 0), (2, 8, 2, 256, 16, 0, 2),
                 (2, 8, 2, 256, 16, 0, 0, 2), (2, 8, 2, 256, 16, 0, 0, 0, 2),
                 # fixed-slot layout: N*E*T_max slots must stay below 2^31
                 (1024, 1024, 1, 8, 2048, 0, 0, 0, 1)]:
        with pytest.raises(mep.MoeError) as ei:
            mep.moe_group_create(*args)
        assert ei.value.status == mep.MOE_ERR_INVALID
    # a null group handle is rejected by every call
    assert lib.moe_dispatch_send(None, 1, None, None, None, None) == mep.MOE_ERR_INVALID
    assert lib.moe_group_timing_enable(None, 1) == mep.MOE_ERR_INVALID
    assert lib.moe_group_status(None, None) == mep.MOE_ERR_INVALID
    assert lib.moe_group_destroy(None) == 0


def test_probe_validation_without_gpu(lib):
    """The measurement probes reject bad arguments before any HIP call."""
    import combine_moe_dispatch_amd as mep
    P = ctypes.c_void_p
    lib.moe_hbm_probe.argtypes = [ctypes.c_int, P, P, ctypes.c_size_t, P]
    for kind, dst, src, n in [(3, 16, 16, 16), (0, 16, 16, 0), (0, 16, 16, 24), (0, 0, 16, 16),
                              (0, 16, 0, 16), (1, 16, 8, 16), (2, 8, 0, 16), (-1, 16, 16, 16)]:
        assert lib.moe_hbm_probe(kind, dst, src, n, None) == mep.MOE_ERR_INVALID, (kind, dst, src, n)
