"""Parity at the limits the header declares: 1024 ranks, 1024 experts, top-64,
hidden 65536, in every combine mode and layout.  These reach code paths the
workload shapes do not: two-wave ranking chunks (E > 512), several rounds of
offset columns and multi-batch column walks (N > 32), the token kernels'
generic-K form, and the widest row shapes."""
import numpy as np
import pytest

from tests.gpu_util import run_cycle, say
from tests.test_gpu_fixed_slot import _check as check_fixed
from tests.test_gpu_parity import _compare_all
from tests.test_gpu_partial import _check as check_partial
from workloads import Config, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402

LIMIT_SHAPES = [
    # name, N, T, H, E, K, dtype, routing
    ("max-ranks-experts-topk", 1024, 2, 8, 1024, 64, "bf16", "uniform"),
    ("max-experts-one-rank", 1, 40, 64, 1024, 8, "bf16", "softmax"),
    ("max-topk-few-ranks", 2, 9, 24, 8, 64, "bf16", "uniform"),
    ("max-hidden", 2, 3, 65536, 4, 2, "bf16", "softmax"),
    ("max-hidden-fp8", 2, 3, 65536, 4, 2, "fp8", "softmax"),
]


@pytest.mark.parametrize("transport", [0, 1])
@pytest.mark.parametrize("shape", LIMIT_SHAPES, ids=[s[0] for s in LIMIT_SHAPES])
def test_limits_receiver_combine(shape, transport):
    name, N, T, H, E, K, dt, routing = shape
    cfg = Config("L", name, N, T, H, E, K, dt, routing, 17)
    say(f"[gpu] limits {cfg.describe()} transport={transport}")
    inp = make_inputs(cfg)
    _compare_all(cfg, inp, run_cycle(torch, mep, cfg, inp, transport=transport))


@pytest.mark.parametrize("transport", [0, 1])
@pytest.mark.parametrize("shape", LIMIT_SHAPES[:3], ids=[s[0] for s in LIMIT_SHAPES[:3]])
def test_limits_partial_combine(shape, transport):
    name, N, T, H, E, K, dt, routing = shape
    cfg = Config("L", name, N, T, H, E, K, dt, routing, 18)
    say(f"[gpu] limits partial {cfg.describe()} transport={transport}")
    inp = make_inputs(cfg)
    check_partial(cfg, inp, run_cycle(torch, mep, cfg, inp, transport=transport,
                                      combine_mode=mep.MOE_COMBINE_PARTIAL))


@pytest.mark.parametrize("transport", [0, 1])
def test_limits_fixed_slot(transport):
    """1024 ranks and experts, top-64 with distinct ids: 1024*1024*2 slots."""
    N, T, H, E, K = 1024, 2, 8, 1024, 64
    cfg = Config("L", "max-fixed-slot", N, T, H, E, K, "bf16", "softmax", 19)
    say(f"[gpu] limits fixed-slot {cfg.describe()} transport={transport}")
    check_fixed(cfg, make_inputs(cfg), T, transport)
