"""The pack's two orders against the oracle.  A sender whose tokens take at
most 2 MiB (T*H*2 bytes) is packed in send-row order: the route plan names
the item of each send row, and the pack gathers the token rows, one XCD run
per sender; a larger sender is packed in token order (each token read once
and written K times).  Shapes on both sides of the boundary (T = 146 and 147
at H = 7168: 2 093 056 and 2 107 392 bytes), bf16 and e4m3, in every
transport, combine and layout.  N = 12 ends the row order's sender runs in a
ragged tile (12 runs in tiles of 8): bf16 28 032 blocks in runs of 2336,
e4m3 14 016 blocks in runs of 1168."""
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

SIDES = {"row-order": 146, "token-order": 147}
MODES = ["staged", "direct", "staged-partial", "direct-partial", "fixed-staged", "fixed-direct"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("side", list(SIDES))
def test_pack_order(side, dtype, mode):
    T = SIDES[side]
    cfg = Config("O", f"pack-{side}-{dtype}", 12, T, 7168, 48, 8, dtype, "softmax", 41)
    transport = mep.MOE_TRANSPORT_DIRECT if "direct" in mode else mep.MOE_TRANSPORT_STAGED
    say(f"[gpu] pack order {cfg.describe()} {mode}")
    inp = make_inputs(cfg)
    if mode.startswith("fixed"):
        check_fixed(cfg, inp, T, transport)
    elif mode.endswith("partial"):
        check_partial(cfg, inp, run_cycle(torch, mep, cfg, inp, transport=transport,
                                          combine_mode=mep.MOE_COMBINE_PARTIAL))
    else:
        _compare_all(cfg, inp, run_cycle(torch, mep, cfg, inp, transport=transport))
