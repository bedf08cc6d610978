"""Parity at the hidden sizes where the token kernels (combine reduce, partial
send, partial reduce) change how a row is split over waves: 8 vectors per lane
(4 waves), 9 (8 waves, ragged last part), 16 (8 waves, even), 17 (back to 4
waves, two rounds per wave).  K = 8 takes the compile-time-K kernels, K = 3
the generic one, in both combine modes and both transports."""
import pytest

from tests.gpu_util import run_cycle, say
from tests.test_gpu_parity import _compare_all
from tests.test_gpu_partial import _check as check_partial
from workloads import Config, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402  (fails loudly if the library is missing)

# hidden size -> 16-byte vectors per row -> vectors per lane over one wave
HIDDEN = [4096, 4104, 8192, 8200]   # 512, 513, 1024, 1025 vectors: 8, 9, 16, 17 per lane


@pytest.mark.parametrize("transport", [mep.MOE_TRANSPORT_STAGED, mep.MOE_TRANSPORT_DIRECT])
@pytest.mark.parametrize("K", [8, 3])
@pytest.mark.parametrize("H", HIDDEN)
def test_row_split_boundaries(H, K, transport):
    cfg = Config("S", "row-split", 3, 7, H, 6, K, "bf16", "uniform", 23 + K)
    inp = make_inputs(cfg)
    say(f"[gpu] row split {cfg.describe()} transport={transport} receiver combine")
    _compare_all(cfg, inp, run_cycle(torch, mep, cfg, inp, T_max=9, transport=transport))
    say(f"[gpu] row split {cfg.describe()} transport={transport} partial combine")
    check_partial(cfg, inp, run_cycle(torch, mep, cfg, inp, T_max=9, transport=transport,
                                      combine_mode=mep.MOE_COMBINE_PARTIAL))
