"""Parity where the XCD-run block remap ends in a ragged tile.  The movers
hand each XCD runs of consecutive blocks (grids of 8192 blocks and more); a
last tile shorter than 8 runs keeps plain order.  The standard workloads all
have power-of-two grids, so these shapes are chosen to end every remapped
grid in a partial tile:

  N=30, T=137, H=7168, E=240, K=8 (bf16): 32 880 rows; shuffle, combine pack
  and combine push 65 760 blocks in tiles of 1024 (64.2 tiles); transfers in
  segments of 36 rows, tiles of 576 blocks (114.2); combine reduce 8220
  blocks in tiles of 256 (32.1); partial transfer segments of 72 blocks,
  tiles of 576 (114.2).
  N=64, T=131, H=7168, E=256, K=8 (fp8): shuffle 67 072 blocks in tiles of
  1024 (65.5); combine reduce 16 768 blocks in tiles of 256 (65.5).
The pack runs in send-row order here (a sender's tokens within 2 MiB), in
runs of one sender: bf16 65 760 blocks in tiles of 17 536 (3.75); its fp8
grid is 8 whole tiles (ragged sender runs: test_gpu_pack_order.py)."""
import pytest

from tests.gpu_util import run_cycle, say
from tests.test_gpu_parity import _compare_all
from tests.test_gpu_partial import _check as check_partial
from workloads import Config, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402

BF16 = Config("G", "ragged-tiles-bf16", 30, 137, 7168, 240, 8, "bf16", "softmax", 61)
FP8 = Config("G", "ragged-tiles-fp8", 64, 131, 7168, 256, 8, "fp8", "softmax", 62)


@pytest.mark.parametrize("transport", [0, 1])
def test_ragged_tiles_receiver_combine(transport):
    say(f"[gpu] ragged tiles {BF16.describe()} transport={transport}")
    inp = make_inputs(BF16)
    _compare_all(BF16, inp, run_cycle(torch, mep, BF16, inp, transport=transport))


@pytest.mark.parametrize("transport", [0, 1])
def test_ragged_tiles_partial_combine(transport):
    say(f"[gpu] ragged tiles partial {BF16.describe()} transport={transport}")
    inp = make_inputs(BF16)
    check_partial(BF16, inp, run_cycle(torch, mep, BF16, inp, transport=transport,
                                       combine_mode=mep.MOE_COMBINE_PARTIAL))


@pytest.mark.parametrize("transport", [0, 1])
def test_ragged_tiles_fp8(transport):
    say(f"[gpu] ragged tiles {FP8.describe()} transport={transport}")
    inp = make_inputs(FP8)
    _compare_all(FP8, inp, run_cycle(torch, mep, FP8, inp, transport=transport))
