"""fp8-e4m3 dispatch on the GPU against the oracle's codec on crafted rows:
every bf16 value of magnitude <= 448 quantised with scale 1 (so every e4m3
code, every midpoint and every tie), blocks with awkward scales, all-zero and
signed-zero blocks, blocks whose largest magnitude is tiny, and blocks whose
largest magnitude walks every bf16 exponent.  Besides equality with the
oracle, every block is held to the codec's own properties (tests/fp8_checks.py:
no NaN code, a normal scale, torch's e4m3 rounding of x * inv, the
dequantisation bound)."""
import numpy as np
import pytest

import oracle
from tests.fp8_checks import check_blocks
from tests.gpu_util import run_cycle, say
from workloads import Config, bf16_bits_from_f32, fp8_exponent_sweep

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_moe_dispatch_amd as mep  # noqa: E402

H = 7168
BLK = 128


def _crafted_rows() -> np.ndarray:
    blocks = []
    # every bf16 pattern with |v| <= 448, 127 per block next to a 448 (inv = 1)
    mags = np.arange(0, 0x43E1, dtype=np.uint16)
    vals = np.concatenate([mags, mags | 0x8000])
    for i in range(0, vals.size, BLK - 1):
        chunk = vals[i:i + BLK - 1]
        blk = np.full(BLK, 0, dtype=np.uint16)
        blk[0] = 0x43E0                               # 448.0
        blk[1:1 + chunk.size] = chunk
        blocks.append(blk)
    g = np.random.default_rng(7)
    # awkward amax values: x * (448 / amax) rounds in fp32 before the encode
    for amax in (1.0, 3.0, 0.1, 1e-3, 1234.5, 65504.0, 3e38, 1e-30, 2.0 ** -120):
        v = (g.standard_normal(BLK) * amax / 3).astype(np.float32)
        v[5] = amax
        blocks.append(bf16_bits_from_f32(v))
    blocks.append(np.zeros(BLK, dtype=np.uint16))                   # all zero
    blocks.append(np.full(BLK, 0x8000, dtype=np.uint16))            # all -0
    tiny = np.zeros(BLK, dtype=np.uint16)
    tiny[3] = 0x0001                                                  # amax subnormal
    tiny[9] = 0x8001
    blocks.append(tiny)
    blocks.extend(fp8_exponent_sweep())
    rows = np.concatenate(blocks)
    n_rows = -(-rows.size // H)
    pad = np.zeros(n_rows * H - rows.size, dtype=np.uint16)
    return np.concatenate([rows, pad]).reshape(n_rows, H)


def test_fp8_encode_exhaustive_on_crafted_rows():
    rows = _crafted_rows()
    T = rows.shape[0]
    # one rank, one expert, top-1: expert rows are the tokens in order
    cfg = Config("X", "fp8-crafted", 1, T, H, 1, 1, "fp8", "uniform", 0)
    say(f"[gpu] fp8 crafted rows {cfg.describe()}")
    inp = {"x": rows[None], "idx": np.zeros((1, T, 1), dtype=np.int32),
           "w": np.ones((1, T, 1), dtype=np.float32)}
    gpu = run_cycle(torch, mep, cfg, inp)
    for t in range(T):
        q, sc = oracle.quant_row_fp8(rows[t])
        bad = np.nonzero(gpu["expert_x"][t] != q)[0]
        assert bad.size == 0, (t, bad[:5], rows[t][bad[:5]], gpu["expert_x"][t][bad[:5]], q[bad[:5]])
        assert np.array_equal(gpu["expert_scale"][t].view(np.uint32), sc.view(np.uint32)), t
    check_blocks(rows.reshape(-1, BLK), gpu["expert_x"].reshape(-1, BLK),
                 gpu["expert_scale"].reshape(-1), "gpu")
