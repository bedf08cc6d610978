"""Pins of the oracle's bf16 and fp8-e4m3 codecs against definitions that do
not come from the oracle: the OCP E4M3 format written out as closed forms,
torch's own CPU casts (a library routine), and tie/saturation cases."""
import numpy as np
import pytest
import torch

import oracle


def _e4m3_closed_form(code: int) -> float:
    # OCP 8-bit FP E4M3: exponent bias 7, 3 mantissa bits, S.1111.111 = NaN
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (8 + m) * 2.0 ** (e - 10)


def test_e4m3_value_table_all_codes():
    for c in range(256):
        a, b = oracle.e4m3_value(c), _e4m3_closed_form(c)
        if np.isnan(b):
            assert np.isnan(a), c
        else:
            assert a == b, (c, a, b)
    # landmarks of the format
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_round_trip_every_finite_code():
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = np.array([_e4m3_closed_form(c) for c in codes], dtype=np.float32)
    vals[codes.index(0x80)] = -0.0
    got = oracle.f32_to_e4m3(vals)
    assert list(got) == codes


def test_e4m3_midpoints_tie_to_even():
    pos = [c for c in range(0x7F)]
    for c in pos[:-1]:
        lo, hi = _e4m3_closed_form(c), _e4m3_closed_form(c + 1)
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2          # exactly representable
        even = c if c % 2 == 0 else c + 1
        assert oracle.f32_to_e4m3(np.array([mid]))[0] == even
        assert oracle.f32_to_e4m3(np.array([-mid]))[0] == even | 0x80
        # just off the midpoint goes to the nearer code
        up = np.nextafter(mid, np.float32(np.inf), dtype=np.float32)
        dn = np.nextafter(mid, np.float32(0), dtype=np.float32)
        assert oracle.f32_to_e4m3(np.array([up]))[0] == c + 1
        assert oracle.f32_to_e4m3(np.array([dn]))[0] == c


def test_e4m3_saturation_and_specials():
    v = np.array([448, 449, 463.9, 464, 465, 480, 1e6, np.inf, -np.inf, -500, np.nan],
                 dtype=np.float32)
    got = oracle.f32_to_e4m3(v)
    assert list(got[:8]) == [0x7E] * 8
    assert got[8] == 0xFE and got[9] == 0xFE
    assert got[10] & 0x7F == 0x7F


def test_e4m3_matches_torch_cast_below_saturation():
    # torch.float8_e4m3fn is round-to-nearest-even and agrees with the format
    # up to 464 (above that torch gives NaN where the oracle saturates).
    g = np.random.default_rng(0)
    parts = [
        g.standard_normal(200_000).astype(np.float32) * 30,
        (g.random(200_000) * 2 - 1).astype(np.float32) * 463.9,
        (g.random(100_000) * 2 - 1).astype(np.float32) * 2.0 ** -6,   # subnormal range
        (g.random(100_000) * 2 - 1).astype(np.float32) * 2.0 ** -9,   # around the smallest code
    ]
    # every midpoint and its neighbours
    vals = np.array([_e4m3_closed_form(c) for c in range(0x7F)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    parts += [mids, -mids, np.nextafter(mids, np.float32(np.inf)),
              np.nextafter(mids, np.float32(0))]
    x = np.concatenate(parts).astype(np.float32)
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.f32_to_e4m3(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_bf16_matches_torch_cast():
    g = np.random.default_rng(1)
    bits = g.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # ties: low 16 bits exactly 0x8000, both parities
    ties = ((g.integers(0, 2 ** 16, 50_000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties, g.standard_normal(100_000).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_bf16_overflow_to_inf_and_exact_values():
    big = np.float32(3.4028235e38)           # FLT_MAX rounds up to +inf in bf16
    assert oracle.f32_to_bf16(np.array([big]))[0] == 0x7F80
    assert oracle.f32_to_bf16(np.array([-big]))[0] == 0xFF80
    assert oracle.f32_to_bf16(np.array([1.0], np.float32))[0] == 0x3F80
    assert oracle.f32_to_bf16(np.array([-0.0], np.float32))[0] == 0x8000
    for b in (0x0001, 0x3F80, 0x7F7F, 0xC0A0):
        assert oracle.bf16_to_f32(b) == np.array([b << 16], np.uint32).view(np.float32)[0]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quant_row_fp8_definition(seed):
    """Block-scaled quantisation: the block's largest magnitude maps to 448
    exactly, scale = amax/448, and the dequantised value is within the e4m3
    rounding bound of the input (2^-4 relative in the normal range, half the
    smallest step times the scale below it)."""
    g = np.random.default_rng(seed)
    H = 1024
    xf = (g.standard_normal(H) * np.exp(g.standard_normal(H))).astype(np.float32)
    xf[128:256] = 0.0                                     # an all-zero block
    xb = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    x = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q, sc = oracle.quant_row_fp8(xb)
    vals = np.array([_e4m3_closed_form(int(c)) for c in q])
    for b in range(H // 128):
        blk = x[b * 128:(b + 1) * 128]
        amax = np.abs(blk).max()
        if amax == 0:
            assert sc[b] == 1.0
            assert np.all((q[b * 128:(b + 1) * 128] & 0x7F) == 0)
            continue
        assert sc[b] == np.float32(np.float32(amax) / np.float32(448.0))
        j = int(np.argmax(np.abs(blk)))
        assert q[b * 128 + j] & 0x7F == 0x7E
        deq = vals[b * 128:(b + 1) * 128] * float(sc[b])
        err = np.abs(deq - blk)
        # e4m3 rounding (half a step) plus four fp32 roundings (x*inv, q*scale
        # and the two divisions), each at most 2^-24 relative
        bound = (np.maximum(np.abs(blk) * 2.0 ** -4, 2.0 ** -10 * float(sc[b])) * (1 + 2.0 ** -16)
                 + 2.0 ** -21 * np.abs(blk))
        assert np.all(err <= bound), (b, err.max())


def test_hand_worked_fp8_block():
    """The block-scaled e4m3 row of the hand-worked example
    (tests/golden/tiny_hand_example.json, "fp8_block"), derived on paper."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "tiny_hand_example.json")))["fp8_block"]
    x = np.zeros(g["H"], dtype=np.uint16)
    for i, v in g["x_nonzero_bf16"].items():
        x[int(i)] = v
    codes, scales = oracle.quant_row_fp8(x)
    want = np.zeros(g["H"], dtype=np.uint8)
    for i, v in g["codes_nonzero"].items():
        want[int(i)] = v
    assert codes.tolist() == want.tolist()
    assert scales.view(np.uint32).tolist() == g["scale_bits"]


def test_quant_row_fp8_total_over_every_bf16_exponent():
    """Blocks whose largest magnitude walks every bf16 exponent, subnormal
    bf16 values included, with and without +-0 elements: no NaN code, a
    finite normal scale, codes equal to torch's e4m3 rounding of x * inv
    under the block rule (the scale held at 2^-126 below amax = 448 * 2^-126),
    and the dequantisation bound (tests/fp8_checks.py, which uses no oracle
    code)."""
    from tests.fp8_checks import CLAMP_BELOW, check_blocks
    from workloads import f32_from_bf16_bits, fp8_exponent_sweep
    blocks = fp8_exponent_sweep()
    q, sc = oracle.quant_row_fp8(blocks.reshape(-1))
    check_blocks(blocks, q.reshape(-1, 128), sc, "oracle")
    amax = np.abs(f32_from_bf16_bits(blocks)).max(axis=1)
    # both regimes are reached, the clamped one from many exponents
    assert (amax < CLAMP_BELOW).sum() >= 2 * 3 * 10 and (amax >= CLAMP_BELOW).sum() > 1000


def test_quant_row_fp8_small_amax_regime_by_hand():
    """Blocks below amax = 448 * 2^-126, worked by hand: the scale is
    2^-126 and each code is the e4m3 value of x * 2^126 (exact).  A block with
    largest magnitude 2^-120 (x * 2^126 = 64 = 2^6: exponent field 6 + 7 = 13,
    code 0x68; 2^-121 -> 32: field 12, code 0x60; -0 -> 0x80) and one of
    subnormal bf16 values (pattern 0x0001 = 2^-133 -> 2^-7 = 4 * 2^-9, an e4m3
    subnormal: code 0x04; -2^-133 -> 0x84; pattern 0x0003 = 3 * 2^-133 ->
    3 * 2^-7 = 1.5 * 2^-6: field 1, mantissa 4, code 0x0C)."""
    x = np.zeros(256, dtype=np.uint16)
    x[0] = 0x0380            # 2^-120: exponent field 7 -> 2^(7-127)
    x[1] = 0x0300            # 2^-121
    x[2] = 0x8000            # -0
    x[128 + 0] = 0x0001
    x[128 + 1] = 0x8001
    x[128 + 2] = 0x0003
    q, sc = oracle.quant_row_fp8(x)
    assert sc.view(np.uint32).tolist() == [0x00800000, 0x00800000]     # 2^-126 both
    assert q[:3].tolist() == [0x68, 0x60, 0x80]
    assert np.all(q[3:128] == 0)
    assert q[128:131].tolist() == [0x04, 0x84, 0x0C]
    assert np.all(q[131:] == 0)


def test_quant_rows_fp8_is_the_row_form_per_row():
    from workloads import fp8_exponent_sweep
    x = fp8_exponent_sweep()[:448].reshape(8, 7168)
    q, sc = oracle.quant_rows_fp8(x)
    for i in range(8):
        q1, s1 = oracle.quant_row_fp8(x[i])
        assert np.array_equal(q[i], q1) and np.array_equal(sc[i].view(np.uint32), s1.view(np.uint32))
