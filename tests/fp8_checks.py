"""Checks of block-scaled e4m3 quantisation that do not use the oracle.

Shared by the CPU pin of the oracle's codec and the GPU test of the pack
kernel.  The block rule checked here (128 elements, one fp32 scale; [EFA]
"Dispatch/combine latency": block-scaled fp8 dispatch):

  amax = max |x| over the block (exact in fp32, x is bf16)
  amax >= 448 * 2^-126:    inv = fp32(448 / amax), scale = fp32(amax / 448)
  0 < amax < 448 * 2^-126: inv = 2^126,             scale = 2^-126
  amax == 0:               inv = 0,                 scale = 1
  code = e4m3_rne_saturating(fp32(x * inv))

The e4m3 rounding is torch's own float8_e4m3fn cast (round to nearest even;
it agrees with the OCP format below 464, and |x * inv| never reaches 464
here), and code values come from the format's closed form.  Beyond the exact
codes, every block is held to the dequantisation bound: |x - value(code) *
scale| <= 2^-4 |x| where the scaled value is an e4m3 normal number, and
<= 2^-10 * scale below that (half the smallest e4m3 step), up to the fp32
roundings of the divisions and of x * inv.
"""
from __future__ import annotations

import numpy as np
import torch

MIN_NORMAL = 2.0 ** -126
CLAMP_BELOW = 448.0 * MIN_NORMAL


def e4m3_values() -> np.ndarray:
    """Value of each of the 256 e4m3 codes (OCP E4M3: bias 7, 3 mantissa
    bits, S.1111.111 = NaN), as float64."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = s * m * 2.0 ** -9
        else:
            out[c] = s * (8 + m) * 2.0 ** (e - 10)
    return out


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def check_blocks(x_bits: np.ndarray, q: np.ndarray, sc: np.ndarray, what: str = "") -> None:
    """x_bits uint16 [nb][128] bf16 patterns (finite), q uint8 [nb][128] codes,
    sc float32 [nb] scales, as produced by a block quantiser under test."""
    x_bits = np.asarray(x_bits, dtype=np.uint16).reshape(-1, 128)
    q = np.asarray(q, dtype=np.uint8).reshape(-1, 128)
    sc = np.asarray(sc, dtype=np.float32).reshape(-1)
    nb = x_bits.shape[0]
    assert q.shape == (nb, 128) and sc.shape == (nb,)
    x32 = (x_bits.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isfinite(x32)), "inputs must be finite"
    # every code is a number, every scale finite and normal (or 1 for a zero block)
    nan_code = (q & 0x7F) == 0x7F
    assert not nan_code.any(), (what, "NaN code", np.argwhere(nan_code)[:5])
    assert np.all(np.isfinite(sc)) and np.all(sc >= MIN_NORMAL), (what, "scale", sc[sc < MIN_NORMAL][:5])

    amax = np.abs(x32).max(axis=1)                                   # fp32, exact
    zero = amax == 0
    clamp = (amax > 0) & (amax < np.float32(CLAMP_BELOW))
    normal = amax >= np.float32(CLAMP_BELOW)
    assert np.all(sc[zero] == 1.0), what
    assert np.all(sc[clamp] == np.float32(MIN_NORMAL)), what
    with np.errstate(divide="ignore"):
        want_sc = (amax / np.float32(448.0)).astype(np.float32)
        inv = np.where(normal, np.float32(448.0) / np.where(normal, amax, 1), 0).astype(np.float32)
    inv[clamp] = np.float32(2.0 ** 126)
    assert np.all(sc[normal] == want_sc[normal]), what

    # the exact codes: torch's e4m3 rounding of the fp32 product
    prod = (x32 * inv[:, None]).astype(np.float32)
    assert np.all(np.abs(prod) < 464)
    want_q = _torch_e4m3(prod).reshape(nb, 128)
    bad = np.argwhere(want_q != q)
    assert bad.size == 0, (what, "codes", bad[:5], q[tuple(bad[:5].T)], want_q[tuple(bad[:5].T)])
    # the largest magnitude of a normal-regime block codes to +-448
    j = np.abs(x32).argmax(axis=1)
    top = q[np.arange(nb), j] & 0x7F
    assert np.all(top[normal] == 0x7E), what

    # the dequantisation bound (float64 arithmetic, exact for these values)
    x = x32.astype(np.float64)
    deq = e4m3_values()[q] * sc.astype(np.float64)[:, None]
    err = np.abs(deq - x)
    s64 = sc.astype(np.float64)[:, None]
    e4m3_half_step = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s64)
    # normal regime: four fp32 roundings (the two divisions, x*inv, q*scale),
    # each at most 2^-24 relative; clamped regime: x*inv and q*scale are exact
    slack = np.where(normal[:, None], 1 + 2.0 ** -16, 1.0)
    rel = np.where(normal[:, None], 2.0 ** -21, 0.0)
    bound = e4m3_half_step * slack + rel * np.abs(x)
    over = np.argwhere(err > bound)
    assert over.size == 0, (what, "bound", over[:5], err[tuple(over[:5].T)], bound[tuple(over[:5].T)])
