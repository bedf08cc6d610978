"""Stand-in for the grouped-GEMM expert between dispatch and combine.

Outside the dispatch/combine path and never timed: it only gives combine a
deterministic input, y[r] = bf16(value * (e+1)) for expert-order row r of
expert e, where value is the bf16 payload or, for e4m3 dispatch, the code's
value times its block scale.  torch elementwise ops on the GPU.
"""
from __future__ import annotations


def e4m3_lut(torch):
    """fp32 value of every e4m3 code, from the format's closed form."""
    vals = []
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            vals.append(float("nan"))
        elif e == 0:
            vals.append(s * m * 2.0 ** -9)
        else:
            vals.append(s * (8 + m) * 2.0 ** (e - 10))
    return torch.tensor(vals, dtype=torch.float32, device="cuda")


def standin_expert(torch, expert_x, expert_scale, expert_offsets, E, H, fp8):
    """Outside the path: y[r] = bf16(value * (e+1)) for row r of expert e
    (value = bf16 payload, or e4m3 value * block scale).  expert_x: uint8
    device tensor holding the rows' bytes; expert_scale: fp32 device tensor
    (e4m3 only)."""
    counts = (expert_offsets[1:] - expert_offsets[:-1]).long()
    factor = torch.repeat_interleave(torch.arange(1, E + 1, device="cuda", dtype=torch.float32),
                                     counts)
    R = int(counts.sum().item())
    raw = expert_x.reshape(-1).view(torch.uint8)
    if fp8:
        lut = e4m3_lut(torch)
        codes = raw[:R * H].reshape(R, H).long()
        scale = expert_scale.reshape(-1)[:R * (H // 128)].reshape(R, H // 128)
        v = lut[codes] * scale.repeat_interleave(128, dim=1)
    else:
        v = raw[:R * 2 * H].view(torch.bfloat16).reshape(R, H).float()
    return (v * factor[:, None]).to(torch.bfloat16)
