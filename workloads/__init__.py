"""Seeded synthetic inputs for the MoE dispatch/combine path.

This module only draws inputs: token activations, router top-K expert ids and
router weights.  It holds none of the dispatch/combine arithmetic, and both the
CPU oracle and the HIP path are fed from it, so they always see identical
inputs.

Pages cited:
  [EPMC] "Efficient and portable Mixture-of-Experts communication" (Perplexity)
  [EFA]  "Enabling trillion-parameter models on AWS EFA" (Perplexity)

The router is a small linear layer producing a probability distribution; the
top-K experts by score are chosen and their probabilities weight the expert
outputs ([EPMC] "Introduction").  The router itself is outside the path, so here
it is replaced by random logits.  The workload shapes follow the models the
pages name: Mixtral 8x7B and DeepSeek R1 ([EPMC] "Introduction"), hidden size
7168 with 128 decode tokens per GPU, block-scaled fp8 dispatch, DeepSeek-V3 and
Kimi-K2 configurations ([EFA] "Dispatch/combine latency").

Randomness: every (config seed, logical rank, stream) triple gets its own
numpy PCG64 stream, so any one rank's inputs can be regenerated alone (the
large prefill shape is checked by sampling ranks).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

__all__ = ["Config", "CONFIGS", "make_tokens", "make_routing", "make_inputs",
           "bf16_bits_from_f32", "f32_from_bf16_bits", "fp8_exponent_sweep"]

_STREAM_X = 0
_STREAM_ROUTE = 1


@dataclass(frozen=True)
class Config:
    """One synthetic workload: N logical ranks, T tokens per rank, hidden H,
    E experts (E/N per rank), top-K routing, dispatch payload dtype."""
    key: str
    name: str
    N: int
    T: int
    H: int
    E: int
    K: int
    dtype: str          # "bf16" or "fp8" (dispatch payload; combine is bf16)
    routing: str        # softmax | softmax_renorm | zipf | worst | uniform
    seed: int

    @property
    def L(self) -> int:
        return self.E // self.N

    @property
    def rows(self) -> int:
        return self.N * self.T * self.K

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    def describe(self) -> str:
        return (f"{self.name} N={self.N} T={self.T} H={self.H} E={self.E} "
                f"K={self.K} {self.dtype}")


CONFIGS = {
    "A": Config("A", "tiny", 2, 16, 256, 8, 2, "bf16", "softmax", 1),
    "B": Config("B", "mixtral-8x7b-decode", 8, 128, 4096, 8, 2, "bf16",
                "softmax_renorm", 2),
    "C": Config("C", "deepseek-r1-decode", 32, 128, 7168, 256, 8, "bf16",
                "softmax", 3),
    "D": Config("D", "deepseek-r1-prefill-fp8", 64, 2048, 7168, 256, 8, "fp8",
                "softmax", 4),
    "E": Config("E", "kimi-k2-zipf-decode", 64, 128, 7168, 384, 8, "bf16",
                "zipf", 5),
    "Ep": Config("Ep", "kimi-k2-all-to-rank0-decode", 64, 128, 7168, 384, 8,
                 "bf16", "worst", 6),
}


def _rng(seed: int, rank: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, rank, stream])))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even, via torch's
    CPU cast.  Used only to synthesise inputs."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_tokens(cfg: Config, rank: int, T: int | None = None) -> np.ndarray:
    """Token activations of one logical rank: fp32 ~ N(0,1) rounded to bf16,
    returned as uint16 bit patterns of shape [T][H]."""
    T = cfg.T if T is None else T
    g = _rng(cfg.seed, rank, _STREAM_X)
    return bf16_bits_from_f32(g.standard_normal((T, cfg.H), dtype=np.float32))


def _softmax_f32(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float32)
    m = z.max(axis=-1, keepdims=True)
    ez = np.exp(z - m, dtype=np.float32)
    return (ez / ez.sum(axis=-1, keepdims=True, dtype=np.float32)).astype(np.float32)


def _topk_desc(score: np.ndarray, K: int) -> np.ndarray:
    # stable sort of the negated score: equal scores keep the lower expert id first
    return np.argsort(-score, axis=-1, kind="stable")[..., :K].astype(np.int32)


def _routing_one_rank(cfg: Config, rank: int, T: int):
    g = _rng(cfg.seed, rank, _STREAM_ROUTE)
    E, K = cfg.E, cfg.K
    if cfg.routing in ("softmax", "softmax_renorm"):
        probs = _softmax_f32(g.standard_normal((T, E), dtype=np.float32))
        idx = _topk_desc(probs, K)
        w = np.take_along_axis(probs, idx, axis=-1).astype(np.float32)
        if cfg.routing == "softmax_renorm":
            w = (w / w.sum(axis=-1, keepdims=True, dtype=np.float32)).astype(np.float32)
    elif cfg.routing == "zipf":
        # expert popularity p_e ~ (e+1)^-1.2 (expert 0 hottest); K distinct
        # experts per token by Gumbel-top-K on log p_e + Gumbel noise, weights =
        # softmax of the K selected keys.
        logp = (-1.2 * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
        u = g.random((T, E), dtype=np.float64)
        gumbel = (-np.log(-np.log(np.clip(u, 1e-300, 1.0 - 1e-16)))).astype(np.float32)
        keys = (logp[None, :] + gumbel).astype(np.float32)
        idx = _topk_desc(keys, K)
        w = _softmax_f32(np.take_along_axis(keys, idx, axis=-1))
    elif cfg.routing == "worst":
        # every token takes all experts of rank 0 plus K-L distinct experts
        # drawn uniformly from the rest; slot order shuffled per token
        L = cfg.L
        assert K >= L
        idx = np.empty((T, K), dtype=np.int32)
        for t in range(T):
            extra = g.choice(np.arange(L, E), size=K - L, replace=False)
            row = np.concatenate([np.arange(L), extra]).astype(np.int32)
            g.shuffle(row)
            idx[t] = row
        w = _softmax_f32(g.standard_normal((T, K), dtype=np.float32))
    elif cfg.routing == "uniform":
        # ids drawn with replacement: duplicates inside a token are allowed
        idx = g.integers(0, E, size=(T, K), dtype=np.int32)
        w = _softmax_f32(g.standard_normal((T, K), dtype=np.float32))
    else:
        raise ValueError(f"unknown routing {cfg.routing!r}")
    return idx.astype(np.int32), w.astype(np.float32)


def make_routing(cfg: Config, T: int | None = None, ranks=None):
    """Top-K expert ids int32 [n][T][K] and weights fp32 [n][T][K] for the
    given ranks (default: all N)."""
    T = cfg.T if T is None else T
    ranks = list(range(cfg.N) if ranks is None else ranks)
    if T == 0:
        return (np.zeros((len(ranks), 0, cfg.K), dtype=np.int32),
                np.zeros((len(ranks), 0, cfg.K), dtype=np.float32))
    idx, w = [], []
    for r in ranks:
        i, ww = _routing_one_rank(cfg, r, T)
        idx.append(i)
        w.append(ww)
    return np.stack(idx), np.stack(w)


def renormalised(w: np.ndarray) -> np.ndarray:
    """Weights scaled to sum to one per token (fp32)."""
    return (w / w.sum(axis=-1, keepdims=True, dtype=np.float32)).astype(np.float32)


def make_inputs(cfg: Config, T: int | None = None) -> dict:
    """All inputs of one workload: x (uint16 bf16 bits [N][T][H]), idx, w."""
    T = cfg.T if T is None else T
    x = np.stack([make_tokens(cfg, r, T) for r in range(cfg.N)]) if T > 0 else \
        np.zeros((cfg.N, 0, cfg.H), dtype=np.uint16)
    idx, w = make_routing(cfg, T)
    return {"x": x, "idx": idx, "w": w}


def fp8_exponent_sweep(seed: int = 3) -> np.ndarray:
    """Blocks of 128 bf16 values (uint16 patterns, [n][128]) whose largest
    magnitude walks every bf16 exponent: for each biased exponent 0..254 and
    mantissas {0, 1, 0x40, 0x7F} (no zero pattern), two blocks with that
    largest magnitude at a random place and random sign, the other elements
    random patterns of no larger magnitude with random signs -- one block
    with no zeros, one with a quarter of its elements +0 or -0.  Inputs for
    the block-scaled e4m3 codec from the subnormal bf16 range to the largest
    finite value."""
    g = _rng(seed, 0, 2)
    blocks = []
    for ex in range(255):
        for mant in (0, 1, 0x40, 0x7F):
            top = (ex << 7) | mant
            if top == 0:
                continue
            for zeros in (False, True):
                mag = g.integers(1, top + 1, size=128, dtype=np.int64)
                if zeros:
                    z = g.choice(128, size=32, replace=False)
                    mag[z] = 0
                j = int(g.integers(128))
                mag[j] = top
                sign = g.integers(0, 2, size=128, dtype=np.int64) << 15
                blocks.append((mag | sign).astype(np.uint16))
    return np.stack(blocks)
