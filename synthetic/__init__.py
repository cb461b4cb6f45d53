"""Seeded synthetic inputs for one rank's fused GEMM + reduce-scatter.

This module only draws random numbers and stores them as BF16 bit patterns
(``numpy.uint16``); it holds none of the method's arithmetic, so both the
oracle and the HIP path take their inputs from here.

Shapes are the ones the problem page "A fused GEMM + reduce-scatter kernel
hiding 90% of communication on 8 H100 GPUs" asks for in "How it gets verified":
tokens M in {512, 2048, 8192, 32768} and (N, K) of the Llama-3 70B and
Mixtral 8x22B projections, one rank of tensor-parallel degree 8 (K_local = K/8),
plus a tiny case that spans several tiles.  Real weights and activations are not
used: entries are N(0, 1) scaled by 1/sqrt(K) (K the unsharded reduction
length) for both X_r and W_r, and the tp-1 peer partials that stand in for the
other ranks' writes are N(0, 1) ("normal" mode) or have the same spread as a
real partial, 1/sqrt(tp*K) ("balanced" mode).  "integer" mode draws small
integers so that every sum on the path is exact in FP32.

Seeds: seed(cfg, tid) = 20260000 + 100*cfg.index + tid with tid 0 = X,
1 = W and 2..tp = peer slots in ascending peer rank.  Shards of the full
unsharded X, W for a given rank r (used to build consistent peers) use
tid = 50 + 2*r (X) and 51 + 2*r (W).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SEED_BASE = 20260000


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    index: int
    M: int          # tokens (rows of X_r and of the full product)
    N: int          # output features
    K_local: int    # reduction length held by one rank (K / tp)
    tp: int = 8
    description: str = ""

    @property
    def K(self) -> int:
        return self.K_local * self.tp

    @property
    def S(self) -> int:
        return self.M // self.tp

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K_local

    @property
    def reduce_bytes(self) -> int:
        # tp-1 peer slices + the local slice read, one output slice written, BF16
        return (self.tp + 1) * self.S * self.N * 2

    @property
    def gemm_bytes(self) -> int:
        # compulsory: X_r and W_r read once, the M x N partial written once, BF16
        return 2 * (self.M * self.K_local + self.N * self.K_local + self.M * self.N)


CONFIGS = {
    c.name: c
    for c in [
        Config("tiny", 0, 128, 1024, 128,
               description="tiny: M=128 N=1024 K_local=128, spans several tiles"),
        Config("o_proj", 1, 512, 8192, 1024,
               description="Llama-3-70B o_proj row-parallel, one rank of TP=8"),
        Config("down_proj", 2, 2048, 8192, 3584,
               description="Llama-3-70B down_proj, one rank of TP=8"),
        Config("mixtral_down", 3, 8192, 6144, 2048,
               description="Mixtral-8x22B-shaped expert down projection, one rank of TP=8"),
        Config("large_prefill", 4, 32768, 8192, 3584,
               description="large prefill, Llama-3-70B down_proj shape, one rank of TP=8"),
    ]
}


def seed(cfg: Config, tid: int) -> int:
    return SEED_BASE + 100 * cfg.index + tid


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Store float32 samples as BF16 bit patterns (torch's CPU conversion)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _normal(s: int, shape, scale: float) -> np.ndarray:
    rng = np.random.default_rng(s)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return to_bf16_bits(a)


def _ints(s: int, shape, lo: int, hi: int) -> np.ndarray:
    rng = np.random.default_rng(s)
    a = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return to_bf16_bits(a)


def make_inputs(cfg: Config, mode: str = "normal", M: int | None = None):
    """Draw X_r [M][K_local], W_r [N][K_local] and tp-1 peer partials [S][N].

    mode: "normal" (peers N(0,1)), "balanced" (peers with a partial's spread),
    "integer" (x, w in {-2..2}, peers in {-8..8}), "zero_peers" (normal X, W,
    peers all +0), "zero_x" (X all +0, normal W and peers).
    M overrides the row count (for a ragged or reduced case); seeds are unchanged.
    """
    M = cfg.M if M is None else M
    S = M // cfg.tp
    xs = (M, cfg.K_local)
    ws = (cfg.N, cfg.K_local)
    ps = (S, cfg.N)
    scale = 1.0 / math.sqrt(cfg.K)
    if mode == "integer":
        x = _ints(seed(cfg, 0), xs, -2, 2)
        w = _ints(seed(cfg, 1), ws, -2, 2)
        peers = [_ints(seed(cfg, 2 + i), ps, -8, 8) for i in range(cfg.tp - 1)]
        return x, w, peers
    x = _normal(seed(cfg, 0), xs, scale)
    w = _normal(seed(cfg, 1), ws, scale)
    if mode == "normal":
        peers = [_normal(seed(cfg, 2 + i), ps, 1.0) for i in range(cfg.tp - 1)]
    elif mode == "balanced":
        ps_scale = 1.0 / math.sqrt(cfg.tp * cfg.K)
        peers = [_normal(seed(cfg, 2 + i), ps, ps_scale) for i in range(cfg.tp - 1)]
    elif mode == "zero_peers":
        peers = [np.zeros(ps, np.uint16) for _ in range(cfg.tp - 1)]
    elif mode == "zero_x":
        x = np.zeros(xs, np.uint16)
        peers = [_normal(seed(cfg, 2 + i), ps, 1.0) for i in range(cfg.tp - 1)]
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return x, w, peers


def make_shards(cfg: Config, integer: bool = True, M: int | None = None):
    """Shards (X_r, W_r) of one unsharded X [M][K], W [N][K] for every rank r.

    Rank r's shard holds columns [r*K_local, (r+1)*K_local) of the reduction
    dimension.  Used to build peers that are the other ranks' real partials.
    """
    M = cfg.M if M is None else M
    scale = 1.0 / math.sqrt(cfg.K)
    shards = []
    for r in range(cfg.tp):
        if integer:
            x = _ints(seed(cfg, 50 + 2 * r), (M, cfg.K_local), -2, 2)
            w = _ints(seed(cfg, 51 + 2 * r), (cfg.N, cfg.K_local), -2, 2)
        else:
            x = _normal(seed(cfg, 50 + 2 * r), (M, cfg.K_local), scale)
            w = _normal(seed(cfg, 51 + 2 * r), (cfg.N, cfg.K_local), scale)
        shards.append((x, w))
    return shards


def small_case(M: int, N: int, K_local: int, tp: int = 8, mode: str = "normal", s: int = 7):
    """Inputs for an arbitrary small shape (odd sizes, ragged tails) with a fixed seed."""
    cfg = Config(f"case_{M}x{N}x{K_local}", 90 + (s % 9), M, N, K_local, tp)
    return cfg, make_inputs(cfg, mode)


# ---- all-gather + GEMM (the column-parallel layer before the row-parallel one)

@dataclasses.dataclass(frozen=True)
class AgConfig:
    """One rank's share of a column-parallel layer at TP degree tp: the
    gathered activations are M x K (tp row slices of S = M / tp rows), the
    weight shard is N x K (N = this rank's output columns)."""
    name: str
    index: int
    M: int
    N: int
    K: int
    tp: int = 8
    description: str = ""

    @property
    def S(self) -> int:
        return self.M // self.tp

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def gather_bytes(self) -> int:
        # the tp-1 peer slices read and written into the gathered buffer, BF16
        return 2 * (self.tp - 1) * self.S * self.K * 2


# The layers that feed each benchmark shape's row-parallel layer in the same
# model: Llama-3-70B's fused q/k/v projection (64 query and 2 x 8 key/value
# heads of 128: N = 10240 / 8) before o_proj, its fused gate/up projection
# (2 x 28672 / 8) before down_proj, and Mixtral-8x22B's expert w1/w3
# (2 x 16384 / 8) before its down projection.
AG_CONFIGS = {
    c.name: c
    for c in [
        AgConfig("ag_tiny", 10, 128, 512, 256,
                 description="tiny all-gather + GEMM: M=128 N=512 K=256, spans several tiles"),
        AgConfig("ag_qkv", 11, 512, 1280, 8192,
                 description="Llama-3-70B q/k/v projection column-parallel, one rank of TP=8"),
        AgConfig("ag_gate_up", 12, 2048, 7168, 8192,
                 description="Llama-3-70B gate/up projection column-parallel, one rank of TP=8"),
        AgConfig("ag_mixtral_w13", 13, 8192, 4096, 6144,
                 description="Mixtral-8x22B-shaped expert w1/w3 column-parallel, one rank of TP=8"),
        AgConfig("ag_large_prefill", 14, 32768, 7168, 8192,
                 description="large prefill, Llama-3-70B gate/up shape, one rank of TP=8"),
    ]
}


def make_ag_inputs(cfg: AgConfig, mode: str = "normal", M: int | None = None):
    """(x_slices, w): tp row slices [S][K] in source-rank order and this rank's
    column shard [N][K] of the weight.  Normal mode: N(0, 1) / sqrt(K) for
    both; integer mode: uniform in {-2..2}.  Seeds: tid 60 + d for slice d,
    tid 70 for the weight."""
    M = cfg.M if M is None else M
    S = M // cfg.tp
    if mode == "integer":
        xs = [_ints(seed(cfg, 60 + d), (S, cfg.K), -2, 2) for d in range(cfg.tp)]
        w = _ints(seed(cfg, 70), (cfg.N, cfg.K), -2, 2)
    elif mode == "normal":
        scale = 1.0 / math.sqrt(cfg.K)
        xs = [_normal(seed(cfg, 60 + d), (S, cfg.K), scale) for d in range(cfg.tp)]
        w = _normal(seed(cfg, 70), (cfg.N, cfg.K), scale)
    else:
        raise ValueError(mode)
    return xs, w

