"""Helpers shared by the GPU tests: device copies of seeded inputs, output
buffers, a run of the library through its C ABI, and comparisons with the
oracle (full or on sampled rows)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synthetic
from tensor_gemm_reduce_amd import gemm_rs as gr

SENTINEL = 0x7FC1  # a NaN pattern no kernel ever produces from finite inputs


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def filled(shape, value=SENTINEL) -> torch.Tensor:
    return torch.full(shape, np.array(value, np.uint16).view(np.int16).item(), dtype=torch.int16,
                      device="cuda")


class Buffers:
    """Device inputs and sentinel-filled outputs for one rank."""

    def __init__(self, x, w, peers, S, N):
        self.x = dev(x)
        self.w = dev(w)
        self.peers = [dev(p) for p in peers]
        self.send = [filled((S, N)) for _ in range(7)]
        self.local = filled((S, N))
        self.out = filled((S, N))

    def refill(self):
        for t in self.send + [self.local, self.out]:
            t.fill_(np.array(SENTINEL, np.uint16).view(np.int16).item())


def run(op: gr.GemmRS, b: Buffers, mode=gr.MODE_FUSED, check_status=True):
    op.run(mode, b.x, b.w, b.send, b.peers, b.out, b.local)
    torch.cuda.synchronize()
    if check_status:
        st = op.status()
        assert st == gr.OK, gr.gemm_rs_strerror(st)


def sample_rows(S: int, bm: int, rng, extra=2):
    rows = {0, S - 1, min(bm, S) - 1, min(bm, S - 1)}
    rows |= set(int(r) for r in rng.integers(0, S, size=extra))
    return np.array(sorted(r for r in rows if 0 <= r < S), np.int64)


def oracle_rows(x, w, peers, rank, S, rows):
    """Oracle local-slice rows, per-destination send rows and out rows for the
    given slice rows.  Returns (local[n][N], send[i][n][N], out[n][N])."""
    tp = 8
    send = []
    for i in range(tp - 1):
        d = oracle.peer_rank(rank, i)
        send.append(oracle.f32_to_bf16(oracle.gemm_f32acc(x, w, rows=d * S + rows)))
    local = oracle.f32_to_bf16(oracle.gemm_f32acc(x, w, rows=rank * S + rows))
    out = oracle.slice_sum(local, [p[rows] for p in peers], tp=tp)
    return local, send, out


def max_rel(a_bits: np.ndarray, b_ref: np.ndarray) -> float:
    """max |a - ref| / max |ref| with a given as BF16 bits and ref as floats."""
    a = oracle.bf16_to_f32(a_bits).astype(np.float64)
    ref = np.asarray(b_ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(a - ref)) / den) if den > 0 else float(np.max(np.abs(a - ref)))


def assert_close_partial(gpu_bits, orc_bits, x, w, rows, tol=1e-2):
    """GPU partial rows vs the oracle's: the stated tolerance (max relative
    error <= tol) and, per element, at most one BF16 ulp plus the FP32
    summation-order bound 2*K*u*sum|x||w|."""
    assert not np.any(gpu_bits == SENTINEL), "unwritten elements"
    g = oracle.bf16_to_f32(gpu_bits).astype(np.float64)
    o = oracle.bf16_to_f32(orc_bits).astype(np.float64)
    assert max_rel(gpu_bits, o) <= tol
    K = x.shape[1]
    xa = np.abs(oracle.bf16_to_f32(x[rows]).astype(np.float64))
    wa = np.abs(oracle.bf16_to_f32(w).astype(np.float64))
    absprod = xa @ wa.T
    mag = np.maximum(np.abs(g), np.abs(o))
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 7), 0.0)
    bound = ulp + 2 * K * 2.0 ** -24 * absprod + 1e-30
    bad = np.abs(g - o) > bound
    assert not np.any(bad), f"{int(bad.sum())} elements beyond one ulp + order bound"
