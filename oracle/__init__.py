"""CPU oracle for one rank's fused BF16 GEMM + reduce-scatter (row-parallel linear).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
``cpu_baseline`` leg use this package; the product library never imports,
links or calls it, and it shares no code with the HIP implementation.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc by
``oracle.build``); this module only marshals numpy arrays.  BF16 arrays are
passed as ``numpy.uint16`` bit patterns.

What is computed follows the problem page "A fused GEMM + reduce-scatter
kernel hiding 90% of communication on 8 H100 GPUs" ("What is asked", "How it
gets verified"): the local partial product X_r * W_r in BF16 with FP32
accumulation, its row slices routed to their owning ranks, and this rank's
slice summed over the partials of all ranks.  Readings where the pages are
silent are listed in ``oracle.c``'s header.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against brute force, exact integer arithmetic, closed forms or library
routines; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def lib():
    """Load liboracle.so, building it first if it is missing."""
    global _LIB
    if _LIB is None:
        _LIB = load()
    return _LIB


def load(path: str | None = None):
    """Open a liboracle build (default: the in-tree one, built if missing)."""
    from . import build as _build

    if path is None:
        path = _build.library_path()
        if not os.path.exists(path):
            _build.build()
    L = ctypes.CDLL(path)
    L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_to_f32.restype = ctypes.c_float
    L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.oracle_f32_to_bf16_array.argtypes = [_f32p, _u16p, _i64]
    L.oracle_bf16_to_f32_array.argtypes = [_u16p, _f32p, _i64]
    L.oracle_gemm_f32acc.argtypes = [_i64, _i64p, _i64, _i64, _u16p, _u16p, _f32p]
    L.oracle_gemm_f32acc.restype = ctypes.c_int
    L.oracle_peer_rank.argtypes = [_i32, _i32]
    L.oracle_peer_rank.restype = ctypes.c_int
    L.oracle_slice_sum.argtypes = [_i64, _i64p, _i64, _i32, _u16p,
                                   ctypes.POINTER(_u16p), _u16p]
    L.oracle_slice_sum.restype = ctypes.c_int
    L.oracle_gemm_rs.argtypes = [_i64, _i64, _i64, _i32, _i32, _u16p, _u16p,
                                 ctypes.POINTER(_u16p), ctypes.POINTER(_u16p),
                                 _u16p, _u16p]
    L.oracle_gemm_rs.restype = ctypes.c_int
    L.oracle_ref_f64.argtypes = [_i64, _i64p, _i64, _i64, _i64, _i32, _i32, _u16p,
                                 _u16p, ctypes.POINTER(_u16p), _f64p]
    L.oracle_ref_f64.restype = ctypes.c_int
    L.oracle_schedule.argtypes = [_i64, _i64, _i32, _i32, _i32, _i32, _i32,
                                  _i32p, _i32p, _i32p, _i32p]
    L.oracle_schedule.restype = ctypes.c_int
    return L


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctype)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def _rows(rows):
    if rows is None:
        return None, None
    r = _c(rows, np.int64)
    return r, _ptr(r, _i64p)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode BF16 bit patterns (uint16) to float32."""
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float32)
    lib().oracle_bf16_to_f32_array(_ptr(b, _u16p), _ptr(out, _f32p), b.size)
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (nearest, ties to even); returns uint16 bit patterns."""
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_f32_to_bf16_array(_ptr(a, _f32p), _ptr(out, _u16p), a.size)
    return out


def gemm_f32acc(x: np.ndarray, w: np.ndarray, rows=None) -> np.ndarray:
    """P = X * W^T over the selected rows of X, FP32 accumulation, k ascending.

    x: [M][K] uint16 (BF16), w: [N][K] uint16 (BF16).  Returns float32 [len(rows) or M][N].
    """
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    M, K = x.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    r, rp = _rows(rows)
    n = M if r is None else r.size
    P = np.empty((n, N), np.float32)
    _check(lib().oracle_gemm_f32acc(n, rp, N, K, _ptr(x, _u16p), _ptr(w, _u16p), _ptr(P, _f32p)),
           "oracle_gemm_f32acc")
    return P


def peer_rank(rank: int, slot: int) -> int:
    """Rank whose partial sits in peer slot ``slot`` of rank ``rank``."""
    return int(lib().oracle_peer_rank(rank, slot))


def _ptr_array(arrs):
    keep = [_c(a, np.uint16) for a in arrs]
    arr = (_u16p * len(keep))(*[_ptr(a, _u16p) for a in keep])
    return keep, arr


def slice_sum(local: np.ndarray, peers, tp: int = 8, rows=None) -> np.ndarray:
    """out = RNE_bf16(sum of peers in ascending peer rank, then local), FP32."""
    local = _c(local, np.uint16)
    S, N = local.shape
    if len(peers) != tp - 1:
        raise ValueError("need tp-1 peer partials")
    keep, parr = _ptr_array(peers)
    for p in keep:
        if p.shape != (S, N):
            raise ValueError("peer shape differs from local slice")
    r, rp = _rows(rows)
    n = S if r is None else r.size
    out = np.empty((n, N), np.uint16)
    _check(lib().oracle_slice_sum(n, rp, N, tp, _ptr(local, _u16p), parr, _ptr(out, _u16p)),
           "oracle_slice_sum")
    return out


def gemm_rs(x: np.ndarray, w: np.ndarray, peers, tp: int, rank: int):
    """Whole path for one rank.  Returns (send[tp-1], local, out), all BF16 bits.

    send[i] is the routed slice for peer rank peer_rank(rank, i); local is this
    rank's own slice of its partial; out is the reduced slice.
    """
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    M, K = x.shape
    N = w.shape[0]
    S = M // tp
    send = [np.empty((S, N), np.uint16) for _ in range(tp - 1)]
    local = np.empty((S, N), np.uint16)
    out = np.empty((S, N), np.uint16)
    keep_p, parr = _ptr_array(peers)
    sarr = (_u16p * (tp - 1))(*[_ptr(s, _u16p) for s in send])
    _check(lib().oracle_gemm_rs(M, N, K, tp, rank, _ptr(x, _u16p), _ptr(w, _u16p), parr, sarr,
                                _ptr(local, _u16p), _ptr(out, _u16p)), "oracle_gemm_rs")
    return send, local, out


def gemm_allreduce(x: np.ndarray, w: np.ndarray, peers, tp: int, rank: int):
    """GEMM + all-reduce for one rank of one node ("mKernel: Fast Multi-GPU,
    Multi-Node Fused Kernels", Sections 3.1 and 4: the local reduction, then
    replication of each GPU's reduced eighth to the others).  The reduction is
    gemm_rs's; the all-gather moves values without arithmetic, so gather[i],
    what peer rank peer_rank(rank, i) receives, is a copy of out.
    Returns (send[tp-1], local, out, gather[tp-1]), all BF16 bits."""
    send, local, out = gemm_rs(x, w, peers, tp, rank)
    return send, local, out, [out.copy() for _ in range(tp - 1)]


def allreduce_result(outs, gathers, rank: int) -> np.ndarray:
    """The M x N all-reduce result held by `rank` after the all-gather: its own
    rows r*S.. from its reduced slice, every other rank q's rows from what q sent
    it (q's gather entry for `rank`).  outs[q], gathers[q] as gemm_allreduce."""
    tp = len(outs)
    rows = []
    for q in range(tp):
        if q == rank:
            rows.append(outs[q])
        else:
            slot = rank if rank < q else rank - 1  # slot of `rank` in q's peer list
            rows.append(gathers[q][slot])
    return np.concatenate(rows, axis=0)


def ref_f64(x: np.ndarray, w: np.ndarray, peers, tp: int, rank: int, rows=None) -> np.ndarray:
    """FP64 value of this rank's slice sum with no BF16 rounding of the local partial.

    peers=None gives the unrounded local partial slice alone.
    """
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    M, K = x.shape
    N = w.shape[0]
    S = M // tp
    r, rp = _rows(rows)
    n = S if r is None else r.size
    ref = np.empty((n, N), np.float64)
    if peers is None:
        parr = None
        keep_p = None
    else:
        keep_p, parr = _ptr_array(peers)
    _check(lib().oracle_ref_f64(n, rp, M, N, K, tp, rank, _ptr(x, _u16p), _ptr(w, _u16p), parr,
                                _ptr(ref, _f64p)), "oracle_ref_f64")
    return ref


def schedule(M: int, N: int, tp: int, rank: int, bm: int, bn: int, group_m: int):
    """Tile schedule: dict of int32 arrays d, tm, tn, flag indexed by slot."""
    S = M // tp
    T = tp * (-(-S // bm)) * (-(-N // bn))
    out = {k: np.empty(T, np.int32) for k in ("d", "tm", "tn", "flag")}
    _check(lib().oracle_schedule(M, N, tp, rank, bm, bn, group_m, _ptr(out["d"], _i32p),
                                 _ptr(out["tm"], _i32p), _ptr(out["tn"], _i32p),
                                 _ptr(out["flag"], _i32p)), "oracle_schedule")
    return out


def gemm_ag(x_slices, w: np.ndarray):
    """AllGather + GEMM for one rank of a column-parallel linear layer.

    FLUX ("FLUX: Fast Software-based Communication Overlap On GPUs Through
    Kernel Fusion", TL;DR) fuses the all-gather into the GEMM as its prologue;
    mKernel ("mKernel: Fast Multi-GPU, Multi-Node Fused Kernels", Section 4)
    computes the local shard's tiles first and the other shards as they
    arrive.  Neither changes what is computed: every rank gathers the tp row
    slices of the activations, rank d's slice at rows d*S .. d*S + S - 1, and
    multiplies the gathered matrix by its own column shard of the weight.

    x_slices: tp arrays [S][K] (BF16 bits) in source-rank order; w: [N][K]
    (this rank's column shard, K contiguous).  Returns (x_gathered [tp*S][K],
    y [tp*S][N]) with y = RNE_bf16(x_gathered * w^T), FP32 accumulation with k
    ascending (gemm_f32acc)."""
    xs = [_c(x, np.uint16) for x in x_slices]
    S, K = xs[0].shape
    for x in xs:
        if x.shape != (S, K):
            raise ValueError("row slices differ in shape")
    xg = np.concatenate(xs, axis=0)
    y = f32_to_bf16(gemm_f32acc(xg, w))
    return xg, y
