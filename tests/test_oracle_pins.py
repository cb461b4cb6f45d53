"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to brute force on tiny inputs, exact integer
arithmetic, a closed form, a hand-derived fixture or a library routine, chosen
so that a dropped term, a wrong sign or index, or a transposed operand fails at
least one of them.  CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from conftest import read_golden

U = 2.0 ** -24  # unit roundoff of FP32


def f32_bits_to_float(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


# ---------------------------------------------------------------- BF16 codec

def test_rne_golden_cases():
    rows = read_golden("bf16_rne_cases.txt")
    assert len(rows) >= 15
    f = f32_bits_to_float([int(r[0], 16) for r in rows])
    want = np.array([int(r[1], 16) for r in rows], np.uint16)
    got = oracle.f32_to_bf16(f)
    bad = [(rows[i][0], rows[i][1], hex(int(got[i]))) for i in range(len(rows)) if got[i] != want[i]]
    assert not bad, bad


def test_rne_nan_stays_nan():
    f = f32_bits_to_float([0x7FC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF])
    got = oracle.f32_to_bf16(f)
    assert np.all((got & 0x7F80) == 0x7F80) and np.all((got & 0x007F) != 0)


def test_rne_matches_torch_on_random_patterns():
    # torch's CPU float -> bfloat16 conversion rounds to nearest even.
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(f)
    assert np.array_equal(got, want)


def test_decode_matches_torch_all_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.bf16_to_f32(b)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


# ---------------------------------------------------------------- GEMM

def _rand_bf16(rng, shape, scale=1.0):
    return synthetic.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale)


@pytest.mark.parametrize("M,N,K", [(37, 53, 29), (5, 3, 1), (16, 64, 300), (1, 1, 1000)])
def test_gemm_within_summation_bound_of_fp64_brute_force(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    x = _rand_bf16(rng, (M, K))
    w = _rand_bf16(rng, (N, K))
    P = oracle.gemm_f32acc(x, w)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wf = oracle.bf16_to_f32(w).astype(np.float64)
    gamma = K * U / (1 - K * U)
    for i in range(M):
        for j in range(N):
            exact = math.fsum(xf[i, k] * wf[j, k] for k in range(K))
            bound = gamma * math.fsum(abs(xf[i, k] * wf[j, k]) for k in range(K))
            assert abs(float(P[i, j]) - exact) <= bound + 1e-300, (i, j)


def test_gemm_k_ascending_fp32_chain_brute_force():
    # One FP32 rounding per addition, k ascending, starting from +0.
    rng = np.random.default_rng(5)
    M, N, K = 3, 4, 257
    x = _rand_bf16(rng, (M, K))
    w = _rand_bf16(rng, (N, K), 1e-3)
    P = oracle.gemm_f32acc(x, w)
    xf = oracle.bf16_to_f32(x)
    wf = oracle.bf16_to_f32(w)
    for i in range(M):
        for j in range(N):
            acc = np.float32(0.0)
            for k in range(K):
                acc = np.float32(acc + np.float32(xf[i, k] * wf[j, k]))
            assert P[i, j].view(np.uint32) == acc.view(np.uint32)


def test_gemm_integer_inputs_exact_vs_int64_matmul():
    rng = np.random.default_rng(3)
    M, N, K = 24, 40, 96
    xi = rng.integers(-2, 3, size=(M, K))
    wi = rng.integers(-2, 3, size=(N, K))
    x = synthetic.to_bf16_bits(xi.astype(np.float32))
    w = synthetic.to_bf16_bits(wi.astype(np.float32))
    P = oracle.gemm_f32acc(x, w)
    assert np.array_equal(P.astype(np.int64), xi @ wi.T)


def test_gemm_row_subset_equals_full():
    rng = np.random.default_rng(4)
    x = _rand_bf16(rng, (20, 33))
    w = _rand_bf16(rng, (17, 33))
    full = oracle.gemm_f32acc(x, w)
    rows = np.array([19, 0, 7, 7], np.int64)
    sub = oracle.gemm_f32acc(x, w, rows=rows)
    assert np.array_equal(sub.view(np.uint32), full[rows].view(np.uint32))


def test_gemm_zero_k_gives_zero():
    x = np.zeros((4, 0), np.uint16)
    w = np.zeros((3, 0), np.uint16)
    assert np.array_equal(oracle.gemm_f32acc(x, w), np.zeros((4, 3), np.float32))


# ---------------------------------------------------------------- slice sum

def test_slice_sum_golden_order():
    rows = read_golden("slice_sum_order.txt")
    for r in rows:
        vals = [int(v, 16) for v in r]
        peers = [np.array([[v]], np.uint16) for v in vals[:7]]
        local = np.array([[vals[7]]], np.uint16)
        out = oracle.slice_sum(local, peers, tp=8)
        assert int(out[0, 0]) == vals[8], r


def test_slice_sum_integer_exact():
    rng = np.random.default_rng(8)
    S, N = 6, 50
    ints = [rng.integers(-8, 9, size=(S, N)) for _ in range(8)]
    bits = [synthetic.to_bf16_bits(a.astype(np.float32)) for a in ints]
    out = oracle.slice_sum(bits[7], bits[:7], tp=8)
    assert np.array_equal(oracle.bf16_to_f32(out).astype(np.int64), sum(ints))


def test_slice_sum_zero_peers_is_identity():
    rng = np.random.default_rng(9)
    local = _rand_bf16(rng, (5, 9))
    zeros = [np.zeros((5, 9), np.uint16)] * 7
    out = oracle.slice_sum(local, zeros, tp=8)
    nz = oracle.bf16_to_f32(local) != 0
    assert np.array_equal(out[nz], local[nz])


def test_slice_sum_within_fp32_bound_of_exact():
    rng = np.random.default_rng(10)
    srcs = [_rand_bf16(rng, (4, 64)) for _ in range(8)]
    out = oracle.f32_to_bf16(np.zeros(1, np.float32))  # warm the library
    out = oracle.slice_sum(srcs[7], srcs[:7], tp=8)
    got = oracle.bf16_to_f32(out).astype(np.float64)
    vals = [oracle.bf16_to_f32(s).astype(np.float64) for s in srcs]
    exact = sum(vals)
    absum = sum(np.abs(v) for v in vals)
    # 8 FP32 additions then one BF16 rounding (half an ulp of 8 significant bits)
    bound = 8 * U * absum * 1.0001 + 2.0 ** -8 * np.abs(exact) * 1.0001
    assert np.all(np.abs(got - exact) <= bound)


# ---------------------------------------------------------------- routing + whole path

def test_worked_example_tp2():
    g = {r[0]: [float(v) for v in r[1:]] for r in read_golden("worked_example_tp2.txt")}
    b = lambda vals, shape: synthetic.to_bf16_bits(np.array(vals, np.float32).reshape(shape))
    x, w = b(g["x"], (2, 2)), b(g["w"], (2, 2))
    peers = [b(g["peer"], (1, 2))]
    send, local, out = oracle.gemm_rs(x, w, peers, tp=2, rank=0)
    assert oracle.bf16_to_f32(send[0]).tolist() == [g["send"]]
    assert oracle.bf16_to_f32(local).tolist() == [g["local"]]
    assert oracle.bf16_to_f32(out).tolist() == [g["out"]]


@pytest.mark.parametrize("rank", range(8))
def test_peer_slot_mapping(rank):
    seen = [oracle.peer_rank(rank, i) for i in range(7)]
    assert sorted(seen) == [r for r in range(8) if r != rank]
    assert seen == sorted(seen)


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_routing_integer_exact(rank):
    cfg = synthetic.CONFIGS["tiny"]
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    send, local, out = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    xi = oracle.bf16_to_f32(x).astype(np.int64)
    wi = oracle.bf16_to_f32(w).astype(np.int64)
    P = xi @ wi.T
    S = cfg.S
    assert np.array_equal(oracle.bf16_to_f32(local).astype(np.int64), P[rank * S:(rank + 1) * S])
    for i in range(7):
        p = oracle.peer_rank(rank, i)
        assert np.array_equal(oracle.bf16_to_f32(send[i]).astype(np.int64), P[p * S:(p + 1) * S])
    want = sum(oracle.bf16_to_f32(pp).astype(np.int64) for pp in peers) + P[rank * S:(rank + 1) * S]
    assert np.array_equal(oracle.bf16_to_f32(out).astype(np.int64), want)


@pytest.mark.parametrize("rank", range(8))
def test_reduce_scatter_invariant_consistent_peers(rank):
    """Reduce-scatter of the 8 ranks' partials equals row slice `rank` of the
    unsharded product X * W^T (exact with integer inputs)."""
    cfg = synthetic.Config("rs_inv", 0, 64, 48, 16)
    shards = synthetic.make_shards(cfg, integer=True)
    S = cfg.S
    # each rank's own partial, routed: rank p's send slot for `rank` holds the
    # partial of slice `rank`
    parts = {}
    for p, (xp, wp) in enumerate(shards):
        zero = [np.zeros((S, cfg.N), np.uint16)] * 7
        send, local, _ = oracle.gemm_rs(xp, wp, zero, tp=8, rank=p)
        parts[p] = (send, local)
    peers = []
    for i in range(7):
        p = oracle.peer_rank(rank, i)
        slot = rank if rank < p else rank - 1  # slot of `rank` in p's send list
        assert oracle.peer_rank(p, slot) == rank
        peers.append(parts[p][0][slot])
    xr, wr = shards[rank]
    _, _, out = oracle.gemm_rs(xr, wr, peers, tp=8, rank=rank)
    X = np.concatenate([oracle.bf16_to_f32(s[0]).astype(np.int64) for s in shards], axis=1)
    W = np.concatenate([oracle.bf16_to_f32(s[1]).astype(np.int64) for s in shards], axis=1)
    full = X @ W.T
    assert np.array_equal(oracle.bf16_to_f32(out).astype(np.int64), full[rank * S:(rank + 1) * S])


def test_allreduce_gives_every_rank_the_unsharded_product():
    """All-reduce invariant: after the reduce-scatter and the all-gather, every
    one of the 8 ranks holds the whole unsharded product X * W^T, rounded once
    to BF16 (exact with integer inputs), and all 8 results are identical."""
    cfg = synthetic.Config("ar_inv", 0, 64, 48, 16)
    shards = synthetic.make_shards(cfg, integer=True)
    S = cfg.S
    parts = {}
    for p, (xp, wp) in enumerate(shards):
        zero = [np.zeros((S, cfg.N), np.uint16)] * 7
        send, local, _ = oracle.gemm_rs(xp, wp, zero, tp=8, rank=p)
        parts[p] = send
    outs, gathers = [], []
    for r, (xr, wr) in enumerate(shards):
        peers = [parts[q][r if r < q else r - 1] for q in (oracle.peer_rank(r, i) for i in range(7))]
        _, _, out, gather = oracle.gemm_allreduce(xr, wr, peers, tp=8, rank=r)
        outs.append(out)
        gathers.append(gather)
    X = np.concatenate([oracle.bf16_to_f32(s[0]).astype(np.int64) for s in shards], axis=1)
    W = np.concatenate([oracle.bf16_to_f32(s[1]).astype(np.int64) for s in shards], axis=1)
    want = oracle.f32_to_bf16((X @ W.T).astype(np.float32))
    results = [oracle.allreduce_result(outs, gathers, r) for r in range(8)]
    for r in range(8):
        assert np.array_equal(results[r], want), r


def test_zero_x_gives_sum_of_peers():
    cfg = synthetic.CONFIGS["tiny"]
    x, w, peers = synthetic.make_inputs(cfg, "zero_x")
    _, local, out = oracle.gemm_rs(x, w, peers, tp=8, rank=2)
    assert not np.any(oracle.bf16_to_f32(local))
    pf = [oracle.bf16_to_f32(p) for p in peers]
    acc = np.zeros_like(pf[0])
    for p in pf:
        acc = (acc + p).astype(np.float32)
    want = torch.from_numpy(acc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, want)


def test_zero_peers_gives_rounded_partial_vs_numpy():
    cfg = synthetic.CONFIGS["tiny"]
    x, w, peers = synthetic.make_inputs(cfg, "zero_peers")
    rank = 6
    _, local, out = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    assert np.array_equal(out[oracle.bf16_to_f32(out) != 0], local[oracle.bf16_to_f32(out) != 0])
    S = cfg.S
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wf = oracle.bf16_to_f32(w).astype(np.float64)
    P = (xf @ wf.T)[rank * S:(rank + 1) * S]
    got = oracle.bf16_to_f32(out).astype(np.float64)
    absP = np.abs(xf) @ np.abs(wf).T
    bound = cfg.K_local * U * 1.01 * absP[rank * S:(rank + 1) * S] + 2.0 ** -8 * np.abs(P)
    assert np.all(np.abs(got - P) <= bound)


# ---------------------------------------------------------------- FP64 reference

def test_ref_f64_matches_fsum_brute_force():
    cfg = synthetic.Config("ref", 0, 16, 12, 20)
    x, w, peers = synthetic.make_inputs(cfg, "normal")
    rank = 3
    ref = oracle.ref_f64(x, w, peers, tp=8, rank=rank)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wf = oracle.bf16_to_f32(w).astype(np.float64)
    pf = [oracle.bf16_to_f32(p).astype(np.float64) for p in peers]
    S = cfg.S
    for i in range(S):
        for j in range(cfg.N):
            terms = [xf[rank * S + i, k] * wf[j, k] for k in range(cfg.K_local)]
            terms += [p[i, j] for p in pf]
            exact = math.fsum(terms)
            assert abs(ref[i, j] - exact) <= 64 * 2.0 ** -53 * math.fsum(abs(t) for t in terms)


def test_ref_f64_local_only_vs_numpy_matmul():
    cfg = synthetic.CONFIGS["tiny"]
    x, w, _ = synthetic.make_inputs(cfg, "normal")
    ref = oracle.ref_f64(x, w, None, tp=8, rank=1)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wf = oracle.bf16_to_f32(w).astype(np.float64)
    want = (xf @ wf.T)[cfg.S:2 * cfg.S]
    assert np.allclose(ref, want, rtol=0, atol=1e-12)


def test_ref_f64_row_subset():
    cfg = synthetic.CONFIGS["tiny"]
    x, w, peers = synthetic.make_inputs(cfg, "normal")
    full = oracle.ref_f64(x, w, peers, tp=8, rank=4)
    rows = np.array([15, 2], np.int64)
    sub = oracle.ref_f64(x, w, peers, tp=8, rank=4, rows=rows)
    assert np.array_equal(sub, full[rows])


def test_oracle_path_error_within_tolerance_of_reference():
    cfg = synthetic.CONFIGS["tiny"]
    for mode in ("normal", "balanced"):
        x, w, peers = synthetic.make_inputs(cfg, mode)
        _, local, out = oracle.gemm_rs(x, w, peers, tp=8, rank=5)
        ref = oracle.ref_f64(x, w, peers, tp=8, rank=5)
        err = np.max(np.abs(oracle.bf16_to_f32(out) - ref)) / np.max(np.abs(ref))
        assert err <= 2.0 ** -8
        ref_local = oracle.ref_f64(x, w, None, tp=8, rank=5)
        err_l = np.max(np.abs(oracle.bf16_to_f32(local) - ref_local)) / np.max(np.abs(ref_local))
        assert err_l <= 2.0 ** -8


# ---------------------------------------------------------------- schedule

SCHED_CASES = [
    (128, 1024, 16, 64, 1), (512, 8192, 64, 128, 4), (2048, 8192, 256, 256, 8),
    (8192, 6144, 256, 256, 8), (8192, 6144, 128, 128, 3), (1024, 640, 32, 64, 5),
]


@pytest.mark.parametrize("M,N,bm,bn,gm", SCHED_CASES)
@pytest.mark.parametrize("rank", [0, 5, 7])
def test_schedule_is_slice_rotated_permutation(M, N, bm, bn, gm, rank):
    tp = 8
    s = oracle.schedule(M, N, tp, rank, bm, bn, gm)
    S = M // tp
    tms, tnc = S // bm, N // bn
    ts = tms * tnc
    T = tp * ts
    assert sorted(s["flag"].tolist()) == list(range(T))
    # every (tm, tn) tile appears once and lies in slice d
    tiles = set(zip(s["tm"].tolist(), s["tn"].tolist()))
    assert len(tiles) == T
    for q in range(T):
        d, tm, tn, f = (int(s[k][q]) for k in ("d", "tm", "tn", "flag"))
        assert d == (rank + q // ts) % tp
        assert d * tms <= tm < (d + 1) * tms and 0 <= tn < tnc
        assert f == d * ts + (tm - d * tms) * tnc + tn
    # own slice first
    assert np.all(s["d"][:ts] == rank)


@pytest.mark.parametrize("M,N,bm,bn", [(1024, 640, 32, 64), (512, 8192, 64, 128)])
def test_schedule_raster_special_cases(M, N, bm, bn):
    tp, rank = 8, 2
    S = M // tp
    tms, tnc = S // bm, N // bn
    ts = tms * tnc
    # group of one tile-row: row-major raster of the slice
    s = oracle.schedule(M, N, tp, rank, bm, bn, 1)
    tm_l, tn = np.unravel_index(np.arange(ts), (tms, tnc), order="C")
    assert np.array_equal(s["tm"][:ts] - rank * tms, tm_l) and np.array_equal(s["tn"][:ts], tn)
    # a group spanning the whole slice: column-major raster
    s = oracle.schedule(M, N, tp, rank, bm, bn, tms)
    tm_l, tn = np.unravel_index(np.arange(ts), (tms, tnc), order="F")
    assert np.array_equal(s["tm"][:ts] - rank * tms, tm_l) and np.array_equal(s["tn"][:ts], tn)


def test_schedule_destinations_form_permutation_across_ranks():
    tp, M, N, bm, bn = 8, 1024, 640, 32, 64
    per_rank = [oracle.schedule(M, N, tp, r, bm, bn, 2)["d"] for r in range(tp)]
    ts = (M // tp // bm) * (N // bn)
    for step in range(tp):
        dests = sorted(int(d[step * ts]) for d in per_rank)
        assert dests == list(range(tp))


def test_schedule_grouped_raster_locality():
    # inside a group of gm tile-rows, gm consecutive slots share one tile column
    M, N, bm, bn, gm = 8192, 6144, 128, 128, 4
    s = oracle.schedule(M, N, 8, 0, bm, bn, gm)
    tms = M // 8 // bm
    for start in range(0, gm * (N // bn), gm):
        cols = s["tn"][start:start + gm]
        assert np.all(cols == cols[0])
        assert sorted((s["tm"][start:start + gm]).tolist()) == list(range(gm))
    assert tms % gm == 0


def test_schedule_rejects_bad_shapes():
    with pytest.raises(RuntimeError):
        oracle.schedule(100, 64, 8, 0, 16, 64, 1)  # M not divisible by tp
    with pytest.raises(RuntimeError):
        oracle.schedule(8, 64, 16, 0, 16, 64, 1)  # empty slice


@pytest.mark.parametrize("M,N,bm,bn,gm", [(8 * 40, 200, 16, 64, 3), (8 * 7, 24, 16, 64, 1),
                                          (8 * 100, 1000, 32, 128, 2)])
def test_schedule_ragged_tiles_cover_slice_exactly_once(M, N, bm, bn, gm):
    # partial last tile row / column: every element of every slice is covered
    # by exactly one tile, and no tile crosses a slice boundary
    tp, rank = 8, 4
    S = M // tp
    s = oracle.schedule(M, N, tp, rank, bm, bn, gm)
    tms = -(-S // bm)
    cover = np.zeros((M, N), np.int32)
    for q in range(s["d"].size):
        d, tm, tn = int(s["d"][q]), int(s["tm"][q]), int(s["tn"][q])
        r0 = d * S + (tm - d * tms) * bm
        r1 = min(r0 + bm, (d + 1) * S)
        cover[r0:r1, tn * bn:min(N, tn * bn + bn)] += 1
    assert np.all(cover == 1)
