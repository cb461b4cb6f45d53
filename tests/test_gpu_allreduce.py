"""GPU parity of the GEMM + all-reduce entry point (gemm_rs_run_allreduce)
against the CPU oracle, through the C ABI: the reduce-scatter of the fused
kernel, whose sum also replicates the reduced slice into the 7 gather buffers
(the all-gather's sends to the peers)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tensor_gemm_reduce_amd import gemm_rs as gr
from gpu_util import SENTINEL, Buffers, filled, host, sample_rows

pytestmark = pytest.mark.gpu

PLACEMENTS = {"tail": dict(num_reducers=0), "coresident": dict(reduce_mode="coresident"),
              "reducers8": dict(num_reducers=8)}


def _op(cfg, **kw):
    return gr.GemmRS(cfg.M, cfg.N, cfg.K_local, **kw)


def _gathers(cfg):
    return [filled((cfg.S, cfg.N)) for _ in range(7)]


def _run(op, b, gather, mode=gr.MODE_FUSED):
    op.run(mode, b.x, b.w, b.send, b.peers, b.out, b.local, gather=gather)
    torch.cuda.synchronize()
    st = op.status()
    assert st == gr.OK, gr.gemm_rs_strerror(st)


@pytest.mark.parametrize("placement", list(PLACEMENTS))
@pytest.mark.parametrize("rank", [0, 5, 7])
def test_tiny_integer_bit_exact(rank, placement):
    cfg = synthetic.CONFIGS["tiny"]
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    op = _op(cfg, rank=rank, **PLACEMENTS[placement])
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    g = _gathers(cfg)
    _run(op, b, g)
    send_o, local_o, out_o, gather_o = oracle.gemm_allreduce(x, w, peers, tp=8, rank=rank)
    for i in range(7):
        assert np.array_equal(host(b.send[i]), send_o[i]), f"send[{i}]"
        assert np.array_equal(host(g[i]), gather_o[i]), f"gather[{i}]"
    assert np.array_equal(host(b.local), local_o)
    assert np.array_equal(host(b.out), out_o)


@pytest.mark.parametrize("placement", ["tail", "reducers8"])
def test_eight_ranks_hold_the_unsharded_product(placement):
    """All 8 ranks run on this GPU with consistent shards; each rank's M x N
    result (its own reduced rows plus what the others sent it) equals the
    unsharded product rounded once to BF16 (exact with integer inputs)."""
    cfg = synthetic.Config("ar_gpu", 0, 8 * 40, 392, 72)
    shards = synthetic.make_shards(cfg, integer=True)
    S, N = cfg.S, cfg.N
    zero = [np.zeros((S, N), np.uint16)] * 7
    # every rank's routed partial slices (its GEMM only)
    parts = []
    for p, (xp, wp) in enumerate(shards):
        op = _op(cfg, rank=p, **PLACEMENTS[placement])
        b = Buffers(xp, wp, zero, S, N)
        _run(op, b, None, gr.MODE_GEMM_ONLY)
        parts.append([host(s) for s in b.send])
    outs, gathers = [], []
    for r, (xr, wr) in enumerate(shards):
        peers = [parts[q][r if r < q else r - 1] for q in (oracle.peer_rank(r, i) for i in range(7))]
        op = _op(cfg, rank=r, **PLACEMENTS[placement])
        b = Buffers(xr, wr, peers, S, N)
        g = _gathers(cfg)
        _run(op, b, g)
        outs.append(host(b.out))
        gathers.append([host(t) for t in g])
    X = np.concatenate([oracle.bf16_to_f32(s[0]).astype(np.int64) for s in shards], axis=1)
    W = np.concatenate([oracle.bf16_to_f32(s[1]).astype(np.int64) for s in shards], axis=1)
    want = oracle.f32_to_bf16((X @ W.T).astype(np.float32))
    for r in range(8):
        assert np.array_equal(oracle.allreduce_result(outs, gathers, r), want), r


def test_modes():
    cfg = synthetic.CONFIGS["tiny"]
    x, w, peers = synthetic.make_inputs(cfg, "normal")
    op = _op(cfg, rank=2)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    g = _gathers(cfg)
    _run(op, b, g)
    fused = host(b.out)
    assert all(np.array_equal(host(t), fused) for t in g)
    # GEMM_ONLY writes no reduced slice: the gather buffers stay untouched
    g2 = _gathers(cfg)
    b.refill()
    _run(op, b, g2, gr.MODE_GEMM_ONLY)
    assert all(np.all(host(t) == SENTINEL) for t in g2)
    # REDUCE_ONLY over that local slice, and SEQUENTIAL, replicate it too
    _run(op, b, g2, gr.MODE_REDUCE_ONLY)
    assert np.array_equal(host(b.out), fused)
    assert all(np.array_equal(host(t), fused) for t in g2)
    g3 = _gathers(cfg)
    b.refill()
    _run(op, b, g3, gr.MODE_SEQUENTIAL)
    assert all(np.array_equal(host(t), fused) for t in g3)


@pytest.mark.parametrize("name", ["o_proj", "down_proj"])
def test_benchmark_shapes(name):
    cfg = synthetic.CONFIGS[name]
    rank = 5
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    op = _op(cfg, rank=rank)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    g = _gathers(cfg)
    _run(op, b, g)
    for t in g:
        assert torch.equal(t, b.out)
    rows = sample_rows(cfg.S, op.info.bm, np.random.default_rng(3))
    local_o = oracle.f32_to_bf16(oracle.gemm_f32acc(x, w, rows=rank * cfg.S + rows))
    assert np.array_equal(host(b.local)[rows], local_o)
    assert np.array_equal(host(b.out)[rows], oracle.slice_sum(local_o, [p[rows] for p in peers]))


def test_gather_arguments_checked():
    cfg = synthetic.CONFIGS["tiny"]
    x, w, peers = synthetic.make_inputs(cfg, "normal")
    op = _op(cfg, rank=1)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    ptr = lambda t: t.data_ptr()
    args = (op.h, gr.MODE_FUSED, ptr(b.x), ptr(b.w), [ptr(s) for s in b.send], [ptr(p) for p in b.peers],
            ptr(b.out), ptr(b.local))
    assert gr.gemm_rs_run_allreduce(*args, None, None) == gr.ERR_INVALID_ARG
    g = _gathers(cfg)
    bad = [ptr(t) for t in g]
    bad[3] += 2
    assert gr.gemm_rs_run_allreduce(*args, bad, None) == gr.ERR_MISALIGNED
    bad[3] = None
    assert gr.gemm_rs_run_allreduce(*args, bad, None) == gr.ERR_INVALID_ARG
    torch.cuda.synchronize()
