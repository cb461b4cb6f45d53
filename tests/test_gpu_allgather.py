"""GPU tests of all-gather + GEMM (gemm_rs_run_allgather) against the oracle.

The column-parallel layer with the all-gather fused as the GEMM's prologue:
the gathered activations must equal the source slices bit for bit, and y the
oracle's product bit for bit on integer inputs (every FP32 sum exact), within
one BF16 ulp plus the FP32 summation-order bound on normal inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tensor_gemm_reduce_amd import gemm_rs as gr
from gpu_util import SENTINEL, assert_close_partial, dev, filled, host

pytestmark = pytest.mark.gpu

RAGGED = synthetic.AgConfig("ag_ragged", 15, 8 * 264, 392, 136)
MID = synthetic.AgConfig("ag_mid", 16, 2048, 4096, 512)   # 128 tiles of 256x256


class AgBuffers:
    def __init__(self, cfg, xs, w, M=None):
        M = cfg.M if M is None else M
        self.xs = [dev(x) for x in xs]
        self.w = dev(w)
        self.xg = filled((M, cfg.K))
        self.y = filled((M, cfg.N))

    def refill(self):
        fill = np.array(SENTINEL, np.uint16).view(np.int16).item()
        self.xg.fill_(fill)
        self.y.fill_(fill)


def _op(cfg, rank, **kw):
    return gr.GemmRS(cfg.M, cfg.N, cfg.K, rank=rank, **kw)


def _run(op, b, mode=gr.MODE_FUSED):
    op.run_allgather(mode, b.xs, b.w, b.xg, b.y)
    torch.cuda.synchronize()
    st = op.status()
    assert st == gr.OK, gr.gemm_rs_strerror(st)


def _exact(cfg, rank, **kw):
    xs, w = synthetic.make_ag_inputs(cfg, "integer")
    op = _op(cfg, rank, **kw)
    b = AgBuffers(cfg, xs, w)
    _run(op, b)
    xg_o, y_o = oracle.gemm_ag(xs, w)
    assert np.array_equal(host(b.xg), xg_o)
    assert np.array_equal(host(b.y), y_o)


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_ag_tiny_integer_bit_exact(rank):
    _exact(synthetic.AG_CONFIGS["ag_tiny"], rank)


@pytest.mark.parametrize("tile", ["16x64", "64x128", "128x128", "128x256", "256x128", "256x256"])
def test_ag_ragged_every_tile_integer_bit_exact(tile):
    _exact(RAGGED, 5, tile=tile)


def test_ag_mid_integer_bit_exact():
    _exact(MID, 2)


def test_ag_modes_agree_bit_exactly():
    cfg = synthetic.AG_CONFIGS["ag_qkv"]
    xs, w = synthetic.make_ag_inputs(cfg, "normal")
    op = _op(cfg, 6)
    b = AgBuffers(cfg, xs, w)
    _run(op, b, gr.MODE_FUSED)
    xg_f, y_f = host(b.xg), host(b.y)
    xg_o = np.concatenate(xs, axis=0)
    assert np.array_equal(xg_f, xg_o)
    b.refill()
    _run(op, b, gr.MODE_SEQUENTIAL)
    assert np.array_equal(host(b.xg), xg_f) and np.array_equal(host(b.y), y_f)
    b.refill()
    _run(op, b, gr.MODE_REDUCE_ONLY)   # the all-gather alone
    assert np.array_equal(host(b.xg), xg_o)
    assert np.all(host(b.y) == SENTINEL)
    _run(op, b, gr.MODE_GEMM_ONLY)     # the GEMM over the gathered buffer
    assert np.array_equal(host(b.y), y_f)
    # and y is the oracle's product within the summation-order bound
    rows = np.array([0, 1, cfg.S - 1, cfg.S, 3 * cfg.S + 7, cfg.M - 1], np.int64)
    y_o = oracle.f32_to_bf16(oracle.gemm_f32acc(xg_o, w, rows=rows))
    assert_close_partial(y_f[rows], y_o, xg_o, w, rows)


def test_ag_alternating_inputs_and_graph_replays():
    """Runs alternate two input sets on one gathered buffer and one output, the
    gathered buffer poisoned before each run: a tile that read its rows before
    they were copied, or a stale cached copy of an earlier run's rows, would
    give a wrong y."""
    cfgs = [synthetic.AgConfig("ag_alt_a", 17, MID.M, MID.N, MID.K),
            synthetic.AgConfig("ag_alt_b", 18, MID.M, MID.N, MID.K)]
    rank = 4
    ins = [synthetic.make_ag_inputs(c, "integer") for c in cfgs]
    want = [dev(oracle.gemm_ag(xs, w)[1]) for xs, w in ins]
    bufs = [AgBuffers(MID, xs, w) for xs, w in ins]
    xg, y = bufs[0].xg, bufs[0].y
    fill = np.array(SENTINEL, np.uint16).view(np.int16).item()
    op = _op(MID, rank)
    bad = 0
    for it in range(20):
        i = it % 2
        xg.fill_(fill)
        op.run_allgather(gr.MODE_FUSED, bufs[i].xs, bufs[i].w, xg, y)
        if not torch.equal(y, want[i]):
            bad += 1
    torch.cuda.synchronize()
    assert op.status() == gr.OK
    assert bad == 0
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        op.run_allgather(gr.MODE_FUSED, bufs[1].xs, bufs[1].w, xg, y)
    torch.cuda.synchronize()
    for it in range(4):
        xg.fill_(fill)
        y.fill_(fill)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert op.status() == gr.OK
        assert torch.equal(y, want[1]), it
        if it % 2:
            op.run_allgather(gr.MODE_FUSED, bufs[0].xs, bufs[0].w, xg, y)
            torch.cuda.synchronize()
            assert torch.equal(y, want[0])


@pytest.mark.parametrize("name,mode", [("ag_gate_up", "normal"), ("ag_gate_up", "integer"),
                                       ("ag_mixtral_w13", "normal"), ("ag_large_prefill", "normal")])
def test_ag_benchmark_shapes_sampled_rows(name, mode):
    cfg = synthetic.AG_CONFIGS[name]
    rank = 5
    xs, w = synthetic.make_ag_inputs(cfg, mode)
    op = _op(cfg, rank)
    b = AgBuffers(cfg, xs, w)
    _run(op, b)
    S = cfg.S
    rng = np.random.default_rng(3)
    rows = sorted({0, S - 1, S, rank * S, rank * S + S - 1, cfg.M - 1} |
                  set(int(r) for r in rng.integers(0, cfg.M, size=4)))
    rows = np.array(rows, np.int64)
    xg_o = np.concatenate(xs, axis=0)
    got_xg = host(b.xg)
    assert np.array_equal(got_xg, xg_o)
    y_o = oracle.f32_to_bf16(oracle.gemm_f32acc(xg_o, w, rows=rows))
    got = host(b.y)[rows]
    if mode == "integer":
        assert np.array_equal(got, y_o)
    else:
        assert_close_partial(got, y_o, xg_o, w, rows)
    assert not bool((b.y == np.array(SENTINEL, np.uint16).view(np.int16).item()).any())


def test_ag_argument_checks():
    cfg = synthetic.AG_CONFIGS["ag_tiny"]
    xs, w = synthetic.make_ag_inputs(cfg, "integer")
    op = _op(cfg, 1)
    b = AgBuffers(cfg, xs, w)
    vp = [t.data_ptr() for t in b.xs]
    assert gr.gemm_rs_run_allgather(op.h, gr.MODE_FUSED, None, b.w.data_ptr(), b.xg.data_ptr(),
                                    b.y.data_ptr(), None) == gr.ERR_INVALID_ARG
    assert gr.gemm_rs_run_allgather(op.h, gr.MODE_FUSED, vp, b.w.data_ptr(), b.xg.data_ptr() + 2,
                                    b.y.data_ptr(), None) == gr.ERR_MISALIGNED
    assert gr.gemm_rs_run_allgather(op.h, 7, vp, b.w.data_ptr(), b.xg.data_ptr(),
                                    b.y.data_ptr(), None) == gr.ERR_INVALID_ARG
    # the fused launch needs x_gathered on a 128-byte line boundary (16 is not
    # enough), the separate copy and GEMM launches do not
    big = torch.zeros(b.xg.numel() + 128, dtype=torch.int16, device="cuda")
    base = (-big.data_ptr()) % 128 // 2
    xg16 = big[base + 8: base + 8 + b.xg.numel()]
    assert xg16.data_ptr() % 128 == 16
    assert gr.gemm_rs_run_allgather(op.h, gr.MODE_FUSED, vp, b.w.data_ptr(), xg16.data_ptr(),
                                    b.y.data_ptr(), None) == gr.ERR_MISALIGNED
    assert gr.gemm_rs_run_allgather(op.h, gr.MODE_SEQUENTIAL, vp, b.w.data_ptr(), xg16.data_ptr(),
                                    b.y.data_ptr(), None) == gr.OK
    # and every slice a whole number of lines: S * K * 2 = 3 * 8 * 2 bytes is not
    odd = gr.GemmRS(24, 64, 8, rank=0)
    zs = [torch.zeros((3, 8), dtype=torch.int16, device="cuda") for _ in range(8)]
    zg = torch.zeros((24, 8), dtype=torch.int16, device="cuda")
    zw = torch.zeros((64, 8), dtype=torch.int16, device="cuda")
    zy = torch.zeros((24, 64), dtype=torch.int16, device="cuda")
    assert gr.gemm_rs_run_allgather(odd.h, gr.MODE_FUSED, [t.data_ptr() for t in zs], zw.data_ptr(),
                                    zg.data_ptr(), zy.data_ptr(), None) == gr.ERR_UNSUPPORTED_SHAPE
    torch.cuda.synchronize()
