"""GPU tests of the co-resident reducers (reduce_mode "coresident"): one
reducer workgroup per CU beside the compute workgroups, whose waves sum the
peers of their items while the GEMM runs and add the local chunk once the
tile's flag is set.

Its results must equal the oracle's bit for bit on integer inputs, and the
sum after the last tile's ("tail") bit for bit on any inputs: both add the
same BF16 values in the same FP32 order.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tensor_gemm_reduce_amd import gemm_rs as gr
from gpu_util import SENTINEL, Buffers, dev, filled, host, run

pytestmark = pytest.mark.gpu

CORES = dict(reduce_mode="coresident")
RAGGED = synthetic.Config("ragged", 5, 8 * 264, 392, 136)


def _outputs(b):
    return [host(t) for t in b.send + [b.local, b.out]]


def _check_integer(cfg, rank, **kw):
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, **CORES, **kw)
    info = op.info
    assert info.reduce_mode == gr.REDUCE_CORESIDENT
    assert info.reducer_wgs > 0 and info.compute_wgs + info.reducer_wgs == info.grid
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b)
    send_o, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    got = _outputs(b)
    for i in range(7):
        assert np.array_equal(got[i], send_o[i]), f"send[{i}]"
    assert np.array_equal(got[7], local_o)
    assert np.array_equal(got[8], out_o)


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_coresident_tiny_integer_bit_exact(rank):
    _check_integer(synthetic.CONFIGS["tiny"], rank)


@pytest.mark.parametrize("tile", ["16x64", "64x128", "128x128"])
def test_coresident_ragged_integer_bit_exact(tile):
    _check_integer(RAGGED, 5, tile=tile)


def test_coresident_o_proj_integer_bit_exact():
    _check_integer(synthetic.CONFIGS["o_proj"], 6)


@pytest.mark.parametrize("tile", ["16x64", "64x128"])
def test_coresident_row_counters_integer_bit_exact(tile):
    # the reducers wait for whole tile rows instead of single tiles
    _check_integer(RAGGED, 2, tile=tile, flag_protocol="row_counter")


def test_coresident_equals_tail_on_normal_inputs():
    cfg = synthetic.CONFIGS["o_proj"]
    x, w, peers = synthetic.make_inputs(cfg, "normal")
    res = []
    for kw in (CORES, dict(reduce_mode="tail")):
        op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=3, **kw)
        b = Buffers(x, w, peers, cfg.S, cfg.N)
        run(op, b)
        res.append(_outputs(b))
        op.close()
    for a_, t_ in zip(*res):
        assert np.array_equal(a_, t_)
    assert np.array_equal(res[0][8], oracle.slice_sum(res[0][7], peers))


def test_coresident_modes_agree_and_all_reduce():
    cfg = synthetic.CONFIGS["o_proj"]
    rank = 2
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, **CORES)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    _, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    for mode in (gr.MODE_SEQUENTIAL, gr.MODE_FUSED):
        b.refill()
        run(op, b, mode)
        assert np.array_equal(host(b.local), local_o)
        assert np.array_equal(host(b.out), out_o)
    b.refill()
    run(op, b, gr.MODE_GEMM_ONLY)
    assert np.array_equal(host(b.local), local_o)
    assert np.all(host(b.out) == SENTINEL)
    gather = [filled((cfg.S, cfg.N)) for _ in range(7)]
    b.refill()
    op.run(gr.MODE_FUSED, b.x, b.w, b.send, b.peers, b.out, b.local, gather=gather)
    torch.cuda.synchronize()
    assert op.status() == gr.OK
    assert np.array_equal(host(b.out), out_o)
    for i, g in enumerate(gather):
        assert np.array_equal(host(g), out_o), f"gather[{i}]"


def test_coresident_alternating_inputs_and_graph_replays():
    base = synthetic.CONFIGS["o_proj"]
    cfgs = [synthetic.Config("alt_a", 1, base.M, base.N, base.K_local),
            synthetic.Config("alt_b", 7, base.M, base.N, base.K_local)]
    rank = 4
    ins = [synthetic.make_inputs(c, "integer") for c in cfgs]
    want = [dev(oracle.gemm_rs(x, w, p, 8, rank)[2]) for x, w, p in ins]
    bufs = [Buffers(x, w, p, base.S, base.N) for x, w, p in ins]
    send, local, out = bufs[0].send, bufs[0].local, bufs[0].out
    fill = np.array(SENTINEL, np.uint16).view(np.int16).item()
    op = gr.GemmRS(base.M, base.N, base.K_local, rank=rank, **CORES)
    bad = 0
    for it in range(40):
        i = it % 2
        local.fill_(fill)
        op.run(gr.MODE_FUSED, bufs[i].x, bufs[i].w, send, bufs[i].peers, out, local)
        if not torch.equal(out, want[i]):
            bad += 1
    torch.cuda.synchronize()
    assert op.status() == gr.OK
    assert bad == 0
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        op.run(gr.MODE_FUSED, bufs[0].x, bufs[0].w, send, bufs[0].peers, out, local)
    torch.cuda.synchronize()
    for it in range(6):
        out.fill_(fill)
        local.fill_(fill)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert op.status() == gr.OK
        assert torch.equal(out, want[0]), it


def test_coresident_watchdog_reports_a_dropped_flag():
    cfg = synthetic.CONFIGS["tiny"]
    rank = 2
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    plan = gr.gemm_rs_plan(gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank))
    sched = oracle.schedule(cfg.M, cfg.N, 8, rank, plan.bm, plan.bn, plan.group_m)
    dropped = int(sched["flag"][0])  # first tile of the own slice: rows [0, bm), columns [0, bn)
    op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, drop_flag=dropped, watchdog_us=2000, **CORES)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b, check_status=False)
    assert op.status() == gr.ERR_TIMEOUT
    _, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    assert np.array_equal(host(b.local), local_o)
    got = host(b.out)
    assert np.all(got[:plan.bm, :plan.bn] == SENTINEL)
    mask = np.ones(got.shape, bool)
    mask[:plan.bm, :plan.bn] = False
    assert np.array_equal(got[mask], out_o[mask])


def test_coresident_rejected_where_no_workgroup_fits_beside():
    cfg = synthetic.CONFIGS["down_proj"]  # 256x256 tile: one workgroup per CU
    with pytest.raises(gr.GemmRSError) as e:
        gr.GemmRS(cfg.M, cfg.N, cfg.K_local, **CORES)
    assert e.value.code == gr.ERR_UNSUPPORTED_SHAPE
