"""GPU tests of the reduce stream: the slice sum issued one operation per K
step from inside the pipelined 256x256 K loop (reduce_mode "stream").

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

STREAM = dict(num_reducers=0, reduce_mode="stream", tile="256x256")
TAIL = dict(num_reducers=0, reduce_mode="tail", tile="256x256")

# ragged: S = 264 and N = 392 leave partial last tiles, K_local = 136 a partial
# last K step (one round of 32 tiles); two rounds: T = 512 tiles on 256
# workgroups, 8 K steps per tile, so items are both streamed and drained
SHAPES = {
    "ragged": synthetic.Config("ragged", 5, 8 * 264, 392, 136),
    "two_rounds": synthetic.Config("two_rounds", 6, 8192, 4096, 512),
}


def _outputs(b):
    return [host(t) for t in b.send + [b.local, b.out]]


def test_stream_is_chosen_only_on_request():
    cfg = SHAPES["two_rounds"]
    info = gr.gemm_rs_plan(gr.make_config(cfg.M, cfg.N, cfg.K_local, num_reducers=0))
    assert (info.bm, info.bn) == (256, 256)
    assert info.reduce_mode == gr.REDUCE_TAIL
    info = gr.gemm_rs_plan(gr.make_config(cfg.M, cfg.N, cfg.K_local, **STREAM))
    assert info.reduce_mode == gr.REDUCE_STREAM


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("rank", [0, 5])
def test_stream_integer_bit_exact(name, rank):
    cfg = SHAPES[name]
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, **STREAM)
    assert op.info.reduce_mode == gr.REDUCE_STREAM
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b)
    send_o, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    got = _outputs(b)
    for i in range(7):
        assert np.array_equal(got[i], send_o[i]), f"send[{i}]"
    assert np.array_equal(got[7], local_o)
    assert np.array_equal(got[8], out_o)


@pytest.mark.parametrize("name", list(SHAPES))
def test_stream_equals_tail_on_normal_inputs(name):
    cfg = SHAPES[name]
    x, w, peers = synthetic.make_inputs(cfg, "normal")
    res = []
    for kw in (STREAM, TAIL):
        op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=3, **kw)
        b = Buffers(x, w, peers, cfg.S, cfg.N)
        run(op, b)
        res.append(_outputs(b))
        op.close()
    for a_, t_ in zip(*res):
        assert np.array_equal(a_, t_)
    # and the sum is the oracle's sum of the GPU's own partial
    assert np.array_equal(res[0][8], oracle.slice_sum(res[0][7], peers))


def test_stream_all_reduce_gathers_equal_out():
    cfg = SHAPES["two_rounds"]
    rank = 2
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, **STREAM)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    gather = [filled((cfg.S, cfg.N)) for _ in range(7)]
    op.run(gr.MODE_FUSED, b.x, b.w, b.send, b.peers, b.out, b.local, gather=gather)
    torch.cuda.synchronize()
    assert op.status() == gr.OK
    _, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    assert np.array_equal(host(b.local), local_o)
    assert np.array_equal(host(b.out), out_o)
    for i, g in enumerate(gather):
        assert np.array_equal(host(g), out_o), f"gather[{i}]"


def test_stream_alternating_inputs_and_graph_replays():
    """Back-to-back runs alternate two input sets with the local slice
    poisoned before each run (a sum that read a tile before its flag, or a
    stale copy, would differ), then the same runs replayed from a graph."""
    base = SHAPES["two_rounds"]
    cfgs = [synthetic.Config("alt_a", 8, base.M, base.N, base.K_local),
            synthetic.Config("alt_b", 9, base.M, base.N, base.K_local)]
    rank = 4
    ins = [synthetic.make_inputs(c, "integer") for c in cfgs]
    want = [dev(oracle.gemm_rs(x, w, p, 8, rank)[2]) for x, w, p in ins]
    bufs = [Buffers(x, w, p, base.S, base.N) for x, w, p in ins]
    send, local, out = bufs[0].send, bufs[0].local, bufs[0].out
    fill = np.array(SENTINEL, np.uint16).view(np.int16).item()
    op = gr.GemmRS(base.M, base.N, base.K_local, rank=rank, **STREAM)
    bad = 0
    for it in range(12):
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
        op.run(gr.MODE_FUSED, bufs[1].x, bufs[1].w, send, bufs[1].peers, out, local)
    torch.cuda.synchronize()
    for it in range(4):
        out.fill_(fill)
        local.fill_(fill)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert op.status() == gr.OK
        assert torch.equal(out, want[1]), it


def test_stream_watchdog_reports_a_dropped_flag():
    cfg = SHAPES["two_rounds"]
    rank = 1
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    plan = gr.gemm_rs_plan(gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank, **STREAM))
    sched = oracle.schedule(cfg.M, cfg.N, 8, rank, plan.bm, plan.bn, plan.group_m)
    dropped = int(sched["flag"][0])  # first tile of the own slice
    t = dropped - rank * plan.tiles_per_slice
    tr, tc = divmod(t, plan.tile_cols)
    op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, drop_flag=dropped, watchdog_us=2000, **STREAM)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b, check_status=False)
    assert op.status() == gr.ERR_TIMEOUT
    _, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    assert np.array_equal(host(b.local), local_o)
    got = host(b.out)
    rs, cs = slice(tr * plan.bm, (tr + 1) * plan.bm), slice(tc * plan.bn, (tc + 1) * plan.bn)
    assert np.all(got[rs, cs] == SENTINEL)
    mask = np.ones(got.shape, bool)
    mask[rs, cs] = False
    assert np.array_equal(got[mask], out_o[mask])
