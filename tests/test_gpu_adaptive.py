"""GPU tests of the adaptive controller (reduce_mode "adaptive", or
num_reducers = -2): every compute workgroup sums slice units at its tile
boundaries, as many per boundary as the controller's target gives, and the
last boundary sums what is left.  Who sums which unit changes from run to run;
the sum of each element does not, so every run must equal the oracle bit for
bit on integer inputs.  The slice-sum stamps of a traced run show the units
summed between the tiles: some own tiles are summed before the GEMM's last
tile is released.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tensor_gemm_reduce_amd import gemm_rs as gr
from gpu_util import SENTINEL, Buffers, dev, filled, host, run

pytestmark = pytest.mark.gpu

# four rounds of 256x256 tiles on 256 CUs, the own slice in the first; and a
# ragged shape (tile rows, columns and K all ragged) of about four and a half
SHAPES = {
    "four_rounds": synthetic.Config("adaptive4", 19, 8 * 1024, 8192, 256),
    "ragged": synthetic.Config("adaptive_rag", 29, 8 * 1500, 6000, 136),
}


def _op(cfg, rank, **kw):
    return gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, reduce_mode="adaptive", **kw)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("rank", [0, 5])
def test_adaptive_runs_equal_the_oracle(name, rank):
    cfg = SHAPES[name]
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    _, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    want = dev(out_o)
    op = _op(cfg, rank)
    info = op.info
    assert info.reduce_mode == gr.REDUCE_ADAPTIVE and info.split_state == 1 and info.reducer_wgs == 0
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    fill = np.array(SENTINEL, np.uint16).view(np.int16).item()
    for it in range(4):
        b.out.fill_(fill)
        run(op, b)
        assert torch.equal(b.out, want), it
    assert np.array_equal(host(b.local), local_o)
    # from a graph, replayed with eager work between the replays
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        op.run(gr.MODE_FUSED, b.x, b.w, b.send, b.peers, b.out, b.local)
    torch.cuda.synchronize()
    for it in range(3):
        b.out.fill_(fill)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert op.status() == gr.OK
        assert torch.equal(b.out, want), it


def test_adaptive_equals_the_num_reducers_spelling_and_the_tail():
    cfg = SHAPES["four_rounds"]
    rank = 3
    x, w, peers = synthetic.make_inputs(cfg, "normal")
    outs = []
    for kw in (dict(reduce_mode="adaptive"), dict(num_reducers=-2), dict(reduce_mode="tail")):
        op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, **kw)
        b = Buffers(x, w, peers, cfg.S, cfg.N)
        run(op, b)
        outs.append([host(t) for t in b.send + [b.local, b.out]])
    for i in range(len(outs[0])):
        assert np.array_equal(outs[0][i], outs[1][i]), i
        assert np.array_equal(outs[0][i], outs[2][i]), i


def test_adaptive_single_round_sums_at_the_end():
    for name in ("tiny", "o_proj"):
        cfg = synthetic.CONFIGS[name]
        x, w, peers = synthetic.make_inputs(cfg, "integer")
        want = oracle.gemm_rs(x, w, peers, tp=8, rank=2)[2]
        op = _op(cfg, 2)
        b = Buffers(x, w, peers, cfg.S, cfg.N)
        run(op, b)
        assert np.array_equal(host(b.out), want), name


def test_adaptive_sum_stamps_show_units_between_the_tiles():
    cfg = SHAPES["four_rounds"]
    rank = 1
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    want = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)[2]
    op = _op(cfg, rank, debug_flags=gr.DEBUG_TRACE)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b)
    run(op, b)  # (stamps of the second run: the first one's are cleared)
    assert np.array_equal(host(b.out), want)
    log, flags, stamps, launch = op.debug_read(sums=True)
    info = op.info
    ipt = info.bm * info.bn // 512
    assert np.all(stamps[:, 3] == ipt)  # every item of every own tile, once
    d = lambda a, b: (a.astype(np.int64) - b.astype(np.int64) + (1 << 31)) % (1 << 32) - (1 << 31)
    poll, acq, done = stamps[:, 0], stamps[:, 1], stamps[:, 2]
    assert np.all(d(acq, poll) >= 0) and np.all(d(done, acq) >= 0)
    # acquire after the tile's release (slot log: flag index, ticket, time)
    rel = {int(f): int(t) for f, t in zip(log[:, 0], log[:, 2])}
    own = [rel[rank * info.tiles_per_slice + t] for t in range(info.tiles_per_slice)]
    assert np.all(d(acq, np.array(own, np.uint32)) >= 0)
    assert np.all(d(poll, np.full_like(poll, launch[0])) >= 0)
    assert np.all(d(np.full_like(done, launch[2]), done) >= 0)
    # units summed at the boundaries: some own tiles are done before the last
    # tile of the GEMM is released
    release = log[:, 2].astype(np.int64) | (log[:, 3].astype(np.int64) << 32)
    last = np.uint32(int(release.max()) & 0xFFFFFFFF)
    early = np.sum(d(done, np.full_like(done, last)) < 0)
    assert early > 0, early


def test_adaptive_all_reduce_stores_every_gather_buffer():
    cfg = SHAPES["four_rounds"]
    rank = 6
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    want = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)[2]
    op = _op(cfg, rank)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    g = [filled((cfg.S, cfg.N)) for _ in range(7)]
    op.run(gr.MODE_FUSED, b.x, b.w, b.send, b.peers, b.out, b.local, gather=g)
    torch.cuda.synchronize()
    assert op.status() == gr.OK
    assert np.array_equal(host(b.out), want)
    for i, t in enumerate(g):
        assert np.array_equal(host(t), want), i


def test_adaptive_dropped_flag_times_out_and_the_rest_is_summed():
    """A tile whose flag is never released: the waves that claimed its units
    give up after the watchdog and report it; every other element is summed."""
    cfg = SHAPES["four_rounds"]
    rank = 2
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    plan = gr.gemm_rs_plan(gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank, reduce_mode="adaptive"))
    sched = oracle.schedule(cfg.M, cfg.N, 8, rank, plan.bm, plan.bn, plan.group_m)
    dropped = int(sched["flag"][0])  # own tile 0: rows [0, bm), columns [0, bn)
    op = _op(cfg, rank, drop_flag=dropped, watchdog_us=2000)
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
