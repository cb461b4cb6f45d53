"""GPU tests of the stream kernel (reduce_mode "stream"): four loader waves
and four stream waves per compute workgroup, the slice sum streamed through
the K loop once the workgroup's own tiles are released, the rest summed after
the last tile.  Shapes cover one round (nothing can stream: all in the
drain), several rounds (the stream latches in a later round), ragged tiles,
and tiles long enough for the stream's groups to run; every result is
compared with the oracle bit for bit (integer inputs) or with the sum after
the last tile (normal inputs, same sum order)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tensor_gemm_reduce_amd import gemm_rs as gr
from gpu_util import SENTINEL, Buffers, dev, host, run

pytestmark = pytest.mark.gpu

STREAM = dict(reduce_mode="stream")
SHAPES = {
    # S = 256: 8 own tiles, 64 tiles in all: one round
    "one_round": synthetic.Config("st_one", 41, 8 * 256, 2048, 512),
    # S = 512: 64 own tiles of 512: two rounds (own tiles in the first)
    "two_rounds": synthetic.Config("st_two", 42, 8 * 512, 8192, 384),
    # S = 2048: 128 own tiles of 1024: four rounds
    "four_rounds": synthetic.Config("st_four", 43, 8 * 2048, 4096, 512),
    # S = 384 (a ragged tile row), N = 4160 (a ragged tile column), 7 K steps
    "ragged": synthetic.Config("st_ragged", 44, 8 * 384, 4160, 448),
}

# Shapes whose tiles are long enough for the stream's groups (four K steps
# each after the probe): with many later tiles the groups begin at a tile's
# start; with few (three rounds) they begin inside the tile whose probe
# latches, after a later probe if the first one came too early.
GROUP_SHAPES = {
    # S = 2048, 128 own tiles of 1024 (four rounds), 48 K steps
    "from_tile_start": synthetic.Config("st_groups_a", 47, 8 * 2048, 4096, 3072),
    # S = 1024, 96 own tiles of 768 (three rounds), 32 K steps
    "in_latching_tile": synthetic.Config("st_groups_b", 48, 8 * 1024, 6144, 2048),
}


def _op(cfg, rank, **kw):
    return gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, **kw)


def test_stream_mode_is_resolved():
    cfg = SHAPES["two_rounds"]
    op = _op(cfg, 0, **STREAM)
    assert op.info.reduce_mode == gr.REDUCE_STREAM
    assert (op.info.bm, op.info.bn) == (256, 256)


@pytest.mark.parametrize("rank", [0, 5])
@pytest.mark.parametrize("name", list(SHAPES))
def test_stream_integer_bit_exact(name, rank):
    cfg = SHAPES[name]
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    op = _op(cfg, rank, **STREAM)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b)
    send_o, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    for i in range(7):
        assert np.array_equal(host(b.send[i]), send_o[i]), f"send[{i}]"
    assert np.array_equal(host(b.local), local_o)
    assert np.array_equal(host(b.out), out_o)


@pytest.mark.parametrize("name", ["two_rounds", "four_rounds", "ragged"])
def test_stream_equals_tail_on_normal_inputs(name):
    cfg = SHAPES[name]
    rank = 3
    x, w, peers = synthetic.make_inputs(cfg, "normal")
    got = {}
    for kw in (STREAM, dict(reduce_mode="tail")):
        op = _op(cfg, rank, **kw)
        b = Buffers(x, w, peers, cfg.S, cfg.N)
        run(op, b)
        got[kw["reduce_mode"]] = [host(t) for t in b.send + [b.local, b.out]]
    for i, (s_, t_) in enumerate(zip(got["stream"], got["tail"])):
        assert np.array_equal(s_, t_), i
    assert np.array_equal(got["stream"][8], oracle.slice_sum(got["stream"][7], peers, tp=8))


@pytest.mark.parametrize("name", ["four_rounds", "in_latching_tile"])
def test_stream_alternating_inputs_and_graph_replays(name):
    """Back-to-back runs alternate two input sets on shared outputs with the
    local slice poisoned before each run (a stream wave that read a tile
    before its release, or a stale copy, would give a wrong slice); then a
    captured run is replayed with eager runs in between."""
    base = {**SHAPES, **GROUP_SHAPES}[name]
    cfgs = [synthetic.Config("st_alt_a", 45, base.M, base.N, base.K_local),
            synthetic.Config("st_alt_b", 46, base.M, base.N, base.K_local)]
    rank = 6
    ins = [synthetic.make_inputs(c, "integer") for c in cfgs]
    want = [dev(oracle.gemm_rs(x, w, p, 8, rank)[2]) for x, w, p in ins]
    bufs = [Buffers(x, w, p, base.S, base.N) for x, w, p in ins]
    send, local, out = bufs[0].send, bufs[0].local, bufs[0].out
    fill = np.array(SENTINEL, np.uint16).view(np.int16).item()
    op = _op(base, rank, **STREAM)
    bad = 0
    for it in range(16):
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
    for it in range(4):
        out.fill_(fill)
        local.fill_(fill)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert op.status() == gr.OK
        assert torch.equal(out, want[0]), it
        op.run(gr.MODE_FUSED, bufs[1].x, bufs[1].w, send, bufs[1].peers, out, local)
        torch.cuda.synchronize()
        assert torch.equal(out, want[1]), it


def test_stream_watchdog_reports_a_dropped_flag():
    """The first own tile's release is dropped: the workgroups whose items lie
    in it never latch, their items go to the sum after the last tile, whose
    wait reports the timeout; every other tile is summed."""
    cfg = SHAPES["two_rounds"]
    rank = 2
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    plan = gr.gemm_rs_plan(gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank, **STREAM))
    sched = oracle.schedule(cfg.M, cfg.N, 8, rank, plan.bm, plan.bn, plan.group_m)
    dropped = int(sched["flag"][0])  # own tile 0: rows [0, bm), columns [0, bn)
    op = _op(cfg, rank, drop_flag=dropped, watchdog_us=2000, **STREAM)
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


def test_stream_modes_agree_and_all_reduce_sums_after_the_last_tile():
    """FUSED equals SEQUENTIAL on a stream handle; the all-reduce's FUSED run
    on the same handle (whose sum also stores every gather buffer) runs the
    sum after the last tile and gives the same slice in out and in gather[]."""
    cfg = SHAPES["two_rounds"]
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    op = _op(cfg, 1, **STREAM)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b, gr.MODE_FUSED)
    fused = [host(t) for t in b.send + [b.local, b.out]]
    b.refill()
    run(op, b, gr.MODE_SEQUENTIAL)
    for i, t in enumerate(b.send + [b.local, b.out]):
        assert np.array_equal(host(t), fused[i]), i
    b.refill()
    g = [torch.full((cfg.S, cfg.N), SENTINEL, dtype=torch.int16, device="cuda") for _ in range(7)]
    op.run(gr.MODE_FUSED, b.x, b.w, b.send, b.peers, b.out, b.local, gather=g)
    torch.cuda.synchronize()
    assert op.status() == 0
    for i, t in enumerate(b.send + [b.local, b.out]):
        assert np.array_equal(host(t), fused[i]), i
    for i, t in enumerate(g):
        assert np.array_equal(host(t), fused[-1]), i
    # and the stream kernel again after it
    b.refill()
    run(op, b, gr.MODE_FUSED)
    assert np.array_equal(host(b.out), fused[-1])


@pytest.mark.parametrize("name", list(GROUP_SHAPES))
def test_stream_groups_sum_the_slice_during_the_gemm(name):
    """Bit-exact on integer inputs, and the slice-sum stamps of a traced run
    show most own tiles summed before the GEMM's last tile is released (the
    sum after the last tile alone would finish none of them before it)."""
    cfg = GROUP_SHAPES[name]
    rank = 4
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    _, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    op = _op(cfg, rank, debug_flags=gr.DEBUG_TRACE, **STREAM)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b)
    run(op, b)  # (stamps of the second run)
    assert np.array_equal(host(b.local), local_o)
    assert np.array_equal(host(b.out), out_o)
    log, flags, stamps, launch = op.debug_read(sums=True)
    info = op.info
    assert np.all(stamps[:, 3] == info.bm * info.bn // 512)
    d = lambda p, q: (p.astype(np.int64) - q.astype(np.int64) + (1 << 31)) % (1 << 32) - (1 << 31)
    release = log[:, 2].astype(np.int64) | (log[:, 3].astype(np.int64) << 32)
    last = np.uint32(int(release.max()) & 0xFFFFFFFF)
    done = stamps[:, 2]
    early = int(np.sum(d(done, np.full_like(done, last)) < 0))
    assert early >= len(done) // 2, (early, len(done))
