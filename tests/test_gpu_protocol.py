"""GPU tests of the tile routing, the ready-flag protocol and the watchdog."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tensor_gemm_reduce_amd import gemm_rs as gr
from gpu_util import SENTINEL, Buffers, dev, host, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,M,kw", [
    ("tiny", None, {}),
    ("o_proj", None, {}),
    ("mixtral_down", 2048, dict(tile="128x128", group_m=3)),
    ("down_proj", None, dict(flag_stride=32)),
    ("down_proj", None, dict(num_reducers=8)),
    ("mixtral_down", 2048, dict(num_reducers=16, flag_stride=32)),
])
def test_slot_log_and_flags_match_oracle_schedule(name, M, kw):
    cfg = synthetic.CONFIGS[name]
    M = cfg.M if M is None else M
    rank = 3
    x, w, peers = synthetic.make_inputs(cfg, "integer", M=M)
    op = gr.GemmRS(M, cfg.N, cfg.K_local, rank=rank, debug_flags=gr.DEBUG_TRACE, **kw)
    b = Buffers(x, w, peers, M // 8, cfg.N)
    for epoch in (1, 2):
        run(op, b)
        log, flags = op.debug_read()
        info = gr.gemm_rs_query(op.h)
        assert info.epoch == epoch
        sched = oracle.schedule(M, cfg.N, 8, rank, info.bm, info.bn, info.group_m)
        # routing: slot q carried exactly the oracle's tile
        assert np.array_equal(log[:, 0].astype(np.int64), sched["flag"].astype(np.int64))
        # every ready flag holds this run's epoch
        assert np.all(flags == epoch)
        # static slot distribution: the l-th compute workgroup of XCD group x
        # holds position p of every round of C slots, p = l*8 + x (strided
        # split) or the group's block offset + l (contiguous split)
        C = info.compute_wgs
        q = np.arange(info.tiles)
        grp = (log[:, 1] >> 16).astype(np.int64)
        loc = (log[:, 1] & 0xFFFF).astype(np.int64)
        if info.xcd_split:
            pos = loc * 8 + grp
        else:
            gq = info.grid // 8
            rq, rr = divmod(info.reducer_wgs, 8)
            pos = grp * (gq - rq) - np.minimum(grp, rr) + loc
        assert np.all(grp < 8)
        assert np.array_equal(pos, q % C)
        # per compute workgroup, releases happen in slot order
        stamp = log[:, 2].astype(np.uint64) | (log[:, 3].astype(np.uint64) << np.uint64(32))
        for c in range(min(C, info.tiles)):
            s = stamp[c::C]
            assert np.all(s[1:] >= s[:-1]), c


@pytest.mark.parametrize("red", [dict(num_reducers=0), dict(num_reducers=8)], ids=["tail", "reducers8"])
def test_watchdog_reports_a_dropped_flag_and_kernel_exits(red):
    cfg = synthetic.CONFIGS["tiny"]
    rank = 2
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    plan = gr.gemm_rs_plan(gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank))
    sched = oracle.schedule(cfg.M, cfg.N, 8, rank, plan.bm, plan.bn, plan.group_m)
    dropped = int(sched["flag"][0])  # first tile of the own slice
    op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, drop_flag=dropped, watchdog_us=2000, **red)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b, check_status=False)
    assert op.status() == gr.ERR_TIMEOUT
    assert op.status() == gr.OK  # reading the status clears it
    # the routed partial is still complete; only the timed-out tile's sum is missing
    send_o, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    assert np.array_equal(host(b.local), local_o)
    # the dropped tile is the first own-slice tile: rows [0, bm), columns [0, bn)
    got = host(b.out)
    assert np.all(got[:plan.bm, :plan.bn] == SENTINEL)
    # every other tile of the slice was still summed
    mask = np.ones(got.shape, bool)
    mask[:plan.bm, :plan.bn] = False
    assert np.array_equal(got[mask], out_o[mask])
    # a fresh handle on the same buffers runs normally afterwards
    op2 = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank)
    run(op2, b)
    assert np.array_equal(host(b.out), out_o)


def test_reducer_timeout_leaves_the_next_run_whole():
    """One dedicated reducer claims every own tile in turn; the first tile's
    release is dropped, so its wait gives up after the (short) watchdog while
    the rest of the slice takes far longer to sum.  Both runs on the handle
    report the timeout and must sum every other tile: the claim counter of a
    run is never reset while that run may still claim from it."""
    cfg = synthetic.Config("reducer_timeout", 22, 4096, 6144, 256)
    rank = 1
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    plan = gr.gemm_rs_plan(gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank))
    sched = oracle.schedule(cfg.M, cfg.N, 8, rank, plan.bm, plan.bn, plan.group_m)
    dropped = int(sched["flag"][0])  # first own tile: rows [0, bm), columns [0, bn)
    op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, num_reducers=1, drop_flag=dropped, watchdog_us=100)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    _, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    mask = np.ones((cfg.S, cfg.N), bool)
    mask[:plan.bm, :plan.bn] = False
    for it in range(2):
        b.refill()
        run(op, b, check_status=False)
        assert op.status() == gr.ERR_TIMEOUT, it
        assert np.array_equal(host(b.local), local_o), it
        got = host(b.out)
        assert np.all(got[:plan.bm, :plan.bn] == SENTINEL), it
        assert np.array_equal(got[mask], out_o[mask]), it


def test_alternating_inputs_never_read_stale_tiles():
    """Back-to-back fused runs alternate two input sets on shared output
    buffers, with the local slice poisoned before each run: a reducer that read
    a tile before its flag (or a stale copy) would produce a wrong slice."""
    base = synthetic.CONFIGS["o_proj"]
    cfg_a = synthetic.Config("alt_a", 1, base.M, base.N, base.K_local)
    cfg_b = synthetic.Config("alt_b", 7, base.M, base.N, base.K_local)
    rank = 4
    ins = [synthetic.make_inputs(c, "integer") for c in (cfg_a, cfg_b)]
    want = [dev(oracle.gemm_rs(x, w, p, 8, rank)[2]) for x, w, p in ins]
    bufs = [Buffers(x, w, p, base.S, base.N) for x, w, p in ins]
    shared_send, shared_local, shared_out = bufs[0].send, bufs[0].local, bufs[0].out
    for kw in (dict(num_reducers=0), dict(num_reducers=0, tile="128x128"), dict(num_reducers=8),
               dict(num_reducers=1), dict(num_reducers=3, tile="128x128"), dict(tile_stores="nt"),
               dict(num_reducers=8, tile_stores="nt"), dict(flag_protocol="row_counter"),
               dict(num_reducers=8, flag_protocol="row_counter")):
        op = gr.GemmRS(base.M, base.N, base.K_local, rank=rank, **kw)
        bad = 0
        for it in range(40):
            i = it % 2
            shared_local.fill_(np.array(SENTINEL, np.uint16).view(np.int16).item())
            op.run(gr.MODE_FUSED, bufs[i].x, bufs[i].w, shared_send, bufs[i].peers, shared_out,
                   shared_local)
            if not torch.equal(shared_out, want[i]):
                bad += 1
        torch.cuda.synchronize()
        assert op.status() == gr.OK
        assert bad == 0, (kw, bad)


@pytest.mark.parametrize("red", [dict(num_reducers=0), dict(num_reducers=8)], ids=["tail", "reducers8"])
def test_graph_replays_match_eager(red):
    """Runs captured into a HIP graph and replayed are new runs each time (the
    epoch and counters live on the device): every replay, with eager runs and
    synchronisations in between, must give the eager result."""
    cfg = synthetic.CONFIGS["o_proj"]
    rank = 6
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    want = dev(oracle.gemm_rs(x, w, peers, 8, rank)[2])
    op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, **red)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    fill = np.array(SENTINEL, np.uint16).view(np.int16).item()
    run(op, b)
    assert torch.equal(b.out, want)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        op.run(gr.MODE_FUSED, b.x, b.w, b.send, b.peers, b.out, b.local)
    torch.cuda.synchronize()
    for it in range(6):
        b.out.fill_(fill)
        b.local.fill_(fill)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert op.status() == gr.OK
        assert torch.equal(b.out, want), it
        if it % 2:
            run(op, b)  # an eager run between replays
            assert torch.equal(b.out, want)
    assert gr.gemm_rs_query(op.h).epoch == 1 + 6 + 3


ROWC = synthetic.Config("rowc", 21, 8 * 64, 1024, 128)


@pytest.mark.parametrize("kw", [dict(), dict(num_reducers=8), dict(flag_stride=32)], ids=["tail", "reducers8", "padded"])
def test_row_counters_count_every_tile_of_every_run(kw):
    """Under the row-counter protocol each (destination slice, tile row) word
    holds runs x tile columns after every run, and the words past the last
    tile row stay zero."""
    cfg = ROWC  # four tile rows per slice
    rank = 3
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    want = oracle.gemm_rs(x, w, peers, 8, rank)[2]
    op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, tile="16x64", flag_protocol="row_counter", **kw)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    info = op.info
    rows = 8 * info.tile_rows_per_slice
    for epoch in (1, 2, 3):
        b.refill()
        run(op, b)
        assert np.array_equal(host(b.out), want)
        _, words = op.debug_read()
        assert np.all(words[:rows] == epoch * info.tile_cols), (epoch, words[:rows])
        assert np.all(words[rows:] == 0)


@pytest.mark.parametrize("red", [dict(num_reducers=0), dict(num_reducers=8)], ids=["tail", "reducers8"])
def test_row_counter_watchdog_skips_the_dropped_row(red):
    """A tile whose release is dropped leaves its row's counter one short: the
    watchdog reports it and the sum skips that whole tile row of the slice;
    every other row is summed."""
    cfg = ROWC  # four tile rows per slice
    rank = 2
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    plan = gr.gemm_rs_plan(gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank, tile="16x64"))
    assert plan.tile_rows_per_slice == 4
    sched = oracle.schedule(cfg.M, cfg.N, 8, rank, plan.bm, plan.bn, plan.group_m)
    dropped = int(sched["flag"][0])  # first tile of the own slice: tile row 0
    op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, tile="16x64", drop_flag=dropped, watchdog_us=2000,
                   flag_protocol="row_counter", **red)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b, check_status=False)
    assert op.status() == gr.ERR_TIMEOUT
    send_o, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    assert np.array_equal(host(b.local), local_o)
    got = host(b.out)
    assert np.all(got[:plan.bm] == SENTINEL)
    assert np.array_equal(got[plan.bm:], out_o[plan.bm:])
