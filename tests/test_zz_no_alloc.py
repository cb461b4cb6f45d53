"""GPU tests of gemm_rs_run_static, the run that allocates nothing: its
results equal gemm_rs_run's on the same config and buffers, on two calls in a
row (the second smaller, so that the static scratch keeps the first call's
contents), under graph capture, and its status words report a watchdog
timeout."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tensor_gemm_reduce_amd import gemm_rs as gr
from gpu_util import SENTINEL, Buffers, host, run

pytestmark = pytest.mark.gpu

BIG = synthetic.Config("static_big", 31, 2048, 6144, 512)     # 256x256 tiles, 8 rounds' worth of flags
SMALL = synthetic.Config("static_small", 32, 512, 1024, 256)  # 64x128 tiles, two workgroups per CU


def _ptrs(b):
    return (b.x.data_ptr(), b.w.data_ptr(), [t.data_ptr() for t in b.send], [t.data_ptr() for t in b.peers],
            b.out.data_ptr(), b.local.data_ptr())


def _run_static(cfg, b, mode=gr.MODE_FUSED, status=None, stream=None):
    x, w, send, peers, out, local = _ptrs(b)
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    return gr.gemm_rs_run_static(cfg, mode, x, w, send, peers, out, local,
                                 status.data_ptr() if status is not None else None, s)


def _outputs(b):
    return [host(t) for t in b.send + [b.local, b.out]]


@pytest.mark.parametrize("kw", [dict(), dict(num_reducers=8), dict(flag_stride=32, tile_stores="nt"),
                                dict(flag_protocol="row_counter"), dict(reduce_mode="adaptive")],
                         ids=["tail", "reducers8", "padded_nt", "rowc", "adaptive"])
def test_static_runs_equal_handle_runs_big_then_small(kw):
    status = torch.full((2,), -99, dtype=torch.int32, device="cuda")
    for cfg, rank, mode in ((BIG, 3, "normal"), (SMALL, 6, "integer")):
        x, w, peers = synthetic.make_inputs(cfg, mode)
        c = gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank, **kw)
        b = Buffers(x, w, peers, cfg.S, cfg.N)
        for mode_ in (gr.MODE_FUSED, gr.MODE_SEQUENTIAL):
            b.refill()
            assert _run_static(c, b, mode_, status) == gr.OK
            torch.cuda.synchronize()
            assert status.tolist() == [0, 0]
            got = _outputs(b)
            op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, **kw)
            b.refill()
            run(op, b, mode_)
            want = _outputs(b)
            op.close()
            for i, (g_, w_) in enumerate(zip(got, want)):
                assert np.array_equal(g_, w_), (cfg.name, mode_, i)
        if mode == "integer":
            send_o, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
            assert np.array_equal(got[7], local_o) and np.array_equal(got[8], out_o)


def test_static_runs_under_graph_capture():
    cfg, rank = BIG, 5
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    c = gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    want = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)[2]
    status = torch.zeros((2,), dtype=torch.int32, device="cuda")
    assert _run_static(c, b, status=status) == gr.OK
    torch.cuda.synchronize()
    assert np.array_equal(host(b.out), want)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        assert _run_static(c, b, status=status, stream=stream.cuda_stream) == gr.OK
    torch.cuda.synchronize()
    small = synthetic.make_inputs(SMALL, "integer")
    bs = Buffers(*small, SMALL.S, SMALL.N)
    cs = gr.make_config(SMALL.M, SMALL.N, SMALL.K_local, rank=1)
    for it in range(5):
        b.refill()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert status.tolist() == [0, 0], it
        assert np.array_equal(host(b.out), want), it
        # an eager call of another shape between replays (the scratch is shared)
        assert _run_static(cs, bs) == gr.OK
        torch.cuda.synchronize()
        assert np.array_equal(host(bs.out), oracle.gemm_rs(*small, tp=8, rank=1)[2])


def test_static_status_reports_a_dropped_flag():
    cfg, rank = SMALL, 2
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    plan = gr.gemm_rs_plan(gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank))
    sched = oracle.schedule(cfg.M, cfg.N, 8, rank, plan.bm, plan.bn, plan.group_m)
    dropped = int(sched["flag"][0])
    c = gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank, drop_flag=dropped, watchdog_us=2000)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    status = torch.zeros((2,), dtype=torch.int32, device="cuda")
    assert _run_static(c, b, status=status) == gr.OK
    torch.cuda.synchronize()
    assert status.tolist() == [gr.ERR_TIMEOUT, dropped]
    out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)[2]
    got = host(b.out)
    assert np.all(got[:plan.bm, :plan.bn] == SENTINEL)
    mask = np.ones(got.shape, bool)
    mask[:plan.bm, :plan.bn] = False
    assert np.array_equal(got[mask], out_o[mask])
    # the next call starts from cleared state
    c2 = gr.make_config(cfg.M, cfg.N, cfg.K_local, rank=rank)
    b.refill()
    assert _run_static(c2, b, status=status) == gr.OK
    torch.cuda.synchronize()
    assert status.tolist() == [0, 0]
    assert np.array_equal(host(b.out), out_o)


def test_static_argument_checks():
    cfg = SMALL
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    c = gr.make_config(cfg.M, cfg.N, cfg.K_local)
    xp, wp, send, pp, out, local = _ptrs(b)
    s = torch.cuda.current_stream().cuda_stream
    assert gr.gemm_rs_run_static(c, gr.MODE_FUSED, xp, wp, send, pp, out, None, None, s) == gr.ERR_INVALID_ARG
    assert gr.gemm_rs_run_static(c, 9, xp, wp, send, pp, out, local, None, s) == gr.ERR_INVALID_ARG
    assert gr.gemm_rs_run_static(c, gr.MODE_FUSED, xp + 2, wp, send, pp, out, local, None, s) == gr.ERR_MISALIGNED
    traced = gr.make_config(cfg.M, cfg.N, cfg.K_local, debug_flags=gr.DEBUG_TRACE)
    assert gr.gemm_rs_run_static(traced, gr.MODE_FUSED, xp, wp, send, pp, out, local, None, s) == gr.ERR_INVALID_ARG
    # ready flags beyond the static array: 16384 tiles of 128x128, each padded to 128 bytes
    big = gr.make_config(32768, 8192, 64, tile="128x128", flag_stride=32)
    assert gr.gemm_rs_run_static(big, gr.MODE_FUSED, None, None, None, None, None, local, None, s) == gr.ERR_SCRATCH
    assert "static" in gr.gemm_rs_strerror(gr.ERR_SCRATCH)
    torch.cuda.synchronize()
