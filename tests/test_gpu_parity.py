"""GPU parity of the fused kernel against the CPU oracle, through the C ABI.

Sizes the oracle finishes in seconds are compared element by element; the
full benchmark shapes are compared on sampled rows (several tiles and the
slice edges) in the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tensor_gemm_reduce_amd import gemm_rs as gr
from gpu_util import (Buffers, SENTINEL, assert_close_partial, host, max_rel, oracle_rows, run,
                      sample_rows)

pytestmark = pytest.mark.gpu

# how the slice is reduced: by the compute workgroups after their last tile
# (default) or by 8 dedicated reducer workgroups
REDUCE = {"tail": dict(num_reducers=0), "reducers8": dict(num_reducers=8)}
REDUCERS = list(REDUCE)
# the automatic placement with the routed tiles stored non-temporally, and
# with device-scope stores only (the automatic store policy picks the
# non-temporal hint for the 256x256 tile when the sum runs after the tiles)
REDUCE["nt"] = dict(tile_stores="nt")
REDUCE["device"] = dict(tile_stores="device")
# the sum streamed through the K loop by four of the eight waves (256x256 tile)
REDUCE["stream"] = dict(reduce_mode="stream")
# the automatic placement with a released-tile counter per tile row
REDUCE["rowc"] = dict(flag_protocol="row_counter")
# the adaptive controller: units of the sum between the tiles
REDUCE["adaptive"] = dict(reduce_mode="adaptive")


def _op(cfg, M=None, **kw):
    M = cfg.M if M is None else M
    return gr.GemmRS(M, cfg.N, cfg.K_local, **kw)


def _full_compare(cfg, mode, rank, **kw):
    x, w, peers = synthetic.make_inputs(cfg, mode)
    op = _op(cfg, rank=rank, **kw)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b)
    send_o, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=rank)
    return op, b, (x, w, peers), (send_o, local_o, out_o)


# ------------------------------------------------------------------ exact (integer inputs)

@pytest.mark.parametrize("red", REDUCERS)
@pytest.mark.parametrize("rank", range(8))
def test_tiny_integer_bit_exact_all_ranks(rank, red):
    cfg = synthetic.CONFIGS["tiny"]
    op, b, _, (send_o, local_o, out_o) = _full_compare(cfg, "integer", rank, **REDUCE[red])
    for i in range(7):
        assert np.array_equal(host(b.send[i]), send_o[i]), f"send[{i}]"
    assert np.array_equal(host(b.local), local_o)
    assert np.array_equal(host(b.out), out_o)


@pytest.mark.parametrize("red", REDUCERS + ["device"])
@pytest.mark.parametrize("tile", ["16x64", "64x128", "128x128", "128x256", "256x128", "256x256"])
def test_every_tile_config_integer_bit_exact(tile, red):
    # ragged: S = 264 is not a multiple of any BM > 8 and N = 392 of no BN;
    # K_local = 136 leaves a partial last K step
    cfg = synthetic.Config("ragged", 5, 8 * 264, 392, 136)
    op, b, _, (send_o, local_o, out_o) = _full_compare(cfg, "integer", 5, tile=tile, **REDUCE[red])
    for i in range(7):
        assert np.array_equal(host(b.send[i]), send_o[i]), f"send[{i}]"
    assert np.array_equal(host(b.local), local_o)
    assert np.array_equal(host(b.out), out_o)


@pytest.mark.parametrize("k_local", [8, 40, 72])
@pytest.mark.parametrize("tile", ["16x64", "64x128", "128x128", "128x256", "256x128", "256x256"])
def test_short_k_every_tile_integer_bit_exact(tile, k_local):
    # one, two or three K steps, the last one partial (BK is 32, 64 or 128)
    cfg = synthetic.Config("short_k", 5, 8 * 264, 392, k_local)
    op, b, _, (send_o, local_o, out_o) = _full_compare(cfg, "integer", 2, tile=tile, num_reducers=0)
    for i in range(7):
        assert np.array_equal(host(b.send[i]), send_o[i]), f"send[{i}]"
    assert np.array_equal(host(b.local), local_o)
    assert np.array_equal(host(b.out), out_o)


def test_reduce_scatter_invariant_consistent_peers():
    """Peers are the other ranks' real partials: out must equal slice `rank` of
    the unsharded product (exact with integer inputs)."""
    cfg = synthetic.CONFIGS["tiny"]
    shards = synthetic.make_shards(cfg, integer=True)
    S, N, rank = cfg.S, cfg.N, 6
    parts = [oracle.gemm_rs(xp, wp, [np.zeros((S, N), np.uint16)] * 7, 8, p)
             for p, (xp, wp) in enumerate(shards)]
    peers = []
    for i in range(7):
        p = oracle.peer_rank(rank, i)
        peers.append(parts[p][0][rank if rank < p else rank - 1])
    x, w = shards[rank]
    op = _op(cfg, rank=rank)
    b = Buffers(x, w, peers, S, N)
    run(op, b)
    X = np.concatenate([oracle.bf16_to_f32(s[0]).astype(np.int64) for s in shards], axis=1)
    W = np.concatenate([oracle.bf16_to_f32(s[1]).astype(np.int64) for s in shards], axis=1)
    full = (X @ W.T)[rank * S:(rank + 1) * S]
    got = oracle.bf16_to_f32(host(b.out)).astype(np.float64)
    # the exact integer sum, rounded once to BF16 by the oracle's codec
    want = oracle.f32_to_bf16(full.astype(np.float32))
    assert np.array_equal(host(b.out), want)
    assert np.all(np.abs(got - full) <= np.abs(full) * 2.0 ** -8)


# ------------------------------------------------------------------ random inputs, full compare

@pytest.mark.parametrize("red", REDUCERS)
@pytest.mark.parametrize("name", ["tiny", "o_proj"])
@pytest.mark.parametrize("mode", ["normal", "balanced"])
def test_full_compare_within_tolerance(name, mode, red):
    cfg = synthetic.CONFIGS[name]
    rank = 5
    op, b, (x, w, peers), (send_o, local_o, out_o) = _full_compare(cfg, mode, rank, **REDUCE[red])
    S = cfg.S
    rows = np.arange(S)
    for i in range(7):
        d = oracle.peer_rank(rank, i)
        assert_close_partial(host(b.send[i]), send_o[i], x, w, d * S + rows)
    assert_close_partial(host(b.local), local_o, x, w, rank * S + rows)
    # reduce stage bit-exact given the GPU's own local slice
    out_given_local = oracle.slice_sum(host(b.local), peers, tp=8)
    assert np.array_equal(host(b.out), out_given_local)
    ref = oracle.ref_f64(x, w, peers, tp=8, rank=rank)
    assert max_rel(host(b.out), ref) <= 1e-2
    assert max_rel(out_o, ref) <= 1e-2


@pytest.mark.parametrize("name", ["tiny", "o_proj", "down_proj", "mixtral_down", "large_prefill"])
@pytest.mark.parametrize("mode", ["normal", "balanced"])
def test_error_within_1p1x_of_unfused_path(name, mode):
    """Fused `out` and local slice against the FP64 reference: no worse than
    1.1x the error of the unfused path (the vendor GEMM with BF16 output,
    then the standalone reduce kernel over its slice), same statistic.  The
    benchmark's launch configuration; slices above 256 rows are compared on
    sampled rows (tile edges, slice edges and random rows)."""
    import torch

    cfg = synthetic.CONFIGS[name]
    rank = 3
    x, w, peers = synthetic.make_inputs(cfg, mode)
    op = _op(cfg, rank=rank)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b)
    fused_out, fused_local = host(b.out), host(b.local)
    S = cfg.S
    y = torch.nn.functional.linear(b.x.view(torch.bfloat16), b.w.view(torch.bfloat16))
    b.local.copy_(y[rank * S:(rank + 1) * S].view(torch.int16))
    b.out.fill_(np.array(SENTINEL, np.uint16).view(np.int16).item())
    run(op, b, gr.MODE_REDUCE_ONLY)
    unfused_out, unfused_local = host(b.out), host(b.local)
    rows = np.arange(S) if S <= 256 else sample_rows(S, op.info.bm, np.random.default_rng(2), extra=6)
    ref_out = oracle.ref_f64(x, w, peers, tp=8, rank=rank, rows=rows)
    ref_local = oracle.ref_f64(x, w, None, tp=8, rank=rank, rows=rows)
    e_fused = max_rel(fused_out[rows], ref_out)
    e_unfused = max_rel(unfused_out[rows], ref_out)
    assert e_fused <= 1e-2
    assert e_fused <= 1.1 * e_unfused, (e_fused, e_unfused)
    l_fused = max_rel(fused_local[rows], ref_local)
    l_unfused = max_rel(unfused_local[rows], ref_local)
    assert l_fused <= 1.1 * l_unfused, (l_fused, l_unfused)


# ------------------------------------------------------------------ full shapes, sampled rows

@pytest.mark.parametrize("red", ["bench", "reducers8", "nt", "device", "rowc", "stream"])
@pytest.mark.parametrize("name", ["o_proj", "down_proj", "mixtral_down", "large_prefill"])
@pytest.mark.parametrize("mode", ["normal", "integer"])
def test_benchmark_shapes_sampled_rows(name, mode, red):
    # "bench": the launch configuration the benchmark times
    cfg = synthetic.CONFIGS[name]
    if red == "stream" and name == "o_proj":
        pytest.skip("the stream kernel needs the 256x256 tile (o_proj has 64-row slices)")
    rank = 5
    x, w, peers = synthetic.make_inputs(cfg, mode)
    op = _op(cfg, rank=rank, **({} if red == "bench" else REDUCE[red]))
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b)
    rng = np.random.default_rng(1)
    rows = sample_rows(cfg.S, op.info.bm, rng)
    local_o, send_o, out_o = oracle_rows(x, w, peers, rank, cfg.S, rows)
    S = cfg.S
    sl = lambda t: host(t)[rows]
    if mode == "integer":
        for i in range(7):
            assert np.array_equal(sl(b.send[i]), send_o[i]), f"send[{i}]"
        assert np.array_equal(sl(b.local), local_o)
        assert np.array_equal(sl(b.out), out_o)
    else:
        for i in range(7):
            d = oracle.peer_rank(rank, i)
            assert_close_partial(sl(b.send[i]), send_o[i], x, w, d * S + rows)
        assert_close_partial(sl(b.local), local_o, x, w, rank * S + rows)
        assert np.array_equal(sl(b.out), oracle.slice_sum(sl(b.local), [p[rows] for p in peers]))
    # every element of every output written (no sentinel left anywhere)
    for t in b.send + [b.local, b.out]:
        assert not bool((t == np.array(SENTINEL, np.uint16).view(np.int16).item()).any())


# ------------------------------------------------------------------ modes and knobs

def test_modes_agree_bit_exactly():
    cfg = synthetic.CONFIGS["o_proj"]
    x, w, peers = synthetic.make_inputs(cfg, "normal")
    op = _op(cfg, rank=2)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b, gr.MODE_FUSED)
    fused = [host(t) for t in b.send + [b.local, b.out]]
    b.refill()
    run(op, b, gr.MODE_SEQUENTIAL)
    seq = [host(t) for t in b.send + [b.local, b.out]]
    for a_, s_ in zip(fused, seq):
        assert np.array_equal(a_, s_)
    b.refill()
    run(op, b, gr.MODE_GEMM_ONLY)
    assert np.array_equal(host(b.local), fused[7])
    assert np.all(host(b.out) == SENTINEL)
    run(op, b, gr.MODE_REDUCE_ONLY)
    assert np.array_equal(host(b.out), fused[8])


@pytest.mark.parametrize("kw", [
    dict(flag_stride=32), dict(num_reducers=1), dict(num_reducers=64), dict(num_reducers=0, group_m=1),
    dict(num_reducers=0, tile="128x128", group_m=3), dict(num_reducers=0, tile="256x256"),
    dict(num_reducers=8, flag_stride=32, tile="128x256"),
    dict(num_reducers=0, flag_stride=32, tile="16x64"), dict(num_reducers=3, tile="16x64"),
    dict(tile_stores="nt"), dict(tile_stores="nt", num_reducers=8), dict(tile_stores="nt", tile="64x128"),
    dict(tile_stores="nt", tile="256x256"), dict(tile_stores="nt", tile="16x64", num_reducers=8),
    dict(flag_protocol="row_counter"), dict(flag_protocol="row_counter", num_reducers=8),
    dict(flag_protocol="row_counter", tile="16x64", flag_stride=32),
])
def test_knobs_keep_results(kw):
    cfg = synthetic.CONFIGS["mixtral_down"]
    cfg = synthetic.Config("mixtral_small", 3, 1024, cfg.N, 512)
    x, w, peers = synthetic.make_inputs(cfg, "integer")
    op = _op(cfg, rank=1, **kw)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b)
    send_o, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=1)
    for i in range(7):
        assert np.array_equal(host(b.send[i]), send_o[i])
    assert np.array_equal(host(b.local), local_o)
    assert np.array_equal(host(b.out), out_o)


def test_caller_local_slice_buffer_and_scratch_agree():
    cfg = synthetic.CONFIGS["tiny"]
    x, w, peers = synthetic.make_inputs(cfg, "normal")
    op = _op(cfg, rank=0)
    b = Buffers(x, w, peers, cfg.S, cfg.N)
    run(op, b)
    out1 = host(b.out)
    op.run(gr.MODE_FUSED, b.x, b.w, b.send, b.peers, b.out, None)  # handle scratch
    torch.cuda.synchronize()
    assert op.status() == gr.OK
    assert np.array_equal(host(b.out), out1)


# ------------------------------------------------------------------ edge cases

def test_zero_k_gives_sum_of_peers():
    cfg = synthetic.Config("k0", 0, 128, 256, 0)
    _, _, peers = synthetic.make_inputs(synthetic.Config("k0p", 0, 128, 256, 8), "normal")
    x = np.zeros((128, 0), np.uint16)
    w = np.zeros((256, 0), np.uint16)
    op = gr.GemmRS(128, 256, 0, rank=3)
    b = Buffers(x, w, peers, 16, 256)
    run(op, b)
    _, local_o, out_o = oracle.gemm_rs(x, w, peers, tp=8, rank=3)
    assert np.array_equal(host(b.local), local_o)
    assert np.array_equal(host(b.out), out_o)


def test_zero_rows_is_a_no_op():
    op = gr.GemmRS(0, 256, 64, rank=0)
    z = torch.zeros((0, 256), dtype=torch.int16, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.int16, device="cuda")
    w = torch.zeros((256, 64), dtype=torch.int16, device="cuda")
    op.run(gr.MODE_FUSED, x, w, [z] * 7, [z] * 7, z, None)
    torch.cuda.synchronize()
    assert op.status() == gr.OK


def test_misaligned_pointer_rejected():
    cfg = synthetic.CONFIGS["tiny"]
    op = _op(cfg)
    buf = torch.zeros(cfg.S * cfg.N + 8, dtype=torch.int16, device="cuda")
    bad = buf[1:1 + cfg.S * cfg.N]
    ok = [torch.zeros((cfg.S, cfg.N), dtype=torch.int16, device="cuda") for _ in range(7)]
    rc = gr.gemm_rs_run(op.h, gr.MODE_REDUCE_ONLY, None, None, None, [t.data_ptr() for t in ok],
                        bad.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    assert rc == gr.ERR_MISALIGNED
    rc = gr.gemm_rs_run(op.h, gr.MODE_REDUCE_ONLY, None, None, None, None, ok[0].data_ptr(), None, None)
    assert rc == gr.ERR_INVALID_ARG


def test_rejects_unsupported_shape():
    with pytest.raises(gr.GemmRSError) as e:
        gr.GemmRS(100, 256, 64)
    assert e.value.code == gr.ERR_UNSUPPORTED_SHAPE
