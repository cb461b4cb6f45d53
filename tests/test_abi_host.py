"""Host-side checks of the C-ABI library (no GPU calls).

- the library loads and exports every function include/gemm_rs.h declares;
- gemm_rs_validate's error codes;
- the schedule the kernels decode (same __host__ __device__ code, run on the
  host through gemm_rs_plan_slots) equals the oracle's schedule bit for bit and
  every tile it produces lies inside its buffers.
"""
import os
import re

import numpy as np
import pytest

import oracle
from conftest import ROOT

gr = pytest.importorskip("tensor_gemm_reduce_amd.gemm_rs")


def declared_functions():
    names = set()
    with open(os.path.join(ROOT, "include", "gemm_rs.h")) as f:
        text = f.read()
    for m in re.finditer(r"^\s*(?:int|void|const char \*)\s*\*?\s*(gemm_rs_\w+)\s*\(", text, re.M):
        names.add(m.group(1))
    return names


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("gemm_rs_create", "gemm_rs_run", "gemm_rs_destroy"):
        assert n in names
    assert names == set(gr.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = gr.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_header_constants_match_binding():
    with open(os.path.join(ROOT, "include", "gemm_rs.h")) as f:
        text = f.read()
    consts = {m.group(1): int(m.group(2)) for m in
              re.finditer(r"#define GEMM_RS_(\w+)\s+\(?(-?\d+)\)?", text)}
    for k, v in consts.items():
        if hasattr(gr, k):
            assert getattr(gr, k) == v, k
    assert consts["ERR_TIMEOUT"] == gr.ERR_TIMEOUT
    assert consts["MODE_SEQUENTIAL"] == gr.MODE_SEQUENTIAL


def cfg(**kw):
    base = dict(M=2048, N=8192, K_local=3584)
    base.update(kw)
    return gr.make_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(), gr.OK),
    (dict(tp=4), gr.ERR_UNSUPPORTED_SHAPE),
    (dict(M=2047), gr.ERR_UNSUPPORTED_SHAPE),
    (dict(N=8191), gr.ERR_UNSUPPORTED_SHAPE),
    (dict(K_local=100), gr.ERR_UNSUPPORTED_SHAPE),
    (dict(rank=8), gr.ERR_INVALID_ARG),
    (dict(rank=-1), gr.ERR_INVALID_ARG),
    (dict(M=-8), gr.ERR_INVALID_ARG),
    (dict(tile=7), gr.ERR_INVALID_ARG),
    (dict(flag_stride=2), gr.ERR_INVALID_ARG),
    (dict(debug_flags=4), gr.ERR_INVALID_ARG),
    (dict(drop_flag=100000), gr.ERR_INVALID_ARG),
    (dict(num_reducers=-3), gr.ERR_INVALID_ARG),
    (dict(num_reducers=-2), gr.OK),
    (dict(num_reducers=-2, reduce_mode="coresident"), gr.ERR_INVALID_ARG),
    (dict(tile_stores="nt"), gr.OK),
    (dict(tile_stores="nt", num_reducers=8), gr.OK),
    (dict(tile_stores=3), gr.ERR_INVALID_ARG),
    (dict(tile_stores="auto"), gr.OK),
    (dict(tile_stores="auto", flag_protocol="row_counter"), gr.OK),
    (dict(tile_stores="auto", reduce_mode="stream"), gr.OK),
    (dict(tile_stores="auto", reduce_mode="adaptive"), gr.OK),
    (dict(tile_stores="auto", num_reducers=-2), gr.OK),
    (dict(tile_stores="device", reduce_mode="stream"), gr.OK),
    (dict(tile_stores=-1), gr.ERR_INVALID_ARG),
    (dict(flag_protocol="row_counter"), gr.OK),
    (dict(flag_protocol="row_counter", num_reducers=8), gr.OK),
    (dict(flag_protocol="row_counter", num_reducers=-2), gr.ERR_INVALID_ARG),  # adaptive: tile flags
    (dict(reduce_mode="adaptive"), gr.OK),
    (dict(reduce_mode="adaptive", num_reducers=-2), gr.OK),
    (dict(reduce_mode="adaptive", tile_stores="nt"), gr.ERR_INVALID_ARG),
    (dict(reduce_mode="adaptive", num_reducers=8), gr.ERR_INVALID_ARG),
    (dict(num_reducers=-2, tile_stores="nt"), gr.ERR_INVALID_ARG),
    (dict(flag_protocol=2), gr.ERR_INVALID_ARG),
    (dict(tile_stores="nt", flag_protocol="row_counter"), gr.ERR_INVALID_ARG),
    (dict(tile_stores="nt", reduce_mode="coresident"), gr.OK),
    (dict(watchdog_us=-1), gr.ERR_INVALID_ARG),
    (dict(reduce_mode=5), gr.ERR_INVALID_ARG),
    (dict(reduce_mode="coresident"), gr.OK),
    (dict(reduce_mode="coresident", num_reducers=8), gr.ERR_INVALID_ARG),
    (dict(reduce_mode="stream"), gr.OK),                                   # 256x256 tile
    (dict(reduce_mode="stream", K_local=384), gr.OK),
    (dict(reduce_mode="stream", K_local=320), gr.ERR_UNSUPPORTED_SHAPE),   # too few K steps
    (dict(reduce_mode="stream", tile="128x128"), gr.ERR_UNSUPPORTED_SHAPE),
    (dict(reduce_mode="stream", M=512, K_local=1024), gr.ERR_UNSUPPORTED_SHAPE),  # o_proj: 64x128
    (dict(reduce_mode="stream", num_reducers=8), gr.ERR_INVALID_ARG),
    (dict(reduce_mode="stream", num_reducers=-2), gr.ERR_INVALID_ARG),
    (dict(reduce_mode="stream", tile_stores="nt"), gr.ERR_INVALID_ARG),
    (dict(reduce_mode="stream", flag_protocol="row_counter"), gr.ERR_INVALID_ARG),
    (dict(reduce_mode=-1), gr.ERR_INVALID_ARG),
    (dict(reduce_mode="tail"), gr.OK),
    (dict(M=0), gr.OK),
    (dict(K_local=0), gr.OK),
])
def test_validate_codes(kw, code):
    assert gr.gemm_rs_validate(cfg(**kw)) == code


def test_strerror_messages():
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -99):
        assert isinstance(gr.gemm_rs_strerror(code), str) and gr.gemm_rs_strerror(code)


SHAPES = [
    (128, 1024, 128, "16x64", 1), (512, 8192, 1024, "64x128", 0), (2048, 8192, 3584, "256x256", 0),
    (8192, 6144, 2048, "256x256", 0), (8192, 6144, 2048, "128x128", 3), (32768, 8192, 3584, "256x256", 0),
    (8 * 200, 1000, 72, "128x128", 2), (8 * 40, 200, 8, "16x64", 0), (8 * 72, 136, 64, "64x128", 0),
]


@pytest.mark.parametrize("M,N,K,tile,gm", SHAPES)
@pytest.mark.parametrize("rank", [0, 5])
def test_kernel_schedule_equals_oracle(M, N, K, tile, gm, rank):
    c = gr.make_config(M, N, K, rank=rank, tile=tile, group_m=gm)
    info = gr.gemm_rs_plan(c)
    got = gr.gemm_rs_plan_slots(c)
    want = oracle.schedule(M, N, 8, rank, info.bm, info.bn, info.group_m)
    for k in ("d", "tm", "tn", "flag"):
        assert np.array_equal(got[k], want[k]), k


@pytest.mark.parametrize("M,N,K,tile,gm", SHAPES)
def test_kernel_tiles_inside_buffers(M, N, K, tile, gm):
    c = gr.make_config(M, N, K, rank=3, tile=tile, group_m=gm)
    info = gr.gemm_rs_plan(c)
    s = gr.gemm_rs_plan_slots(c)
    S = M // 8
    bm, bn, tms = info.bm, info.bn, info.tile_rows_per_slice
    assert info.tiles == 8 * tms * info.tile_cols
    assert sorted(s["flag"].tolist()) == list(range(info.tiles))
    for q in range(info.tiles):
        d, tm, tn = int(s["d"][q]), int(s["tm"][q]), int(s["tn"][q])
        tml = tm - d * tms
        rows = min(bm, S - tml * bm)
        cols = min(bn, N - tn * bn)
        assert 0 < rows and 0 < cols
        r0 = d * S + tml * bm                      # rows of X / of the partial
        assert 0 <= r0 and r0 + rows <= (d + 1) * S <= M
        assert 0 <= tml * bm and tml * bm + rows <= S   # rows of the slice buffer
        assert 0 <= tn * bn and tn * bn + cols <= N


@pytest.mark.parametrize("kw,mode", [
    (dict(), gr.REDUCE_TAIL),                        # automatic: the sum after the last tile
    (dict(reduce_mode="tail"), gr.REDUCE_TAIL),
    (dict(reduce_mode="coresident"), gr.REDUCE_CORESIDENT),
    (dict(reduce_mode="stream"), gr.REDUCE_STREAM),
    (dict(num_reducers=8), gr.REDUCE_TAIL),           # dedicated reducers run the sum
    (dict(M=512, K_local=1024), gr.REDUCE_TAIL),     # o_proj: 64x128 tile
    # automatic: the stream from 768 tiles of 256x256 (three rounds of 256 CUs)
    # with K_local below 3072; the sum after the last tile from there on
    (dict(M=8192, N=6144, K_local=2048), gr.REDUCE_STREAM),          # 768 tiles
    (dict(M=32768, N=8192, K_local=2048), gr.REDUCE_STREAM),
    (dict(M=32768, N=8192, K_local=3008), gr.REDUCE_STREAM),
    (dict(M=32768, N=8192, K_local=3072), gr.REDUCE_TAIL),
    (dict(M=32768, N=8192, K_local=3584), gr.REDUCE_TAIL),           # large prefill
    (dict(M=8192, N=5888, K_local=2048), gr.REDUCE_TAIL),            # 736 tiles
    (dict(M=8192, N=6144, K_local=320), gr.REDUCE_TAIL),             # five K steps
    (dict(M=8192, N=6144, K_local=2048, num_reducers=-2), gr.REDUCE_ADAPTIVE),  # the controller
    (dict(reduce_mode="adaptive"), gr.REDUCE_ADAPTIVE),
    (dict(M=512, K_local=1024, num_reducers=-2), gr.REDUCE_ADAPTIVE),
    (dict(M=8192, N=6144, K_local=2048, num_reducers=8), gr.REDUCE_TAIL),
    (dict(M=8192, N=6144, K_local=2048, tile="128x128"), gr.REDUCE_TAIL),
    (dict(M=8192, N=6144, K_local=2048, reduce_mode="tail"), gr.REDUCE_TAIL),
])
def test_plan_resolves_reduce_mode(kw, mode):
    assert gr.gemm_rs_plan(cfg(**kw)).reduce_mode == mode


@pytest.mark.parametrize("kw,stores", [
    (dict(M=32768, N=8192, K_local=3584), gr.STORES_NONTEMPORAL),    # large prefill: 4096 tiles, tail
    (dict(M=8192, N=8192, K_local=3584), gr.STORES_NONTEMPORAL),     # 1024 tiles
    (dict(M=8192, N=7936, K_local=3584), gr.STORES_DEVICE),          # 992 tiles
    (dict(M=2048, N=8192, K_local=3584), gr.STORES_DEVICE),          # down_proj: one round
    (dict(M=512, N=8192, K_local=1024), gr.STORES_DEVICE),           # o_proj: 64x128 tile
    (dict(M=8192, N=6144, K_local=2048), gr.STORES_DEVICE),          # the stream
    (dict(M=32768, N=8192, K_local=2048), gr.STORES_DEVICE),         # the stream
    (dict(M=32768, N=8192, K_local=2048, reduce_mode="tail"), gr.STORES_NONTEMPORAL),
    (dict(M=32768, N=8192, K_local=3584, num_reducers=8), gr.STORES_NONTEMPORAL),
    (dict(M=32768, N=8192, K_local=3584, flag_protocol="row_counter"), gr.STORES_DEVICE),
    (dict(M=32768, N=8192, K_local=3584, reduce_mode="adaptive"), gr.STORES_DEVICE),
    (dict(M=32768, N=8192, K_local=3584, tile="128x128"), gr.STORES_DEVICE),
    (dict(M=32768, N=8192, K_local=3584, tile_stores="device"), gr.STORES_DEVICE),
    (dict(M=512, N=8192, K_local=1024, tile_stores="nt"), gr.STORES_NONTEMPORAL),
])
def test_plan_resolves_tile_stores(kw, stores):
    # the automatic store policy (the binding's default): the non-temporal hint
    # for the 256x256 tile from 1024 tiles when the sum runs after the tiles,
    # tile flags
    assert gr.make_config(1, 1, 8).tile_stores == gr.STORES_AUTO
    assert gr.gemm_rs_plan(cfg(**kw)).tile_stores == stores


def test_plan_resolves_auto_tile():
    for name, (M, N, K) in {"tiny": (128, 1024, 128), "o_proj": (512, 8192, 1024),
                            "down": (2048, 8192, 3584)}.items():
        info = gr.gemm_rs_plan(gr.make_config(M, N, K))
        assert (M // 8) % info.bm == 0 and N % info.bn == 0, name
        assert info.bk == 64
