"""ctypes binding of libgemm_rs.so (include/gemm_rs.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
the library.  PyTorch provides device memory and the stream.  The functions
keep the C names; ``GemmRS`` wraps a handle for torch tensors.

If the library is missing this module raises ImportError: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

# ---- constants mirrored from include/gemm_rs.h ------------------------------
OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED_SHAPE = -2
ERR_MISALIGNED = -3
ERR_NO_DEVICE = -4
ERR_HIP = -5
ERR_TIMEOUT = -6
ERR_NO_MEMORY = -7
ERR_SCRATCH = -8

STATIC_SCRATCH_BYTES = 1 << 20

MODE_FUSED = 0
MODE_GEMM_ONLY = 1
MODE_REDUCE_ONLY = 2
MODE_SEQUENTIAL = 3

TILE_AUTO = 0
TILE_16x64 = 1
TILE_64x128 = 2
TILE_128x128 = 3
TILE_128x256 = 4
TILE_256x128 = 5
TILE_256x256 = 6
TILES = {"auto": 0, "16x64": 1, "64x128": 2, "128x128": 3, "128x256": 4, "256x128": 5, "256x256": 6}

REDUCE_AUTO = 0
REDUCE_TAIL = 1
REDUCE_CORESIDENT = 2
REDUCE_STREAM = 3
REDUCE_ADAPTIVE = 4
REDUCE_MODES = {"auto": 0, "tail": 1, "coresident": 2, "stream": 3, "adaptive": 4}

STORES_DEVICE = 0
STORES_NONTEMPORAL = 1
STORES_AUTO = 2
TILE_STORES = {"device": 0, "nt": 1, "auto": 2}

FLAGS_TILE = 0
FLAGS_ROW_COUNTER = 1
FLAG_PROTOCOLS = {"tile": 0, "row_counter": 1}

DEBUG_TRACE = 1

EXPORTS = ("gemm_rs_validate", "gemm_rs_plan", "gemm_rs_plan_slots", "gemm_rs_create",
           "gemm_rs_run", "gemm_rs_run_allreduce", "gemm_rs_run_allgather", "gemm_rs_run_static",
           "gemm_rs_status", "gemm_rs_query", "gemm_rs_debug_read", "gemm_rs_destroy", "gemm_rs_strerror")


class gemm_rs_config(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int32), ("N", ctypes.c_int32), ("K_local", ctypes.c_int32),
                ("tp", ctypes.c_int32), ("rank", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("group_m", ctypes.c_int32), ("num_reducers", ctypes.c_int32),
                ("debug_flags", ctypes.c_int32),
                ("drop_flag", ctypes.c_int32), ("flag_stride", ctypes.c_int32),
                ("watchdog_us", ctypes.c_int64), ("reduce_mode", ctypes.c_int32),
                ("tile_stores", ctypes.c_int32), ("flag_protocol", ctypes.c_int32)]


class gemm_rs_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "bm", "bn", "bk", "group_m", "tiles", "tiles_per_slice", "tile_rows_per_slice",
        "tile_cols", "grid", "compute_wgs", "reducer_wgs", "num_cus", "wgs_per_cu",
        "lds_bytes", "reduce_grid", "xcd_split")] + [("epoch", ctypes.c_uint32),
                                                     ("reduce_mode", ctypes.c_int32),
                                                     ("split_state", ctypes.c_int32),
                                                     ("tile_stores", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_LIB = None


def library_path() -> str:
    return _build.library_path()


def lib():
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it with `python -m tensor_gemm_reduce_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        cfgp = ctypes.POINTER(gemm_rs_config)
        infop = ctypes.POINTER(gemm_rs_info)
        i32p = ctypes.POINTER(ctypes.c_int32)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        L.gemm_rs_validate.argtypes = [cfgp]
        L.gemm_rs_plan.argtypes = [cfgp, infop]
        L.gemm_rs_plan_slots.argtypes = [cfgp, i32p, i32p, i32p, i32p, ctypes.c_size_t]
        L.gemm_rs_create.argtypes = [cfgp, ctypes.POINTER(vp)]
        L.gemm_rs_run.argtypes = [vp, ctypes.c_int32, vp, vp, ctypes.POINTER(vp),
                                  ctypes.POINTER(vp), vp, vp, vp]
        L.gemm_rs_run_allreduce.argtypes = [vp, ctypes.c_int32, vp, vp, ctypes.POINTER(vp),
                                            ctypes.POINTER(vp), vp, vp, ctypes.POINTER(vp), vp]
        L.gemm_rs_run_allgather.argtypes = [vp, ctypes.c_int32, ctypes.POINTER(vp), vp, vp, vp, vp]
        L.gemm_rs_run_static.argtypes = [cfgp, ctypes.c_int32, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                         vp, vp, vp, vp]
        L.gemm_rs_status.argtypes = [vp]
        L.gemm_rs_query.argtypes = [vp, infop]
        L.gemm_rs_debug_read.argtypes = [vp, u32p, ctypes.c_size_t, u32p, ctypes.c_size_t]
        L.gemm_rs_destroy.argtypes = [vp]
        L.gemm_rs_destroy.restype = None
        L.gemm_rs_strerror.argtypes = [ctypes.c_int]
        L.gemm_rs_strerror.restype = ctypes.c_char_p
        for name in ("gemm_rs_validate", "gemm_rs_plan", "gemm_rs_plan_slots", "gemm_rs_create",
                     "gemm_rs_run", "gemm_rs_run_allreduce", "gemm_rs_run_allgather", "gemm_rs_run_static",
                     "gemm_rs_status", "gemm_rs_query", "gemm_rs_debug_read"):
            getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


class GemmRSError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {gemm_rs_strerror(code)} ({code})")


def _check(code: int, what: str) -> int:
    if code != OK:
        raise GemmRSError(code, what)
    return code


def make_config(M, N, K_local, tp=8, rank=0, tile=TILE_AUTO, group_m=0, num_reducers=-1,
                debug_flags=0, drop_flag=-1, flag_stride=1,
                watchdog_us=0, reduce_mode=REDUCE_AUTO, tile_stores=STORES_AUTO,
                flag_protocol=FLAGS_TILE) -> gemm_rs_config:
    if isinstance(tile, str):
        tile = TILES[tile]
    if isinstance(reduce_mode, str):
        reduce_mode = REDUCE_MODES[reduce_mode]
    if isinstance(tile_stores, str):
        tile_stores = TILE_STORES[tile_stores]
    if isinstance(flag_protocol, str):
        flag_protocol = FLAG_PROTOCOLS[flag_protocol]
    return gemm_rs_config(M, N, K_local, tp, rank, tile, group_m, num_reducers,
                          debug_flags, drop_flag, flag_stride, watchdog_us, reduce_mode, tile_stores,
                          flag_protocol)


# ---- C names ------------------------------------------------------------------

def gemm_rs_validate(cfg: gemm_rs_config) -> int:
    return lib().gemm_rs_validate(ctypes.byref(cfg))


def gemm_rs_plan(cfg: gemm_rs_config) -> gemm_rs_info:
    info = gemm_rs_info()
    _check(lib().gemm_rs_plan(ctypes.byref(cfg), ctypes.byref(info)), "gemm_rs_plan")
    return info


def gemm_rs_plan_slots(cfg: gemm_rs_config):
    """Schedule as the kernels decode it: dict of int32 numpy arrays d, tm, tn, flag."""
    import numpy as np

    T = gemm_rs_plan(cfg).tiles
    out = {k: np.zeros(max(T, 1), np.int32) for k in ("d", "tm", "tn", "flag")}
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _check(lib().gemm_rs_plan_slots(ctypes.byref(cfg), p(out["d"]), p(out["tm"]), p(out["tn"]),
                                    p(out["flag"]), max(T, 1)), "gemm_rs_plan_slots")
    return {k: v[:T] for k, v in out.items()}


def gemm_rs_create(cfg: gemm_rs_config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(lib().gemm_rs_create(ctypes.byref(cfg), ctypes.byref(h)), "gemm_rs_create")
    return h


def gemm_rs_run(h, mode: int, x: int, w: int, send, peers, out: int, local: int | None,
                stream: int | None) -> int:
    """Pointers are integers (device addresses); send/peers are lists of 7 of them."""
    vp = ctypes.c_void_p
    send_arr = (vp * 7)(*send) if send is not None else None
    peer_arr = (vp * 7)(*peers) if peers is not None else None
    return lib().gemm_rs_run(h, mode, x, w, send_arr, peer_arr, out, local, stream)


def gemm_rs_run_allreduce(h, mode: int, x: int, w: int, send, peers, out: int, local: int | None,
                          gather, stream: int | None) -> int:
    """As gemm_rs_run, plus gather: a list of 7 device addresses (or None)."""
    vp = ctypes.c_void_p
    send_arr = (vp * 7)(*send) if send is not None else None
    peer_arr = (vp * 7)(*peers) if peers is not None else None
    gather_arr = (vp * 7)(*gather) if gather is not None else None
    return lib().gemm_rs_run_allreduce(h, mode, x, w, send_arr, peer_arr, out, local, gather_arr, stream)


def gemm_rs_run_allgather(h, mode: int, x_slices, w: int | None, x_gathered: int, y: int | None,
                          stream: int | None) -> int:
    """All-gather + GEMM; x_slices: a list of tp device addresses in source-rank order."""
    vp = ctypes.c_void_p
    xs = (vp * len(x_slices))(*x_slices) if x_slices is not None else None
    return lib().gemm_rs_run_allgather(h, mode, xs, w, x_gathered, y, stream)


def gemm_rs_run_static(cfg: gemm_rs_config, mode: int, x: int | None, w: int | None, send, peers,
                       out: int | None, local: int | None, status: int | None, stream: int | None) -> int:
    """The allocation-free run: no handle; pointers are integers (device
    addresses), send/peers lists of 7 of them, status the device address of
    two int32 words (or None)."""
    vp = ctypes.c_void_p
    send_arr = (vp * 7)(*send) if send is not None else None
    peer_arr = (vp * 7)(*peers) if peers is not None else None
    return lib().gemm_rs_run_static(ctypes.byref(cfg), mode, x, w, send_arr, peer_arr, out, local, status, stream)


def gemm_rs_status(h) -> int:
    return lib().gemm_rs_status(h)


def gemm_rs_query(h) -> gemm_rs_info:
    info = gemm_rs_info()
    _check(lib().gemm_rs_query(h, ctypes.byref(info)), "gemm_rs_query")
    return info


def gemm_rs_debug_read(h, tiles: int, own_tiles=None):
    """Returns (slot_log [tiles][4] uint32, flags [tiles] uint32) as numpy arrays;
    with own_tiles (tiles per slice) also the slice-sum stamps [own_tiles][4]
    (poll, acquire, done, items) and the launch's [first, -, last, -] words."""
    import numpy as np

    extra = 0 if own_tiles is None else own_tiles + 1
    log = np.zeros((max(tiles + extra, 1), 4), np.uint32)
    flags = np.zeros(max(tiles, 1), np.uint32)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))
    _check(lib().gemm_rs_debug_read(h, p(log), log.size, p(flags), flags.size), "gemm_rs_debug_read")
    if own_tiles is None:
        return log[:tiles], flags[:tiles]
    return log[:tiles], flags[:tiles], log[tiles:tiles + own_tiles], log[tiles + own_tiles]


def gemm_rs_destroy(h) -> None:
    lib().gemm_rs_destroy(h)


def gemm_rs_strerror(code: int) -> str:
    return lib().gemm_rs_strerror(code).decode()


# ---- torch convenience wrapper ----------------------------------------------------

def _ptr(t) -> int:
    return t.data_ptr()


class GemmRS:
    """One handle bound to the current device; tensors are torch BF16 (or 16-bit
    integer views of BF16 bits), contiguous, on that device.

    run(mode, x, w, send, peers, out, local=None, stream=None) enqueues a run on
    ``stream`` (default: torch's current stream) and returns immediately.
    """

    def __init__(self, M, N, K_local, tp=8, rank=0, **kw):
        import torch

        if not torch.cuda.is_available():
            raise RuntimeError("GemmRS needs a HIP device")
        self.cfg = make_config(M, N, K_local, tp, rank, **kw)
        self.h = gemm_rs_create(self.cfg)
        self.info = gemm_rs_query(self.h)
        self.S = M // tp

    def _check_tensor(self, t, shape, name):
        import torch

        if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise TypeError(f"{name}: expected a 16-bit tensor of BF16 bits, got {t.dtype}")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name}: must be a contiguous device tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")

    def run(self, mode, x=None, w=None, send=None, peers=None, out=None, local=None, stream=None,
            gather=None):
        """One run; with `gather` (7 [S][N] tensors) the all-reduce variant, whose
        sum also stores the reduced slice into every gather buffer."""
        import torch

        c = self.cfg
        SN = (self.S, c.N)
        if mode != MODE_REDUCE_ONLY:
            self._check_tensor(x, (c.M, c.K_local), "x")
            self._check_tensor(w, (c.N, c.K_local), "w")
            if len(send) != c.tp - 1:
                raise ValueError("send: need tp-1 buffers")
            for i, s in enumerate(send):
                self._check_tensor(s, SN, f"send[{i}]")
        if mode != MODE_GEMM_ONLY:
            if len(peers) != c.tp - 1:
                raise ValueError("peers: need tp-1 buffers")
            for i, p in enumerate(peers):
                self._check_tensor(p, SN, f"peers[{i}]")
            self._check_tensor(out, SN, "out")
            if gather is not None:
                if len(gather) != c.tp - 1:
                    raise ValueError("gather: need tp-1 buffers")
                for i, g in enumerate(gather):
                    self._check_tensor(g, SN, f"gather[{i}]")
        if local is not None:
            self._check_tensor(local, SN, "local")
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        args = (self.h, mode,
                _ptr(x) if x is not None else None, _ptr(w) if w is not None else None,
                [_ptr(s) for s in send] if send is not None else None,
                [_ptr(p) for p in peers] if peers is not None else None,
                _ptr(out) if out is not None else None,
                _ptr(local) if local is not None else None)
        if gather is None:
            _check(gemm_rs_run(*args, stream), "gemm_rs_run")
        else:
            _check(gemm_rs_run_allreduce(*args, [_ptr(g) for g in gather], stream), "gemm_rs_run_allreduce")

    def run_allgather(self, mode, x_slices, w, x_gathered, y, stream=None):
        """All-gather + GEMM with this handle's M (gathered rows), N (output
        columns) and K_local read as the layer's K: x_slices are tp [S][K]
        tensors in source-rank order, w [N][K], x_gathered [M][K], y [M][N]."""
        import torch

        c = self.cfg
        if len(x_slices) != c.tp:
            raise ValueError("x_slices: need tp row slices")
        for i, t in enumerate(x_slices):
            self._check_tensor(t, (self.S, c.K_local), f"x_slices[{i}]")
        self._check_tensor(x_gathered, (c.M, c.K_local), "x_gathered")
        if mode != MODE_REDUCE_ONLY:
            self._check_tensor(w, (c.N, c.K_local), "w")
            self._check_tensor(y, (c.M, c.N), "y")
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        _check(gemm_rs_run_allgather(self.h, mode, [_ptr(t) for t in x_slices],
                                     _ptr(w) if w is not None else None, _ptr(x_gathered),
                                     _ptr(y) if y is not None else None, stream), "gemm_rs_run_allgather")

    def status(self) -> int:
        return gemm_rs_status(self.h)

    def debug_read(self, sums=False):
        return gemm_rs_debug_read(self.h, self.info.tiles, self.info.tiles_per_slice if sums else None)

    def close(self):
        if self.h is not None:
            gemm_rs_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
