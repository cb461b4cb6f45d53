/*
 * gemm_rs.h -- C ABI of the fused BF16 GEMM + reduce-scatter library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is one rank's share of a tensor-parallel row-parallel linear
 * layer (problem page "A fused GEMM + reduce-scatter kernel hiding 90% of
 * communication on 8 H100 GPUs", sections "What is asked" and "How it gets
 * verified"): rank r holds X_r (M x K_local) and its weight shard W_r, computes
 * the partial product P_r = X_r * W_r in BF16 with FP32 accumulation, and the
 * partials of all tp ranks are summed so that rank d keeps row slice d of the
 * total.  Following FLUX (TL;DR of "FLUX: Fast Software-based Communication
 * Overlap On GPUs Through Kernel Fusion": reduce-scatter fused as a GEMM
 * epilogue, tile coordinate swizzling) and mKernel ("mKernel: Fast Multi-GPU,
 * Multi-Node Fused Kernels", sections 3 and 3.2: compute and communication
 * roles inside one persistent kernel, tile readiness flags), one persistent
 * kernel both computes the GEMM tiles and reduces this rank's slice:
 *
 *   compute workgroups  walk the tile schedule, run the MFMA main loop, round
 *                       each finished tile to BF16, store it into the buffer of
 *                       its destination slice and release its ready flag;
 *   reducers            wait for the flags of this rank's own slice and sum each
 *                       tile with the tp-1 peer partials into `out`: by default
 *                       the compute workgroups themselves after their last
 *                       tile, optionally in dedicated workgroups (num_reducers)
 *                       or in co-resident ones (reduce_mode).
 *
 * On one GPU the tp-1 peer partials are buffers already resident in HBM that
 * stand in for the other ranks' remote writes, and the tp-1 send buffers stand
 * in for remote stores; there is no inter-GPU traffic.
 *
 * Numerics (fixed so that results are reproducible bit for bit):
 *   - partial tiles: FP32 MFMA accumulation, rounded to BF16 to nearest-even;
 *   - slice sum: FP32 additions in the order (((0 + peer_0) + peer_1) + ...
 *     + peer_{tp-2}) + local, then one round-to-nearest-even to BF16, where
 *     peer slot i holds peer rank p_i = (i < rank ? i : i + 1).
 *
 * Layouts (all row-major BF16, raw 16-bit patterns, device memory):
 *   x      [M][K_local]        this rank's activations X_r
 *   w      [N][K_local]        this rank's weight shard, K contiguous (the
 *                              layout of a linear layer's weight; the product
 *                              is X_r * W_r with W_r = w^T)
 *   send[i], peers[i], out, local_slice: [S][N] with S = M / tp
 * Every pointer must be 16-byte aligned; K_local and N must be multiples of 8;
 * M * K_local, N * K_local and S * N must stay below 2^30 elements.
 *
 * Errors: every function returns GEMM_RS_OK (0) or a negative GEMM_RS_ERR_*
 * code; nothing aborts and nothing throws across the ABI.  gemm_rs_strerror
 * gives a message (for GEMM_RS_ERR_HIP it includes the last HIP error).
 *
 * Threading: a handle may be used from one host thread at a time, and runs on
 * one handle must not overlap on the device (they share the ready flags and
 * the handle's device counters): issue them on one stream, or synchronise
 * between streams.  The run epoch and all counters live in device memory and
 * are advanced by the kernel itself, so runs may be captured into a HIP graph
 * and replayed; each replay is a new run.  A fused run needs its whole grid
 * resident at once (the grid is sized to the device: CUs x workgroups per CU),
 * as a persistent kernel whose workgroups wait for each other's flags.  This
 * is not checked at launch: a kernel that holds CUs on another stream can
 * delay part of the grid, and a reducer that then waits longer than the
 * watchdog reports GEMM_RS_ERR_TIMEOUT with `out` incomplete.
 */
#ifndef GEMM_RS_H
#define GEMM_RS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes -------------------------------------------------------- */
#define GEMM_RS_OK 0
#define GEMM_RS_ERR_INVALID_ARG (-1)       /* null pointer, bad enum, bad size  */
#define GEMM_RS_ERR_UNSUPPORTED_SHAPE (-2) /* tp != 8, M % tp, N or K % 8, ... */
#define GEMM_RS_ERR_MISALIGNED (-3)        /* a buffer is not 16-byte aligned   */
#define GEMM_RS_ERR_NO_DEVICE (-4)         /* current device is not gfx950      */
#define GEMM_RS_ERR_HIP (-5)               /* a HIP runtime call failed         */
#define GEMM_RS_ERR_TIMEOUT (-6)           /* a reducer gave up waiting (watchdog) */
#define GEMM_RS_ERR_NO_MEMORY (-7)         /* device or host allocation failed  */
#define GEMM_RS_ERR_SCRATCH (-8)           /* gemm_rs_run_static: the problem's
                                              state exceeds the static scratch   */

/* Device bytes of the static scratch gemm_rs_run_static uses per GPU. */
#define GEMM_RS_STATIC_SCRATCH_BYTES 1048576 /* 1 MiB */

/* ---- run modes ---------------------------------------------------------- */
#define GEMM_RS_MODE_FUSED 0       /* one persistent kernel: compute + reducers  */
#define GEMM_RS_MODE_GEMM_ONLY 1   /* the same GEMM on all CUs, no flags, no sum */
#define GEMM_RS_MODE_REDUCE_ONLY 2 /* standalone slice sum of local + peers      */
#define GEMM_RS_MODE_SEQUENTIAL 3  /* GEMM_ONLY then REDUCE_ONLY on one stream   */

/* ---- tile configurations (BM x BN output tile) ---------------------------- */
#define GEMM_RS_TILE_AUTO 0
#define GEMM_RS_TILE_16x64 1
#define GEMM_RS_TILE_64x128 2
#define GEMM_RS_TILE_128x128 3
#define GEMM_RS_TILE_128x256 4
#define GEMM_RS_TILE_256x128 5
#define GEMM_RS_TILE_256x256 6
#define GEMM_RS_TILE_COUNT 7

/* ---- where the slice sum runs without dedicated reducers ------------------ */
#define GEMM_RS_REDUCE_AUTO 0   /* STREAM for the 256x256 tile with
                                   384 <= K_local < 3072 and at least 768 tiles
                                   (three rounds of a 256-CU device) unless
                                   num_reducers is -2; TAIL otherwise            */
#define GEMM_RS_REDUCE_TAIL 1   /* each compute workgroup sums its share of the
                                   slice after its last tile                      */
#define GEMM_RS_REDUCE_CORESIDENT 2 /* one reducer workgroup per CU beside the
                                   compute workgroups (tiles whose kernel fits one
                                   more workgroup per CU, else gemm_rs_create gives
                                   GEMM_RS_ERR_UNSUPPORTED_SHAPE); each reducer wave
                                   sums the peers of its items while the GEMM runs,
                                   then adds the local chunk once the tile's flag
                                   is set                                          */
#define GEMM_RS_REDUCE_STREAM 3 /* 256x256 tile, K_local >= 384: four of the eight
                                   waves of each compute workgroup issue no stage
                                   loads and stream the slice sum between their
                                   MFMAs (two loads and a store per K step, each
                                   load in flight for two steps) once the
                                   workgroup's own tiles are released; the rest
                                   is summed after the last tile.  Tile flags and
                                   device-scope stores only.  The all-reduce's
                                   FUSED runs on such a handle sum after the last
                                   tile (TAIL)                                    */
#define GEMM_RS_REDUCE_ADAPTIVE 4 /* every compute workgroup changes role at its
                                   tile boundaries and sums a share of the slice
                                   there: each wave owns every (W G)-th 512-
                                   element item in release order and, at a
                                   boundary, sums an even share of what it has
                                   left over the boundaries it has left, limited
                                   to released rounds and, by its cycle counter,
                                   to a quarter of a tile's time; the last
                                   boundary sums the rest (mKernel, "mKernel:
                                   Fast Multi-GPU, Multi-Node Fused Kernels",
                                   section 3.2: roles change at task boundaries
                                   under a target from progress and cost
                                   counters).  Also selected by num_reducers ==
                                   -2.  Tile flags and device-scope stores only   */

/* ---- cache policy of the routed tile stores ------------------------------ */
#define GEMM_RS_STORES_DEVICE 0      /* device scope, written through L2        */
#define GEMM_RS_STORES_NONTEMPORAL 1 /* device scope with the non-temporal hint:
                                        the tiles are not kept in L2 for reuse.
                                        A separate kernel variant (also of
                                        GEMM_ONLY); not with row counters      */
#define GEMM_RS_STORES_AUTO 2        /* NONTEMPORAL for the 256x256 tile with at
                                        least 1024 tiles when the sum runs
                                        after the tiles (TAIL, also with
                                        dedicated reducers) with tile flags;
                                        DEVICE otherwise.  Measured: 0.3-2.5%
                                        faster from 8 rounds of 256x256 tiles,
                                        no gain below, 1% slower on o_proj's
                                        64x128 tile                           */

/* ---- how a released tile is signalled ------------------------------------ */
#define GEMM_RS_FLAGS_TILE 0        /* one ready flag per tile, set to the run's
                                       epoch                                    */
#define GEMM_RS_FLAGS_ROW_COUNTER 1 /* one counter per tile row (destination
                                       slice, tile row), atomically incremented
                                       per released tile and never reset; a tile
                                       is summed once its row's counter reaches
                                       epoch x tile columns.  A separate kernel
                                       variant.  After a watchdog timeout the
                                       counters are one short for good: create a
                                       new handle.                              */

/* ---- debug flags -------------------------------------------------------- */
#define GEMM_RS_DEBUG_TRACE 1 /* record, per schedule slot, the tile's flag index,
                                 the compute workgroup and a release timestamp */

typedef struct gemm_rs_config {
    int32_t M;            /* tokens: rows of X_r and of the partial product   */
    int32_t N;            /* output features (columns of the product)         */
    int32_t K_local;      /* this rank's share of the reduction dimension     */
    int32_t tp;           /* tensor-parallel degree; must be 8                */
    int32_t rank;         /* this rank, 0 <= rank < tp                        */
    int32_t tile;         /* GEMM_RS_TILE_*                                   */
    int32_t group_m;      /* tile rows per raster group; 0 = automatic        */
    int32_t num_reducers; /* dedicated reducer workgroups in FUSED mode (they
                             sum while the others compute, then stop);
                             -1 = automatic (none); -2 = the adaptive
                             controller (GEMM_RS_REDUCE_ADAPTIVE)             */
    int32_t debug_flags;  /* GEMM_RS_DEBUG_* bits                             */
    int32_t drop_flag;    /* debug: index of a ready flag the producer never
                             releases, to exercise the watchdog; -1 = none    */
    int32_t flag_stride;  /* 32-bit words between ready flags (1 or 32)       */
    int64_t watchdog_us;  /* reducer wait limit per tile in microseconds;
                             0 = default (2 000 000)                          */
    int32_t reduce_mode;  /* GEMM_RS_REDUCE_*; all but AUTO and TAIL need
                             num_reducers <= 0                               */
    int32_t tile_stores;  /* GEMM_RS_STORES_*: cache policy of the tile stores
                             into the destination slices (every mode and entry
                             point that routes tiles)                        */
    int32_t flag_protocol; /* GEMM_RS_FLAGS_*                                 */
} gemm_rs_config;

typedef struct gemm_rs_info {
    int32_t bm, bn, bk;       /* resolved tile                                 */
    int32_t group_m;          /* resolved raster group                         */
    int32_t tiles;            /* T: tiles of the whole M x N partial           */
    int32_t tiles_per_slice;  /* T_s                                           */
    int32_t tile_rows_per_slice, tile_cols;
    int32_t grid;             /* workgroups launched in FUSED mode             */
    int32_t compute_wgs;      /* of which compute                              */
    int32_t reducer_wgs;      /* of which reducers                             */
    int32_t num_cus;          /* compute units of the device                   */
    int32_t wgs_per_cu;       /* resident workgroups per CU for this kernel    */
    int32_t lds_bytes;        /* LDS per workgroup                             */
    int32_t reduce_grid;      /* workgroups of the standalone reduce kernel    */
    int32_t xcd_split;        /* how a round of slots is split over the 8 XCDs:
                                 0 contiguous blocks, 1 every 8th slot         */
    uint32_t epoch;           /* value the last FUSED run stored in its flags
                                 (read from the device; waits for the stream) */
    int32_t reduce_mode;      /* resolved GEMM_RS_REDUCE_* of a FUSED run with
                                 no dedicated reducers                        */
    int32_t split_state;      /* 0: fixed reducer count; 1: the adaptive
                                 controller decides on the device           */
    int32_t tile_stores;      /* resolved GEMM_RS_STORES_* (never AUTO)      */
} gemm_rs_info;

typedef struct gemm_rs_handle gemm_rs_handle;

/* Checks a configuration without touching the GPU (pure host code).
 * Returns GEMM_RS_OK, GEMM_RS_ERR_INVALID_ARG or GEMM_RS_ERR_UNSUPPORTED_SHAPE. */
int gemm_rs_validate(const gemm_rs_config *cfg);

/* Resolves the tile and raster group that gemm_rs_create would pick, on the
 * host only (no GPU).  info fields that need a device are left 0. */
int gemm_rs_plan(const gemm_rs_config *cfg, gemm_rs_info *info);

/* Host-only enumeration of the tile schedule (the same code the kernels run):
 * for each slot q < tiles, the destination slice, the tile row in the M x N
 * partial (units of bm rows counted per slice: d * tile_rows_per_slice + row
 * inside the slice), the tile column and the ready-flag index.  Any output may
 * be NULL; n is the capacity of each array (>= tiles). */
int gemm_rs_plan_slots(const gemm_rs_config *cfg, int32_t *slot_d, int32_t *slot_tm,
                       int32_t *slot_tn, int32_t *slot_flag, size_t n);

/* Creates a handle on the current HIP device: validates cfg, checks that the
 * device is gfx950, and allocates the handle-owned device state (ready flags
 * and per-workgroup finish marks zeroed, arrival tickets, status word, trace
 * log, and a [S][N] BF16 scratch used as the local slice when gemm_rs_run gets
 * local_slice == NULL).  The handle is the persistent kernel's setup: mKernel
 * ("mKernel: Fast Multi-GPU, Multi-Node Fused Kernels", section 3) splits one
 * persistent kernel's blocks into compute and communication roles that
 * coordinate through per-tile readiness flags in GPU memory; the flags, the
 * role tickets and the grid size (CUs x workgroups per CU, all resident at
 * once) are fixed here.
 * On success *out receives the handle; on failure *out is set to NULL.
 * Errors: INVALID_ARG / UNSUPPORTED_SHAPE (as gemm_rs_validate), NO_DEVICE,
 * NO_MEMORY, HIP. */
int gemm_rs_create(const gemm_rs_config *cfg, gemm_rs_handle **out);

/* Enqueues one run on `stream` (a hipStream_t; NULL = the null stream) and
 * returns without waiting.  A FUSED run is the operation of the problem page
 * ("A fused GEMM + reduce-scatter kernel hiding 90% of communication on 8 H100
 * GPUs", "What is asked"): the local GEMM and the reduce-scatter of its
 * partial in one kernel, partial tiles handed on as they are finished; the
 * other modes are the unfused baselines the same page's "How it gets
 * verified" compares against (the GEMM alone, then the reduction).
 *   mode         GEMM_RS_MODE_*.
 *   x, w         device inputs (see Layouts); unused by REDUCE_ONLY.
 *   send         host array of tp-1 device pointers; send[i] receives the
 *                partial's slice for peer rank p_i.  Unused by REDUCE_ONLY.
 *   peers        host array of tp-1 device pointers to the peer partials of
 *                this rank's slice; unused by GEMM_ONLY.
 *   out          device [S][N]: the reduced slice; unused by GEMM_ONLY.
 *   local_slice  device [S][N]: this rank's own slice of its partial (written by
 *                the GEMM, read by the sum); NULL = the handle's scratch.
 * The caller owns every buffer and keeps it alive until the stream work is
 * done.  Runs on one handle must not overlap on the device.
 * M == 0 or N == 0 enqueues nothing; K_local == 0 gives a zero partial. */
int gemm_rs_run(gemm_rs_handle *h, int32_t mode, const void *x, const void *w,
                void *const *send, const void *const *peers, void *out,
                void *local_slice, void *stream);

/* GEMM + all-reduce for one node (mKernel, "mKernel: Fast Multi-GPU,
 * Multi-Node Fused Kernels", Sections 3.1 and 4: the local reduction is followed
 * by replication, each GPU sending its reduced eighth of the output to the
 * others).  The same run as gemm_rs_run, and every chunk of the reduced slice
 * that the sum stores into `out` is also stored, in the same launch, into
 * gather[0..tp-2]:
 *   gather       host array of tp-1 device pointers, each [S][N] BF16, 16-byte
 *                aligned; gather[i] receives this rank's reduced slice for peer
 *                rank p_i (the all-gather's send to that peer: rows
 *                rank*S .. rank*S+S-1 of the peer's M x N result).  Required
 *                (GEMM_RS_ERR_INVALID_ARG if NULL) except for GEMM_ONLY, which
 *                writes no reduced slice and ignores it.
 * In a caller that passes for `out` the rows rank*S .. of its own M x N
 * result, that buffer holds this rank's part of the all-reduce; the other
 * ranks' parts are what they send.  Same ownership and error behaviour as
 * gemm_rs_run; REDUCE_ONLY and SEQUENTIAL fill gather[] too. */
int gemm_rs_run_allreduce(gemm_rs_handle *h, int32_t mode, const void *x, const void *w,
                          void *const *send, const void *const *peers, void *out,
                          void *local_slice, void *const *gather, void *stream);

/* All-gather + GEMM: the column-parallel linear layer that precedes the
 * row-parallel one, with the all-gather fused as the GEMM's prologue (FLUX,
 * "FLUX: Fast Software-based Communication Overlap On GPUs Through Kernel
 * Fusion", TL;DR; mKernel, "mKernel: Fast Multi-GPU, Multi-Node Fused
 * Kernels", Section 4: the local shard's tiles first, the others as their rows
 * arrive).  The handle's config is read as: M gathered rows (tp row slices of
 * S = M / tp), N this rank's output columns, K_local the layer's reduction
 * length K (the activations are not sharded along K).
 *   x_slices    host array of tp device pointers, in source-rank order, each
 *               [S][K] BF16: x_slices[rank] is this rank's own row slice, the
 *               others stand in for what the peers send.
 *   w           [N][K] BF16, this rank's column shard of the weight.
 *   x_gathered  [M][K] BF16 output: the gathered activations, slice d at rows
 *               d*S .. d*S + S - 1.
 *   y           [M][N] BF16 output: RNE(x_gathered * w^T), FP32 accumulation.
 * Modes: FUSED is one persistent launch: every workgroup copies its share of
 * the slices into x_gathered (in the order the tiles need them) and bumps a
 * per-block counter, then runs the GEMM; tiles of this rank's slice start at
 * once, the others wait for their rows.  GEMM_ONLY runs the GEMM over an
 * already complete x_gathered (only x_slices[rank] is read); REDUCE_ONLY runs
 * the standalone all-gather copy alone; SEQUENTIAL runs the copy then the
 * GEMM.  M * N * 2 must stay below 2^31 (else GEMM_RS_ERR_UNSUPPORTED_SHAPE).
 * Ownership, alignment and errors as gemm_rs_run; a FUSED all-gather run may
 * not overlap another run of the same handle on the device. */
int gemm_rs_run_allgather(gemm_rs_handle *h, int32_t mode, const void *const *x_slices, const void *w,
                          void *x_gathered, void *y, void *stream);

/* gemm_rs_run without a handle and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  It calls no hipMalloc, hipFree or
 * other allocating routine.  The run state, the per-workgroup finish marks and
 * the ready flags live in a static device array of
 * GEMM_RS_STATIC_SCRATCH_BYTES per GPU, kept until the process ends; a run
 * whose state does not fit (ready flags: tiles x flag_stride words, finish
 * marks: one word per workgroup of the grid) returns GEMM_RS_ERR_SCRATCH.
 * Every call on one GPU shares that GPU's array: each run first clears it
 * with a small kernel on `stream`, so calls that overlap on one GPU race and
 * must be ordered by the caller (one stream, or synchronisation).
 *   cfg          as for gemm_rs_create; any debug_flags are refused
 *                (GEMM_RS_ERR_INVALID_ARG).
 *   mode, x, w, send, peers, out, stream: as for gemm_rs_run.
 *   local_slice  required (there is no handle scratch): device [S][N].
 *   status       NULL, or a 4-byte aligned device array of 2 int32 that the
 *                run zeroes first and in which a watchdog timeout leaves
 *                GEMM_RS_ERR_TIMEOUT and the flag index (read it after the
 *                stream work is done); with NULL a timeout is not reported.
 * Results are those of gemm_rs_run with the same config and buffers. */
int gemm_rs_run_static(const gemm_rs_config *cfg, int32_t mode, const void *x, const void *w,
                       void *const *send, const void *const *peers, void *out,
                       void *local_slice, int32_t *status, void *stream);

/* Waits for the handle's last run and returns its device status:
 * GEMM_RS_OK, or GEMM_RS_ERR_TIMEOUT if a reducer gave up waiting for a ready
 * flag (the kernel still exits; `out` is then incomplete).  Reading the status
 * clears it.  The waits it reports are the readiness-flag waits of mKernel's
 * communication roles ("mKernel: Fast Multi-GPU, Multi-Node Fused Kernels",
 * section 4: tiles signal completion through flags that consumers poll), here
 * bounded by a watchdog.  A wait also times out when the grid is not wholly
 * resident, for instance while other kernels hold CUs on another stream: the
 * persistent launch assumes every workgroup runs at once.
 * Errors: INVALID_ARG (h NULL), HIP. */
int gemm_rs_status(gemm_rs_handle *h);

/* Fills *info with the resolved launch parameters of a handle. */
int gemm_rs_query(gemm_rs_handle *h, gemm_rs_info *info);

/* Copies debug state of the last run to host memory (waits for it first):
 * the per-tile release times and flag values that make the overlap and the
 * flag order visible (the progress counters mKernel's controller reads,
 * "mKernel: Fast Multi-GPU, Multi-Node Fused Kernels", section 3.2; the flag
 * order fixed by FLUX's tile coordinate swizzling, TL;DR of "FLUX: Fast
 * Software-based Communication Overlap On GPUs Through Kernel Fusion").
 *   slot_log   if non-NULL, 4 words per schedule slot: the tile's flag index,
 *              the compute workgroup's ticket, and the 64-bit release time
 *              (100 MHz counter; low word then high word).  Written only when
 *              the run had GEMM_RS_DEBUG_TRACE; slot_words >= 4 * tiles.
 *              With slot_words >= 4 * (tiles + T_s + 1) (T_s: tiles per
 *              slice) the slice-sum stamps of the last FUSED run follow: per
 *              own tile (slice order, row-major) the earliest flag check, the
 *              earliest time it was seen released, the latest sum store and
 *              the number of 512-element items summed (low words of the same
 *              counter; all ones / zero where none), then the launch's first
 *              workgroup start, an unused word, its last workgroup end and an
 *              unused word.  The stream records a wave's items at the tile
 *              boundary after it has summed them all.
 *   flags      if non-NULL, the current value of each ready flag;
 *              flag_words >= tiles. */
int gemm_rs_debug_read(gemm_rs_handle *h, uint32_t *slot_log, size_t slot_words,
                       uint32_t *flags, size_t flag_words);

/* Waits for outstanding work and frees the handle's device state (what
 * gemm_rs_create set up for the persistent kernel of mKernel, "mKernel: Fast
 * Multi-GPU, Multi-Node Fused Kernels", section 3).  NULL is a no-op; nothing
 * is returned, and a HIP error while waiting is ignored. */
void gemm_rs_destroy(gemm_rs_handle *h);

/* Message for an error code (static storage; for GEMM_RS_ERR_HIP the last HIP
 * error seen by this thread). */
const char *gemm_rs_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_RS_H */
