// gemm_rs.hip -- host side of the C ABI declared in include/gemm_rs.h, and the
// kernel instantiations for gfx950.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <type_traits>

#include "gemm_rs.h"
#include "kernels.hpp"
#include "plan.hpp"

using namespace gemm_rs;

namespace {

thread_local char g_hip_msg[256] = "";

int hip_fail(hipError_t e, const char* what)
{
    snprintf(g_hip_msg, sizeof g_hip_msg, "%s: %s", what, hipGetErrorString(e));
    return GEMM_RS_ERR_HIP;
}

#define HIP_TRY(call)                                   \
    do {                                                \
        hipError_t e_ = (call);                         \
        if (e_ != hipSuccess) return hip_fail(e_, #call); \
    } while (0)

// Tile table: id -> tile shape, stage depth and the kernel instantiations.
//                      BM   BN   BK  NS  waves  MFMA
typedef TileCfg<16, 64, 128, 2, 1, 4, 16> Tile16x64;
typedef TileCfg<64, 128, 64, 2, 2, 2, 32> Tile64x128;
typedef TileCfg<128, 128, 32, 3, 2, 2, 32> Tile128x128;
typedef TileCfg<128, 256, 32, 4, 2, 2, 32> Tile128x256;
typedef TileCfg<256, 128, 32, 4, 2, 2, 32> Tile256x128;
// four waves, one per SIMD, on the long-tail K loop (tile_kloop_long)
typedef TileCfg<256, 256, 64, 2, 2, 2, 32> Tile256x256;
// the stream kernel of the 256x256 tile: eight waves, four of them loading
// the stages and four streaming the slice sum
typedef TileCfg<256, 256, 64, 2, 2, 4, 32, 4> Tile256x256S;

struct TileDesc {
    int bm, bn, bk;
    int threads;               // workgroup size
    int wgs_per_cu;            // workgroups per CU the kernels are built for
    int lds_bytes;             // stages
    const void* kernel;        // fused (every reducer placement)
    const void* gemm_kernel;   // the same GEMM without flags or reduction
    const void* kernel_nt;     // `kernel` storing routed tiles non-temporally
    const void* gemm_kernel_nt;  // `gemm_kernel` storing routed tiles non-temporally
    const void* kernel_rows;   // `kernel` reading row counters
    const void* ag_kernel;     // all-gather + GEMM: copy phase, then the GEMM waiting for rows
    const void* ag_gemm_kernel;  // the same GEMM over an already gathered buffer
    const void* stream_kernel;   // fused, reduce_mode STREAM (or null)
    const void* kernel_dyn;      // fused, reduce_mode ADAPTIVE (the sum between the tiles)
    int stream_lds_bytes;        // its stages, stream slots and probe area
    int stream_threads;          // its workgroup size
    int fused_lds_bytes;         // LDS of `kernel` (set by variant_desc)
    int fused_threads;           // workgroup size of `kernel` (set by variant_desc)
};

// Eight-wave tiles run one workgroup per CU with two waves per SIMD; four-wave
// tiles that cannot fit two workgroups per CU get the occupancy-1 kernel (one
// wave per SIMD, the whole register file).
template <class C, bool FUSED, bool TWO_PER_CU, int VAR = 0>
const void* kernel_for()
{
    if constexpr (C::WAVES == 8)
        return reinterpret_cast<const void*>(&fused_kernel_8w<C, FUSED, VAR>);
    else if constexpr (TWO_PER_CU)
        return reinterpret_cast<const void*>(&fused_kernel<C, FUSED, VAR>);
    else
        return reinterpret_cast<const void*>(&fused_kernel_1w<C, FUSED, VAR>);
}

template <class C, bool FUSED, bool TWO_PER_CU>
const void* ag_kernel_for()
{
    if constexpr (C::WAVES == 8)
        return reinterpret_cast<const void*>(&ag_kernel_8w<C, FUSED>);
    else if constexpr (TWO_PER_CU)
        return reinterpret_cast<const void*>(&ag_kernel<C, FUSED>);
    else
        return reinterpret_cast<const void*>(&ag_kernel_1w<C, FUSED>);
}

template <class C, class CS = void>
TileDesc desc()
{
    static_assert(C::LDS_BYTES <= 160 * 1024 - 64, "LDS of one workgroup");
    // occupancy is set by the stages
    constexpr bool two = C::LDS_BYTES <= 80 * 1024 - 64;
    const void* sk = nullptr;
    int slds = 0, sthreads = 0;
    if constexpr (!std::is_void<CS>::value) {
        static_assert(CS::BM == C::BM && CS::BN == C::BN && CS::LDS_BYTES + kStreamLds <= 160 * 1024 - 256,
                      "the stream kernel's tile and LDS");
        sk = reinterpret_cast<const void*>(&fused_kernel_8w<CS, true>);
        slds = CS::LDS_BYTES + kStreamLds;
        sthreads = CS::THREADS;
    }
    return TileDesc{C::BM, C::BN, C::BK, C::THREADS, C::WAVES == 4 && two ? 2 : 1, C::LDS_BYTES,
                    kernel_for<C, true, two>(), kernel_for<C, false, two>(),
                    kernel_for<C, true, two, kVarNt>(), kernel_for<C, false, two, kVarNt>(),
                    kernel_for<C, true, two, kVarRows>(),
                    ag_kernel_for<C, true, two>(), ag_kernel_for<C, false, two>(), sk,
                    kernel_for<C, true, two, kVarDyn>(), slds, sthreads, C::LDS_BYTES, C::THREADS};
}

TileDesc tile_desc(int id)
{
    switch (id) {
    case GEMM_RS_TILE_16x64: return desc<Tile16x64>();
    case GEMM_RS_TILE_64x128: return desc<Tile64x128>();
    case GEMM_RS_TILE_128x128: return desc<Tile128x128>();
    case GEMM_RS_TILE_128x256: return desc<Tile128x256>();
    case GEMM_RS_TILE_256x128: return desc<Tile256x128>();
    case GEMM_RS_TILE_256x256: return desc<Tile256x256, Tile256x256S>();
    default:
        return TileDesc{0, 0, 0, 0, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, 0, 0};
    }
}

// Host-only tile geometry (no kernel pointer needed).
void tile_shape(int id, int* bm, int* bn)
{
    static const int shapes[GEMM_RS_TILE_COUNT][2] = {
        {0, 0}, {16, 64}, {64, 128}, {128, 128}, {128, 256}, {256, 128}, {256, 256}};
    *bm = (id > 0 && id < GEMM_RS_TILE_COUNT) ? shapes[id][0] : 0;
    *bn = (id > 0 && id < GEMM_RS_TILE_COUNT) ? shapes[id][1] : 0;
}

int auto_tile(const gemm_rs_config& c)
{
    const int S = c.M / c.tp;
    if (S >= 256 && c.N >= 256) return GEMM_RS_TILE_256x256;
    if (S >= 128 && c.N >= 128) return GEMM_RS_TILE_128x128;
    if (S >= 64 && c.N >= 128) return GEMM_RS_TILE_64x128;
    return GEMM_RS_TILE_16x64;
}

int resolve_tile(const gemm_rs_config& c) { return c.tile == GEMM_RS_TILE_AUTO ? auto_tile(c) : c.tile; }

// Where the slice sum of a fused run without dedicated reducers runs.
// AUTO: the stream where it can run beside the GEMM and pays for its slower
// GEMM: the 256x256 tile, at least kProbe + 2 K steps, three or more rounds of
// tiles on a 256-CU device (768 tiles; the own slice, an eighth of them, is
// released during the first rounds and the stream runs in the later ones),
// and K_local below kAutoStreamMaxK.  The stream kernel is the eight-wave
// tile (four waves stream); the sum after the last tile runs on the faster
// four-wave tile, whose lead grows with K while the sum's share of the work
// shrinks as 1/K_local (measured: the stream ahead at K_local = 2048, behind
// at 3584).  Otherwise the sum after the last tile.
constexpr int kAutoStreamTiles = 3 * 256;
constexpr int kAutoStreamMaxK = 3072;

int resolve_reduce_mode(const gemm_rs_config& c)
{
    if (c.num_reducers > 0) return GEMM_RS_REDUCE_TAIL;
    if (c.num_reducers == -2) return GEMM_RS_REDUCE_ADAPTIVE;
    if (c.reduce_mode == GEMM_RS_REDUCE_AUTO) {
        if (resolve_tile(c) != GEMM_RS_TILE_256x256 || c.K_local < (kProbe + 2) * 64)
            return GEMM_RS_REDUCE_TAIL;
        const int64_t S = c.M / c.tp;
        const int64_t tiles = (int64_t)c.tp * ((S + 255) / 256) * (((int64_t)c.N + 255) / 256);
        return tiles >= kAutoStreamTiles && c.K_local < kAutoStreamMaxK ? GEMM_RS_REDUCE_STREAM
                                                                          : GEMM_RS_REDUCE_TAIL;
    }
    return c.reduce_mode;
}

// The store policy a config runs (GEMM_RS_STORES_AUTO resolved): the
// non-temporal hint pays on the 256x256 tile from four rounds of tiles when
// the sum runs after the tiles (measured 0.3-0.8% at 16 rounds, 2.5% at 8;
// nothing at one or three rounds, 1% slower on the 64x128 tile, no gain on
// the stream's).
constexpr int kAutoNtTiles = 4 * 256;

int resolve_stores(const gemm_rs_config& c)
{
    if (c.tile_stores != GEMM_RS_STORES_AUTO) return c.tile_stores;
    if (resolve_tile(c) != GEMM_RS_TILE_256x256 || resolve_reduce_mode(c) != GEMM_RS_REDUCE_TAIL ||
        c.flag_protocol != GEMM_RS_FLAGS_TILE)
        return GEMM_RS_STORES_DEVICE;
    const int64_t S = c.M / c.tp;
    const int64_t tiles = (int64_t)c.tp * ((S + 255) / 256) * (((int64_t)c.N + 255) / 256);
    return tiles >= kAutoNtTiles ? GEMM_RS_STORES_NONTEMPORAL : GEMM_RS_STORES_DEVICE;
}

Geometry geometry_of(const gemm_rs_config& c)
{
    int bm, bn;
    tile_shape(resolve_tile(c), &bm, &bn);
    int gm = c.group_m;
    const int S = c.M / c.tp;
    const int tms = S > 0 ? ceil_div(S, bm) : 0;
    if (gm <= 0) gm = tms < 8 ? (tms > 0 ? tms : 1) : 8;
    return make_geometry(c.M, c.N, c.K_local, c.tp, c.rank, bm, bn, 64, gm);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }


}  // namespace

struct gemm_rs_handle {
    gemm_rs_config cfg;
    Geometry g;
    int tile_id;
    TileDesc td;
    int device;
    int num_cus;
    int wgs_per_cu;
    int fused_lds;
    int gemm_grid;         // workgroups of a GEMM-only launch
    // a STREAM handle's all-reduce runs: the tile's kernel summing after the
    // last tile (the stream stores only into `out`)
    const void* tail_kernel;
    int tail_lds;
    // all-gather + GEMM runs
    uint32_t* agflags;     // tp * tile rows per slice copy counters
    uint32_t* agfinished;  // per workgroup of ag_grid
    int ag_grid;
    int ag_strided;
    int ag_units;
    uint32_t ag_unit_bytes;
    int reduce_mode;       // resolved GEMM_RS_REDUCE_* (TAIL when dedicated reducers run the sum)
    int grid;
    int compute_wgs;
    int reducer_wgs;
    int reduce_grid;
    int flag_stride;
    int strided;
    uint32_t* flags;
    DeviceState* state;
    uint32_t* trace;
    uint32_t* finished;
    uint16_t* scratch;
    hipStream_t last_stream;
};

namespace {

// Distinct tile rows plus tile columns that one XCD touches in the first round
// of the schedule (a proxy for its L2 footprint per K step) under the
// contiguous or the strided split of the round.
long xcd_footprint(const Geometry& g, int grid, int R, bool strided)
{
    long worst = 0;
    const int C = grid - R;
    const int n = C < g.tiles ? C : g.tiles;
    for (int x = 0; x < kGroups; ++x) {
        const int gq = grid / kGroups, rq = R / kGroups, rr = R % kGroups;
        const int cnt = gq - rq - (x < rr ? 1 : 0);
        const int base = x * (gq - rq) - (x < rr ? x : rr);
        // at most 64 tile rows and 512 columns are tracked exactly
        unsigned char rowseen[8 * 64] = {0};
        static thread_local unsigned char colseen[512];
        memset(colseen, 0, sizeof colseen);
        long rowsn = 0, colsn = 0;
        for (int l = 0; l < cnt; ++l) {
            const int q = strided ? l * kGroups + x : base + l;
            if (q >= n) continue;
            const TileCoord t = decode_slot(g, q);
            const int rk = (t.d * g.tms + t.tml) % (8 * 64), ck = t.tn % 512;
            if (!rowseen[rk]) { rowseen[rk] = 1; ++rowsn; }
            if (!colseen[ck]) { colseen[ck] = 1; ++colsn; }
        }
        const long fp = rowsn * g.bm + colsn * g.bn;
        if (fp > worst) worst = fp;
    }
    return worst;
}

}  // namespace

extern "C" {

int gemm_rs_validate(const gemm_rs_config* c)
{
    if (!c) return GEMM_RS_ERR_INVALID_ARG;
    if (c->M < 0 || c->N < 0 || c->K_local < 0) return GEMM_RS_ERR_INVALID_ARG;
    if (c->rank < 0 || c->rank >= c->tp) return GEMM_RS_ERR_INVALID_ARG;
    if (c->tile < 0 || c->tile >= GEMM_RS_TILE_COUNT) return GEMM_RS_ERR_INVALID_ARG;
    if (c->group_m < 0) return GEMM_RS_ERR_INVALID_ARG;
    if (c->num_reducers < -2) return GEMM_RS_ERR_INVALID_ARG;
    // num_reducers -2 is the adaptive controller, as reduce_mode ADAPTIVE
    if (c->num_reducers == -2 && c->reduce_mode != GEMM_RS_REDUCE_AUTO && c->reduce_mode != GEMM_RS_REDUCE_ADAPTIVE)
        return GEMM_RS_ERR_INVALID_ARG;
    if (c->debug_flags & ~GEMM_RS_DEBUG_TRACE) return GEMM_RS_ERR_INVALID_ARG;
    if (c->drop_flag < -1) return GEMM_RS_ERR_INVALID_ARG;
    if (c->flag_stride != 0 && c->flag_stride != 1 && c->flag_stride != 32) return GEMM_RS_ERR_INVALID_ARG;
    if (c->watchdog_us < 0) return GEMM_RS_ERR_INVALID_ARG;
    if (c->tile_stores != GEMM_RS_STORES_DEVICE && c->tile_stores != GEMM_RS_STORES_NONTEMPORAL &&
        c->tile_stores != GEMM_RS_STORES_AUTO)
        return GEMM_RS_ERR_INVALID_ARG;
    if (c->flag_protocol != GEMM_RS_FLAGS_TILE && c->flag_protocol != GEMM_RS_FLAGS_ROW_COUNTER)
        return GEMM_RS_ERR_INVALID_ARG;
    if (c->reduce_mode < GEMM_RS_REDUCE_AUTO || c->reduce_mode > GEMM_RS_REDUCE_ADAPTIVE)
        return GEMM_RS_ERR_INVALID_ARG;
    // (AUTO resolves to a policy every placement accepts)
    const int stores = resolve_stores(*c);
    // both are kernel variants of the fused kernel (and, for the stores, of
    // the GEMM-only kernel); one at a time
    if (stores == GEMM_RS_STORES_NONTEMPORAL && c->flag_protocol == GEMM_RS_FLAGS_ROW_COUNTER)
        return GEMM_RS_ERR_INVALID_ARG;
    // the stream and the adaptive kernels are the default store policy with
    // tile flags
    const bool adaptive = c->num_reducers == -2 || c->reduce_mode == GEMM_RS_REDUCE_ADAPTIVE;
    if ((c->reduce_mode == GEMM_RS_REDUCE_STREAM || adaptive) &&
        (stores != GEMM_RS_STORES_DEVICE || c->flag_protocol != GEMM_RS_FLAGS_TILE))
        return GEMM_RS_ERR_INVALID_ARG;
    if (c->reduce_mode != GEMM_RS_REDUCE_AUTO && c->reduce_mode != GEMM_RS_REDUCE_TAIL && c->num_reducers > 0)
        return GEMM_RS_ERR_INVALID_ARG;
    if (c->tp != 8) return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
    if (c->M % c->tp != 0) return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
    if (c->N % 8 != 0 || c->K_local % 8 != 0) return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
    // every row-major element offset must fit the kernels' 64-bit arithmetic
    // and every tile count a 32-bit int
    const int64_t S = c->M / c->tp;
    if ((int64_t)c->M * c->K_local > ((int64_t)1 << 40) || (int64_t)c->N * c->K_local > ((int64_t)1 << 40) ||
        S * (int64_t)c->N > ((int64_t)1 << 40))
        return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
    // slice buffers are written through buffer resources with 31-bit byte
    // offsets
    if ((int64_t)(c->M / c->tp) * c->N * 2 >= ((int64_t)1 << 31)) return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
    // X_r and W_r are read through buffer resources with 31-bit byte offsets
    if ((int64_t)c->M * c->K_local * 2 >= ((int64_t)1 << 31) ||
        (int64_t)c->N * c->K_local * 2 >= ((int64_t)1 << 31))
        return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
    int bm, bn;
    tile_shape(resolve_tile(*c), &bm, &bn);
    const int64_t tiles = (int64_t)c->tp * ((S + bm - 1) / bm) * (((int64_t)c->N + bn - 1) / bn);
    if (tiles > (1 << 30)) return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
    if (c->drop_flag >= 0 && c->drop_flag >= tiles) return GEMM_RS_ERR_INVALID_ARG;
    // the stream kernel: the 256x256 tile, and at least kProbe + 2 K steps per
    // tile (its waits count the stream loads of the previous tile's last
    // steps, and the readiness probe is read at step kProbe)
    if (c->reduce_mode == GEMM_RS_REDUCE_STREAM &&
        (resolve_tile(*c) != GEMM_RS_TILE_256x256 || c->K_local < (kProbe + 2) * 64))
        return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
    return GEMM_RS_OK;
}

int gemm_rs_plan(const gemm_rs_config* c, gemm_rs_info* info)
{
    int rc = gemm_rs_validate(c);
    if (rc != GEMM_RS_OK) return rc;
    if (!info) return GEMM_RS_ERR_INVALID_ARG;
    memset(info, 0, sizeof *info);
    const Geometry g = geometry_of(*c);
    info->bm = g.bm;
    info->bn = g.bn;
    info->bk = g.bk;
    info->group_m = g.group_m;
    info->tiles = g.tiles;
    info->tiles_per_slice = g.ts;
    info->tile_rows_per_slice = g.tms;
    info->tile_cols = g.tnc;
    info->reduce_mode = resolve_reduce_mode(*c);
    info->tile_stores = resolve_stores(*c);
    return GEMM_RS_OK;
}

int gemm_rs_plan_slots(const gemm_rs_config* c, int32_t* slot_d, int32_t* slot_tm, int32_t* slot_tn,
                       int32_t* slot_flag, size_t n)
{
    int rc = gemm_rs_validate(c);
    if (rc != GEMM_RS_OK) return rc;
    const Geometry g = geometry_of(*c);
    if ((size_t)g.tiles > n) return GEMM_RS_ERR_INVALID_ARG;
    for (int q = 0; q < g.tiles; ++q) {
        const TileCoord t = decode_slot(g, q);
        if (slot_d) slot_d[q] = t.d;
        if (slot_tm) slot_tm[q] = t.d * g.tms + t.tml;
        if (slot_tn) slot_tn[q] = t.tn;
        if (slot_flag) slot_flag[q] = t.flag;
    }
    return GEMM_RS_OK;
}

const char* gemm_rs_strerror(int code)
{
    switch (code) {
    case GEMM_RS_OK: return "success";
    case GEMM_RS_ERR_INVALID_ARG: return "invalid argument";
    case GEMM_RS_ERR_UNSUPPORTED_SHAPE: return "unsupported shape (tp must be 8, M a multiple of tp, N and K_local multiples of 8)";
    case GEMM_RS_ERR_MISALIGNED: return "buffer not 16-byte aligned";
    case GEMM_RS_ERR_NO_DEVICE: return "current HIP device is not a gfx950 GPU";
    case GEMM_RS_ERR_HIP: return g_hip_msg[0] ? g_hip_msg : "HIP runtime error";
    case GEMM_RS_ERR_TIMEOUT: return "a reducer timed out waiting for a tile's ready flag";
    case GEMM_RS_ERR_NO_MEMORY: return "out of memory";
    case GEMM_RS_ERR_SCRATCH:
        return "the problem needs more device scratch (ready flags, finish marks, run state) than the "
               "allocation-free entry point's static array holds (GEMM_RS_STATIC_SCRATCH_BYTES)";
    default: return "unknown error";
    }
}

// Sets the dedicated-reducer count of fused launches (and the XCD split that
// goes with it).
static void set_split(gemm_rs_handle* h, int red)
{
    if (red >= h->grid) red = h->grid - 1;
    h->reducer_wgs = red;
    h->compute_wgs = h->grid - red;
    h->strided = (h->reducer_wgs % kGroups == 0 && h->g.tiles > 0 &&
                  xcd_footprint(h->g, h->grid, h->reducer_wgs, true) <
                      xcd_footprint(h->g, h->grid, h->reducer_wgs, false))
                     ? 1 : 0;
}

static void free_state(gemm_rs_handle* h)
{
    if (h->flags) (void)hipFree(h->flags);
    if (h->state) (void)hipFree(h->state);
    if (h->trace) (void)hipFree(h->trace);
    if (h->finished) (void)hipFree(h->finished);
    if (h->scratch) (void)hipFree(h->scratch);
    if (h->agflags) (void)hipFree(h->agflags);
    if (h->agfinished) (void)hipFree(h->agfinished);
}

// The tile and kernel variant a (valid) config runs: the store policy, the
// flag protocol or the stream selects a separate instantiation of the fused
// kernel.
static TileDesc variant_desc(const gemm_rs_config& c, int* variant)
{
    TileDesc td = tile_desc(resolve_tile(c));
    *variant = 0;
    const int mode = resolve_reduce_mode(c);
    if (mode == GEMM_RS_REDUCE_STREAM) {
        td.kernel = td.stream_kernel;
        td.fused_lds_bytes = td.stream_lds_bytes;
        td.fused_threads = td.stream_threads;
        *variant = 3;
    } else if (mode == GEMM_RS_REDUCE_ADAPTIVE) {
        td.kernel = td.kernel_dyn;
        *variant = 4;
    } else if (resolve_stores(c) == GEMM_RS_STORES_NONTEMPORAL) {
        td.kernel = td.kernel_nt;
        td.gemm_kernel = td.gemm_kernel_nt;
        *variant = 1;
    } else if (c.flag_protocol == GEMM_RS_FLAGS_ROW_COUNTER) {
        td.kernel = td.kernel_rows;
        *variant = 2;
    }
    return td;
}

// Gives the fused and GEMM-only kernels of td their dynamic LDS size and
// returns in *occ how many fused workgroups fit on one CU.
static int kernel_setup(const TileDesc& td, int* occ)
{
    HIP_TRY(hipFuncSetAttribute(td.kernel, hipFuncAttributeMaxDynamicSharedMemorySize, td.fused_lds_bytes));
    HIP_TRY(hipFuncSetAttribute(td.gemm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, td.lds_bytes));
    HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, td.kernel, td.fused_threads, td.fused_lds_bytes));
    return GEMM_RS_OK;
}

// Fills the launch plan of a handle for a valid config on device dev (no
// allocation, no device call): tile, kernels, persistent grid, reducer split.
// occ: fused workgroups per CU (kernel_setup).
static int plan_launch(gemm_rs_handle* h, const gemm_rs_config* c, int dev, int num_cus, int occ)
{
    int variant = 0;
    h->cfg = *c;
    h->g = geometry_of(*c);
    h->tile_id = resolve_tile(*c);
    h->td = variant_desc(*c, &variant);
    h->device = dev;
    h->num_cus = num_cus;
    h->flag_stride = c->flag_stride == 0 ? 1 : c->flag_stride;
    // automatic: no dedicated reducers, the compute workgroups sum the slice
    const int red_req = c->num_reducers < 0 ? 0 : c->num_reducers;
    h->reduce_mode = resolve_reduce_mode(*c);
    h->fused_lds = h->td.fused_lds_bytes;
    {
        const TileDesc base = tile_desc(h->tile_id);
        h->tail_kernel = base.kernel;
        h->tail_lds = base.lds_bytes;
    }
    // the persistent grid holds the workgroups per CU the kernel was built for
    // (more would share a SIMD's registers between more waves than planned)
    h->wgs_per_cu = occ < 1 ? 1 : (occ > h->td.wgs_per_cu ? h->td.wgs_per_cu : occ);
    // a whole number of workgroups per XCD group
    h->grid = (h->num_cus * h->wgs_per_cu) / kGroups * kGroups;
    if (h->grid < kGroups) h->grid = kGroups;
    h->gemm_grid = h->grid;
    int red = red_req;
    if (h->reduce_mode == GEMM_RS_REDUCE_CORESIDENT) {
        // one more workgroup per CU, which must fit beside the compute ones
        if (occ < h->wgs_per_cu + 1) return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
        red = h->num_cus / kGroups * kGroups;
        h->grid += red;
        h->wgs_per_cu += 1;
    }
    if (red >= h->grid) red = h->grid - 1;
    h->reduce_grid = h->num_cus * 8;
    set_split(h, red);
    // a stream workgroup probes the flags of its items' own tiles in one
    // 64-lane load: its items may span at most 64 tiles
    if (h->reduce_mode == GEMM_RS_REDUCE_STREAM && h->g.ts > 0 &&
        (h->g.ts + h->compute_wgs - 1) / h->compute_wgs + 1 > 64)
        return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
    return GEMM_RS_OK;
}

int gemm_rs_create(const gemm_rs_config* c, gemm_rs_handle** out)
{
    if (!out) return GEMM_RS_ERR_INVALID_ARG;
    *out = nullptr;
    int rc = gemm_rs_validate(c);
    if (rc != GEMM_RS_OK) return rc;

    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, dev));
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_RS_ERR_NO_DEVICE;

    int variant = 0, occ = 0;
    const TileDesc vd = variant_desc(*c, &variant);
    rc = kernel_setup(vd, &occ);
    if (rc != GEMM_RS_OK) return rc;
    if (variant == 3) {
        const TileDesc base = tile_desc(resolve_tile(*c));
        HIP_TRY(hipFuncSetAttribute(base.kernel, hipFuncAttributeMaxDynamicSharedMemorySize, base.lds_bytes));
    }
    gemm_rs_handle* h = new (std::nothrow) gemm_rs_handle();
    if (!h) return GEMM_RS_ERR_NO_MEMORY;
    rc = plan_launch(h, c, dev, prop.multiProcessorCount, occ);
    if (rc != GEMM_RS_OK) { delete h; return rc; }
    hipError_t e = hipSuccess;
    // all-gather + GEMM launches: the compute grid of the same tile (no reducers)
    for (const void* k : {h->td.ag_kernel, h->td.ag_gemm_kernel}) {
        e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, h->td.lds_bytes);
        if (e != hipSuccess) { delete h; return hip_fail(e, "hipFuncSetAttribute"); }
    }
    int ag_occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&ag_occ, h->td.ag_kernel, h->td.threads, h->td.lds_bytes);
    if (e != hipSuccess) { delete h; return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor"); }
    {
        const int per_cu = ag_occ < 1 ? 1 : (ag_occ > h->td.wgs_per_cu ? h->td.wgs_per_cu : ag_occ);
        h->ag_grid = (h->num_cus * per_cu) / kGroups * kGroups;
        if (h->ag_grid < kGroups) h->ag_grid = kGroups;
    }
    h->ag_strided = (h->g.tiles > 0 && xcd_footprint(h->g, h->ag_grid, 0, true) <
                                           xcd_footprint(h->g, h->ag_grid, 0, false)) ? 1 : 0;
    // copy units of 64 KiB: a tile-row block of BM rows is split into ag_units
    h->ag_unit_bytes = 64u << 10;
    {
        const int64_t blk = (int64_t)h->g.bm * h->g.K * 2;
        h->ag_units = (int)((blk + h->ag_unit_bytes - 1) / h->ag_unit_bytes);
        if (h->ag_units < 1) h->ag_units = 1;
    }
    const size_t agblocks = (size_t)h->g.tp * (size_t)(h->g.tms > 0 ? h->g.tms : 1);

    const size_t tiles = (size_t)(h->g.tiles > 0 ? h->g.tiles : 1);
    // the slot log, then the slice-sum stamps of the own tiles and the launch
    const size_t trace_words = ((size_t)h->g.tiles + (size_t)h->g.ts + 1) * 4;
    const size_t slice = (size_t)h->g.S * (size_t)h->g.N;
    if (hipMalloc(&h->agflags, agblocks * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc(&h->agfinished, (size_t)h->ag_grid * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc(&h->flags, tiles * h->flag_stride * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc(&h->state, sizeof(DeviceState)) != hipSuccess ||
        hipMalloc(&h->trace, trace_words * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc(&h->finished, (size_t)h->grid * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc(&h->scratch, (slice > 0 ? slice : 8) * sizeof(uint16_t)) != hipSuccess) {
        free_state(h);
        delete h;
        return GEMM_RS_ERR_NO_MEMORY;
    }
    if (hipMemset(h->agflags, 0, agblocks * sizeof(uint32_t)) != hipSuccess ||
        hipMemset(h->agfinished, 0, (size_t)h->ag_grid * sizeof(uint32_t)) != hipSuccess ||
        hipMemset(h->flags, 0, tiles * h->flag_stride * sizeof(uint32_t)) != hipSuccess ||
        hipMemset(h->state, 0, sizeof(DeviceState)) != hipSuccess ||
        hipMemset(h->trace, 0, trace_words * sizeof(uint32_t)) != hipSuccess ||
        hipMemset(h->finished, 0, (size_t)h->grid * sizeof(uint32_t)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        free_state(h);
        delete h;
        return hip_fail(hipGetLastError(), "hipMemset");
    }
    h->last_stream = nullptr;
    *out = h;
    return GEMM_RS_OK;
}

static void fill_args(gemm_rs_handle* h, Args& a, const void* x, const void* w, void* const* send,
                      const void* const* peers, void* out, uint16_t* local, void* const* gather)
{
    memset(&a, 0, sizeof a);
    a.x = static_cast<const uint16_t*>(x);
    a.w = static_cast<const uint16_t*>(w);
    const int r = h->g.rank;
    for (int d = 0; d < h->g.tp; ++d) {
        if (d == r)
            a.dst[d] = local;
        else
            a.dst[d] = send ? static_cast<uint16_t*>(send[d < r ? d : d - 1]) : nullptr;
    }
    for (int i = 0; i < kPeers; ++i) a.peers[i] = peers ? static_cast<const uint16_t*>(peers[i]) : nullptr;
    a.out = static_cast<uint16_t*>(out);
    a.gather_on = gather ? 1 : 0;
    for (int i = 0; i < kPeers; ++i) a.gather[i] = gather ? static_cast<uint16_t*>(gather[i]) : nullptr;
    a.flags = h->flags;
    a.state = h->state;
    a.status = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(h->state) + offsetof(DeviceState, status));
    a.trace = h->trace;
    a.sum_trace = h->trace ? h->trace + (int64_t)h->g.tiles * 4 : nullptr;
    a.finished = h->finished;
    a.g = h->g;
    a.x_bytes = (uint32_t)((int64_t)h->g.M * h->g.K * 2);
    a.w_bytes = (uint32_t)((int64_t)h->g.N * h->g.K * 2);
    a.slice_bytes = (uint32_t)((int64_t)h->g.S * h->g.N * 2);
    a.strided = h->strided;
    const int64_t us = h->cfg.watchdog_us > 0 ? h->cfg.watchdog_us : 2000000;
    a.watchdog_ticks = us * 100;  // 100 MHz real-time counter
    a.flag_stride = h->flag_stride;
    a.drop_flag = h->cfg.drop_flag;
    a.trace_on = (h->cfg.debug_flags & GEMM_RS_DEBUG_TRACE) ? 1 : 0;
    a.coresident = h->reduce_mode == GEMM_RS_REDUCE_CORESIDENT ? 1 : 0;
}

static int launch_gemm(gemm_rs_handle* h, Args& a, bool fused, hipStream_t s, bool tail = false)
{
    a.fused = fused ? 1 : 0;
    a.num_compute = fused ? h->compute_wgs : h->grid;
    a.num_reducers = fused ? h->reducer_wgs : 0;
    // GEMM_ONLY has no reducers, so its groups always split evenly
    if (!fused) a.strided = h->strided;
    void* params[] = {&a};
    const void* k = fused ? (tail ? h->tail_kernel : h->td.kernel) : h->td.gemm_kernel;
    // (a GEMM-only launch runs on the compute workgroups' grid: the
    // co-resident reducers' extra workgroup per CU is not part of the GEMM)
    if (!fused) a.num_compute = h->gemm_grid;
    HIP_TRY(hipLaunchKernel(k, dim3(fused ? h->grid : h->gemm_grid),
                            dim3(fused && !tail ? h->td.fused_threads : h->td.threads), params,
                            fused ? (tail ? h->tail_lds : h->fused_lds) : h->td.lds_bytes, s));
    return GEMM_RS_OK;
}

static int launch_reduce(gemm_rs_handle* h, Args& a, hipStream_t s)
{
    const int64_t chunks = (int64_t)h->g.S * h->g.N / 8;
    int64_t want = (chunks + kReduceThreads - 1) / kReduceThreads;
    int grid = (int)(want < h->reduce_grid ? want : h->reduce_grid);
    if (grid < 1) grid = 1;
    void* params[] = {&a};
    HIP_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&reduce_kernel), dim3(grid), dim3(kReduceThreads), params,
                            0, s));
    return GEMM_RS_OK;
}

// The buffers of a run of a valid mode on a non-empty problem: present where
// the mode uses them, 16-byte aligned, and the current device the handle's.
static int check_run(const gemm_rs_handle* h, int32_t mode, const void* x, const void* w, void* const* send,
                     const void* const* peers, const void* out, const void* local, void* const* gather)
{
    const bool needs_gemm = mode != GEMM_RS_MODE_REDUCE_ONLY;
    const bool needs_sum = mode != GEMM_RS_MODE_GEMM_ONLY;
    if (!aligned16(local)) return GEMM_RS_ERR_MISALIGNED;
    if (needs_gemm) {
        // with K_local == 0 the inputs are never read and may be NULL
        if (!send || ((!x || !w) && h->g.K > 0)) return GEMM_RS_ERR_INVALID_ARG;
        if (!aligned16(x) || !aligned16(w)) return GEMM_RS_ERR_MISALIGNED;
        for (int i = 0; i < kPeers; ++i) {
            if (!send[i]) return GEMM_RS_ERR_INVALID_ARG;
            if (!aligned16(send[i])) return GEMM_RS_ERR_MISALIGNED;
        }
    }
    if (needs_sum) {
        if (!out || !peers) return GEMM_RS_ERR_INVALID_ARG;
        if (!aligned16(out)) return GEMM_RS_ERR_MISALIGNED;
        for (int i = 0; i < kPeers; ++i) {
            if (!peers[i]) return GEMM_RS_ERR_INVALID_ARG;
            if (!aligned16(peers[i])) return GEMM_RS_ERR_MISALIGNED;
        }
        if (gather) {
            for (int i = 0; i < kPeers; ++i) {
                if (!gather[i]) return GEMM_RS_ERR_INVALID_ARG;
                if (!aligned16(gather[i])) return GEMM_RS_ERR_MISALIGNED;
            }
        }
    }
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev != h->device) return GEMM_RS_ERR_INVALID_ARG;
    return GEMM_RS_OK;
}

// Enqueues a checked run; status, if set, replaces the handle's status words.
static int launch_run(gemm_rs_handle* h, int32_t mode, const void* x, const void* w, void* const* send,
                      const void* const* peers, void* out, uint16_t* local, void* const* gather, int32_t* status,
                      hipStream_t s)
{
    const bool needs_sum = mode != GEMM_RS_MODE_GEMM_ONLY;
    Args a;
    fill_args(h, a, x, w, send, peers, out, local, needs_sum ? gather : nullptr);
    if (status) a.status = status;
    if (mode == GEMM_RS_MODE_FUSED && a.trace_on) {
        // the slice-sum stamps start empty (a fill kernel: safe in a captured graph)
        void* params[] = {&a.sum_trace, &h->g.ts};
        HIP_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&sum_trace_clear_kernel), dim3(1), dim3(256), params, 0,
                                s));
    }
    int rc = GEMM_RS_OK;
    switch (mode) {
    case GEMM_RS_MODE_FUSED:
        // (the all-reduce's sum also stores every gather buffer: on a STREAM
        // handle it runs after the last tile)
        rc = launch_gemm(h, a, true, s, needs_sum && gather && h->reduce_mode == GEMM_RS_REDUCE_STREAM);
        break;
    case GEMM_RS_MODE_GEMM_ONLY: rc = launch_gemm(h, a, false, s); break;
    case GEMM_RS_MODE_REDUCE_ONLY: rc = launch_reduce(h, a, s); break;
    case GEMM_RS_MODE_SEQUENTIAL:
        rc = launch_gemm(h, a, false, s);
        if (rc == GEMM_RS_OK) rc = launch_reduce(h, a, s);
        break;
    }
    return rc;
}

static int run_impl(gemm_rs_handle* h, int32_t mode, const void* x, const void* w, void* const* send,
                    const void* const* peers, void* out, void* local_slice, void* const* gather, void* stream)
{
    if (!h) return GEMM_RS_ERR_INVALID_ARG;
    if (mode < GEMM_RS_MODE_FUSED || mode > GEMM_RS_MODE_SEQUENTIAL) return GEMM_RS_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    h->last_stream = s;
    // an empty slice or no columns: nothing is read or written, buffers may be NULL
    if (h->g.S == 0 || h->g.N == 0) return GEMM_RS_OK;
    uint16_t* local = static_cast<uint16_t*>(local_slice ? local_slice : h->scratch);
    const int rc = check_run(h, mode, x, w, send, peers, out, local, gather);
    if (rc != GEMM_RS_OK) return rc;
    return launch_run(h, mode, x, w, send, peers, out, local, gather, nullptr, s);
}

int gemm_rs_run(gemm_rs_handle* h, int32_t mode, const void* x, const void* w, void* const* send,
                const void* const* peers, void* out, void* local_slice, void* stream)
{
    return run_impl(h, mode, x, w, send, peers, out, local_slice, nullptr, stream);
}

int gemm_rs_run_allreduce(gemm_rs_handle* h, int32_t mode, const void* x, const void* w, void* const* send,
                          const void* const* peers, void* out, void* local_slice, void* const* gather,
                          void* stream)
{
    if (mode != GEMM_RS_MODE_GEMM_ONLY && !gather) return GEMM_RS_ERR_INVALID_ARG;
    return run_impl(h, mode, x, w, send, peers, out, local_slice, gather, stream);
}

int gemm_rs_run_allgather(gemm_rs_handle* h, int32_t mode, const void* const* x_slices, const void* w,
                          void* x_gathered, void* y, void* stream)
{
    if (!h) return GEMM_RS_ERR_INVALID_ARG;
    if (mode < GEMM_RS_MODE_FUSED || mode > GEMM_RS_MODE_SEQUENTIAL) return GEMM_RS_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    h->last_stream = s;
    if (h->g.S == 0) return GEMM_RS_OK;
    // y [M][N] is written through a buffer resource with 31-bit byte offsets
    if ((int64_t)h->g.M * h->g.N * 2 >= ((int64_t)1 << 31)) return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
    const bool needs_copy = mode != GEMM_RS_MODE_GEMM_ONLY;
    const bool needs_gemm = mode != GEMM_RS_MODE_REDUCE_ONLY;
    if (!x_slices || !x_gathered) return GEMM_RS_ERR_INVALID_ARG;
    if (!aligned16(x_gathered)) return GEMM_RS_ERR_MISALIGNED;
    if (mode == GEMM_RS_MODE_FUSED) {
        // the fused launch's no-stale-line argument needs every 128-byte line of
        // x_gathered inside one copy block: the buffer and each slice aligned
        if ((reinterpret_cast<uintptr_t>(x_gathered) & 127u) != 0) return GEMM_RS_ERR_MISALIGNED;
        if (((int64_t)h->g.S * h->g.K * 2) % 128 != 0) return GEMM_RS_ERR_UNSUPPORTED_SHAPE;
    }
    for (int d = 0; d < h->g.tp; ++d) {
        // GEMM_ONLY reads only this rank's own slice (the rest from x_gathered)
        if (!needs_copy && d != h->g.rank) continue;
        if (!x_slices[d] && h->g.K > 0) return GEMM_RS_ERR_INVALID_ARG;
        if (!aligned16(x_slices[d])) return GEMM_RS_ERR_MISALIGNED;
    }
    if (needs_gemm) {
        if (!y || (!w && h->g.K > 0)) return GEMM_RS_ERR_INVALID_ARG;
        if (!aligned16(y) || !aligned16(w)) return GEMM_RS_ERR_MISALIGNED;
    }
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev != h->device) return GEMM_RS_ERR_INVALID_ARG;

    Args a;
    memset(&a, 0, sizeof a);
    a.w = static_cast<const uint16_t*>(w);
    for (int d = 0; d < h->g.tp; ++d) a.xsrc[d] = static_cast<const uint16_t*>(x_slices[d]);
    a.xg = static_cast<uint16_t*>(x_gathered);
    a.y = static_cast<uint16_t*>(y);
    a.agflags = h->agflags;
    a.agfinished = h->agfinished;
    a.state = h->state;
    a.g = h->g;
    a.x_bytes = (uint32_t)((int64_t)h->g.M * h->g.K * 2);
    a.w_bytes = (uint32_t)((int64_t)h->g.N * h->g.K * 2);
    a.xs_bytes = (uint32_t)((int64_t)h->g.S * h->g.K * 2);
    a.y_bytes = (uint32_t)((int64_t)h->g.M * h->g.N * 2);
    a.strided = h->ag_strided;
    const int64_t us = h->cfg.watchdog_us > 0 ? h->cfg.watchdog_us : 2000000;
    a.watchdog_ticks = us * 100;
    a.ag_units = h->ag_units;
    a.ag_unit_bytes = h->ag_unit_bytes;
    a.num_compute = h->ag_grid;
    void* params[] = {&a};
    if (mode == GEMM_RS_MODE_FUSED) {
        HIP_TRY(hipLaunchKernel(h->td.ag_kernel, dim3(h->ag_grid), dim3(h->td.threads), params, h->td.lds_bytes, s));
        return GEMM_RS_OK;
    }
    if (needs_copy) {
        const int64_t chunks = (int64_t)h->g.S * h->g.K / 8;
        int64_t want = (chunks + kReduceThreads - 1) / kReduceThreads;
        int grid = (int)(want < h->reduce_grid ? want : h->reduce_grid);
        if (grid < 1) grid = 1;
        HIP_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&ag_copy_kernel), dim3(grid), dim3(kReduceThreads),
                                params, 0, s));
    }
    if (needs_gemm)
        HIP_TRY(hipLaunchKernel(h->td.ag_gemm_kernel, dim3(h->ag_grid), dim3(h->td.threads), params, h->td.lds_bytes,
                                s));
    return GEMM_RS_OK;
}

int gemm_rs_status(gemm_rs_handle* h)
{
    if (!h) return GEMM_RS_ERR_INVALID_ARG;
    HIP_TRY(hipStreamSynchronize(h->last_stream));
    int32_t st[2] = {0, 0};
    char* dev_status = reinterpret_cast<char*>(h->state) + offsetof(DeviceState, status);
    HIP_TRY(hipMemcpy(st, dev_status, sizeof st, hipMemcpyDeviceToHost));
    if (st[0] != 0) {
        HIP_TRY(hipMemset(dev_status, 0, sizeof st));
        HIP_TRY(hipDeviceSynchronize());
        return st[0];
    }
    return GEMM_RS_OK;
}

int gemm_rs_query(gemm_rs_handle* h, gemm_rs_info* info)
{
    if (!h || !info) return GEMM_RS_ERR_INVALID_ARG;
    memset(info, 0, sizeof *info);
    info->bm = h->g.bm;
    info->bn = h->g.bn;
    info->bk = h->g.bk;
    info->group_m = h->g.group_m;
    info->tiles = h->g.tiles;
    info->tiles_per_slice = h->g.ts;
    info->tile_rows_per_slice = h->g.tms;
    info->tile_cols = h->g.tnc;
    info->grid = h->grid;
    info->compute_wgs = h->compute_wgs;
    info->reducer_wgs = h->reducer_wgs;
    info->num_cus = h->num_cus;
    info->wgs_per_cu = h->wgs_per_cu;
    info->lds_bytes = h->fused_lds;
    info->reduce_grid = h->reduce_grid;
    info->xcd_split = h->strided;
    info->reduce_mode = h->reduce_mode;
    info->split_state = h->reduce_mode == GEMM_RS_REDUCE_ADAPTIVE ? 1 : 0;
    info->tile_stores = resolve_stores(h->cfg);
    // every workgroup's finish mark holds the epoch of the last fused launch
    HIP_TRY(hipStreamSynchronize(h->last_stream));
    HIP_TRY(hipMemcpy(&info->epoch, h->finished, sizeof info->epoch, hipMemcpyDeviceToHost));
    return GEMM_RS_OK;
}

int gemm_rs_debug_read(gemm_rs_handle* h, uint32_t* slot_log, size_t slot_words, uint32_t* flags,
                       size_t flag_words)
{
    if (!h) return GEMM_RS_ERR_INVALID_ARG;
    const size_t tiles = (size_t)h->g.tiles;
    if (slot_log && slot_words < 4 * tiles) return GEMM_RS_ERR_INVALID_ARG;
    if (flags && flag_words < tiles) return GEMM_RS_ERR_INVALID_ARG;
    HIP_TRY(hipStreamSynchronize(h->last_stream));
    // with room for them, the slice-sum stamps follow the slot log
    const size_t words = 4 * (tiles + (size_t)h->g.ts + 1);
    if (slot_log && tiles)
        HIP_TRY(hipMemcpy(slot_log, h->trace, (slot_words >= words ? words : 4 * tiles) * sizeof(uint32_t),
                          hipMemcpyDeviceToHost));
    if (flags && tiles) {
        if (h->flag_stride == 1) {
            HIP_TRY(hipMemcpy(flags, h->flags, tiles * sizeof(uint32_t), hipMemcpyDeviceToHost));
        } else {
            HIP_TRY(hipMemcpy2D(flags, sizeof(uint32_t), h->flags, h->flag_stride * sizeof(uint32_t),
                                sizeof(uint32_t), tiles, hipMemcpyDeviceToHost));
        }
    }
    return GEMM_RS_OK;
}

void gemm_rs_destroy(gemm_rs_handle* h)
{
    if (!h) return;
    (void)hipDeviceSynchronize();
    free_state(h);
    delete h;
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free runs
//
// gemm_rs_run_static keeps what a handle allocates (the run state, the
// per-workgroup finish marks and the ready flags) in this array instead.  In
// host code `scratch` names a host-side stand-in: its device address on each
// GPU comes from hipGetSymbolAddress, taken once per device and used for
// every kernel argument.
static __device__ __align__(256) uint32_t scratch[GEMM_RS_STATIC_SCRATCH_BYTES / 4];

// Zeroes n words at p and, if st is set, the two status words there (a kernel
// rather than a memset, so that a captured graph holds no memset node).
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, uint32_t n, int32_t* st)
{
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
    if (st && blockIdx.x == 0 && threadIdx.x < 2) st[threadIdx.x] = 0;
}

namespace {

constexpr int kMaxDevices = 64;
constexpr int kVariants = 5;

// Per device, filled on the first allocation-free call there.
struct StaticDevice {
    bool ready;
    bool gfx950;
    int num_cus;
    uint32_t* ptr;                                  // the device's copy of `scratch`
    int occ[GEMM_RS_TILE_COUNT][kVariants];         // fused workgroups per CU; -1: not yet set up
};

std::mutex g_static_mu;
StaticDevice g_static[kMaxDevices];

}  // namespace

extern "C" int gemm_rs_run_static(const gemm_rs_config* c, int32_t mode, const void* x, const void* w,
                                  void* const* send, const void* const* peers, void* out, void* local_slice,
                                  int32_t* status, void* stream)
{
    int rc = gemm_rs_validate(c);
    if (rc != GEMM_RS_OK) return rc;
    if (mode < GEMM_RS_MODE_FUSED || mode > GEMM_RS_MODE_SEQUENTIAL) return GEMM_RS_ERR_INVALID_ARG;
    // no trace log (its buffer)
    if (c->debug_flags != 0) return GEMM_RS_ERR_INVALID_ARG;
    if (!local_slice) return GEMM_RS_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(status) & 3u) != 0) return GEMM_RS_ERR_MISALIGNED;
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return GEMM_RS_ERR_INVALID_ARG;
    int variant = 0;
    const TileDesc td = variant_desc(*c, &variant);
    const int tile = resolve_tile(*c);
    StaticDevice sd;
    {
        std::lock_guard<std::mutex> lock(g_static_mu);
        StaticDevice& e = g_static[dev];
        if (!e.ready) {
            hipDeviceProp_t prop;
            HIP_TRY(hipGetDeviceProperties(&prop, dev));
            void* p = nullptr;
            HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
            e.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            e.num_cus = prop.multiProcessorCount;
            e.ptr = static_cast<uint32_t*>(p);
            for (int i = 0; i < GEMM_RS_TILE_COUNT; ++i)
                for (int j = 0; j < kVariants; ++j) e.occ[i][j] = -1;
            e.ready = true;
        }
        if (e.gfx950 && e.occ[tile][variant] < 0) {
            int occ = 0;
            rc = kernel_setup(td, &occ);
            if (rc != GEMM_RS_OK) return rc;
            e.occ[tile][variant] = occ;
        }
        sd = e;
    }
    if (!sd.gfx950) return GEMM_RS_ERR_NO_DEVICE;

    gemm_rs_handle h{};
    rc = plan_launch(&h, c, dev, sd.num_cus, sd.occ[tile][variant]);
    if (rc != GEMM_RS_OK) return rc;
    // layout: run state, finish marks, ready flags (each 256-byte aligned)
    const size_t state_words = (sizeof(DeviceState) + 255) / 256 * 64;
    const size_t fin_words = ((size_t)h.grid + 63) / 64 * 64;
    const size_t flag_words = (size_t)(h.g.tiles > 0 ? h.g.tiles : 1) * (size_t)h.flag_stride;
    if (state_words + fin_words + flag_words > GEMM_RS_STATIC_SCRATCH_BYTES / 4) return GEMM_RS_ERR_SCRATCH;
    h.state = reinterpret_cast<DeviceState*>(sd.ptr);
    h.finished = sd.ptr + state_words;
    h.flags = h.finished + fin_words;

    hipStream_t s = static_cast<hipStream_t>(stream);
    h.last_stream = s;
    if (h.g.S == 0 || h.g.N == 0) return GEMM_RS_OK;
    uint16_t* local = static_cast<uint16_t*>(local_slice);
    rc = check_run(&h, mode, x, w, send, peers, out, local, nullptr);
    if (rc != GEMM_RS_OK) return rc;
    // every run starts from zeroed flags and finish marks (run epoch 1): a
    // call before it may have had another geometry
    const uint32_t nclear = (uint32_t)(state_words + fin_words + flag_words);
    {
        void* args[] = {&sd.ptr, const_cast<uint32_t*>(&nclear), &status};
        const int blocks = (int)((nclear + 255) / 256 < 1024 ? (nclear + 255) / 256 : 1024);
        HIP_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&clear_words_kernel), dim3(blocks), dim3(256), args, 0,
                                s));
    }
    // the kernels report a timeout into the caller's words, if any
    int32_t* st_dev = status ? status
                             : reinterpret_cast<int32_t*>(reinterpret_cast<char*>(h.state) + offsetof(DeviceState, status));
    return launch_run(&h, mode, x, w, send, peers, out, local, nullptr, st_dev, s);
}
