// kernels.hpp -- gfx950 device code of the fused BF16 GEMM + reduce-scatter.
//
// One persistent kernel holds two workgroup roles, in the spirit of mKernel's
// compute / communication roles ("mKernel: Fast Multi-GPU, Multi-Node Fused
// Kernels", sections 3 and 3.2) and of FLUX's reduce-scatter epilogue (TL;DR of
// "FLUX: Fast Software-based Communication Overlap On GPUs Through Kernel
// Fusion"):
//   compute   GEMM tiles on bf16 MFMA with FP32 accumulators.  A and B tiles go
//             from HBM straight into LDS (buffer loads with the LDS-direct bit),
//             NS stages deep, so several BK steps of loads are in flight while
//             the MFMAs consume the oldest stage.  The epilogue rounds the tile
//             to BF16, stores it into its destination slice buffer at device
//             scope and publishes the tile's ready flag;
//   reducer   sums this rank's slice with the tp-1 peer partials, tile by tile
//             as the ready flags arrive.
// The reduction runs either in dedicated reducer workgroups or, by default,
// inside the compute workgroups: there the first half of the waves ("loader"
// waves) issue every stage load of the GEMM and the second half ("engine"
// waves) run the reduce engine between their MFMAs.  Vector-memory operations
// of one wave retire in issue order, so an HBM load issued by a wave that also
// waits for stage loads would hold every later stage of that wave behind one
// HBM round trip; engine waves wait for stage loads only through the barrier.
//
// Workgroup g belongs to group g % 8, which is the XCD it runs on (workgroups
// are dispatched to the 8 XCDs round-robin).  Each group hands out its own
// arrival tickets: the first C_x arrivals of group x compute, the next R_x
// reduce.  A reducer therefore exists only after every compute workgroup of its
// group is resident, and compute workgroups never wait, so reducers cannot
// starve their producers.  Compute slots are split so that the workgroups of
// one XCD work on tiles that share rows of X or columns of W in that XCD's L2.
//
// The run epoch, the tickets and the reducer work counter live in device
// memory (see fused_body), so a launch needs no host-side state and can be
// replayed from a captured graph.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace gemm_rs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kReduceThreads = 256;  // standalone reduce kernel
constexpr int kPeers = 7;      // tp - 1 with tp = 8
constexpr int kGroups = 8;     // XCDs of an MI355X
constexpr int kStatusTimeout = -6;  // GEMM_RS_ERR_TIMEOUT
// A buffer offset at or past the resource's byte count reads as zero and
// drops a store.
constexpr uint32_t kOob = 0x80000000u;
// Third descriptor word of a raw buffer resource on gfx9-family GPUs.
constexpr int kRsrcFlags = 0x00020000;
// Cache-policy bits of a buffer store: sc1 makes it device scope (written
// through this XCD's L2 to the memory side, where a device-scope load on any
// XCD sees it once the store has completed -- no L2 write-back is needed to
// publish a tile).
constexpr int kStoreDevice = 16;
// Cache-policy bits of the engine's loads and stores: peer partials are read
// once and sums written once (non-temporal); the local slice and the flags are
// read at device scope (sc1), so a copy left in this XCD's L2 by an earlier
// run is never used.
constexpr int kAuxNt = 2;
constexpr int kAuxSc1 = 16;
// Routed tile stores with the non-temporal hint on top of device scope: the
// tile is not read back through this XCD's L2 (the sum reads the local slice
// at device scope, the send buffers leave the GPU), so it need not displace
// the GEMM's operands there.
constexpr int kStoreDeviceNt = kStoreDevice | kAuxNt;

// Kernel variants (a template parameter of the fused and GEMM kernels, so that
// the default kernel carries no code of the others): bit 0 stores routed tiles
// with kStoreDeviceNt, bit 1 reads row counters instead of tile flags.
constexpr int kVarNt = 1;
constexpr int kVarRows = 2;

// Reduce engine: 16-byte loads per operation (one per lane each), LDS bytes an
// operation lands in, operations in flight per engine wave.
constexpr int kEngLoads = 2;
constexpr int kEngAreaBytes = kEngLoads * 1024;
constexpr int kEngAreas = 2;

// Handle-owned device state, zeroed at creation.
struct DeviceState {
    uint32_t pad1;
    uint32_t role[kGroups];   // per-group arrival tickets (dedicated reducers only)
    uint32_t unit;            // next reducer unit to claim
    uint32_t pad0;
    int32_t status[2];        // [0] error code, [1] flag index that timed out
    uint32_t pad[3];
};

struct Args {
    const uint16_t* x;       // [M][K]
    const uint16_t* w;       // [N][K]
    uint16_t* dst[8];        // destination slice buffers by destination rank
    const uint16_t* peers[kPeers];
    uint16_t* out;           // [S][N]
    uint16_t* gather[kPeers];  // all-reduce runs: [S][N] copies of out, one per peer
    int32_t gather_on;       // 1: every summed chunk is also stored into gather[]
    uint32_t* flags;         // ready flags, flag_stride words apart
    DeviceState* state;
    uint32_t* trace;         // 4 words per slot (debug)
    uint32_t* finished;      // per workgroup: epoch of the last fused launch it finished
    Geometry g;
    uint32_t x_bytes, w_bytes;
    uint32_t slice_bytes;    // S * N * 2
    int64_t watchdog_ticks;  // 100 MHz ticks
    int32_t num_compute;     // C: compute workgroups in the grid
    int32_t num_reducers;    // R
    int32_t strided;         // XCD split of a round: 0 contiguous, 1 strided
    int32_t flag_stride;
    int32_t fused;           // 1: release flags, reducers run, epoch advances
    int32_t drop_flag;
    int32_t trace_on;
    int32_t engine_every;    // K steps between reduce-engine slots (0: reduce after the last tile)
    int32_t coresident;      // 1: the reducer workgroups sit beside the compute workgroups of
                             // their CUs and sum a static share of items (peers first)
    // all-gather + GEMM runs (the column-parallel layer): M x K gathered
    // activations times this rank's N x K weight shard
    const uint16_t* xsrc[8];  // row slice [S][K] of source rank d; xsrc[rank] is this rank's own
    uint16_t* xg;            // gathered activations [M][K] (x_bytes long)
    uint16_t* y;             // output [M][N]
    uint32_t* agflags;       // per (source rank, tile row): copy units done, summed over runs
    uint32_t* agfinished;    // per workgroup: count of all-gather launches it finished
    uint32_t y_bytes;        // M * N * 2
    uint32_t xs_bytes;       // S * K * 2
    uint32_t ag_unit_bytes;  // bytes of one copy unit
    int32_t ag_units;        // copy units per tile-row block (BM rows of one slice)
};

// BM x BN output tile, BK deep stages, NS stages in LDS, WAVES_M x WAVES_N
// waves (4: one wave per SIMD, 8: two), MF x MF MFMA output blocks (32:
// v_mfma_f32_32x32x16_bf16, 16: v_mfma_f32_16x16x32_bf16).  The first LW waves
// issue the stage loads (LW = 0: all of them); the other EW waves run the
// reduce engine.
template <int BM_, int BN_, int BK_, int NS_, int WAVES_M_, int WAVES_N_, int MF_, int LW_ = 0>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, NS = NS_;
    static_assert(NS >= 2 && NS <= 4, "stage depth");
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static_assert(WAVES == 4 || WAVES == 8, "four or eight waves per workgroup");
    static constexpr int LW = LW_ > 0 ? LW_ : WAVES;
    static constexpr int EW = WAVES - LW;
    static constexpr int LTHREADS = 64 * LW;
    static constexpr int MF = MF_;
    static constexpr int KF = MF_ == 32 ? 16 : 32;  // k per MFMA
    static constexpr int KSUB = BK / KF;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / MF, FN = WTN / MF;
    static_assert(FM >= 1 && FN >= 1 && WTM % MF == 0 && WTN % MF == 0, "wave tile");
    static constexpr int CPR = BK / 8;               // 16-byte chunks per LDS row
    static constexpr int ROW_BYTES = BK * 2;
    static constexpr int A_CHUNKS = BM * CPR, B_CHUNKS = BN * CPR;
    static_assert(A_CHUNKS % LTHREADS == 0 && B_CHUNKS % LTHREADS == 0, "whole load rounds");
    static constexpr int A_LD = A_CHUNKS / LTHREADS, B_LD = B_CHUNKS / LTHREADS;
    static constexpr int LPS = A_LD + B_LD;          // loads per loader thread per stage
    static_assert(LPS * (NS - 1) <= 63, "vmcnt range");
    static constexpr int A_BYTES = BM * ROW_BYTES;
    static constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;
    static constexpr int LDS_BYTES = NS * STAGE_BYTES;
    static_assert(CPR == 4 || CPR == 8 || CPR == 16, "swizzle defined for BK = 32, 64, 128");
    // Epilogue.  With 32x32 MFMA blocks and wave tiles a whole number of 64
    // columns wide, the BF16 tile goes through a per-wave 4 KiB LDS area (32
    // rows x 64 columns per pass) so that each store instruction writes 8 full
    // 128-byte row segments; otherwise every lane stores its own 8 bytes.
    // STORES is the number of store instructions per wave per tile (issued
    // unconditionally: lanes outside a ragged tile store out of bounds).
    static constexpr bool STAGED_EPI = MF == 32 && WTN % 64 == 0;
    static constexpr int EPI_AREA = 4096;
    static constexpr int STORES = STAGED_EPI ? FM * (WTN / 64) * 4 : FM * FN * (MF == 32 ? 4 : 1);
    static_assert(!STAGED_EPI || WAVES * EPI_AREA <= STAGE_BYTES, "epilogue staging fits one stage buffer");
    static_assert((NS - 2) * LPS + STORES <= 63, "vmcnt range");
    static constexpr int ENG_LDS = EW * kEngAreas * kEngAreaBytes;
    // One workgroup per CU (four waves whose stages fit only once, or eight
    // waves) with every wave loading: the K loop is pipelined across steps.
    static constexpr bool XP = EW == 0 && LDS_BYTES > 80 * 1024 - 64 && KSUB % 2 == 0;
};

template <int MF> struct AccT;
template <> struct AccT<32> { typedef f32x16 type; static constexpr int N = 16; };
template <> struct AccT<16> { typedef f32x4 type; static constexpr int N = 4; };

// LDS swizzle: the 16-byte chunk c of row r is stored at chunk c ^ swz(r).  The
// MFMA fragment reads take one chunk from each of 16 or 32 consecutive rows;
// these functions spread any 8 aligned consecutive rows (and the 8 rows of one
// parity among 16) over distinct chunks, so the reads hit distinct banks whether
// a b128 read is served 8 or 16 lanes at a time.
template <int CPR>
__host__ __device__ inline int swz(int r)
{
    if constexpr (CPR == 4) return ((r >> 1) ^ (r >> 3)) & 3;
    else if constexpr (CPR == 8) return ((r >> 1) & 7) ^ ((r & 1) << 2);
    else return ((r >> 1) & 7) ^ ((r & 1) << 3);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most n of this wave's vector-memory instructions are
// outstanding; n above 15 waits for 15 (longer than needed, never shorter).
__device__ __forceinline__ void wait_vmcnt_upto(uint32_t n)
{
    switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<15>(); break;
    }
}

// Execution barrier without the memory fence __syncthreads() implies (which
// would wait for every LDS-direct load in flight).  The asm memory clobber
// keeps the compiler from moving LDS reads of a stage above it.
__device__ __forceinline__ void stage_barrier()
{
    __asm__ __volatile__("s_barrier" ::: "memory");
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Two FP32 values to two BF16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
// A pointer every lane holds the same value of, made visibly uniform: buffer
// resources built from it then stay in scalar registers (a resource the
// compiler takes for divergent wraps every buffer access in a readfirstlane
// loop).
__device__ __forceinline__ const void* uni_ptr(const void* p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------- GEMM tile

template <class C>
struct TileState {
    typename AccT<C::MF>::type acc[C::FM][C::FN];
};

// Per-thread load plan of one tile (loader threads): byte offset of each chunk
// this thread moves at k = 0 (kOob for rows past the tile's valid extent) and
// the chunk's k offset (for the K tail).
template <class C>
struct LoadPlan {
    uint32_t a_off[C::A_LD], b_off[C::B_LD];
    uint16_t a_k[C::A_LD], b_k[C::B_LD];
};

template <class C>
__device__ __forceinline__ void make_plan(const Args& a, LoadPlan<C>& lp, int row0, int rows, int n0, int cols)
{
    const int tid = threadIdx.x;
    const uint32_t K = (uint32_t)a.g.K;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
        const int p = i * C::LTHREADS + tid;
        const int r = p / C::CPR;
        const int c = (p % C::CPR) ^ swz<C::CPR>(r);
        lp.a_k[i] = (uint16_t)(c * 8);
        lp.a_off[i] = r < rows ? ((uint32_t)(row0 + r) * K + (uint32_t)c * 8u) * 2u : kOob;
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
        const int p = i * C::LTHREADS + tid;
        const int r = p / C::CPR;
        const int c = (p % C::CPR) ^ swz<C::CPR>(r);
        lp.b_k[i] = (uint16_t)(c * 8);
        lp.b_off[i] = r < cols ? ((uint32_t)(n0 + r) * K + (uint32_t)c * 8u) * 2u : kOob;
    }
}

// Issue the LDS-direct loads of the BK slice starting at k0 into stage buffer
// `stage` (LPS loads per loader thread).  Each wave instruction fills 1 KiB of
// LDS: lane l writes bytes [16 l, 16 l + 16) after the wave's base.
//
// Branch-free: a chunk whose k lies at or past K (the K tail, or a whole stage
// past the end) gets an offset past the resource and reads as zero; rows past
// the tile carry kOob already, and kOob + 2 k0 stays past the resource.
template <class C>
__device__ __forceinline__ void issue_stage(const LoadPlan<C>& lp, __amdgpu_buffer_rsrc_t rx,
                                            __amdgpu_buffer_rsrc_t rw, char* stage, int k0, int K)
{
    // (uniform: the LDS destination, and with it M0, is scalar arithmetic)
    const int wave = uni((int)(threadIdx.x >> 6));
    const int lim = K - k0;  // chunks with k offset >= lim are past K
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
        const uint32_t off = (int)lp.a_k[i] < lim ? lp.a_off[i] + (uint32_t)k0 * 2u : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (lds_void_t*)(stage + (i * C::LTHREADS + wave * 64) * 16), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
        const uint32_t off = (int)lp.b_k[i] < lim ? lp.b_off[i] + (uint32_t)k0 * 2u : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (lds_void_t*)(stage + C::A_BYTES + (i * C::LTHREADS + wave * 64) * 16), 16, off, 0, 0, 0);
    }
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;

// Fragments of one MFMA k-substep s of a stage: FM X fragments and FN W
// fragments, one 16-byte LDS read each.
template <class C>
__device__ __forceinline__ void load_frags(const char* stage, int s, bf16x8 (&xf)[C::FM], bf16x8 (&wf)[C::FN])
{
    const int lane = threadIdx.x & 63;
    const int wave = uni((int)(threadIdx.x >> 6));
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const char* sa = stage;
    const char* sb = stage + C::A_BYTES;
    const int lr = lane % C::MF;
    const int c = s * (C::KF / 8) + lane / C::MF;  // logical chunk of this lane
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int r = wm * C::WTM + i * C::MF + lr;
        xf[i] = *reinterpret_cast<const bf16x8*>(sa + r * C::ROW_BYTES + ((c ^ swz<C::CPR>(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
        const int r = wn * C::WTN + j * C::MF + lr;
        wf[j] = *reinterpret_cast<const bf16x8*>(sb + r * C::ROW_BYTES + ((c ^ swz<C::CPR>(r)) << 4));
    }
}

// The W fragment is the MFMA's A operand and the X fragment its B operand, so
// the accumulator holds the transposed tile: lane l owns output row m = l % MF
// and, per group of four registers, four consecutive output columns.
template <class C>
__device__ __forceinline__ void mfma_substep(TileState<C>& st, const bf16x8 (&xf)[C::FM], const bf16x8 (&wf)[C::FN])
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            if constexpr (C::MF == 32)
                st.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], st.acc[i][j], 0, 0, 0);
            else
                st.acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf[i], st.acc[i][j], 0, 0, 0);
        }
}

// One K step: a loader wave refills the buffer of stage kt-1 with stage
// kt+NS-1; then the MFMAs of stage kt with the fragments of substep s+1 read
// while substep s computes.  The scheduling groups place the substep-0 reads
// first, then every direct load of the refill (the earlier they are issued,
// the longer they have to land before the next step waits for them:
// measured 4% on the large shape), then one LDS read after each MFMA, so no
// MFMA waits on a full LDS round trip.
template <class C, bool LOADER>
__device__ __forceinline__ void kstep(const LoadPlan<C>& lp, __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw,
                                      char* refill, int k_refill, int K, const char* cur, TileState<C>& st)
{
    bf16x8 xf[2][C::FM], wf[2][C::FN];
    load_frags<C>(cur, 0, xf[0], wf[0]);
    if constexpr (LOADER) issue_stage<C>(lp, rx, rw, refill, k_refill, K);
#pragma unroll
    for (int s = 0; s < C::KSUB; ++s) {
        if (s + 1 < C::KSUB) load_frags<C>(cur, s + 1, xf[(s + 1) & 1], wf[(s + 1) & 1]);
        mfma_substep<C>(st, xf[s & 1], wf[s & 1]);
    }
    constexpr int kMfmas = C::KSUB * C::FM * C::FN;
    constexpr int kFill = (C::KSUB - 1) * (C::FM + C::FN) + (LOADER ? C::LPS : 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, C::FM + C::FN, 0);
    if constexpr (LOADER) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, C::LPS, 0);
    constexpr int kFillDs = (C::KSUB - 1) * (C::FM + C::FN);
#pragma unroll
    for (int m = 0; m < kMfmas; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (m < kFillDs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
}

// Round the accumulators to BF16 and store the valid part of the tile into the
// destination slice buffer behind `rd` (byte offsets from the slice start) at
// device scope; the tile's first row is slice row `row0`.  Exactly C::STORES
// store instructions per wave, whatever the tile's valid extent: the vector-
// memory wait counts of the next tile rely on that.
//
// Staged path: per pass (one 32-row block i, one 64-column chunk c of the wave
// tile) each lane writes its 4 x 2 packed groups (row l % 32, 8-byte halves of
// 16-byte chunks) into the wave's LDS area, chunk k of row r at k ^ ((r>>1)&7)
// so that both the 32-row writes and the 8-row reads spread over all banks;
// then the wave reads 8 rows x 8 chunks per instruction and stores them.
// AUX: the stores' cache-policy bits.
template <class C, int AUX = kStoreDevice>
__device__ __forceinline__ void store_tile(const Args& a, const TileState<C>& st, char* area,
                                           __amdgpu_buffer_rsrc_t rd, int row0, int rows, int n0, int cols)
{
    const int lane = threadIdx.x & 63;
    const int wave = uni((int)(threadIdx.x >> 6));
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const uint32_t N = (uint32_t)a.g.N;
    if constexpr (C::STAGED_EPI) {
        char* buf = area + wave * C::EPI_AREA;
        const int r = lane & 31, h = lane >> 5;    // writer: row, chunk half
        const int rr = lane >> 3, ck = lane & 7;   // reader: row in an 8-row group, chunk
        char* wbase = buf + r * 128 + h * 8;
        const int wsw = (r >> 1) & 7;
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int c = 0; c < C::WTN / 64; ++c) {
#pragma unroll
                for (int j2 = 0; j2 < 2; ++j2)
#pragma unroll
                    for (int grp = 0; grp < 4; ++grp) {
                        const auto& acc = st.acc[i][c * 2 + j2];
                        const u32x2 v = {pack_bf16x2(acc[grp * 4 + 0], acc[grp * 4 + 1]),
                                         pack_bf16x2(acc[grp * 4 + 2], acc[grp * 4 + 3])};
                        *reinterpret_cast<u32x2*>(wbase + (((j2 * 4 + grp) ^ wsw) << 4)) = v;
                    }
                // LDS operations of one wave complete in order: the reads below
                // see the writes above, and the next pass's writes come after
                // these reads
                __asm__ __volatile__("" ::: "memory");
                const int n = wn * C::WTN + c * 64 + ck * 8;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int row = s4 * 8 + rr;
                    const u32x4 d = *reinterpret_cast<const u32x4*>(buf + row * 128 + ((ck ^ ((row >> 1) & 7)) << 4));
                    const int m = wm * C::WTM + i * 32 + row;
                    const uint32_t off =
                        (m < rows && n < cols) ? (((uint32_t)(row0 + m) * N + (uint32_t)(n0 + n)) * 2u) : kOob;
                    __builtin_amdgcn_raw_buffer_store_b128(d, rd, off, 0, AUX);
                }
                __asm__ __volatile__("" ::: "memory");
            }
    } else {
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            const int m = wm * C::WTM + i * C::MF + (lane % C::MF);
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                constexpr int G = C::MF == 32 ? 4 : 1;
#pragma unroll
                for (int grp = 0; grp < G; ++grp) {
                    const int n = C::MF == 32 ? wn * C::WTN + j * 32 + grp * 8 + (lane / 32) * 4
                                              : wn * C::WTN + j * 16 + (lane / 16) * 4;
                    const u32x2 v = {pack_bf16x2(st.acc[i][j][grp * 4 + 0], st.acc[i][j][grp * 4 + 1]),
                                     pack_bf16x2(st.acc[i][j][grp * 4 + 2], st.acc[i][j][grp * 4 + 3])};
                    const uint32_t off =
                        (m < rows && n < cols) ? (((uint32_t)(row0 + m) * N + (uint32_t)(n0 + n)) * 2u) : kOob;
                    __builtin_amdgcn_raw_buffer_store_b64(v, rd, off, 0, AUX);
                }
            }
        }
    }
}

// Publish a finished tile by storing its ready flag (device scope).  Called by
// one thread once every wave's stores of the tile have completed.  ROWS: the
// row-counter protocol (the tile's row counter is incremented instead).
template <bool ROWS = false>
__device__ __forceinline__ void publish(const Args& a, int q, int flag, uint32_t who, uint32_t epoch)
{
    if (a.trace_on) {
        const uint64_t now = wall_clock64();
        uint32_t* tr = a.trace + (int64_t)q * 4;
        tr[0] = (uint32_t)flag;
        tr[1] = who;
        tr[2] = (uint32_t)now;
        tr[3] = (uint32_t)(now >> 32);
    }
    if (flag != a.drop_flag) {
        if constexpr (ROWS)
            __hip_atomic_fetch_add(a.flags + (int64_t)(flag / a.g.tnc) * a.flag_stride, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        else
            __hip_atomic_store(a.flags + (int64_t)flag * a.flag_stride, epoch, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The word that says whether tile `flag` of this run is released: its own
// flag, or under the row-counter protocol its tile row's counter.
template <bool ROWS>
__device__ __forceinline__ const uint32_t* ready_word(const Args& a, int flag)
{
    const int idx = ROWS ? flag / a.g.tnc : flag;
    return a.flags + (int64_t)idx * a.flag_stride;
}

// Whether a ready word read in run `epoch` releases the tile: the flag holds
// the epoch, or the row counter has reached epoch * (tiles per row) -- every
// run adds one per tile, so the counter passes that value exactly when the
// whole row of this run is stored (compared modulo 2^32).
template <bool ROWS>
__device__ __forceinline__ bool released(const Args& a, uint32_t v, uint32_t epoch)
{
    if constexpr (ROWS)
        return (int32_t)(v - epoch * (uint32_t)a.g.tnc) >= 0;
    else
        return v == epoch;
}

// ---------------------------------------------------------------- slice sum

// acc + the 8 BF16 values packed in v (exact widening, one FP32 rounding per
// element).
__device__ __forceinline__ f32x8 add8(f32x8 acc, const u32x4& v)
{
    f32x8 b;
    b[0] = bf16_bits_to_f32(v.x & 0xFFFFu);
    b[1] = bf16_bits_to_f32(v.x >> 16);
    b[2] = bf16_bits_to_f32(v.y & 0xFFFFu);
    b[3] = bf16_bits_to_f32(v.y >> 16);
    b[4] = bf16_bits_to_f32(v.z & 0xFFFFu);
    b[5] = bf16_bits_to_f32(v.z >> 16);
    b[6] = bf16_bits_to_f32(v.w & 0xFFFFu);
    b[7] = bf16_bits_to_f32(v.w >> 16);
    return acc + b;
}

__device__ __forceinline__ u32x4 pack8(const f32x8& acc)
{
    u32x4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    return o;
}

// Stores one summed 16-byte chunk at byte offset boff of the slice: into
// `out` and, in an all-reduce run, also into the 7 gather buffers (the
// all-gather that follows the reduce-scatter replicates this rank's reduced
// slice to every peer).  Returns the number of store instructions issued.
__device__ __forceinline__ int store_sum(const Args& a, const u32x4& v, uint32_t boff)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, __builtin_amdgcn_make_buffer_rsrc(a.out, 0, a.slice_bytes, kRsrcFlags),
                                           boff, 0, kAuxNt);
    if (!a.gather_on) return 1;
#pragma unroll
    for (int i = 0; i < kPeers; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(
            v, __builtin_amdgcn_make_buffer_rsrc(a.gather[i], 0, a.slice_bytes, kRsrcFlags), boff, 0, kAuxNt);
    return 1 + kPeers;
}

template <int AUX>
__device__ __forceinline__ void lds_load16(const uint16_t* g, const char* slot)
{
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)slot, 16, 0, AUX);
}

__device__ __forceinline__ void lds_load_flag(const uint32_t* g, const char* slot)
{
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)slot, 4, 0, kAuxSc1);
}

// out = RNE( (((0 + peer_0) + ... + peer_6) + local ) for 8 elements at `off`
// (standalone reduce kernel; plain loads are coherent after the kernel
// boundary).
__device__ __forceinline__ void sum_chunk(const Args& a, const uint16_t* local, int64_t off)
{
    uint4 v[kPeers + 1];
#pragma unroll
    for (int s = 0; s < kPeers; ++s) v[s] = *reinterpret_cast<const uint4*>(a.peers[s] + off);
    v[kPeers] = *reinterpret_cast<const uint4*>(local + off);
    f32x8 acc = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s <= kPeers; ++s) {
        const u32x4 w = {v[s].x, v[s].y, v[s].z, v[s].w};
        acc = add8(acc, w);
    }
    const u32x4 o = pack8(acc);
    *reinterpret_cast<uint4*>(a.out + off) = make_uint4(o.x, o.y, o.z, o.w);
    if (a.gather_on) {
#pragma unroll
        for (int i = 0; i < kPeers; ++i) *reinterpret_cast<uint4*>(a.gather[i] + off) = make_uint4(o.x, o.y, o.z, o.w);
    }
}

// Sum a rows x cols block of the slice starting at (row0, col0), 16-byte
// chunks distributed over `nthreads` threads starting at `tid`.
__device__ __forceinline__ void sum_block(const Args& a, int row0, int rows, int col0, int cols, int tid,
                                          int nthreads)
{
    const uint16_t* local = a.dst[a.g.rank];
    const int cpr = cols >> 3;
    const int total = rows * cpr;
    const int64_t N = a.g.N;
    int c = tid;
    for (; c + nthreads < total; c += 2 * nthreads) {
        const int r0 = c / cpr, r1 = (c + nthreads) / cpr;
        const int64_t o0 = (int64_t)(row0 + r0) * N + col0 + (c - r0 * cpr) * 8;
        const int64_t o1 = (int64_t)(row0 + r1) * N + col0 + (c + nthreads - r1 * cpr) * 8;
        sum_chunk(a, local, o0);
        sum_chunk(a, local, o1);
    }
    if (c < total) {
        const int r0 = c / cpr;
        sum_chunk(a, local, (int64_t)(row0 + r0) * N + col0 + (c - r0 * cpr) * 8);
    }
}

// ---------------------------------------------------------------- reduce engine
//
// The slice sum is cut into items: item i covers 64 16-byte chunks (512
// elements) of own-slice tile t = i / IPT, one chunk per lane, where own tiles
// are numbered row-major (t = tile row * tile columns + tile column, so own
// tile t carries ready flag rank * tiles_per_slice + t); an item spans
// 64 / (BN/8) consecutive rows of the tile, so a lane's offset inside an item
// is a constant and the item's base offset is wave-uniform.  Engine wave gw (of
// W) owns items gw, gw + W, gw + 2W, ... -- tile order.
//
// Between MFMAs an engine wave sums the items whose tile is flagged, in four
// steps of two loads each, in the sum order:
//   step 0: peers 0, 1      acc = (0 + p0) + p1
//   step 1: peers 2, 3      acc = (acc + p2) + p3
//   step 2: peers 4, 5      acc = (acc + p4) + p5
//   step 3: peer 6, local   acc = (acc + p6) + local, rounded and stored to out
// and otherwise polls: POLL reads 64 consecutive ready flags (own tiles
// anchor .. anchor+63, one per lane).  Operations are issued and consumed in
// order, two in flight: each engine slot consumes the older operation and
// issues a new one.  The loads land in the wave's two LDS areas (LDS-direct
// global loads), so no register is live while they fly; the consumer waits
// with s_waitcnt until at most the vector-memory instructions issued after the
// operation are outstanding (the wave counts every one it issues: engine
// loads, out stores, epilogue stores).  Every lane issues every load and store
// (lanes without a valid chunk read the slice's first chunk and store out of
// bounds), so the count is exact.  Items still open after the wave's last
// tile are summed by engine_drain.

enum EngineOp { kOpNone = 0, kOpStep = 1, kOpPoll = 2 };

struct EngOp {
    int op, step, area, anchor;
    uint32_t soff;    // STEP 3: this lane's byte offset in out (kOob: no valid chunk)
    uint32_t vm_end;  // the wave's vector-memory count right after the operation's issue
};

// Where an item lies: item i is chunk row (i % IPT) * RPI .. of own tile
// i / IPT, tile t = tile row * tile columns + tile column.
struct ItemMap {
    int nitems;         // items of the slice
    int ipt_log2;       // log2(items per tile)
    int rpi;            // tile rows per item
    int lane_row, lane_col, lane_off;  // this lane's place inside an item
    uint32_t div_m;     // t / tile_cols = (umulhi(t, div_m) + t) >> div_l
    int div_l;
};

__device__ __forceinline__ ItemMap item_map(const Args& a)
{
    ItemMap m;
    const int lane = threadIdx.x & 63;
    const int cpr = a.g.bn >> 3;  // 16-byte chunks per tile row (8 .. 32)
    m.rpi = 64 / cpr;
    m.ipt_log2 = __builtin_ctz(a.g.bm / m.rpi);
    m.nitems = a.g.ts << m.ipt_log2;
    m.lane_row = lane / cpr;
    m.lane_col = (lane % cpr) * 8;
    m.lane_off = m.lane_row * a.g.N + m.lane_col;
    // multiply-shift division by the tile-column count d (exact for t < 2^31):
    // l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1
    const uint32_t d = (uint32_t)(a.g.tnc > 0 ? a.g.tnc : 1);
    m.div_l = d == 1 ? 0 : 32 - __builtin_clz(d - 1);
    m.div_m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << m.div_l) - d)) / d + 1);
    return m;
}

// Byte offset of this lane's chunk of an item in the slice; kOob if the chunk
// lies outside the possibly ragged tile or the item past the last one.
__device__ __forceinline__ uint32_t item_boff(const ItemMap& m, const Args& a, int item)
{
    const uint32_t t = (uint32_t)(item >> m.ipt_log2);
    const int j = item & ((1 << m.ipt_log2) - 1);
    const int tml = (int)((__umulhi(t, m.div_m) + t) >> m.div_l);
    const int tn = (int)t - tml * a.g.tnc;
    const int row = j * m.rpi;
    const int trows = min(a.g.bm, a.g.S - tml * a.g.bm);
    const int tcols = min(a.g.bn, a.g.N - tn * a.g.bn);
    const bool valid = item < m.nitems && row + m.lane_row < trows && m.lane_col < tcols;
    const uint32_t base = (uint32_t)(tml * a.g.bm + row) * (uint32_t)a.g.N + (uint32_t)(tn * a.g.bn);
    return valid ? (base + (uint32_t)m.lane_off) * 2u : kOob;
}

struct Engine {
    char* areas;    // kEngAreas LDS areas of kEngAreaBytes
    ItemMap m;
    int next;       // next owned item not yet started
    int stride;     // engine waves W
    int nitems, ipt, ipt_log2;  // copies of m's (items per tile: a power of two)
    // issue side
    int i_item;     // item being issued, -1 if none
    int i_step;     // its next step
    uint32_t i_off; // this lane's element offset in the slice (0 if no valid chunk)
    uint32_t i_soff;
    int anchor;     // tile of bit 0 of `ready`
    uint64_t ready; // ready tiles anchor .. anchor+63
    int area;       // area of the next operation
    // consume side
    f32x8 acc;
    // in flight, oldest first
    EngOp o0, o1;
    uint32_t vm;         // vector-memory instructions issued by this wave
    uint32_t vm_stores;  // vm right after this wave's last epilogue stores
    uint32_t epoch;
};

// Element offset of this lane's chunk of an item in the slice (0 if the chunk
// lies outside the possibly ragged tile) and its byte offset for a store
// (kOob then).
__device__ __forceinline__ void item_offsets(const Engine& e, const Args& a, int item, uint32_t& off,
                                             uint32_t& soff)
{
    soff = item_boff(e.m, a, item);
    off = soff == kOob ? 0u : soff >> 1;
}

__device__ __forceinline__ void engine_init(Engine& e, const Args& a, char* areas, int gw, int waves,
                                            uint32_t epoch)
{
    e.areas = areas;
    e.m = item_map(a);
    e.ipt_log2 = e.m.ipt_log2;
    e.ipt = 1 << e.ipt_log2;
    e.nitems = e.m.nitems;
    e.next = uni(gw);
    e.stride = waves;
    e.i_item = -1;
    e.i_step = 0;
    e.i_off = 0;
    e.i_soff = kOob;
    e.anchor = 0;
    e.ready = 0;
    e.area = 0;
    e.o0 = EngOp{kOpNone, 0, 0, 0, kOob, 0u};
    e.o1 = e.o0;
    e.vm = 0;
    e.vm_stores = 0;
    e.epoch = epoch;
}

__device__ __forceinline__ bool tile_ready(const Engine& e, int tile)
{
    const int b = tile - e.anchor;
    return b >= 0 && b < 64 && ((e.ready >> b) & 1ull);
}

// Move the ready window so that it starts at the oldest tile still needed.
__device__ __forceinline__ void engine_reanchor(Engine& e)
{
    int want = e.i_item >= 0 ? e.i_item : e.next;
    if (want > e.nitems) want = e.nitems;
    want >>= e.ipt_log2;
    const int sh = want - e.anchor;
    if (sh > 0) {
        e.ready = sh >= 64 ? 0ull : (e.ready >> sh);
        e.anchor = want;
    }
}

__device__ __forceinline__ char* area_ptr(const Engine& e, int area) { return e.areas + area * kEngAreaBytes; }

__device__ __forceinline__ u32x4 engine_chunk(const Engine& e, int area, int k)
{
    return *reinterpret_cast<const u32x4*>(area_ptr(e, area) + k * 1024 + (threadIdx.x & 63) * 16);
}

// Consume an operation whose loads have completed.
__device__ __forceinline__ void engine_consume(Engine& e, const Args& a, const EngOp& o)
{
    if (o.op == kOpStep) {
        f32x8 acc = o.step == 0 ? f32x8{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f} : e.acc;
        acc = add8(acc, engine_chunk(e, o.area, 0));
        acc = add8(acc, engine_chunk(e, o.area, 1));
        if (o.step < 3) {
            e.acc = acc;
        } else {
            e.vm += store_sum(a, pack8(acc), o.soff);
        }
    } else if (o.op == kOpPoll) {
        const int lane = threadIdx.x & 63;
        const uint32_t f = *reinterpret_cast<const uint32_t*>(area_ptr(e, o.area) + lane * 4);
        const bool mine = o.anchor + lane < a.g.ts;
        const uint64_t bits = __builtin_amdgcn_ballot_w64(mine && f == e.epoch);
        // the window has only moved forward since the poll was issued
        const int sh = e.anchor - o.anchor;
        if (sh < 64) e.ready |= bits >> sh;
    }
}

// Choose and issue the next operation; with `start` false no new item is
// begun and no flag is polled.
__device__ __forceinline__ EngOp engine_issue(Engine& e, const Args& a, bool start)
{
    EngOp o{kOpNone, 0, e.area, e.anchor, kOob, 0u};
    if (start && e.i_item < 0 && e.next < e.nitems && tile_ready(e, e.next >> e.ipt_log2)) {
        e.i_item = e.next;
        e.i_step = 0;
        e.next += e.stride;
        item_offsets(e, a, e.i_item, e.i_off, e.i_soff);
    }
    char* ar = area_ptr(e, o.area);
    if (e.i_item >= 0) {
        o.op = kOpStep;
        o.step = e.i_step;
        o.soff = e.i_soff;
        const uint32_t off = e.i_off;
        switch (e.i_step) {
        case 0:
            lds_load16<kAuxNt>(a.peers[0] + off, ar);
            lds_load16<kAuxNt>(a.peers[1] + off, ar + 1024);
            break;
        case 1:
            lds_load16<kAuxNt>(a.peers[2] + off, ar);
            lds_load16<kAuxNt>(a.peers[3] + off, ar + 1024);
            break;
        case 2:
            lds_load16<kAuxNt>(a.peers[4] + off, ar);
            lds_load16<kAuxNt>(a.peers[5] + off, ar + 1024);
            break;
        default:
            lds_load16<kAuxNt>(a.peers[6] + off, ar);
            lds_load16<kAuxSc1>(a.dst[a.g.rank] + off, ar + 1024);
            break;
        }
        e.vm += 2;
        if (++e.i_step == 4) e.i_item = -1;
    } else if (start && e.next < e.nitems) {
        o.op = kOpPoll;
        const int lane = threadIdx.x & 63;
        const int t = e.anchor + lane < a.g.ts ? e.anchor + lane : 0;
        lds_load_flag(a.flags + (int64_t)(a.g.rank * a.g.ts + t) * a.flag_stride, ar);
        e.vm += 1;
    }
    o.vm_end = e.vm;
    if (o.op != kOpNone) e.area ^= 1;
    engine_reanchor(e);
    // keep the issue order of these loads against later memory operations
    __builtin_amdgcn_sched_barrier(0);
    return o;
}

// One engine slot: consume the older operation in flight, issue a new one.
__device__ __forceinline__ void engine_step(Engine& e, const Args& a, bool start)
{
    if (e.o0.op != kOpNone) {
        wait_vmcnt_upto(e.vm - e.o0.vm_end);
        engine_consume(e, a, e.o0);
    }
    e.o0 = e.o1;
    e.o1 = engine_issue(e, a, start);
}

// Waits (device-scope polls, short sleeps) until own tile t is flagged.  The
// first wait that exceeds the watchdog limit reports the tile and sets
// gave_up; after that no wait blocks, so a drain never waits longer than one
// watchdog period in total.  ROWS: the row-counter protocol.
template <int SLEEP = 2, bool ROWS = false>
__device__ __forceinline__ bool wait_tile(const Args& a, uint32_t epoch, int t, bool& gave_up)
{
    const int flag = a.g.rank * a.g.ts + t;
    const uint32_t* f = ready_word<ROWS>(a, flag);
    if (released<ROWS>(a, __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), epoch)) return true;
    if (gave_up) return false;
    const uint64_t t0 = wall_clock64();
    while (!released<ROWS>(a, __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), epoch)) {
        __builtin_amdgcn_s_sleep(SLEEP);
        if ((int64_t)(wall_clock64() - t0) > a.watchdog_ticks) {
            gave_up = true;
            if ((threadIdx.x & 63) == 0 && atomicCAS(&a.state->status[0], 0, kStatusTimeout) == 0)
                atomicExch(&a.state->status[1], flag);
            return false;
        }
    }
    return true;
}

// Sums items first, first + stride, ... with plain loads (no LDS), BATCH items
// at a time: a batch's peer chunks are loaded before its tiles' flags are
// checked (they need none), then its local chunks, in the sum order.  A tile
// whose flag does not arrive within the watchdog limit is reported and its
// items are skipped.
// SLEEP: s_sleep argument between flag polls (64 clocks each); ROWS: the
// row-counter protocol.
template <int BATCH, int SLEEP = 2, bool ROWS = false>
__device__ __forceinline__ void drain_items(const Args& a, const ItemMap& m, int first, int stride, uint32_t epoch)
{
    constexpr int kDrainBatch = BATCH;
    bool gave_up = false;
    const __amdgpu_buffer_rsrc_t rl =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.dst[a.g.rank], 0, a.slice_bytes, kRsrcFlags);
    for (int base = first; base < m.nitems; base += kDrainBatch * stride) {
        uint32_t boff[kDrainBatch];
        u32x4 v[kDrainBatch][kPeers + 1];
#pragma unroll
        for (int b = 0; b < kDrainBatch; ++b) {
            boff[b] = item_boff(m, a, base + b * stride);
#pragma unroll
            for (int s = 0; s < kPeers; ++s) {
                const __amdgpu_buffer_rsrc_t rp =
                    __builtin_amdgcn_make_buffer_rsrc((void*)a.peers[s], 0, a.slice_bytes, kRsrcFlags);
                v[b][s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, boff[b], 0, kAuxNt));
            }
        }
#pragma unroll
        for (int b = 0; b < kDrainBatch; ++b) {
            const int item = base + b * stride;
            const bool ok = item < m.nitems && wait_tile<SLEEP, ROWS>(a, epoch, item >> m.ipt_log2, gave_up);
            boff[b] = ok ? boff[b] : kOob;
            v[b][kPeers] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, boff[b], 0, kAuxSc1));
        }
#pragma unroll
        for (int b = 0; b < kDrainBatch; ++b) {
            f32x8 acc = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s <= kPeers; ++s) acc = add8(acc, v[b][s]);
            store_sum(a, pack8(acc), boff[b]);
        }
    }
}

// After the last tile of an engine wave that ran in-loop slots: settle the
// operations in flight and the item being summed (its tile is flagged), then
// drain the wave's remaining items.
__device__ __forceinline__ void engine_drain(Engine& e, const Args& a)
{
    while (e.o0.op != kOpNone || e.o1.op != kOpNone || e.i_item >= 0) engine_step(e, a, false);
    wait_vmcnt<0>();
    drain_items<2>(a, e.m, e.next, e.stride, e.epoch);
}

// ---------------------------------------------------------------- reduce stream
//
// The slice sum streamed through the cross-step pipelined K loop (eight-wave
// workgroups, two stages).  With kStreamOps = 1 every wave streams; with 2
// one wave per SIMD (waves 0..3) does, at twice the rate, so that the sibling
// wave on its SIMD keeps the matrix core fed while the streaming wave runs the
// sum's bookkeeping (measured: no better).  Streaming wave gw of TW owns a
// contiguous range of items, [gw * n / TW, (gw + 1) * n / TW) of n, and per K
// step issues at most kStreamOps vector-memory instructions of the sum, right
// after its stage refill.  With two stages the next step's wait then lets
// those instructions stay outstanding (and only those), so an operation issued
// at step k has completed by the wait of step k + 2, where it is consumed: the
// sum adds nothing to the stage waits.  Loads land in the wave's LDS slots
// (LDS-direct loads), so nothing but the running FP32 sum is held in registers
// while they fly.
//
// Per item, in the sum order: poll the tile's ready flag (unless the wave has
// already seen that tile flagged), load peers 0..6 (they need no flag), load
// the local chunk once the flag has been seen, then store the rounded sum into
// `out` and, in an all-reduce run, into the 7 gather buffers, one store per
// step.  A poll that finds the tile not yet flagged is repeated only after
// kStreamBackoff steps; a step with nothing to issue and nothing in flight
// runs no stream code at all.  Items a streaming wave has not finished when
// the workgroup's last tile is done are summed by drain_items, split between
// that wave and the waves that do not stream on its SIMD.

constexpr int kStreamOps = 1;                      // per streaming wave and K step
constexpr int kStreamQueue = 2 * kStreamOps;       // operations in flight (two steps)
constexpr int kStreamSlots = kStreamQueue + 1;     // 1 KiB LDS slots per streaming wave
constexpr int kStreamLds = kStreamSlots * 1024;
constexpr int kStreamBackoff = 8;                  // K steps between polls of one tile

enum StreamOp { kSoNone = 0, kSoPeer = 1, kSoPoll = 2, kSoLocal = 3 };

struct Stream {
    char* slots;          // this wave's kStreamSlots LDS slots
    const uint16_t* local;
    ItemMap m;
    int item, end;        // next item to finish, end of the wave's range
    int phase;            // 0..6: load peer `phase`; 7: load local; 8: local in flight; 9..: stores
    int nst;              // stores per item (1, or 8 in an all-reduce run)
    int ready_tile;       // the last tile seen flagged (-1: none)
    int poll_tile;        // tile of the poll in flight (-1: none)
    int poll_wait;        // steps before the next poll may be issued
    int slot;             // slot of the next operation
    int q[kStreamQueue];  // operations in flight, oldest first (kSoNone: none)
    int nissued;          // vector-memory instructions the last step issued
    uint32_t soff;        // this lane's byte offset of the item's chunk (kOob: none)
    uint32_t epoch;
    int gw0, tw;          // the workgroup's first streaming wave, streaming waves in all
    f32x8 acc;
};

// arr[i] for a wave-uniform i in 0..6, as a chain of selects: a switch would
// merge the pointers through control flow, which the compiler may keep in
// vector registers (and then wrap every buffer access of the loop in a
// per-lane loop over its resource).
template <class T>
__device__ __forceinline__ T pick7(T const (&arr)[kPeers], int i)
{
    T r = arr[0];
#pragma unroll
    for (int k = 1; k < kPeers; ++k) r = i == k ? arr[k] : r;
    return r;
}

__device__ __forceinline__ void stream_item_start(Stream& s, const Args& a)
{
    s.phase = 0;
    s.soff = s.item < s.end ? item_boff(s.m, a, s.item) : kOob;
}

// Streaming wave gw of tw (gw0: the workgroup's first); a wave that does not
// stream passes active = false and gets an empty range.
__device__ __forceinline__ void stream_init(Stream& s, const Args& a, char* slots, int gw0, int gw, int tw,
                                            bool active, uint32_t epoch)
{
    s.slots = slots;
    s.local = a.dst[a.g.rank];
    s.m = item_map(a);
    s.gw0 = gw0;
    s.tw = tw;
    const int64_t n = s.m.nitems;
    s.item = active ? uni((int)(n * gw / tw)) : 0;
    s.end = active ? uni((int)(n * (gw + 1) / tw)) : 0;
    s.nst = a.gather_on ? 1 + kPeers : 1;
    s.ready_tile = -1;
    s.poll_tile = -1;
    s.poll_wait = 0;
    s.slot = 0;
#pragma unroll
    for (int i = 0; i < kStreamQueue; ++i) s.q[i] = kSoNone;
    s.nissued = 0;
    // (the epoch comes from an LDS read: make it provably uniform, so that
    // the whole stream state stays in scalar registers)
    s.epoch = (uint32_t)uni((int)epoch);
    s.acc = f32x8{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    stream_item_start(s, a);
}

// Operation code: kind | slot << 4 | peer << 8.
__device__ __forceinline__ void stream_consume(Stream& s, int code)
{
    const int kind = code & 15;
    if (kind == kSoNone) return;
    const char* slot = s.slots + ((code >> 4) & 7) * 1024;
    if (kind == kSoPoll) {
        const uint32_t f = (uint32_t)uni((int)*reinterpret_cast<const uint32_t*>(slot));
        if (f == s.epoch)
            s.ready_tile = s.poll_tile;
        else
            s.poll_wait = kStreamBackoff;
        s.poll_tile = -1;
        return;
    }
    const u32x4 v = *reinterpret_cast<const u32x4*>(slot + (threadIdx.x & 63) * 16);
    if (kind == kSoPeer && (code >> 8) == 0) s.acc = f32x8{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    s.acc = add8(s.acc, v);
    if (kind == kSoLocal) s.phase = 9;
}

// Issues the next operation, if any; returns its code (kSoNone when nothing
// was issued).
__device__ __forceinline__ int stream_issue(Stream& s, const Args& a)
{
    char* slot = s.slots + s.slot * 1024;
    const uint32_t off = s.soff == kOob ? 0u : s.soff >> 1;  // element offset of a valid chunk
    int code = kSoNone;
    bool issued = false;
    if (s.item < s.end) {
        const int tile = s.item >> s.m.ipt_log2;
        const bool ready = tile == s.ready_tile;
        if (!ready && s.poll_tile < 0 && s.poll_wait == 0 && (s.phase == 0 || s.phase == 7)) {
            lds_load_flag(a.flags + (int64_t)(a.g.rank * a.g.ts + tile) * a.flag_stride, slot);
            s.poll_tile = tile;
            code = kSoPoll;
            issued = true;
        } else if (s.phase < 7) {
            lds_load16<kAuxNt>(pick7(a.peers, s.phase) + off, slot);
            code = kSoPeer | (s.phase << 8);
            ++s.phase;
            issued = true;
        } else if (s.phase == 7 && ready) {
            lds_load16<kAuxSc1>(s.local + off, slot);
            code = kSoLocal;
            s.phase = 8;
            issued = true;
        } else if (s.phase >= 9) {
            const u32x4 v = pack8(s.acc);
            uint16_t* dst = s.phase == 9 ? a.out : pick7(a.gather, s.phase - 10);
            __builtin_amdgcn_raw_buffer_store_b128(v, __builtin_amdgcn_make_buffer_rsrc(dst, 0, a.slice_bytes, kRsrcFlags),
                                                   s.soff, 0, kAuxNt);
            issued = true;
            if (++s.phase == 9 + s.nst) {
                ++s.item;
                stream_item_start(s, a);
            }
        }
    }
    if (!issued) return kSoNone;
    ++s.nissued;
    code |= s.slot << 4;
    s.slot = s.slot == kStreamSlots - 1 ? 0 : s.slot + 1;
    return code;
}

// One K step of the stream, after the step's refill: kStreamOps times,
// consume the operation issued two steps ago and issue the next.  Nothing
// runs once the wave's items are done and nothing is in flight.
__device__ __forceinline__ void stream_step(Stream& s, const Args& a)
{
    __builtin_amdgcn_sched_barrier(0);
    bool busy = s.item < s.end;
#pragma unroll
    for (int i = 0; i < kStreamQueue; ++i) busy = busy || s.q[i] != kSoNone;
    s.nissued = 0;
    if (busy) {
        if (s.poll_wait > 0) --s.poll_wait;
#pragma unroll
        for (int k = 0; k < kStreamOps; ++k) {
            stream_consume(s, s.q[0]);
#pragma unroll
            for (int i = 0; i + 1 < kStreamQueue; ++i) s.q[i] = s.q[i + 1];
            s.q[kStreamQueue - 1] = stream_issue(s, a);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Wait for the stage refill issued by the previous step, letting the stream
// instructions issued after it stay in flight.
template <int B>
__device__ __forceinline__ void stream_wait(const Stream& s)
{
    static_assert(kStreamOps <= 2, "wait counts below");
    if (s.nissued == 0)
        wait_vmcnt<B>();
    else if (s.nissued == 1)
        wait_vmcnt<B + 1>();
    else
        wait_vmcnt<B + 2>();
}

// After a wait for every vector-memory instruction: consume what is in flight.
__device__ __forceinline__ void stream_settle(Stream& s)
{
#pragma unroll
    for (int i = 0; i < kStreamQueue; ++i) {
        stream_consume(s, s.q[i]);
        s.q[i] = kSoNone;
    }
    s.nissued = 0;
}

// After the last tile, in every wave of the workgroup: the items the streaming
// waves have not finished (an item in progress restarts) are split between
// each streaming wave w and the waves w + SW, w + 2 SW, ... on its SIMD.
// `progress` is an LDS array of SW entries; called by all waves, it holds one
// workgroup barrier.
template <int WAVES>
__device__ __forceinline__ void stream_drain(const Stream& s, const Args& a, int wave, int* progress)
{
    constexpr int SW = WAVES / kStreamOps;
    if (wave < SW && (threadIdx.x & 63) == 0) progress[wave] = s.item;
    __syncthreads();
    const int w = wave % SW, part = wave / SW;
    const int64_t n = s.m.nitems;
    const int gw = s.gw0 + w;
    const int end = (int)(n * (gw + 1) / s.tw);
    const int cur = uni(progress[w]);
    ItemMap m = s.m;
    m.nitems = cur + (end - cur) * (part + 1) / kStreamOps;
    drain_items<2>(a, m, cur + (end - cur) * part / kStreamOps, 1, s.epoch);
}


// ---------------------------------------------------------------- sum in the epilogue
//
// reduce_mode EPILOGUE (four-wave tiles small enough to keep a tile's peer
// chunks in registers): the workgroup that computes an own-slice tile sums it
// in its epilogue, from its accumulators, the way FLUX fuses the
// reduce-scatter into the GEMM epilogue (TL;DR of "FLUX: Fast Software-based
// Communication Overlap On GPUs Through Kernel Fusion").  Each lane loads the
// 7 peers' values of exactly the output elements its accumulators hold (the
// same element map as the unstaged tile store) before the tile's first stage
// loads, so they arrive with the first stage; the epilogue forms
// (((0 + p_0) + ...) + p_6) + RNE_bf16(acc) in FP32, the oracle's order, and
// stores it rounded to `out` (and the gather buffers in an all-reduce run).
// No flag is polled: the producer sums its own tile.

template <class C>
struct PeerFrag {
    static constexpr int G = C::MF == 32 ? 4 : 1;  // groups of four columns per MFMA block
    u32x2 v[kPeers][C::FM][C::FN][G];
};

// Loads the peer values of tile (srow0.., n0..) that this lane's accumulators
// hold; elements outside the (ragged) tile read as zero.
template <class C>
__device__ __forceinline__ void epi_load_peers(const Args& a, PeerFrag<C>& pf, int srow0, int rows, int n0, int cols)
{
    const int lane = threadIdx.x & 63;
    const int wave = uni((int)(threadIdx.x >> 6));
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const uint32_t N = (uint32_t)a.g.N;
#pragma unroll
    for (int s = 0; s < kPeers; ++s) {
        const __amdgpu_buffer_rsrc_t rp =
            __builtin_amdgcn_make_buffer_rsrc((void*)a.peers[s], 0, a.slice_bytes, kRsrcFlags);
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            const int m = wm * C::WTM + i * C::MF + (lane % C::MF);
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int grp = 0; grp < PeerFrag<C>::G; ++grp) {
                    const int n = C::MF == 32 ? wn * C::WTN + j * 32 + grp * 8 + (lane / 32) * 4
                                              : wn * C::WTN + j * 16 + (lane / 16) * 4;
                    const uint32_t off =
                        (m < rows && n < cols) ? (((uint32_t)(srow0 + m) * N + (uint32_t)(n0 + n)) * 2u) : kOob;
                    pf.v[s][i][j][grp] =
                        __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rp, off, 0, kAuxNt));
                }
        }
    }
}

// os = (((0 + p_0) + ... ) + p_6) + RNE_bf16(st), element by element (FP32).
template <class C>
__device__ __forceinline__ void epi_sum(const PeerFrag<C>& pf, const TileState<C>& st, TileState<C>& os)
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int grp = 0; grp < PeerFrag<C>::G; ++grp)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float acc = 0.0f;
#pragma unroll
                    for (int s = 0; s < kPeers; ++s) {
                        const uint32_t w = e < 2 ? pf.v[s][i][j][grp].x : pf.v[s][i][j][grp].y;
                        acc += bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu));
                    }
                    const int k = grp * 4 + e;
                    const float local = bf16_bits_to_f32(pack_bf16x2(st.acc[i][j][k], 0.0f) & 0xFFFFu);
                    os.acc[i][j][k] = acc + local;
                }
}

// The epilogue's sum stores: the rounded sums into `out` and, in an all-reduce
// run, into the gather buffers (each through the tile store's LDS staging).
template <class C>
__device__ __forceinline__ void epi_store(const Args& a, const TileState<C>& os, char* area, int srow0, int rows,
                                          int n0, int cols)
{
    store_tile<C>(a, os, area, __builtin_amdgcn_make_buffer_rsrc(a.out, 0, a.slice_bytes, kRsrcFlags), srow0, rows,
                  n0, cols);
    if (a.gather_on) {
#pragma unroll 1
        for (int g = 0; g < kPeers; ++g)
            store_tile<C>(a, os, area,
                          __builtin_amdgcn_make_buffer_rsrc(pick7(a.gather, g), 0, a.slice_bytes, kRsrcFlags),
                          srow0, rows, n0, cols);
    }
}

// ---------------------------------------------------------------- tile loop

// Per-tile state shared by the K loop and the role loop.
struct StepHooks {
    bool interleave; // engine waves run the reduce engine between MFMAs
    int eng_countdown;  // K steps to the next engine slot
    bool stores;     // the previous tile's epilogue stores are still in flight
    int pend_q;      // slot of the previous tile, whose flag is still to be stored
    int pend_flag;
    uint32_t who, epoch;
};

// Stage wait of a loader wave: B = (NS-2)*LPS younger direct loads may stay in
// flight, plus the previous tile's C::STORES epilogue stores while they are
// younger than the stage waited for (steps before NS-1).
template <class C>
__device__ __forceinline__ void wait_stage(bool stores)
{
    constexpr int B = (C::NS - 2) * C::LPS;
    if (stores)
        wait_vmcnt<B + C::STORES>();
    else
        wait_vmcnt<B>();
}

// The K loop of one tile is split in two so that the next tile's first stages
// can be issued before the current tile's epilogue stores (see compute_waves).
// Stage kt lives in buffer kt % NS and NS-1 stages are always in flight
// (stages past the end load zeros), so every step of a loader wave waits for
// the same count; the barrier then certifies that every loader's loads of stage
// kt have landed and that every wave has finished reading stage kt-1, whose
// buffer the step refills.  Engine waves issue no stage loads: their waits
// cover only their own epilogue stores (before a flag is published) and their
// engine operations (inside engine_step).
template <class C>
struct TileJob {
    LoadPlan<C> lp;
    int nk;
    const void* xp;    // the buffer the tile's X rows come from, and its bytes
    uint32_t xbytes;
};

// X rows come from `xp` (xbytes long, row0 counted in it); by default from a.x.
template <class C, bool LOADER>
__device__ __forceinline__ void tile_prologue(const Args& a, char* lds, TileJob<C>& job, int row0, int rows,
                                              int n0, int cols, const void* xp = nullptr, uint32_t xbytes = 0)
{
    const int K = a.g.K;
    job.nk = (K + C::BK - 1) / C::BK;
    job.xp = xp ? xp : (const void*)a.x;
    job.xbytes = xp ? xbytes : a.x_bytes;
    if constexpr (LOADER) {
        if (job.nk == 0) return;
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)uni_ptr(job.xp), 0, (uint32_t)uni((int)job.xbytes), kRsrcFlags);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.w, 0, a.w_bytes, kRsrcFlags);
        make_plan<C>(a, job.lp, row0, rows, n0, cols);
#pragma unroll
        for (int s = 0; s < C::NS - 1; ++s) issue_stage<C>(job.lp, rx, rw, lds + s * C::STAGE_BYTES, s * C::BK, K);
    }
}

// Wait until this wave's epilogue stores have completed.
template <bool LOADER>
__device__ __forceinline__ void wait_own_stores(const Engine& eng)
{
    if constexpr (LOADER)
        wait_vmcnt<0>();
    else
        wait_vmcnt_upto(eng.vm - eng.vm_stores);
}

// Runs the K loop of a tile whose prologue has been issued.  The previous
// tile's epilogue stores were issued after this tile's prologue and before the
// first refill, so they have completed once the refill issued at step 0 has:
// at step NS-1 (or after the loop) its flag is published.
template <class C, bool LOADER, bool ROWS = false>
__device__ __forceinline__ void tile_kloop(const Args& a, char* lds, TileState<C>& st, const TileJob<C>& job,
                                           StepHooks& hk, Engine& eng)
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int e = 0; e < AccT<C::MF>::N; ++e) st.acc[i][j][e] = 0.0f;

    const int K = a.g.K;
    const int nk = job.nk;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)uni_ptr(job.xp), 0, (uint32_t)uni((int)job.xbytes), kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.w, 0, a.w_bytes, kRsrcFlags);
    for (int kt = 0; kt < nk; ++kt) {
        if constexpr (LOADER)
            wait_stage<C>(hk.stores && kt < C::NS - 1);
        else if (hk.stores && kt == C::NS - 1)
            wait_own_stores<false>(eng);
        stage_barrier();
        if (kt == C::NS - 1) {
            hk.stores = false;
            if (hk.pend_flag >= 0) {
                if (threadIdx.x == 0) publish<ROWS>(a, hk.pend_q, hk.pend_flag, hk.who, hk.epoch);
                hk.pend_flag = -1;
            }
        }
        if constexpr (!LOADER) {
            if (hk.interleave && --hk.eng_countdown == 0) {
                hk.eng_countdown = a.engine_every;
                engine_step(eng, a, true);
            }
        }
        const int nxt = kt + C::NS - 1;
        kstep<C, LOADER>(job.lp, rx, rw, lds + (nxt % C::NS) * C::STAGE_BYTES, nxt * C::BK, K,
                         lds + (kt % C::NS) * C::STAGE_BYTES, st);
    }
    // loaders drain the zero-filling loads past the end; every wave finishes
    // reading LDS before the next tile's loads overwrite it; a flag still
    // pending (nk < NS) is published here
    if constexpr (LOADER)
        wait_vmcnt<0>();
    else if (hk.stores)
        wait_own_stores<false>(eng);
    stage_barrier();
    hk.stores = false;
    if (hk.pend_flag >= 0) {
        if (threadIdx.x == 0) publish<ROWS>(a, hk.pend_q, hk.pend_flag, hk.who, hk.epoch);
        hk.pend_flag = -1;
    }
}

// Wait until this wave's LDS reads (and other LGKM operations) have completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4)); }

// Publishes the previous tile's flag once a barrier has certified its stores.
template <bool ROWS = false>
__device__ __forceinline__ void publish_pending(const Args& a, StepHooks& hk)
{
    hk.stores = false;
    if (hk.pend_flag >= 0) {
        if (threadIdx.x == 0) publish<ROWS>(a, hk.pend_q, hk.pend_flag, hk.who, hk.epoch);
        hk.pend_flag = -1;
    }
}

// The K loop of a tile for kernels with one workgroup per CU (every wave
// loads), pipelined across K steps: substep 0 of step kt+1 is read while the
// last substep of step kt computes, so no wave starts a step with an LDS round
// trip (with one wave per SIMD no sibling covers it; with two, both waves of a
// SIMD leave the same barrier together).  The step's wait and barrier therefore sit
// before its last substep: they certify that every wave's loads of stage kt+1
// have landed and that every wave has read all of stage kt (each wave waits for
// its LDS reads first), whose buffer is refilled right after the barrier with
// stage kt+NS.  The vector-memory wait counts follow tile_kloop: NS-2 younger
// stages, plus the previous tile's stores while they are younger than the
// stage waited for (stages of the prologue).  The first barrier that covers
// those stores (the one waiting for stage NS-1, the first refill) publishes
// the previous tile's flag.
//
// With STREAM every step also runs one step of the reduce stream after its
// refill (and its sched barriers keep those instructions younger than every
// load of the refill), so a step's wait allows as many more outstanding
// instructions as the previous step's stream issued.
template <class C, bool STREAM, bool ROWS = false>
__device__ __forceinline__ void tile_kloop_xp(const Args& a, char* lds, TileState<C>& st, const TileJob<C>& job,
                                              StepHooks& hk, Stream& rs)
{
    static_assert(C::KSUB % 2 == 0, "substep s of every step uses fragment buffer s % 2");
    static_assert(C::EW == 0, "every wave loads stages");
    static_assert(!STREAM || C::NS == 2, "the reduce stream's wait counts assume two stages");
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int e = 0; e < AccT<C::MF>::N; ++e) st.acc[i][j][e] = 0.0f;

    const int K = a.g.K;
    const int nk = job.nk;
    constexpr int B = (C::NS - 2) * C::LPS;
    constexpr int kMf = C::FM * C::FN;   // MFMAs per substep
    constexpr int kDs = C::FM + C::FN;   // fragment reads per substep
    if (nk > 0) {
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)uni_ptr(job.xp), 0, (uint32_t)uni((int)job.xbytes), kRsrcFlags);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.w, 0, a.w_bytes, kRsrcFlags);
        bf16x8 xf[2][C::FM], wf[2][C::FN];
        // stage 0 came from the prologue, before the previous tile's stores
        if (hk.stores)
            wait_vmcnt<B + C::STORES>();
        else
            wait_vmcnt<B>();
        stage_barrier();
        issue_stage<C>(job.lp, rx, rw, lds + (C::NS - 1) * C::STAGE_BYTES, (C::NS - 1) * C::BK, K);
        load_frags<C>(lds, 0, xf[0], wf[0]);
        for (int kt = 0; kt + 1 < nk; ++kt) {
            const char* cur = lds + (kt % C::NS) * C::STAGE_BYTES;
#pragma unroll
            for (int s = 0; s + 1 < C::KSUB; ++s) {
                load_frags<C>(cur, s + 1, xf[(s + 1) & 1], wf[(s + 1) & 1]);
                mfma_substep<C>(st, xf[s & 1], wf[s & 1]);
            }
#pragma unroll
            for (int s = 0; s + 1 < C::KSUB; ++s)
#pragma unroll
                for (int m = 0; m < kMf; ++m) {
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    if (m < kDs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
                }
            if constexpr (STREAM) {
                // (the previous step's stream instructions may stay in flight)
                stream_wait<B>(rs);
            } else if (hk.stores && kt + 1 < C::NS - 1) {
                wait_vmcnt<B + C::STORES>();
            } else {
                wait_vmcnt<B>();
            }
            wait_lgkm0();
            stage_barrier();
            if (kt + 1 == C::NS - 1) publish_pending<ROWS>(a, hk);
            // raised issue priority from the barrier to the end of the step,
            // while the wave issues the refill (measured: ~1% faster than
            // without, and than raising it over the MFMA-only part)
            __builtin_amdgcn_s_setprio(1);
            issue_stage<C>(job.lp, rx, rw, lds + (kt % C::NS) * C::STAGE_BYTES, (kt + C::NS) * C::BK, K);
            load_frags<C>(lds + ((kt + 1) % C::NS) * C::STAGE_BYTES, 0, xf[0], wf[0]);
            mfma_substep<C>(st, xf[(C::KSUB - 1) & 1], wf[(C::KSUB - 1) & 1]);
            // the refill's loads one per MFMA (any excess first), then the
            // next step's first fragments
            if constexpr (C::LPS > kMf) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, C::LPS - kMf, 0);
#pragma unroll
            for (int m = 0; m < kMf; ++m) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                if (m < C::LPS) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
                if (m < kDs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
            __builtin_amdgcn_s_setprio(0);
            if constexpr (STREAM) stream_step(rs, a);
        }
        // the last step
        const char* cur = lds + ((nk - 1) % C::NS) * C::STAGE_BYTES;
#pragma unroll
        for (int s = 0; s < C::KSUB; ++s) {
            if (s + 1 < C::KSUB) load_frags<C>(cur, s + 1, xf[(s + 1) & 1], wf[(s + 1) & 1]);
            mfma_substep<C>(st, xf[s & 1], wf[s & 1]);
        }
    }
    // the zero-filling loads past the end drain; every wave finishes reading
    // LDS before the next tile's loads overwrite it; a flag still pending
    // (nk < NS) is published here
    wait_vmcnt<0>();
    stage_barrier();
    if constexpr (STREAM) stream_settle(rs);
    publish_pending<ROWS>(a, hk);
}

// Every group holds G/8 workgroups; group x has R_x = R/8 + (x < R%8) reducers
// and C_x = G/8 - R_x compute workgroups, so the groups' compute counts add up
// to C = G - R whatever R is.
struct GroupSplit {
    int compute, reducers, base;  // base: first position of the group in a round
    int rbase;                    // index of the group's first reducer among all R
};

__device__ __forceinline__ GroupSplit group_split(int grid, int reducers, int grp)
{
    const int gq = grid / kGroups;
    const int rq = reducers / kGroups, rr = reducers % kGroups;
    GroupSplit s;
    s.reducers = rq + (grp < rr ? 1 : 0);
    s.compute = gq - s.reducers;
    s.base = grp * (gq - rq) - (grp < rr ? grp : rr);
    s.rbase = grp * rq + (grp < rr ? grp : rr);
    return s;
}

// The tile loop of one wave of a compute workgroup at position `pos` of a
// round.  Round r covers slots [r*C, r*C + C).  A tile's flag is stored once
// the next tile's waits have covered the tile's stores: publishing costs no
// extra wait.  Loader and engine waves run the same loop (the same barriers);
// engine waves also run the reduce engine.
template <class C, bool FUSED, bool LOADER, bool STREAM, bool EPI = false, int VAR = 0>
__device__ __forceinline__ void compute_waves(const Args& a, char* lds, int pos, uint32_t who, uint32_t epoch,
                                              bool interleave)
{
    static_assert(!EPI || (FUSED && C::WAVES == 4 && C::EW == 0), "the epilogue sum: four-wave fused tiles");
    const int Ctot = a.num_compute;
    const int wave = uni((int)(threadIdx.x >> 6));
    Engine eng;
    Stream rs;
    if constexpr (STREAM) {
        constexpr int SW = C::WAVES / kStreamOps;  // streaming waves
        stream_init(rs, a, lds + C::LDS_BYTES + (wave % SW) * kStreamLds, pos * SW, pos * SW + wave % SW,
                    Ctot * SW, wave < SW, epoch);
    }
    if constexpr (!LOADER) {
        const int ew = wave - C::LW;
        engine_init(eng, a, lds + C::LDS_BYTES + ew * kEngAreas * kEngAreaBytes, pos * C::EW + ew, Ctot * C::EW,
                    epoch);
    }
    StepHooks hk;
    hk.interleave = interleave && C::EW > 0 && a.engine_every > 0;
    hk.eng_countdown = 1;
    hk.stores = false;
    hk.pend_q = -1;
    hk.pend_flag = -1;
    hk.who = who;
    hk.epoch = epoch;
    TileState<C> st;
    TileJob<C> job;
    PeerFrag<C> pf;
    int q = pos;
    TileCoord t;
    if (q < a.g.tiles) {
        t = decode_slot(a.g, q);
        // (the peer values load ahead of the first stage, which waits for them)
        if constexpr (EPI)
            if (t.d == a.g.rank)
                epi_load_peers<C>(a, pf, t.tml * C::BM, tile_rows(a.g, t), t.tn * C::BN, tile_cols(a.g, t));
        tile_prologue<C, LOADER>(a, lds, job, tile_row0(a.g, t), tile_rows(a.g, t), t.tn * C::BN,
                                 tile_cols(a.g, t));
    }
    while (q < a.g.tiles) {
        if constexpr (C::XP)
            tile_kloop_xp<C, STREAM, (VAR & kVarRows) != 0>(a, lds, st, job, hk, rs);
        else
            tile_kloop<C, LOADER, (VAR & kVarRows) != 0>(a, lds, st, job, hk, eng);
        // issue the next tile's first stages before this tile's stores
        const int qn = q + Ctot;
        TileCoord tn = t;
        if (qn < a.g.tiles) {
            tn = decode_slot(a.g, qn);
            tile_prologue<C, LOADER>(a, lds, job, tile_row0(a.g, tn), tile_rows(a.g, tn), tn.tn * C::BN,
                                     tile_cols(a.g, tn));
        }
        // the stage buffer the next tile's prologue left free holds the
        // epilogue staging areas
        const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(a.dst[t.d], 0, a.slice_bytes, kRsrcFlags);
        store_tile<C, (VAR & kVarNt) ? kStoreDeviceNt : kStoreDevice>(
            a, st, lds + (C::NS - 1) * C::STAGE_BYTES, rd, t.tml * C::BM, tile_rows(a.g, t), t.tn * C::BN,
            tile_cols(a.g, t));
        if constexpr (EPI) {
            if (t.d == a.g.rank) {
                TileState<C> os;
                epi_sum<C>(pf, st, os);
                epi_store<C>(a, os, lds + (C::NS - 1) * C::STAGE_BYTES, t.tml * C::BM, tile_rows(a.g, t),
                             t.tn * C::BN, tile_cols(a.g, t));
            }
            // a later own tile's peer values load behind these stores (its
            // stage waits then cover them)
            if (qn < a.g.tiles && tn.d == a.g.rank)
                epi_load_peers<C>(a, pf, tn.tml * C::BM, tile_rows(a.g, tn), tn.tn * C::BN, tile_cols(a.g, tn));
        }
        hk.stores = true;
        if constexpr (!LOADER) {
            eng.vm += C::STORES;
            eng.vm_stores = eng.vm;
        }
        if (FUSED) {
            hk.pend_q = q;
            hk.pend_flag = t.flag;
        }
        q = qn;
        t = tn;
    }
    if (hk.pend_flag >= 0) {
        wait_own_stores<LOADER>(eng);
        stage_barrier();
        if (threadIdx.x == 0) publish<(VAR & kVarRows) != 0>(a, hk.pend_q, hk.pend_flag, who, epoch);
    }
    if constexpr (EPI) {
        // every own tile was summed by its producer
    } else if constexpr (STREAM) {
        // the items the stream has not finished
        __shared__ int s_progress[C::WAVES / kStreamOps];
        stream_drain<C::WAVES>(rs, a, wave, s_progress);
    } else if (interleave) {
        if (hk.interleave) {
            // in-loop slots: the engine waves own the items
            if constexpr (!LOADER) engine_drain(eng, a);
        } else {
            // every wave sums a share of the slice after its last tile
            const int wave = uni((int)(threadIdx.x >> 6));
            // (sixteen items in flight per CU for the eight-wave and one-per-CU
            // tiles; one per wave for four-wave tiles at two per CU, whose
            // shapes leave about one item per wave: a second, empty slot of a
            // batch still issues its eight loads and lengthens the wait)
            drain_items<(C::WAVES == 4 && C::LDS_BYTES <= 80 * 1024 - 64) ? 1 : 16 / C::WAVES, 2,
                        (VAR & kVarRows) != 0>(a, item_map(a), pos * C::WAVES + wave, a.num_compute * C::WAVES,
                                               epoch);
        }
    }
}

// Compute role of the l-th compute workgroup of group grp: its position in a
// round is either the group's block offset + l (contiguous split) or
// l * 8 + grp (strided, used when all C_x are equal).
template <class C, bool FUSED, bool STREAM, bool EPI = false, int VAR = 0>
__device__ __forceinline__ void compute_role(const Args& a, char* lds, int grp, int l, uint32_t epoch, int base)
{
    const int pos = uni(a.strided ? (l * kGroups + grp) : (base + l));
    const uint32_t who = ((uint32_t)grp << 16) | (uint32_t)l;
    // without dedicated reducers the compute workgroups reduce the slice
    const bool interleave = FUSED && a.num_reducers == 0;
    const int wave = uni((int)(threadIdx.x >> 6));
    if (C::EW == 0 || wave < C::LW)
        compute_waves<C, FUSED, true, STREAM, EPI, VAR>(a, lds, pos, who, epoch, interleave);
    else if constexpr (C::EW > 0)
        compute_waves<C, FUSED, false, false, false, VAR>(a, lds, pos, who, epoch, interleave);
}

// Dedicated reducer role (used when reducers are requested): claim own-slice
// tiles in schedule order, wait for each tile's flag (thread 0 polls with
// device-scope loads and short sleeps, bounded by the watchdog), then sum the
// tile, reading the local slice at device scope.
template <bool ROWS>
__device__ void reducer_role(const Args& a, uint32_t epoch)
{
    __shared__ int s_unit;
    __shared__ int s_abort;
    for (;;) {
        if (threadIdx.x == 0) {
            const int u = (int)atomicAdd(&a.state->unit, 1u);
            int abort_now = 0;
            if (u < a.g.ts) {
                const TileCoord t = decode_slot(a.g, u);
                const uint32_t* f = ready_word<ROWS>(a, t.flag);
                if (!released<ROWS>(a, __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), epoch)) {
                    const uint64_t t0 = wall_clock64();
                    while (!released<ROWS>(a, __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), epoch)) {
                        __builtin_amdgcn_s_sleep(2);
                        if ((int64_t)(wall_clock64() - t0) > a.watchdog_ticks) {
                            abort_now = 1;
                            break;
                        }
                    }
                }
                if (abort_now && atomicCAS(&a.state->status[0], 0, kStatusTimeout) == 0)
                    atomicExch(&a.state->status[1], t.flag);
            }
            s_unit = u;
            s_abort = abort_now;
        }
        __syncthreads();
        const int u = s_unit;
        const int abort_now = s_abort;
        __syncthreads();  // s_unit / s_abort are rewritten by the next claim
        if (u >= a.g.ts) return;
        if (abort_now) continue;
        const TileCoord t = decode_slot(a.g, u);
        const int rows = tile_rows(a.g, t), cols = tile_cols(a.g, t);
        const int cpr = cols >> 3;
        const uint16_t* local = a.dst[a.g.rank];
        for (int c = threadIdx.x; c < rows * cpr; c += (int)blockDim.x) {
            const int r = c / cpr;
            const int64_t off = (int64_t)(t.tml * a.g.bm + r) * a.g.N + t.tn * a.g.bn + (c - r * cpr) * 8;
            u32x4 v[kPeers + 1];
#pragma unroll
            for (int s = 0; s < kPeers; ++s)
                v[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.peers[s] + off));
            // the local slice at device scope (two 8-byte relaxed agent-scope loads)
            const uint64_t* lp = reinterpret_cast<const uint64_t*>(local + off);
            const uint64_t l0 = __hip_atomic_load(lp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t l1 = __hip_atomic_load(lp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v[kPeers] = u32x4{(uint32_t)l0, (uint32_t)(l0 >> 32), (uint32_t)l1, (uint32_t)(l1 >> 32)};
            f32x8 acc = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s <= kPeers; ++s) acc = add8(acc, v[s]);
            const u32x4 o = pack8(acc);
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(a.out + off));
            if (a.gather_on) {
#pragma unroll
                for (int i = 0; i < kPeers; ++i) __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(a.gather[i] + off));
            }
        }
    }
}

// Role dispatch and end-of-launch bookkeeping, with no device atomics on the
// default path.  Without dedicated reducers every workgroup computes and its
// position follows from its index.  With reducers, per-group arrival tickets
// hand out the roles (a reducer exists only once its group's compute
// workgroups are all resident), and workgroup 0 resets the tickets once every
// workgroup has finished.
//
// The run epoch: each workgroup keeps, in its own word of `finished`, the
// epoch of the last fused launch it finished.  A launch reads that word at
// the start and uses the next value; every workgroup of the previous fused
// launch stored the same value, so all workgroups of a launch agree on its
// epoch without communicating (the words change only at kernel ends).  A
// GEMM-only launch has no flags and touches none of this.
template <class C, bool FUSED, bool STREAM = false, bool EPI = false, int VAR = 0>
__device__ __forceinline__ void fused_body(const Args& a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ uint32_t s_ticket, s_epoch;
    const int grp = blockIdx.x % kGroups;
    // co-resident reducers take their role from their index (the whole grid
    // fits on the device at once, and compute workgroups never wait for
    // reducers), so they need no tickets
    const bool tickets = FUSED && a.num_reducers > 0 && !a.coresident;
    if (threadIdx.x == 0) {
        s_ticket = tickets ? atomicAdd(&a.state->role[grp], 1u) : (uint32_t)(blockIdx.x / kGroups);
        s_epoch = FUSED ? __hip_atomic_load(a.finished + blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : 0u;
    }
    __syncthreads();
    // (read through readfirstlane so that the compiler sees them uniform: the
    // tile loop and the reduce stream then stay in scalar registers)
    const uint32_t ticket = (uint32_t)uni((int)s_ticket);
    const uint32_t epoch = (uint32_t)uni((int)s_epoch) + 1u;  // value this run's flags carry
    const GroupSplit split = group_split((int)gridDim.x, uni(a.num_reducers), grp);
    if (ticket < (uint32_t)split.compute)
        compute_role<C, FUSED, STREAM, EPI, VAR>(a, lds, grp, (int)ticket, epoch, split.base);
    else if (FUSED && ticket - (uint32_t)split.compute < (uint32_t)split.reducers) {
        if (a.coresident) {
            // reducer r of R owns items r*W + wave, + R*W, ...: its peer chunks
            // are loaded and summed while the GEMM runs, before the flags are
            // checked; once a tile is flagged only its local chunks remain
            const int r = split.rbase + (int)(ticket - (uint32_t)split.compute);
            const int wave = uni((int)(threadIdx.x >> 6));
            drain_items<2, 1, (VAR & kVarRows) != 0>(a, item_map(a), r * C::WAVES + wave,
                                                     uni(a.num_reducers) * C::WAVES, epoch);
        } else {
            reducer_role<(VAR & kVarRows) != 0>(a, epoch);
        }
    }

    if constexpr (FUSED) {
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_store(a.finished + blockIdx.x, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tickets && blockIdx.x == 0) {
            // every finish mark arrives (each workgroup's own waits are
            // bounded by the watchdog; this one is bounded too)
            const uint64_t t0 = wall_clock64();
            for (int i = threadIdx.x; i < (int)gridDim.x; i += blockDim.x)
                while (__hip_atomic_load(a.finished + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch &&
                       (int64_t)(wall_clock64() - t0) <= 2 * a.watchdog_ticks)
                    __builtin_amdgcn_s_sleep(2);
            __syncthreads();
            if (threadIdx.x == 0) {
                for (int i = 0; i < kGroups; ++i)
                    __hip_atomic_store(&a.state->role[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&a.state->unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// Tiles that fit two workgroups per CU keep two waves per SIMD resident.
template <class C, bool FUSED, bool EPI = false, int VAR = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fused_kernel(Args a)
{
    fused_body<C, FUSED, false, EPI, VAR>(a);
}

// Eight-wave workgroups (one per CU): two waves per SIMD, so one wave's
// MFMAs run while its sibling waits on LDS, a barrier or the reduce engine.
template <class C, bool FUSED, bool STREAM = false, int VAR = 0>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fused_kernel_8w(Args a)
{
    fused_body<C, FUSED, STREAM, false, VAR>(a);
}

// Large tiles run one workgroup (one wave per SIMD) per CU: let the compiler
// use the whole register file for latency hiding.
template <class C, bool FUSED, int VAR = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fused_kernel_1w(Args a)
{
    fused_body<C, FUSED, false, false, VAR>(a);
}

// Standalone slice sum: every workgroup reduces, no flags, grid-stride over the
// whole [S][N] slice.
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(Args a)
{
    sum_block(a, 0, a.g.S, 0, a.g.N, blockIdx.x * kReduceThreads + threadIdx.x, gridDim.x * kReduceThreads);
}

// ---------------------------------------------------------------- all-gather + GEMM
//
// The column-parallel linear layer that precedes the row-parallel one, with
// the all-gather fused as the GEMM's prologue (TL;DR of "FLUX: Fast
// Software-based Communication Overlap On GPUs Through Kernel Fusion";
// "mKernel: Fast Multi-GPU, Multi-Node Fused Kernels", Section 4: the local
// shard's tiles first, the others as their rows arrive).  Rank r holds its
// activation row slice; the other tp-1 slices arrive from the peers.  On one
// GPU they are resident buffers, and the copy phase below stands in for the
// peers' writes into this rank's gathered buffer: every workgroup first
// copies its share of copy units (in the order the tiles need them: slice
// r+1 first, this rank's own slice last), each unit followed by one
// device-scope increment of its tile-row block's counter.  The GEMM then runs
// the reduce-scatter's tile schedule (own slice first, then rotated by rank):
// an own tile reads the local slice directly; any other tile waits until its
// block's counter reaches runs * units (counters are never reset, so a launch
// can be replayed from a graph), then reads the gathered buffer.  Lines of the
// gathered buffer left in an XCD's L2 by an earlier run would be stale, so
// every workgroup invalidates its caches once at its start (agent-scope
// acquire), before anything of this run is cached; later lines of the buffer
// can only come from reads made after their rows were copied.  Output tiles
// go to y [M][N]; there is no reduction.

// Copies units first, first + stride, ... (all threads of the workgroup).
template <class C>
__device__ __forceinline__ void ag_copy(const Args& a, int first, int stride)
{
    const int tp = a.g.tp, r = a.g.rank, S = a.g.S, K = a.g.K, tms = a.g.tms;
    const int U = a.ag_units;
    const uint32_t UB = a.ag_unit_bytes;
    const int nunits = tp * tms * U;
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void*)a.xg, 0, a.x_bytes, kRsrcFlags);
    const uint32_t tid16 = threadIdx.x * 16u;
    constexpr uint32_t kPass = (uint32_t)C::THREADS * 16u;
    for (int gu = first; gu < nunits; gu += stride) {
        const int blk = gu / U, u = gu - blk * U;
        const int k = blk / tms, tml = blk - k * tms;
        const int d = uni((r + 1 + k) % tp);  // this rank's own slice last
        const int rows = min(C::BM, S - tml * C::BM);
        const uint32_t blk_bytes = (uint32_t)rows * (uint32_t)K * 2u;
        const uint32_t src0 = (uint32_t)(tml * C::BM) * (uint32_t)K * 2u;
        const uint32_t dst0 = (uint32_t)(d * S + tml * C::BM) * (uint32_t)K * 2u;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)a.xsrc[d], 0, a.xs_bytes, kRsrcFlags);
        const uint32_t u0 = (uint32_t)u * UB;
        const uint32_t u1 = min(u0 + UB, blk_bytes);
        // (eight 16-byte loads in flight per thread: a workgroup's copy is
        // bound by how much it has in flight)
        for (uint32_t o = u0 + tid16; o < u1; o += 8 * kPass) {
            u32x4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t oi = o + (uint32_t)i * kPass;
                v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, oi < u1 ? src0 + oi : kOob, 0, kAuxNt));
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t oi = o + (uint32_t)i * kPass;
                __builtin_amdgcn_raw_buffer_store_b128(v[i], rd, oi < u1 ? dst0 + oi : kOob, 0, kStoreDevice);
            }
        }
        // every wave's stores of the unit have completed (device scope, written
        // through to the memory side) before the block's counter moves
        wait_vmcnt<0>();
        __syncthreads();
        if (threadIdx.x == 0 && d != r)
            __hip_atomic_fetch_add(a.agflags + d * tms + tml, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Waits (device-scope polls) until block `blk`'s counter reaches `target`;
// reports a timeout through the status word and returns false.
__device__ __forceinline__ bool ag_wait(const Args& a, int blk, uint32_t target)
{
    const uint32_t* f = a.agflags + blk;
    if ((int32_t)(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - target) >= 0) return true;
    const uint64_t t0 = wall_clock64();
    while ((int32_t)(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - target) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if ((int64_t)(wall_clock64() - t0) > a.watchdog_ticks) {
            if ((threadIdx.x & 63) == 0 && atomicCAS(&a.state->status[0], 0, kStatusTimeout) == 0)
                atomicExch(&a.state->status[1], blk);
            return false;
        }
    }
    return true;
}

// Issues the first stages of tile t: X rows from the local slice (own tile)
// or from the gathered buffer once the block has arrived (FUSED) or because
// the buffer is already complete (GEMM only).
template <class C, bool FUSED>
__device__ __forceinline__ void ag_prologue(const Args& a, char* lds, TileJob<C>& job, const TileCoord& t,
                                            uint32_t target)
{
    const int rows = tile_rows(a.g, t), cols = tile_cols(a.g, t);
    if (t.d == a.g.rank) {
        tile_prologue<C, true>(a, lds, job, t.tml * C::BM, rows, t.tn * C::BN, cols, a.xsrc[a.g.rank], a.xs_bytes);
        return;
    }
    if constexpr (FUSED) ag_wait(a, t.d * a.g.tms + t.tml, target);
    tile_prologue<C, true>(a, lds, job, t.d * a.g.S + t.tml * C::BM, rows, t.tn * C::BN, cols, a.xg, a.x_bytes);
}

template <class C, bool FUSED>
__device__ __forceinline__ void ag_body(const Args& a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ uint32_t s_runs;
    if (threadIdx.x < 64) {
        // drop lines an earlier run left in this CU's L1 and this XCD's L2
        if constexpr (FUSED) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (threadIdx.x == 0)
            s_runs = FUSED ? __hip_atomic_load(a.agfinished + blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0u;
    }
    __syncthreads();
    const uint32_t run = (uint32_t)uni((int)s_runs) + 1u;  // this launch's count
    const int grp = blockIdx.x % kGroups;
    const int l = blockIdx.x / kGroups;
    const int G = (int)gridDim.x;
    const int pos = uni(a.strided ? (l * kGroups + grp) : (grp * (G / kGroups) + l));
    // copy units go to the workgroups from the last position down: those
    // hold the fewest tiles (a round's last positions), or none
    if constexpr (FUSED) ag_copy<C>(a, G - 1 - pos, G);
    const uint32_t target = run * (uint32_t)a.ag_units;

    StepHooks hk;
    hk.interleave = false;
    hk.eng_countdown = 1;
    hk.stores = false;
    hk.pend_q = -1;
    hk.pend_flag = -1;
    hk.who = 0;
    hk.epoch = run;
    Engine eng;
    Stream rs;
    TileState<C> st;
    TileJob<C> job;
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc((void*)a.y, 0, a.y_bytes, kRsrcFlags);
    int q = pos;
    TileCoord t;
    if (q < a.g.tiles) {
        t = decode_slot(a.g, q);
        ag_prologue<C, FUSED>(a, lds, job, t, target);
    }
    while (q < a.g.tiles) {
        if constexpr (C::XP)
            tile_kloop_xp<C, false>(a, lds, st, job, hk, rs);
        else
            tile_kloop<C, true>(a, lds, st, job, hk, eng);
        const int qn = q + G;
        TileCoord tn = t;
        if (qn < a.g.tiles) {
            tn = decode_slot(a.g, qn);
            ag_prologue<C, FUSED>(a, lds, job, tn, target);
        }
        store_tile<C>(a, st, lds + (C::NS - 1) * C::STAGE_BYTES, ry, t.d * a.g.S + t.tml * C::BM, tile_rows(a.g, t),
                      t.tn * C::BN, tile_cols(a.g, t));
        hk.stores = true;
        q = qn;
        t = tn;
    }
    if constexpr (FUSED) {
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_store(a.agfinished + blockIdx.x, run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <class C, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void ag_kernel(Args a)
{
    ag_body<C, FUSED>(a);
}

template <class C, bool FUSED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void ag_kernel_8w(Args a)
{
    ag_body<C, FUSED>(a);
}

template <class C, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void ag_kernel_1w(Args a)
{
    ag_body<C, FUSED>(a);
}

// Standalone all-gather: copies the tp slices into the gathered buffer,
// grid-stride over 16-byte chunks of each slice in turn (no counters).
__global__ __launch_bounds__(kReduceThreads) void ag_copy_kernel(Args a)
{
    const int64_t chunks = (int64_t)a.g.S * a.g.K / 8;  // per slice
    for (int d = 0; d < a.g.tp; ++d) {
        const uint16_t* src = a.xsrc[d];
        uint16_t* dst = a.xg + (int64_t)d * a.g.S * a.g.K;
        for (int64_t c = blockIdx.x * (int64_t)kReduceThreads + threadIdx.x; c < chunks;
             c += (int64_t)gridDim.x * kReduceThreads)
            *reinterpret_cast<uint4*>(dst + c * 8) = *reinterpret_cast<const uint4*>(src + c * 8);
    }
}

}  // namespace gemm_rs
