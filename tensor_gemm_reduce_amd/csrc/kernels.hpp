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
// By default the compute workgroups themselves sum the slice after their last
// tile; dedicated reducer workgroups (arrival tickets) and co-resident reducer
// workgroups (one more per CU, role by index) are the other placements.
//
// Workgroup g belongs to group g % 8, which is the XCD it runs on (workgroups
// are dispatched to the 8 XCDs round-robin).  With dedicated reducers each
// group hands out its own arrival tickets: the first C_x arrivals of group x
// compute, the next R_x reduce.  A reducer therefore exists only after every
// compute workgroup of its group is resident, and compute workgroups never
// wait, so reducers cannot starve their producers.  Compute slots are split so
// that the workgroups of one XCD work on tiles that share rows of X or columns
// of W in that XCD's L2.
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
// Cache-policy bits of the slice sum's loads and stores: peer partials are
// read once and sums written once (non-temporal); the local slice and the
// flags are read at device scope (sc1), so a copy left in this XCD's L2 by an
// earlier run is never used.
constexpr int kAuxNt = 2;
constexpr int kAuxSc1 = 16;
// Routed tile stores with the non-temporal hint on top of device scope: the
// tile is not read back through this XCD's L2 (the sum reads the local slice
// at device scope, the send buffers leave the GPU), so it need not displace
// the GEMM's operands there.
constexpr int kStoreDeviceNt = kStoreDevice | kAuxNt;

// Kernel variants (a template parameter of the fused and GEMM kernels, so that
// the default kernel carries no code of the others): bit 0 stores routed tiles
// with kStoreDeviceNt, bit 1 reads row counters instead of tile flags, bit 2
// interleaves the slice sum with the tiles under the adaptive controller
// (sum_units).
constexpr int kVarNt = 1;
constexpr int kVarRows = 2;
constexpr int kVarDyn = 4;


// Handle-owned device state, zeroed at creation.  The arrival tickets and the
// reducer claim counter exist twice: run e uses set e & 1 and clears set
// (e + 1) & 1 for the next run, which no workgroup of run e touches (runs of
// one handle do not overlap), so no counter is ever reset while a run may
// still use it.
struct DeviceState {
    uint32_t role[2][kGroups];  // per-group arrival tickets (dedicated reducers only)
    uint32_t unit[2];           // next reducer unit to claim
    int32_t status[2];          // [0] error code, [1] flag index that timed out
    uint32_t pad[12];
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
    int32_t* status;         // [0] error code, [1] flag index that timed out
    uint32_t* trace;         // 4 words per slot (debug)
    uint32_t* sum_trace;     // 4 words per own tile, then 4 for the launch (debug)
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
// issue the stage loads (LW = 0: all of them); the other EW waves issue none.
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
    // One workgroup per CU (four waves whose stages fit only once, or eight
    // waves) with every wave loading: the K loop is pipelined across steps.
    static constexpr bool XP = LDS_BYTES > 80 * 1024 - 64 && KSUB % 2 == 0;
    // Four waves (one per SIMD) with four substeps per stage of two: the
    // barrier follows a step's first substep and the refill spreads over the
    // other three (tile_kloop_long).
    static constexpr bool LT = XP && WAVES == 4 && KSUB == 4 && NS == 2;
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

// Per-thread load plan of one tile (loader threads).  Thread tid moves the
// chunks p = i * LTHREADS + tid (i = 0 .. LD-1) of each operand: tile row
// r_i = tid / CPR + i * LTHREADS / CPR and 16-byte column c = (tid % CPR) ^
// swz(r_i).  The swizzle depends on r mod 16 only and LTHREADS / CPR is a
// multiple of 16, so c is the same for every i, and the plan is one byte
// offset per operand (chunk i = 0 at k = 0) plus the chunk's k offset.  Rows
// past the tile's valid extent are loaded like the others: they are rows of
// the next slice or columns of the next tile, never stored, or lie past the
// end of the buffer and read as zero.
template <class C>
struct LoadPlan {
    uint32_t a_off, b_off;
    int kc;
};

template <class C>
__device__ __forceinline__ void make_plan(const Args& a, LoadPlan<C>& lp, int row0, int n0)
{
    static_assert((C::LTHREADS / C::CPR) % 16 == 0, "one swizzled column per thread");
    const int tid = threadIdx.x;
    const uint32_t K = (uint32_t)a.g.K;
    const int r = tid / C::CPR;
    const int c = (tid % C::CPR) ^ swz<C::CPR>(r);
    lp.kc = c * 8;
    lp.a_off = ((uint32_t)(row0 + r) * K + (uint32_t)c * 8u) * 2u;
    lp.b_off = ((uint32_t)(n0 + r) * K + (uint32_t)c * 8u) * 2u;
}

// Issue the LDS-direct loads of the BK slice starting at k0 into stage buffer
// `stage` (LPS loads per loader thread).  Each wave instruction fills 1 KiB of
// LDS: lane l writes bytes [16 l, 16 l + 16) after the wave's base.
//
// Branch-free: a chunk whose k lies at or past K (the K tail, or a whole stage
// past the end) gets an offset past the resource and reads as zero (kOob plus
// the rows of a tile stays past any resource of these kernels).
template <class C>
__device__ __forceinline__ void issue_stage(const LoadPlan<C>& lp, __amdgpu_buffer_rsrc_t rx,
                                            __amdgpu_buffer_rsrc_t rw, char* stage, int k0, int K)
{
    // (uniform: the LDS destination, and with it M0, is scalar arithmetic)
    const int wave = uni((int)(threadIdx.x >> 6));
    const bool in_k = lp.kc < K - k0;
    const uint32_t a0 = in_k ? lp.a_off + (uint32_t)k0 * 2u : kOob;
    const uint32_t b0 = in_k ? lp.b_off + (uint32_t)k0 * 2u : kOob;
    // bytes between the rows of chunks i and i + 1
    const uint32_t step = (uint32_t)uni((C::LTHREADS / C::CPR) * K * 2);
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (lds_void_t*)(stage + (i * C::LTHREADS + wave * 64) * 16), 16, a0 + (uint32_t)i * step, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (lds_void_t*)(stage + C::A_BYTES + (i * C::LTHREADS + wave * 64) * 16), 16, b0 + (uint32_t)i * step,
            0, 0, 0);
}

// The last substep of an XP step after its barrier, with the refill of the
// stage buffer just read and the next step's first fragments: MFMA m is
// followed by direct load m and fragment read m, in that order (scheduling
// fences hold it; left to the scheduler, the loads bunch together and the
// fragment reads come last).  The fragments are read in load_frags' order.
template <class C>
__device__ __forceinline__ void xp_tail(TileState<C>& st, const bf16x8 (&xl)[C::FM], const bf16x8 (&wl)[C::FN],
                                        bf16x8 (&xn)[C::FM], bf16x8 (&wn)[C::FN], const char* next,
                                        const LoadPlan<C>& lp, __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw,
                                        char* refill, int k0, int K)
{
    constexpr int kMf = C::FM * C::FN, kDs = C::FM + C::FN;
    constexpr int kSlots = kMf > C::LPS ? kMf : C::LPS;
    const int wave = uni((int)(threadIdx.x >> 6));
    // the refill, as in issue_stage
    const bool in_k = lp.kc < K - k0;
    const uint32_t a0 = in_k ? lp.a_off + (uint32_t)k0 * 2u : kOob;
    const uint32_t b0 = in_k ? lp.b_off + (uint32_t)k0 * 2u : kOob;
    const uint32_t step = (uint32_t)uni((C::LTHREADS / C::CPR) * K * 2);
    // the fragments, as in load_frags (substep 0)
    const int lane = threadIdx.x & 63;
    const int wm = wave / C::WAVES_N, wc = wave % C::WAVES_N;
    const int lr = lane % C::MF, c = lane / C::MF;
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
        if (m < kMf) {
            const int i = m / C::FN, j = m % C::FN;
            if constexpr (C::MF == 32)
                st.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wl[j], xl[i], st.acc[i][j], 0, 0, 0);
            else
                st.acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl[j], xl[i], st.acc[i][j], 0, 0, 0);
        }
        if (m < C::A_LD)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(refill + (m * C::LTHREADS + wave * 64) * 16), 16,
                                                     a0 + (uint32_t)m * step, 0, 0, 0);
        else if (m < C::LPS)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (lds_void_t*)(refill + C::A_BYTES + ((m - C::A_LD) * C::LTHREADS + wave * 64) * 16), 16,
                b0 + (uint32_t)(m - C::A_LD) * step, 0, 0, 0);
        if (m < C::FM) {
            const int r = wm * C::WTM + m * C::MF + lr;
            xn[m] = *reinterpret_cast<const bf16x8*>(next + r * C::ROW_BYTES + ((c ^ swz<C::CPR>(r)) << 4));
        } else if (m < kDs) {
            const int r = wc * C::WTN + (m - C::FM) * C::MF + lr;
            wn[m - C::FM] =
                *reinterpret_cast<const bf16x8*>(next + C::A_BYTES + r * C::ROW_BYTES + ((c ^ swz<C::CPR>(r)) << 4));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedAlu = 0x001;
constexpr int kSchedValu = 0x002;
constexpr int kSchedSalu = 0x004;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedVmemWrite = 0x040;
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

// ---------------------------------------------------------------- slice-sum items
//
// The slice sum is cut into items: item i covers 64 16-byte chunks (512
// elements) of own-slice tile t = i / IPT, one chunk per lane, where own tiles
// are numbered row-major (t = tile row * tile columns + tile column, so own
// tile t carries ready flag rank * tiles_per_slice + t); an item spans
// 64 / (BN/8) consecutive rows of the tile, so a lane's offset inside an item
// is a constant and the item's base offset is wave-uniform.

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
            if ((threadIdx.x & 63) == 0 && atomicCAS(&a.status[0], 0, kStatusTimeout) == 0)
                atomicExch(&a.status[1], flag);
            return false;
        }
    }
    return true;
}

// Fills the slice-sum stamps of ts own tiles and the launch (below) with
// their starting values, before a traced fused run.
__global__ void sum_trace_clear_kernel(uint32_t* st, int ts)
{
    for (int i = threadIdx.x; i < (ts + 1) * 4; i += blockDim.x) st[i] = (i & 3) < 2 ? 0xFFFFFFFFu : 0u;
}

// Slice-sum trace (debug runs only): per own tile t, words 4t .. 4t+3 hold the
// earliest time a wave checked its flag for a sum, the earliest time a wave
// saw it released, the latest time a wave stored a sum of it, and the number
// of items summed (100 MHz counter, low words); words 4 ts, 4 ts + 1 hold the
// launch's first and last workgroup times.  The host fills the minima with
// all ones and the rest with zeros before a traced run.
__device__ __forceinline__ uint32_t now32() { return (uint32_t)wall_clock64(); }

__device__ __forceinline__ void trace_sum(const Args& a, int t, uint32_t poll, uint32_t acq, uint32_t done, uint32_t n)
{
    uint32_t* w = a.sum_trace + (int64_t)t * 4;
    atomicMin(w, poll);
    atomicMin(w + 1, acq);
    atomicMax(w + 2, done);
    atomicAdd(w + 3, n);
}

// Sums the items item[0 .. B-1] (slice item indices; past the last item or
// negative: none) with plain loads: every peer chunk first (they need no flag),
// then each item's tile flag is checked and its local chunk loaded, in the sum
// order.  An item whose flag does not arrive within the watchdog limit is
// reported and skipped (`gave_up` then skips later unreleased items without
// waiting).
template <int B, int SLEEP = 2, bool ROWS = false>
__device__ __forceinline__ void sum_batch(const Args& a, const ItemMap& m, const int (&item)[B], uint32_t epoch,
                                          bool& gave_up)
{
    const __amdgpu_buffer_rsrc_t rl =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.dst[a.g.rank], 0, a.slice_bytes, kRsrcFlags);
    uint32_t boff[B];
    u32x4 v[B][kPeers + 1];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        boff[b] = item[b] >= 0 ? item_boff(m, a, item[b]) : kOob;
#pragma unroll
        for (int s = 0; s < kPeers; ++s) {
            const __amdgpu_buffer_rsrc_t rp =
                __builtin_amdgcn_make_buffer_rsrc((void*)a.peers[s], 0, a.slice_bytes, kRsrcFlags);
            v[b][s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, boff[b], 0, kAuxNt));
        }
    }
    // every item's ready word first, in one round trip; a tile not yet
    // released is then waited for
    uint32_t tp[B], ta[B], fw[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const bool in = item[b] >= 0 && item[b] < m.nitems;
        fw[b] = in ? __hip_atomic_load(ready_word<ROWS>(a, a.g.rank * a.g.ts + (item[b] >> m.ipt_log2)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : 0u;
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const bool in = item[b] >= 0 && item[b] < m.nitems;
        if (a.trace_on) tp[b] = now32();
        const bool ok = in && (released<ROWS>(a, fw[b], epoch) ||
                               wait_tile<SLEEP, ROWS>(a, epoch, item[b] >> m.ipt_log2, gave_up));
        if (a.trace_on) ta[b] = ok ? now32() : 0xFFFFFFFFu;
        boff[b] = ok ? boff[b] : kOob;
        v[b][kPeers] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, boff[b], 0, kAuxSc1));
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
        f32x8 acc = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s <= kPeers; ++s) acc = add8(acc, v[b][s]);
        store_sum(a, pack8(acc), boff[b]);
        if (a.trace_on && item[b] >= 0 && item[b] < m.nitems && (threadIdx.x & 63) == 0)
            trace_sum(a, item[b] >> m.ipt_log2, tp[b], ta[b], now32(), ta[b] != 0xFFFFFFFFu ? 1u : 0u);
    }
}

// Sums items first, first + stride, ... BATCH at a time (sum_batch).
// SLEEP: s_sleep argument between flag polls (64 clocks each); ROWS: the
// row-counter protocol.
template <int BATCH, int SLEEP = 2, bool ROWS = false>
__device__ __forceinline__ void drain_items(const Args& a, const ItemMap& m, int first, int stride, uint32_t epoch)
{
    bool gave_up = false;
    for (int base = first; base < m.nitems; base += BATCH * stride) {
        int item[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) item[b] = base + b * stride;
        sum_batch<BATCH, SLEEP, ROWS>(a, m, item, epoch, gave_up);
    }
}


// ---------------------------------------------------------------- slice-sum stream
//
// reduce_mode STREAM (256x256 tile, eight waves): waves 0-3 issue every stage
// load of the GEMM ("loader" waves), waves 4-7 issue none and instead stream
// the slice sum while all eight run the MFMAs.  Vector-memory operations of a
// wave retire in issue order, so a wave that waits for its stage loads every
// K step could not keep an HBM load in flight across steps; a stream wave
// only ever waits for its own stream operations.
//
// Stream wave w of the TW in the grid owns items [n w / TW, n (w + 1) / TW)
// and sums one item per group of four K steps.  Step PH of a group (0..3)
// issues two device-scope loads of the group's item, in the oracle's sum
// order: peers 0, 1 | peers 2, 3 | peers 4, 5 | peer 6, local; and consumes
// the two loads issued two steps earlier (from the previous group at PH 0, 1):
//   PH 0: acc = (acc + p4) + p5                        (previous item)
//   PH 1: acc = (acc + p6) + local, stored to out     (previous item)
//   PH 2: acc = ((0 + p0) + p1)                        (this item)
//   PH 3: acc = (acc + p2) + p3                        (this item)
// The stream waves' K loop is unrolled by four, so the sources, the reset,
// the store and the wait counts are constants of the step's code, which has
// no branch and is interleaved with the step's MFMAs.  A tile runs the
// groups if the workgroup has latched (below) when the tile begins and the
// wave still has items, or, when the workgroup's later tiles hold fewer
// groups than the wave has items left, from the step after the tile's probe
// latches; other tiles run the plain loop, and a wave whose last item was
// begun in the previous tile finishes it first.  A group past
// the wave's last item issues the same instructions through an empty buffer
// resource (they read zeros) and its store goes past its resource.  Loads land in two 2 KiB LDS slot pairs, pair PH & 1: a step
// reads the pair of the step two back at its start and refills it once the
// values are used.  The stream step runs after the step's first substep, not
// right after the barrier, where the loader waves' refill fills the load
// queue.  The steps of a
// tile that do not fill a group run without stream code; the loads of a
// group's last two steps are consumed in the next group, possibly after the
// tile's epilogue stores (counted in the waits of a tile's first group).
//
// The local partial of an item may be read only once its tile is released.
// A workgroup's four stream waves own consecutive items, spanning own tiles
// t_lo .. t_hi; until all of them are released (latched once seen), tiles
// run the plain loop.  Loader wave 0 probes the tiles' flags with device-scope
// loads into LDS right after the barrier of step kProbe - 1 (and of every
// fourth step after it), while the workgroup has not latched; the wait of the
// next step covers them, and after its barrier every wave reads the probe and
// latches together.  A tile's groups begin at its start, or, when the later
// tiles cannot hold a wave's remaining items, right after the latching step.
// The previous
// tile's flag is published after the barrier of step kPub: the stream waves'
// epilogue stores are older than the loads its wait covers.  Items a stream
// wave has not finished after the workgroup's last tile are summed there by
// the stream wave and its SIMD's loader wave.
constexpr int kSPairLds = 2048;        // two 1 KiB slots
constexpr int kSWaveLds = 2 * kSPairLds;
constexpr int kProbeLds = 256;         // 64 flags
constexpr int kProbe = 4;              // step whose barrier certifies the probe
constexpr int kPub = 2;                // step whose barrier publishes the previous tile's flag
constexpr int kStreamLds = 4 * kSWaveLds + kProbeLds;

struct Stream {
    char* slots;          // this wave's two slot pairs
    const char* probe;    // the workgroup's probe area (one flag per lane)
    ItemMap m;
    int first, end;       // this wave's item range
    int item;             // next item to begin
    int real_cur;         // this group's loads are real (its item exists and is released)
    int real_prev;        // the previous group's
    uint32_t ioff, coff;  // this lane's byte offset of this / the previous group's item (kOob: none)
    bool latched;         // every own tile of the workgroup's items is released
    int tiles_left;       // the workgroup's tiles after the current one
    int t_lo, t_hi;       // own tiles of the workgroup's items (t_hi < t_lo: none)
    uint32_t epoch;
    uint32_t slice_bytes;
    f32x8 acc;
};

// Eight BF16 values to FP32 (exact).
__device__ __forceinline__ f32x8 widen8(const u32x4& v)
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
    return b;
}

// Item range of stream wave gw of tw over n items.
__device__ __forceinline__ int stream_bound(int64_t n, int gw, int tw) { return (int)(n * gw / tw); }

// Every wave of a stream workgroup sets this up (the loader waves use the
// probe fields only).  pos: the workgroup's position in a round, sw: the
// stream wave index 0..3 (loader waves pass 0), C: compute workgroups.
__device__ __forceinline__ void stream_init(Stream& s, const Args& a, char* stream_lds, int pos, int sw, int C,
                                            uint32_t epoch)
{
    s.m = item_map(a);
    const int64_t n = s.m.nitems;
    const int tw = 4 * C;
    s.slots = stream_lds + sw * kSWaveLds;
    s.probe = stream_lds + 4 * kSWaveLds;
    s.first = uni(stream_bound(n, pos * 4 + sw, tw));
    s.end = uni(stream_bound(n, pos * 4 + sw + 1, tw));
    const int wfirst = stream_bound(n, pos * 4, tw), wend = stream_bound(n, pos * 4 + 4, tw);
    s.t_lo = uni(wfirst >> s.m.ipt_log2);
    s.t_hi = uni(wend > wfirst ? (wend - 1) >> s.m.ipt_log2 : s.t_lo - 1);
    s.item = s.first;
    s.real_cur = 0;
    s.real_prev = 0;
    s.ioff = kOob;
    s.coff = kOob;
    s.latched = s.t_hi < s.t_lo;  // nothing to wait for
    s.tiles_left = uni(pos < a.g.tiles ? (a.g.tiles - pos + C - 1) / C : 0);
    s.epoch = (uint32_t)uni((int)epoch);
    s.slice_bytes = a.slice_bytes;
    s.acc = f32x8{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
}

// Loader wave 0: device-scope loads of the flags of own tiles t_lo + lane
// (lanes past t_hi read zero) into the probe area.
__device__ __forceinline__ void stream_probe_issue(const Stream& s, const Args& a)
{
    const int lane = threadIdx.x & 63;
    const int t = s.t_lo + lane;
    const uint32_t fbytes = (uint32_t)a.g.tiles * (uint32_t)a.flag_stride * 4u;
    const __amdgpu_buffer_rsrc_t rf = __builtin_amdgcn_make_buffer_rsrc((void*)a.flags, 0, fbytes, kRsrcFlags);
    const uint32_t off = t <= s.t_hi ? (uint32_t)((a.g.rank * a.g.ts + t) * a.flag_stride) * 4u : kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rf, (lds_void_t*)s.probe, 4, off, 0, 0, kAuxSc1);
}

// Every wave, after the barrier that certifies the probe: latch once every
// probed tile holds this run's epoch.
__device__ __forceinline__ void stream_probe_read(Stream& s)
{
    const int lane = threadIdx.x & 63;
    const uint32_t f = *reinterpret_cast<const uint32_t*>(s.probe + lane * 4);
    const bool ok = s.t_lo + lane > s.t_hi || f == s.epoch;
    s.latched = __builtin_amdgcn_ballot_w64(ok) == ~0ull;
}

// A wave-uniform mask the compiler cannot see through: selects written as
// bit operations on it stay selects (a known 0 / -1 mask would be folded into
// a select, and a select between expensive values into a branch, which would
// split the step's code from the MFMAs it is meant to run between).
__device__ __forceinline__ uint32_t opaque_mask(int cond)
{
    uint32_t m = (uint32_t)uni(cond ? -1 : 0);
    __asm__("" : "+s"(m));
    return m;
}

__device__ __forceinline__ uint32_t bsel(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

// This lane's byte offset of item `item`'s chunk (kOob outside the ragged
// tile or past the last item), branch-free: item_boff with its selects as bit
// operations.
__device__ __forceinline__ uint32_t item_boff_nb(const ItemMap& m, const Args& a, int item)
{
    const uint32_t t = (uint32_t)(item >> m.ipt_log2);
    const int j = item & ((1 << m.ipt_log2) - 1);
    const int tml = (int)((__umulhi(t, m.div_m) + t) >> m.div_l);
    const int tn = (int)t - tml * a.g.tnc;
    const int row = j * m.rpi;
    const int trows = min(a.g.bm, a.g.S - tml * a.g.bm);
    const int tcols = min(a.g.bn, a.g.N - tn * a.g.bn);
    const uint32_t base = (uint32_t)(tml * a.g.bm + row) * (uint32_t)a.g.N + (uint32_t)(tn * a.g.bn);
    const uint32_t in_item = opaque_mask(item < m.nitems ? 1 : 0);
    const uint32_t in_tile = (row + m.lane_row < trows && m.lane_col < tcols) ? ~0u : 0u;
    return bsel(in_item & in_tile, (base + (uint32_t)m.lane_off) * 2u, kOob);
}

// Stream wave, before the step's MFMAs: wait for the loads of the step two
// back.  Younger vector-memory instructions: the step one back's two loads,
// plus the store of a group's step 1 (consumed at steps 2 and 3), plus the
// previous tile's epilogue stores in a tile's first group (steps 0 and 1).
template <int PH, int STORES>
__device__ __forceinline__ void stream_wait(bool first_group)
{
    constexpr int kYoung = (PH == 0 || PH == 1) ? 2 : 3;
    if constexpr (PH <= 1) {
        if (first_group)
            wait_vmcnt<kYoung + STORES>();
        else
            wait_vmcnt<kYoung>();
    } else {
        wait_vmcnt<kYoung>();
    }
}

// Stream wave, at the start of a step (after stream_wait): read the loads of
// the step two back (pair PH & 1); stream_step uses them before it refills
// the pair.
template <int PH>
__device__ __forceinline__ void stream_read(const Stream& s, u32x4& va, u32x4& vb)
{
    const char* pair = s.slots + (PH & 1) * kSPairLds + (threadIdx.x & 63) * 16;
    va = *reinterpret_cast<const u32x4*>(pair);
    vb = *reinterpret_cast<const u32x4*>(pair + 1024);
}

// Stream wave, after the first substep of step PH of a group: begin the group
// (PH 0), consume the loads read at the step's start, issue the step's two
// loads into the same pair PH & 1, store the previous item (PH 1).
template <int PH>
__device__ __forceinline__ void stream_step(Stream& s, const Args& a, const u32x4& va, const u32x4& vb)
{
    if constexpr (PH == 0) {
        const int item = uni(s.item);
        const int real = (s.latched ? 1 : 0) & (item < s.end ? 1 : 0);
        s.real_prev = s.real_cur;
        s.real_cur = uni(real);
        s.coff = s.ioff;
        s.ioff = item_boff_nb(s.m, a, item);
        s.item = item + real;
    }
    // consume (an idle step's loads read zeros and leave the sum as it is)
    const f32x8 wa = widen8(va), wb = widen8(vb);
    if constexpr (PH == 2) {
        const f32x8 z = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        s.acc = (z + wa) + wb;
    } else {
        s.acc = (s.acc + wa) + wb;
    }
    // (the slot pair is refilled below only after its values were used)
    __builtin_amdgcn_sched_barrier(0);
    // issue
    const uint16_t* pa = PH == 0 ? a.peers[0] : PH == 1 ? a.peers[2] : PH == 2 ? a.peers[4] : a.peers[6];
    const uint16_t* pb = PH == 0 ? a.peers[1] : PH == 1 ? a.peers[3] : PH == 2 ? a.peers[5] : a.dst[a.g.rank];
    const uint32_t nrec = s.slice_bytes & opaque_mask(s.real_cur);
    char* pair = s.slots + (PH & 1) * kSPairLds;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void*)pa, 0, nrec, kRsrcFlags),
                                             (lds_void_t*)pair, 16, s.ioff, 0, 0, kAuxSc1 | kAuxNt);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void*)pb, 0, nrec, kRsrcFlags),
                                             (lds_void_t*)(pair + 1024), 16, s.ioff, 0, 0, kAuxSc1 | kAuxNt);
    if constexpr (PH == 1) {
        const uint32_t soff = bsel(opaque_mask(s.real_prev), s.coff, kOob);
        __builtin_amdgcn_raw_buffer_store_b128(pack8(s.acc),
                                               __builtin_amdgcn_make_buffer_rsrc(a.out, 0, s.slice_bytes, kRsrcFlags),
                                               soff, 0, kAuxNt);
    }
}

// Stream wave, after its last tile: wait for everything in flight, then
// finish the last group (its steps 2 and 3 were never consumed) and store its
// item if it was real.
__device__ __forceinline__ void stream_settle(Stream& s, const Args& a)
{
    wait_vmcnt<0>();
    const int lane16 = (threadIdx.x & 63) * 16;
    const f32x8 w4 = widen8(*reinterpret_cast<const u32x4*>(s.slots + lane16));
    const f32x8 w5 = widen8(*reinterpret_cast<const u32x4*>(s.slots + 1024 + lane16));
    const f32x8 w6 = widen8(*reinterpret_cast<const u32x4*>(s.slots + kSPairLds + lane16));
    const f32x8 wl = widen8(*reinterpret_cast<const u32x4*>(s.slots + kSPairLds + 1024 + lane16));
    const f32x8 acc = (((s.acc + w4) + w5) + w6) + wl;
    const uint32_t soff = s.real_cur ? s.ioff : kOob;
    __builtin_amdgcn_raw_buffer_store_b128(pack8(acc), __builtin_amdgcn_make_buffer_rsrc(a.out, 0, s.slice_bytes, kRsrcFlags),
                                           soff, 0, kAuxNt);
    s.real_cur = 0;
}

// (trace) Records stamps for a stream wave's items [first, last) on every own
// tile they cover: a probe read (poll; acq if it latched) or, with n, the
// items summed by `done`.
__device__ __forceinline__ void stream_trace(const Args& a, const Stream& s, int first, int last, uint32_t poll,
                                             uint32_t acq, uint32_t done, bool count)
{
    if (last <= first || (threadIdx.x & 63) != 0) return;
    const int ipt = 1 << s.m.ipt_log2;
    for (int t = first >> s.m.ipt_log2; t <= (last - 1) >> s.m.ipt_log2; ++t) {
        const int lo = max(first, t * ipt), hi = min(last, (t + 1) * ipt);
        trace_sum(a, t, poll, acq, done, count ? (uint32_t)(hi - lo) : 0u);
    }
}

// ---------------------------------------------------------------- tile loop

// State carried from one tile to the next: whether the previous tile's
// epilogue stores may still be in flight, and its flag, which is stored once a
// wait has covered those stores.
struct StepHooks {
    bool stores;     // the previous tile's epilogue stores are still in flight
    int pend_q;      // slot of the previous tile, whose flag is still to be stored
    int pend_flag;
    uint32_t who, epoch;
};

// Stage wait: B = (NS-2)*LPS younger direct loads may stay in flight, plus the
// previous tile's C::STORES epilogue stores while they are younger than the
// stage waited for (steps before NS-1).
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
// (stages past the end load zeros), so every step waits for the same count;
// the barrier then certifies that every wave's loads of stage kt have landed
// and that every wave has finished reading stage kt-1, whose buffer the step
// refills.
template <class C>
struct TileJob {
    LoadPlan<C> lp;
    int nk;
    const void* xp;    // the buffer the tile's X rows come from, and its bytes
    uint32_t xbytes;
};

// X rows come from `xp` (xbytes long, row0 counted in it); by default from a.x.
// ISSUE: this wave issues stage loads (every wave but a stream kernel's
// stream waves).
template <class C, bool ISSUE = true>
__device__ __forceinline__ void tile_prologue(const Args& a, char* lds, TileJob<C>& job, int row0, int rows,
                                              int n0, int cols, const void* xp = nullptr, uint32_t xbytes = 0)
{
    const int K = a.g.K;
    job.nk = (K + C::BK - 1) / C::BK;
    job.xp = xp ? xp : (const void*)a.x;
    job.xbytes = xp ? xbytes : a.x_bytes;
    if (!ISSUE || job.nk == 0) return;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)uni_ptr(job.xp), 0, (uint32_t)uni((int)job.xbytes), kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.w, 0, a.w_bytes, kRsrcFlags);
    make_plan<C>(a, job.lp, row0, n0);
#pragma unroll
    for (int s = 0; s < C::NS - 1; ++s) issue_stage<C>(job.lp, rx, rw, lds + s * C::STAGE_BYTES, s * C::BK, K);
}

// Runs the K loop of a tile whose prologue has been issued.  The previous
// tile's epilogue stores were issued after this tile's prologue and before the
// first refill, so they have completed once the refill issued at step 0 has:
// at step NS-1 (or after the loop) its flag is published.
template <class C, bool ROWS = false>
__device__ __forceinline__ void tile_kloop(const Args& a, char* lds, TileState<C>& st, const TileJob<C>& job,
                                           StepHooks& hk)
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
        wait_stage<C>(hk.stores && kt < C::NS - 1);
        stage_barrier();
        if (kt == C::NS - 1) {
            hk.stores = false;
            if (hk.pend_flag >= 0) {
                if (threadIdx.x == 0) publish<ROWS>(a, hk.pend_q, hk.pend_flag, hk.who, hk.epoch);
                hk.pend_flag = -1;
            }
        }
        const int nxt = kt + C::NS - 1;
        kstep<C, true>(job.lp, rx, rw, lds + (nxt % C::NS) * C::STAGE_BYTES, nxt * C::BK, K,
                       lds + (kt % C::NS) * C::STAGE_BYTES, st);
    }
    // the zero-filling loads past the end drain; every wave finishes reading
    // LDS before the next tile's loads overwrite it; a flag still pending
    // (nk < NS) is published here
    wait_vmcnt<0>();
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
// The K loop of the four-wave two-stage tiles (C::LT).  With one wave per
// SIMD nothing else fills the MFMA pipe while a wave stalls on issuing a
// direct load, and a refill issued in a burst fills the TA's command queue
// (measured on the two-stage eight-wave loop: the queue full a quarter of the
// cycles).  So the barrier follows a step's first substep, which reads the
// fragments of substeps 2 and 3; the other three substeps form the tail,
// where MFMA m is followed by refill load m/3 (every third slot) and, from
// slot 1 on, every third slot by a fragment read of the next step's
// substeps 0 and 1, in that order.  Four fragment sets, one per substep; a
// set is rewritten only after its substep's MFMAs have been issued.
template <class C, bool ROWS = false>
__device__ __forceinline__ void tile_kloop_long(const Args& a, char* lds, TileState<C>& st, const TileJob<C>& job,
                                                StepHooks& hk)
{
    static_assert(C::LT && C::EW == 0, "four waves, four substeps, two stages");
    constexpr int kMf = C::FM * C::FN;  // MFMAs per substep
    constexpr int kDs = C::FM + C::FN;  // fragment reads per substep
    constexpr int kLs = 3;              // tail slots per refill load
    static_assert(C::LPS * kLs <= 3 * kMf && 1 + 3 * (2 * kDs - 1) < 3 * kMf, "the tail holds the refill and the reads");
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int e = 0; e < AccT<C::MF>::N; ++e) st.acc[i][j][e] = 0.0f;

    const int K = a.g.K;
    const int nk = job.nk;
    if (nk > 0) {
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)uni_ptr(job.xp), 0, (uint32_t)uni((int)job.xbytes), kRsrcFlags);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.w, 0, a.w_bytes, kRsrcFlags);
        bf16x8 x0[C::FM], w0[C::FN], x1[C::FM], w1[C::FN], x2[C::FM], w2[C::FN], x3[C::FM], w3[C::FN];
        const int wave = uni((int)(threadIdx.x >> 6));
        const int lane = threadIdx.x & 63;
        const int wm = wave / C::WAVES_N, wc = wave % C::WAVES_N;
        const int lr = lane % C::MF;
        const uint32_t step = (uint32_t)uni((C::LTHREADS / C::CPR) * K * 2);
        // stage 0 came from the prologue, before the previous tile's stores
        if (hk.stores)
            wait_vmcnt<C::STORES>();
        else
            wait_vmcnt<0>();
        stage_barrier();
        issue_stage<C>(job.lp, rx, rw, lds + C::STAGE_BYTES, C::BK, K);
        load_frags<C>(lds, 0, x0, w0);
        load_frags<C>(lds, 1, x1, w1);
        for (int kt = 0; kt + 1 < nk; ++kt) {
            char* cur = lds + (kt & 1) * C::STAGE_BYTES;
            const char* nxt = lds + ((kt + 1) & 1) * C::STAGE_BYTES;
            load_frags<C>(cur, 2, x2, w2);
            load_frags<C>(cur, 3, x3, w3);
            mfma_substep<C>(st, x0, w0);
#pragma unroll
            for (int m = 0; m < kMf; ++m) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                if (m < 2 * kDs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kDs > kMf ? 2 : 1, 0);
            }
            wait_vmcnt<0>();
            wait_lgkm0();
            stage_barrier();
            if (kt == 0) publish_pending<ROWS>(a, hk);
            // the refill of this step's buffer with stage kt + 2, as in issue_stage
            const int k0 = (kt + 2) * C::BK;
            const bool in_k = job.lp.kc < K - k0;
            const uint32_t a0 = in_k ? job.lp.a_off + (uint32_t)k0 * 2u : kOob;
            const uint32_t b0 = in_k ? job.lp.b_off + (uint32_t)k0 * 2u : kOob;
#pragma unroll
            for (int m = 0; m < 3 * kMf; ++m) {
                const int ss = m / kMf, i = (m % kMf) / C::FN, j = m % C::FN;
                if (ss == 0)
                    st.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1[j], x1[i], st.acc[i][j], 0, 0, 0);
                else if (ss == 1)
                    st.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w2[j], x2[i], st.acc[i][j], 0, 0, 0);
                else
                    st.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w3[j], x3[i], st.acc[i][j], 0, 0, 0);
                if (m % kLs == 0 && m / kLs < C::LPS) {
                    const int li = m / kLs;
                    if (li < C::A_LD)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rx, (lds_void_t*)(cur + (li * C::LTHREADS + wave * 64) * 16), 16, a0 + (uint32_t)li * step, 0,
                            0, 0);
                    else
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rw, (lds_void_t*)(cur + C::A_BYTES + ((li - C::A_LD) * C::LTHREADS + wave * 64) * 16), 16,
                            b0 + (uint32_t)(li - C::A_LD) * step, 0, 0, 0);
                }
                if (m >= 1 && (m - 1) % 3 == 0 && (m - 1) / 3 < 2 * kDs) {
                    // the next step's substep sb fragment di, as in load_frags
                    const int dd = (m - 1) / 3, sb = dd / kDs, di = dd % kDs;
                    const int c = sb * (C::KF / 8) + lane / C::MF;
                    if (di < C::FM) {
                        const int r = wm * C::WTM + di * C::MF + lr;
                        const bf16x8 v =
                            *reinterpret_cast<const bf16x8*>(nxt + r * C::ROW_BYTES + ((c ^ swz<C::CPR>(r)) << 4));
                        if (sb == 0) x0[di] = v; else x1[di] = v;
                    } else {
                        const int r = wc * C::WTN + (di - C::FM) * C::MF + lr;
                        const bf16x8 v = *reinterpret_cast<const bf16x8*>(nxt + C::A_BYTES + r * C::ROW_BYTES +
                                                                          ((c ^ swz<C::CPR>(r)) << 4));
                        if (sb == 0) w0[di - C::FM] = v; else w1[di - C::FM] = v;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the last step (its substep 0 and 1 fragments are in sets 0 and 1)
        const char* cur = lds + ((nk - 1) & 1) * C::STAGE_BYTES;
        load_frags<C>(cur, 2, x2, w2);
        load_frags<C>(cur, 3, x3, w3);
        mfma_substep<C>(st, x0, w0);
        mfma_substep<C>(st, x1, w1);
        mfma_substep<C>(st, x2, w2);
        mfma_substep<C>(st, x3, w3);
    }
    // the zero-filling loads past the end drain; every wave finishes reading
    // LDS before the next tile's loads overwrite it; a flag still pending
    // (nk < 2) is published here
    wait_vmcnt<0>();
    stage_barrier();
    publish_pending<ROWS>(a, hk);
}

template <class C, bool ROWS = false>
__device__ __forceinline__ void tile_kloop_xp(const Args& a, char* lds, TileState<C>& st, const TileJob<C>& job,
                                              StepHooks& hk)
{
    if constexpr (C::LT) {
        tile_kloop_long<C, ROWS>(a, lds, st, job, hk);
        return;
    }
    static_assert(C::KSUB % 2 == 0, "substep s of every step uses fragment buffer s % 2");
    static_assert(C::EW == 0, "every wave loads stages");
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
            if (hk.stores && kt + 1 < C::NS - 1)
                wait_vmcnt<B + C::STORES>();
            else
                wait_vmcnt<B>();
            wait_lgkm0();
            stage_barrier();
            if (kt + 1 == C::NS - 1) publish_pending<ROWS>(a, hk);
            // raised issue priority from the barrier to the end of the step,
            // while the wave issues the refill (measured: ~1% faster than
            // without, and than raising it over the MFMA-only part)
            __builtin_amdgcn_s_setprio(1);
            xp_tail<C>(st, xf[(C::KSUB - 1) & 1], wf[(C::KSUB - 1) & 1], xf[0], wf[0],
                       lds + ((kt + 1) % C::NS) * C::STAGE_BYTES, job.lp, rx, rw, lds + (kt % C::NS) * C::STAGE_BYTES,
                       (kt + C::NS) * C::BK, K);
            __builtin_amdgcn_s_setprio(0);
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
    publish_pending<ROWS>(a, hk);
}

// The K loop of a tile in the stream kernel (four loader waves, four stream
// waves, two stages), pipelined across steps like tile_kloop_xp.  Loader waves
// wait for their stage loads (and at step 0 for their previous epilogue
// stores) and issue the refill; stream waves issue no stage loads, wait only
// for their own stream loads, and run the steps of a tile in groups of four
// (a stream step each), then the remaining steps without stream code.  The
// previous tile's flag is published after the barrier of step kPub, the first
// that certifies the stream waves' epilogue stores (at the tile's end if the
// loop is shorter).
template <class C>
struct SplitLoop {
    static_assert(C::KSUB % 2 == 0 && C::NS == 2 && C::WAVES == 8 && C::LW == 4, "stream kernel tile");
    static constexpr int kMf = C::FM * C::FN;   // MFMAs per substep
    static constexpr int kDs = C::FM + C::FN;   // fragment reads per substep

    // Substeps 0 .. KSUB-2 of step kt (MFMAs with the next substep's
    // fragment reads between them).
    static __device__ __forceinline__ void head(TileState<C>& st, const char* cur, bf16x8 (&xf)[2][C::FM],
                                                bf16x8 (&wf)[2][C::FN])
    {
#pragma unroll
        for (int ss = 0; ss + 1 < C::KSUB; ++ss) {
            load_frags<C>(cur, ss + 1, xf[(ss + 1) & 1], wf[(ss + 1) & 1]);
            mfma_substep<C>(st, xf[ss & 1], wf[ss & 1]);
        }
#pragma unroll
        for (int ss = 0; ss + 1 < C::KSUB; ++ss)
#pragma unroll
            for (int m = 0; m < kMf; ++m) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                if (m < kDs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
    }

    // After the barrier of step kt: the flag publish and the readiness probe.
    static __device__ __forceinline__ void control(const Args& a, StepHooks& hk, Stream& s, int kt, bool prober)
    {
        if (kt == kPub) publish_pending<false>(a, hk);
        if (!s.latched) {
            // a probe after the barrier of step kProbe - 1 + 4j, read after
            // the next one, until the workgroup latches
            if (kt >= kProbe - 1 && ((kt - (kProbe - 1)) & 3) == 0 && prober) stream_probe_issue(s, a);
            if (kt >= kProbe && ((kt - kProbe) & 3) == 0) {
                stream_probe_read(s);
                // (stamps: a tile's first probe and the latching one; stamping
                // every probe would crowd the stamp words with atomics)
                if (a.trace_on && threadIdx.x >= C::LW * 64 && (kt == kProbe || s.latched)) {
                    const uint32_t t = now32();
                    stream_trace(a, s, s.first, s.end, t, s.latched ? t : 0xFFFFFFFFu, 0u, false);
                }
            }
        }
    }

    // The last substep of step kt and the next step's first fragments.
    static __device__ __forceinline__ void tail(TileState<C>& st, const char* lds, int kt, bf16x8 (&xf)[2][C::FM],
                                                bf16x8 (&wf)[2][C::FN])
    {
        load_frags<C>(lds + ((kt + 1) & 1) * C::STAGE_BYTES, 0, xf[0], wf[0]);
        mfma_substep<C>(st, xf[(C::KSUB - 1) & 1], wf[(C::KSUB - 1) & 1]);
    }

    // One step of a stream wave with stream phase PH.  The stream step runs
    // after the step's first substep, away from the barrier, where the loader
    // waves' refill (issued right after it) has left the load queue.
    template <int PH>
    static __device__ __forceinline__ void stream_step_k(const Args& a, char* lds, TileState<C>& st, StepHooks& hk,
                                                         Stream& s, int kt, bool first_group,
                                                         bf16x8 (&xf)[2][C::FM], bf16x8 (&wf)[2][C::FN])
    {
        stream_wait<PH, C::STORES>(first_group);
        u32x4 va, vb;
        stream_read<PH>(s, va, vb);
        const char* cur = lds + (kt & 1) * C::STAGE_BYTES;
        load_frags<C>(cur, 1, xf[1], wf[1]);
        mfma_substep<C>(st, xf[0], wf[0]);
#pragma unroll
        for (int m = 0; m < kMf; ++m) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (m < kDs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        stream_step<PH>(s, a, va, vb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ss = 1; ss + 1 < C::KSUB; ++ss) {
            load_frags<C>(cur, ss + 1, xf[(ss + 1) & 1], wf[(ss + 1) & 1]);
            mfma_substep<C>(st, xf[ss & 1], wf[ss & 1]);
        }
#pragma unroll
        for (int ss = 1; ss + 1 < C::KSUB; ++ss)
#pragma unroll
            for (int m = 0; m < kMf; ++m) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                if (m < kDs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
        wait_lgkm0();
        stage_barrier();
        control(a, hk, s, kt, false);
        tail(st, lds, kt, xf, wf);
#pragma unroll
        for (int m = 0; m < kMf; ++m) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (m < kDs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
    }

    // One step of a stream wave without stream code.
    static __device__ __forceinline__ void plain_step(const Args& a, char* lds, TileState<C>& st, StepHooks& hk,
                                                      Stream& s, int kt, bf16x8 (&xf)[2][C::FM],
                                                      bf16x8 (&wf)[2][C::FN])
    {
        head(st, lds + (kt & 1) * C::STAGE_BYTES, xf, wf);
        wait_lgkm0();
        stage_barrier();
        control(a, hk, s, kt, false);
        tail(st, lds, kt, xf, wf);
#pragma unroll
        for (int m = 0; m < kMf; ++m) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (m < kDs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
    }

    // One step of a loader wave: wait for the stage, refill, compute.
    static __device__ __forceinline__ void loader_step(const Args& a, char* lds, TileState<C>& st, StepHooks& hk,
                                                       Stream& s, const TileJob<C>& job, __amdgpu_buffer_rsrc_t rx,
                                                       __amdgpu_buffer_rsrc_t rw, int kt, bool prober,
                                                       bf16x8 (&xf)[2][C::FM], bf16x8 (&wf)[2][C::FN])
    {
        head(st, lds + (kt & 1) * C::STAGE_BYTES, xf, wf);
        wait_vmcnt<0>();
        wait_lgkm0();
        stage_barrier();
        control(a, hk, s, kt, prober);
        __builtin_amdgcn_s_setprio(1);
        issue_stage<C>(job.lp, rx, rw, lds + (kt & 1) * C::STAGE_BYTES, (kt + 2) * C::BK, a.g.K);
        tail(st, lds, kt, xf, wf);
        // the refill's loads, two per MFMA, then the next step's first fragments
#pragma unroll
        for (int m = 0; m < kMf; ++m) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (2 * m < C::LPS) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 2, 0);
            if (m < kDs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_s_setprio(0);
    }
};

template <class C, bool STREAMER>
__device__ __forceinline__ void tile_kloop_split(const Args& a, char* lds, TileState<C>& st, const TileJob<C>& job,
                                                 StepHooks& hk, Stream& s)
{
    typedef SplitLoop<C> L;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int e = 0; e < AccT<C::MF>::N; ++e) st.acc[i][j][e] = 0.0f;

    const int nk = job.nk;
    const int wave = uni((int)(threadIdx.x >> 6));
    if (nk > 0) {
        bf16x8 xf[2][C::FM], wf[2][C::FN];
        if constexpr (!STREAMER) {
            const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)uni_ptr(job.xp), 0, (uint32_t)uni((int)job.xbytes), kRsrcFlags);
            const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.w, 0, a.w_bytes, kRsrcFlags);
            // stage 0 came from the prologue, before the previous tile's stores
            if (hk.stores)
                wait_vmcnt<C::STORES>();
            else
                wait_vmcnt<0>();
            stage_barrier();
            issue_stage<C>(job.lp, rx, rw, lds + C::STAGE_BYTES, C::BK, a.g.K);
            load_frags<C>(lds, 0, xf[0], wf[0]);
            for (int kt = 0; kt + 1 < nk; ++kt) L::loader_step(a, lds, st, hk, s, job, rx, rw, kt, wave == 0, xf, wf);
        } else {
            // a tile runs the stream's groups only while this wave has items
            // to sum and the slice's tiles are ready; otherwise the plain
            // loop, after finishing an item begun in the previous tile
            s.tiles_left -= 1;
            bool active = s.latched && s.item < s.end;
            if (!active && s.real_cur) stream_settle(s, a);
            // (trace: a wave that has summed all its items records them at the
            // next tile start; its range then starts at its end)
            if (a.trace_on && !active && s.latched && s.first < s.item) {
                stream_trace(a, s, s.first, s.item, 0xFFFFFFFFu, 0xFFFFFFFFu, now32(), true);
                s.first = s.item;
            }
            stage_barrier();
            load_frags<C>(lds, 0, xf[0], wf[0]);
            int kt = 0;
            if (!s.latched && (int64_t)s.tiles_left * ((nk - 1) / 4) < (int64_t)(s.end - s.item)) {
                // the later tiles' groups cannot hold this wave's items: begin
                // the groups in this tile, after the step whose probe latches
                for (; kt + 1 < nk && kt < kProbe; ++kt) L::plain_step(a, lds, st, hk, s, kt, xf, wf);
                for (; kt + 1 < nk && !s.latched; ++kt) L::plain_step(a, lds, st, hk, s, kt, xf, wf);
                active = s.latched && s.item < s.end;
            }
            if (active)
            for (; kt + 4 < nk; kt += 4) {
                // (the previous tile's epilogue stores are younger than the
                // previous group's loads only in a tile's first group)
                const bool first = kt == 0;
                L::template stream_step_k<0>(a, lds, st, hk, s, kt, first, xf, wf);
                L::template stream_step_k<1>(a, lds, st, hk, s, kt + 1, first, xf, wf);
                L::template stream_step_k<2>(a, lds, st, hk, s, kt + 2, first, xf, wf);
                L::template stream_step_k<3>(a, lds, st, hk, s, kt + 3, first, xf, wf);
            }
            for (; kt + 1 < nk; ++kt) L::plain_step(a, lds, st, hk, s, kt, xf, wf);
        }
        // the last step
        const char* cur = lds + ((nk - 1) & 1) * C::STAGE_BYTES;
#pragma unroll
        for (int ss = 0; ss < C::KSUB; ++ss) {
            if (ss + 1 < C::KSUB) load_frags<C>(cur, ss + 1, xf[(ss + 1) & 1], wf[(ss + 1) & 1]);
            mfma_substep<C>(st, xf[ss & 1], wf[ss & 1]);
        }
    }
    // loader waves drain the zero-filling loads past the end; stream waves
    // keep their loads in flight unless the previous tile's flag is still to
    // be published (a loop shorter than kPub + 1 steps); every wave finishes
    // reading LDS before the next tile's loads overwrite it
    if (!STREAMER || hk.pend_flag >= 0) wait_vmcnt<0>();
    stage_barrier();
    publish_pending<false>(a, hk);
}

// ---------------------------------------------------------------- adaptive controller
//
// Reading of mKernel's adaptive role split ("mKernel: Fast Multi-GPU,
// Multi-Node Fused Kernels", section 3.2: cost estimates from cycle counters,
// a communication target, role changes at task boundaries) for one GPU whose
// tiles fill whole rounds of the grid: a dedicated reducer workgroup takes its
// CU out of the GEMM for the rest of the launch, which adds a round of tiles
// whenever the tile count is a multiple of the grid (every workload here).
// Instead every compute workgroup changes role at its tile boundaries and sums
// a share of the slice there.  The slice's items are taken in release order
// (own tiles in schedule order); wave w of the W * G owns items w, w + W G, ...
// of that order, so every wave's share spreads over the whole release
// timeline and no wave claims anything at run time.  At a boundary a wave sums
// batches of four of its items: an even share of what it has left over the
// boundaries it has left, limited to items of rounds already released (slots
// below j * G after its j-th tile) and, once it has measured a batch with the
// 100 MHz counter, to a quarter of its last tile's time.  The last boundary
// sums everything left, as the tail does.
constexpr int kUnitItems = 4;

struct UnitCtl {
    int n;             // this wave's next item (the n-th of its share)
    uint32_t t_tile;   // this wave's last tile time (ticks)
    uint32_t t_batch;  // this wave's last batch time (ticks; 0: none yet)
    bool gave_up;      // a flag wait timed out (later ones are not waited for)
};

// The slice item of release-order item v (v = s * items_per_tile + i, s an
// own tile's schedule slot).
__device__ __forceinline__ int release_item(const Args& a, const ItemMap& m, int v)
{
    const TileCoord t = decode_slot(a.g, v >> m.ipt_log2);
    return ((t.tml * a.g.tnc + t.tn) << m.ipt_log2) + (v & ((1 << m.ipt_log2) - 1));
}

// One wave at a boundary with nb boundaries left (this one included; nb == 1
// is the last).  Its share: release-order items base, base + stride, ...;
// `frontier`: release-order items below it are released.
template <bool ROWS>
__device__ __forceinline__ void sum_units(const Args& a, const ItemMap& m, UnitCtl& c, int nb, int frontier,
                                          int base, int stride, uint32_t epoch)
{
    const int total = m.nitems;
    const int mine = base < total ? (total - base + stride - 1) / stride : 0;
    const int rem = mine - c.n;
    if (rem <= 0) return;
    int batches = (rem + kUnitItems * nb - 1) / (kUnitItems * nb);
    if (nb > 1 && c.t_batch > 0u) batches = min(batches, max((int)((c.t_tile / 4u) / c.t_batch), 1));
    for (int bt = 0; bt < batches; ++bt) {
        int item[kUnitItems];
        int cnt = 0;
#pragma unroll
        for (int q = 0; q < kUnitItems; ++q) {
            const int nn = c.n + q;
            const int v = base + nn * stride;
            const bool take = nn < mine && (nb == 1 || v < frontier);
            item[q] = take ? release_item(a, m, v) : -1;
            cnt += take ? 1 : 0;
        }
        if (cnt == 0) return;
        const uint32_t t0 = now32();
        sum_batch<kUnitItems, 1, ROWS>(a, m, item, epoch, c.gave_up);
        c.t_batch = now32() - t0;
        c.n += cnt;
    }
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

// The tile loop of a compute workgroup at position `pos` of a round.  Round r
// covers slots [r*C, r*C + C).  A tile's flag is stored once the next tile's
// waits have covered the tile's stores: publishing costs no extra wait.  With
// `sum_tail` every wave then sums a share of the slice.
template <class C, bool FUSED, int VAR = 0>
__device__ __forceinline__ void compute_waves(const Args& a, char* lds, int pos, uint32_t who, uint32_t epoch,
                                              bool sum_tail)
{
    // the stream kernel: waves 0..LW-1 load stages, the others stream the sum
    constexpr bool SPLIT = C::EW > 0;
    static_assert(!SPLIT || (FUSED && VAR == 0), "the stream kernel is a fused kernel");
    const int Ctot = a.num_compute;
    const int wave = uni((int)(threadIdx.x >> 6));
    const bool loader = !SPLIT || wave < C::LW;
    StepHooks hk;
    hk.stores = false;
    hk.pend_q = -1;
    hk.pend_flag = -1;
    hk.who = who;
    hk.epoch = epoch;
    TileState<C> st;
    TileJob<C> job;
    Stream sm;
    if constexpr (SPLIT) stream_init(sm, a, lds + C::LDS_BYTES, pos, loader ? 0 : wave - C::LW, Ctot, epoch);
    // the adaptive controller: units at the boundaries from j0 on (once the
    // rounds holding own tiles are released)
    constexpr bool DYN = FUSED && (VAR & kVarDyn) != 0;
    const ItemMap um = item_map(a);
    UnitCtl uc = {0, 0u, 0u, false};
    const int ubase = pos * C::WAVES + wave, ustride = Ctot * C::WAVES;
    const int ntile = pos < a.g.tiles ? (a.g.tiles - pos + Ctot - 1) / Ctot : 0;
    const int j0 = a.g.ts > 0 ? (a.g.ts - 1) / Ctot + 1 : ntile;
    int j = 0;
    int q = pos;
    TileCoord t;
    if (q < a.g.tiles) {
        t = decode_slot(a.g, q);
        if (loader)
            tile_prologue<C>(a, lds, job, tile_row0(a.g, t), tile_rows(a.g, t), t.tn * C::BN, tile_cols(a.g, t));
        else
            tile_prologue<C, false>(a, lds, job, tile_row0(a.g, t), tile_rows(a.g, t), t.tn * C::BN,
                                    tile_cols(a.g, t));
    }
    while (q < a.g.tiles) {
        const uint32_t t_start = DYN ? now32() : 0u;
        if constexpr (SPLIT) {
            if (loader)
                tile_kloop_split<C, false>(a, lds, st, job, hk, sm);
            else
                tile_kloop_split<C, true>(a, lds, st, job, hk, sm);
        } else if constexpr (C::XP) {
            tile_kloop_xp<C, (VAR & kVarRows) != 0>(a, lds, st, job, hk);
        } else {
            tile_kloop<C, (VAR & kVarRows) != 0>(a, lds, st, job, hk);
        }
        // issue the next tile's first stages before this tile's stores
        const int qn = q + Ctot;
        TileCoord tn = t;
        if (qn < a.g.tiles) {
            tn = decode_slot(a.g, qn);
            if (loader)
                tile_prologue<C>(a, lds, job, tile_row0(a.g, tn), tile_rows(a.g, tn), tn.tn * C::BN,
                                 tile_cols(a.g, tn));
            else
                tile_prologue<C, false>(a, lds, job, tile_row0(a.g, tn), tile_rows(a.g, tn), tn.tn * C::BN,
                                        tile_cols(a.g, tn));
        }
        // the stage buffer the next tile's prologue left free holds the
        // epilogue staging areas
        const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(a.dst[t.d], 0, a.slice_bytes, kRsrcFlags);
        store_tile<C, (VAR & kVarNt) ? kStoreDeviceNt : kStoreDevice>(
            a, st, lds + (C::NS - 1) * C::STAGE_BYTES, rd, t.tml * C::BM, tile_rows(a.g, t), t.tn * C::BN,
            tile_cols(a.g, t));
        hk.stores = true;
        if (FUSED) {
            hk.pend_q = q;
            hk.pend_flag = t.flag;
        }
        if constexpr (DYN) {
            uc.t_tile = now32() - t_start;
            if (j >= j0 && j + 1 < ntile)
                sum_units<(VAR & kVarRows) != 0>(a, um, uc, ntile - j, (int)min((int64_t)j * Ctot << um.ipt_log2,
                                                                                 (int64_t)um.nitems),
                                                 ubase, ustride, epoch);
        }
        ++j;
        q = qn;
        t = tn;
    }
    if (hk.pend_flag >= 0) {
        wait_vmcnt<0>();
        stage_barrier();
        if (threadIdx.x == 0) publish<(VAR & kVarRows) != 0>(a, hk.pend_q, hk.pend_flag, who, epoch);
    }
    if constexpr (SPLIT) {
        // the stream waves settle their loads in flight; the items they have
        // not finished (an item begun restarts) are split between each stream
        // wave and the loader wave on its SIMD
        __shared__ int s_progress[C::EW];
        if (!loader) {
            stream_settle(sm, a);
            if (a.trace_on) stream_trace(a, sm, sm.first, sm.item, 0xFFFFFFFFu, 0xFFFFFFFFu, now32(), true);
            if ((threadIdx.x & 63) == 0) s_progress[wave - C::LW] = sm.item;
        }
        __syncthreads();
        const int sw = wave % C::EW, half = wave / C::EW;
        const int64_t n = sm.m.nitems;
        const int end = stream_bound(n, pos * C::EW + sw + 1, C::EW * Ctot);
        const int cur = uni(s_progress[sw]);
        const int mid = cur + (end - cur) / 2;
        ItemMap m = sm.m;
        m.nitems = half ? end : mid;
        drain_items<2>(a, m, half ? mid : cur, 1, epoch);
    } else if (DYN) {
        // the last boundary: units until none is left
        sum_units<(VAR & kVarRows) != 0>(a, um, uc, 1, um.nitems, ubase, ustride, epoch);
    } else if (sum_tail) {
        // every wave sums a share of the slice after its last tile (sixteen
        // items in flight per CU for the eight-wave and one-per-CU tiles; one
        // per wave for four-wave tiles at two per CU, whose shapes leave about
        // one item per wave: a second, empty slot of a batch still issues its
        // eight loads and lengthens the wait)
        const int wave = uni((int)(threadIdx.x >> 6));
        drain_items<(C::WAVES == 4 && C::LDS_BYTES <= 80 * 1024 - 64) ? 1 : 16 / C::WAVES, 2,
                    (VAR & kVarRows) != 0>(a, item_map(a), pos * C::WAVES + wave, a.num_compute * C::WAVES, epoch);
    }
}

// Compute role of the l-th compute workgroup of group grp: its position in a
// round is either the group's block offset + l (contiguous split) or
// l * 8 + grp (strided, used when all C_x are equal).  Without dedicated
// reducers the compute workgroups sum the slice after their last tile.
template <class C, bool FUSED, int VAR = 0>
__device__ __forceinline__ void compute_role(const Args& a, char* lds, int grp, int l, uint32_t epoch, int base)
{
    const int pos = uni(a.strided ? (l * kGroups + grp) : (base + l));
    const uint32_t who = ((uint32_t)grp << 16) | (uint32_t)l;
    compute_waves<C, FUSED, VAR>(a, lds, pos, who, epoch, FUSED && a.num_reducers == 0);
}

// Dedicated reducer role (used when reducers are requested): claim own-slice
// tiles in schedule order from this run's claim counter, wait for each tile's
// flag (thread 0 polls with device-scope loads and short sleeps, bounded by the
// watchdog), then sum the tile, reading the local slice at device scope.  The
// first wait that exceeds the watchdog reports the tile and latches: later
// unreleased tiles are skipped without waiting, so one reducer never waits
// longer than one watchdog period in total.
template <bool ROWS>
__device__ void reducer_role(const Args& a, uint32_t epoch)
{
    __shared__ int s_unit;
    __shared__ int s_skip;
    uint32_t* unit = &a.state->unit[epoch & 1u];
    bool gave_up = false;  // (thread 0's)
    uint32_t tp = 0u, ta = 0u;  // (thread 0's trace stamps of the unit)
    for (;;) {
        if (threadIdx.x == 0) {
            const int u = (int)atomicAdd(unit, 1u);
            int skip = 0;
            if (a.trace_on) tp = now32();
            if (u < a.g.ts) {
                const TileCoord t = decode_slot(a.g, u);
                const uint32_t* f = ready_word<ROWS>(a, t.flag);
                if (!released<ROWS>(a, __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), epoch)) {
                    if (gave_up) {
                        skip = 1;
                    } else {
                        const uint64_t t0 = wall_clock64();
                        while (!released<ROWS>(a, __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                               epoch)) {
                            __builtin_amdgcn_s_sleep(2);
                            if ((int64_t)(wall_clock64() - t0) > a.watchdog_ticks) {
                                skip = 1;
                                gave_up = true;
                                if (atomicCAS(&a.status[0], 0, kStatusTimeout) == 0)
                                    atomicExch(&a.status[1], t.flag);
                                break;
                            }
                        }
                    }
                }
            }
            if (a.trace_on) ta = skip ? 0xFFFFFFFFu : now32();
            s_unit = u;
            s_skip = skip;
        }
        __syncthreads();
        const int u = s_unit;
        const int skip = s_skip;
        __syncthreads();  // s_unit / s_skip are rewritten by the next claim
        if (u >= a.g.ts) return;
        if (skip) continue;
        const TileCoord t = decode_slot(a.g, u);
        const int rows = tile_rows(a.g, t), cols = tile_cols(a.g, t);
        const int cpr = cols >> 3;
        const int n = rows * cpr;
        const uint16_t* local = a.dst[a.g.rank];
        // four chunks per thread and pass: all their loads are issued before
        // any sum is stored (the stores could alias the loads of a later
        // pass, so the compiler keeps passes apart).  A reducer workgroup has
        // a CU to itself; the loads in flight set its share of HBM bandwidth.
        constexpr int kCh = 4;
        for (int c0 = threadIdx.x; c0 < n; c0 += kCh * (int)blockDim.x) {
            int64_t off[kCh];
            bool on[kCh];
            u32x4 v[kCh][kPeers + 1];
#pragma unroll
            for (int h = 0; h < kCh; ++h) {
                const int c = c0 + h * (int)blockDim.x;
                on[h] = c < n;
                const int cc = on[h] ? c : c0;
                const int r = cc / cpr;
                off[h] = (int64_t)(t.tml * a.g.bm + r) * a.g.N + t.tn * a.g.bn + (cc - r * cpr) * 8;
#pragma unroll
                for (int s = 0; s < kPeers; ++s)
                    v[h][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.peers[s] + off[h]));
                // the local slice at device scope (two 8-byte relaxed agent-scope loads)
                const uint64_t* lp = reinterpret_cast<const uint64_t*>(local + off[h]);
                const uint64_t l0 = __hip_atomic_load(lp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t l1 = __hip_atomic_load(lp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                v[h][kPeers] = u32x4{(uint32_t)l0, (uint32_t)(l0 >> 32), (uint32_t)l1, (uint32_t)(l1 >> 32)};
            }
#pragma unroll
            for (int h = 0; h < kCh; ++h) {
                if (!on[h]) continue;
                f32x8 acc = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s <= kPeers; ++s) acc = add8(acc, v[h][s]);
                const u32x4 o = pack8(acc);
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(a.out + off[h]));
                if (a.gather_on) {
#pragma unroll
                    for (int i = 0; i < kPeers; ++i)
                        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(a.gather[i] + off[h]));
                }
            }
        }
        if (a.trace_on) {
            __syncthreads();
            if (threadIdx.x == 0)
                trace_sum(a, t.tml * a.g.tnc + t.tn, tp, ta, now32(), (uint32_t)((a.g.bm * a.g.bn) >> 9));
        }
    }
}

// Role dispatch, with no device atomics on the default path.  Without
// dedicated reducers every workgroup computes and its position follows from
// its index.  With reducers, per-group arrival tickets hand out the roles (a
// reducer exists only once its group's compute workgroups are all resident).
//
// The run epoch: each workgroup keeps, in its own word of `finished`, the
// epoch of the last fused launch it finished.  A launch reads that word at
// the start and uses the next value; every workgroup of the previous fused
// launch stored the same value, so all workgroups of a launch agree on its
// epoch without communicating (the words change only at kernel ends).  The
// tickets and the claim counter of the next run are cleared by workgroup 0 of
// every fused run (the next run may use them even if this one does not).  A
// GEMM-only launch has no flags and touches none of this.
template <class C, bool FUSED, int VAR = 0>
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
        const uint32_t e = FUSED ? __hip_atomic_load(a.finished + blockIdx.x, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) + 1u
                                 : 0u;
        s_epoch = e;
        s_ticket = tickets ? atomicAdd(&a.state->role[e & 1u][grp], 1u) : (uint32_t)(blockIdx.x / kGroups);
        // (every fused run clears the next run's set, whether or not it uses
        // tickets itself: the next run may)
        if (FUSED && blockIdx.x == 0) {
            const uint32_t nx = (e + 1u) & 1u;
            for (int i = 0; i < kGroups; ++i)
                __hip_atomic_store(&a.state->role[nx][i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.state->unit[nx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (FUSED && a.trace_on && threadIdx.x == 0) atomicMin(a.sum_trace + (int64_t)a.g.ts * 4, now32());
    __syncthreads();
    // (read through readfirstlane so that the compiler sees them uniform: the
    // tile loop then stays in scalar registers)
    const uint32_t ticket = (uint32_t)uni((int)s_ticket);
    const uint32_t epoch = (uint32_t)uni((int)s_epoch);  // value this run's flags carry
    const GroupSplit split = group_split((int)gridDim.x, uni(a.num_reducers), grp);
    if (ticket < (uint32_t)split.compute)
        compute_role<C, FUSED, VAR>(a, lds, grp, (int)ticket, epoch, split.base);
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
        if (threadIdx.x == 0) {
            if (a.trace_on) atomicMax(a.sum_trace + (int64_t)a.g.ts * 4 + 2, now32());
            __hip_atomic_store(a.finished + blockIdx.x, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Tiles that fit two workgroups per CU keep two waves per SIMD resident.
template <class C, bool FUSED, int VAR = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fused_kernel(Args a)
{
    fused_body<C, FUSED, VAR>(a);
}

// Eight-wave workgroups (one per CU): two waves per SIMD, so one wave's
// MFMAs run while its sibling waits on LDS or a barrier.
template <class C, bool FUSED, int VAR = 0>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fused_kernel_8w(Args a)
{
    fused_body<C, FUSED, VAR>(a);
}

// Large tiles run one workgroup (one wave per SIMD) per CU: let the compiler
// use the whole register file for latency hiding.
template <class C, bool FUSED, int VAR = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fused_kernel_1w(Args a)
{
    fused_body<C, FUSED, VAR>(a);
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
// can only come from reads made after their rows were copied.  That holds per
// 128-byte line only if no line spans two tile-row blocks (a line cached when
// the first block is read could miss the second block's copy), so the host
// requires x_gathered to be 128-byte aligned and every slice, S * K * 2 bytes,
// a whole number of lines (a block of BM >= 16 rows of K % 8 == 0 elements
// always is).  Output tiles go to y [M][N]; there is no reduction.

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
            if ((threadIdx.x & 63) == 0 && atomicCAS(&a.status[0], 0, kStatusTimeout) == 0)
                atomicExch(&a.status[1], blk);
            return false;
        }
    }
    return true;
}

// Issues the first stages of tile t: X rows from the local slice (own tile)
// or from the gathered buffer once the block has arrived (FUSED) or because
// the buffer is already complete (GEMM only).  If the block's counter never
// arrives (the wait timed out and the status word says so), the tile reads
// its X rows as zeros rather than rows that may be only partly copied.
template <class C, bool FUSED>
__device__ __forceinline__ void ag_prologue(const Args& a, char* lds, TileJob<C>& job, const TileCoord& t,
                                            uint32_t target)
{
    const int rows = tile_rows(a.g, t), cols = tile_cols(a.g, t);
    if (t.d == a.g.rank) {
        tile_prologue<C>(a, lds, job, t.tml * C::BM, rows, t.tn * C::BN, cols, a.xsrc[a.g.rank], a.xs_bytes);
        return;
    }
    bool arrived = true;
    if constexpr (FUSED) arrived = ag_wait(a, t.d * a.g.tms + t.tml, target);
    tile_prologue<C>(a, lds, job, t.d * a.g.S + t.tml * C::BM, rows, t.tn * C::BN, cols, a.xg,
                     arrived ? a.x_bytes : 0u);
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
    hk.stores = false;
    hk.pend_q = -1;
    hk.pend_flag = -1;
    hk.who = 0;
    hk.epoch = run;
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
            tile_kloop_xp<C>(a, lds, st, job, hk);
        else
            tile_kloop<C>(a, lds, st, job, hk);
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
