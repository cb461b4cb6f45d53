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
//             to BF16, stores it into its destination slice buffer and releases
//             the tile's ready flag at agent scope;
//   reducer   claims own-slice tiles in schedule order, waits (acquire) for
//             their flags and sums each with the tp-1 peer partials.
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
// memory; the last workgroup to finish resets the counters and publishes the
// new epoch, so a launch needs no host-side state and can be replayed from a
// captured graph.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace gemm_rs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kReduceThreads = 256;  // standalone reduce kernel
constexpr int kPeers = 7;      // tp - 1 with tp = 8
constexpr int kGroups = 8;     // XCDs of an MI355X
constexpr int kStatusTimeout = -6;  // GEMM_RS_ERR_TIMEOUT
// A buffer-load offset at or past the resource's byte count reads as zero.
constexpr uint32_t kOob = 0x80000000u;
// Third descriptor word of a raw buffer resource on gfx9-family GPUs.
constexpr int kRsrcFlags = 0x00020000;

// Handle-owned device state, zeroed at creation.
struct DeviceState {
    uint32_t epoch;           // epoch of the last completed fused run
    uint32_t role[kGroups];   // per-group arrival tickets
    uint32_t unit;            // next reducer unit to claim
    uint32_t done;            // workgroups that finished this launch
    int32_t status[2];        // [0] error code, [1] flag index that timed out
    uint32_t pad[3];
};

struct Args {
    const uint16_t* x;       // [M][K]
    const uint16_t* w;       // [N][K]
    uint16_t* dst[8];        // destination slice buffers by destination rank
    const uint16_t* peers[kPeers];
    uint16_t* out;           // [S][N]
    uint32_t* flags;         // ready flags, flag_stride words apart
    DeviceState* state;
    uint32_t* trace;         // 4 words per slot (debug)
    Geometry g;
    uint32_t x_bytes, w_bytes;
    int64_t watchdog_ticks;  // 100 MHz ticks
    int32_t num_compute;     // C: compute workgroups in the grid
    int32_t num_reducers;    // R
    int32_t strided;         // XCD split of a round: 0 contiguous, 1 strided
    int32_t flag_stride;
    int32_t fused;           // 1: release flags, reducers run, epoch advances
    int32_t protocol;        // 0: per-wave release fence, 1: one release store
    int32_t drop_flag;
    int32_t trace_on;
};

// BM x BN output tile, BK deep stages, NS stages in LDS, WAVES_M x WAVES_N
// waves (4: one wave per SIMD, 8: two), MF x MF MFMA output blocks (32:
// v_mfma_f32_32x32x16_bf16, 16: v_mfma_f32_16x16x32_bf16).
template <int BM_, int BN_, int BK_, int NS_, int WAVES_M_, int WAVES_N_, int MF_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, NS = NS_;
    static_assert(NS >= 2 && NS <= 4, "stage depth");
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static_assert(WAVES == 4 || WAVES == 8, "four or eight waves per workgroup");
    static constexpr int MF = MF_;
    static constexpr int KF = MF_ == 32 ? 16 : 32;  // k per MFMA
    static constexpr int KSUB = BK / KF;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / MF, FN = WTN / MF;
    static_assert(FM >= 1 && FN >= 1 && WTM % MF == 0 && WTN % MF == 0, "wave tile");
    static constexpr int CPR = BK / 8;               // 16-byte chunks per LDS row
    static constexpr int ROW_BYTES = BK * 2;
    static constexpr int A_CHUNKS = BM * CPR, B_CHUNKS = BN * CPR;
    static_assert(A_CHUNKS % THREADS == 0 && B_CHUNKS % THREADS == 0, "whole load rounds");
    static constexpr int A_LD = A_CHUNKS / THREADS, B_LD = B_CHUNKS / THREADS;
    static constexpr int LPS = A_LD + B_LD;          // loads per thread per stage
    static_assert(LPS * (NS - 1) <= 63, "vmcnt range");
    static constexpr int A_BYTES = BM * ROW_BYTES;
    static constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;
    static constexpr int LDS_BYTES = NS * STAGE_BYTES;
    static_assert(CPR == 4 || CPR == 8 || CPR == 16, "swizzle defined for BK = 32, 64, 128");
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

// ---------------------------------------------------------------- GEMM tile

template <class C>
struct TileState {
    typename AccT<C::MF>::type acc[C::FM][C::FN];
};

// Per-thread load plan of one tile: byte offset of each chunk this thread
// moves at k = 0 (kOob for rows past the tile's valid extent) and the chunk's
// k offset (for the K tail).
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
        const int p = i * C::THREADS + tid;
        const int r = p / C::CPR;
        const int c = (p % C::CPR) ^ swz<C::CPR>(r);
        lp.a_k[i] = (uint16_t)(c * 8);
        lp.a_off[i] = r < rows ? ((uint32_t)(row0 + r) * K + (uint32_t)c * 8u) * 2u : kOob;
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
        const int p = i * C::THREADS + tid;
        const int r = p / C::CPR;
        const int c = (p % C::CPR) ^ swz<C::CPR>(r);
        lp.b_k[i] = (uint16_t)(c * 8);
        lp.b_off[i] = r < cols ? ((uint32_t)(n0 + r) * K + (uint32_t)c * 8u) * 2u : kOob;
    }
}

// Issue the LDS-direct loads of the BK slice starting at k0 into stage buffer
// `stage` (LPS loads per thread).  Each wave instruction fills 1 KiB of LDS:
// lane l writes bytes [16 l, 16 l + 16) after the wave's base.
//
// Branch-free: a chunk whose k lies at or past K (the K tail, or a whole stage
// past the end) gets an offset past the resource and reads as zero; rows past
// the tile carry kOob already, and kOob + 2 k0 stays past the resource.
template <class C>
__device__ __forceinline__ void issue_stage(const LoadPlan<C>& lp, __amdgpu_buffer_rsrc_t rx,
                                   __amdgpu_buffer_rsrc_t rw, char* stage, int k0, int K)
{
    const int wave = threadIdx.x >> 6;
    const int lim = K - k0;  // chunks with k offset >= lim are past K
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
        const uint32_t off = (int)lp.a_k[i] < lim ? lp.a_off[i] + (uint32_t)k0 * 2u : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (lds_void_t*)(stage + (i * C::THREADS + wave * 64) * 16), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
        const uint32_t off = (int)lp.b_k[i] < lim ? lp.b_off[i] + (uint32_t)k0 * 2u : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (lds_void_t*)(stage + C::A_BYTES + (i * C::THREADS + wave * 64) * 16), 16, off, 0, 0, 0);
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
    const int wave = threadIdx.x >> 6;
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
// and, per group of four registers, four consecutive output columns -- one
// 8-byte store per group in the epilogue.
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

// One K step: refill the buffer of stage kt-1 with stage kt+NS-1, then the
// MFMAs of stage kt with the fragments of substep s+1 read while substep s
// computes.  The scheduling groups place the substep-0 reads first and then
// one LDS read or one direct load after each MFMA, so neither waits on a full
// LDS round trip in the middle of the MFMA stream.
template <class C>
__device__ __forceinline__ void kstep(const LoadPlan<C>& lp, __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw,
                             char* refill, int k_refill, int K, const char* cur, TileState<C>& st)
{
    bf16x8 xf[2][C::FM], wf[2][C::FN];
    load_frags<C>(cur, 0, xf[0], wf[0]);
    issue_stage<C>(lp, rx, rw, refill, k_refill, K);
#pragma unroll
    for (int s = 0; s < C::KSUB; ++s) {
        if (s + 1 < C::KSUB) load_frags<C>(cur, s + 1, xf[(s + 1) & 1], wf[(s + 1) & 1]);
        mfma_substep<C>(st, xf[s & 1], wf[s & 1]);
    }
    constexpr int kMfmas = C::KSUB * C::FM * C::FN;
    constexpr int kFill = (C::KSUB - 1) * (C::FM + C::FN) + C::LPS;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, C::FM + C::FN, 0);
#pragma unroll
    for (int m = 0; m < kMfmas; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (m < kFill) __builtin_amdgcn_sched_group_barrier(kSchedDsRead | kSchedVmemRead, 1, 0);
    }
}

// Round the accumulators to BF16 and store the valid part of the tile at
// dst[m][n0 + n] (dst already points at the tile's first row).  The stores are
// device-scope (sc1): they write through this XCD's L2 to the memory side,
// where a device-scope load on any XCD sees them once they have completed --
// no L2 write-back is needed to publish the tile.
template <class C, bool DEVICE_SCOPE>
__device__ __forceinline__ void store_tile(const Args& a, const TileState<C>& st, uint16_t* dst, int rows, int n0,
                                  int cols)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t N = a.g.N;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int m = wm * C::WTM + i * C::MF + (lane % C::MF);
        if (m >= rows) continue;
        uint16_t* drow = dst + (int64_t)m * N + n0;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            constexpr int G = C::MF == 32 ? 4 : 1;
#pragma unroll
            for (int grp = 0; grp < G; ++grp) {
                const int n = C::MF == 32 ? wn * C::WTN + j * 32 + grp * 8 + (lane / 32) * 4
                                          : wn * C::WTN + j * 16 + (lane / 16) * 4;
                if (n < cols) {
                    const uint64_t v = (uint64_t)pack_bf16x2(st.acc[i][j][grp * 4 + 0], st.acc[i][j][grp * 4 + 1]) |
                                       ((uint64_t)pack_bf16x2(st.acc[i][j][grp * 4 + 2], st.acc[i][j][grp * 4 + 3]) << 32);
                    if constexpr (DEVICE_SCOPE)
                        __hip_atomic_store(reinterpret_cast<uint64_t*>(drow + n), v, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    else
                        *reinterpret_cast<uint64_t*>(drow + n) = v;
                }
            }
        }
    }
}

// Publish a finished tile by storing its ready flag (device scope).  Called by
// one thread once every wave's stores of the tile have completed.
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
    if (flag != a.drop_flag)
        __hip_atomic_store(a.flags + (int64_t)flag * a.flag_stride, epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- slice sum

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

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

// Engine loads go straight into a per-wave LDS area (LDS-direct global
// loads), never through registers the compiler would consider live: the data is
// read back with ds_read only after the step wait has certified its arrival.
// Peer partials are read once (non-temporal: kept out of L2); the local slice
// and the flags are read at device scope (sc1), so a copy left in this XCD's
// L2 by an earlier run is never used.
constexpr int kAuxNt = 2;
constexpr int kAuxSc1 = 16;
constexpr int kEngineSlotBytes = 1024;               // one 16-byte chunk per lane
constexpr int kEngineSlots = 2;                      // per wave

template <int AUX>
__device__ __forceinline__ void lds_load16(const uint16_t* g, char* slot)
{
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)slot, 16, 0, AUX);
}

__device__ __forceinline__ void lds_load_flag(const uint32_t* g, char* slot)
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
// elements) of own-slice tile u = i / IPT (schedule slot u), one chunk per lane;
// an item spans 64 / (BN/8) consecutive rows of the tile, so a lane's offset
// inside an item is a constant and the item's base offset is wave-uniform.
// Compute wave gw (of W) owns items gw, gw + W, gw + 2W, ... -- tile order.
// An item is summed in four steps of two loads each, in the sum order:
//   step 0: peers 0, 1    acc = (0 + p0) + p1
//   step 1: peers 2, 3    acc = (acc + p2) + p3
//   step 2: peers 4, 5    acc = (acc + p4) + p5
//   step 3: peer 6 and, if the item's tile is flagged, the local partial:
//           acc = (acc + p6) + local, stored to out; otherwise acc + p6 is
//           parked in registers and a later FINISH adds the local partial.
// POLL reads 64 ready flags (tiles anchor .. anchor+63, one per lane).  Peer
// loads need no flag, so a wave pre-sums while its tiles are still being
// computed.  Between MFMAs, every NS-1 K steps, a wave consumes its previous
// operation and issues the next; the loads go straight into two per-wave LDS
// slots and have completed by consumption time, because vector-memory
// operations complete in issue order and the stage wait NS-1 steps later
// covers a younger load.  After its last tile a wave drains its remaining
// items, polling flags under the watchdog.

enum EngineOp { kOpNone = 0, kOpStep = 1, kOpFinish = 2, kOpPoll = 3 };
constexpr int kPark = 2;  // parked FP32 partials per wave

struct Engine {
    char* slots;    // this wave's kEngineSlots LDS slots
    int next;       // next owned item not yet started (wave-uniform)
    int stride;     // compute waves W
    int nitems;     // items of the slice
    int ipt;        // items per tile
    int rpi;        // tile rows per item
    int lane_row, lane_col, lane_off;  // this lane's place inside an item
    int op;         // operation in flight
    int op_item, op_step, op_local;
    int loads;      // vector loads the last engine step issued
    int anchor;     // tile of bit 0 of `ready`
    uint64_t ready; // ready tiles anchor .. anchor+63
    int cur_item;   // item being summed, -1 if none
    int cur_step;   // its next step
    f32x8 cur;
    int park_n;
    int park_item[kPark];
    f32x8 park[kPark];
    uint32_t epoch;
};

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Wave-uniform base offset of an item in the slice and whether this lane's
// chunk lies inside the (possibly ragged) tile.
__device__ __forceinline__ int64_t item_base(const Engine& e, const Args& a, int item, bool& valid)
{
    const int u = item / e.ipt;
    const int j = item - u * e.ipt;
    const TileCoord t = decode_slot(a.g, u);
    const int row = j * e.rpi;
    valid = row + e.lane_row < tile_rows(a.g, t) && e.lane_col < tile_cols(a.g, t);
    return (int64_t)(t.tml * a.g.bm + row) * a.g.N + t.tn * a.g.bn;
}

__device__ __forceinline__ void engine_init(Engine& e, const Args& a, char* slots, int gw, int waves,
                                            uint32_t epoch)
{
    const int lane = threadIdx.x & 63;
    const int cpr = a.g.bn >> 3;  // 16-byte chunks per tile row (8 .. 32)
    e.slots = slots;
    e.rpi = 64 / cpr;
    e.ipt = a.g.bm / e.rpi;
    e.nitems = a.g.ts * e.ipt;
    e.lane_row = lane / cpr;
    e.lane_col = (lane % cpr) * 8;
    e.lane_off = e.lane_row * a.g.N + e.lane_col;
    e.next = uni(gw);
    e.stride = waves;
    e.op = kOpNone;
    e.op_item = 0;
    e.op_step = 0;
    e.op_local = 0;
    e.loads = 0;
    e.anchor = 0;
    e.ready = 0;
    e.cur_item = -1;
    e.cur_step = 0;
    e.park_n = 0;
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
    int want = e.park_n > 0 ? e.park_item[0] : e.next;
    if (e.cur_item >= 0 && e.cur_item < want) want = e.cur_item;
    if (want > e.nitems) want = e.nitems;
    want /= e.ipt;
    const int sh = want - e.anchor;
    if (sh > 0) {
        e.ready = sh >= 64 ? 0ull : (e.ready >> sh);
        e.anchor = want;
    }
}

__device__ __forceinline__ void store_out(const Engine& e, const Args& a, int item, const f32x8& acc)
{
    bool valid;
    const int64_t base = item_base(e, a, item, valid);
    if (valid) __builtin_nontemporal_store(pack8(acc), reinterpret_cast<u32x4*>(a.out + base + e.lane_off));
}

__device__ __forceinline__ void park_pop(Engine& e)
{
#pragma unroll
    for (int p = 0; p + 1 < kPark; ++p) {
        e.park_item[p] = e.park_item[p + 1];
        e.park[p] = e.park[p + 1];
    }
    --e.park_n;
}

__device__ __forceinline__ u32x4 engine_slot(const Engine& e, int k)
{
    return *reinterpret_cast<const u32x4*>(e.slots + k * kEngineSlotBytes + (threadIdx.x & 63) * 16);
}

// Consume the operation in flight (its loads have completed).
__device__ __forceinline__ void engine_consume(Engine& e, const Args& a)
{
    const int op = e.op;
    if (op == kOpStep) {
        const int s = e.op_step;
        f32x8 acc = e.cur;
        if (s == 0) acc = f32x8{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        acc = add8(acc, engine_slot(e, 0));
        if (s < 3 || e.op_local) acc = add8(acc, engine_slot(e, 1));
        if (s < 3) {
            e.cur = acc;
            e.cur_step = s + 1;
        } else if (e.op_local) {
            store_out(e, a, e.op_item, acc);
            e.cur_item = -1;
        } else {
            // a value select per slot (no indexed store) keeps the parked
            // partials in registers
#pragma unroll
            for (int p = 0; p < kPark; ++p) {
                const bool here = p == e.park_n;
                e.park[p] = here ? acc : e.park[p];
                e.park_item[p] = here ? e.op_item : e.park_item[p];
            }
            ++e.park_n;
            e.cur_item = -1;
        }
    } else if (op == kOpFinish) {
        store_out(e, a, e.park_item[0], add8(e.park[0], engine_slot(e, 1)));
        park_pop(e);
    } else if (op == kOpPoll) {
        const int lane = threadIdx.x & 63;
        const uint32_t f = *reinterpret_cast<const uint32_t*>(e.slots + lane * 4);
        const bool mine = e.anchor + lane < a.g.ts;
        e.ready |= __builtin_amdgcn_ballot_w64(mine && f == e.epoch);
    }
    e.op = kOpNone;
    engine_reanchor(e);
}

// Choose and issue the next operation.  Every lane issues every load (lanes
// without a valid chunk read the slice's first chunk), so the number of
// vector-memory instructions equals e.loads exactly.
__device__ __forceinline__ void engine_issue(Engine& e, const Args& a)
{
    int op = kOpNone, item = 0, step = 0, local = 0;
    if (e.park_n > 0 && tile_ready(e, e.park_item[0] / e.ipt)) {
        op = kOpFinish;
        item = e.park_item[0];
    } else if (e.cur_item >= 0) {
        item = e.cur_item;
        step = e.cur_step;
        if (step < 3) {
            op = kOpStep;
        } else if (tile_ready(e, item / e.ipt)) {
            op = kOpStep;
            local = 1;
        } else {
            op = e.park_n < kPark ? kOpStep : kOpPoll;
        }
    } else if (e.next < e.nitems && (e.park_n < kPark || tile_ready(e, e.next / e.ipt))) {
        op = kOpStep;
        item = e.next;
        e.cur_item = e.next;
        e.cur_step = 0;
        e.next += e.stride;
    } else if (e.park_n > 0 || e.next < e.nitems) {
        op = kOpPoll;
    }
    e.op = op;
    e.op_item = item;
    e.op_step = step;
    e.op_local = local;
    e.loads = 0;
    if (op == kOpStep || op == kOpFinish) {
        bool valid;
        const int64_t base = item_base(e, a, item, valid);
        // lanes outside the (ragged) tile read the slice's first chunk
        const int64_t off = valid ? base + e.lane_off : 0;
        if (op == kOpStep) {
            const int p = 2 * step;
            lds_load16<kAuxNt>(a.peers[p] + off, e.slots);
            e.loads = 1;
            if (step < 3) {
                lds_load16<kAuxNt>(a.peers[p + 1] + off, e.slots + kEngineSlotBytes);
                e.loads = 2;
            }
        }
        if (local || op == kOpFinish) {
            lds_load16<kAuxSc1>(a.dst[a.g.rank] + off, e.slots + kEngineSlotBytes);
            e.loads += 1;
        }
    } else if (op == kOpPoll) {
        const int lane = threadIdx.x & 63;
        const int u = e.anchor + lane < a.g.ts ? e.anchor + lane : 0;
        lds_load_flag(a.flags + (int64_t)decode_slot(a.g, u).flag * a.flag_stride, e.slots);
        e.loads = 1;
    }
    // keep every later memory operation (the stage's direct loads) behind these
    // in issue order: completion is inferred from in-order vmcnt
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ bool engine_busy(const Engine& e)
{
    return e.op != kOpNone || e.cur_item >= 0 || e.park_n > 0 || e.next < e.nitems;
}

// After the last tile: finish the wave's items, waiting for flags.  A tile
// whose flag does not arrive within the watchdog limit is reported and its
// items are skipped; after one timeout the wave waits no more (a later tile
// that is still not flagged is skipped at once), so a drain never waits longer
// than one watchdog period in total.
__device__ __forceinline__ void engine_drain(Engine& e, const Args& a)
{
    uint64_t t0 = wall_clock64();
    int last_anchor = -1;
    uint64_t last_ready = 0;
    bool gave_up = false;
    while (engine_busy(e)) {
        if (e.op == kOpNone) engine_issue(e, a);
        wait_vmcnt<0>();
        const bool polled = e.op == kOpPoll;
        engine_consume(e, a);
        if (!polled) {
            t0 = wall_clock64();
            continue;
        }
        if (e.anchor != last_anchor || e.ready != last_ready) {
            last_anchor = e.anchor;
            last_ready = e.ready;
            t0 = wall_clock64();
            continue;
        }
        __builtin_amdgcn_s_sleep(2);
        if (gave_up || (int64_t)(wall_clock64() - t0) > a.watchdog_ticks) {
            gave_up = true;
            // give up on the oldest pending item's tile
            const int stuck = (e.park_n > 0 ? e.park_item[0] : (e.cur_item >= 0 ? e.cur_item : e.next)) / e.ipt;
            if ((threadIdx.x & 63) == 0 && atomicCAS(&a.state->status[0], 0, kStatusTimeout) == 0)
                atomicExch(&a.state->status[1], decode_slot(a.g, stuck).flag);
#pragma unroll
            for (int p = 0; p < kPark; ++p)
                if (e.park_n > 0 && e.park_item[0] / e.ipt == stuck) park_pop(e);
            if (e.cur_item >= 0 && e.cur_item / e.ipt == stuck) e.cur_item = -1;
            while (e.cur_item < 0 && e.park_n == 0 && e.next < e.nitems && e.next / e.ipt == stuck)
                e.next += e.stride;
            engine_reanchor(e);
            t0 = wall_clock64();
        }
    }
}

// Per-tile hooks run by the K loop right after a stage barrier.
struct StepHooks {
    bool interleave; // run the reduce engine between MFMAs
    int pend_q;      // slot of the previous tile, whose flag is still to be stored
    int pend_flag;
    uint32_t who, epoch;
};

// Extra loads the reduce engine may have in flight inside the stage window.
template <class C>
__device__ __forceinline__ void wait_stage(int extra)
{
    constexpr int B = (C::NS - 2) * C::LPS;
    static_assert(B + 2 <= 63, "vmcnt range");
    switch (extra) {
    case 1: wait_vmcnt<B + 1>(); break;
    case 2: wait_vmcnt<B + 2>(); break;
    default: wait_vmcnt<B>(); break;
    }
}

// The K loop of one tile is split in two so that the next tile's first stages
// can be issued before the current tile's epilogue stores (see compute_role).
// Stage kt lives in buffer kt % NS and NS-1 stages are always in flight
// (stages past the end load zeros), so every step waits for the same count:
// this thread's loads of stage kt are done once at most (NS-2)*LPS newer loads
// (plus the engine's, see below) are outstanding.  The barrier then certifies
// that every thread's loads of stage kt have landed and that every wave has
// finished reading stage kt-1, whose buffer the step refills.
template <class C>
struct TileJob {
    LoadPlan<C> lp;
    int nk;
};

template <class C>
__device__ __forceinline__ void tile_prologue(const Args& a, char* lds, TileJob<C>& job, int row0, int rows,
                                              int n0, int cols)
{
    const int K = a.g.K;
    job.nk = (K + C::BK - 1) / C::BK;
    if (job.nk == 0) return;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, 0, a.x_bytes, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.w, 0, a.w_bytes, kRsrcFlags);
    make_plan<C>(a, job.lp, row0, rows, n0, cols);
#pragma unroll
    for (int s = 0; s < C::NS - 1; ++s) issue_stage<C>(job.lp, rx, rw, lds + s * C::STAGE_BYTES, s * C::BK, K);
}

// Runs the K loop of a tile whose prologue has been issued.  The previous
// tile's epilogue stores were issued after this tile's prologue and before the
// first refill, so they have completed once the refill issued at step 0 has:
// at step NS-1 (or after the loop) its flag is published.
template <class C>
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
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, 0, a.x_bytes, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.w, 0, a.w_bytes, kRsrcFlags);
    constexpr int E = C::NS - 1 > 0 ? C::NS - 1 : 1;  // K steps between engine operations
    for (int kt = 0; kt < nk; ++kt) {
        // engine loads issued inside the stage window (steps kt-NS+2 .. kt-1)
        // may stay in flight: that is the engine step at kt - kt % E if kt % E
        // is not 0 (with NS == 2 the window is empty)
        const int extra = (C::NS > 2 && hk.interleave && kt % E != 0) ? eng.loads : 0;
        wait_stage<C>(extra);
        stage_barrier();
        if (kt == C::NS - 1 && hk.pend_flag >= 0) {
            if (threadIdx.x == 0) publish(a, hk.pend_q, hk.pend_flag, hk.who, hk.epoch);
            hk.pend_flag = -1;
        }
        if (hk.interleave && kt % E == 0) {
            engine_consume(eng, a);
            engine_issue(eng, a);
        }
        const int nxt = kt + C::NS - 1;
        kstep<C>(job.lp, rx, rw, lds + (nxt % C::NS) * C::STAGE_BYTES, nxt * C::BK, K,
                 lds + (kt % C::NS) * C::STAGE_BYTES, st);
    }
    // drain the zero-filling loads past the end (and any engine loads), and
    // let every wave finish reading LDS before the next tile's loads
    // overwrite it; a flag still pending (nk < NS) is published here
    wait_vmcnt<0>();
    stage_barrier();
    if (hk.pend_flag >= 0) {
        if (threadIdx.x == 0) publish(a, hk.pend_q, hk.pend_flag, hk.who, hk.epoch);
        hk.pend_flag = -1;
    }
}

// Every group holds G/8 workgroups; group x has R_x = R/8 + (x < R%8) reducers
// and C_x = G/8 - R_x compute workgroups, so the groups' compute counts add up
// to C = G - R whatever R is.
struct GroupSplit {
    int compute, reducers, base;  // base: first position of the group in a round
};

__device__ __forceinline__ GroupSplit group_split(int grid, int reducers, int grp)
{
    const int gq = grid / kGroups;
    const int rq = reducers / kGroups, rr = reducers % kGroups;
    GroupSplit s;
    s.reducers = rq + (grp < rr ? 1 : 0);
    s.compute = gq - s.reducers;
    s.base = grp * (gq - rq) - (grp < rr ? grp : rr);
    return s;
}

// Compute role of the l-th compute workgroup of group grp.  Round r covers
// slots [r*C, r*C + C); the group's share of a round is its C_x slots, either a
// contiguous block or every 8th slot (strided, used when all C_x are equal).
// A tile's flag is stored after the next tile's first stage wait, which has
// already waited for the tile's stores: publishing costs no extra wait.  With
// no dedicated reducers, the waves also run the reduce engine.
template <class C, bool FUSED>
__device__ __forceinline__ void compute_role(const Args& a, char* lds, int grp, int l, uint32_t epoch, int base)
{
    const int Ctot = a.num_compute;
    const int pos = a.strided ? (l * kGroups + grp) : (base + l);
    const uint32_t who = ((uint32_t)grp << 16) | (uint32_t)l;
    const bool interleave = FUSED && a.num_reducers == 0;
    Engine eng;
    const int wave = uni((int)(threadIdx.x >> 6));
    engine_init(eng, a, lds + C::LDS_BYTES + wave * kEngineSlots * kEngineSlotBytes, pos * C::WAVES + wave,
                Ctot * C::WAVES, epoch);
    StepHooks hk;
    hk.interleave = interleave;
    hk.pend_q = -1;
    hk.pend_flag = -1;
    hk.who = who;
    hk.epoch = epoch;
    TileState<C> st;
    TileJob<C> job;
    int q = pos;
    TileCoord t;
    if (q < a.g.tiles) {
        t = decode_slot(a.g, q);
        tile_prologue<C>(a, lds, job, tile_row0(a.g, t), tile_rows(a.g, t), t.tn * C::BN, tile_cols(a.g, t));
    }
    while (q < a.g.tiles) {
        tile_kloop<C>(a, lds, st, job, hk, eng);
        // issue the next tile's first stages before this tile's stores
        const int qn = q + Ctot;
        TileCoord tn = t;
        if (qn < a.g.tiles) {
            tn = decode_slot(a.g, qn);
            tile_prologue<C>(a, lds, job, tile_row0(a.g, tn), tile_rows(a.g, tn), tn.tn * C::BN,
                             tile_cols(a.g, tn));
        }
        uint16_t* dst = a.dst[t.d] + (int64_t)t.tml * C::BM * a.g.N;
        store_tile<C, FUSED>(a, st, dst, tile_rows(a.g, t), t.tn * C::BN, tile_cols(a.g, t));
        if (FUSED) {
            hk.pend_q = q;
            hk.pend_flag = t.flag;
        }
        q = qn;
        t = tn;
    }
    if (hk.pend_flag >= 0) {
        wait_vmcnt<0>();
        stage_barrier();
        if (threadIdx.x == 0) publish(a, hk.pend_q, hk.pend_flag, who, epoch);
    }
    if (interleave) engine_drain(eng, a);
}

// Dedicated reducer role (used when reducers are requested): claim own-slice
// tiles in schedule order, wait for each tile's flag (thread 0 polls with
// device-scope loads and short sleeps, bounded by the watchdog), then sum the
// tile, reading the local slice at device scope.
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
                const uint32_t* f = a.flags + (int64_t)t.flag * a.flag_stride;
                if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
                    const uint64_t t0 = wall_clock64();
                    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
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
            __builtin_nontemporal_store(pack8(acc), reinterpret_cast<u32x4*>(a.out + off));
        }
    }
}

// Role dispatch and end-of-launch bookkeeping.
template <class C, bool FUSED>
__device__ __forceinline__ void fused_body(const Args& a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ uint32_t s_ticket, s_epoch;
    const int grp = blockIdx.x % kGroups;
    if (threadIdx.x == 0) {
        s_ticket = atomicAdd(&a.state->role[grp], 1u);
        s_epoch = __hip_atomic_load(&a.state->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const uint32_t ticket = s_ticket;
    const uint32_t epoch = s_epoch + 1u;  // value this run's flags carry
    const GroupSplit split = group_split((int)gridDim.x, a.num_reducers, grp);
    if (ticket < (uint32_t)split.compute)
        compute_role<C, FUSED>(a, lds, grp, (int)ticket, epoch, split.base);
    else if (FUSED && ticket - (uint32_t)split.compute < (uint32_t)split.reducers)
        reducer_role(a, epoch);

    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t finished = atomicAdd(&a.state->done, 1u);
        if (finished == gridDim.x - 1) {
            // every other workgroup has finished: reset for the next launch
            for (int i = 0; i < kGroups; ++i) __hip_atomic_store(&a.state->role[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.state->unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.state->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (FUSED) __hip_atomic_store(&a.state->epoch, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Tiles that fit two workgroups per CU keep two waves per SIMD resident.
template <class C, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fused_kernel(Args a)
{
    fused_body<C, FUSED>(a);
}

// Eight-wave workgroups (one per CU): two waves per SIMD, so one wave's
// MFMAs run while its sibling waits on LDS, a barrier or the reduce engine.
template <class C, bool FUSED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fused_kernel_8w(Args a)
{
    fused_body<C, FUSED>(a);
}

// Large tiles run one workgroup (one wave per SIMD) per CU: let the compiler
// use the whole register file for latency hiding.
template <class C, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fused_kernel_1w(Args a)
{
    fused_body<C, FUSED>(a);
}

// Standalone slice sum: every workgroup reduces, no flags, grid-stride over the
// whole [S][N] slice.
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(Args a)
{
    sum_block(a, 0, a.g.S, 0, a.g.N, blockIdx.x * kReduceThreads + threadIdx.x, gridDim.x * kReduceThreads);
}

}  // namespace gemm_rs
