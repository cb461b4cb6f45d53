// kernels.hpp -- gfx950 device code of the fused BF16 GEMM + reduce-scatter.
//
// One persistent kernel holds two workgroup roles, in the spirit of mKernel's
// compute / communication roles ("mKernel: Fast Multi-GPU, Multi-Node Fused
// Kernels", sections 3 and 3.2) and of FLUX's reduce-scatter epilogue (TL;DR of
// "FLUX: Fast Software-based Communication Overlap On GPUs Through Kernel
// Fusion"):
//   compute   GEMM tiles on bf16 MFMA (FP32 accumulators), A/B tiles staged
//             through double-buffered LDS; the epilogue rounds the tile to BF16,
//             stores it into its destination slice buffer and releases the
//             tile's ready flag (agent scope);
//   reducer   waits (acquire) for the ready flags of this rank's own slice, in
//             schedule order, and sums each tile with the tp-1 peer partials.
// Roles come from an arrival ticket, so every compute workgroup is resident
// before any reducer starts to wait: reducers can never starve the producers
// they wait for, whatever the grid size.
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

constexpr int kThreads = 256;  // 4 wave64 per workgroup
constexpr int kPeers = 7;      // tp - 1 with tp = 8

constexpr int kStatusTimeout = -6;  // GEMM_RS_ERR_TIMEOUT

struct Args {
    const uint16_t* x;       // [M][K]
    const uint16_t* w;       // [N][K]
    uint16_t* dst[8];        // destination slice buffers by destination rank
    const uint16_t* peers[kPeers];
    uint16_t* out;           // [S][N]
    uint32_t* flags;         // ready flags, flag_stride words apart
    uint32_t* ticket;        // arrival counter
    int32_t* status;         // [0] error code, [1] flag index that timed out
    uint32_t* trace;         // 4 words per slot (debug)
    Geometry g;
    int64_t watchdog_ticks;  // 100 MHz ticks
    uint32_t epoch;
    uint32_t ticket_base;
    int32_t num_compute;
    int32_t num_reducers;
    int32_t flag_stride;
    int32_t flags_on;
    int32_t protocol;        // 0 = per-wave fence, 1 = single release store
    int32_t drop_flag;
    int32_t trace_on;
};

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int MF_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 64;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
    static constexpr int MF = MF_;                   // MFMA output edge
    static constexpr int KF = MF_ == 32 ? 16 : 32;   // k per MFMA
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / MF, FN = WTN / MF;
    static_assert(FM >= 1 && FN >= 1 && WTM % MF == 0 && WTN % MF == 0, "wave tile");
    static constexpr int LDS_ROW = BK + 8;           // padded row, elements
    static constexpr int STAGE = (BM + BN) * LDS_ROW;
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static constexpr int CHUNKS_PER_ROW = BK / 8;    // 16-byte chunks
    static constexpr int A_CHUNKS = BM * CHUNKS_PER_ROW;
    static constexpr int B_CHUNKS = BN * CHUNKS_PER_ROW;
    static constexpr int A_PER_T = (A_CHUNKS + kThreads - 1) / kThreads;
    static constexpr int B_PER_T = (B_CHUNKS + kThreads - 1) / kThreads;
};

template <int MF> struct AccT;
template <> struct AccT<32> { typedef f32x16 type; static constexpr int N = 16; };
template <> struct AccT<16> { typedef f32x4 type; static constexpr int N = 4; };

__device__ inline float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Two FP32 values to two BF16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// ---------------------------------------------------------------- GEMM tile

template <class C>
struct TileState {
    typename AccT<C::MF>::type acc[C::FM][C::FN];
    uint4 ra[C::A_PER_T];
    uint4 rb[C::B_PER_T];
};

// Global -> registers for one BK slice of the A (X rows) and B (W rows) tiles.
// Rows past the tile's valid extent and k past K read as zero.
template <class C>
__device__ inline void load_ab(const Args& a, TileState<C>& st, int row0, int rows, int n0,
                               int cols, int k0)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        const int c = tid + i * kThreads;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (C::A_CHUNKS % kThreads == 0 || c < C::A_CHUNKS) {
            const int r = c / C::CHUNKS_PER_ROW;
            const int k = k0 + (c % C::CHUNKS_PER_ROW) * 8;
            if (r < rows && k < a.g.K)
                v = *reinterpret_cast<const uint4*>(a.x + (int64_t)(row0 + r) * a.g.K + k);
        }
        st.ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
        const int c = tid + i * kThreads;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (C::B_CHUNKS % kThreads == 0 || c < C::B_CHUNKS) {
            const int r = c / C::CHUNKS_PER_ROW;
            const int k = k0 + (c % C::CHUNKS_PER_ROW) * 8;
            if (r < cols && k < a.g.K)
                v = *reinterpret_cast<const uint4*>(a.w + (int64_t)(n0 + r) * a.g.K + k);
        }
        st.rb[i] = v;
    }
}

template <class C>
__device__ inline void store_ab(uint16_t* stage, const TileState<C>& st)
{
    const int tid = threadIdx.x;
    uint16_t* sa = stage;
    uint16_t* sb = stage + C::BM * C::LDS_ROW;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        const int c = tid + i * kThreads;
        if (C::A_CHUNKS % kThreads == 0 || c < C::A_CHUNKS) {
            const int r = c / C::CHUNKS_PER_ROW, kc = c % C::CHUNKS_PER_ROW;
            *reinterpret_cast<uint4*>(sa + r * C::LDS_ROW + kc * 8) = st.ra[i];
        }
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
        const int c = tid + i * kThreads;
        if (C::B_CHUNKS % kThreads == 0 || c < C::B_CHUNKS) {
            const int r = c / C::CHUNKS_PER_ROW, kc = c % C::CHUNKS_PER_ROW;
            *reinterpret_cast<uint4*>(sb + r * C::LDS_ROW + kc * 8) = st.rb[i];
        }
    }
}

// MFMA over one LDS stage.  The W fragment is the MFMA's A operand and the X
// fragment its B operand, so the accumulator holds the transposed tile:
// lane l owns output row m = l % MF and, per group of four registers, four
// consecutive output columns -- one 8-byte store per group in the epilogue.
template <class C>
__device__ inline void mma_stage(const uint16_t* stage, TileState<C>& st)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const uint16_t* sa = stage;
    const uint16_t* sb = stage + C::BM * C::LDS_ROW;
    const int lr = lane % C::MF;          // fragment row
    const int lk = (lane / C::MF) * 8;    // fragment k offset
#pragma unroll
    for (int kk = 0; kk < C::BK; kk += C::KF) {
        bf16x8 xf[C::FM], wf[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
            xf[i] = *reinterpret_cast<const bf16x8*>(sa + (wm * C::WTM + i * C::MF + lr) * C::LDS_ROW + kk + lk);
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            wf[j] = *reinterpret_cast<const bf16x8*>(sb + (wn * C::WTN + j * C::MF + lr) * C::LDS_ROW + kk + lk);
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
}

// Full K loop of one tile: prologue load, then per BK step prefetch the next
// slice into registers while the MFMAs consume the current LDS stage.
template <class C>
__device__ inline void gemm_tile(const Args& a, uint16_t* smem, TileState<C>& st, int row0,
                                 int rows, int n0, int cols)
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int e = 0; e < AccT<C::MF>::N; ++e) st.acc[i][j][e] = 0.0f;

    const int nk = (a.g.K + C::BK - 1) / C::BK;
    if (nk == 0) return;
    load_ab<C>(a, st, row0, rows, n0, cols, 0);
    store_ab<C>(smem, st);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        uint16_t* cur = smem + (kt & 1) * C::STAGE;
        uint16_t* nxt = smem + ((kt + 1) & 1) * C::STAGE;
        const bool more = kt + 1 < nk;
        if (more) load_ab<C>(a, st, row0, rows, n0, cols, (kt + 1) * C::BK);
        mma_stage<C>(cur, st);
        if (more) store_ab<C>(nxt, st);
        __syncthreads();
    }
}

// Round the accumulators to BF16 and store the valid part of the tile at
// dst[(tile row) ...][n0 ...] (dst already points at the tile's first row).
template <class C>
__device__ inline void store_tile(const Args& a, const TileState<C>& st, uint16_t* dst, int rows,
                                  int n0, int cols)
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
            if constexpr (C::MF == 32) {
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    const int n = wn * C::WTN + j * 32 + grp * 8 + (lane / 32) * 4;
                    if (n < cols) {
                        uint2 v;
                        v.x = pack_bf16x2(st.acc[i][j][grp * 4 + 0], st.acc[i][j][grp * 4 + 1]);
                        v.y = pack_bf16x2(st.acc[i][j][grp * 4 + 2], st.acc[i][j][grp * 4 + 3]);
                        *reinterpret_cast<uint2*>(drow + n) = v;
                    }
                }
            } else {
                const int n = wn * C::WTN + j * 16 + (lane / 16) * 4;
                if (n < cols) {
                    uint2 v;
                    v.x = pack_bf16x2(st.acc[i][j][0], st.acc[i][j][1]);
                    v.y = pack_bf16x2(st.acc[i][j][2], st.acc[i][j][3]);
                    *reinterpret_cast<uint2*>(drow + n) = v;
                }
            }
        }
    }
}

// Publish a finished tile: all of its stores become visible at agent scope
// before the flag does.
__device__ inline void release_flag(const Args& a, int q, const TileCoord& t, uint32_t ticket)
{
    if (a.protocol == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0 && a.flags_on) {
        if (a.trace_on) {
            const uint64_t now = wall_clock64();
            uint32_t* tr = a.trace + (int64_t)q * 4;
            tr[0] = (uint32_t)t.flag;
            tr[1] = ticket;
            tr[2] = (uint32_t)now;
            tr[3] = (uint32_t)(now >> 32);
        }
        if (t.flag != a.drop_flag) {
            uint32_t* f = a.flags + (int64_t)t.flag * a.flag_stride;
            if (a.protocol == 0)
                __hip_atomic_store(f, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                __hip_atomic_store(f, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <class C>
__device__ void compute_role(const Args& a, uint16_t* smem, uint32_t ticket)
{
    TileState<C> st;
    for (int q = (int)ticket; q < a.g.tiles; q += a.num_compute) {
        const TileCoord t = decode_slot(a.g, q);
        const int rows = tile_rows(a.g, t), cols = tile_cols(a.g, t);
        const int row0 = tile_row0(a.g, t);
        const int n0 = t.tn * C::BN;
        gemm_tile<C>(a, smem, st, row0, rows, n0, cols);
        uint16_t* dst = a.dst[t.d] + (int64_t)t.tml * C::BM * a.g.N;
        store_tile<C>(a, st, dst, rows, n0, cols);
        release_flag(a, q, t, ticket);
    }
}

// ---------------------------------------------------------------- slice sum

__device__ inline void add8(float (&acc)[8], const uint4& v)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] = acc[2 * i] + bf16_bits_to_f32(w[i] & 0xFFFFu);
        acc[2 * i + 1] = acc[2 * i + 1] + bf16_bits_to_f32(w[i] >> 16);
    }
}

// out = RNE( (((0 + peer_0) + ... + peer_6) + local ) for 8 elements at `off`.
__device__ inline void sum_chunk(const Args& a, const uint16_t* local, int64_t off)
{
    uint4 v[kPeers + 1];
#pragma unroll
    for (int s = 0; s < kPeers; ++s) v[s] = *reinterpret_cast<const uint4*>(a.peers[s] + off);
    v[kPeers] = *reinterpret_cast<const uint4*>(local + off);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int s = 0; s <= kPeers; ++s) add8(acc, v[s]);
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(a.out + off) = o;
}

// Sum a rows x cols block of the slice starting at (row0, col0), 16-byte
// chunks distributed over `nthreads` threads starting at `tid`.
__device__ inline void sum_block(const Args& a, int row0, int rows, int col0, int cols, int tid,
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

// Reducer role: own-slice tiles in schedule order (slots 0 .. ts-1), strided
// over the reducer workgroups.  Thread 0 polls the flag (relaxed loads, short
// sleeps, a wall-clock limit); after the barrier every wave takes an agent-
// scope acquire fence before reading the tile.
template <class C>
__device__ void reducer_role(const Args& a, int rid)
{
    __shared__ int s_abort;
    for (int u = rid; u < a.g.ts; u += a.num_reducers) {
        const TileCoord t = decode_slot(a.g, u);
        if (threadIdx.x == 0) {
            const uint32_t* f = a.flags + (int64_t)t.flag * a.flag_stride;
            int abort_now = 0;
            if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.epoch) {
                const uint64_t t0 = wall_clock64();
                while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.epoch) {
                    __builtin_amdgcn_s_sleep(2);
                    if ((int64_t)(wall_clock64() - t0) > a.watchdog_ticks) {
                        abort_now = 1;
                        break;
                    }
                }
            }
            if (abort_now) {
                if (atomicCAS(a.status, 0, kStatusTimeout) == 0) atomicExch(a.status + 1, t.flag);
            }
            s_abort = abort_now;
        }
        __syncthreads();
        const int abort_now = s_abort;
        if (abort_now) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        sum_block(a, t.tml * a.g.bm, tile_rows(a.g, t), t.tn * a.g.bn, tile_cols(a.g, t),
                  threadIdx.x, kThreads);
        __syncthreads();  // s_abort is rewritten for the next unit
    }
}

template <class C>
__global__ __launch_bounds__(kThreads) void fused_kernel(Args a)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    __shared__ uint32_t s_ticket;
    if (threadIdx.x == 0) s_ticket = atomicAdd(a.ticket, 1u) - a.ticket_base;
    __syncthreads();
    const uint32_t ticket = s_ticket;
    if (ticket < (uint32_t)a.num_compute)
        compute_role<C>(a, smem, ticket);
    else if (ticket - (uint32_t)a.num_compute < (uint32_t)a.num_reducers)
        reducer_role<C>(a, (int)(ticket - (uint32_t)a.num_compute));
}

// Standalone slice sum: every workgroup reduces, no flags, grid-stride over the
// whole [S][N] slice.
__global__ __launch_bounds__(kThreads) void reduce_kernel(Args a)
{
    sum_block(a, 0, a.g.S, 0, a.g.N, blockIdx.x * kThreads + threadIdx.x, gridDim.x * kThreads);
}

}  // namespace gemm_rs
