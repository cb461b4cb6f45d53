/*
 * oracle.c -- plain CPU oracle for one rank's share of a tensor-parallel
 * row-parallel linear layer: a BF16 GEMM with FP32 accumulation whose output
 * rows are split into tp row slices, one per rank, followed by the sum of this
 * rank's slice over all tp partial products (a reduce-scatter).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's
 * cpu_baseline leg do.  It shares no code, header, table or constant with the
 * HIP implementation.
 *
 * Sources (the pages' text):
 *   - problem page "A fused GEMM + reduce-scatter kernel hiding 90% of
 *     communication on 8 H100 GPUs", sections "What is asked" (each GPU
 *     computes a partial product, the partials are summed across GPUs and each
 *     GPU keeps one slice of the total) and "How it gets verified" (row-
 *     parallel linear, GEMM then reduce-scatter, BF16 inputs, FP32
 *     accumulation, tensor-parallel degree 8);
 *   - FLUX summary "FLUX: Fast Software-based Communication Overlap On GPUs
 *     Through Kernel Fusion", TL;DR (reduce-scatter fused as a GEMM epilogue,
 *     tile coordinate swizzling).
 *
 * Where the pages are silent the oracle fixes one plain reading:
 *   - slices are contiguous blocks of S = M/tp rows; slice d belongs to rank d;
 *   - every partial (peers' and this rank's own) is handed over as BF16,
 *     rounded to nearest-even from its FP32 accumulator;
 *   - the slice sum is FP32, starting from +0.0, adding the tp-1 received
 *     partials in ascending peer-rank order and this rank's own partial last,
 *     with a single round-to-nearest-even to BF16 at the end;
 *   - the GEMM accumulates each output element in FP32 with k ascending.
 *
 * Layouts (row-major, BF16 passed as raw uint16 bit patterns):
 *   X [M][K]   this rank's activations X_r
 *   W [N][K]   this rank's weight shard W_r, K contiguous (the product is
 *              X_r * W_r with W_r read as its K x N transpose)
 *   peers[i], send[i], local, out: [S][N]
 *   peer slot i belongs to peer rank p_i = i for i < rank, i + 1 otherwise.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/* ---- BF16 codec ------------------------------------------------------- */

/* A BF16 value is the upper half of the FP32 bit pattern. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* IEEE-754 round-to-nearest, ties-to-even, of an FP32 value to BF16: add
 * half an ulp of the result (0x7FFF) plus the result's lowest kept bit, then
 * truncate.  A carry out of the mantissa moves into the exponent, so values
 * above the largest finite BF16 round to infinity.  NaNs stay NaN (quiet bit
 * forced, sign and upper payload kept). */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + keep_lsb) >> 16);
}

void oracle_f32_to_bf16_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(in[i]);
}

void oracle_bf16_to_f32_array(const uint16_t *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_f32(in[i]);
}

/* ---- GEMM with FP32 accumulation -------------------------------------- */

/* P[ii][j] = sum_{k=0}^{K-1} X[i][k] * W[j][k] for i = rows[ii] (or i = ii
 * when rows is NULL), accumulated in FP32 with k ascending.  A product of two
 * BF16 values has at most 16 significant bits, so it is exact in FP32 and the
 * only rounding is the one in each addition.  Output rows are independent and
 * are shared among threads; the arithmetic of one element is unchanged. */
int oracle_gemm_f32acc(int64_t nrows, const int64_t *rows, int64_t N, int64_t K,
                       const uint16_t *X, const uint16_t *W, float *P)
{
    if (nrows < 0 || N < 0 || K < 0) return ORACLE_EINVAL;
    if (nrows == 0 || N == 0) return ORACLE_OK;
    float *wt = (float *)malloc((size_t)(K > 0 ? K : 1) * (size_t)N * sizeof(float));
    if (!wt) return ORACLE_ENOMEM;
    /* wt[k][j] = W[j][k]: W read as the K x N operand. */
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k)
            wt[k * N + j] = oracle_bf16_to_f32(W[j * K + k]);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ii = 0; ii < nrows; ++ii) {
        int64_t i = rows ? rows[ii] : ii;
        float *p = P + ii * N;
        for (int64_t j = 0; j < N; ++j)
            p[j] = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = oracle_bf16_to_f32(X[i * K + k]);
            const float *wk = wt + k * N;
            for (int64_t j = 0; j < N; ++j)
                p[j] = p[j] + a * wk[j];
        }
    }
    free(wt);
    return ORACLE_OK;
}

/* ---- routing and the slice sum ---------------------------------------- */

/* Peer slot i (0..tp-2) holds the partial of peer rank p_i. */
static int peer_rank_of_slot(int rank, int slot)
{
    return slot < rank ? slot : slot + 1;
}

int oracle_peer_rank(int32_t rank, int32_t slot)
{
    return peer_rank_of_slot(rank, slot);
}

/* out[i][j] = RNE_bf16( (((0 + peer_0) + peer_1) + ... + peer_{tp-2}) + local ),
 * FP32 additions in that order (received partials in ascending peer rank,
 * this rank's own partial last).  rows/nrows select slice rows (NULL = all S). */
int oracle_slice_sum(int64_t nrows, const int64_t *rows, int64_t N, int32_t tp,
                     const uint16_t *local, const uint16_t *const *peers, uint16_t *out)
{
    if (nrows < 0 || N < 0 || tp < 1) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t ii = 0; ii < nrows; ++ii) {
        int64_t i = rows ? rows[ii] : ii;
        for (int64_t j = 0; j < N; ++j) {
            float acc = 0.0f;
            for (int s = 0; s < tp - 1; ++s)
                acc = acc + oracle_bf16_to_f32(peers[s][i * N + j]);
            acc = acc + oracle_bf16_to_f32(local[i * N + j]);
            out[ii * N + j] = oracle_f32_to_bf16(acc);
        }
    }
    return ORACLE_OK;
}

/* The whole path for one rank: P = X * W (FP32 accumulation), partial rounded
 * to BF16, rows [d*S, (d+1)*S) routed to destination d (send slot i for peer
 * rank p_i, `local` for d == rank), then the slice sum into `out`.
 * send may be NULL (routing not returned); each send[i] may be NULL too. */
int oracle_gemm_rs(int64_t M, int64_t N, int64_t K, int32_t tp, int32_t rank,
                   const uint16_t *X, const uint16_t *W,
                   const uint16_t *const *peers, uint16_t *const *send,
                   uint16_t *local, uint16_t *out)
{
    if (M < 0 || N < 0 || K < 0 || tp < 1 || rank < 0 || rank >= tp) return ORACLE_EINVAL;
    if (M % tp != 0) return ORACLE_EINVAL;
    const int64_t S = M / tp;
    float *P = (float *)malloc((size_t)(S > 0 ? S : 1) * (size_t)(N > 0 ? N : 1) * sizeof(float));
    int64_t *rows = (int64_t *)malloc((size_t)(S > 0 ? S : 1) * sizeof(int64_t));
    if (!P || !rows) { free(P); free(rows); return ORACLE_ENOMEM; }

    int rc = ORACLE_OK;
    for (int d = 0; d < tp && rc == ORACLE_OK; ++d) {
        uint16_t *dst;
        if (d == rank) {
            dst = local;
        } else {
            int slot = d < rank ? d : d - 1;
            dst = send ? send[slot] : NULL;
        }
        if (!dst) continue;
        for (int64_t i = 0; i < S; ++i) rows[i] = (int64_t)d * S + i;
        rc = oracle_gemm_f32acc(S, rows, N, K, X, W, P);
        if (rc == ORACLE_OK) oracle_f32_to_bf16_array(P, dst, S * N);
    }
    if (rc == ORACLE_OK && out)
        rc = oracle_slice_sum(S, NULL, N, tp, local, peers, out);
    free(P);
    free(rows);
    return rc;
}

/* ---- high-precision reference for the error statistics ----------------- */

/* ref[ii][j] = sum_s peer_s[i][j] + sum_k X[rank*S + i][k] * W[j][k], in
 * FP64 with no BF16 rounding of the local partial (the exact value of the
 * unrounded computation up to FP64 rounding).  peers may be NULL (then only
 * the local partial).  rows selects slice rows (NULL = all S). */
int oracle_ref_f64(int64_t nrows, const int64_t *rows, int64_t M, int64_t N, int64_t K,
                   int32_t tp, int32_t rank, const uint16_t *X, const uint16_t *W,
                   const uint16_t *const *peers, double *ref)
{
    if (M < 0 || N < 0 || K < 0 || tp < 1 || rank < 0 || rank >= tp || M % tp) return ORACLE_EINVAL;
    const int64_t S = M / tp;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ii = 0; ii < nrows; ++ii) {
        int64_t i = rows ? rows[ii] : ii;
        int64_t xi = (int64_t)rank * S + i;
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)oracle_bf16_to_f32(X[xi * K + k]) *
                       (double)oracle_bf16_to_f32(W[j * K + k]);
            if (peers)
                for (int s = 0; s < tp - 1; ++s)
                    acc += (double)oracle_bf16_to_f32(peers[s][i * N + j]);
            ref[ii * N + j] = acc;
        }
    }
    return ORACLE_OK;
}

/* ---- tile schedule ------------------------------------------------------ */

/* The pages name tile-coordinate swizzling (FLUX TL;DR) without details.  The
 * schedule fixed here: the output is cut into BM x BN tiles that never cross a
 * slice boundary; a slice has TMs = ceil(S/BM) tile rows and TN = ceil(N/BN)
 * tile columns, the last of each possibly partial; slot q of the T = tp*TMs*TN
 * slots visits destination slices in the order rank, rank+1, ... (mod tp), so
 * this rank's own slice comes first and every rank targets a different
 * destination at each step; within a slice, tiles are visited in groups of
 * group_m tile-rows, column-major inside a group (a grouped raster).
 *
 * For each slot q the arrays receive: d (destination slice), tm (global tile
 * row, in units of BM rows of the M x N product), tn (tile column) and flag
 * (index of the tile's ready flag, d*T_s + tm_local*TN + tn).  Any output
 * array may be NULL. */
int oracle_schedule(int64_t M, int64_t N, int32_t tp, int32_t rank, int32_t bm, int32_t bn,
                    int32_t group_m, int32_t *slot_d, int32_t *slot_tm, int32_t *slot_tn,
                    int32_t *slot_flag)
{
    if (M <= 0 || N <= 0 || tp < 1 || rank < 0 || rank >= tp || bm <= 0 || bn <= 0 || group_m <= 0)
        return ORACLE_EINVAL;
    if (M % tp) return ORACLE_EINVAL;
    const int64_t S = M / tp;
    if (S == 0) return ORACLE_EINVAL;
    const int64_t tms = (S + bm - 1) / bm, tn_count = (N + bn - 1) / bn, ts = tms * tn_count;
    const int64_t total = (int64_t)tp * ts;
    for (int64_t q = 0; q < total; ++q) {
        int64_t step = q / ts;
        int64_t d = (rank + step) % tp;
        int64_t w = q % ts;
        int64_t group = w / ((int64_t)group_m * tn_count);
        int64_t rows_in_group = tms - group * group_m;
        if (rows_in_group > group_m) rows_in_group = group_m;
        int64_t v = w % ((int64_t)group_m * tn_count);
        int64_t tm_local = group * group_m + v % rows_in_group;
        int64_t tn = v / rows_in_group;
        if (slot_d) slot_d[q] = (int32_t)d;
        if (slot_tm) slot_tm[q] = (int32_t)(d * tms + tm_local);
        if (slot_tn) slot_tn[q] = (int32_t)tn;
        if (slot_flag) slot_flag[q] = (int32_t)(d * ts + tm_local * tn_count + tn);
    }
    return ORACLE_OK;
}
