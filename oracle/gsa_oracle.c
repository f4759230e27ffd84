/*
 * gsa_oracle.c -- CPU oracle for one rank's fused GEMV + one-shot AllReduce.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite, the
 * package smoke check and the benchmark's CPU-baseline leg load this library.
 * It shares no source, header, constant or helper with the HIP library; the
 * two meet only at the seeded inputs.
 *
 * Plain, slow and meant to be checked by eye: fp64 accumulation, ascending
 * loop order, no blocking, no threads, no vector tricks.
 *
 * What it computes (the sources it follows):
 *  - "Overlapping Collective Communication with Dependent Computation ...
 *    using GPU-Initiated Intra-Kernel Networking" (summary of Punniyamurthy
 *    et al., "Optimizing Distributed ML Communication with Fused
 *    Computation-Collective Operations"), Abstract: the fused GEMV + AllReduce
 *    operator for Transformers.  One rank computes its partial product and the
 *    partials of all ranks are summed.
 *  - "Bay.Area.AI: Tensor and 2D Parallelism" talk, Megatron-style MLP
 *    segment: a column-wise shard followed by a row-wise shard needs no
 *    collective in between and one all-reduce at the end.  So rank r holds
 *    the input-dimension slice A_r (N x K/W) of the weight and the matching
 *    slice x_r of the activation, and its partial is y_r = A_r x_r.
 *  - "PyTorch Symmetric Memory" documentation, section on writing your own
 *    kernel (the Triton one_shot_all_reduce_kernel): the accumulator starts
 *    at zero and the loop visits every rank's buffer in rank order 0..W-1,
 *    the local one included.  The "PyTorch Symmetric Memory" talk says the
 *    same (inner loop over all ranks, local or remote alike).
 *  - "PyTorch Symmetric Memory" documentation, section on higher-precision
 *    reduction: bf16 inputs are accumulated in fp32.  The oracle goes further
 *    and accumulates in fp64, so it is the exact value up to fp64 rounding.
 *
 *  - "PyTorch Symmetric Memory" talk, the real-model example near its end:
 *    the all-reduce is followed by a bias addition (elementwise, so it joins
 *    the reduction loop) and an RMSNorm, all in one kernel.  The pages do not
 *    write RMSNorm out; gsa_oracle_bias_rmsnorm uses its textbook definition
 *    over the hidden dimension (the N output rows of one token).
 *  - "PyTorch Symmetric Memory" documentation, op reference of
 *    two_shot_all_reduce_ (a two-stage all-reduce; the talk mentions a
 *    two-shot version too): read as reduce-scatter then all-gather.  Rank p
 *    owns one tile-aligned chunk of the rows, sums it over all ranks in rank
 *    order from zero (the one-shot rule) and publishes it; every rank copies
 *    the other chunks from their owners (gsa_oracle_two_shot).
 *  - "PyTorch Symmetric Memory" documentation, higher-precision reduction:
 *    accumulate in fp32, hand the result back in the input precision (bf16),
 *    which gsa_oracle_scale_f32 rounds to nearest, ties to even.  The same
 *    section read for the all-reduce itself: bf16 partials in the slots are
 *    widened and summed in fp32 (gsa_oracle_fold_bf16), and the sum is
 *    handed back in bf16 (gsa_oracle_f32_to_bf16).
 *
 *  - "Overlapping Collective Communication ..." (the fused-operators page),
 *    Abstract: a third fused operator, GEMM + All-to-All for mixture-of-
 *    experts models.  "PyTorch Symmetric Memory" documentation, op reference
 *    of all_to_all_vdev_2d and all_to_all_vdev_2d_offset: the dispatch
 *    shuffle lays tokens out expert-major (each local expert's segments from
 *    source ranks 0..W-1), with splits and offsets given on the device; the
 *    combine is its inverse, sending every segment back to its source rank
 *    at an offset that rank chose.  gsa_oracle_moe_combine computes each
 *    local expert's product of its dispatched rows with its weight and
 *    places every result row where the combine puts it.
 *
 * Layouts (plain readings, the pages fix none): A_r is N x Ks row-major,
 * x is B x Ks row-major (one token's activation slice is contiguous),
 * slots are W x N x B with element (n, b) of rank r at r*N*B + n*B + b,
 * outputs are N x B.  bf16 values arrive as their 16 raw bits.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

/* A bf16 value is the upper half of an fp32 word: widening is exact. */
static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/*
 * y64[n*B+b]   = sum_k A_r[n][k] * x[b][k]          (fp64, ascending k)
 * abs64[n*B+b] = sum_k |A_r[n][k] * x[b][k]|        (for the error bound)
 * Returns 0, or -1 on a bad size.
 */
int gsa_oracle_gemv(const uint16_t *A_r, const uint16_t *x,
                    int64_t N, int64_t Ks, int B,
                    double *y64, double *abs64)
{
    if (N < 0 || Ks < 0 || B < 1)
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        for (int b = 0; b < B; ++b) {
            double sum = 0.0;
            double sum_abs = 0.0;
            for (int64_t k = 0; k < Ks; ++k) {
                double a = bf16_bits_to_double(A_r[n * Ks + k]);
                double v = bf16_bits_to_double(x[(int64_t)b * Ks + k]);
                double p = a * v;
                sum += p;
                sum_abs += fabs(p);
            }
            y64[n * B + b] = sum;
            abs64[n * B + b] = sum_abs;
        }
    }
    return 0;
}

/*
 * The whole call of rank `rank`: its partial y_r, then the one-shot sum
 *   out64[i] = sum_{r=0..W-1} (r == rank ? y64[i] : slots[r][i])
 * in ascending r, starting from 0.  Slot `rank` of the input is ignored: it
 * is what the call itself publishes.
 */
int gsa_oracle_gemv_allreduce(const uint16_t *A_r, const uint16_t *x,
                              const float *slots, int W, int rank,
                              int64_t N, int64_t Ks, int B,
                              double *y64, double *abs64, double *out64)
{
    if (W < 1 || rank < 0 || rank >= W)
        return -1;
    if (gsa_oracle_gemv(A_r, x, N, Ks, B, y64, abs64) != 0)
        return -1;
    int64_t NB = N * (int64_t)B;
    for (int64_t i = 0; i < NB; ++i) {
        double acc = 0.0;
        for (int r = 0; r < W; ++r) {
            double term = (r == rank) ? y64[i] : (double)slots[(int64_t)r * NB + i];
            acc += term;
        }
        out64[i] = acc;
    }
    return 0;
}

/*
 * The one-shot sum as fp32 arithmetic over given slots, in the pages' order:
 *   acc = +0.0f; for r = 0..W-1: acc = fl32(acc + slots[r][i]); out[i] = acc
 * Given the fp32 partials a GPU published, this result is unique, so it is
 * the bit-exact reference for the reduction step.
 */
void gsa_oracle_fold_f32(const float *slots, int W, int64_t NB, float *out)
{
    for (int64_t i = 0; i < NB; ++i) {
        float acc = 0.0f;
        for (int r = 0; r < W; ++r)
            acc = acc + slots[(int64_t)r * NB + i];
        out[i] = acc;
    }
}

/*
 * The fused epilogue: bias, then RMSNorm over n, for every token column b.
 *   z[n][b]   = fl32(out[n][b] + bias[n])                (bias NULL: 0)
 *   inv64[b]  = 1 / sqrt((sum_n z[n][b]^2) / N + eps)    (fp64, ascending n)
 *   y64[n][b] = z[n][b] * inv64[b] * w[n]                (fp64; w NULL: 1)
 * out, z: N x B fp32; bias, w: N fp32.  Returns 0, or -1 on a bad size.
 */
int gsa_oracle_bias_rmsnorm(const float *out, const float *bias, const float *w,
                            double eps, int64_t N, int B,
                            float *z, double *inv64, double *y64)
{
    if (N < 1 || B < 1 || !(eps >= 0.0))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        for (int b = 0; b < B; ++b) {
            float add = bias ? bias[n] : 0.0f;
            z[n * B + b] = out[n * B + b] + add;
        }
    }
    for (int b = 0; b < B; ++b) {
        double ssq = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double v = (double)z[n * B + b];
            ssq += v * v;
        }
        inv64[b] = 1.0 / sqrt(ssq / (double)N + eps);
    }
    for (int64_t n = 0; n < N; ++n) {
        double wn = w ? (double)w[n] : 1.0;
        for (int b = 0; b < B; ++b)
            y64[n * B + b] = (double)z[n * B + b] * inv64[b] * wn;
    }
    return 0;
}

/* fp32 to bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN. */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/*
 * fp32 to bf16 for a whole array: out[i] = round-to-nearest-even of in[i]
 * to the bf16 grid (a quiet NaN stays a quiet NaN).
 */
void gsa_oracle_f32_to_bf16(const float *in, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16_rne(in[i]);
}

/*
 * The one-shot sum over bf16 slots with fp32 accumulation, in the pages'
 * order: sum = +0.0f; for r = 0..W-1: sum = fl32(sum + widen(slots[r][i]));
 * out[i] = sum.  Widening bf16 to fp32 is exact.  Given the bf16 partials a
 * GPU published, this result (and its bf16 rounding) is unique.
 */
void gsa_oracle_fold_bf16(const uint16_t *slots, int W, int64_t NB, float *out)
{
    for (int64_t i = 0; i < NB; ++i) {
        float sum = 0.0f;
        for (int r = 0; r < W; ++r) {
            uint32_t word = (uint32_t)slots[(int64_t)r * NB + i] << 16;
            float v;
            memcpy(&v, &word, sizeof v);
            sum = sum + v;
        }
        out[i] = sum;
    }
}

/*
 * The normalised output in fp32, given one 1/rms value per column, in the
 * evaluation order y = fl32(fl32(z * inv[b]) * w[n]) (w NULL: the second
 * product is skipped), plus its bf16 rounding.  Given the same inv, this
 * result is unique.
 */
void gsa_oracle_scale_f32(const float *z, const float *inv, const float *w,
                          int64_t N, int B, float *y, uint16_t *y_bf16)
{
    for (int64_t n = 0; n < N; ++n) {
        for (int b = 0; b < B; ++b) {
            float v = z[n * B + b] * inv[b];
            if (w)
                v = v * w[n];
            y[n * B + b] = v;
            y_bf16[n * B + b] = f32_to_bf16_rne(v);
        }
    }
}

/*
 * Rows owned by each rank in the two-shot variant: chunks of
 * chunk_rows = ceil(ceil(N / W) / 16) * 16 rows (whole 16-row tiles), rank p
 * owning rows [p * chunk_rows, min(N, (p + 1) * chunk_rows)); rows past
 * W * chunk_rows cannot occur.  Returns chunk_rows.
 */
int64_t gsa_oracle_two_shot_chunk_rows(int64_t N, int W)
{
    int64_t per_rank = (N + W - 1) / W;
    return (per_rank + 15) / 16 * 16;
}

/*
 * Two-shot all-reduce at one rank's share, given the slots as published
 * (W x N x B fp32, the calling rank's own slot included) and what every
 * rank published as its reduced chunk (`gathered`, N x B: rows of chunk p
 * hold rank p's values; the calling rank's rows are ignored):
 *   rows of the own chunk:   out = fp32 fold of the W slots in rank order
 *                            from +0 (as gsa_oracle_fold_f32), also the
 *                            chunk this rank publishes (mine)
 *   rows of chunk p != rank: out = gathered (rank p's published values)
 * out, mine: N x B fp32 (mine is written only on the own chunk's rows).
 */
void gsa_oracle_two_shot(const float *slots, const float *gathered, int W, int rank,
                         int64_t N, int B, float *out, float *mine)
{
    int64_t cr = gsa_oracle_two_shot_chunk_rows(N, W);
    int64_t NB = N * (int64_t)B;
    for (int64_t n = 0; n < N; ++n) {
        int64_t owner = n / cr;
        for (int b = 0; b < B; ++b) {
            int64_t i = n * B + b;
            if (owner == rank) {
                float acc = 0.0f;
                for (int r = 0; r < W; ++r)
                    acc = acc + slots[(int64_t)r * NB + i];
                out[i] = acc;
                mine[i] = acc;
            } else {
                out[i] = gathered[i];
            }
        }
    }
}

/*
 * Mixture-of-experts down-projection fused with the combine all-to-all, at
 * one rank's share.  This rank holds ne experts; expert e's weight Wd[e] is
 * H x F (H output features of F inputs, row-major).  The dispatched rows X
 * (rows_in x F) hold, for local expert e and source rank s, len[e*W + s] rows
 * starting at row in_off[e*W + s].  Row i of that segment goes back to rank
 * s as row dst_off[s*ne + e] + i of its combine buffer (rows_out x H):
 *   y64[(s*rows_out + dst_off[s*ne+e] + i)*H + n]
 *       = sum_k X[in_off[e*W+s] + i][k] * Wd[e][n][k]      (fp64, ascending k)
 *   abs64[...] = sum_k |X[..][k] * Wd[e][n][k]|            (for the error bound)
 *   written[s*rows_out + row] = 1 for every row a segment fills.
 * Other entries are left as the caller set them.  Returns 0; -1 if a length
 * or offset is negative or a segment leaves X or a combine buffer; -2 if two
 * segments fill the same row of a combine buffer.
 */
int gsa_oracle_moe_combine(const uint16_t *X, const uint16_t *Wd, const int32_t *len,
                           const int32_t *in_off, const int32_t *dst_off, int W, int ne,
                           int64_t H, int64_t F, int64_t rows_in, int64_t rows_out,
                           double *y64, double *abs64, uint8_t *written)
{
    if (W < 1 || ne < 1 || H < 1 || F < 1)
        return -1;
    for (int s = 0; s < W; ++s) {
        for (int e = 0; e < ne; ++e) {
            int64_t n_rows = len[e * W + s];
            int64_t src = in_off[e * W + s];
            int64_t dst = dst_off[s * ne + e];
            if (n_rows < 0 || src < 0 || dst < 0 || src + n_rows > rows_in ||
                dst + n_rows > rows_out)
                return -1;
            for (int64_t i = 0; i < n_rows; ++i) {
                int64_t orow = (int64_t)s * rows_out + dst + i;
                if (written[orow])
                    return -2;
                written[orow] = 1;
                const uint16_t *xr = X + (src + i) * F;
                for (int64_t n = 0; n < H; ++n) {
                    const uint16_t *wr = Wd + ((int64_t)e * H + n) * F;
                    double acc = 0.0;
                    double acc_abs = 0.0;
                    for (int64_t k = 0; k < F; ++k) {
                        double q = bf16_bits_to_double(xr[k]) * bf16_bits_to_double(wr[k]);
                        acc += q;
                        acc_abs += fabs(q);
                    }
                    y64[orow * H + n] = acc;
                    abs64[orow * H + n] = acc_abs;
                }
            }
        }
    }
    return 0;
}
