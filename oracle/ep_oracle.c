/*
 * CPU oracle for MoE expert-parallel dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library. The product
 * path (the HIP library) never calls it and shares no code with it.
 *
 * Plain, slow, obviously correct loops in the order the method describes
 * them. Source: "Enabling trillion-parameter models on AWS EFA" (Perplexity,
 * 2025-11-04):
 *   - section "Dispatch and combine": the dispatch kernel takes the tokens
 *     and each token's experts and forwards every token to the ranks that
 *     host its experts; after the experts run, combine brings the tokens
 *     back to their source rank and forms their routing-weighted average;
 *   - section "Send and receive buffers": a rank can receive at most
 *     N*T*max(R, E/N) tokens; senders must place writes contiguously, which
 *     needs per-expert token counts exchanged first, from which each rank
 *     derives where its writes go and at which offset it receives from each
 *     peer;
 *   - section "Dispatch and combine" (timing figures): per-expert counts,
 *     then a running prefix sum gives the offsets that fill per-peer send
 *     buffers; the receiver shuffles tokens from its receive buffer into the
 *     grouped-GEMM input; combine accumulates the tokens of the receive
 *     buffer into the output tensor;
 *   - section "Evaluation": hidden 7168, block-scaled fp8 dispatch, bf16
 *     combine.
 *
 * Readings where the page is silent (each one also listed in the design
 * notes): expert e lives on rank e / L with L = E/N; one row moves per
 * (token, expert) slot; within an expert, rows keep slot order (token, then
 * choice); the receive buffer of rank d holds the segments of sources
 * 0..N-1 in order; the grouped layout orders rows by (local expert, source,
 * token, choice) with no padding; the weighted average is the plain sum of
 * weight * value over the R choices (the weights already sum to one);
 * out-of-range expert ids and rows beyond the capacity are dropped and
 * flagged.
 *
 * Floating point: combine accumulates in double and rounds once to bf16
 * (round to nearest, ties to even). The stand-in expert ops (scale,
 * dequantise) multiply in float and round to bf16, the way an expert
 * kernel emitting bf16 would.
 */
#include "ep_oracle.h"

#include <fenv.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* Number formats, written from their definitions.                          */
/* ---------------------------------------------------------------------- */

/* bf16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits; the top
 * half of an IEEE-754 binary32. Decoding is exact. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a double to the nearest bf16 value, ties to even, in one step.
 * Finite results only; values beyond the largest bf16 round to infinity
 * as IEEE-754 prescribes. */
uint16_t oracle_f64_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    if (v == 0.0)
        return signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    int e2;
    frexp(a, &e2);           /* a = m * 2^e2 with m in [0.5, 1) */
    int e = e2 - 1;          /* 2^e <= a < 2^(e+1) */
    if (e < -126)
        e = -126;            /* subnormal range: fixed quantum 2^-133 */
    double quantum = ldexp(1.0, e - 7);     /* 8 significant bits */
    double n = a / quantum;                  /* exact: power-of-two scale */
    double r = nearbyint(n);                 /* default mode: ties to even */
    double q = r * quantum;
    const double bf16_max = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
    const double halfway = ldexp(511.0, 119);    /* bf16_max + half ulp */
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    if (a >= halfway)
        return sign | 0x7F80;                    /* rounds to infinity */
    if (q > bf16_max)
        q = bf16_max;
    float f = (float)q;                          /* exact: q is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

uint16_t oracle_f32_to_bf16(float f)
{
    return oracle_f64_to_bf16((double)f);
}

/* OCP 8-bit floating point, E4M3 ("e4m3fn"): 1 sign, 4 exponent bits
 * (bias 7), 3 fraction bits; no infinities; S.1111.111 is NaN; exponent
 * field 0 encodes subnormals m/8 * 2^-6. */
float oracle_e4m3_to_f32(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int ex = (c >> 3) & 0xF;
    int m = c & 7;
    double v;
    if (ex == 0xF && m == 7)
        return NAN;
    if (ex == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, ex - 7);
    return (float)(sign ? -v : v);
}

/* Nearest OCP e4m3fn value to v, ties to the even code; magnitudes beyond the
 * largest finite value (448) saturate to it; NaN gives 0x7F. Written as a
 * search over the 127 non-negative finite codes, which are ordered like
 * their values. */
uint8_t oracle_f32_to_e4m3(float v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (isinf(a))
        return sign | 0x7E;            /* saturates like any finite overflow */
    uint8_t best = 0;
    double best_d = a;                 /* distance to code 0 (value 0) */
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs((double)oracle_e4m3_to_f32((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) != 0)) {
            best = (uint8_t)c;
            best_d = d;
        }
    }
    return sign | best;
}

/* Block-scaled fp8 ("Evaluation": block-scaled fp8 dispatch), for one row of
 * H bf16 values: per block of 128, amax = max |x|, scale = amax / 448 in
 * float (1 when amax is 0), code = e4m3(x / scale) with the quotient formed
 * in float and clamped to +-448. codes: H bytes; scales: H/128 floats.
 * Non-finite inputs (the page is silent; reading adopted): a NaN is never
 * larger than amax, so it is left out of it, and its quotient is NaN, code
 * 0x7F; an infinite value makes amax and the scale infinite, its own
 * quotient inf/inf is NaN (0x7F) and the finite values of its block divide
 * to signed zeros. */
void oracle_quantize_b128(int H, const uint16_t *x, uint8_t *codes, float *scales)
{
    for (int b = 0; b < H / 128; ++b) {
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) {
            float a = fabsf(oracle_bf16_to_f32(x[b * 128 + i]));
            if (a > amax)
                amax = a;
        }
        float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
        scales[b] = scale;
        for (int i = 0; i < 128; ++i) {
            float q = oracle_bf16_to_f32(x[b * 128 + i]) / scale;
            if (q > 448.0f)
                q = 448.0f;
            if (q < -448.0f)
                q = -448.0f;
            codes[b * 128 + i] = oracle_f32_to_e4m3(q);
        }
    }
}

/* Sender with the quantisation fused: the fp8 planes of token (s, t) go to
 * its R send slots. x: bf16 [N][T][H]; codes: [N][T*R][H];
 * scales: [N][T*R][H/128]. */
void oracle_dispatch_pack_quant(int N, int T, int R, int H, const uint16_t *x,
                                const int32_t *send_pos, uint8_t *codes,
                                float *scales)
{
    uint8_t *qc = (uint8_t *)malloc((size_t)H);
    float *qs = (float *)malloc((size_t)(H / 128) * sizeof(float));
    if (!qc || !qs) {
        free(qc);
        free(qs);
        return;
    }
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t) {
            oracle_quantize_b128(H, x + ((size_t)s * T + t) * H, qc, qs);
            for (int k = 0; k < R; ++k) {
                int32_t p = send_pos[((size_t)s * T + t) * R + k];
                if (p < 0)
                    continue;
                size_t row = (size_t)s * T * R + (size_t)p;
                memcpy(codes + row * H, qc, (size_t)H);
                memcpy(scales + row * (H / 128), qs, (size_t)(H / 128) * sizeof(float));
            }
        }
    free(qc);
    free(qs);
}

/* ---------------------------------------------------------------------- */
/* Plan: counts, prefix sums, positions, exchange, receive offsets.         */
/* ---------------------------------------------------------------------- */

int64_t oracle_recv_bound(int N, int T, int E, int R)
{
    /* worst case from "Send and receive buffers": N * T * max(R, E/N) */
    int64_t L = E / N;
    int64_t m = R > L ? R : L;
    return (int64_t)N * T * m;
}

int oracle_plan(int N, int T, int E, int R, int64_t cap,
                const int32_t *idx, int32_t *cnt, int32_t *send_off,
                int32_t *send_pos, int32_t *recv_off, int32_t *grp_off,
                int32_t *grp_pos, int32_t *status)
{
    if (N <= 0 || T < 0 || E <= 0 || R <= 0 || E % N != 0 || cap < 0)
        return -1;
    const int L = E / N;
    int32_t st = 0;

    /* Per-expert token counts of every source rank. Slots whose expert id
     * is out of range are not routed anywhere. */
    for (int s = 0; s < N; ++s)
        for (int e = 0; e < E; ++e)
            cnt[(size_t)s * E + e] = 0;
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < R; ++k) {
                int32_t e = idx[((size_t)s * T + t) * R + k];
                if (e < 0 || e >= E) {
                    st |= ORACLE_STATUS_BAD_EXPERT;
                    continue;
                }
                cnt[(size_t)s * E + e] += 1;
            }

    /* Send offsets: exclusive prefix sum of the counts over experts. Since
     * experts of rank d are d*L .. d*L+L-1, the rows for rank d form one
     * contiguous segment [send_off[d*L], send_off[(d+1)*L]). */
    for (int s = 0; s < N; ++s) {
        int32_t *so = send_off + (size_t)s * (E + 1);
        so[0] = 0;
        for (int e = 0; e < E; ++e)
            so[e + 1] = so[e] + cnt[(size_t)s * E + e];
    }

    /* Send position of each slot: its expert's offset plus the number of
     * earlier slots of the same source routed to the same expert (slot
     * order = token, then choice). */
    int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!seen)
        return -2;
    for (int s = 0; s < N; ++s) {
        memset(seen, 0, (size_t)E * sizeof(int32_t));
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < R; ++k) {
                size_t i = ((size_t)s * T + t) * R + k;
                int32_t e = idx[i];
                if (e < 0 || e >= E) {
                    send_pos[i] = -1;
                    continue;
                }
                send_pos[i] = send_off[(size_t)s * (E + 1) + e] + seen[e];
                seen[e] += 1;
            }
    }
    free(seen);

    /* Exchange: destination d learns rows(s -> d) from every source and
     * receives source s's segment at recv_off[d][s] (sources in order). */
    for (int d = 0; d < N; ++d) {
        int32_t *ro = recv_off + (size_t)d * (N + 1);
        ro[0] = 0;
        for (int s = 0; s < N; ++s) {
            const int32_t *so = send_off + (size_t)s * (E + 1);
            int32_t rows = so[(d + 1) * L] - so[d * L];
            ro[s + 1] = ro[s] + rows;
        }
        if ((int64_t)ro[N] > cap)
            st |= ORACLE_STATUS_CAPACITY;
    }

    /* Grouped layout offsets of destination d: local expert j owns rows
     * [grp_off[d][j], grp_off[d][j+1]); its size is the column sum of the
     * counts over all sources. */
    for (int d = 0; d < N; ++d) {
        int32_t *go = grp_off + (size_t)d * (L + 1);
        go[0] = 0;
        for (int j = 0; j < L; ++j) {
            int32_t col = 0;
            for (int s = 0; s < N; ++s)
                col += cnt[(size_t)s * E + d * L + j];
            go[j + 1] = go[j] + col;
        }
    }

    /* Grouped position of each slot: expert offset, plus the rows that
     * earlier sources sent to the same expert, plus the slot's rank among
     * its own source's rows for that expert. Rows that do not fit the
     * capacity are dropped (-1). */
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < R; ++k) {
                size_t i = ((size_t)s * T + t) * R + k;
                int32_t e = idx[i];
                if (e < 0 || e >= E) {
                    grp_pos[i] = -1;
                    continue;
                }
                int d = e / L, j = e % L;
                int64_t before = 0;
                for (int s2 = 0; s2 < s; ++s2)
                    before += cnt[(size_t)s2 * E + e];
                int64_t rank = send_pos[i] - send_off[(size_t)s * (E + 1) + e];
                int64_t g = grp_off[(size_t)d * (L + 1) + j] + before + rank;
                grp_pos[i] = (g < cap) ? (int32_t)g : -1;
            }

    *status = st;
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Payload movement (opaque bytes; one call per payload plane).             */
/* ---------------------------------------------------------------------- */

/* Sender: copy each token row into its send slots, so the rows for one
 * destination sit contiguously in the source's send buffer.
 * x: [N][T][row], send: [N][T*R][row]. */
void oracle_dispatch_pack(int N, int T, int R, int64_t row,
                          const uint8_t *x, const int32_t *send_pos,
                          uint8_t *send)
{
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < R; ++k) {
                int32_t p = send_pos[((size_t)s * T + t) * R + k];
                if (p < 0)
                    continue;
                memcpy(send + ((size_t)s * T * R + (size_t)p) * row,
                       x + ((size_t)s * T + t) * row, (size_t)row);
            }
}

/* The network write: for every pair (s, d) one bulk copy of s's segment
 * for d into d's receive buffer at recv_off[d][s].
 * recv: [N][recv_rows][row]; rows beyond recv_rows are not written. */
void oracle_transfer(int N, int T, int E, int R, int64_t row,
                     int64_t recv_rows, const uint8_t *send,
                     const int32_t *send_off, const int32_t *recv_off,
                     uint8_t *recv)
{
    const int L = E / N;
    for (int s = 0; s < N; ++s)
        for (int d = 0; d < N; ++d) {
            const int32_t *so = send_off + (size_t)s * (E + 1);
            int64_t first = so[d * L];
            int64_t rows = so[(d + 1) * L] - so[d * L];
            int64_t dst = recv_off[(size_t)d * (N + 1) + s];
            for (int64_t i = 0; i < rows; ++i) {
                if (dst + i >= recv_rows)
                    break;
                memcpy(recv + ((size_t)d * recv_rows + dst + i) * row,
                       send + ((size_t)s * T * R + first + i) * row,
                       (size_t)row);
            }
        }
}

/* Receiver: shuffle rows from the receive buffer into the grouped layout.
 * Source s's segment holds its rows for local experts j = 0..L-1 in turn;
 * they go to expert j's region after the rows of sources 0..s-1.
 * grouped: [N][cap][row]. A grouped row below cap whose receive-buffer row
 * lies at or beyond recv_rows (the transfer dropped it: more rows arrived
 * than the buffer holds) is written as zeros; the page is silent on what an
 * overflowing receiver holds, and zeros make the slot add nothing to its
 * token downstream. */
void oracle_unpack(int N, int T, int E, int R, int64_t row,
                   int64_t recv_rows, int64_t cap, const uint8_t *recv,
                   const int32_t *cnt, const int32_t *send_off,
                   const int32_t *recv_off, const int32_t *grp_off,
                   uint8_t *grouped)
{
    (void)T;
    (void)R;
    const int L = E / N;
    for (int d = 0; d < N; ++d)
        for (int s = 0; s < N; ++s) {
            const int32_t *so = send_off + (size_t)s * (E + 1);
            int64_t seg = recv_off[(size_t)d * (N + 1) + s];
            for (int j = 0; j < L; ++j) {
                int e = d * L + j;
                int64_t in_seg = so[e] - so[d * L];
                int64_t before = 0;
                for (int s2 = 0; s2 < s; ++s2)
                    before += cnt[(size_t)s2 * E + e];
                int64_t g0 = grp_off[(size_t)d * (L + 1) + j] + before;
                for (int64_t i = 0; i < cnt[(size_t)s * E + e]; ++i) {
                    int64_t src = seg + in_seg + i;
                    int64_t dst = g0 + i;
                    if (dst >= cap)
                        continue;
                    if (src >= recv_rows) {
                        memset(grouped + ((size_t)d * cap + dst) * row, 0, (size_t)row);
                        continue;
                    }
                    memcpy(grouped + ((size_t)d * cap + dst) * row,
                           recv + ((size_t)d * recv_rows + src) * row,
                           (size_t)row);
                }
            }
        }
}

/* ---------------------------------------------------------------------- */
/* Stand-in expert (the grouped GEMM is out of scope).                      */
/* ---------------------------------------------------------------------- */

/* y row of expert e from one grouped bf16 row: identity or a per-expert
 * scalar scale alpha[e] (float multiply, bf16 rounding). */
void oracle_expert_bf16(int H, const uint16_t *in, const float *alpha, int e,
                        uint16_t *out)
{
    for (int h = 0; h < H; ++h) {
        if (!alpha) {
            out[h] = in[h];
        } else {
            float v = oracle_bf16_to_f32(in[h]) * alpha[e];
            out[h] = oracle_f32_to_bf16(v);
        }
    }
}

/* Dequantising expert: bf16(e4m3(code) * scale of its 128-element block). */
void oracle_expert_fp8(int H, const uint8_t *codes, const float *scales,
                       uint16_t *out)
{
    for (int h = 0; h < H; ++h) {
        float v = oracle_e4m3_to_f32(codes[h]) * scales[h / 128];
        out[h] = oracle_f32_to_bf16(v);
    }
}

/* Apply the stand-in expert to every delivered grouped row of every
 * destination. The expert of grouped row r of d is d*L + j where
 * grp_off[d][j] <= r < grp_off[d][j+1].
 * payload 0: grouped0 bf16 [N][cap][H]; payload 1: grouped0 e4m3 [N][cap][H]
 * and grouped1 fp32 [N][cap][H/128]. y: bf16 [N][cap][H]. */
void oracle_expert_op(int N, int E, int H, int64_t cap, int payload,
                      const void *grouped0, const void *grouped1,
                      const float *alpha, const int32_t *grp_off,
                      uint16_t *y)
{
    const int L = E / N;
    for (int d = 0; d < N; ++d)
        for (int j = 0; j < L; ++j) {
            int64_t r0 = grp_off[(size_t)d * (L + 1) + j];
            int64_t r1 = grp_off[(size_t)d * (L + 1) + j + 1];
            if (r1 > cap)
                r1 = cap;
            for (int64_t r = r0; r < r1; ++r) {
                size_t row = (size_t)d * cap + r;
                if (payload == 0)
                    oracle_expert_bf16(H, (const uint16_t *)grouped0 + row * H,
                                       alpha, d * L + j, y + row * H);
                else
                    oracle_expert_fp8(H, (const uint8_t *)grouped0 + row * H,
                                      (const float *)grouped1 + row * (H / 128),
                                      y + row * H);
            }
        }
}

/* ---------------------------------------------------------------------- */
/* Combine.                                                                 */
/* ---------------------------------------------------------------------- */

/* One output token from its R expert rows: sum_k w[k] * y_k, k ascending,
 * accumulated in double, rounded once to bf16. Rows given as NULL (dropped
 * slots) contribute nothing. */
void oracle_combine_token(int H, int R, const float *w,
                          const uint16_t *const *rows, uint16_t *out)
{
    for (int h = 0; h < H; ++h) {
        double acc = 0.0;
        for (int k = 0; k < R; ++k) {
            if (!rows[k])
                continue;
            acc += (double)w[k] * (double)oracle_bf16_to_f32(rows[k][h]);
        }
        out[h] = oracle_f64_to_bf16(acc);
    }
}

/* Combine on the receiver: each source token gathers the expert outputs of
 * its R slots (at grp_pos on the hosting rank) and takes their weighted
 * sum. y: bf16 [N][cap][H]; w: fp32 [N][T][R]; out: bf16 [N][T][H]. */
void oracle_combine(int N, int T, int E, int R, int H, int64_t cap,
                    const int32_t *idx, const int32_t *grp_pos,
                    const uint16_t *y, const float *w, uint16_t *out)
{
    const int L = E / N;
    const uint16_t **rows = (const uint16_t **)malloc((size_t)R * sizeof *rows);
    if (!rows)
        return;
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t) {
            size_t tok = (size_t)s * T + t;
            for (int k = 0; k < R; ++k) {
                int32_t e = idx[tok * R + k];
                int32_t g = grp_pos[tok * R + k];
                if (e < 0 || e >= E || g < 0) {
                    rows[k] = NULL;
                    continue;
                }
                rows[k] = y + ((size_t)(e / L) * cap + g) * H;
            }
            oracle_combine_token(H, R, w + tok * R, rows, out + tok * H);
        }
    free(rows);
}

/* Combine with partial sums on the expert side (the sender-side
 * accumulation the "Evaluation" section contrasts with receiver-only
 * accumulation). Reading adopted: for one token, the slots whose experts sit
 * on the same rank d form a group; the expert rank sums its group in float
 * (fused multiply-add, slot order k ascending, from 0) and rounds the sum
 * once to bf16, which is what travels back; the group's row is kept at the
 * slot of its first member (its leader). The source rank then adds the
 * partial rows in float in leader order (k ascending, from 0) and rounds
 * once to bf16. Dropped slots (grp_pos < 0 or a bad id) belong to no group.
 * rows[k], rank[k]: the slot's expert-output row and hosting rank (rows[k]
 * NULL for a dropped slot). partial: R rows of H (leader rows written, the
 * others untouched). */
void oracle_combine_presum_token(int H, int R, const float *w,
                                 const uint16_t *const *rows, const int *rank,
                                 uint16_t *partial, uint16_t *out)
{
    for (int k = 0; k < R; ++k) {
        if (!rows[k])
            continue;
        int leader = 1;
        for (int k2 = 0; k2 < k; ++k2)
            if (rows[k2] && rank[k2] == rank[k])
                leader = 0;
        if (!leader)
            continue;
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int k2 = k; k2 < R; ++k2)
                if (rows[k2] && rank[k2] == rank[k])
                    acc = fmaf(w[k2], oracle_bf16_to_f32(rows[k2][h]), acc);
            partial[(size_t)k * H + h] = oracle_f32_to_bf16(acc);
        }
    }
    for (int h = 0; h < H; ++h) {
        float acc = 0.0f;
        for (int k = 0; k < R; ++k) {
            if (!rows[k])
                continue;
            int leader = 1;
            for (int k2 = 0; k2 < k; ++k2)
                if (rows[k2] && rank[k2] == rank[k])
                    leader = 0;
            if (leader)
                acc = acc + oracle_bf16_to_f32(partial[(size_t)k * H + h]);
        }
        out[h] = oracle_f32_to_bf16(acc);
    }
}

/* The whole partial-sum combine. y: bf16 [N][cap][H]; w: fp32 [N][T][R];
 * partial: bf16 [N][T*R][H] (leader rows written); out: bf16 [N][T][H]. */
void oracle_combine_presum(int N, int T, int E, int R, int H, int64_t cap,
                           const int32_t *idx, const int32_t *grp_pos,
                           const uint16_t *y, const float *w, uint16_t *partial,
                           uint16_t *out)
{
    const int L = E / N;
    const uint16_t **rows = (const uint16_t **)malloc((size_t)R * sizeof *rows);
    int *rank = (int *)malloc((size_t)R * sizeof *rank);
    if (!rows || !rank) {
        free(rows);
        free(rank);
        return;
    }
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t) {
            size_t tok = (size_t)s * T + t;
            for (int k = 0; k < R; ++k) {
                int32_t e = idx[tok * R + k];
                int32_t g = grp_pos[tok * R + k];
                rank[k] = -1;
                rows[k] = NULL;
                if (e < 0 || e >= E || g < 0)
                    continue;
                rank[k] = e / L;
                rows[k] = y + ((size_t)(e / L) * cap + g) * H;
            }
            oracle_combine_presum_token(H, R, w + tok * R, rows, rank,
                                        partial + tok * R * (size_t)H, out + tok * H);
        }
    free(rows);
    free(rank);
}

/* ---------------------------------------------------------------------- */
/* KV-block push ("vLLMにおける分離型推論のTTFTとTPOTを改善するプッシュ型KV転送",   */
/* 「スレッドモデル」: block ids are mapped to memory descriptors and        */
/* contiguous blocks are merged into larger transfer regions, one write per  */
/* region).                                                                  */
/* ---------------------------------------------------------------------- */

/* Byte offset of token i of a request in a pool of blocks of `bs` tokens of
 * `tok` bytes each, given the request's block table. */
static int64_t kv_addr(int64_t i, int64_t tok, int64_t bs, const int32_t *blocks)
{
    return ((int64_t)blocks[i / bs] * bs + i % bs) * tok;
}

/* Regions of a request of n tokens: maximal runs of consecutive tokens
 * whose source and destination bytes both continue where the previous
 * token's ended. Writes up to n regions (src_off, dst_off, bytes) and
 * returns their number. */
int64_t oracle_kv_regions(int64_t n, int64_t tok, int64_t bs_src,
                          const int32_t *src_blocks, int64_t bs_dst,
                          const int32_t *dst_blocks, int64_t *src_off,
                          int64_t *dst_off, int64_t *bytes)
{
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t a = kv_addr(i, tok, bs_src, src_blocks);
        int64_t b = kv_addr(i, tok, bs_dst, dst_blocks);
        if (m > 0 && src_off[m - 1] + bytes[m - 1] == a &&
            dst_off[m - 1] + bytes[m - 1] == b) {
            bytes[m - 1] += tok;
        } else {
            src_off[m] = a;
            dst_off[m] = b;
            bytes[m] = tok;
            ++m;
        }
    }
    return m;
}

/* Apply the regions for every tensor-parallel rank r: rank r's pools start
 * at r * src_rank_bytes and r * dst_rank_bytes. */
void oracle_kv_copy(int ranks, int64_t m, const int64_t *src_off,
                    const int64_t *dst_off, const int64_t *bytes,
                    const uint8_t *src, int64_t src_rank_bytes, uint8_t *dst,
                    int64_t dst_rank_bytes)
{
    for (int r = 0; r < ranks; ++r)
        for (int64_t j = 0; j < m; ++j)
            memcpy(dst + r * dst_rank_bytes + dst_off[j],
                   src + r * src_rank_bytes + src_off[j], (size_t)bytes[j]);
}

int oracle_rounding_mode_is_nearest(void)
{
    return fegetround() == FE_TONEAREST;
}
