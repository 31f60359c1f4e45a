/*
 * CPU oracle for the GPU-resident-metadata all-to-allv (MoE dispatch and combine).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is loaded by tests/, by the smoke check in
 * __graft_entry__ and by the cpu_baseline leg of bench.py; nothing on the product path
 * links it, calls it or includes it, and it includes nothing from the product path.
 * It is plain single-threaded C11, built with gcc -O2 and no fast-math, and computes
 * floating point in double (fp64); values are rounded to the storage dtype only where
 * the method stores them.
 *
 * What it computes, step by step, in the order the pages give it:
 *
 *   [abhik.ai "Collective Communication for 100k+ GPUs", section "Inference: small
 *    messages, unknown sizes", Figure 13; qiguanping.github.io "NCCLX", section 7,
 *    figures 13-18; notes.yuuk.io, paper section 6.1]
 *
 *   1. A router has chosen top-k experts per token (an input here: ids[R][T][k]).
 *   2. On every rank the tokens are sorted by expert into a send buffer
 *      (oracle_dispatch, phase "sort").
 *   3. An all-to-allv sends every row to the rank that holds its expert; the
 *      per-peer counts are device data, read when the exchange runs, and the counts
 *      each rank received are handed back (oracle_dispatch, phase "exchange").
 *   4. Experts run on the received rows (a harness stand-in: oracle_expert).
 *   5. The return all-to-all brings expert outputs back to the token's home rank
 *      (oracle_return), and the combine merges each token's k results
 *      (oracle_combine).  The pages name this combine step without defining it; the
 *      reading taken here is the gate-weighted sum over the k slots.
 *
 * Readings of points the pages leave open (each is also listed in the design notes):
 *   - expert e lives on rank owner(e) = e / experts_per_rank (contiguous blocks);
 *   - "sorted by expert" is a stable sort by (expert, token, slot);
 *   - a receive buffer is laid out source-major (rows from rank 0 first), keeping the
 *     sender's order inside each source segment, as any all-to-allv does; the
 *     expert-major layout (an option) groups a receiver's rows by its local expert,
 *     then by source rank, then in the sender's order, which is the grouping an
 *     expert's computation right after the dispatch wants (abhik.ai page, Figure 13:
 *     tokens travel to the GPU that holds their expert);
 *   - counts and offsets are in rows (int32);
 *   - a token whose k experts share a rank is sent k times (no de-duplication);
 *   - an expert id outside [0, E) is dropped (status bit 1), and its slot adds
 *     nothing to the combine;
 *   - a receive row at or beyond the per-rank capacity is dropped (status bit 2), and
 *     its slot adds nothing to the combine;
 *   - combine: y = sum_j g[j] * z_j in exact-as-possible fp64, rounded once to the
 *     output dtype (round to nearest, ties to even).
 *
 * Pins (tests/test_oracle_*.py, run without a GPU): library bincount/cumsum for the
 * counts and offsets; a library stable argsort for the send order at one rank; tagged
 * rows (each token appears exactly k times, at the predicted place); brute force over
 * every id pattern for two ranks against an independent nested-loop formulation; the
 * round trip dispatch -> return; unit-gate identities; exact rational arithmetic for
 * the combine; brute-force nearest search for the bf16 rounding.
 */
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#include <math.h>

#define ORACLE_F32  0
#define ORACLE_BF16 1

#define ORACLE_ST_EXPERT_RANGE  1u
#define ORACLE_ST_RECV_OVERFLOW 2u

#define ORACLE_LAYOUT_SOURCE_MAJOR 0
#define ORACLE_LAYOUT_EXPERT_MAJOR 1

/* First place of expert e's rows in sender s's expert-sorted order: the rows s sends
 * to experts below e. */
static int64_t sender_expert_start(const int32_t* cnt, int32_t E, int32_t s, int32_t e)
{
    int64_t run = 0;
    for (int32_t e2 = 0; e2 < e; ++e2) run += cnt[(int64_t)s * E + e2];
    return run;
}

/* ---------------------------------------------------------------------------------
 * Number formats.  bf16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent
 * bits, 7 stored fraction bits.
 * ------------------------------------------------------------------------------- */

/* bf16 bits -> double; exact (every bf16 value is a binary32 value). */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> bf16 bits, round to nearest, ties to even, in one rounding step from the
 * double (no detour through binary32, which would round twice).  Finite inputs only;
 * overflow saturates to infinity as IEEE rounding does. */
uint16_t oracle_double_to_bf16(double v)
{
    if (v != v) return 0x7FC0u;                       /* NaN */
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int ex;
    (void)frexp(a, &ex);          /* a = m * 2^ex, m in [0.5, 1) */
    /* bf16 keeps 8 significant bits: the unit in the last place is 2^(ex-8) for a
     * normal result.  Below the smallest normal (2^-126) the spacing is fixed at the
     * subnormal step 2^-133. */
    int ulp_exp = ex - 8;
    if (ulp_exp < -133) ulp_exp = -133;
    double scaled = ldexp(a, -ulp_exp);               /* exact: a power-of-two scale */
    double r = nearbyint(scaled);                     /* default mode: ties to even  */
    double q = ldexp(r, ulp_exp);                     /* exactly representable in bf16 */
    if (q >= 0x1.0p128) return (uint16_t)(sign | 0x7F80u);   /* rounds past the max */
    float f = (float)q;                               /* exact: q has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFFu));
}

static double load_elem(const uint8_t* row, int64_t h, int dtype)
{
    if (dtype == ORACLE_BF16) {
        uint16_t b;
        memcpy(&b, row + 2 * h, 2);
        return oracle_bf16_to_double(b);
    }
    float f;
    memcpy(&f, row + 4 * h, 4);
    return (double)f;
}

static void store_elem(uint8_t* row, int64_t h, int dtype, double v)
{
    if (dtype == ORACLE_BF16) {
        uint16_t b = oracle_double_to_bf16(v);
        memcpy(row + 2 * h, &b, 2);
    } else {
        float f = (float)v;                           /* C conversion: round to nearest even */
        memcpy(row + 4 * h, &f, 4);
    }
}

static int64_t elem_bytes(int dtype) { return dtype == ORACLE_BF16 ? 2 : 4; }

/* ---------------------------------------------------------------------------------
 * Dispatch: sort by expert into send buffers, then the all-to-allv.
 *
 *   x        [R][T][row_bytes]   token rows of every rank (raw bytes: rows are copied,
 *                                never interpreted, so any payload works, tags included)
 *   ids      [R][T][k]           expert ids chosen by the router
 *   cnt      [R][E]    out       rows rank s sends to expert e (the split table)
 *   send_off [R][R+1]  out       row offset of the segment for rank d in s's send buffer
 *   pos      [R][T][k] out       place of assignment (t, j) in s's send buffer, -1 if dropped
 *   send     [R][T*k][row_bytes] out  send buffers (expert-sorted)
 *   recv_counts [R][R] out       recv_counts[d][s] = rows rank d receives from rank s
 *   recv_off [R][R+1]  out       exclusive prefix of recv_counts[d][.] over s
 *   recv_eoff [R][epr+1] out     rows rank d receives for its local experts below le
 *                                (exclusive prefix; where expert groups start in the
 *                                expert-major layout)
 *   recv     [R][cap][row_bytes] out  receive buffers (layout: source- or expert-major);
 *                                rows past the received count untouched
 *   status   out                 OR of ORACLE_ST_* bits
 * Returns 0, or -1 for unusable arguments.
 * ------------------------------------------------------------------------------- */
int oracle_dispatch(int32_t R, int32_t T, int32_t k, int32_t epr, int64_t row_bytes, int64_t cap, int32_t layout,
                    const uint8_t* x, const int32_t* ids,
                    int32_t* cnt, int32_t* send_off, int32_t* pos, uint8_t* send,
                    int32_t* recv_counts, int32_t* recv_off, int32_t* recv_eoff, uint8_t* recv, uint32_t* status)
{
    if (R < 1 || T < 0 || k < 1 || epr < 1 || row_bytes < 1 || cap < 0) return -1;
    if (layout != ORACLE_LAYOUT_SOURCE_MAJOR && layout != ORACLE_LAYOUT_EXPERT_MAJOR) return -1;
    const int32_t E = R * epr;
    const int64_t TK = (int64_t)T * k;
    uint32_t st = 0;

    /* Sort by expert, rank by rank (each rank works on its own data only). */
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor) return -1;
    for (int32_t s = 0; s < R; ++s) {
        const int32_t* ids_s = ids + (int64_t)s * TK;
        int32_t* cnt_s = cnt + (int64_t)s * E;

        /* Histogram: how many of this rank's assignments chose each expert. */
        for (int32_t e = 0; e < E; ++e) cnt_s[e] = 0;
        for (int64_t a = 0; a < TK; ++a) {
            int32_t e = ids_s[a];
            if (e < 0 || e >= E) { st |= ORACLE_ST_EXPERT_RANGE; continue; }
            cnt_s[e] += 1;
        }

        /* Where each expert's rows start in the send buffer (exclusive prefix), and
         * where each destination's segment starts: the segment for rank d holds the
         * rows of d's experts d*epr .. d*epr+epr-1, which are consecutive. */
        int32_t run = 0;
        for (int32_t e = 0; e < E; ++e) { cursor[e] = run; run += cnt_s[e]; }
        for (int32_t d = 0; d < R; ++d) send_off[(int64_t)s * (R + 1) + d] = cursor[d * epr];
        send_off[(int64_t)s * (R + 1) + R] = run;

        /* Stable placement: visit (t, j) in order, each row goes to its expert's next
         * free place. */
        for (int32_t t = 0; t < T; ++t) {
            for (int32_t j = 0; j < k; ++j) {
                int64_t a = (int64_t)t * k + j;
                int32_t e = ids_s[a];
                if (e < 0 || e >= E) { pos[(int64_t)s * TK + a] = -1; continue; }
                int32_t p = cursor[e]++;
                pos[(int64_t)s * TK + a] = p;
                memcpy(send + ((int64_t)s * TK + p) * row_bytes,
                       x + ((int64_t)s * T + t) * row_bytes, (size_t)row_bytes);
            }
        }
    }
    free(cursor);

    /* The all-to-allv.  The count rank d receives from rank s is what s put in its
     * segment for d; the receive buffer of d is the concatenation of the segments
     * from s = 0, 1, ..., R-1. */
    for (int32_t d = 0; d < R; ++d) {
        int32_t run = 0;
        for (int32_t s = 0; s < R; ++s) {
            int32_t c = send_off[(int64_t)s * (R + 1) + d + 1] - send_off[(int64_t)s * (R + 1) + d];
            recv_counts[(int64_t)d * R + s] = c;
            recv_off[(int64_t)d * (R + 1) + s] = run;
            run += c;
        }
        recv_off[(int64_t)d * (R + 1) + R] = run;
    }
    for (int32_t d = 0; d < R; ++d) {
        int32_t run = 0;
        for (int32_t le = 0; le < epr; ++le) {
            recv_eoff[(int64_t)d * (epr + 1) + le] = run;
            for (int32_t s = 0; s < R; ++s) run += cnt[(int64_t)s * E + d * epr + le];
        }
        recv_eoff[(int64_t)d * (epr + 1) + epr] = run;
    }
    for (int32_t d = 0; d < R; ++d) {
        if (layout == ORACLE_LAYOUT_SOURCE_MAJOR) {
            /* segment from s = 0 first, each segment in the sender's order */
            for (int32_t s = 0; s < R; ++s) {
                int32_t c = recv_counts[(int64_t)d * R + s];
                for (int32_t i = 0; i < c; ++i) {
                    int64_t q = (int64_t)recv_off[(int64_t)d * (R + 1) + s] + i;
                    int64_t p = (int64_t)send_off[(int64_t)s * (R + 1) + d] + i;
                    if (q >= cap) { st |= ORACLE_ST_RECV_OVERFLOW; continue; }
                    memcpy(recv + ((int64_t)d * cap + q) * row_bytes,
                           send + ((int64_t)s * TK + p) * row_bytes, (size_t)row_bytes);
                }
            }
        } else {
            /* local expert 0 first; inside an expert, source 0 first; inside a source,
             * the sender's order */
            int64_t q = 0;
            for (int32_t le = 0; le < epr; ++le) {
                int32_t e = d * epr + le;
                for (int32_t s = 0; s < R; ++s) {
                    int64_t p0 = sender_expert_start(cnt, E, s, e);
                    for (int32_t i = 0; i < cnt[(int64_t)s * E + e]; ++i, ++q) {
                        if (q >= cap) { st |= ORACLE_ST_RECV_OVERFLOW; continue; }
                        memcpy(recv + ((int64_t)d * cap + q) * row_bytes,
                               send + ((int64_t)s * TK + p0 + i) * row_bytes, (size_t)row_bytes);
                    }
                }
            }
        }
    }
    if (status) *status |= st;
    return 0;
}

/* ---------------------------------------------------------------------------------
 * Expert stand-in on the received rows (harness).  mode 0: identity.  mode 1: scale by
 * 1 + e/256 where e is the row's expert, computed in double and rounded once to the
 * dtype.  The expert of a received row follows from the layout: inside the segment
 * from rank s, rows are sorted by expert, with cnt[s][e] rows for each of d's experts.
 *   recv, z  [R][cap][H] of dtype; only the first min(recv_off[d][R], cap) rows of
 *   each rank are read and written.
 * ------------------------------------------------------------------------------- */
int oracle_expert(int32_t R, int32_t epr, int64_t H, int32_t dtype, int64_t cap, int32_t mode, int32_t layout,
                  const int32_t* cnt, const int32_t* recv_off,
                  const uint8_t* recv, uint8_t* z)
{
    if (R < 1 || epr < 1 || H < 1 || cap < 0 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return -1;
    if (layout != ORACLE_LAYOUT_SOURCE_MAJOR && layout != ORACLE_LAYOUT_EXPERT_MAJOR) return -1;
    const int32_t E = R * epr;
    const int64_t rb = H * elem_bytes(dtype);
    for (int32_t d = 0; d < R; ++d) {
        int64_t q = 0;
        /* visit the received rows of d in their layout's order, with their expert */
        for (int32_t outer = 0; outer < (layout == ORACLE_LAYOUT_SOURCE_MAJOR ? R : epr); ++outer) {
            for (int32_t inner = 0; inner < (layout == ORACLE_LAYOUT_SOURCE_MAJOR ? epr : R); ++inner) {
                int32_t s = layout == ORACLE_LAYOUT_SOURCE_MAJOR ? outer : inner;
                int32_t le = layout == ORACLE_LAYOUT_SOURCE_MAJOR ? inner : outer;
                int32_t e = d * epr + le;
                int32_t c = cnt[(int64_t)s * E + e];
                double scale = 1.0 + (double)e / 256.0;
                if (layout == ORACLE_LAYOUT_SOURCE_MAJOR && le == 0) q = recv_off[(int64_t)d * (R + 1) + s];
                for (int32_t i = 0; i < c; ++i, ++q) {
                    if (q >= cap) continue;
                    const uint8_t* in = recv + ((int64_t)d * cap + q) * rb;
                    uint8_t* out = z + ((int64_t)d * cap + q) * rb;
                    if (mode == 0) { memmove(out, in, (size_t)rb); continue; }
                    for (int64_t h = 0; h < H; ++h)
                        store_elem(out, h, dtype, load_elem(in, h, dtype) * scale);
                }
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------
 * Return all-to-all: the inverse of the exchange.  Every received row goes back to the
 * place its row had in the sender's send order (source-major: row i of the segment d
 * received from s goes to place send_off[s][d] + i; expert-major: row i of the block
 * of expert e from s goes to the sender's first place for e plus i).  A row that was
 * dropped for lack of capacity comes back as zeros.
 *   z   [R][cap][row_bytes];  ret [R][T*k][row_bytes]
 * ------------------------------------------------------------------------------- */
int oracle_return(int32_t R, int32_t T, int32_t k, int32_t epr, int64_t row_bytes, int64_t cap, int32_t layout,
                  const int32_t* cnt, const int32_t* send_off, const int32_t* recv_off,
                  const uint8_t* z, uint8_t* ret)
{
    if (R < 1 || T < 0 || k < 1 || epr < 1 || row_bytes < 1 || cap < 0) return -1;
    if (layout != ORACLE_LAYOUT_SOURCE_MAJOR && layout != ORACLE_LAYOUT_EXPERT_MAJOR) return -1;
    const int64_t TK = (int64_t)T * k;
    const int32_t E = R * epr;
    if (layout == ORACLE_LAYOUT_SOURCE_MAJOR) {
        for (int32_t s = 0; s < R; ++s) {
            for (int32_t d = 0; d < R; ++d) {
                int64_t p0 = send_off[(int64_t)s * (R + 1) + d];
                int64_t c = send_off[(int64_t)s * (R + 1) + d + 1] - p0;
                int64_t q0 = recv_off[(int64_t)d * (R + 1) + s];
                for (int64_t i = 0; i < c; ++i) {
                    uint8_t* out = ret + ((int64_t)s * TK + p0 + i) * row_bytes;
                    if (q0 + i >= cap) { memset(out, 0, (size_t)row_bytes); continue; }
                    memcpy(out, z + ((int64_t)d * cap + q0 + i) * row_bytes, (size_t)row_bytes);
                }
            }
        }
        return 0;
    }
    for (int32_t d = 0; d < R; ++d) {
        int64_t q = 0;
        for (int32_t le = 0; le < epr; ++le) {
            int32_t e = d * epr + le;
            for (int32_t s = 0; s < R; ++s) {
                int64_t p0 = sender_expert_start(cnt, E, s, e);
                for (int32_t i = 0; i < cnt[(int64_t)s * E + e]; ++i, ++q) {
                    uint8_t* out = ret + ((int64_t)s * TK + p0 + i) * row_bytes;
                    if (q >= cap) { memset(out, 0, (size_t)row_bytes); continue; }
                    memcpy(out, z + ((int64_t)d * cap + q) * row_bytes, (size_t)row_bytes);
                }
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------
 * Combine: y[s][t] = sum over slots j of gates[s][t][j] * ret_s[pos[s][t][j]], summed
 * in double and rounded once to the dtype.  Dropped slots (pos < 0) add nothing.
 *   ret [R][T*k][H]; pos, gates [R][T][k]; y [R][T][H]
 * ------------------------------------------------------------------------------- */
int oracle_combine(int32_t R, int32_t T, int32_t k, int64_t H, int32_t dtype,
                   const int32_t* pos, const float* gates, const uint8_t* ret, uint8_t* y)
{
    if (R < 1 || T < 0 || k < 1 || H < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return -1;
    const int64_t TK = (int64_t)T * k;
    const int64_t rb = H * elem_bytes(dtype);
    for (int32_t s = 0; s < R; ++s) {
        for (int32_t t = 0; t < T; ++t) {
            uint8_t* out = y + ((int64_t)s * T + t) * rb;
            for (int64_t h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int32_t j = 0; j < k; ++j) {
                    int64_t a = (int64_t)s * TK + (int64_t)t * k + j;
                    int32_t p = pos[a];
                    if (p < 0) continue;
                    acc += (double)gates[a] * load_elem(ret + ((int64_t)s * TK + p) * rb, h, dtype);
                }
                store_elem(out, h, dtype, acc);
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------
 * The same end result written without any layout: for every token, apply the expert
 * stand-in of each of its k experts to the token's own row and take the gate-weighted
 * sum.  The combine does not depend on how rows were placed in between, so this is a
 * second, independent formulation of dispatch -> expert -> return -> combine when no
 * row is dropped for capacity.  Tokens [tok_begin, tok_end) of the flattened [R*T]
 * range are computed; y holds their rows only (row 0 of y is token tok_begin).
 * ------------------------------------------------------------------------------- */
int oracle_closed_form(int32_t R, int32_t T, int32_t k, int32_t epr, int64_t H, int32_t dtype,
                       int32_t mode, const uint8_t* x, const int32_t* ids, const float* gates,
                       uint8_t* y, int64_t tok_begin, int64_t tok_end)
{
    if (R < 1 || T < 0 || k < 1 || epr < 1 || H < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return -1;
    const int32_t E = R * epr;
    const int64_t rb = H * elem_bytes(dtype);
    const int64_t N = (int64_t)R * T;
    if (tok_begin < 0) tok_begin = 0;
    if (tok_end > N) tok_end = N;
    for (int64_t n = tok_begin; n < tok_end; ++n) {
        const uint8_t* in = x + n * rb;
        uint8_t* out = y + (n - tok_begin) * rb;
        for (int64_t h = 0; h < H; ++h) {
            double v = load_elem(in, h, dtype);
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                int32_t e = ids[n * k + j];
                if (e < 0 || e >= E) continue;
                double f = v;
                if (mode == 1) {
                    /* the expert's output is stored in the dtype before it is returned */
                    uint8_t tmp[4];
                    store_elem(tmp, 0, dtype, v * (1.0 + (double)e / 256.0));
                    f = load_elem(tmp, 0, dtype);
                }
                acc += (double)gates[n * k + j] * f;
            }
            store_elem(out, h, dtype, acc);
        }
    }
    return 0;
}
