/*
 * oracle.c -- plain, slow, single-threaded CPU reference for the MoE token
 * dispatch/combine path.
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library.  The HIP
 * library never links it and shares no source with it.
 *
 * Every function is a direct loop over the definition of the operation.
 * Sources (page titles; the section or table named):
 *   [EPA] "DeepEP-Ascend" README -- "API Overview" table
 *         (get_dispatch_layout / dispatch / combine / low_latency_*),
 *         "Environment Variables" table (MOE_EXPERT_TOKEN_NUMS_TYPE:
 *         count vs prefix sum; MOE_ENABLE_TOPK_NEG_ONE: -1 = not
 *         dispatched), "Quantization Modes in Normal Dispatch" table
 *         (float8_e4m3fn payload with float32 scales).
 *   [ECR] "[Feature Request] Support Expert-Choice Routing via Native
 *         Expert-Centric API ([num_experts, capacity])" -- "Proposed
 *         Solutions", Solution 1 (token_indices [num_experts, capacity]
 *         int32 plus expert weights).
 * Where the pages leave a step open (index dtype, row order inside an
 * expert, capacity overflow, the 128-channel fp8 group and scale rule,
 * accumulation precision), the reading taken is stated at the function.
 *
 * Floating point: built with -O2 -ffp-contract=off, no fast-math, SSE
 * arithmetic (no excess precision).
 *
 * Threads: the plain build is single-threaded.  The same source is built a
 * second time with -fopenmp for the all-host-cores CPU baseline; then the
 * token-major loops (the dispatch copies and their quantisation, the
 * combines, the expert-choice copy) run their tokens or entries in
 * parallel, each iteration writing its own rows, so the results are the
 * same bytes.  Layout, slots, the inverse map and the rank pack stay serial
 * (a running count), and the OpenMP pragmas are ignored by the plain
 * build.  fp32 is used exactly where the method
 * fixes it (the fp8 scale and the value that is rounded to e4m3); sums are
 * accumulated in fp64 and rounded once.
 *
 * Parity pins (tests/test_oracle_*.py): numpy brute force on tiny inputs,
 * hand-derived fixtures in tests/golden/, closed forms (unit-weight round
 * trip = bf16(multiplicity * x), the amax element encodes to +-448), the
 * e4m3 converter against a nearest-code search and against torch's
 * float8_e4m3fn cast, and the bf16 rounding against torch's cast.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the parallel loops use (1 in the plain build). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 bits -> fp32: the bf16 pattern is the top half of an fp32 pattern. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a real number (given as fp64) to the nearest bf16 value, ties to
 * the even significand, and return its bit pattern.  bf16 keeps 8
 * significant bits and fp32's exponent range; below 2^-126 the spacing is
 * the subnormal quantum 2^-133.  Overflow gives infinity (never reached by
 * in-contract inputs; NaN input is out of contract). */
uint16_t oracle_bf16_from_f64(double v)
{
    if (v == 0.0)
        return signbit(v) ? 0x8000u : 0x0000u;
    double a = fabs(v);
    int e;
    frexp(a, &e);            /* a in [2^(e-1), 2^e) */
    int ex = e - 1;          /* floor(log2(a)) */
    int qexp = (ex < -126) ? -133 : ex - 7;
    double q = nearbyint(ldexp(a, -qexp));   /* exact scaling, then RNE */
    double r = ldexp(q, qexp);
    float f = (float)r;      /* exact: r is a bf16 value (or overflows to inf) */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t h = (uint16_t)(u >> 16);
    return signbit(v) ? (uint16_t)(h | 0x8000u) : h;
}

/* fp32 -> OCP 8-bit E4M3 ("float8_e4m3fn") code, round to nearest, ties to
 * the even code.  E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; no infinities; S.1111.111 is NaN, so the largest finite magnitude is
 * 1.75 * 2^8 = 448; subnormals are m * 2^-9, m = 1..7.
 * Magnitudes >= 464 (the midpoint above 448) saturate to 448 (readings: the
 * format has no infinity, and in-contract inputs never exceed 448*(1+2^-23),
 * which rounds to 448 anyway).  The sign of zero is kept. */
uint8_t oracle_e4m3_from_f32(float v)
{
    uint8_t sign = signbit(v) ? 0x80u : 0x00u;
    double a = fabs((double)v);              /* exact */
    if (a >= 464.0)
        return (uint8_t)(sign | 0x7Eu);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);
    int ex = e - 1;                          /* floor(log2(a)) */
    int qexp = (ex < -6) ? -9 : ex - 3;      /* 4 significant bits, or the subnormal quantum */
    double q = nearbyint(ldexp(a, -qexp));   /* RNE to an integer multiple of 2^qexp */
    double r = ldexp(q, qexp);               /* the chosen e4m3 value */
    if (r == 0.0)
        return sign;
    frexp(r, &e);
    ex = e - 1;                              /* may have carried into the next binade */
    if (ex < -6)                             /* subnormal: r = m * 2^-9 */
        return (uint8_t)(sign | (uint8_t)ldexp(r, 9));
    int m = (int)ldexp(r, 3 - ex) - 8;       /* r = (8 + m) * 2^(ex-3) */
    return (uint8_t)(sign | (uint8_t)(((ex + 7) << 3) | m));
}

/* Value of an E4M3 code (NaN codes return NaN). */
float oracle_e4m3_to_f32(uint8_t c)
{
    int s = (c >> 7) & 1, ef = (c >> 3) & 15, m = c & 7;
    double v;
    if (ef == 15 && m == 7)
        return NAN;
    if (ef == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(8.0 + m, ef - 7 - 3);
    return (float)(s ? -v : v);
}

/* Array forms, for tests. */
void oracle_e4m3_from_f32_array(const float *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_from_f32(in[i]);
}

void oracle_bf16_from_f64_array(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_from_f64(in[i]);
}

/* ------------------------------------------------------------------ */
/* Token choice                                                        */
/* ------------------------------------------------------------------ */

/* Dispatch layout ([EPA] API Overview, get_dispatch_layout; Environment
 * Variables, MOE_EXPERT_TOKEN_NUMS_TYPE and MOE_ENABLE_TOPK_NEG_ONE).
 *   topk_idx [T,K] int32.  -1 = padding (not dispatched).  Any other value
 *   outside [0,E) is invalid: counted in num_invalid and treated like -1.
 *   counts[e]   = number of valid (t,k) with topk_idx[t,k] == e   (count form)
 *   offsets[e]  = sum of counts[0..e-1], offsets[E] = N           (prefix form)
 *   Experts are split into R equal contiguous blocks (rank r owns experts
 *   [r*E/R, (r+1)*E/R)); is_token_in_rank[t,r] = 1 when token t has at least
 *   one valid slot on rank r; tokens_per_rank[r] = sum over t of that.
 * tokens_per_rank / is_token_in_rank may be NULL. */
void oracle_layout(const int32_t *topk_idx, int T, int K, int E, int R,
                   int32_t *counts, int32_t *offsets, int32_t *tokens_per_rank,
                   uint8_t *is_token_in_rank, int32_t *num_invalid)
{
    int per_rank = E / R;
    uint8_t *row = (uint8_t *)calloc((size_t)R, 1);
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    if (tokens_per_rank)
        for (int r = 0; r < R; ++r)
            tokens_per_rank[r] = 0;
    *num_invalid = 0;
    for (int t = 0; t < T; ++t) {
        memset(row, 0, (size_t)R);
        for (int k = 0; k < K; ++k) {
            int32_t e = topk_idx[(int64_t)t * K + k];
            if (e == -1)
                continue;
            if (e < 0 || e >= E) {
                (*num_invalid)++;
                continue;
            }
            counts[e]++;
            row[e / per_rank] = 1;
        }
        for (int r = 0; r < R; ++r) {
            if (is_token_in_rank)
                is_token_in_rank[(int64_t)t * R + r] = row[r];
            if (tokens_per_rank)
                tokens_per_rank[r] += row[r];
        }
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    free(row);
}

/* Slot assignment: the receive row of every (t,k) ([EPA] API Overview,
 * dispatch returns the handle that combine must use; low_latency_dispatch
 * takes a per-expert capacity, num_max_dispatch_tokens_per_rank).
 * Readings: rows of one expert are in ascending (t,k) order (a stable
 * scatter), experts in ascending order.  With r = number of earlier valid
 * (t',k') < (t,k) that chose the same expert e:
 *   contiguous (padded == 0): slot = offsets[e] + r, kept only if
 *       slot < max_rows (the receive buffer's row count);
 *   padded (padded != 0):     slot = e*cap + r, kept only if r < cap.
 * A slot that is not kept is -1 and counts in num_dropped; padding and
 * invalid entries get -1 and are not counted.  recv_src[slot] = t. */
void oracle_slots(const int32_t *topk_idx, int T, int K, int E, int padded,
                  int cap_or_max_rows, int32_t *slot, int32_t *recv_src,
                  int32_t *num_dropped)
{
    int32_t *counts = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int32_t *offsets = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
    int32_t *cursor = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int32_t inval;
    oracle_layout(topk_idx, T, K, E, 1, counts, offsets, NULL, NULL, &inval);
    *num_dropped = 0;
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t i = (int64_t)t * K + k;
            int32_t e = topk_idx[i];
            if (e < 0 || e >= E) {
                slot[i] = -1;
                continue;
            }
            int r = cursor[e]++;
            int64_t s;
            if (padded)
                s = (r < cap_or_max_rows) ? (int64_t)e * cap_or_max_rows + r : -1;
            else
                s = ((int64_t)offsets[e] + r < cap_or_max_rows) ? (int64_t)offsets[e] + r : -1;
            if (s < 0) {
                (*num_dropped)++;
                slot[i] = -1;
                continue;
            }
            slot[i] = (int32_t)s;
            if (recv_src)
                recv_src[s] = t;
        }
    }
    free(counts);
    free(offsets);
    free(cursor);
}

/* bf16 dispatch ([EPA] API Overview, dispatch; Quantization Modes, "bf16"):
 * recv[slot[t,k], :] = x[t, :] for every kept slot.  A byte copy. */
void oracle_dispatch_bf16(const uint16_t *x, int T, int H, const int32_t *slot, int K,
                          uint16_t *recv)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int32_t s = slot[(int64_t)t * K + k];
            if (s < 0)
                continue;
            memcpy(recv + (int64_t)s * H, x + (int64_t)t * H, (size_t)H * sizeof(uint16_t));
        }
}

/* fp8 dispatch ([EPA] Quantization Modes: float8_e4m3fn payload with float32
 * scales).  The 128-channel group and its scale rule are not on the pages
 * (they list per-token and per-32 granularity); the rule taken is:
 * per token t and group g (channels 128g .. 128g+127)
 *   a = max |x|                 (exact)
 *   a == 0: s = 0 and every code is 0x00
 *   else:   s = a / 448         (fp32 division, round to nearest even)
 *           q_i = e4m3(x_i / s) (fp32 division, then the RNE encoder above)
 * and q, s are written to every kept slot of t: recv_q [rows, H] codes,
 * recv_s [rows, H/128] fp32. */
void oracle_dispatch_fp8(const uint16_t *x, int T, int H, const int32_t *slot, int K,
                         uint8_t *recv_q, float *recv_s)
{
    int G = H / 128;
#pragma omp parallel
    {
    uint8_t *q = (uint8_t *)malloc((size_t)H + 1);
    float *s = (float *)malloc(((size_t)G + 1) * sizeof(float));
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
        const uint16_t *xr = x + (int64_t)t * H;
        for (int g = 0; g < G; ++g) {
            float a = 0.0f;
            for (int i = 0; i < 128; ++i) {
                float v = fabsf(oracle_bf16_to_f32(xr[128 * g + i]));
                if (v > a)
                    a = v;
            }
            if (a == 0.0f) {
                s[g] = 0.0f;
                for (int i = 0; i < 128; ++i)
                    q[128 * g + i] = 0x00;
                continue;
            }
            float sg = a / 448.0f;
            s[g] = sg;
            for (int i = 0; i < 128; ++i) {
                float v = oracle_bf16_to_f32(xr[128 * g + i]);
                q[128 * g + i] = oracle_e4m3_from_f32(v / sg);
            }
        }
        for (int k = 0; k < K; ++k) {
            int32_t sl = slot[(int64_t)t * K + k];
            if (sl < 0)
                continue;
            memcpy(recv_q + (int64_t)sl * H, q, (size_t)H);
            memcpy(recv_s + (int64_t)sl * G, s, (size_t)G * sizeof(float));
        }
    }
    free(q);
    free(s);
    }
}

/* ------------------------------------------------------------------ */
/* The other quantisation modes of [EPA] "Quantization Modes in Normal    */
/* Dispatch": INT8 dynamic (int8, float32 scale, per token), scalar FP8   */
/* (float8_e4m3fn, float32 scale, per token), MXFP8 per-block             */
/* (float8_e4m3fn or float8_e5m2 with a float8_e8m0fnu scale per 32       */
/* elements) and MXFP4 (float4_e2m1fn_x2 with the same scales).  The      */
/* table fixes formats and granularities only; the rules taken are stated */
/* at each function.                                                      */
/* ------------------------------------------------------------------ */

/* Round a >= 0 (fp64, exact) to the nearest value of a binary format with
 * `mbits` fraction bits and smallest normal exponent `emin` (so the
 * subnormal quantum is 2^(emin - mbits)), ties to the even significand;
 * results above `maxv` saturate to `maxv`. */
static double round_to_format(double a, int mbits, int emin, double maxv)
{
    if (a == 0.0)
        return 0.0;
    int e;
    frexp(a, &e);
    int ex = e - 1;                                   /* floor(log2(a)) */
    int qexp = (ex < emin) ? emin - mbits : ex - mbits;
    double r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);
    return r > maxv ? maxv : r;
}

/* The code (without sign) of a value r of that format, exponent bias `bias`. */
static unsigned code_of(double r, int mbits, int emin, int bias)
{
    if (r == 0.0)
        return 0u;
    int e;
    frexp(r, &e);
    int ex = e - 1;
    if (ex < emin)                                    /* subnormal: r = m * 2^(emin - mbits) */
        return (unsigned)ldexp(r, mbits - emin);
    unsigned m = (unsigned)ldexp(r, mbits - ex) - (1u << mbits);
    return ((unsigned)(ex + bias) << mbits) | m;
}

/* OCP 8-bit E5M2 ("float8_e5m2"): bias 15, 2 fraction bits, largest finite
 * 1.75 * 2^15 = 57344, subnormals m * 2^-16.  Round to nearest even; the
 * format has infinities, but magnitudes beyond 57344 saturate to it
 * (reading: a quantised payload stays finite, as with E4M3).  Sign of zero
 * kept. */
uint8_t oracle_e5m2_from_f32(float v)
{
    unsigned sign = signbit(v) ? 0x80u : 0u;
    double r = round_to_format(fabs((double)v), 2, -14, 57344.0);
    return (uint8_t)(sign | code_of(r, 2, -14, 15));
}

float oracle_e5m2_to_f32(uint8_t c)
{
    int s = (c >> 7) & 1, ef = (c >> 2) & 31, m = c & 3;
    double v;
    if (ef == 31)
        return m ? NAN : (s ? -INFINITY : INFINITY);
    v = ef == 0 ? ldexp((double)m, -16) : ldexp(4.0 + m, ef - 15 - 2);
    return (float)(s ? -v : v);
}

/* OCP 4-bit E2M1 ("float4_e2m1fn"): bias 1, 1 fraction bit; the magnitudes
 * are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7), bit 3 is the sign.  Round to
 * nearest even; beyond 6 saturates to 6.  Sign of zero kept. */
uint8_t oracle_e2m1_from_f32(float v)
{
    unsigned sign = signbit(v) ? 0x8u : 0u;
    double r = round_to_format(fabs((double)v), 1, 0, 6.0);
    return (uint8_t)(sign | code_of(r, 1, 0, 1));
}

float oracle_e2m1_to_f32(uint8_t c)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double v = mag[c & 7];
    return (float)((c & 8) ? -v : v);
}

/* int8 code of v: round to nearest, ties to even, clamped to [-127, 127]
 * (reading: the symmetric range, so that -q is always a code). */
int8_t oracle_int8_from_f32(float v)
{
    double q = nearbyint((double)v);
    if (q > 127.0)
        q = 127.0;
    if (q < -127.0)
        q = -127.0;
    return (int8_t)q;
}

void oracle_e5m2_from_f32_array(const float *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e5m2_from_f32(in[i]);
}

void oracle_e2m1_from_f32_array(const float *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e2m1_from_f32(in[i]);
}

/* Per-token scaled dispatch: INT8 dynamic (fmt 1) and scalar FP8 (fmt 0).
 * Rule taken (the same shape as the 128-channel fp8 rule, over the whole
 * row): per token t
 *   a = max over the row of |x|                         (exact)
 *   a == 0: s = 0 and every code is 0
 *   else:   s = a / Q  (fp32 division, RNE), Q = 448 (e4m3) or 127 (int8)
 *           q_i = enc(x_i / s)  (fp32 division, then the RNE encoder)
 * recv_q [rows, H] codes (int8 as two's complement bytes), recv_s [rows]. */
void oracle_dispatch_token_quant(const uint16_t *x, int T, int H, const int32_t *slot, int K,
                                 int fmt, uint8_t *recv_q, float *recv_s)
{
    const float Q = fmt == 1 ? 127.0f : 448.0f;
#pragma omp parallel
    {
    uint8_t *q = (uint8_t *)malloc((size_t)H + 1);
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
        const uint16_t *xr = x + (int64_t)t * H;
        float a = 0.0f;
        for (int i = 0; i < H; ++i) {
            float v = fabsf(oracle_bf16_to_f32(xr[i]));
            if (v > a)
                a = v;
        }
        float st = 0.0f;
        if (a == 0.0f) {
            memset(q, 0, (size_t)H);
        } else {
            st = a / Q;
            for (int i = 0; i < H; ++i) {
                float v = oracle_bf16_to_f32(xr[i]) / st;
                q[i] = fmt == 1 ? (uint8_t)oracle_int8_from_f32(v) : oracle_e4m3_from_f32(v);
            }
        }
        for (int k = 0; k < K; ++k) {
            int32_t sl = slot[(int64_t)t * K + k];
            if (sl < 0)
                continue;
            memcpy(recv_q + (int64_t)sl * H, q, (size_t)H);
            recv_s[sl] = st;
        }
    }
    free(q);
    }
}

/* MX dispatch (MXFP8 e4m3: fmt 0, MXFP8 e5m2: fmt 1, MXFP4 e2m1: fmt 2).
 * Rule taken (the shared-scale rule of the OCP microscaling formats): per
 * token and block b of 32 consecutive channels
 *   a = max |x| over the block
 *   E = floor(log2(a)) - emax, emax = 8 (e4m3), 15 (e5m2), 2 (e2m1),
 *       clamped to [-127, 127]; an all-zero block takes E = -127
 *   scale code = E + 127 (float8_e8m0fnu: the value 2^E)
 *   element i = enc(x_i * 2^-E)  (exact power-of-two scaling, then the RNE
 *               encoder, saturating)
 * recv_q rows are H bytes (fp8) or H/2 bytes (fp4: channel 2i in the low
 * nibble of byte i, channel 2i+1 in the high nibble); recv_e [rows, H/32]. */
void oracle_dispatch_mx(const uint16_t *x, int T, int H, const int32_t *slot, int K, int fmt,
                        uint8_t *recv_q, uint8_t *recv_e)
{
    static const int emax_of[3] = {8, 15, 2};
    const int emax = emax_of[fmt];
    const int nb = H / 32;
    const int rb = fmt == 2 ? H / 2 : H;
#pragma omp parallel
    {
    uint8_t *q = (uint8_t *)malloc((size_t)rb + 1);
    uint8_t *ec = (uint8_t *)malloc((size_t)nb + 1);
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
        const uint16_t *xr = x + (int64_t)t * H;
        memset(q, 0, (size_t)rb);
        for (int b = 0; b < nb; ++b) {
            double a = 0.0;
            for (int i = 0; i < 32; ++i) {
                double v = fabs((double)oracle_bf16_to_f32(xr[32 * b + i]));
                if (v > a)
                    a = v;
            }
            int E = -127;
            if (a > 0.0) {
                int e;
                frexp(a, &e);
                E = (e - 1) - emax;
                if (E < -127)
                    E = -127;
                if (E > 127)
                    E = 127;
            }
            ec[b] = (uint8_t)(E + 127);
            for (int i = 0; i < 32; ++i) {
                const int c = 32 * b + i;
                float v = (float)ldexp((double)oracle_bf16_to_f32(xr[c]), -E);
                if (fmt == 0)
                    q[c] = oracle_e4m3_from_f32(v);
                else if (fmt == 1)
                    q[c] = oracle_e5m2_from_f32(v);
                else
                    q[c >> 1] |= (uint8_t)(oracle_e2m1_from_f32(v) << (4 * (c & 1)));
            }
        }
        for (int k = 0; k < K; ++k) {
            int32_t sl = slot[(int64_t)t * K + k];
            if (sl < 0)
                continue;
            memcpy(recv_q + (int64_t)sl * rb, q, (size_t)rb);
            memcpy(recv_e + (int64_t)sl * nb, ec, (size_t)nb);
        }
    }
    free(q);
    free(ec);
    }
}

/* Combine ([EPA] API Overview: combine reduces the dispatched rows through
 * the handle; low_latency_combine also takes topk_weights):
 *   out[t, h] = bf16( sum over k with slot >= 0 of w[t,k] * y[slot[t,k], h] )
 * w == NULL means unit weights (the plain normal-mode sum).  The sum is the
 * exact real sum up to fp64 rounding (products of an fp32 weight and a bf16
 * value are exact in fp64), rounded once to bf16.  A token with no kept slot
 * gives +0. */
void oracle_combine(const uint16_t *y, int H, const int32_t *slot, const float *w,
                    int T, int K, uint16_t *out)
{
#pragma omp parallel
    {
    double *acc = (double *)malloc(((size_t)H + 1) * sizeof(double));
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h)
            acc[h] = 0.0;
        for (int k = 0; k < K; ++k) {
            int32_t s = slot[(int64_t)t * K + k];
            if (s < 0)
                continue;
            double wk = w ? (double)w[(int64_t)t * K + k] : 1.0;
            const uint16_t *yr = y + (int64_t)s * H;
            for (int h = 0; h < H; ++h)
                acc[h] += wk * (double)oracle_bf16_to_f32(yr[h]);
        }
        for (int h = 0; h < H; ++h)
            out[(int64_t)t * H + h] = oracle_bf16_from_f64(acc[h]);
    }
    free(acc);
    }
}

/* ------------------------------------------------------------------ */
/* Expert choice ([ECR] Solution 1)                                    */
/* ------------------------------------------------------------------ */

/* recv[e, c, :] = x[token_indices[e, c], :].  Entries equal to -1 are empty
 * and leave their row untouched; other values outside [0,T) are invalid:
 * counted and skipped (reading).  Duplicates are allowed. */
void oracle_ec_dispatch(const uint16_t *x, int T, int H, const int32_t *token_indices,
                        int E, int C, uint16_t *recv, int32_t *num_invalid)
{
    int32_t inval = 0;
#pragma omp parallel for schedule(static) reduction(+ : inval)
    for (int64_t j = 0; j < (int64_t)E * C; ++j) {
        int32_t i = token_indices[j];
        if (i == -1)
            continue;
        if (i < 0 || i >= T) {
            inval++;
            continue;
        }
        memcpy(recv + j * H, x + (int64_t)i * H, (size_t)H * sizeof(uint16_t));
    }
    *num_invalid = inval;
}

/* Token -> entries map (the inverse of token_indices, kept as the handle for
 * combine): for token t the flat entries j = e*C + c with
 * token_indices[j] == t, ascending in j, stored in
 * tok_ent[tok_off[t] .. tok_off[t+1]); tok_off[T] = number of valid entries. */
void oracle_ec_invert(const int32_t *token_indices, int E, int C, int T,
                      int32_t *tok_off, int32_t *tok_ent)
{
    int64_t n = (int64_t)E * C;
    int32_t *cursor = (int32_t *)calloc((size_t)T + 1, sizeof(int32_t));
    for (int t = 0; t <= T; ++t)
        tok_off[t] = 0;
    for (int64_t j = 0; j < n; ++j) {
        int32_t i = token_indices[j];
        if (i >= 0 && i < T)
            tok_off[i + 1]++;
    }
    for (int t = 0; t < T; ++t)
        tok_off[t + 1] += tok_off[t];
    for (int64_t j = 0; j < n; ++j) {
        int32_t i = token_indices[j];
        if (i >= 0 && i < T)
            tok_ent[tok_off[i] + cursor[i]++] = (int32_t)j;
    }
    free(cursor);
}

/* out[t, h] = bf16( sum over j with token_indices[j] == t, j ascending, of
 * w[j] * y[j, h] ) with y [E*C, H]; tokens that no expert chose give +0.
 * Accumulation as in oracle_combine.  Only tokens in `tokens` (n_tokens of
 * them; NULL = all T in order) are computed, into consecutive rows of out. */
void oracle_ec_combine(const uint16_t *y, const float *w, const int32_t *token_indices,
                       int E, int C, int H, int T, const int32_t *tokens, int n_tokens,
                       uint16_t *out)
{
    int64_t n = (int64_t)E * C;
    int count = tokens ? n_tokens : T;
#pragma omp parallel
    {
    double *acc = (double *)malloc(((size_t)H + 1) * sizeof(double));
#pragma omp for schedule(static)
    for (int o = 0; o < count; ++o) {
        int t = tokens ? tokens[o] : o;
        for (int h = 0; h < H; ++h)
            acc[h] = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            if (token_indices[j] != t)
                continue;
            const uint16_t *yr = y + j * H;
            for (int h = 0; h < H; ++h)
                acc[h] += (double)w[j] * (double)oracle_bf16_to_f32(yr[h]);
        }
        for (int h = 0; h < H; ++h)
            out[(int64_t)o * H + h] = oracle_bf16_from_f64(acc[h]);
    }
    free(acc);
    }
}

/* ------------------------------------------------------------------ */
/* One rank's share of the expert-parallel exchange ([EPA] API         */
/* Overview: get_dispatch_layout returns num_tokens_per_rank and       */
/* is_token_in_rank, dispatch sends the tokens to the ranks of their   */
/* experts and combine reduces what comes back).  Rank r owns experts  */
/* [r*E/R, (r+1)*E/R).  The exchange itself is not here: what a sender */
/* packs for rank r is what rank r receives from it.                   */
/* ------------------------------------------------------------------ */

/* Sender pack: the rows to send, grouped by destination rank.
 * Readings: a token goes once to each rank that holds at least one of its
 * valid entries (the is_token_in_rank of the layout), with its whole row
 * and its entries rewritten for that rank: the local expert id e - r*E/R
 * where the entry's expert is on r, -1 elsewhere (padding and invalid
 * entries included), and the entry's weight (1 when w is NULL; 0 where the
 * id is -1).  Rows are ordered by destination rank, then by token.  With
 * n_r = tokens sent to rank r, rank_offsets[r] = n_0 + ... + n_{r-1}
 * (rank_offsets[R] = all rows); the row of (t, r) is rank_offsets[r] +
 * (number of earlier tokens sent to r), kept only if below max_rows (else
 * counted in num_dropped, as a contiguous receive buffer drops rows).
 *   send_x [rows, H], send_src [rows] = t, send_idx / send_w [rows, K]
 *   (send_w may be NULL), pack_pos [T, R] = the row of (t, r) or -1. */
void oracle_rank_pack(const uint16_t *x, int T, int H, const int32_t *topk_idx, const float *w,
                      int K, int E, int R, int max_rows, int32_t *rank_offsets, uint16_t *send_x,
                      int32_t *send_src, int32_t *send_idx, float *send_w, int32_t *pack_pos,
                      int32_t *num_dropped)
{
    int per_rank = E / R;
    int64_t row = 0;
    *num_dropped = 0;
    for (int64_t i = 0; i < (int64_t)T * R; ++i)
        pack_pos[i] = -1;
    for (int r = 0; r < R; ++r) {
        rank_offsets[r] = (int32_t)row;
        for (int t = 0; t < T; ++t) {
            int on_rank = 0;
            for (int k = 0; k < K; ++k) {
                int32_t e = topk_idx[(int64_t)t * K + k];
                if (e >= 0 && e < E && e / per_rank == r)
                    on_rank = 1;
            }
            if (!on_rank)
                continue;
            int64_t p = row++;
            if (p >= max_rows) {
                (*num_dropped)++;
                continue;
            }
            pack_pos[(int64_t)t * R + r] = (int32_t)p;
            memcpy(send_x + p * H, x + (int64_t)t * H, (size_t)H * sizeof(uint16_t));
            send_src[p] = t;
            for (int k = 0; k < K; ++k) {
                int32_t e = topk_idx[(int64_t)t * K + k];
                int here = e >= 0 && e < E && e / per_rank == r;
                send_idx[p * K + k] = here ? e - r * per_rank : -1;
                if (send_w)
                    send_w[p * K + k] = here ? (w ? w[(int64_t)t * K + k] : 1.0f) : 0.0f;
            }
        }
    }
    rank_offsets[R] = (int32_t)row;
}

/* The receiving rank's combine before the reverse exchange: per received
 * row p, partial[p, h] = sum over k with slot >= 0 of w[p,k] * y[slot[p,k], h]
 * (w NULL = unit weights), taken as the exact sum up to fp64 rounding and
 * rounded once to fp32.  Reading: the partial sums cross the exchange in
 * fp32, the accumulator precision of the combine, so the sender's sum of
 * them is an fp32-accumulated combine as well.  A row with no kept slot
 * gives +0. */
void oracle_combine_partial(const uint16_t *y, int H, const int32_t *slot, const float *w, int S,
                            int K, float *partial)
{
#pragma omp parallel
    {
    double *acc = (double *)malloc(((size_t)H + 1) * sizeof(double));
#pragma omp for schedule(static)
    for (int p = 0; p < S; ++p) {
        for (int h = 0; h < H; ++h)
            acc[h] = 0.0;
        for (int k = 0; k < K; ++k) {
            int32_t s = slot[(int64_t)p * K + k];
            if (s < 0)
                continue;
            double wk = w ? (double)w[(int64_t)p * K + k] : 1.0;
            const uint16_t *yr = y + (int64_t)s * H;
            for (int h = 0; h < H; ++h)
                acc[h] += wk * (double)oracle_bf16_to_f32(yr[h]);
        }
        for (int h = 0; h < H; ++h)
            partial[(int64_t)p * H + h] = (float)acc[h];
    }
    free(acc);
    }
}

/* The sender's final sum after the reverse exchange: for token t,
 * out[t, h] = bf16( sum over r ascending with pack_pos[t,r] in [0, rows) of
 * partial[pack_pos[t,r], h] ), exact up to fp64 rounding, rounded once; a
 * token that no rank received gives +0. */
void oracle_combine_ranks(const float *partial, int rows, int H, const int32_t *pack_pos, int T,
                          int R, uint16_t *out)
{
#pragma omp parallel
    {
    double *acc = (double *)malloc(((size_t)H + 1) * sizeof(double));
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h)
            acc[h] = 0.0;
        for (int r = 0; r < R; ++r) {
            int32_t p = pack_pos[(int64_t)t * R + r];
            if (p < 0 || p >= rows)
                continue;
            for (int h = 0; h < H; ++h)
                acc[h] += (double)partial[(int64_t)p * H + h];
        }
        for (int h = 0; h < H; ++h)
            out[(int64_t)t * H + h] = oracle_bf16_from_f64(acc[h]);
    }
    free(acc);
    }
}
