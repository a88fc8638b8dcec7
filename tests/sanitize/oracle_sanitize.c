/* Drives every function of oracle/oracle.c on seeded random and edge-case
 * inputs, with each buffer malloc'd at exactly the size the function's
 * contract states, so that an AddressSanitizer + UndefinedBehaviorSanitizer
 * build reports any access outside a buffer, leak, signed overflow, bad
 * shift or out-of-range float conversion.  A few cross-checks between the
 * functions' outputs are made as well.  Exit status 0 = clean.
 * Test infrastructure: built and run by tests/test_oracle_sanitize.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_bf16_from_f64(double v);
uint8_t oracle_e4m3_from_f32(float v);
float oracle_e4m3_to_f32(uint8_t c);
uint8_t oracle_e5m2_from_f32(float v);
float oracle_e5m2_to_f32(uint8_t c);
uint8_t oracle_e2m1_from_f32(float v);
float oracle_e2m1_to_f32(uint8_t c);
int8_t oracle_int8_from_f32(float v);
void oracle_layout(const int32_t *topk_idx, int T, int K, int E, int R, int32_t *counts,
                   int32_t *offsets, int32_t *tokens_per_rank, uint8_t *is_token_in_rank,
                   int32_t *num_invalid);
void oracle_slots(const int32_t *topk_idx, int T, int K, int E, int padded, int cap_or_max_rows,
                  int32_t *slot, int32_t *recv_src, int32_t *num_dropped);
void oracle_dispatch_bf16(const uint16_t *x, int T, int H, const int32_t *slot, int K,
                          uint16_t *recv);
void oracle_dispatch_fp8(const uint16_t *x, int T, int H, const int32_t *slot, int K,
                         uint8_t *recv_q, float *recv_s);
void oracle_dispatch_token_quant(const uint16_t *x, int T, int H, const int32_t *slot, int K,
                                 int fmt, uint8_t *recv_q, float *recv_s);
void oracle_dispatch_mx(const uint16_t *x, int T, int H, const int32_t *slot, int K, int fmt,
                        uint8_t *recv_q, uint8_t *recv_e);
void oracle_combine(const uint16_t *y, int H, const int32_t *slot, const float *w, int T, int K,
                    uint16_t *out);
void oracle_ec_dispatch(const uint16_t *x, int T, int H, const int32_t *token_indices, int E,
                        int C, uint16_t *recv, int32_t *num_invalid);
void oracle_ec_invert(const int32_t *token_indices, int E, int C, int T, int32_t *tok_off,
                      int32_t *tok_ent);
void oracle_ec_combine(const uint16_t *y, const float *w, const int32_t *token_indices, int E,
                       int C, int H, int T, const int32_t *tokens, int n_tokens, uint16_t *out);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint32_t rnd(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(rng_state >> 33);
}

static int rnd_int(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }

static void *must(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int failures = 0;

static void expect(int ok, const char *what, int case_no)
{
    if (!ok) {
        fprintf(stderr, "case %d: %s\n", case_no, what);
        failures++;
    }
}

/* A finite bf16 value: zeros, subnormals, ordinary and large magnitudes. */
static uint16_t rnd_bf16(void)
{
    uint32_t kind = rnd() % 16;
    uint16_t sign = (uint16_t)((rnd() & 1u) << 15);
    if (kind == 0)
        return sign;                                          /* +-0 */
    if (kind == 1)
        return (uint16_t)(sign | (rnd() % 0x7Fu + 1u));       /* subnormal */
    if (kind == 2)
        return (uint16_t)(sign | (rnd() % (0x7F7Fu - 0x7000u) + 0x7000u)); /* huge */
    uint16_t e = (uint16_t)rnd_int(100, 140);                 /* ordinary */
    return (uint16_t)(sign | (e << 7) | (rnd() & 0x7Fu));
}

static void token_choice_case(int case_no)
{
    const int T = rnd_int(0, 40), K = rnd_int(1, 9), E = rnd_int(1, 40);
    int R = rnd_int(1, E);
    while (E % R)
        --R;
    const int mode = rnd_int(0, 2);        /* bf16 rows, 128-channel groups, 32-channel blocks */
    const int H = mode == 1 ? 128 * rnd_int(1, 3) : (mode == 2 ? 32 * rnd_int(1, 5) : 8 * rnd_int(1, 40));
    const int64_t TK = (int64_t)T * K;

    int32_t *idx = must((size_t)TK * sizeof(int32_t));
    for (int64_t i = 0; i < TK; ++i) {
        uint32_t u = rnd() % 100;
        idx[i] = u < 10 ? -1 : (u < 14 ? (rnd() & 1 ? E + rnd_int(0, 5) : -2 - rnd_int(0, 5))
                                       : rnd_int(0, E - 1));
    }
    uint16_t *x = must((size_t)T * H * sizeof(uint16_t));
    for (int64_t i = 0; i < (int64_t)T * H; ++i)
        x[i] = rnd_bf16();

    int32_t *counts = must((size_t)E * sizeof(int32_t));
    int32_t *offsets = must(((size_t)E + 1) * sizeof(int32_t));
    int32_t *tpr = must((size_t)R * sizeof(int32_t));
    uint8_t *itr = must((size_t)T * R);
    int32_t ninv = -1;
    oracle_layout(idx, T, K, E, R, counts, offsets, rnd() & 1 ? tpr : NULL,
                  rnd() & 1 ? itr : NULL, &ninv);
    oracle_layout(idx, T, K, E, R, counts, offsets, tpr, itr, &ninv);
    int64_t valid = 0, inval = 0;
    for (int64_t i = 0; i < TK; ++i) {
        valid += idx[i] >= 0 && idx[i] < E;
        inval += idx[i] != -1 && (idx[i] < 0 || idx[i] >= E);
    }
    expect(offsets[E] == valid, "offsets[E] is the number of valid entries", case_no);
    expect(ninv == inval, "num_invalid", case_no);

    const int padded = rnd() & 1;
    const int cap = padded ? rnd_int(0, 6) : (rnd() & 1 ? (int)TK : rnd_int(0, (int)valid + 1));
    const int64_t rows = padded ? (int64_t)E * cap : cap;
    int32_t *slot = must((size_t)TK * sizeof(int32_t));
    int32_t *src = must((size_t)rows * sizeof(int32_t));
    int32_t nd = -1;
    oracle_slots(idx, T, K, E, padded, cap, slot, src, &nd);
    for (int64_t i = 0; i < TK; ++i)
        expect(slot[i] >= -1 && slot[i] < rows, "slot inside the receive rows", case_no);

    uint16_t *recv = must((size_t)rows * H * sizeof(uint16_t));
    memset(recv, 0, (size_t)rows * H * sizeof(uint16_t));
    oracle_dispatch_bf16(x, T, H, slot, K, recv);
    float *w = must((size_t)TK * sizeof(float));
    for (int64_t i = 0; i < TK; ++i)
        w[i] = (float)(rnd() % 1000) / 997.0f;
    uint16_t *out = must((size_t)T * H * sizeof(uint16_t));
    oracle_combine(recv, H, slot, rnd() & 1 ? w : NULL, T, K, out);

    if (mode == 1) {
        uint8_t *q = must((size_t)rows * H);
        float *s = must((size_t)rows * (H / 128) * sizeof(float));
        oracle_dispatch_fp8(x, T, H, slot, K, q, s);
        free(q);
        free(s);
    }
    for (int fmt = 0; fmt < 2; ++fmt) {
        uint8_t *q = must((size_t)rows * H);
        float *s = must((size_t)rows * sizeof(float));
        oracle_dispatch_token_quant(x, T, H, slot, K, fmt, q, s);
        free(q);
        free(s);
    }
    if (mode == 2)
        for (int fmt = 0; fmt < 3; ++fmt) {
            const int rb = fmt == 2 ? H / 2 : H;
            uint8_t *q = must((size_t)rows * rb);
            uint8_t *e = must((size_t)rows * (H / 32));
            oracle_dispatch_mx(x, T, H, slot, K, fmt, q, e);
            free(q);
            free(e);
        }
    free(idx);
    free(x);
    free(counts);
    free(offsets);
    free(tpr);
    free(itr);
    free(slot);
    free(src);
    free(recv);
    free(w);
    free(out);
}

static void expert_choice_case(int case_no)
{
    const int T = rnd_int(0, 50), E = rnd_int(1, 12), C = rnd_int(1, 12), H = 8 * rnd_int(1, 20);
    const int64_t n = (int64_t)E * C;
    int32_t *ti = must((size_t)n * sizeof(int32_t));
    for (int64_t j = 0; j < n; ++j) {
        uint32_t u = rnd() % 100;
        ti[j] = u < 10 ? -1 : (u < 14 ? T + rnd_int(0, 3) : (T ? rnd_int(0, T - 1) : -1));
    }
    uint16_t *x = must((size_t)T * H * sizeof(uint16_t));
    for (int64_t i = 0; i < (int64_t)T * H; ++i)
        x[i] = rnd_bf16();
    uint16_t *recv = must((size_t)n * H * sizeof(uint16_t));
    memset(recv, 0, (size_t)n * H * sizeof(uint16_t));
    int32_t ninv = -1;
    oracle_ec_dispatch(x, T, H, ti, E, C, recv, &ninv);
    int32_t *off = must(((size_t)T + 1) * sizeof(int32_t));
    int32_t *ent = must((size_t)n * sizeof(int32_t));
    oracle_ec_invert(ti, E, C, T, off, ent);
    int64_t valid = 0;
    for (int64_t j = 0; j < n; ++j)
        valid += ti[j] >= 0 && ti[j] < T;
    expect(off[T] == valid, "tok_off[T] is the number of valid entries", case_no);
    float *w = must((size_t)n * sizeof(float));
    for (int64_t j = 0; j < n; ++j)
        w[j] = (float)(rnd() % 1000) / 991.0f;
    uint16_t *out = must((size_t)T * H * sizeof(uint16_t));
    oracle_ec_combine(recv, w, ti, E, C, H, T, NULL, 0, out);
    if (T > 0) {
        int32_t some[3] = {rnd_int(0, T - 1), rnd_int(0, T - 1), T - 1};
        uint16_t *out3 = must((size_t)3 * H * sizeof(uint16_t));
        oracle_ec_combine(recv, w, ti, E, C, H, T, some, 3, out3);
        expect(memcmp(out3 + 2 * H, out + (int64_t)(T - 1) * H, (size_t)H * 2) == 0,
               "a listed token's row equals the full combine's", case_no);
        free(out3);
    }
    free(ti);
    free(x);
    free(recv);
    free(off);
    free(ent);
    free(w);
    free(out);
}

static void encoders(void)
{
    /* every 4099th fp32 pattern, both signs, all finite; plus the bf16 set */
    for (uint64_t b = 0; b < 0x7F800000ull; b += 4099) {
        for (uint32_t sgn = 0; sgn < 2; ++sgn) {
            uint32_t bits = (uint32_t)b | (sgn << 31);
            float v;
            memcpy(&v, &bits, sizeof v);
            uint8_t c = oracle_e4m3_from_f32(v);
            (void)oracle_e4m3_to_f32(c);
            c = oracle_e5m2_from_f32(v);
            (void)oracle_e5m2_to_f32(c);
            c = oracle_e2m1_from_f32(v);
            (void)oracle_e2m1_to_f32(c);
            (void)oracle_int8_from_f32(v);
            (void)oracle_bf16_from_f64((double)v);
        }
    }
    for (uint32_t b = 0; b < 0x10000u; ++b)
        if ((b & 0x7F80u) != 0x7F80u)
            (void)oracle_bf16_from_f64((double)oracle_bf16_to_f32((uint16_t)b));
    const double edges[] = {0.0, -0.0, 1e-300, -1e-300, 1e300, -1e300, 3.3895313892515355e38,
                            3.4e38, -3.4e38, INFINITY, -INFINITY};
    for (size_t i = 0; i < sizeof edges / sizeof edges[0]; ++i)
        (void)oracle_bf16_from_f64(edges[i]);
    const float fedges[] = {INFINITY, -INFINITY, 3.4e38f, -3.4e38f, 127.5f, -127.5f, 128.0f};
    for (size_t i = 0; i < sizeof fedges / sizeof fedges[0]; ++i) {
        (void)oracle_int8_from_f32(fedges[i]);
        (void)oracle_e4m3_from_f32(fedges[i]);
        (void)oracle_e5m2_from_f32(fedges[i]);
        (void)oracle_e2m1_from_f32(fedges[i]);
    }
}

int main(void)
{
    encoders();
    for (int i = 0; i < 400; ++i)
        token_choice_case(i);
    for (int i = 0; i < 200; ++i)
        expert_choice_case(i);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitize run clean\n");
    return 0;
}
