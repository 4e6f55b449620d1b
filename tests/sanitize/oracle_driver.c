/* Drives every function of the C oracle on small inputs (worked examples,
 * random vectors with ties and zeros, empty and one-element segments,
 * corrupt streams) so that a build with -fsanitize=address,undefined sees
 * each memory access and integer operation they make.  Exit status 0 when
 * every check holds; a sanitizer report aborts the run.                    */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t orc_keep_count(int64_t n, uint32_t ppm);
int64_t orc_sample_count(int64_t n, uint32_t sample_div, uint32_t sample_min);
int64_t orc_warmup_ppm(int64_t t, int64_t steps, uint32_t start, uint32_t end);
double orc_rice_expected_bits(int32_t b, double p);
int32_t orc_rice_param(double p);
void orc_accumulate(const float* g, float* r, int64_t n);
void orc_momentum_correct(float beta, const float* g, float* u, int64_t n);
void orc_momentum_mask(float* u, const int32_t* sent_idx, int64_t count);
int64_t orc_compress_exact(const float* g, float* r, const int64_t* seg_off, int32_t nseg, int32_t scope,
                           uint32_t ppm, int32_t* out_idx, float* out_val, int64_t cap, int64_t* out_counts);
int64_t orc_compress_sampled(const float* g, float* r, const int64_t* seg_off, int32_t nseg, int32_t scope,
                             uint32_t ppm, uint32_t sample_div, uint32_t sample_min, int32_t* out_idx,
                             float* out_val, int64_t cap, int64_t* out_counts, uint32_t* status);
int64_t orc_binarize(const int32_t* idx, const float* val, const int64_t* counts, int32_t nseg, int32_t mode,
                     float* r, int32_t* out_idx, int64_t* out_counts, float* out_means, uint32_t* out_codes);
int32_t orc_encode(const int32_t* idx, const int64_t* counts, const int64_t* seg_off, int32_t nseg,
                   int32_t scope, int32_t b, uint32_t* words, int64_t word_cap, uint64_t* word_off,
                   uint64_t* nbits, uint64_t* chunk_off, int64_t chunk_cap);
int32_t orc_decode_stream(const uint32_t* words, uint64_t nbits, int64_t count, int32_t b, int64_t numel,
                          const uint64_t* chunk_off, int64_t* out_pos, uint32_t* status);
int32_t orc_accumulate_message(float* out, const int64_t* seg_off, int32_t nseg, int32_t golomb, int32_t scope,
                               int32_t b, int32_t vkind, const int64_t* counts, const int32_t* idx,
                               const float* val, const uint32_t* codes, const float* means,
                               const uint32_t* words, const uint64_t* word_off, const uint64_t* nbits,
                               const uint64_t* chunk_off, uint32_t* status);

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 11);
}
static float draw(void)
{
    static const float vals[] = {0.0f, -0.0f, 0.5f, -0.5f, 0.25f, -1.0f, 3.0f, 1e-40f, -2.0f};
    uint32_t u = next_u32();
    if (u % 3 == 0) return vals[(u >> 8) % 9];
    return ((float)(u % 20001) - 10000.0f) * 1e-4f;
}

/* One case: a random layout, a compress (exact or sampled, either scope),
 * binarize (SBC / 2-bit), encode with every scope, decode and accumulate. */
static void one_case(int nseg, const int64_t* sizes, uint32_t ppm, int sampled, int scope, int b)
{
    int64_t seg_off[16];
    seg_off[0] = 0;
    for (int t = 0; t < nseg; ++t) seg_off[t + 1] = seg_off[t] + sizes[t];
    const int64_t n = seg_off[nseg];
    const int64_t m = n > 0 ? n : 1;
    float* g = malloc(m * sizeof(float));
    float* r = malloc(m * sizeof(float));
    float* u = malloc(m * sizeof(float));
    int32_t* idx = malloc(m * sizeof(int32_t));
    float* val = malloc(m * sizeof(float));
    int64_t counts[17];
    for (int64_t i = 0; i < n; ++i) {
        g[i] = draw();
        r[i] = draw();
        u[i] = draw();
    }
    orc_momentum_correct(0.9f, g, u, n);
    orc_accumulate(g, r, n);
    int64_t got;
    uint32_t st = 0;
    if (sampled)
        got = orc_compress_sampled(u, r, seg_off, nseg, scope, ppm, 7, 5, idx, val, n, counts, &st);
    else
        got = orc_compress_exact(u, r, seg_off, nseg, scope, ppm, idx, val, n, counts);
    CHECK(got >= 0 && got == counts[nseg]);
    if (got < 0) goto done;
    orc_momentum_mask(u, idx, got);
    for (int64_t j = 1; j < got; ++j) CHECK(idx[j] > idx[j - 1]);

    /* SBC and 2-bit on copies of the residual */
    {
        float* r2 = malloc(m * sizeof(float));
        int32_t* oidx = malloc((got > 0 ? got : 1) * sizeof(int32_t));
        uint32_t* codes = malloc(((got + 15) / 16 + 1) * sizeof(uint32_t));
        float means[32];
        int64_t oc[17];
        memcpy(r2, r, m * sizeof(float));
        int64_t sent = orc_binarize(idx, val, counts, nseg, 0, r2, oidx, oc, means, codes);
        CHECK(sent >= 0 && sent <= got);
        memcpy(r2, r, m * sizeof(float));
        CHECK(orc_binarize(idx, val, counts, nseg, 1, r2, oidx, oc, means, codes) == got);
        /* 2-bit message accumulated raw */
        float* out = calloc(m, sizeof(float));
        uint32_t ast = 0;
        CHECK(orc_accumulate_message(out, seg_off, nseg, 0, 0, 0, 2, oc, idx, NULL, codes, means, NULL, NULL,
                                     NULL, NULL, &ast) == 0);
        CHECK(ast == 0);
        free(out);
        free(r2);
        free(oidx);
        free(codes);
    }

    /* Rice: both scopes, round trip through the decoder and the accumulator */
    for (int sc = 0; sc < 2; ++sc) {
        const int ns = sc == 0 ? 1 : nseg;
        const int64_t wcap = (got * (b + 1) + n) / 32 + 2 * ns + 2;
        const int64_t ccap = 2 * (got / 256 + ns + 1);
        uint32_t* words = malloc(wcap * sizeof(uint32_t));
        uint64_t word_off[17], nbits[16];
        uint64_t* chunk = malloc(ccap * sizeof(uint64_t));
        CHECK(orc_encode(idx, counts, seg_off, nseg, sc, b, words, wcap, word_off, nbits, chunk, ccap) == 0);
        if (sc == 0) {
            int64_t* pos = malloc((got > 0 ? got : 1) * sizeof(int64_t));
            uint32_t dst = 0;
            orc_decode_stream(words, nbits[0], got, b, n, chunk, pos, &dst);
            CHECK(dst == 0);
            for (int64_t j = 0; j < got && dst == 0; ++j) CHECK(pos[j] == idx[j]);
            /* a stream cut short by one bit is corrupt, and reads stay inside it */
            if (nbits[0] > 0) {
                dst = 0;
                orc_decode_stream(words, nbits[0] - 1, got, b, n, NULL, pos, &dst);
                CHECK(dst != 0);
            }
            free(pos);
        }
        float* out = calloc(m, sizeof(float));
        uint32_t ast = 0;
        CHECK(orc_accumulate_message(out, seg_off, nseg, 1, sc, b, 0, counts, NULL, val, NULL, NULL, words,
                                     word_off, nbits, chunk, &ast) == 0);
        CHECK(ast == 0);
        for (int64_t j = 0; j < got; ++j) CHECK(memcmp(&out[idx[j]], &val[j], 4) == 0 || val[j] == 0.0f);
        free(out);
        free(words);
        free(chunk);
    }
done:
    free(g);
    free(r);
    free(u);
    free(idx);
    free(val);
}

int main(void)
{
    CHECK(orc_keep_count(1 << 20, 10000) == 10486);
    CHECK(orc_keep_count(0, 10000) == 0);
    CHECK(orc_sample_count(65537, 1000, 65536) == 65536);
    CHECK(orc_warmup_ppm(1, 6, 250000, 1000) == 82861);
    CHECK(orc_warmup_ppm(-1, 6, 250000, 1000) == -1);
    CHECK(orc_rice_param(0.01) == 6);
    CHECK(fabs(orc_rice_expected_bits(7, 0.01) - 8.3817) < 1e-3);

    static const uint32_t ppms[] = {0, 1, 100000, 250000, 500000, 999999, 1000000};
    for (int c = 0; c < 300; ++c) {
        int nseg = 1 + (int)(next_u32() % 5);
        int64_t sizes[16];
        for (int t = 0; t < nseg; ++t) sizes[t] = next_u32() % 4 == 0 ? 0 : (int64_t)(next_u32() % 700);
        one_case(nseg, sizes, ppms[next_u32() % 7], (int)(next_u32() & 1), (int)(next_u32() & 1),
                 (int)(next_u32() % 11));
    }
    /* a corrupt 2-bit code (3) and out-of-range raw indices are flagged */
    {
        int64_t seg_off[2] = {0, 8}, counts[2] = {2, 2};
        int32_t idx[2] = {1, 9};
        float val[2] = {1.0f, 2.0f}, out[8] = {0};
        uint32_t st = 0;
        CHECK(orc_accumulate_message(out, seg_off, 1, 0, 0, 0, 0, counts, idx, val, NULL, NULL, NULL, NULL, NULL,
                                     NULL, &st) == 0);
        CHECK(st != 0);
        uint32_t codes[1] = {0xF};
        float means[2] = {1.0f, -1.0f};
        int32_t idx2[2] = {1, 2};
        st = 0;
        CHECK(orc_accumulate_message(out, seg_off, 1, 0, 0, 0, 2, counts, idx2, NULL, codes, means, NULL, NULL,
                                     NULL, NULL, &st) == 0);
        CHECK(st != 0);
    }
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver ok\n");
    return 0;
}
