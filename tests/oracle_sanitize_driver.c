/*
 * Drives every entry point of the CPU oracle (oracle/stv_oracle.c) on small
 * inputs that reach its edge cases, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles and
 * runs it).  The sanitizers check memory safety and defined behaviour, the
 * property the elpis-lossless page assumes of its kernels ("Trust base":
 * H_mem); the driver adds a few invariants of its own on the way:
 *   - every code at every position of a block reads back as written;
 *   - a chain tree equals the causal chunk bit for bit;
 *   - partials over a partition of the keys merge to the whole call;
 *   - a commit of the identity path leaves the cache unchanged.
 * Exit status 0 when all hold; the sanitizers abort on their own findings.
 * Inputs come from a fixed linear congruential generator.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_code_get(const uint32_t *w, int e);
void orc_code_set(uint32_t *w, int e, int code);
uint16_t orc_f32_to_f16(float x);
double orc_f16_to_f64(uint16_t h);
void orc_quantize_q_row(const float *q, int D, int8_t *qi8, float *sq);
uint16_t orc_quantize_kv_block(const float *x, uint32_t *w);
void orc_k_quant_pack(const float *x, int n_tok, int pos0, uint32_t *codes, uint16_t *scales,
                      int Hkv, int D, int cap);
void orc_v_quant_pack(const float *x, int n_tok, int pos0, uint32_t *codes, uint16_t *scales,
                      int Hkv, int D, int cap);
int orc_attention(const float *q, int T, int Hq, const uint32_t *kc, const uint16_t *ks,
                  const uint32_t *vc, const uint16_t *vs, int Hkv, int D, int cap, int L,
                  const uint64_t *mask, double scale, int k_begin, int k_end,
                  const int32_t *rows, int n_rows, double *out, double *lse, int64_t *logits,
                  int8_t *qi8_out, float *sq_out);
int orc_set_threads(int n);
void orc_merge(const double *part_o, const double *part_lse, int S, int rows, int D,
               double *out, double *out_lse);
int orc_tree_accept(const uint64_t *mask, int T, const int32_t *draft, const int32_t *target,
                    int32_t *path, int32_t *bonus);
int orc_kv_commit(uint32_t *kc, uint16_t *ks, uint32_t *vc, uint16_t *vs, int Hkv, int D,
                  int cap, int L, int T, const int32_t *path, int n);
void orc_lookup_draft(const int32_t *hist, const int32_t *len, int B, int stride, int n_min,
                      int n_max, int k, int32_t *tokens, int32_t *count, int32_t *match,
                      int32_t *pos);
uint16_t orc_quantize_kv4_row(const float *x, int D, uint32_t *w);
void orc_k4_quant_pack(const float *x, int n_tok, int pos0, uint32_t *codes, uint16_t *scales,
                       int Hkv, int D, int cap);
void orc_v4_quant_pack(const float *x, int n_tok, int pos0, uint32_t *codes, uint16_t *scales,
                       int Hkv, int D, int cap);
int orc_attention_i4(const float *q, int T, int Hq, const uint32_t *kc, const uint16_t *ks,
                     const uint32_t *vc, const uint16_t *vs, int Hkv, int D, int cap, int L,
                     const uint64_t *mask, double scale, int k_begin, int k_end,
                     const int32_t *rows, int n_rows, double *out, double *lse,
                     int64_t *logits, int8_t *qi8_out, float *sq_out);
int orc_kv4_commit(uint32_t *kc, uint16_t *ks, uint32_t *vc, uint16_t *vs, int Hkv, int D,
                   int cap, int L, int T, const int32_t *path, int n);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(rng_state >> 32);
}
static float next_normalish(void)
{
    /* sum of four uniforms, centred: enough spread for quantizer inputs */
    float s = 0.0f;
    for (int i = 0; i < 4; ++i)
        s += (float)(next_u32() >> 8) / 16777216.0f;
    return (s - 2.0f) * 1.7f;
}

static int failures = 0;
#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);          \
            fprintf(stderr, __VA_ARGS__);                                 \
            fprintf(stderr, "\n");                                        \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static void *xcalloc(size_t n, size_t sz)
{
    void *p = calloc(n ? n : 1, sz);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void test_codes_and_fp16(void)
{
    for (int e = 0; e < 32; ++e)
        for (int c = 0; c < 8; ++c) {
            uint32_t w[3] = {next_u32(), next_u32(), next_u32()};
            orc_code_set(w, e, c);
            CHECK(orc_code_get(w, e) == c, "code %d at %d", c, e);
        }
    const float xs[] = {0.0f, -0.0f, 1e-8f, 5.96e-8f, 6.1e-5f, 1.0f, 65504.0f, 65520.0f,
                        1e30f, -3.5f, INFINITY, NAN};
    for (size_t i = 0; i < sizeof xs / sizeof xs[0]; ++i) {
        uint16_t h = orc_f32_to_f16(xs[i]);
        double back = orc_f16_to_f64(h);
        if (isfinite(xs[i]) && fabsf(xs[i]) <= 65504.0f)
            CHECK(fabs(back - xs[i]) <= fabs(xs[i]) * 1e-3 + 6e-8, "fp16 of %g", xs[i]);
    }
}

static void test_quantizers(void)
{
    for (int D = 32; D <= 256; D *= 2) {
        float *q = xcalloc(D, sizeof(float));
        int8_t *qi = xcalloc(D, 1);
        float sq = -1.0f;
        orc_quantize_q_row(q, D, qi, &sq);                /* zero row */
        CHECK(sq == 0.0f && qi[0] == 0, "zero row");
        for (int i = 0; i < D; ++i)
            q[i] = next_normalish();
        orc_quantize_q_row(q, D, qi, &sq);
        CHECK(sq > 0.0f, "scale of a normal row");
        free(q);
        free(qi);
    }
    float blk[32];
    uint32_t w[3];
    const float mags[] = {0.0f, 1e-9f, 1e-3f, 1.0f, 1e6f};
    for (size_t m = 0; m < sizeof mags / sizeof mags[0]; ++m) {
        for (int i = 0; i < 32; ++i)
            blk[i] = next_normalish() * mags[m];
        uint16_t s = orc_quantize_kv_block(blk, w);
        for (int i = 0; i < 32; ++i)
            CHECK(orc_code_get(w, i) >= 0 && orc_code_get(w, i) <= 7, "code range");
        (void)s;
    }
    float row[256];
    uint32_t w4[32];
    for (int i = 0; i < 256; ++i)
        row[i] = next_normalish();
    (void)orc_quantize_kv4_row(row, 256, w4);
}

/* One cache of either format, filled by the oracle's own pack, then
 * attention in every mode the entry point offers. */
static void test_attention(int four_bit, int Hq, int Hkv, int D, int L, int T)
{
    int nb = D / 32, cap = L + T + 3, ng = (cap + 31) / 32, N = L + T;
    size_t kwords = four_bit ? (size_t)Hkv * cap * (D / 8) : (size_t)Hkv * cap * nb * 3;
    size_t vwords = four_bit ? (size_t)Hkv * ng * D * 4 : (size_t)Hkv * ng * D * 3;
    size_t kscales = four_bit ? (size_t)Hkv * cap : (size_t)Hkv * cap * nb;
    size_t vscales = four_bit ? (size_t)Hkv * cap : (size_t)Hkv * ng * nb * 32;
    uint32_t *kc = xcalloc(kwords, 4), *vc = xcalloc(vwords, 4);
    uint16_t *ks = xcalloc(kscales, 2), *vs = xcalloc(vscales, 2);
    float *x = xcalloc((size_t)N * Hkv * D, sizeof(float));
    for (size_t i = 0; i < (size_t)N * Hkv * D; ++i)
        x[i] = next_normalish();
    /* appends in two ragged pieces */
    int cut = L / 3 + 1 < N ? L / 3 + 1 : N;
    if (four_bit) {
        orc_k4_quant_pack(x, cut, 0, kc, ks, Hkv, D, cap);
        orc_k4_quant_pack(x + (size_t)cut * Hkv * D, N - cut, cut, kc, ks, Hkv, D, cap);
        orc_v4_quant_pack(x, cut, 0, vc, vs, Hkv, D, cap);
        orc_v4_quant_pack(x + (size_t)cut * Hkv * D, N - cut, cut, vc, vs, Hkv, D, cap);
    } else {
        orc_k_quant_pack(x, cut, 0, kc, ks, Hkv, D, cap);
        orc_k_quant_pack(x + (size_t)cut * Hkv * D, N - cut, cut, kc, ks, Hkv, D, cap);
        orc_v_quant_pack(x, cut, 0, vc, vs, Hkv, D, cap);
        orc_v_quant_pack(x + (size_t)cut * Hkv * D, N - cut, cut, vc, vs, Hkv, D, cap);
    }
    float *q = xcalloc((size_t)T * Hq * D, sizeof(float));
    for (size_t i = 0; i < (size_t)T * Hq * D; ++i)
        q[i] = next_normalish();
    memset(q, 0, (size_t)D * sizeof(float));                 /* a zero row */

    int R = T * Hq;
    double *out = xcalloc((size_t)R * D, 8), *out2 = xcalloc((size_t)R * D, 8);
    double *lse = xcalloc(R, 8), *lse2 = xcalloc(R, 8);
    size_t nlog = four_bit ? (size_t)R * N : (size_t)R * N * nb;
    int64_t *logits = xcalloc(nlog, 8);
    int8_t *qi8 = xcalloc((size_t)R * D, 1);
    float *sq = xcalloc(R, sizeof(float));
    uint64_t *chain = xcalloc(T, 8), *forest = xcalloc(T, 8);
    for (int i = 0; i < T; ++i) {
        chain[i] = i == 63 ? ~0ull : ((1ull << (i + 1)) - 1);
        /* a forest: every third row starts a new tree, others hang below i-1 */
        forest[i] = (i % 3 == 0 || i == 0) ? (1ull << i) : (forest[i - 1] | (1ull << i));
    }
    int (*attn)(const float *, int, int, const uint32_t *, const uint16_t *, const uint32_t *,
                const uint16_t *, int, int, int, int, const uint64_t *, double, int, int,
                const int32_t *, int, double *, double *, int64_t *, int8_t *, float *) =
        four_bit ? orc_attention_i4 : orc_attention;
    double scale = 1.0 / sqrt((double)D);

    CHECK(attn(q, T, Hq, kc, ks, vc, vs, Hkv, D, cap, L, chain, scale, 0, N, NULL, 0, out, lse,
               logits, qi8, sq) == 0, "chain");
    CHECK(attn(q, T, Hq, kc, ks, vc, vs, Hkv, D, cap, L, NULL, scale, 0, N, NULL, 0, out2,
               lse2, NULL, NULL, NULL) == 0, "causal");
    CHECK(memcmp(out, out2, (size_t)R * D * 8) == 0 && memcmp(lse, lse2, (size_t)R * 8) == 0,
          "chain equals causal");
    CHECK(attn(q, T, Hq, kc, ks, vc, vs, Hkv, D, cap, L, forest, scale, 0, N, NULL, 0, out,
               lse, logits, qi8, sq) == 0, "forest");

    /* partials over three ranges (one may be empty) merge to the whole */
    int cuts[4] = {0, N / 3, N / 3, N};
    double *po = xcalloc((size_t)3 * R * D, 8), *pl = xcalloc((size_t)3 * R, 8);
    for (int s = 0; s < 3; ++s)
        CHECK(attn(q, T, Hq, kc, ks, vc, vs, Hkv, D, cap, L, forest, scale, cuts[s],
                   cuts[s + 1], NULL, 0, po + (size_t)s * R * D, pl + (size_t)s * R, NULL, NULL,
                   NULL) == 0, "partial %d", s);
    orc_merge(po, pl, 3, R, D, out2, lse2);
    for (size_t i = 0; i < (size_t)R * D; ++i)
        CHECK(fabs(out2[i] - out[i]) <= 1e-12 * (1.0 + fabs(out[i])), "merge %zu", i);

    /* a subset of rows, in reverse order */
    int32_t rows[3] = {R - 1, R / 2, 0};
    int n_list = R < 3 ? R : 3;                     /* outputs hold R rows */
    CHECK(attn(q, T, Hq, kc, ks, vc, vs, Hkv, D, cap, L, forest, scale, 0, N, rows, n_list,
               out2, lse2, logits, qi8, sq) == 0, "rows");
    /* rejected arguments: a kv head count that does not divide Hq */
    CHECK(attn(q, T, Hq, kc, ks, vc, vs, Hq + 1, D, cap, L, forest, scale, 0, N, NULL, 0, out,
               lse, NULL, NULL, NULL) != 0, "bad head counts rejected");

    /* commit: identity path leaves the cache as it was; a real path moves */
    if (T >= 2) {
        int32_t path[64];
        for (int i = 0; i < T; ++i)
            path[i] = i;
        uint32_t *kc0 = xcalloc(kwords, 4), *vc0 = xcalloc(vwords, 4);
        memcpy(kc0, kc, kwords * 4);
        memcpy(vc0, vc, vwords * 4);
        int rc = four_bit ? orc_kv4_commit(kc, ks, vc, vs, Hkv, D, cap, L, T, path, T)
                          : orc_kv_commit(kc, ks, vc, vs, Hkv, D, cap, L, T, path, T);
        CHECK(rc == 0 && memcmp(kc0, kc, kwords * 4) == 0 && memcmp(vc0, vc, vwords * 4) == 0,
              "identity commit");
        path[0] = 0;
        path[1] = T - 1;
        rc = four_bit ? orc_kv4_commit(kc, ks, vc, vs, Hkv, D, cap, L, T, path, 2)
                      : orc_kv_commit(kc, ks, vc, vs, Hkv, D, cap, L, T, path, 2);
        CHECK(rc == 0, "commit of two");
        path[1] = T;                                    /* out of range: rejected */
        rc = four_bit ? orc_kv4_commit(kc, ks, vc, vs, Hkv, D, cap, L, T, path, 2)
                      : orc_kv_commit(kc, ks, vc, vs, Hkv, D, cap, L, T, path, 2);
        CHECK(rc != 0, "bad path rejected");
        free(kc0);
        free(vc0);
    }
    free(po); free(pl); free(chain); free(forest); free(sq); free(qi8); free(logits);
    free(lse2); free(lse); free(out2); free(out); free(q); free(x);
    free(vs); free(ks); free(vc); free(kc);
}

static void test_merge_edges(void)
{
    enum { S = 4, R = 5, D = 7 };
    double po[S * R * D], pl[S * R], out[R * D], ol[R];
    for (int i = 0; i < S * R * D; ++i)
        po[i] = next_normalish();
    for (int i = 0; i < S * R; ++i)
        pl[i] = (next_u32() % 3 == 0) ? -INFINITY : next_normalish() * 4.0;
    for (int s = 0; s < S; ++s)
        pl[s * R] = -INFINITY;                          /* a row no split saw */
    orc_merge(po, pl, S, R, D, out, ol);
    CHECK(ol[0] == -INFINITY && out[0] == 0.0, "empty row");
    orc_merge(po, pl, S, R, D, out, NULL);
}

static void test_accept_and_lookup(void)
{
    uint64_t mask[64];
    int32_t draft[64], target[64], path[64], bonus;
    for (int T = 1; T <= 64; T += 9) {
        for (int i = 0; i < T; ++i) {
            int p = i == 0 ? -1 : (int)(next_u32() % (unsigned)i);
            if (i > 0 && next_u32() % 7 == 0)
                p = -1;                                 /* a second root */
            mask[i] = (p < 0 ? 0 : mask[p]) | (1ull << i);
            draft[i] = (int32_t)(next_u32() % 3);
            target[i] = (int32_t)(next_u32() % 3);
        }
        int n = orc_tree_accept(mask, T, draft, target, path, &bonus);
        CHECK(n >= 1 && n <= T, "accept n");
    }
    CHECK(orc_tree_accept(mask, 0, draft, target, path, &bonus) == 0, "T = 0 rejected");

    enum { B = 4, STRIDE = 300, K = 8 };
    int32_t *hist = xcalloc((size_t)B * STRIDE, 4);
    int32_t len[B] = {0, 1, 13, STRIDE + 5};            /* empty, one, short, clamped */
    for (int i = 0; i < B * STRIDE; ++i)
        hist[i] = (int32_t)(next_u32() % 4);
    int32_t tokens[B * K], count[B], match[B], pos[B];
    orc_lookup_draft(hist, len, B, STRIDE, 1, 12, K, tokens, count, match, pos);
    CHECK(count[0] == 0 && pos[0] == -1, "empty history");
    orc_lookup_draft(hist, len, B, STRIDE, 6, 12, 0, tokens, count, match, pos);
    free(hist);
}

int main(void)
{
    orc_set_threads(2);
    test_codes_and_fp16();
    test_quantizers();
    test_attention(0, 4, 1, 64, 70, 8);
    test_attention(0, 6, 2, 128, 0, 5);
    test_attention(0, 4, 2, 64, 33, 64);
    test_attention(0, 2, 1, 256, 1, 1);
    test_attention(1, 4, 1, 64, 50, 8);
    test_attention(1, 6, 3, 128, 0, 3);
    test_merge_edges();
    test_accept_and_lookup();
    if (failures) {
        fprintf(stderr, "%d invariant failures\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all entry points exercised, invariants hold\n");
    return 0;
}
