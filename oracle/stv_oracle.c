/*
 * stv_oracle.c -- plain CPU oracle for verify-round attention over a 3-bit
 * KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The GPU path never
 * calls it and shares no code, header, table or helper with it.
 *
 * What it computes (the elpis pages: "Why fast" for int8 Q.K^T over 3-bit K
 * codes widened to int8 and for split-K with a merge; elpis-lossless
 * "Lossless" and "Trust base" for fp32-accumulated P.V and row
 * independence; "How" for the 8-row token tree):
 *
 *   for every query row (t, h), with kv head g = h / (Hq / Hkv):
 *     (q_i8, sq)  = per-row int8 quantization of q[t][h]            (c1)
 *     S_b[j]      = sum_{d in block b} q_i8[d] * (kcode[j][d] - 4)   int64
 *     x[j]        = scale * sq * sum_b sk[j][b] * S_b[j]             fp64
 *     visible(j)  = j < L, or the tree/causal rule for the new rows
 *     out         = sum_j softmax(x)_j * vs[j][b(d)] * (vcode[j][d] - 4)
 *     lse         = log sum_j exp(x[j])                              fp64
 *
 * It is the definition written out: no tiling, no splitting, no online
 * rescaling.  Integer parts are int64, softmax and P.V are fp64, keys are
 * visited in ascending order.  The only fp32 steps are the two quantizers,
 * because they define integers and fp16 scales that the GPU must reproduce
 * bit for bit; they use one correctly rounded IEEE division, one multiply
 * and round-half-even, with no contraction (built with -ffp-contract=off).
 *
 * Readings where the pages are silent (each also listed in the design
 * notes):
 *  (c1) Q quantizer: amax = max|q|; amax == 0 gives sq = 0 and all-zero
 *       codes; else inv = 127/amax, q_i8 = clamp(rint(q*inv), -127, 127),
 *       sq = amax/127.
 *  (c2) codes are offset binary with zero point 4: value = s * (c - 4).
 *  (c3) bit layout of one 32-element block in three 32-bit words, the
 *       "byte-plane" layout: element e = 4*qq + i (qq = e/4, i = e%4)
 *         qq = 0,1 : word 0, bits [8i + 3qq, +3)
 *         qq = 2,3 : word 1, bits [8i + 3(qq-2), +3)
 *         qq = 4,5 : word 2, bits [8i + 3(qq-4), +3)
 *         qq = 6   : code bits 0-1 at word 0 bits [8i+6, 8i+8),
 *                    code bit 2 at word 2 bit 8i+6
 *         qq = 7   : code bits 0-1 at word 1 bits [8i+6, 8i+8),
 *                    code bit 2 at word 2 bit 8i+7
 *  (c4) K/V quantizer per 32-element block: s16 = fp16_rne(amax/3) (the
 *       largest finite fp16 if that overflows), code = clamp(rint(x/s), -4,
 *       3) + 4, and code 4 everywhere when s16 is zero.
 *  (c6) the K scale is one fp16 per 32 consecutive elements of one (token,
 *       kv head) row; the softmax scale is a caller argument.
 *  (c8) storage: K is token-major, codes [Hkv][cap][D/32][3 words] and scales
 *       [Hkv][cap][D/32]; V is key-transposed in groups of 32 keys, codes
 *       [Hkv][ng][D][3 words] where element d of key 32*grp + e is code e of
 *       the block (grp, d), and scales [Hkv][ng][D/32][32] (ng = ceil(cap/32)).
 *       The bit layout of a three-word block is the same for both.
 *  (c7) tree keys sit at L + node index; key L + a is visible to row i iff
 *       bit a of mask[i] is set; a NULL mask means the causal chunk rule
 *       (key L + u visible to row t iff u <= t).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXPORT __attribute__((visibility("default")))

/* ---------------------------------------------------------------- format */

/* Bit position of bit k (0..2) of the code of element e (0..31). */
static void code_bit_pos(int e, int k, int *word, int *bit)
{
    int qq = e / 4, i = e % 4;
    if (qq < 6) {
        *word = qq / 2;
        *bit = 8 * i + 3 * (qq % 2) + k;
    } else if (k < 2) {
        *word = qq - 6;              /* qq 6 -> word 0, qq 7 -> word 1 */
        *bit = 8 * i + 6 + k;
    } else {
        *word = 2;
        *bit = 8 * i + 6 + (qq - 6);
    }
}

ORC_EXPORT int orc_code_get(const uint32_t *w, int e)
{
    int c = 0;
    for (int k = 0; k < 3; ++k) {
        int word, bit;
        code_bit_pos(e, k, &word, &bit);
        c |= (int)((w[word] >> bit) & 1u) << k;
    }
    return c;
}

ORC_EXPORT void orc_code_set(uint32_t *w, int e, int code)
{
    for (int k = 0; k < 3; ++k) {
        int word, bit;
        code_bit_pos(e, k, &word, &bit);
        w[word] &= ~(1u << bit);
        w[word] |= (uint32_t)((code >> k) & 1) << bit;
    }
}

/* ------------------------------------------------------------------ fp16 */

/* IEEE binary16 round-to-nearest-even of a float. */
ORC_EXPORT uint16_t orc_f32_to_f16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00u);
    double a = fabs((double)x);
    if (a >= 65520.0)                   /* halfway to 2^16 rounds up: inf */
        return (uint16_t)(sign | 0x7C00u);
    if (a < 0x1p-14) {                  /* subnormal range, quantum 2^-24 */
        double n = rint(a / 0x1p-24);   /* exact quotient, ties to even */
        return (uint16_t)(sign | (uint16_t)n);  /* n == 1024 is 2^-14 */
    }
    int E;
    frexp(a, &E);                       /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                      /* a in [2^e, 2^(e+1)) */
    double n = rint(ldexp(a, 10 - e));  /* 11-bit significand, exact input */
    if (n == 2048.0) {
        n = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024.0));
}

ORC_EXPORT double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1, ex = (h >> 10) & 0x1F, man = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man + 1024), ex - 25);
    return sign ? -v : v;
}

/* -------------------------------------------------------------- quantizers */

ORC_EXPORT void orc_quantize_q_row(const float *q, int D, int8_t *qi8, float *sq)
{
    float amax = 0.0f;
    for (int d = 0; d < D; ++d) {
        float a = fabsf(q[d]);
        if (a > amax)
            amax = a;
    }
    if (amax == 0.0f) {
        for (int d = 0; d < D; ++d)
            qi8[d] = 0;
        *sq = 0.0f;
        return;
    }
    float inv = 127.0f / amax;
    for (int d = 0; d < D; ++d) {
        float t = rintf(q[d] * inv);
        if (t > 127.0f) t = 127.0f;
        if (t < -127.0f) t = -127.0f;
        qi8[d] = (int8_t)t;
    }
    *sq = amax / 127.0f;
}

/* Quantize one 32-element block; returns the fp16 scale bits. */
ORC_EXPORT uint16_t orc_quantize_kv_block(const float *x, uint32_t *w)
{
    float amax = 0.0f;
    for (int e = 0; e < 32; ++e) {
        float a = fabsf(x[e]);
        if (a > amax)
            amax = a;
    }
    uint16_t s16 = orc_f32_to_f16(amax / 3.0f);
    if ((s16 & 0x7FFFu) == 0x7C00u)
        s16 = 0x7BFFu;                  /* saturate to the largest finite */
    float s = (float)orc_f16_to_f64(s16);
    w[0] = w[1] = w[2] = 0;
    for (int e = 0; e < 32; ++e) {
        int c = 4;
        if (s != 0.0f) {
            float t = rintf(x[e] / s);
            if (t > 3.0f) t = 3.0f;
            if (t < -4.0f) t = -4.0f;
            c = (int)t + 4;
        }
        orc_code_set(w, e, c);
    }
    return s16;
}

/* Number of 32-key groups of the V layout for a capacity. */
static size_t n_groups(int cap) { return ((size_t)cap + 31) / 32; }

/* K: x [n_tok][Hkv][D] fp32 into codes [Hkv][cap][D/32][3], scales
 * [Hkv][cap][D/32]; writes positions pos0 .. pos0+n_tok-1 only. */
ORC_EXPORT void orc_k_quant_pack(const float *x, int n_tok, int pos0, uint32_t *codes,
                                 uint16_t *scales, int Hkv, int D, int cap)
{
    int nb = D / 32;
    for (int t = 0; t < n_tok; ++t)
        for (int g = 0; g < Hkv; ++g)
            for (int b = 0; b < nb; ++b) {
                size_t pos = (size_t)g * cap + (size_t)(pos0 + t);
                scales[pos * nb + b] = orc_quantize_kv_block(
                    x + ((size_t)t * Hkv + g) * D + 32 * b, codes + (pos * nb + b) * 3);
            }
}

/* V: the same rule per (token, head, block); stored key-transposed, codes
 * [Hkv][ng][D][3] and scales [Hkv][ng][D/32][32].  Only the bits and scales of
 * keys pos0 .. pos0+n_tok-1 change. */
ORC_EXPORT void orc_v_quant_pack(const float *x, int n_tok, int pos0, uint32_t *codes,
                                 uint16_t *scales, int Hkv, int D, int cap)
{
    int nb = D / 32;
    size_t ng = n_groups(cap);
    for (int t = 0; t < n_tok; ++t)
        for (int g = 0; g < Hkv; ++g)
            for (int b = 0; b < nb; ++b) {
                int pos = pos0 + t, grp = pos / 32, e = pos % 32;
                uint32_t w[3];
                uint16_t s16 = orc_quantize_kv_block(x + ((size_t)t * Hkv + g) * D + 32 * b, w);
                scales[(((size_t)g * ng + grp) * nb + b) * 32 + e] = s16;
                for (int i = 0; i < 32; ++i) {
                    int d = 32 * b + i;
                    uint32_t *dst = codes + (((size_t)g * ng + grp) * D + d) * 3;
                    orc_code_set(dst, e, orc_code_get(w, i));
                }
            }
}

/* Code and scale of V element d of key j (kv head g). */
static int v_code(const uint32_t *vc, size_t ng, int D, int g, int j, int d)
{
    return orc_code_get(vc + (((size_t)g * ng + (size_t)(j / 32)) * D + d) * 3, j % 32);
}

static double v_scale(const uint16_t *vs, size_t ng, int nb, int g, int j, int b)
{
    return orc_f16_to_f64(vs[(((size_t)g * ng + (size_t)(j / 32)) * nb + b) * 32 + j % 32]);
}

/* ------------------------------------------------------------- attention */

/* Returns 0 on success, -1 on bad arguments.
 * q: [T][Hq][D]; caches as in (c8); mask: [T] (NULL = causal chunk rule).
 * Only keys j in [k_begin, k_end) take part (a split-K partial); pass
 * 0, L+T for the whole call.  rows: flattened t*Hq + h (NULL = all rows in
 * order).  Outputs are per listed row: out [n][D], lse [n], and optionally
 * logits [n][L+T][D/32] (every key, visible or not), qi8 [n][D], sq [n]. */
ORC_EXPORT int orc_attention(const float *q, int T, int Hq,
                             const uint32_t *kc, const uint16_t *ks,
                             const uint32_t *vc, const uint16_t *vs,
                             int Hkv, int D, int cap, int L,
                             const uint64_t *mask, double scale,
                             int k_begin, int k_end,
                             const int32_t *rows, int n_rows,
                             double *out, double *lse, int64_t *logits,
                             int8_t *qi8_out, float *sq_out)
{
    if (T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || D % 32 || L < 0 ||
        L + T > cap || (mask && T > 64))
        return -1;
    int nb = D / 32, G = Hq / Hkv, N = L + T;
    size_t ng = n_groups(cap);
    if (!rows)
        n_rows = T * Hq;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < n_rows; ++r) {
        int flat = rows ? rows[r] : r;
        if (flat < 0 || flat >= T * Hq) {
            bad = 1;
            continue;
        }
        int t = flat / Hq, h = flat % Hq, g = h / G;
        int8_t *qi = (int8_t *)malloc((size_t)D);
        double *x = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        char *vis = (char *)malloc((size_t)(N > 0 ? N : 1));
        float sq;
        orc_quantize_q_row(q + ((size_t)t * Hq + h) * D, D, qi, &sq);
        if (qi8_out)
            memcpy(qi8_out + (size_t)r * D, qi, (size_t)D);
        if (sq_out)
            sq_out[r] = sq;

        double m = -INFINITY;
        for (int j = 0; j < N; ++j) {
            const uint32_t *kw = kc + (((size_t)g * cap + j) * nb) * 3;
            const uint16_t *ksj = ks + ((size_t)g * cap + j) * nb;
            double acc = 0.0;
            for (int b = 0; b < nb; ++b) {
                int64_t s = 0;
                for (int e = 0; e < 32; ++e)
                    s += (int64_t)qi[32 * b + e] * (int64_t)(orc_code_get(kw + 3 * b, e) - 4);
                if (logits)
                    logits[((size_t)r * N + j) * nb + b] = s;
                acc += orc_f16_to_f64(ksj[b]) * (double)s;
            }
            x[j] = scale * (double)sq * acc;
            int v = (j >= k_begin && j < k_end);
            if (v && j >= L) {
                int a = j - L;
                v = mask ? (int)((mask[t] >> a) & 1u) : (a <= t);
            }
            vis[j] = (char)v;
            if (v && x[j] > m)
                m = x[j];
        }

        double *o = out + (size_t)r * D;
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        if (m == -INFINITY) {
            lse[r] = -INFINITY;
        } else {
            double l = 0.0;
            for (int j = 0; j < N; ++j) {
                if (!vis[j])
                    continue;
                double p = exp(x[j] - m);
                l += p;
                for (int b = 0; b < nb; ++b) {
                    double sv = v_scale(vs, ng, nb, g, j, b);
                    for (int e = 0; e < 32; ++e)
                        o[32 * b + e] += p * (sv * (double)(v_code(vc, ng, D, g, j, 32 * b + e) - 4));
                }
            }
            for (int d = 0; d < D; ++d)
                o[d] /= l;
            lse[r] = m + log(l);
        }
        free(qi);
        free(x);
        free(vis);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------- threading */

#ifdef _OPENMP
#include <omp.h>
#endif

/* Sets the OpenMP thread count of the row loop; returns the count in use. */
ORC_EXPORT int orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ----------------------------------------------------------------- merge */

/* part_o: [S][rows][D] (each normalised), part_lse: [S][rows] (natural log,
 * -inf for a split that saw no key).  out = sum_s e^(lse_s - LSE) O_s with
 * LSE = log sum_s e^lse_s; out_lse may be NULL. */
ORC_EXPORT void orc_merge(const double *part_o, const double *part_lse, int S, int rows,
                          int D, double *out, double *out_lse)
{
    for (int r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int s = 0; s < S; ++s)
            if (part_lse[(size_t)s * rows + r] > M)
                M = part_lse[(size_t)s * rows + r];
        double *o = out + (size_t)r * D;
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        if (M == -INFINITY) {
            if (out_lse)
                out_lse[r] = -INFINITY;
            continue;
        }
        double W = 0.0;
        for (int s = 0; s < S; ++s) {
            double ls = part_lse[(size_t)s * rows + r];
            if (ls == -INFINITY)
                continue;
            double w = exp(ls - M);
            W += w;
            const double *os = part_o + ((size_t)s * rows + r) * D;
            for (int d = 0; d < D; ++d)
                o[d] += w * os[d];
        }
        for (int d = 0; d < D; ++d)
            o[d] /= W;
        if (out_lse)
            out_lse[r] = M + log(W);
    }
}

/* ---------------------------------------------------- tree acceptance */

/* Greedy acceptance over a token tree (elpis "Why fast" and elpis-lossless
 * "How": the 8-row tree, best-first nodes, commit the longest matching path
 * plus one token; acceptance compares token ids exactly).  Readings:
 *  (a1) node 0 is the round's root, already decided, and always committed;
 *  (a2) node i > 0 matches when its draft token equals the target's greedy
 *       token at its parent row (parent = highest other bit of mask[i]);
 *  (a3) a node is acceptable when it descends from node 0 and every node on
 *       its path other than node 0 matches;
 *  (a4) the committed path ends at the acceptable node of greatest depth
 *       (number of nodes on its path), the lowest node index among equals;
 *  (a5) the extra token is the target's token at that node's row.
 * path[0 .. n-1] receives the path's node indices in increasing order and
 * path[n .. T-1] = -1.  Returns n (>= 1), or 0 on bad arguments. */
ORC_EXPORT int orc_tree_accept(const uint64_t *mask, int T, const int32_t *draft,
                               const int32_t *target, int32_t *path, int32_t *bonus)
{
    if (T < 1 || T > 64)
        return 0;
    int best = 0, best_depth = 1;
    for (int i = 0; i < T; ++i) {
        if (!((mask[i] >> 0) & 1ull))
            continue;                                   /* not below node 0 */
        int ok = 1, depth = 0;
        for (int j = 0; j <= i; ++j) {
            if (!((mask[i] >> j) & 1ull))
                continue;
            ++depth;
            if (j == 0)
                continue;
            int parent = -1;                            /* highest other bit */
            for (int k = j - 1; k >= 0; --k)
                if ((mask[j] >> k) & 1ull) {
                    parent = k;
                    break;
                }
            if (parent < 0 || draft[j] != target[parent])
                ok = 0;
        }
        if (ok && depth > best_depth) {
            best = i;
            best_depth = depth;
        }
    }
    int n = 0;
    for (int j = 0; j < T; ++j)
        if ((mask[best] >> j) & 1ull)
            path[n++] = j;
    for (int j = n; j < T; ++j)
        path[j] = -1;
    *bonus = target[best];
    return n;
}

/* Accepted-path commit: for j = 0 .. n-1 the K and V of cache position
 * L + path[j] move to position L + j, in every kv head; everything else in
 * the cache keeps its value (elpis-lossless "How": only the committed
 * tokens' K/V stay in the cache, at consecutive positions).  All sources are
 * read before any position is written.  Layouts as in (c8).  Returns 0, or
 * -1 on bad arguments. */
ORC_EXPORT int orc_kv_commit(uint32_t *kc, uint16_t *ks, uint32_t *vc, uint16_t *vs, int Hkv,
                             int D, int cap, int L, int T, const int32_t *path, int n)
{
    int nb = D / 32;
    size_t ng = n_groups(cap);
    if (n < 1 || n > T || L < 0 || L + T > cap)
        return -1;
    for (int j = 0; j < n; ++j)
        if (path[j] < 0 || path[j] >= T)
            return -1;
    size_t kwords = (size_t)n * nb * 3;
    uint32_t *kbuf = malloc(kwords * sizeof(uint32_t) + 1);
    uint16_t *kbs = malloc((size_t)n * nb * sizeof(uint16_t) + 1);
    int *vcode = malloc((size_t)n * D * sizeof(int) + 1);
    uint16_t *vsb = malloc((size_t)n * nb * sizeof(uint16_t) + 1);
    if (!kbuf || !kbs || !vcode || !vsb) {
        free(kbuf); free(kbs); free(vcode); free(vsb);
        return -1;
    }
    for (int g = 0; g < Hkv; ++g) {
        /* read every source first */
        for (int j = 0; j < n; ++j) {
            int src = L + path[j];
            for (int b = 0; b < nb; ++b) {
                size_t blk = ((size_t)g * cap + (size_t)src) * nb + b;
                memcpy(kbuf + ((size_t)j * nb + b) * 3, kc + blk * 3, 3 * sizeof(uint32_t));
                kbs[(size_t)j * nb + b] = ks[blk];
                vsb[(size_t)j * nb + b] =
                    vs[(((size_t)g * ng + (size_t)(src / 32)) * nb + b) * 32 + src % 32];
            }
            for (int d = 0; d < D; ++d)
                vcode[(size_t)j * D + d] = v_code(vc, ng, D, g, src, d);
        }
        /* then write the destinations */
        for (int j = 0; j < n; ++j) {
            int dst = L + j;
            for (int b = 0; b < nb; ++b) {
                size_t blk = ((size_t)g * cap + (size_t)dst) * nb + b;
                memcpy(kc + blk * 3, kbuf + ((size_t)j * nb + b) * 3, 3 * sizeof(uint32_t));
                ks[blk] = kbs[(size_t)j * nb + b];
                vs[(((size_t)g * ng + (size_t)(dst / 32)) * nb + b) * 32 + dst % 32] =
                    vsb[(size_t)j * nb + b];
            }
            for (int d = 0; d < D; ++d)
                orc_code_set(vc + (((size_t)g * ng + (size_t)(dst / 32)) * D + d) * 3, dst % 32,
                             vcode[(size_t)j * D + d]);
        }
    }
    free(kbuf); free(kbs); free(vcode); free(vsb);
    return 0;
}

/* ------------------------------------------------------- lookup drafting */

/* Lookup drafting over a token history (u/iamMess, lookup-augmented
 * drafting: scan the request's own history for the most recent earlier
 * occurrence of its last 6-12 tokens and propose the tokens that followed;
 * elpis, the drafter-free n-gram chains).  Readings:
 *  (l1) a candidate is an end position e <= N-2 (so at least one token
 *       follows it); its match length m(e) is the number of tokens, at most
 *       n_max and at most e+1, for which h[e-i] == h[N-1-i], i = 0, 1, ...;
 *  (l2) candidates need m(e) >= n_min; the longest match wins, the most
 *       recent (largest e) among equals;
 *  (l3) the proposal is h[e+1 .. e+count] with count = min(k, N-1-e);
 *       without a candidate: count 0, match 0, position -1.
 * tokens[k] gets the proposal, then -1.  Per sequence b of a batch, history
 * row b of `stride` tokens holds N = len[b] valid tokens. */
ORC_EXPORT void orc_lookup_draft(const int32_t *hist, const int32_t *len, int B, int stride,
                                 int n_min, int n_max, int k, int32_t *tokens, int32_t *count,
                                 int32_t *match, int32_t *pos)
{
    for (int b = 0; b < B; ++b) {
        const int32_t *h = hist + (size_t)b * stride;
        int N = len[b] < 0 ? 0 : (len[b] > stride ? stride : len[b]);
        int best_m = 0, best_e = -1;
        for (int e = 0; e <= N - 2; ++e) {
            int cap = n_max < e + 1 ? n_max : e + 1;
            int m = 0;
            while (m < cap && h[e - m] == h[N - 1 - m])
                ++m;
            if (m >= n_min && (m > best_m || (m == best_m && e > best_e))) {
                best_m = m;
                best_e = e;
            }
        }
        int c = 0;
        if (best_e >= 0) {
            c = N - 1 - best_e;
            if (c > k)
                c = k;
        }
        for (int j = 0; j < k; ++j)
            tokens[(size_t)b * k + j] = j < c ? h[best_e + 1 + j] : -1;
        count[b] = c;
        match[b] = best_e >= 0 ? best_m : 0;
        pos[b] = best_e;
    }
}

/* ------------------------------------- second KV format: 4-bit per token-head */

/* The 4-bit per-token-head cache ("Qwen3.8-27B on one RTX 3090", the int4 KV
 * section: 4-bit codes with one scale per token and KV head).  The pages give
 * the granularity only; readings:
 *  (i1) codes c in [0, 15] stand for s * (c - 8);
 *  (i2) per (token, KV head) row of D elements: s16 = fp16_rne(amax / 7)
 *       saturated to the largest finite fp16, code = clamp(rint(x / s), -8,
 *       7) + 8, all codes 8 when s16 is zero (the 3-bit rule with 7 = 2^3 - 1);
 *  (i3) K token-major: codes uint32 [Hkv][cap][D/8], element 8w + i in bits
 *       [4i, 4i+4) of word w; scales fp16 [Hkv][cap].  V key-transposed in
 *       32-key groups: codes uint32 [Hkv][ng][D][4], key 32*grp + e of
 *       element d in word e/8 bits [4(e%8), +4) of row (grp, d); scales fp16
 *       [Hkv][cap];
 *  (i4) Q.K^T is one int64 sum over the whole row, x = scale * sq * sk * S. */
static int nib_get(const uint32_t *w, int e) { return (int)((w[e / 8] >> (4 * (e % 8))) & 15u); }

static void nib_set(uint32_t *w, int e, int c)
{
    w[e / 8] &= ~(15u << (4 * (e % 8)));
    w[e / 8] |= (uint32_t)(c & 15) << (4 * (e % 8));
}

ORC_EXPORT uint16_t orc_quantize_kv4_row(const float *x, int D, uint32_t *w)
{
    float amax = 0.0f;
    for (int e = 0; e < D; ++e) {
        float a = fabsf(x[e]);
        if (a > amax)
            amax = a;
    }
    uint16_t s16 = orc_f32_to_f16(amax / 7.0f);
    if ((s16 & 0x7FFFu) == 0x7C00u)
        s16 = (uint16_t)((s16 & 0x8000u) | 0x7BFFu);
    float s = (float)orc_f16_to_f64(s16);
    for (int i = 0; i < D / 8; ++i)
        w[i] = 0;
    for (int e = 0; e < D; ++e) {
        int c = 8;
        if (s != 0.0f) {
            float r = rintf(x[e] / s);
            if (r < -8.0f)
                r = -8.0f;
            if (r > 7.0f)
                r = 7.0f;
            c = (int)r + 8;
        }
        nib_set(w, e, c);
    }
    return s16;
}

ORC_EXPORT void orc_k4_quant_pack(const float *x, int n_tok, int pos0, uint32_t *codes,
                                  uint16_t *scales, int Hkv, int D, int cap)
{
    for (int t = 0; t < n_tok; ++t)
        for (int g = 0; g < Hkv; ++g) {
            size_t pos = (size_t)g * cap + (size_t)(pos0 + t);
            scales[pos] = orc_quantize_kv4_row(x + ((size_t)t * Hkv + g) * D, D,
                                               codes + pos * (size_t)(D / 8));
        }
}

ORC_EXPORT void orc_v4_quant_pack(const float *x, int n_tok, int pos0, uint32_t *codes,
                                  uint16_t *scales, int Hkv, int D, int cap)
{
    size_t ng = n_groups(cap);
    uint32_t *w = malloc((size_t)(D / 8) * sizeof(uint32_t) + 1);
    if (!w)
        return;
    for (int t = 0; t < n_tok; ++t)
        for (int g = 0; g < Hkv; ++g) {
            int pos = pos0 + t, grp = pos / 32, e = pos % 32;
            scales[(size_t)g * cap + pos] = orc_quantize_kv4_row(x + ((size_t)t * Hkv + g) * D, D, w);
            for (int d = 0; d < D; ++d)
                nib_set(codes + (((size_t)g * ng + grp) * D + d) * 4, e, nib_get(w, d));
        }
    free(w);
}

/* As orc_attention, for the 4-bit per-token-head cache; logits [n][L+T]
 * (one int64 sum per key). */
ORC_EXPORT int orc_attention_i4(const float *q, int T, int Hq,
                                const uint32_t *kc, const uint16_t *ks,
                                const uint32_t *vc, const uint16_t *vs,
                                int Hkv, int D, int cap, int L,
                                const uint64_t *mask, double scale,
                                int k_begin, int k_end,
                                const int32_t *rows, int n_rows,
                                double *out, double *lse, int64_t *logits,
                                int8_t *qi8_out, float *sq_out)
{
    if (T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || D % 32 || L < 0 ||
        L + T > cap || (mask && T > 64))
        return -1;
    int G = Hq / Hkv, N = L + T;
    size_t ng = n_groups(cap);
    if (!rows)
        n_rows = T * Hq;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < n_rows; ++r) {
        int flat = rows ? rows[r] : r;
        if (flat < 0 || flat >= T * Hq) {
            bad = 1;
            continue;
        }
        int t = flat / Hq, h = flat % Hq, g = h / G;
        int8_t *qi = (int8_t *)malloc((size_t)D);
        double *x = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        char *vis = (char *)malloc((size_t)(N > 0 ? N : 1));
        float sq;
        orc_quantize_q_row(q + ((size_t)t * Hq + h) * D, D, qi, &sq);
        if (qi8_out)
            memcpy(qi8_out + (size_t)r * D, qi, (size_t)D);
        if (sq_out)
            sq_out[r] = sq;

        double m = -INFINITY;
        for (int j = 0; j < N; ++j) {
            const uint32_t *kw = kc + ((size_t)g * cap + j) * (size_t)(D / 8);
            int64_t s = 0;
            for (int d = 0; d < D; ++d)
                s += (int64_t)qi[d] * (int64_t)(nib_get(kw, d) - 8);
            if (logits)
                logits[(size_t)r * N + j] = s;
            x[j] = scale * (double)sq * orc_f16_to_f64(ks[(size_t)g * cap + j]) * (double)s;
            int v = (j >= k_begin && j < k_end);
            if (v && j >= L) {
                int a = j - L;
                v = mask ? (int)((mask[t] >> a) & 1u) : (a <= t);
            }
            vis[j] = (char)v;
            if (v && x[j] > m)
                m = x[j];
        }

        double *o = out + (size_t)r * D;
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        if (m == -INFINITY) {
            lse[r] = -INFINITY;
        } else {
            double l = 0.0;
            for (int j = 0; j < N; ++j) {
                if (!vis[j])
                    continue;
                double p = exp(x[j] - m);
                l += p;
                double sv = orc_f16_to_f64(vs[(size_t)g * cap + j]);
                for (int d = 0; d < D; ++d) {
                    const uint32_t *vw = vc + (((size_t)g * ng + (size_t)(j / 32)) * D + d) * 4;
                    o[d] += p * (sv * (double)(nib_get(vw, j % 32) - 8));
                }
            }
            for (int d = 0; d < D; ++d)
                o[d] /= l;
            lse[r] = m + log(l);
        }
        free(qi);
        free(x);
        free(vis);
    }
    return bad ? -1 : 0;
}

/* Accepted-path commit for the 4-bit per-token-head cache (as
 * orc_kv_commit; layouts as in (i3)). */
ORC_EXPORT int orc_kv4_commit(uint32_t *kc, uint16_t *ks, uint32_t *vc, uint16_t *vs, int Hkv,
                              int D, int cap, int L, int T, const int32_t *path, int n)
{
    size_t ng = n_groups(cap);
    int kw = D / 8;
    if (n < 1 || n > T || L < 0 || L + T > cap)
        return -1;
    for (int j = 0; j < n; ++j)
        if (path[j] < 0 || path[j] >= T)
            return -1;
    uint32_t *kbuf = malloc((size_t)n * kw * sizeof(uint32_t) + 1);
    uint16_t *ksb = malloc((size_t)n * sizeof(uint16_t) + 1);
    uint16_t *vsb = malloc((size_t)n * sizeof(uint16_t) + 1);
    int *vcode = malloc((size_t)n * D * sizeof(int) + 1);
    if (!kbuf || !ksb || !vsb || !vcode) {
        free(kbuf); free(ksb); free(vsb); free(vcode);
        return -1;
    }
    for (int g = 0; g < Hkv; ++g) {
        for (int j = 0; j < n; ++j) {
            int src = L + path[j];
            memcpy(kbuf + (size_t)j * kw, kc + ((size_t)g * cap + src) * kw, (size_t)kw * 4);
            ksb[j] = ks[(size_t)g * cap + src];
            vsb[j] = vs[(size_t)g * cap + src];
            for (int d = 0; d < D; ++d)
                vcode[(size_t)j * D + d] =
                    nib_get(vc + (((size_t)g * ng + (size_t)(src / 32)) * D + d) * 4, src % 32);
        }
        for (int j = 0; j < n; ++j) {
            int dst = L + j;
            memcpy(kc + ((size_t)g * cap + dst) * kw, kbuf + (size_t)j * kw, (size_t)kw * 4);
            ks[(size_t)g * cap + dst] = ksb[j];
            vs[(size_t)g * cap + dst] = vsb[j];
            for (int d = 0; d < D; ++d)
                nib_set(vc + (((size_t)g * ng + (size_t)(dst / 32)) * D + d) * 4, dst % 32,
                        vcode[(size_t)j * D + d]);
        }
    }
    free(kbuf); free(ksb); free(vsb); free(vcode);
    return 0;
}
