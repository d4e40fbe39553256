// C-ABI host layer: argument validation (all before any HIP call), the
// split plan, and kernel launches.  See include/stv.h for the contract.
#include "stv.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "stv_accept.h"
#include "stv_lookup.h"
#include "stv_internal.h"

namespace stv {
// the split plan for L context keys followed by n_after more (defined below)
Plan make_plan_keys(int T, int Hq, int Hkv, int D, int L, bool causal, int n_splits_req, int fmt,
                    int n_after);
}  // namespace stv

namespace {

thread_local char g_err[512] = "";
constexpr int kKeyTileC = stv::kKeyTile;

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return STV_OK;
}

bool head_dim_ok(int D) { return D == 64 || D == 128 || D == 256; }

int check_heads(int Hq, int Hkv, int D) {
    if (Hkv <= 0 || Hq <= 0) return fail(STV_EINVAL, "head counts must be positive (Hq=%d, Hkv=%d)", Hq, Hkv);
    if (Hq % Hkv) return fail(STV_EINVAL, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", Hq, Hkv);
    if (!head_dim_ok(D)) return fail(STV_EINVAL, "head_dim %d unsupported (64, 128 or 256)", D);
    return STV_OK;
}

// Rows must form a forest: own bit set, no higher bit, and the remaining
// bits equal to the mask of the highest of them (the parent).
int check_mask(const uint64_t *m, int T) {
    for (int i = 0; i < T; ++i) {
        const uint64_t own = 1ull << i;
        if (!(m[i] & own)) return fail(STV_EMASK, "anc_mask[%d] lacks its own bit", i);
        if (i < 63 && (m[i] >> (i + 1))) return fail(STV_EMASK, "anc_mask[%d] has a bit above row %d", i, i);
        const uint64_t rest = m[i] & ~own;
        if (rest) {
            const int p = 63 - __builtin_clzll(rest);
            if (m[p] != rest)
                return fail(STV_EMASK, "anc_mask[%d] is not its parent's (row %d) mask plus itself", i, p);
        }
    }
    return STV_OK;
}

int check_kv(const stv_kv_layer *kv, int Hq, int L, int T) {
    if (!kv) return fail(STV_EINVAL, "kv is NULL");
    if (!kv->k_codes || !kv->k_scales || !kv->v_codes || !kv->v_scales)
        return fail(STV_EINVAL, "kv has a NULL array");
    int rc = check_heads(Hq, kv->n_kv_heads, kv->head_dim);
    if (rc) return rc;
    if (kv->capacity <= 0) return fail(STV_EINVAL, "capacity must be positive");
    if (kv->kv_format != STV_KV_3BIT && kv->kv_format != STV_KV_4BIT_TOKEN)
        return fail(STV_EINVAL, "kv_format %d unknown", kv->kv_format);
    if (kv->kv_format == STV_KV_4BIT_TOKEN &&
        ((reinterpret_cast<uintptr_t>(kv->k_codes) | reinterpret_cast<uintptr_t>(kv->v_codes)) & 15u))
        return fail(STV_EINVAL, "4-bit k_codes and v_codes must be 16-byte aligned");
    if (L < 0) return fail(STV_EINVAL, "ctx_len must be >= 0");
    if ((long long)L + T > kv->capacity)
        return fail(STV_ECAPACITY, "ctx_len + T = %lld exceeds capacity %d", (long long)L + T, kv->capacity);
    return STV_OK;
}

// With partials_o set, every split (even when S == 1) writes its partial to
// partials_o / partials_lse and no merge runs.  ctx_only: the T rows see
// keys 0 .. L-1 only (a context slice without tree keys; no mask).
int attention_common(const float *q, int T, int Hq, const stv_kv_layer *kv, int L,
                     const uint64_t *mask, bool causal, float scale, float *out, float *out_lse,
                     void *ws, size_t ws_bytes, int n_splits, int32_t *dbg_logits, int8_t *dbg_q,
                     float *dbg_qscale, void *stream, float *partials_o = nullptr,
                     float *partials_lse = nullptr, bool pv16 = false, bool ctx_only = false,
                     bool noalloc = false) {
    const bool partials_only = partials_o != nullptr;
    if (!q || (!out && !partials_only)) return fail(STV_EINVAL, "q and out must not be NULL");
    if (partials_only && !partials_lse) return fail(STV_EINVAL, "part_lse must not be NULL");
    // the kernels move q, out and the partials in 16-byte vectors
    if (((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) |
          reinterpret_cast<uintptr_t>(partials_o) | reinterpret_cast<uintptr_t>(ws)) & 15u) != 0)
        return fail(STV_EINVAL, "q, out, workspace and part_o must be 16-byte aligned");
    if (T < 1) return fail(STV_EINVAL, "T must be >= 1 (got %d)", T);
    if (!causal && T > STV_MAX_TREE_ROWS) return fail(STV_EINVAL, "verify supports at most 64 tree rows (got %d)", T);
    if ((long long)T * Hq >= (1ll << 31)) return fail(STV_EINVAL, "T * n_q_heads too large");
    if (n_splits < 0) return fail(STV_EINVAL, "n_splits must be >= 0");
    if (!(scale > 0.0f) || !isfinite(scale)) return fail(STV_EINVAL, "softmax_scale must be positive and finite");
    if (ctx_only && L < 1) return fail(STV_EINVAL, "n_keys must be >= 1");
    int rc = check_kv(kv, Hq, L, ctx_only ? 0 : T);
    if (rc) return rc;
    if (!causal && !ctx_only) {
        if (!mask) return fail(STV_EINVAL, "anc_mask must not be NULL");
        rc = check_mask(mask, T);
        if (rc) return rc;
    }
    const int D = kv->head_dim, Hkv = kv->n_kv_heads;
    if (dbg_logits && (long long)T * Hq * (L + T) * (D / 32) >= (1ll << 40))
        return fail(STV_EINVAL, "dbg_logits would be too large");
    const int fmt = kv->kv_format;
    if (pv16 && fmt != STV_KV_3BIT)
        return fail(STV_EINVAL, "fp16-accumulated P.V reads the 3-bit format only");
    stv::Plan plan = stv::make_plan_keys(T, Hq, Hkv, D, L, causal, n_splits, fmt, ctx_only ? 0 : T);
    if (noalloc && plan.S > 1 && plan.part_bytes > stv::kNoAllocScratchBytes) {
        // the partials go to the library's fixed scratch: the automatic plan
        // takes as many splits as it holds; an explicit count beyond that fails
        const size_t per_split = (size_t)T * Hq * ((size_t)D + 1) * sizeof(float);
        const long long fit = (long long)(stv::kNoAllocScratchBytes / per_split);
        if (n_splits > 0)
            return fail(STV_EWORKSPACE,
                        "the no-alloc scratch (%zu bytes) holds at most %lld splits of this call "
                        "(%d requested)", stv::kNoAllocScratchBytes, fit, n_splits);
        plan = stv::make_plan_keys(T, Hq, Hkv, D, L, causal, fit > 1 ? (int)fit : 1, fmt,
                                   ctx_only ? 0 : T);
    }
    if (noalloc && plan.S > 1) {
        hipError_t e = hipSuccess;
        ws = stv::noalloc_scratch(&e);
        if (!ws) return fail(STV_EHIP, "no-alloc scratch unavailable: %s", hipGetErrorString(e));
        ws_bytes = stv::kNoAllocScratchBytes;
    }
    if (!partials_only && plan.S > 1 && (!ws || ws_bytes < plan.part_bytes))
        return fail(STV_EWORKSPACE, "workspace of %zu bytes needed for %d splits (got %zu)",
                    plan.part_bytes, plan.S, ws ? ws_bytes : (size_t)0);

    stv::AttnArgs a;
    memset(&a, 0, sizeof a);
    a.q = q;
    a.kc = kv->k_codes;
    a.ks = kv->k_scales;
    a.vc = kv->v_codes;
    a.vs = kv->v_scales;
    a.out = out;
    a.out_lse = out_lse;
    const size_t rows = (size_t)T * Hq;
    if (partials_only) {
        a.part_o = partials_o;
        a.part_lse = partials_lse;
    } else if (plan.S > 1) {
        a.part_o = static_cast<float *>(ws);
        a.part_lse = a.part_o + (size_t)plan.S * rows * D;
    }
    a.dbg_logits = dbg_logits;
    a.dbg_q = dbg_q;
    a.dbg_qscale = dbg_qscale;
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.cap = kv->capacity;
    a.ngroups = (kv->capacity + kKeyTileC - 1) / kKeyTileC;
    a.L = L;
    a.N = ctx_only ? L : L + T;
    a.R = T * a.G;
    a.S = plan.S;
    a.split_len = plan.split_len;
    a.NRG = plan.NRG;
    a.n_hs_pad = ((Hkv * plan.S + 7) / 8) * 8;
    a.scale_log2 = scale * 1.44269504088896340736f;
    if (!causal && !ctx_only)
        for (int i = 0; i < T; ++i) a.mask[i] = mask[i];

    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool debug = dbg_logits || dbg_q || dbg_qscale;
    // tile images when the plan asks for them and the workspace holds them
    // (otherwise every row group unpacks the tiles itself)
    if (plan.pre && !debug && !partials_only && !noalloc && ws && ws_bytes >= plan.ws_bytes) {
        unsigned char *img = static_cast<unsigned char *>(ws) + plan.img_offset;
        a.img = img;
        a.img_tiles = (a.N + kKeyTileC - 1) / kKeyTileC;
        hipError_t e = stv::launch_tile_images(a, D, fmt, img, st);
        if (e != hipSuccess) return fail(STV_EHIP, "tile image launch failed: %s", hipGetErrorString(e));
    }
    hipError_t e = plan.dec   ? stv::launch_attention_dec(a, D, causal, debug, pv16, fmt, st)
                   : plan.s16 ? stv::launch_attention_s16(a, D, causal, debug, pv16, st)
                              : stv::launch_attention(a, D, plan.NW, causal, debug, fmt, pv16, st);
    if (e != hipSuccess) return fail(STV_EHIP, "attention launch failed: %s", hipGetErrorString(e));
    if (!partials_only && plan.S > 1) {
        e = stv::launch_merge(a.part_o, a.part_lse, plan.S, (int)rows, D, out, out_lse, st);
        if (e != hipSuccess) return fail(STV_EHIP, "merge launch failed: %s", hipGetErrorString(e));
    }
    return ok();
}

}  // namespace

namespace stv {

long long attention_slots(int D, int NW, bool causal, int kind, int fmt) {
    // MI355X: 256 CUs; the D = 256 four-wave kernels hold two work-groups per
    // CU, the wave-specialized kernel one.
    const long long kFallback = kind == 3 ? 256LL : 256LL * 2;
    struct Entry {
        int dev, D, NW;
        bool causal;
        int kind, fmt;
        long long slots;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0, count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0 || hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return kFallback;
    }
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry &e : cache)
        if (e.dev == dev && e.D == D && e.NW == NW && e.causal == causal && e.kind == kind &&
            e.fmt == fmt)
            return e.slots;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
        (void)hipGetLastError();
        return kFallback;
    }
    const int per_cu = kind == 1   ? attention_dec_wgs_per_cu(D, causal, fmt)
                       : kind == 2 ? attention_s16_wgs_per_cu(D, causal)
                       : kind == 3 ? attention_ws_wgs_per_cu(D)
                                   : attention_wgs_per_cu(D, NW, causal, fmt);
    const long long slots = per_cu > 0 ? (long long)cus * per_cu : kFallback;
    cache.push_back({dev, D, NW, causal, kind, fmt, slots});
    return slots;
}

// n_after: keys after the L context keys (T for verify and prefill, 0 for a
// context slice).
Plan make_plan_keys(int T, int Hq, int Hkv, int D, int L, bool causal, int n_splits_req, int fmt,
                    int n_after) {
    Plan p;
    const int G = Hq / Hkv;
    const long long R = (long long)T * G;
    // the few-row kernel: up to 16 rows per KV head (3-bit), 64 (4-bit)
    p.dec = R <= (fmt == 1 ? kDecMaxRows4 : kDecMaxRows);
    p.s16 = !p.dec && R <= kS16MaxRows && fmt == 0;
    p.ws = false;
    if (p.dec) {
        p.NW = 4;
        p.NRG = (int)((R + 15) / 16);
    } else if (p.s16) {
        p.NW = 4;
        p.NRG = (int)((R + 63) / 64);
    } else {
        const long long row_tiles = (R + kRowTile - 1) / kRowTile;
        p.NW = row_tiles >= 4 ? 4 : (row_tiles >= 2 ? 2 : 1);
        p.NRG = (int)((row_tiles + p.NW - 1) / p.NW);
        p.ws = !causal && fmt == 0 && p.NW == 4 && D == 256;
    }
    const long long N = (long long)L + n_after;
    const long long n_tiles = (N + kKeyTile - 1) / kKeyTile;
    long long S;
    if (n_splits_req > 0) {
        S = n_splits_req;
    } else if (p.ws) {
        // The wave-specialized kernel holds one work-group per CU, and
        // work-group i runs on XCD i mod 8; each XCD takes a run of
        // ceil(work-groups / 8) of them, which sets the number of rounds.  A
        // round costs its work-groups' tiles plus a fixed part (prologue,
        // prefetch fill, epilogue: about kWsRoundTiles tiles, measured), so
        // pick the split count that minimises rounds x (tiles per split +
        // that part), preferring fewer splits.
        const long long slots = attention_slots(D, p.NW, causal, 3, fmt);
        const long long xcds = slots % 8 == 0 ? 8 : 1;
        const long long per_xcd = slots / xcds;
        const long long max_s = n_tiles / 4 > 0 ? n_tiles / 4 : 1;
        const long long groups = (long long)Hkv * p.NRG;
        long long s_hi = 4 * ((slots + groups - 1) / groups);
        if (s_hi > max_s) s_hi = max_s;
        if (s_hi < 1) s_hi = 1;
        S = 1;
        long long best = -1;
        for (long long s = 1; s <= s_hi; ++s) {
            const long long fullest = (p.NRG * Hkv * s + xcds - 1) / xcds;
            const long long rounds = (fullest + per_xcd - 1) / per_xcd;
            const long long cost = rounds * ((n_tiles + s - 1) / s + kWsRoundTiles);
            if (best < 0 || cost < best) {
                best = cost;
                S = s;
            }
        }
    } else {
        // Fill the device's resident work-group slots exactly once: one
        // round of equal work-groups, no straggling partial round.  Splits
        // keep at least four tiles.
        const long long slots = attention_slots(D, p.NW, causal, p.dec ? 1 : (p.s16 ? 2 : 0), fmt);
        const long long groups = (long long)Hkv * p.NRG;
        if (groups < slots) {
            S = slots / groups;
        } else {
            // More row groups than slots: pick the split count (1..4) that
            // wastes the least of the last round, preferring fewer splits.
            S = 1;
            double best = 1e30;
            for (long long s = 1; s <= 4; ++s) {
                const double rounds_per_split = (double)((groups * s + slots - 1) / slots) / (double)s;
                if (rounds_per_split < best - 1e-9) {
                    best = rounds_per_split;
                    S = s;
                }
            }
        }
        const long long max_s = n_tiles / 4 > 0 ? n_tiles / 4 : 1;
        if (S > max_s) S = max_s;
    }
    if (S < 1) S = 1;
    if (S > n_tiles) S = n_tiles > 0 ? n_tiles : 1;
    // Whole tiles per split; dropping splits that would be empty, then
    // spreading the tiles evenly over the rest, keeps S and makes split s
    // cover keys [s*P, min(N, (s+1)*P)) with P = 32*ceil(ceil(N/32)/S).
    long long tiles_per_split = (n_tiles + S - 1) / S;
    S = (n_tiles + tiles_per_split - 1) / tiles_per_split;
    if (S < 1) S = 1;
    tiles_per_split = (n_tiles + S - 1) / S;
    p.split_len = (int)(tiles_per_split * kKeyTile);
    p.S = (int)S;
    const size_t rows = (size_t)T * Hq;
    p.part_bytes = p.S > 1 ? (size_t)p.S * rows * ((size_t)D + 1) * sizeof(float) : 0;
    // the causal chunk with many row groups: each tile unpacked once, into
    // images after the partials (256-byte aligned)
    // (3-bit format only: the 4-bit unpack is cheap enough that images
    // measured no faster)
    p.pre = causal && fmt == 0 && !p.dec && !p.s16 && p.NW == 4 && p.NRG >= kPreMinRowGroups;
    p.img_offset = (p.part_bytes + 255) / 256 * 256;
    p.ws_bytes = p.pre ? p.img_offset + (size_t)Hkv * (size_t)n_tiles * tile_image_bytes(D)
                       : p.part_bytes;
    return p;
}

Plan make_plan(int T, int Hq, int Hkv, int D, int L, bool causal, int n_splits_req, int fmt) {
    return make_plan_keys(T, Hq, Hkv, D, L, causal, n_splits_req, fmt, T);
}

}  // namespace stv

extern "C" {

const char *stv_last_error(void) { return g_err; }

int32_t stv_abi_version(void) { return 5; }

int stv_kv_quant_pack(const float *x, int32_t n_tok, int32_t pos0, int32_t which,
                      uint32_t *codes, uint16_t *scales, int32_t n_kv_heads, int32_t head_dim,
                      int32_t capacity, void *stream) {
    if (which != STV_K && which != STV_V && which != STV_K4 && which != STV_V4)
        return fail(STV_EINVAL, "which must be STV_K, STV_V, STV_K4 or STV_V4");
    if (n_tok < 0) return fail(STV_EINVAL, "n_tok must be >= 0");
    if (n_kv_heads <= 0) return fail(STV_EINVAL, "n_kv_heads must be positive");
    if (!head_dim_ok(head_dim)) return fail(STV_EINVAL, "head_dim %d unsupported (64, 128 or 256)", head_dim);
    if (capacity <= 0) return fail(STV_EINVAL, "capacity must be positive");
    if (pos0 < 0 || (long long)pos0 + n_tok > capacity)
        return fail(STV_ECAPACITY, "positions %d..%lld outside capacity %d", pos0,
                    (long long)pos0 + n_tok - 1, capacity);
    if (n_tok == 0) return ok();
    if (!x || !codes || !scales) return fail(STV_EINVAL, "x, codes and scales must not be NULL");
    if ((reinterpret_cast<uintptr_t>(x) & 15u) != 0) return fail(STV_EINVAL, "x must be 16-byte aligned");
    const bool four = which == STV_K4 || which == STV_V4;
    const bool is_v = which == STV_V || which == STV_V4;
    hipError_t e = four ? stv::launch_kv_pack4(x, n_tok, pos0, codes, scales, n_kv_heads, head_dim,
                                               capacity, is_v, static_cast<hipStream_t>(stream))
                        : stv::launch_kv_pack(x, n_tok, pos0, codes, scales, n_kv_heads, head_dim,
                                              capacity, is_v, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(STV_EHIP, "kv pack launch failed: %s", hipGetErrorString(e));
    return ok();
}

int stv_attention_plan(int32_t T, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                       int32_t ctx_len, int32_t causal, int32_t kv_format, int32_t n_splits_req,
                       int32_t *n_splits_out, size_t *workspace_bytes_out) {
    if (kv_format != STV_KV_3BIT && kv_format != STV_KV_4BIT_TOKEN)
        return fail(STV_EINVAL, "kv_format %d unknown", kv_format);
    if (T < 1) return fail(STV_EINVAL, "T must be >= 1");
    if (!causal && T > STV_MAX_TREE_ROWS) return fail(STV_EINVAL, "verify supports at most 64 tree rows");
    int rc = check_heads(n_q_heads, n_kv_heads, head_dim);
    if (rc) return rc;
    if (ctx_len < 0) return fail(STV_EINVAL, "ctx_len must be >= 0");
    if (n_splits_req < 0) return fail(STV_EINVAL, "n_splits must be >= 0");
    if ((long long)T * n_q_heads >= (1ll << 31)) return fail(STV_EINVAL, "T * n_q_heads too large");
    const stv::Plan p = stv::make_plan(T, n_q_heads, n_kv_heads, head_dim, ctx_len, causal != 0,
                                       n_splits_req, kv_format);
    if (n_splits_out) *n_splits_out = p.S;
    if (workspace_bytes_out) *workspace_bytes_out = p.ws_bytes;
    return ok();
}

size_t stv_workspace_bytes(int32_t T, int32_t n_q_heads, int32_t head_dim, int32_t n_splits) {
    if (T < 1) return fail(STV_EINVAL, "T must be >= 1"), (size_t)0;
    if (n_q_heads < 1) return fail(STV_EINVAL, "n_q_heads must be >= 1"), (size_t)0;
    if (!head_dim_ok(head_dim))
        return fail(STV_EINVAL, "head_dim %d unsupported (64, 128 or 256)", head_dim), (size_t)0;
    if (n_splits < 1)
        return fail(STV_EINVAL, "n_splits must be >= 1 (stv_attention_plan chooses it)"), (size_t)0;
    if ((long long)T * n_q_heads >= (1ll << 31))
        return fail(STV_EINVAL, "T * n_q_heads too large"), (size_t)0;
    ok();
    if (n_splits == 1) return 0;
    return (size_t)n_splits * (size_t)T * (size_t)n_q_heads * ((size_t)head_dim + 1) * sizeof(float);
}

int stv_verify_attention(const float *q, int32_t T, int32_t n_q_heads, const stv_kv_layer *kv,
                         int32_t ctx_len, const uint64_t *anc_mask, float softmax_scale,
                         float *out, float *out_lse, void *workspace, size_t workspace_bytes,
                         int32_t n_splits, int32_t *dbg_logits, int8_t *dbg_q,
                         float *dbg_qscale, void *stream) {
    return attention_common(q, T, n_q_heads, kv, ctx_len, anc_mask, false, softmax_scale, out,
                            out_lse, workspace, workspace_bytes, n_splits, dbg_logits, dbg_q,
                            dbg_qscale, stream);
}

int stv_verify_attention_noalloc(const float *q, int32_t T, int32_t n_q_heads,
                                 const stv_kv_layer *kv, int32_t ctx_len,
                                 const uint64_t *anc_mask, float softmax_scale, float *out,
                                 float *out_lse, int32_t n_splits, void *stream) {
    return attention_common(q, T, n_q_heads, kv, ctx_len, anc_mask, false, softmax_scale, out,
                            out_lse, nullptr, 0, n_splits, nullptr, nullptr, nullptr, stream,
                            nullptr, nullptr, false, false, true);
}

size_t stv_noalloc_scratch_bytes(void) { return stv::kNoAllocScratchBytes; }

int stv_verify_attention_fp16acc(const float *q, int32_t T, int32_t n_q_heads,
                                 const stv_kv_layer *kv, int32_t ctx_len,
                                 const uint64_t *anc_mask, float softmax_scale, float *out,
                                 float *out_lse, void *workspace, size_t workspace_bytes,
                                 int32_t n_splits, void *stream) {
    return attention_common(q, T, n_q_heads, kv, ctx_len, anc_mask, false, softmax_scale, out,
                            out_lse, workspace, workspace_bytes, n_splits, nullptr, nullptr,
                            nullptr, stream, nullptr, nullptr, true);
}

int stv_prefill_attention(const float *q, int32_t T, int32_t n_q_heads, const stv_kv_layer *kv,
                          int32_t ctx_len, float softmax_scale, float *out, float *out_lse,
                          void *workspace, size_t workspace_bytes, int32_t n_splits,
                          int32_t *dbg_logits, int8_t *dbg_q, float *dbg_qscale, void *stream) {
    return attention_common(q, T, n_q_heads, kv, ctx_len, nullptr, true, softmax_scale, out,
                            out_lse, workspace, workspace_bytes, n_splits, dbg_logits, dbg_q,
                            dbg_qscale, stream);
}

int stv_attention_partials(const float *q, int32_t T, int32_t n_q_heads,
                           const stv_kv_layer *kv, int32_t ctx_len, const uint64_t *anc_mask,
                           float softmax_scale, int32_t n_splits, float *part_o,
                           float *part_lse, void *stream) {
    if (!part_o) return fail(STV_EINVAL, "part_o must not be NULL");
    return attention_common(q, T, n_q_heads, kv, ctx_len, anc_mask, anc_mask == nullptr,
                            softmax_scale, nullptr, nullptr, nullptr, 0, n_splits, nullptr,
                            nullptr, nullptr, stream, part_o, part_lse);
}

int stv_context_plan(int32_t T, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     int32_t n_keys, int32_t kv_format, int32_t n_splits_req,
                     int32_t *n_splits_out, size_t *workspace_bytes_out) {
    if (kv_format != STV_KV_3BIT && kv_format != STV_KV_4BIT_TOKEN)
        return fail(STV_EINVAL, "kv_format %d unknown", kv_format);
    if (T < 1 || T > STV_MAX_TREE_ROWS) return fail(STV_EINVAL, "T must be in 1..64");
    int rc = check_heads(n_q_heads, n_kv_heads, head_dim);
    if (rc) return rc;
    if (n_keys < 1) return fail(STV_EINVAL, "n_keys must be >= 1");
    if (n_splits_req < 0) return fail(STV_EINVAL, "n_splits must be >= 0");
    const stv::Plan p = stv::make_plan_keys(T, n_q_heads, n_kv_heads, head_dim, n_keys, false,
                                            n_splits_req, kv_format, 0);
    if (n_splits_out) *n_splits_out = p.S;
    if (workspace_bytes_out) *workspace_bytes_out = p.ws_bytes;
    return ok();
}

int stv_context_partials(const float *q, int32_t T, int32_t n_q_heads, const stv_kv_layer *kv,
                         int32_t n_keys, float softmax_scale, int32_t n_splits, float *part_o,
                         float *part_lse, void *stream) {
    if (!part_o) return fail(STV_EINVAL, "part_o must not be NULL");
    return attention_common(q, T, n_q_heads, kv, n_keys, nullptr, false, softmax_scale, nullptr,
                            nullptr, nullptr, 0, n_splits, nullptr, nullptr, nullptr, stream,
                            part_o, part_lse, false, true);
}

int stv_split_merge(const float *part_o, const float *part_lse, int32_t S, int32_t rows,
                    int32_t D, float *out, float *out_lse, void *stream) {
    if (S < 1) return fail(STV_EINVAL, "S must be >= 1");
    if (rows < 0) return fail(STV_EINVAL, "rows must be >= 0");
    if (D < 1 || D > 1024) return fail(STV_EINVAL, "D must be in 1..1024");
    if (rows == 0) return ok();
    if (!part_o || !part_lse || !out) return fail(STV_EINVAL, "part_o, part_lse and out must not be NULL");
    if ((D & 3) == 0 &&
        ((reinterpret_cast<uintptr_t>(part_o) | reinterpret_cast<uintptr_t>(out)) & 15u) != 0)
        return fail(STV_EINVAL, "part_o and out must be 16-byte aligned when D %% 4 == 0");
    hipError_t e = stv::launch_merge(part_o, part_lse, S, rows, D, out, out_lse,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(STV_EHIP, "merge launch failed: %s", hipGetErrorString(e));
    return ok();
}

int stv_tree_accept(const uint64_t *anc_mask, int32_t T, const int32_t *draft,
                    const int32_t *target, int32_t *path, int32_t *n_accepted, int32_t *bonus,
                    void *stream) {
    if (T < 1 || T > STV_MAX_TREE_ROWS) return fail(STV_EINVAL, "T must be in 1..64 (got %d)", T);
    if (!anc_mask) return fail(STV_EINVAL, "anc_mask must not be NULL");
    if (!draft || !target || !path || !n_accepted || !bonus)
        return fail(STV_EINVAL, "draft, target, path, n_accepted and bonus must not be NULL");
    int rc = check_mask(anc_mask, T);
    if (rc) return rc;
    stv::AcceptArgs a;
    memset(&a, 0, sizeof a);
    for (int i = 0; i < T; ++i) a.mask[i] = anc_mask[i];
    a.T = T;
    a.draft = draft;
    a.target = target;
    a.path = path;
    a.n_accepted = n_accepted;
    a.bonus = bonus;
    hipError_t e = stv::launch_tree_accept(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(STV_EHIP, "tree_accept launch failed: %s", hipGetErrorString(e));
    return ok();
}

int stv_kv_commit(const stv_kv_layer *kv, int32_t ctx_len, int32_t T, const int32_t *path,
                  const int32_t *n_accepted, void *stream) {
    if (!kv) return fail(STV_EINVAL, "kv is NULL");
    if (!kv->k_codes || !kv->k_scales || !kv->v_codes || !kv->v_scales)
        return fail(STV_EINVAL, "kv has a NULL array");
    if (T < 1 || T > STV_MAX_TREE_ROWS) return fail(STV_EINVAL, "T must be in 1..64 (got %d)", T);
    if (!path || !n_accepted) return fail(STV_EINVAL, "path and n_accepted must not be NULL");
    const int D = kv->head_dim;
    if (D != 64 && D != 128 && D != 256) return fail(STV_EINVAL, "head_dim must be 64, 128 or 256");
    if (kv->n_kv_heads < 1) return fail(STV_EINVAL, "n_kv_heads must be >= 1");
    if (kv->capacity <= 0) return fail(STV_EINVAL, "capacity must be positive");
    if (kv->kv_format != STV_KV_3BIT && kv->kv_format != STV_KV_4BIT_TOKEN)
        return fail(STV_EINVAL, "kv_format %d unknown", kv->kv_format);
    if (ctx_len < 0) return fail(STV_EINVAL, "ctx_len must be >= 0");
    if ((long long)ctx_len + T > kv->capacity)
        return fail(STV_ECAPACITY, "ctx_len + T = %lld exceeds capacity %d", (long long)ctx_len + T,
                    kv->capacity);
    stv::CommitArgs a;
    // the layer's arrays are the caller's writable device memory; this call
    // is the one that writes through them
    a.kc = const_cast<uint32_t *>(kv->k_codes);
    a.ks = const_cast<uint16_t *>(kv->k_scales);
    a.vc = const_cast<uint32_t *>(kv->v_codes);
    a.vs = const_cast<uint16_t *>(kv->v_scales);
    a.Hkv = kv->n_kv_heads;
    a.D = D;
    a.cap = kv->capacity;
    a.ngroups = (kv->capacity + 31) / 32;
    a.fmt = kv->kv_format;
    a.L = ctx_len;
    a.T = T;
    a.path = path;
    a.n_accepted = n_accepted;
    hipError_t e = stv::launch_kv_commit(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(STV_EHIP, "kv_commit launch failed: %s", hipGetErrorString(e));
    return ok();
}

int stv_lookup_plan(int32_t batch, int32_t stride, size_t *workspace_bytes) {
    if (batch < 0 || batch > 65535) return fail(STV_EINVAL, "batch must be in 0..65535 (got %d)", batch);
    if (stride < 1) return fail(STV_EINVAL, "stride must be >= 1 (got %d)", stride);
    if (!workspace_bytes) return fail(STV_EINVAL, "workspace_bytes must not be NULL");
    *workspace_bytes = (size_t)batch * (size_t)stv::lookup_chunks(stride) * sizeof(uint64_t);
    return ok();
}

int stv_lookup_draft(const int32_t *history, const int32_t *lengths, int32_t batch,
                     int32_t stride, int32_t n_min, int32_t n_max, int32_t k, int32_t *tokens,
                     int32_t *count, int32_t *match, int32_t *pos, void *workspace,
                     size_t workspace_bytes, void *stream) {
    size_t need = 0;
    int rc = stv_lookup_plan(batch, stride, &need);
    if (rc) return rc;
    if (n_min < 1 || n_max < n_min || n_max > stv::kLookupMaxN)
        return fail(STV_EINVAL, "need 1 <= n_min <= n_max <= %d (got %d, %d)", stv::kLookupMaxN,
                    n_min, n_max);
    if (k < 0 || k > 4096) return fail(STV_EINVAL, "k must be in 0..4096 (got %d)", k);
    if (batch == 0) return ok();
    if (!history || !lengths || !count || !match || !pos || (k > 0 && !tokens))
        return fail(STV_EINVAL, "history, lengths, tokens, count, match and pos must not be NULL");
    if (!workspace || workspace_bytes < need)
        return fail(STV_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    stv::LookupArgs a;
    a.hist = history;
    a.len = lengths;
    a.B = batch;
    a.stride = stride;
    a.n_min = n_min;
    a.n_max = n_max;
    a.k = k;
    a.n_chunks = stv::lookup_chunks(stride);
    a.vec16 = (stride % 4) == 0 && (reinterpret_cast<uintptr_t>(history) & 15u) == 0;
    a.ws = static_cast<uint64_t *>(workspace);
    a.tokens = tokens;
    a.count = count;
    a.match = match;
    a.pos = pos;
    hipError_t e = stv::launch_lookup(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(STV_EHIP, "lookup launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
