/*
 * stv.h -- C ABI of the speculative tree-verify attention library for
 * MI355X (gfx950).
 *
 * The operation: in a speculative verify round, a block of draft-tree query
 * rows attends over a long KV cache quantized to 3 bits with one fp16 scale
 * per 32 elements (elpis, "Setup": 3-bit KV, 262,144-token context; "How": an
 * 8-row token tree whose rows see their ancestors).  Q.K^T is computed
 * exactly in int8/int32 with the 3-bit K codes widened to int8 (elpis, "Why
 * fast": decode verify and prefill int8 Q.K^T on integer matrix units),
 * softmax runs in fp32 and P.V accumulates in fp32 (elpis, "What fast
 * means": fp16-accumulated P.V was not shipped; elpis-lossless, "Lossless":
 * fp32 sums), and the context is split across work-groups whose partial
 * results are joined by a log-sum-exp merge (elpis-lossless, "Trust base":
 * the split-K barrier; elpis, "Why fast": the prefill merge).
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless marked [host].
 *  - The caller owns all memory.  The library never allocates or frees.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream).  No entry point synchronizes the host.
 *  - Every argument is validated on the host before any HIP call, so every
 *    error path returns without touching the GPU.  The return value is
 *    STV_OK or a negative STV_E* code; stv_last_error() (thread-local) then
 *    describes the failure.
 *  - Results are deterministic: a call with the same arguments produces
 *    bitwise identical outputs (fixed split partition, fixed merge order).
 *  - NaN or Inf in the inputs is not checked and propagates.
 *
 * Cache layout (one layer).  A "block" is three 32-bit words holding 32
 * codes c in [0, 7]; a code stands for scale * (c - 4).
 *  K, token-major:
 *    k_codes  uint32 [Hkv][capacity][D/32][3]   block (key, b): elements 32b..32b+31
 *    k_scales uint16 [Hkv][capacity][D/32]      fp16 bits, one per block
 *  V, key-transposed in groups of 32 keys (ng = ceil(capacity / 32)):
 *    v_codes  uint32 [Hkv][ng][D][3]            block (group, d): element d of
 *                                               keys 32*group .. 32*group+31
 *    v_scales uint16 [Hkv][ng][D/32][32]        fp16 bits: scale of elements
 *                                               32b..32b+31 of each key
 * K streams with the model dimension contiguous, V with the key dimension
 * contiguous: the dimension each product contracts over.
 * Bit layout of a block ("byte-plane"), code e = 4*qq + i:
 *   qq 0,1: word 0 bits [8i + 3qq, +3)      qq 2,3: word 1 bits [8i + 3(qq-2), +3)
 *   qq 4,5: word 2 bits [8i + 3(qq-4), +3)
 *   qq 6:   code bits 0-1 at word 0 bits [8i+6, 8i+8), bit 2 at word 2 bit 8i+6
 *   qq 7:   code bits 0-1 at word 1 bits [8i+6, 8i+8), bit 2 at word 2 bit 8i+7
 * so that one shift and one mask yield four codes in the four bytes of a
 * word.  Supported head_dim: 64, 128, 256.
 */
#ifndef STV_H
#define STV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STV_OK 0
#define STV_EINVAL (-1)     /* bad shape, pointer or argument */
#define STV_EMASK (-2)      /* ancestor mask is not a forest of root-to-node paths */
#define STV_ECAPACITY (-3)  /* ctx_len + T exceeds the cache capacity */
#define STV_EWORKSPACE (-4) /* workspace missing or too small for the split plan */
#define STV_EHIP (-5)       /* the HIP runtime reported an error at launch */

#define STV_MAX_TREE_ROWS 64

#define STV_K 0              /* stv_kv_quant_pack: K, 3-bit format */
#define STV_V 1              /* stv_kv_quant_pack: V, 3-bit format */
#define STV_K4 2             /* stv_kv_quant_pack: K, 4-bit per-token-head format */
#define STV_V4 3             /* stv_kv_quant_pack: V, 4-bit per-token-head format */

/*
 * Cache formats.
 *  STV_KV_3BIT (the layout above): 3-bit codes, one fp16 scale per 32
 *    elements of a (token, KV head) row.
 *  STV_KV_4BIT_TOKEN: 4-bit codes c in [0, 15] standing for s * (c - 8), one
 *    fp16 scale per (token, KV head) (the int4 per-token-head cache of the
 *    "Qwen3.8-27B on one RTX 3090" page, int4 KV section):
 *      k_codes  uint32 [Hkv][capacity][D/8]   element 8w + i in bits [4i, 4i+4)
 *                                             of word w
 *      k_scales uint16 [Hkv][capacity]        fp16 bits, one per (key, head)
 *      v_codes  uint32 [Hkv][ng][D][4]        row (group, d): element d of the
 *                                             group's 32 keys, key e in word
 *                                             e/8 bits [4(e%8), +4)
 *      v_scales uint16 [Hkv][capacity]        fp16 bits, one per (key, head)
 *    k_codes and v_codes must be 16-byte aligned.  Q.K^T is one exact int32
 *    sum per (row, key) over the whole head dimension.
 */
#define STV_KV_3BIT 0
#define STV_KV_4BIT_TOKEN 1

/* One layer's quantized cache (layouts above).  Passed by [host] pointer. */
typedef struct stv_kv_layer {
    const uint32_t *k_codes;
    const uint16_t *k_scales;
    const uint32_t *v_codes;
    const uint16_t *v_scales;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t capacity;
    int32_t kv_format;      /* STV_KV_3BIT or STV_KV_4BIT_TOKEN */
} stv_kv_layer;

/* Description of the last failure on the calling thread ("" after success). */
const char *stv_last_error(void);

/* ABI version; bumped on any change of the interface.  Currently 5. */
int32_t stv_abi_version(void);

/*
 * stv_kv_quant_pack -- write new tokens' K or V rows into the 3-bit cache
 * (the 3-bit KV cache of elpis, "Setup"; the pages do not state the rule).
 * Call once for K (which = STV_K) and once for V (which = STV_V).
 *   x       fp32 [n_tok][n_kv_heads][head_dim], the new rows
 *   pos0    first cache position written; positions pos0 .. pos0+n_tok-1
 *           are overwritten, every other position is left untouched (for V
 *           only those keys' bits and scales change in the shared blocks)
 *   codes, scales   the cache arrays of that tensor (layout above)
 * Rule per 32-element block: s = fp16_rne(amax / 3) (the largest finite fp16
 * if that overflows), code = clamp(rint(x / s), -4, 3) + 4, all codes 4 when
 * s is zero; the division is correctly rounded and rint rounds half to even.
 * which = STV_K4 / STV_V4 write the 4-bit per-token-head format instead:
 * one scale per (token, head) row of head_dim elements, s = fp16_rne(amax /
 * 7) (saturated likewise), code = clamp(rint(x / s), -8, 7) + 8, all codes 8
 * when s is zero; scales are [n_kv_heads][capacity] for K and V alike.
 * Calls for the same tensor that touch the same 32-key group of V must not
 * run concurrently (they rewrite shared words).  x must be 16-byte aligned.
 * Errors: STV_EINVAL (null pointer, n_tok < 0, bad head_dim, heads or
 * which), STV_ECAPACITY (pos0 < 0 or pos0 + n_tok > capacity), STV_EHIP.
 */
int stv_kv_quant_pack(const float *x, int32_t n_tok, int32_t pos0, int32_t which,
                      uint32_t *codes, uint16_t *scales, int32_t n_kv_heads,
                      int32_t head_dim, int32_t capacity, void *stream);

/*
 * stv_attention_plan -- the split plan a verify (causal = 0) or prefill
 * (causal = 1) call with these sizes and cache format (STV_KV_3BIT or
 * STV_KV_4BIT_TOKEN) will use, and the workspace it needs.
 *   n_splits_req  0 lets the library choose; otherwise the requested number
 *                 of context splits (the effective count may be lower: each
 *                 split covers a whole number of 32-key tiles)
 *   n_splits_out  [host] effective split count S
 *   workspace_bytes_out [host] bytes of workspace the call needs (0 when S = 1):
 *                 stv_workspace_bytes(T, n_q_heads, head_dim, S), except for
 *                 a prefill call on the 3-bit format with eight or more groups
 *                 of 128 query rows per KV head (T * n_q_heads / n_kv_heads >
 *                 896).  There it adds, after the partials rounded up to 256
 *                 bytes, one unpacked image of every 32-key tile per KV head
 *                 (ceil((ctx_len + T) / 32) * n_kv_heads images, a whole number
 *                 of KiB each: about 31 KiB at head_dim 256): the call then
 *                 unpacks each tile once instead of once per row group.  A
 *                 workspace that holds the partials only still works (every
 *                 row group unpacks the tiles itself); the results are the
 *                 same bit for bit.
 * Errors: STV_EINVAL, STV_ECAPACITY is not checked here (no capacity given).
 */
int stv_attention_plan(int32_t T, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                       int32_t ctx_len, int32_t causal, int32_t kv_format, int32_t n_splits_req,
                       int32_t *n_splits_out, size_t *workspace_bytes_out);

/*
 * stv_workspace_bytes -- workspace a verify or prefill call with a known
 * split count S needs: the split partials O_s (fp32 [S][T * n_q_heads]
 * [head_dim]) followed by their log-sum-exps (fp32 [S][T * n_q_heads]),
 * i.e. S * T * n_q_heads * (head_dim + 1) * 4 bytes, or 0 when S = 1 (one
 * split writes the output directly).  Split-K with a merge of the partials:
 * elpis-lossless, "Trust base" (the split-K barrier); elpis, "Why fast" (the
 * prefill merge).  stv_attention_plan gives S (and this same size, plus
 * tile images for a large 3-bit prefill chunk) for a call whose split count
 * the library chooses.
 *   T, n_q_heads  query rows and heads of the call (T >= 1, n_q_heads >= 1)
 *   head_dim      64, 128 or 256
 *   n_splits      the call's effective split count S >= 1
 * Returns the byte count; on invalid arguments returns 0 and sets
 * stv_last_error.  No HIP call, no allocation.
 */
size_t stv_workspace_bytes(int32_t T, int32_t n_q_heads, int32_t head_dim, int32_t n_splits);

/*
 * stv_verify_attention -- attention of T draft-tree rows over the cache
 * (elpis, "Why fast": decode verify with int8 Q.K^T; "How": the token tree).
 *   q           fp32 [T][n_q_heads][head_dim]; query head h reads kv head
 *               h / (n_q_heads / n_kv_heads)
 *   T           1 .. 64 tree rows
 *   kv          [host] the layer's cache.  Keys 0 .. ctx_len-1 are the
 *               context; the T rows' own K/V must already sit at positions
 *               ctx_len .. ctx_len+T-1 (written with stv_kv_quant_pack)
 *   anc_mask    [host] uint64 [T]: bit a of anc_mask[i] is set iff tree row a
 *               is row i or an ancestor of it.  Every row must have its own
 *               bit and no bit above it, and the rest of its bits must be
 *               exactly the mask of its highest other row (its parent), so
 *               the rows form a forest and each row sees a root-to-node path
 *   softmax_scale  positive, multiplies the logits (commonly 1/sqrt(head_dim))
 *   out         fp32 [T][n_q_heads][head_dim]
 *   out_lse     nullable fp32 [T][n_q_heads]: natural-log log-sum-exp of each
 *               row's scaled logits, for merging with results over other
 *               key ranges
 *   workspace, workspace_bytes  device scratch of at least the plan's bytes
 *               (may be NULL when the plan has S = 1)
 *   n_splits    0 = automatic, else requested split count (see the plan)
 *   dbg_logits  nullable int32 [T][n_q_heads][ctx_len+T][head_dim/32]: the
 *               exact per-block integer Q.K^T sums (3-bit format), or
 *               [T][n_q_heads][ctx_len+T]: the exact whole-row sums (4-bit
 *               format); entries of keys a row cannot see are unspecified
 *   dbg_q       nullable int8 [T][n_q_heads][head_dim]: the quantized Q
 *   dbg_qscale  nullable fp32 [T][n_q_heads]: the Q scales
 * q, out and workspace must be 16-byte aligned (the kernels move them in
 * 16-byte vectors).
 * Per-row Q quantizer: amax = max|q|; inv = 127 / amax (correctly rounded);
 * q8 = clamp(rint(q * inv), -127, 127); sq = amax / 127; a zero row gives
 * sq = 0 and zero codes.  Logit of key j: softmax_scale * sq *
 * sum_b k_scale[j][b] * S_b[j] with S_b the int32 block sums.
 * Value range: P.V takes fp16 operands (elpis-lossless, "Trust base": the
 * m16n8k16 fp16 shape).  Calls of more than 16 rows per kv head (3-bit
 * format) and the 4-bit format above 64 rows dequantize V to fp16 s (c - 4)
 * (4-bit: s (c - 8)), so V scales must stay at or below 16,376 (4-bit:
 * 8,188); beyond that the result is undefined.  Calls of up to 16 rows per
 * kv head (4-bit: 64) accept every finite V scale.
 * Errors: STV_EINVAL, STV_EMASK, STV_ECAPACITY, STV_EWORKSPACE, STV_EHIP.
 */
int stv_verify_attention(const float *q, int32_t T, int32_t n_q_heads,
                         const stv_kv_layer *kv, int32_t ctx_len, const uint64_t *anc_mask,
                         float softmax_scale, float *out, float *out_lse, void *workspace,
                         size_t workspace_bytes, int32_t n_splits, int32_t *dbg_logits,
                         int8_t *dbg_q, float *dbg_qscale, void *stream);

/*
 * stv_verify_attention_noalloc -- stv_verify_attention for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The split partials go to a
 * file-scope device array of the library, STV_NOALLOC_SCRATCH_BYTES (64 MiB)
 * per GPU, held from the library's first such call on that GPU until the
 * process ends; the call allocates nothing.  Every call on a GPU shares that
 * GPU's array, which keeps the last call's contents: calls that overlap on
 * one GPU (on different streams, or from different threads) race and give
 * undefined results.  The caller still passes q, out and out_lse.
 *   n_splits  0 = automatic, capped at the splits whose partials
 *             (n_splits * T * n_q_heads * (head_dim + 1) * 4 bytes) fit the
 *             array; an explicit count that does not fit is STV_EWORKSPACE
 * Other arguments, results (bit for bit, at the same split count) and
 * errors as for stv_verify_attention, without the debug outputs.
 */
#define STV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int stv_verify_attention_noalloc(const float *q, int32_t T, int32_t n_q_heads,
                                 const stv_kv_layer *kv, int32_t ctx_len,
                                 const uint64_t *anc_mask, float softmax_scale, float *out,
                                 float *out_lse, int32_t n_splits, void *stream);
/* Bytes of the array above (STV_NOALLOC_SCRATCH_BYTES).  No HIP call. */
size_t stv_noalloc_scratch_bytes(void);

/*
 * stv_verify_attention_fp16acc -- stv_verify_attention with P.V accumulated
 * in fp16 (elpis, "What fast means": the fp16-accumulated P.V decode kernel,
 * left unresolved there and not shipped).  Each 32-key tile's P.V product
 * is computed in fp32, rounded to fp16 and added into fp16 accumulators; the
 * running max follows every increase, so P <= 1.  An accumulator overflows
 * to inf when a split's sum of P * |V| passes 65504 (all keys of a split
 * about equally likely and |V| large); the result is then undefined.
 * Arguments, workspace (same plan) and errors as for stv_verify_attention,
 * without the debug outputs; the 3-bit format only (STV_EINVAL otherwise).
 */
int stv_verify_attention_fp16acc(const float *q, int32_t T, int32_t n_q_heads,
                                 const stv_kv_layer *kv, int32_t ctx_len,
                                 const uint64_t *anc_mask, float softmax_scale, float *out,
                                 float *out_lse, void *workspace, size_t workspace_bytes,
                                 int32_t n_splits, void *stream);

/*
 * stv_prefill_attention -- the chunked-prefill variant (elpis, "Why fast":
 * prefill int8 Q.K^T, the K/V double-buffered ring, the prefill merge): T
 * new rows, row t sees keys 0 .. ctx_len+t.  Arguments as for
 * stv_verify_attention without anc_mask; T may be any positive count with
 * T * n_q_heads < 2^31.  The workspace must hold the partials
 * (stv_workspace_bytes); with the plan's full size (stv_attention_plan) a
 * chunk of many row groups per KV head unpacks each tile once into it.
 * Errors: STV_EINVAL, STV_ECAPACITY, STV_EWORKSPACE, STV_EHIP.
 */
int stv_prefill_attention(const float *q, int32_t T, int32_t n_q_heads,
                          const stv_kv_layer *kv, int32_t ctx_len, float softmax_scale,
                          float *out, float *out_lse, void *workspace, size_t workspace_bytes,
                          int32_t n_splits, int32_t *dbg_logits, int8_t *dbg_q,
                          float *dbg_qscale, void *stream);

/*
 * stv_attention_partials -- the split phase alone: each of the S context
 * splits of the plan writes its normalised partial output and its
 * log-sum-exp, to be joined by stv_split_merge (elpis-lossless, "Trust
 * base": split-K; the same partials serve a context range computed on
 * another device).  stv_verify_attention with S > 1 is exactly this call
 * followed by stv_split_merge.
 *   q, T, n_q_heads, kv, ctx_len, softmax_scale, n_splits: as for
 *               stv_verify_attention / stv_prefill_attention
 *   anc_mask    [host] uint64 [T] tree masks (as for verify), or NULL for
 *               the causal chunk rule of prefill
 *   part_o      fp32 [S][T][n_q_heads][head_dim], S from stv_attention_plan;
 *               16-byte aligned, as are q
 *   part_lse    fp32 [S][T][n_q_heads], natural log; -inf where a split saw
 *               no key of that row (its part_o row is then zero)
 * Split s covers keys [s*P, min(ctx_len+T, (s+1)*P)) with
 * P = 32 * ceil(ceil((ctx_len+T)/32) / S).
 * Errors: STV_EINVAL, STV_EMASK, STV_ECAPACITY, STV_EHIP.
 */
int stv_attention_partials(const float *q, int32_t T, int32_t n_q_heads,
                           const stv_kv_layer *kv, int32_t ctx_len, const uint64_t *anc_mask,
                           float softmax_scale, int32_t n_splits, float *part_o,
                           float *part_lse, void *stream);

/*
 * stv_context_plan / stv_context_partials -- the split phase over a slice of
 * the context with no tree keys: every one of the T rows sees keys
 * 0 .. n_keys-1 of kv (elpis-lossless, "Trust base": split-K over the
 * context; the partials of a context range held elsewhere, e.g. on another
 * device, joined by stv_split_merge with those of the slice that holds the
 * tree keys, which stv_attention_partials computes).
 *   q, T (1 .. 64), n_q_heads, softmax_scale, n_splits: as for
 *               stv_attention_partials
 *   n_keys      keys of the slice (>= 1, at most the cache capacity)
 *   part_o, part_lse  as for stv_attention_partials, S from stv_context_plan;
 *               split s covers keys [s*P, min(n_keys, (s+1)*P)) with
 *               P = 32 * ceil(ceil(n_keys/32) / S)
 * A slice whose length is a multiple of 32 gives, split for split, the same
 * partials bit for bit as the matching splits of one call over the whole
 * context.  Errors: STV_EINVAL, STV_ECAPACITY, STV_EHIP.
 */
int stv_context_plan(int32_t T, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     int32_t n_keys, int32_t kv_format, int32_t n_splits_req,
                     int32_t *n_splits_out, size_t *workspace_bytes_out);
int stv_context_partials(const float *q, int32_t T, int32_t n_q_heads, const stv_kv_layer *kv,
                         int32_t n_keys, float softmax_scale, int32_t n_splits, float *part_o,
                         float *part_lse, void *stream);

/*
 * stv_split_merge -- join split partials with a log-sum-exp merge
 * (elpis-lossless, "Trust base": the split-K barrier; elpis, "Why fast":
 * the prefill merge).
 *   part_o    fp32 [S][rows][D], each split's normalised output
 *   part_lse  fp32 [S][rows], natural log; -inf marks a split that saw no key
 *   out       fp32 [rows][D] = sum_s exp(lse_s - LSE) * part_o[s], with
 *             LSE = log sum_s exp(lse_s); rows whose splits are all -inf
 *             get zeros
 *   out_lse   nullable fp32 [rows], receives LSE
 * The summation order depends only on S and D (no atomics), so results are
 * reproducible bit for bit.  D: 1 .. 1024; part_o and out 16-byte aligned
 * when D is a multiple of 4.
 * Errors: STV_EINVAL, STV_EHIP.
 */
int stv_split_merge(const float *part_o, const float *part_lse, int32_t S, int32_t rows,
                    int32_t D, float *out, float *out_lse, void *stream);

/*
 * stv_tree_accept -- greedy acceptance over the draft tree (elpis, "Why
 * fast": the 8-row token tree, commit the longest matching path plus one
 * token; elpis-lossless, "Lossless": token ids are compared exactly, nothing
 * is sampled or thresholded).
 *   anc_mask    [host] uint64 [T], the verify call's tree masks (same rules)
 *   T           1 .. 64 tree rows; node 0 is the round's root, already decided
 *   draft       int32 [T], token id of each tree node
 *   target      int32 [T], the target's greedy token at each tree row (the
 *               token that follows the node's path)
 *   path        int32 [T] out: the committed nodes in increasing order, then
 *               -1 in the entries past the count
 *   n_accepted  int32 [1] out: number of committed nodes, >= 1 (the root)
 *   bonus       int32 [1] out: the extra token, target[last committed node]
 * Node i > 0 matches when draft[i] == target[parent of i]; a node can end
 * the path when it lies below node 0 and every node on its path below node 0
 * matches; the deepest such node wins, the lowest index among equals.
 * Errors: STV_EINVAL, STV_EMASK, STV_EHIP.
 */
int stv_tree_accept(const uint64_t *anc_mask, int32_t T, const int32_t *draft,
                    const int32_t *target, int32_t *path, int32_t *n_accepted, int32_t *bonus,
                    void *stream);

/*
 * stv_kv_commit -- keep only the committed tree tokens in the cache, at
 * consecutive positions (elpis-lossless, "How": the accepted path's K/V is
 * what stays; the rejected nodes' rows are free again).
 *   kv          [host] the layer's cache, written in place through its
 *               arrays; the tree's K/V sits at ctx_len + i
 *   ctx_len, T  context before the tree, tree rows (1 .. 64);
 *               ctx_len + T <= capacity
 *   path, n_accepted  device outputs of stv_tree_accept (read on the device,
 *               so the call needs no host synchronisation)
 * For j < n: the K codes, K scales, V codes and V scales of position
 * ctx_len + path[j] move to position ctx_len + j in every KV head; all
 * sources are read before any destination is written.  Every other cache
 * entry keeps its value.  The next round continues at ctx_len + n.  A count
 * outside [1, T] or a path entry outside [0, T) found on the device leaves
 * the cache unchanged.
 * Errors: STV_EINVAL, STV_ECAPACITY, STV_EHIP.
 */
int stv_kv_commit(const stv_kv_layer *kv, int32_t ctx_len, int32_t T, const int32_t *path,
                  const int32_t *n_accepted, void *stream);

/*
 * stv_lookup_plan / stv_lookup_draft -- lookup drafting: propose draft
 * tokens by finding the latest earlier occurrence of a request's last
 * tokens in its own history and copying what followed (u/iamMess,
 * lookup-augmented drafting, which scans for the last 6-12 tokens; elpis,
 * the drafter-free n-gram chains).  Batched over B sequences.
 *   history     int32 [B][stride] token ids; row b holds lengths[b] tokens
 *   lengths     int32 [B] (device), clamped to [0, stride] on the device
 *   n_min, n_max  1 <= n_min <= n_max <= 64 (6 and 12 on the pages)
 *   k           0 .. 4096 proposed tokens per sequence
 *   tokens      int32 [B][k] out: the proposal, then -1
 *   count, match, pos  int32 [B] out: proposal length, match length, end
 *               position e of the matched occurrence (-1 when none)
 *   workspace   device bytes, at least stv_lookup_plan's figure
 *               (B * ceil((stride-1)/4096) * 8); contents are scratch
 * An end position e <= N-2 matches m(e) tokens when h[e-i] == h[N-1-i] for
 * i < m(e), with m(e) <= min(n_max, e+1); candidates have m(e) >= n_min; the
 * longest match wins, then the largest e; the proposal is h[e+1 ..], at most
 * k tokens and never past the history's end.  B <= 65535.
 * Errors: STV_EINVAL, STV_EWORKSPACE, STV_EHIP.
 */
int stv_lookup_plan(int32_t batch, int32_t stride, size_t *workspace_bytes);
int stv_lookup_draft(const int32_t *history, const int32_t *lengths, int32_t batch,
                     int32_t stride, int32_t n_min, int32_t n_max, int32_t k, int32_t *tokens,
                     int32_t *count, int32_t *match, int32_t *pos, void *workspace,
                     size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* STV_H */
