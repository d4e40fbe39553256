// HIP kernels for gfx950 (MI355X): K/V pack (3-bit blocks and 4-bit
// per-token-head), split attention with an int8 MFMA Q.K^T stage and an
// fp16-in / fp32-accumulate MFMA P.V stage, and the log-sum-exp merge of
// split partials.  Three attention kernels share that scheme:
// attn_split_kernel (32-row tiles, more than 64 rows per KV head: the 64-node
// tree, the prefill chunk), attn_split16_kernel (16-row tiles, 17..64 rows,
// 3-bit: the 8-row tree) and attn_dec_kernel (at most 16 rows, one token; up to
// 64 rows for the 4-bit format; per-wave tiles without work-group barriers).
//
// Method (elpis, "Why fast": decode-verify and prefill int8 Q.K^T with the
// 3-bit K codes widened to exact int8, the double-buffered K/V ring, the
// prefill merge; elpis-lossless, "Lossless" / "Trust base": fp32 sums,
// split-K with a barrier, rows computed from their own data only):
//   per (kv head, row group, context split) work-group
//     prologue: quantize each query row to int8 with an fp32 scale
//     per 32-key tile: stream codes+scales HBM -> registers (one tile ahead)
//       -> unpack into LDS (K as int8 c-4, V^T as fp16 s*(c-4))
//       -> per wave: int8 MFMA per 32-element block, fp32 scale epilogue,
//          visibility mask, online softmax (base 2), fp16 P into an fp32
//          MFMA accumulator over V^T
//     epilogue: normalise, write the partial (or the output when S = 1)
//   merge: out = sum_s exp(lse_s - LSE) O_s, splits in fixed order.
#include "stv_codes.h"
#include "stv_internal.h"

#include <math.h>

#include <mutex>
#include <type_traits>

namespace stv {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer descriptor on gfx9: 32-bit data format, no swizzle.
constexpr int kBufWord3 = 0x00020000;

// Four codes c in [0, 7] (one per byte) -> four int8 values c - 4, by one
// v_perm_b32 byte select from the table {-4, -3, -2, -1, 0, 1, 2, 3}.
constexpr uint32_t kI8Lo = 0xFFFEFDFCu;     // codes 0..3 -> -4..-1
constexpr uint32_t kI8Hi = 0x03020100u;     // codes 4..7 ->  0..3
__device__ __forceinline__ uint32_t codes_to_i8(uint32_t o) {
    return __builtin_amdgcn_perm(kI8Hi, kI8Lo, o);
}

// High bytes of the binary16 values c - 4 for c = 0..7 (-4, -3, -2, -1, 0,
// 1, 2, 3: 0xC400 0xC200 0xC000 0xBC00 0x0000 0x3C00 0x4000 0x4200), as the
// two source words of a v_perm_b32 byte select (bytes 0-3 from kC4Lo).
constexpr uint32_t kC4Lo = 0xBCC0C2C4u;
constexpr uint32_t kC4Hi = 0x42403C00u;

// Combine a value with the same lane of the other 32-lane half.
// Maximum over lanes l and l ^ 16: v_permlane16_swap trades rows 2k + 1 of
// one copy with rows 2k of the other, so the two results hold, per lane, the
// values of both rows of its pair (a VALU exchange, no LDS round trip).
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A lane's part of one Q row for the int8 quantization in the attention
// prologues: C four-element chunks of every 32-element block b, at
// row + 32b + 4j.  All chunks load at once (one memory round trip, where a
// load under a per-lane condition was issued and waited for one chunk at a
// time), and the codes come from the same registers.  `row` must be readable
// for every lane, also where the lane's row is past the last one (the kernels
// point such lanes at a real row); valid = false gives a zero maximum and zero
// codes for them.
template <int NB, int C>
struct QPart {
    f32x4 v[NB][C];
    __device__ __forceinline__ void load(const float *row) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < C; ++j) v[b][j] = *reinterpret_cast<const f32x4 *>(row + 32 * b + 4 * j);
    }
    // largest magnitude of the lane's elements
    __device__ __forceinline__ float absmax(bool valid) const {
        float m = 0.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const f32x4 x = v[b][j];
                m = fmaxf(m, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
            }
        return valid ? m : 0.0f;
    }
    // int8 codes of chunk (b, j), element 4j + i in byte i: x * inv rounded
    // to nearest even, clamped to [-127, 127]
    __device__ __forceinline__ uint32_t codes(int b, int j, float inv, bool valid) const {
        const f32x4 x = v[b][j];
        const float e[4] = {x.x, x.y, x.z, x.w};
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float r = rintf(e[i] * inv);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            word |= ((uint32_t)(int)r & 0xFFu) << (8 * i);
        }
        return valid ? word : 0u;
    }
};

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// ---- integer form of a key's fp16 block scales (3-bit format).
//
// A finite binary16 scale is s = m * 2^(e - 25), with e its exponent field
// (1 for subnormals) and m its integer significand (hidden bit included for
// normals).  Over the nonzero scales of one key, with emin the smallest e,
// s_b = M_b * 2^(emin - 25) and M_b = m_b << (e_b - emin).  When every
// e_b - emin <= 3, M_b <= 2047 * 8 < 2^14, and with |S_b| <= 32 * 127 * 4 =
// 16,256 the key's whole sum  sum_b M_b * S_b  stays below 2^31 in magnitude:
// the block-scaled logit is one exact int32 sum, converted and scaled once.
// Keys whose exponents spread wider, or with an Inf/NaN scale, flag their
// tile for the per-block fp32 epilogue instead.
constexpr uint32_t kScaleNoExp = 31u;      // exponent of a zero scale: constrains nothing
constexpr uint32_t kScaleMaxShift = 3u;

// v_mad_i32_i16: sext(s[15:0]) * sext(16-bit half HI of m) + acc, exact for
// the operands above (|S_b| < 2^15, 0 <= M_b < 2^15, sums below 2^31).
//
// s is an MFMA result.  The compiler inserts the wait states a VALU read of
// an MFMA result needs only before instructions it can see, not before
// inline asm, so every asm read of an MFMA's results takes as an extra
// input `ready`, the result of a compiler-visible VALU read of the same
// MFMA (mfma_ready): the asm is then ordered after that read and its waits.
template <int HI>
__device__ __forceinline__ int32_t mad_i16(int32_t s, uint32_t m, int32_t acc, int32_t ready) {
    int32_t d;
    if constexpr (HI)
        asm("v_mad_i32_i16 %0, %1, %2, %3 op_sel:[0,1,0,0]"
            : "=v"(d) : "v"(s), "v"(m), "v"(acc), "v"(ready));
    else
        asm("v_mad_i32_i16 %0, %1, %2, %3" : "=v"(d) : "v"(s), "v"(m), "v"(acc), "v"(ready));
    return d;
}
// A compiler-visible VALU read of one result register of an MFMA (all of an
// MFMA's result registers are written when it completes).
__device__ __forceinline__ int32_t mfma_ready(int32_t s0) { return s0 & 1; }

// Minimum over the NB consecutive lanes (NB = 2, 4 or 8, aligned) holding
// the blocks of one key: quad permutations, then a half-row mirror.
template <int NB>
__device__ __forceinline__ uint32_t min_over_blocks(uint32_t v) {
    if constexpr (NB >= 2)
        v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    if constexpr (NB >= 4)
        v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    if constexpr (NB >= 8)
        v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    return v;
}

struct ScaleInt {
    uint32_t e, m;      // exponent field (1 for subnormals; kScaleNoExp when m == 0), significand
    bool special;       // Inf or NaN
};
__device__ __forceinline__ ScaleInt scale_int(uint16_t s16) {
    const uint32_t E = (s16 >> 10) & 31u, man = s16 & 1023u;
    ScaleInt r;
    r.special = E == 31u;
    r.m = E ? (man | 1024u) : man;
    r.e = r.m ? (E ? E : 1u) : kScaleNoExp;
    return r;
}
// 2^(emin - 25) as fp32 (emin in [1, 31])
__device__ __forceinline__ float scale_unit(uint32_t emin) {
    return __uint_as_float((emin + 102u) << 23);
}

// ------------------------------------------------------------- kv pack

// Quantize the 32 elements v[] with the symmetric rule: scale fp16(amax / 3)
// saturated to the largest finite value; code clamp(rint(x / s), -4, 3) + 4,
// all 4 when the scale is zero.  Divisions are IEEE correctly rounded.
__device__ __forceinline__ uint16_t block_scale(const float v[32]) {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
    _Float16 sh = (_Float16)(amax / 3.0f);            // RNE to binary16
    uint16_t s16 = __builtin_bit_cast(uint16_t, sh);
    if ((s16 & 0x7FFFu) == 0x7C00u) s16 = 0x7BFFu;     // saturate to 65504
    return s16;
}

__device__ __forceinline__ uint32_t code_of(float x, float s) {
    if (s == 0.0f) return 4u;
    float r = rintf(x / s);
    r = fminf(fmaxf(r, -4.0f), 3.0f);
    return (uint32_t)((int)r + 4);
}

__device__ __forceinline__ void load32(const float *src, float v[32]) {
    const f32x4 *p = reinterpret_cast<const f32x4 *>(src);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const f32x4 f = p[j];
        v[4 * j + 0] = f.x;
        v[4 * j + 1] = f.y;
        v[4 * j + 2] = f.z;
        v[4 * j + 3] = f.w;
    }
}

// K: one thread per (token, head, block); token-major layout.
__global__ void k_pack_kernel(const float *__restrict__ x, int n_tok, int pos0,
                              uint32_t *__restrict__ codes, uint16_t *__restrict__ scales,
                              int Hkv, int D, int cap) {
    const int NB = D / 32;
    const long long total = (long long)n_tok * Hkv * NB;
    const long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= total) return;
    const int b = (int)(id % NB);
    const int g = (int)((id / NB) % Hkv);
    const int t = (int)(id / ((long long)NB * Hkv));
    float v[32];
    load32(x + ((size_t)t * Hkv + g) * D + 32 * b, v);
    const uint16_t s16 = block_scale(v);
    const float s = half_bits_to_float(s16);
    uint32_t o[8];
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) word |= code_of(v[4 * qq + i], s) << (8 * i);
        o[qq] = word;
    }
    uint32_t w0, w1, w2;
    pack_bytes(o, w0, w1, w2);
    const size_t pos = (size_t)g * cap + (size_t)(pos0 + t);
    uint32_t *dst = codes + (pos * NB + b) * 3;
    dst[0] = w0;
    dst[1] = w1;
    dst[2] = w2;
    scales[pos * NB + b] = s16;
}

// V: one work-group of D threads per (head, 32-key group that holds new
// keys); the key-transposed layout puts the codes of 32 keys in each element
// row's three words, so one thread owns a row's read-modify-write.  The
// group's new rows are staged in LDS; thread i = (key e = i / NB, block
// b = i % NB) computes that block's scale from its 32 elements and writes it
// to the scale layout [Hkv][ng][D/32][32]; then thread d rewrites the three
// words of element row d, changing only the new keys.  The old code words are
// loaded first, so their latency overlaps the rows'.
__global__ __launch_bounds__(256) void v_pack_kernel(const float *__restrict__ x, int n_tok, int pos0,
                                                     uint32_t *__restrict__ codes,
                                                     uint16_t *__restrict__ scales, int Hkv, int D,
                                                     int ng, int grp0) {
    __shared__ float xs[32][8][33];      // [key][block][element], one float of padding per block
    __shared__ uint16_t ss[32][8];       // [key][block] scales
    const int NB = D / 32;
    const int g = (int)blockIdx.x % Hkv;
    const int grp = grp0 + (int)blockIdx.x / Hkv;
    const int d = threadIdx.x;           // element row (and, for the scales, key d / NB, block d % NB)
    const int e0 = max(0, pos0 - grp * 32), e1 = min(32, pos0 + n_tok - grp * 32);
    uint32_t *w = codes + (((size_t)g * ng + grp) * D + d) * 3;
    uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
    // every key's row is loaded (keys outside the new ones read a real new row,
    // unused), so all loads are issued before the first wait
    float xv[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        const int r = min(max(grp * 32 + e - pos0, 0), n_tok - 1);
        xv[e] = x[((size_t)r * Hkv + g) * D + d];
    }
#pragma unroll
    for (int e = 0; e < 32; ++e)
        if (e >= e0 && e < e1) xs[e][d >> 5][d & 31] = xv[e];
    __syncthreads();
    {
        const int e = d / NB, b = d - (d / NB) * NB;
        if (e >= e0 && e < e1) {
            float v[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) v[k] = xs[e][b][k];
            const uint16_t s16 = block_scale(v);
            ss[e][b] = s16;
            scales[(((size_t)g * ng + grp) * NB + b) * 32 + e] = s16;
        }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 32; ++e)
        if (e >= e0 && e < e1) set_code(w0, w1, w2, e, code_of(xv[e], half_bits_to_float(ss[e][d >> 5])));
    w[0] = w0;
    w[1] = w1;
    w[2] = w2;
}

// ---- 4-bit per-token-head pack.  One wave per (token, head): lane l holds
// elements 8l .. 8l+7 (l < D/8); scale fp16(amax / 7) saturated, code
// clamp(rint(x / s), -8, 7) + 8, all 8 when the scale is zero.  K writes its
// word directly; V writes the scales here and the codes in v4_code_kernel.
__device__ __forceinline__ uint16_t row_scale4(float amax) {
    _Float16 sh = (_Float16)(amax / 7.0f);              // RNE to binary16
    uint16_t s16 = __builtin_bit_cast(uint16_t, sh);
    if ((s16 & 0x7FFFu) == 0x7C00u) s16 = 0x7BFFu;
    return s16;
}

__device__ __forceinline__ uint32_t code4_of(float x, float s) {
    if (s == 0.0f) return 8u;
    float r = rintf(x / s);
    r = fminf(fmaxf(r, -8.0f), 7.0f);
    return (uint32_t)((int)r + 8);
}

template <bool IS_V>
__global__ __launch_bounds__(64) void kv4_pack_kernel(const float *__restrict__ x, int pos0,
                                                      uint32_t *__restrict__ codes,
                                                      uint16_t *__restrict__ scales, int Hkv,
                                                      int D, int cap) {
    // one work-group per (new token t, KV head g): the grid is n_tok * Hkv
    const int t = blockIdx.x / Hkv, g = blockIdx.x - (blockIdx.x / Hkv) * Hkv;
    const int l = threadIdx.x;
    const bool act = l < D / 8;
    const float *xr = x + ((size_t)t * Hkv + g) * D + 8 * l;
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float amax = 0.0f;
    if (act) {
        const f32x4 a0 = *reinterpret_cast<const f32x4 *>(xr);
        const f32x4 a1 = *reinterpret_cast<const f32x4 *>(xr + 4);
        v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
        v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const uint16_t s16 = row_scale4(amax);
    const size_t pos = (size_t)g * cap + (size_t)(pos0 + t);
    if (l == 0) scales[pos] = s16;
    if (!IS_V && act) {
        const float s = half_bits_to_float(s16);
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) w |= code4_of(v[e], s) << (4 * e);
        codes[pos * (size_t)(D / 8) + l] = w;
    }
}

// V codes: one thread per (group, head, d) row of four words, over the new
// keys of that group; scales come from kv4_pack_kernel<true>.
__global__ void v4_code_kernel(const float *__restrict__ x, int n_tok, int pos0,
                               uint32_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                               int Hkv, int D, int cap, int ng, int grp0, int n_grp) {
    const long long total = (long long)n_grp * Hkv * D;
    const long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= total) return;
    const int d = (int)(id % D);
    const int g = (int)((id / D) % Hkv);
    const int grp = grp0 + (int)(id / ((long long)D * Hkv));
    uint32_t *w = codes + (((size_t)g * ng + grp) * D + d) * 4;
    const int e0 = max(0, pos0 - grp * 32), e1 = min(32, pos0 + n_tok - grp * 32);
    float xv[32];
    uint16_t sv[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        xv[e] = 0.0f;
        sv[e] = 0;
        if (e >= e0 && e < e1) {
            xv[e] = x[((size_t)(grp * 32 + e - pos0) * Hkv + g) * D + d];
            sv[e] = scales[(size_t)g * cap + grp * 32 + e];
        }
    }
    uint32_t ww[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        if (e >= e0 && e < e1) {
            const uint32_t c = code4_of(xv[e], half_bits_to_float(sv[e]));
            ww[e / 8] = (ww[e / 8] & ~(15u << (4 * (e % 8)))) | (c << (4 * (e % 8)));
        }
    }
    w[0] = ww[0];
    w[1] = ww[1];
    w[2] = ww[2];
    w[3] = ww[3];
}

// ------------------------------------------------------------ attention

typedef float f32x2 __attribute__((ext_vector_type(2)));

// LDS layout of one 32-key tile.
//   kq : int8 K, [32 keys][D + 16] bytes (row pad keeps the A-operand reads
//        of 16 consecutive lanes on distinct banks)
//   vt : fp16 V^T, element (d, key) at d*VTS + (d/32)*VBPAD + key halves.
//        VTS = 40 keeps the B128 operand reads conflict-free; the per-block
//        pad of 16 dwords spreads the four blocks written by one wave over
//        all 64 banks.
//   skh: fp16 K scales, [D/32][32 keys] (3-bit format); skf: fp32 K scale
//        per key (4-bit per-token-head format)
//   skm, skf: the 3-bit K scales in integer form (M [D/32][32 keys], and the
//        key's unit 2^(emin - 25)); wide_kb flags a tile that needs skh
//   svs: fp16 V scales as stored, [D/32][32 keys]
//   S16: the 16-row kernel's layout, set by what its operand reads measure
//        on gfx950 (8-byte reads: 64 banks, 32 lanes a cycle).
//        K: its Q.K^T operand read takes rows 8(i / 4) + i % 4 (+ 4) for
//        lanes i = 0..15, so rows 16 apart meet in one read; with a 272-byte
//        stride they share banks.  Rows of 296 bytes, with row k's data
//        shifted by 8 (k % 4) bytes, put the 8-byte reads on distinct banks.
//        V^T: its P.V operand read takes 16 bytes (keys 8q .. 8q + 7) of
//        rows d .. d + 15; 40-key rows measure two cycles per read where
//        one suffices.  Unpadded 32-key rows with the 16-byte chunk q stored
//        at q ^ ((d >> 1) & 3) measure one.
template <int D, bool S16 = false>
struct TileLds {
    static constexpr int NB = D / 32;
    static constexpr int KQS = S16 ? D + 40 : D + 16;
    static constexpr int VTS = S16 ? kKeyTile : kKeyTile + 8;
    static constexpr int VBPAD = S16 ? 0 : 32;
    int8_t kq[kKeyTile * KQS];
    _Float16 vt[D * VTS + NB * VBPAD];
    // fp32 K scale per key (4-bit format); the key's unit 2^(emin - 25) (3-bit)
    float skf[kKeyTile];
    alignas(16) _Float16 skh[NB * kKeyTile];  // fp16 K scales [D/32][32 keys] (3-bit format)
    alignas(16) uint16_t skm[NB * kKeyTile];  // integer K scales M [D/32][32 keys] (3-bit)
    int wide_kb;                          // = the tile's first key when a key needs the fp32 epilogue
    // the tile's V scales: [D/32][32 keys] (3-bit), or per wave [NW][32 keys]
    // (4-bit per-token-head)
    alignas(16) uint16_t svs[D > 128 ? D : 128];
};

// One (key, block) item of the K side: 3 code words and the fp16 scale.
struct KItem {
    uint32_t w[3];
    uint16_t s;
};
// One element row d of the V side: the 3 words holding element d of the
// tile's 32 keys, and one of the tile's V scales (entry d: block d / 32,
// key d % 32), which the thread's own wave needs for its rows.
struct VItem {
    uint32_t w[3];
    uint16_t s;
};

// A wave-local handoff through LDS: the wave's own earlier LDS writes are
// visible to all of its lanes afterwards.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One K item (key kk, block b) of a tile into LDS: the int8 values c - 4 of
// its 32 codes (row stride KQS bytes; S16: the 16-row kernel's shifted rows),
// its fp16 scale, and with INT_SCALES the integer form of the key's scales
// (M of the block; the key's unit, from the item with b == 0).  kb: the
// tile's first key, written to *wide when the key has no exact integer scale
// form.  The NB items of a key sit on NB consecutive lanes, all present or all
// absent (min_over_blocks).
template <int NB, int KQS, bool INT_SCALES, bool S16>
__device__ __forceinline__ void unpack_k_item(const KItem &it, int kk, int b, int8_t *kq,
                                              _Float16 *skh, uint16_t *skm, float *skf, int *wide,
                                              int kb) {
    uint32_t o[8];
    unpack_bytes(it.w[0], it.w[1], it.w[2], o);
    if constexpr (S16) {
        // 8-byte pieces: the row shift keeps them 8-byte aligned only
        int8_t *row = kq + kk * KQS + 8 * (kk & 3) + 32 * b;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<u32x2 *>(row + 8 * c) =
                u32x2{codes_to_i8(o[2 * c]), codes_to_i8(o[2 * c + 1])};
    } else {
        const u32x4 lo = {codes_to_i8(o[0]), codes_to_i8(o[1]), codes_to_i8(o[2]), codes_to_i8(o[3])};
        const u32x4 hi = {codes_to_i8(o[4]), codes_to_i8(o[5]), codes_to_i8(o[6]), codes_to_i8(o[7])};
        *reinterpret_cast<u32x4 *>(kq + kk * KQS + 32 * b) = lo;
        *reinterpret_cast<u32x4 *>(kq + kk * KQS + 32 * b + 16) = hi;
    }
    skh[b * kKeyTile + kk] = __builtin_bit_cast(_Float16, it.s);
    if constexpr (INT_SCALES) {
        const ScaleInt si = scale_int(it.s);
        const uint32_t emin = min_over_blocks<NB>(si.e);
        const uint32_t shift = si.e - emin;      // 0 .. 30 (zero scales: M = 0)
        skm[b * kKeyTile + kk] = (uint16_t)(shift <= kScaleMaxShift ? si.m << shift : 0u);
        if (b == 0) skf[kk] = scale_unit(emin);
        if (si.special || (si.m != 0u && shift > kScaleMaxShift)) *wide = kb;
    }
}

// Element row d of a tile's V side into LDS as fp16 V^ = s * (c - 4), keys in
// order (row stride VTS halves, plus VBPAD per 32-row block; S16: 16-byte
// chunks swizzled by row).  svs: the tile's V scales [D/32][32 keys], written
// by the same wave and made visible by a wave-local sync.
template <int VTS, int VBPAD, bool S16>
__device__ __forceinline__ void unpack_v_row(const VItem &it, int d, _Float16 *vt,
                                             const uint16_t *svs) {
    uint32_t o[8];
    unpack_bytes(it.w[0], it.w[1], it.w[2], o);   // keys 4qq..4qq+3 in o[qq]
    const uint32_t *sv32 = reinterpret_cast<const uint32_t *>(svs + (d & ~31));
    uint32_t row[16];
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) {
        // Byte-select table lookup: code c -> high byte of the binary16
        // value c - 4 (whose low byte is zero).
        const uint32_t tt = __builtin_amdgcn_perm(kC4Hi, kC4Lo, o[qq]);
        const uint32_t p01 = __builtin_amdgcn_perm(tt, tt, 0x010C000Cu);
        const uint32_t p23 = __builtin_amdgcn_perm(tt, tt, 0x030C020Cu);
        const f16x2 v01 = __builtin_bit_cast(f16x2, p01) * __builtin_bit_cast(f16x2, sv32[2 * qq]);
        const f16x2 v23 = __builtin_bit_cast(f16x2, p23) * __builtin_bit_cast(f16x2, sv32[2 * qq + 1]);
        row[2 * qq] = __builtin_bit_cast(uint32_t, v01);
        row[2 * qq + 1] = __builtin_bit_cast(uint32_t, v23);
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(vt + d * VTS + (d / 32) * VBPAD);
    const int sw = S16 ? (d >> 1) & 3 : 0;      // chunk swizzle of the S16 layout
#pragma unroll
    for (int j = 0; j < 4; ++j)
        dst[j ^ sw] = u32x4{row[4 * j], row[4 * j + 1], row[4 * j + 2], row[4 * j + 3]};
}

// INT_SCALES: also stage the K scales in integer form (the 32-row kernel's
// epilogue); the 16-row kernel, whose unpack sits between two barriers on
// its critical path, uses the fp16 scales only.
template <int D, int NT, bool INT_SCALES, bool S16 = false>
struct TileIo {
    static constexpr int NB = D / 32;
    static constexpr int KI = kKeyTile * NB;           // K items per tile
    static constexpr int VI = D;                        // V rows per tile (= V scales)
    static constexpr int KPT = (KI + NT - 1) / NT;
    static constexpr int VPT = (VI + NT - 1) / NT;
    KItem k[KPT];
    VItem v[VPT];

    // Loads go through buffer descriptors based at the tile and sized to the
    // keys below k1 (zero size for a tile at or past k1, based at k0), so
    // entries past the range read as zero and every lane issues the same
    // loads: the waits for one register set never wait for another.  The V
    // scales past the range are zeroed by store().
    __device__ __forceinline__ void load(const AttnArgs &a, int head, int kb, int k0, int k1,
                                         int tid) {
        const bool valid = kb < k1;
        const int kt = valid ? kb : k0;
        const int nk = valid ? min(kKeyTile, k1 - kb) : 0;
        const size_t head_base = (size_t)head * a.cap;
        const size_t grp = (size_t)head * a.ngroups + (size_t)(kt / kKeyTile);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.kc + (head_base + kt) * NB * 3), (short)0, nk * NB * 12, kBufWord3);
        const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.ks + (head_base + kt) * NB), (short)0, nk * NB * 2, kBufWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.vc + grp * D * 3), (short)0, valid ? D * 12 : 0, kBufWord3);
        const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.vs + grp * D), (short)0, valid ? D * 2 : 0, kBufWord3);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int item = tid + i * NT;      // (key item / NB, block item % NB)
            const u32x3 w = __builtin_amdgcn_raw_buffer_load_b96(rk, item * 12, 0, 0);
            k[i].w[0] = w[0];
            k[i].w[1] = w[1];
            k[i].w[2] = w[2];
            k[i].s = __builtin_amdgcn_raw_buffer_load_b16(rks, item * 2, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int d = tid + i * NT;
            const u32x3 w = __builtin_amdgcn_raw_buffer_load_b96(rv, d * 12, 0, 0);
            v[i].w[0] = w[0];
            v[i].w[1] = w[1];
            v[i].w[2] = w[2];
            v[i].s = __builtin_amdgcn_raw_buffer_load_b16(rvs, d * 2, 0, 0);
        }
    }

    // nk: keys of the tile below k1 (V scales of later keys become 0); kb:
    // the tile's first key, written to t.wide_kb when a key of the tile has
    // no exact integer scale form (the NB items of a key sit on NB
    // consecutive lanes, all present or all absent)
    __device__ __forceinline__ void store(TileLds<D, S16> &t, int tid, int nk, int kb) const {
        using L = TileLds<D, S16>;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int item = tid + i * NT;
            if (item < KI)
                unpack_k_item<NB, L::KQS, INT_SCALES, S16>(k[i], item / NB, item % NB, t.kq, t.skh,
                                                           t.skm, t.skf, &t.wide_kb, kb);
        }
        // V scales: every wave stages the entries its own rows need; keys
        // past the range get scale 0, so their V^ is exactly 0.
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int d = tid + i * NT;
            if (d < VI) t.svs[d] = (d & 31) < nk ? v[i].s : (uint16_t)0;
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int d = tid + i * NT;
            if (d < VI) unpack_v_row<L::VTS, L::VBPAD, S16>(v[i], d, t.vt, t.svs);
        }
    }
};

// The 16-row kernel's tile I/O (256 threads, 3-bit format): thread tid
// holds K item tid and, with V, element rows of the V side: row tid, or
// (VWAVE) rows lane + 64i, i < D / 64, of the one wave that unpacks all of
// them (the kernel gives them to its fourth wave when that wave has no query
// rows, so the wave that would idle through the math takes the V unpack and
// the three computing waves only the K items).
template <int D, bool VWAVE>
struct Split16Io {
    static constexpr int NB = D / 32;
    static constexpr int KI = kKeyTile * NB;           // K items per tile (at most 256)
    static constexpr int NV = VWAVE ? D / 64 : 1;
    static_assert(KI <= 256 && D <= 256 && D % 64 == 0, "one K item per thread");
    using L = TileLds<D, true>;
    KItem k;
    VItem v[NV];

    __device__ __forceinline__ static int vrow(int tid, int i) {
        return VWAVE ? (tid & 63) + 64 * i : tid;
    }

    // Buffer-descriptor loads as in TileIo: zeros past k1 (and for rows
    // d >= D, which are not stored), nothing for a tile at or past k1.
    __device__ __forceinline__ void load(const AttnArgs &a, int head, int kb, int k0, int k1,
                                         int tid, bool with_v) {
        const bool valid = kb < k1;
        const int kt = valid ? kb : k0;
        const int nk = valid ? min(kKeyTile, k1 - kb) : 0;
        const size_t head_base = (size_t)head * a.cap;
        const size_t grp = (size_t)head * a.ngroups + (size_t)(kt / kKeyTile);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.kc + (head_base + kt) * NB * 3), (short)0, nk * NB * 12, kBufWord3);
        const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.ks + (head_base + kt) * NB), (short)0, nk * NB * 2, kBufWord3);
        const u32x3 w = __builtin_amdgcn_raw_buffer_load_b96(rk, tid * 12, 0, 0);
        k.w[0] = w[0];
        k.w[1] = w[1];
        k.w[2] = w[2];
        k.s = __builtin_amdgcn_raw_buffer_load_b16(rks, tid * 2, 0, 0);
        if (!with_v) return;
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.vc + grp * D * 3), (short)0, valid ? D * 12 : 0, kBufWord3);
        const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.vs + grp * D), (short)0, valid ? D * 2 : 0, kBufWord3);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int d = vrow(tid, i);
            const u32x3 x = __builtin_amdgcn_raw_buffer_load_b96(rv, d * 12, 0, 0);
            v[i].w[0] = x[0];
            v[i].w[1] = x[1];
            v[i].w[2] = x[2];
            v[i].s = __builtin_amdgcn_raw_buffer_load_b16(rvs, d * 2, 0, 0);
        }
    }

    // Tile into one LDS buffer: K int8 rows kq, fp16 K scales skh, V^ rows
    // vt; svs stages the V scales.  nk: keys of the tile below k1 (V scales
    // of later keys become 0, so their V^ is exactly 0).  The V scales a
    // wave's rows read are the ones that wave wrote (one row per thread:
    // entries 64w .. 64w + 63, blocks 2w and 2w + 1; VWAVE: all of them), so
    // a wave-local sync orders them.
    __device__ __forceinline__ void store(int8_t *kq, _Float16 *skh, _Float16 *vt, uint16_t *svs,
                                          int tid, int nk, bool with_v) const {
        if (tid < KI)
            unpack_k_item<NB, L::KQS, false, true>(k, tid / NB, tid % NB, kq, skh, nullptr, nullptr,
                                                   nullptr, 0);
        if (!with_v || vrow(tid, 0) >= D) return;       // (wave-uniform)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int d = vrow(tid, i);
            svs[d] = (d & 31) < nk ? v[i].s : (uint16_t)0;
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < NV; ++i)
            unpack_v_row<L::VTS, L::VBPAD, true>(v[i], vrow(tid, i), vt, svs);
    }
};

// ---- the 4-bit per-token-head format: 8 codes per word (element 8w + i in
// bits 4i), one fp16 scale per (token, KV head) for K and for V.
struct KItem4 {
    uint32_t w[4];      // elements 32b .. 32b+31 of one key
    uint16_t s;         // the key's scale (items with b == 0), else 0
};
struct VItem4 {
    uint32_t w[4];      // element d of the tile's 32 keys
};

// K codes become int8 (c - 8) * 16 = (c ^ 8) << 4, with the even elements
// of each 8-element group first: bytes e0 e2 e4 e6 | e1 e3 e5 e7.  The Q
// operand uses the same order, so the int32 sums are those of the natural
// order times 16 (exact; the 1/16 goes into the key's scale).
template <int D, int NT>
struct TileIo4 {
    static constexpr int NB = D / 32;
    static constexpr int KI = kKeyTile * NB;
    static constexpr int VI = D;
    static constexpr int KPT = (KI + NT - 1) / NT;
    static constexpr int VPT = (VI + NT - 1) / NT;
    KItem4 k[KPT];
    VItem4 v[VPT];
    uint16_t vs;        // V scale of key (lane % 32) of the tile (lanes 0..31 of each wave use it)

    // Buffer-descriptor loads as in TileIo: zeros past k1, the same loads
    // on every lane.
    __device__ __forceinline__ void load(const AttnArgs &a, int head, int kb, int k0, int k1,
                                         int tid) {
        const bool valid = kb < k1;
        const int kt = valid ? kb : k0;
        const int nk = valid ? min(kKeyTile, k1 - kb) : 0;
        const size_t head_base = (size_t)head * a.cap;
        const size_t grp = (size_t)head * a.ngroups + (size_t)(kt / kKeyTile);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.kc + (head_base + kt) * (D / 8)), (short)0, nk * (D / 2), kBufWord3);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.ks + head_base + kt), (short)0, nk * 2, kBufWord3);
        const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.vs + head_base + kt), (short)0, nk * 2, kBufWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.vc + grp * D * 4), (short)0, valid ? D * 16 : 0, kBufWord3);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int item = tid + i * NT;
            const int kk = item / NB, b = item % NB;
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rk, (kk * (D / 8) + 4 * b) * 4, 0, 0);
            k[i].w[0] = w[0];
            k[i].w[1] = w[1];
            k[i].w[2] = w[2];
            k[i].w[3] = w[3];
            k[i].s = __builtin_amdgcn_raw_buffer_load_b16(rs, kk * 2, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int d = tid + i * NT;
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rv, d * 16, 0, 0);
            v[i].w[0] = w[0];
            v[i].w[1] = w[1];
            v[i].w[2] = w[2];
            v[i].w[3] = w[3];
        }
        // key (lane % 32)'s V scale; zero past the range
        vs = __builtin_amdgcn_raw_buffer_load_b16(rvs, (tid & 31) * 2, 0, 0);
    }

    __device__ __forceinline__ void store(TileLds<D> &t, int tid, int, int) const {
        using L = TileLds<D>;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int item = tid + i * NT;
            if (item < KI) {
                const int kk = item / NB, b = item % NB;
                uint32_t o[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    o[2 * j] = ((k[i].w[j] << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
                    o[2 * j + 1] = (k[i].w[j] & 0xF0F0F0F0u) ^ 0x80808080u;
                }
                *reinterpret_cast<u32x4 *>(t.kq + kk * L::KQS + 32 * b) = u32x4{o[0], o[1], o[2], o[3]};
                *reinterpret_cast<u32x4 *>(t.kq + kk * L::KQS + 32 * b + 16) = u32x4{o[4], o[5], o[6], o[7]};
                if (b == 0) t.skf[kk] = half_bits_to_float(k[i].s) * 0.0625f;
            }
        }
        // V scales: every wave stages the tile's 32 key scales for its rows.
        const int wave = tid >> 6, lane = tid & 63;
        if (lane < kKeyTile) t.svs[wave * kKeyTile + lane] = vs;
        wave_lds_sync();
        const uint32_t *sv32 = reinterpret_cast<const uint32_t *>(t.svs + wave * kKeyTile);
        const f16x2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int d = tid + i * NT;
            if (d < VI) {
                uint32_t row[16];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // keys 8j + 2m (low nibbles) and 8j + 2m + 1 (high nibbles)
                    const uint32_t lo = v[i].w[j] & 0x0F0F0F0Fu;
                    const uint32_t hi = (v[i].w[j] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        // binary16 bits 0x6400 | c = 1024 + c; minus 1032 is c - 8, exactly
                        const uint32_t sel = (uint32_t)m | 0x0C00u | ((uint32_t)(4 + m) << 16) | 0x0C000000u;
                        const uint32_t pr = __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;
                        const uint32_t sw = sv32[4 * j + m];
                        const f16x2 val = (__builtin_bit_cast(f16x2, pr) + off) *
                                          __builtin_bit_cast(f16x2, sw);
                        row[4 * j + m] = __builtin_bit_cast(uint32_t, val);
                    }
                }
                u32x4 *dst = reinterpret_cast<u32x4 *>(t.vt + d * L::VTS + (d / 32) * L::VBPAD);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    dst[j] = u32x4{row[4 * j], row[4 * j + 1], row[4 * j + 2], row[4 * j + 3]};
            }
        }
    }
};

template <int D, int NT, int FMT>
using TileIoOf = typename std::conditional<FMT == 0, TileIo<D, NT, true>, TileIo4<D, NT>>::type;

// ---- unpacked tile images (the causal chunk with many row groups).
//
// Every row group of a KV head unpacks the same tiles; with hundreds of row
// groups per head (a prefill chunk) a pre-pass unpacks each tile once into
// the workspace, laid out exactly as the 32-row kernel's LDS tile, and the
// kernel copies images into LDS with direct buffer-to-LDS loads (no VGPRs,
// no VALU).  An image is a K part (int8 K rows, K scales in fp32 unit, fp16
// and integer form, the fp32-epilogue flag) and a V part (fp16 V^T), each
// padded to whole 1 KiB chunks: one 16-byte load per lane moves one chunk.
template <int D>
struct PreLayout {
    using L = TileLds<D>;
    static constexpr int NB = D / 32;
    static constexpr int KQ = 0;
    static constexpr int SKF = kKeyTile * L::KQS;
    static constexpr int SKH = SKF + 4 * kKeyTile;
    static constexpr int SKM = SKH + 2 * NB * kKeyTile;
    static constexpr int WIDE = SKM + 2 * NB * kKeyTile;
    static constexpr int KP = (WIDE + 16 + 1023) / 1024 * 1024;
    static constexpr int VT = KP;
    static constexpr int VP = (2 * (D * L::VTS + NB * L::VBPAD) + 1023) / 1024 * 1024;
    static constexpr int BYTES = KP + VP;
    static_assert(L::KQS % 16 == 0 && (2 * NB * kKeyTile) % 16 == 0, "16-byte pieces");
};

template <int N>
__device__ __forceinline__ void copy16(unsigned char *dst, const void *src, int tid, int nt) {
    static_assert(N % 16 == 0, "whole 16-byte pieces");
    const u32x4 *s = reinterpret_cast<const u32x4 *>(src);
    u32x4 *d = reinterpret_cast<u32x4 *>(dst);
    for (int i = tid; i < N / 16; i += nt) d[i] = s[i];
}

// Chunks wave, wave + NW, ... of NC 1 KiB chunks of an image from src into
// LDS at dst, one 16-byte direct buffer-to-LDS load per lane and chunk.
template <int NC, int NW>
__device__ __forceinline__ void image_to_lds(const unsigned char *src, unsigned char *dst, int wave,
                                             int lane) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char *>(src), (short)0, NC * 1024, kBufWord3);
    for (int c = wave; c < NC; c += NW)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void *)(dst + 1024 * c), 16, 16 * lane, 1024 * c, 0, 0);
}

// A lane's direct-to-LDS loads have written LDS once its vector-memory count is 0.
__device__ __forceinline__ void vmem_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One work-group per (tile, KV head): the 32-row kernel's unpack into LDS,
// then the tile's image out to img.  Keys at or past N read as zero.
template <int D, int FMT>
__global__ __launch_bounds__(256) void tile_image_kernel(const AttnArgs a, unsigned char *img) {
    using L = TileLds<D>;
    using PL = PreLayout<D>;
    __shared__ __attribute__((aligned(16))) L t;
    const int tid = threadIdx.x;
    const int tile = blockIdx.x, head = blockIdx.y;
    const int kb = tile * kKeyTile;
    TileIoOf<D, 256, FMT> io;
    io.load(a, head, kb, 0, a.N, tid);
    if (tid == 0) t.wide_kb = -1;
    __syncthreads();
    io.store(t, tid, min(kKeyTile, a.N - kb), kb);
    __syncthreads();
    unsigned char *dst = img + ((size_t)head * a.img_tiles + tile) * PL::BYTES;
    copy16<kKeyTile * L::KQS>(dst + PL::KQ, t.kq, tid, 256);
    copy16<4 * kKeyTile>(dst + PL::SKF, t.skf, tid, 256);
    copy16<2 * PL::NB * kKeyTile>(dst + PL::SKH, t.skh, tid, 256);
    copy16<2 * PL::NB * kKeyTile>(dst + PL::SKM, t.skm, tid, 256);
    copy16<2 * (D * L::VTS + PL::NB * L::VBPAD)>(dst + PL::VT, t.vt, tid, 256);
    if (tid == 0) *reinterpret_cast<int *>(dst + PL::WIDE) = t.wide_kb;
}

// PV16 selects the fp16-accumulated P.V variant (3-bit, verify only): each
// 32-key tile's P.V product still comes out of an fp32 MFMA, but it is
// rounded to fp16 and added into fp16 accumulators, and the running max
// follows every increase (so P <= 1 and the fp16 sums stay in range).
//
// NG groups of NW waves per work-group.  Each group owns one (kv head, row
// group of NW x 32 rows, context split) item, its own Q and tile in LDS, and
// walks its tiles in three phases: U (store the held tile to LDS, fetch the
// next), C (Q.K^T, block-scale epilogue, mask, online softmax) and P (P.V).
// Every phase ends at a work-group barrier.  With NG = 2 the second group
// runs one phase behind the first, and wave w of each group sits on SIMD
// w, so the two waves a SIMD holds are always in different phases: the
// VALU-heavy C of one beside the MFMA-only P or the lighter U of the other.
// (Two independent work-groups per CU would drift into the same phase,
// since each is held together by its own barriers.)  With NG = 1 the
// phases C and P fuse and a tile takes two barriers.
template <int D, int NW, int NG, bool CAUSAL, bool DEBUG, int FMT, bool PV16, bool PRE = false>
__global__ __launch_bounds__(NG * NW * 64) __attribute__((amdgpu_waves_per_eu(D == 256 && NG * NW > 1 && !DEBUG ? 2 : 1)))
void attn_split_kernel(const AttnArgs a) {
    constexpr int NB = D / 32;
    constexpr int KT = kKeyTile;
    constexpr int NT = NW * 64;
    using L = TileLds<D>;
    using PL = PreLayout<D>;
    // the tile: TileLds, or with PRE the image layout in two arrays, the K
    // part and the V part (distinct objects, so the compiler can tell the
    // image loads into one from the reads of the other and does not wait
    // for them)
    constexpr int TSZ = PRE ? 16 : ((int)sizeof(L) + 15) / 16 * 16;
    __shared__ __attribute__((aligned(16))) unsigned char tile_raw[NG * TSZ];
    __shared__ __attribute__((aligned(16))) unsigned char kimg[PRE ? PL::KP : 16];
    __shared__ __attribute__((aligned(16))) unsigned char vimg[PRE ? PL::VP : 16];
    // int8 Q of each wave's 32 rows, [NG][NW][32 rows][D + 16] bytes: read
    // back as the B operand of every Q.K^T MFMA, which keeps 32 VGPRs free
    // for double-buffering the MFMA results.
    __shared__ __attribute__((aligned(16))) int8_t qlds_g[NG * NW * kRowTile * L::KQS];

    const int grp = NG == 2 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x / NT) : 0;
    const int tid = threadIdx.x - grp * NT;
    unsigned char *const tbase = tile_raw + grp * TSZ;
    L &lds = *reinterpret_cast<L *>(tbase);
    int8_t *const t_kq = PRE ? reinterpret_cast<int8_t *>(kimg + PL::KQ) : lds.kq;
    _Float16 *const t_vt = PRE ? reinterpret_cast<_Float16 *>(vimg) : lds.vt;
    float *const t_skf = PRE ? reinterpret_cast<float *>(kimg + PL::SKF) : lds.skf;
    _Float16 *const t_skh = PRE ? reinterpret_cast<_Float16 *>(kimg + PL::SKH) : lds.skh;
    uint16_t *const t_skm = PRE ? reinterpret_cast<uint16_t *>(kimg + PL::SKM) : lds.skm;
    int *const t_wide = PRE ? reinterpret_cast<int *>(kimg + PL::WIDE) : &lds.wide_kb;
    int8_t *qlds = qlds_g + grp * NW * kRowTile * L::KQS;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int l32 = lane & 31;

    // ---- work item of each group.  Items ("virtual work-groups") map to
    // (kv head, split, row group) so that the row groups of one (head,
    // split) get ids 8 apart; a work-group takes items v and v + 8 (NG = 2),
    // so both sit on one XCD (work-group i runs on XCD i mod 8) and they
    // usually share a key range, hence a tile count.
    // An item with no visible key (a causal row group whose rows end before
    // its split) still writes its empty partial: zeros with lse = -inf.
    struct Item {
        int head, split, rg, k0, k1, n_tiles;
        bool valid;
    };
    auto item_of = [&](int g) {
        Item it{0, 0, 0, 0, 0, 0, false};
        const int v = NG == 2 ? 16 * ((int)blockIdx.x >> 3) + ((int)blockIdx.x & 7) + 8 * g
                              : (int)blockIdx.x;
        const int chunk = v / (8 * a.NRG);
        const int within = v - chunk * 8 * a.NRG;
        const int hs = chunk * 8 + (within & 7);
        if (hs >= a.Hkv * a.S) return it;
        it.valid = true;
        it.rg = within >> 3;
        it.head = hs / a.S;
        it.split = hs - it.head * a.S;
        it.k0 = it.split * a.split_len;
        int k1 = min(a.N, it.k0 + a.split_len);
        if (CAUSAL) {
            const int rho_last = min(a.R, (it.rg + 1) * NW * kRowTile) - 1;
            k1 = min(k1, a.L + rho_last / a.G + 1);
        }
        it.k1 = max(k1, it.k0);
        it.n_tiles = (it.k1 - it.k0 + KT - 1) / KT;
        return it;
    };
    const Item me = item_of(grp);
    const int n_other = NG == 2 ? item_of(1 - grp).n_tiles : 0;
    const int head = me.head, split = me.split, rg = me.rg, k0 = me.k0, k1 = me.k1;

    const int rho = (rg * NW + wave) * kRowTile + l32;
    const bool row_ok = me.valid && rho < a.R;
    const int t = row_ok ? rho / a.G : 0;
    const int g = row_ok ? rho - t * a.G : 0;
    const int flat = t * a.Hq + head * a.G + g;
    const bool wave_active = me.valid && (rg * NW + wave) * kRowTile < a.R;
    const int vis_from = min(k1, a.L);   // keys below this need no mask test

    // ---- prologue: per-row int8 quantization of Q.  Lane (l32, hl) holds
    // row l32 of the wave and elements 32b + 16hl + [0, 16) of every block b:
    // the B operand layout of the 32x32x32 int8 MFMA.
    float sq = 0.0f;
    int8_t *q_lane = qlds + (wave * kRowTile + l32) * L::KQS + 16 * hl;
    {
        i32x4 qreg[NB];
        QPart<NB, 4> qp;
        qp.load(a.q + (size_t)flat * D + 16 * hl);
        float amax = qp.absmax(row_ok);
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
        sq = amax / 127.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) qreg[b][j] = (int32_t)qp.codes(b, j, inv, row_ok);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            i32x4 w = qreg[b];
            if constexpr (FMT == 1) {
                // even elements of each 8-element group first, as the K codes
                const uint32_t q0 = (uint32_t)w[0], q1 = (uint32_t)w[1];
                const uint32_t q2 = (uint32_t)w[2], q3 = (uint32_t)w[3];
                w[0] = (int32_t)__builtin_amdgcn_perm(q1, q0, 0x06040200u);
                w[1] = (int32_t)__builtin_amdgcn_perm(q1, q0, 0x07050301u);
                w[2] = (int32_t)__builtin_amdgcn_perm(q3, q2, 0x06040200u);
                w[3] = (int32_t)__builtin_amdgcn_perm(q3, q2, 0x07050301u);
            }
            *reinterpret_cast<i32x4 *>(q_lane + 32 * b) = w;
        }
        if (DEBUG && split == 0 && row_ok) {
            if (a.dbg_q) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    *reinterpret_cast<i32x4 *>(a.dbg_q + (size_t)flat * D + 32 * b + 16 * hl) =
                        qreg[b];
            }
            if (a.dbg_qscale && hl == 0) a.dbg_qscale[flat] = sq;
        }
    }
    const float c_row = sq * a.scale_log2;

    // the row's ancestor mask (t < T for every lane: rows past the end use row 0)
    const uint64_t mrow = CAUSAL ? 0 : a.mask[t];

    // Key order inside a tile: MFMA row i of the Q.K^T product reads key
    // kperm(i), chosen so that output registers r = 0..7 of lane half hl hold
    // keys 8hl + r and registers 8..15 hold keys 16 + 8hl + (r - 8); those
    // are exactly the key runs the P.V MFMA wants from that lane.
    const int ai = l32 >> 3;
    const int krow = 16 * (ai >> 1) + 8 * ((l32 >> 2) & 1) + 4 * (ai & 1) + (l32 & 3);
    const int8_t *kq_lane = t_kq + krow * L::KQS + 16 * hl;
    const _Float16 *vt_lane = t_vt + l32 * L::VTS + 8 * hl;

    f32x16 oacc[NB];
#pragma unroll
    for (int dt = 0; dt < NB; ++dt) oacc[dt] = f32x16{};
    f16x2 oh[PV16 ? NB : 1][8];          // fp16 accumulators of the PV16 variant
#pragma unroll
    for (int dt = 0; dt < (PV16 ? NB : 1); ++dt)
#pragma unroll
        for (int j = 0; j < 8; ++j) oh[dt][j] = f16x2{};
    // Running max in base-2 logit units.  It only moves when a tile's max
    // exceeds it by more than 8 (so exp2 stays below 256, well inside fp16),
    // which makes rescaling the accumulators rare.  PV16: by any amount.
    constexpr float kLazy = PV16 ? 0.0f : 8.0f;
    float m_run = -INFINITY;
    float l_run = 0.0f;
    f16x8 pk[2];                          // the tile's P, from phase C to phase P

    // Tile data is prefetched into registers one tile ahead: phase U stores
    // the held tile to LDS and issues the next tile's loads, which then have
    // the rest of the tile's phases to arrive.
    TileIoOf<D, NT, FMT> io;
    if constexpr (!PRE) io.load(a, head, k0, k0, k1, tid);

    // ---- phase C: Q.K^T, mask, online softmax of tile kb (P left in pk)
    auto phase_c = [&](int kb) {
        f32x16 acc = f32x16{};
        const bool exact_int = FMT == 0 && __builtin_amdgcn_readfirstlane(*t_wide) != kb;
        if (exact_int) {
            // ---- Q.K^T: one int8 MFMA per 32-element block; the block
            // scales in integer form, so the key's logit is one int32
            // sum (one v_mad_i32_i16 per block), converted and scaled
            // once.  The MFMA of block b + 1 is issued before block b's
            // sums read its results.
            i32x16 iacc = i32x16{};
            i32x16 s_cur = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                *reinterpret_cast<const i32x4 *>(kq_lane),
                *reinterpret_cast<const i32x4 *>(q_lane), i32x16{}, 0, 0, 0);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                i32x16 s_next;
                if (b + 1 < NB)
                    s_next = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        *reinterpret_cast<const i32x4 *>(kq_lane + 32 * (b + 1)),
                        *reinterpret_cast<const i32x4 *>(q_lane + 32 * (b + 1)), i32x16{}, 0, 0, 0);
                // M of keys 8hl + [0, 8) and 16 + 8hl + [0, 8), two per word
                const u32x4 m0 = *reinterpret_cast<const u32x4 *>(t_skm + b * KT + 8 * hl);
                const u32x4 m1 = *reinterpret_cast<const u32x4 *>(t_skm + b * KT + 16 + 8 * hl);
                const int32_t ready = mfma_ready(s_cur[0]);
#pragma unroll
                for (int r = 0; r < 8; r += 2) {
                    iacc[r] = mad_i16<0>(s_cur[r], m0[r >> 1], iacc[r], ready);
                    iacc[r + 1] = mad_i16<1>(s_cur[r + 1], m0[r >> 1], iacc[r + 1], ready);
                    iacc[8 + r] = mad_i16<0>(s_cur[8 + r], m1[r >> 1], iacc[8 + r], ready);
                    iacc[9 + r] = mad_i16<1>(s_cur[9 + r], m1[r >> 1], iacc[9 + r], ready);
                }
                if (DEBUG && a.dbg_logits && row_ok) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb + (r < 8 ? 8 * hl + r : 16 + 8 * hl + (r - 8));
                        if (key < k1)
                            a.dbg_logits[((size_t)flat * a.N + key) * NB + b] = s_cur[r];
                    }
                }
                if (b + 1 < NB) s_cur = s_next;
            }
            const f32x4 u0 = *reinterpret_cast<const f32x4 *>(t_skf + 8 * hl);
            const f32x4 u1 = *reinterpret_cast<const f32x4 *>(t_skf + 8 * hl + 4);
            const f32x4 u2 = *reinterpret_cast<const f32x4 *>(t_skf + 16 + 8 * hl);
            const f32x4 u3 = *reinterpret_cast<const f32x4 *>(t_skf + 16 + 8 * hl + 4);
            const float unit[16] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w,
                                    u2.x, u2.y, u2.z, u2.w, u3.x, u3.y, u3.z, u3.w};
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = unit[r] * (float)iacc[r];
        } else if constexpr (FMT == 0) {
            // ---- the per-block fp32 epilogue, for tiles with a key
            // whose scales have no exact integer form (rare: kept short,
            // without the MFMA pipelining, to spare registers)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const i32x16 s_cur = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                    *reinterpret_cast<const i32x4 *>(kq_lane + 32 * b),
                    *reinterpret_cast<const i32x4 *>(q_lane + 32 * b), i32x16{}, 0, 0, 0);
                // fp16 scales of keys 8hl + [0, 8) and 16 + 8hl + [0, 8); the FMA
                // widens them in the instruction (v_fma_mix_f32)
                const f16x8 h0 = *reinterpret_cast<const f16x8 *>(t_skh + b * KT + 8 * hl);
                const f16x8 h1 = *reinterpret_cast<const f16x8 *>(t_skh + b * KT + 16 + 8 * hl);
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    acc[r] = fmaf((float)h0[r], (float)s_cur[r], acc[r]);
                    acc[8 + r] = fmaf((float)h1[r], (float)s_cur[8 + r], acc[8 + r]);
                }
                if (DEBUG && a.dbg_logits && row_ok) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb + (r < 8 ? 8 * hl + r : 16 + 8 * hl + (r - 8));
                        if (key < k1)
                            a.dbg_logits[((size_t)flat * a.N + key) * NB + b] = s_cur[r];
                    }
                }
            }
        } else {
            // ---- 4-bit per-token-head: the int8 MFMAs of all blocks
            // accumulate one int32 sum per (row, key), scaled once.
            i32x16 s_acc = i32x16{};
#pragma unroll
            for (int b = 0; b < NB; ++b)
                s_acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                    *reinterpret_cast<const i32x4 *>(kq_lane + 32 * b),
                    *reinterpret_cast<const i32x4 *>(q_lane + 32 * b), s_acc, 0, 0, 0);
            const f32x4 s0 = *reinterpret_cast<const f32x4 *>(t_skf + 8 * hl);
            const f32x4 s1 = *reinterpret_cast<const f32x4 *>(t_skf + 8 * hl + 4);
            const f32x4 s2 = *reinterpret_cast<const f32x4 *>(t_skf + 16 + 8 * hl);
            const f32x4 s3 = *reinterpret_cast<const f32x4 *>(t_skf + 16 + 8 * hl + 4);
            const float skr[16] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w,
                                   s2.x, s2.y, s2.z, s2.w, s3.x, s3.y, s3.z, s3.w};
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = skr[r] * (float)s_acc[r];
            if (DEBUG && a.dbg_logits && row_ok) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + (r < 8 ? 8 * hl + r : 16 + 8 * hl + (r - 8));
                    if (key < k1) a.dbg_logits[(size_t)flat * a.N + key] = s_acc[r] >> 4;
                }
            }
        }

        // ---- mask, online softmax in base 2.  c_row >= 0, so the row max
        // of the scaled logits is c_row times the max of acc.
        const bool masked = kb + KT > vis_from;
        if (masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb + (r < 8 ? 8 * hl + r : 16 + 8 * hl + (r - 8));
                bool vis = key < k1;
                if (vis && key >= a.L) {
                    const int u = key - a.L;
                    vis = CAUSAL ? (u <= t) : (((mrow >> u) & 1ull) != 0ull);
                }
                if (!vis) acc[r] = -INFINITY;
            }
        }
        float amax = acc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) amax = fmaxf(amax, acc[r]);
        amax = max_halves(amax);
        // a row with c_row == 0 has all visible logits 0
        const float tmax = amax == -INFINITY ? -INFINITY : amax * c_row;
        const float m_new = tmax > m_run + kLazy ? tmax : m_run;
        if (__any(m_new != m_run)) {
            const float alpha = m_new != m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            l_run *= alpha;
            if constexpr (PV16) {
#pragma unroll
                for (int dt = 0; dt < NB; ++dt)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        oh[dt][j] = __builtin_convertvector(
                            __builtin_convertvector(oh[dt][j], f32x2) * alpha, f16x2);
            } else {
#pragma unroll
                for (int dt = 0; dt < NB; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            }
            m_run = m_new;
        }
        const float mm = m_run == -INFINITY ? 0.0f : m_run;
        float p[16];
        if (masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                p[r] = acc[r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fmaf(acc[r], c_row, -mm));
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(acc[r], c_row, -mm));
        }
        // P for the B operand of P.V (lane = row, 8 keys per k-step); the
        // row sum adds the same fp16 values the MFMA multiplies.
        float psum = 0.0f;
        const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const f16x2 h2 = __builtin_convertvector(f32x2{p[8 * ks + e], p[8 * ks + e + 1]}, f16x2);
                pk[ks][e] = h2.x;
                pk[ks][e + 1] = h2.y;
                psum = __builtin_amdgcn_fdot2(h2, ones, psum, false);
            }
        l_run += psum;
    };

    // ---- phase P: O += P.V over the tile (A operand = V^T rows)
    auto phase_p = [&]() {
        __builtin_amdgcn_s_setprio(1);
        if constexpr (PV16) {
            // the tile's 32 keys in one fp32 product, then one fp16
            // rounding and one fp16 add per accumulator
#pragma unroll
            for (int dt = 0; dt < NB; ++dt) {
                const _Float16 *vrow = vt_lane + (dt * 32) * L::VTS + dt * L::VBPAD;
                f32x16 tp = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    *reinterpret_cast<const f16x8 *>(vrow), pk[0], f32x16{}, 0, 0, 0);
                tp = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    *reinterpret_cast<const f16x8 *>(vrow + 16), pk[1], tp, 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    oh[dt][j] += __builtin_convertvector(f32x2{tp[2 * j], tp[2 * j + 1]}, f16x2);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int dt = 0; dt < NB; ++dt) {
                    const f16x8 vop = *reinterpret_cast<const f16x8 *>(
                        vt_lane + (dt * 32) * L::VTS + dt * L::VBPAD + 16 * ks);
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, pk[ks], oacc[dt], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- the tile loop: U, barrier, C, barrier (NG = 2 only), P, barrier.
    // A barrier pairs with whichever barrier the other waves reach next, so
    // group 1 takes one extra barrier before its first tile and runs one
    // phase behind group 0 from then on; at the end each group takes the
    // barriers the other group's remaining tiles still need, so every wave
    // takes NPH * max(n) + NG - 1 barriers after the first.
    if constexpr (PRE) {
        // ---- tiles from their images: the K part of tile i + 1 streams into
        // LDS during tile i's P.V, the V part during tile i + 1's Q.K^T; each
        // wave moves every NW-th 1 KiB chunk (one 16-byte load per lane).
        static_assert(NG == 1, "images feed one group per work-group");
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        auto copy_img = [&](int kb, bool kpart, bool vpart) {
            const unsigned char *src =
                a.img + ((size_t)head * a.img_tiles + (size_t)(kb / KT)) * PL::BYTES;
            if (kpart) image_to_lds<PL::KP / 1024, NW>(src, kimg, wv, lane);
            if (vpart) image_to_lds<PL::VP / 1024, NW>(src + PL::KP, vimg, wv, lane);
        };
        if (me.n_tiles > 0) copy_img(k0, true, true);
        vmem_wait();
        __syncthreads();
        for (int kb = k0; kb < k1; kb += KT) {
            const bool more = kb + KT < k1;
            if (wave_active) phase_c(kb);
            vmem_wait();
            __syncthreads();
            if (more) copy_img(kb + KT, true, false);
            if (wave_active) phase_p();
            vmem_wait();
            __syncthreads();
            if (more) copy_img(kb + KT, false, true);
        }
    } else {
        constexpr int NPH = NG == 2 ? 3 : 2;
        if constexpr (FMT == 0) {
            if (tid == 0) lds.wide_kb = -1;
        }
        __syncthreads();
        if (NG == 2 && grp == 1) __syncthreads();
        for (int kb = k0; kb < k1; kb += KT) {
            io.store(lds, tid, min(KT, k1 - kb), kb);
            io.load(a, head, kb + KT, k0, k1, tid);
            __syncthreads();
            if (wave_active) phase_c(kb);
            if constexpr (NG == 2) __syncthreads();
            if (wave_active) phase_p();
            __syncthreads();
        }
        const int rest = NPH * (max(me.n_tiles, n_other) - me.n_tiles) + (NG == 2 && grp == 0 ? 1 : 0);
        for (int i = 0; i < rest; ++i) __syncthreads();
    }

    // ---- epilogue
    if (!wave_active) return;
    if constexpr (PV16) {
#pragma unroll
        for (int dt = 0; dt < NB; ++dt)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                oacc[dt][2 * j] = (float)oh[dt][j].x;
                oacc[dt][2 * j + 1] = (float)oh[dt][j].y;
            }
    }
    const float l_tot = sum_halves(l_run);
    const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    const size_t rows_total = (size_t)a.T * a.Hq;
    const bool partial = a.part_o != nullptr;
    float *const out_base = partial ? a.part_o + (size_t)split * rows_total * D : a.out;
    if (row_ok && hl == 0) {
        if (partial)
            a.part_lse[(size_t)split * rows_total + flat] = lse;
        else if (a.out_lse)
            a.out_lse[flat] = lse;
    }
    // The output goes out through the wave's own Q slot in LDS (no longer
    // read), one 32-column tile at a time: the MFMA layout gives a lane 16
    // bytes of a row per store, while read back row-major, eight lanes write
    // a row's whole 128-byte segment in one store instruction.  (head_dim
    // 64, whose Q slot is too small, stores from the MFMA layout.)
    constexpr int SS = 36;                     // staging row stride in floats (144 bytes)
    if constexpr (SS * 4 <= L::KQS) {
        float *stage = reinterpret_cast<float *>(qlds_g + (grp * NW + wave) * kRowTile * L::KQS);
        const int rr = lane >> 3, cq = lane & 7;    // read-back: rows rr + 8j, columns 4cq..4cq+3
        float *dst_row[4];
        bool ok_row[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rho_j = (rg * NW + wave) * kRowTile + rr + 8 * j;
            ok_row[j] = rho_j < a.R;
            const int t_j = ok_row[j] ? rho_j / a.G : 0;
            const int g_j = ok_row[j] ? rho_j - t_j * a.G : 0;
            dst_row[j] = out_base + (size_t)(t_j * a.Hq + head * a.G + g_j) * D + 4 * cq;
        }
#pragma unroll
        for (int dt = 0; dt < NB; ++dt) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 v = {oacc[dt][4 * r4 + 0] * inv_l, oacc[dt][4 * r4 + 1] * inv_l,
                                 oacc[dt][4 * r4 + 2] * inv_l, oacc[dt][4 * r4 + 3] * inv_l};
                *reinterpret_cast<f32x4 *>(stage + l32 * SS + 8 * r4 + 4 * hl) = v;
            }
            wave_lds_sync();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(stage + (rr + 8 * j) * SS + 4 * cq);
                if (ok_row[j]) *reinterpret_cast<f32x4 *>(dst_row[j] + dt * 32) = v;
            }
            wave_lds_sync();
        }
    } else {
        if (!row_ok) return;
        float *dst = out_base + (size_t)flat * D;
#pragma unroll
        for (int dt = 0; dt < NB; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = dt * 32 + 8 * r4 + 4 * hl;
                const f32x4 v = {oacc[dt][4 * r4 + 0] * inv_l, oacc[dt][4 * r4 + 1] * inv_l,
                                 oacc[dt][4 * r4 + 2] * inv_l, oacc[dt][4 * r4 + 3] * inv_l};
                *reinterpret_cast<f32x4 *>(dst + d0) = v;
            }
    }
}

// ------------------------------------------ attention, 32-row tiles, wave-specialized
//
// The 32-row tile kernel's work for the 3-bit format at head_dim 256, split by
// role over three waves per row tile (four row tiles, 128 rows, per work-group of
// twelve waves):
//   score waves 0-3 (row tile w): Q in registers, Q.K^T with the integer
//     block-scale epilogue, the mask and the online softmax; they hand P (fp16,
//     in the P.V operand layout) and the step's row rescale to the output waves
//     through LDS;
//   output waves 4-11 (row tile (w - 4) mod 4, half (w - 4) / 4 of D): P.V into
//     32 rows x D/2 fp32 accumulators, and the unpack -- waves 4-7 the K items of
//     the next tile, waves 8-11 the V rows of the current one.
// K, V and P are double-buffered in LDS, so one step (Q.K^T of tile j, P.V of
// tile j - 1, the unpack of K of tile j + 1 and of V of tile j) ends at one
// barrier.  The score waves' chain is the step's critical path; the output
// waves' MFMAs and unpack run beside it (wave w sits on SIMD w mod 4, so a SIMD
// holds one row tile's three waves).  No wave holds both Q and accumulators, or
// more than 32 x D/2 accumulators, so three waves fit per SIMD.  Raw code words
// are fetched three tiles ahead into registers.
template <int D>
struct WsLds {
    using L = TileLds<D>;
    static constexpr int NB = D / 32;
    static constexpr int NRT = 4;        // row tiles per work-group
    struct KBuf {
        int8_t kq[kKeyTile * L::KQS];
        float skf[kKeyTile];
        alignas(16) _Float16 skh[NB * kKeyTile];
        alignas(16) uint16_t skm[NB * kKeyTile];
        int wide_kb;
    };
    struct VBuf {
        _Float16 vt[D * L::VTS + NB * L::VBPAD];
        alignas(16) uint16_t svs[D];
    };
    struct PBuf {
        f16x8 p[2][64];          // [k-step][lane]: the score wave's P.V operand registers
        float alpha[kRowTile];   // the step's row rescale (when rescale is set)
        int rescale;
    };
    alignas(16) KBuf k[2];
    alignas(16) VBuf v[2];
    alignas(16) PBuf p[2][NRT];  // [buffer][row tile]
};

template <int D, bool CAUSAL, bool DEBUG>
__global__ __launch_bounds__(kWsThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void attn_ws_kernel(const AttnArgs a) {
    constexpr int NB = D / 32;
    constexpr int KT = kKeyTile;
    using L = TileLds<D>;
    using W = WsLds<D>;
    constexpr int NRT = W::NRT;
    constexpr int NH = NB / 2;               // 32-column d-tiles of an output wave
    __shared__ __attribute__((aligned(16))) W sh;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    const bool score = wave < NRT;
    const int rt = score ? wave : (wave - NRT) % NRT;
    const int dh = score ? 0 : (wave - NRT) / NRT;

    // ---- work item w = (head * S + split) * NRG + row group.  Work-group i
    // runs on XCD i mod 8; XCD x takes the run of items [x Q, x Q + Q), Q =
    // ceil(items / 8), so the row groups of one (head, split) share an XCD's
    // L2 (except where a run ends) and no XCD holds more than Q of them.
    const int n_items = a.Hkv * a.S * a.NRG;
    const int per_xcd = (n_items + 7) / 8;
    const int w_item = ((int)blockIdx.x & 7) * per_xcd + ((int)blockIdx.x >> 3);
    if (w_item >= n_items) return;
    const int hs = w_item / a.NRG;
    const int rg = w_item - hs * a.NRG;
    const int head = hs / a.S;
    const int split = hs - head * a.S;
    const int k0 = split * a.split_len;
    int k1 = min(a.N, k0 + a.split_len);
    if (CAUSAL) {
        const int rho_last = min(a.R, (rg + 1) * NRT * kRowTile) - 1;
        k1 = min(k1, a.L + rho_last / a.G + 1);
    }
    k1 = max(k1, k0);
    const int n_tiles = (k1 - k0 + KT - 1) / KT;

    const int rho = (rg * NRT + rt) * kRowTile + l32;
    const bool row_ok = rho < a.R;
    const int t = row_ok ? rho / a.G : 0;
    const int g = row_ok ? rho - t * a.G : 0;
    const int flat = t * a.Hq + head * a.G + g;
    const bool tile_active = (rg * NRT + rt) * kRowTile < a.R;
    const size_t rows_total = (size_t)a.T * a.Hq;
    const bool partial = a.part_o != nullptr;

    if (score) {
        __builtin_amdgcn_s_setprio(1);
        // ---- Q row l32 of the row tile to int8 with one fp32 scale; lane
        // (l32, hl) holds elements 32b + 16hl + [0, 16) of every block b (the B
        // operand of the 32x32x32 int8 MFMA)
        i32x4 qreg[NB];
        float sq = 0.0f;
        {
            QPart<NB, 4> qp;
            qp.load(a.q + (size_t)flat * D + 16 * hl);
            float amax = qp.absmax(row_ok);
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
            sq = amax / 127.0f;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) qreg[b][j] = (int32_t)qp.codes(b, j, inv, row_ok);
            if (DEBUG && split == 0 && row_ok) {
                if (a.dbg_q) {
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        *reinterpret_cast<i32x4 *>(a.dbg_q + (size_t)flat * D + 32 * b + 16 * hl) = qreg[b];
                }
                if (a.dbg_qscale && hl == 0) a.dbg_qscale[flat] = sq;
            }
        }
        const float c_row = sq * a.scale_log2;
        // the row's ancestor mask (t < T for every lane: rows past the end use row 0)
        const uint64_t mrow = CAUSAL ? 0 : a.mask[t];
        const int vis_from = min(k1, a.L);
        // MFMA row i of Q.K^T reads key krow(i): output registers r = 0..7 of
        // lane half hl hold keys 8hl + r, registers 8..15 keys 16 + 8hl + r - 8,
        // the key runs of the P.V operand
        const int ai = l32 >> 3;
        const int krow = 16 * (ai >> 1) + 8 * ((l32 >> 2) & 1) + 4 * (ai & 1) + (l32 & 3);
        constexpr float kLazy = 8.0f;
        float m_run = -INFINITY;
        float l_run = 0.0f;

        if (tid == 0) {
            sh.k[0].wide_kb = -1;
            sh.k[1].wide_kb = -1;
        }
        __syncthreads();     // the flags are set before any unpack
        __syncthreads();     // K of the first tile is in LDS
        for (int j = 0; j <= n_tiles; ++j) {
            if (j < n_tiles && tile_active) {
                const int kb = k0 + j * KT;
                const typename W::KBuf &kt = sh.k[j & 1];
                typename W::PBuf &pb = sh.p[j & 1][rt];
                const int8_t *kq_lane = kt.kq + krow * L::KQS + 16 * hl;
                f32x16 acc = f32x16{};
                // the first operands go out with the read of the tile's flag
                // (LDS returns in order: the flag's wait leaves them in flight)
                const int wide_kb = kt.wide_kb;
                i32x4 kop[3];
                u32x4 mop[2][2];
                kop[0] = *reinterpret_cast<const i32x4 *>(kq_lane);
                kop[1] = *reinterpret_cast<const i32x4 *>(kq_lane + 32);
                mop[0][0] = *reinterpret_cast<const u32x4 *>(kt.skm + 8 * hl);
                mop[0][1] = *reinterpret_cast<const u32x4 *>(kt.skm + 16 + 8 * hl);
                if (__builtin_amdgcn_readfirstlane(wide_kb) != kb) {
                    // Q.K^T, one int8 MFMA per block; the block scales in
                    // integer form make the logit one exact int32 sum (one
                    // v_mad_i32_i16 per block), converted and scaled once.  The
                    // MFMA of block b + 1 is issued before block b's sums, and
                    // the LDS operands run ahead of their use (K two blocks, M
                    // one), so no read waits right before its MFMA or sums.
                    i32x16 iacc = i32x16{};
                    i32x16 s_cur = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[0], qreg[0], i32x16{}, 0, 0, 0);
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        if (b + 2 < NB) kop[(b + 2) % 3] = *reinterpret_cast<const i32x4 *>(kq_lane + 32 * (b + 2));
                        if (b + 1 < NB) {
                            mop[(b + 1) & 1][0] = *reinterpret_cast<const u32x4 *>(kt.skm + (b + 1) * KT + 8 * hl);
                            mop[(b + 1) & 1][1] = *reinterpret_cast<const u32x4 *>(kt.skm + (b + 1) * KT + 16 + 8 * hl);
                        }
                        i32x16 s_next;
                        if (b + 1 < NB)
                            s_next = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[(b + 1) % 3], qreg[b + 1], i32x16{}, 0, 0, 0);
                        // M of keys 8hl + [0, 8) and 16 + 8hl + [0, 8), two per word
                        const u32x4 m0 = mop[b & 1][0];
                        const u32x4 m1 = mop[b & 1][1];
                        const int32_t ready = mfma_ready(s_cur[0]);
#pragma unroll
                        for (int r = 0; r < 8; r += 2) {
                            iacc[r] = mad_i16<0>(s_cur[r], m0[r >> 1], iacc[r], ready);
                            iacc[r + 1] = mad_i16<1>(s_cur[r + 1], m0[r >> 1], iacc[r + 1], ready);
                            iacc[8 + r] = mad_i16<0>(s_cur[8 + r], m1[r >> 1], iacc[8 + r], ready);
                            iacc[9 + r] = mad_i16<1>(s_cur[9 + r], m1[r >> 1], iacc[9 + r], ready);
                        }
                        if (DEBUG && a.dbg_logits && row_ok) {
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int key = kb + (r < 8 ? 8 * hl + r : 16 + 8 * hl + (r - 8));
                                if (key < k1) a.dbg_logits[((size_t)flat * a.N + key) * NB + b] = s_cur[r];
                            }
                        }
                        if (b + 1 < NB) s_cur = s_next;
                    }
                    const f32x4 u0 = *reinterpret_cast<const f32x4 *>(kt.skf + 8 * hl);
                    const f32x4 u1 = *reinterpret_cast<const f32x4 *>(kt.skf + 8 * hl + 4);
                    const f32x4 u2 = *reinterpret_cast<const f32x4 *>(kt.skf + 16 + 8 * hl);
                    const f32x4 u3 = *reinterpret_cast<const f32x4 *>(kt.skf + 16 + 8 * hl + 4);
                    const float unit[16] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w,
                                            u2.x, u2.y, u2.z, u2.w, u3.x, u3.y, u3.z, u3.w};
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[r] = unit[r] * (float)iacc[r];
                } else {
                    // the per-block fp32 epilogue, for a tile with a key whose
                    // scales have no exact integer form
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        const i32x16 s_cur = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                            *reinterpret_cast<const i32x4 *>(kq_lane + 32 * b), qreg[b], i32x16{}, 0, 0, 0);
                        const f16x8 h0 = *reinterpret_cast<const f16x8 *>(kt.skh + b * KT + 8 * hl);
                        const f16x8 h1 = *reinterpret_cast<const f16x8 *>(kt.skh + b * KT + 16 + 8 * hl);
#pragma unroll
                        for (int r = 0; r < 8; ++r) {
                            acc[r] = fmaf((float)h0[r], (float)s_cur[r], acc[r]);
                            acc[8 + r] = fmaf((float)h1[r], (float)s_cur[8 + r], acc[8 + r]);
                        }
                        if (DEBUG && a.dbg_logits && row_ok) {
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int key = kb + (r < 8 ? 8 * hl + r : 16 + 8 * hl + (r - 8));
                                if (key < k1) a.dbg_logits[((size_t)flat * a.N + key) * NB + b] = s_cur[r];
                            }
                        }
                    }
                }

                // ---- mask, online softmax in base 2 (c_row >= 0: the row max of
                // the scaled logits is c_row times the max of acc)
                const bool masked = kb + KT > vis_from;
                if (masked) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb + (r < 8 ? 8 * hl + r : 16 + 8 * hl + (r - 8));
                        bool vis = key < k1;
                        if (vis && key >= a.L) {
                            const int u = key - a.L;
                            vis = CAUSAL ? (u <= t) : (((mrow >> u) & 1ull) != 0ull);
                        }
                        if (!vis) acc[r] = -INFINITY;
                    }
                }
                // the row max as a tree of three-way maxima (short dependency chain)
                float m3[6];
#pragma unroll
                for (int i = 0; i < 5; ++i) m3[i] = fmaxf(fmaxf(acc[3 * i], acc[3 * i + 1]), acc[3 * i + 2]);
                m3[5] = acc[15];
                float amax = fmaxf(fmaxf(fmaxf(m3[0], m3[1]), m3[2]), fmaxf(fmaxf(m3[3], m3[4]), m3[5]));
                amax = max_halves(amax);
                const float tmax = amax == -INFINITY ? -INFINITY : amax * c_row;
                const float m_new = tmax > m_run + kLazy ? tmax : m_run;
                // the running max moves (rarely): the output waves scale their
                // accumulators by alpha before adding this tile's P.V
                const bool moved = __any(m_new != m_run);
                if (moved) {
                    const float alpha = m_new != m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
                    l_run *= alpha;
                    m_run = m_new;
                    if (hl == 0) pb.alpha[l32] = alpha;
                }
                if (lane == 0) pb.rescale = moved ? 1 : 0;
                const float mm = m_run == -INFINITY ? 0.0f : m_run;
                float p[16];
                if (masked) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        p[r] = acc[r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fmaf(acc[r], c_row, -mm));
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(acc[r], c_row, -mm));
                }
                // P for the B operand of P.V (lane = row, 8 keys per k-step); the
                // row sum adds the same fp16 values the MFMA multiplies
                // (four independent pair sums, then a tree: a short chain)
                const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
                f16x8 pk[2];
                float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const f16x2 h2 = __builtin_convertvector(f32x2{p[8 * ks + e], p[8 * ks + e + 1]}, f16x2);
                        pk[ks][e] = h2.x;
                        pk[ks][e + 1] = h2.y;
                        const int c = (4 * ks + e / 2) & 3;
                        ps[c] = __builtin_amdgcn_fdot2(h2, ones, ps[c], false);
                    }
                l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
                pb.p[0][lane] = pk[0];
                pb.p[1][lane] = pk[1];
            }
            __syncthreads();
        }
        // ---- epilogue: 1 / (row sum) to the output waves, the lse out
        const float l_tot = sum_halves(l_run);
        if (tile_active && hl == 0) sh.p[0][rt].alpha[l32] = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        if (tile_active && row_ok && hl == 0) {
            const float lse = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
            if (partial)
                a.part_lse[(size_t)split * rows_total + flat] = lse;
            else if (a.out_lse)
                a.out_lse[flat] = lse;
        }
        __syncthreads();
        return;
    }

    // ---- output waves
    const int item = (tid - NRT * 64) & 255;     // K item (waves 4-7) or V row d (waves 8-11)
    const bool kthr = dh == 0;
    f32x16 oacc[NH];
#pragma unroll
    for (int dt = 0; dt < NH; ++dt) oacc[dt] = f32x16{};

    // Buffer-descriptor loads as in TileIo: entries past k1 read as zero, a
    // tile at or past k1 reads nothing (zero-size descriptors based at k0).
    auto load_k = [&](KItem &r, int kb) {
        const bool valid = kb < k1;
        const int kt = valid ? kb : k0;
        const int nk = valid ? min(KT, k1 - kb) : 0;
        const size_t head_base = (size_t)head * a.cap;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.kc + (head_base + kt) * NB * 3), (short)0, nk * NB * 12, kBufWord3);
        const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.ks + (head_base + kt) * NB), (short)0, nk * NB * 2, kBufWord3);
        const u32x3 w = __builtin_amdgcn_raw_buffer_load_b96(rk, item * 12, 0, 0);
        r.w[0] = w[0];
        r.w[1] = w[1];
        r.w[2] = w[2];
        r.s = __builtin_amdgcn_raw_buffer_load_b16(rks, item * 2, 0, 0);
    };
    auto load_v = [&](VItem &r, int kb) {
        const bool valid = kb < k1;
        const int kt = valid ? kb : k0;
        const size_t grp = (size_t)head * a.ngroups + (size_t)(kt / KT);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.vc + grp * D * 3), (short)0, valid ? D * 12 : 0, kBufWord3);
        const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.vs + grp * D), (short)0, valid ? D * 2 : 0, kBufWord3);
        const u32x3 w = __builtin_amdgcn_raw_buffer_load_b96(rv, item * 12, 0, 0);
        r.w[0] = w[0];
        r.w[1] = w[1];
        r.w[2] = w[2];
        r.s = __builtin_amdgcn_raw_buffer_load_b16(rvs, item * 2, 0, 0);
    };
    // V scales of keys past the range become 0, so their V^ is exactly 0
    auto store_v = [&](const VItem &r, typename W::VBuf &vb, int kb) {
        const int nk = min(KT, k1 - kb);
        vb.svs[item] = (item & 31) < nk ? r.s : (uint16_t)0;
        wave_lds_sync();
        unpack_v_row<L::VTS, L::VBPAD, false>(r, item, vb.vt, vb.svs);
    };
    auto store_k = [&](const KItem &r, typename W::KBuf &kbuf, int kb) {
        unpack_k_item<NB, L::KQS, true, false>(r, item / NB, item % NB, kbuf.kq, kbuf.skh, kbuf.skm,
                                               kbuf.skf, &kbuf.wide_kb, kb);
    };
    // P.V of a tile: this wave's d-tiles dh * NH + [0, NH)
    auto phase_p = [&](const typename W::VBuf &vb, const typename W::PBuf &pb) {
        if (__builtin_amdgcn_readfirstlane(pb.rescale)) {
            const float al = pb.alpha[l32];
#pragma unroll
            for (int dt = 0; dt < NH; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= al;
        }
        const f16x8 p0 = pb.p[0][lane];
        const f16x8 p1 = pb.p[1][lane];
        const _Float16 *vt_lane = vb.vt + l32 * L::VTS + 8 * hl;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int dt = 0; dt < NH; ++dt) {
                const int gd = dh * NH + dt;
                const f16x8 vop = *reinterpret_cast<const f16x8 *>(vt_lane + (gd * 32) * L::VTS +
                                                                   gd * L::VBPAD + 16 * ks);
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, ks ? p1 : p0, oacc[dt], 0, 0, 0);
            }
        }
    };

    // Step j: K of tile j + 1 (waves 4-7) or V of tile j (waves 8-11) into
    // LDS from one of three register sets, which is then refilled with the
    // tile three steps ahead (loads of tiles past the range read nothing), and
    // P.V of tile j - 1.  Each role runs its own loop over triples of steps,
    // so that the register sets stay put and every path into a step has that
    // step's set loaded first: a step waits only for its own set's loads.
    if (kthr) {
        KItem r0, r1, r2;
        load_k(r0, k0);
        load_k(r1, k0 + KT);
        load_k(r2, k0 + 2 * KT);
        __syncthreads();     // the flags are set
        if (n_tiles > 0) store_k(r0, sh.k[0], k0);
        load_k(r0, k0 + 3 * KT);
        __syncthreads();     // K of the first tile is in LDS
        auto step = [&](int j, KItem &r) {
            if (j + 1 < n_tiles) store_k(r, sh.k[(j + 1) & 1], k0 + (j + 1) * KT);
            load_k(r, k0 + (j + 4) * KT);
            if (j >= 1 && tile_active) phase_p(sh.v[(j - 1) & 1], sh.p[(j - 1) & 1][rt]);
            __syncthreads();
        };
        int j = 0;
        for (; j + 2 <= n_tiles; j += 3) {
            step(j, r1);
            step(j + 1, r2);
            step(j + 2, r0);
        }
        if (j <= n_tiles) step(j, r1);
        if (j + 1 <= n_tiles) step(j + 1, r2);
    } else {
        VItem r0, r1, r2;
        load_v(r0, k0);
        load_v(r1, k0 + KT);
        load_v(r2, k0 + 2 * KT);
        __syncthreads();
        __syncthreads();
        auto step = [&](int j, VItem &r) {
            if (j < n_tiles) store_v(r, sh.v[j & 1], k0 + j * KT);
            load_v(r, k0 + (j + 3) * KT);
            if (j >= 1 && tile_active) phase_p(sh.v[(j - 1) & 1], sh.p[(j - 1) & 1][rt]);
            __syncthreads();
        };
        int j = 0;
        for (; j + 2 <= n_tiles; j += 3) {
            step(j, r0);
            step(j + 1, r1);
            step(j + 2, r2);
        }
        if (j <= n_tiles) step(j, r0);
        if (j + 1 <= n_tiles) step(j + 1, r1);
    }
    __syncthreads();     // the score waves' 1 / (row sum) is in LDS
    if (!tile_active) return;
    const float inv_l = sh.p[0][rt].alpha[l32];
    float *const out_base = partial ? a.part_o + (size_t)split * rows_total * D : a.out;
    // The output goes out through LDS (the V buffers, free after the last
    // P.V), one 32-column tile at a time: read back row-major, eight lanes
    // write a row's whole 128-byte segment in one store instruction.
    constexpr int SS = 36;                       // staging row stride in floats
    static_assert(8 * kRowTile * SS * 4 <= (int)sizeof(sh.v), "staging fits the V buffers");
    float *stage = reinterpret_cast<float *>(&sh.v[0]) + (wave - NRT) * kRowTile * SS;
    const int rr = lane >> 3, cq = lane & 7;     // read-back: rows rr + 8j, columns 4cq..4cq+3
    float *dst_row[4];
    bool ok_row[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int rho_j = (rg * NRT + rt) * kRowTile + rr + 8 * j;
        ok_row[j] = rho_j < a.R;
        const int t_j = ok_row[j] ? rho_j / a.G : 0;
        const int g_j = ok_row[j] ? rho_j - t_j * a.G : 0;
        dst_row[j] = out_base + (size_t)(t_j * a.Hq + head * a.G + g_j) * D + 4 * cq;
    }
#pragma unroll
    for (int dt = 0; dt < NH; ++dt) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 v = {oacc[dt][4 * r4 + 0] * inv_l, oacc[dt][4 * r4 + 1] * inv_l,
                             oacc[dt][4 * r4 + 2] * inv_l, oacc[dt][4 * r4 + 3] * inv_l};
            *reinterpret_cast<f32x4 *>(stage + l32 * SS + 8 * r4 + 4 * hl) = v;
        }
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(stage + (rr + 8 * j) * SS + 4 * cq);
            if (ok_row[j]) *reinterpret_cast<f32x4 *>(dst_row[j] + (dh * NH + dt) * 32) = v;
        }
        wave_lds_sync();
    }
}

// ------------------------------------------ attention, 16-row tiles, shared tiles
//
// For 17..64 query rows per KV head (the 8-row tree: 48 rows): the split
// kernel's shared tile (one unpack per work-group into LDS: int8 K, fp16
// V^ = s * (c - 4), fp16 K scales) feeding four waves of 16 rows each, with
// 16x16 MFMAs: Q.K^T on v_mfma_i32_16x16x32_i8 (exact int32 per 32-element
// block), P.V on v_mfma_f32_16x16x32_f16.  A wave holds 16 rows x D fp32
// accumulators (64 VGPRs at D = 256, half the 32-row tile's), which with Q in
// registers and the tile in LDS leaves room for three waves per SIMD.
// 3-bit format (the 4-bit format's small shapes run the few-row kernel).
// PV16: the fp16-accumulated P.V variant, as in the split kernel.
typedef int32_t i32x4s __attribute__((ext_vector_type(4)));
typedef int64_t i64_t;

// The 16-row kernel's LDS: two tile buffers (the unpack of tile j + 1 runs
// beside the math of tile j, one barrier per tile) and the V scale staging;
// 52 KB at D = 256, so three work-groups share a CU.
template <int D>
struct S16Lds {
    using L = TileLds<D, true>;
    struct Buf {
        int8_t kq[kKeyTile * L::KQS];
        alignas(16) _Float16 vt[D * L::VTS];
        alignas(16) _Float16 skh[(D / 32) * kKeyTile];   // fp16 K scales [D/32][32 keys]
    };
    alignas(16) Buf b[2];
    alignas(16) uint16_t svs[D];
};

template <int D, bool CAUSAL, bool DEBUG, bool PV16>
__global__ __launch_bounds__(256) void attn_split16_kernel(const AttnArgs a) {
    constexpr int NB = D / 32;
    constexpr int NDT = D / 16;
    constexpr int KT = kKeyTile;
    constexpr int NW = 4;
    constexpr int NT = NW * 64;
    using L = TileLds<D, true>;
    using SL = S16Lds<D>;
    __shared__ __attribute__((aligned(16))) SL lds;

    // ---- work-group -> (kv head, split, group of 64 rows); the row groups of
    // one (head, split) get ids 8 apart so they share an XCD and its L2.
    const int id = blockIdx.x;
    const int chunk = id / (8 * a.NRG);
    const int within = id - chunk * 8 * a.NRG;
    const int rg = within >> 3;
    const int hs = chunk * 8 + (within & 7);
    if (hs >= a.Hkv * a.S) return;
    const int head = hs / a.S;
    const int split = hs - head * a.S;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i16 = lane & 15;          // row of this lane in the wave's 16 (MFMA column)
    const int qc = lane >> 4;           // 8-element chunk / 8-key group of this lane
    const int row0 = (rg * NW + wave) * 16;
    const bool wave_active = row0 < a.R;
    const bool row_ok = row0 + i16 < a.R;
    const int t = row_ok ? (row0 + i16) / a.G : 0;
    const int g = row_ok ? row0 + i16 - t * a.G : 0;
    const int flat = t * a.Hq + head * a.G + g;

    const int k0 = split * a.split_len;
    int k1 = min(a.N, k0 + a.split_len);
    if (CAUSAL) {
        const int rho_last = min(a.R, (rg + 1) * NW * 16) - 1;
        k1 = min(k1, a.L + rho_last / a.G + 1);
    }
    const int vis_from = min(k1, a.L);
    const int n_tiles = k1 > k0 ? (k1 - k0 + KT - 1) / KT : 0;

    // Step j stores tile j + 1 (fetched into registers during step j - 1)
    // into buffer (j + 1) & 1, fetches tile j + 2, and runs the math of tile
    // j from buffer j & 1; one barrier ends the step.  With at most 48 rows
    // in the work-group its fourth wave, which has no rows, unpacks all V
    // rows in a loop of its own (the same barriers), and the other waves only
    // the K items.
    const bool vw = (rg * NW + NW - 1) * 16 >= a.R;
    if (vw && wave == NW - 1) {
        Split16Io<D, true> vio;
        vio.load(a, head, k0, k0, k1, tid, true);
        if (n_tiles > 0)
            vio.store(lds.b[0].kq, lds.b[0].skh, lds.b[0].vt, lds.svs, tid, min(KT, k1 - k0), true);
        vio.load(a, head, k0 + KT, k0, k1, tid, true);
        __syncthreads();
        for (int j = 0; j < n_tiles; ++j) {
            if (j + 1 < n_tiles) {
                typename SL::Buf &nb = lds.b[(j + 1) & 1];
                const int kn = k0 + (j + 1) * KT;
                vio.store(nb.kq, nb.skh, nb.vt, lds.svs, tid, min(KT, k1 - kn), true);
            }
            vio.load(a, head, k0 + (j + 2) * KT, k0, k1, tid, true);
            __syncthreads();
        }
        return;
    }
    // ---- Q: lane (row i16, chunk qc) quantizes and holds elements
    // 32b + 8qc + [0, 8) of every block b (B operand of the 16x16x32 MFMA)
    i64_t qop[NB];
    float sq;
    {
        QPart<NB, 2> qp;
        qp.load(a.q + (size_t)flat * D + 8 * qc);
        float amax = qp.absmax(row_ok);
        amax = max_xor16(amax);
        amax = max_halves(amax);
        const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
        sq = amax / 127.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            qop[b] = (i64_t)((uint64_t)qp.codes(b, 0, inv, row_ok) | ((uint64_t)qp.codes(b, 1, inv, row_ok) << 32));
        if (DEBUG && split == 0 && row_ok) {
            if (a.dbg_q) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    *reinterpret_cast<i64_t *>(a.dbg_q + (size_t)flat * D + 32 * b + 8 * qc) = qop[b];
            }
            if (a.dbg_qscale && qc == 0) a.dbg_qscale[flat] = sq;
        }
    }
    const float c_row = sq * a.scale_log2;
    // the row's ancestor mask (t < T for every lane: rows past the end use row 0)
    const uint64_t mrow = CAUSAL ? 0 : a.mask[t];

    // A operand row m of key half kh reads key 8(m / 4) + 4kh + m % 4, so the
    // result registers of lane (i16, qc) hold keys 8qc + 4kh + [0, 4): its
    // eight logits are keys 8qc + [0, 8), the run the P.V operand wants.
    const int krow0 = 8 * (i16 >> 2) + (i16 & 3);
    // (row shift: rows krow0 and krow0 + 4 both start 8 (i16 % 4) bytes in)
    const int kq_off = krow0 * L::KQS + 8 * (i16 & 3) + 8 * qc;

    f32x4 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    f16x2 oh[PV16 ? NDT : 1][2];
#pragma unroll
    for (int dt = 0; dt < (PV16 ? NDT : 1); ++dt) oh[dt][0] = oh[dt][1] = f16x2{};
    // base-2 running max; moves by more than 8 only (PV16: by any amount)
    constexpr float kLazy = PV16 ? 0.0f : 8.0f;
    float m_run = -INFINITY;
    float l_run = 0.0f;

    Split16Io<D, false> io;
    io.load(a, head, k0, k0, k1, tid, !vw);
    if (n_tiles > 0)
        io.store(lds.b[0].kq, lds.b[0].skh, lds.b[0].vt, lds.svs, tid, min(KT, k1 - k0), !vw);
    io.load(a, head, k0 + KT, k0, k1, tid, !vw);
    __syncthreads();
    for (int j = 0; j < n_tiles; ++j) {
        const int kb = k0 + j * KT;
        if (j + 1 < n_tiles) {
            typename SL::Buf &nb = lds.b[(j + 1) & 1];
            io.store(nb.kq, nb.skh, nb.vt, lds.svs, tid, min(KT, k1 - (kb + KT)), !vw);
        }
        io.load(a, head, kb + 2 * KT, k0, k1, tid, !vw);
        const typename SL::Buf &cb = lds.b[j & 1];
        const int8_t *kq_lane = cb.kq + kq_off;

        if (wave_active) {
            float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            // ---- Q.K^T, one int8 MFMA per (block, key half), fp32 epilogue
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const f16x8 h = *reinterpret_cast<const f16x8 *>(cb.skh + b * KT + 8 * qc);
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    const i64_t kop = *reinterpret_cast<const i64_t *>(kq_lane + 4 * kh * L::KQS + 32 * b);
                    const i32x4s sres = __builtin_amdgcn_mfma_i32_16x16x32_i8(kop, qop[b], i32x4s{}, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[4 * kh + e] = fmaf((float)h[4 * kh + e], (float)sres[e], acc[4 * kh + e]);
                    if (DEBUG && a.dbg_logits && row_ok) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int key = kb + 8 * qc + 4 * kh + e;
                            if (key < k1) a.dbg_logits[((size_t)flat * a.N + key) * NB + b] = sres[e];
                        }
                    }
                }
            }

            // ---- mask, online softmax in base 2
            const bool masked = kb + KT > vis_from;
            if (masked) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int key = kb + 8 * qc + r;
                    bool vis = key < k1;
                    if (vis && key >= a.L) {
                        const int u = key - a.L;
                        vis = CAUSAL ? (u <= t) : (((mrow >> u) & 1ull) != 0ull);
                    }
                    if (!vis) acc[r] = -INFINITY;
                }
            }
            float amax = acc[0];
#pragma unroll
            for (int r = 1; r < 8; ++r) amax = fmaxf(amax, acc[r]);
            amax = max_xor16(amax);
            amax = max_halves(amax);
            const float tmax = amax == -INFINITY ? -INFINITY : amax * c_row;
            const float m_new = tmax > m_run + kLazy ? tmax : m_run;
            if (__any(m_new != m_run)) {
                const float alpha = m_new != m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
                l_run *= alpha;
                if constexpr (PV16) {
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            oh[dt][j] = __builtin_convertvector(
                                __builtin_convertvector(oh[dt][j], f32x2) * alpha, f16x2);
                } else {
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
                }
                m_run = m_new;
            }
            const float mm = m_run == -INFINITY ? 0.0f : m_run;
            f16x8 pk;
            float psum = 0.0f;
            const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
            // only a tile holding masked keys (the split's last) has -inf logits
            float pe[8];
            if (masked) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pe[e] = acc[e] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fmaf(acc[e], c_row, -mm));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(acc[e], c_row, -mm));
            }
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const f16x2 h2 = __builtin_convertvector(f32x2{pe[e], pe[e + 1]}, f16x2);
                pk[e] = h2.x;
                pk[e + 1] = h2.y;
                psum = __builtin_amdgcn_fdot2(h2, ones, psum, false);
            }
            l_run += psum;

            // ---- P.V: A operand = V^T rows d = 16dt + i16, keys 8qc + [0, 8)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int d = 16 * dt + i16;
                // (d >> 1) & 3 = (i16 >> 1) & 3: the layout's chunk swizzle
                const f16x8 vop = *reinterpret_cast<const f16x8 *>(cb.vt + d * L::VTS + 8 * (qc ^ ((i16 >> 1) & 3)));
                if constexpr (PV16) {
                    const f32x4 tp = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pk, f32x4{}, 0, 0, 0);
                    oh[dt][0] += __builtin_convertvector(f32x2{tp[0], tp[1]}, f16x2);
                    oh[dt][1] += __builtin_convertvector(f32x2{tp[2], tp[3]}, f16x2);
                } else {
                    oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pk, oacc[dt], 0, 0, 0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        __syncthreads();
    }

    // ---- epilogue: row sums over the four key groups of the row
    if (!wave_active) return;
    if constexpr (PV16) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            oacc[dt] = f32x4{(float)oh[dt][0].x, (float)oh[dt][0].y, (float)oh[dt][1].x,
                             (float)oh[dt][1].y};
    }
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot = sum_halves(l_tot);
    const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    if (!row_ok) return;
    const size_t rows_total = (size_t)a.T * a.Hq;
    const bool partial = a.part_o != nullptr;
    float *dst = (partial ? a.part_o + (size_t)split * rows_total * D : a.out) + (size_t)flat * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4 *>(dst + 16 * dt + 4 * qc) = oacc[dt] * inv_l;
    if (qc == 0) {
        if (partial)
            a.part_lse[(size_t)split * rows_total + flat] = lse;
        else if (a.out_lse)
            a.out_lse[flat] = lse;
    }
}

// ------------------------------------------------- attention, few query rows
//
// For at most 16 query rows per KV head (one token, or a few tree rows): the
// streaming of the cache bounds the call, so every wave works on its own
// 32-key tiles with no work-group barrier.  A lane quantizes and holds its
// rows' int8 Q in registers; the wave unpacks its tile into its own LDS
// region (int8 K chunks, V code chunks, scales) and runs 16x16 MFMAs:
// Q.K^T with v_mfma_i32_16x16x32_i8 (exact int32 per 32-element block) and
// P.V with v_mfma_f32_16x16x32_f16.  P.V takes the V codes' values c - 4
// (exact in fp16, built by table lookup) as one operand and P times the V
// scales of each 32-element block as the other, so sv * (c - 4) is never
// formed.  The four waves of a work-group stride over the split's tiles and
// merge their softmax states through LDS at the end.

typedef int32_t i32x4v __attribute__((ext_vector_type(4)));

constexpr int kDecWaves = 4;

template <int D>
struct DecWaveLds {
    static constexpr int NB = D / 32;
    static constexpr int NDT = D / 16;
    // int8 K, [block][chunk of 8 elements][32 keys + 4 pad][8 bytes]: the A
    // operand read of lane (key i, chunk q) lands on distinct banks.
    uint32_t kq[NB][4][36][2];
    // V codes (one byte per key, codes 0..7), [d-tile][chunk slot][d % 16][8
    // keys]; chunk q of d-tile dt sits in slot q ^ (dt & 3).
    uint32_t vc[NDT][4][16][2];
    float skf[NB][32];
    alignas(16) uint16_t svs[NB][32];
};

// PV16: the fp16-accumulated P.V variant (3-bit only), as in the split
// kernel.  FMT 1: the 4-bit per-token-head format: the K chunks become int8
// 16 (c - 8) in the split kernel's even/odd order (Q permuted alike), the
// eight block MFMAs of a key half chain into one int32 sum scaled once per
// key, V code words are expanded to fp16 c - 8 by the 0x6400 | c pattern,
// and P times the key's V scale serves all blocks.
template <int D, bool CAUSAL, bool DEBUG, bool PV16, int FMT>
__global__ __launch_bounds__(kDecWaves * 64) void attn_dec_kernel(const AttnArgs a) {
    constexpr int NB = D / 32;
    constexpr int NDT = D / 16;
    constexpr int KT = kKeyTile;
    using W = DecWaveLds<D>;
    static_assert(sizeof(W) >= 16 * D * sizeof(float) + 64 * sizeof(float),
                  "the merge stages a wave's 16 x D outputs in its tile region");
    __shared__ __attribute__((aligned(16))) W wl[kDecWaves];

    // ---- work-group -> (kv head, split, group of 16 rows).  The row groups
    // of one (head, split) get ids 8 apart, so they run on one XCD and read
    // the split's tiles through its L2.
    const int id = blockIdx.x;
    const int chunk = id / (8 * a.NRG);
    const int within = id - chunk * 8 * a.NRG;
    const int rg = within >> 3;
    const int hs = chunk * 8 + (within & 7);
    if (hs >= a.Hkv * a.S) return;
    const int head = hs / a.S;
    const int split = hs - head * a.S;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: tile bases stay scalar
    const int i16 = lane & 15;          // row of this lane in the group (MFMA row/column index)
    const int qc = lane >> 4;           // 8-element chunk / 4-key group of this lane
    W &my = wl[wave];
    const int row0 = rg * 16;           // first row (t * G + g order) of the group

    const bool row_ok = row0 + i16 < a.R;
    const int t = row_ok ? (row0 + i16) / a.G : 0;
    const int g = row_ok ? row0 + i16 - t * a.G : 0;
    const int flat = t * a.Hq + head * a.G + g;

    const int k0 = split * a.split_len;
    int k1 = min(a.N, k0 + a.split_len);
    if (CAUSAL) k1 = min(k1, a.L + (min(a.R, row0 + 16) - 1) / a.G + 1);
    const int vis_from = min(k1, a.L);

    // ---- Q: lane (row i16, chunk qc) holds elements 32b + 8qc + [0, 8) of
    // every block b, the B operand layout of the 16x16x32 int8 MFMA.
    i64_t qop[NB];
    float sq;
    {
        QPart<NB, 2> qp;
        qp.load(a.q + (size_t)flat * D + 8 * qc);
        float amax = qp.absmax(row_ok);
        amax = max_xor16(amax);
        amax = max_halves(amax);
        const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
        sq = amax / 127.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            qop[b] = (i64_t)((uint64_t)qp.codes(b, 0, inv, row_ok) | ((uint64_t)qp.codes(b, 1, inv, row_ok) << 32));
        if (DEBUG && split == 0 && wave == 0 && row_ok) {
            if (a.dbg_q) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    *reinterpret_cast<i64_t *>(a.dbg_q + (size_t)flat * D + 32 * b + 8 * qc) = qop[b];
            }
            if (a.dbg_qscale && qc == 0) a.dbg_qscale[flat] = sq;
        }
        if constexpr (FMT == 1) {
            // even elements of the 8-element chunk first, as the K codes
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint64_t w = (uint64_t)qop[b];
                const uint32_t q0 = (uint32_t)w, q1 = (uint32_t)(w >> 32);
                const uint32_t e = __builtin_amdgcn_perm(q1, q0, 0x06040200u);
                const uint32_t o = __builtin_amdgcn_perm(q1, q0, 0x07050301u);
                qop[b] = (i64_t)((uint64_t)e | ((uint64_t)o << 32));
            }
        }
    }
    const float c_row = sq * a.scale_log2;
    // the row's ancestor mask (t < T for every lane: rows past the end use row 0)
    const uint64_t mrow = CAUSAL ? 0 : a.mask[t];

    f32x4 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    f16x2 oh[PV16 ? NDT : 1][2];
#pragma unroll
    for (int dt = 0; dt < (PV16 ? NDT : 1); ++dt) oh[dt][0] = oh[dt][1] = f16x2{};
    constexpr float kLazy = PV16 ? 0.0f : 8.0f;
    float m_run = -INFINITY;
    float l_run = 0.0f;
    float lv_run = 0.0f;        // 4-bit: running sum of P times the V scale (this lane's keys)

    // ---- per-wave register prefetch of one tile: 4 K items, 4 V rows and
    // 4 V scales per lane
    constexpr int PER = (KT * NB) / 64;     // = D / 64
    // 3-bit: three code words per K item and V row, a K and a V scale per
    // item.  4-bit: four words each; one K and one V scale per key (lane % 32).
    constexpr int KW = FMT == 1 ? 4 : 3;
    struct TileRegs {
        uint32_t k[PER][KW], v[PER][KW];
        uint16_t ks[PER], vs[PER];
    };
    // Loads go through buffer descriptors whose base is the tile and whose
    // size ends at the split's last key, so entries past it read as zero
    // (code 0 with scale 0 for K) without a per-lane branch.
    const size_t head_k = (size_t)head * a.cap;
    // A tile at or past k1 gets descriptors of size 0 (based at the split's
    // first tile): its loads read nothing and return zeros.  Issuing them
    // anyway keeps the number of loads in flight the same on every path, so
    // the waits for one register set never wait for the other.
    auto load_tile = [&](TileRegs &r, int kb) {
        const bool valid = kb < k1;
        const int kt = valid ? kb : k0;
        const int nk = valid ? min(KT, k1 - kb) : 0;
        const size_t grp = (size_t)head * a.ngroups + (size_t)(kt / KT);
        if constexpr (FMT == 1) {
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint32_t *>(a.kc + (head_k + kt) * (D / 8)), (short)0, nk * (D / 2), kBufWord3);
            const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t *>(a.ks + head_k + kt), (short)0, nk * 2, kBufWord3);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint32_t *>(a.vc + grp * D * 4), (short)0, valid ? D * 16 : 0, kBufWord3);
            const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t *>(a.vs + head_k + kt), (short)0, nk * 2, kBufWord3);
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                // K item = (key item % 32, block item / 32): 16 bytes of the
                // key's codes; V row d = item of the key-transposed group
                const int item = lane + 64 * i;
                const int key = item & 31, b = item >> 5;
                const u32x4 kw = __builtin_amdgcn_raw_buffer_load_b128(rk, (key * (D / 8) + 4 * b) * 4, 0, 0);
                const u32x4 vw = __builtin_amdgcn_raw_buffer_load_b128(rv, item * 16, 0, 0);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    r.k[i][w] = kw[w];
                    r.v[i][w] = vw[w];
                }
            }
            // key lane % 32's scales (the same key for every item of a lane)
            r.ks[0] = __builtin_amdgcn_raw_buffer_load_b16(rks, (lane & 31) * 2, 0, 0);
            r.vs[0] = __builtin_amdgcn_raw_buffer_load_b16(rvs, (lane & 31) * 2, 0, 0);
            return;
        }
        const int vbytes = valid ? D * 12 : 0, vsbytes = valid ? D * 2 : 0;
        const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.kc + (head_k + kt) * NB * 3), (short)0, nk * NB * 12, kBufWord3);
        const __amdgpu_buffer_rsrc_t rss = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.ks + (head_k + kt) * NB), (short)0, nk * NB * 2, kBufWord3);
        const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.vc + grp * D * 3), (short)0, vbytes, kBufWord3);
        const __amdgpu_buffer_rsrc_t rsvs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.vs + grp * D), (short)0, vsbytes, kBufWord3);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            // K: item = (key item % 32, block item / 32), so that the LDS
            // writes of a load's 32 keys fall on distinct banks.  V: row
            // d = item of the key-transposed group, and scale entry item =
            // (block item / 32, key item % 32); the unpack zeroes the scales
            // past the key range (no use of loaded data here, so the loads
            // stay in flight).
            const int item = lane + 64 * i;
            const int koff = (item & 31) * NB + (item >> 5);
            const u32x3 kw = __builtin_amdgcn_raw_buffer_load_b96(rsk, koff * 12, 0, 0);
            r.k[i][0] = kw[0];
            r.k[i][1] = kw[1];
            r.k[i][2] = kw[2];
            r.ks[i] = __builtin_amdgcn_raw_buffer_load_b16(rss, koff * 2, 0, 0);
            const u32x3 vw = __builtin_amdgcn_raw_buffer_load_b96(rsv, item * 12, 0, 0);
            r.v[i][0] = vw[0];
            r.v[i][1] = vw[1];
            r.v[i][2] = vw[2];
            r.vs[i] = __builtin_amdgcn_raw_buffer_load_b16(rsvs, item * 2, 0, 0);
        }
    };

    // Each wave keeps two tiles in flight: tile i is unpacked from one
    // register set while the other set's loads (tile i + 1) are outstanding,
    // and the freed set is refilled with tile i + 2 right after the unpack.
    const int stride = kDecWaves * KT;
    auto process = [&](TileRegs &r, int kb) {
        // ---- unpack the held tile into this wave's LDS region
        const int nk = min(KT, k1 - kb);
        // P.V multiplies P by the V scales in fp16 (below).  With the lazy
        // max, P reaches 2^kLazy = 256, so a V scale of 256 or more (fp16
        // bits >= 0x5C00; sign-bit patterns count as large too) could carry
        // the product past 65504.  A tile holding such a scale moves the
        // running max to its own max, which bounds P by 1 and the product by
        // the scale itself.  (Read here: the registers are refilled with a
        // later tile right after the unpack.)
        bool big_sv = false;
#pragma unroll
        for (int i = 0; i < (FMT == 1 ? 1 : PER); ++i) big_sv |= r.vs[i] >= (uint16_t)0x5C00u;
        const float lazy = __any(big_sv) ? 0.0f : kLazy;
        wave_lds_sync();
        if constexpr (FMT == 1) {
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int item = lane + 64 * i;
                const int key = item & 31, b = item >> 5;
                const int d = item, dt = d >> 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // K chunk j: int8 16 (c - 8) = (c ^ 8) << 4, even elements first
                    my.kq[b][j][key][0] = ((r.k[i][j] << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
                    my.kq[b][j][key][1] = (r.k[i][j] & 0xF0F0F0F0u) ^ 0x80808080u;
                    // V row d, keys 8j .. 8j + 7 (key 8j + e in bits 4e)
                    my.vc[dt][j ^ (dt & 3)][d & 15][0] = r.v[i][j];
                }
            }
            if (lane < KT) {
                my.skf[0][lane] = half_bits_to_float(r.ks[0]) * 0.0625f;
                my.svs[0][lane] = lane < nk ? r.vs[0] : (uint16_t)0;
            }
        } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int item = lane + 64 * i;
            const int kkey = item & 31, kbk = item >> 5;
            uint32_t o[8];
            unpack_bytes(r.k[i][0], r.k[i][1], r.k[i][2], o);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                my.kq[kbk][c][kkey][0] = codes_to_i8(o[2 * c]);
                my.kq[kbk][c][kkey][1] = codes_to_i8(o[2 * c + 1]);
            }
            my.skf[kbk][kkey] = half_bits_to_float(r.ks[i]);
            const int key = item & 31, b = item >> 5;
            const int d = item, dt = d >> 4;
            unpack_bytes(r.v[i][0], r.v[i][1], r.v[i][2], o);    // keys 4qq..4qq+3 in o[qq]
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                my.vc[dt][c ^ (dt & 3)][d & 15][0] = o[2 * c];
                my.vc[dt][c ^ (dt & 3)][d & 15][1] = o[2 * c + 1];
            }
            my.svs[b][key] = key < nk ? r.vs[i] : (uint16_t)0;
        }
        }
        wave_lds_sync();
        // the registers are free again: fetch the tile two strides ahead
        load_tile(r, kb + 2 * stride);

        // ---- Q.K^T: two 16-key halves per block; lane (i16, qc) gets keys
        // 8qc + 4kh + [0, 4) for half kh, so its 8 logits are keys 8qc + [0, 8)
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        const int krow0 = 8 * (i16 >> 2) + (i16 & 3);
        if constexpr (FMT == 1) {
            // the block MFMAs of each key half chain into one int32 sum
            // (16 times the natural one; the 1/16 sits in the K scale)
            i32x4v sacc[2] = {i32x4v{}, i32x4v{}};
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
                    sacc[kh] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                        *reinterpret_cast<const i64_t *>(&my.kq[b][qc][krow0 + 4 * kh][0]), qop[b],
                        sacc[kh], 0, 0, 0);
            const f32x4 sk0 = *reinterpret_cast<const f32x4 *>(&my.skf[0][8 * qc]);
            const f32x4 sk1 = *reinterpret_cast<const f32x4 *>(&my.skf[0][8 * qc + 4]);
            const float skr[8] = {sk0.x, sk0.y, sk0.z, sk0.w, sk1.x, sk1.y, sk1.z, sk1.w};
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[4 * kh + e] = skr[4 * kh + e] * (float)sacc[kh][e];
            if (DEBUG && a.dbg_logits && row_ok) {
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = kb + 8 * qc + 4 * kh + e;
                        if (key < k1) a.dbg_logits[(size_t)flat * a.N + key] = sacc[kh][e] >> 4;
                    }
            }
        } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const f32x4 sk0 = *reinterpret_cast<const f32x4 *>(&my.skf[b][8 * qc]);
            const f32x4 sk1 = *reinterpret_cast<const f32x4 *>(&my.skf[b][8 * qc + 4]);
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const i64_t kop = *reinterpret_cast<const i64_t *>(&my.kq[b][qc][krow0 + 4 * kh][0]);
                const i32x4v sres = __builtin_amdgcn_mfma_i32_16x16x32_i8(kop, qop[b], i32x4v{}, 0, 0, 0);
                const f32x4 sk = kh ? sk1 : sk0;
                acc[4 * kh + 0] = fmaf(sk.x, (float)sres[0], acc[4 * kh + 0]);
                acc[4 * kh + 1] = fmaf(sk.y, (float)sres[1], acc[4 * kh + 1]);
                acc[4 * kh + 2] = fmaf(sk.z, (float)sres[2], acc[4 * kh + 2]);
                acc[4 * kh + 3] = fmaf(sk.w, (float)sres[3], acc[4 * kh + 3]);
                if (DEBUG && a.dbg_logits && row_ok) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = kb + 8 * qc + 4 * kh + e;
                        if (key < k1) a.dbg_logits[((size_t)flat * a.N + key) * NB + b] = sres[e];
                    }
                }
            }
        }
        }

        // ---- mask, online softmax in base 2 (running max moves by > 8 only;
        // PV16: by any amount)
        const bool masked = kb + KT > vis_from;
        if (masked) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int key = kb + 8 * qc + r;
                bool vis = key < k1;
                if (vis && key >= a.L) {
                    const int u = key - a.L;
                    vis = CAUSAL ? (u <= t) : (((mrow >> u) & 1ull) != 0ull);
                }
                if (!vis) acc[r] = -INFINITY;
            }
        }
        float amax = acc[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) amax = fmaxf(amax, acc[r]);
        amax = max_xor16(amax);
        amax = max_halves(amax);
        const float tmax = amax == -INFINITY ? -INFINITY : amax * c_row;
        const float m_new = tmax > m_run + lazy ? tmax : m_run;
        if (__any(m_new != m_run)) {
            const float alpha = m_new != m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            l_run *= alpha;
            lv_run *= alpha;
            if constexpr (PV16) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        oh[dt][j] = __builtin_convertvector(
                            __builtin_convertvector(oh[dt][j], f32x2) * alpha, f16x2);
            } else {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
            }
            m_run = m_new;
        }
        const float mm = m_run == -INFINITY ? 0.0f : m_run;
        f16x8 pk;
        float psum = 0.0f;
        const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
        // only a tile holding masked keys (the split's last) has -inf logits
        float pe[8];
        if (masked) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pe[e] = acc[e] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fmaf(acc[e], c_row, -mm));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(acc[e], c_row, -mm));
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const f16x2 h2 = __builtin_convertvector(f32x2{pe[e], pe[e + 1]}, f16x2);
            pk[e] = h2.x;
            pk[e + 1] = h2.y;
            psum = __builtin_amdgcn_fdot2(h2, ones, psum, false);
        }
        l_run += psum;

        // ---- P.V: A operand = the codes' values c - 4 (exact in fp16) of
        // V^T rows d = 16dt + i16, keys 8qc + [0, 8); B operand = P times the
        // V scales of those keys in block d / 32 (keys 8qc + [0, 8), row i16).
        __builtin_amdgcn_s_setprio(1);
        if constexpr (FMT == 1) {
            // 4-bit: one V scale per key, so P times it serves every d-tile.
            // The A operand holds the codes c as fp16 bit patterns, i.e. the
            // subnormals c * 2^-24 (exact; the MFMA keeps subnormal inputs):
            // the product is 2^-24 sum pb c, and sum pb (c - 8) = 2^24 acc -
            // 8 sum pb, with sum pb kept per row in lv_run.
            const u32x4 svw = *reinterpret_cast<const u32x4 *>(&my.svs[0][8 * qc]);
            const uint32_t s01 = svw[0], s23 = svw[1], s45 = svw[2], s67 = svw[3];
            const f16x2 p01 = f16x2{pk[0], pk[1]} * __builtin_bit_cast(f16x2, s01);
            const f16x2 p23 = f16x2{pk[2], pk[3]} * __builtin_bit_cast(f16x2, s23);
            const f16x2 p45 = f16x2{pk[4], pk[5]} * __builtin_bit_cast(f16x2, s45);
            const f16x2 p67 = f16x2{pk[6], pk[7]} * __builtin_bit_cast(f16x2, s67);
            const f16x8 pb = {p01.x, p01.y, p23.x, p23.y, p45.x, p45.y, p67.x, p67.y};
            float lsum = __builtin_amdgcn_fdot2(p01, ones, 0.0f, false);
            lsum = __builtin_amdgcn_fdot2(p23, ones, lsum, false);
            lsum = __builtin_amdgcn_fdot2(p45, ones, lsum, false);
            lv_run += __builtin_amdgcn_fdot2(p67, ones, lsum, false);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const uint32_t w = my.vc[dt][qc ^ (dt & 3)][i16][0];
                const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
                // keys 2m (low nibbles) and 2m + 1 (high nibbles) as two fp16
                const uint32_t v0 = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u);
                const uint32_t v1 = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u);
                const uint32_t v2 = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u);
                const uint32_t v3 = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u);
                const f16x8 vop = __builtin_bit_cast(f16x8, u32x4{v0, v1, v2, v3});
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pb, oacc[dt], 0, 0, 0);
            }
        } else {
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            // Scales of keys 8qc + [0, 8), two per word.  Each word goes
            // through a scalar: clang bit-casts a vector component
            // (v.y, v.z, ...) as if it were component 0.
            const u32x4 svw = *reinterpret_cast<const u32x4 *>(&my.svs[bb][8 * qc]);
            const uint32_t s01 = svw[0], s23 = svw[1], s45 = svw[2], s67 = svw[3];
            const f16x2 p01 = f16x2{pk[0], pk[1]} * __builtin_bit_cast(f16x2, s01);
            const f16x2 p23 = f16x2{pk[2], pk[3]} * __builtin_bit_cast(f16x2, s23);
            const f16x2 p45 = f16x2{pk[4], pk[5]} * __builtin_bit_cast(f16x2, s45);
            const f16x2 p67 = f16x2{pk[6], pk[7]} * __builtin_bit_cast(f16x2, s67);
            const f16x8 pb = {p01.x, p01.y, p23.x, p23.y, p45.x, p45.y, p67.x, p67.y};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int dt = 2 * bb + h;
                const uint32_t *cw = my.vc[dt][qc ^ (dt & 3)][i16];
                const uint32_t w0 = cw[0], w1 = cw[1];
                const uint32_t ta = __builtin_amdgcn_perm(kC4Hi, kC4Lo, w0);
                const uint32_t tb = __builtin_amdgcn_perm(kC4Hi, kC4Lo, w1);
                const uint32_t v0 = __builtin_amdgcn_perm(ta, ta, 0x010C000Cu);
                const uint32_t v1 = __builtin_amdgcn_perm(ta, ta, 0x030C020Cu);
                const uint32_t v2 = __builtin_amdgcn_perm(tb, tb, 0x010C000Cu);
                const uint32_t v3 = __builtin_amdgcn_perm(tb, tb, 0x030C020Cu);
                const f16x8 vop = __builtin_bit_cast(f16x8, u32x4{v0, v1, v2, v3});
                if constexpr (PV16) {
                    const f32x4 tp = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pb, f32x4{}, 0, 0, 0);
                    oh[dt][0] += __builtin_convertvector(f32x2{tp[0], tp[1]}, f16x2);
                    oh[dt][1] += __builtin_convertvector(f32x2{tp[2], tp[3]}, f16x2);
                } else {
                    oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pb, oacc[dt], 0, 0, 0);
                }
            }
        }
        }
        __builtin_amdgcn_s_setprio(0);
    };
    TileRegs r0, r1;
    const int kb0 = k0 + wave * KT;
    load_tile(r0, kb0);
    load_tile(r1, kb0 + stride);
    for (int kb = kb0; kb < k1; kb += 2 * stride) {
        process(r0, kb);
        if (kb + stride >= k1) break;
        process(r1, kb + stride);
    }

    if constexpr (PV16) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            oacc[dt] = f32x4{(float)oh[dt][0].x, (float)oh[dt][0].y, (float)oh[dt][1].x,
                             (float)oh[dt][1].y};
    }
    if constexpr (FMT == 1) {
        // sum pb (c - 8) = 2^24 acc - 8 sum pb, per row
        float lv = lv_run + __shfl_xor(lv_run, 16);
        lv = sum_halves(lv);
        const float corr = -8.0f * lv;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) oacc[dt][i] = fmaf(oacc[dt][i], 16777216.0f, corr);
    }
    // ---- merge the four waves' softmax states through LDS, in wave order
    float l_row = l_run + __shfl_xor(l_run, 16);
    l_row = sum_halves(l_row);
    __syncthreads();                                   // tile regions are free now
    float *ostage = reinterpret_cast<float *>(&my);    // [16 rows][D], then m[16], l[16]
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4 *>(ostage + i16 * D + 16 * dt + 4 * qc) = oacc[dt];
    if (qc == 0) {
        ostage[16 * D + i16] = m_run;
        ostage[16 * D + 16 + i16] = l_row;
    }
    __syncthreads();
    // thread -> (row r, 16 consecutive elements)
    const int r = tid >> 4;
    const int c0 = (tid & 15) * (D / 16);
    if (row0 + r >= a.R) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w)
        M = fmaxf(M, reinterpret_cast<const float *>(&wl[w])[16 * D + r]);
    float wt[kDecWaves];
    float Lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
        const float *st = reinterpret_cast<const float *>(&wl[w]);
        const float mw = st[16 * D + r];
        wt[w] = (M == -INFINITY || mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        Lsum += wt[w] * st[16 * D + 16 + r];
    }
    const float inv_l = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
    const float lse = Lsum > 0.0f ? (M + log2f(Lsum)) * 0.69314718055994531f : -INFINITY;
    const int tr = (row0 + r) / a.G, gr = row0 + r - tr * a.G;
    const int flat_r = tr * a.Hq + head * a.G + gr;
    const size_t rows_total = (size_t)a.T * a.Hq;
    const bool partial = a.part_o != nullptr;
    float *dst = (partial ? a.part_o + (size_t)split * rows_total * D : a.out) + (size_t)flat_r * D;
#pragma unroll
    for (int j = 0; j < D / 16; j += 4) {
        f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(
                reinterpret_cast<const float *>(&wl[w]) + r * D + c0 + j);
            o += wt[w] * v;
        }
        *reinterpret_cast<f32x4 *>(dst + c0 + j) = o * inv_l;
    }
    if ((tid & 15) == 0) {
        if (partial)
            a.part_lse[(size_t)split * rows_total + flat_r] = lse;
        else if (a.out_lse)
            a.out_lse[flat_r] = lse;
    }
}

// ---------------------------------------------------------------- merge

// One work-group per output row, or per (row, chunk of CC column groups of
// four) when rows are few: then the row's partials stream through D / 4CC
// CUs instead of one.  The weights exp(lse_s - M) come from a block-wide max
// and sum; then thread (g, c) accumulates column group c over the splits
// s = g, g + G, g + 2G, ... (four loads in flight), and the G partial sums
// are added in order g = 0, 1, ... through LDS, so the result does not
// depend on timing.  G grows with S so that few rows with many splits still
// keep many loads in flight.
constexpr int kMergeMaxThreads = 1024;
constexpr int kMergeWeights = 1024;      // weights cached in LDS for s < this
constexpr int kMergePre = 8;             // partial vectors a thread loads up front
constexpr int kMergeChunkRows = 1024;    // fewer rows: a row's columns split over work-groups

__device__ __forceinline__ float block_reduce(float v, float *red, bool is_max) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_waves = blockDim.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float w = __shfl_xor(v, o);
        v = is_max ? fmaxf(v, w) : v + w;
    }
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
    for (int i = 1; i < n_waves; ++i) v = is_max ? fmaxf(v, red[i]) : v + red[i];
    return v;
}

__device__ __forceinline__ float merge_weight(const float *part_lse, const float *wgt, int s,
                                              int rows, int row, float M) {
    if (s < kMergeWeights) return wgt[s];
    const float ls = part_lse[(size_t)s * rows + row];
    return ls == -INFINITY ? 0.0f : expf(ls - M);
}

// Few splits (S <= kMergeSmallS, D % 4 == 0): one thread per (row, 4
// columns), several rows per work-group; each thread reads the row's S lse
// values itself, so there is no block reduction, barrier or LDS, and many
// rows run per CU (the chunked prefill merges ~10^5 rows over 2 splits).
constexpr int kMergeSmallS = 8;
constexpr int kMergeSmallThreads = 256;

__global__ __launch_bounds__(kMergeSmallThreads) void merge_small_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse, int S, int rows, int D,
    float *__restrict__ out, float *__restrict__ out_lse) {
    const int C = D / 4;
    const int per_wg = kMergeSmallThreads / C;
    if ((int)threadIdx.x >= per_wg * C) return;
    const int row = blockIdx.x * per_wg + threadIdx.x / C;
    const int c = threadIdx.x % C;
    if (row >= rows) return;
    float ls[kMergeSmallS];
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMergeSmallS; ++s) {
        ls[s] = s < S ? part_lse[(size_t)s * rows + row] : -INFINITY;
        M = fmaxf(M, ls[s]);
    }
    f32x4 *dst = reinterpret_cast<f32x4 *>(out + (size_t)row * D + 4 * c);
    if (M == -INFINITY) {
        *dst = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (out_lse && c == 0) out_lse[row] = -INFINITY;
        return;
    }
    // An empty split (lse = -inf) has weight 0 and an all-zero partial.
    float W = 0.0f;
    f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < kMergeSmallS; ++s) {
        if (s < S) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(part_o + ((size_t)s * rows + row) * D + 4 * c);
            const float w = ls[s] == -INFINITY ? 0.0f : expf(ls[s] - M);
            W += w;
            o += w * v;
        }
    }
    const float invW = W > 0.0f ? 1.0f / W : 0.0f;
    *dst = o * invW;
    if (out_lse && c == 0) out_lse[row] = M + logf(W);
}

__global__ __launch_bounds__(kMergeMaxThreads) void merge_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse, int S, int rows, int D,
    int G, int CC, float *__restrict__ out, float *__restrict__ out_lse) {
    __shared__ float red[kMergeMaxThreads / 64];
    __shared__ float wgt[kMergeWeights];
    __shared__ f32x4 acc_lds[kMergeMaxThreads];
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    // Vector path: thread (g, c) owns column group c of splits g, g + G, ...
    // Its first kMergePre partial vectors are loaded before the weights are
    // known, so their latency overlaps the two block reductions.
    const bool vec = (D & 3) == 0;
    const int C = vec ? CC : 1;
    const int g = tid / C, c = tid - (tid / C) * C;
    const bool gv = vec && g < G;
    const int c0 = vec ? (int)blockIdx.y * CC : 0;      // first column group of the chunk
    const size_t split_stride = (size_t)rows * D;
    const float *col = part_o + (size_t)row * D + 4 * (c0 + c);
    f32x4 pre[kMergePre];
#pragma unroll
    for (int u = 0; u < kMergePre; ++u) {
        const int s = g + u * G;
        pre[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (gv && s < S) pre[u] = *reinterpret_cast<const f32x4 *>(col + (size_t)s * split_stride);
    }
    // lse values of this thread's splits s = tid, tid + nt, ... (the first
    // one kept in a register for the second pass)
    const float ls0 = tid < S ? part_lse[(size_t)tid * rows + row] : -INFINITY;
    float M = ls0;
    for (int s = tid + nt; s < S; s += nt) M = fmaxf(M, part_lse[(size_t)s * rows + row]);
    M = block_reduce(M, red, true);
    float W = 0.0f;
    if (M != -INFINITY)
        for (int s = tid; s < S; s += nt) {
            const float ls = s == tid ? ls0 : part_lse[(size_t)s * rows + row];
            const float w = ls == -INFINITY ? 0.0f : expf(ls - M);
            W += w;
            if (s < kMergeWeights) wgt[s] = w;
        }
    W = block_reduce(W, red, false);
    const float invW = W > 0.0f ? 1.0f / W : 0.0f;
    if (out_lse && tid == 0 && blockIdx.y == 0) out_lse[row] = M == -INFINITY ? -INFINITY : M + logf(W);
    __syncthreads();
    if (M == -INFINITY) {
        const int d_end = vec ? 4 * (c0 + CC) : D;
        for (int d = 4 * c0 + tid; d < d_end; d += nt) out[(size_t)row * D + d] = 0.0f;
        return;
    }
    if (vec) {
        // An empty split (lse = -inf) has weight 0 and an all-zero partial.
        f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
        if (gv) {
#pragma unroll
            for (int u = 0; u < kMergePre; ++u) {
                const int s = g + u * G;
                if (s < S) o += merge_weight(part_lse, wgt, s, rows, row, M) * pre[u];
            }
            for (int s0 = g + kMergePre * G; s0 < S; s0 += 4 * G) {
                f32x4 v[4];
                float w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int s = s0 + u * G;
                    v[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    w[u] = 0.0f;
                    if (s < S) {
                        v[u] = *reinterpret_cast<const f32x4 *>(col + (size_t)s * split_stride);
                        w[u] = merge_weight(part_lse, wgt, s, rows, row, M);
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) o += w[u] * v[u];
            }
        }
        acc_lds[tid] = o;
        __syncthreads();
        if (g == 0) {
            f32x4 sum = acc_lds[c];
            for (int k = 1; k < G; ++k) sum += acc_lds[k * C + c];
            *reinterpret_cast<f32x4 *>(out + (size_t)row * D + 4 * (c0 + c)) = sum * invW;
        }
    } else {
        for (int d = tid; d < D; d += nt) {
            float o = 0.0f;
            for (int s = 0; s < S; ++s)
                o += merge_weight(part_lse, wgt, s, rows, row, M) *
                     part_o[((size_t)s * rows + row) * D + d];
            out[(size_t)row * D + d] = o * invW;
        }
    }
}

// Row groups per work-group.  Paired four-wave groups (NG = 2, items v and
// v + 8 of each block of 16) measured slower than two independent
// work-groups per CU on the 64-node tree over 262K (645 against 610 us; the
// extra barrier per tile and each phase waiting for the slower group cost
// more than the overlap of complementary phases gains), so every variant
// runs one group; NG = 2 stays available to the template.
template <int NW, bool DEBUG>
constexpr int kGroups = 1;

// The wave-specialized kernel serves the 3-bit verify rows at head_dim 256 in
// groups of four row tiles; the other shapes run attn_split_kernel.
template <int D, int NW, bool CAUSAL, int FMT>
constexpr bool kWaveSpecialized = D == 256 && NW == 4 && FMT == 0 && !CAUSAL;

template <int D, bool CAUSAL, bool DEBUG>
hipError_t launch_ws_t(const AttnArgs &a, hipStream_t stream) {
    // eight runs of ceil(items / 8) work-groups, one per XCD
    const int per_xcd = (a.Hkv * a.S * a.NRG + 7) / 8;
    hipLaunchKernelGGL((attn_ws_kernel<D, CAUSAL, DEBUG>), dim3(8 * per_xcd), dim3(kWsThreads), 0, stream, a);
    return hipGetLastError();
}

template <int D, int NW, bool CAUSAL, bool DEBUG, int FMT, bool PV16 = false, bool PRE = false>
hipError_t launch_t(const AttnArgs &a, hipStream_t stream) {
    if constexpr (kWaveSpecialized<D, NW, CAUSAL, FMT> && !PV16 && !PRE) return launch_ws_t<D, CAUSAL, DEBUG>(a, stream);
    constexpr int NG = kGroups<NW, DEBUG>;
    const int items = a.n_hs_pad * a.NRG;
    const int grid = NG == 2 ? 8 * ((items + 15) / 16) : items;
    hipLaunchKernelGGL((attn_split_kernel<D, NW, NG, CAUSAL, DEBUG, FMT, PV16, PRE>), dim3(grid),
                       dim3(NG * NW * 64), 0, stream, a);
    return hipGetLastError();
}

// The PV16 variant exists for the 3-bit format, verify rows, no debug output.
template <int D, int NW, int FMT>
hipError_t launch_d(const AttnArgs &a, bool causal, bool debug, bool pv16, hipStream_t s) {
    if (pv16) {
        if constexpr (FMT == 0) {
            if (!causal && !debug) return launch_t<D, NW, false, false, 0, true>(a, s);
        }
        return hipErrorInvalidValue;
    }
    if (causal) {
        if constexpr (NW == 4 && FMT == 0) {
            // the causal chunk reading tile images (a.img set by the caller)
            if (a.img && !debug) return launch_t<D, NW, true, false, FMT, false, true>(a, s);
        }
        return debug ? launch_t<D, NW, true, true, FMT>(a, s) : launch_t<D, NW, true, false, FMT>(a, s);
    }
    if (a.img) return hipErrorInvalidValue;
    return debug ? launch_t<D, NW, false, true, FMT>(a, s) : launch_t<D, NW, false, false, FMT>(a, s);
}

template <int D, int FMT>
hipError_t launch_nw(const AttnArgs &a, int NW, bool causal, bool debug, bool pv16, hipStream_t s) {
    switch (NW) {
        case 1: return launch_d<D, 1, FMT>(a, causal, debug, pv16, s);
        case 2: return launch_d<D, 2, FMT>(a, causal, debug, pv16, s);
        case 4: return launch_d<D, 4, FMT>(a, causal, debug, pv16, s);
        default: return hipErrorInvalidValue;
    }
}

// Resident items (row groups of NW waves) per CU.
template <int D, int NW, bool CAUSAL, int FMT>
int occupancy_t() {
    constexpr int NG = kGroups<NW, false>;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void *>(&attn_split_kernel<D, NW, NG, CAUSAL, false, FMT, false>),
            NG * NW * 64, 0) != hipSuccess)
        return 0;
    return n * NG;
}

template <int D, int FMT>
int occupancy_d(int NW, bool causal) {
    switch (NW) {
        case 1: return causal ? occupancy_t<D, 1, true, FMT>() : occupancy_t<D, 1, false, FMT>();
        case 2: return causal ? occupancy_t<D, 2, true, FMT>() : occupancy_t<D, 2, false, FMT>();
        case 4: return causal ? occupancy_t<D, 4, true, FMT>() : occupancy_t<D, 4, false, FMT>();
        default: return 0;
    }
}

template <int D, bool CAUSAL, bool DEBUG, bool PV16 = false>
hipError_t launch_s16_t(const AttnArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((attn_split16_kernel<D, CAUSAL, DEBUG, PV16>), dim3(a.n_hs_pad * a.NRG),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
}

// The PV16 variant: verify rows, no debug output.
template <int D>
hipError_t launch_s16_d(const AttnArgs &a, bool causal, bool debug, bool pv16, hipStream_t s) {
    if (pv16) {
        if (causal || debug) return hipErrorInvalidValue;
        return launch_s16_t<D, false, false, true>(a, s);
    }
    if (causal) return debug ? launch_s16_t<D, true, true>(a, s) : launch_s16_t<D, true, false>(a, s);
    return debug ? launch_s16_t<D, false, true>(a, s) : launch_s16_t<D, false, false>(a, s);
}

template <int D, bool CAUSAL>
int occupancy_s16_t() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void *>(&attn_split16_kernel<D, CAUSAL, false, false>), 256,
            0) != hipSuccess)
        return 0;
    return n;
}

template <int D, bool CAUSAL, bool DEBUG, int FMT, bool PV16 = false>
hipError_t launch_dec_t(const AttnArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((attn_dec_kernel<D, CAUSAL, DEBUG, PV16, FMT>), dim3(a.n_hs_pad * a.NRG),
                       dim3(kDecWaves * 64), 0, stream, a);
    return hipGetLastError();
}

// The PV16 variant exists for the 3-bit format, verify rows, no debug output.
template <int D, int FMT>
hipError_t launch_dec_d(const AttnArgs &a, bool causal, bool debug, bool pv16, hipStream_t s) {
    if (pv16) {
        if constexpr (FMT == 0) {
            if (!causal && !debug) return launch_dec_t<D, false, false, 0, true>(a, s);
        }
        return hipErrorInvalidValue;
    }
    if (causal)
        return debug ? launch_dec_t<D, true, true, FMT>(a, s) : launch_dec_t<D, true, false, FMT>(a, s);
    return debug ? launch_dec_t<D, false, true, FMT>(a, s) : launch_dec_t<D, false, false, FMT>(a, s);
}

template <int D, bool CAUSAL, int FMT>
int occupancy_dec_t() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void *>(&attn_dec_kernel<D, CAUSAL, false, false, FMT>),
            kDecWaves * 64, 0) != hipSuccess)
        return 0;
    return n;
}

}  // namespace

int attention_ws_wgs_per_cu(int D) {
    if (D != 256) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void *>(&attn_ws_kernel<256, false, false>), kWsThreads, 0) != hipSuccess)
        return 0;
    return n;
}

int attention_s16_wgs_per_cu(int D, bool causal) {
    switch (D) {
        case 64: return causal ? occupancy_s16_t<64, true>() : occupancy_s16_t<64, false>();
        case 128: return causal ? occupancy_s16_t<128, true>() : occupancy_s16_t<128, false>();
        case 256: return causal ? occupancy_s16_t<256, true>() : occupancy_s16_t<256, false>();
        default: return 0;
    }
}

hipError_t launch_attention_s16(const AttnArgs &a, int D, bool causal, bool debug, bool pv16,
                                hipStream_t stream) {
    switch (D) {
        case 64: return launch_s16_d<64>(a, causal, debug, pv16, stream);
        case 128: return launch_s16_d<128>(a, causal, debug, pv16, stream);
        case 256: return launch_s16_d<256>(a, causal, debug, pv16, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int FMT>
int dec_wgs_per_cu_f(int D, bool causal) {
    switch (D) {
        case 64: return causal ? occupancy_dec_t<64, true, FMT>() : occupancy_dec_t<64, false, FMT>();
        case 128: return causal ? occupancy_dec_t<128, true, FMT>() : occupancy_dec_t<128, false, FMT>();
        case 256: return causal ? occupancy_dec_t<256, true, FMT>() : occupancy_dec_t<256, false, FMT>();
        default: return 0;
    }
}

int attention_dec_wgs_per_cu(int D, bool causal, int fmt) {
    return fmt == 1 ? dec_wgs_per_cu_f<1>(D, causal) : dec_wgs_per_cu_f<0>(D, causal);
}

template <int FMT>
hipError_t launch_dec_f(const AttnArgs &a, int D, bool causal, bool debug, bool pv16,
                        hipStream_t stream) {
    switch (D) {
        case 64: return launch_dec_d<64, FMT>(a, causal, debug, pv16, stream);
        case 128: return launch_dec_d<128, FMT>(a, causal, debug, pv16, stream);
        case 256: return launch_dec_d<256, FMT>(a, causal, debug, pv16, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attention_dec(const AttnArgs &a, int D, bool causal, bool debug, bool pv16,
                                int fmt, hipStream_t stream) {
    return fmt == 1 ? launch_dec_f<1>(a, D, causal, debug, pv16, stream)
                    : launch_dec_f<0>(a, D, causal, debug, pv16, stream);
}

int attention_wgs_per_cu(int D, int NW, bool causal, int fmt) {
    if (fmt == 1) {
        switch (D) {
            case 64: return occupancy_d<64, 1>(NW, causal);
            case 128: return occupancy_d<128, 1>(NW, causal);
            case 256: return occupancy_d<256, 1>(NW, causal);
            default: return 0;
        }
    }
    switch (D) {
        case 64: return occupancy_d<64, 0>(NW, causal);
        case 128: return occupancy_d<128, 0>(NW, causal);
        case 256: return occupancy_d<256, 0>(NW, causal);
        default: return 0;
    }
}

size_t tile_image_bytes(int D) {
    switch (D) {
        case 64: return PreLayout<64>::BYTES;
        case 128: return PreLayout<128>::BYTES;
        case 256: return PreLayout<256>::BYTES;
        default: return 0;
    }
}

template <int D, int FMT>
hipError_t launch_img_t(const AttnArgs &a, unsigned char *img, hipStream_t s) {
    hipLaunchKernelGGL((tile_image_kernel<D, FMT>), dim3(a.img_tiles, a.Hkv), dim3(256), 0, s, a, img);
    return hipGetLastError();
}

// (3-bit format only)
hipError_t launch_tile_images(const AttnArgs &a, int D, int fmt, unsigned char *img, hipStream_t s) {
    if (a.img_tiles <= 0) return hipSuccess;
    if (fmt != 0) return hipErrorInvalidValue;
    switch (D) {
        case 64: return launch_img_t<64, 0>(a, img, s);
        case 128: return launch_img_t<128, 0>(a, img, s);
        case 256: return launch_img_t<256, 0>(a, img, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attention(const AttnArgs &a, int D, int NW, bool causal, bool debug, int fmt,
                            bool pv16, hipStream_t stream) {
    if (fmt == 1) {
        switch (D) {
            case 64: return launch_nw<64, 1>(a, NW, causal, debug, pv16, stream);
            case 128: return launch_nw<128, 1>(a, NW, causal, debug, pv16, stream);
            case 256: return launch_nw<256, 1>(a, NW, causal, debug, pv16, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (D) {
        case 64: return launch_nw<64, 0>(a, NW, causal, debug, pv16, stream);
        case 128: return launch_nw<128, 0>(a, NW, causal, debug, pv16, stream);
        case 256: return launch_nw<256, 0>(a, NW, causal, debug, pv16, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_merge(const float *part_o, const float *part_lse, int S, int rows, int D,
                        float *out, float *out_lse, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    if ((D & 3) == 0 && S <= kMergeSmallS && D / 4 <= kMergeSmallThreads) {
        const int per_wg = kMergeSmallThreads / (D / 4);
        hipLaunchKernelGGL(merge_small_kernel, dim3((rows + per_wg - 1) / per_wg),
                           dim3(kMergeSmallThreads), 0, stream, part_o, part_lse, S, rows, D, out,
                           out_lse);
        return hipGetLastError();
    }
    // Vector path: C = D / 4 column groups times G split groups, about
    // eight splits per group (so many rows keep blocks small), at most 1024
    // threads.  Fewer rows than kMergeChunkRows: the columns split into
    // chunks of 16 groups, one work-group each, with the same G (so the same
    // order of the sums).  Scalar path (D % 4 != 0): 256 threads over the
    // columns.
    int G = 1, threads = 256, CC = 1, chunks = 1;
    if ((D & 3) == 0) {
        const int C = D / 4;
        G = (S + 7) / 8;
        if (G > kMergeMaxThreads / C) G = kMergeMaxThreads / C;
        if (G < 1) G = 1;
        CC = C;
        if (rows < kMergeChunkRows && C % 16 == 0) CC = 16;
        chunks = C / CC;
        threads = ((CC * G + 63) / 64) * 64;
    }
    hipLaunchKernelGGL(merge_kernel, dim3(rows, chunks), dim3(threads), 0, stream, part_o, part_lse,
                       S, rows, D, G, CC, out, out_lse);
    return hipGetLastError();
}

hipError_t launch_kv_pack(const float *x, int n_tok, int pos0, uint32_t *codes, uint16_t *scales,
                          int Hkv, int D, int cap, bool is_v, hipStream_t stream) {
    const long long items = (long long)n_tok * Hkv * (D / 32);
    if (items == 0) return hipSuccess;
    const int threads = 256;
    if (!is_v) {
        hipLaunchKernelGGL(k_pack_kernel, dim3((unsigned)((items + threads - 1) / threads)),
                           dim3(threads), 0, stream, x, n_tok, pos0, codes, scales, Hkv, D, cap);
        return hipGetLastError();
    }
    // V: one work-group of D (64, 128 or 256) threads per (head, touched group)
    const int ng = (cap + 31) / 32;
    const int grp0 = pos0 / 32, n_grp = (pos0 + n_tok - 1) / 32 - grp0 + 1;
    hipLaunchKernelGGL(v_pack_kernel, dim3((unsigned)((long long)n_grp * Hkv)), dim3(D), 0, stream, x, n_tok,
                       pos0, codes, scales, Hkv, D, ng, grp0);
    return hipGetLastError();
}

hipError_t launch_kv_pack4(const float *x, int n_tok, int pos0, uint32_t *codes, uint16_t *scales,
                           int Hkv, int D, int cap, bool is_v, hipStream_t stream) {
    if (n_tok == 0) return hipSuccess;
    const int rows = n_tok * Hkv;
    if (!is_v) {
        hipLaunchKernelGGL(kv4_pack_kernel<false>, dim3(rows), dim3(64), 0, stream, x, pos0, codes,
                           scales, Hkv, D, cap);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(kv4_pack_kernel<true>, dim3(rows), dim3(64), 0, stream, x, pos0, codes,
                       scales, Hkv, D, cap);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ng = (cap + 31) / 32;
    const int grp0 = pos0 / 32, n_grp = (pos0 + n_tok - 1) / 32 - grp0 + 1;
    const long long items = (long long)n_grp * Hkv * D;
    const int threads = 256;
    hipLaunchKernelGGL(v4_code_kernel, dim3((unsigned)((items + threads - 1) / threads)),
                       dim3(threads), 0, stream, x, n_tok, pos0, codes, scales, Hkv, D, cap, ng,
                       grp0, n_grp);
    return hipGetLastError();
}

// ------------------------------------------- scratch of the no-alloc entry

// Split partials of stv_verify_attention_noalloc: a file-scope device array,
// one per GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

void *noalloc_scratch(hipError_t *err) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *ptr[kMaxDevices];
    *err = hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = e != hipSuccess ? e : hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        // with device `dev` current (hipGetDevice above): its own copy
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        ptr[dev] = p;
    }
    return ptr[dev];
}

}  // namespace stv
