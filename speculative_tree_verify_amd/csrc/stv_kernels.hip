// HIP kernels for gfx950 (MI355X): 3-bit K/V pack, split attention with an
// int8 MFMA Q.K^T stage and an fp16-in / fp32-accumulate MFMA P.V stage,
// and the log-sum-exp merge of split partials.
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
#include "stv_internal.h"

#include <math.h>

namespace stv {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ 3-bit blocks
// Byte-plane layout: byte i of word qq' below holds the code of element
// 4*qq + i.  Words 0..2 of a block give codes qq = 0..7 as follows.
__device__ __forceinline__ void unpack_bytes(uint32_t w0, uint32_t w1, uint32_t w2,
                                             uint32_t o[8]) {
    const uint32_t m3 = 0x07070707u, m2 = 0x03030303u, mh = 0x04040404u;
    o[0] = w0 & m3;
    o[1] = (w0 >> 3) & m3;
    o[2] = w1 & m3;
    o[3] = (w1 >> 3) & m3;
    o[4] = w2 & m3;
    o[5] = (w2 >> 3) & m3;
    o[6] = ((w0 >> 6) & m2) | ((w2 >> 4) & mh);
    o[7] = ((w1 >> 6) & m2) | ((w2 >> 5) & mh);
}

__device__ __forceinline__ void pack_bytes(const uint32_t o[8], uint32_t &w0, uint32_t &w1,
                                           uint32_t &w2) {
    const uint32_t m2 = 0x03030303u, mh = 0x04040404u;
    w0 = o[0] | (o[1] << 3) | ((o[6] & m2) << 6);
    w1 = o[2] | (o[3] << 3) | ((o[7] & m2) << 6);
    w2 = o[4] | (o[5] << 3) | ((o[6] & mh) << 4) | ((o[7] & mh) << 5);
}

// Four codes c in [0, 7] (one per byte) -> four int8 values c - 4.  Setting
// bit 7 of every byte first keeps the byte-wise subtraction borrow-free.
__device__ __forceinline__ uint32_t codes_to_i8(uint32_t o) {
    return ((o | 0x80808080u) - 0x04040404u) ^ 0x80808080u;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// ------------------------------------------------------------- kv pack

__global__ void kv_pack_kernel(const float *__restrict__ x, int n_tok, int pos0,
                               uint32_t *__restrict__ codes, uint16_t *__restrict__ scales,
                               int Hkv, int D, int cap) {
    const int NB = D / 32;
    const long long total = (long long)n_tok * Hkv * NB;
    const long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= total) return;
    const int b = (int)(id % NB);
    const int g = (int)((id / NB) % Hkv);
    const int t = (int)(id / ((long long)NB * Hkv));
    const f32x4 *src = reinterpret_cast<const f32x4 *>(x + ((size_t)t * Hkv + g) * D + 32 * b);
    float v[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        f32x4 f = src[j];
        v[4 * j + 0] = f.x;
        v[4 * j + 1] = f.y;
        v[4 * j + 2] = f.z;
        v[4 * j + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
    _Float16 sh = (_Float16)(amax / 3.0f);            // RNE to binary16
    uint16_t s16 = __builtin_bit_cast(uint16_t, sh);
    if ((s16 & 0x7FFFu) == 0x7C00u) s16 = 0x7BFFu;     // saturate to 65504
    const float s = half_bits_to_float(s16);
    uint32_t o[8];
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int c = 4;
            if (s != 0.0f) {
                float r = rintf(v[4 * qq + i] / s);
                r = fminf(fmaxf(r, -4.0f), 3.0f);
                c = (int)r + 4;
            }
            word |= (uint32_t)c << (8 * i);
        }
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

// ------------------------------------------------------------ attention

template <int D, int NW, bool CAUSAL, bool DEBUG>
__global__ __launch_bounds__(NW * 64) void attn_split_kernel(const AttnArgs a) {
    constexpr int NB = D / 32;
    constexpr int KT = kKeyTile;
    constexpr int KQS = D + 16;           // bytes per key row of the int8 K tile
    constexpr int VTS = KT + 8;           // halves per d row of the V^T tile
    constexpr int PAIRS = KT * NB;        // (key, block) pairs per tile
    constexpr int NT = NW * 64;
    constexpr int PPT = (PAIRS + NT - 1) / NT;

    __shared__ __attribute__((aligned(16))) int8_t kq[KT * KQS];
    __shared__ __attribute__((aligned(16))) _Float16 vt[D * VTS];
    __shared__ __attribute__((aligned(16))) float skf[NB * KT];

    // ---- work-group -> (kv head, split, row group).  Row groups of one
    // (head, split) get ids 8 apart so they share an XCD and its L2.
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
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int l32 = lane & 31;

    const int rho = (rg * NW + wave) * kRowTile + l32;
    const bool row_ok = rho < a.R;
    const int t = row_ok ? rho / a.G : 0;
    const int g = row_ok ? rho - t * a.G : 0;
    const int flat = t * a.Hq + head * a.G + g;
    const bool wave_active = (rg * NW + wave) * kRowTile < a.R;

    // ---- key range of this work-group
    int k0 = split * a.split_len;
    int k1 = min(a.N, k0 + a.split_len);
    if (CAUSAL) {
        const int rho_last = min(a.R, (rg + 1) * NW * kRowTile) - 1;
        k1 = min(k1, a.L + rho_last / a.G + 1);
    }
    const int vis_from = min(k1, a.L);   // keys below this need no mask test

    // ---- prologue: per-row int8 quantization of Q.  Lane (l32, hl) holds
    // row l32 of the wave and elements 32b + 16hl + [0, 16) of every block b:
    // the B operand layout of the 32x32x32 int8 MFMA.
    i32x4 qreg[NB];
    float sq = 0.0f;
    {
        const float *qrow = a.q + (size_t)flat * D + 16 * hl;
        float amax = 0.0f;
        if (row_ok) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x4 v = *reinterpret_cast<const f32x4 *>(qrow + 32 * b + 4 * j);
                    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)),
                                             fmaxf(fabsf(v.z), fabsf(v.w))));
                }
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
        sq = amax / 127.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t word = 0;
                if (row_ok) {
                    f32x4 v = *reinterpret_cast<const f32x4 *>(qrow + 32 * b + 4 * j);
                    float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float r = rintf(e[i] * inv);
                        r = fminf(fmaxf(r, -127.0f), 127.0f);
                        word |= ((uint32_t)(int)r & 0xFFu) << (8 * i);
                    }
                }
                qreg[b][j] = (int32_t)word;
            }
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

    uint64_t mrow = 0;
    if (!CAUSAL) {
        for (int tt = 0; tt < a.T; ++tt)
            if (tt == t) mrow = a.mask[tt];
    }

    // Key order inside a tile: MFMA row i of the Q.K^T product reads key
    // kperm(i), chosen so that output registers r = 0..7 of lane half hl hold
    // keys 8hl + r and registers 8..15 hold keys 16 + 8hl + (r - 8); those
    // are exactly the key runs the P.V MFMA wants from that lane.
    const int ai = l32 >> 3;
    const int krow = 16 * (ai >> 1) + 8 * ((l32 >> 2) & 1) + 4 * (ai & 1) + (l32 & 3);

    f32x16 oacc[NB];
#pragma unroll
    for (int dt = 0; dt < NB; ++dt) oacc[dt] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.0f;

    const size_t head_base = (size_t)head * a.cap;

    // ---- register prefetch of one tile
    uint32_t rk[PPT][3], rv[PPT][3];
    uint16_t rks[PPT], rvs[PPT];
    auto load_tile = [&](int kb) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + i * NT;
            const int key = kb + p / NB;
            const int b = p % NB;
            rk[i][0] = rk[i][1] = rk[i][2] = 0u;
            rv[i][0] = rv[i][1] = rv[i][2] = 0u;
            rks[i] = 0;
            rvs[i] = 0;
            if (p < PAIRS && key < k1) {
                const size_t blk = (head_base + key) * NB + b;
                const uint32_t *kw = a.kc + blk * 3;
                const uint32_t *vw = a.vc + blk * 3;
                rk[i][0] = kw[0];
                rk[i][1] = kw[1];
                rk[i][2] = kw[2];
                rv[i][0] = vw[0];
                rv[i][1] = vw[1];
                rv[i][2] = vw[2];
                rks[i] = a.ks[blk];
                rvs[i] = a.vs[blk];
            }
        }
    };

    if (k0 < k1) load_tile(k0);

    for (int kb = k0; kb < k1; kb += KT) {
        // ---- unpack the tile held in registers into LDS
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + i * NT;
            if (p < PAIRS) {
                const int kk = p / NB;
                const int b = p % NB;
                uint32_t o[8];
                unpack_bytes(rk[i][0], rk[i][1], rk[i][2], o);
                u32x4 lo = {codes_to_i8(o[0]), codes_to_i8(o[1]), codes_to_i8(o[2]),
                            codes_to_i8(o[3])};
                u32x4 hi = {codes_to_i8(o[4]), codes_to_i8(o[5]), codes_to_i8(o[6]),
                            codes_to_i8(o[7])};
                *reinterpret_cast<u32x4 *>(kq + kk * KQS + 32 * b) = lo;
                *reinterpret_cast<u32x4 *>(kq + kk * KQS + 32 * b + 16) = hi;
                skf[b * KT + kk] = half_bits_to_float(rks[i]);

                unpack_bytes(rv[i][0], rv[i][1], rv[i][2], o);
                const _Float16 sv = __builtin_bit_cast(_Float16, rvs[i]);
                const f16x2 svp = {sv, sv};
                const f16x2 off = {(_Float16)1028.0f, (_Float16)1028.0f};
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    // 0x6400 | c is the binary16 value 1024 + c; minus 1028 is c - 4.
                    const uint32_t lo_bits = (o[qq] & 0x00070007u) | 0x64006400u;
                    const uint32_t hi_bits = ((o[qq] >> 8) & 0x00070007u) | 0x64006400u;
                    const f16x2 vlo = (__builtin_bit_cast(f16x2, lo_bits) - off) * svp;
                    const f16x2 vhi = (__builtin_bit_cast(f16x2, hi_bits) - off) * svp;
                    _Float16 *col = vt + (32 * b + 4 * qq) * VTS + kk;
                    col[0 * VTS] = vlo.x;
                    col[2 * VTS] = vlo.y;
                    col[1 * VTS] = vhi.x;
                    col[3 * VTS] = vhi.y;
                }
            }
        }
        __syncthreads();

        if (kb + KT < k1) load_tile(kb + KT);

        if (wave_active) {
            // ---- Q.K^T: one int8 MFMA per 32-element block, fp32 epilogue
            f32x16 acc = f32x16{};
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const i32x4 kop = *reinterpret_cast<const i32x4 *>(kq + krow * KQS + 32 * b + 16 * hl);
                const i32x16 s = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop, qreg[b], i32x16{}, 0, 0, 0);
                const f32x4 s0 = *reinterpret_cast<const f32x4 *>(skf + b * KT + 8 * hl);
                const f32x4 s1 = *reinterpret_cast<const f32x4 *>(skf + b * KT + 8 * hl + 4);
                const f32x4 s2 = *reinterpret_cast<const f32x4 *>(skf + b * KT + 16 + 8 * hl);
                const f32x4 s3 = *reinterpret_cast<const f32x4 *>(skf + b * KT + 16 + 8 * hl + 4);
                const float skr[16] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w,
                                       s2.x, s2.y, s2.z, s2.w, s3.x, s3.y, s3.z, s3.w};
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] += skr[r] * (float)s[r];
                if (DEBUG && a.dbg_logits && row_ok) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb + (r < 8 ? 8 * hl + r : 16 + 8 * hl + (r - 8));
                        if (key < k1)
                            a.dbg_logits[((size_t)flat * a.N + key) * NB + b] = s[r];
                    }
                }
            }

            // ---- scale, mask, online softmax in base 2
            float y[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) y[r] = acc[r] * c_row;
            if (kb + KT > vis_from) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + (r < 8 ? 8 * hl + r : 16 + 8 * hl + (r - 8));
                    bool vis = key < k1;
                    if (vis && key >= a.L) {
                        const int u = key - a.L;
                        vis = CAUSAL ? (u <= t) : (((mrow >> u) & 1ull) != 0ull);
                    }
                    if (!vis) y[r] = -INFINITY;
                }
            }
            float tmax = y[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, y[r]);
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float m_new = fmaxf(m_run, tmax);
            float alpha = 1.0f;
            float p[16];
            if (m_new == -INFINITY) {
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = 0.0f;
            } else {
                alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(y[r] - m_new);
            }
            float psum = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) psum += p[r];
            l_run = l_run * alpha + psum;
            if (__any(alpha != 1.0f)) {
#pragma unroll
                for (int dt = 0; dt < NB; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            }
            m_run = m_new;

            // ---- P.V: B operand = P (lane = row, 8 keys), A operand = V^T rows
            f16x8 pk[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) pk[ks][e] = (_Float16)p[8 * ks + e];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int dt = 0; dt < NB; ++dt) {
                    const f16x8 vop = *reinterpret_cast<const f16x8 *>(
                        vt + (dt * 32 + l32) * VTS + 16 * ks + 8 * hl);
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, pk[ks], oacc[dt], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue
    if (!wave_active) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    if (!row_ok) return;
    const size_t rows_total = (size_t)a.T * a.Hq;
    const bool partial = a.part_o != nullptr;
    float *dst = partial ? a.part_o + (size_t)split * rows_total * D : a.out;
    dst += (size_t)flat * D;
#pragma unroll
    for (int dt = 0; dt < NB; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = dt * 32 + 8 * r4 + 4 * hl;
            f32x4 v = {oacc[dt][4 * r4 + 0] * inv_l, oacc[dt][4 * r4 + 1] * inv_l,
                       oacc[dt][4 * r4 + 2] * inv_l, oacc[dt][4 * r4 + 3] * inv_l};
            *reinterpret_cast<f32x4 *>(dst + d0) = v;
        }
    if (hl == 0) {
        if (partial)
            a.part_lse[(size_t)split * rows_total + flat] = lse;
        else if (a.out_lse)
            a.out_lse[flat] = lse;
    }
}

// ---------------------------------------------------------------- merge

__global__ void merge_kernel(const float *__restrict__ part_o, const float *__restrict__ part_lse,
                             int S, int rows, int D, float *__restrict__ out,
                             float *__restrict__ out_lse) {
    const int row = blockIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, part_lse[(size_t)s * rows + row]);
    float W = 0.0f;
    if (M != -INFINITY)
        for (int s = 0; s < S; ++s) W += expf(part_lse[(size_t)s * rows + row] - M);
    const float invW = W > 0.0f ? 1.0f / W : 0.0f;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float o = 0.0f;
        if (M != -INFINITY)
            for (int s = 0; s < S; ++s) {
                const float ls = part_lse[(size_t)s * rows + row];
                if (ls != -INFINITY)
                    o += expf(ls - M) * part_o[((size_t)s * rows + row) * D + d];
            }
        out[(size_t)row * D + d] = o * invW;
    }
    if (out_lse && threadIdx.x == 0) out_lse[row] = M == -INFINITY ? -INFINITY : M + logf(W);
}

template <int D, int NW, bool CAUSAL, bool DEBUG>
hipError_t launch_t(const AttnArgs &a, hipStream_t stream) {
    const int grid = a.n_hs_pad * a.NRG;
    hipLaunchKernelGGL((attn_split_kernel<D, NW, CAUSAL, DEBUG>), dim3(grid), dim3(NW * 64), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_d(const AttnArgs &a, bool causal, bool debug, hipStream_t s) {
    if (causal) return debug ? launch_t<D, NW, true, true>(a, s) : launch_t<D, NW, true, false>(a, s);
    return debug ? launch_t<D, NW, false, true>(a, s) : launch_t<D, NW, false, false>(a, s);
}

template <int D>
hipError_t launch_nw(const AttnArgs &a, int NW, bool causal, bool debug, hipStream_t s) {
    switch (NW) {
        case 1: return launch_d<D, 1>(a, causal, debug, s);
        case 2: return launch_d<D, 2>(a, causal, debug, s);
        case 4: return launch_d<D, 4>(a, causal, debug, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, int D, int NW, bool causal, bool debug,
                            hipStream_t stream) {
    switch (D) {
        case 64: return launch_nw<64>(a, NW, causal, debug, stream);
        case 128: return launch_nw<128>(a, NW, causal, debug, stream);
        case 256: return launch_nw<256>(a, NW, causal, debug, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_merge(const float *part_o, const float *part_lse, int S, int rows, int D,
                        float *out, float *out_lse, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int threads = D >= 256 ? 256 : ((D + 63) / 64) * 64;
    hipLaunchKernelGGL(merge_kernel, dim3(rows), dim3(threads), 0, stream, part_o, part_lse, S,
                       rows, D, out, out_lse);
    return hipGetLastError();
}

hipError_t launch_kv_pack(const float *x, int n_tok, int pos0, uint32_t *codes, uint16_t *scales,
                          int Hkv, int D, int cap, hipStream_t stream) {
    const long long total = (long long)n_tok * Hkv * (D / 32);
    if (total == 0) return hipSuccess;
    const int threads = 256;
    const long long blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(kv_pack_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, x, n_tok,
                       pos0, codes, scales, Hkv, D, cap);
    return hipGetLastError();
}

}  // namespace stv
