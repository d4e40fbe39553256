// HIP kernels for the end of a verify round on gfx950: greedy acceptance over
// the token tree and the commit of the accepted path's 3-bit K/V.
//
// Method (elpis, "Why fast": an 8-row token tree whose longest matching path
// is committed plus one token; elpis-lossless, "How" and "Lossless": token
// ids compared exactly, only committed tokens stay in the cache).
//
// tree_accept_kernel: one wave, lane i = tree node i.  A node matches when
//   its draft token equals the target's token at its parent row; the wave
//   ballots the matches, so node i is acceptable when its ancestor mask
//   holds no unmatched node.  The deepest acceptable node (lowest index among
//   equals) ends the path; each lane on it writes its own position in the
//   path, given by a popcount of the lower path bits.
// kv_commit_kernel: one work-group per KV head, for either cache format.
//   Phase 1 reads every committed source token (K code words, K and V
//   scales into LDS; V codes of row d by thread d into LDS); after one
//   barrier, phase 2 writes them to positions L, L+1, ...  A thread owns V
//   row d across all groups, so its read-modify-writes of 3- or 4-bit fields
//   never race.
#include "stv_accept.h"
#include "stv_codes.h"

namespace stv {
namespace {

__global__ __launch_bounds__(64) void tree_accept_kernel(const AcceptArgs a) {
    const int i = threadIdx.x;
    const bool node = i < a.T;
    const uint64_t m = node ? a.mask[i] : 0ull;
    const uint64_t others = m & ~(1ull << i);
    const int parent = others ? 63 - __clzll((long long)others) : -1;
    bool matched = false;
    if (node) matched = i == 0 || (parent >= 0 && a.draft[i] == a.target[parent]);
    const uint64_t matched_mask = __ballot(matched);
    const bool ok = node && (m & 1ull) && (m & ~matched_mask) == 0ull;
    // deepest first, then the lowest index: key = depth * 256 + (255 - i)
    int key = ok ? (__popcll(m) << 8) | (255 - i) : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o));
    const int best = key ? 255 - (key & 255) : 0;   // node 0 is always acceptable
    const uint64_t pm = a.mask[best];
    const int n = __popcll(pm);
    if (node) {
        if ((pm >> i) & 1ull) a.path[__popcll(pm & ((1ull << i) - 1ull))] = i;
        if (i >= n) a.path[i] = -1;
    }
    if (i == 0) {
        *a.n_accepted = n;
        *a.bonus = a.target[best];
    }
}

constexpr int kCommitThreads = 256;
constexpr int kMaxNb = 8;               // D <= 256

// FMT 0: 3-bit blocks (K [cap][D/32][3] + scales [cap][D/32]; V key-
// transposed 3-bit rows + scales [ng][D/32][32]).  FMT 1: 4-bit per-token-head
// (K [cap][D/8] + scale [cap]; V key-transposed nibble rows [ng][D][4] +
// scale [cap]).  K words per key: NB*3 or D/8; at most 32 for D <= 256.
template <int FMT>
__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(const CommitArgs a) {
    constexpr int kMaxKWords = 32;
    __shared__ uint32_t kbuf[64][kMaxKWords];
    __shared__ uint16_t kscale[64][kMaxNb];
    __shared__ uint16_t vscale[64][kMaxNb];
    __shared__ uint8_t vcode[kCommitThreads][64];
    __shared__ int src_pos[64];

    const int g = blockIdx.x;
    const int tid = threadIdx.x;
    const int NB = a.D / 32;
    const int kwords = FMT == 0 ? NB * 3 : a.D / 8;     // K code words per key
    const int nsc = FMT == 0 ? NB : 1;                   // scales per key (K and V)
    // The path and count come from device memory: a malformed pair (count
    // outside [1, T] or a node outside [0, T)) leaves the cache untouched.
    const int n = *a.n_accepted;
    if (n < 1 || n > a.T) return;
    bool bad = false;
    for (int j = 0; j < n; ++j) {
        const int p = a.path[j];
        bad |= p < 0 || p >= a.T;
    }
    if (bad) return;
    if (tid < n) src_pos[tid] = a.L + a.path[tid];
    __syncthreads();

    const size_t head_k = (size_t)g * a.cap;
    const size_t head_v = (size_t)g * a.ngroups;
    auto vscale_at = [&](int pos, int b) -> size_t {
        return FMT == 0 ? ((head_v + pos / 32) * NB + b) * 32 + pos % 32 : head_k + pos;
    };
    // ---- phase 1: read every source
    for (int it = tid; it < n * kwords; it += kCommitThreads) {
        const int j = it / kwords, w = it - (it / kwords) * kwords;
        kbuf[j][w] = a.kc[(head_k + src_pos[j]) * kwords + w];
    }
    for (int it = tid; it < n * nsc; it += kCommitThreads) {
        const int j = it / nsc, b = it - (it / nsc) * nsc;
        kscale[j][b] = a.ks[(head_k + src_pos[j]) * nsc + b];
        vscale[j][b] = a.vs[vscale_at(src_pos[j], b)];
    }
    if (tid < a.D) {
        const int d = tid;
        for (int j = 0; j < n; ++j) {
            const int src = src_pos[j];
            if constexpr (FMT == 0) {
                const uint32_t *w = a.vc + ((head_v + src / 32) * a.D + d) * 3;
                vcode[d][j] = (uint8_t)get_code(w[0], w[1], w[2], src % 32);
            } else {
                const uint32_t *w = a.vc + ((head_v + src / 32) * a.D + d) * 4;
                const int e = src % 32;
                vcode[d][j] = (uint8_t)((w[e / 8] >> (4 * (e % 8))) & 15u);
            }
        }
    }
    __syncthreads();
    // ---- phase 2: write positions L .. L + n - 1
    for (int it = tid; it < n * kwords; it += kCommitThreads) {
        const int j = it / kwords, w = it - (it / kwords) * kwords;
        a.kc[(head_k + a.L + j) * kwords + w] = kbuf[j][w];
    }
    for (int it = tid; it < n * nsc; it += kCommitThreads) {
        const int j = it / nsc, b = it - (it / nsc) * nsc;
        a.ks[(head_k + a.L + j) * nsc + b] = kscale[j][b];
        a.vs[vscale_at(a.L + j, b)] = vscale[j][b];
    }
    if (tid < a.D) {
        const int d = tid;
        const int g0 = a.L / 32, g1 = (a.L + n - 1) / 32;
        for (int grp = g0; grp <= g1; ++grp) {
            const int j0 = max(0, grp * 32 - a.L), j1 = min(n, grp * 32 + 32 - a.L);
            if constexpr (FMT == 0) {
                uint32_t *w = a.vc + ((head_v + grp) * a.D + d) * 3;
                uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
                for (int j = j0; j < j1; ++j) set_code(w0, w1, w2, (a.L + j) % 32, vcode[d][j]);
                w[0] = w0;
                w[1] = w1;
                w[2] = w2;
            } else {
                uint32_t *w = a.vc + ((head_v + grp) * a.D + d) * 4;
                uint32_t ww[4] = {w[0], w[1], w[2], w[3]};
                for (int j = j0; j < j1; ++j) {
                    const int e = (a.L + j) % 32;
                    ww[e / 8] = (ww[e / 8] & ~(15u << (4 * (e % 8)))) |
                                ((uint32_t)vcode[d][j] << (4 * (e % 8)));
                }
                w[0] = ww[0];
                w[1] = ww[1];
                w[2] = ww[2];
                w[3] = ww[3];
            }
        }
    }
}

}  // namespace

hipError_t launch_tree_accept(const AcceptArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(tree_accept_kernel, dim3(1), dim3(64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_kv_commit(const CommitArgs &a, hipStream_t stream) {
    if (a.D > kMaxNb * 32 || a.D > kCommitThreads || a.T > 64) return hipErrorInvalidValue;
    if (a.fmt == 1)
        hipLaunchKernelGGL(kv_commit_kernel<1>, dim3(a.Hkv), dim3(kCommitThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(kv_commit_kernel<0>, dim3(a.Hkv), dim3(kCommitThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace stv
