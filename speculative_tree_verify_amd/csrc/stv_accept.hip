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
// kv_commit_kernel: one work-group per KV head.  Phase 1 reads every
//   committed source token (K blocks, K scales, V scales into LDS; V codes
//   of row d by thread d into LDS); after one barrier, phase 2 writes them
//   to positions L, L+1, ...  A thread owns V row d across all groups, so
//   its read-modify-writes of 3-bit fields never race.
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

__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(const CommitArgs a) {
    __shared__ uint32_t kbuf[64 * kMaxNb][3];
    __shared__ uint16_t kscale[64 * kMaxNb];
    __shared__ uint16_t vscale[64 * kMaxNb];
    __shared__ uint8_t vcode[kCommitThreads][64];
    __shared__ int src_pos[64];

    const int g = blockIdx.x;
    const int tid = threadIdx.x;
    const int NB = a.D / 32;
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
    // ---- phase 1: read every source
    for (int it = tid; it < n * NB; it += kCommitThreads) {
        const int j = it / NB, b = it - (it / NB) * NB;
        const int src = src_pos[j];
        const size_t blk = (head_k + src) * NB + b;
        kbuf[it][0] = a.kc[blk * 3 + 0];
        kbuf[it][1] = a.kc[blk * 3 + 1];
        kbuf[it][2] = a.kc[blk * 3 + 2];
        kscale[it] = a.ks[blk];
        vscale[it] = a.vs[((head_v + src / 32) * NB + b) * 32 + src % 32];
    }
    if (tid < a.D) {
        const int d = tid;
        for (int j = 0; j < n; ++j) {
            const int src = src_pos[j];
            const uint32_t *w = a.vc + ((head_v + src / 32) * a.D + d) * 3;
            vcode[d][j] = (uint8_t)get_code(w[0], w[1], w[2], src % 32);
        }
    }
    __syncthreads();
    // ---- phase 2: write positions L .. L + n - 1
    for (int it = tid; it < n * NB; it += kCommitThreads) {
        const int j = it / NB, b = it - (it / NB) * NB;
        const int dst = a.L + j;
        const size_t blk = (head_k + dst) * NB + b;
        a.kc[blk * 3 + 0] = kbuf[it][0];
        a.kc[blk * 3 + 1] = kbuf[it][1];
        a.kc[blk * 3 + 2] = kbuf[it][2];
        a.ks[blk] = kscale[it];
        a.vs[((head_v + dst / 32) * NB + b) * 32 + dst % 32] = vscale[it];
    }
    if (tid < a.D) {
        const int d = tid;
        const int g0 = a.L / 32, g1 = (a.L + n - 1) / 32;
        for (int grp = g0; grp <= g1; ++grp) {
            uint32_t *w = a.vc + ((head_v + grp) * a.D + d) * 3;
            uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
            const int j0 = max(0, grp * 32 - a.L), j1 = min(n, grp * 32 + 32 - a.L);
            for (int j = j0; j < j1; ++j) set_code(w0, w1, w2, (a.L + j) % 32, vcode[d][j]);
            w[0] = w0;
            w[1] = w1;
            w[2] = w2;
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
    hipLaunchKernelGGL(kv_commit_kernel, dim3(a.Hkv), dim3(kCommitThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace stv
