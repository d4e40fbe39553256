// HIP kernels for lookup drafting on gfx950: scan each request's token
// history for the latest earlier occurrence of its last tokens and propose
// the tokens that followed (u/iamMess, lookup-augmented drafting; elpis, the
// drafter-free n-gram chains).
//
// lookup_scan_kernel: one work-group per (4,096 end positions, sequence).
//   Coalesced loads of h[e]; only positions whose token equals the last
//   token extend the comparison backwards (a rare, divergent path), so the
//   scan streams the history at HBM speed.  The candidate key
//   (match length << 32 | e) is max-reduced over the work-group: the longest
//   match wins, then the largest e.
// lookup_finalize_kernel: one wave per sequence reduces the chunk keys in
//   the workspace and gathers the proposed tokens.
#include "stv_lookup.h"

namespace stv {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanPer = kLookupChunk / kScanThreads;

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t w = __shfl_xor(v, o);
        v = w > v ? w : v;
    }
    return v;
}

__device__ __forceinline__ int clamp_len(int n, int stride) {
    return n < 0 ? 0 : (n > stride ? stride : n);
}

__global__ __launch_bounds__(kScanThreads) void lookup_scan_kernel(const LookupArgs a) {
    __shared__ int32_t tail[kLookupMaxN];
    __shared__ uint64_t red[kScanThreads / 64];
    const int b = blockIdx.y;
    const int chunk = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t *h = a.hist + (size_t)b * a.stride;
    const int N = clamp_len(a.len[b], a.stride);
    // Thread tid covers positions c0 + 4*(tid + 256 j) + [0, 4): one 16-byte
    // load per four positions when every row starts 16-byte aligned (checked
    // on the host), else four 4-byte loads.  All of them are issued before
    // the tail is read, so the chunk's loads overlap the tail's latency.
    // Positions past N - 2 hold a token that cannot match (fixed below).
    constexpr int J = kScanPer / 4;
    const int c0 = chunk * kLookupChunk;
    int v[J][4];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e4 = c0 + 4 * (tid + j * kScanThreads);
        if (a.vec16 && e4 + 3 <= N - 2) {
            const int4 q = *reinterpret_cast<const int4 *>(h + e4);
            v[j][0] = q.x;
            v[j][1] = q.y;
            v[j][2] = q.z;
            v[j][3] = q.w;
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[j][u] = e4 + u <= N - 2 ? h[e4 + u] : 0;
        }
    }
    // tail[i] = h[N-1-i]; only i <= N-2 is ever compared
    if (tid < a.n_max && tid < N) tail[tid] = h[N - 1 - tid];
    __syncthreads();
    uint64_t best = 0;
    if (N >= 2) {
        const int last = tail[0];
#pragma unroll
        for (int j = 0; j < J; ++j) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = c0 + 4 * (tid + j * kScanThreads) + u;
                if (v[j][u] == last && e <= N - 2) {
                    const int cap = min(a.n_max, e + 1);
                    int m = 1;
                    while (m < cap && h[e - m] == tail[m]) ++m;
                    if (m >= a.n_min) {
                        const uint64_t key = ((uint64_t)m << 32) | (uint32_t)e;
                        best = key > best ? key : best;
                    }
                }
            }
        }
    }
    best = wave_max_u64(best);
    if ((tid & 63) == 0) red[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
        uint64_t w = red[0];
        for (int i = 1; i < kScanThreads / 64; ++i) w = red[i] > w ? red[i] : w;
        a.ws[(size_t)b * a.n_chunks + chunk] = w;
    }
}

__global__ __launch_bounds__(64) void lookup_finalize_kernel(const LookupArgs a) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t *h = a.hist + (size_t)b * a.stride;
    const int N = clamp_len(a.len[b], a.stride);
    uint64_t key = 0;
    for (int c = lane; c < a.n_chunks; c += 64) {
        const uint64_t v = a.ws[(size_t)b * a.n_chunks + c];
        key = v > key ? v : key;
    }
    key = wave_max_u64(key);
    const bool found = key != 0;          // a candidate has match >= n_min >= 1
    const int m = (int)(key >> 32);
    const int e = (int)(uint32_t)key;
    const int cnt = found ? min(a.k, N - 1 - e) : 0;
    for (int j = lane; j < a.k; j += 64)
        a.tokens[(size_t)b * a.k + j] = j < cnt ? h[e + 1 + j] : -1;
    if (lane == 0) {
        a.count[b] = cnt;
        a.match[b] = found ? m : 0;
        a.pos[b] = found ? e : -1;
    }
}

}  // namespace

hipError_t launch_lookup(const LookupArgs &a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    hipLaunchKernelGGL(lookup_scan_kernel, dim3(a.n_chunks, a.B), dim3(kScanThreads), 0, stream,
                       a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lookup_finalize_kernel, dim3(a.B), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace stv
