// HIP kernels for lookup drafting on gfx950: scan each request's token
// history for the latest earlier occurrence of its last tokens and propose
// the tokens that followed (u/iamMess, lookup-augmented drafting; elpis, the
// drafter-free n-gram chains).
//
// lookup_scan_kernel: one work-group per (2,048 end positions, sequence).
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
    // tail[i] = h[N-1-i]; only i <= N-2 is ever compared
    if (tid < a.n_max && tid < N) tail[tid] = h[N - 1 - tid];
    __syncthreads();
    uint64_t best = 0;
    if (N >= 2) {
        const int last = tail[0];
        const int e0 = chunk * kLookupChunk + tid;
#pragma unroll
        for (int j = 0; j < kScanPer; ++j) {
            const int e = e0 + j * kScanThreads;
            if (e <= N - 2 && h[e] == last) {
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
    best = wave_max_u64(best);
    if ((tid & 63) == 0) red[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
        uint64_t v = red[0];
        for (int w = 1; w < kScanThreads / 64; ++w) v = red[w] > v ? red[w] : v;
        a.ws[(size_t)b * a.n_chunks + chunk] = v;
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
