// Internal interface of the lookup-drafting kernels (not part of the
// public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace stv {

constexpr int kLookupChunk = 4096;      // end positions per scan work-group
constexpr int kLookupMaxN = 64;         // largest n_max

struct LookupArgs {
    const int32_t *hist;    // [B][stride]
    const int32_t *len;     // [B], clamped to [0, stride] on the device
    int B, stride, n_min, n_max, k, n_chunks;
    bool vec16;             // every row starts on a 16-byte boundary
    uint64_t *ws;           // [B][n_chunks] best (match << 32 | end) per chunk
    int32_t *tokens;        // [B][k]
    int32_t *count, *match, *pos;   // [B]
};

inline int lookup_chunks(int stride) {
    const int ends = stride > 1 ? stride - 1 : 1;
    return (ends + kLookupChunk - 1) / kLookupChunk;
}

hipError_t launch_lookup(const LookupArgs &a, hipStream_t stream);

}  // namespace stv
