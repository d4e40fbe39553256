// Internal interface of the acceptance and commit kernels (not part of the
// public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stv {

struct AcceptArgs {
    uint64_t mask[64];          // ancestor masks, validated on the host
    int T;
    const int32_t *draft;       // [T]
    const int32_t *target;      // [T]
    int32_t *path;              // [T] out
    int32_t *n_accepted;        // [1] out
    int32_t *bonus;             // [1] out
};

struct CommitArgs {
    uint32_t *kc;
    uint16_t *ks;
    uint32_t *vc;
    uint16_t *vs;
    int Hkv, D, cap, ngroups;
    int fmt;                    // 0 = 3-bit blocks, 1 = 4-bit per-token-head
    int L, T;
    const int32_t *path;        // [T] device
    const int32_t *n_accepted;  // [1] device
};

hipError_t launch_tree_accept(const AcceptArgs &a, hipStream_t stream);
hipError_t launch_kv_commit(const CommitArgs &a, hipStream_t stream);

}  // namespace stv
