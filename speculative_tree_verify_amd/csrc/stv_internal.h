// Internal interface between the C-ABI host layer (stv_abi.cpp) and the HIP
// kernels (stv_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "stv.h"

namespace stv {

constexpr int kKeyTile = 32;     // keys per tile: the M side of one 32x32 MFMA
constexpr int kRowTile = 32;     // query rows per wave: the N side of one 32x32 MFMA

// Arguments of the split attention kernel.  Rows are ordered per kv head as
// rho = t * G + g (tree row t, query head h = head * G + g); the flat output
// row is t * Hq + h.
struct AttnArgs {
    const float *q;
    const uint32_t *kc;
    const uint16_t *ks;
    const uint32_t *vc;
    const uint16_t *vs;
    float *out;          // [T*Hq][D], written when part_o is NULL (then S == 1)
    float *out_lse;      // nullable [T*Hq], written when part_o is NULL
    float *part_o;       // nullable [S][T*Hq][D]: set, every split writes its partial
    float *part_lse;     // [S][T*Hq] when part_o is set
    int32_t *dbg_logits; // nullable [T*Hq][N][D/32]
    int8_t *dbg_q;       // nullable [T*Hq][D]
    float *dbg_qscale;   // nullable [T*Hq]
    int32_t T, Hq, Hkv, G, cap, ngroups, L, N, R;
    int32_t S, split_len, NRG, n_hs_pad;
    float scale_log2;    // softmax_scale * log2(e)
    const unsigned char *img;  // unpacked tile images [Hkv][img_tiles] (causal chunk), or NULL
    int32_t img_tiles;         // ceil(N / 32): images per KV head
    uint64_t mask[64];   // verify only: ancestor masks of the tree rows
};

// Query rows per KV head up to which the few-row kernel (16-row MFMA tiles,
// per-wave key tiles, one work-group per group of 16 rows) runs instead of
// the 32-row tile kernel.
constexpr int kDecMaxRows = 16;
// The same for the 4-bit format, whose cheaper unpack and one-scale-per-key
// epilogue make a separate unpack per 16-row group pay (the 8-row tree:
// 48 rows).
constexpr int kDecMaxRows4 = 64;
// Query rows per KV head up to which the 16-row shared-tile kernel runs for
// the 3-bit format (above the few-row kernel's range); above it, and for the
// 4-bit format above kDecMaxRows4, the 32-row tile kernel.
constexpr int kS16MaxRows = 64;

// The wave-specialized 32-row kernel (3-bit verify rows at head_dim 256, four
// row tiles per work-group): twelve waves, one work-group per CU.
constexpr int kWsThreads = 768;
// Fixed cost of one round of its work-groups, in tile steps (measured: the
// 64-node tree over 32K and 262K keys).
constexpr int kWsRoundTiles = 12;

struct Plan {
    bool dec;        // few-row kernel (then NW = 4 waves and NRG groups of 16 rows)
    bool s16;        // 16-row shared-tile kernel (then NW = 4 waves and NRG groups of 64 rows)
    bool ws;         // wave-specialized 32-row kernel (3-bit, head_dim 256, NW = 4, verify rows)
    int NW;          // waves (32-row tiles) per work-group
    int NRG;         // row groups per kv head
    int S;           // context splits
    int split_len;   // keys per split, a multiple of kKeyTile
    size_t ws_bytes; // workspace of the call: the partials, then the tile images when pre is set
    size_t part_bytes;   // the partials alone (the least workspace the call accepts)
    bool pre;            // the causal chunk with many row groups: unpack each tile once into
                         // images in the workspace (used when the workspace holds them)
    size_t img_offset;   // where the images start in the workspace
};

// Row groups per KV head from which a causal chunk unpacks its tiles once, in
// a pre-pass, instead of in every row group.
constexpr int kPreMinRowGroups = 8;

// Work-groups of the attention kernels that fit on one CU at once, from the
// runtime's occupancy calculator; 0 when no device answers.
// fmt: 0 = 3-bit codes with per-32-element scales, 1 = 4-bit codes with
// per-token-head scales.
int attention_wgs_per_cu(int D, int NW, bool causal, int fmt);
int attention_dec_wgs_per_cu(int D, bool causal, int fmt);
int attention_s16_wgs_per_cu(int D, bool causal);     // 3-bit format
int attention_ws_wgs_per_cu(int D);                   // 3-bit format, verify rows

// Resident work-group slots of the current device for a kernel variant
// (CUs x work-groups per CU); a fixed MI355X figure when no device answers.
// kind: 0 = 32-row tile kernel, 1 = few-row kernel, 2 = 16-row shared-tile kernel,
// 3 = wave-specialized 32-row kernel.
long long attention_slots(int D, int NW, bool causal, int kind, int fmt);

Plan make_plan(int T, int Hq, int Hkv, int D, int L, bool causal, int n_splits_req, int fmt);

// Launchers return the hipError_t of the launch.  pv16 selects the
// fp16-accumulated P.V variant (3-bit format, verify rows, no debug output;
// anything else with pv16 set is hipErrorInvalidValue).
hipError_t launch_attention(const AttnArgs &a, int D, int NW, bool causal, bool debug, int fmt,
                            bool pv16, hipStream_t stream);
hipError_t launch_attention_dec(const AttnArgs &a, int D, bool causal, bool debug, bool pv16,
                                int fmt, hipStream_t stream);
hipError_t launch_attention_s16(const AttnArgs &a, int D, bool causal, bool debug, bool pv16,
                                hipStream_t stream);   // 3-bit format
// Bytes of the device array that holds the split partials of
// stv_verify_attention_noalloc (one per device), and its device address for
// the current device (resolved once per device; NULL with *err set when the
// runtime cannot resolve it).
constexpr size_t kNoAllocScratchBytes = STV_NOALLOC_SCRATCH_BYTES;
void *noalloc_scratch(hipError_t *err);

// The pre-pass: images of tiles 0 .. a.img_tiles - 1 of every KV head into img.
hipError_t launch_tile_images(const AttnArgs &a, int D, int fmt, unsigned char *img, hipStream_t s);
size_t tile_image_bytes(int D);
hipError_t launch_merge(const float *part_o, const float *part_lse, int S, int rows, int D,
                        float *out, float *out_lse, hipStream_t stream);
hipError_t launch_kv_pack(const float *x, int n_tok, int pos0, uint32_t *codes,
                          uint16_t *scales, int Hkv, int D, int cap, bool is_v,
                          hipStream_t stream);
hipError_t launch_kv_pack4(const float *x, int n_tok, int pos0, uint32_t *codes,
                           uint16_t *scales, int Hkv, int D, int cap, bool is_v,
                           hipStream_t stream);

}  // namespace stv
