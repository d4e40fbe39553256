// Device helpers for the 3-bit block layout shared by the HIP sources:
// 32 codes c in [0, 7] in three 32-bit words, "byte-plane" order.  Element
// e = 4*qq + i (qq = e / 4, i = e % 4):
//   qq = 0,1 : word 0, bits [8i + 3qq, +3)
//   qq = 2,3 : word 1, bits [8i + 3(qq-2), +3)
//   qq = 4,5 : word 2, bits [8i + 3(qq-4), +3)
//   qq = 6   : code bits 0-1 at word 0 bits [8i+6, +2), bit 2 at word 2 bit 8i+6
//   qq = 7   : code bits 0-1 at word 1 bits [8i+6, +2), bit 2 at word 2 bit 8i+7
// so one byte of each word holds parts of the codes of elements 4qq + i.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stv {

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

// Set element e's code in a three-word block (byte-plane layout).
__device__ __forceinline__ void set_code(uint32_t &w0, uint32_t &w1, uint32_t &w2, int e,
                                         uint32_t c) {
    const int qq = e >> 2, i = e & 3;
    if (qq < 6) {
        const int sh = 8 * i + 3 * (qq & 1);
        const uint32_t m = 7u << sh;
        uint32_t &w = qq < 2 ? w0 : (qq < 4 ? w1 : w2);
        w = (w & ~m) | (c << sh);
    } else {
        const int sh = 8 * i + 6;
        uint32_t &w = qq == 6 ? w0 : w1;
        w = (w & ~(3u << sh)) | ((c & 3u) << sh);
        const int hb = 8 * i + 6 + (qq - 6);
        w2 = (w2 & ~(1u << hb)) | ((c >> 2) << hb);
    }
}

// Code of element e of a three-word block.
__device__ __forceinline__ uint32_t get_code(uint32_t w0, uint32_t w1, uint32_t w2, int e) {
    const int qq = e >> 2, i = e & 3;
    if (qq < 6) {
        const uint32_t w = qq < 2 ? w0 : (qq < 4 ? w1 : w2);
        return (w >> (8 * i + 3 * (qq & 1))) & 7u;
    }
    const uint32_t lo = ((qq == 6 ? w0 : w1) >> (8 * i + 6)) & 3u;
    const uint32_t hi = (w2 >> (8 * i + 6 + (qq - 6))) & 1u;
    return lo | (hi << 2);
}

}  // namespace stv
