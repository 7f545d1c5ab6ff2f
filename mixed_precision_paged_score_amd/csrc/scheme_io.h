// Slot-level reads and writes of precision-scheme pages, shared by the scheme page writers
// (prompt and re-tier placement), the scheme append and the scheme generation step.
//
// Layout (this project's own, include/kvc.h): keys slot-major, slot s's 128 codes of kb bits
// at bytes [16 kb s, 16 kb (s + 1)), code i at bits [i kb, (i + 1) kb); values from byte
// 16 kb S (S = 16 HIGH or 32 LOW slots) in blocks of 16 slots, 256 vb bytes each: lane
// L = 16 g + c of block f owns bytes [4 vb L, 4 vb (L + 1)), the codes of channels 16 n + c
// (n < 8) of slots 16 f + 4 g + r (r < 4), code (n, r) at bit
// 32 (n / p) + 16 (r % 2) + vb (2 (n % p) + r / 2), p = 8 / vb; parameters and positions at the
// default layout's offsets.
#pragma once

#include "kvc_internal.h"
#include "page_io.h"

namespace kvc {

// the lane's 8 codes (b bits each, channels 8c .. 8c + 7) as b bytes at dst (b = 1, 2, 4, 8:
// naturally aligned stores)
__device__ __forceinline__ void store_codes(uint8_t *dst, uint64_t w, int b) {
    if (b == 8) st_page8(dst, uint32_t(w), uint32_t(w >> 32));
    else if (b == 4) st_page4(dst, uint32_t(w));
    else if (b == 2) *reinterpret_cast<uint16_t *>(dst) = uint16_t(w);
    else *dst = uint8_t(w);
}

// one lane's share of a value block (16 slots) in the decode's operand order: lane L = 16 g + c
// packs the codes of channels 16 n + c (n < 8) for slots 16 f + 4 g + r (r < 4), code (n, r)
// at bit 32 (n / p) + 16 (r % 2) + VB (2 (n % p) + r / 2) with p = 8 / VB, and stores its
// 4 VB bytes at dst (naturally aligned)
template <int VB>
__device__ __forceinline__ void pack_value_block(uint8_t *dst, const uint8_t (*vc)[D], int f,
                                                 int g, int c) {
    constexpr int P = 8 / VB;
    uint32_t w[VB];
#pragma unroll
    for (int j = 0; j < VB; ++j) w[j] = 0u;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t code = vc[16 * f + 4 * g + r][16 * n + c];
            w[n / P] |= code << (16 * (r & 1) + VB * (2 * (n % P) + (r >> 1)));
        }
    if constexpr (VB == 8) {
        st_page16(dst, w[0], w[1], w[2], w[3]);
        st_page16(dst + 16, w[4], w[5], w[6], w[7]);
    } else if constexpr (VB == 4) {
        st_page16(dst, w[0], w[1], w[2], w[3]);
    } else if constexpr (VB == 2) {
        st_page8(dst, w[0], w[1]);
    } else {
        st_page4(dst, w[0]);
    }
}

// bit offset, within a value lane's 4 vb bytes, of code (n, r); p = 8 / vb
__device__ __forceinline__ int sch_vbit(int vb, int n, int r) {
    const int lp = vb == 8 ? 0 : vb == 4 ? 1 : vb == 2 ? 2 : 3;      // log2(8 / vb)
    return 32 * (n >> lp) + 16 * (r & 1) + vb * (2 * (n & ((1 << lp) - 1)) + (r >> 1));
}

// the value lane of (slot s, channel group c) in a page of S slots: its byte offset
__device__ __forceinline__ int sch_vlane_off(int kb, int vb, int S, int s, int c) {
    const int f = s >> 4, g = (s & 15) >> 2;
    return 16 * kb * S + 256 * vb * f + 4 * vb * (16 * g + c);
}

// the 4 vb bytes of a value lane as 32-bit words (w[k] for k < vb)
__device__ __forceinline__ void sch_vlane_load(const uint8_t *src, int vb, uint32_t (&w)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = 0u;
    if (vb == 8) {
        const uint4 a = *reinterpret_cast<const uint4 *>(src);
        const uint4 b = *reinterpret_cast<const uint4 *>(src + 16);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if (vb == 4) {
        const uint4 a = *reinterpret_cast<const uint4 *>(src);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else if (vb == 2) {
        const uint2 a = *reinterpret_cast<const uint2 *>(src);
        w[0] = a.x; w[1] = a.y;
    } else {
        w[0] = *reinterpret_cast<const uint32_t *>(src);
    }
}
__device__ __forceinline__ void sch_vlane_store(uint8_t *dst, int vb, const uint32_t (&w)[8]) {
    if (vb == 8) {
        *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint4 *>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
    } else if (vb == 4) {
        *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if (vb == 2) {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
    } else {
        *reinterpret_cast<uint32_t *>(dst) = w[0];
    }
}

// slot s's key codes of channels 8c .. 8c + 7 (kb bits each)
__device__ __forceinline__ void sch_key_codes(const uint8_t *pg, int kb, int s, int c,
                                              uint32_t (&kc)[8]) {
    const uint8_t *src = pg + 16 * kb * s + c * kb;
    uint64_t w;
    if (kb == 8) w = *reinterpret_cast<const uint64_t *>(src);
    else if (kb == 4) w = *reinterpret_cast<const uint32_t *>(src);
    else if (kb == 2) w = *reinterpret_cast<const uint16_t *>(src);
    else w = *src;
    const uint32_t mask = (1u << kb) - 1u;
#pragma unroll
    for (int e = 0; e < 8; ++e) kc[e] = uint32_t(w >> (kb * e)) & mask;
}

// slot s's value codes of channels 16 n + c (n < 8), in a page of S slots
__device__ __forceinline__ void sch_val_codes(const uint8_t *pg, int kb, int vb, int S, int s,
                                              int c, uint32_t (&vc)[8]) {
    uint32_t w[8];
    sch_vlane_load(pg + sch_vlane_off(kb, vb, S, s, c), vb, w);
    const int r = s & 3;
    const uint32_t mask = (1u << vb) - 1u;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int bit = sch_vbit(vb, n, r);
        vc[n] = (w[bit >> 5] >> (bit & 31)) & mask;
    }
}

// writes slot s's value codes of channels 16 n + c (n < 8) into its lane's words, the other
// slots' codes kept (fresh: the page was just cleared, nothing to read)
__device__ __forceinline__ void sch_set_val_codes(uint8_t *pg, int kb, int vb, int S, int s,
                                                  int c, const uint32_t (&vc)[8], bool fresh) {
    uint8_t *dst = pg + sch_vlane_off(kb, vb, S, s, c);
    uint32_t w[8];
    if (fresh) {
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = 0u;
    } else {
        sch_vlane_load(dst, vb, w);
    }
    const int r = s & 3;
    const uint32_t mask = (1u << vb) - 1u;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int bit = sch_vbit(vb, n, r);
        w[bit >> 5] = (w[bit >> 5] & ~(mask << (bit & 31))) | ((vc[n] & mask) << (bit & 31));
    }
    sch_vlane_store(dst, vb, w);
}

}  // namespace kvc
