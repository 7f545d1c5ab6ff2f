// Slot-level reads and whole-page writes of the unified page (layout in include/kvc.h), shared
// by the page writers (prompt and re-tier placement, the generation step).
#pragma once

#include "kvc_internal.h"

#pragma clang fp contract(off)

namespace kvc {

typedef unsigned int pio_u2 __attribute__((ext_vector_type(2)));
typedef unsigned int pio_u4 __attribute__((ext_vector_type(4)));
// Page stores are non-temporal: a page image is written once and read back only by a later
// launch, so streaming it out keeps a prompt round's hundreds of MB from filling the caches
// with dirty lines that the next kernel would have to write back first.
__device__ __forceinline__ void st_page4(uint8_t *p, uint32_t a) {
    __builtin_nontemporal_store(a, reinterpret_cast<uint32_t *>(p));
}
__device__ __forceinline__ void st_page8(uint8_t *p, uint32_t a, uint32_t b) {
    __builtin_nontemporal_store(pio_u2{a, b}, reinterpret_cast<pio_u2 *>(p));
}
__device__ __forceinline__ void st_page16(uint8_t *p, uint32_t a, uint32_t b, uint32_t c,
                                          uint32_t d) {
    __builtin_nontemporal_store(pio_u4{a, b, c, d}, reinterpret_cast<pio_u4 *>(p));
}

__device__ __forceinline__ int k_nib(int e) { return (e & 1) + 2 * (e >> 2) + 4 * ((e >> 1) & 1); }

// codes of the lane's 8 channels 8c..8c+7 of slot `so` in an old page of tier `t`
__device__ __forceinline__ void old_codes(const uint8_t *pg, int t, int so, int c, uint32_t (&kc)[8],
                                          uint32_t (&vc)[8], uint32_t &kpar, uint32_t &vpar) {
    if (t == HIGH) {
        const uint2 kw = *reinterpret_cast<const uint2 *>(pg + K_OFF + so * 128 + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kc[e] = (kw.x >> (8 * e)) & 255u;
            kc[4 + e] = (kw.y >> (8 * e)) & 255u;
        }
    } else {
        const uint32_t kw = *reinterpret_cast<const uint32_t *>(pg + K_OFF + so * 64 + 4 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) kc[e] = (kw >> (4 * k_nib(e))) & 15u;
    }
    const int n = c >> 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int dl = 8 * (c & 1) + e;
        if (t == HIGH) {
            const int j = so >> 2, r = so & 3;
            const uint32_t w = *reinterpret_cast<const uint32_t *>(pg + V_OFF + 16 * (16 * j + dl) + 4 * (n >> 1));
            vc[e] = (w >> (4 * (2 * (n & 1) + (r >> 1) + 4 * (r & 1)))) & 15u;
        } else {
            const int f = so >> 4, j = (so & 15) >> 2, r = so & 3;
            const uint32_t w = *reinterpret_cast<const uint32_t *>(pg + V_OFF + 16 * (16 * j + dl) + 4 * (2 * f + (n >> 2)));
            vc[e] = (w >> (2 * (2 * (n & 3) + (r >> 1) + 8 * (r & 1)))) & 3u;
        }
    }
    const uint2 par = *reinterpret_cast<const uint2 *>(pg + PARAM_OFF + 8 * so);
    kpar = par.x;
    vpar = par.y;
}

// The codes of slot `so` of an old page of tier t from words already loaded: kw its key
// words (HIGH: 8 bytes, LOW: the first 4), u the 16 value units (256 B) of its unit group,
// units 16 ((so & 15) >> 2) .. + 15 of the page, staged in LDS by the slot's 16 lanes (one
// 16-byte unit each) in place of 8 scattered 4-byte loads per lane
__device__ __forceinline__ void old_codes_staged(uint2 kw, const uint4 *u, int t, int so, int c,
                                                 uint32_t (&kc)[8], uint32_t (&vc)[8]) {
    if (t == HIGH) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kc[e] = (kw.x >> (8 * e)) & 255u;
            kc[4 + e] = (kw.y >> (8 * e)) & 255u;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kc[e] = (kw.x >> (4 * k_nib(e))) & 15u;
    }
    const int n = c >> 1, r = so & 3;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t *uw = reinterpret_cast<const uint32_t *>(u + 8 * (c & 1) + e);
        if (t == HIGH) {
            vc[e] = (uw[n >> 1] >> (4 * (2 * (n & 1) + (r >> 1) + 4 * (r & 1)))) & 15u;
        } else {
            const int f = so >> 4;
            vc[e] = (uw[2 * f + (n >> 2)] >> (2 * (2 * (n & 3) + (r >> 1) + 8 * (r & 1)))) & 3u;
        }
    }
}

// fp16 rounding of a code's reconstruction code*scale + zero (one float32 rounding, then RNE)
__device__ __forceinline__ float recon16(uint32_t code, uint32_t par) {
    const float r = fmaf(float(code), h2f(uint16_t(par & 0xffffu)), h2f(uint16_t(par >> 16)));
    return h2f(f2h_rn(r));
}

// one slot's outputs: key codes straight to the page (an empty slot writes zeros), value
// codes and the four fp16 parameters to the wave's LDS staging
__device__ __forceinline__ void store_slot(uint8_t *pg, uint8_t *sv, uint16_t (*par)[4], bool high,
                                           int s, int c, bool live, uint32_t kw0, uint32_t kw1,
                                           uint32_t vw0, uint32_t vw1, uint16_t ks, uint16_t kz,
                                           uint16_t vs, uint16_t vz) {
    if (!live) kw0 = kw1 = vw0 = vw1 = 0;
    if (high) st_page8(pg + K_OFF + s * 128 + 8 * c, kw0, kw1);
    else st_page4(pg + K_OFF + s * 64 + 4 * c, kw0);
    *reinterpret_cast<uint2 *>(sv + s * D + 8 * c) = make_uint2(vw0, vw1);
    if (c == 0) {
        par[s][0] = live ? ks : 0;
        par[s][1] = live ? kz : 0;
        par[s][2] = live ? vs : 0;
        par[s][3] = live ? vz : 0;
    }
}

// value codes of a whole page from the wave's LDS staging sv[slot][channel] (one code per
// byte): lane = value unit (j, l), 16 bytes at V_OFF + 16 * lane, in the decode kernel's
// operand order
__device__ __forceinline__ void pack_values(uint8_t *pg, const uint8_t *sv, bool high, int lane) {
    const int j = lane >> 4, l = lane & 15;
    uint32_t w[4] = {0, 0, 0, 0};
    if (high) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int nn = 0; nn < 2; ++nn)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = 2 * q + nn;
                    const uint32_t code = sv[(4 * j + r) * D + 16 * n + l];
                    w[q] |= code << (4 * (2 * nn + (r >> 1) + 4 * (r & 1)));
                }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int nn = 0; nn < 4; ++nn)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int f = q >> 1, n = 4 * (q & 1) + nn;
                    const uint32_t code = sv[(16 * f + 4 * j + r) * D + 16 * n + l];
                    w[q] |= code << (2 * (2 * nn + (r >> 1) + 8 * (r & 1)));
                }
    }
    st_page16(pg + V_OFF + 16 * lane, w[0], w[1], w[2], w[3]);
}

}  // namespace kvc
