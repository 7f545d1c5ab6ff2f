// The per-token quantizer shared by the page writers: one 128-channel key or value row per
// 16-lane group, 8 channels per lane (one 128-bit load).  float32 with round-to-nearest-even
// and no contraction: s = fp16(fl(fl(max - min) / (2^b - 1))) (2^-24 if that rounds to 0
// while max > min), z = min (+0 for -0), code = min(rint(fl(fl(x - z) * fl(1/s))), 2^b - 1).
#pragma once

#include "kvc_internal.h"

#pragma clang fp contract(off)

namespace kvc {

struct RowQ {
    float z, inv, lq;
    uint16_t s16, z16;
};

__device__ __forceinline__ RowQ row_params(const float (&x)[8], float lq) {
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
        mn = fminf(mn, x[e]);
        mx = fmaxf(mx, x[e]);
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m, 64));
        mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    }
    RowQ q;
    const float rng = mx - mn;
    const float s32 = rng / lq;                   // correctly rounded float32 division
    uint16_t s16 = f2h_rn(s32);
    if (s16 == 0 && mx > mn) s16 = 1;             // smallest fp16 subnormal, 2^-24
    const float sf = h2f(s16);
    q.inv = sf > 0.0f ? 1.0f / sf : 0.0f;
    q.z = mn + 0.0f;                              // a -0 minimum is stored as +0
    q.z16 = f2h_rn(q.z);
    q.s16 = s16;
    q.lq = lq;
    return q;
}

__device__ __forceinline__ uint32_t code_of(float x, const RowQ &q) {
    const float d = x - q.z;
    const float y = d * q.inv;
    return uint32_t(fminf(rintf(y), q.lq));
}

__device__ __forceinline__ void load_row8(const uint16_t *src, bool live, float (&x)[8]) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (live) u = *reinterpret_cast<const uint4 *>(src);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = h2f(uint16_t(w[e] & 0xffffu));
        x[2 * e + 1] = h2f(uint16_t(w[e] >> 16));
    }
}

}  // namespace kvc
