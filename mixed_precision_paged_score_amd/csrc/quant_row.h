// The per-token quantizer shared by the page writers: one 128-channel key or value row per
// 16-lane group, 8 channels per lane (one 128-bit load).  float32 with round-to-nearest-even
// and no contraction: s = fp16(fl(fl(max - min) / (2^b - 1))) (2^-24 if that rounds to 0
// while max > min), z = min (+0 for -0), code = min(rint(fl(fl(x - z) * fl(1/s))), 2^b - 1),
// with every fl() correctly rounded.
#pragma once

#include "kvc_internal.h"

#pragma clang fp contract(off)

namespace kvc {

struct RowQ {
    float z, inv, lq;
    uint16_t s16, z16;
};

// min and max over the 16 lanes of each row of the wave (lanes 16 r .. 16 r + 15; the whole
// row must be active): four steps within the row (quad xor 1, quad xor 2, half-row mirror,
// row mirror), each one v_min_f32 / v_max_f32 reading its first operand through a DPP
// permute.  The s_nop gives the two wait states a DPP read needs after a VALU write of its
// source.
#define KVC_ROW_STEP(op, x, ctrl) \
    asm("s_nop 1\n\t" op "_dpp %0, %0, %0 " ctrl " row_mask:0xf bank_mask:0xf" : "+v"(x))
__device__ __forceinline__ void row_minmax16(float &mn, float &mx) {
    KVC_ROW_STEP("v_min_f32", mn, "quad_perm:[1,0,3,2]");
    KVC_ROW_STEP("v_max_f32", mx, "quad_perm:[1,0,3,2]");
    KVC_ROW_STEP("v_min_f32", mn, "quad_perm:[2,3,0,1]");
    KVC_ROW_STEP("v_max_f32", mx, "quad_perm:[2,3,0,1]");
    KVC_ROW_STEP("v_min_f32", mn, "row_half_mirror");
    KVC_ROW_STEP("v_max_f32", mx, "row_half_mirror");
    KVC_ROW_STEP("v_min_f32", mn, "row_mirror");
    KVC_ROW_STEP("v_max_f32", mx, "row_mirror");
}
#undef KVC_ROW_STEP

// x / d, correctly rounded, for d in {1, 3, 15, 255} and x >= 0 finite: q0 = x * RN(1/d), then
// one FMA correction of the remainder (checked exhaustively against IEEE division for every
// positive finite float x and each d)
__device__ __forceinline__ float div_levels(float x, float d) {
    const float c = d == 255.0f ? 1.0f / 255.0f : d == 15.0f ? 1.0f / 15.0f
                  : d == 3.0f ? 1.0f / 3.0f : 1.0f;
    if (d != 1.0f && d != 3.0f && d != 15.0f && d != 255.0f) return x / d;
    const float q0 = x * c;
    const float r = fmaf(-q0, d, x);
    return fmaf(r, c, q0);
}

// 1 / y, correctly rounded, for y a positive finite fp16 value: the hardware reciprocal and
// one Newton step with FMAs (exact for every such y from any seed within 2 ulp; the
// instruction's seed is within 1 ulp)
__device__ __forceinline__ float rcp_half(float y) {
    const float r0 = __builtin_amdgcn_rcpf(y);
    const float e = fmaf(-y, r0, 1.0f);
    return fmaf(e, r0, r0);
}

__device__ __forceinline__ RowQ row_params(const float (&x)[8], float lq) {
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
        mn = fminf(mn, x[e]);
        mx = fmaxf(mx, x[e]);
    }
    row_minmax16(mn, mx);
    RowQ q;
    const float rng = mx - mn;
    const float s32 = div_levels(rng, lq);        // = rng / lq, correctly rounded
    uint16_t s16 = f2h_rn(s32);
    if (s16 == 0 && mx > mn) s16 = 1;             // smallest fp16 subnormal, 2^-24
    const float sf = h2f(s16);
    q.inv = sf > 0.0f ? rcp_half(sf) : 0.0f;      // = 1 / sf, correctly rounded
    q.z = mn + 0.0f;                              // a -0 minimum is stored as +0
    q.z16 = f2h_rn(q.z);
    q.s16 = s16;
    q.lq = lq;
    return q;
}

// the code of x as the low bits of the float 2^23 + code (0x4B000000 above them):
// min(rint(y), lq) = rint(min(y, lq)) for y >= 0 and integer lq, and adding 2^23 rounds
// 0 <= y < 2^22 to the nearest integer, ties to even, as rint does
__device__ __forceinline__ uint32_t code_bits(float x, const RowQ &q) {
    const float y = fminf((x - q.z) * q.inv, q.lq);
    return __float_as_uint(y + 8388608.0f);
}

__device__ __forceinline__ uint32_t code_of(float x, const RowQ &q) {
    return code_bits(x, q) & 0xffu;
}

// the low bytes of four code_bits words as one word, a in byte 0
__device__ __forceinline__ uint32_t gather4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return (__builtin_amdgcn_perm(d, c, 0x0c0c0400u) << 16) | __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
}

// one fp16 row slice of 8 channels; a non-temporal load, since the prompt's K/V rows are
// read once and streaming them keeps the caches for the page images and tables
typedef unsigned int qr_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load_row8(const uint16_t *src, bool live, float (&x)[8]) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (live) {
        const qr_u4 x = __builtin_nontemporal_load(reinterpret_cast<const qr_u4 *>(src));
        u = make_uint4(x[0], x[1], x[2], x[3]);
    }
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = h2f(uint16_t(w[e] & 0xffffu));
        x[2 * e + 1] = h2f(uint16_t(w[e] >> 16));
    }
}

}  // namespace kvc
