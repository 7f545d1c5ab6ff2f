// kvc_paged_decode_attention: one decode query per request over mixed-precision pages.
//
// Keys and values are reconstructed on the fly from the unified pages (K8V4 HIGH pages,
// K4V2 LOW pages) as code*scale + zero and attended with an online softmax (DiffKV review
// page: the memory manager serves attention over the compressed paged cache; "Assumptions"
// lists standard causal multi-head attention, the page's Eq. 1).
//
// Matrix-core design (gfx950, wave64, v_mfma_f32_16x16x32_f16):
//   * a tile is 16 tokens: one HIGH page, or one half of a LOW page;
//   * S^T = K_codes * Q^T on MFMA: rows are the tile's tokens, columns the G query heads of
//     the KV head (padded to 16).  Codes become exact fp16 operands with one bit trick
//     (0x6400 | code is the fp16 number 1024 + code); the pages' byte order puts each lane's
//     32 key channels in one contiguous 32-byte (K8) or 16-byte (K4) run, so codes go
//     straight from a 128-bit load into operand registers, without LDS;
//     q.k_hat = scale_k * (q . code) + zero_k * sum(q);
//   * P' = p * scale_v is split into fp16 hi + lo parts (two MFMAs) so the value weights keep
//     ~22 bits; O += P' * V_codes on MFMA, with the values' page layout already in the
//     operand's token-major order (value codes enter as exact small integers); the zero_v
//     term is added back per query head from a running sum;
//   * the running max is only moved when a tile exceeds it by more than 8 (in log2 units),
//     so the accumulator rescale (a cross-lane shuffle) is rare; it is also forced for a pair
//     holding a value scale above 65504 / 2^8, which keeps P' = p * scale_v within fp16;
//   * split-K with a per-head plan: a head's tiles are weighed in work units (HIGH 3, LOW 2,
//     their measured relative cost) and the head takes one workgroup per ~wt units of its
//     workgroup slots (long heads of a ragged batch get more); four waves per workgroup take
//     consecutive slices of the workgroup's range and merge in LDS; each wave keeps a pair
//     of tiles in flight in registers, with the page ids of up to 64 tiles preloaded in one
//     lane-indexed register (no load waits on another load);
//   * a second kernel merges each query head's S (max, sum, output) partials in float32 (a
//     fused last-workgroup merge needs device-scope fences, which on a multi-XCD part write
//     back and invalidate L2 and cost more than the extra launch).
#include <mutex>

#include "kvc_internal.h"
#include "page_load.h"
#include "workspace.h"

namespace kvc {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_MARGIN = 8.0f;      // log2 units
constexpr float VS_LAZY_MAX = 255.875f;     // 65504 / 2^RESCALE_MARGIN: larger value
                                            // scales force the rescale (p <= 1)
constexpr float M_INIT = -1.0e30f;          // finite "minus infinity" for the running max
#ifndef KVC_DEC_WAVES
#define KVC_DEC_WAVES 4
#endif
#ifndef KVC_DEC_OCC
#define KVC_DEC_OCC 3
#endif
constexpr int DEC_WAVES = KVC_DEC_WAVES;    // waves per workgroup (slices of one head)

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ h8 cat4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(h8, make_uint4(a, b, c, d));
}
__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pick4(const uint4 &u, int k) {
    return k == 0 ? u.x : k == 1 ? u.y : k == 2 ? u.z : u.w;
}
__device__ __forceinline__ float half_lo(uint32_t u) { return h2f(uint16_t(u & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t u) { return h2f(uint16_t(u >> 16)); }

// A 4- or 2-bit code moved to mantissa bits 6..9 of each fp16 half and OR-ed with 16.0
// (0x4C00) is the exact fp16 number 16 + code.  SH > 0 shifts left, < 0 right.  `mg` holds
// 0x4C004C00 in a register the compiler cannot see through, so shift + v_and_or_b32 is two
// instructions per pair of codes.
template <int SH, uint32_t MASK>
__device__ __forceinline__ uint32_t code16(uint32_t w, uint32_t mg) {
    const uint32_t x = SH >= 0 ? (w << SH) : (w >> (-SH));
    return (x & MASK) | mg;
}
constexpr uint32_t NIB = 0x03C003C0u;    // bits 6..9 of both halves
constexpr uint32_t CRB = 0x00C000C0u;    // bits 6..7 of both halves
constexpr float KOFF_HIGH = 1024.0f;     // 8-bit key codes: byte -> 1024 + code
constexpr float COFF = 16.0f;            // 4/2-bit codes: 16 + code

// Per-lane bytes of a pair of 16-token tiles (A, B) of one tier, in two parts so the next
// pair's value/parameter loads can reuse the registers of the current pair's keys.  A HIGH
// tile is one HIGH page; a LOW tile is one half (16 slots) of a LOW page.  Keys and values of
// both tiles are needed by every lane (matrix operands); parameters only for its own tile.
template <bool HIGH> struct Keys;
template <> struct Keys<true> {
    uint4 ka0, ka1, kb0, kb1;   // channels 32j..32j+31 of token (lane & 15), 8-bit codes
};
template <> struct Keys<false> {
    uint4 ka, kb;               // channels 32j..32j+31 of token (lane & 15), 4-bit codes
};
template <bool HIGH> struct Vals;
template <> struct Vals<true> {
    uint4 va, vb;               // value unit 16j + (lane & 15): tokens 4j..4j+3, 8 channels
    uint4 p0, p1;               // parameters of tokens 4j..4j+3 of the lane's tile
    uint32_t ps;                // (score accumulation) position of token 4j + (lane & 3)
};
template <> struct Vals<false> {
    uint2 va, vb;               // the tiles' halves of value unit 16j + (lane & 15)
    uint4 p0, p1;
    uint32_t ps;
};

template <bool HIGH>
__device__ __forceinline__ Keys<HIGH> load_keys(__amdgpu_buffer_rsrc_t ra,
                                                __amdgpu_buffer_rsrc_t rb, int fa, int fb,
                                                int lane) {
    const uint32_t j = lane >> 4, tok = lane & 15;
    Keys<HIGH> d;
    if constexpr (HIGH) {
        const uint32_t o = K_OFF + tok * 128 + 32 * j;
        d.ka0 = ld16(ra, o);
        d.ka1 = ld16(ra, o + 16);
        d.kb0 = ld16(rb, o);
        d.kb1 = ld16(rb, o + 16);
    } else {
        d.ka = ld16(ra, K_OFF + (16 * uint32_t(fa) + tok) * 64 + 16 * j);
        d.kb = ld16(rb, K_OFF + (16 * uint32_t(fb) + tok) * 64 + 16 * j);
    }
    return d;
}

// LG: also the position of token 4j + (lane & 3) of the lane's own tile.  own: the page of
// the lane's own tile (HIGH: page A or B by lane; read by per-lane addresses, since a buffer
// descriptor chosen per lane would make the compiler serialize the load over the two pages)
template <bool HIGH, bool LG>
__device__ __forceinline__ Vals<HIGH> load_vals(__amdgpu_buffer_rsrc_t ra,
                                                __amdgpu_buffer_rsrc_t rb, int fa, int fb,
                                                int lane, bool own_b, const uint8_t *own) {
    const uint32_t j = lane >> 4;
    Vals<HIGH> d;
    d.ps = 0;
    if constexpr (HIGH) {
        d.va = ld16(ra, V_OFF + 16 * uint32_t(lane));
        d.vb = ld16(rb, V_OFF + 16 * uint32_t(lane));
        // parameters of the lane's own tile: each half-wave reads its tile's page
        const uint4 *op = reinterpret_cast<const uint4 *>(own + PARAM_OFF + 32 * j);
        d.p0 = op[0];
        d.p1 = op[1];
        if constexpr (LG)
            d.ps = *reinterpret_cast<const uint32_t *>(own + POS_OFF + 4 * (4 * j + (lane & 3)));
    } else {
        // the two LOW tiles of a pair are the halves of one page (ra and rb are the same)
        d.va = ld8(ra, V_OFF + 16 * uint32_t(lane) + 8 * uint32_t(fa));
        d.vb = ld8(rb, V_OFF + 16 * uint32_t(lane) + 8 * uint32_t(fb));
        const uint32_t o = PARAM_OFF + 8 * (16 * uint32_t(own_b ? fb : fa) + 4 * j);
        d.p0 = ld16(ra, o);
        d.p1 = ld16(ra, o + 16);
        if constexpr (LG)
            d.ps = ld4(ra, POS_OFF + 4 * (16 * uint32_t(own_b ? fb : fa) + 4 * j + (lane & 3)));
    }
    return d;
}

// key operand of 16x16x32 MFMA m (0..3): channels 32j + 8m + {0,2,1,3,4,6,5,7}
__device__ __forceinline__ h8 key_op_high(const uint4 &k0, const uint4 &k1, int m, uint32_t mg) {
    const uint32_t w0 = m < 2 ? pick4(k0, 2 * m) : pick4(k1, 2 * m - 4);
    const uint32_t w1 = m < 2 ? pick4(k0, 2 * m + 1) : pick4(k1, 2 * m - 3);
    // mg = 0x64646464: byte b of a key word becomes the fp16 number 1024 + b
    return cat4(__builtin_amdgcn_perm(mg, w0, 0x04020400u), __builtin_amdgcn_perm(mg, w0, 0x04030401u),
                __builtin_amdgcn_perm(mg, w1, 0x04020400u), __builtin_amdgcn_perm(mg, w1, 0x04030401u));
}
__device__ __forceinline__ h8 key_op_low(const uint4 &k, int m, uint32_t mg) {
    const uint32_t w = pick4(k, m);    // nibble p holds channel order {0,1,4,5,2,3,6,7}
    return cat4(code16<6, NIB>(w, mg), code16<2, NIB>(w, mg), code16<-2, NIB>(w, mg),
                code16<-6, NIB>(w, mg));
}

// value operand (B, tokens x channels) of 16x16x32 MFMA n: k = 8j + e, e < 4 tile A token
// 4j + e, e >= 4 tile B token 4j + e - 4, channel 16n + (lane & 15); entries 16 + code
__device__ __forceinline__ void val_pair_high(uint32_t w, int nlow, uint32_t mg, uint32_t &r01,
                                              uint32_t &r23) {
    // unit word: channel-block n = 2q + nlow, token r at nibble 2*nlow + (r>>1) + 4*(r&1)
    if (nlow == 0) {
        r01 = code16<6, NIB>(w, mg);
        r23 = code16<2, NIB>(w, mg);
    } else {
        r01 = code16<-2, NIB>(w, mg);
        r23 = code16<-6, NIB>(w, mg);
    }
}
__device__ __forceinline__ h8 val_op_high(const uint4 &va, const uint4 &vb, int n, uint32_t mg) {
    uint32_t a01, a23, b01, b23;
    val_pair_high(pick4(va, n >> 1), n & 1, mg, a01, a23);
    val_pair_high(pick4(vb, n >> 1), n & 1, mg, b01, b23);
    return cat4(a01, a23, b01, b23);
}
template <int NL>
__device__ __forceinline__ void val_pair_low(uint32_t w, uint32_t mg, uint32_t &r01,
                                             uint32_t &r23) {
    // 2-bit field 2*NL + (r>>1) + 8*(r&1) of the word; fields f, f+8 share a 16-bit lane
    r01 = code16<6 - 4 * NL, CRB>(w, mg);
    r23 = code16<4 - 4 * NL, CRB>(w, mg);
}
template <int N>
__device__ __forceinline__ h8 val_op_low(const uint2 &va, const uint2 &vb, uint32_t mg) {
    const uint32_t wa = (N >> 2) == 0 ? va.x : va.y, wb = (N >> 2) == 0 ? vb.x : vb.y;
    uint32_t a01, a23, b01, b23;
    val_pair_low<N & 3>(wa, mg, a01, a23);
    val_pair_low<N & 3>(wb, mg, b01, b23);
    return cat4(a01, a23, b01, b23);
}

struct WaveState {
    f4 o[8];         // O[row 4j + r][16n + (lane & 15)]; row c < 8: tile-A half, >= 8: tile-B half
    float m;         // running max (log2 units) of query head (lane & 7), shared by c and c^8
    float l, lz, lp; // partial sums of the lane's own scores: p, p*zero_v, P' (offset removal)
};

__device__ __forceinline__ float fmax_raw(float a, float b) {   // no NaNs here: plain v_max
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// max over the lanes of one score column: the four 16-lane groups (xor 16, xor 32) and the
// two tile halves (xor 8), with lane swaps and a row rotation instead of LDS permutes
__device__ __forceinline__ float max_over_column(float x) {
    uint32_t u = __float_as_uint(x);
    const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = fmax_raw(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    u = __float_as_uint(x);
    const auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmax_raw(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    const float y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf,
                                                             false));   // row_ror:8
    return fmax_raw(x, y);
}

struct Magic {
    uint32_t k8;     // 0x64646464 (key bytes -> 1024 + code)
    uint32_t c16;    // 0x4C004C00 (4/2-bit codes -> 16 + code)
};

// S^T for a pair of tiles.  The query operands live in LDS (shared by the workgroup's waves):
// qa holds the 8 query heads in columns 0..7 (zero in 8..15), qb in columns 8..15, so lane
// column c = lane & 15 gets tile A's scores when c < 8 and tile B's when c >= 8 and every
// lane's softmax work is useful although G <= 8.
template <bool HIGH>
__device__ __forceinline__ f4 pair_scores(const Keys<HIGH> &d, const uint4 (*s_qa)[64],
                                          const uint4 (*s_qb)[64], int lane, const Magic &mg,
                                          float acc0) {
    f4 acc = {acc0, acc0, acc0, acc0};      // -code offset * sum(q): removes the offset
    // an opaque lane index keeps the compiler from hoisting the LDS reads out of the loop
    // (which would pin 32 registers for the operands)
    int li = lane;
    asm volatile("" : "+v"(li));
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const h8 qa = __builtin_bit_cast(h8, s_qa[m][li]);
        const h8 qb = __builtin_bit_cast(h8, s_qb[m][li]);
        if constexpr (HIGH) {
            acc = mfma32(key_op_high(d.ka0, d.ka1, m, mg.k8), qa, acc);
            acc = mfma32(key_op_high(d.kb0, d.kb1, m, mg.k8), qb, acc);
        } else {
            acc = mfma32(key_op_low(d.ka, m, mg.c16), qa, acc);
            acc = mfma32(key_op_low(d.kb, m, mg.c16), qb, acc);
        }
    }
    return acc;
}

// LG: the lane also stores its four logits (log2 units, -inf for empty slots) as one 16-byte
// store at lg when lg_on, and lanes with ps_on the position of token 4j + (lane & 3) of its
// tile at lg - ps_off, when lg is not null (the score-accumulating variant)
template <bool HIGH, bool LG>
__device__ __forceinline__ void pair_softmax_pv(const f4 &acc, const Vals<HIGH> &d, int live_own,
                                                float sumq, float scale_log2, int lane,
                                                const Magic &mg, WaveState &st, float *lg,
                                                bool lg_on, bool ps_on, int ps_off) {
    const int j = lane >> 4, c = lane & 15;
    const bool own_b = c >= 8;
    const uint32_t pw[8] = {d.p0.x, d.p0.y, d.p0.z, d.p0.w, d.p1.x, d.p1.y, d.p1.z, d.p1.w};
    float L[4], vs[4], vz[4];
    float tmax = M_INIT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float ks = half_lo(pw[2 * r]), kz = half_hi(pw[2 * r]);
        vs[r] = half_lo(pw[2 * r + 1]);
        vz[r] = half_hi(pw[2 * r + 1]);
        // q.k_hat * scale * log2(e); sumq is already scaled by scale * log2(e)
        const float x = ks * (acc[r] * scale_log2) + kz * sumq;
        L[r] = (4 * j + r < live_own) ? x : -__builtin_inff();
        tmax = fmaxf(tmax, L[r]);
    }
    if constexpr (LG) {
        if (lg) {          // tokens 4j..4j+3 of the lane's tile and query head, contiguous
            if (lg_on) *reinterpret_cast<float4 *>(lg) = make_float4(L[0], L[1], L[2], L[3]);
            if (ps_on) reinterpret_cast<uint32_t *>(lg)[-ps_off] = d.ps;
        }
    }
    tmax = max_over_column(tmax);
    // P' = p * scale_v enters the value product as fp16.  With the lazy running max p can
    // reach 2^RESCALE_MARGIN, so a value scale above 65504 / 2^8 could overflow fp16: a pair
    // holding such a scale forces the rescale, after which p <= 1 and P' <= scale_v <= 65504
    // (value rows spanning more than ~3,800 at 4 bits or ~770 at 2 bits; never for data of
    // unit scale, whose path is unchanged)
    const bool big = fmaxf(fmaxf(vs[0], vs[1]), fmaxf(vs[2], vs[3])) > VS_LAZY_MAX;
    // the branch is uniform, but written as a per-lane condition (an opaque lane value that
    // is always 1) the compiler predicates it instead of splitting the accumulators' live
    // ranges, which would copy all 32 of them on the common path
    int one = 1;
    asm volatile("" : "+v"(one));
    if (one && __ballot(tmax > st.m + RESCALE_MARGIN || big) != 0ull) {
        const float mn = fmaxf(st.m, tmax);
        const float corr = __builtin_amdgcn_exp2f(st.m - mn);
        st.l *= corr;
        st.lz *= corr;
        st.lp *= corr;
        st.m = mn;
        float cr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * j + r, 64);
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) st.o[n][r] *= cr[r];
    }
    // P' = p * scale_v, as fp16 hi + lo, placed in the lane's half of the k dimension
    _Float16 hi[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(L[r] - st.m);     // exp2(-inf) = 0
        const float pv = p * vs[r];
        hi[r] = _Float16(pv);
        lo[r] = _Float16(pv - float(hi[r]));
        st.l += p;
        st.lz += p * vz[r];
        st.lp += pv;          // the 16 + code offset is removed with this sum at the end
    }
    const uint32_t h01 = __builtin_bit_cast(uint32_t, h2{hi[0], hi[1]});
    const uint32_t h23 = __builtin_bit_cast(uint32_t, h2{hi[2], hi[3]});
    const uint32_t l01 = __builtin_bit_cast(uint32_t, h2{lo[0], lo[1]});
    const uint32_t l23 = __builtin_bit_cast(uint32_t, h2{lo[2], lo[3]});
    const h8 phi = cat4(own_b ? 0u : h01, own_b ? 0u : h23, own_b ? h01 : 0u, own_b ? h23 : 0u);
    const h8 plo = cat4(own_b ? 0u : l01, own_b ? 0u : l23, own_b ? l01 : 0u, own_b ? l23 : 0u);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        h8 vop;
        if constexpr (HIGH) {
            vop = val_op_high(d.va, d.vb, n, mg.c16);
        } else {
            switch (n) {
                case 0: vop = val_op_low<0>(d.va, d.vb, mg.c16); break;
                case 1: vop = val_op_low<1>(d.va, d.vb, mg.c16); break;
                case 2: vop = val_op_low<2>(d.va, d.vb, mg.c16); break;
                case 3: vop = val_op_low<3>(d.va, d.vb, mg.c16); break;
                case 4: vop = val_op_low<4>(d.va, d.vb, mg.c16); break;
                case 5: vop = val_op_low<5>(d.va, d.vb, mg.c16); break;
                case 6: vop = val_op_low<6>(d.va, d.vb, mg.c16); break;
                default: vop = val_op_low<7>(d.va, d.vb, mg.c16); break;
            }
        }
        st.o[n] = mfma32(phi, vop, st.o[n]);
        st.o[n] = mfma32(plo, vop, st.o[n]);
    }
}

// tiles [t0, t1) of one tier of a head, two at a time; page ids of up to 64 pages come from
// one lane-indexed register, so no load waits on another load.  The next pair's keys are
// requested before this pair's scores, its values and parameters before this pair's softmax
// (reusing the registers of the keys just consumed).
// page ids of the first chunk (up to 64 pages) of tiles [t0, t1) of one tier: lane k holds
// the id of page t0 / TPP + k (0 beyond the chunk)
template <bool HIGH>
__device__ __forceinline__ int first_chunk_pids(int t0, int t1, const int32_t *row, int C,
                                                int lane) {
    constexpr int TPP = HIGH ? 1 : 2;
    if (t0 >= t1) return 0;
    const int c1 = min(t1, t0 + 64 * TPP);
    const int p0 = t0 / TPP;
    const int np = (c1 - 1) / TPP - p0 + 1;
    return lane < np ? (HIGH ? row[p0 + lane] : row[C - 1 - (p0 + lane)]) : 0;
}

// lgh (LG only): the head's tile records [tile][16 positions, then GT query heads x 16
// tokens of logits] offset to this tier's first tile, the lane's query head and first token
template <bool HIGH, bool LG>
__device__ __forceinline__ void attend_range(int t0, int t1, int n_tier, const int32_t *row,
                                             int C, const uint8_t *pages,
                                             const uint4 (*s_qa)[64], const uint4 (*s_qb)[64],
                                             float sumq, float scale_log2, int lane,
                                             const Magic &mg, WaveState &st, float *lgh,
                                             int lg_tile_stride, bool lg_on,
                                             bool ps_on, int ps_off, int pid_first) {
    constexpr int TPP = HIGH ? 1 : 2;             // tiles per page
    const bool own_b = (lane & 15) >= 8;
    const float acc0 = -(HIGH ? KOFF_HIGH : COFF) * sumq;   // the key codes' offset
    const float sumq_s = sumq * scale_log2;
    for (int c0 = t0; c0 < t1; c0 += 64 * TPP) {
        const int c1 = min(t1, c0 + 64 * TPP);
        const int p0 = c0 / TPP;
        const int np = (c1 - 1) / TPP - p0 + 1;
        int pid = pid_first;     // the first chunk's ids were requested by the caller early
        if (c0 != t0) pid = lane < np ? (HIGH ? row[p0 + lane] : row[C - 1 - (p0 + lane)]) : 0;
        auto page_of = [&](int t) -> const uint8_t * {
            return pages + int64_t(__builtin_amdgcn_readlane(pid, t / TPP - p0)) * PAGE;
        };
        auto live_of = [&](int t) -> int {
            return t >= c1 ? 0 : (HIGH ? min(HS, n_tier - HS * t) : min(16, n_tier - 16 * t));
        };
        auto tb_of = [&](int t) -> int { return t + 1 < c1 ? t + 1 : t; };  // missing B: reuse A
        // pair starting at tile t; past the last pair the loads repeat the last pair (cache
        // hits), which keeps the loop free of branches around loads and of register copies
        const int tlast = c0 + ((c1 - 1 - c0) & ~1);
        auto keys_at = [&](int t) {
            t = min(t, tlast);
            const int tb = tb_of(t);
            return load_keys<HIGH>(page_rsrc(page_of(t)), page_rsrc(page_of(tb)), t & 1, tb & 1,
                                   lane);
        };
        auto vals_at = [&](int t) {
            t = min(t, tlast);
            const int tb = tb_of(t);
            const uint8_t *pa = page_of(t), *pb = page_of(tb);
            return load_vals<HIGH, LG>(page_rsrc(pa), page_rsrc(pb), t & 1, tb & 1, lane, own_b,
                                       own_b ? pb : pa);
        };
        // the lane's logit slot for the pair starting at tile t (its own tile of the pair)
        auto lg_at = [&](int t) -> float * {
            if constexpr (!LG) {
                return nullptr;
            } else {
                const int own = own_b ? t + 1 : t;
                return (lgh && own < c1) ? lgh + int64_t(own) * lg_tile_stride : nullptr;
            }
        };
        Keys<HIGH> ka = keys_at(c0), kb;
        Vals<HIGH> va = vals_at(c0), vb;
        for (int t = c0;;) {
            kb = keys_at(t + 2);
            f4 acc = pair_scores<HIGH>(ka, s_qa, s_qb, lane, mg, acc0);
            vb = vals_at(t + 2);
            pair_softmax_pv<HIGH, LG>(acc, va, own_b ? live_of(t + 1) : live_of(t), sumq_s,
                                      scale_log2, lane, mg, st, lg_at(t), lg_on, ps_on, ps_off);
            t += 2;
            if (t >= c1) break;
            ka = keys_at(t + 2);
            acc = pair_scores<HIGH>(kb, s_qa, s_qb, lane, mg, acc0);
            va = vals_at(t + 2);
            pair_softmax_pv<HIGH, LG>(acc, vb, own_b ? live_of(t + 1) : live_of(t), sumq_s,
                                      scale_log2, lane, mg, st, lg_at(t), lg_on, ps_on, ps_off);
            t += 2;
            if (t >= c1) break;
        }
    }
}

// grid: S workgroup slots per (request, KV head, group of up to 8 query heads), of which the
// head uses active_splits(); the 4 waves of a workgroup take consecutive slices of its share
// of the head's tiles, weighed in work units (a HIGH tile DEC_UH, a LOW tile DEC_UL)
// LG: also store, per tile of the head (HIGH tiles, then LOW tiles), its 16 slots' positions
// and every token's logit per query head: lg [head][tile][16 + GT * 16] (positions, then per
// query head its 16 tokens), for the score accumulation
template <bool LG>
__global__ __launch_bounds__(64 * DEC_WAVES) __attribute__((amdgpu_waves_per_eu(KVC_DEC_OCC)))
void decode_mfma_kernel(const uint16_t *__restrict__ q, float scale_log2,
                        const uint8_t *__restrict__ pages, const int32_t *__restrict__ rows_l,
                        const int32_t *__restrict__ count_l, int Hkv, int GT, int C, int S,
                        int wt, float *__restrict__ part, float *__restrict__ lg,
                        int64_t tiles_cap) {
    __shared__ float s_o[DEC_WAVES][8][D];      // [wave][query head][channel]
    __shared__ float s_m[DEC_WAVES][16], s_l[DEC_WAVES][16], s_lz[DEC_WAVES][16],
        s_lp[DEC_WAVES][16];
    __shared__ uint4 s_qa[4][64], s_qb[4][64];
    const int lane = threadIdx.x & 63;
    // the wave index is the same in all lanes: reading it from lane 0 tells the compiler so,
    // which keeps the tile ranges, the loop control and page-id lookups in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, j = lane >> 4, gq = c & 7;
    const int NGP = (GT + 7) >> 3;             // groups of 8 query heads per KV head
    const int gp = (blockIdx.x / S) % NGP;
    const int i = blockIdx.x / (S * NGP);      // head index b*Hkv + h
    const int b = i / Hkv, h = i - b * Hkv;
    const int Hq = Hkv * GT;
    const int G = min(8, GT - 8 * gp);         // query heads of this group
    const int g0 = 8 * gp;
    // the query rows and the head's counts are requested together, before either is used
    uint4 qv[4] = {};
    if (gq < G) {
        const uint4 *qp = reinterpret_cast<const uint4 *>(q + (int64_t(b) * Hq + h * GT + g0 + gq) * D + 32 * j);
        qv[0] = qp[0]; qv[1] = qp[1]; qv[2] = qp[2]; qv[3] = qp[3];
    }
    const int nh = count_l[2 * i], nl = count_l[2 * i + 1];
    const int SH = active_splits(nh, nl, S, wt);   // the head's workgroups; the rest exit
    const int s = split_of_slot(blockIdx.x % S, i, SH, S);
    if (s >= SH) return;
    const int qH = ceil_div(nh, HS);
    const int tL = ceil_div(nl, 16);
    // work units: a HIGH tile (one page) weighs DEC_UH, a LOW tile (half a page) DEC_UL;
    // slices start on even LOW tiles (pairs stay in a page)
    const int64_t WH = int64_t(DEC_UH) * qH;
    const int64_t W = WH + int64_t(DEC_UL) * tL;
    const int NC = SH * DEC_WAVES;
    const int cc = s * DEC_WAVES + wave;
    auto tile_of = [&](int64_t x) -> int {
        int t = x <= WH ? int((x + DEC_UH - 1) / DEC_UH)
                        : qH + int((x - WH + DEC_UL - 1) / DEC_UL);
        if (t > qH) t = qH + ((t - qH + 1) & ~1);     // LOW pairs start on even LOW tiles
        return min(t, qH + tL);
    };
    const int u0 = tile_of(W * cc / NC), u1 = tile_of(W * (cc + 1) / NC);

    // query operands: lane (c, j) holds q[gq][32j + 8m + {0,2,1,3,4,6,5,7}], gq = c & 7,
    // kept in LDS for the whole workgroup (all its waves serve the same head): qa in columns
    // 0..7, qb in columns 8..15
    // the first page ids of both tiers are requested before the workgroup waits on its barrier
    const int32_t *row = rows_l + int64_t(i) * C;
    const int pid_h = first_chunk_pids<true>(u0, min(u1, qH), row, C, lane);
    const int pid_l = first_chunk_pids<false>(max(u0, qH) - qH, u1 - qH, row, C, lane);
    float sumq = 0.0f;
    {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const h2 x0 = as_h2(qv[m].x), x1 = as_h2(qv[m].y), x2 = as_h2(qv[m].z), x3 = as_h2(qv[m].w);
            const h8 o = {x0[0], x1[0], x0[1], x1[1], x2[0], x3[0], x2[1], x3[1]};
#pragma unroll
            for (int e = 0; e < 8; ++e) sumq += float(o[e]);
            if (wave == 0) {
                const uint4 ov = __builtin_bit_cast(uint4, o);
                const bool lo_half = c < 8;
                s_qa[m][lane] = make_uint4(lo_half ? ov.x : 0u, lo_half ? ov.y : 0u,
                                           lo_half ? ov.z : 0u, lo_half ? ov.w : 0u);
                s_qb[m][lane] = make_uint4(lo_half ? 0u : ov.x, lo_half ? 0u : ov.y,
                                           lo_half ? 0u : ov.z, lo_half ? 0u : ov.w);
            }
        }
        sumq += __shfl_xor(sumq, 16, 64);
        sumq += __shfl_xor(sumq, 32, 64);
    }
    __syncthreads();

    WaveState st;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = f4{0.f, 0.f, 0.f, 0.f};
    st.m = M_INIT;
    st.l = st.lz = st.lp = 0.0f;

    Magic mg{0x64646464u, 0x4C004C00u};
    asm volatile("" : "+v"(mg.k8), "+v"(mg.c16));   // keep the constants in VGPRs
    // LG: tile records of 16 (GT + 1) words; the lane's logit words of tokens 4j..4j+3,
    // query head g0 + gq in tile 0 of the head (stored when gq < G); lanes gq < 4 of the first
    // group also store the position of token 4j + gq, ps_off words before those logits
    const int lg_stride = 16 * (GT + 1);
    float *lgh = nullptr;
    if constexpr (LG)
        lgh = lg + int64_t(i) * tiles_cap * lg_stride + 16 + 16 * (g0 + gq) + 4 * j;
    const bool lg_on = gq < G, ps_on = g0 == 0 && gq < 4;
    const int ps_off = 16 + 15 * gq;
    attend_range<true, LG>(u0, min(u1, qH), nh, row, C, pages, s_qa, s_qb, sumq, scale_log2,
                           lane, mg, st, lgh, lg_stride, lg_on, ps_on, ps_off, pid_h);
    attend_range<false, LG>(max(u0, qH) - qH, u1 - qH, nl, row, C, pages, s_qa, s_qb, sumq,
                            scale_log2, lane, mg, st,
                            lgh ? lgh + int64_t(qH) * lg_stride : nullptr, lg_stride, lg_on,
                            ps_on, ps_off, pid_l);
    // per query head gq: sums over the lane's 4 groups and over the two column halves
#pragma unroll
    for (int o = 8; o <= 32; o <<= 1) {
        if (o == 8 || o == 16 || o == 32) {
            st.l += __shfl_xor(st.l, o, 64);
            st.lz += __shfl_xor(st.lz, o, 64);
            st.lp += __shfl_xor(st.lp, o, 64);
        }
    }
    // ---- merge the four waves in LDS and write this workgroup's partial --------------------
    // rows gg (tile A half, lanes 0..31) and gg + 8 (tile B half, lanes 32..63) of the
    // accumulator belong to the same query head
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.o[n][r] += __shfl_xor(st.o[n][r], 32, 64);
    if (lane < 32) {
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) s_o[wave][4 * j + r][16 * n + c] = st.o[n][r];
    }
    if (lane < 8) {
        s_m[wave][lane] = st.m;
        s_l[wave][lane] = st.l;
        s_lz[wave][lane] = st.lz;
        s_lp[wave][lane] = st.lp;
    }
    __syncthreads();
    float *hp = part + int64_t(i) * S * GT * PART_STRIDE;    // this head's partials [s][g]
    for (int e = threadIdx.x; e < G * D; e += 64 * DEC_WAVES) {
        const int gg = e / D, d = e - gg * D;
        float M = M_INIT;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, s_m[w][gg]);
        float Ls = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_m[w][gg] - M);
            O += (s_o[w][gg][d] - COFF * s_lp[w][gg] + s_lz[w][gg]) * f;
            Ls += s_l[w][gg] * f;
        }
        float *pp = hp + (int64_t(s) * GT + g0 + gg) * PART_STRIDE;
        if (d == 0) {
            pp[0] = M;
            pp[1] = Ls;
        }
        pp[4 + d] = O;
    }
}

// merge the S partials of one (request, query head): one wave per query head; lane s < S
// holds split s's max, the weights are broadcast, each lane accumulates 2 channels
// one wave per (request, query head): lanes first hold the splits' (m, l) (S <= 64), then
// two output channels each; the splits' partial rows are loaded eight at a time, all
// independent, and weighted with exp2(m_s - M) read from the owning lane
__device__ __forceinline__ void combine_block(int bx, const float *__restrict__ part, int Hq,
                                              int G, int S, int nqh, void *out, int out_fp32,
                                              float *__restrict__ mls,
                                              const int32_t *__restrict__ count_l, int wt) {
    const int lane = threadIdx.x & 63;
    const int qh = bx * 4 + (threadIdx.x >> 6);            // b*Hq + hq
    if (qh >= nqh) return;
    const int b = qh / Hq, hq = qh - b * Hq;
    const int h = hq / G, gg = hq - h * G;
    const int Hkv = Hq / G;
    const int64_t sstride = int64_t(G) * PART_STRIDE;
    const float *hp = part + ((int64_t(b) * Hkv + h) * S * G + gg) * PART_STRIDE;
    // The head's split count first; then its splits' (max, sum) and the first PRE splits'
    // outputs are requested together, so the merge waits for two round trips (a slot past
    // SH reloads split SH - 1, a cache hit, and gets weight 0)
    const int64_t hi = int64_t(b) * Hkv + h;
    const int SH = active_splits(count_l[2 * hi], count_l[2 * hi + 1], S, wt);
    float ms = M_INIT, ls = 0.0f;
    if (lane < SH) {
        ms = hp[lane * sstride];
        ls = hp[lane * sstride + 1];
    }
    constexpr int PRE = 16;
    float2 vp[PRE];
#pragma unroll
    for (int u = 0; u < PRE; ++u)
        vp[u] = *reinterpret_cast<const float2 *>(hp + min(u, SH - 1) * sstride + 4 + 2 * lane);
    float M = ms;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float w = lane < SH ? __builtin_amdgcn_exp2f(ms - M) : 0.0f;
    float Ls = ls * w;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) Ls += __shfl_xor(Ls, o, 64);
    float r0 = 0.0f, r1 = 0.0f;
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
        const float wf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
        if (u < SH) {
            r0 += vp[u].x * wf;
            r1 += vp[u].y * wf;
        }
    }
    for (int k0 = PRE; k0 < SH; k0 += 8) {
        float2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = min(k0 + u, SH - 1);          // past the end: reload, weight 0
            v[u] = *reinterpret_cast<const float2 *>(hp + k * sstride + 4 + 2 * lane);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int wk = __builtin_amdgcn_readlane(__float_as_int(w), min(k0 + u, 63));
            const float wf = k0 + u < SH ? __int_as_float(wk) : 0.0f;
            r0 += v[u].x * wf;
            r1 += v[u].y * wf;
        }
    }
    const int64_t idx = int64_t(qh) * D + 2 * lane;
    const float o0 = Ls > 0.0f ? r0 / Ls : 0.0f, o1 = Ls > 0.0f ? r1 / Ls : 0.0f;
    if (mls && lane == 0) *reinterpret_cast<float2 *>(mls + 2 * int64_t(qh)) = make_float2(M, Ls);
    if (out_fp32) {
        *reinterpret_cast<float2 *>(static_cast<float *>(out) + idx) = make_float2(o0, o1);
    } else {
        const uint32_t v = uint32_t(f2h_rn(o0)) | (uint32_t(f2h_rn(o1)) << 16);
        *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(out) + idx) = v;
    }
}

__global__ __launch_bounds__(256) void decode_combine_kernel(const float *__restrict__ part,
                                                             int Hq, int G, int S, int nqh,
                                                             void *out, int out_fp32,
                                                             float *__restrict__ mls,
                                                             const int32_t *__restrict__ count_l,
                                                             int wt) {
    combine_block(blockIdx.x, part, Hq, G, S, nqh, out, out_fp32, mls, count_l, wt);
}

// ---- score accumulation: acc_sum[cu[b] + pos][hq] += exp2(logit - M) / L -------------------
// The decode kernel leaves, per tile of each head (HIGH tiles, then LOW tiles of 16 slots),
// the tile's 16 positions and its logits; one accumulator row holds all query heads of one
// position.  The update therefore runs over
// chunks of ACC_R positions of one request: a workgroup loads the chunk's rows (ACC_R x Hq
// floats, contiguous) into LDS, adds the weights of every head's live tokens whose positions
// fall in the chunk, and writes the rows back whole.  Within a head and tier the slots are in
// ascending position order, so the tokens of a chunk are one slot range per head and tier;
// acc_index finds these ranges: start[c] = number of slots with position < c * ACC_R.

// grid (B*Hkv, 2 * ACC_IDX_BLOCKS): y even = HIGH, odd = LOW.  Thread for slot s (position
// p, previous slot's position prev, both from the tile records the decode kernel wrote)
// writes start[c] = s for every c with prev < c*R <= p; the last slot also writes
// start[c] = n for c*R > p up to c = ceil(N/R).
constexpr int ACC_IDX_BLOCKS = 16;
__device__ __forceinline__ void index_block(
    int i, int by, const int32_t *__restrict__ count_l, const int32_t *__restrict__ cu, int Hkv,
    int G, int max_seqlen, int nch_cap, const float *__restrict__ lg, int64_t tiles_cap,
    int32_t *__restrict__ idx, int32_t *status) {
    const bool high = (by & 1) == 0;
    const int part = by >> 1;
    const int b = i / Hkv;
    const int N = cu[b + 1] - cu[b];
    if (N < 0 || N > max_seqlen) {
        if (by == 0 && threadIdx.x == 0) atomicOr(status, KVC_DEV_SEQLEN);
        return;
    }
    const int nh = count_l[2 * i];
    const int n = high ? nh : count_l[2 * i + 1];
    const int nch = ceil_div(N, ACC_R);
    int32_t *st = idx + (int64_t(i) * 2 + (high ? 0 : 1)) * nch_cap;
    if (n == 0) {
        for (int c = part * 256 + threadIdx.x; c <= nch; c += ACC_IDX_BLOCKS * 256) st[c] = 0;
        return;
    }
    const int64_t ts = 16 * (G + 1);
    const int32_t *rec = reinterpret_cast<const int32_t *>(lg) +
                         (int64_t(i) * tiles_cap + (high ? 0 : ceil_div(nh, HS))) * ts;
    auto pos_of = [&](int sl) { return rec[int64_t(sl >> 4) * ts + (sl & 15)]; };
    const int ntl = ceil_div(n, 16);
    for (int sl = part * 256 + threadIdx.x; sl < n; sl += ACC_IDX_BLOCKS * 256) {
        if ((high ? 0 : ceil_div(nh, HS)) + ntl > tiles_cap) break;
        const int p = pos_of(sl);
        const int prev = sl > 0 ? pos_of(sl - 1) : -1;
        if (p <= prev || p >= N) {
            atomicOr(status, KVC_DEV_SEQLEN);
            continue;
        }
        const int c_hi = p / ACC_R;
        for (int c = prev < 0 ? 0 : prev / ACC_R + 1; c <= c_hi; ++c) st[c] = sl;
        if (sl == n - 1)
            for (int c = c_hi + 1; c <= nch; ++c) st[c] = n;
    }
}

__global__ __launch_bounds__(256) void acc_index_kernel(
    const int32_t *__restrict__ count_l, const int32_t *__restrict__ cu, int Hkv, int G,
    int max_seqlen, int nch_cap, const float *__restrict__ lg, int64_t tiles_cap,
    int32_t *__restrict__ idx, int32_t *status) {
    index_block(blockIdx.x, blockIdx.y, count_l, cu, Hkv, G, max_seqlen, nch_cap, lg, tiles_cap,
                idx, status);
}

// The combine and the chunk index of a score-accumulating decode in one launch (both read
// only what the main kernel wrote): workgroups [0, ncomb) combine four query heads each, the
// rest are the index's (head, part and tier) workgroups, head fastest
__global__ __launch_bounds__(256) void combine_index_kernel(
    int ncomb, int nidx_x, const float *__restrict__ part, int Hq, int G, int S, int nqh,
    void *out, int out_fp32, float *__restrict__ mls, const int32_t *__restrict__ count_l,
    int wt, const int32_t *__restrict__ cu, int Hkv, int max_seqlen, int nch_cap,
    const float *__restrict__ lg, int64_t tiles_cap, int32_t *__restrict__ idx,
    int32_t *status) {
    if (int(blockIdx.x) < ncomb) {
        combine_block(blockIdx.x, part, Hq, G, S, nqh, out, out_fp32, mls, count_l, wt);
    } else {
        const int k = int(blockIdx.x) - ncomb;
        index_block(k % nidx_x, k / nidx_x, count_l, cu, Hkv, G, max_seqlen, nch_cap, lg,
                    tiles_cap, idx, status);
    }
}

// the GT query heads' logits of one slot (16 words apart in the tile record)
template <int GT>
__device__ __forceinline__ void load_logits(const float *src, float (&l)[GT]) {
#pragma unroll
    for (int g = 0; g < GT; ++g) l[g] = src[16 * g];
}

// grid (ceil(max_seqlen / R), B), 4 waves, dynamic LDS ACC_R * Hq + 2 * Hq floats.  The
// (head, tier) ranges are the jobs: wave w takes jobs w, w + 4, ...; a range holds at most
// ACC_R = 64 slots (the chunk's positions), so lane k takes slot s0 + k and all G query heads
// of its head.  Each (position, query head) has one live slot at most, so every LDS word is
// added to by one lane: no atomics, deterministic.
// LDS row stride of the staged accumulator rows (words).  The lanes of a job hold distinct
// positions of the chunk, i.e. distinct rows, and add into the same columns: with an odd
// stride the rows of any 64 lanes fall on distinct banks
__host__ __device__ inline int acc_ldr(int Hq) { return Hq | 1; }

template <int GT>
__global__ __launch_bounds__(256) void acc_update_kernel(
    const int32_t *__restrict__ count_l, const int32_t *__restrict__ cu, int Hkv, int G_rt,
    int max_seqlen, int nch_cap, const int32_t *__restrict__ idx,
    const float *__restrict__ lg, int64_t tiles_cap,
    const float *__restrict__ mls, float *__restrict__ acc, int32_t *status) {
    extern __shared__ float s_acc[];                 // [ACC_R][ldr], then [Hq][2] (M, L)
    const int G = GT > 0 ? GT : G_rt;
    const int b = blockIdx.y, c = blockIdx.x;
    const int lo = cu[b], N = cu[b + 1] - lo;
    if (N <= 0 || N > max_seqlen) return;
    const int t0 = c * ACC_R;
    if (t0 >= N) return;
    const int nr = min(ACC_R, N - t0);
    const int Hq = Hkv * G;
    const int ldr = acc_ldr(Hq);
    float *s_ml = s_acc + ACC_R * ldr;
    float *arow = acc + (int64_t(lo) + t0) * Hq;
    const int nw = nr * Hq;
    if ((Hq & 3) == 0) {
        // the chunk's rows: every thread's loads are issued before the first LDS write
        constexpr int SU = 4;
        const int q4 = Hq >> 2, n4 = nw / 4;
        for (int k0 = threadIdx.x; k0 < n4; k0 += SU * 256) {
            float4 x[SU];
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int k = k0 + u * 256;
                if (k < n4) x[u] = reinterpret_cast<const float4 *>(arow)[k];
            }
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int k = k0 + u * 256;
                if (k < n4) {
                    const int r = k / q4, c4 = k - r * q4;
                    float *d = s_acc + r * ldr + 4 * c4;
                    d[0] = x[u].x;
                    d[1] = x[u].y;
                    d[2] = x[u].z;
                    d[3] = x[u].w;
                }
            }
        }
    } else {
        for (int k = threadIdx.x; k < nw; k += 256) s_acc[(k / Hq) * ldr + k % Hq] = arow[k];
    }
    for (int k = threadIdx.x; k < 2 * Hq; k += 256) s_ml[k] = mls[int64_t(b) * 2 * Hq + k];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar loads
    // per job: its slot, position and logits.  All of a pass's jobs' counts and chunk bounds
    // (scalar loads) are requested together, then all of their lanes' records (a lane past
    // its range reads a record of the head's first tile and drops it), so a pass waits for
    // two round trips, and the first pass's before the barrier
    constexpr int JMAX = 4;                          // jobs per wave per pass (Hkv <= 8)
    for (int j0 = 0; j0 < 2 * Hkv; j0 += 4 * JMAX) {
        int nh_j[JMAX], n_j[JMAX], st0[JMAX], st1[JMAX];
#pragma unroll
        for (int u = 0; u < JMAX; ++u) {
            const int seg = min(j0 + wave + 4 * u, 2 * Hkv - 1);
            const bool high = (seg & 1) == 0;
            const int i = b * Hkv + (seg >> 1);
            nh_j[u] = count_l[2 * i];
            n_j[u] = count_l[2 * i + 1];
            const int32_t *st = idx + (int64_t(i) * 2 + (high ? 0 : 1)) * nch_cap;
            st0[u] = st[c];
            st1[u] = st[c + 1];
        }
        int pj[JMAX], hj[JMAX];
        int64_t lj[JMAX];                            // the slot's logits: lg + lj
        float l[JMAX][GT > 0 ? GT : 1];
#pragma unroll
        for (int u = 0; u < JMAX; ++u) {
            const int seg = j0 + wave + 4 * u;
            hj[u] = seg >> 1;
            const bool high = (seg & 1) == 0;
            const int i = b * Hkv + (min(seg, 2 * Hkv - 1) >> 1);
            const int nh = nh_j[u], n = high ? nh : n_j[u];
            const int s0 = min(max(st0[u], 0), n), s1 = min(max(st1[u], s0), n);
            const int sl = s0 + lane;
            const int tile = (high ? 0 : ceil_div(nh, HS)) + (sl >> 4);
            const bool live = seg < 2 * Hkv && sl < s1 && tile < tiles_cap;
            const int64_t rb = (int64_t(i) * tiles_cap + (live ? tile : 0)) * (16 * (G + 1));
            const int32_t pos = reinterpret_cast<const int32_t *>(lg)[rb + (sl & 15)];
            lj[u] = rb + 16 + (sl & 15);
            if constexpr (GT > 0) load_logits<GT>(lg + lj[u], l[u]);
            pj[u] = live ? pos : -1;
        }
        if (j0 == 0) __syncthreads();                // the rows and (M, L) are in LDS
#pragma unroll
        for (int u = 0; u < JMAX; ++u) {
            const int p = pj[u];
            if (p < 0) continue;                      // no slot for this lane
            if (p < t0 || p >= t0 + nr) {
                atomicOr(status, KVC_DEV_SEQLEN);
                continue;
            }
            float *dst = s_acc + (p - t0) * ldr + hj[u] * G;
            const float *ml = s_ml + 2 * hj[u] * G;
            if constexpr (GT > 0) {
#pragma unroll
                for (int g = 0; g < GT; ++g)
                    if (ml[2 * g + 1] > 0.0f)
                        dst[g] += __builtin_amdgcn_exp2f(l[u][g] - ml[2 * g]) / ml[2 * g + 1];
            } else {
                for (int g = 0; g < G; ++g)
                    if (ml[2 * g + 1] > 0.0f)
                        dst[g] += __builtin_amdgcn_exp2f(lg[lj[u] + 16 * g] - ml[2 * g]) /
                                  ml[2 * g + 1];
            }
        }
    }
    __syncthreads();
    if ((Hq & 3) == 0) {
        const int q4 = Hq >> 2;
        for (int k = threadIdx.x; k < nw / 4; k += 256) {
            const int r = k / q4, c4 = k - r * q4;
            const float *d = s_acc + r * ldr + 4 * c4;
            reinterpret_cast<float4 *>(arow)[k] = make_float4(d[0], d[1], d[2], d[3]);
        }
    } else {
        for (int k = threadIdx.x; k < nw; k += 256) arow[k] = s_acc[(k / Hq) * ldr + k % Hq];
    }
}

// The combine and the score accumulation after a decode that wrote its partials and tile
// records: one launch for the combine (which writes each query head's (M, L)) and the chunk
// index, then the accumulator update (shared with the precision-scheme decode)
int launch_combine_and_accumulation(const kvc_geom *g, const kvc_pool *p, const float *part,
                                    int S, int wt, void *out, int out_fp32,
                                    const int32_t *count_l, const int32_t *cu, int max_seqlen,
                                    float *acc_sum, char *w, hipStream_t s) {
    const DecodeWs L(g, true, max_seqlen);
    const int B = g->batch, Hkv = g->num_kv_heads, Hq = g->num_q_heads, G = Hq / Hkv;
    float *mls = reinterpret_cast<float *>(w + L.mls);
    const float *lg = reinterpret_cast<const float *>(w + L.lg);
    int32_t *idx = reinterpret_cast<int32_t *>(w + L.idx);
    const int nqh = B * Hq, ncomb = (nqh + 3) / 4, nidx_x = B * Hkv;
    const int nblk = max_seqlen == 0 ? ncomb : ncomb + nidx_x * 2 * ACC_IDX_BLOCKS;
    hipLaunchKernelGGL(combine_index_kernel, dim3(nblk), dim3(256), 0, s, ncomb, nidx_x, part, Hq,
                       G, S, nqh, out, out_fp32, mls, count_l, wt, cu, Hkv, max_seqlen,
                       L.nch_cap, lg, L.tiles_cap, idx, p->dev_status);
    int rc = launch_check("score accumulation/combine and index");
    if (rc || max_seqlen == 0) return rc;
    const size_t lds = sizeof(float) * (size_t(ACC_R) * acc_ldr(g->num_q_heads) +
                                        2 * size_t(g->num_q_heads));
    auto upd = G == 8 ? acc_update_kernel<8> : G == 4 ? acc_update_kernel<4>
             : G == 16 ? acc_update_kernel<16> : G == 2 ? acc_update_kernel<2>
             : G == 1 ? acc_update_kernel<1> : acc_update_kernel<0>;
    hipLaunchKernelGGL(upd, dim3(L.nch_cap - 1, B), dim3(256), lds, s, count_l, cu, Hkv, G,
                       max_seqlen, L.nch_cap, idx, lg, L.tiles_cap, mls, acc_sum, p->dev_status);
    return launch_check("score accumulation/update");
}

// the combine launch of a split-K decode (shared with the precision-scheme decode)
int launch_decode_combine(const float *part, int Hq, int G, int S, int B, void *out,
                          int out_fp32, float *mls, const int32_t *count_l, int wt,
                          hipStream_t s) {
    const int nqh = B * Hq;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((nqh + 3) / 4), dim3(256), 0, s, part, Hq, G,
                       S, nqh, out, out_fp32, mls, count_l, wt);
    return launch_check("decode/combine");
}

}  // namespace kvc

using namespace kvc;

namespace {

int decode_impl(const kvc_geom *g, int32_t layer, const kvc_pool *p, const uint16_t *q,
                float softmax_scale, void *out, int32_t out_is_fp32, float *acc_sum,
                const int32_t *cu, int32_t max_seqlen, void *ws, size_t ws_bytes,
                kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    if (!q || !out) return KVC_E_NULL;
    const bool accum = acc_sum != nullptr || cu != nullptr;
    if (accum && (!acc_sum || !cu)) return KVC_E_NULL;
    if (!aligned16(q) || !aligned16(out)) return KVC_E_ALIGN;
    if (accum && !aligned16(acc_sum)) return KVC_E_ALIGN;
    if (layer < 0 || layer >= g->num_layers) return KVC_E_SHAPE;
    const int G = g->num_q_heads / g->num_kv_heads;
    if (G > 16) return KVC_E_SHAPE;
    if (accum && (max_seqlen < 0 || g->num_q_heads > ACC_MAX_HQ)) return KVC_E_SHAPE;
    DecodeWs L(g, accum, max_seqlen);
    if (!ws || ws_bytes < L.bytes) return KVC_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return KVC_E_ALIGN;
    char *w = static_cast<char *>(ws);
    float *part = reinterpret_cast<float *>(w + L.part);
    float *mls = accum ? reinterpret_cast<float *>(w + L.mls) : nullptr;
    float *lg = accum ? reinterpret_cast<float *>(w + L.lg) : nullptr;
    const int B = g->batch, Hkv = g->num_kv_heads, C = g->row_capacity;
    const int nheads = B * Hkv;
    const int32_t *rows_l = p->page_table + int64_t(layer) * nheads * C;
    const int32_t *count_l = p->count + int64_t(layer) * nheads * 2;
    hipStream_t s = (hipStream_t)stream;
    const int ngp = (G + 7) / 8;
    const dim3 grid(L.splits * nheads * ngp), block(64 * DEC_WAVES);
    if (accum)
        hipLaunchKernelGGL(decode_mfma_kernel<true>, grid, block, 0, s, q,
                           softmax_scale * LOG2E, p->pages, rows_l, count_l, Hkv, G, C, L.splits,
                           L.wt, part, lg, L.tiles_cap);
    else
        hipLaunchKernelGGL(decode_mfma_kernel<false>, grid, block, 0, s, q,
                           softmax_scale * LOG2E, p->pages, rows_l, count_l, Hkv, G, C, L.splits,
                           L.wt, part, nullptr, int64_t(0));
    rc = launch_check("kvc_paged_decode_attention/main");
    if (rc) return rc;
    if (accum)
        return launch_combine_and_accumulation(g, p, part, L.splits, L.wt, out, out_is_fp32,
                                               count_l, cu, max_seqlen, acc_sum, w, s);
    return launch_decode_combine(part, g->num_q_heads, G, L.splits, B, out, out_is_fp32, mls,
                                 count_l, L.wt, s);
}

}  // namespace

extern "C" int kvc_paged_decode_attention(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                                          const uint16_t *q, float softmax_scale, void *out,
                                          int32_t out_is_fp32, void *ws, size_t ws_bytes,
                                          kvc_stream_t stream) {
    return decode_impl(g, layer, p, q, softmax_scale, out, out_is_fp32, nullptr, nullptr, 0, ws,
                       ws_bytes, stream);
}

// ---- the decode without a workspace argument ------------------------------------------------
// The split-K partials live in this file-scope device array instead (one per GPU the library
// runs on, held until the process ends).  Host code never passes `scratch` itself to a kernel
// (on the host the name is a stand-in, not a device address): the device address is looked up
// once per device with hipGetSymbolAddress and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[KVC_STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch[MAX_DEVICES] = {};

// the current device's scratch address (looked up on its first use); nullptr on failure
void *scratch_of_current_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_error("kvc_paged_decode_attention_static/hipGetDevice", e);
        return nullptr;
    }
    if (dev < 0 || dev >= MAX_DEVICES) {
        set_error("kvc_paged_decode_attention_static/device index", hipErrorInvalidDevice);
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            set_error("kvc_paged_decode_attention_static/hipGetSymbolAddress", e);
            return nullptr;
        }
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}
}  // namespace

extern "C" int kvc_paged_decode_attention_static(const kvc_geom *g, int32_t layer,
                                                 const kvc_pool *p, const uint16_t *q,
                                                 float softmax_scale, void *out,
                                                 int32_t out_is_fp32, kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    // the size check needs no device: a geometry whose partials exceed the array is refused
    // before anything touches the GPU
    if (DecodeWs(g, false).bytes > size_t(KVC_STATIC_SCRATCH_BYTES)) return KVC_E_WORKSPACE;
    rc = check_pool(p);
    if (rc) return rc;
    if (!q || !out) return KVC_E_NULL;
    void *ws = scratch_of_current_device();
    if (!ws) return KVC_E_HIP;
    return decode_impl(g, layer, p, q, softmax_scale, out, out_is_fp32, nullptr, nullptr, 0, ws,
                       size_t(KVC_STATIC_SCRATCH_BYTES), stream);
}

extern "C" int kvc_paged_decode_attention_acc(const kvc_geom *g, int32_t layer,
                                              const kvc_pool *p, const uint16_t *q,
                                              float softmax_scale, void *out, int32_t out_is_fp32,
                                              float *acc_sum, const int32_t *cu_seqlens,
                                              int32_t max_seqlen, void *ws, size_t ws_bytes,
                                              kvc_stream_t stream) {
    if (!acc_sum || !cu_seqlens) return KVC_E_NULL;
    return decode_impl(g, layer, p, q, softmax_scale, out, out_is_fp32, acc_sum, cu_seqlens,
                       max_seqlen, ws, ws_bytes, stream);
}
