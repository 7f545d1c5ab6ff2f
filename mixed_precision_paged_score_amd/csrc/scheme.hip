// kvc_paged_decode_attention_scheme: decode attention over pages written in a precision
// scheme's layout (kvc_quantize_and_place_scheme: keys slot-major, values channel-major).
//
// DiffKV review page: the free-parameter ledger's comparison of precision schemes (K8V4, K4V8,
// K8V2, K4V2, K2V4, K4V1); "Assumptions" for the attention itself.  Codes enter the matrix
// products as exact fp16 numbers and the per-token scales and zeros are applied around them.
// Keys: 1024 + code, q.k_hat = s_k (q.(1024 + code) - 1024 sum(q)) + z_k sum(q).  Values:
// sum_t p_t v_hat_t = sum_t (p_t s_v) code_t + sum_t p_t z_v, with p s_v split into fp16 hi +
// lo; 2- and 4-bit codes enter as 1024 + 2^(10-b) code against p s_v 2^-(10-b) (an offset of
// 2^b code steps that the fp32 sums remove at the end), other widths as the code itself.
//
// Grid: S workgroup slots per (request, KV head), 4 waves each, with the default decode's
// per-head plan: the head uses SH of them (more for a long head), and its 16-slot tiles (HIGH
// pages, then LOW half-pages) are cut into 4 SH contiguous ranges, one per wave; each wave runs its HIGH tiles, then its LOW tiles, in two loops
// compiled for the tiers' widths.  Per tile, with v_mfma_f32_16x16x32_f16 and operands read
// straight from the page (buffer loads; the next tile's are requested before this tile's
// products): S^T = codes . q^T (lane (c, g): 32 channels of the token in score row c as the
// A operand, query head c's same channels as B; D: query head c, score rows 4 g + r), an
// online softmax per query-head column, and O^T += V^T . P^T with k = the lane's four tokens
// against the high parts of p s_v, then the same tokens against the low parts (A: channel
// 16 dt + c's codes of those tokens, from one 32-bit word of the channel's run).  The four
// waves merge in LDS into the default decode's partials; its combine kernel finishes.
#include <type_traits>

#include "kvc_internal.h"
#include "page_load.h"
#include "workspace.h"

#pragma clang fp contract(off)

namespace kvc {
namespace sch {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = 4;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float MARGIN = 8.0f;
constexpr float VS_LAZY_MAX = 255.875f;   // 65504 / 2^MARGIN
constexpr float M_INIT = -1.0e30f;
constexpr float CODE_OFF = 1024.0f;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ h8 cat(h4 a, h4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}


__device__ __forceinline__ float max_col(float x) {
    uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    u = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// 32 codes of b bits (4 b bytes at offset o of a page, naturally aligned) into w[0 .. b-1]
template <int KB>
__device__ __forceinline__ void load_codes32(__amdgpu_buffer_rsrc_t rs, uint32_t o, int b,
                                             uint32_t (&w)[KB ? KB : 8]) {
    if (KB == 8 || (KB == 0 && b == 8)) {
        const uint4 x = ld16(rs, o), y = ld16(rs, o + 16);
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
        if constexpr (KB == 8 || KB == 0) {
            w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
        }
    } else if (KB == 4 || (KB == 0 && b == 4)) {
        const uint4 x = ld16(rs, o);
        w[0] = x.x;
        if constexpr (KB >= 4 || KB == 0) {
            w[1] = x.y; w[2] = x.z; w[3] = x.w;
        }
    } else if (KB == 2 || (KB == 0 && b == 2)) {
        const uint2 x = ld8(rs, o);
        w[0] = x.x;
        if constexpr (KB >= 2 || KB == 0) w[1] = x.y;
    } else {
        w[0] = ld4(rs, o);
    }
}

// Key operands.  Codes of b < 8 bits enter the score product as the fp16 numbers
// 1024 + 2^(10-b) code (the code in the top bits of the mantissa), 8-bit codes as 1024 + code;
// the tier's key scales are multiplied by key_factor = 2^-(10-b) (exact), so the offset that
// the float32 sums cancel (1024 sum(q)) is 2^b code steps rather than 1024, which keeps the
// cancellation error of narrow keys as small as that of 8-bit ones.
template <int KB>
__device__ __forceinline__ float key_factor(int kb_rt) {
    const int b = KB ? KB : kb_rt;
    return b == 8 ? 1.0f : 1.0f / float(1 << (10 - b));
}
// four b-bit codes starting at bit 0 of w as key operand numbers (an h4 operand)
__device__ __forceinline__ uint2 codes4(uint32_t w, int b) {
    const uint32_t m = (1u << b) - 1u;
    const int t = b == 8 ? 0 : 10 - b;
    const uint32_t c0 = (w & m) << t, c1 = ((w >> b) & m) << t, c2 = ((w >> (2 * b)) & m) << t,
                   c3 = ((w >> (3 * b)) & m) << t;
    return make_uint2((c0 | 0x6400u) | ((c1 | 0x6400u) << 16),
                      (c2 | 0x6400u) | ((c3 | 0x6400u) << 16));
}

template <int N> using ic = std::integral_constant<int, N>;

// For widths known at compile time, codes are converted two at a time: one shift (or
// rotation) and one and-or turn two codes 16 bits apart into an fp16 pair (byte permutes for
// 8-bit codes).  Keys: k-step ks of the score product takes channels key_chan(ks, 0..3) of the
// lane's 32, and the query operand is permuted the same way (once per tier).  Values: the page
// stores each lane's codes in the operand order (channels 16 n + c, slots 4 g + r of a
// 16-slot block, code (n, r) at bit 32 (n / p) + 16 (r % 2) + vb (2 (n % p) + r / 2), p = 8 / vb),
// so one load per tile brings all of them.  Width 0 (run-time widths) converts code by code.
template <int KB>
__device__ __forceinline__ constexpr int key_chan(int ks, int e) {
    if constexpr (KB == 0 || KB == 8) {
        return 4 * ks + e;
    } else {
        constexpr int n = 32 / KB, ppw = 16 / KB, hpw = 8 / KB;
        const int base = (ks / hpw) * n + 2 * (ks % hpw);
        return e == 0 ? base : e == 1 ? base + ppw : e == 2 ? base + 1 : base + 1 + ppw;
    }
}
constexpr uint32_t MAGIC = 0x64006400u;   // fp16 1024 in both halves
__device__ __forceinline__ uint32_t rotr(uint32_t x, uint32_t n) {
    return __builtin_amdgcn_alignbit(x, x, n);
}
// bytes 0, 1 and 2, 3 of x as fp16 pairs (1024 + byte)
__device__ __forceinline__ h4 bytes4(uint32_t x) {
    return __builtin_bit_cast(h4, make_uint2(__builtin_amdgcn_perm(0x64646464u, x, 0x04010400u),
                                             __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)));
}
template <int KB>
__device__ __forceinline__ h4 key_op(const uint32_t (&w)[KB ? KB : 8], int ks, int kb_rt) {
    if constexpr (KB == 8) {
        return bytes4(w[ks]);
    } else if constexpr (KB > 0) {
        // a rotation brings each pair of codes (16 bits apart) to the top of the mantissas
        constexpr int hpw = 8 / KB, T = 10 - KB;
        constexpr uint32_t M = (((1u << KB) - 1u) << T) * 0x00010001u;
        const uint32_t x = w[ks / hpw];
        const int u = ks % hpw;
        return __builtin_bit_cast(h4, make_uint2(
            (rotr(x, uint32_t(2 * KB * u - T) & 31u) & M) | MAGIC,
            (rotr(x, uint32_t(KB * (2 * u + 1) - T) & 31u) & M) | MAGIC));
    } else {
        const uint32_t word = kb_rt == 8 ? w[ks] : kb_rt == 4 ? w[ks >> 1]
                            : kb_rt == 2 ? w[ks >> 2] : w[0];
        return __builtin_bit_cast(h4, codes4(word >> ((4 * ks * kb_rt) & 31), kb_rt));
    }
}
// Value operands.  For 1-, 2- and 4-bit codes a rotation puts a pair of codes in the top bits
// of the fp16 mantissas, 1024 + 2^(10-b) code, and the tier's value scales are multiplied by
// 2^-(10-b) (exact), so a product term is p s_v (2^b + code): the offset that the fp32 sums
// cancel at the end (1024 per unit of the scaled p s_v) is 2^b code steps, not 1024.  8-bit
// and run-time widths convert to 1024 + code and subtract 1024 in fp16 (exact): no offset.
template <int VB>
__device__ __forceinline__ constexpr bool val_offset() { return VB == 1 || VB == 2 || VB == 4; }
template <int VB>
__device__ __forceinline__ constexpr float val_scale() {
    return VB == 4 ? 1.0f / 64.0f : VB == 2 ? 1.0f / 256.0f : VB == 1 ? 1.0f / 512.0f : 1.0f;
}
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t minus1024(uint32_t x) {
    const h2 r = __builtin_bit_cast(h2, x) - h2{(_Float16)1024.0f, (_Float16)1024.0f};
    return __builtin_bit_cast(uint32_t, r);
}
// the lane's value words of one 16-slot block: VB of them (run-time widths: vb)
template <int VB>
__device__ __forceinline__ void load_val_words(__amdgpu_buffer_rsrc_t rs, uint32_t o, int vb,
                                               uint32_t (&w)[VB ? VB : 8]) {
    load_codes32<VB>(rs, o, vb, w);   // 4 vb bytes, naturally aligned: the same shapes as keys
}
// rows r = 0..3 (slots 4 g + r) of channel 16 n + c as an h4 operand
template <int VB>
__device__ __forceinline__ h4 val_op(const uint32_t (&w)[VB ? VB : 8], int n, int vb_rt) {
    if constexpr (VB == 1 || VB == 2 || VB == 4) {
        constexpr int P = 8 / VB, T = 10 - VB;
        constexpr uint32_t M = (((1u << VB) - 1u) << T) * 0x00010001u;
        const uint32_t x = w[n / P];
        const int s0 = VB * 2 * (n % P);
        return __builtin_bit_cast(h4, make_uint2((rotr(x, uint32_t(s0 - T) & 31u) & M) | MAGIC,
                                                 (rotr(x, uint32_t(s0 + VB - T) & 31u) & M) | MAGIC));
    } else if constexpr (VB == 8) {
        // bytes (r0, r2, r1, r3)
        const uint32_t x = w[n];
        return __builtin_bit_cast(h4, make_uint2(
            minus1024(__builtin_amdgcn_perm(0x64646464u, x, 0x04020400u)),
            minus1024(__builtin_amdgcn_perm(0x64646464u, x, 0x04030401u))));
    } else {
        const int vb = vb_rt, p = 8 / vb;
        const uint32_t x = vb == 8 ? w[n] : vb == 4 ? w[n >> 1] : vb == 2 ? w[n >> 2] : w[0];
        const int s0 = vb * 2 * (n % p);
        const uint32_t m = (1u << vb) - 1u;
        const uint32_t c0 = (x >> s0) & m, c2 = (x >> (s0 + vb)) & m;
        const uint32_t c1 = (x >> (s0 + 16)) & m, c3 = (x >> (s0 + vb + 16)) & m;
        return __builtin_bit_cast(h4, make_uint2(minus1024((c0 | 0x6400u) | ((c1 | 0x6400u) << 16)),
                                                 minus1024((c2 | 0x6400u) | ((c3 | 0x6400u) << 16))));
    }
}

// one tile's raw operands: the key codes of row c's slot (the lane's 32 channels), the
// parameters of the lane's four tokens (slots 4 g .. 4 g + 3), and its value words
template <int KB, int VB>
struct Tile {
    uint32_t wk[KB ? KB : 8];
    uint4 pa, pb;
    uint32_t wv[VB ? VB : 8];
    int live;
};

// the four waves' partial results of one workgroup (split sp of head i) merged into the
// default decode's partials: per query head the max m, the sum l and 128 output sums
__device__ __forceinline__ void merge_waves(const float (*s_o)[16][D], const float (*s_m)[16],
                                            const float (*s_l)[16], float *part, int i, int sp,
                                            int S, int G) {
    float *hp = part + int64_t(i) * S * G * PART_STRIDE;
    for (int e = threadIdx.x; e < G * D; e += 64 * WAVES) {
        const int gg = e / D, d = e - gg * D;
        float M = M_INIT;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][gg]);
        float Ls = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_m[w][gg] - M);
            O += s_o[w][gg][d] * f;
            Ls += s_l[w][gg] * f;
        }
        float *pp = hp + (int64_t(sp) * G + gg) * PART_STRIDE;
        if (d == 0) {
            pp[0] = M;
            pp[1] = Ls;
        }
        pp[4 + d] = O;
    }
}

// grid (S * B * Hkv), 256 threads; workgroup x: head x / S, split x % S.  KH, VH, KL, VL: the
// scheme's bit widths when compiled for it (0: taken from the arguments at run time).
template <int KH, int VH, int KL, int VL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void scheme_decode_kernel(
    const uint16_t *__restrict__ q, float scale_log2, const uint8_t *__restrict__ pages,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l, int Hkv, int G,
    int C, int S, int wt, int kh_rt, int vh_rt, int kl_rt, int vl_rt, float *__restrict__ part,
    float *__restrict__ /* lg: no records (groups above 8 heads) */, int64_t /* tiles_cap */) {
    const int kh = KH ? KH : kh_rt, vh = VH ? VH : vh_rt, kl = KL ? KL : kl_rt,
              vl = VL ? VL : vl_rt;
    __shared__ float s_o[WAVES][16][D];
    __shared__ float s_m[WAVES][16], s_l[WAVES][16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int i = blockIdx.x / S;
    const int b = i / Hkv, h = i - b * Hkv;
    const int Hq = Hkv * G;
    const int nh = count_l[2 * i], nl = count_l[2 * i + 1];
    const int SH = active_splits(nh, nl, S, wt);   // the head's workgroups; the rest exit
    const int sp = split_of_slot(blockIdx.x - i * S, i, SH, S);
    if (sp >= SH) return;
    const int qH = ceil_div(nh, HS), tL = ceil_div(nl, 16);
    const int T = qH + tL;
    const int cc = sp * WAVES + wave, NC = SH * WAVES;
    const int t0 = int(int64_t(T) * cc / NC), t1 = int(int64_t(T) * (cc + 1) / NC);
    const int32_t *row = rows_l + int64_t(i) * C;

    // query: the lane's channels 32 g .. 32 g + 31 of query head c (zero beyond G), natural
    // order; each tier's loop permutes them into its key order
    h4 qn[8];
    float sumq = 0.f;
    {
        uint4 u[4] = {};
        if (c < G) {
            const uint4 *qp = reinterpret_cast<const uint4 *>(q + (int64_t(b) * Hq + h * G + c) * D + 32 * g);
            u[0] = qp[0]; u[1] = qp[1]; u[2] = qp[2]; u[3] = qp[3];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            qn[2 * j] = __builtin_bit_cast(h4, make_uint2(u[j].x, u[j].y));
            qn[2 * j + 1] = __builtin_bit_cast(h4, make_uint2(u[j].z, u[j].w));
        }
#pragma unroll
        for (int p = 0; p < 32; ++p) sumq += float(qn[p >> 2][p & 3]);
        sumq += __shfl_xor(sumq, 16, 64);
        sumq += __shfl_xor(sumq, 32, 64);
    }
    const float acc0 = -CODE_OFF * sumq;
    f4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float m = M_INIT, l = 0.f, lz = 0.f, lp = 0.f;

    // tiles [ta, tb) of one tier (HIGH: tile t = page row[t]; LOW: tile t = half t % 2 of page
    // row[C - 1 - t / 2]), two register sets: the next tile's operands are requested before
    // this tile's products
    auto run_tier = [&](int ta, int tb, auto highc, auto kbc, auto vbc) {
        constexpr bool HIGH = decltype(highc)::value;
        constexpr int KB = decltype(kbc)::value, VB = decltype(vbc)::value;
        if (ta >= tb) return;
        const int kb = KB ? KB : (HIGH ? kh : kl), vb = VB ? VB : (HIGH ? vh : vl);
        const float kf = key_factor<KB>(kb);
        constexpr int Sp = HIGH ? HS : LS;
        // 16x16x32 product m2: k-steps 2 m2 and 2 m2 + 1 of the key order
        h8 qop[4];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ch = key_chan<KB>(ks, e);
                qop[ks >> 1][4 * (ks & 1) + e] = qn[ch >> 2][ch & 3];
            }
        auto load = [&](Tile<KB, VB> &r, int t) {
            const int page = HIGH ? row[t] : row[C - 1 - (t >> 1)];
            const uint32_t f = HIGH ? 0u : uint32_t(t & 1);     // 16-slot block of the page
            r.live = min(16, (HIGH ? nh : nl) - 16 * t);
            const __amdgpu_buffer_rsrc_t rs = page_rsrc(pages + int64_t(page) * PAGE);
            load_codes32<KB>(rs, 16 * kb * (16 * f + c) + 4 * g * kb, kb, r.wk);
            r.pa = ld16(rs, PARAM_OFF + 8 * (16 * f + 4 * g));
            r.pb = ld16(rs, PARAM_OFF + 8 * (16 * f + 4 * g + 2));
            load_val_words<VB>(rs, 16 * kb * Sp + 256 * vb * f + 4 * vb * lane, vb, r.wv);
        };
        auto compute = [&](const Tile<KB, VB> &r, int t) {
            f4 acc = f4{acc0, acc0, acc0, acc0};
#pragma unroll
            for (int m2 = 0; m2 < 4; ++m2)
                acc = mfma(cat(key_op<KB>(r.wk, 2 * m2, kb), key_op<KB>(r.wk, 2 * m2 + 1, kb)),
                           qop[m2], acc);
            const uint2 par[4] = {make_uint2(r.pa.x, r.pa.y), make_uint2(r.pa.z, r.pa.w),
                                  make_uint2(r.pb.x, r.pb.y), make_uint2(r.pb.z, r.pb.w)};
            float x[4], vs[4], vz[4];
            float mx = -__builtin_inff();
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float ksc = h2f(uint16_t(par[q4].x & 0xffffu)) * kf;
                const float kz = h2f(uint16_t(par[q4].x >> 16));
                vs[q4] = h2f(uint16_t(par[q4].y & 0xffffu)) * val_scale<VB>();
                vz[q4] = h2f(uint16_t(par[q4].y >> 16));
                const float xv = (ksc * acc[q4] + kz * sumq) * scale_log2;
                x[q4] = 4 * g + q4 < r.live ? xv : -__builtin_inff();
                mx = fmaxf(mx, x[q4]);
            }
            mx = fmaxf(max_col(mx), M_INIT);
            // the branch is uniform; written as a per-lane condition (an opaque lane value that
            // is always 1) the compiler predicates it instead of splitting the accumulators'
            // live ranges, which would copy all 32 of them on the common path
            // P' = p s_v enters the value product as fp16.  For 1-, 2- and 4-bit values the
            // scale carries 2^-(10-b), which keeps P' below 65504 for any fp16 input although
            // the lazy running max lets p reach 2^MARGIN; with unscaled (8-bit or run-time)
            // widths a pair holding a scale above 65504 / 2^MARGIN forces the rescale, after
            // which p <= 1
            bool big = false;
            if constexpr (!val_offset<VB>())
                big = fmaxf(fmaxf(vs[0], vs[1]), fmaxf(vs[2], vs[3])) > VS_LAZY_MAX;
            int one = 1;
            asm volatile("" : "+v"(one));
            if (one && __ballot(mx > m + MARGIN || big) != 0ull) {
                const float mn = fmaxf(m, mx);
                const float corr = __builtin_amdgcn_exp2f(m - mn);
                m = mn;
                l *= corr;
                lz *= corr;
                lp *= corr;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[dt] *= corr;
            }
            _Float16 hi[4], lo[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float p = __builtin_amdgcn_exp2f(x[q4] - m);
                const float pv = p * vs[q4];
                hi[q4] = _Float16(pv);
                lo[q4] = _Float16(pv - float(hi[q4]));
                l += p;
                lz += p * vz[q4];
                if constexpr (val_offset<VB>()) lp += pv;
            }
            // k = 8 g + e: the lane's four tokens with P' = p s_v's fp16 high parts (e < 4),
            // then the same tokens with its low parts (e >= 4)
            const h8 bp = h8{hi[0], hi[1], hi[2], hi[3], lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const h4 a = val_op<VB>(r.wv, dt, vb);
                o[dt] = mfma(cat(a, a), bp, o[dt]);
            }
        };
        // past the tier's last tile the loads repeat it (cache hits), which keeps the loop
        // free of branches around loads and of register copies
        const int tl = tb - 1;
        Tile<KB, VB> ra, rb;
        load(ra, ta);
        for (int t = ta;;) {
            load(rb, min(t + 1, tl));
            compute(ra, t);
            if (++t >= tb) break;
            load(ra, min(t + 1, tl));
            compute(rb, t);
            if (++t >= tb) break;
        }
    };
    run_tier(t0, min(t1, qH), ic<1>{}, ic<KH>{}, ic<VH>{});
    run_tier(max(t0, qH) - qH, t1 - qH, ic<0>{}, ic<KL>{}, ic<VL>{});
    // column sums over the four lane groups, then the four waves' merge
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    lz += __shfl_xor(lz, 16, 64);
    lz += __shfl_xor(lz, 32, 64);
    lp += __shfl_xor(lp, 16, 64);
    lp += __shfl_xor(lp, 32, 64);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            s_o[wave][c][16 * dt + 4 * g + r] = o[dt][r] - CODE_OFF * lp + lz;
    if (g == 0) {
        s_m[wave][c] = m;
        s_l[wave][c] = l;
    }
    __syncthreads();
    merge_waves(s_o, s_m, s_l, part, i, sp, S, G);
}


// Two tiles per pass (query groups of at most 8 heads).  Tile A's scores fill columns 0..7 of
// the score product and tile B's columns 8..15 (query operands qa, qb: the lane's head in
// its half, zero in the other), so every lane's softmax work is useful: lane (c, g) scores
// tokens 4 g + r of tile (c < 8 ? A : B) for query head c % 8, and columns c and c ^ 8 share
// one running max.  O = P . V: A = P with rows c < 8 tile A's heads and c >= 8 tile B's
// (k = 8 g + e: tile A's tokens 4 g + e, then tile B's, the other tile's half zero), B = the
// value codes of channel 16 n + c (tile A's four tokens, then tile B's); rows h and h + 8 of
// O add up at the end.
template <int KB, int VB>
struct PairTiles {
    uint32_t wka[KB ? KB : 8], wkb[KB ? KB : 8];
    uint32_t wva[VB ? VB : 8], wvb[VB ? VB : 8];
    uint4 pa, pb;        // the lane's own tile's parameters (slots 4 g .. 4 g + 3)
    int live;            // the lane's own tile's live tokens
    int tile;            // the lane's own tile (-1: none)
    int ps;              // LG: the position of slot 4 g + (c & 3) of the own tile
};

// LG: also store, per tile of the head (HIGH tiles, then LOW tiles), its 16 slots' positions
// and every token's logit per query head, in the default decode's record layout
// lg [head][tile][16 + G * 16], for the score accumulation
template <int KH, int VH, int KL, int VL, bool LG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void scheme_pair_kernel(
    const uint16_t *__restrict__ q, float scale_log2, const uint8_t *__restrict__ pages,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l, int Hkv, int G,
    int C, int S, int wt, int kh_rt, int vh_rt, int kl_rt, int vl_rt, float *__restrict__ part,
    float *__restrict__ lg, int64_t tiles_cap) {
    const int kh = KH ? KH : kh_rt, vh = VH ? VH : vh_rt, kl = KL ? KL : kl_rt,
              vl = VL ? VL : vl_rt;
    __shared__ float s_o[WAVES][16][D];
    __shared__ float s_m[WAVES][16], s_l[WAVES][16];
    __shared__ uint4 s_q[2][2][4][64];     // [tier: HIGH, LOW][tile A, B][product][lane]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, g = lane >> 4, hc = c & 7;
    const bool own_b = c >= 8;
    const int i = blockIdx.x / S;
    const int b = i / Hkv, h = i - b * Hkv;
    const int Hq = Hkv * G;
    const int nh = count_l[2 * i], nl = count_l[2 * i + 1];
    const int SH = active_splits(nh, nl, S, wt);   // the head's workgroups; the rest exit
    const int sp = split_of_slot(blockIdx.x - i * S, i, SH, S);
    if (sp >= SH) return;
    const int qH = ceil_div(nh, HS), tL = ceil_div(nl, 16);
    const int T = qH + tL;
    const int cc = sp * WAVES + wave, NC = SH * WAVES;
    const int t0 = int(int64_t(T) * cc / NC), t1 = int(int64_t(T) * (cc + 1) / NC);
    const int32_t *row = rows_l + int64_t(i) * C;

    // query head hc's channels 32 g .. 32 g + 31 (zero beyond G); wave 0 stores both tiers'
    // operands in their key orders
    float sumq = 0.f;
    {
        uint4 u[4] = {};
        if (hc < G) {
            const uint4 *qp = reinterpret_cast<const uint4 *>(q + (int64_t(b) * Hq + h * G + hc) * D + 32 * g);
            u[0] = qp[0]; u[1] = qp[1]; u[2] = qp[2]; u[3] = qp[3];
        }
        h4 qn[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            qn[2 * j] = __builtin_bit_cast(h4, make_uint2(u[j].x, u[j].y));
            qn[2 * j + 1] = __builtin_bit_cast(h4, make_uint2(u[j].z, u[j].w));
        }
#pragma unroll
        for (int p = 0; p < 32; ++p) sumq += float(qn[p >> 2][p & 3]);
        sumq += __shfl_xor(sumq, 16, 64);
        sumq += __shfl_xor(sumq, 32, 64);
        if (wave == 0) {
            auto store = [&](int tier, auto kbc) {
                constexpr int KB = decltype(kbc)::value;
#pragma unroll
                for (int m2 = 0; m2 < 4; ++m2) {
                    h8 v;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int ch = key_chan<KB>(2 * m2 + (e >> 2), e & 3);
                        v[e] = qn[ch >> 2][ch & 3];
                    }
                    const uint4 w = __builtin_bit_cast(uint4, v);
                    s_q[tier][0][m2][lane] = own_b ? make_uint4(0, 0, 0, 0) : w;
                    s_q[tier][1][m2][lane] = own_b ? w : make_uint4(0, 0, 0, 0);
                }
            };
            store(0, ic<KH>{});
            store(1, ic<KL>{});
        }
    }
    __syncthreads();
    const float acc0 = -CODE_OFF * sumq;
    f4 o[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] = f4{0.f, 0.f, 0.f, 0.f};
    float m = M_INIT, l = 0.f, lz = 0.f, lp = 0.f;

    // tile pairs (t, t + 1) of tiles [ta, tb) of one tier; a missing tile B repeats tile A's
    // loads with no live token
    auto run_tier = [&](int ta, int tb, auto highc, auto kbc, auto vbc) {
        constexpr bool HIGH = decltype(highc)::value;
        constexpr int KB = decltype(kbc)::value, VB = decltype(vbc)::value;
        constexpr int TIER = HIGH ? 0 : 1;
        if (ta >= tb) return;
        const int kb = KB ? KB : (HIGH ? kh : kl), vb = VB ? VB : (HIGH ? vh : vl);
        const float kf = key_factor<KB>(kb);
        constexpr int Sp = HIGH ? HS : LS;
        const int nt = HIGH ? nh : nl;
        auto page_of = [&](int t) -> const uint8_t * {
            return pages + int64_t(HIGH ? row[t] : row[C - 1 - (t >> 1)]) * PAGE;
        };
        auto block_of = [&](int t) -> uint32_t { return HIGH ? 0u : uint32_t(t & 1); };
        auto load = [&](PairTiles<KB, VB> &r, int t) {
            const int tbb = t + 1 < tb ? t + 1 : t;
            const uint8_t *pga = page_of(t), *pgb = page_of(tbb);
            const uint32_t fa = block_of(t), fb = block_of(tbb);
            const __amdgpu_buffer_rsrc_t ra = page_rsrc(pga), rb = page_rsrc(pgb);
            load_codes32<KB>(ra, 16 * kb * (16 * fa + c) + 4 * g * kb, kb, r.wka);
            load_codes32<KB>(rb, 16 * kb * (16 * fb + c) + 4 * g * kb, kb, r.wkb);
            const uint32_t vo = 16 * kb * Sp + 4 * vb * lane;
            load_val_words<VB>(ra, vo + 256 * vb * fa, vb, r.wva);
            load_val_words<VB>(rb, vo + 256 * vb * fb, vb, r.wvb);
            // the lane's own tile's parameters, read by per-lane address (a buffer descriptor
            // chosen per lane would make the compiler serialize the load over both pages)
            const uint8_t *own = own_b ? pgb : pga;
            const uint4 *op = reinterpret_cast<const uint4 *>(
                own + PARAM_OFF + 8 * (16 * (own_b ? fb : fa) + 4 * g));
            r.pa = op[0];
            r.pb = op[1];
            const int tl = own_b ? (t + 1 < tb ? t + 1 : -1) : t;
            r.live = tl < 0 ? 0 : min(16, nt - 16 * tl);
            r.tile = tl;
            if constexpr (LG) {
                r.ps = -1;
                if (tl >= 0 && hc < 4)
                    r.ps = reinterpret_cast<const int32_t *>(own + POS_OFF)[16 * (own_b ? fb : fa) +
                                                                           4 * g + hc];
            }
        };
        auto compute = [&](const PairTiles<KB, VB> &r) {
            // an opaque lane index keeps the compiler from hoisting the query reads out of the
            // loop (which would pin 32 registers)
            int li = lane;
            asm volatile("" : "+v"(li));
            f4 acc = f4{acc0, acc0, acc0, acc0};
#pragma unroll
            for (int m2 = 0; m2 < 4; ++m2) {
                const h8 qa = __builtin_bit_cast(h8, s_q[TIER][0][m2][li]);
                const h8 qb = __builtin_bit_cast(h8, s_q[TIER][1][m2][li]);
                acc = mfma(cat(key_op<KB>(r.wka, 2 * m2, kb), key_op<KB>(r.wka, 2 * m2 + 1, kb)), qa, acc);
                acc = mfma(cat(key_op<KB>(r.wkb, 2 * m2, kb), key_op<KB>(r.wkb, 2 * m2 + 1, kb)), qb, acc);
            }
            const uint2 par[4] = {make_uint2(r.pa.x, r.pa.y), make_uint2(r.pa.z, r.pa.w),
                                  make_uint2(r.pb.x, r.pb.y), make_uint2(r.pb.z, r.pb.w)};
            float x[4], vs[4], vz[4];
            float mx = -__builtin_inff();
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float ksc = h2f(uint16_t(par[q4].x & 0xffffu)) * kf;
                const float kz = h2f(uint16_t(par[q4].x >> 16));
                vs[q4] = h2f(uint16_t(par[q4].y & 0xffffu)) * val_scale<VB>();
                vz[q4] = h2f(uint16_t(par[q4].y >> 16));
                const float xv = (ksc * acc[q4] + kz * sumq) * scale_log2;
                x[q4] = 4 * g + q4 < r.live ? xv : -__builtin_inff();
                mx = fmaxf(mx, x[q4]);
            }
            if constexpr (LG) {
                if (r.tile >= 0) {
                    float *rec = lg + (int64_t(i) * tiles_cap + (HIGH ? 0 : qH) + r.tile) *
                                          (16 * (G + 1));
                    if (hc < G)
                        *reinterpret_cast<float4 *>(rec + 16 + 16 * hc + 4 * g) =
                            make_float4(x[0], x[1], x[2], x[3]);
                    if (hc < 4) reinterpret_cast<int32_t *>(rec)[4 * g + hc] = r.ps;
                }
            }
            mx = max_col(mx);
            mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0x128, 0xf,
                                                                   0xf, false)));   // row_ror:8
            mx = fmaxf(mx, M_INIT);
            // P' = p s_v enters the value product as fp16.  For 1-, 2- and 4-bit values the
            // scale carries 2^-(10-b), which keeps P' below 65504 for any fp16 input although
            // the lazy running max lets p reach 2^MARGIN; with unscaled (8-bit or run-time)
            // widths a pair holding a scale above 65504 / 2^MARGIN forces the rescale, after
            // which p <= 1
            bool big = false;
            if constexpr (!val_offset<VB>())
                big = fmaxf(fmaxf(vs[0], vs[1]), fmaxf(vs[2], vs[3])) > VS_LAZY_MAX;
            int one = 1;
            asm volatile("" : "+v"(one));
            if (one && __ballot(mx > m + MARGIN || big) != 0ull) {
                const float mn = fmaxf(m, mx);
                const float corr = __builtin_amdgcn_exp2f(m - mn);
                m = mn;
                l *= corr;
                lz *= corr;
                lp *= corr;
                // O's row 4 g + r holds query head (4 g + r) % 8: its factor from that column
                float cr[4];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) cr[r4] = __shfl(corr, (4 * g + r4) & 7, 64);
#pragma unroll
                for (int n = 0; n < 8; ++n)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) o[n][r4] *= cr[r4];
            }
            _Float16 hi[4], lo[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float p = __builtin_amdgcn_exp2f(x[q4] - m);
                const float pv = p * vs[q4];
                hi[q4] = _Float16(pv);
                lo[q4] = _Float16(pv - float(hi[q4]));
                l += p;
                lz += p * vz[q4];
                if constexpr (val_offset<VB>()) lp += pv;
            }
            const h4 z4 = h4{0, 0, 0, 0};
            const h4 ph = h4{hi[0], hi[1], hi[2], hi[3]}, pl = h4{lo[0], lo[1], lo[2], lo[3]};
            const h8 ah = own_b ? cat(z4, ph) : cat(ph, z4);
            const h8 al = own_b ? cat(z4, pl) : cat(pl, z4);
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const h8 bv = cat(val_op<VB>(r.wva, n, vb), val_op<VB>(r.wvb, n, vb));
                o[n] = mfma(ah, bv, o[n]);
                o[n] = mfma(al, bv, o[n]);
            }
        };
        // past the last pair the loads repeat it (cache hits): no branch around a load
        const int tlast = ta + ((tb - 1 - ta) & ~1);
        PairTiles<KB, VB> ra, rb;
        load(ra, ta);
        for (int t = ta;;) {
            load(rb, min(t + 2, tlast));
            compute(ra);
            t += 2;
            if (t >= tb) break;
            load(ra, min(t + 2, tlast));
            compute(rb);
            t += 2;
            if (t >= tb) break;
        }
    };
    run_tier(t0, min(t1, qH), ic<1>{}, ic<KH>{}, ic<VH>{});
    run_tier(max(t0, qH) - qH, t1 - qH, ic<0>{}, ic<KL>{}, ic<VL>{});

    // per query head: sums over the lane groups and the two column halves; O rows h and h + 8
    // (tile A's and tile B's parts of head h) added across the wave's halves
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    l += __shfl_xor(l, 8, 64);
    lz += __shfl_xor(lz, 16, 64);
    lz += __shfl_xor(lz, 32, 64);
    lz += __shfl_xor(lz, 8, 64);
    lp += __shfl_xor(lp, 16, 64);
    lp += __shfl_xor(lp, 32, 64);
    lp += __shfl_xor(lp, 8, 64);
    // per row head (4 g + r) % 8: its sums from that column
    float lzr[4], lpr[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        lzr[r4] = __shfl(lz, (4 * g + r4) & 7, 64);
        lpr[r4] = __shfl(lp, (4 * g + r4) & 7, 64);
    }
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const float other = __shfl_xor(o[n][r4], 32, 64);   // rows 4 g + r + 8
            if (g < 2) s_o[wave][4 * g + r4][16 * n + c] = o[n][r4] + other - CODE_OFF * lpr[r4] + lzr[r4];
        }
    if (g == 0 && c < 8) {
        s_m[wave][c] = m;
        s_l[wave][c] = l;
    }
    __syncthreads();
    merge_waves(s_o, s_m, s_l, part, i, sp, S, G);
}

}  // namespace sch
}  // namespace kvc

using namespace kvc;

namespace {

int scheme_decode_impl(const kvc_geom *g, const kvc_scheme *sc, int32_t layer,
                       const kvc_pool *p, const uint16_t *q, float softmax_scale, void *out,
                       int32_t out_is_fp32, float *acc_sum, const int32_t *cu,
                       int32_t max_seqlen, void *ws, size_t ws_bytes, kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    rc = check_scheme(sc);
    if (rc) return rc;
    if (!q || !out) return KVC_E_NULL;
    const bool accum = acc_sum != nullptr || cu != nullptr;
    if (accum && (!acc_sum || !cu)) return KVC_E_NULL;
    if (!aligned16(q) || !aligned16(out)) return KVC_E_ALIGN;
    if (accum && !aligned16(acc_sum)) return KVC_E_ALIGN;
    if (layer < 0 || layer >= g->num_layers) return KVC_E_SHAPE;
    const int G = g->num_q_heads / g->num_kv_heads;
    if (G > 16) return KVC_E_SHAPE;
    if (accum && G > 8) return KVC_E_UNSUPPORTED;
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
    // the schemes the pages compare are compiled with their widths (others run the generic
    // instance); the accumulating variant runs the same instance with the record stores
    const int key = sc->k_bits_high * 1000 + sc->v_bits_high * 100 + sc->k_bits_low * 10 +
                    sc->v_bits_low;
    // query groups of up to 8 heads take two tiles per pass
    auto kern = accum ? sch::scheme_pair_kernel<0, 0, 0, 0, true>
              : G <= 8 ? sch::scheme_pair_kernel<0, 0, 0, 0, false>
                       : sch::scheme_decode_kernel<0, 0, 0, 0>;
#define KVC_SCHEME_CASE(k, a, b, c2, d)                                                      \
    case k:                                                                                  \
        kern = accum ? sch::scheme_pair_kernel<a, b, c2, d, true>                            \
             : G <= 8 ? sch::scheme_pair_kernel<a, b, c2, d, false>                          \
                      : sch::scheme_decode_kernel<a, b, c2, d>;                              \
        break;
    switch (key) {
        KVC_SCHEME_CASE(8442, 8, 4, 4, 2)
        KVC_SCHEME_CASE(4824, 4, 8, 2, 4)
        KVC_SCHEME_CASE(8241, 8, 2, 4, 1)
        KVC_SCHEME_CASE(4241, 4, 2, 4, 1)
        KVC_SCHEME_CASE(8441, 8, 4, 4, 1)
        KVC_SCHEME_CASE(8424, 8, 4, 2, 4)
        default: break;
    }
#undef KVC_SCHEME_CASE
    hipLaunchKernelGGL(kern, dim3(L.splits * nheads), dim3(256), 0, s, q,
                       softmax_scale * sch::LOG2E, p->pages, rows_l, count_l, Hkv, G, C, L.splits,
                       L.wt, sc->k_bits_high, sc->v_bits_high, sc->k_bits_low, sc->v_bits_low, part,
                       lg, L.tiles_cap);
    rc = launch_check("kvc_paged_decode_attention_scheme/main");
    if (rc) return rc;
    if (accum)
        return launch_combine_and_accumulation(g, p, part, L.splits, L.wt, out, out_is_fp32,
                                               count_l, cu, max_seqlen, acc_sum, w, s);
    return launch_decode_combine(part, g->num_q_heads, G, L.splits, B, out, out_is_fp32, mls,
                                 count_l, L.wt, s);
}

}  // namespace

extern "C" int kvc_paged_decode_attention_scheme(const kvc_geom *g, const kvc_scheme *sc,
                                                 int32_t layer, const kvc_pool *p,
                                                 const uint16_t *q, float softmax_scale,
                                                 void *out, int32_t out_is_fp32, void *ws,
                                                 size_t ws_bytes, kvc_stream_t stream) {
    return scheme_decode_impl(g, sc, layer, p, q, softmax_scale, out, out_is_fp32, nullptr,
                              nullptr, 0, ws, ws_bytes, stream);
}

extern "C" int kvc_paged_decode_attention_scheme_acc(const kvc_geom *g, const kvc_scheme *sc,
                                                     int32_t layer, const kvc_pool *p,
                                                     const uint16_t *q, float softmax_scale,
                                                     void *out, int32_t out_is_fp32,
                                                     float *acc_sum, const int32_t *cu_seqlens,
                                                     int32_t max_seqlen, void *ws,
                                                     size_t ws_bytes, kvc_stream_t stream) {
    if (!acc_sum || !cu_seqlens) return KVC_E_NULL;
    return scheme_decode_impl(g, sc, layer, p, q, softmax_scale, out, out_is_fp32, acc_sum,
                              cu_seqlens, max_seqlen, ws, ws_bytes, stream);
}
