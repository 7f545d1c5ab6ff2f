// kvc_paged_decode_attention_scheme: decode attention over pages written in a precision
// scheme's layout (kvc_quantize_and_place_scheme: keys slot-major, values channel-major).
//
// DiffKV review page: the free-parameter ledger's comparison of precision schemes (K8V4, K4V8,
// K8V2, K4V2, K2V4, K4V1); "Assumptions" for the attention itself.  The arithmetic is the
// default decode's: codes enter the matrix products as the fp16 numbers 1024 + code (exact),
// the offset and the per-token scales and zeros are applied around them:
// q.k_hat = s_k (q.(1024 + code) - 1024 sum(q)) + z_k sum(q), and
// sum_t p_t v_hat_t = sum_t (p_t s_v)(1024 + code_t) - 1024 sum_t p_t s_v + sum_t p_t z_v,
// with p s_v split into fp16 hi + lo.
//
// Grid: S workgroups per (request, KV head) (the default decode's split count), 4 waves each;
// the head's 16-slot tiles (HIGH pages, then LOW half-pages) are cut into 4 S contiguous
// ranges, one per wave.  Per tile, with v_mfma_f32_16x16x16_f16 and operands straight from the
// page: S^T = codes . q^T (lane (c, g): token c's 32 channels 32 g .. 32 g + 31 as the A
// operand, query head c's same channels as B; D: query head c, tokens 4 g + r), an online
// softmax per query-head column, and O^T += V^T . P^T (A: channel 16 dt + c's codes of tokens
// 4 g .. 4 g + 3, one 32-bit word of the channel's run; B: the lane's own P^T entries).  The
// four waves merge in LDS into the default decode's partials; its combine kernel finishes.
#include "kvc_internal.h"
#include "workspace.h"

#pragma clang fp contract(off)

namespace kvc {
namespace sch {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = 4;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float MARGIN = 8.0f;
constexpr float M_INIT = -1.0e30f;
constexpr float CODE_OFF = 1024.0f;

__device__ __forceinline__ f4 mfma(h4 a, h4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max_col(float x) {
    uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    u = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// 32 codes of b bits (4 b bytes at p, naturally aligned) into w[0 .. b-1]
__device__ __forceinline__ void load_codes32(const uint8_t *p, int b, uint32_t (&w)[8]) {
    if (b == 8) {
        const uint4 x = reinterpret_cast<const uint4 *>(p)[0], y = reinterpret_cast<const uint4 *>(p)[1];
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w; w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
    } else if (b == 4) {
        const uint4 x = *reinterpret_cast<const uint4 *>(p);
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    } else if (b == 2) {
        const uint2 x = *reinterpret_cast<const uint2 *>(p);
        w[0] = x.x; w[1] = x.y;
    } else {
        w[0] = *reinterpret_cast<const uint32_t *>(p);
    }
}

// four b-bit codes starting at bit 0 of w as the fp16 numbers 1024 + code (an h4 operand)
__device__ __forceinline__ uint2 codes4(uint32_t w, int b) {
    const uint32_t m = (1u << b) - 1u;
    const uint32_t c0 = w & m, c1 = (w >> b) & m, c2 = (w >> (2 * b)) & m, c3 = (w >> (3 * b)) & m;
    return make_uint2((c0 | 0x6400u) | ((c1 | 0x6400u) << 16),
                      (c2 | 0x6400u) | ((c3 | 0x6400u) << 16));
}

// grid (S * B * Hkv), 256 threads; workgroup x: head x / S, split x % S.  KH, VH, KL, VL: the
// scheme's bit widths when compiled for it (0: taken from the arguments at run time).
template <int KH, int VH, int KL, int VL>
__global__ __launch_bounds__(256) void scheme_decode_kernel(
    const uint16_t *__restrict__ q, float scale_log2, const uint8_t *__restrict__ pages,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l, int Hkv, int G,
    int C, int S, int kh_rt, int vh_rt, int kl_rt, int vl_rt, float *__restrict__ part) {
    const int kh = KH ? KH : kh_rt, vh = VH ? VH : vh_rt, kl = KL ? KL : kl_rt,
              vl = VL ? VL : vl_rt;
    __shared__ float s_o[WAVES][16][D];
    __shared__ float s_m[WAVES][16], s_l[WAVES][16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int i = blockIdx.x / S, sp = blockIdx.x - i * S;
    const int b = i / Hkv, h = i - b * Hkv;
    const int Hq = Hkv * G;
    const int nh = count_l[2 * i], nl = count_l[2 * i + 1];
    const int qH = ceil_div(nh, HS), tL = ceil_div(nl, 16);
    const int T = qH + tL;
    const int cc = sp * WAVES + wave, NC = S * WAVES;
    const int t0 = int(int64_t(T) * cc / NC), t1 = int(int64_t(T) * (cc + 1) / NC);
    const int32_t *row = rows_l + int64_t(i) * C;

    // query operands: column c = query head (zero beyond G), channels 32 g + 4 ks + e
    h4 qop[8];
    float sumq = 0.f;
    {
        uint4 u[4] = {};
        if (c < G) {
            const uint4 *qp = reinterpret_cast<const uint4 *>(q + (int64_t(b) * Hq + h * G + c) * D + 32 * g);
            u[0] = qp[0]; u[1] = qp[1]; u[2] = qp[2]; u[3] = qp[3];
        }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const uint4 &x = u[ks >> 1];
            qop[ks] = __builtin_bit_cast(h4, (ks & 1) ? make_uint2(x.z, x.w) : make_uint2(x.x, x.y));
#pragma unroll
            for (int e = 0; e < 4; ++e) sumq += float(qop[ks][e]);
        }
        sumq += __shfl_xor(sumq, 16, 64);
        sumq += __shfl_xor(sumq, 32, 64);
    }
    const float acc0 = -CODE_OFF * sumq;
    f4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float m = M_INIT, l = 0.f, lz = 0.f, lp = 0.f;

    // one tile's raw operands: key codes of token c (channels 32 g ..), parameters of tokens
    // 4 g .. 4 g + 3, and the value-code words of channels 16 dt + c
    struct Raw {
        uint32_t wk[8];
        uint4 pa, pb;
        uint32_t wv[8];
        int live, kb, vb, vsh;
    };
    auto load_tile = [&](Raw &r, int t) {
        const bool high = t < qH;
        const int page = high ? row[t] : row[C - 1 - ((t - qH) >> 1)];
        const int slot0 = high ? 0 : 16 * ((t - qH) & 1);
        r.live = high ? min(16, nh - 16 * t) : min(16, nl - 16 * (t - qH));
        r.kb = high ? kh : kl;
        r.vb = high ? vh : vl;
        const int Sp = high ? HS : LS;
        const uint8_t *pg = pages + int64_t(page) * PAGE;
        load_codes32(pg + 16 * r.kb * (slot0 + c) + 4 * g * r.kb, r.kb, r.wk);
        r.pa = *reinterpret_cast<const uint4 *>(pg + PARAM_OFF + 8 * (slot0 + 4 * g));
        r.pb = *reinterpret_cast<const uint4 *>(pg + PARAM_OFF + 8 * (slot0 + 4 * g) + 16);
        // 4 vb bits of one naturally aligned word of channel 16 dt + c's run (a 2-byte run,
        // 16 slots of 1 bit, is read as such)
        const int run = Sp * r.vb / 8;
        const uint8_t *vbase = pg + 16 * r.kb * Sp;
        const int vbit = (slot0 + 4 * g) * r.vb;
        r.vsh = vbit & 31;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const uint8_t *vr = vbase + (16 * dt + c) * run;
            r.wv[dt] = run == 2 ? uint32_t(*reinterpret_cast<const uint16_t *>(vr))
                                : *reinterpret_cast<const uint32_t *>(vr + 4 * (vbit >> 5));
        }
    };
    auto compute = [&](const Raw &r) {
        f4 acc = f4{acc0, acc0, acc0, acc0};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            // channels 4 ks .. 4 ks + 3 of the lane's 32: bits 4 ks kb .. of the run; the word
            // index is chosen from the four widths so that every register index is static
            const uint32_t word = r.kb == 8 ? r.wk[ks] : r.kb == 4 ? r.wk[ks >> 1]
                                : r.kb == 2 ? r.wk[ks >> 2] : r.wk[0];
            const h4 a = __builtin_bit_cast(h4, codes4(word >> ((4 * ks * r.kb) & 31), r.kb));
            acc = mfma(a, qop[ks], acc);
        }
        const uint32_t pw[8] = {r.pa.x, r.pa.y, r.pa.z, r.pa.w, r.pb.x, r.pb.y, r.pb.z, r.pb.w};
        float x[4], vs[4], vz[4];
        float mx = -__builtin_inff();
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float ksc = h2f(uint16_t(pw[2 * q4] & 0xffffu));
            const float kz = h2f(uint16_t(pw[2 * q4] >> 16));
            vs[q4] = h2f(uint16_t(pw[2 * q4 + 1] & 0xffffu));
            vz[q4] = h2f(uint16_t(pw[2 * q4 + 1] >> 16));
            x[q4] = 4 * g + q4 < r.live ? (ksc * acc[q4] + kz * sumq) * scale_log2
                                        : -__builtin_inff();
            mx = fmaxf(mx, x[q4]);
        }
        mx = fmaxf(max_col(mx), M_INIT);
        if (__ballot(mx > m + MARGIN) != 0ull) {
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
            lp += pv;
        }
        const h4 bh = h4{hi[0], hi[1], hi[2], hi[3]}, bl = h4{lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const h4 a = __builtin_bit_cast(h4, codes4(r.wv[dt] >> r.vsh, r.vb));
            o[dt] = mfma(a, bh, o[dt]);
            o[dt] = mfma(a, bl, o[dt]);
        }
    };
    // two register sets: the next tile's operands are requested before this tile's products
    if (t0 < t1) {
        Raw ra, rb;
        load_tile(ra, t0);
        for (int t = t0;;) {
            if (t + 1 < t1) load_tile(rb, t + 1);
            compute(ra);
            if (++t >= t1) break;
            if (t + 1 < t1) load_tile(ra, t + 1);
            compute(rb);
            if (++t >= t1) break;
        }
    }
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

}  // namespace sch
}  // namespace kvc

using namespace kvc;

extern "C" int kvc_paged_decode_attention_scheme(const kvc_geom *g, const kvc_scheme *sc,
                                                 int32_t layer, const kvc_pool *p,
                                                 const uint16_t *q, float softmax_scale,
                                                 void *out, int32_t out_is_fp32, void *ws,
                                                 size_t ws_bytes, kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    rc = check_scheme(sc);
    if (rc) return rc;
    if (!q || !out) return KVC_E_NULL;
    if (!aligned16(q) || !aligned16(out)) return KVC_E_ALIGN;
    if (layer < 0 || layer >= g->num_layers) return KVC_E_SHAPE;
    const int G = g->num_q_heads / g->num_kv_heads;
    if (G > 16) return KVC_E_SHAPE;
    DecodeWs L(g, false);
    if (!ws || ws_bytes < L.bytes) return KVC_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return KVC_E_ALIGN;
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + L.part);
    const int B = g->batch, Hkv = g->num_kv_heads, C = g->row_capacity;
    const int nheads = B * Hkv;
    const int32_t *rows_l = p->page_table + int64_t(layer) * nheads * C;
    const int32_t *count_l = p->count + int64_t(layer) * nheads * 2;
    hipStream_t s = (hipStream_t)stream;
    // the schemes the pages compare are compiled with their widths; others run the generic
    // instance
    auto kern = sch::scheme_decode_kernel<0, 0, 0, 0>;
    const int key = sc->k_bits_high * 1000 + sc->v_bits_high * 100 + sc->k_bits_low * 10 +
                    sc->v_bits_low;
    switch (key) {
        case 8442: kern = sch::scheme_decode_kernel<8, 4, 4, 2>; break;
        case 4824: kern = sch::scheme_decode_kernel<4, 8, 2, 4>; break;
        case 8241: kern = sch::scheme_decode_kernel<8, 2, 4, 1>; break;
        case 4241: kern = sch::scheme_decode_kernel<4, 2, 4, 1>; break;
        case 8441: kern = sch::scheme_decode_kernel<8, 4, 4, 1>; break;
        case 8424: kern = sch::scheme_decode_kernel<8, 4, 2, 4>; break;
        default: break;
    }
    hipLaunchKernelGGL(kern, dim3(L.splits * nheads), dim3(256), 0, s, q,
                       softmax_scale * sch::LOG2E, p->pages, rows_l, count_l, Hkv, G, C, L.splits,
                       sc->k_bits_high, sc->v_bits_high, sc->k_bits_low, sc->v_bits_low, part);
    rc = launch_check("kvc_paged_decode_attention_scheme/main");
    if (rc) return rc;
    return launch_decode_combine(part, g->num_q_heads, G, L.splits, B, out, out_is_fp32, nullptr,
                                 s);
}
