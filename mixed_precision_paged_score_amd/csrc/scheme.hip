// kvc_paged_decode_attention_scheme: decode attention over pages written in a precision
// scheme's slot-major layout (kvc_quantize_and_place_scheme).
//
// DiffKV review page: the free-parameter ledger's comparison of precision schemes (K8V4, K4V8,
// K8V2, K4V2, K2V4, K4V1); "Assumptions" for the attention itself.  The arithmetic is the
// default decode's: keys and values enter the matrix products as their integer codes (exact in
// fp16), the per-token scales and zeros are applied around them: q.k_hat = s_k (q.code) +
// z_k sum(q), and sum_t p_t v_hat_t = sum_t (p_t s_v) code_t + sum_t p_t z_v with p s_v split
// into fp16 hi + lo.
//
// Grid: S workgroups per (request, KV head) (the default decode's split count), 4 waves each;
// the head's 16-slot tiles (HIGH pages, then LOW half-pages) are cut into 4 S contiguous
// ranges, one per wave.  Per tile a wave unpacks the codes into its own LDS area (keys
// row-major, values transposed), then S^T = codes . q^T with v_mfma_f32_16x16x16_f16 (lane:
// query head column c, tokens 4g + r), an online softmax per column, and O^T += V^T . P^T.
// The four waves merge in LDS into the default decode's partials; its combine kernel finishes.
#include "kvc_internal.h"
#include "workspace.h"

#pragma clang fp contract(off)

namespace kvc {
namespace sch {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = 4;
constexpr int KR = D + 8;          // LDS key code row stride (halves)
constexpr int VR = 16 + 4;         // LDS transposed value code row stride (halves)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float MARGIN = 8.0f;
constexpr float M_INIT = -1.0e30f;

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

// 32 codes of b bits (4 b bytes at p, 4-byte aligned) into w[0 .. b-1]
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
__device__ __forceinline__ _Float16 code_at(const uint32_t (&w)[8], int b, int e) {
    const int bit = b * e;
    const uint32_t word = w[bit >> 5];
    return _Float16(float((word >> (bit & 31)) & ((1u << b) - 1u)));
}

struct WaveLds {
    _Float16 k[16 * KR];       // key codes [token][channel]
    _Float16 vt[D * VR];       // value codes [channel][token]
    float par[16][4];          // k scale, k zero, v scale, v zero
};

// grid (S * B * Hkv), 256 threads; workgroup x: head x / S, split x % S
__global__ __launch_bounds__(256) void scheme_decode_kernel(
    const uint16_t *__restrict__ q, float scale_log2, const uint8_t *__restrict__ pages,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l, int Hkv, int G,
    int C, int S, int kh, int vh, int kl, int vl, float *__restrict__ part) {
    __shared__ WaveLds s_w[WAVES];
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
    WaveLds &L = s_w[wave];

    // query operands: column c = query head (zero beyond G), dims 16 ks + 4 g + e
    h4 qop[8];
    float sumq = 0.f;
    {
        const uint16_t *qp = q + (int64_t(b) * Hq + h * G + c) * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            uint2 u = make_uint2(0, 0);
            if (c < G) u = *reinterpret_cast<const uint2 *>(qp + 16 * ks + 4 * g);
            qop[ks] = __builtin_bit_cast(h4, u);
#pragma unroll
            for (int e = 0; e < 4; ++e) sumq += float(qop[ks][e]);
        }
        sumq += __shfl_xor(sumq, 16, 64);
        sumq += __shfl_xor(sumq, 32, 64);
    }
    f4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float m = M_INIT, l = 0.f, lz = 0.f;

    for (int t = t0; t < t1; ++t) {
        const bool high = t < qH;
        const int page = high ? row[t] : row[C - 1 - ((t - qH) >> 1)];
        const int slot0 = high ? 0 : 16 * ((t - qH) & 1);
        const int live = high ? min(16, nh - 16 * t) : min(16, nl - 16 * (t - qH));
        const int kb = high ? kh : kl, vb = high ? vh : vl;
        const int sbytes = 16 * (kb + vb);
        const uint8_t *pg = pages + int64_t(page) * PAGE;
        // unpack: lane (slot sl = lane / 4, quarter qq = lane % 4) takes channels 32 qq .. + 31
        {
            const int sl = lane >> 2, qq = lane & 3;
            const uint8_t *base = pg + (slot0 + sl) * sbytes;
            uint32_t wk[8], wv[8];
            load_codes32(base + 4 * qq * kb, kb, wk);
            load_codes32(base + 16 * kb + 4 * qq * vb, vb, wv);
            _Float16 *kd = L.k + sl * KR + 32 * qq;
#pragma unroll
            for (int e4 = 0; e4 < 8; ++e4) {
                const h4 x = h4{code_at(wk, kb, 4 * e4), code_at(wk, kb, 4 * e4 + 1),
                                code_at(wk, kb, 4 * e4 + 2), code_at(wk, kb, 4 * e4 + 3)};
                *reinterpret_cast<h4 *>(kd + 4 * e4) = x;
            }
#pragma unroll
            for (int e = 0; e < 32; ++e) L.vt[(32 * qq + e) * VR + sl] = code_at(wv, vb, e);
            if (qq == 0) {
                const uint2 pr = *reinterpret_cast<const uint2 *>(pg + PARAM_OFF + 8 * (slot0 + sl));
                L.par[sl][0] = h2f(uint16_t(pr.x & 0xffffu));
                L.par[sl][1] = h2f(uint16_t(pr.x >> 16));
                L.par[sl][2] = h2f(uint16_t(pr.y & 0xffffu));
                L.par[sl][3] = h2f(uint16_t(pr.y >> 16));
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // S^T = codes . q^T: lane (c, g) holds tokens 4 g + r of query head c
        f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const h4 a = *reinterpret_cast<const h4 *>(L.k + c * KR + 16 * ks + 4 * g);
            acc = mfma(a, qop[ks], acc);
        }
        float x[4], vs[4], vz[4];
        float mx = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tk = 4 * g + r;
            const float ksc = L.par[tk][0], kz = L.par[tk][1];
            vs[r] = L.par[tk][2];
            vz[r] = L.par[tk][3];
            x[r] = tk < live ? (ksc * acc[r] + kz * sumq) * scale_log2 : -__builtin_inff();
            mx = fmaxf(mx, x[r]);
        }
        mx = fmaxf(max_col(mx), M_INIT);
        if (__ballot(mx > m + MARGIN) != 0ull) {
            const float mn = fmaxf(m, mx);
            const float corr = __builtin_amdgcn_exp2f(m - mn);
            m = mn;
            l *= corr;
            lz *= corr;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) o[dt] *= corr;
        }
        _Float16 hi[4], lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(x[r] - m);
            const float pv = p * vs[r];
            hi[r] = _Float16(pv);
            lo[r] = _Float16(pv - float(hi[r]));
            l += p;
            lz += p * vz[r];
        }
        const h4 bh = h4{hi[0], hi[1], hi[2], hi[3]}, bl = h4{lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const h4 a = *reinterpret_cast<const h4 *>(L.vt + (16 * dt + c) * VR + 4 * g);
            o[dt] = mfma(a, bh, o[dt]);
            o[dt] = mfma(a, bl, o[dt]);
        }
        // the next tile's unpack overwrites this wave's LDS area
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // column sums over the four lane groups, then the four waves' merge
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    lz += __shfl_xor(lz, 16, 64);
    lz += __shfl_xor(lz, 32, 64);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_o[wave][c][16 * dt + 4 * g + r] = o[dt][r] + lz;
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
    hipLaunchKernelGGL(sch::scheme_decode_kernel, dim3(L.splits * nheads), dim3(256), 0, s, q,
                       softmax_scale * sch::LOG2E, p->pages, rows_l, count_l, Hkv, G, C, L.splits,
                       sc->k_bits_high, sc->v_bits_high, sc->k_bits_low, sc->v_bits_low, part);
    rc = launch_check("kvc_paged_decode_attention_scheme/main");
    if (rc) return rc;
    return launch_decode_combine(part, g->num_q_heads, G, L.splits, B, out, out_is_fp32, nullptr,
                                 s);
}
