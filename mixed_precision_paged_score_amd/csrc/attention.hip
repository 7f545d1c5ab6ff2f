// kvc_paged_decode_attention: one decode query per request over mixed-precision pages.
//
// Keys and values are reconstructed on the fly from the unified pages (K8V4 HIGH pages,
// K4V2 LOW pages) as code*scale + zero and attended with an online softmax (DiffKV review
// page: the memory manager serves attention over the compressed paged cache; "Assumptions"
// lists standard causal multi-head attention, the page's Eq. 1).
//
// Matrix-core design (gfx950, wave64, v_mfma_f32_16x16x16_f16):
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
//   * the running max is only moved when a tile exceeds it by more than 2^8 (in log2 units),
//     so the accumulator rescale (a cross-lane shuffle) is rare;
//   * four waves per workgroup take consecutive slices of one head's tiles (balanced by
//     bytes: a HIGH tile counts twice a LOW tile) and merge in LDS; a second kernel merges
//     the workgroups' (max, sum, output) partials of each query head in float32.
#include "kvc_internal.h"
#include "workspace.h"

namespace kvc {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_MARGIN = 8.0f;      // log2 units
constexpr int DEC_WAVES = 4;
constexpr float MAGIC = 1024.0f;

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ h4 cat(h2 a, h2 b) { return h4{a[0], a[1], b[0], b[1]}; }
__device__ __forceinline__ f4 mfma16(h4 a, h4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// raw per-lane bytes of one tile
struct Tile {
    uint4 k0, k1;      // HIGH: 32 key bytes (8-bit codes); LOW: k0 = 16 key bytes (4-bit)
    uint4 v;           // HIGH: value unit (4 words); LOW: v.x, v.y = this half's 2 words
    uint4 p0, p1;      // parameters of the lane group's 4 tokens (8 bytes each)
};

struct TileRef {
    const uint8_t *pg;
    int high, f, live;  // f: half of a LOW page (slots 16f..16f+15)
};

__device__ __forceinline__ TileRef tile_ref(int u, int qH, int nh, int nl,
                                            const int32_t *row, int C,
                                            const uint8_t *pages) {
    TileRef t;
    if (u < qH) {
        t.high = 1;
        t.f = 0;
        t.live = min(HS, nh - HS * u);
        t.pg = pages + int64_t(row[u]) * PAGE;
    } else {
        const int v = u - qH, lp = v >> 1;
        t.high = 0;
        t.f = v & 1;
        t.live = min(16, nl - LS * lp - 16 * t.f);
        t.pg = pages + int64_t(row[C - 1 - lp]) * PAGE;
    }
    return t;
}

__device__ __forceinline__ Tile load_tile(const TileRef &t, int lane) {
    const int j = lane >> 4, tok = lane & 15;
    Tile d;
    if (t.high) {
        const uint4 *kp = reinterpret_cast<const uint4 *>(t.pg + K_OFF + tok * 128 + 32 * j);
        d.k0 = kp[0];
        d.k1 = kp[1];
        d.v = *reinterpret_cast<const uint4 *>(t.pg + V_OFF + 16 * lane);
        const uint4 *pp = reinterpret_cast<const uint4 *>(t.pg + PARAM_OFF + 32 * j);
        d.p0 = pp[0];
        d.p1 = pp[1];
    } else {
        const int slot = 16 * t.f + tok;
        d.k0 = *reinterpret_cast<const uint4 *>(t.pg + K_OFF + slot * 64 + 16 * j);
        d.k1 = make_uint4(0, 0, 0, 0);
        const uint2 vv = *reinterpret_cast<const uint2 *>(t.pg + V_OFF + 16 * lane + 8 * t.f);
        d.v = make_uint4(vv.x, vv.y, 0, 0);
        const uint4 *pp = reinterpret_cast<const uint4 *>(t.pg + PARAM_OFF + 8 * (16 * t.f + 4 * j));
        d.p0 = pp[0];
        d.p1 = pp[1];
    }
    return d;
}

// key operand of MFMA m: channels 32j + 4m + {0, 2, 1, 3} of the lane's token, as 1024 + code
__device__ __forceinline__ h4 key_operand(const Tile &d, int high, int m) {
    if (high) {
        const uint32_t w = m == 0 ? d.k0.x : m == 1 ? d.k0.y : m == 2 ? d.k0.z : m == 3 ? d.k0.w
                         : m == 4 ? d.k1.x : m == 5 ? d.k1.y : m == 6 ? d.k1.z : d.k1.w;
        const uint32_t a = (w & 0x00FF00FFu) | 0x64006400u;          // channels 0, 2
        const uint32_t b = ((w >> 8) & 0x00FF00FFu) | 0x64006400u;   // channels 1, 3
        return cat(as_h2(a), as_h2(b));
    }
    const uint32_t w = (m >> 1) == 0 ? d.k0.x : (m >> 1) == 1 ? d.k0.y : (m >> 1) == 2 ? d.k0.z : d.k0.w;
    const int sh = 8 * (m & 1);
    const uint32_t a = ((w >> sh) & 0x000F000Fu) | 0x64006400u;        // channels 0, 2
    const uint32_t b = ((w >> (sh + 4)) & 0x000F000Fu) | 0x64006400u;  // channels 1, 3
    return cat(as_h2(a), as_h2(b));
}

// value operand of MFMA n: tokens 4j + {0,1,2,3} of channel 16n + (lane & 15), as the exact
// code (1024 + code built by the bit trick, then 1024 subtracted exactly in fp16: the output
// is a small difference of large sums, so the offset must not reach the accumulator)
__device__ __forceinline__ h4 value_operand(const Tile &d, int high, int n) {
    const h2 off = {_Float16(MAGIC), _Float16(MAGIC)};
    uint32_t a, b;
    if (high) {
        const uint32_t w = (n >> 1) == 0 ? d.v.x : (n >> 1) == 1 ? d.v.y : (n >> 1) == 2 ? d.v.z : d.v.w;
        const int sh = 8 * (n & 1);
        a = ((w >> sh) & 0x000F000Fu) | 0x64006400u;
        b = ((w >> (sh + 4)) & 0x000F000Fu) | 0x64006400u;
    } else {
        const uint32_t w = (n >> 2) == 0 ? d.v.x : d.v.y;
        const int sh = 4 * (n & 3);
        a = ((w >> sh) & 0x00030003u) | 0x64006400u;
        b = ((w >> (sh + 2)) & 0x00030003u) | 0x64006400u;
    }
    return cat(as_h2(a) - off, as_h2(b) - off);
}

__device__ __forceinline__ float half_lo(uint32_t u) { return h2f(uint16_t(u & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t u) { return h2f(uint16_t(u >> 16)); }

struct WaveState {
    f4 o[8];                  // O[g = 4j + r][16n + (lane & 15)], n = 0..7
    float m, l, lz;           // per column g = lane & 15: running max (log2), sums
};

__global__ __launch_bounds__(64 * DEC_WAVES) void decode_mfma_kernel(
    const uint16_t *__restrict__ q, float scale_log2, const uint8_t *__restrict__ pages,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l, int Hkv, int G,
    int C, int S, float *__restrict__ part) {
    __shared__ float s_o[DEC_WAVES][32][64];
    __shared__ float s_m[DEC_WAVES][16], s_l[DEC_WAVES][16], s_lz[DEC_WAVES][16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane & 15, j = lane >> 4;
    // block -> (split, KV head, request)
    const int s = blockIdx.x % S;
    const int i = blockIdx.x / S;             // head index b*Hkv + h
    const int b = i / Hkv, h = i - b * Hkv;
    const int Hq = Hkv * G;
    const int nh = count_l[2 * i], nl = count_l[2 * i + 1];
    const int qH = ceil_div(nh, HS);
    const int tL = ceil_div(nl, 16);
    const int64_t W = 2 * int64_t(qH) + tL;   // work units: HIGH tile 2, LOW tile 1
    const int NC = S * DEC_WAVES;
    const int c = s * DEC_WAVES + wave;
    auto tile_of = [&](int64_t x) -> int {
        return x <= 2 * int64_t(qH) ? int((x + 1) >> 1) : qH + int(x - 2 * int64_t(qH));
    };
    const int u0 = tile_of(W * c / NC), u1 = tile_of(W * (c + 1) / NC);

    // query operand: lane (g, j) holds q[g][32j + 4m + {0,2,1,3}] for m = 0..7
    h4 qop[8];
    float sumq = 0.0f;
    {
        uint4 qa[4] = {};
        if (g < G) {
            const uint4 *qp = reinterpret_cast<const uint4 *>(q + (int64_t(b) * Hq + h * G + g) * D + 32 * j);
            qa[0] = qp[0]; qa[1] = qp[1]; qa[2] = qp[2]; qa[3] = qp[3];
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint4 &u = qa[m >> 1];
            const uint32_t w0 = (m & 1) ? u.z : u.x, w1 = (m & 1) ? u.w : u.y;  // ch 0,1 | 2,3
            const h2 a = as_h2(w0), bq = as_h2(w1);
            qop[m] = h4{a[0], bq[0], a[1], bq[1]};
            sumq += float(a[0]) + float(a[1]) + float(bq[0]) + float(bq[1]);
        }
        sumq += __shfl_xor(sumq, 16, 64);
        sumq += __shfl_xor(sumq, 32, 64);
    }

    WaveState st;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = f4{0.f, 0.f, 0.f, 0.f};
    st.m = -__builtin_inff();
    st.l = st.lz = 0.0f;

    const int32_t *row = rows_l + int64_t(i) * C;
    if (u0 < u1) {
        TileRef tr = tile_ref(u0, qH, nh, nl, row, C, pages);
        Tile cur = load_tile(tr, lane);
        for (int u = u0; u < u1; ++u) {
            const TileRef trc = tr;
            Tile nxt = cur;
            if (u + 1 < u1) {
                tr = tile_ref(u + 1, qH, nh, nl, row, C, pages);
                nxt = load_tile(tr, lane);
            }
            // ---- S^T = K * Q^T (codes offset by 1024) -------------------------------------
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 8; ++m) acc = mfma16(key_operand(cur, trc.high, m), qop[m], acc);
            const uint32_t pw[8] = {cur.p0.x, cur.p0.y, cur.p0.z, cur.p0.w,
                                    cur.p1.x, cur.p1.y, cur.p1.z, cur.p1.w};
            float L[4], vs[4], vz[4];
            float tmax = -__builtin_inff();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ks = half_lo(pw[2 * r]), kz = half_hi(pw[2 * r]);
                vs[r] = half_lo(pw[2 * r + 1]);
                vz[r] = half_hi(pw[2 * r + 1]);
                const float dot = acc[r] - MAGIC * sumq;           // q . code
                const float x = (ks * dot + kz * sumq) * scale_log2;
                L[r] = (4 * j + r < trc.live) ? x : -__builtin_inff();
                tmax = fmaxf(tmax, L[r]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            // ---- lazy rescale of the running max --------------------------------------------
            if (__ballot(tmax > st.m + RESCALE_MARGIN) != 0ull) {
                const float mn = fmaxf(st.m, tmax);
                const float corr = (st.m == -__builtin_inff()) ? 0.0f : exp2f(st.m - mn);
                st.l *= corr;
                st.lz *= corr;
                st.m = mn;
                float cr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * j + r, 64);
#pragma unroll
                for (int n = 0; n < 8; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r) st.o[n][r] *= cr[r];
            }
            // ---- P' = p * scale_v as fp16 hi + lo ---------------------------------------------
            h4 phi, plo;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = (L[r] == -__builtin_inff()) ? 0.0f : exp2f(L[r] - st.m);
                const float pv = p * vs[r];
                const _Float16 hi = _Float16(pv);
                const _Float16 lo = _Float16(pv - float(hi));
                phi[r] = hi;
                plo[r] = lo;
                st.l += p;
                st.lz += p * vz[r];
            }
            // ---- O += P' * V_codes ----------------------------------------------------------
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const h4 vop = value_operand(cur, trc.high, n);
                st.o[n] = mfma16(phi, vop, st.o[n]);
                st.o[n] = mfma16(plo, vop, st.o[n]);
            }
            cur = nxt;
        }
    }
    // column sums over the four lane groups
    st.l += __shfl_xor(st.l, 16, 64);
    st.l += __shfl_xor(st.l, 32, 64);
    st.lz += __shfl_xor(st.lz, 16, 64);
    st.lz += __shfl_xor(st.lz, 32, 64);
    // ---- merge the four waves in LDS and write this workgroup's partial --------------------
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_o[wave][4 * n + r][lane] = st.o[n][r];
    if (lane < 16) {
        s_m[wave][lane] = st.m;
        s_l[wave][lane] = st.l;
        s_lz[wave][lane] = st.lz;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < G * D; e += 64 * DEC_WAVES) {
        const int gg = e / D, d = e - gg * D;
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, s_m[w][gg]);
        float Ls = 0.0f, O = 0.0f;
        if (M != -__builtin_inff()) {
            const int n = d >> 4, dl = d & 15, jj = gg >> 2, r = gg & 3;
#pragma unroll
            for (int w = 0; w < DEC_WAVES; ++w) {
                const float mw = s_m[w][gg];
                if (mw == -__builtin_inff()) continue;
                const float f = exp2f(mw - M);
                const float ow = s_o[w][4 * n + r][16 * jj + dl] + s_lz[w][gg];
                O += ow * f;
                Ls += s_l[w][gg] * f;
            }
        }
        float *pp = part + ((int64_t(b) * Hq + h * G + gg) * S + s) * PART_STRIDE;
        if (d == 0) {
            pp[0] = M;
            pp[1] = Ls;
        }
        pp[4 + d] = O;
    }
}

// merge the S partials of one (request, query head); m is in log2 units
__global__ __launch_bounds__(128) void decode_combine_kernel(const float *__restrict__ part,
                                                             int Hq, int S, void *out,
                                                             int out_fp32) {
    const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const float *pp = part + (int64_t(b) * Hq + hq) * S * PART_STRIDE;
    float M = -__builtin_inff();
    for (int s = 0; s < S; ++s) M = fmaxf(M, pp[s * PART_STRIDE]);
    float L = 0.0f, O = 0.0f;
    if (M != -__builtin_inff()) {
        for (int s = 0; s < S; ++s) {
            const float ms = pp[s * PART_STRIDE];
            if (ms == -__builtin_inff()) continue;
            const float w = exp2f(ms - M);
            L += pp[s * PART_STRIDE + 1] * w;
            O += pp[s * PART_STRIDE + 4 + d] * w;
        }
    }
    const float r = L > 0.0f ? O / L : 0.0f;
    const int64_t idx = (int64_t(b) * Hq + hq) * D + d;
    if (out_fp32) static_cast<float *>(out)[idx] = r;
    else static_cast<uint16_t *>(out)[idx] = f2h_rn(r);
}

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_paged_decode_attention(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                                          const uint16_t *q, float softmax_scale, void *out,
                                          int32_t out_is_fp32, void *ws, size_t ws_bytes,
                                          kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    if (!q || !out) return KVC_E_NULL;
    if (!aligned16(q) || !aligned16(out)) return KVC_E_ALIGN;
    if (layer < 0 || layer >= g->num_layers) return KVC_E_SHAPE;
    const int G = g->num_q_heads / g->num_kv_heads;
    if (G > 16) return KVC_E_SHAPE;
    DecodeWs L(g);
    if (!ws || ws_bytes < L.bytes) return KVC_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return KVC_E_ALIGN;
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + L.part);
    const int B = g->batch, Hkv = g->num_kv_heads, C = g->row_capacity;
    const int nheads = B * Hkv;
    const int32_t *rows_l = p->page_table + int64_t(layer) * nheads * C;
    const int32_t *count_l = p->count + int64_t(layer) * nheads * 2;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(decode_mfma_kernel, dim3(L.splits * nheads), dim3(64 * DEC_WAVES), 0, s,
                       q, softmax_scale * LOG2E, p->pages, rows_l, count_l, Hkv, G, C, L.splits,
                       part);
    rc = launch_check("kvc_paged_decode_attention/main");
    if (rc) return rc;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(g->num_q_heads, B), dim3(128), 0, s, part,
                       g->num_q_heads, L.splits, out, out_is_fp32);
    return launch_check("kvc_paged_decode_attention/combine");
}
