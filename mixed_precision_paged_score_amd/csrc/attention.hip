// kvc_paged_decode_attention: one decode query per request over mixed-precision pages.
//
// Keys and values are reconstructed on the fly from the unified pages (K8V4 HIGH pages,
// K4V2 LOW pages) as code*scale + zero and attended with a numerically stable online
// softmax.  Each head's live tokens are split across workgroups (split-K); a second kernel
// merges the per-split (max, sum, output) triples in float32.
#include "kvc_internal.h"
#include "workspace.h"

namespace kvc {

constexpr int MAXG = 16;
constexpr float LOG2E = 1.4426950408889634f;

// ---- reference-grade vector path: one wave per (split, KV head, request), 2 channels/lane --
__device__ __forceinline__ uint32_t k_code(const uint8_t *pg, bool high, int slot, int d) {
    if (high) return pg[K_OFF + slot * 128 + d];
    const int w = d >> 3, e = d & 7;
    const int nib = (e >> 1) + 4 * (e & 1);
    const uint32_t word = *reinterpret_cast<const uint32_t *>(pg + K_OFF + slot * 64 + 4 * w);
    return (word >> (4 * nib)) & 15u;
}

__device__ __forceinline__ uint32_t v_code(const uint8_t *pg, bool high, int slot, int d) {
    const int n = d >> 4, l = d & 15;
    if (high) {
        const int j = slot >> 2, r = slot & 3;
        const int q = n >> 1, field = 2 * (n & 1) + (r >> 1) + 4 * (r & 1);
        const uint32_t word =
            *reinterpret_cast<const uint32_t *>(pg + V_OFF + 16 * (16 * j + l) + 4 * q);
        return (word >> (4 * field)) & 15u;
    }
    const int f = slot >> 4, j = (slot & 15) >> 2, r = slot & 3;
    const int q = 2 * f + (n >> 2), field = 2 * (n & 3) + (r >> 1) + 8 * (r & 1);
    const uint32_t word = *reinterpret_cast<const uint32_t *>(pg + V_OFF + 16 * (16 * j + l) + 4 * q);
    return (word >> (2 * field)) & 3u;
}

__global__ __launch_bounds__(64) void decode_vector_kernel(
    const uint16_t *__restrict__ q, float scale, const uint8_t *__restrict__ pages,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l, int Hkv, int G,
    int C, int S, float *__restrict__ part) {
    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int i = b * Hkv + h;
    const int nh = count_l[2 * i], nl = count_l[2 * i + 1];
    const int n = nh + nl;
    const int chunk = (n + S - 1) / S;
    const int u0 = s * chunk, u1 = min(n, u0 + chunk);
    const int Hq = Hkv * G;
    const int d0 = 2 * lane;
    float qf[MAXG][2], o[MAXG][2], m[MAXG], l[MAXG];
    for (int g = 0; g < G; ++g) {
        const uint16_t *qp = q + (int64_t(b) * Hq + h * G + g) * D;
        qf[g][0] = h2f(qp[d0]) * scale * LOG2E;
        qf[g][1] = h2f(qp[d0 + 1]) * scale * LOG2E;
        o[g][0] = o[g][1] = 0.0f;
        m[g] = -__builtin_inff();
        l[g] = 0.0f;
    }
    const int32_t *row = rows_l + int64_t(i) * C;
    for (int u = u0; u < u1; ++u) {
        const bool high = u < nh;
        const int su = high ? u : u - nh;
        const int slot = high ? (su & 15) : (su & 31);
        const int page = high ? row[su >> 4] : row[C - 1 - (su >> 5)];
        const uint8_t *pg = pages + int64_t(page) * PAGE;
        const uint16_t *par = reinterpret_cast<const uint16_t *>(pg + PARAM_OFF + 8 * slot);
        const float ks = h2f(par[0]), kz = h2f(par[1]), vs = h2f(par[2]), vz = h2f(par[3]);
        const float k0 = fmaf(float(k_code(pg, high, slot, d0)), ks, kz);
        const float k1 = fmaf(float(k_code(pg, high, slot, d0 + 1)), ks, kz);
        const float v0 = fmaf(float(v_code(pg, high, slot, d0)), vs, vz);
        const float v1 = fmaf(float(v_code(pg, high, slot, d0 + 1)), vs, vz);
        for (int g = 0; g < G; ++g) {
            float dot = qf[g][0] * k0 + qf[g][1] * k1;
#pragma unroll
            for (int msk = 32; msk >= 1; msk >>= 1) dot += __shfl_xor(dot, msk, 64);
            const float mn = fmaxf(m[g], dot);
            const float corr = exp2f(m[g] - mn);
            const float p = exp2f(dot - mn);
            l[g] = l[g] * corr + p;
            o[g][0] = o[g][0] * corr + p * v0;
            o[g][1] = o[g][1] * corr + p * v1;
            m[g] = mn;
        }
    }
    for (int g = 0; g < G; ++g) {
        float *pp = part + ((int64_t(b) * Hq + h * G + g) * S + s) * PART_STRIDE;
        if (lane == 0) {
            pp[0] = m[g];
            pp[1] = l[g];
        }
        pp[4 + d0] = o[g][0];
        pp[4 + d0 + 1] = o[g][1];
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
            const float w = exp2f(pp[s * PART_STRIDE] - M);
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
    if (G > MAXG) return KVC_E_SHAPE;
    DecodeWs L(g);
    if (!ws || ws_bytes < L.bytes) return KVC_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return KVC_E_ALIGN;
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + L.part);
    const int B = g->batch, Hkv = g->num_kv_heads, C = g->row_capacity;
    const int nheads = B * Hkv;
    const int32_t *rows_l = p->page_table + int64_t(layer) * nheads * C;
    const int32_t *count_l = p->count + int64_t(layer) * nheads * 2;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(decode_vector_kernel, dim3(L.splits, Hkv, B), dim3(64), 0, s, q,
                       softmax_scale, p->pages, rows_l, count_l, Hkv, G, C, L.splits, part);
    rc = launch_check("kvc_paged_decode_attention/main");
    if (rc) return rc;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(g->num_q_heads, B), dim3(128), 0, s, part,
                       g->num_q_heads, L.splits, out, out_is_fp32);
    return launch_check("kvc_paged_decode_attention/combine");
}
