// kvc_append_tokens: place one new token per (request, KV head) as K8V4 during decoding.
//
// DiffKV review page, free-parameter ledger: the most recent W tokens are always kept at high
// precision, so a freshly generated token enters its head's HIGH tier; "What carries the
// argument": pages come from the circular free list by prefix sum.  The token takes the next
// HIGH slot (it has the largest position, so slot order stays ascending); a head whose last
// HIGH page is full gets one new page in the same kind of allocation round as
// kvc_compact_pages (grow mode: no head is rebuilt).
//
// Launches: append_demand (counts + 1 HIGH), the three allocation kernels, append_place (one
// wave per head: quantize key and value rows, write the slot; a fresh page is written whole,
// so its empty slots are zero / -1 like every other page).
#include "kvc_internal.h"
#include "quant_row.h"
#include "scheme_io.h"
#include "workspace.h"

#pragma clang fp contract(off)

namespace kvc {

__global__ void append_demand_kernel(const int32_t *__restrict__ count_l,
                                     int32_t *__restrict__ new_count,
                                     uint8_t *__restrict__ changed, int nheads) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nheads) return;
    new_count[2 * i] = count_l[2 * i] + 1;
    new_count[2 * i + 1] = count_l[2 * i + 1];
    changed[i] = 0;
}

constexpr int AP_WAVES = 4;

// wave w of block x appends to head 4x + w.  Lanes 0..15 quantize the key row, lanes 16..31
// the value row (8 channels per lane); lanes 32..63 only help with the whole-page writes.
__global__ __launch_bounds__(64 * AP_WAVES) void append_place_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ positions, int Hkv, int C, int nheads,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l,
    const int32_t *__restrict__ new_count, uint8_t *__restrict__ pages) {
    __shared__ uint8_t s_v[AP_WAVES][D];
    __shared__ uint16_t s_par[AP_WAVES][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = blockIdx.x * AP_WAVES + wave;
    if (i >= nheads) return;
    // the allocation round commits the new count only on success
    if (count_l[2 * i] != new_count[2 * i] || count_l[2 * i + 1] != new_count[2 * i + 1]) return;
    const int b = i / Hkv;
    const int s = count_l[2 * i] - 1;          // the new token's HIGH slot
    const int sp = s & (HS - 1);
    uint8_t *pg = pages + int64_t(rows_l[int64_t(i) * C + (s >> 4)]) * PAGE;
    const int rg = lane >> 4, c = lane & 15;
    const uint16_t *src = (rg == 0 ? K : V) + int64_t(i) * D + 8 * c;
    float x[8];
    load_row8(src, rg < 2, x);
    const RowQ q = row_params(x, rg == 0 ? 255.0f : 15.0f);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) w0 |= code_of(x[e], q) << (8 * e);
#pragma unroll
    for (int e = 0; e < 4; ++e) w1 |= code_of(x[4 + e], q) << (8 * e);
    if (rg == 1) *reinterpret_cast<uint2 *>(&s_v[wave][8 * c]) = make_uint2(w0, w1);
    if (c == 0 && rg < 2) {
        s_par[wave][2 * rg] = q.s16;
        s_par[wave][2 * rg + 1] = q.z16;
    }
    if (sp == 0) {
        // a fresh page: clear it whole first (3456 B = 216 x 16 B)
        for (int k = lane; k < PAGE / 16; k += 64)
            reinterpret_cast<uint4 *>(pg)[k] = make_uint4(0, 0, 0, 0);
        if (lane < LS) reinterpret_cast<int32_t *>(pg + POS_OFF)[lane] = -1;
        __threadfence_block();                  // the clears land before the slot's bytes
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (rg == 0) *reinterpret_cast<uint2 *>(pg + K_OFF + sp * 128 + 8 * c) = make_uint2(w0, w1);
    if (rg == 1) {
        // value unit (j, l = c): this token's nibble of channels 16n + l, n = 0..7
        const int j = sp >> 2, r = sp & 3;
        uint32_t *u = reinterpret_cast<uint32_t *>(pg + V_OFF + 16 * (16 * j + c));
        uint32_t wv[4] = {0u, 0u, 0u, 0u};          // a fresh page holds only this token
        if (sp != 0) {
            const uint4 old = *reinterpret_cast<const uint4 *>(u);
            wv[0] = old.x; wv[1] = old.y; wv[2] = old.z; wv[3] = old.w;
        }
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int sh = 4 * (2 * (n & 1) + (r >> 1) + 4 * (r & 1));
            const uint32_t code = s_v[wave][16 * n + c];
            wv[n >> 1] = (wv[n >> 1] & ~(15u << sh)) | (code << sh);
        }
        *reinterpret_cast<uint4 *>(u) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    if (lane == 32) {
        const uint32_t a = uint32_t(s_par[wave][0]) | (uint32_t(s_par[wave][1]) << 16);
        const uint32_t bb = uint32_t(s_par[wave][2]) | (uint32_t(s_par[wave][3]) << 16);
        *reinterpret_cast<uint2 *>(pg + PARAM_OFF + 8 * sp) = make_uint2(a, bb);
        reinterpret_cast<int32_t *>(pg + POS_OFF)[sp] = positions[b];
    }
}

// The same in a precision scheme's layout (kh-bit keys, vh-bit values for HIGH): lanes 0..15
// quantize the key row, lanes 16..31 the value row; the value codes go through LDS to the 16
// lanes that own the slot's value words (16 n + c, n < 8), which set its codes in place.
__global__ __launch_bounds__(64 * AP_WAVES) void append_place_scheme_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ positions, int Hkv, int C, int nheads,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l,
    const int32_t *__restrict__ new_count, int kh, int vh, uint8_t *__restrict__ pages) {
    __shared__ uint8_t s_v[AP_WAVES][D];
    __shared__ uint16_t s_par[AP_WAVES][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = blockIdx.x * AP_WAVES + wave;
    if (i >= nheads) return;
    if (count_l[2 * i] != new_count[2 * i] || count_l[2 * i + 1] != new_count[2 * i + 1]) return;
    const int b = i / Hkv;
    const int s = count_l[2 * i] - 1;          // the new token's HIGH slot
    const int sp = s & (HS - 1);
    uint8_t *pg = pages + int64_t(rows_l[int64_t(i) * C + (s >> 4)]) * PAGE;
    const int rg = lane >> 4, c = lane & 15;
    const uint16_t *src = (rg == 0 ? K : V) + int64_t(i) * D + 8 * c;
    float x[8];
    load_row8(src, rg < 2, x);
    const RowQ q = row_params(x, float((1 << (rg == 0 ? kh : vh)) - 1));
    uint64_t wk = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) wk |= uint64_t(code_of(x[e], q)) << (kh * e);
    if (rg == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s_v[wave][8 * c + e] = uint8_t(code_of(x[e], q));
    }
    if (c == 0 && rg < 2) {
        s_par[wave][2 * rg] = q.s16;
        s_par[wave][2 * rg + 1] = q.z16;
    }
    if (sp == 0) {
        // a fresh page: clear it whole first (3456 B = 216 x 16 B)
        for (int k = lane; k < PAGE / 16; k += 64)
            reinterpret_cast<uint4 *>(pg)[k] = make_uint4(0, 0, 0, 0);
        if (lane < LS) reinterpret_cast<int32_t *>(pg + POS_OFF)[lane] = -1;
        __threadfence_block();                  // the clears land before the slot's bytes
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (rg == 0) store_codes(pg + 16 * kh * sp + c * kh, wk, kh);
    if (rg == 1) {
        uint32_t vc[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) vc[n] = s_v[wave][16 * n + c];
        sch_set_val_codes(pg, kh, vh, HS, sp, c, vc, sp == 0);
    }
    if (lane == 32) {
        const uint32_t a = uint32_t(s_par[wave][0]) | (uint32_t(s_par[wave][1]) << 16);
        const uint32_t bb = uint32_t(s_par[wave][2]) | (uint32_t(s_par[wave][3]) << 16);
        *reinterpret_cast<uint2 *>(pg + PARAM_OFF + 8 * sp) = make_uint2(a, bb);
        reinterpret_cast<int32_t *>(pg + POS_OFF)[sp] = positions[b];
    }
}

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_append_tokens(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                                 const uint16_t *k_new, const uint16_t *v_new,
                                 const int32_t *positions, void *ws, size_t ws_bytes,
                                 kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    if (!k_new || !v_new || !positions) return KVC_E_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVC_E_ALIGN;
    if (layer < 0 || layer >= g->num_layers) return KVC_E_SHAPE;
    AppendWs L(g);
    if (!ws || ws_bytes < L.bytes) return KVC_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return KVC_E_ALIGN;
    char *w = static_cast<char *>(ws);
    int32_t *new_count = reinterpret_cast<int32_t *>(w + L.new_count);
    uint8_t *changed = reinterpret_cast<uint8_t *>(w + L.changed);
    const int nheads = g->batch * g->num_kv_heads, C = g->row_capacity;
    const int32_t *rows_l = p->page_table + int64_t(layer) * nheads * C;
    const int32_t *count_l = p->count + int64_t(layer) * nheads * 2;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(append_demand_kernel, dim3((nheads + 255) / 256), dim3(256), 0, s, count_l,
                       new_count, changed, nheads);
    rc = launch_check("kvc_append_tokens/demand");
    if (rc) return rc;
    rc = launch_compact(g, layer, p, new_count, changed, nullptr, nullptr, w + L.compact, s);
    if (rc) return rc;
    hipLaunchKernelGGL(append_place_kernel, dim3((nheads + AP_WAVES - 1) / AP_WAVES),
                       dim3(64 * AP_WAVES), 0, s, k_new, v_new, positions, g->num_kv_heads, C,
                       nheads, rows_l, count_l, new_count, p->pages);
    return launch_check("kvc_append_tokens/place");
}

extern "C" int kvc_append_tokens_scheme(const kvc_geom *g, const kvc_scheme *sc, int32_t layer,
                                        const kvc_pool *p, const uint16_t *k_new,
                                        const uint16_t *v_new, const int32_t *positions,
                                        void *ws, size_t ws_bytes, kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    rc = check_scheme(sc);
    if (rc) return rc;
    if (!k_new || !v_new || !positions) return KVC_E_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVC_E_ALIGN;
    if (layer < 0 || layer >= g->num_layers) return KVC_E_SHAPE;
    AppendWs L(g);
    if (!ws || ws_bytes < L.bytes) return KVC_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return KVC_E_ALIGN;
    char *w = static_cast<char *>(ws);
    int32_t *new_count = reinterpret_cast<int32_t *>(w + L.new_count);
    uint8_t *changed = reinterpret_cast<uint8_t *>(w + L.changed);
    const int nheads = g->batch * g->num_kv_heads, C = g->row_capacity;
    const int32_t *rows_l = p->page_table + int64_t(layer) * nheads * C;
    const int32_t *count_l = p->count + int64_t(layer) * nheads * 2;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(append_demand_kernel, dim3((nheads + 255) / 256), dim3(256), 0, s, count_l,
                       new_count, changed, nheads);
    rc = launch_check("kvc_append_tokens_scheme/demand");
    if (rc) return rc;
    rc = launch_compact(g, layer, p, new_count, changed, nullptr, nullptr, w + L.compact, s);
    if (rc) return rc;
    hipLaunchKernelGGL(append_place_scheme_kernel, dim3((nheads + AP_WAVES - 1) / AP_WAVES),
                       dim3(64 * AP_WAVES), 0, s, k_new, v_new, positions, g->num_kv_heads, C,
                       nheads, rows_l, count_l, new_count, sc->k_bits_high, sc->v_bits_high,
                       p->pages);
    return launch_check("kvc_append_tokens_scheme/place");
}
