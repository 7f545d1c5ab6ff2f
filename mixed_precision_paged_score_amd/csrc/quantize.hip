// kvc_quantize_and_place (prompt mode): K8V4 / K4V2 codes written into unified pages.
//
// DiffKV review page, "Core claim": important tokens are stored as K8V4, moderately
// important ones as K4V2, both tiers in one unified page format.  The per-token quantizer
// is asymmetric min/max over the 128 channels of a key or value row, in float32 with
// round-to-nearest-even, scale and zero stored as fp16.
//
// Four launches on the caller's stream:
//   1. quant_count   per (request, 256-token tile): #HIGH and #LOW per KV head (LDS atomics)
//   2. quant_scan    per (request, KV head): exclusive prefix of the tile counts; checks the
//                    totals against the pool's counts (mismatch: head skipped, status bit)
//   3. quant_select  per tile and head: a wave ranks the tile's tokens of each tier with
//                    64-lane ballots and writes the token positions into a per-head list
//                    (HIGH ranks from the front, LOW ranks from the back)
//   4. quant_pages   one wave per page: gathers the page's 16 (HIGH) or 32 (LOW) tokens by
//                    position, quantizes them (16 lanes per 256-byte row, 128-bit loads,
//                    cross-lane min/max), packs keys in registers, stages value codes in LDS
//                    and writes the page whole: keys, values in the decode kernel's
//                    operand order, parameters and positions; empty slots are zero / -1.
#include "kvc_internal.h"
#include "workspace.h"

#pragma clang fp contract(off)

namespace kvc {

__global__ __launch_bounds__(256) void quant_count_kernel(
    const uint8_t *__restrict__ tier, const int32_t *__restrict__ cu, int Hkv, int ntq,
    int max_seqlen, const int32_t *status, int32_t *__restrict__ tile_cnt,
    int32_t *__restrict__ entry, int nheads) {
    __shared__ int s_cnt[512];
    const int b = blockIdx.y, tq = blockIdx.x;
    if (b == 0 && tq == 0 && threadIdx.x == 0) entry[nheads] = *status;
    const int lo = cu[b], N = cu[b + 1] - lo;
    const int t0 = tq * QTILE;
    if (N > max_seqlen || t0 >= N) return;
    for (int i = threadIdx.x; i < 2 * Hkv; i += blockDim.x) s_cnt[i] = 0;
    __syncthreads();
    const int nt = min(QTILE, N - t0);
    const uint8_t *tb = tier + (int64_t(lo) + t0) * Hkv;
    for (int idx = threadIdx.x; idx < nt * Hkv; idx += blockDim.x) {
        const int x = tb[idx];
        const int h = idx % Hkv;
        if (x == HIGH) atomicAdd(&s_cnt[2 * h], 1);
        else if (x == LOW) atomicAdd(&s_cnt[2 * h + 1], 1);
    }
    __syncthreads();
    int32_t *out = tile_cnt + (int64_t(b) * ntq + tq) * Hkv * 2;
    for (int i = threadIdx.x; i < 2 * Hkv; i += blockDim.x) out[i] = s_cnt[i];
}

// grid (Hkv, B): exclusive scan over the request's tiles of the (HIGH, LOW) columns of one
// head.  Thread (k, c) sums chunk c of column k; chunk sums are scanned serially in LDS.
__global__ __launch_bounds__(256) void quant_scan_kernel(
    const int32_t *__restrict__ tile_cnt, const int32_t *__restrict__ cu, int Hkv, int ntq,
    int max_seqlen, const int32_t *__restrict__ count_l, int32_t *__restrict__ tile_base,
    int32_t *__restrict__ ok, int32_t *status) {
    __shared__ int s_sum[2][128];
    __shared__ int s_tot[2];
    const int h = blockIdx.x, b = blockIdx.y;
    const int i = b * Hkv + h;
    if (ok[gridDim.x * gridDim.y] != 0) {      // pool status was set on entry: no-op
        if (threadIdx.x == 0) ok[i] = 0;
        return;
    }
    const int N = cu[b + 1] - cu[b];
    if (N > max_seqlen) {
        if (threadIdx.x == 0) {
            ok[i] = 0;
            atomicOr(status, KVC_DEV_SEQLEN);
        }
        return;
    }
    const int nt = (N + QTILE - 1) / QTILE;
    const int k = threadIdx.x >> 7, c = threadIdx.x & 127;
    const int cs = (nt + 127) / 128;
    const int j0 = c * cs, j1 = min(nt, j0 + cs);
    const int64_t col = (int64_t(b) * ntq) * Hkv * 2 + h * 2 + k;
    int sum = 0;
    for (int j = j0; j < j1; ++j) sum += tile_cnt[col + int64_t(j) * Hkv * 2];
    s_sum[k][c] = sum;
    __syncthreads();
    if (threadIdx.x < 2) {
        int run = 0;
        for (int q = 0; q < 128; ++q) {
            const int v = s_sum[threadIdx.x][q];
            s_sum[threadIdx.x][q] = run;
            run += v;
        }
        s_tot[threadIdx.x] = run;
    }
    __syncthreads();
    int run = s_sum[k][c];
    for (int j = j0; j < j1; ++j) {
        const int v = tile_cnt[col + int64_t(j) * Hkv * 2];
        tile_base[col + int64_t(j) * Hkv * 2] = run;
        run += v;
    }
    if (threadIdx.x == 0) {
        const int good = s_tot[0] == count_l[2 * i] && s_tot[1] == count_l[2 * i + 1];
        ok[i] = good;
        if (!good) atomicOr(status, KVC_DEV_COUNT_MISMATCH);
    }
}

// grid (ntq, B), 4 waves: wave w ranks heads w, w+4, ... over the tile's tokens
__global__ __launch_bounds__(256) void quant_select_kernel(
    const uint8_t *__restrict__ tier, const int32_t *__restrict__ cu, int Hkv, int ntq,
    int max_seqlen, const int32_t *__restrict__ tile_base, const int32_t *__restrict__ ok,
    int32_t *__restrict__ poslist) {
    const int b = blockIdx.y, tq = blockIdx.x;
    const int lo = cu[b], N = cu[b + 1] - lo;
    const int t0 = tq * QTILE;
    if (N > max_seqlen || t0 >= N) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nt = min(QTILE, N - t0);
    const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    for (int h = wave; h < Hkv; h += 4) {
        const int i = b * Hkv + h;
        if (!ok[i]) continue;
        const int32_t *base = tile_base + ((int64_t(b) * ntq + tq) * Hkv + h) * 2;
        int rH = base[0], rL = base[1];
        int32_t *pl = poslist + int64_t(i) * max_seqlen;
        for (int c0 = 0; c0 < nt; c0 += 64) {
            const int tt = c0 + lane;
            const int x = tt < nt ? tier[(int64_t(lo) + t0 + tt) * Hkv + h] : PRUNE;
            const uint64_t mH = __ballot(x == HIGH);
            const uint64_t mL = __ballot(x == LOW);
            if (x == HIGH) pl[rH + __popcll(mH & lt)] = t0 + tt;
            else if (x == LOW) pl[max_seqlen - 1 - (rL + __popcll(mL & lt))] = t0 + tt;
            rH += __popcll(mH);
            rL += __popcll(mL);
        }
    }
}

// ---- the quantizer (one 128-channel row per 16-lane group, 8 channels per lane) --------
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

constexpr int QP_WAVES = 4;
constexpr int VST_BYTES = LS * D;     // per-wave staging of value codes (LOW page size)

// grid (ceil(C / 4), B*Hkv): wave w of block x handles page index 4x + w of head y
__global__ __launch_bounds__(256) void quant_pages_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ cu, int Hkv, int C, int max_seqlen,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l,
    const int32_t *__restrict__ ok, const int32_t *__restrict__ poslist,
    uint8_t *__restrict__ pages) {
    __shared__ uint8_t s_v[QP_WAVES][VST_BYTES];
    __shared__ uint16_t s_par[QP_WAVES][LS][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = blockIdx.y;
    const int nheads = gridDim.y;
    if (ok[nheads] != 0 || !ok[i]) return;     // pool failed earlier, or head mismatched
    const int b = i / Hkv, h = i - b * Hkv;
    const int nh = count_l[2 * i], nl = count_l[2 * i + 1];
    const int qH = ceil_div(nh, HS), qL = ceil_div(nl, LS);
    const int pi = blockIdx.x * QP_WAVES + wave;
    bool high;
    int first, m, page;
    if (pi < qH) {
        high = true;
        first = pi * HS;
        m = min(HS, nh - first);
        page = rows_l[int64_t(i) * C + pi];
    } else if (pi - qH < qL) {
        high = false;
        const int lp = pi - qH;
        first = lp * LS;
        m = min(LS, nl - first);
        page = rows_l[int64_t(i) * C + C - 1 - lp];
    } else {
        return;
    }
    uint8_t *pg = pages + int64_t(page) * PAGE;
    const int32_t *pl = poslist + int64_t(i) * max_seqlen;
    const int lo = cu[b];
    const int rg = lane >> 4, c = lane & 15;
    const int nslots = high ? HS : LS;
    uint8_t *sv = s_v[wave];
    // positions of this page's tokens: HIGH ranks from the front, LOW ranks from the back
    for (int pass = 0; pass < nslots / 4; ++pass) {
        const int s = pass * 4 + rg;
        const bool live = s < m;
        int pos = 0;
        if (live) pos = high ? pl[first + s] : pl[max_seqlen - 1 - (first + s)];
        const int64_t roff = ((int64_t(lo) + pos) * Hkv + h) * D + 8 * c;
        // key row
        float x[8];
        load_row8(K + roff, live, x);
        RowQ q = row_params(x, high ? 255.0f : 15.0f);
        if (high) {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) w0 |= code_of(x[e], q) << (8 * e);
#pragma unroll
            for (int e = 0; e < 4; ++e) w1 |= code_of(x[4 + e], q) << (8 * e);
            if (!live) w0 = w1 = 0;
            *reinterpret_cast<uint2 *>(pg + K_OFF + s * 128 + 8 * c) = make_uint2(w0, w1);
        } else {
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                w |= code_of(x[e], q) << (4 * ((e & 1) + 2 * (e >> 2) + 4 * ((e >> 1) & 1)));
            if (!live) w = 0;
            *reinterpret_cast<uint32_t *>(pg + K_OFF + s * 64 + 4 * c) = w;
        }
        if (c == 0) {
            s_par[wave][s][0] = live ? q.s16 : 0;
            s_par[wave][s][1] = live ? q.z16 : 0;
        }
        // value row: codes staged in LDS as bytes [slot][channel]
        load_row8(V + roff, live, x);
        q = row_params(x, high ? 15.0f : 3.0f);
        uint32_t v0 = 0, v1 = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) v0 |= code_of(x[e], q) << (8 * e);
#pragma unroll
        for (int e = 0; e < 4; ++e) v1 |= code_of(x[4 + e], q) << (8 * e);
        if (!live) v0 = v1 = 0;
        *reinterpret_cast<uint2 *>(sv + s * D + 8 * c) = make_uint2(v0, v1);
        if (c == 0) {
            s_par[wave][s][2] = live ? q.s16 : 0;
            s_par[wave][s][3] = live ? q.z16 : 0;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // value unit (j, l) = lane: 16 bytes at V_OFF + 16*lane
    {
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
        *reinterpret_cast<uint4 *>(pg + V_OFF + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    // parameters and positions of all 32 slots (slots >= m, and 16..31 of a HIGH page, empty)
    if (lane < LS) {
        const int s = lane;
        uint32_t a = 0, bb = 0;
        int32_t pos = -1;
        if (s < m) {
            a = uint32_t(s_par[wave][s][0]) | (uint32_t(s_par[wave][s][1]) << 16);
            bb = uint32_t(s_par[wave][s][2]) | (uint32_t(s_par[wave][s][3]) << 16);
            pos = high ? pl[first + s] : pl[max_seqlen - 1 - (first + s)];
        }
        *reinterpret_cast<uint2 *>(pg + PARAM_OFF + 8 * s) = make_uint2(a, bb);
        *reinterpret_cast<int32_t *>(pg + POS_OFF + 4 * s) = pos;
    }
    // a HIGH page's key area beyond slot 15 does not exist; its value area is complete
}

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_quantize_and_place(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                                      const uint16_t *k, const uint16_t *v, const int32_t *cu,
                                      int64_t total_tokens, int32_t max_seqlen,
                                      const uint8_t *tier, const uint8_t *prev_tier,
                                      const uint8_t *changed, const int32_t *old_rows,
                                      const int32_t *old_count, void *ws, size_t ws_bytes,
                                      kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    if (prev_tier || changed || old_rows || old_count) return KVC_E_UNSUPPORTED;
    if (!cu) return KVC_E_NULL;
    if (total_tokens > 0 && (!k || !v || !tier)) return KVC_E_NULL;
    if (layer < 0 || layer >= g->num_layers || max_seqlen < 0 || total_tokens < 0)
        return KVC_E_SHAPE;
    if (g->num_kv_heads > 256) return KVC_E_SHAPE;
    if ((k && !aligned16(k)) || (v && !aligned16(v))) return KVC_E_ALIGN;
    QuantWs L(g, max_seqlen);
    if (!ws || ws_bytes < L.bytes) return KVC_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return KVC_E_ALIGN;
    char *w = static_cast<char *>(ws);
    int32_t *tile_cnt = reinterpret_cast<int32_t *>(w + L.tile_cnt);
    int32_t *tile_base = reinterpret_cast<int32_t *>(w + L.tile_base);
    int32_t *ok = reinterpret_cast<int32_t *>(w + L.ok);
    int32_t *poslist = reinterpret_cast<int32_t *>(w + L.poslist);
    const int B = g->batch, Hkv = g->num_kv_heads, C = g->row_capacity;
    const int nheads = B * Hkv;
    const int32_t *rows_l = p->page_table + int64_t(layer) * nheads * C;
    const int32_t *count_l = p->count + int64_t(layer) * nheads * 2;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(quant_count_kernel, dim3(L.ntq, B), dim3(256), 0, s, tier, cu, Hkv,
                       L.ntq, max_seqlen, p->dev_status, tile_cnt, ok, nheads);
    rc = launch_check("kvc_quantize_and_place/count");
    if (rc) return rc;
    hipLaunchKernelGGL(quant_scan_kernel, dim3(Hkv, B), dim3(256), 0, s, tile_cnt, cu, Hkv,
                       L.ntq, max_seqlen, count_l, tile_base, ok, p->dev_status);
    rc = launch_check("kvc_quantize_and_place/scan");
    if (rc) return rc;
    hipLaunchKernelGGL(quant_select_kernel, dim3(L.ntq, B), dim3(256), 0, s, tier, cu, Hkv,
                       L.ntq, max_seqlen, tile_base, ok, poslist);
    rc = launch_check("kvc_quantize_and_place/select");
    if (rc) return rc;
    hipLaunchKernelGGL(quant_pages_kernel, dim3((C + QP_WAVES - 1) / QP_WAVES, nheads),
                       dim3(64 * QP_WAVES), 0, s, k, v, cu, Hkv, C, max_seqlen, rows_l,
                       count_l, ok, poslist, p->pages);
    return launch_check("kvc_quantize_and_place/pages");
}
