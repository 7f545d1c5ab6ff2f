// kvc_score_tokens: significance score, GQA max and three-tier decision.
//
// DiffKV review page, "What carries the argument": the score of a token is the mean
// attention it receives from subsequent tokens, max-aggregated across the GQA heads of its
// KV head, compared with alpha_h/N and alpha_l/N.  Free-parameter ledger: the most recent
// W tokens are always high precision.  Referee major comment 3: demotion is irreversible.
//
// HBM-bound streaming kernel: each (token, KV head) reads its G float32 accumulators
// (contiguous, 16-byte vector loads when G % 4 == 0) and writes one tier byte.  Because a
// correctly rounded division is monotone, max_g fl(a_g/cnt) == fl(max_g a_g / cnt), so one
// division per (token, head) suffices.  Per-head counts are reduced in LDS and added to
// global memory with one atomic per (workgroup, head, tier).
#include "kvc_internal.h"
#include "workspace.h"

namespace kvc {

#ifndef KVC_SCORE_UNROLL
#define KVC_SCORE_UNROLL 4       // (token, head) items per thread whose loads are in flight together
#endif
#ifndef KVC_SCORE_TILE
#define KVC_SCORE_TILE 256
#endif
constexpr int SCORE_TILE = KVC_SCORE_TILE;   // tokens per workgroup
constexpr int SCORE_THREADS = 256;
constexpr int MAX_HKV_LDS = 256;

__global__ void score_zero_kernel(int32_t *count, int n, uint8_t *changed, int nc) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) count[i] = 0;
    if (changed && i < nc) changed[i] = 0;
}

// TILES (the fused round): instead of adding the workgroup's counts into count[B][Hkv][2] and
// setting changed[B][Hkv], store them per tile: count -> [B][ntq][Hkv][2] (new tiers),
// count2 -> the same for the previous tiers, changed -> [B][ntq][Hkv] (a tier dropped)
template <int G, bool TILES>   // G > 0: compile-time group size; G == 0: runtime group size `g`
__global__ __launch_bounds__(SCORE_THREADS) void score_kernel(
    const float *__restrict__ acc, const int32_t *__restrict__ cu, int B, int Hkv, int g,
    int max_seqlen, float alpha_h, float alpha_l, int window,
    const uint8_t *__restrict__ prev, uint8_t *__restrict__ tier, int32_t *__restrict__ count,
    uint8_t *__restrict__ changed, int32_t *status, int32_t *__restrict__ count2) {
    __shared__ int s_cnt[MAX_HKV_LDS * 2];
    __shared__ int s_cnt2[TILES ? MAX_HKV_LDS * 2 : 1];
    __shared__ int s_chg[MAX_HKV_LDS];
    const int b = blockIdx.y;
    const int lo = cu[b];
    const int N = cu[b + 1] - lo;
    if (N > max_seqlen) {
        if (blockIdx.x == 0 && threadIdx.x == 0 && status) atomicOr(status, KVC_DEV_SEQLEN);
        return;
    }
    const int t0 = blockIdx.x * SCORE_TILE;
    if (t0 >= N) return;
    const int gs = G > 0 ? G : g;
    const int Hq = Hkv * gs;
    for (int i = threadIdx.x; i < Hkv * 2; i += blockDim.x) s_cnt[i] = 0;
    if constexpr (TILES)
        for (int i = threadIdx.x; i < Hkv * 2; i += blockDim.x) s_cnt2[i] = 0;
    for (int i = threadIdx.x; i < Hkv; i += blockDim.x) s_chg[i] = 0;
    __syncthreads();
    const float fN = float(N);
    const float th = alpha_h / fN;   // correctly rounded float32 division
    const float tl = alpha_l / fN;
    const int nt = min(SCORE_TILE, N - t0);
    const int total = nt * Hkv;
    // SU items per thread per pass: every item's accumulators (and previous tier) are requested
    // before the first is used, so a pass waits for one round trip, not one per item (an item
    // past the tile loads the tile's last item and is dropped)
    constexpr int SU = (G > 0 && G % 4 == 0) ? KVC_SCORE_UNROLL : 1;
    for (int base = threadIdx.x; base < total; base += SU * blockDim.x) {
    float mxs[SU];
    int pvs[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
        const int idx = min(base + u * int(blockDim.x), total - 1);
        const int tt = idx / Hkv, h = idx - tt * Hkv;
        const int64_t r = int64_t(lo) + t0 + tt;
        const float *a = acc + r * Hq + h * gs;
        float mx;
        if constexpr (G > 0 && G % 4 == 0) {
            float4 v = *reinterpret_cast<const float4 *>(a);
            mx = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
#pragma unroll
            for (int k = 4; k < G; k += 4) {
                float4 w = *reinterpret_cast<const float4 *>(a + k);
                mx = fmaxf(mx, fmaxf(fmaxf(w.x, w.y), fmaxf(w.z, w.w)));
            }
        } else {
            mx = a[0];
            for (int k = 1; k < gs; ++k) mx = fmaxf(mx, a[k]);
        }
        mxs[u] = mx;
        pvs[u] = prev ? int(prev[r * Hkv + h]) : 0;
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
        const int idx = base + u * int(blockDim.x);
        if (idx >= total) break;
        const int tt = idx / Hkv, h = idx - tt * Hkv;
        const int t = t0 + tt;
        const int64_t r = int64_t(lo) + t;
        const float mx = mxs[u];
        const int cnt = N - 1 - t;
        const float score = cnt == 0 ? __builtin_inff() : mx / float(cnt);
        int x = score >= th ? HIGH : (score >= tl ? LOW : PRUNE);
        if (t >= N - window) x = HIGH;
        if (prev) {
            const int p = pvs[u];
            if constexpr (TILES) {
                if (p == HIGH) atomicAdd(&s_cnt2[2 * h], 1);
                else if (p == LOW) atomicAdd(&s_cnt2[2 * h + 1], 1);
            }
            if (p != FRESH) {
                if (x < p) s_chg[h] = 1;
                x = min(x, p);
            } else if (x != PRUNE) {
                s_chg[h] = 1;                  // a fresh token joins the head's pages
            }
        }
        tier[r * Hkv + h] = uint8_t(x);
        if (x == HIGH) atomicAdd(&s_cnt[2 * h], 1);
        else if (x == LOW) atomicAdd(&s_cnt[2 * h + 1], 1);
    }
    }
    __syncthreads();
    if constexpr (TILES) {
        const int64_t tb = int64_t(b) * gridDim.x + blockIdx.x;      // (request, tile)
        for (int i = threadIdx.x; i < Hkv * 2; i += blockDim.x) {
            count[tb * Hkv * 2 + i] = s_cnt[i];
            if (prev) count2[tb * Hkv * 2 + i] = s_cnt2[i];
        }
        if (prev)
            for (int i = threadIdx.x; i < Hkv; i += blockDim.x)
                changed[tb * Hkv + i] = uint8_t(s_chg[i]);
    } else {
        for (int i = threadIdx.x; i < Hkv * 2; i += blockDim.x) {
            const int c = s_cnt[i];
            if (c) atomicAdd(&count[(b * Hkv) * 2 + i], c);
        }
        if (changed)
            for (int i = threadIdx.x; i < Hkv; i += blockDim.x)
                if (s_chg[i]) changed[b * Hkv + i] = 1;
    }
}

static_assert(SCORE_TILE == QTILE, "a fused round's score tiles are its rank tiles");

// the score launch of a fused round: tiers, per-tile counts (new and previous tiers) and
// per-tile dropped-tier flags; grid (ntq, B) with ntq = ceil(max_seqlen / QTILE)
int launch_round_score(const kvc_geom *g, const float *acc, const int32_t *cu, int max_seqlen,
                       float alpha_h, float alpha_l, int window, const uint8_t *prev_tier,
                       uint8_t *tier, int32_t *tile_cnt, int32_t *tile_cnt2, uint8_t *tile_chg,
                       int32_t *status, hipStream_t s) {
    const int B = g->batch, Hkv = g->num_kv_heads, G = g->num_q_heads / g->num_kv_heads;
    const int ntq = max(1, (max_seqlen + QTILE - 1) / QTILE);
    const dim3 grid(ntq, B), block(SCORE_THREADS);
#define KVC_ROUND_SCORE(GG)                                                                    \
    hipLaunchKernelGGL((score_kernel<GG, true>), grid, block, 0, s, acc, cu, B, Hkv, G,         \
                       max_seqlen, alpha_h, alpha_l, window, prev_tier, tier, tile_cnt, tile_chg, \
                       status, tile_cnt2)
    switch (G) {
        case 4: KVC_ROUND_SCORE(4); break;
        case 8: KVC_ROUND_SCORE(8); break;
        case 16: KVC_ROUND_SCORE(16); break;
        default: KVC_ROUND_SCORE(0); break;
    }
#undef KVC_ROUND_SCORE
    return launch_check("kvc_compaction_round/score");
}

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_score_tokens(const kvc_geom *g, const float *acc, const int32_t *cu,
                                int64_t total_tokens, int32_t max_seqlen, float alpha_h,
                                float alpha_l, int32_t window, const uint8_t *prev_tier,
                                uint8_t *tier, int32_t *new_count, uint8_t *changed,
                                int32_t *dev_status, kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    if (!cu || !new_count || (total_tokens > 0 && (!acc || !tier))) return KVC_E_NULL;
    if (prev_tier && !changed) return KVC_E_NULL;
    if (total_tokens < 0 || window < 0 || max_seqlen < 0) return KVC_E_SHAPE;
    if (g->num_kv_heads > MAX_HKV_LDS) return KVC_E_SHAPE;
    if (acc && ((reinterpret_cast<uintptr_t>(acc) & 15u) != 0)) return KVC_E_ALIGN;
    const int B = g->batch, Hkv = g->num_kv_heads, G = g->num_q_heads / g->num_kv_heads;
    hipStream_t s = (hipStream_t)stream;
    const int nc = B * Hkv * 2;
    hipLaunchKernelGGL(score_zero_kernel, dim3((nc + 255) / 256), dim3(256), 0, s, new_count,
                       nc, changed, B * Hkv);
    rc = launch_check("kvc_score_tokens/zero");
    if (rc) return rc;
    if (max_seqlen == 0 || total_tokens == 0) return KVC_OK;
    dim3 grid((max_seqlen + SCORE_TILE - 1) / SCORE_TILE, B);
    dim3 block(SCORE_THREADS);
#define KVC_SCORE_LAUNCH(GG)                                                                  \
    hipLaunchKernelGGL((score_kernel<GG, false>), grid, block, 0, s, acc, cu, B, Hkv, G,      \
                       max_seqlen, alpha_h, alpha_l, window, prev_tier, tier, new_count,      \
                       changed, dev_status, nullptr)
    switch (G) {
        case 4: KVC_SCORE_LAUNCH(4); break;
        case 8: KVC_SCORE_LAUNCH(8); break;
        case 16: KVC_SCORE_LAUNCH(16); break;
        default: KVC_SCORE_LAUNCH(0); break;
    }
#undef KVC_SCORE_LAUNCH
    return launch_check("kvc_score_tokens");
}
