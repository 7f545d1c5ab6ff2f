// Internal definitions shared by the libkvc HIP sources (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <string.h>

#include "../../include/kvc.h"

namespace kvc {

constexpr int D = KVC_HEAD_DIM;
constexpr int PAGE = KVC_PAGE_BYTES;
constexpr int HS = KVC_HIGH_SLOTS;   // HIGH tokens per page
constexpr int LS = KVC_LOW_SLOTS;    // LOW tokens per page
constexpr int K_OFF = 0;
constexpr int V_OFF = 2048;
constexpr int PARAM_OFF = 3072;      // 8 bytes per slot: k_scale, k_zero, v_scale, v_zero
constexpr int POS_OFF = 3328;        // int32 per slot

constexpr int PRUNE = KVC_PRUNE, LOW = KVC_LOW, HIGH = KVC_HIGH, FRESH = KVC_FRESH;

void set_error(const char *what, hipError_t e);

// one allocation round (compact.hip); arguments already validated
int launch_compact(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                   const int32_t *new_count, const uint8_t *changed, int32_t *old_rows_out,
                   int32_t *old_count_out, void *ws, hipStream_t s);

// the launches of a fused round (score.hip, compact.hip), arguments already validated
int launch_round_score(const kvc_geom *g, const float *acc, const int32_t *cu, int max_seqlen,
                       float alpha_h, float alpha_l, int window, const uint8_t *prev_tier,
                       uint8_t *tier, int32_t *tile_cnt, int32_t *tile_cnt2, uint8_t *tile_chg,
                       int32_t *status, hipStream_t s);
int launch_round_commit(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                        const int32_t *cnt0, const int32_t *new_count, const uint8_t *changed,
                        int32_t *ok, int32_t *old_rows_out, void *compact_ws, hipStream_t s);

// the combine and the score accumulation after a score-accumulating decode (attention.hip):
// w is the decode workspace laid out by DecodeWs(g, true, max_seqlen), its partials and tile
// records already written
int launch_combine_and_accumulation(const kvc_geom *g, const kvc_pool *p, const float *part,
                                    int S, int wt, void *out, int out_fp32,
                                    const int32_t *count_l, const int32_t *cu, int max_seqlen,
                                    float *acc_sum, char *w, hipStream_t s);
// the combine launch of a split-K decode (attention.hip); partials [B*Hkv][S][G][132], of
// which head i's first active_splits(count_l[2i], count_l[2i+1], S, wt) were written
int launch_decode_combine(const float *part, int Hq, int G, int S, int B, void *out,
                          int out_fp32, float *mls, const int32_t *count_l, int wt,
                          hipStream_t s);

inline int launch_check(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error(what, e);
        return KVC_E_HIP;
    }
    return KVC_OK;
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int check_geom(const kvc_geom *g) {
    if (!g) return KVC_E_NULL;
    if (g->num_layers <= 0 || g->batch <= 0 || g->num_q_heads <= 0 || g->num_kv_heads <= 0 ||
        g->row_capacity <= 0 || g->num_pages <= 0)
        return KVC_E_SHAPE;
    if (g->num_q_heads % g->num_kv_heads) return KVC_E_SHAPE;
    if (g->num_pages >= (int64_t(1) << 31)) return KVC_E_SHAPE;
    int64_t rows = int64_t(g->num_layers) * g->batch * g->num_kv_heads * g->row_capacity;
    if (rows >= (int64_t(1) << 31)) return KVC_E_SHAPE;
    return KVC_OK;
}

inline bool scheme_bits_ok(int b) { return b == 1 || b == 2 || b == 4 || b == 8; }
inline int check_scheme(const kvc_scheme *sc) {
    if (!sc) return KVC_E_NULL;
    if (!scheme_bits_ok(sc->k_bits_high) || !scheme_bits_ok(sc->v_bits_high) ||
        !scheme_bits_ok(sc->k_bits_low) || !scheme_bits_ok(sc->v_bits_low))
        return KVC_E_SHAPE;
    if (HS * 16 * (sc->k_bits_high + sc->v_bits_high) > PARAM_OFF) return KVC_E_SHAPE;
    if (LS * 16 * (sc->k_bits_low + sc->v_bits_low) > PARAM_OFF) return KVC_E_SHAPE;
    return KVC_OK;
}

inline int check_pool(const kvc_pool *p) {
    if (!p || !p->pages || !p->page_table || !p->count || !p->owner || !p->free_ring ||
        !p->ring_ctr || !p->dev_status)
        return KVC_E_NULL;
    if (!aligned16(p->pages)) return KVC_E_ALIGN;
    return KVC_OK;
}

// ---- device helpers -------------------------------------------------------------------

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// request index owning global row r, by binary search over cu_seqlens[0..B]
__device__ __forceinline__ int find_request(const int32_t *cu, int B, int64_t r) {
    int lo = 0, hi = B;   // cu[lo] <= r < cu[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (cu[mid] <= r) lo = mid; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ float h2f(uint16_t b) {
    return __half2float(__ushort_as_half(b));
}
// fp16 rounding (nearest, ties to even) of the float32 value f.  The empty asm makes f a
// finished float32 value: without it the compiler may fuse the multiply-add that produced f
// into an fp16-result v_fma_mix, one rounding of the exact result instead of the float32
// rounding followed by the fp16 one (they differ where the float32 value is an fp16 tie)
__device__ __forceinline__ uint16_t f2h_rn(float f) {
    asm("" : "+v"(f));
    return __half_as_ushort(__float2half_rn(f));
}

}  // namespace kvc
