// kvc_generation_step: one decode step under the per-step tier policy.
//
// DiffKV review page: Algorithm 1 (as the referee report describes it, major comment 2 and
// minor comment 4) scores, in the generation phase, the candidate token t_c that has just left
// the recent window against alpha_h/N and alpha_l/N; the free-parameter ledger keeps the most
// recent W tokens at high precision; "What carries the argument": the score is the mean
// attention a token received from later tokens, max-aggregated over its GQA group, and pages
// come from the circular free list by prefix sum.
//
// Every request's new token enters its head's HIGH tier at the end (it has the largest
// position).  t_c = N-1-W is the oldest window token, so it holds HIGH rank n_high - W; it
// keeps HIGH, or goes to LOW (re-quantized from its K8V4 reconstruction, appended after every
// older LOW token) or is dropped.  A HIGH count never shrinks in a step (+1 new, -1 leaving),
// so the allocation is a growth round like kvc_append_tokens.
//
// Launches: gen_decide (per head: the leaving token's tier and the new counts), the three
// allocation kernels, gen_place (one workgroup per head: the head's HIGH tail pages, from
// t_c's page on, are gathered into LDS as per-slot codes, shifted over t_c, extended by the
// new token and written back whole; the demoted token goes into the next LOW slot).  Up to
// 256 heads take two launches instead: gen_plan (decisions and the allocation scan in one
// workgroup) and gen_place<FUSED> (each workgroup commits its head's allocation, then places).
#include "compact_dev.h"
#include "kvc_internal.h"
#include "page_io.h"
#include "quant_row.h"
#include "scheme_io.h"
#include "workspace.h"

#pragma clang fp contract(off)

namespace kvc {

constexpr int GEN_NONE = 255;               // no token left the window
constexpr int GEN_TAIL = GEN_MAX_WINDOW + 16; // HIGH slots a step may rewrite

// head i's decision: the leaving token's tier (GEN_NONE if none left), the new counts
__device__ __forceinline__ void decide_head(int i, const int32_t *__restrict__ count_l,
                                            const int32_t *__restrict__ rows_l, int C,
                                            const uint8_t *__restrict__ pages,
                                            const int32_t *__restrict__ positions,
                                            const float *__restrict__ acc,
                                            const int32_t *__restrict__ cu, int Hkv, int G,
                                            float alpha_h, float alpha_l, int window,
                                            int32_t *__restrict__ new_count,
                                            int32_t *__restrict__ old_count,
                                            uint8_t *__restrict__ changed,
                                            uint8_t *__restrict__ decided,
                                            uint8_t *__restrict__ tier_out, int32_t *status) {
    const int b = i / Hkv, h = i - b * Hkv;
    const int nh = count_l[2 * i], nl = count_l[2 * i + 1];
    old_count[2 * i] = nh;
    old_count[2 * i + 1] = nl;
    changed[i] = 0;
    const int pos = positions[b];               // the new token's position, N = pos + 1
    const int N = pos + 1;
    const int t_c = pos - window;
    int d = GEN_NONE;
    if (t_c >= 0) {
        const int lo = cu[b];
        if (cu[b + 1] - lo < N) {
            atomicOr(status, KVC_DEV_SEQLEN);     // the accumulators do not cover this request
        } else if (nh < window ||
                   reinterpret_cast<const int32_t *>(
                       pages + int64_t(rows_l[int64_t(i) * C + ((nh - window) >> 4)]) * PAGE +
                       POS_OFF)[(nh - window) & (HS - 1)] != t_c) {
            // the last `window` HIGH slots must hold positions t_c .. pos-1
            atomicOr(status, KVC_DEV_COUNT_MISMATCH);
        } else {
            const float *a = acc + (int64_t(lo) + t_c) * (int64_t(Hkv) * G) + int64_t(h) * G;
            float mx = a[0];
            for (int g = 1; g < G; ++g) mx = fmaxf(mx, a[g]);
            const float score = mx / float(N - 1 - t_c);    // correctly rounded float32
            const float th = alpha_h / float(N), tl = alpha_l / float(N);
            d = score >= th ? HIGH : (score >= tl ? LOW : PRUNE);
        }
    }
    decided[i] = uint8_t(d);
    tier_out[i] = uint8_t(d);
    const bool leaves = d == LOW || d == PRUNE;
    new_count[2 * i] = nh + 1 - (leaves ? 1 : 0);
    new_count[2 * i + 1] = nl + (d == LOW ? 1 : 0);
}

__global__ void gen_decide_kernel(const int32_t *__restrict__ count_l,
                                  const int32_t *__restrict__ rows_l, int C,
                                  const uint8_t *__restrict__ pages,
                                  const int32_t *__restrict__ positions,
                                  const float *__restrict__ acc, const int32_t *__restrict__ cu,
                                  int Hkv, int G, float alpha_h, float alpha_l, int window,
                                  int nheads, int32_t *__restrict__ new_count,
                                  int32_t *__restrict__ old_count, uint8_t *__restrict__ changed,
                                  uint8_t *__restrict__ decided, uint8_t *__restrict__ tier_out,
                                  int32_t *status) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nheads) return;
    decide_head(i, count_l, rows_l, C, pages, positions, acc, cu, Hkv, G, alpha_h, alpha_l,
                window, new_count, old_count, changed, decided, tier_out, status);
}

// up to 256 heads in one workgroup: every head's decision, then the allocation round's scan
// (the heads' page demands, their exclusive prefix sums and the round's totals) without the
// multi-tile look-back of compact_scan
__global__ __launch_bounds__(256) void gen_plan_kernel(
    const int32_t *__restrict__ count_l, const int32_t *__restrict__ rows_l, int C,
    const uint8_t *__restrict__ pages, const int32_t *__restrict__ positions,
    const float *__restrict__ acc, const int32_t *__restrict__ cu, int Hkv, int G, float alpha_h,
    float alpha_l, int window, int nheads, int32_t *__restrict__ new_count,
    int32_t *__restrict__ old_count, uint8_t *__restrict__ changed,
    uint8_t *__restrict__ decided, uint8_t *__restrict__ tier_out, int32_t *status,
    const uint64_t *ctr, CompactHdr *hdr, int32_t *__restrict__ off, int32_t *__restrict__ foff) {
    __shared__ int s_wa[4], s_wf[4];
    __shared__ uint32_t s_err;
    if (threadIdx.x == 0) s_err = 0u;
    __syncthreads();
    const int i = threadIdx.x;
    HeadDemand d{};
    if (i < nheads) {
        decide_head(i, count_l, rows_l, C, pages, positions, acc, cu, Hkv, G, alpha_h, alpha_l,
                    window, new_count, old_count, changed, decided, tier_out, status);
        d = head_demand(count_l, new_count, changed, i, C);
        if (d.err) atomicOr(&s_err, uint32_t(d.err));
    }
    int a = d.alloc, f = d.free;
    block_scan2(a, f, s_wa, s_wf);       // inclusive; the last thread holds the totals
    if (i < nheads) {
        off[i] = a - d.alloc;
        foff[i] = f - d.free;
    }
    __syncthreads();
    if (threadIdx.x == blockDim.x - 1) {
        hdr->err = s_err;
        hdr->total_alloc = a;
        hdr->total_free = f;
        hdr->head0 = ctr[0];
        hdr->tail0 = ctr[1];
        // the decisions' status bits included (set by this workgroup's atomics)
        hdr->entry_status = __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// the bit widths of a precision-scheme layer; kh == 0: the default K8V4 / K4V2 layout
struct SchBits {
    int kh, vh, kl, vl;
};

// one workgroup (4 waves) per head.  FUSED: the workgroup first commits its head's part of
// the allocation round (gen_plan_kernel did the scan), then places
template <bool FUSED>
__global__ __launch_bounds__(256) void gen_place_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ positions, int Hkv, int C, int nheads, int window,
    int32_t *__restrict__ rows_l, int32_t *__restrict__ count_l,
    const int32_t *__restrict__ new_count, const int32_t *__restrict__ old_count,
    const uint8_t *__restrict__ decided, uint8_t *__restrict__ pages, int32_t *status,
    const uint8_t *__restrict__ changed, int64_t P, int layer_gid0, uint64_t *ctr,
    int32_t *__restrict__ ring, int32_t *__restrict__ owner, const CompactHdr *hdr,
    const int32_t *__restrict__ off, const int32_t *__restrict__ foff, SchBits sb) {
    __shared__ uint8_t s_k[GEN_TAIL][D];            // key codes per slot (one per byte)
    __shared__ uint8_t s_v[GEN_TAIL][D];            // value codes per slot
    __shared__ uint32_t s_par[GEN_TAIL][2];         // (key scale|zero, value scale|zero)
    __shared__ int32_t s_pos[GEN_TAIL];
    __shared__ uint8_t s_lk[D], s_lv[D];            // the demoted token's LOW codes
    __shared__ uint32_t s_lpar[2];
    const int i = blockIdx.x;
    if (i >= nheads) return;
    if constexpr (FUSED) {
        // a round that does not commit (status bits at its start, the decisions' included,
        // or a failed allocation) leaves every page as it was
        if (!commit_head(i, rows_l, count_l, new_count, changed, C, P, layer_gid0, status, ctr,
                         ring, owner, hdr, off, foff, nullptr, nullptr))
            return;
        __syncthreads();                             // the head's new row and counts
    } else {
        // any status bit (set before this call, by the decision or by the allocation round)
        // means the round committed nothing: the step leaves every page as it was
        if (*status != 0) return;
        if (count_l[2 * i] != new_count[2 * i] || count_l[2 * i + 1] != new_count[2 * i + 1])
            return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = lane >> 4, c = lane & 15;
    const int b = i / Hkv;
    const int d = decided[i];
    // a scheme layer reads and writes its own layout; its value codes of a slot come to a lane
    // as channels 16 n + c (the default layout's as 8 c + n)
    const bool sch = sb.kh != 0;
    const int kh = sch ? sb.kh : 8, vh = sch ? sb.vh : 4, kl = sch ? sb.kl : 4,
              vl = sch ? sb.vl : 2;
    const int nh0 = old_count[2 * i], nl0 = old_count[2 * i + 1];
    const int32_t *row = rows_l + int64_t(i) * C;
    const int pos = positions[b];
    const bool leaves = d == LOW || d == PRUNE;
    const int end = leaves ? nh0 : nh0 + 1;          // HIGH slots after the step
    const int rc = nh0 - window;                     // the leaving token's HIGH rank
    const int base = leaves ? (rc & ~(HS - 1)) : (nh0 & ~(HS - 1));
    const int ns = end - base;                       // slots rewritten, <= window + 16
    const int ns16 = (ns + HS - 1) & ~(HS - 1);
    // the head's row entries for the HIGH pages the step reads and writes (pages base / 16 ..),
    // loaded once, so that no pass of the gather waits for a page id
    __shared__ int32_t s_row[GEN_TAIL / HS + 2];
    const int pg0 = base >> 4;
    const int npg = max((end - 1) >> 4, (nh0 - 1) >> 4) - pg0 + 1;
    for (int k = threadIdx.x; k < npg; k += blockDim.x) s_row[k] = row[pg0 + k];
    __syncthreads();
    // ---- gather: 16 lanes per slot, 16 slots per pass -----------------------------------
    for (int d0 = 0; d0 < ns16; d0 += 16) {
        const int dd = d0 + 4 * wave + rg;           // destination slot, relative to base
        if (dd >= ns) {
            // padding up to the page end: empty slots (zero codes, -1 position)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s_k[dd][8 * c + e] = 0;
                s_v[dd][8 * c + e] = 0;
            }
            if (c == 0) {
                s_par[dd][0] = s_par[dd][1] = 0u;
                s_pos[dd] = -1;
            }
            continue;
        }
        const int da = base + dd;                    // absolute HIGH rank after the step
        if (da == end - 1) {
            // the new token, quantized from its fp16 rows (K8V4)
            float xk[8], xv[8];
            load_row8(K + int64_t(i) * D + 8 * c, true, xk);
            load_row8(V + int64_t(i) * D + 8 * c, true, xv);
            const RowQ qk = row_params(xk, float((1 << kh) - 1));
            const RowQ qv = row_params(xv, float((1 << vh) - 1));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s_k[dd][8 * c + e] = uint8_t(code_of(xk[e], qk));
                s_v[dd][8 * c + e] = uint8_t(code_of(xv[e], qv));
            }
            if (c == 0) {
                s_par[dd][0] = uint32_t(qk.s16) | (uint32_t(qk.z16) << 16);
                s_par[dd][1] = uint32_t(qv.s16) | (uint32_t(qv.z16) << 16);
                s_pos[dd] = pos;
            }
        } else {
            // an existing token: its old rank skips the leaving token
            const int src = (leaves && da >= rc) ? da + 1 : da;
            const uint8_t *pg = pages + int64_t(s_row[(src >> 4) - pg0]) * PAGE;
            uint32_t kc[8], vc[8], kp, vp;
            if (sch) {
                sch_key_codes(pg, kh, src & (HS - 1), c, kc);
                sch_val_codes(pg, kh, vh, HS, src & (HS - 1), c, vc);
                const uint2 par = *reinterpret_cast<const uint2 *>(pg + PARAM_OFF +
                                                                   8 * (src & (HS - 1)));
                kp = par.x;
                vp = par.y;
            } else {
                old_codes(pg, HIGH, src & (HS - 1), c, kc, vc, kp, vp);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s_k[dd][8 * c + e] = uint8_t(kc[e]);
                s_v[dd][sch ? 16 * e + c : 8 * c + e] = uint8_t(vc[e]);
            }
            if (c == 0) {
                s_par[dd][0] = kp;
                s_par[dd][1] = vp;
                s_pos[dd] = reinterpret_cast<const int32_t *>(pg + POS_OFF)[src & (HS - 1)];
            }
        }
    }
    if (leaves && wave == 0 && rg == 0) {
        // the leaving token (its position was checked by gen_decide): LOW re-quantizes the
        // fp16 rounding of its K8V4 reconstruction
        const uint8_t *pg = pages + int64_t(s_row[(rc >> 4) - pg0]) * PAGE;
        const int so = rc & (HS - 1);
        if (d == LOW) {
            uint32_t kc[8], vc[8], kp, vp;
            if (sch) {
                sch_key_codes(pg, kh, so, c, kc);
                sch_val_codes(pg, kh, vh, HS, so, c, vc);
                const uint2 par = *reinterpret_cast<const uint2 *>(pg + PARAM_OFF + 8 * so);
                kp = par.x;
                vp = par.y;
            } else {
                old_codes(pg, HIGH, so, c, kc, vc, kp, vp);
            }
            float xk[8], xv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xk[e] = recon16(kc[e], kp);
                xv[e] = recon16(vc[e], vp);
            }
            const RowQ qk = row_params(xk, float((1 << kl) - 1));
            const RowQ qv = row_params(xv, float((1 << vl) - 1));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s_lk[8 * c + e] = uint8_t(code_of(xk[e], qk));
                s_lv[sch ? 16 * e + c : 8 * c + e] = uint8_t(code_of(xv[e], qv));
            }
            if (c == 0) {
                s_lpar[0] = uint32_t(qk.s16) | (uint32_t(qk.z16) << 16);
                s_lpar[1] = uint32_t(qv.s16) | (uint32_t(qv.z16) << 16);
            }
        }
    }
    __syncthreads();
    // ---- HIGH tail pages, written whole: wave w takes pages base/16 + w, + 4, ... ----------
    const int p_last = (end - 1) >> 4;
    for (int p = (base >> 4) + wave; p <= p_last; p += 4) {
        uint8_t *pg = pages + int64_t(s_row[p - pg0]) * PAGE;
        const int s0 = HS * p - base;
        const int live = min(HS, end - HS * p);
        if (sch) {
            // keys slot-major at kh bits: (slot, channel group) items, 4 per lane
            for (int k = lane; k < HS * 16; k += 64) {
                const int slot = k >> 4, cg = k & 15;
                uint64_t wk = 0;
                if (slot < live) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        wk |= uint64_t(s_k[s0 + slot][8 * cg + e]) << (kh * e);
                }
                store_codes(pg + 16 * kh * slot + cg * kh, wk, kh);
            }
            // one value block (16 slots); rows past `live` hold the padding's zero codes
            uint8_t *dst = pg + 16 * kh * HS + 4 * vh * lane;
            const uint8_t (*vc)[D] = reinterpret_cast<const uint8_t (*)[D]>(&s_v[s0][0]);
            if (vh == 8) pack_value_block<8>(dst, vc, 0, rg, c);
            else if (vh == 4) pack_value_block<4>(dst, vc, 0, rg, c);
            else if (vh == 2) pack_value_block<2>(dst, vc, 0, rg, c);
            else pack_value_block<1>(dst, vc, 0, rg, c);
            for (int k = HS * (kh + vh) + lane; k < PARAM_OFF / 16; k += 64)
                st_page16(pg + 16 * k, 0u, 0u, 0u, 0u);
        } else {
            for (int k = lane; k < HS * 8; k += 64) {          // keys: 16 slots x 8 x 16 B
                const int slot = k >> 3, off = (k & 7) * 16;
                uint4 x = make_uint4(0, 0, 0, 0);
                if (slot < live) x = *reinterpret_cast<const uint4 *>(&s_k[s0 + slot][off]);
                *reinterpret_cast<uint4 *>(pg + K_OFF + slot * 128 + off) = x;
            }
            pack_values(pg, &s_v[s0][0], true, lane);
        }
        if (lane < LS) {
            const bool on = lane < live;
            const uint2 par = on ? make_uint2(s_par[s0 + lane][0], s_par[s0 + lane][1])
                                 : make_uint2(0u, 0u);
            *reinterpret_cast<uint2 *>(pg + PARAM_OFF + 8 * lane) = par;
            reinterpret_cast<int32_t *>(pg + POS_OFF)[lane] = on ? s_pos[s0 + lane] : -1;
        }
    }
    // ---- the demoted token: next LOW slot (its page is not one of the HIGH pages) ---------
    if (d == LOW && wave == (p_last - (base >> 4) + 1) % 4) {
        uint8_t *pg = pages + int64_t(row[C - 1 - (nl0 >> 5)]) * PAGE;
        const int so = nl0 & (LS - 1);
        if (so == 0) {
            // a fresh page: clear it whole first (3456 B = 216 x 16 B)
            for (int k = lane; k < PAGE / 16; k += 64)
                reinterpret_cast<uint4 *>(pg)[k] = make_uint4(0, 0, 0, 0);
            if (lane < LS) reinterpret_cast<int32_t *>(pg + POS_OFF)[lane] = -1;
            __threadfence_block();
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < 16 && sch) {
            uint64_t wk = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) wk |= uint64_t(s_lk[8 * c + e]) << (kl * e);
            store_codes(pg + 16 * kl * so + c * kl, wk, kl);
            uint32_t vc[8];
#pragma unroll
            for (int n = 0; n < 8; ++n) vc[n] = s_lv[16 * n + c];
            sch_set_val_codes(pg, kl, vl, LS, so, c, vc, so == 0);
        } else if (lane < 16) {
            // keys: lane c packs channels 8c..8c+7 (nibble order of a LOW key word)
            uint32_t kw = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) kw |= uint32_t(s_lk[8 * c + e]) << (4 * k_nib(e));
            *reinterpret_cast<uint32_t *>(pg + K_OFF + so * 64 + 4 * c) = kw;
            // values: unit (j, l = c) holds this slot's 2-bit codes of channels 16n + l
            const int f = so >> 4, j = (so & 15) >> 2, r = so & 3;
            uint32_t *u = reinterpret_cast<uint32_t *>(pg + V_OFF + 16 * (16 * j + c));
            uint32_t wv[4] = {0u, 0u, 0u, 0u};
            if (so != 0) {
                const uint4 old = *reinterpret_cast<const uint4 *>(u);
                wv[0] = old.x; wv[1] = old.y; wv[2] = old.z; wv[3] = old.w;
            }
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const int q = 2 * f + (n >> 2);
                const int sh = 2 * (2 * (n & 3) + (r >> 1) + 8 * (r & 1));
                wv[q] = (wv[q] & ~(3u << sh)) | (uint32_t(s_lv[16 * n + c]) << sh);
            }
            *reinterpret_cast<uint4 *>(u) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
        if (lane == 32) {
            *reinterpret_cast<uint2 *>(pg + PARAM_OFF + 8 * so) = make_uint2(s_lpar[0], s_lpar[1]);
            reinterpret_cast<int32_t *>(pg + POS_OFF)[so] = pos - window;
        }
    }
}

}  // namespace kvc

using namespace kvc;

namespace {

int generation_step_impl(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                         const uint16_t *k_new, const uint16_t *v_new, const int32_t *positions,
                         const float *acc_sum, const int32_t *cu_seqlens, float alpha_h,
                         float alpha_l, int32_t window, uint8_t *tier_out, void *ws,
                         size_t ws_bytes, SchBits sb, kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    if (!k_new || !v_new || !positions || !acc_sum || !cu_seqlens || !tier_out)
        return KVC_E_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVC_E_ALIGN;
    if (layer < 0 || layer >= g->num_layers) return KVC_E_SHAPE;
    if (window < 1 || window > GEN_MAX_WINDOW) return KVC_E_SHAPE;
    GenWs L(g);
    if (!ws || ws_bytes < L.bytes) return KVC_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return KVC_E_ALIGN;
    char *w = static_cast<char *>(ws);
    int32_t *new_count = reinterpret_cast<int32_t *>(w + L.new_count);
    int32_t *old_count = reinterpret_cast<int32_t *>(w + L.old_count);
    uint8_t *changed = reinterpret_cast<uint8_t *>(w + L.changed);
    uint8_t *decided = reinterpret_cast<uint8_t *>(w + L.decided);
    const int nheads = g->batch * g->num_kv_heads, C = g->row_capacity;
    const int G = g->num_q_heads / g->num_kv_heads;
    const int32_t *rows_l = p->page_table + int64_t(layer) * nheads * C;
    const int32_t *count_l = p->count + int64_t(layer) * nheads * 2;
    hipStream_t s = (hipStream_t)stream;
    int32_t *rows_w = p->page_table + int64_t(layer) * nheads * C;
    int32_t *count_w = p->count + int64_t(layer) * nheads * 2;
    if (nheads <= 256) {
        // two launches: decisions + scan in one workgroup, then commit + placement per head
        const CompactWs Lc(g);
        char *wc = w + L.compact;
        CompactHdr *hdr = reinterpret_cast<CompactHdr *>(wc + Lc.hdr);
        int32_t *off = reinterpret_cast<int32_t *>(wc + Lc.off);
        int32_t *foff = reinterpret_cast<int32_t *>(wc + Lc.foff);
        hipLaunchKernelGGL(gen_plan_kernel, dim3(1), dim3(256), 0, s, count_l, rows_l, C,
                           p->pages, positions, acc_sum, cu_seqlens, g->num_kv_heads, G, alpha_h,
                           alpha_l, window, nheads, new_count, old_count, changed, decided,
                           tier_out, p->dev_status, p->ring_ctr, hdr, off, foff);
        rc = launch_check("kvc_generation_step/plan");
        if (rc) return rc;
        hipLaunchKernelGGL(gen_place_kernel<true>, dim3(nheads), dim3(256), 0, s, k_new, v_new,
                           positions, g->num_kv_heads, C, nheads, window, rows_w, count_w,
                           new_count, old_count, decided, p->pages, p->dev_status, changed,
                           g->num_pages, layer * nheads, p->ring_ctr, p->free_ring, p->owner, hdr,
                           off, foff, sb);
        return launch_check("kvc_generation_step/place");
    }
    hipLaunchKernelGGL(gen_decide_kernel, dim3((nheads + 255) / 256), dim3(256), 0, s, count_l,
                       rows_l, C, p->pages, positions, acc_sum, cu_seqlens, g->num_kv_heads, G, alpha_h, alpha_l,
                       window, nheads, new_count, old_count, changed, decided, tier_out,
                       p->dev_status);
    rc = launch_check("kvc_generation_step/decide");
    if (rc) return rc;
    rc = launch_compact(g, layer, p, new_count, changed, nullptr, nullptr, w + L.compact, s);
    if (rc) return rc;
    hipLaunchKernelGGL(gen_place_kernel<false>, dim3(nheads), dim3(256), 0, s, k_new, v_new,
                       positions, g->num_kv_heads, C, nheads, window, rows_w, count_w, new_count,
                       old_count, decided, p->pages, p->dev_status, nullptr, int64_t(0), 0,
                       nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, sb);
    return launch_check("kvc_generation_step/place");
}

}  // namespace

extern "C" int kvc_generation_step(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                                   const uint16_t *k_new, const uint16_t *v_new,
                                   const int32_t *positions, const float *acc_sum,
                                   const int32_t *cu_seqlens, float alpha_h, float alpha_l,
                                   int32_t window, uint8_t *tier_out, void *ws, size_t ws_bytes,
                                   kvc_stream_t stream) {
    return generation_step_impl(g, layer, p, k_new, v_new, positions, acc_sum, cu_seqlens,
                                alpha_h, alpha_l, window, tier_out, ws, ws_bytes,
                                SchBits{0, 0, 0, 0}, stream);
}

extern "C" int kvc_generation_step_scheme(const kvc_geom *g, const kvc_scheme *sc, int32_t layer,
                                          const kvc_pool *p, const uint16_t *k_new,
                                          const uint16_t *v_new, const int32_t *positions,
                                          const float *acc_sum, const int32_t *cu_seqlens,
                                          float alpha_h, float alpha_l, int32_t window,
                                          uint8_t *tier_out, void *ws, size_t ws_bytes,
                                          kvc_stream_t stream) {
    const int rc = check_scheme(sc);
    if (rc) return rc;
    return generation_step_impl(g, layer, p, k_new, v_new, positions, acc_sum, cu_seqlens,
                                alpha_h, alpha_l, window, tier_out, ws, ws_bytes,
                                SchBits{sc->k_bits_high, sc->v_bits_high, sc->k_bits_low,
                                        sc->v_bits_low}, stream);
}
