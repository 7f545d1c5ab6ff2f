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
#include "quant_row.h"
#include "page_io.h"
#include "scheme_io.h"
#include "compact_dev.h"

#pragma clang fp contract(off)

namespace kvc {

// grid (ntq, B): per 256-token tile, #HIGH and #LOW per KV head of `tier` (and of `prev`)
__global__ __launch_bounds__(256) void quant_count_kernel(
    const uint8_t *__restrict__ tier, const uint8_t *__restrict__ prev,
    const int32_t *__restrict__ cu, int Hkv, int ntq, int max_seqlen, const int32_t *status,
    int32_t *__restrict__ tile_cnt, int32_t *__restrict__ tile_cnt2,
    int32_t *__restrict__ entry, int nheads) {
    __shared__ int s_cnt[2][512];
    const int b = blockIdx.y, tq = blockIdx.x;
    if (b == 0 && tq == 0 && threadIdx.x == 0) entry[nheads] = *status;
    const int lo = cu[b], N = cu[b + 1] - lo;
    const int t0 = tq * QTILE;
    if (N > max_seqlen || t0 >= N) return;
    for (int i = threadIdx.x; i < 2 * Hkv; i += blockDim.x) s_cnt[0][i] = s_cnt[1][i] = 0;
    __syncthreads();
    const int nt = min(QTILE, N - t0);
    const int64_t base = (int64_t(lo) + t0) * Hkv;
    for (int idx = threadIdx.x; idx < nt * Hkv; idx += blockDim.x) {
        const int h = idx % Hkv;
        const int x = tier[base + idx];
        if (x == HIGH) atomicAdd(&s_cnt[0][2 * h], 1);
        else if (x == LOW) atomicAdd(&s_cnt[0][2 * h + 1], 1);
        if (prev) {
            const int y = prev[base + idx];
            if (y == HIGH) atomicAdd(&s_cnt[1][2 * h], 1);
            else if (y == LOW) atomicAdd(&s_cnt[1][2 * h + 1], 1);
        }
    }
    __syncthreads();
    const int64_t o = (int64_t(b) * ntq + tq) * Hkv * 2;
    for (int i = threadIdx.x; i < 2 * Hkv; i += blockDim.x) {
        tile_cnt[o + i] = s_cnt[0][i];
        if (prev) tile_cnt2[o + i] = s_cnt[1][i];
    }
}

// exclusive scan over a request's tiles of the (HIGH, LOW) columns of one head; returns the
// totals.  Thread (k, c) sums chunk c of column k; chunk sums are scanned serially in LDS.
__device__ void scan_columns(const int32_t *__restrict__ cnt, int32_t *__restrict__ out,
                             int64_t col0, int Hkv, int nt, int (&s_sum)[2][128], int (&tot)[2]) {
    const int k = threadIdx.x >> 7, c = threadIdx.x & 127;
    const int cs = (nt + 127) / 128;
    const int j0 = c * cs, j1 = min(nt, j0 + cs);
    const int64_t col = col0 + k;
    int sum = 0;
    for (int j = j0; j < j1; ++j) sum += cnt[col + int64_t(j) * Hkv * 2];
    s_sum[k][c] = sum;
    __syncthreads();
    if (threadIdx.x < 2) {
        int run = 0;
        for (int q = 0; q < 128; ++q) {
            const int v = s_sum[threadIdx.x][q];
            s_sum[threadIdx.x][q] = run;
            run += v;
        }
        tot[threadIdx.x] = run;
    }
    __syncthreads();
    int run = s_sum[k][c];
    for (int j = j0; j < j1; ++j) {
        const int v = cnt[col + int64_t(j) * Hkv * 2];
        out[col + int64_t(j) * Hkv * 2] = run;
        run += v;
    }
    __syncthreads();
}

// grid (Hkv, B).  ok[i] = 1 when head i's pages are to be written: its tier counts match the
// pool's (and, re-tiering, its previous counts match the snapshot and the head is rebuilt).
__global__ __launch_bounds__(256) void quant_scan_kernel(
    const int32_t *__restrict__ tile_cnt, const int32_t *__restrict__ tile_cnt2,
    const int32_t *__restrict__ cu, int Hkv, int ntq, int max_seqlen,
    const int32_t *__restrict__ count_l, const uint8_t *__restrict__ changed,
    const int32_t *__restrict__ old_count, int32_t *__restrict__ tile_base,
    int32_t *__restrict__ tile_base2, int32_t *__restrict__ ok, int32_t *status) {
    __shared__ int s_sum[2][128];
    __shared__ int s_tot[2], s_tot2[2];
    const int h = blockIdx.x, b = blockIdx.y;
    const int i = b * Hkv + h;
    const bool rebuild = tile_cnt2 != nullptr;
    if (ok[gridDim.x * gridDim.y] != 0 || (rebuild && !changed[i])) {
        // pool status set on entry (no-op), or a head that keeps its pages
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
    const int64_t col0 = (int64_t(b) * ntq) * Hkv * 2 + h * 2;
    scan_columns(tile_cnt, tile_base, col0, Hkv, nt, s_sum, s_tot);
    if (rebuild) scan_columns(tile_cnt2, tile_base2, col0, Hkv, nt, s_sum, s_tot2);
    if (threadIdx.x == 0) {
        bool good = s_tot[0] == count_l[2 * i] && s_tot[1] == count_l[2 * i + 1];
        if (rebuild) good = good && s_tot2[0] == old_count[2 * i] && s_tot2[1] == old_count[2 * i + 1];
        ok[i] = good;
        if (!good) atomicOr(status, KVC_DEV_COUNT_MISMATCH);
    }
}

// The per-head launch of a fused round: grid (Hkv, B).  The head's tier totals over its
// request's tiles (new_count, the round's counts), the tiles' exclusive bases for the rank
// kernel, for the previous tiers too when re-tiering (with the changed flag: some tile dropped
// a tier), and ok[i] = the head's pages are written (every head in prompt mode, a changed one
// when re-tiering; the planning launch clears the round's ok[nheads] when it does not commit).
__global__ __launch_bounds__(256) void round_head_kernel(
    const int32_t *__restrict__ tile_cnt, const int32_t *__restrict__ tile_cnt2,
    const uint8_t *__restrict__ tile_chg, const int32_t *__restrict__ cu, int Hkv, int ntq,
    int max_seqlen, int32_t *__restrict__ tile_base, int32_t *__restrict__ tile_base2,
    int32_t *__restrict__ new_count, uint8_t *__restrict__ changed, int32_t *__restrict__ ok,
    const int32_t *status, const uint64_t *ctr, CompactHdr *snap,
    const int32_t *__restrict__ rows_l, int C, int32_t *__restrict__ old_rows,
    const int32_t *__restrict__ count_l, int32_t *__restrict__ cnt0) {
    __shared__ int s_sum[2][128];
    __shared__ int s_tot[2], s_tot2[2];
    __shared__ int s_chg;
    const int h = blockIdx.x, b = blockIdx.y;
    if (h == 0 && b == 0 && threadIdx.x == 0) {
        // the round's start for the commit launch: the pool status (the score launch's bits
        // included) and the ring counters, before any commit of this round moves them
        snap->entry_status = __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        snap->head0 = ctr[0];
        snap->tail0 = ctr[1];
    }
    const int i = b * Hkv + h;
    const bool retier = tile_cnt2 != nullptr;
    const int N = cu[b + 1] - cu[b];
    // a request longer than max_seqlen was skipped by the score launch (its status bit set)
    const int nt = (N < 0 || N > max_seqlen) ? 0 : (N + QTILE - 1) / QTILE;
    if (threadIdx.x == 0) s_chg = 0;
    const int64_t col0 = (int64_t(b) * ntq) * Hkv * 2 + h * 2;
    scan_columns(tile_cnt, tile_base, col0, Hkv, nt, s_sum, s_tot);
    if (retier) {
        scan_columns(tile_cnt2, tile_base2, col0, Hkv, nt, s_sum, s_tot2);
        for (int tq = threadIdx.x; tq < nt; tq += blockDim.x)
            if (tile_chg[(int64_t(b) * ntq + tq) * Hkv + h]) s_chg = 1;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        new_count[2 * i] = s_tot[0];
        new_count[2 * i + 1] = s_tot[1];
        if (retier) changed[i] = uint8_t(s_chg);
        ok[i] = retier ? s_chg : 1;
        // the head's counts before the round, for the commit launch's demands
        cnt0[2 * i] = count_l[2 * i];
        cnt0[2 * i + 1] = count_l[2 * i + 1];
    }
    // re-tier: a changed head's row as it stands before this round's commit, where the rank
    // launch looks up the old page of every kept token (the commit then overwrites the row)
    if (old_rows && s_chg) {
        const int32_t *row = rows_l + int64_t(i) * C;
        for (int p = threadIdx.x; p < C; p += blockDim.x) old_rows[int64_t(i) * C + p] = row[p];
    }
}

// grid (ntq, B), 4 waves: wave w ranks heads w, w+4, ... over the tile's tokens with 64-lane
// ballots.  poslist: HIGH ranks from the front, LOW ranks from the back (positions).
// Re-tiering: srcdesc at the same index as poslist tells the page writer where a kept token's
// codes are: its previous tier, its rank among that tier (so its old page, through the old
// row, and its slot there); FRESH and invalid previous tiers carry page 0.
__device__ __forceinline__ void select_block(
    const int tq, const int b, const uint8_t *__restrict__ tier, const uint8_t *__restrict__ prev,
    const int32_t *__restrict__ cu, int Hkv, int ntq, int max_seqlen,
    const int32_t *__restrict__ tile_base, const int32_t *__restrict__ tile_base2,
    const int32_t *__restrict__ ok, const int32_t *__restrict__ old_rows, int C,
    int32_t *__restrict__ poslist, uint2 *__restrict__ srcdesc) {
    const int lo = cu[b], N = cu[b + 1] - lo;
    const int t0 = tq * QTILE;
    if (N > max_seqlen || t0 >= N) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar loads
    const int nt = min(QTILE, N - t0);
    const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    constexpr int NC = QTILE / 64;          // 64-token chunks of a tile
    constexpr int HW = 2;                   // heads per wave per pass
    for (int h0 = wave; h0 < Hkv; h0 += 4 * HW) {
        // every load of the pass's heads is requested before any is used: the heads' flags
        // and rank bases (scalar), the tier bytes of every chunk (a lane past the tile reads
        // its last token and counts as PRUNE)
        int okh[HW], bH[HW], bL[HW], b2H[HW], b2L[HW];
        int xs[HW][NC], ys[HW][NC];
#pragma unroll
        for (int j = 0; j < HW; ++j) {
            const int h = min(h0 + 4 * j, Hkv - 1);
            const int i = b * Hkv + h;
            okh[j] = ok[i];
            const int64_t tb = ((int64_t(b) * ntq + tq) * Hkv + h) * 2;
            bH[j] = tile_base[tb];
            bL[j] = tile_base[tb + 1];
            b2H[j] = prev ? tile_base2[tb] : 0;
            b2L[j] = prev ? tile_base2[tb + 1] : 0;
#pragma unroll
            for (int q = 0; q < NC; ++q) {
                const int64_t r = (int64_t(lo) + t0 + min(64 * q + lane, nt - 1)) * Hkv + h;
                xs[j][q] = tier[r];
                ys[j][q] = prev ? prev[r] : int(PRUNE);
            }
        }
#pragma unroll
        for (int j = 0; j < HW; ++j) {
            const int h = h0 + 4 * j;
            if (h >= Hkv || !okh[j]) continue;
            const int i = b * Hkv + h;
            int rH = bH[j], rL = bL[j], oH = b2H[j], oL = b2L[j];
            int32_t *pl = poslist + int64_t(i) * max_seqlen;
            uint2 *sd = prev ? srcdesc + int64_t(i) * max_seqlen : nullptr;
            const int32_t *orow = prev ? old_rows + int64_t(i) * C : nullptr;
            // re-tier: each chunk's record (index in the head's list, old row entry, tag), the
            // old page ids then loaded together
            int sk[NC], so[NC];
            uint32_t stag[NC];
#pragma unroll
            for (int q = 0; q < NC; ++q) sk[q] = -1;
#pragma unroll
            for (int q = 0; q < NC; ++q) {
                const int tt = 64 * q + lane;
                if (64 * q >= nt) break;
                const int x = tt < nt ? xs[j][q] : int(PRUNE);
                const uint64_t mH = __ballot(x == HIGH);
                const uint64_t mL = __ballot(x == LOW);
                int k = -1;                                  // the token's index in poslist
                if (x == HIGH) k = rH + __popcll(mH & lt);
                else if (x == LOW) k = max_seqlen - 1 - (rL + __popcll(mL & lt));
                if (k >= 0) pl[k] = t0 + tt;
                rH += __popcll(mH);
                rL += __popcll(mL);
                if (prev) {
                    const int y = tt < nt ? ys[j][q] : int(PRUNE);
                    const uint64_t nH = __ballot(y == HIGH);
                    const uint64_t nL = __ballot(y == LOW);
                    // the old rank is below the head's old count (checked by the scan), so
                    // the old page index stays within the head's old row
                    int orw = -1, osl = 0;
                    if (y == HIGH) {
                        const int o = oH + __popcll(nH & lt);
                        osl = o & (HS - 1);
                        orw = o / HS;
                    } else if (y == LOW) {
                        const int o = oL + __popcll(nL & lt);
                        osl = o & (LS - 1);
                        orw = C - 1 - o / LS;
                    }
                    sk[q] = k;
                    so[q] = orw;
                    stag[q] = uint32_t((y << 8) | osl);
                    oH += __popcll(nH);
                    oL += __popcll(nL);
                }
            }
            if (prev) {
                int pg[NC];
#pragma unroll
                for (int q = 0; q < NC; ++q) pg[q] = (sk[q] >= 0 && so[q] >= 0) ? orow[so[q]] : 0;
#pragma unroll
                for (int q = 0; q < NC; ++q)
                    if (sk[q] >= 0) sd[sk[q]] = make_uint2(uint32_t(pg[q]), stag[q]);
            }
        }
    }
}

__global__ __launch_bounds__(256) void quant_select_kernel(
    const uint8_t *__restrict__ tier, const uint8_t *__restrict__ prev,
    const int32_t *__restrict__ cu, int Hkv, int ntq, int max_seqlen,
    const int32_t *__restrict__ tile_base, const int32_t *__restrict__ tile_base2,
    const int32_t *__restrict__ ok, const int32_t *__restrict__ old_rows, int C,
    int32_t *__restrict__ poslist, uint2 *__restrict__ srcdesc) {
    select_block(blockIdx.x, blockIdx.y, tier, prev, cu, Hkv, ntq, max_seqlen, tile_base,
                 tile_base2, ok, old_rows, C, poslist, srcdesc);
}

// The commits (workgroups 0 .. nheads - 1, one per head) and the ranks (the rest, one per
// (request, 256-token tile)) of a fused round in one launch.  The ranks read only what the
// per-head scan launch wrote (tile bases, head flags and, when re-tiering, the changed heads'
// old rows) and write the position lists and source records, none of which the commits read
// or write, so the two need no order between them.
__global__ __launch_bounds__(256) void round_commit_select_kernel(
    int nheads, int32_t *__restrict__ rows_l, int32_t *__restrict__ count_l,
    const int32_t *__restrict__ cnt0, const int32_t *__restrict__ new_count,
    const uint8_t *__restrict__ changed, int C, int64_t P,
    int layer_gid0, int32_t *status, uint64_t *ctr, int32_t *__restrict__ ring,
    int32_t *__restrict__ owner, const CompactHdr *snap, int32_t *__restrict__ ok,
    const uint8_t *__restrict__ tier, const uint8_t *__restrict__ prev,
    const int32_t *__restrict__ cu, int Hkv, int ntq, int max_seqlen,
    const int32_t *__restrict__ tile_base, const int32_t *__restrict__ tile_base2,
    const int32_t *__restrict__ old_rows, int32_t *__restrict__ poslist,
    uint2 *__restrict__ srcdesc) {
    const int x = blockIdx.x;
    if (x < nheads) {
        round_commit_block(x, nheads, rows_l, count_l, cnt0, new_count, changed, C, P,
                           layer_gid0, status, ctr, ring, owner, snap, ok, nullptr, nullptr);
    } else {
        const int k = x - nheads;
        select_block(k % ntq, k / ntq, tier, prev, cu, Hkv, ntq, max_seqlen, tile_base,
                     tile_base2, ok, old_rows, C, poslist, srcdesc);
    }
}

constexpr int QP_WAVES = 4;
#ifndef KVC_ROUND_MERGE
#define KVC_ROUND_MERGE 1        // prompt-mode rounds: commits and ranks in one launch
#endif
#ifndef KVC_RB_AHEAD
#define KVC_RB_AHEAD 1
#endif
// re-tier passes whose old words are in flight ahead of the pass being written: at 1 the
// re-tier kernel fits 72 VGPRs when asked for 6 or more waves per EU, so 7 waves per SIMD run
// (the LDS staging allows no more); 2 and 3 measured slower on the chain-of-thought re-tier
// round (284 us against 278 at the time) once every slot's source record is requested at once
constexpr int RB_AHEAD = KVC_RB_AHEAD;
constexpr int VST_BYTES = LS * D;     // per-wave staging of value codes (LOW page size)

// prompt placement of one page: NP passes of 4 slots (one 16-lane group per slot).  The
// slots' positions are all loaded first, and each pass's K/V rows (16 bytes of each per lane)
// are requested while the pass before is quantized.
template <int NP, typename Page, typename Emit>
__device__ __forceinline__ void fresh_slots(const uint16_t *__restrict__ K,
                                            const uint16_t *__restrict__ V,
                                            const int32_t *__restrict__ pl, int lo, int Hkv, int h,
                                            int max_seqlen, int first, int m, bool high, int rg,
                                            int c, Page &load_page, Emit &emit) {
    int pos[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int s = 4 * p + rg;
        pos[p] = 0;
        if (s < m) pos[p] = high ? pl[first + s] : pl[max_seqlen - 1 - (first + s)];
    }
    load_page();
    // the rows of pass p + 1 are requested before pass p is quantized (a slot past the page's
    // tokens reads the rows of position 0, unconditionally, and is written as zeros)
    typedef unsigned int fs_u4 __attribute__((ext_vector_type(4)));
    fs_u4 rk[NP], rv[NP];
    auto issue = [&](int p) {
        const int64_t roff = ((int64_t(lo) + pos[p]) * Hkv + h) * D + 8 * c;
        rk[p] = __builtin_nontemporal_load(reinterpret_cast<const fs_u4 *>(K + roff));
        rv[p] = __builtin_nontemporal_load(reinterpret_cast<const fs_u4 *>(V + roff));
    };
    issue(0);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        if (p + 1 < NP) issue(p + 1);
        const bool live = 4 * p + rg < m;
        float xk[8], xv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xk[2 * e] = h2f(uint16_t(rk[p][e] & 0xffffu));
            xk[2 * e + 1] = h2f(uint16_t(rk[p][e] >> 16));
            xv[2 * e] = h2f(uint16_t(rv[p][e] & 0xffffu));
            xv[2 * e + 1] = h2f(uint16_t(rv[p][e] >> 16));
        }
        emit(4 * p + rg, live, xk, xv);
    }
}

// grid (ceil(C / 4), B*Hkv): wave w of block x writes page index 4x + w of head y, whole.
// REBUILD: each token's codes come from the fp16 rows (previous tier FRESH), are copied from
// its old page (tier unchanged), or are re-quantized from its old K8V4 codes (HIGH -> LOW).
// (at least 6 waves per EU requested: the re-tier instance then fits 7, which measured 5%
// faster on the chain-of-thought re-tier round than the compiler's own 77-VGPR choice)
template <bool REBUILD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6))) void quant_pages_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ cu, int Hkv, int C, int max_seqlen,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l,
    const int32_t *__restrict__ ok, const int32_t *__restrict__ poslist,
    const uint2 *__restrict__ srcdesc, uint8_t *__restrict__ pages, int32_t *status) {
    __shared__ uint8_t s_v[QP_WAVES][VST_BYTES];
    __shared__ uint16_t s_par[QP_WAVES][LS][4];
    __shared__ uint4 s_ov[REBUILD ? QP_WAVES : 1][4][16];   // re-tier: old value unit groups
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = blockIdx.y;
    const int nheads = gridDim.y;
    // the flags and the head's counts are requested together (no branch between them)
    const int ok_all = ok[nheads], ok_i = ok[i];
    const int nh = count_l[2 * i], nl = count_l[2 * i + 1];
    asm volatile("" ::"s"(nh), "s"(nl));   // (keeps the counts' loads above the branch)
    if (ok_all != 0 || !ok_i) return;     // pool failed earlier, head mismatched or kept
    const int b = i / Hkv, h = i - b * Hkv;
    const int qH = ceil_div(nh, HS), qL = ceil_div(nl, LS);
    const int pi = blockIdx.x * QP_WAVES + wave;
    if (pi >= qH + qL) return;
    // HIGH page pi of the head's row, or LOW page lp = pi - qH (taken from the row's end);
    // no branch around the page id's load, so it is in flight with the slots' first loads
    const bool high = pi < qH;
    const int lp = high ? pi : pi - qH;
    const int first = lp * (high ? HS : LS);
    const int m = min(high ? HS : LS, (high ? nh : nl) - first);
    const int64_t row_at = int64_t(i) * C + (high ? pi : C - 1 - lp);
    const int T = high ? HIGH : LOW;
    // the page id is loaded after each path's first per-slot loads (positions or source
    // records), so that no wait for it stands before them
    uint8_t *pg = nullptr;
    int32_t pos_end = -1;     // position of slot `lane` (lanes < LS), for the final store
    const int32_t *pl = poslist + int64_t(i) * max_seqlen;
    auto load_page = [&]() {
        asm volatile("" ::: "memory");
        pg = pages + int64_t(rows_l[row_at]) * PAGE;
        const int sl = min(lane, m - 1);
        pos_end = pl[high ? first + sl : max_seqlen - 1 - (first + sl)];
    };
    const int lo = cu[b];
    const int rg = lane >> 4, c = lane & 15;
    uint8_t *sv = s_v[wave];
    // quantize the lane's 8 channels of slot s from float rows (or store a zero slot), write
    // the key codes to the page and stage value codes and parameters in LDS
    auto emit_fresh = [&](int s, bool live, const float (&xk)[8], const float (&xv)[8]) {
        uint32_t kw0 = 0, kw1 = 0;
        const RowQ qk = row_params(xk, high ? 255.0f : 15.0f);
        uint32_t kb[8], vb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) kb[e] = code_bits(xk[e], qk);
        if (high) {
            kw0 = gather4(kb[0], kb[1], kb[2], kb[3]);
            kw1 = gather4(kb[4], kb[5], kb[6], kb[7]);
        } else {
            // nibble k_nib(e) holds channel e: bytes (c0 c1) (c4 c5) (c2 c3) (c6 c7), low first
            kw0 = gather4(kb[0], kb[4], kb[2], kb[6]) | (gather4(kb[1], kb[5], kb[3], kb[7]) << 4);
        }
        const RowQ qv = row_params(xv, high ? 15.0f : 3.0f);
#pragma unroll
        for (int e = 0; e < 8; ++e) vb[e] = code_bits(xv[e], qv);
        const uint32_t vw0 = gather4(vb[0], vb[1], vb[2], vb[3]);
        const uint32_t vw1 = gather4(vb[4], vb[5], vb[6], vb[7]);
        store_slot(pg, sv, s_par[wave], high, s, c, live, kw0, kw1, vw0, vw1, qk.s16, qk.z16,
                   qv.s16, qv.z16);
    };
    if constexpr (!REBUILD) {
        // every row of the page is requested before the first one is quantized
        if (high) fresh_slots<HS / 4>(K, V, pl, lo, Hkv, h, max_seqlen, first, m, true, rg, c, load_page, emit_fresh);
        else fresh_slots<LS / 4>(K, V, pl, lo, Hkv, h, max_seqlen, first, m, false, rg, c, load_page, emit_fresh);
    } else {
    // re-tier placement.  Every slot's position and source (previous tier, old page id, old
    // slot) are loaded for all of the page's passes first; then each pass reads its old codes
    // (or fp16 rows) and emits.
    auto rebuild = [&](auto np_c) {
        constexpr int NP = decltype(np_c)::value;
        // (a FRESH slot's position, needed only for its fp16 rows, is loaded when used)
        int sy[NP], opg[NP];     // sy: previous tier << 8 | old slot
        auto index_of = [&](int s) -> int64_t { return high ? first + s : max_seqlen - 1 - (first + s); };
        // every pass's record is requested before any is used: a slot past the page's tokens
        // reads the page's last token's record (in the list, no branch around the load) and
        // then counts as empty
        uint2 d[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p)
            d[p] = srcdesc[int64_t(i) * max_seqlen + index_of(min(4 * p + rg, m - 1))];
        load_page();
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const bool in = 4 * p + rg < m;
            opg[p] = in ? int(d[p].x) : 0;
            sy[p] = in ? int(d[p].y) : int(FRESH) << 8;
        }
        auto src_of = [&](int p) { return sy[p] >> 8; };
        // a pass's slot validity and, for a slot read from an old page, its old-page words:
        // the 16-byte value unit this lane loads for the row (the row's 16 lanes share the
        // slot and load its 256-byte unit group), key words and parameters
        auto valid_of = [&](int p) {
            if (4 * p + rg >= m) return false;
            // a tier never rises, and a fresh token needs its fp16 rows
            return src_of(p) == T || (src_of(p) == HIGH && T == LOW) || (src_of(p) == FRESH && K != nullptr);
        };
        auto old_words = [&](int p, uint4 &ov, uint2 &okw, uint2 &opar) {
            ov = make_uint4(0u, 0u, 0u, 0u);
            okw = opar = make_uint2(0u, 0u);
            if (!valid_of(p) || src_of(p) == FRESH) return;
            const uint8_t *op = pages + int64_t(opg[p]) * PAGE;
            const int osl = sy[p] & 255;
            ov = *reinterpret_cast<const uint4 *>(op + V_OFF + 16 * (16 * ((osl & 15) >> 2) + c));
            if (src_of(p) == HIGH)
                okw = *reinterpret_cast<const uint2 *>(op + K_OFF + osl * 128 + 8 * c);
            else
                okw.x = *reinterpret_cast<const uint32_t *>(op + K_OFF + osl * 64 + 4 * c);
            opar = *reinterpret_cast<const uint2 *>(op + PARAM_OFF + 8 * osl);
        };
        // the old words of pass p + RB_AHEAD are requested before pass p waits on its LDS
        // staging (the loop is unrolled: the arrays are registers, RB_AHEAD + 1 sets live)
        uint4 ov[NP];
        uint2 okw[NP], opar[NP];
#pragma unroll
        for (int p = 0; p < RB_AHEAD && p < NP; ++p) old_words(p, ov[p], okw[p], opar[p]);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int s = 4 * p + rg;
            const bool valid = valid_of(p);
            if (4 * p + rg < m && !valid && c == 0) atomicOr(status, KVC_DEV_BAD_TIER);
            if (p + RB_AHEAD < NP)
                old_words(p + RB_AHEAD, ov[p + RB_AHEAD], okw[p + RB_AHEAD], opar[p + RB_AHEAD]);
            const int osl = sy[p] & 255;                                   // old slot
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            s_ov[wave][rg][c] = ov[p];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (!valid) {
                store_slot(pg, sv, s_par[wave], high, s, c, false, 0, 0, 0, 0, 0, 0, 0, 0);
            } else if (src_of(p) == T) {
                // unchanged tier: copy the token's codes and parameters from its old page
                uint32_t kw0 = 0, kw1 = 0, vw0 = 0, vw1 = 0;
                uint32_t kc[8], vc[8];
                old_codes_staged(okw[p], s_ov[wave][rg], T, osl, c, kc, vc);
                const uint32_t kp = opar[p].x, vp = opar[p].y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vw0 |= vc[e] << (8 * e);
                    vw1 |= vc[4 + e] << (8 * e);
                }
                if (high) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kw0 |= kc[e] << (8 * e);
                        kw1 |= kc[4 + e] << (8 * e);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) kw0 |= kc[e] << (4 * k_nib(e));
                }
                store_slot(pg, sv, s_par[wave], high, s, c, true, kw0, kw1, vw0, vw1,
                           uint16_t(kp & 0xffffu), uint16_t(kp >> 16), uint16_t(vp & 0xffffu),
                           uint16_t(vp >> 16));
            } else {
                // fresh rows, or a HIGH -> LOW demotion from the old K8V4 reconstruction
                float xk[8], xv[8];
                if (src_of(p) == FRESH) {
                    const int64_t roff = ((int64_t(lo) + pl[index_of(s)]) * Hkv + h) * D + 8 * c;
                    load_row8(K + roff, true, xk);
                    load_row8(V + roff, true, xv);
                } else {
                    uint32_t kc[8], vc[8];
                    old_codes_staged(okw[p], s_ov[wave][rg], HIGH, osl, c, kc, vc);
                    const uint32_t kp = opar[p].x, vp = opar[p].y;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        xk[e] = recon16(kc[e], kp);
                        xv[e] = recon16(vc[e], vp);
                    }
                }
                emit_fresh(s, true, xk, xv);
            }
        }
    };
    if (high) rebuild(std::integral_constant<int, HS / 4>{});
    else rebuild(std::integral_constant<int, LS / 4>{});
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    pack_values(pg, sv, high, lane);
    // parameters and positions of all 32 slots (slots >= m, and 16..31 of a HIGH page, empty)
    if (lane < LS) {
        const int s = lane;
        uint32_t a = 0, bb = 0;
        int32_t pos = -1;
        if (s < m) {
            a = uint32_t(s_par[wave][s][0]) | (uint32_t(s_par[wave][s][1]) << 16);
            bb = uint32_t(s_par[wave][s][2]) | (uint32_t(s_par[wave][s][3]) << 16);
            pos = pos_end;
        }
        st_page8(pg + PARAM_OFF + 8 * s, a, bb);
        st_page4(pg + POS_OFF + 4 * s, uint32_t(pos));
    }
}

// ---- precision schemes: slot-major pages --------------------------------------------------
// grid (ceil(C / 4), B*Hkv): wave w of block x writes page index 4x + w of head y, whole.
// Keys slot-major (16 lanes per row, channels 8c .. 8c + 7, four slots per pass, stored from
// registers); values in blocks of 16 slots in the decode's operand order: the slots' codes
// are staged in LDS (one byte per code), then every lane packs its share of each block
// (pack_value_block); the code bytes past the values are zero, parameters and positions of
// all 32 slot indices as in the default layout.
__global__ __launch_bounds__(256) void scheme_pages_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ cu, int Hkv, int C, int max_seqlen,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l,
    const int32_t *__restrict__ ok, const int32_t *__restrict__ poslist, int kh, int vh, int kl,
    int vl, uint8_t *__restrict__ pages) {
    __shared__ uint8_t s_vc[QP_WAVES][LS][D];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = blockIdx.y;
    const int nheads = gridDim.y;
    if (ok[nheads] != 0 || !ok[i]) return;
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
        first = (pi - qH) * LS;
        m = min(LS, nl - first);
        page = rows_l[int64_t(i) * C + C - 1 - (pi - qH)];
    } else {
        return;
    }
    const int kb = high ? kh : kl, vb = high ? vh : vl;
    const int S = high ? HS : LS;
    uint8_t *pg = pages + int64_t(page) * PAGE;
    const int32_t *pl = poslist + int64_t(i) * max_seqlen;
    const int lo = cu[b];
    const int rg = lane >> 4, c = lane & 15;
    const float lk = float((1 << kb) - 1), lv = float((1 << vb) - 1);
    uint8_t (*vc)[D] = s_vc[wave];
    for (int pass = 0; pass < S / 4; ++pass) {
        const int sl = 4 * pass + rg;
        const bool live = sl < m;
        int pos = 0;
        if (live) pos = high ? pl[first + sl] : pl[max_seqlen - 1 - (first + sl)];
        const int64_t roff = ((int64_t(lo) + pos) * Hkv + h) * D + 8 * c;
        float xk[8], xv[8];
        load_row8(K + roff, live, xk);
        load_row8(V + roff, live, xv);
        const RowQ qk = row_params(xk, lk);
        const RowQ qv = row_params(xv, lv);
        uint64_t wk = 0;
        uint32_t v0 = 0, v1 = 0;
        if (live) {
#pragma unroll
            for (int e = 0; e < 8; ++e) wk |= uint64_t(code_of(xk[e], qk)) << (kb * e);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v0 |= code_of(xv[e], qv) << (8 * e);
                v1 |= code_of(xv[4 + e], qv) << (8 * e);
            }
        }
        store_codes(pg + 16 * kb * sl + c * kb, wk, kb);
        *reinterpret_cast<uint2 *>(&vc[sl][8 * c]) = make_uint2(v0, v1);
        if (c == 0) {
            const uint32_t a = live ? uint32_t(qk.s16) | (uint32_t(qk.z16) << 16) : 0u;
            const uint32_t bb = live ? uint32_t(qv.s16) | (uint32_t(qv.z16) << 16) : 0u;
            st_page8(pg + PARAM_OFF + 8 * sl, a, bb);
            st_page4(pg + POS_OFF + 4 * sl, uint32_t(live ? pos : -1));
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // value blocks of 16 slots, 256 vb bytes each
    uint8_t *vbase = pg + 16 * kb * S;
    for (int f = 0; f < S / 16; ++f) {
        uint8_t *dst = vbase + 256 * vb * f + 4 * vb * lane;
        if (vb == 8) pack_value_block<8>(dst, vc, f, rg, c);
        else if (vb == 4) pack_value_block<4>(dst, vc, f, rg, c);
        else if (vb == 2) pack_value_block<2>(dst, vc, f, rg, c);
        else pack_value_block<1>(dst, vc, f, rg, c);
    }
    // code bytes past the values (16 S (kb + vb) is a multiple of 16), slots S..31's fields
    for (int k = S * (kb + vb) + lane; k < PARAM_OFF / 16; k += 64)
        st_page16(pg + 16 * k, 0u, 0u, 0u, 0u);
    if (lane >= S && lane < LS) {
        st_page8(pg + PARAM_OFF + 8 * lane, 0u, 0u);
        st_page4(pg + POS_OFF + 4 * lane, uint32_t(-1));
    }
}

// Re-tier placement in a precision scheme's layout (grid and waves as scheme_pages_kernel).
// Each slot of a rebuilt head comes from its source record (quant_select): its codes and
// parameters copied bit for bit from its old page when its tier is unchanged (the key bytes
// as they are, the value codes through the LDS staging), re-quantized at the LOW widths from
// the fp16 rounding of its HIGH reconstruction when demoted, or quantized from its fp16 rows
// when FRESH.
__global__ __launch_bounds__(256) void scheme_rebuild_pages_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ cu, int Hkv, int C, int max_seqlen,
    const int32_t *__restrict__ rows_l, const int32_t *__restrict__ count_l,
    const int32_t *__restrict__ ok, const int32_t *__restrict__ poslist,
    const uint2 *__restrict__ srcdesc, int kh, int vh, int kl, int vl,
    uint8_t *__restrict__ pages, int32_t *status) {
    __shared__ uint8_t s_vc[QP_WAVES][LS][D];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = blockIdx.y;
    const int nheads = gridDim.y;
    if (ok[nheads] != 0 || !ok[i]) return;
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
        first = (pi - qH) * LS;
        m = min(LS, nl - first);
        page = rows_l[int64_t(i) * C + C - 1 - (pi - qH)];
    } else {
        return;
    }
    const int T = high ? HIGH : LOW;
    const int kb = high ? kh : kl, vb = high ? vh : vl;
    const int S = high ? HS : LS;
    uint8_t *pg = pages + int64_t(page) * PAGE;
    const int32_t *pl = poslist + int64_t(i) * max_seqlen;
    const uint2 *sd = srcdesc + int64_t(i) * max_seqlen;
    const int lo = cu[b];
    const int rg = lane >> 4, c = lane & 15;
    const float lk = float((1 << kb) - 1), lv = float((1 << vb) - 1);
    uint8_t (*vc)[D] = s_vc[wave];
    for (int pass = 0; pass < S / 4; ++pass) {
        const int sl = 4 * pass + rg;
        const bool live = sl < m;
        const int64_t x = high ? first + sl : max_seqlen - 1 - (first + sl);
        int pos = 0, src = FRESH, osl = 0;
        const uint8_t *op = pages;
        if (live) {
            pos = pl[x];
            const uint2 d = sd[x];
            op = pages + int64_t(d.x) * PAGE;
            src = int(d.y >> 8);
            osl = int(d.y & 255u);
        }
        // a tier never rises, and a fresh token needs its fp16 rows
        const bool valid = live && (src == T || (src == HIGH && T == LOW) ||
                                    (src == FRESH && K != nullptr));
        if (live && !valid && c == 0) atomicOr(status, KVC_DEV_BAD_TIER);
        uint64_t wk = 0;
        uint32_t a = 0u, bb = 0u;
        uint32_t vcode[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        bool by16 = true;            // vcode[n] is channel 16 n + c (else 8 c + n)
        if (valid && src == T) {
            // unchanged tier: the old slot's key bytes as they are, its value codes unpacked
            const uint8_t *ks = op + 16 * kb * osl + c * kb;
            if (kb == 8) wk = *reinterpret_cast<const uint64_t *>(ks);
            else if (kb == 4) wk = *reinterpret_cast<const uint32_t *>(ks);
            else if (kb == 2) wk = *reinterpret_cast<const uint16_t *>(ks);
            else wk = *ks;
            sch_val_codes(op, kb, vb, S, osl, c, vcode);
            const uint2 par = *reinterpret_cast<const uint2 *>(op + PARAM_OFF + 8 * osl);
            a = par.x;
            bb = par.y;
        } else if (valid) {
            float xk[8], xv[8];
            if (src == HIGH) {
                // HIGH -> LOW: the fp16 rounding of the old HIGH page's reconstruction
                uint32_t kc[8], vo[8];
                sch_key_codes(op, kh, osl, c, kc);
                sch_val_codes(op, kh, vh, HS, osl, c, vo);
                const uint2 par = *reinterpret_cast<const uint2 *>(op + PARAM_OFF + 8 * osl);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xk[e] = recon16(kc[e], par.x);
                    xv[e] = recon16(vo[e], par.y);
                }
            } else {
                const int64_t roff = ((int64_t(lo) + pos) * Hkv + h) * D + 8 * c;
                load_row8(K + roff, true, xk);
                load_row8(V + roff, true, xv);
                by16 = false;
            }
            const RowQ qk = row_params(xk, lk);
            const RowQ qv = row_params(xv, lv);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                wk |= uint64_t(code_of(xk[e], qk)) << (kb * e);
                vcode[e] = code_of(xv[e], qv);
            }
            a = uint32_t(qk.s16) | (uint32_t(qk.z16) << 16);
            bb = uint32_t(qv.s16) | (uint32_t(qv.z16) << 16);
        }
        store_codes(pg + 16 * kb * sl + c * kb, wk, kb);
#pragma unroll
        for (int n = 0; n < 8; ++n) vc[sl][by16 ? 16 * n + c : 8 * c + n] = uint8_t(vcode[n]);
        if (c == 0) {
            st_page8(pg + PARAM_OFF + 8 * sl, a, bb);
            st_page4(pg + POS_OFF + 4 * sl, uint32_t(valid ? pos : -1));
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint8_t *vbase = pg + 16 * kb * S;
    for (int f = 0; f < S / 16; ++f) {
        uint8_t *dst = vbase + 256 * vb * f + 4 * vb * lane;
        if (vb == 8) pack_value_block<8>(dst, vc, f, rg, c);
        else if (vb == 4) pack_value_block<4>(dst, vc, f, rg, c);
        else if (vb == 2) pack_value_block<2>(dst, vc, f, rg, c);
        else pack_value_block<1>(dst, vc, f, rg, c);
    }
    for (int k = S * (kb + vb) + lane; k < PARAM_OFF / 16; k += 64)
        st_page16(pg + 16 * k, 0u, 0u, 0u, 0u);
    if (lane >= S && lane < LS) {
        st_page8(pg + PARAM_OFF + 8 * lane, 0u, 0u);
        st_page4(pg + POS_OFF + 4 * lane, uint32_t(-1));
    }
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
    const bool rebuild = prev_tier != nullptr;
    if (rebuild && (!changed || !old_rows || !old_count)) return KVC_E_NULL;
    if (!rebuild && (changed || old_rows || old_count)) return KVC_E_UNSUPPORTED;
    if (!cu) return KVC_E_NULL;
    if (total_tokens > 0 && !tier) return KVC_E_NULL;
    if (!rebuild && total_tokens > 0 && (!k || !v)) return KVC_E_NULL;
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
    int32_t *tile_cnt2 = rebuild ? reinterpret_cast<int32_t *>(w + L.tile_cnt2) : nullptr;
    int32_t *tile_base2 = rebuild ? reinterpret_cast<int32_t *>(w + L.tile_base2) : nullptr;
    int32_t *ok = reinterpret_cast<int32_t *>(w + L.ok);
    int32_t *poslist = reinterpret_cast<int32_t *>(w + L.poslist);
    uint2 *srcdesc = rebuild ? reinterpret_cast<uint2 *>(w + L.srcdesc) : nullptr;
    const int B = g->batch, Hkv = g->num_kv_heads, C = g->row_capacity;
    const int nheads = B * Hkv;
    const int32_t *rows_l = p->page_table + int64_t(layer) * nheads * C;
    const int32_t *count_l = p->count + int64_t(layer) * nheads * 2;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(quant_count_kernel, dim3(L.ntq, B), dim3(256), 0, s, tier, prev_tier, cu,
                       Hkv, L.ntq, max_seqlen, p->dev_status, tile_cnt, tile_cnt2, ok, nheads);
    rc = launch_check("kvc_quantize_and_place/count");
    if (rc) return rc;
    hipLaunchKernelGGL(quant_scan_kernel, dim3(Hkv, B), dim3(256), 0, s, tile_cnt, tile_cnt2, cu,
                       Hkv, L.ntq, max_seqlen, count_l, changed, old_count, tile_base,
                       tile_base2, ok, p->dev_status);
    rc = launch_check("kvc_quantize_and_place/scan");
    if (rc) return rc;
    hipLaunchKernelGGL(quant_select_kernel, dim3(L.ntq, B), dim3(256), 0, s, tier, prev_tier, cu,
                       Hkv, L.ntq, max_seqlen, tile_base, tile_base2, ok, old_rows, C,
                       poslist, srcdesc);
    rc = launch_check("kvc_quantize_and_place/select");
    if (rc) return rc;
    const dim3 grid((C + QP_WAVES - 1) / QP_WAVES, nheads);
    if (rebuild)
        hipLaunchKernelGGL(quant_pages_kernel<true>, grid, dim3(64 * QP_WAVES), 0, s, k, v, cu, Hkv,
                           C, max_seqlen, rows_l, count_l, ok, poslist, srcdesc, p->pages,
                           p->dev_status);
    else
        hipLaunchKernelGGL(quant_pages_kernel<false>, grid, dim3(64 * QP_WAVES), 0, s, k, v, cu,
                           Hkv, C, max_seqlen, rows_l, count_l, ok, poslist, nullptr, p->pages,
                           p->dev_status);
    return launch_check("kvc_quantize_and_place/pages");
}

extern "C" int kvc_quantize_and_place_scheme(const kvc_geom *g, const kvc_scheme *sc,
                                             int32_t layer, const kvc_pool *p, const uint16_t *k,
                                             const uint16_t *v, const int32_t *cu,
                                             int64_t total_tokens, int32_t max_seqlen,
                                             const uint8_t *tier, const uint8_t *prev_tier,
                                             const uint8_t *changed, const int32_t *old_rows,
                                             const int32_t *old_count, void *ws, size_t ws_bytes,
                                             kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    rc = check_scheme(sc);
    if (rc) return rc;
    const bool rebuild = prev_tier != nullptr;
    if (rebuild && (!changed || !old_rows || !old_count)) return KVC_E_NULL;
    if (!rebuild && (changed || old_rows || old_count)) return KVC_E_UNSUPPORTED;
    if (!cu) return KVC_E_NULL;
    if (total_tokens > 0 && !tier) return KVC_E_NULL;
    if (!rebuild && total_tokens > 0 && (!k || !v)) return KVC_E_NULL;
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
    int32_t *tile_cnt2 = rebuild ? reinterpret_cast<int32_t *>(w + L.tile_cnt2) : nullptr;
    int32_t *tile_base2 = rebuild ? reinterpret_cast<int32_t *>(w + L.tile_base2) : nullptr;
    int32_t *ok = reinterpret_cast<int32_t *>(w + L.ok);
    int32_t *poslist = reinterpret_cast<int32_t *>(w + L.poslist);
    uint2 *srcdesc = rebuild ? reinterpret_cast<uint2 *>(w + L.srcdesc) : nullptr;
    const int B = g->batch, Hkv = g->num_kv_heads, C = g->row_capacity;
    const int nheads = B * Hkv;
    const int32_t *rows_l = p->page_table + int64_t(layer) * nheads * C;
    const int32_t *count_l = p->count + int64_t(layer) * nheads * 2;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(quant_count_kernel, dim3(L.ntq, B), dim3(256), 0, s, tier, prev_tier, cu,
                       Hkv, L.ntq, max_seqlen, p->dev_status, tile_cnt, tile_cnt2, ok, nheads);
    rc = launch_check("kvc_quantize_and_place_scheme/count");
    if (rc) return rc;
    hipLaunchKernelGGL(quant_scan_kernel, dim3(Hkv, B), dim3(256), 0, s, tile_cnt, tile_cnt2, cu,
                       Hkv, L.ntq, max_seqlen, count_l, changed, old_count, tile_base,
                       tile_base2, ok, p->dev_status);
    rc = launch_check("kvc_quantize_and_place_scheme/scan");
    if (rc) return rc;
    hipLaunchKernelGGL(quant_select_kernel, dim3(L.ntq, B), dim3(256), 0, s, tier, prev_tier, cu,
                       Hkv, L.ntq, max_seqlen, tile_base, tile_base2, ok, old_rows, C, poslist,
                       srcdesc);
    rc = launch_check("kvc_quantize_and_place_scheme/select");
    if (rc) return rc;
    const dim3 grid((C + QP_WAVES - 1) / QP_WAVES, nheads);
    if (rebuild)
        hipLaunchKernelGGL(scheme_rebuild_pages_kernel, grid, dim3(64 * QP_WAVES), 0, s, k, v, cu,
                           Hkv, C, max_seqlen, rows_l, count_l, ok, poslist, srcdesc,
                           sc->k_bits_high, sc->v_bits_high, sc->k_bits_low, sc->v_bits_low,
                           p->pages, p->dev_status);
    else
        hipLaunchKernelGGL(scheme_pages_kernel, grid, dim3(64 * QP_WAVES), 0, s, k, v, cu, Hkv,
                           C, max_seqlen, rows_l, count_l, ok, poslist, sc->k_bits_high,
                           sc->v_bits_high, sc->k_bits_low, sc->v_bits_low, p->pages);
    return launch_check("kvc_quantize_and_place_scheme/pages");
}

// ---- the fused compaction round -------------------------------------------------------------
// kvc_score_tokens -> kvc_compact_pages -> kvc_quantize_and_place in four launches for up to
// ROUND_MAX_HEADS heads: score with per-tile counts (no counters to clear, no separate count
// launch), the per-head tile scans (totals, rank bases, a changed head's old row; the first
// workgroup also takes the round's start: pool status and ring counters), the commits (every
// workgroup makes the page demands' scan and the commit decision for itself) with the ranks
// beside them in the same launch, and the page writer.  (A round with no tokens runs the
// commits alone, as the separate commit launch, which also keeps the old rows.)
extern "C" int kvc_compaction_round(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                                    const float *acc, const int32_t *cu, int64_t total_tokens,
                                    int32_t max_seqlen, float alpha_h, float alpha_l,
                                    int32_t window, const uint16_t *k, const uint16_t *v,
                                    const uint8_t *prev_tier, uint8_t *tier, int32_t *new_count,
                                    uint8_t *changed, void *ws, size_t ws_bytes,
                                    kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    const bool retier = prev_tier != nullptr;
    if (!cu || !new_count || (total_tokens > 0 && (!acc || !tier))) return KVC_E_NULL;
    if (retier && !changed) return KVC_E_NULL;
    if (!retier && total_tokens > 0 && (!k || !v)) return KVC_E_NULL;
    if (total_tokens < 0 || window < 0 || max_seqlen < 0) return KVC_E_SHAPE;
    if (layer < 0 || layer >= g->num_layers) return KVC_E_SHAPE;
    const int B = g->batch, Hkv = g->num_kv_heads, C = g->row_capacity;
    const int nheads = B * Hkv;
    if (Hkv > 256 || nheads > ROUND_MAX_HEADS) return KVC_E_SHAPE;
    if (int64_t(nheads) * C >= (int64_t(1) << 31)) return KVC_E_SHAPE;
    if (acc && (reinterpret_cast<uintptr_t>(acc) & 15u) != 0) return KVC_E_ALIGN;
    if ((k && !aligned16(k)) || (v && !aligned16(v))) return KVC_E_ALIGN;
    RoundWs R(g, max_seqlen);
    if (!ws || ws_bytes < R.bytes) return KVC_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return KVC_E_ALIGN;
    char *w = static_cast<char *>(ws);
    const QuantWs L(g, max_seqlen);
    int32_t *tile_cnt = reinterpret_cast<int32_t *>(w + R.quant + L.tile_cnt);
    int32_t *tile_base = reinterpret_cast<int32_t *>(w + R.quant + L.tile_base);
    int32_t *tile_cnt2 = retier ? reinterpret_cast<int32_t *>(w + R.quant + L.tile_cnt2) : nullptr;
    int32_t *tile_base2 = retier ? reinterpret_cast<int32_t *>(w + R.quant + L.tile_base2) : nullptr;
    int32_t *ok = reinterpret_cast<int32_t *>(w + R.quant + L.ok);
    int32_t *poslist = reinterpret_cast<int32_t *>(w + R.quant + L.poslist);
    uint2 *srcdesc = retier ? reinterpret_cast<uint2 *>(w + R.quant + L.srcdesc) : nullptr;
    uint8_t *tile_chg = reinterpret_cast<uint8_t *>(w + R.tile_chg);
    int32_t *old_rows = retier ? reinterpret_cast<int32_t *>(w + R.old_rows) : nullptr;
    // every head's counts before the round (written by the per-head scans, read by the commits)
    int32_t *cnt0 = reinterpret_cast<int32_t *>(w + R.old_count);
    const int32_t *rows_l = p->page_table + int64_t(layer) * nheads * C;
    const int32_t *count_l = p->count + int64_t(layer) * nheads * 2;
    hipStream_t s = (hipStream_t)stream;
    rc = launch_round_score(g, acc, cu, max_seqlen, alpha_h, alpha_l, window, prev_tier, tier,
                            tile_cnt, tile_cnt2, tile_chg, p->dev_status, s);
    if (rc) return rc;
    const CompactWs CL(g);
    const bool work = max_seqlen > 0 && total_tokens > 0;
    const bool merge = KVC_ROUND_MERGE && work;
    hipLaunchKernelGGL(round_head_kernel, dim3(Hkv, B), dim3(256), 0, s, tile_cnt, tile_cnt2,
                       tile_chg, cu, Hkv, L.ntq, max_seqlen, tile_base, tile_base2, new_count,
                       retier ? changed : nullptr, ok, p->dev_status, p->ring_ctr,
                       reinterpret_cast<CompactHdr *>(w + R.compact + CL.hdr), rows_l, C,
                       merge ? old_rows : nullptr, count_l, cnt0);
    rc = launch_check("kvc_compaction_round/heads");
    if (rc) return rc;
    if (merge) {
        // commits and ranks in one launch (the old rows were taken by the per-head scans)
        hipLaunchKernelGGL(round_commit_select_kernel, dim3(nheads + L.ntq * B), dim3(256), 0, s,
                           nheads, p->page_table + int64_t(layer) * nheads * C,
                           p->count + int64_t(layer) * nheads * 2, cnt0, new_count,
                           retier ? changed : nullptr, C, g->num_pages, layer * nheads,
                           p->dev_status, p->ring_ctr, p->free_ring, p->owner,
                           reinterpret_cast<const CompactHdr *>(w + R.compact + CL.hdr), ok, tier,
                           prev_tier, cu, Hkv, L.ntq, max_seqlen, tile_base, tile_base2, old_rows,
                           poslist, srcdesc);
        rc = launch_check("kvc_compaction_round/commit+select");
        if (rc) return rc;
    } else {
        rc = launch_round_commit(g, layer, p, cnt0, new_count, retier ? changed : nullptr, ok,
                                 old_rows, w + R.compact, s);
        if (rc) return rc;
        if (!work) return KVC_OK;
        hipLaunchKernelGGL(quant_select_kernel, dim3(L.ntq, B), dim3(256), 0, s, tier, prev_tier,
                           cu, Hkv, L.ntq, max_seqlen, tile_base, tile_base2, ok, old_rows, C,
                           poslist, srcdesc);
        rc = launch_check("kvc_compaction_round/select");
        if (rc) return rc;
    }
    const dim3 grid((C + QP_WAVES - 1) / QP_WAVES, nheads);
    if (retier)
        hipLaunchKernelGGL(quant_pages_kernel<true>, grid, dim3(64 * QP_WAVES), 0, s, k, v, cu, Hkv,
                           C, max_seqlen, rows_l, count_l, ok, poslist, srcdesc, p->pages,
                           p->dev_status);
    else
        hipLaunchKernelGGL(quant_pages_kernel<false>, grid, dim3(64 * QP_WAVES), 0, s, k, v, cu,
                           Hkv, C, max_seqlen, rows_l, count_l, ok, poslist, nullptr, p->pages,
                           p->dev_status);
    return launch_check("kvc_compaction_round/pages");
}
