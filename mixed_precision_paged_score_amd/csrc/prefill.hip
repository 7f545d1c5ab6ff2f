// kvc_prefill_attention: causal prefill attention of the prompt, and the prompt's significance
// accumulators (the step before scoring).
//
// DiffKV review page: "Assumptions" (standard causal multi-head attention, the page's Eq. 1);
// "What carries the argument" (a token's significance is the mean of the attention it
// receives from subsequent tokens; referee major comment 2 counts the N - i later queries).
// acc_sum[t][hq] is therefore the sum, over the strictly later queries i > t of the same
// request, of query i's softmax weight on key t.
//
// Two launches:
//   prefill_fwd     flash-attention forward (one workgroup per 128 queries of one request and
//                   query head; 64-key blocks double-buffered in LDS): the output rows and
//                   each row's softmax max and sum (log2 units) into the workspace.
//   prefill_colsum  one workgroup per 256 keys of one request and query head (64 per wave):
//                   the scores against every later 32-query tile (staged once in LDS for the
//                   four waves) are recomputed, normalized with the rows' max and sum, and
//                   summed per key; each accumulator is written once.
// Matrix products are v_mfma_f32_16x16x32_f16 on S^T = K Q^T (a lane owns one query column,
// so row statistics and rescales stay in the lane) and O^T = V^T P^T (P^T is already in the
// operand layout: its k index is the key order of two S^T tiles).
#include "kvc_internal.h"
#include "workspace.h"

#pragma clang fp contract(off)

namespace kvc {
namespace pf {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

#ifndef KVC_PF_WAVES
#define KVC_PF_WAVES 8           // forward waves per workgroup (32 queries each)
#endif
constexpr int BN = 64;           // keys per block
// LDS row stride (halves) of the staged key and query tiles.  A lane of the 16x16x32 products
// reads 16 bytes of row c (c < 16) at column group g (g < 4); measured on gfx950 with
// SQ_LDS_BANK_CONFLICT, 16 such rows 272 bytes apart (D + 8) cost ~3.9 conflict cycles per
// ds_read_b128 and 288 bytes apart (D + 16) none
constexpr int KS = D + 16;
// LDS row stride (halves) of the transposed value tile.  Within each 32-key block the keys are
// stored permuted (vt_pos) so that the 8 keys one lane feeds to a V^T P^T product are one
// 16-byte run: one ds_read_b128 per operand, rows 160 bytes apart, which measured free of bank
// conflicts (two 8-byte reads 32 bytes apart in 144-byte rows cost ~7.9 conflict cycles each)
constexpr int VS = BN + 16;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float MARGIN = 8.0f;   // the running max moves only when exceeded by this (log2)
constexpr float M_INIT = -1.0e30f;

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four row groups of one query column): each
// permlane swap leaves the lane's own value in one operand and its partner's in the other.
// Written out so that the maxima skip the NaN quieting a library max adds (scores are never
// NaN); the two wait states before each swap are the ones it needs after a VALU write.
__device__ __forceinline__ float max_col(float x) {
    float t;
    asm("v_mov_b32 %1, %0\n\t"
        "s_nop 1\n\t"
        "v_permlane32_swap_b32 %0, %1\n\t"
        "v_max_f32 %0, %0, %1\n\t"
        "v_mov_b32 %1, %0\n\t"
        "s_nop 1\n\t"
        "v_permlane16_swap_b32 %0, %1\n\t"
        "v_max_f32 %0, %0, %1"
        : "+v"(x), "=&v"(t));
    return x;
}

// Workgroups are dispatched to the 8 XCDs round-robin by flat index, and each XCD has its own
// L2.  Both kernels therefore decode their flat index L as (XCD x = L % 8, slot j = L / 8) and
// give XCD x the groups x, x + 8, ... whole, W workgroups each: workgroups that stream the same
// keys and values (forward) or the same queries (column sums) share one L2.  Returns the
// group (or -1 past the last one) and the workgroup's index r within it.
constexpr int XCDS = 8;
__device__ __forceinline__ int xcd_group(int L, int W, int ngroups, int &r) {
    const int x = L % XCDS, j = L / XCDS;
    const int grp = x + XCDS * (j / W);
    r = j % W;
    return grp < ngroups ? grp : -1;
}
__host__ __device__ inline int xcd_grid(int ngroups, int W) {
    return XCDS * ((ngroups + XCDS - 1) / XCDS) * W;
}

// ---- staging of one key block (64 keys of one request and KV head) ----------------------
// K: thread t loads row (t / 16) + 16i, 16 bytes at column 8 (t % 16); stored row-major.
// V: thread t loads rows 2m, 2m + 1 (m = t % 32) at column 8d (d = t / 32 + 8i) and stores
// them transposed, a word holding both rows' halves of one column.
struct KBlock {
    uint4 k[4];
};
struct VBlock {
    uint4 v[4];
};

__device__ __forceinline__ uint4 ld_row(const uint16_t *base, int64_t row, bool ok, int col8) {
    return ok ? *reinterpret_cast<const uint4 *>(base + row * D + 8 * col8)
              : make_uint4(0, 0, 0, 0);
}

// NT threads stage a block: K rows (tid / 16) + (NT / 16) i, V row pairs (tid % 32) at
// columns 8 ((tid / 32) + (NT / 32) i).  Rows past the request's end (last block only) read
// as zeros; every other block loads without a per-row test.  Keys and values are requested
// together in either case, so that neither waits for the other.
template <int NT, bool FULL>
__device__ __forceinline__ void load_kv_rows(KBlock &kb, VBlock &vb, const uint16_t *K,
                                             const uint16_t *V, int64_t lo, int N, int kb0,
                                             int Hkv, int h, int tid) {
#pragma unroll
    for (int i = 0; i < 1024 / NT; ++i) {
        const int key = (tid >> 4) + (NT / 16) * i;
        kb.k[i] = ld_row(K, (lo + kb0 + key) * Hkv + h, FULL || kb0 + key < N, tid & 15);
    }
    const int m = tid & 31;
#pragma unroll
    for (int i = 0; i < 512 / NT; ++i) {
        const int d8 = (tid >> 5) + (NT / 32) * i;
        vb.v[2 * i] = ld_row(V, (lo + kb0 + 2 * m) * Hkv + h, FULL || kb0 + 2 * m < N, d8);
        vb.v[2 * i + 1] =
            ld_row(V, (lo + kb0 + 2 * m + 1) * Hkv + h, FULL || kb0 + 2 * m + 1 < N, d8);
    }
}
template <int NT>
__device__ __forceinline__ void load_kv(KBlock &kb, VBlock &vb, const uint16_t *K,
                                        const uint16_t *V, int64_t lo, int N, int kb0, int Hkv,
                                        int h, int tid) {
    if (kb0 + BN <= N)
        load_kv_rows<NT, true>(kb, vb, K, V, lo, N, kb0, Hkv, h, tid);
    else
        load_kv_rows<NT, false>(kb, vb, K, V, lo, N, kb0, Hkv, h, tid);
}
template <int NT>
__device__ __forceinline__ void store_k(const KBlock &kb, _Float16 *s_k, int tid) {
#pragma unroll
    for (int i = 0; i < 1024 / NT; ++i)
        *reinterpret_cast<uint4 *>(s_k + ((tid >> 4) + (NT / 16) * i) * KS + 8 * (tid & 15)) =
            kb.k[i];
}
// position of key k (within the 64-key block) in a transposed value row: the lane (c, g) of
// operand u reads keys 32u + 4g + e and 32u + 16 + 4g + e (e < 4) as positions 32u + 8g .. + 7
__device__ __forceinline__ int vt_pos(int k) {
    return (k & ~31) + 8 * ((k & 15) >> 2) + 4 * ((k >> 4) & 1) + (k & 3);
}
template <int NT>
__device__ __forceinline__ void store_v(const VBlock &vb, _Float16 *s_vt, int tid) {
    const int m = tid & 31;
    const int pm = vt_pos(2 * m);            // keys 2m, 2m + 1 stay adjacent
#pragma unroll
    for (int i = 0; i < 512 / NT; ++i) {
        const int d8 = (tid >> 5) + (NT / 32) * i;
        const uint32_t a[4] = {vb.v[2 * i].x, vb.v[2 * i].y, vb.v[2 * i].z, vb.v[2 * i].w};
        const uint32_t b[4] = {vb.v[2 * i + 1].x, vb.v[2 * i + 1].y, vb.v[2 * i + 1].z,
                               vb.v[2 * i + 1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // half e of row 2m in the low 16 bits, of row 2m + 1 in the high 16 (byte select)
            const uint32_t w = __builtin_amdgcn_perm(b[e >> 1], a[e >> 1],
                                                     (e & 1) ? 0x07060302u : 0x05040100u);
            *reinterpret_cast<uint32_t *>(s_vt + (8 * d8 + e) * VS + pm) = w;
        }
    }
}

// query operands of 32 queries (two column tiles) starting at q0: lane (c, g) holds query
// q0 + 16 qt + c, dims 32 ks + 8 g .. + 7
__device__ __forceinline__ void load_q(h8 (&qop)[2][4], const uint16_t *Q, int64_t lo, int N,
                                       int q0, int Hq, int hq, int lane) {
    const int c = lane & 15, g = lane >> 4;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int qi = q0 + 16 * qt + c;
        const bool ok = qi < N;
        const uint16_t *row = Q + ((lo + qi) * Hq + hq) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint4 u = ok ? *reinterpret_cast<const uint4 *>(row + 32 * ks)
                               : make_uint4(0, 0, 0, 0);
            qop[qt][ks] = __builtin_bit_cast(h8, u);
        }
    }
}

// S^T tiles of 64 keys x 32 queries: s[kt][qt], lane (c, g) holds query 16 qt + c, keys
// 16 kt + 4 g + r.  Key operands from LDS rows (16 kt + c), dims 32 ks + 8 g.
__device__ __forceinline__ void scores(f4 (&s)[4][2], const _Float16 *s_k,
                                       const h8 (&qop)[2][4], int lane) {
    const int c = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) s[kt][qt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const h8 a = *reinterpret_cast<const h8 *>(s_k + (16 * kt + c) * KS + 32 * ks + 8 * g);
            s[kt][0] = mfma(a, qop[0][ks], s[kt][0]);
            s[kt][1] = mfma(a, qop[1][ks], s[kt][1]);
        }
}

// flat grid xcd_grid(B * Hkv, nqb * G), 64 NW threads; group = (request, KV head), its
// workgroups (query block, query head of the group) in the order: query blocks last-first
// (the longest key ranges start first), the G query heads of a block together.  Wave w takes
// queries q0 + 32 w .. + 31 of the workgroup's block.
template <int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void prefill_fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ cu, int Hq, int Hkv,
    int max_seqlen, int B, float scale_log2, void *__restrict__ out, int out_fp32,
    float *__restrict__ ml, int32_t *status) {
    __shared__ __attribute__((aligned(16))) _Float16 s_k[2][BN * KS];
    __shared__ __attribute__((aligned(16))) _Float16 s_vt[2][D * VS];
    constexpr int NT = 64 * NW, BQ = 32 * NW;
    const int G = Hq / Hkv;
    const int nqb = (max_seqlen + BQ - 1) / BQ;
    int r;
    const int grp = xcd_group(blockIdx.x, nqb * G, B * Hkv, r);
    if (grp < 0) return;
    const int b = grp / Hkv, h = grp - b * Hkv;
    const int hq = h * G + r % G;
    const int64_t lo = cu[b];
    const int N = cu[b + 1] - cu[b];
    if (N > max_seqlen) {
        if (status && r == 0 && threadIdx.x == 0) atomicOr(status, KVC_DEV_SEQLEN);
        return;
    }
    const int q0 = (nqb - 1 - r / G) * BQ;
    if (q0 >= N) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int qw = q0 + 32 * wave;                   // the wave's first query
    const int nblk = (min(q0 + BQ, N) - 1) / BN + 1; // key blocks 0 .. nblk-1

    h8 qop[2][4];
    load_q(qop, Q, lo, N, qw, Hq, hq, lane);
    KBlock kb;
    VBlock vb;
    load_kv<NT>(kb, vb, K, V, lo, N, 0, Hkv, h, tid);
    store_k<NT>(kb, s_k[0], tid);
    store_v<NT>(vb, s_vt[0], tid);
    __syncthreads();

    f4 o[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt][0] = o[dt][1] = f4{0.f, 0.f, 0.f, 0.f};
    float m[2] = {M_INIT, M_INIT}, l[2] = {0.f, 0.f};

    // softmax of one block's S^T tiles into the P^T operands [qt][u], rescaling o, m, l when the
    // running max moves
    auto softmax_block = [&](const f4 (&s)[4][2], int kb0, h8 (&pb)[2][2]) {
        const bool diag = kb0 + BN - 1 > qw;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            // raw scores; keys after the query (diagonal blocks only) become -inf.  The max
            // is taken before scaling (scale_log2 > 0 and rounding are monotone)
            float x[16];
            float mx = -__builtin_inff();
            if (diag) {
                // key kb0 + 16 kt + 4 g + r is after query qw + 16 qt + c when 16 kt + r > thr
                const int thr = qw + 16 * qt + c - kb0 - 4 * g;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = 16 * kt + r > thr ? -__builtin_inff() : s[kt][qt][r];
                        x[4 * kt + r] = v;
                        mx = fmaxf(mx, v);
                    }
            } else {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        x[4 * kt + r] = s[kt][qt][r];
                        mx = fmaxf(mx, s[kt][qt][r]);
                    }
            }
            mx = fmaxf(max_col(mx) * scale_log2, M_INIT);
            if (__ballot(mx > m[qt] + MARGIN) != 0ull) {
                const float mn = fmaxf(m[qt], mx);
                const float corr = __builtin_amdgcn_exp2f(m[qt] - mn);
                m[qt] = mn;
                l[qt] *= corr;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[dt][qt] *= corr;
            }
            float pe[16];
            _Float16 p[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], scale_log2, -m[qt]));
                p[e] = _Float16(pe[e]);
            }
            float ls = pe[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) ls += pe[e];
            l[qt] += ls;
            // P^T operand u: keys 32u + 4g + e (e < 4) from tile 2u, 32u + 16 + 4g + e - 4
            // from tile 2u + 1
#pragma unroll
            for (int u = 0; u < 2; ++u)
                pb[qt][u] = h8{p[8 * u], p[8 * u + 1], p[8 * u + 2], p[8 * u + 3],
                               p[8 * u + 4], p[8 * u + 5], p[8 * u + 6], p[8 * u + 7]};
        }
    };
    // O^T += V^T P^T; V^T operand: dim row 16 dt + c, keys in the same order as P^T's k
    // (32u + 4g + e, then 32u + 16 + 4g + e), stored contiguously by vt_pos
    auto pv_block = [&](const h8 (&pb)[2][2], const _Float16 *vt) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const _Float16 *vrow = vt + (16 * dt + c) * VS + 8 * g;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const h8 a = *reinterpret_cast<const h8 *>(vrow + 32 * u);
                o[dt][0] = mfma(a, pb[0][u], o[dt][0]);
                o[dt][1] = mfma(a, pb[1][u], o[dt][1]);
            }
        }
    };

    for (int j = 0; j < nblk; ++j) {
        const int cur = j & 1;
        const int kb0 = j * BN;
        const bool more = j + 1 < nblk;
        bool issued = false;
        if (kb0 <= qw + 31) {                        // else every key is after the wave's queries
            f4 s[4][2];
            scores(s, s_k[cur], qop, lane);
            h8 pb[2][2];                             // P^T operands [qt][u]
            softmax_block(s, kb0, pb);
            // the next block's rows are requested now (the score registers are free) and land
            // while the PV products run
            if (more) {
                load_kv<NT>(kb, vb, K, V, lo, N, kb0 + BN, Hkv, h, tid);
                issued = true;
            }
            pv_block(pb, s_vt[cur]);
        }
        if (more) {
            if (!issued) {
                load_kv<NT>(kb, vb, K, V, lo, N, kb0 + BN, Hkv, h, tid);
            }
            store_k<NT>(kb, s_k[cur ^ 1], tid);
            store_v<NT>(vb, s_vt[cur ^ 1], tid);
        }
        __syncthreads();
    }

#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        float lt = l[qt];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        const int qi = qw + 16 * qt + c;
        if (qi >= N) continue;
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        const int64_t row = (lo + qi) * Hq + hq;
        if (g == 0) *reinterpret_cast<float2 *>(ml + 2 * row) = make_float2(m[qt], lt);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const int d0 = 16 * dt + 4 * g;
            const f4 v = o[dt][qt] * inv;
            if (out_fp32) {
                *reinterpret_cast<float4 *>(static_cast<float *>(out) + row * D + d0) =
                    make_float4(v[0], v[1], v[2], v[3]);
            } else {
                const uint32_t w0 = uint32_t(f2h_rn(v[0])) | (uint32_t(f2h_rn(v[1])) << 16);
                const uint32_t w1 = uint32_t(f2h_rn(v[2])) | (uint32_t(f2h_rn(v[3])) << 16);
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + row * D + d0) =
                    make_uint2(w0, w1);
            }
        }
    }
}

// flat grid xcd_grid(B * Hq, nkb), 256 threads; group = (request, query head), its workgroups
// the key blocks.  Wave w owns keys kb0 + 64 w .. + 63, their operands in registers; all four
// waves walk the same 32-query tiles, each tile's rows and statistics staged once in LDS
// (double-buffered) for the four waves.  The walk runs from the request's last tile back to
// kb0, so the group's workgroups on one XCD read the same query tiles at about the same time.
constexpr int CK = 4 * BN;       // keys per column-sum workgroup
constexpr int QT = 32;           // queries per staged tile
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_colsum_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const int32_t *__restrict__ cu,
    int Hq, int Hkv, int max_seqlen, int B, float scale_log2, const float *__restrict__ ml,
    float *__restrict__ acc) {
    __shared__ __attribute__((aligned(16))) _Float16 s_q[2][QT * KS];
    __shared__ float s_m[2][QT];
    const int nkb = (max_seqlen + CK - 1) / CK;
    int r;
    const int grp = xcd_group(blockIdx.x, nkb, B * Hq, r);
    if (grp < 0) return;
    const int b = grp / Hq, hq = grp - b * Hq;
    const int64_t lo = cu[b];
    const int N = cu[b + 1] - cu[b];
    if (N > max_seqlen) return;
    const int kb0 = r * CK;
    if (kb0 >= N) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int h = hq / (Hq / Hkv);
    const int kw = kb0 + BN * wave;                  // the wave's first key
    // key operands [kt][ks]: row 16 kt + c of the wave's keys, dims 32 ks + 8 g
    h8 ka[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        const int ki = kw + 16 * kt + c;
        const uint16_t *row = K + ((lo + ki) * Hkv + h) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            ka[kt][ks] = __builtin_bit_cast(
                h8, ki < N ? *reinterpret_cast<const uint4 *>(row + 32 * ks) : make_uint4(0, 0, 0, 0));
    }
    float cs[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) cs[kt][r] = 0.f;
    // staging: thread t loads query row t / 8 of the tile, 32 bytes at column 16 (t % 8); lanes
    // 0..31 of wave 0 also load the rows' (max, sum), stored as m + log2(sum) (+inf past the end)
    // (only the last tile, staged first, can run past the end: `full` skips the row tests)
    // per-thread row addresses at query 0; a tile adds q0 rows (uniform) to them
    const uint16_t *qbase = Q + ((lo + (tid >> 3)) * Hq + hq) * D + 16 * (tid & 7);
    const float *mlbase = ml + 2 * ((lo + tid) * Hq + hq);
    const int64_t qstep = int64_t(Hq) * D;
    auto load_tile = [&](uint4 (&u)[2], float &mq, int q0, bool full) {
        const int qi = q0 + (tid >> 3);
        const uint16_t *row = qbase + q0 * qstep;
        const bool ok = full || qi < N;
        u[0] = ok ? *reinterpret_cast<const uint4 *>(row) : make_uint4(0, 0, 0, 0);
        u[1] = ok ? *reinterpret_cast<const uint4 *>(row + 8) : make_uint4(0, 0, 0, 0);
        mq = __builtin_inff();
        if (tid < QT && (full || q0 + tid < N)) {
            const float2 x = *reinterpret_cast<const float2 *>(mlbase + 2 * int64_t(q0) * Hq);
            mq = x.y > 0.f ? x.x + __builtin_amdgcn_logf(x.y) : __builtin_inff();
        }
    };
    auto store_tile = [&](const uint4 (&u)[2], float mq, int buf) {
        _Float16 *dst = s_q[buf] + (tid >> 3) * KS + 16 * (tid & 7);
        reinterpret_cast<uint4 *>(dst)[0] = u[0];
        reinterpret_cast<uint4 *>(dst)[1] = u[1];
        if (tid < QT) s_m[buf][tid] = mq;
    };
    uint4 u[2];
    float mq;
    const int ntile = (N - kb0 + QT - 1) / QT;
    load_tile(u, mq, kb0 + QT * (ntile - 1), false);
    store_tile(u, mq, 0);
    __syncthreads();
    for (int it = 0; it < ntile; ++it) {
        const int buf = it & 1;
        const int q0 = kb0 + QT * (ntile - 1 - it);  // last tile first
        const bool more = it + 1 < ntile;
        if (more) load_tile(u, mq, q0 - QT, true);
        // queries q0 .. q0 + 31 against the wave's keys: nothing if every query precedes or
        // is the first key; masks only where the ranges overlap
        if (q0 + QT - 1 > kw) {
            const _Float16 *sq = s_q[buf];
            f4 sc[4][2];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) sc[kt][0] = sc[kt][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const h8 b0 = *reinterpret_cast<const h8 *>(sq + c * KS + 32 * ks + 8 * g);
                const h8 b1 = *reinterpret_cast<const h8 *>(sq + (16 + c) * KS + 32 * ks + 8 * g);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    sc[kt][0] = mfma(ka[kt][ks], b0, sc[kt][0]);
                    sc[kt][1] = mfma(ka[kt][ks], b1, sc[kt][1]);
                }
            }
            const bool diag = q0 <= kw + BN - 1;
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const float m = s_m[buf][16 * qt + c];
                if (diag) {
                    // query q0 + 16 qt + c is after key kw + 16 kt + 4 g + r when 16 kt + r < thr
                    const int thr = q0 + 16 * qt + c - kw - 4 * g;
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float p = __builtin_amdgcn_exp2f(
                                __builtin_fmaf(sc[kt][qt][r], scale_log2, -m));
                            cs[kt][r] += 16 * kt + r < thr ? p : 0.f;
                        }
                } else {
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            cs[kt][r] += __builtin_amdgcn_exp2f(
                                __builtin_fmaf(sc[kt][qt][r], scale_log2, -m));
                }
            }
        }
        if (more) store_tile(u, mq, buf ^ 1);
        __syncthreads();
    }
    // sum over the 16 query columns of each lane group; lane c == 0 of group g holds keys
    // 16 kt + 4 g + r of the wave
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float x = cs[kt][r];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, 64);
            const int ki = kw + 16 * kt + 4 * g + r;
            if (c == 0 && ki < N) acc[(lo + ki) * Hq + hq] = x;
        }
}

}  // namespace pf
}  // namespace kvc

using namespace kvc;

extern "C" int kvc_prefill_attention(const kvc_geom *g, const uint16_t *q, const uint16_t *k,
                                     const uint16_t *v, const int32_t *cu_seqlens,
                                     int32_t max_seqlen, float softmax_scale, void *out,
                                     int32_t out_is_fp32, float *acc_sum, int32_t *dev_status,
                                     void *ws, size_t ws_bytes, kvc_stream_t stream) {
    if (!g) return KVC_E_NULL;
    if (g->batch <= 0 || g->num_q_heads <= 0 || g->num_kv_heads <= 0 ||
        g->num_q_heads % g->num_kv_heads)
        return KVC_E_SHAPE;
    if (!q || !k || !v || !cu_seqlens || !out) return KVC_E_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return KVC_E_ALIGN;
    if (max_seqlen < 0) return KVC_E_SHAPE;
    PrefillWs L(g, max_seqlen);
    if (!ws || ws_bytes < L.bytes) return KVC_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return KVC_E_ALIGN;
    if (max_seqlen == 0) return KVC_OK;
    float *ml = reinterpret_cast<float *>(static_cast<char *>(ws) + L.ml);
    hipStream_t s = (hipStream_t)stream;
    const int Hq = g->num_q_heads, Hkv = g->num_kv_heads, B = g->batch;
    const float sl2 = softmax_scale * pf::LOG2E;
    constexpr int NW = KVC_PF_WAVES;
    const int nqb = (max_seqlen + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL(pf::prefill_fwd_kernel<NW>, dim3(pf::xcd_grid(B * Hkv, nqb * (Hq / Hkv))),
                       dim3(64 * NW), 0, s, q, k, v, cu_seqlens, Hq, Hkv, max_seqlen, B, sl2, out,
                       out_is_fp32, ml, dev_status);
    int rc = launch_check("kvc_prefill_attention/forward");
    if (rc || !acc_sum) return rc;
    const int nkb = (max_seqlen + pf::CK - 1) / pf::CK;
    hipLaunchKernelGGL(pf::prefill_colsum_kernel, dim3(pf::xcd_grid(B * Hq, nkb)), dim3(256), 0,
                       s, q, k, cu_seqlens, Hq, Hkv, max_seqlen, B, sl2, ml, acc_sum);
    return launch_check("kvc_prefill_attention/column sums");
}
