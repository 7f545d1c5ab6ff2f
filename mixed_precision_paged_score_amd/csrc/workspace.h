// Workspace layouts of the libkvc calls.  Each call carves its caller-provided workspace
// into the arrays below (offsets 256-byte aligned); kvc_workspace_bytes() reports the size.
#pragma once

#include "kvc_internal.h"

namespace kvc {

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- compact_pages -------------------------------------------------------------------
constexpr int SCAN_TILE = 256;    // heads per scan workgroup (one per thread)

struct CompactHdr {
    uint32_t ticket;       // dynamic tile index counter (tiles start in ticket order)
    uint32_t err;          // KVC_DEV_* bits found by the scan (row overflow, shrink)
    int64_t total_alloc;   // pages handed out by the whole call
    int64_t total_free;    // pages returned by the whole call
    uint64_t head0, tail0; // ring counters when the call started
    int32_t entry_status;  // pool status when the call started
};

struct CompactWs {
    int nheads, ntiles;
    size_t hdr, st, off, foff, bytes;
    explicit CompactWs(const kvc_geom *g) {
        nheads = g->batch * g->num_kv_heads;
        ntiles = (nheads + SCAN_TILE - 1) / SCAN_TILE;
        hdr = 0;
        st = align256(sizeof(CompactHdr));
        off = st + align256(sizeof(uint64_t) * ntiles);
        foff = off + align256(sizeof(int32_t) * nheads);
        bytes = foff + align256(sizeof(int32_t) * nheads);
    }
};

// ---- append_tokens ----------------------------------------------------------------------
struct AppendWs {
    size_t compact, new_count, changed, bytes;
    explicit AppendWs(const kvc_geom *g) {
        const size_t heads = size_t(g->batch) * g->num_kv_heads;
        compact = 0;
        new_count = CompactWs(g).bytes;
        changed = new_count + align256(sizeof(int32_t) * 2 * heads);
        bytes = changed + align256(heads);
    }
};

// ---- generation_step ---------------------------------------------------------------------
constexpr int GEN_MAX_WINDOW = KVC_GEN_MAX_WINDOW;

struct GenWs {
    size_t compact, new_count, old_count, changed, decided, bytes;
    explicit GenWs(const kvc_geom *g) {
        const size_t heads = size_t(g->batch) * g->num_kv_heads;
        compact = 0;
        new_count = CompactWs(g).bytes;
        old_count = new_count + align256(sizeof(int32_t) * 2 * heads);
        changed = old_count + align256(sizeof(int32_t) * 2 * heads);
        decided = changed + align256(heads);
        bytes = decided + align256(heads);
    }
};

// ---- prefill_attention -------------------------------------------------------------------
struct PrefillWs {
    size_t ml, bytes;
    PrefillWs(const kvc_geom *g, int max_seqlen) {
        ml = 0;            // float [T][Hq][2]: each query row's softmax max (log2) and sum
        bytes = align256(sizeof(float) * 2 * size_t(g->batch) * size_t(max_seqlen > 0 ? max_seqlen : 1) *
                         size_t(g->num_q_heads));
    }
};

// ---- quantize_and_place ----------------------------------------------------------------
constexpr int QTILE = 256;        // tokens per rank tile (and per score tile of a fused round)

struct QuantWs {
    int ntq;
    size_t tile_cnt, tile_base, tile_cnt2, tile_base2, ok, poslist, srcdesc, bytes;
    QuantWs(const kvc_geom *g, int max_seqlen) {
        ntq = (max_seqlen + QTILE - 1) / QTILE;
        if (ntq < 1) ntq = 1;
        const size_t cnt = align256(sizeof(int32_t) * size_t(g->batch) * ntq * g->num_kv_heads * 2);
        const size_t heads = size_t(g->batch) * g->num_kv_heads;
        const size_t pl = align256(sizeof(int32_t) * heads * size_t(max_seqlen > 0 ? max_seqlen : 1));
        tile_cnt = 0;                       // per tile (HIGH, LOW) counts of the new tiers
        tile_base = tile_cnt + cnt;         // their exclusive prefix over tiles
        tile_cnt2 = tile_base + cnt;        // the same for the previous tiers (re-tiering)
        tile_base2 = tile_cnt2 + cnt;
        ok = tile_base2 + cnt;              // per head: write its pages; [heads] = entry status
        poslist = ok + align256(sizeof(int32_t) * (heads + 1));
        // re-tiering: per head and new slot index (as poslist) where the token's codes come
        // from, {old page id, previous tier << 8 | slot in the old page}
        srcdesc = poslist + pl;
        bytes = srcdesc + 2 * pl;
    }
};

// ---- the fused compaction round (kvc_compaction_round) -----------------------------------
constexpr int ROUND_MAX_HEADS = 1024;    // the planning workgroup's heads: 4 per thread
struct RoundWs {
    size_t quant, compact, tile_chg, old_rows, old_count, bytes;
    RoundWs(const kvc_geom *g, int max_seqlen) {
        const QuantWs Q(g, max_seqlen);
        const size_t heads = size_t(g->batch) * g->num_kv_heads;
        quant = 0;                        // the QuantWs layout: tile counts, bases, ok, lists
        compact = Q.bytes;                // the CompactWs layout: header, offsets
        tile_chg = compact + CompactWs(g).bytes;     // per tile and head: a tier dropped
        old_rows = tile_chg + align256(size_t(g->batch) * Q.ntq * g->num_kv_heads);
        old_count = old_rows + align256(sizeof(int32_t) * heads * size_t(g->row_capacity));
        bytes = old_count + align256(sizeof(int32_t) * 2 * heads);
    }
};

// ---- paged_decode_attention ------------------------------------------------------------
constexpr int PART_STRIDE = 132;  // floats per partial: m, l, pad, pad, o[128]

#ifndef KVC_DEC_SPLIT_TARGET
#define KVC_DEC_SPLIT_TARGET 2048      // workgroups per decode launch to aim for
#endif
#ifndef KVC_DEC_SLOTS_MAX
#define KVC_DEC_SLOTS_MAX 8192         // workgroup slots per decode launch at most
#endif
#ifndef KVC_DEC_WT_MIN
#define KVC_DEC_WT_MIN 128             // work units per workgroup at least (about 50 tiles)
#endif
#ifndef KVC_DEC_WT_MAX
#define KVC_DEC_WT_MAX 256             // work units per workgroup at most (about 100 tiles)
#endif
#ifndef KVC_DEC_UH
#define KVC_DEC_UH 3
#endif
#ifndef KVC_DEC_UL
#define KVC_DEC_UL 2
#endif
constexpr int DEC_UH = KVC_DEC_UH, DEC_UL = KVC_DEC_UL;   // work units of a HIGH / LOW tile

// Split-K plan of the decode.  The grid has `splits` workgroup slots per head; head h uses
// active_splits() = min(splits, ceil(W_h / wt)) of them, W_h its work units (HIGH tiles weigh
// DEC_UH, LOW half-page tiles DEC_UL), so that a long head gets more workgroups than a short
// one and every workgroup about wt units; the other slots exit at once.  The slot count is
// the batch's share of the workgroup target, at least 16 and at most 64 (16 and 32 are
// multiples of the 8 XCDs, which the kernels' slot order relies on), and no more than the
// largest possible head needs (its tiles are at most the row capacity C + 1), nor more than
// KVC_DEC_SLOTS_MAX over all heads (a batch of more than 512 heads gets fewer than 16); wt
// spreads that largest head over the slots, within [KVC_DEC_WT_MIN, KVC_DEC_WT_MAX] units per
// workgroup: below the minimum a batch of many short heads would be cut into tens of
// thousands of workgroups of a tile or two.
struct DecodePlan {
    int splits, wt;
};
inline DecodePlan decode_plan(const kvc_geom *g) {
    const int heads = g->batch * g->num_kv_heads;
    int s0 = (KVC_DEC_SPLIT_TARGET + heads - 1) / heads;
    if (s0 < 16) s0 = 16;
    if (s0 > 64) s0 = 64;
    const int64_t wmax = int64_t(DEC_UH) * (int64_t(g->row_capacity) + 1);
    int64_t wt = (wmax + s0 - 1) / s0;
    if (wt > KVC_DEC_WT_MAX) wt = KVC_DEC_WT_MAX;
    if (wt < KVC_DEC_WT_MIN) wt = KVC_DEC_WT_MIN;
    if (wt < 1) wt = 1;
    int64_t splits = (wmax + wt - 1) / wt;
    if (splits > s0) splits = s0;
    // at most KVC_DEC_SLOTS_MAX slots per launch: a slot a head leaves unused still costs a
    // workgroup launch, which a batch of thousands of heads would pay tens of thousands of times
    const int64_t cap = KVC_DEC_SLOTS_MAX / heads;
    if (splits > cap) splits = cap;
    if (splits < 1) splits = 1;
    return {int(splits), int(wt)};
}
// the workgroups head (nh HIGH, nl LOW tokens) uses of its `splits` (at least one)
__host__ __device__ inline int active_splits(int nh, int nl, int splits, int wt) {
    const int64_t w = int64_t(DEC_UH) * ((nh + HS - 1) / HS) + int64_t(DEC_UL) * ((nl + 15) / 16);
    const int64_t a = (w + wt - 1) / wt;
    return int(a < 1 ? 1 : (a > splits ? splits : a));
}
// The split that workgroup slot `slot` of head i serves (>= SH: none).  Workgroups go to the
// XCDs round-robin, so with a slot count that is a multiple of 8 slot k of every head runs on
// XCD k mod 8.  A head that uses all its slots keeps that order (the fastest measured for
// batches of equal heads); a head that uses fewer turns its splits by its index, so that the
// workgroups of short heads spread over all the XCDs instead of crowding the first ones.
__device__ inline int split_of_slot(int slot, int i, int SH, int splits) {
    if (SH == splits) return slot;
    const int s = slot - i % splits;
    return s < 0 ? s + splits : s;
}

constexpr int ACC_R = 64;          // positions per score-accumulation chunk
constexpr int ACC_MAX_HQ = 512;    // query heads the accumulation's LDS rows hold

struct DecodeWs {
    int splits, wt;
    int64_t tiles_cap;     // tiles per head the logit buffer holds (HIGH pages + 2 x LOW pages)
    int nch_cap;           // chunk-start entries per head and tier: ceil(max_seqlen / R) + 1
    size_t part, mls, lg, idx, bytes;
    // acc: also the buffers of the score-accumulating variant (requests up to max_seqlen)
    DecodeWs(const kvc_geom *g, bool acc, int max_seqlen = 0) {
        const DecodePlan pl = decode_plan(g);
        splits = pl.splits;
        wt = pl.wt;
        tiles_cap = 2 * int64_t(g->row_capacity);
        part = 0;          // float [B][Hkv][S][G][PART_STRIDE]
        bytes = align256(sizeof(float) * PART_STRIDE * size_t(g->batch) * g->num_q_heads *
                         splits);
        mls = bytes;       // float [B][Hq][2]: the softmax's max and sum per query head
        lg = mls;          // per head and tile (the head's tile order): 16 int32 positions,
                           // then float logits [16][G]
        idx = mls;         // int32 [B*Hkv][2][nch_cap]: first slot of each position chunk
        nch_cap = (max_seqlen + ACC_R - 1) / ACC_R + 1;
        if (acc) {
            lg = mls + align256(sizeof(float) * 2 * size_t(g->batch) * g->num_q_heads);
            const size_t G = size_t(g->num_q_heads / g->num_kv_heads);
            idx = lg + align256(sizeof(float) * size_t(g->batch) * g->num_kv_heads *
                                size_t(tiles_cap) * 16 * (G + 1));
            bytes = idx + align256(sizeof(int32_t) * 2 * size_t(g->batch) * g->num_kv_heads *
                                   size_t(nch_cap));
        }
    }
};

}  // namespace kvc
