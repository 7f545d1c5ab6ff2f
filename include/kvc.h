/*
 * kvc.h -- C ABI of libkvc: differentiated KV compaction and mixed-precision paged decode
 * attention for AMD Instinct MI355X (gfx950).
 *
 * The method is DiffKV's (pith.science review of arXiv 2412.03131, "DiffKV: Differentiated
 * Memory Management for Large Language Models with Parallel KV Compaction"):
 *   - "What carries the argument": a token's significance is the mean attention it receives
 *     from subsequent tokens, max-aggregated over its GQA group, compared with alpha_h/N
 *     and alpha_l/N (high precision, low precision, pruned); after every head has decided
 *     how many high- and low-precision pages it needs, a parallel prefix sum over the
 *     circular free page list gives each head a disjoint contiguous region of page ids.
 *   - "Core claim": K8V4 high tier, K4V2 low tier, unified pages, a circular free page list
 *     and a bidirectional page table, all GPU-resident.
 *   - free-parameter ledger: the most recent W = 64 tokens are always high precision.
 *
 * Conventions for every call
 *   - Pointers are device pointers unless stated otherwise.  Every buffer is owned by the
 *     caller; the library allocates nothing, keeps no pointer after returning, and never
 *     synchronizes: all work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream).
 *   - A negative return value is a synchronous error: nothing was enqueued.
 *   - Errors found on the device are sticky bits OR-ed into pool->dev_status (and, for
 *     kvc_score_tokens, into its own dev_status argument).  Every kernel that changes pool
 *     state first reads dev_status and does nothing if any bit is set, so a failed call
 *     leaves the pool exactly as it was and turns the rest of the round into no-ops.  The
 *     caller reads the word after a stream synchronization and clears it.
 *   - Calls that share a pool must be ordered on one stream (or by the caller's events).
 *   - Query head hq reads KV head hq / G, G = num_q_heads / num_kv_heads.
 *   - Head dimension is fixed at 128.  K, V and q are IEEE fp16 bit patterns.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *kvc_stream_t; /* hipStream_t */

/* synchronous status codes */
enum {
    KVC_OK = 0,
    KVC_E_NULL = -1,        /* a required pointer is NULL                                   */
    KVC_E_ALIGN = -2,       /* K/V/q/pages/out not 16-byte aligned                          */
    KVC_E_SHAPE = -3,       /* inconsistent geometry or sizes (see each call)               */
    KVC_E_WORKSPACE = -4,   /* workspace NULL or smaller than kvc_workspace_bytes()         */
    KVC_E_HIP = -5,         /* a HIP launch failed; kvc_last_error() has the message        */
    KVC_E_UNSUPPORTED = -6  /* argument combination not implemented                         */
};

/* device-side status bits (OR-ed into *dev_status) */
enum {
    KVC_DEV_POOL_EXHAUSTED = 1, /* compaction needs more pages than are free                */
    KVC_DEV_ROW_OVERFLOW = 2,   /* a head would need more than row_capacity pages           */
    KVC_DEV_SHRINK = 4,         /* a head not marked changed would lose pages               */
    KVC_DEV_COUNT_MISMATCH = 8, /* tier array disagrees with the pool's per-head counts     */
    KVC_DEV_SEQLEN = 16,        /* a request is longer than the max_seqlen argument         */
    KVC_DEV_INTERNAL = 32,      /* a scan's look-back gave up waiting (a library bug)       */
    KVC_DEV_BAD_TIER = 64       /* re-tiering: a tier rose, or a fresh token had no fp16 row */
};

/* tier codes */
enum { KVC_PRUNE = 0, KVC_LOW = 1, KVC_HIGH = 2, KVC_FRESH = 3 };

/* unified page format (both tiers share one 3456-byte page):
 *   [   0, 2048)  key codes: HIGH 16 slots x 128 B (8-bit), LOW 32 slots x 64 B (4-bit)
 *   [2048, 3072)  value codes, 64 units of 16 B laid out for the decode kernel's matrix
 *                 operands: unit 16j + l (j < 4, l < 16) holds channels l, l+16, ..., l+112;
 *                 HIGH (4-bit): slot 4j + r, channel 16n + l in word n >> 1, nibble
 *                 2(n & 1) + (r >> 1) + 4(r & 1); LOW (2-bit): slot 16f + 4j + r in word
 *                 2f + (n >> 2), 2-bit field 2(n & 3) + (r >> 1) + 8(r & 1)
 *   key codes of a LOW slot: word w (little-endian) holds channels 8w..8w+7, channel
 *                 8w + e in nibble (e & 1) + 2(e >> 2) + 4((e >> 1) & 1)
 *   [3072, 3328)  per slot: key scale, key zero, value scale, value zero (fp16)
 *   [3328, 3456)  per slot: token position (int32), -1 for an empty slot            */
#define KVC_HEAD_DIM 128
#define KVC_HIGH_SLOTS 16
#define KVC_LOW_SLOTS 32
#define KVC_PAGE_BYTES 3456
#define KVC_GEN_MAX_WINDOW 112  /* largest recent window kvc_generation_step accepts      */

typedef struct {
    int32_t num_layers;   /* L: layers sharing the pool                                   */
    int32_t batch;        /* B: requests                                                  */
    int32_t num_q_heads;  /* Hq                                                           */
    int32_t num_kv_heads; /* Hkv (Hq % Hkv == 0)                                          */
    int32_t row_capacity; /* C: page-table slots per (layer, request, KV head)            */
    int64_t num_pages;    /* P: pages in the pool                                         */
} kvc_geom;

typedef struct {
    uint8_t *pages;      /* [P][3456]                                                      */
    int32_t *page_table; /* [L][B][Hkv][C]: HIGH page ids from position 0 upward, LOW page
                            ids from position C-1 downward, -1 elsewhere                    */
    int32_t *count;      /* [L][B][Hkv][2]: live (#HIGH, #LOW) tokens per head              */
    int32_t *owner;      /* [P]: reverse map, gid*C + row position with
                            gid = (layer*B + b)*Hkv + h; -1 for a free page                */
    int32_t *free_ring;  /* [P]: circular free list; free pages are
                            free_ring[(head + k) % P] for k < tail - head                  */
    uint64_t *ring_ctr;  /* [2]: head, tail (monotone counters)                            */
    int32_t *dev_status; /* [1]: sticky KVC_DEV_* bits                                     */
} kvc_pool;

/* Precision scheme of the two tiers (key and value bits: 1, 2, 4 or 8).  A tier's format must
 * fit its page: 16 slots * 16 (k + v) bytes <= 3072 for HIGH, 32 slots * 16 (k + v) <= 3072
 * for LOW; e.g. K8V4, K4V8, K8V2 for HIGH and K4V2, K2V4, K4V1 for LOW. */
typedef struct {
    int32_t k_bits_high, v_bits_high, k_bits_low, v_bits_low;
} kvc_scheme;

/* Operation ids for kvc_workspace_bytes */
enum { KVC_OP_COMPACT = 1, KVC_OP_QUANTIZE = 2, KVC_OP_DECODE = 3, KVC_OP_APPEND = 4,
       KVC_OP_DECODE_ACC = 5, KVC_OP_GENERATE = 6, KVC_OP_PREFILL = 7, KVC_OP_ROUND = 8 };

/* Version string of the library. */
const char *kvc_version(void);

/* Message of the last KVC_E_HIP failure in this thread ("" if none). */
const char *kvc_last_error(void);

/* Bytes of workspace `op` needs for this geometry.  max_seqlen is the longest request
 * (KVC_OP_QUANTIZE, KVC_OP_DECODE_ACC, KVC_OP_PREFILL, KVC_OP_ROUND), unused otherwise.
 * Returns 0 for an unknown op. */
size_t kvc_workspace_bytes(const kvc_geom *geom, int32_t op, int32_t max_seqlen);

/* Empty pool: free_ring = 0..P-1, head = 0, tail = P, page table and owner = -1,
 * counts = 0, dev_status = 0.  Page bytes are left as they are.
 * Errors: KVC_E_NULL, KVC_E_SHAPE (non-positive sizes, L*B*Hkv*C >= 2^31, P >= 2^31). */
int kvc_pool_init(const kvc_geom *geom, const kvc_pool *pool, kvc_stream_t stream);

/* Significance score and tier of every (token, KV head) of one layer (DiffKV review page,
 * "What carries the argument"; free-parameter ledger for W).
 *   acc_sum    float32 [T][Hq]: for each token, the sum of the softmax weight it received
 *              from strictly later queries of each query head (>= 0, finite)
 *   cu_seqlens int32 [B+1]: request b owns rows cu[b]..cu[b+1]-1, positions 0..N_b-1
 *   For token t of request b (N = N_b, cnt = N-1-t): score = +inf if cnt == 0, else
 *   max over the G query heads of fl32(acc/cnt); tier = HIGH if score >= fl32(alpha_h/N),
 *   LOW if score >= fl32(alpha_l/N), else PRUNE; HIGH when t >= N - window; with
 *   prev_tier (uint8 [T][Hkv], or NULL), tier = min(tier, prev) wherever prev != FRESH.
 *   Outputs: tier uint8 [T][Hkv]; new_count int32 [B][Hkv][2] = (#HIGH, #LOW);
 *   changed uint8 [B][Hkv] = 1 where some already-tiered token dropped a tier or a FRESH
 *   token was kept, i.e. where the head's pages must be rebuilt (may be NULL when prev_tier
 *   is NULL).  max_seqlen bounds every N_b (else KVC_DEV_SEQLEN is set in
 *   *dev_status and the request is skipped; dev_status may be NULL).
 * Errors: KVC_E_NULL, KVC_E_SHAPE (Hq % Hkv, window < 0, total_tokens < 0). */
int kvc_score_tokens(const kvc_geom *geom, const float *acc_sum, const int32_t *cu_seqlens,
                     int64_t total_tokens, int32_t max_seqlen, float alpha_h, float alpha_l,
                     int32_t window, const uint8_t *prev_tier, uint8_t *tier,
                     int32_t *new_count, uint8_t *changed, int32_t *dev_status,
                     kvc_stream_t stream);

/* Causal prefill attention of a batch of prompts, and the prompt's significance
 * accumulators (DiffKV review page: "Assumptions", standard causal multi-head attention;
 * "What carries the argument", a token's score is the mean of the attention it receives from
 * subsequent tokens, so the sums over strictly later queries are what kvc_score_tokens reads).
 * For request b (rows cu[b] .. cu[b+1]-1) and query head hq (KV head hq / G), query row i
 * attends to keys j <= i of its request: p_ij = softmax_j(softmax_scale * q_i . k_j);
 *   out[i][hq]    = sum_j p_ij v_j   (fp16 or float32 [T][Hq][128]);
 *   acc_sum[t][hq] = sum over i > t of p_it   (float32 [T][Hq], overwritten; NULL: skipped).
 * Scores and sums in float32 from fp16 inputs (matrix cores); the probabilities that weight V
 * are rounded to fp16.  Each accumulator is summed by one workgroup in a fixed order:
 * deterministic.
 *   q fp16 [T][Hq][128]; k, v fp16 [T][Hkv][128]; all 16-byte aligned, as is out
 *   max_seqlen  bounds every request length (a longer request is skipped and sets
 *               KVC_DEV_SEQLEN in *dev_status; dev_status may be NULL)
 *   workspace >= kvc_workspace_bytes(geom, KVC_OP_PREFILL, max_seqlen) bytes, 256-B aligned
 *               (each row's softmax max and sum); geom's batch, num_q_heads and num_kv_heads
 *               are used
 * Errors: KVC_E_NULL, KVC_E_ALIGN, KVC_E_SHAPE (Hq % Hkv, max_seqlen < 0), KVC_E_WORKSPACE. */
int kvc_prefill_attention(const kvc_geom *geom, const uint16_t *q, const uint16_t *k,
                          const uint16_t *v, const int32_t *cu_seqlens, int32_t max_seqlen,
                          float softmax_scale, void *out, int32_t out_is_fp32, float *acc_sum,
                          int32_t *dev_status, void *workspace, size_t workspace_bytes,
                          kvc_stream_t stream);

/* One allocation round for one layer: prefix sums over the B*Hkv heads (request-major) of
 * their page demand give each head a contiguous segment of the circular free list
 * (DiffKV review page, "What carries the argument").  Per head, pages needed are
 * ceil(n_high/16) HIGH and ceil(n_low/32) LOW.  With changed == NULL (prompt mode) or
 * changed[b][h] != 0 the head is rebuilt: it takes fresh pages for all its tokens and its
 * old pages are returned to the ring's tail (HIGH in row order, then LOW from the right
 * end); other heads grow in place.  Only pages free when the call starts are handed out,
 * so old pages stay readable until the next call.  All or nothing: on exhaustion, row
 * overflow or a shrink of a non-rebuilt head, a KVC_DEV_* bit is set and nothing changes.
 *   new_count      int32 [B][Hkv][2] (from kvc_score_tokens)
 *   old_rows_out   int32 [B][Hkv][C] or NULL: the layer's page table before the call
 *   old_count_out  int32 [B][Hkv][2] or NULL: the layer's counts before the call
 *   workspace      >= kvc_workspace_bytes(geom, KVC_OP_COMPACT, 0) bytes, 256-B aligned
 * Errors: KVC_E_NULL, KVC_E_SHAPE (layer out of range), KVC_E_WORKSPACE. */
int kvc_compact_pages(const kvc_geom *geom, int32_t layer, const kvc_pool *pool,
                      const int32_t *new_count, const uint8_t *changed,
                      int32_t *old_rows_out, int32_t *old_count_out, void *workspace,
                      size_t workspace_bytes, kvc_stream_t stream);

/* Quantize and place one layer's kept tokens into the pages compact_pages assigned.  HIGH
 * tokens are K8V4, LOW tokens K4V2 (DiffKV review page, "Core claim"): per token and head,
 * asymmetric min/max codes over the 128 channels, scale and zero computed in float32 with
 * round-to-nearest-even and stored as fp16.  Within a head and a tier, tokens take slots in
 * ascending position order; every page of a written head is written whole (empty slots
 * zeroed, position -1).
 *   k, v       fp16 [T][Hkv][128] (T = cu_seqlens[B]), 16-byte aligned
 *   tier       uint8 [T][Hkv] (from kvc_score_tokens)
 * Prompt mode (prev_tier, changed, old_rows, old_count all NULL): every head is written, all
 * tokens quantized from k, v.
 * Re-tier mode (all four given; after kvc_compact_pages with the same `changed`): only heads
 * with changed[b][h] != 0 are written.  A token whose tier is unchanged keeps its codes and
 * parameters bit for bit (copied from its old page, found through old_rows / old_count from
 * kvc_compact_pages); a HIGH token demoted to LOW is re-quantized from the fp16 rounding of its
 * K8V4 reconstruction (referee major comment 3: demotion is irreversible); a FRESH token is
 * quantized from k, v (which may be NULL when no token is FRESH).  A token whose tier rose,
 * or a FRESH one without k/v, is left zero and sets KVC_DEV_BAD_TIER.
 *   A head whose tier counts differ from the pool's counts is skipped and
 *   KVC_DEV_COUNT_MISMATCH is set.
 * Errors: KVC_E_NULL, KVC_E_ALIGN, KVC_E_SHAPE, KVC_E_WORKSPACE, KVC_E_UNSUPPORTED (only some
 * of the four re-tier arguments given). */
int kvc_quantize_and_place(const kvc_geom *geom, int32_t layer, const kvc_pool *pool,
                           const uint16_t *k, const uint16_t *v, const int32_t *cu_seqlens,
                           int64_t total_tokens, int32_t max_seqlen, const uint8_t *tier,
                           const uint8_t *prev_tier, const uint8_t *changed,
                           const int32_t *old_rows, const int32_t *old_count,
                           void *workspace, size_t workspace_bytes, kvc_stream_t stream);

/* One whole compaction round of a layer: kvc_score_tokens, kvc_compact_pages and
 * kvc_quantize_and_place in sequence (DiffKV review page, "What carries the argument": score,
 * per-head page demand, prefix-sum allocation over the circular free list, placement), with the
 * same results bit for bit, in four launches instead of nine: the score also counts each
 * 256-token tile's tiers per head (nothing to clear, no separate count launch), a per-head
 * launch turns the tile counts into the heads' totals and rank bases (and, re-tiering, keeps
 * each changed head's old row), one launch holds the commits, each commit workgroup making
 * the allocation scan for itself, beside the ranks, and the last writes the pages.  For
 * batches of at most 1024 KV heads
 * (KVC_E_SHAPE above: use the three calls).
 *   prev_tier NULL: prompt mode (every head rebuilt, the layer's previous pages returned first;
 *     k, v required, changed may be NULL); else re-tier mode (changed required; k, v only for
 *     FRESH tokens; the old rows and counts are kept in the workspace).
 *   Inputs and outputs as in the three calls: acc_sum fp32 [T][Hq] (16-byte aligned), tier u8
 *   [T][Hkv], new_count i32 [B][Hkv][2], changed u8 [B][Hkv]; device failures are the same
 *   status bits in pool->dev_status, the score's included (a request longer than max_seqlen:
 *   KVC_DEV_SEQLEN, as kvc_score_tokens given the pool's status), and a round that does not
 *   commit changes nothing.
 *   workspace >= kvc_workspace_bytes(geom, KVC_OP_ROUND, max_seqlen) bytes, 256-B aligned
 * Errors: the union of the three calls' errors. */
int kvc_compaction_round(const kvc_geom *geom, int32_t layer, const kvc_pool *pool,
                         const float *acc_sum, const int32_t *cu_seqlens, int64_t total_tokens,
                         int32_t max_seqlen, float alpha_h, float alpha_l, int32_t window,
                         const uint16_t *k, const uint16_t *v, const uint8_t *prev_tier,
                         uint8_t *tier, int32_t *new_count, uint8_t *changed, void *workspace,
                         size_t workspace_bytes, kvc_stream_t stream);

/* Placement under a precision scheme (DiffKV review page: the free-parameter ledger's
 * comparison of K8V4, K4V8, K8V2, K4V2, K2V4 and K4V1; referee minor comment 5 for the
 * K8V4-K4V2 / K8V4-Prune configurations).  Same contract as kvc_quantize_and_place, in prompt
 * mode and in re-tier mode (same ranks, pages and slots; the K8V4-Prune and no-prune
 * configurations are threshold settings of kvc_score_tokens), but each tier is quantized at
 * the scheme's bit widths with the same per-token min/max quantizer (2^b - 1 levels) and
 * written in the layout below.  In re-tier mode the layer's pages must hold this scheme's
 * layout: a token whose tier is unchanged keeps its codes and parameters bit for bit, a HIGH
 * token demoted to LOW is re-quantized at the LOW widths from the fp16 rounding of its HIGH
 * reconstruction (referee major comment 3), a FRESH one is quantized from k, v.  Layout (bits
 * counted little-endian from a field's first byte; S = 16 slots for HIGH, 32 for LOW):
 *   keys, slot-major: slot s's 128 codes at bytes [16 kb s, 16 kb (s + 1)), code i at bits
 *     [i kb, (i + 1) kb);
 *   values from byte 16 kb S in blocks of 16 slots (S / 16 of them), 256 vb bytes each, in the
 *     decode's operand order: bytes [4 vb L, 4 vb (L + 1)) of block f, L = 16 g + c (g < 4,
 *     c < 16), hold the codes of channels 16 n + c (n < 8) for slots 16 f + 4 g + r (r < 4),
 *     code (n, r) at bit 32 (n / p) + 16 (r % 2) + vb (2 (n % p) + r / 2), p = 8 / vb;
 *   the bytes after the values up to 3072 are zero; parameters and positions as in the
 *   default layout.
 * Pages written this way are read by kvc_paged_decode_attention_scheme only.
 *   workspace >= kvc_workspace_bytes(geom, KVC_OP_QUANTIZE, max_seqlen)
 * Errors: as kvc_quantize_and_place, and KVC_E_SHAPE for a scheme that does not fit. */
int kvc_quantize_and_place_scheme(const kvc_geom *geom, const kvc_scheme *scheme, int32_t layer,
                                  const kvc_pool *pool, const uint16_t *k, const uint16_t *v,
                                  const int32_t *cu_seqlens, int64_t total_tokens,
                                  int32_t max_seqlen, const uint8_t *tier,
                                  const uint8_t *prev_tier, const uint8_t *changed,
                                  const int32_t *old_rows, const int32_t *old_count,
                                  void *workspace, size_t workspace_bytes, kvc_stream_t stream);

/* Decode attention over pages written by kvc_quantize_and_place_scheme with the same scheme:
 * the contract of kvc_paged_decode_attention (codes reconstructed as code * scale + zero, all
 * live tokens, a head with none yields zeros), G <= 16.
 *   workspace >= kvc_workspace_bytes(geom, KVC_OP_DECODE, 0)
 * Errors: as kvc_paged_decode_attention, and KVC_E_SHAPE for a scheme that does not fit or
 * G > 16. */
int kvc_paged_decode_attention_scheme(const kvc_geom *geom, const kvc_scheme *scheme,
                                      int32_t layer, const kvc_pool *pool, const uint16_t *q,
                                      float softmax_scale, void *out, int32_t out_is_fp32,
                                      void *workspace, size_t workspace_bytes,
                                      kvc_stream_t stream);

/* kvc_paged_decode_attention_acc over pages written in a precision scheme's layout (with the
 * same scheme): the scheme decode's output, and every live token's softmax weight per query
 * head added into acc_sum (the contract, workspace and errors of
 * kvc_paged_decode_attention_acc), for groups of up to 8 query heads per KV head
 * (KVC_E_UNSUPPORTED above). */
int kvc_paged_decode_attention_scheme_acc(const kvc_geom *geom, const kvc_scheme *scheme,
                                          int32_t layer, const kvc_pool *pool,
                                          const uint16_t *q, float softmax_scale, void *out,
                                          int32_t out_is_fp32, float *acc_sum,
                                          const int32_t *cu_seqlens, int32_t max_seqlen,
                                          void *workspace, size_t workspace_bytes,
                                          kvc_stream_t stream);

/* Append one freshly generated token per (request, KV head) to layer `layer` during
 * decoding: the token enters its head's HIGH tier (DiffKV review page, free-parameter ledger:
 * the recent window is always high precision) as K8V4 codes in the next HIGH slot; a head
 * whose last HIGH page is full first receives one page from the circular free list in an
 * allocation round like kvc_compact_pages (no head is rebuilt).  The slot's position field
 * is positions[b].  On pool exhaustion or row overflow the round sets its status bit and no
 * token is written.
 *   k_new, v_new  fp16 [B][Hkv][128], 16-byte aligned;  positions int32 [B]
 *   workspace >= kvc_workspace_bytes(geom, KVC_OP_APPEND, 0) bytes, 256-B aligned
 * Errors: KVC_E_NULL, KVC_E_ALIGN, KVC_E_SHAPE, KVC_E_WORKSPACE. */
int kvc_append_tokens(const kvc_geom *geom, int32_t layer, const kvc_pool *pool,
                      const uint16_t *k_new, const uint16_t *v_new, const int32_t *positions,
                      void *workspace, size_t workspace_bytes, kvc_stream_t stream);

/* kvc_append_tokens for a layer whose pages hold a precision scheme's layout (written by
 * kvc_quantize_and_place_scheme with the same scheme): the new token's codes are quantized at
 * the scheme's HIGH widths and set into its slot (keys slot-major, values into the slot's
 * value words, the other slots' codes kept).  Same allocation, workspace and errors, and
 * KVC_E_SHAPE for a scheme that does not fit. */
int kvc_append_tokens_scheme(const kvc_geom *geom, const kvc_scheme *scheme, int32_t layer,
                             const kvc_pool *pool, const uint16_t *k_new, const uint16_t *v_new,
                             const int32_t *positions, void *workspace, size_t workspace_bytes,
                             kvc_stream_t stream);

/* Decode attention of one new query per request over its KV head's live tokens (HIGH
 * slots < n_high, LOW slots < n_low), keys and values reconstructed on the fly as
 * code*scale + zero: o = softmax(softmax_scale * q.k) v.  No mask (every cached token
 * precedes the query).  A head with no live token yields zeros.
 *   q    fp16 [B][Hq][128];  out  [B][Hq][128], float32 if out_is_fp32 else fp16
 *   workspace >= kvc_workspace_bytes(geom, KVC_OP_DECODE, 0) bytes, 256-B aligned (split
 *        partials); calls that share a decode workspace must not overlap.
 * Errors: KVC_E_NULL, KVC_E_ALIGN, KVC_E_SHAPE, KVC_E_WORKSPACE. */
int kvc_paged_decode_attention(const kvc_geom *geom, int32_t layer, const kvc_pool *pool,
                               const uint16_t *q, float softmax_scale, void *out,
                               int32_t out_is_fp32, void *workspace, size_t workspace_bytes,
                               kvc_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): kvc_paged_decode_attention without a workspace
 * argument.  The split partials go to a device array inside the library, KVC_STATIC_SCRATCH_BYTES
 * per GPU, which each GPU the call runs on holds until the process ends; its device address is
 * looked up on the first call on that GPU (the current device, which must be the stream's).
 * The call allocates nothing and needs nothing cleared: every partial the combine reads is
 * written first by the same call.  All calls on one GPU share its array, so calls that overlap
 * on one GPU (other streams, other threads) race; order them on one stream.  Same arguments,
 * results and errors as kvc_paged_decode_attention, and KVC_E_WORKSPACE (before any device
 * work) when kvc_workspace_bytes(geom, KVC_OP_DECODE, 0) exceeds KVC_STATIC_SCRATCH_BYTES
 * (every batch of up to 8,192 KV heads with G <= 8 fits); KVC_E_HIP if the device or the
 * array's address cannot be queried. */
#define KVC_STATIC_SCRATCH_BYTES (64u << 20)
int kvc_paged_decode_attention_static(const kvc_geom *geom, int32_t layer, const kvc_pool *pool,
                                      const uint16_t *q, float softmax_scale, void *out,
                                      int32_t out_is_fp32, kvc_stream_t stream);

/* The same decode attention, and it adds each cached token's attention weight from this
 * query into the significance accumulators: the query is a later token for every cached
 * token, so acc_sum[cu_seqlens[b] + pos][hq] += softmax weight of (b, hq) on the live token at
 * position pos (DiffKV review page, "What carries the argument": a token's score is the mean
 * of the attention it receives from subsequent tokens).  The weights are the ones the output
 * uses: exp(s*q.k_hat - max) / sum over the head's live tokens.  Pruned tokens get nothing.
 *   acc_sum     float32 [T][Hq], the layout kvc_score_tokens reads, 16-byte aligned;
 *               updated in place
 *   cu_seqlens  int32 [B+1]: request b owns rows cu[b] .. cu[b+1]-1 (N_b rows: its length, or
 *               any larger capacity, so that a generation loop can keep one padded buffer;
 *               every row of the range is read and written back); a live token with
 *               position >= N_b, or out of ascending order within its head and tier, is
 *               skipped and sets KVC_DEV_SEQLEN
 *   max_seqlen  bounds every N_b (a longer request gets no update and sets KVC_DEV_SEQLEN)
 *   workspace >= kvc_workspace_bytes(geom, KVC_OP_DECODE_ACC, max_seqlen) bytes, 256-B aligned
 *        (split partials, softmax max/sum per query head, logits of every live token, the
 *        first slot of every 64-position chunk per head and tier).
 * The accumulator rows are updated 64 positions at a time, each row read and written whole
 * once; every (token, query head) is added by one thread: no atomics, deterministic.
 * Errors: as kvc_paged_decode_attention; KVC_E_NULL if acc_sum or cu_seqlens is NULL,
 * KVC_E_ALIGN if acc_sum is not 16-byte aligned, KVC_E_SHAPE if max_seqlen < 0 or
 * Hq > 512. */
int kvc_paged_decode_attention_acc(const kvc_geom *geom, int32_t layer, const kvc_pool *pool,
                                   const uint16_t *q, float softmax_scale, void *out,
                                   int32_t out_is_fp32, float *acc_sum,
                                   const int32_t *cu_seqlens, int32_t max_seqlen,
                                   void *workspace, size_t workspace_bytes,
                                   kvc_stream_t stream);

/* One decode step under the per-step tier policy (DiffKV review page: Algorithm 1 as the
 * referee report describes it, major comment 2 and minor comment 4; free-parameter ledger
 * for the window; "What carries the argument" for the score and the allocation round).
 * For each request b the new token (position positions[b], so N = positions[b] + 1 tokens
 * after it) enters every KV head's HIGH tier as K8V4, like kvc_append_tokens.  The token
 * t_c = N-1-window, which leaves the recent window in this step, is scored when t_c >= 0:
 * score = max over the G query heads of fl32(acc_sum[cu[b] + t_c][hq] / (N-1-t_c)); it stays
 * HIGH if score >= fl32(alpha_h/N), goes to LOW if score >= fl32(alpha_l/N), else it is
 * dropped.  A token moved to LOW is re-quantized as K4V2 from the fp16 rounding of its K8V4
 * reconstruction and takes the next LOW slot (every older LOW token has a smaller position);
 * the HIGH slots after it move down by one so that slot order stays ascending.  Pages come
 * from one allocation round of the kvc_compact_pages kind (no head is rebuilt; a HIGH count
 * never shrinks in a step).
 *   k_new, v_new  fp16 [B][Hkv][128], 16-byte aligned;  positions int32 [B]
 *   acc_sum       float32 [T][Hq], e.g. filled by kvc_paged_decode_attention_acc; read only
 *   cu_seqlens    int32 [B+1]: request b's accumulator rows are cu[b] .. cu[b+1]-1, at least
 *                 N of them (its length after the new token, or a larger capacity: the same
 *                 padded layout as the accumulating decode's); fewer set KVC_DEV_SEQLEN
 *   window        1 .. KVC_GEN_MAX_WINDOW; the head's last `window` HIGH slots must hold
 *                 positions t_c .. N-2 (else KVC_DEV_COUNT_MISMATCH)
 *   tier_out      uint8 [B][Hkv]: the tier given to t_c, 255 where no token left the window
 *   workspace >= kvc_workspace_bytes(geom, KVC_OP_GENERATE, 0) bytes, 256-B aligned
 * All or nothing: when any KVC_DEV_* bit is set (before the call, by the checks above, or by
 * the allocation round on exhaustion or row overflow) no page, count or table entry changes.
 * Errors: KVC_E_NULL, KVC_E_ALIGN, KVC_E_SHAPE (layer, window), KVC_E_WORKSPACE. */
int kvc_generation_step(const kvc_geom *geom, int32_t layer, const kvc_pool *pool,
                        const uint16_t *k_new, const uint16_t *v_new, const int32_t *positions,
                        const float *acc_sum, const int32_t *cu_seqlens, float alpha_h,
                        float alpha_l, int32_t window, uint8_t *tier_out, void *workspace,
                        size_t workspace_bytes, kvc_stream_t stream);

/* kvc_generation_step for a layer whose pages hold a precision scheme's layout: the new token
 * enters at the scheme's HIGH widths, a token leaving the window that goes LOW is re-quantized
 * at its LOW widths from the fp16 rounding of its HIGH reconstruction, and the rewritten pages
 * keep the scheme's layout.  Same workspace, outputs and errors, and KVC_E_SHAPE (or
 * KVC_E_NULL) for a scheme that does not fit (or is missing). */
int kvc_generation_step_scheme(const kvc_geom *geom, const kvc_scheme *scheme, int32_t layer,
                               const kvc_pool *pool, const uint16_t *k_new,
                               const uint16_t *v_new, const int32_t *positions,
                               const float *acc_sum, const int32_t *cu_seqlens, float alpha_h,
                               float alpha_l, int32_t window, uint8_t *tier_out,
                               void *workspace, size_t workspace_bytes, kvc_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
