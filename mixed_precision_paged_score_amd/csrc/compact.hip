// kvc_compact_pages: GPU-resident page allocation by prefix sum over the circular free list.
//
// DiffKV review page, "What carries the argument": after each head decides how many high-
// and low-precision pages it needs, a parallel prefix sum over the circular free page list
// assigns every head a disjoint contiguous region of page ids, so allocation and recycling
// happen on the GPU in one coordinated step.  "Core claim": circular free list and
// bidirectional page table (page table rows + the owner reverse map).
//
// Three launches on the caller's stream (up to 256 heads, one scan tile: compact_scan1, one
// workgroup doing the whole scan with nothing to clear, then the commit):
//   1. compact_zero   clears the scan header and tile descriptors (a fill kernel, so the
//                     sequence stays valid inside a captured graph)
//   2. compact_scan   single-pass scan over heads: LDS block scan of (alloc, free) per
//                     256-head tile plus decoupled look-back across tiles (Merrill & Garland,
//                     "Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016);
//                     tiles take their index from an atomic ticket, so every predecessor a
//                     tile waits on has already started and never waits on it.
//   3. compact_commit all-or-nothing commit: if the pool status was clear, no head overflowed
//                     or shrank and the total demand fits the free pages, each workgroup
//                     rewrites one head's row, its ring segments and the reverse map.
// The alloc region [head0, head0 + total_alloc) and the return region
// [tail0, tail0 + total_free) of the ring are disjoint modulo P (the returned pages are live
// pages, so tail0 + total_free <= head0 + P), so the commit has no cross-workgroup hazards.
#include "compact_dev.h"
#include "kvc_internal.h"
#include "workspace.h"

namespace kvc {

// tile descriptor: bits 62..63 flag, 31..61 free sum, 0..30 alloc sum
constexpr uint64_t FLAG_AGG = 1ull << 62, FLAG_INC = 2ull << 62, FLAG_MASK = 3ull << 62;
constexpr uint64_t SUM_MASK = (1ull << 31) - 1;

__device__ __forceinline__ uint64_t pack_desc(uint64_t flag, int64_t a, int64_t f) {
    return flag | (uint64_t(f) << 31) | uint64_t(a);
}

__global__ void compact_zero_kernel(CompactHdr *hdr, uint64_t *st, int ntiles) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) {
        hdr->ticket = 0;
        hdr->err = 0;
        hdr->total_alloc = 0;
        hdr->total_free = 0;
        hdr->head0 = 0;
        hdr->tail0 = 0;
        hdr->entry_status = 0;
    }
    if (i < ntiles) st[i] = 0;
}

__global__ __launch_bounds__(SCAN_TILE) void compact_scan_kernel(
    const int32_t *__restrict__ count_l, const int32_t *__restrict__ new_count,
    const uint8_t *__restrict__ changed, int nheads, int C, const int32_t *status,
    const uint64_t *ctr, CompactHdr *hdr, uint64_t *st, int32_t *off, int32_t *foff) {
    __shared__ int s_tile;
    __shared__ int s_wa[4], s_wf[4];
    __shared__ long long s_pa, s_pf;
    if (threadIdx.x == 0) s_tile = int(atomicAdd(&hdr->ticket, 1u));
    __syncthreads();
    const int tile = s_tile;
    const int i = tile * SCAN_TILE + threadIdx.x;
    HeadDemand d{};
    if (i < nheads) d = head_demand(count_l, new_count, changed, i, C);
    if (d.err) atomicOr(&hdr->err, uint32_t(d.err));
    int a = d.alloc, f = d.free;
    block_scan2(a, f, s_wa, s_wf);       // inclusive within the tile
    if (threadIdx.x == SCAN_TILE - 1) {
        // publish the tile aggregate, then look back for the exclusive prefix
        int64_t pa = 0, pf = 0;
        if (tile == 0) {
            __hip_atomic_store(&st[0], pack_desc(FLAG_INC, a, f), __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
        } else {
            __hip_atomic_store(&st[tile], pack_desc(FLAG_AGG, a, f), __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
            uint32_t spins = 0;
            for (int j = tile - 1; j >= 0;) {
                uint64_t v = __hip_atomic_load(&st[j], __ATOMIC_ACQUIRE,
                                               __HIP_MEMORY_SCOPE_AGENT);
                uint64_t flag = v & FLAG_MASK;
                if (flag == 0) {
                    // a predecessor holds an earlier ticket, so it is running and publishes
                    // without waiting; the bound only turns a broken invariant into an error
                    if (++spins > (1u << 24)) {
                        atomicOr(&hdr->err, uint32_t(KVC_DEV_INTERNAL));
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                    continue;
                }
                pa += int64_t(v & SUM_MASK);
                pf += int64_t((v >> 31) & SUM_MASK);
                if (flag == FLAG_INC) break;
                --j;
            }
            __hip_atomic_store(&st[tile], pack_desc(FLAG_INC, pa + a, pf + f),
                               __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
        s_pa = pa;
        s_pf = pf;
        if (tile == gridDim.x - 1) {
            hdr->total_alloc = pa + a;
            hdr->total_free = pf + f;
            hdr->head0 = ctr[0];
            hdr->tail0 = ctr[1];
            hdr->entry_status = *status;
        }
    }
    __syncthreads();
    if (i < nheads) {
        off[i] = int32_t(s_pa + a - d.alloc);    // exclusive
        foff[i] = int32_t(s_pf + f - d.free);
    }
}

// up to SCAN_TILE heads: the whole scan in one workgroup (no look-back state to clear)
__global__ __launch_bounds__(SCAN_TILE) void compact_scan1_kernel(
    const int32_t *__restrict__ count_l, const int32_t *__restrict__ new_count,
    const uint8_t *__restrict__ changed, int nheads, int C, const int32_t *status,
    const uint64_t *ctr, CompactHdr *hdr, int32_t *off, int32_t *foff) {
    __shared__ int s_wa[4], s_wf[4];
    __shared__ uint32_t s_err;
    if (threadIdx.x == 0) s_err = 0u;
    __syncthreads();
    const int i = threadIdx.x;
    HeadDemand d{};
    if (i < nheads) {
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
    if (threadIdx.x == SCAN_TILE - 1) {
        hdr->err = s_err;
        hdr->total_alloc = a;
        hdr->total_free = f;
        hdr->head0 = ctr[0];
        hdr->tail0 = ctr[1];
        hdr->entry_status = *status;
    }
}

// one workgroup per head: snapshot the old row, then (if the call commits) rewrite it
__global__ __launch_bounds__(256) void compact_commit_kernel(
    int32_t *__restrict__ rows_l, int32_t *__restrict__ count_l,
    const int32_t *__restrict__ new_count, const uint8_t *__restrict__ changed, int C,
    int64_t P, int layer_gid0, int32_t *status, uint64_t *ctr, int32_t *__restrict__ ring,
    int32_t *__restrict__ owner, const CompactHdr *hdr, const int32_t *__restrict__ off,
    const int32_t *__restrict__ foff, int32_t *__restrict__ old_rows,
    int32_t *__restrict__ old_count) {
    commit_head(blockIdx.x, rows_l, count_l, new_count, changed, C, P, layer_gid0, status, ctr,
                ring, owner, hdr, off, foff, old_rows, old_count);
}

// The planning and the commits of a fused round (kvc_compaction_round) in one launch, one
// workgroup per head: every workgroup sums all heads' demands itself (thread t takes heads
// 4t .. 4t + 3, as the planning workgroup did) for the round's totals, error bits and its
// own head's offsets, so no planning launch stands between the per-head scans and the
// commits.  The pool status and ring counters at the round's start come from *snap, taken by
// the per-head scan launch: no workgroup here reads them after another may have moved them.
// Workgroup 0 records in ok[nheads] whether the round commits (0) or not (1).
__global__ __launch_bounds__(256) void round_commit_kernel(
    int nheads, int32_t *__restrict__ rows_l, int32_t *__restrict__ count_l,
    const int32_t *__restrict__ cnt0, const int32_t *__restrict__ new_count,
    const uint8_t *__restrict__ changed, int C, int64_t P, int layer_gid0, int32_t *status,
    uint64_t *ctr, int32_t *__restrict__ ring, int32_t *__restrict__ owner,
    const CompactHdr *snap, int32_t *__restrict__ ok, int32_t *__restrict__ old_rows) {
    round_commit_block(blockIdx.x, nheads, rows_l, count_l, cnt0, new_count, changed, C, P,
                       layer_gid0, status, ctr, ring, owner, snap, ok, old_rows, nullptr);
}

}  // namespace kvc

using namespace kvc;

namespace kvc {

// the planning and commit launch of a fused round (round_commit_kernel); the round's start
// was snapshotted into the compact workspace's header by the per-head scan launch
int launch_round_commit(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                        const int32_t *cnt0, const int32_t *new_count, const uint8_t *changed,
                        int32_t *ok, int32_t *old_rows_out, void *compact_ws, hipStream_t s) {
    const CompactWs L(g);
    char *w = static_cast<char *>(compact_ws);
    const int C = g->row_capacity;
    int32_t *rows_l = p->page_table + int64_t(layer) * L.nheads * C;
    int32_t *count_l = p->count + int64_t(layer) * L.nheads * 2;
    hipLaunchKernelGGL(round_commit_kernel, dim3(L.nheads), dim3(256), 0, s, L.nheads, rows_l,
                       count_l, cnt0, new_count, changed, C, g->num_pages, layer * L.nheads,
                       p->dev_status, p->ring_ctr, p->free_ring, p->owner,
                       reinterpret_cast<const CompactHdr *>(w + L.hdr), ok, old_rows_out);
    return launch_check("kvc_compaction_round/commit");
}

// the three launches of one allocation round (arguments already validated)
int launch_compact(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                   const int32_t *new_count, const uint8_t *changed, int32_t *old_rows_out,
                   int32_t *old_count_out, void *ws, hipStream_t s) {
    CompactWs L(g);
    char *w = static_cast<char *>(ws);
    CompactHdr *hdr = reinterpret_cast<CompactHdr *>(w + L.hdr);
    uint64_t *st = reinterpret_cast<uint64_t *>(w + L.st);
    int32_t *off = reinterpret_cast<int32_t *>(w + L.off);
    int32_t *foff = reinterpret_cast<int32_t *>(w + L.foff);
    const int C = g->row_capacity;
    int32_t *rows_l = p->page_table + int64_t(layer) * L.nheads * C;
    int32_t *count_l = p->count + int64_t(layer) * L.nheads * 2;
    int rc;
    if (L.ntiles == 1) {
        hipLaunchKernelGGL(compact_scan1_kernel, dim3(1), dim3(SCAN_TILE), 0, s, count_l,
                           new_count, changed, L.nheads, C, p->dev_status, p->ring_ctr, hdr, off,
                           foff);
        rc = launch_check("compact/scan1");
    } else {
        hipLaunchKernelGGL(compact_zero_kernel, dim3((L.ntiles + 255) / 256), dim3(256), 0, s,
                           hdr, st, L.ntiles);
        rc = launch_check("compact/zero");
        if (rc) return rc;
        hipLaunchKernelGGL(compact_scan_kernel, dim3(L.ntiles), dim3(SCAN_TILE), 0, s, count_l,
                           new_count, changed, L.nheads, C, p->dev_status, p->ring_ctr, hdr, st,
                           off, foff);
        rc = launch_check("compact/scan");
    }
    if (rc) return rc;
    hipLaunchKernelGGL(compact_commit_kernel, dim3(L.nheads), dim3(256), 0, s, rows_l, count_l,
                       new_count, changed, C, g->num_pages, layer * L.nheads, p->dev_status,
                       p->ring_ctr, p->free_ring, p->owner, hdr, off, foff, old_rows_out,
                       old_count_out);
    return launch_check("compact/commit");
}

}  // namespace kvc

extern "C" int kvc_compact_pages(const kvc_geom *g, int32_t layer, const kvc_pool *p,
                                 const int32_t *new_count, const uint8_t *changed,
                                 int32_t *old_rows_out, int32_t *old_count_out, void *ws,
                                 size_t ws_bytes, kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    if (!new_count) return KVC_E_NULL;
    if (layer < 0 || layer >= g->num_layers) return KVC_E_SHAPE;
    CompactWs L(g);
    if (!ws || ws_bytes < L.bytes) return KVC_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return KVC_E_ALIGN;
    // sums of pages per call must fit 31 bits
    if (int64_t(L.nheads) * g->row_capacity >= (int64_t(1) << 31)) return KVC_E_SHAPE;
    return launch_compact(g, layer, p, new_count, changed, old_rows_out, old_count_out, ws,
                          (hipStream_t)stream);
}
