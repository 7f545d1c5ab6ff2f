// kvc_compact_pages: GPU-resident page allocation by prefix sum over the circular free list.
//
// DiffKV review page, "What carries the argument": after each head decides how many high-
// and low-precision pages it needs, a parallel prefix sum over the circular free page list
// assigns every head a disjoint contiguous region of page ids, so allocation and recycling
// happen on the GPU in one coordinated step.  "Core claim": circular free list and
// bidirectional page table (page table rows + the owner reverse map).
//
// Three launches on the caller's stream:
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

struct HeadDemand {
    int pH, pL, qH, qL, alloc, free, rebuilt, err;
};

__device__ __forceinline__ HeadDemand head_demand(const int32_t *count_l,
                                                  const int32_t *new_count,
                                                  const uint8_t *changed, int i, int C) {
    HeadDemand d;
    const int nh = count_l[2 * i], nl = count_l[2 * i + 1];
    const int mh = new_count[2 * i], ml = new_count[2 * i + 1];
    d.pH = ceil_div(nh, HS);
    d.pL = ceil_div(nl, LS);
    d.qH = ceil_div(mh, HS);
    d.qL = ceil_div(ml, LS);
    d.rebuilt = changed == nullptr || changed[i] != 0;
    d.err = 0;
    if (d.rebuilt) {
        d.alloc = d.qH + d.qL;
        d.free = d.pH + d.pL;
    } else {
        if (d.qH < d.pH || d.qL < d.pL) d.err |= KVC_DEV_SHRINK;
        d.alloc = max(d.qH - d.pH, 0) + max(d.qL - d.pL, 0);
        d.free = 0;
    }
    if (d.qH + d.qL > C || mh < 0 || ml < 0) d.err |= KVC_DEV_ROW_OVERFLOW;
    if (d.err) d.alloc = d.free = 0;   // keep sums in range; the call fails anyway
    return d;
}

// inclusive block scan of two ints over 256 threads (4 wave64s): wave scans by shuffles,
// then a scan of the 4 wave totals in LDS
__device__ __forceinline__ void block_scan2(int &a, int &f, int *s_wa, int *s_wf) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int ua = __shfl_up(a, o, 64), uf = __shfl_up(f, o, 64);
        if (lane >= o) {
            a += ua;
            f += uf;
        }
    }
    if (lane == 63) {
        s_wa[wave] = a;
        s_wf[wave] = f;
    }
    __syncthreads();
    int pa = 0, pf = 0;
    for (int w = 0; w < wave; ++w) {
        pa += s_wa[w];
        pf += s_wf[w];
    }
    a += pa;
    f += pf;
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

// one workgroup per head: snapshot the old row, then (if the call commits) rewrite it
__global__ __launch_bounds__(256) void compact_commit_kernel(
    int32_t *__restrict__ rows_l, int32_t *__restrict__ count_l,
    const int32_t *__restrict__ new_count, const uint8_t *__restrict__ changed, int C,
    int64_t P, int layer_gid0, int32_t *status, uint64_t *ctr, int32_t *__restrict__ ring,
    int32_t *__restrict__ owner, const CompactHdr *hdr, const int32_t *__restrict__ off,
    const int32_t *__restrict__ foff, int32_t *__restrict__ old_rows,
    int32_t *__restrict__ old_count) {
    const int i = blockIdx.x;
    if (hdr->entry_status != 0) return;               // sticky failure: no-op
    int32_t *row = rows_l + int64_t(i) * C;
    if (old_rows)
        for (int p = threadIdx.x; p < C; p += blockDim.x) old_rows[int64_t(i) * C + p] = row[p];
    if (old_count && threadIdx.x < 2) old_count[2 * i + threadIdx.x] = count_l[2 * i + threadIdx.x];
    const uint64_t head0 = hdr->head0, tail0 = hdr->tail0;
    uint32_t err = hdr->err;
    if (uint64_t(hdr->total_alloc) > tail0 - head0) err |= KVC_DEV_POOL_EXHAUSTED;
    if (err) {
        if (i == 0 && threadIdx.x == 0) atomicOr(status, int(err));
        return;
    }
    const HeadDemand d = head_demand(count_l, new_count, changed, i, C);
    __syncthreads();   // every thread has read the old counts and row before they change
    const int gid = layer_gid0 + i;
    if (d.rebuilt) {
        // return the old pages to the ring's tail: HIGH in row order, then LOW from the end
        const int64_t base = int64_t(tail0 % uint64_t(P)) + foff[i];
        for (int k = threadIdx.x; k < d.free; k += blockDim.x) {
            const int p = k < d.pH ? k : C - 1 - (k - d.pH);
            const int page = row[p];
            ring[(base + k) % P] = page;
            owner[page] = -1;
        }
        __syncthreads();
        for (int p = threadIdx.x; p < C; p += blockDim.x) row[p] = -1;
        __syncthreads();
    }
    const int h0 = d.rebuilt ? 0 : d.pH;       // first new HIGH row position
    const int l0 = d.rebuilt ? 0 : d.pL;       // first new LOW page index (from the right)
    const int nH = d.qH - h0;
    const int64_t abase = int64_t(head0 % uint64_t(P)) + off[i];
    for (int k = threadIdx.x; k < d.alloc; k += blockDim.x) {
        const int page = ring[(abase + k) % P];
        const int p = k < nH ? h0 + k : C - 1 - (l0 + (k - nH));
        row[p] = page;
        owner[page] = gid * C + p;
    }
    if (threadIdx.x < 2) count_l[2 * i + threadIdx.x] = new_count[2 * i + threadIdx.x];
    if (i == 0 && threadIdx.x == 0) {
        ctr[0] = head0 + uint64_t(hdr->total_alloc);
        ctr[1] = tail0 + uint64_t(hdr->total_free);
    }
}

}  // namespace kvc

using namespace kvc;

namespace kvc {

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
    hipLaunchKernelGGL(compact_zero_kernel, dim3((L.ntiles + 255) / 256), dim3(256), 0, s, hdr,
                       st, L.ntiles);
    int rc = launch_check("compact/zero");
    if (rc) return rc;
    hipLaunchKernelGGL(compact_scan_kernel, dim3(L.ntiles), dim3(SCAN_TILE), 0, s, count_l,
                       new_count, changed, L.nheads, C, p->dev_status, p->ring_ctr, hdr, st,
                       off, foff);
    rc = launch_check("compact/scan");
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
