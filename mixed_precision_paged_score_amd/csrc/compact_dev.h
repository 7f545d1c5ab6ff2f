// Per-head pieces of the page allocation round (kvc_compact_pages), shared by the allocation
// kernels and the generation step's fused kernels.
#pragma once

#include "kvc_internal.h"
#include "workspace.h"

namespace kvc {

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

// The commit of head i given the round's inputs (entry status, ring counters, the OR of every
// head's error bits, the round's totals, the head's demand d and its offsets oi / fi into the
// round's allocation and free regions); commit_head below loads them from a scan's header.
__device__ __forceinline__ bool commit_head_with(
    int i, int32_t *__restrict__ rows_l, int32_t *__restrict__ count_l,
    const int32_t *__restrict__ new_count, int C, int64_t P, int layer_gid0, int32_t *status,
    uint64_t *ctr, int32_t *__restrict__ ring, int32_t *__restrict__ owner, int32_t entry,
    uint64_t head0, uint64_t tail0, uint32_t herr, int64_t total_alloc, int64_t total_free,
    const HeadDemand &d, int oi, int fi, int32_t *__restrict__ old_rows,
    int32_t *__restrict__ old_count) {
    if (entry != 0) return false;                      // sticky failure: no-op
    int32_t *row = rows_l + int64_t(i) * C;
    constexpr int U = 4;                               // loads in flight per thread
    if (old_rows) {
        for (int p0 = threadIdx.x; p0 < C; p0 += U * blockDim.x) {
            int v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = p0 + u * blockDim.x;
                v[u] = p < C ? row[p] : 0;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = p0 + u * blockDim.x;
                if (p < C) old_rows[int64_t(i) * C + p] = v[u];
            }
        }
    }
    if (old_count && threadIdx.x < 2) old_count[2 * i + threadIdx.x] = count_l[2 * i + threadIdx.x];
    uint32_t err = herr;
    if (uint64_t(total_alloc) > tail0 - head0) err |= KVC_DEV_POOL_EXHAUSTED;
    if (err) {
        if (i == 0 && threadIdx.x == 0) atomicOr(status, int(err));
        return false;
    }
    __syncthreads();   // every thread has read the old counts and row before they change
    const int gid = layer_gid0 + i;
    // ring index base + k modulo P for base < 2P, k < P
    auto wrap = [&](int64_t j) {
        j -= j >= P ? P : 0;
        return j >= P ? j - P : j;
    };
    if (d.rebuilt) {
        // return the old pages to the ring's tail: HIGH in row order, then LOW from the end
        const int64_t base = int64_t(tail0 % uint64_t(P)) + fi;
        for (int k0 = threadIdx.x; k0 < d.free; k0 += U * blockDim.x) {
            int page[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + u * blockDim.x;
                page[u] = k < d.free ? row[k < d.pH ? k : C - 1 - (k - d.pH)] : 0;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + u * blockDim.x;
                if (k < d.free) {
                    ring[wrap(base + k)] = page[u];
                    owner[page[u]] = -1;
                }
            }
        }
        __syncthreads();
        for (int p = threadIdx.x; p < C; p += blockDim.x) row[p] = -1;
        __syncthreads();
    }
    const int h0 = d.rebuilt ? 0 : d.pH;       // first new HIGH row position
    const int l0 = d.rebuilt ? 0 : d.pL;       // first new LOW page index (from the right)
    const int nH = d.qH - h0;
    const int64_t abase = int64_t(head0 % uint64_t(P)) + oi;
    for (int k0 = threadIdx.x; k0 < d.alloc; k0 += U * blockDim.x) {
        int page[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + u * blockDim.x;
            page[u] = k < d.alloc ? ring[wrap(abase + k)] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + u * blockDim.x;
            if (k < d.alloc) {
                const int p = k < nH ? h0 + k : C - 1 - (l0 + (k - nH));
                row[p] = page[u];
                owner[page[u]] = gid * C + p;
            }
        }
    }
    if (threadIdx.x < 2) count_l[2 * i + threadIdx.x] = new_count[2 * i + threadIdx.x];
    if (i == 0 && threadIdx.x == 0) {
        ctr[0] = head0 + uint64_t(total_alloc);
        ctr[1] = tail0 + uint64_t(total_free);
    }
    return true;
}

// Head i's commit by one workgroup (all its threads call it): snapshot the old row and counts
// when asked, then, if the round commits (pool status clear at entry, no head overflowed or
// shrank, the total demand fits the free pages), return the rebuilt head's old pages to the
// ring's tail, take its new pages from the ring's head (off[i] / foff[i] into the round's
// regions), rewrite its row, the reverse map and its counts; head 0 moves the ring counters.
// Returns whether the round committed (the same answer in every workgroup).
__device__ __forceinline__ bool commit_head(
    int i, int32_t *__restrict__ rows_l, int32_t *__restrict__ count_l,
    const int32_t *__restrict__ new_count, const uint8_t *__restrict__ changed, int C, int64_t P,
    int layer_gid0, int32_t *status, uint64_t *ctr, int32_t *__restrict__ ring,
    int32_t *__restrict__ owner, const CompactHdr *hdr, const int32_t *__restrict__ off,
    const int32_t *__restrict__ foff, int32_t *__restrict__ old_rows,
    int32_t *__restrict__ old_count) {
    // every input of the head's commit is requested at once: the round's header, the head's
    // old and new counts and changed flag, and its offsets into the round's regions
    const int32_t entry = hdr->entry_status;
    const uint64_t head0 = hdr->head0, tail0 = hdr->tail0;
    const uint32_t herr = hdr->err;
    const int64_t total_alloc = hdr->total_alloc, total_free = hdr->total_free;
    const HeadDemand d = head_demand(count_l, new_count, changed, i, C);
    const int oi = off[i], fi = foff[i];
    asm volatile("" ::"s"(entry), "s"(d.alloc), "s"(d.free), "s"(oi), "s"(fi));
    return commit_head_with(i, rows_l, count_l, new_count, C, P, layer_gid0, status, ctr, ring,
                            owner, entry, head0, tail0, herr, total_alloc, total_free, d, oi, fi,
                            old_rows, old_count);
}

// one workgroup (256 threads) of the fused round's commit launch, for head i.  Every head's
// demand comes from cnt0, the old counts as the per-head scan launch recorded them: count_l
// itself is rewritten by each head's workgroup as it commits, and another workgroup may still
// be summing the demands then.
__device__ __forceinline__ void round_commit_block(
    int i, int nheads, int32_t *__restrict__ rows_l, int32_t *__restrict__ count_l,
    const int32_t *__restrict__ cnt0,
    const int32_t *__restrict__ new_count, const uint8_t *__restrict__ changed, int C,
    int64_t P, int layer_gid0, int32_t *status, uint64_t *ctr, int32_t *__restrict__ ring,
    int32_t *__restrict__ owner, const CompactHdr *snap, int32_t *__restrict__ ok,
    int32_t *__restrict__ old_rows, int32_t *__restrict__ old_count) {
    __shared__ int s_r[4][4];
    __shared__ uint32_t s_err[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t entry = snap->entry_status;
    const uint64_t head0 = snap->head0, tail0 = snap->tail0;
    const HeadDemand mine = head_demand(cnt0, new_count, changed, i, C);
    int ta = 0, tf = 0, pa = 0, pf = 0;
    uint32_t err = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int j = 4 * threadIdx.x + k;
        if (j >= nheads) continue;
        const HeadDemand d = head_demand(cnt0, new_count, changed, j, C);
        err |= uint32_t(d.err);
        ta += d.alloc;
        tf += d.free;
        if (j < i) {
            pa += d.alloc;
            pf += d.free;
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        ta += __shfl_xor(ta, o, 64);
        tf += __shfl_xor(tf, o, 64);
        pa += __shfl_xor(pa, o, 64);
        pf += __shfl_xor(pf, o, 64);
        err |= uint32_t(__shfl_xor(int(err), o, 64));
    }
    if (lane == 0) {
        s_r[wave][0] = ta;
        s_r[wave][1] = tf;
        s_r[wave][2] = pa;
        s_r[wave][3] = pf;
        s_err[wave] = err;
    }
    __syncthreads();
    ta = tf = pa = pf = 0;
    err = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        ta += s_r[w][0];
        tf += s_r[w][1];
        pa += s_r[w][2];
        pf += s_r[w][3];
        err |= s_err[w];
    }
    if (i == 0 && threadIdx.x == 0)
        ok[nheads] = (entry == 0 && err == 0 && uint64_t(ta) <= tail0 - head0) ? 0 : 1;
    commit_head_with(i, rows_l, count_l, new_count, C, P, layer_gid0, status, ctr, ring, owner,
                     entry, head0, tail0, err, ta, tf, mine, pa, pf, old_rows, old_count);
}


}  // namespace kvc
