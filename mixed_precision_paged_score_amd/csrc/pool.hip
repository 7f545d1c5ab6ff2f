// Pool initialisation, version, error text and workspace sizing for libkvc.
#include "kvc_internal.h"
#include "workspace.h"

#include <stdio.h>

namespace kvc {

static thread_local char g_err[256] = "";

void set_error(const char *what, hipError_t e) {
    snprintf(g_err, sizeof g_err, "%s: %s", what, hipGetErrorString(e));
}

// Empty pool: the ring lists every page once (0..P-1), head = 0, tail = P; the page table,
// the reverse map and the counts are cleared.  Grid-stride over the largest array.
__global__ void pool_init_kernel(int32_t *ring, int32_t *owner, int64_t P, int32_t *table,
                                 int64_t table_n, int32_t *count, int64_t count_n,
                                 uint64_t *ctr, int32_t *status) {
    int64_t n = P > table_n ? P : table_n;
    if (count_n > n) n = count_n;
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        if (i < P) {
            ring[i] = int32_t(i);
            owner[i] = -1;
        }
        if (i < table_n) table[i] = -1;
        if (i < count_n) count[i] = 0;
        if (i == 0) {
            ctr[0] = 0;
            ctr[1] = uint64_t(P);
            status[0] = 0;
        }
    }
}

}  // namespace kvc

using namespace kvc;

extern "C" const char *kvc_version(void) { return "libkvc 0.1 (gfx950)"; }

extern "C" const char *kvc_last_error(void) { return g_err; }

extern "C" size_t kvc_workspace_bytes(const kvc_geom *g, int32_t op, int32_t max_seqlen) {
    if (check_geom(g) != KVC_OK) return 0;
    switch (op) {
        case KVC_OP_COMPACT: return CompactWs(g).bytes;
        case KVC_OP_QUANTIZE: return max_seqlen < 0 ? 0 : QuantWs(g, max_seqlen).bytes;
        case KVC_OP_DECODE: return DecodeWs(g, false).bytes;
        case KVC_OP_DECODE_ACC: return max_seqlen < 0 ? 0 : DecodeWs(g, true, max_seqlen).bytes;
        case KVC_OP_APPEND: return AppendWs(g).bytes;
        case KVC_OP_GENERATE: return GenWs(g).bytes;
        case KVC_OP_PREFILL: return max_seqlen < 0 ? 0 : PrefillWs(g, max_seqlen).bytes;
        case KVC_OP_ROUND: return max_seqlen < 0 ? 0 : RoundWs(g, max_seqlen).bytes;
        default: return 0;
    }
}

extern "C" int kvc_pool_init(const kvc_geom *g, const kvc_pool *p, kvc_stream_t stream) {
    int rc = check_geom(g);
    if (rc) return rc;
    rc = check_pool(p);
    if (rc) return rc;
    int64_t table_n = int64_t(g->num_layers) * g->batch * g->num_kv_heads * g->row_capacity;
    int64_t count_n = int64_t(g->num_layers) * g->batch * g->num_kv_heads * 2;
    int64_t n = g->num_pages > table_n ? g->num_pages : table_n;
    if (count_n > n) n = count_n;
    int blocks = int((n + 255) / 256);
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(pool_init_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       p->free_ring, p->owner, g->num_pages, p->page_table, table_n, p->count,
                       count_n, p->ring_ctr, p->dev_status);
    return launch_check("kvc_pool_init");
}
