// Page reads by buffer loads, shared by the decode kernels: one descriptor per page
// (wave-uniform, scalar registers: the page's address and its size as the range) and a 32-bit
// per-lane offset, so no lane does 64-bit address arithmetic, and an offset outside the page
// reads zeros.
#pragma once

#include "kvc_internal.h"

namespace kvc {

typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
constexpr int BUF_FLAGS = 0x00020000;      // raw (untyped) 32-bit access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t *page) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(page), 0, PAGE, BUF_FLAGS);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u4v x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u2v x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(x[0], x[1]);
}
__device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

}  // namespace kvc
