// Device pieces shared by the prefill kernels (ssd_prefill.hip) and the fused
// scan walk (ssd_scan_walk.hip): the B^T fragment order, the XCD-aware item
// order and raw buffer access.
#pragma once

#include "ssd_device.h"

namespace ssd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// B^T of a chunk is kept in the order the chunk_state MFMAs consume it: for
// n-tile nt (32 values of n), k-step s (16 tokens) and lane l = 32 half + col
// the eight tokens 16 s + 8 half + j (j < 8) of row n = 32 nt + col are
// consecutive, so each wave-wide 16-byte-per-lane load reads one contiguous
// fragment.  Element (n, t) of chunk k, group g sits at
//   bt[(k G + g) ntp Q + ((nt (Q/16) + s) 64 + l) 8 + j].
__host__ __device__ constexpr int bt_frag(int Q, int nt, int s, int lane) {
    return ((nt * (Q / 16) + s) * 64 + lane) * 8;
}

// Grid order: item i of a chunk-major work list runs as workgroup L with
// i = (L % 8) * per_xcd + L / 8.  Workgroups are dealt to the 8 XCDs round
// robin, so each XCD walks a contiguous range of items: the heads and column
// tiles of one chunk run together and share its C.B^T, C and B^T in that
// XCD's L2.
__device__ inline int64_t xcd_item(int per_xcd) {
    return (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
}

// Raw buffer access (gfx9 descriptor: untyped 32-bit data format word).
constexpr int kBufferWord3 = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// A raw buffer offset past any descriptor's range (accesses there are dropped).
constexpr int kOutOfRange = 0x7ffffff0;

// Four consecutive outputs through a raw buffer descriptor (byte offset voff).
// These stores carry the non-temporal hint: y and the per-chunk states are
// written once and not read again by the same kernel, so they should not
// displace its inputs from the caches.
constexpr int kNonTemporal = 2;  // cache-policy bit of gfx9.4+ buffer instructions
template <typename TY>
__device__ inline void buffer_store4(f32x4 v, __amdgpu_buffer_rsrc_t r, int voff);
template <>
__device__ inline void buffer_store4<float>(f32x4 v, __amdgpu_buffer_rsrc_t r, int voff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, 0, kNonTemporal);
}
template <>
__device__ inline void buffer_store4<bf16_t>(f32x4 v, __amdgpu_buffer_rsrc_t r, int voff) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, Tr<bf16_t>::narrow4(v)), r, voff, 0,
                                          kNonTemporal);
}

// Eight consecutive elements through a raw buffer descriptor (byte offset voff).
template <typename T>
__device__ inline typename Tr<T>::v8 buffer_ld8(__amdgpu_buffer_rsrc_t r, int voff);
template <>
__device__ inline bf16x8 buffer_ld8<bf16_t>(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
template <>
__device__ inline f32x8 buffer_ld8<float>(__amdgpu_buffer_rsrc_t r, int voff) {
    const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
    const f32x4 b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, 0, 0));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The x rows of one chunk as a buffer: uniform base, 32-bit lane offsets.
template <typename T>
__device__ inline __amdgpu_buffer_rsrc_t chunk_x_rsrc(const T* x, const ChunkDesc& cd, int H, int P) {
    return buffer_rsrc(x + (size_t)cd.row0 * H * P, (uint32_t)((size_t)cd.len * H * P * sizeof(T)));
}

}  // namespace ssd
