// Device-side helpers for the gfx950 (CDNA4) SSD kernels: element traits,
// the 32x32 MFMA step, wave64 prefix scan and the chunk/segment descriptors.
#pragma once

#include <hip/hip_runtime.h>

#include "ssd_internal.h"

namespace ssd {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- elements
// Tr<T> gives the 8-element operand vector of element type T and the moves
// between it and fp32.  bf16 widening is exact; narrowing rounds to nearest
// even (v_cvt_pk_bf16_f32).
template <typename T>
struct Tr;

template <>
struct Tr<bf16_t> {
    typedef bf16_t elem;
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    __device__ static inline v4 ld4raw(const bf16_t* p) { return *(const v4*)p; }
    __device__ static inline v8 ld8(const bf16_t* p) { return *(const v8*)p; }
    __device__ static inline void st8(bf16_t* p, v8 v) { *(v8*)p = v; }
    __device__ static inline f32x8 widen(v8 v) { return __builtin_convertvector(v, f32x8); }
    __device__ static inline v8 narrow(f32x8 v) { return __builtin_convertvector(v, v8); }
    __device__ static inline f32x4 ld4(const bf16_t* p) {
        return __builtin_convertvector(*(const bf16x4*)p, f32x4);
    }
    __device__ static inline void st4(bf16_t* p, f32x4 v) {
        *(bf16x4*)p = __builtin_convertvector(v, bf16x4);
    }
    __device__ static inline v4 narrow4(f32x4 v) { return __builtin_convertvector(v, bf16x4); }
    __device__ static inline f32x4 widen4(v4 v) { return __builtin_convertvector(v, f32x4); }
    __device__ static inline void st4raw(bf16_t* p, v4 v) { *(v4*)p = v; }
};

template <>
struct Tr<float> {
    typedef float elem;
    typedef f32x8 v8;
    typedef f32x4 v4;
    __device__ static inline v4 ld4raw(const float* p) { return *(const v4*)p; }
    __device__ static inline v8 ld8(const float* p) {
        f32x4 a = *(const f32x4*)p;
        f32x4 b = *(const f32x4*)(p + 4);
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    __device__ static inline void st8(float* p, v8 v) {
        *(f32x4*)p = __builtin_shufflevector(v, v, 0, 1, 2, 3);
        *(f32x4*)(p + 4) = __builtin_shufflevector(v, v, 4, 5, 6, 7);
    }
    __device__ static inline f32x8 widen(v8 v) { return v; }
    __device__ static inline v8 narrow(f32x8 v) { return v; }
    __device__ static inline f32x4 ld4(const float* p) { return *(const f32x4*)p; }
    __device__ static inline void st4(float* p, f32x4 v) { *(f32x4*)p = v; }
    __device__ static inline v4 narrow4(f32x4 v) { return v; }
    __device__ static inline f32x4 widen4(v4 v) { return v; }
    __device__ static inline void st4raw(float* p, v4 v) { *(v4*)p = v; }
};

// ---------------------------------------------------------------- MFMA
// One K=16 step of a 32x32 fp32-accumulated tile product, D += A(32x16) B(16x32).
// Operand fragment convention (both dtypes): lane l holds 8 values of row
// (A) or column (B) l%32, at k = 8*(l/32) + i, i = 0..7.  Accumulator: lane l,
// register v holds D[8*(v/4) + 4*(l/32) + v%4][l%32].
// bf16: one v_mfma_f32_32x32x16_bf16.  fp32: eight v_mfma_f32_32x32x2_f32, step
// i pairing k = i (lanes 0-31) with k = 8 + i (lanes 32-63); the sum over the
// eight steps covers all sixteen k of the step exactly once.
__device__ inline void mma16(f32x16& acc, bf16x8 a, bf16x8 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ inline void mma16(f32x16& acc, f32x8 a, f32x8 b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
}

__device__ inline int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// ---------------------------------------------------------------- wave scan
// Inclusive prefix sum over the 64 lanes of a wave with DPP: Hillis-Steele
// shifts inside each row of 16 lanes, then row_bcast:15 / row_bcast:31 carry
// the row totals upward (the classic GCN wave scan).
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_take(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}
__device__ inline float wave_inclusive_scan(float v) {
    v += dpp_take<0x111, 0xf>(v);  // row_shr:1
    v += dpp_take<0x112, 0xf>(v);  // row_shr:2
    v += dpp_take<0x114, 0xf>(v);  // row_shr:4
    v += dpp_take<0x118, 0xf>(v);  // row_shr:8
    v += dpp_take<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_take<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// ---------------------------------------------------------------- dt activation
// softplus(raw + bias[h]) clamped to [lo, hi] when a.on (raw as given
// otherwise); softplus(v) = log(1 + exp(v)), v itself above 20.
__device__ inline float dt_activate(const DtAct& a, float raw, int h) {
    if (!a.on) return raw;
    const float v = raw + (a.bias ? a.bias[h] : 0.f);
    const float sp = v > 20.f ? v : log1pf(expf(v));
    return fminf(fmaxf(sp, a.lo), a.hi);
}

// ---------------------------------------------------------------- descriptors
struct ChunkDesc {
    int32_t seq;   // -1: no such chunk
    int32_t len;
    int64_t row0;
    int32_t idx;   // chunk index inside its sequence
};

__device__ inline ChunkDesc chunk_desc(const Plan& pl, int k) {
    ChunkDesc d;
    if (pl.dense) {
        if (k >= pl.nchunk_ub) { d.seq = -1; d.len = 0; d.row0 = 0; d.idx = 0; return d; }
        const int s = k / pl.cpseq;
        const int c = k - s * pl.cpseq;
        const int64_t t0 = (int64_t)c * pl.Q;
        d.seq = s;
        d.row0 = (int64_t)s * pl.L + t0;
        d.len = (int32_t)min((int64_t)pl.Q, pl.L - t0);
        d.idx = c;
        return d;
    }
    const int4 e = ((const int4*)pl.chunk_tab)[k];
    d.seq = e.x;
    d.row0 = e.y;
    d.len = e.z;
    d.idx = e.w;
    return d;
}

// The descriptor of a workgroup's chunk is the same for every lane; saying so
// lets the compiler keep it in scalar registers (buffer descriptors built from
// it then need no per-lane handling).
__device__ inline ChunkDesc uniform_desc(ChunkDesc d) {
    ChunkDesc u;
    u.seq = __builtin_amdgcn_readfirstlane(d.seq);
    u.len = __builtin_amdgcn_readfirstlane(d.len);
    u.idx = __builtin_amdgcn_readfirstlane(d.idx);
    const uint64_t r = (uint64_t)d.row0;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)r);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(r >> 32));
    u.row0 = (int64_t)(((uint64_t)hi << 32) | lo);
    return u;
}

// Sequence s: first chunk and chunk count.
__device__ inline int2 seq_chunks(const Plan& pl, int s) {
    if (pl.dense) return make_int2(s * pl.cpseq, pl.cpseq);
    const int4 q = ((const int4*)pl.seq_tab)[s];
    return make_int2(q.x, q.y);
}

// Sequence s: first chunk, chunk count, first token row and token count.
struct SeqExtent {
    int32_t chunk0, nchunks, len;
    int64_t row0;
};

__device__ inline SeqExtent seq_extent(const Plan& pl, int s) {
    SeqExtent e;
    if (pl.dense) {
        e.chunk0 = s * pl.cpseq;
        e.nchunks = pl.cpseq;
        e.len = (int32_t)pl.L;
        e.row0 = (int64_t)s * pl.L;
        return e;
    }
    const int4 q = ((const int4*)pl.seq_tab)[s];
    e.chunk0 = q.x;
    e.nchunks = q.y;
    e.row0 = q.z;
    e.len = q.w;
    return e;
}

}  // namespace ssd
