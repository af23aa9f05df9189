// O(1) cached decode step on gfx950: one token per sequence, state updated in
// place ("Compiler-First State Space Duality...", abstract: cached decode with
// a cost independent of the sequence length; recurrence from "Engineering
// hybrid state-space models", section 2):
//   S[p][:] <- exp(dt A) S[p][:] + (dt x[p]) B[:] ;  y[p] = S[p][:].C[:] + D x[p]
//
// The step is bound by HBM bandwidth: the fp32 state is read once and written
// once (the read-D + write-D accounting of the SketchSSM page, Table 4).  One
// wave streams one (sequence, head) block of P x N floats with 128-bit
// non-temporal loads and stores, several in flight per lane; the dot product
// with C is reduced across the row's lanes with DPP moves.  No MFMA: one
// multiply-add per element.
#include "ssd_device.h"

namespace ssd {

namespace {

constexpr int kDecThreads = 256;  // four waves, one (sequence, head) state block each
constexpr int kBatch = 8;         // 128-bit state loads in flight per lane

// Sum over aligned groups of TPR lanes with DPP moves (no LDS): quad swaps,
// half-row and row mirrors, then row broadcasts across 16-lane rows.  The
// group's last lane always holds the group sum.
template <int TPR>
__device__ inline float group_sum(float v) {
    if (TPR >= 2) v += dpp_take<0xB1, 0xf>(v);   // quad_perm [1,0,3,2]
    if (TPR >= 4) v += dpp_take<0x4E, 0xf>(v);   // quad_perm [2,3,0,1]
    if (TPR >= 8) v += dpp_take<0x141, 0xf>(v);  // row_half_mirror
    if (TPR >= 16) v += dpp_take<0x140, 0xf>(v); // row_mirror
    if (TPR >= 32) v += dpp_take<0x142, 0xa>(v); // row_bcast:15 into rows 1 and 3
    if (TPR >= 64) v += dpp_take<0x143, 0xc>(v); // row_bcast:31 into rows 2 and 3
    return v;
}

// Raw buffer descriptor (gfx9 untyped data word) and an offset beyond any
// descriptor's range: stores there are dropped by the hardware.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kOutOfRange = 0x7ffffff0;
constexpr int kNonTemporal = 2;  // cache-policy bit of gfx9.4+ buffer instructions: streaming store
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// Wave w of block L updates the state block (b, h) = 4L + w: P rows of N
// floats, contiguous.  Lane l owns columns n = 4 (l % TPR) .. +3 of the rows
// p = RPI i + l / TPR, so each wave instruction moves 64 x 16 contiguous bytes
// and B, C, dt, A are loaded once per lane.  Rows go in batches of kBatch
// instructions; the next batch is loaded before the current one is stored,
// and every lane issues every store (rows past P, columns past N and the
// lanes that do not own a y element get an out-of-range offset), so the wait
// for a batch never includes the previous batch's stores.
template <typename T, int TPR>
__global__ __launch_bounds__(kDecThreads) void ssd_decode_kernel(
    int64_t nbh, int H, int P, int N, int G, float* __restrict__ state, const T* __restrict__ x,
    const float* __restrict__ dt, const float* __restrict__ A, const T* __restrict__ B,
    const T* __restrict__ C, const float* __restrict__ D, void* __restrict__ y, int y_f32, DtAct act) {
    constexpr int RPI = 64 / TPR;  // rows per wave instruction
    constexpr int RPB = RPI * kBatch;  // rows per batch
    const int lane = threadIdx.x & 63;
    const int64_t bh = (int64_t)blockIdx.x * (kDecThreads / 64) + (threadIdx.x >> 6);
    if (bh >= nbh) return;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int j = lane % TPR, rsub = lane / TPR;
    const bool nv = 4 * j < N;
    const int n = nv ? 4 * j : N - 4;
    const float d = dt_activate(act, dt[bh], h);
    const float a = __expf(d * A[h]);
    const float Dh = D[h];
    const f32x4 bv = nv ? Tr<T>::ld4(B + (b * G + g) * N + n) : f32x4{};
    const f32x4 cv = nv ? Tr<T>::ld4(C + (b * G + g) * N + n) : f32x4{};
    float* sb = state + bh * P * N;
    const T* xb = x + bh * P;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(sb, (uint32_t)(P * N * sizeof(float)));
    const __amdgpu_buffer_rsrc_t ry =
        buffer_rsrc((char*)y + bh * P * (y_f32 ? 4 : 2), (uint32_t)(P * (y_f32 ? 4 : 2)));
    f32x4 s[kBatch], sn[kBatch];
    float xv[kBatch], xn[kBatch];
    auto load = [&](int p0, f32x4 (&dst)[kBatch], float (&xd)[kBatch]) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int p = min(p0 + u * RPI + rsub, P - 1);
            dst[u] = __builtin_nontemporal_load((const f32x4*)(sb + (int64_t)p * N + n));
            xd[u] = (float)xb[p];
        }
    };
    load(0, s, xv);
    for (int p0 = 0; p0 < P; p0 += RPB) {
        load(min(p0 + RPB, P - 1), sn, xn);  // next batch (repeats the last rows at the end)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int p = p0 + u * RPI + rsub;
            const f32x4 ns = a * s[u] + (d * xv[u]) * bv;
            const float tot = group_sum<TPR>(ns[0] * cv[0] + ns[1] * cv[1] + ns[2] * cv[2] + ns[3] * cv[3]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ns), rs,
                                                   (p < P && nv) ? (p * N + n) * 4 : kOutOfRange, 0, kNonTemporal);
            const float o = tot + Dh * xv[u];
            const bool yo = j == TPR - 1 && p < P;
            if (y_f32)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o), ry, yo ? p * 4 : kOutOfRange,
                                                      0, kNonTemporal);
            else
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16_t)o), ry,
                                                      yo ? p * 2 : kOutOfRange, 0, kNonTemporal);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            s[u] = sn[u];
            xv[u] = xn[u];
        }
    }
}

template <typename T, int TPR>
hipError_t run(const DecodeArgs& a, hipStream_t stream) {
    const int64_t nbh = a.batch * a.H;
    const int64_t blocks = (nbh + kDecThreads / 64 - 1) / (kDecThreads / 64);
    hipLaunchKernelGGL((ssd_decode_kernel<T, TPR>), dim3((unsigned)blocks), dim3(kDecThreads), 0, stream,
                       nbh, a.H, a.P, a.N, a.G, a.state, (const T*)a.x, a.dt, a.A, (const T*)a.B,
                       (const T*)a.C, a.D, a.y, a.y_f32, a.act);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const DecodeArgs& a, hipStream_t stream) {
    const int need = (a.N + 3) / 4;  // 128-bit groups per row
    if (need <= 2) return run<T, 2>(a, stream);
    if (need <= 4) return run<T, 4>(a, stream);
    if (need <= 8) return run<T, 8>(a, stream);
    if (need <= 16) return run<T, 16>(a, stream);
    if (need <= 32) return run<T, 32>(a, stream);
    if (need <= 64) return run<T, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.batch * a.H * a.P == 0) return hipSuccess;
    if (a.dtype == 1) return dispatch<bf16_t>(a, stream);
    return dispatch<float>(a, stream);
}

}  // namespace ssd
