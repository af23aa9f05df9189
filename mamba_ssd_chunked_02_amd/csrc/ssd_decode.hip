// O(1) cached decode step on gfx950: one token per sequence, state updated in
// place ("Compiler-First State Space Duality...", abstract: cached decode with
// a cost independent of the sequence length; recurrence from "Engineering
// hybrid state-space models", section 2):
//   S[p][:] <- exp(dt A) S[p][:] + (dt x[p]) B[:] ;  y[p] = S[p][:].C[:] + D x[p]
//
// The step is bound by HBM bandwidth: the fp32 state is read once and written
// once (the read-D + write-D accounting of the SketchSSM page, Table 4).  Each
// state row (b, h, p) of N floats is handled by TPR lanes with one 128-bit
// non-temporal load and store per lane; the dot product with C is reduced
// across those lanes with shuffles.  No MFMA: one multiply-add per element.
#include "ssd_device.h"

namespace ssd {

namespace {

constexpr int kDecThreads = 256;
constexpr int kRowsPerThread = 4;  // independent rows in flight per lane

template <typename T, int TPR>
__global__ __launch_bounds__(kDecThreads) void ssd_decode_kernel(
    int64_t rows, int H, int P, int N, int G, float* __restrict__ state, const T* __restrict__ x,
    const float* __restrict__ dt, const float* __restrict__ A, const T* __restrict__ B,
    const T* __restrict__ C, const float* __restrict__ D, void* __restrict__ y, int y_f32) {
    constexpr int RPP = kDecThreads / TPR;  // rows per pass of the block
    const int lr = threadIdx.x / TPR, j = threadIdx.x % TPR;
    const int n = 4 * j;
    const int hpg = H / G;
    f32x4 s[kRowsPerThread], bv[kRowsPerThread], cv[kRowsPerThread];
    float xv[kRowsPerThread], a[kRowsPerThread], u[kRowsPerThread];
    int64_t r[kRowsPerThread];
    // issue every load first so each lane keeps several 128-bit loads in flight
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
        r[i] = ((int64_t)blockIdx.x * kRowsPerThread + i) * RPP + lr;
        s[i] = f32x4{};
        bv[i] = f32x4{};
        cv[i] = f32x4{};
        xv[i] = 0.f;
        a[i] = 0.f;
        u[i] = 0.f;
        if (r[i] < rows) {
            const int64_t bh = r[i] / P;
            const int h = (int)(bh % H);
            const int64_t b = bh / H;
            const int g = h / hpg;
            const float d = dt[bh];
            xv[i] = (float)x[r[i]];
            a[i] = __expf(d * A[h]);
            u[i] = d * xv[i];
            if (n < N) {
                s[i] = __builtin_nontemporal_load((const f32x4*)(state + r[i] * N + n));
                bv[i] = Tr<T>::ld4(B + (b * G + g) * N + n);
                cv[i] = Tr<T>::ld4(C + (b * G + g) * N + n);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
        const f32x4 ns = a[i] * s[i] + u[i] * bv[i];
        float part = ns[0] * cv[i][0] + ns[1] * cv[i][1] + ns[2] * cv[i][2] + ns[3] * cv[i][3];
#pragma unroll
        for (int m = TPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, TPR);
        if (r[i] < rows) {
            if (n < N) __builtin_nontemporal_store(ns, (f32x4*)(state + r[i] * N + n));
            if (j == 0) {
                const int h = (int)((r[i] / P) % H);
                const float o = part + D[h] * xv[i];
                if (y_f32) ((float*)y)[r[i]] = o;
                else ((bf16_t*)y)[r[i]] = (bf16_t)o;
            }
        }
    }
}

template <typename T, int TPR>
hipError_t run(const DecodeArgs& a, hipStream_t stream) {
    const int64_t rows = a.batch * a.H * a.P;
    constexpr int per_block = (kDecThreads / TPR) * kRowsPerThread;
    const int64_t blocks = (rows + per_block - 1) / per_block;
    hipLaunchKernelGGL((ssd_decode_kernel<T, TPR>), dim3((unsigned)blocks), dim3(kDecThreads), 0, stream,
                       rows, a.H, a.P, a.N, a.G, a.state, (const T*)a.x, a.dt, a.A, (const T*)a.B,
                       (const T*)a.C, a.D, a.y, a.y_f32);
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
