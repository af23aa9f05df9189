// Causal depthwise conv1d + SiLU on gfx950, the step before the scan in the
// Mamba-2 block ("Engineering Hybrid State-Space Models", section 3,
// architecture figure: width-4 1D convolution and SiLU; section 4: a conv
// state of the last dConv - 1 inputs per channel):
//   v[t, c] = bias[c] + sum_{k<K} w[c, k] xp[t + k, c],  out = v sigmoid(v)
// over xp = [conv state (K-1 rows); x] per sequence.
//
// One multiply-add per tap and element: the prefill is an HBM stream (read x
// once, write the output once), so it is laid out for bandwidth, not MFMA.
// Rows are token-major [rows, C].  A lane owns 8 consecutive channels (one
// 16-byte bf16 vector) and walks a block of kTokBlock tokens; a wave covers
// 512 channels of a row, so every wave load and store is 1 KB (bf16) of
// contiguous row.  Rows go in batches of 8, the next batch in flight while
// the current one is computed; one register array holds the K-1 inputs
// before the batch and the batch's 8 rows, so every tap is a compile-time
// index.  A batch with no sequence start inside takes a path with no
// per-row test; otherwise sequence starts, which are the same for the whole
// wave (rows are uniform), switch to the next sequence's incoming state on a
// scalar branch.
#include <type_traits>

#include "ssd_device.h"

namespace ssd {

namespace {

constexpr int kConvThreads = 256;        // four waves: four token blocks of one channel tile
constexpr int kTokBlock = 64;            // tokens per wave
constexpr int kRowBatch = 8;             // rows in flight per lane
constexpr int kChanPerLane = 8;
constexpr int kChanPerWave = 64 * kChanPerLane;

// Eight channels of one row, widened to fp32.
template <typename T>
__device__ inline f32x8 ld_row8(const T* p) {
    return Tr<T>::widen(Tr<T>::ld8(p));
}

// Eight channels of x with the streaming cache hint (x is read once; only the
// K-1 rows before a block are read again, by that block).
template <typename T>
__device__ inline typename Tr<T>::v8 ld_stream8(const T* p);
template <>
__device__ inline bf16x8 ld_stream8<bf16_t>(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const f32x4*)p));
}
template <>
__device__ inline f32x8 ld_stream8<float>(const float* p) {
    const f32x4 a = __builtin_nontemporal_load((const f32x4*)p);
    const f32x4 b = __builtin_nontemporal_load((const f32x4*)(p + 4));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <typename Y>
__device__ inline void st_row8(Y* p, f32x8 v);
template <>
__device__ inline void st_row8<bf16_t>(bf16_t* p, f32x8 v) {
    __builtin_nontemporal_store(Tr<bf16_t>::narrow(v), (bf16x8*)p);
}
template <>
__device__ inline void st_row8<float>(float* p, f32x8 v) {
    __builtin_nontemporal_store(__builtin_shufflevector(v, v, 0, 1, 2, 3), (f32x4*)p);
    __builtin_nontemporal_store(__builtin_shufflevector(v, v, 4, 5, 6, 7), (f32x4*)(p + 4));
}

// First row, end row of sequence s.  Device offsets are clamped into
// [0, T] with the end no earlier than the start (an offset list that
// decreases or leaves the stream makes that sequence empty), so no row or
// state index derived from them leaves its array.
__device__ inline void seq_rows(const ConvArgs& a, int64_t s, int64_t& r0, int64_t& r1) {
    if (!a.cu) {
        r0 = s * a.L;
        r1 = r0 + a.L;
    } else {
        r0 = min(max((int64_t)a.cu[s], (int64_t)0), a.T);
        r1 = min(max((int64_t)a.cu[s + 1], r0), a.T);
    }
}

// The sequence holding row r (the last sequence starting at or before r that
// is not empty): binary search over cu_seqlens.
__device__ inline int64_t seq_of_row(const ConvArgs& a, int64_t r) {
    if (!a.cu) return r / a.L;
    int64_t lo = 0, hi = a.nseq - 1;  // cu[lo] <= r < cu[nseq]
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (a.cu[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The lane's output part: base pointer of its 8 channels in row 0 and the
// part's row stride (elements).
template <typename Y>
__device__ inline Y* out_base(const ConvArgs& a, int c0, int64_t& stride) {
    int off = 0;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        if (p + 1 < a.nparts && c0 >= off + a.part_ch[p]) off += a.part_ch[p];
        else {
            stride = a.part_ch[p];
            return (Y*)a.out[p] + (c0 - off);
        }
    }
    stride = a.part_ch[2];
    return (Y*)a.out[2] + (c0 - off);
}

template <int K>
struct Taps {
    float w[K][kChanPerLane];
    float b[kChanPerLane];
};

// weight [C, K] row-major: the lane's 8 channels are 8K contiguous floats.
template <int K>
__device__ inline void load_taps(const ConvArgs& a, int c0, Taps<K>& tp) {
    float raw[kChanPerLane * K];
    const f32x4* wp = (const f32x4*)(a.weight + (int64_t)c0 * K);
#pragma unroll
    for (int i = 0; i < 2 * K; ++i) {
        const f32x4 v = wp[i];
        raw[4 * i] = v[0];
        raw[4 * i + 1] = v[1];
        raw[4 * i + 2] = v[2];
        raw[4 * i + 3] = v[3];
    }
#pragma unroll
    for (int e = 0; e < kChanPerLane; ++e)
#pragma unroll
        for (int k = 0; k < K; ++k) tp.w[k][e] = raw[e * K + k];
    if (a.bias) {
        const f32x4 b0 = *(const f32x4*)(a.bias + c0);
        const f32x4 b1 = *(const f32x4*)(a.bias + c0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tp.b[e] = b0[e];
            tp.b[4 + e] = b1[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < kChanPerLane; ++e) tp.b[e] = 0.f;
    }
}

// SiLU with the hardware reciprocal (1 ulp): v / (1 + exp(-v)).  For very
// negative v, exp(-v) overflows to +inf and the result is -0.
__device__ inline float silu_f(float v) { return v * __builtin_amdgcn_rcpf(1.f + __expf(-v)); }

// One output row from inputs h[0..K-1] (h[K-1] the current token).
template <int K, bool SILU>
__device__ inline f32x8 conv_row(const Taps<K>& tp, const f32x8* h) {
    f32x8 v;
#pragma unroll
    for (int e = 0; e < kChanPerLane; ++e) {
        float acc = tp.b[e];
#pragma unroll
        for (int k = 0; k < K; ++k) acc += tp.w[k][e] * h[k][e];
        v[e] = SILU ? silu_f(acc) : acc;
    }
    return v;
}

template <typename T, typename Y, int K, bool SILU>
__global__ __launch_bounds__(kConvThreads) void ssd_conv1d_kernel(ConvArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t r0 = ((int64_t)blockIdx.x * (kConvThreads / 64) + wave) * kTokBlock;
    if (r0 >= a.T) return;
    const int64_t r1 = min(r0 + kTokBlock, a.T);
    const int c0 = blockIdx.y * kChanPerWave + lane * kChanPerLane;
    if (c0 >= a.C) return;
    const T* xb = (const T*)a.x + c0;
    Taps<K> tp;
    load_taps<K>(a, c0, tp);
    int64_t ostride;
    Y* ob = out_base<Y>(a, c0, ostride);

    // hist[0..K-2]: the K-1 inputs before the current batch of rows;
    // hist[K-1+u]: row u of the batch.  Output row u reads hist[u..u+K-1].
    f32x8 hist[K - 1 + kRowBatch];
    int64_t s = seq_of_row(a, r0), sb, se;
    seq_rows(a, s, sb, se);
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
        // padded index of the j-th previous input (negative only when the
        // offsets are invalid and r0 lies outside every sequence)
        const int64_t i = r0 - sb + j;
        hist[j] = i < K - 1 ? ((a.state_in && i >= 0) ? ld_row8((const T*)a.state_in + (s * (K - 1) + i) * a.C + c0)
                                                     : f32x8{})
                            : ld_row8(xb + (r0 + j - (K - 1)) * a.C);
    }

    typename Tr<T>::v8 cur[kRowBatch], nxt[kRowBatch];
    auto load = [&](int64_t rb, typename Tr<T>::v8 (&dst)[kRowBatch]) {
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) dst[u] = ld_stream8<T>(xb + min(rb + u, r1 - 1) * a.C);
    };
    // A batch of rows with no sequence start and no block end inside takes
    // the straight path; the others check every row.
    auto batch = [&](int64_t rb, auto edges) {
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) hist[K - 1 + u] = Tr<T>::widen(cur[u]);
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
            const int64_t r = rb + u;
            if constexpr (decltype(edges)::value) {
                if (r >= r1) break;
                if (r == se) {
                    // the next non-empty sequence starts at row u: the inputs
                    // before it are that sequence's incoming state
                    while (s + 1 < a.nseq) {
                        ++s;
                        seq_rows(a, s, sb, se);
                        if (se > r) break;
                    }
#pragma unroll
                    for (int j = 0; j < K - 1; ++j)
                        hist[u + j] = a.state_in ? ld_row8((const T*)a.state_in + (s * (K - 1) + j) * a.C + c0)
                                                 : f32x8{};
                }
            }
            st_row8<Y>(ob + r * ostride, conv_row<K, SILU>(tp, hist + u));
        }
#pragma unroll
        for (int j = 0; j < K - 1; ++j) hist[j] = hist[kRowBatch + j];
    };
    load(r0, cur);
    for (int64_t rb = r0; rb < r1; rb += kRowBatch) {
        load(min(rb + kRowBatch, r1 - 1), nxt);  // next rows (repeats the last one at the end)
        if (rb + kRowBatch <= r1 && se >= rb + kRowBatch) batch(rb, std::false_type{});
        else batch(rb, std::true_type{});
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) cur[u] = nxt[u];
    }
}

// Final conv state of every sequence: the last K-1 rows of [state_in; x].
// All reads of a thread come before its writes, so state_out may be state_in.
template <typename T, int K>
__global__ __launch_bounds__(kConvThreads) void ssd_conv1d_state_kernel(ConvArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    const int64_t groups = a.C / kChanPerLane;
    if (gid >= a.nseq * groups) return;
    const int64_t s = gid / groups;
    const int c0 = (int)(gid - s * groups) * kChanPerLane;
    int64_t sb, se;
    seq_rows(a, s, sb, se);
    const int64_t len = se - sb;
    typename Tr<T>::v8 v[K - 1];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
        const int64_t i = len + j;  // padded index
        if (i < K - 1)
            v[j] = a.state_in ? Tr<T>::ld8((const T*)a.state_in + (s * (K - 1) + i) * a.C + c0)
                              : Tr<T>::narrow(f32x8{});
        else
            v[j] = Tr<T>::ld8((const T*)a.x + (sb + i - (K - 1)) * a.C + c0);
    }
#pragma unroll
    for (int j = 0; j < K - 1; ++j) Tr<T>::st8((T*)a.state_out + (s * (K - 1) + j) * a.C + c0, v[j]);
}

// Decode step: one token per sequence, state [nseq, K-1, C] shifted in place.
template <typename T, typename Y, int K, bool SILU>
__global__ __launch_bounds__(kConvThreads) void ssd_conv1d_step_kernel(ConvArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    const int64_t groups = a.C / kChanPerLane;
    if (gid >= a.nseq * groups) return;
    const int64_t s = gid / groups;
    const int c0 = (int)(gid - s * groups) * kChanPerLane;
    T* st = (T*)a.state_out + s * (K - 1) * a.C + c0;
    typename Tr<T>::v8 raw[K - 1];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) raw[j] = Tr<T>::ld8(st + j * a.C);
    const typename Tr<T>::v8 xr = Tr<T>::ld8((const T*)a.x + s * a.C + c0);
    Taps<K> tp;
    load_taps<K>(a, c0, tp);
    f32x8 h[K];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) h[j] = Tr<T>::widen(raw[j]);
    h[K - 1] = Tr<T>::widen(xr);
    int64_t ostride;
    Y* ob = out_base<Y>(a, c0, ostride);
    st_row8<Y>(ob + s * ostride, conv_row<K, SILU>(tp, h));
#pragma unroll
    for (int j = 0; j < K - 2; ++j) Tr<T>::st8(st + j * a.C, raw[j + 1]);
    Tr<T>::st8(st + (K - 2) * a.C, xr);
}

template <typename T, typename Y, int K, bool SILU>
hipError_t run_conv(const ConvArgs& a, hipStream_t stream) {
    if (a.T > 0) {
        const int64_t blocks = (a.T + kTokBlock - 1) / kTokBlock;
        const dim3 grid((unsigned)((blocks + kConvThreads / 64 - 1) / (kConvThreads / 64)),
                        (unsigned)((a.C + kChanPerWave - 1) / kChanPerWave));
        hipLaunchKernelGGL((ssd_conv1d_kernel<T, Y, K, SILU>), grid, dim3(kConvThreads), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.state_out && a.nseq > 0) {
        const int64_t n = a.nseq * (a.C / kChanPerLane);
        hipLaunchKernelGGL((ssd_conv1d_state_kernel<T, K>), dim3((unsigned)((n + kConvThreads - 1) / kConvThreads)),
                           dim3(kConvThreads), 0, stream, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename T, typename Y, int K, bool SILU>
hipError_t run_step(const ConvArgs& a, hipStream_t stream) {
    const int64_t n = a.nseq * (a.C / kChanPerLane);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL((ssd_conv1d_step_kernel<T, Y, K, SILU>),
                       dim3((unsigned)((n + kConvThreads - 1) / kConvThreads)), dim3(kConvThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, typename Y, int K>
hipError_t by_activation(const ConvArgs& a, hipStream_t stream, bool step) {
    if (a.silu) return step ? run_step<T, Y, K, true>(a, stream) : run_conv<T, Y, K, true>(a, stream);
    return step ? run_step<T, Y, K, false>(a, stream) : run_conv<T, Y, K, false>(a, stream);
}

template <typename T, typename Y>
hipError_t by_width(const ConvArgs& a, hipStream_t stream, bool step) {
    switch (a.K) {
        case 2: return by_activation<T, Y, 2>(a, stream, step);
        case 3: return by_activation<T, Y, 3>(a, stream, step);
        case 4: return by_activation<T, Y, 4>(a, stream, step);
        default: return hipErrorInvalidValue;
    }
}

hipError_t dispatch_conv(const ConvArgs& a, hipStream_t stream, bool step) {
    if (a.dtype == 1)
        return a.y_f32 ? by_width<bf16_t, float>(a, stream, step) : by_width<bf16_t, bf16_t>(a, stream, step);
    return a.y_f32 ? by_width<float, float>(a, stream, step) : by_width<float, bf16_t>(a, stream, step);
}

}  // namespace

hipError_t launch_conv1d(const ConvArgs& a, hipStream_t stream) { return dispatch_conv(a, stream, false); }

hipError_t launch_conv1d_step(const ConvArgs& a, hipStream_t stream) { return dispatch_conv(a, stream, true); }

}  // namespace ssd
