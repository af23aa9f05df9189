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

// Decode step: eight waves per workgroup, one (sequence, head) state block
// each.  At the 2.7B decode shape (20 480 blocks), in interleaved A/B runs,
// this streamed 1.5% faster than two waves per workgroup and 2.7% faster
// than sixteen.
constexpr int kDecThreads = 512;
// Windowed step: four waves per workgroup, one state block each.
constexpr int kWinThreads = 256;

// dt_activate with the head's bias already loaded (0 when there is none), so
// the kernel can issue that load together with its others.
__device__ inline float dt_activate_b(const DtAct& a, float raw, float bias) {
    if (!a.on) return raw;
    const float v = raw + bias;
    const float sp = v > 20.f ? v : log1pf(expf(v));
    return fminf(fmaxf(sp, a.lo), a.hi);
}
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

// Wave w of block L updates the state block (b, h) = 8L + w: P rows of N
// floats, contiguous.  Lane l owns columns n = 4 (l % TPR) .. +3 of the rows
// p = RPI i + l / TPR, so each wave instruction moves 64 x 16 contiguous bytes
// and B, C, dt, A are loaded once per lane.  Rows go in batches of kBatch
// instructions; the next batch is loaded before the current one is stored,
// and every lane issues every state store (rows past P and columns past N get
// an out-of-range offset), so the wait for a batch never includes the
// previous batch's stores.  The block's x (P <= 128 values) is loaded once
// into the wave's LDS row and its y collected there, then stored with one
// coalesced store per 64 rows: per batch the wave issues only the state's
// loads and stores to memory.  The wave index is made uniform so the buffer
// descriptors are scalar.
template <typename T, int TPR>
__global__ __launch_bounds__(kDecThreads) void ssd_decode_kernel(
    int64_t nbh, int H, int P, int N, int G, float* __restrict__ state, const T* __restrict__ x,
    const float* __restrict__ dt, const float* __restrict__ A, const T* __restrict__ B,
    const T* __restrict__ C, const float* __restrict__ D, void* __restrict__ y, int y_f32, DtAct act) {
    constexpr int RPI = 64 / TPR;  // rows per wave instruction
    constexpr int RPB = RPI * kBatch;  // rows per batch
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = (int64_t)blockIdx.x * (kDecThreads / 64) + wave;
    if (bh >= nbh) return;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int j = lane % TPR, rsub = lane / TPR;
    const bool nv = 4 * j < N;
    const int n = nv ? 4 * j : N - 4;
    float* sb = state + bh * P * N;
    const T* xb = x + bh * P;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(sb, (uint32_t)(P * N * sizeof(float)));
    const __amdgpu_buffer_rsrc_t ry =
        buffer_rsrc((char*)y + bh * P * (y_f32 ? 4 : 2), (uint32_t)(P * (y_f32 ? 4 : 2)));
    __shared__ float xsh[kDecThreads / 64][128];
    __shared__ float ysh[kDecThreads / 64][128];
    float* xs = xsh[wave];
    float* ys = ysh[wave];
    const float xl0 = (float)xb[min(lane, P - 1)];
    const float xl1 = (float)xb[min(lane + 64, P - 1)];
    f32x4 s[kBatch], sn[kBatch];
    auto load = [&](int p0, f32x4 (&dst)[kBatch]) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int p = min(p0 + u * RPI + rsub, P - 1);
            dst[u] = __builtin_nontemporal_load((const f32x4*)(sb + (int64_t)p * N + n));
        }
    };
    // the first state rows go out first; then every per-step operand, with
    // no load waiting on another (B, C columns clamped in range, masked after)
    load(0, s);
    xs[lane] = xl0;
    xs[lane + 64] = xl1;
    const float draw = dt[bh], Ah = A[h], Dh = D[h];
    const float braw = *(act.bias ? act.bias + h : A + h);
    const typename Tr<T>::v4 bq = Tr<T>::ld4raw(B + (b * G + g) * N + n);
    const typename Tr<T>::v4 cq = Tr<T>::ld4raw(C + (b * G + g) * N + n);
    const float d = dt_activate_b(act, draw, act.bias ? braw : 0.f);
    const float a = __expf(d * Ah);
    const f32x4 bv = nv ? Tr<T>::widen4(bq) : f32x4{};
    const f32x4 cv = nv ? Tr<T>::widen4(cq) : f32x4{};
    // xs is read across lanes below: keep its writes ahead of those reads
    __builtin_amdgcn_wave_barrier();
    for (int p0 = 0; p0 < P; p0 += RPB) {
        load(min(p0 + RPB, P - 1), sn);  // next batch (repeats the last rows at the end)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int p = p0 + u * RPI + rsub;
            const float xp = xs[min(p, P - 1)];
            const f32x4 ns = a * s[u] + (d * xp) * bv;
            const float tot = group_sum<TPR>(ns[0] * cv[0] + ns[1] * cv[1] + ns[2] * cv[2] + ns[3] * cv[3]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ns), rs,
                                                   (p < P && nv) ? (p * N + n) * 4 : kOutOfRange, 0, kNonTemporal);
            const float o = tot + Dh * xp;
            if (j == TPR - 1 && p < P) ys[p] = o;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) s[u] = sn[u];
    }
    // ys rows were written by other lanes
    __builtin_amdgcn_wave_barrier();
    const float y0 = ys[min(lane, P - 1)], y1 = ys[min(lane + 64, P - 1)];
    if (y_f32) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, y0), ry, lane < P ? lane * 4 : kOutOfRange,
                                              0, kNonTemporal);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, y1), ry,
                                              lane + 64 < P ? (lane + 64) * 4 : kOutOfRange, 0, kNonTemporal);
    } else {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16_t)y0), ry,
                                              lane < P ? lane * 2 : kOutOfRange, 0, kNonTemporal);
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16_t)y1), ry,
                                              lane + 64 < P ? (lane + 64) * 2 : kOutOfRange, 0, kNonTemporal);
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

// ------------------------------------------------------------------ windowed decode
// Exact windowed update ("SketchSSM: Write to the Full State...", Fig. 3(a),
// Fig. 4 and Table 4: the full state S0 is read every step and written once
// per window of W tokens).  The window holds the tokens since the last flush
// (slots 0..t, the current token in slot t).  With cs_s = sum_{u<=s} dt_u A,
//   y_t = exp(cs_t) (S0 C_t) + sum_{s<=t} exp(cs_t - cs_s) dt_s (B_s . C_t) x_s + D x_t
// and on a flush step
//   S0 <- exp(cs_t) S0 + sum_{s<=t} exp(cs_t - cs_s) dt_s x_s (outer) B_s.
// Same traversal as the decode step: one wave per (sequence, head), lanes
// own 4 columns of a row.  Per-token scalars of the window (decay sums,
// weights, B_s . C_t) are wave-uniform; the window's x rows sit in LDS.
constexpr int kWinMax = 16;
constexpr int kWinPitch = kWinMax + 4;  // floats per x row of the window in LDS (16-byte aligned rows)

// Every step streams the state block once for y (and, with FLUSH, writes the
// new state in the same pass), with the streaming cache hint on its loads.
// The prologue reduces the window to per-lane constants: C_t, the decay
// exp(cs_t), y's intra-window part per row (LDS) and, with FLUSH,
// u_s = exp(cs_t - cs_s) dt_s B_s and the window's x rows (LDS, one row of W
// values per p).  Rows are streamed as in the decode step: batches of kBatch
// 128-bit loads, the next batch in flight while the current one is used.
// Each row's y replaces its intra-window part in LDS, and the block's y goes
// out at the end with one coalesced store per 64 rows.
template <typename T, int TPR, bool FLUSH>
__global__ __launch_bounds__(kWinThreads, FLUSH ? 2 : (sizeof(T) == 2 ? 4 : 3)) void ssd_decode_window_kernel(
    int64_t nbh, int H, int P, int N, int G, int W, int t, float* __restrict__ state,
    const T* __restrict__ xw, const float* __restrict__ dtw, const float* __restrict__ A,
    const T* __restrict__ Bw, const T* __restrict__ Cw, const float* __restrict__ D, void* __restrict__ y,
    int y_f32, DtAct act) {
    constexpr int RPI = 64 / TPR;      // rows per wave instruction
    constexpr int RPB = RPI * kBatch;  // rows per batch
    // x of the window, transposed: row p holds x_s[p] for s = 0..15 (zero past t).
    // The flush step reads a row with 128-bit loads (16-byte aligned pitch);
    // the other step only reads it once per lane, with an odd pitch that keeps
    // the transposing writes free of bank conflicts.
    constexpr int XPITCH = FLUSH ? kWinPitch : kWinMax + 1;
    __shared__ __align__(16) float yis[kWinThreads / 64][128];
    __shared__ __align__(16) float xts[kWinThreads / 64][128][XPITCH];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t bh = (int64_t)blockIdx.x * (kWinThreads / 64) + wave;
    if (bh >= nbh) return;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int j = lane % TPR, rsub = lane / TPR;
    const bool nv = 4 * j < N;
    const int n = nv ? 4 * j : N - 4;
    float* yi = yis[wave];
    float* sb = state + bh * P * N;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(sb, (uint32_t)(P * N * sizeof(float)));
    const __amdgpu_buffer_rsrc_t ry =
        buffer_rsrc((char*)y + bh * P * (y_f32 ? 4 : 2), (uint32_t)(P * (y_f32 ? 4 : 2)));
    f32x4 s0[kBatch], sn[kBatch];
    auto load = [&](int p0, f32x4 (&dst)[kBatch]) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int p = min(p0 + u * RPI + rsub, P - 1);
            dst[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (p * N + n) * 4, 0,
                                                                                   kNonTemporal));
        }
    };
    // the first state rows go out first: their latency covers the window set-up
    load(0, s0);
    // Window inputs: every slot is loaded (slots past t repeat slot t and are
    // masked afterwards), so the loads issue back to back with no branch.
    // lane s (< 16) takes window slot s's dt
    const float rawl = dtw[(b * W + min(lane & (kWinMax - 1), t)) * H + h];
    typename Tr<T>::v4 bq[kWinMax];
#pragma unroll
    for (int s = 0; s < kWinMax; ++s) bq[s] = Tr<T>::ld4raw(Bw + ((b * W + min(s, t)) * G + g) * N + n);
    const typename Tr<T>::v4 cq = Tr<T>::ld4raw(Cw + ((b * W + t) * G + g) * N + n);
    // x of the window: P/8 chunks of 8 values per slot, at most 4 per lane
    const int cpr = P >> 3, nch = kWinMax * cpr;
    typename Tr<T>::v8 xq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = min(lane + 64 * i, nch - 1);
        const int sl = c / cpr, q = c - sl * cpr;
        xq[i] = Tr<T>::ld8(xw + ((b * W + min(sl, t)) * H + h) * P + 8 * q);
    }
    const f32x4 ct = nv ? Tr<T>::widen4(cq) : f32x4{};
    // window scalars, one slot per lane: dt, decay sums cs_s (a prefix scan
    // over the lanes), weights w_s = exp(cs_t - cs_s) dt_s; zero past t
    const float dl = lane <= t ? dt_activate(act, rawl, h) : 0.f;
    const float csl = wave_inclusive_scan(dl * A[h]);
    const float cst = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, csl), t));
    const float wl = lane <= t ? __expf(cst - csl) * dl : 0.f;
    float k[kWinMax];
    f32x4 us[FLUSH ? kWinMax : 1];
#pragma unroll
    for (int s = 0; s < kWinMax; ++s) {
        const f32x4 bv = nv ? Tr<T>::widen4(bq[s]) : f32x4{};
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s));
        const float dot = group_sum<TPR>(bv[0] * ct[0] + bv[1] * ct[1] + bv[2] * ct[2] + bv[3] * ct[3]);
        // the group's last lane holds the dot product; it is the same for every row
        k[s] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dot), TPR - 1)) * w;
        if constexpr (FLUSH) us[s] = w * bv;
    }
    const float Dh = D[h];
    float(*xt)[XPITCH] = xts[wave];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
            const int sl = c / cpr, q = c - sl * cpr;
            const f32x8 v = Tr<T>::widen(xq[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) xt[8 * q + e][sl] = sl <= t ? v[e] : 0.f;
        }
    }
    __builtin_amdgcn_wave_barrier();
    // per row p: y's window part sum_s k_s x_s[p] + D x_t[p]
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int p = lane + 64 * m;
        if (p < P) {
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < kWinMax; ++s) acc += k[s] * xt[p][s];
            yi[p] = acc + Dh * xt[p][t];
        }
    }
    // rows written by one lane are read by others below (same wave, in-order LDS)
    __builtin_amdgcn_wave_barrier();
    const float et = __expf(cst);
    for (int p0 = 0; p0 < P; p0 += RPB) {
        load(min(p0 + RPB, P - 1), sn);  // next batch (repeats the last rows at the end)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int p = p0 + u * RPI + rsub;
            const int pc = min(p, P - 1);
            const float tot = group_sum<TPR>(s0[u][0] * ct[0] + s0[u][1] * ct[1] + s0[u][2] * ct[2] + s0[u][3] * ct[3]);
            const float o = et * tot + yi[pc];
            if (j == TPR - 1 && p < P) yi[p] = o;
            if constexpr (FLUSH) {
                const f32x4* xr = (const f32x4*)xt[pc];
                f32x4 ns = et * s0[u];
#pragma unroll
                for (int q = 0; q < kWinMax / 4; ++q) {
                    const f32x4 xq = xr[q];
                    ns += xq[0] * us[4 * q] + xq[1] * us[4 * q + 1] + xq[2] * us[4 * q + 2] + xq[3] * us[4 * q + 3];
                }
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ns), rs,
                                                       (p < P && nv) ? (p * N + n) * 4 : kOutOfRange, 0,
                                                       kNonTemporal);
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) s0[u] = sn[u];
    }
    __builtin_amdgcn_wave_barrier();
    const float y0 = yi[min(lane, P - 1)], y1 = yi[min(lane + 64, P - 1)];
    if (y_f32) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, y0), ry, lane < P ? lane * 4 : kOutOfRange,
                                              0, kNonTemporal);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, y1), ry,
                                              lane + 64 < P ? (lane + 64) * 4 : kOutOfRange, 0, kNonTemporal);
    } else {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16_t)y0), ry,
                                              lane < P ? lane * 2 : kOutOfRange, 0, kNonTemporal);
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16_t)y1), ry,
                                              lane + 64 < P ? (lane + 64) * 2 : kOutOfRange, 0, kNonTemporal);
    }
}

template <typename T, int TPR>
hipError_t run_window(const WindowArgs& a, hipStream_t stream) {
    const int64_t nbh = a.batch * a.H;
    const int64_t blocks = (nbh + kWinThreads / 64 - 1) / (kWinThreads / 64);
    auto* k = a.flush ? ssd_decode_window_kernel<T, TPR, true> : ssd_decode_window_kernel<T, TPR, false>;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kWinThreads), 0, stream, nbh, a.H, a.P, a.N, a.G, a.W, a.t,
                       a.state, (const T*)a.x, a.dt, a.A, (const T*)a.B, (const T*)a.C, a.D, a.y, a.y_f32, a.act);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_window(const WindowArgs& a, hipStream_t stream) {
    const int need = (a.N + 3) / 4;
    if (need <= 2) return run_window<T, 2>(a, stream);
    if (need <= 4) return run_window<T, 4>(a, stream);
    if (need <= 8) return run_window<T, 8>(a, stream);
    if (need <= 16) return run_window<T, 16>(a, stream);
    if (need <= 32) return run_window<T, 32>(a, stream);
    if (need <= 64) return run_window<T, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_window(const WindowArgs& a, hipStream_t stream) {
    if (a.batch * a.H * a.P == 0) return hipSuccess;
    if (a.dtype == 1) return dispatch_window<bf16_t>(a, stream);
    return dispatch_window<float>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.batch * a.H * a.P == 0) return hipSuccess;
    if (a.dtype == 1) return dispatch<bf16_t>(a, stream);
    return dispatch<float>(a, stream);
}

}  // namespace ssd
