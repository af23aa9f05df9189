// Chunked SSD prefill on gfx950 (CDNA4).
//
// The scan computes, per sequence and head, S_t = exp(dt_t A) S_{t-1} +
// dt_t x_t (outer) B_t and y_t = S_t C_t + D x_t ("Engineering hybrid
// state-space models", section 2), regrouped over chunks of Q tokens as the
// SSD duality allows (same section: Y = (M o CB^T) X with a 1-semiseparable
// decay mask M; "Compiler-First State Space Duality...", abstract: fixed-size
// chunking, einsum-dominated compute).  With cs the per-chunk inclusive sum
// of dt*A:
//   chunk state   S_c = sum_k exp(cs_last - cs_k) dt_k x_k (outer) B_k
//   passing       h_{c+1} = exp(cs_last) h_c + S_c
//   chunk output  y_t = exp(cs_t) C_t h_c + sum_{k<=t} (C_t.B_k) exp(cs_t-cs_k) dt_k x_k + D x_t
//
// Kernels (queued in this order on one stream):
//   plan           packed batches only: chunk / segment / sequence tables
//   cumsum         cs and dt per (chunk, head), wave64 DPP prefix scan
//   cb             C.B^T per (chunk, group) on MFMA, and B^T per chunk
//   chunk_state    own state of every segment that is not a sequence's last
//   state_passing  sequential over segments, parallel over (head, P, N)
//   chunk_scan     per (segment, head): walks the segment's chunks carrying
//                  the fp32 state in registers, writes y and final states
// The contractions run on 32x32 MFMA tiles (bf16 inputs: 32x32x16 bf16; fp32
// inputs: 32x32x2 f32), fp32 accumulation everywhere.
#include "ssd_device.h"

namespace ssd {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------ plan
// One workgroup.  Sequence s covers rows [cu[s], cu[s+1]); an offset list that
// is decreasing or leaves [0, T] makes that sequence empty, so no later kernel
// can address memory outside the token arrays.
__global__ __launch_bounds__(kThreads) void ssd_plan_kernel(Plan pl) {
    __shared__ int s_a[kThreads], s_b[kThreads], s_c[kThreads];
    __shared__ int s_carry[3];
    const int tid = threadIdx.x;
    if (tid == 0) s_carry[0] = s_carry[1] = s_carry[2] = 0;
    __syncthreads();
    for (int base = 0; base < pl.nseq; base += kThreads) {
        const int s = base + tid;
        int nc = 0, ns = 0, nsl = 0;
        if (s < pl.nseq) {
            const int a = pl.cu[s], b = pl.cu[s + 1];
            const int len = (a >= 0 && b >= a && (int64_t)b <= pl.T) ? b - a : 0;
            nc = (len + pl.Q - 1) / pl.Q;
            ns = (nc + pl.cps - 1) / pl.cps;
            nsl = ns > 0 ? ns - 1 : 0;
        }
        s_a[tid] = nc;
        s_b[tid] = ns;
        s_c[tid] = nsl;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {  // inclusive block scan
            int va = 0, vb = 0, vc = 0;
            if (tid >= off) { va = s_a[tid - off]; vb = s_b[tid - off]; vc = s_c[tid - off]; }
            __syncthreads();
            s_a[tid] += va;
            s_b[tid] += vb;
            s_c[tid] += vc;
            __syncthreads();
        }
        if (s < pl.nseq) {
            int4 e;
            e.x = s_carry[0] + s_a[tid] - nc;
            e.y = nc;
            e.z = s_carry[1] + s_b[tid] - ns;
            e.w = s_carry[2] + s_c[tid] - nsl;
            ((int4*)pl.seq_tab)[s] = e;
        }
        __syncthreads();
        if (tid == kThreads - 1) {
            s_carry[0] += s_a[tid];
            s_carry[1] += s_b[tid];
            s_carry[2] += s_c[tid];
        }
        __syncthreads();
    }
    int nchunks = s_carry[0], nsegs = s_carry[1];
    if (nchunks > pl.nchunk_ub || nsegs > pl.nseg_ub) {
        // the offsets describe more tokens than the stream holds (overlapping
        // sequences): treat every sequence as empty rather than index past the
        // workspace regions sized for T tokens
        for (int s = tid; s < pl.nseq; s += kThreads) ((int4*)pl.seq_tab)[s] = make_int4(0, 0, 0, 0);
        nchunks = 0;
        nsegs = 0;
    }
    // chunk and segment entries; the owning sequence is the last one whose
    // first index is <= the entry (empty sequences share it with a successor)
    for (int k = tid; k < pl.nchunk_ub; k += kThreads) {
        int4 e = make_int4(-1, 0, 0, 0);
        if (k < nchunks) {
            int lo = 0, hi = pl.nseq - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (((const int4*)pl.seq_tab)[mid].x <= k) lo = mid; else hi = mid - 1;
            }
            const int4 q = ((const int4*)pl.seq_tab)[lo];
            const int c = k - q.x;
            const int a = pl.cu[lo];
            const int len = pl.cu[lo + 1] - a;
            e = make_int4(lo, a + c * pl.Q, min(pl.Q, len - c * pl.Q), q.z + c / pl.cps);
        }
        ((int4*)pl.chunk_tab)[k] = e;
    }
    for (int j = tid; j < pl.nseg_ub; j += kThreads) {
        int4 e = make_int4(-1, 0, 0, 0);
        if (j < nsegs) {
            int lo = 0, hi = pl.nseq - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (((const int4*)pl.seq_tab)[mid].z <= j) lo = mid; else hi = mid - 1;
            }
            const int4 q = ((const int4*)pl.seq_tab)[lo];
            const int i = j - q.z;
            e = make_int4(lo, q.x + i * pl.cps, min(pl.cps, q.y - i * pl.cps), i);
        }
        ((int4*)pl.seg_tab)[j] = e;
    }
}

// ------------------------------------------------------------------ cumsum
// grid (chunks, ceil(H/4)); wave w of the block handles head 4*blockIdx.y + w.
// cs[q] = sum_{s<=q} dt_s A_h inside the chunk; positions past the chunk end
// repeat the last value (dt = 0 there), dtc holds dt with zeros past the end.
__global__ __launch_bounds__(kThreads) void ssd_cumsum_kernel(Plan pl, const float* __restrict__ dt,
                                                               const float* __restrict__ A,
                                                               float* __restrict__ cs,
                                                               float* __restrict__ dtc) {
    const int k = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = blockIdx.y * 4 + wave;
    const ChunkDesc cd = chunk_desc(pl, k);
    if (cd.seq < 0 || h >= pl.H) return;
    const int Q = pl.Q, H = pl.H;
    const float a = A[h];
    const int ppl = Q >= 64 ? Q / 64 : 1;  // consecutive positions per lane
    float d[4];
    float own = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d[i] = 0.f;
        const int q = lane * ppl + i;
        if (i < ppl && q < cd.len) d[i] = dt[(cd.row0 + q) * H + h];
        own += d[i] * a;
    }
    float run = wave_inclusive_scan(own) - own;  // exclusive prefix of lane totals
    float* csr = cs + ((size_t)k * H + h) * Q;
    float* dtr = dtc + ((size_t)k * H + h) * Q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = lane * ppl + i;
        if (i < ppl && q < Q) {
            run += d[i] * a;
            csr[q] = run;
            dtr[q] = d[i];
        }
    }
}

// ------------------------------------------------------------------ C.B^T
// grid (chunks, G, Q/32), one wave: row tile ti of cb = C B^T for column
// tiles kj <= ti (the causal part the chunk scan reads), plus columns
// [32 ti, 32 ti + 32) of B^T.  Rows/columns past the chunk end are zero.
template <typename T>
__global__ __launch_bounds__(64) void ssd_cb_kernel(Plan pl, const T* __restrict__ B,
                                                    const T* __restrict__ C, float* __restrict__ cb,
                                                    T* __restrict__ bt) {
    const int k = blockIdx.x, g = blockIdx.y, ti = blockIdx.z;
    const ChunkDesc cd = chunk_desc(pl, k);
    if (cd.seq < 0) return;
    const int Q = pl.Q, N = pl.N, G = pl.G;
    const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;
    typedef typename Tr<T>::v8 v8;
    const int t = 32 * ti + col;
    const bool tv = t < cd.len;
    const T* crow = C + ((cd.row0 + t) * G + g) * N;
    float* out = cb + ((size_t)k * G + g) * Q * Q;
    for (int kj = 0; kj <= ti; ++kj) {
        f32x16 acc = {};
        const int kk = 32 * kj + col;
        const bool kv = kk < cd.len;
        const T* brow = B + ((cd.row0 + kk) * G + g) * N;
        for (int n0 = 0; n0 < N; n0 += 16) {
            const int n = n0 + 8 * half;
            v8 a = {}, b = {};
            if (tv && n < N) a = Tr<T>::ld8(crow + n);
            if (kv && n < N) b = Tr<T>::ld8(brow + n);
            mma16(acc, a, b);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) out[(size_t)(32 * ti + acc_row(v, lane)) * Q + 32 * kj + col] = acc[v];
    }
    T* btk = bt + ((size_t)k * G + g) * N * Q;
    for (int idx = lane; idx < 32 * (N / 8); idx += 64) {
        const int kk = idx & 31, ng = idx >> 5;
        const int kr = 32 * ti + kk;
        v8 b = {};
        if (kr < cd.len) b = Tr<T>::ld8(B + ((cd.row0 + kr) * G + g) * N + 8 * ng);
#pragma unroll
        for (int i = 0; i < 8; ++i) btk[(size_t)(8 * ng + i) * Q + kr] = b[i];
    }
}

// ------------------------------------------------------------------ x staging
// Operand precision.  x, B and C are exact in their dtype.  A product with a
// per-token fp32 factor (x * w for the state update) and the fp32 state used
// as an operand are not: for bf16 operands each is carried as a hi/lo pair of
// bf16 values (hi = rn(v), lo = rn(v - hi)) and contracted with two MFMAs, so
// the operand error is ~2^-16 relative instead of 2^-8.  fp32 operands need
// no split.
template <typename T>
struct Split {
    static constexpr bool on = !__is_same(T, float);
};

// Writes the chunk's x tile of head h transposed into LDS (rows p, PT of them,
// zero past P; k contiguous, pitch LP; tokens past the chunk end are zero):
//   RAW:    xr[p][k] = x[k][p]                     (exact)
//   WITH_W: xh[p][k] + xl[p][k] = x[k][p] * w[k]   (hi/lo pair; xl unused for fp32)
// Each thread owns 8 tokens x 8 columns per step.
template <typename T, int PT, bool RAW, bool WITH_W>
__device__ inline void stage_x(const T* __restrict__ x, const ChunkDesc& cd, int H, int P, int h,
                               int Q, T* xr, const float* w, T* xh, T* xl, int LP) {
    typedef typename Tr<T>::v8 v8;
    constexpr int NPB = PT / 8;
    const int nunits = (Q / 8) * NPB;
    for (int u = threadIdx.x; u < nunits; u += kThreads) {
        const int pb = u % NPB, kb = u / NPB;
        const int p0 = pb * 8, k0 = kb * 8;
        v8 raw[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            raw[r] = v8{};
            const int kk = k0 + r;
            if (kk < cd.len && p0 < P) raw[r] = Tr<T>::ld8(x + ((cd.row0 + kk) * H + h) * P + p0);
        }
        float ws[8];
        if (WITH_W) {
#pragma unroll
            for (int r = 0; r < 8; ++r) ws[r] = w[k0 + r];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (RAW) {
                v8 o;
#pragma unroll
                for (int r = 0; r < 8; ++r) o[r] = raw[r][i];
                Tr<T>::st8(xr + (p0 + i) * LP + k0, o);
            }
            if (WITH_W) {
                f32x8 o;
#pragma unroll
                for (int r = 0; r < 8; ++r) o[r] = (float)raw[r][i] * ws[r];
                const v8 hi = Tr<T>::narrow(o);
                Tr<T>::st8(xh + (p0 + i) * LP + k0, hi);
                if (Split<T>::on) Tr<T>::st8(xl + (p0 + i) * LP + k0, Tr<T>::narrow(o - Tr<T>::widen(hi)));
            }
        }
    }
}

// State tiles: the (N x P) transposed state S^T is NT/32 x PT/32 tiles of 32x32;
// wave w owns tiles w*TPW .. w*TPW+TPW-1 (index u -> nt = u / NPT, pt = u % NPT).
// Accumulator register v of tile (nt, pt) holds S[p = 32pt + lane%32]
// [n = 32nt + 8(v/4) + 4(lane/32) + v%4].

// S^T(tile) <- dec * S^T + B^T(rows n) . xw(cols p) over the chunk's Q tokens,
// xw given as the hi/lo pair xh/xl in LDS (pitch LP).
template <typename T>
__device__ inline void state_update_tile(f32x16& st, float dec, const T* __restrict__ btk, int n, int N,
                                         int Q, const T* xh, const T* xl, int p, int LP, int half) {
    typedef typename Tr<T>::v8 v8;
    st *= dec;
    for (int k0 = 0; k0 < Q; k0 += 16) {
        v8 a = {};
        if (n < N) a = Tr<T>::ld8(btk + (size_t)n * Q + k0 + 8 * half);
        mma16(st, a, Tr<T>::ld8(xh + p * LP + k0 + 8 * half));
        if (Split<T>::on) mma16(st, a, Tr<T>::ld8(xl + p * LP + k0 + 8 * half));
    }
}

// ------------------------------------------------------------------ chunk_state
// grid (segments, H).  For every segment that is not the last of its sequence,
// the state that the segment alone produces from a zero state:
//   S <- exp(cs_last) S + B^T diag(exp(cs_last - cs_k) dt_k) X   per chunk.
template <typename T, int PT, int NT>
__global__ __launch_bounds__(kThreads) void ssd_chunk_state_kernel(
    Plan pl, const T* __restrict__ x, const float* __restrict__ cs, const float* __restrict__ dtc,
    const T* __restrict__ bt, float* __restrict__ sbuf) {
    extern __shared__ __align__(16) char smem[];
    const SegDesc sd = seg_desc(pl, blockIdx.x);
    const int h = blockIdx.y;
    if (sd.seq < 0 || sd.last) return;
    constexpr int NPT = PT / 32, NNT = NT / 32, NTILE = NPT * NNT, TPW = (NTILE + 3) / 4;
    const int Q = pl.Q, P = pl.P, N = pl.N, H = pl.H, G = pl.G;
    const int g = h / pl.hpg;
    const int LP = Q + 8;
    T* xh = (T*)smem;
    T* xl = xh + PT * LP;
    float* wl = (float*)(xl + (Split<T>::on ? PT * LP : 0));
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    f32x16 st[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) st[i] = f32x16{};
    for (int c = 0; c < sd.nchunks; ++c) {
        const int kc = sd.chunk0 + c;
        const ChunkDesc cd = chunk_desc(pl, kc);
        const float* csk = cs + ((size_t)kc * H + h) * Q;
        const float* dtk = dtc + ((size_t)kc * H + h) * Q;
        const float cl = csk[Q - 1];
        for (int q = threadIdx.x; q < Q; q += kThreads) wl[q] = __expf(cl - csk[q]) * dtk[q];
        __syncthreads();
        stage_x<T, PT, false, true>(x, cd, H, P, h, Q, nullptr, wl, xh, xl, LP);
        __syncthreads();
        const float dec = __expf(cl);
        const T* btk = bt + ((size_t)kc * G + g) * N * Q;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int u = wave * TPW + i;
            if (u < NTILE)
                state_update_tile<T>(st[i], dec, btk, 32 * (u / NPT) + col, N, Q, xh, xl,
                                     32 * (u % NPT) + col, LP, half);
        }
        __syncthreads();
    }
    float* out = sbuf + ((size_t)sd.slot_out * H + h) * P * N;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int u = wave * TPW + i;
        if (u < NTILE) {
            const int nt = u / NPT, pt = u % NPT;
            const int p = 32 * pt + col;
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                const int n = 32 * nt + 8 * vg + 4 * half;
                if (p < P && n < N)
                    *(f32x4*)(out + (size_t)p * N + n) =
                        f32x4{st[i][4 * vg], st[i][4 * vg + 1], st[i][4 * vg + 2], st[i][4 * vg + 3]};
            }
        }
    }
}

// ------------------------------------------------------------------ state_passing
// grid (ceil(P*N/4/256), H, nseq).  Sequential over the segments of one
// sequence, four (p, n) elements per thread, fp32:
//   h <- exp(sum of cs_last over segment j) h + S_j;  slot_j <- h, the state
//   entering segment j+1 (S_j is what slot_j held before).
// A sequence without tokens gets final = initial state here.
__global__ __launch_bounds__(kThreads) void ssd_state_passing_kernel(
    Plan pl, const float* __restrict__ cs, float* __restrict__ sbuf, const float* __restrict__ init,
    float* __restrict__ fin) {
    const int s = blockIdx.z, h = blockIdx.y;
    const int PN = pl.P * pl.N;
    const int e = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (e >= PN) return;
    const int4 si = seq_info(pl, s);
    const size_t off = ((size_t)s * pl.H + h) * PN + e;
    f32x4 st = {};
    if (init) st = *(const f32x4*)(init + off);
    if (si.y == 0) {
        if (fin) *(f32x4*)(fin + off) = st;
        return;
    }
    const int nseg = (si.y + pl.cps - 1) / pl.cps;
    for (int j = 0; j + 1 < nseg; ++j) {
        float lsum = 0.f;
        const int c0 = si.x + j * pl.cps;
        for (int c = 0; c < pl.cps; ++c) lsum += cs[((size_t)(c0 + c) * pl.H + h) * pl.Q + pl.Q - 1];
        const float dec = __expf(lsum);
        float* slot = sbuf + ((size_t)(si.w + j) * pl.H + h) * PN + e;
        const f32x4 own = *(const f32x4*)slot;
        st = dec * st + own;
        *(f32x4*)slot = st;
    }
}

// ------------------------------------------------------------------ chunk_scan
// grid (segments, H).  For each chunk of the segment, in order:
//   Y^T[p][t]  = exp(cs_t) sum_n S[p][n] C[t][n]                        (state term)
//              + sum_{k<=t} x[k][p] cb[t][k] exp(cs_t - cs_k) dt_k        (causal intra-chunk term)
//   y[t][p]    = Y^T[p][t] + D x[t][p]                                   (written in fp32 or bf16)
//   S^T       <- exp(cs_last) S^T + B^T (x dt exp(cs_last - cs_k))       (carry to the next chunk)
// The state lives in fp32 accumulators; its operand copy sits in LDS as a
// hi/lo pair sh/sl[p][n].  The decay-weighted mask is built in registers from
// cb, one bf16 rounding per element.  t-tiles are dealt to waves in snake
// order so the causal work balances.
template <typename T, int PT, int NT>
__global__ __launch_bounds__(kThreads) void ssd_chunk_scan_kernel(
    Plan pl, const T* __restrict__ x, const float* __restrict__ cs, const float* __restrict__ dtc,
    const T* __restrict__ Cm, const float* __restrict__ cb, const T* __restrict__ bt,
    const float* __restrict__ D, const float* __restrict__ init, const float* __restrict__ sbuf,
    void* __restrict__ yv, int y_f32, float* __restrict__ fin) {
    extern __shared__ __align__(16) char smem[];
    const SegDesc sd = seg_desc(pl, blockIdx.x);
    const int h = blockIdx.y;
    if (sd.seq < 0) return;
    constexpr bool SP = Split<T>::on;
    constexpr int NPT = PT / 32, NNT = NT / 32, NTILE = NPT * NNT, TPW = (NTILE + 3) / 4;
    typedef typename Tr<T>::v8 v8;
    const int Q = pl.Q, P = pl.P, N = pl.N, H = pl.H, G = pl.G;
    const int g = h / pl.hpg;
    const int LP = Q + 8, LS = NT + 8;
    T* xr = (T*)smem;
    T* xh = xr + PT * LP;
    T* xl = xh + PT * LP;
    T* sh = xl + (SP ? PT * LP : 0);
    T* sl = sh + PT * LS;
    float* csl = (float*)(sl + (SP ? PT * LS : 0));
    float* dtl = csl + Q;
    float* wl = dtl + Q;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    const bool need_final = sd.last && fin != nullptr;
    const float Dh = D[h];

    // entering state: previous segment's passed state, else the initial state
    const float* src = nullptr;
    if (sd.slot_in >= 0) src = sbuf + ((size_t)sd.slot_in * H + h) * P * N;
    else if (init) src = init + ((size_t)sd.seq * H + h) * P * N;
    bool zero_state = (src == nullptr);
    f32x16 st[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        st[i] = f32x16{};
        const int u = wave * TPW + i;
        if (src && u < NTILE) {
            const int nt = u / NPT, pt = u % NPT;
            const int p = 32 * pt + col;
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                const int n = 32 * nt + 8 * vg + 4 * half;
                if (p < P && n < N) {
                    const f32x4 v = *(const f32x4*)(src + (size_t)p * N + n);
                    st[i][4 * vg] = v[0];
                    st[i][4 * vg + 1] = v[1];
                    st[i][4 * vg + 2] = v[2];
                    st[i][4 * vg + 3] = v[3];
                }
            }
        }
    }
    auto state_to_lds = [&]() {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int u = wave * TPW + i;
            if (u < NTILE) {
                const int nt = u / NPT, pt = u % NPT;
                const int p = 32 * pt + col;
#pragma unroll
                for (int vg = 0; vg < 4; ++vg) {
                    const int n = 32 * nt + 8 * vg + 4 * half;
                    const f32x4 v = f32x4{st[i][4 * vg], st[i][4 * vg + 1], st[i][4 * vg + 2],
                                          st[i][4 * vg + 3]};
                    if (SP) {
                        const bf16x4 hi = __builtin_convertvector(v, bf16x4);
                        *(bf16x4*)((bf16_t*)sh + p * LS + n) = hi;
                        *(bf16x4*)((bf16_t*)sl + p * LS + n) =
                            __builtin_convertvector(v - __builtin_convertvector(hi, f32x4), bf16x4);
                    } else {
                        Tr<T>::st4(sh + p * LS + n, v);
                    }
                }
            }
        }
    };
    if (!zero_state) state_to_lds();

    const int nti = Q / 32;
    for (int c = 0; c < sd.nchunks; ++c) {
        const int kc = sd.chunk0 + c;
        const ChunkDesc cd = chunk_desc(pl, kc);
        const bool update = (c + 1 < sd.nchunks) || need_final;
        const float* csk = cs + ((size_t)kc * H + h) * Q;
        const float* dtk = dtc + ((size_t)kc * H + h) * Q;
        const float cl = csk[Q - 1];
        for (int q = threadIdx.x; q < Q; q += kThreads) {
            const float a = csk[q], d = dtk[q];
            csl[q] = a;
            dtl[q] = d;
            wl[q] = __expf(cl - a) * d;
        }
        __syncthreads();
        if (update) stage_x<T, PT, true, true>(x, cd, H, P, h, Q, xr, wl, xh, xl, LP);
        else stage_x<T, PT, true, false>(x, cd, H, P, h, Q, xr, nullptr, nullptr, nullptr, LP);
        __syncthreads();

        const float* cbk = cb + ((size_t)kc * G + g) * Q * Q;
        for (int ti = 0; ti < nti; ++ti) {
            const int owner = ((ti >> 2) & 1) ? 3 - (ti & 3) : (ti & 3);
            if (owner != wave) continue;
            f32x16 ya[NPT];
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) ya[pt] = f32x16{};
            const int t = 32 * ti + col;
            const bool tv = t < cd.len;
            const float cst = csl[t];
            if (!zero_state) {
                const T* crow = Cm + ((cd.row0 + t) * G + g) * N;
                for (int n0 = 0; n0 < NT; n0 += 16) {
                    const int n = n0 + 8 * half;
                    v8 b = {};
                    if (tv && n < N) b = Tr<T>::ld8(crow + n);
#pragma unroll
                    for (int pt = 0; pt < NPT; ++pt) {
                        const int off = (32 * pt + col) * LS + n0 + 8 * half;
                        mma16(ya[pt], Tr<T>::ld8(sh + off), b);
                        if (SP) mma16(ya[pt], Tr<T>::ld8(sl + off), b);
                    }
                }
                const float e = __expf(cst);
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) ya[pt] *= e;
            }
            const float* grow = cbk + (size_t)t * Q;
            for (int kj = 0; kj <= ti; ++kj) {
                const bool diag = (kj == ti);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int kb = 32 * kj + 16 * ks + 8 * half;
                    const f32x4 g0 = *(const f32x4*)(grow + kb);
                    const f32x4 g1 = *(const f32x4*)(grow + kb + 4);
                    f32x8 m;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int kk = kb + i;
                        const float gv = i < 4 ? g0[i] : g1[i - 4];
                        const bool keep = !diag || kk <= t;
                        const float e = keep ? __expf(cst - csl[kk]) : 0.f;
                        m[i] = keep ? gv * e * dtl[kk] : 0.f;
                    }
                    const v8 b = Tr<T>::narrow(m);
#pragma unroll
                    for (int pt = 0; pt < NPT; ++pt) mma16(ya[pt], Tr<T>::ld8(xr + (32 * pt + col) * LP + kb), b);
                }
            }
            if (tv) {
                const T* xrow = x + ((cd.row0 + t) * H + h) * P;
                const size_t yoff = ((cd.row0 + t) * H + h) * P;
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) {
#pragma unroll
                    for (int vg = 0; vg < 4; ++vg) {
                        const int p = 32 * pt + 8 * vg + 4 * half;
                        if (p < P) {
                            const f32x4 xv = Tr<T>::ld4(xrow + p);
                            const f32x4 o = f32x4{ya[pt][4 * vg], ya[pt][4 * vg + 1], ya[pt][4 * vg + 2],
                                                  ya[pt][4 * vg + 3]} + Dh * xv;
                            if (y_f32) *(f32x4*)((float*)yv + yoff + p) = o;
                            else Tr<bf16_t>::st4((bf16_t*)yv + yoff + p, o);
                        }
                    }
                }
            }
        }
        if (update) {
            __syncthreads();  // all reads of the state operand sh/sl are done
            const float dec = __expf(cl);
            const T* btk = bt + ((size_t)kc * G + g) * N * Q;
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int u = wave * TPW + i;
                if (u < NTILE)
                    state_update_tile<T>(st[i], dec, btk, 32 * (u / NPT) + col, N, Q, xh, xl,
                                         32 * (u % NPT) + col, LP, half);
            }
            state_to_lds();
            zero_state = false;
        }
        __syncthreads();
    }
    if (need_final) {
        float* out = fin + ((size_t)sd.seq * H + h) * P * N;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int u = wave * TPW + i;
            if (u < NTILE) {
                const int nt = u / NPT, pt = u % NPT;
                const int p = 32 * pt + col;
#pragma unroll
                for (int vg = 0; vg < 4; ++vg) {
                    const int n = 32 * nt + 8 * vg + 4 * half;
                    if (p < P && n < N)
                        *(f32x4*)(out + (size_t)p * N + n) =
                            f32x4{st[i][4 * vg], st[i][4 * vg + 1], st[i][4 * vg + 2], st[i][4 * vg + 3]};
                }
            }
        }
    }
}

template <typename T, int PT, int NT>
size_t scan_lds(int Q) {
    const size_t nx = Split<T>::on ? 3 : 2, ns = Split<T>::on ? 2 : 1;
    return nx * PT * (Q + 8) * sizeof(T) + ns * PT * (NT + 8) * sizeof(T) + 3 * Q * sizeof(float);
}
template <typename T, int PT>
size_t state_lds(int Q) {
    const size_t nx = Split<T>::on ? 2 : 1;
    return nx * PT * (Q + 8) * sizeof(T) + Q * sizeof(float);
}

template <typename F>
hipError_t allow_lds(F* fn, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, int PT, int NT>
hipError_t run_prefill(const Plan& pl, const Layout& lay, const ScanArgs& a, hipStream_t stream,
                       hipEvent_t* marks) {
    char* ws = a.ws;
    const T* x = (const T*)a.x;
    const T* B = (const T*)a.B;
    const T* C = (const T*)a.C;
    float* cs = (float*)(ws + lay.cs);
    float* dtc = (float*)(ws + lay.dtc);
    float* cbm = (float*)(ws + lay.cb);
    T* bt = (T*)(ws + lay.bt);
    float* sbuf = (float*)(ws + lay.sbuf);
    hipError_t err;
    auto mark = [&](int i) -> hipError_t { return marks ? hipEventRecord(marks[i], stream) : hipSuccess; };
    if ((err = mark(0)) != hipSuccess) return err;
    if (!pl.dense && pl.nseq > 0) {
        hipLaunchKernelGGL(ssd_plan_kernel, dim3(1), dim3(kThreads), 0, stream, pl);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(1)) != hipSuccess) return err;
    if (pl.nchunk_ub > 0) {
        hipLaunchKernelGGL(ssd_cumsum_kernel, dim3(pl.nchunk_ub, (pl.H + 3) / 4), dim3(kThreads), 0,
                           stream, pl, a.dt, a.A, cs, dtc);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(2)) != hipSuccess) return err;
    if (pl.nchunk_ub > 0) {
        hipLaunchKernelGGL(ssd_cb_kernel<T>, dim3(pl.nchunk_ub, pl.G, pl.Q / 32), dim3(64), 0, stream,
                           pl, B, C, cbm, bt);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(3)) != hipSuccess) return err;
    if (a.run_passing) {
        if (pl.nseg_ub > 0 && pl.nslot_ub > 0) {
            const size_t lds = state_lds<T, PT>(pl.Q);
            auto* k2 = ssd_chunk_state_kernel<T, PT, NT>;
            if ((err = allow_lds(k2, lds)) != hipSuccess) return err;
            hipLaunchKernelGGL(k2, dim3(pl.nseg_ub, pl.H), dim3(kThreads), lds, stream, pl, x, cs, dtc,
                               bt, sbuf);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
    }
    if ((err = mark(4)) != hipSuccess) return err;
    if (a.run_passing) {
        const int pn4 = pl.P * pl.N / 4;
        hipLaunchKernelGGL(ssd_state_passing_kernel, dim3((pn4 + kThreads - 1) / kThreads, pl.H, pl.nseq),
                           dim3(kThreads), 0, stream, pl, cs, sbuf, a.init, a.final_state);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(5)) != hipSuccess) return err;
    if (pl.nseg_ub > 0) {
        const size_t lds = scan_lds<T, PT, NT>(pl.Q);
        auto* k4 = ssd_chunk_scan_kernel<T, PT, NT>;
        if ((err = allow_lds(k4, lds)) != hipSuccess) return err;
        hipLaunchKernelGGL(k4, dim3(pl.nseg_ub, pl.H), dim3(kThreads), lds, stream, pl, x, cs, dtc, C,
                           cbm, bt, a.D, a.init, sbuf, a.y, a.y_f32, a.final_state);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(6)) != hipSuccess) return err;
    return hipSuccess;
}

template <typename T>
hipError_t dispatch_nt(const Plan& pl, const Layout& lay, const ScanArgs& a, hipStream_t s,
                       hipEvent_t* marks) {
    const int PT = pl.P <= 32 ? 32 : pl.P <= 64 ? 64 : 128;
    const int NT = pl.N <= 32 ? 32 : pl.N <= 64 ? 64 : pl.N <= 128 ? 128 : 256;
#define SSD_CASE(pt, nt) \
    if (PT == pt && NT == nt) return run_prefill<T, pt, nt>(pl, lay, a, s, marks);
    SSD_CASE(32, 32) SSD_CASE(32, 64) SSD_CASE(32, 128) SSD_CASE(32, 256)
    SSD_CASE(64, 32) SSD_CASE(64, 64) SSD_CASE(64, 128) SSD_CASE(64, 256)
    SSD_CASE(128, 32) SSD_CASE(128, 64) SSD_CASE(128, 128) SSD_CASE(128, 256)
#undef SSD_CASE
    return hipErrorInvalidValue;
}

}  // namespace

size_t chunk_scan_lds_bytes(int dtype, int P, int N, int Q) {
    const int PT = P <= 32 ? 32 : P <= 64 ? 64 : 128;
    const int NT = N <= 32 ? 32 : N <= 64 ? 64 : N <= 128 ? 128 : 256;
    const size_t es = dtype == 1 ? 2 : 4;
    const size_t nx = dtype == 1 ? 3 : 2, ns = dtype == 1 ? 2 : 1;  // bf16 keeps hi/lo pairs
    return nx * PT * (Q + 8) * es + ns * PT * (NT + 8) * es + 3 * Q * sizeof(float);
}

hipError_t launch_prefill(const Plan& plan, const Layout& lay, const ScanArgs& a, hipStream_t stream,
                          hipEvent_t* marks) {
    if (a.dtype == 1) return dispatch_nt<bf16_t>(plan, lay, a, stream, marks);
    return dispatch_nt<float>(plan, lay, a, stream, marks);
}

}  // namespace ssd
