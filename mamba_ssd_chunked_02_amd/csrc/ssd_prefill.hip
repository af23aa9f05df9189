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
//   plan           packed batches only: chunk and sequence tables
//   cumsum         cs and dt per (chunk, head), wave64 DPP prefix scan
//   cb             C.B^T per (chunk, group) on MFMA, and B^T per chunk
//   chunk_state    S_c per (chunk, head, 32-column tile of P), MFMA
//   state_passing  sequential over the chunks of a sequence, parallel over
//                  (head, P, N); replaces S_c by h_c, writes final states
//   chunk_scan     y per (chunk, head, 32-column tile of P), MFMA
// chunk_state and chunk_scan have no dependence between chunks, so every
// (chunk, head, tile) is an independent workgroup.  The contractions run on
// 32x32 MFMA tiles (bf16 inputs: 32x32x16 bf16; fp32 inputs: 32x32x2 f32),
// fp32 accumulation everywhere.
#include <algorithm>

#include "ssd_device.h"

namespace ssd {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------ plan
// One workgroup.  Sequence s covers rows [cu[s], cu[s+1]); an offset list that
// is decreasing or leaves [0, T] makes that sequence empty, so no later kernel
// can address memory outside the token arrays.
__global__ __launch_bounds__(kThreads) void ssd_plan_kernel(Plan pl) {
    __shared__ int s_a[kThreads];
    __shared__ int s_carry;
    const int tid = threadIdx.x;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base < pl.nseq; base += kThreads) {
        const int s = base + tid;
        int nc = 0;
        if (s < pl.nseq) {
            const int a = pl.cu[s], b = pl.cu[s + 1];
            const int len = (a >= 0 && b >= a && (int64_t)b <= pl.T) ? b - a : 0;
            nc = (len + pl.Q - 1) / pl.Q;
        }
        s_a[tid] = nc;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {  // inclusive block scan
            const int va = tid >= off ? s_a[tid - off] : 0;
            __syncthreads();
            s_a[tid] += va;
            __syncthreads();
        }
        if (s < pl.nseq) ((int4*)pl.seq_tab)[s] = make_int4(s_carry + s_a[tid] - nc, nc, 0, 0);
        __syncthreads();
        if (tid == kThreads - 1) s_carry += s_a[tid];
        __syncthreads();
    }
    int nchunks = s_carry;
    if (nchunks > pl.nchunk_ub) {
        // the offsets describe more tokens than the stream holds (overlapping
        // sequences): treat every sequence as empty rather than index past the
        // workspace regions sized for T tokens
        for (int s = tid; s < pl.nseq; s += kThreads) ((int4*)pl.seq_tab)[s] = make_int4(0, 0, 0, 0);
        nchunks = 0;
    }
    // chunk entries; the owning sequence is the last one whose first chunk is
    // <= the entry (empty sequences share it with a successor)
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
            e = make_int4(lo, a + c * pl.Q, min(pl.Q, len - c * pl.Q), c);
        }
        ((int4*)pl.chunk_tab)[k] = e;
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
// grid (chunks, G, Q/32), one wave: row tile ti of cb = C B^T (stored in the
// input dtype) for column tiles kj <= ti, the causal part the chunk scan
// reads; plus columns [32 ti, 32 ti + 32) of B^T with rows padded with zeros
// to ntp (a multiple of 32).  Rows/columns past the chunk end are zero.
template <typename T>
__global__ __launch_bounds__(64) void ssd_cb_kernel(Plan pl, int ntp, const T* __restrict__ B,
                                                    const T* __restrict__ C, T* __restrict__ cb,
                                                    T* __restrict__ bt) {
    const int k = blockIdx.x, g = blockIdx.y, ti = blockIdx.z;
    const ChunkDesc cd = chunk_desc(pl, k);
    if (cd.seq < 0) return;
    const int Q = pl.Q, N = pl.N, G = pl.G;
    const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;
    typedef typename Tr<T>::v8 v8;
    const int t = 32 * ti + col;
    const bool tv = t < cd.len;
    const T* crow = C + ((cd.row0 + (tv ? t : 0)) * G + g) * N;
    T* out = cb + ((size_t)k * G + g) * Q * Q;
    for (int kj = 0; kj <= ti; ++kj) {
        f32x16 acc = {};
        const int kk = 32 * kj + col;
        const bool kv = kk < cd.len;
        const T* brow = B + ((cd.row0 + (kv ? kk : 0)) * G + g) * N;
        for (int n0 = 0; n0 < N; n0 += 16) {
            const int n = n0 + 8 * half;
            const bool nv = n < N;
            const v8 a0 = Tr<T>::ld8(crow + (nv ? n : 0));
            const v8 b0 = Tr<T>::ld8(brow + (nv ? n : 0));
            mma16(acc, (tv && nv) ? a0 : v8{}, (kv && nv) ? b0 : v8{});
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) out[(size_t)(32 * ti + acc_row(v, lane)) * Q + 32 * kj + col] = (T)acc[v];
    }
    T* btk = bt + ((size_t)k * G + g) * ntp * Q;
    for (int idx = lane; idx < 32 * (ntp / 8); idx += 64) {
        const int kk = idx & 31, ng = idx >> 5;
        const int kr = 32 * ti + kk;
        const bool ok = kr < cd.len && 8 * ng < N;
        const v8 bv = Tr<T>::ld8(B + ((cd.row0 + (ok ? kr : 0)) * G + g) * N + (ok ? 8 * ng : 0));
        const v8 b = ok ? bv : v8{};
#pragma unroll
        for (int i = 0; i < 8; ++i) btk[(size_t)(8 * ng + i) * Q + kr] = b[i];
    }
}

// ------------------------------------------------------------------ shared pieces
// Operand precision.  x, B, C are exact in their dtype.  Three products are
// rounded to the operand dtype: C.B^T (once, by the cb kernel), x scaled by a
// per-token fp32 weight, and the fp32 state used as an operand.  For bf16 the
// chunk state's x * weight and the state operand of y are carried as hi/lo
// pairs (hi = rn(v), lo = rn(v - hi)) and contracted with two MFMAs, which
// keeps their error ~2^-16 relative; the intra-chunk term of y uses the hi
// part only.  fp32 operands are not split.
template <typename T>
struct Split {
    static constexpr bool on = !__is_same(T, float);
};

// Grid order: item i of a chunk-major work list runs as workgroup L with
// i = (L % 8) * per_xcd + L / 8.  Workgroups are dealt to the 8 XCDs round
// robin, so each XCD walks a contiguous range of items: the heads and column
// tiles of one chunk run together and share its C.B^T, C and B^T in that
// XCD's L2.
__device__ inline int64_t xcd_item(int per_xcd) {
    return (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
}

// Workgroup-cooperative transposed copy of x * w for the columns
// [32pt, 32pt+32) of head h in one chunk:
//   xh[pl][k] (+ xl[pl][k]) = x[row0+k][h][32pt+pl] * w[k]     (pitch LP)
// zero past the chunk end and past P; xl (the rounding residue) only when LO.
// One unit = 4 tokens x 8 columns; Q units, spread over the NTHR threads.
template <typename T, bool LO, int Q, int NTHR>
__device__ inline void stage_xw(const T* __restrict__ x, const ChunkDesc& cd, int H, int P, int h, int pt,
                                const float* w, T* xh, T* xl, int LP, int tid) {
    typedef typename Tr<T>::v8 v8;
    typedef typename Tr<T>::v4 v4;
#pragma unroll
    for (int u0 = 0; u0 < Q; u0 += NTHR) {
        const int u = u0 + tid;
        if (Q % NTHR != 0 && u >= Q) break;
        const int pb = u & 3, k0 = 4 * (u >> 2);
        const int pc = 32 * pt + 8 * pb;
        const bool pok = pc < P;
        const int p0 = pok ? pc : 0;
        v8 raw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int kk = min(k0 + r, cd.len - 1);
            raw[r] = Tr<T>::ld8(x + ((cd.row0 + kk) * H + h) * P + p0);
        }
        const f32x4 wv = *(const f32x4*)(w + k0);
        f32x8 f[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) f[r] = Tr<T>::widen(raw[r]) * ((pok && k0 + r < cd.len) ? wv[r] : 0.f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 o = {f[0][i], f[1][i], f[2][i], f[3][i]};
            const v4 hi = Tr<T>::narrow4(o);
            Tr<T>::st4raw(xh + (8 * pb + i) * LP + k0, hi);
            if (LO) Tr<T>::st4raw(xl + (8 * pb + i) * LP + k0, Tr<T>::narrow4(o - Tr<T>::widen4(hi)));
        }
    }
}

// ------------------------------------------------------------------ chunk_state
// Workgroup per (chunk k, head h, tile pt of 32 columns of P):
//   S_k[p][n] = sum_t exp(cs_last - cs_t) dt_t x[t][p] B[t][n]
// for p in the tile and every n < N, as a (32 x Q) . (Q x NT) MFMA product:
// A = (x w)^T from LDS (hi/lo pair when split), B = the B^T rows the cb
// kernel wrote.  The weight w_t = exp(cs_last - cs_t) dt_t <= dt_t never
// overflows.  Wave w computes the 32-wide n-tiles w, w + waves, ...
__host__ __device__ constexpr int state_waves(int NT) { return NT / 32 < 4 ? NT / 32 : 4; }

template <typename T>
__host__ __device__ constexpr size_t chunk_state_lds_bytes(int Q) {
    return (size_t)Q * sizeof(float) + (size_t)(Split<T>::on ? 2 : 1) * 32 * (Q + 8) * sizeof(T);
}

template <typename T, int NT, int NTI>
__global__ __launch_bounds__(64 * state_waves(NT)) void ssd_chunk_state_kernel(
    Plan pl, int per_xcd, int npt, const T* __restrict__ x, const float* __restrict__ cs,
    const float* __restrict__ dtc, const T* __restrict__ bt, float* __restrict__ states) {
    extern __shared__ __align__(16) char smem[];
    constexpr bool SP = Split<T>::on;
    constexpr int NNT = NT / 32, Q = 32 * NTI, LP = Q + 8;
    constexpr int NW = state_waves(NT), NTHR = 64 * NW;
    typedef typename Tr<T>::v8 v8;
    const int64_t item = xcd_item(per_xcd);
    if (item >= (int64_t)pl.nchunk_ub * pl.H * npt) return;
    const int pt = (int)(item % npt);
    const int64_t kh = item / npt;
    const int h = (int)(kh % pl.H), k = (int)(kh / pl.H);
    const ChunkDesc cd = chunk_desc(pl, k);
    if (cd.seq < 0) return;
    const int P = pl.P, N = pl.N, H = pl.H, G = pl.G;
    const int g = h / pl.hpg;
    const int tid = threadIdx.x;
    float* w = (float*)smem;
    T* xh = (T*)(smem + Q * sizeof(float));
    T* xl = xh + 32 * LP;
    const float* csk = cs + ((size_t)k * H + h) * Q;
    const float* dtk = dtc + ((size_t)k * H + h) * Q;
    const float clast = csk[Q - 1];
    for (int q = tid; q < Q; q += NTHR) w[q] = __expf(clast - csk[q]) * dtk[q];
    __syncthreads();
    stage_xw<T, SP, Q, NTHR>(x, cd, H, P, h, pt, w, xh, xl, LP, tid);
    __syncthreads();
    const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const T* btk = bt + ((size_t)k * G + g) * NT * Q;
    float* out = states + ((size_t)k * H + h) * P * N;
    const T* arow = xh + col * LP + 8 * half;
    const T* lrow = xl + col * LP + 8 * half;
    for (int nt = wave; nt < NNT; nt += NW) {
        f32x16 acc = {};
        const T* brow = btk + (size_t)(32 * nt + col) * Q + 8 * half;
#pragma unroll 8
        for (int s = 0; s < Q / 16; ++s) {
            const v8 b = Tr<T>::ld8(brow + 16 * s);
            mma16(acc, Tr<T>::ld8(arow + 16 * s), b);
            if (SP) mma16(acc, Tr<T>::ld8(lrow + 16 * s), b);
        }
        // acc: row p = 32pt + acc_row(v), column n = 32nt + col
        const int n = 32 * nt + col;
        if (n < N) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int p = 32 * pt + acc_row(v, lane);
                if (p < P) out[(size_t)p * N + n] = acc[v];
            }
        }
    }
}

// ------------------------------------------------------------------ state_passing
// Flat grid over (sequence, head, block of 1024 elements of P*N); each thread
// owns four consecutive (p, n) elements in fp32 and walks the sequence's
// chunks in order:
//   h <- initial state (or 0);  per chunk c:  slot_c <- h,  h <- exp(cs_last,c) h + S_c
// where slot_c held S_c.  Afterwards slot_c holds the state entering chunk c
// and h is the state after the sequence (a sequence without tokens passes its
// initial state through).  The S_c of a batch of chunks are loaded before any
// of them is combined, so each thread keeps several loads in flight.
__global__ __launch_bounds__(kThreads) void ssd_state_passing_kernel(Plan pl, int nblk,
                                                                      const float* __restrict__ cs,
                                                                      float* __restrict__ states,
                                                                      const float* __restrict__ init,
                                                                      float* __restrict__ fin) {
    const int b = (int)(blockIdx.x % nblk);
    const int sh = (int)(blockIdx.x / nblk);
    const int h = sh % pl.H, s = sh / pl.H;
    const int PN = pl.P * pl.N;
    const int e = (b * kThreads + threadIdx.x) * 4;
    if (e >= PN) return;
    const int2 sc = seq_chunks(pl, s);
    const size_t off = ((size_t)s * pl.H + h) * PN + e;
    f32x4 st = {};
    if (init) st = *(const f32x4*)(init + off);
    constexpr int kBatch = 8;
    for (int c0 = 0; c0 < sc.y; c0 += kBatch) {
        f32x4 own[kBatch];
        float last[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const size_t kc = (size_t)sc.x + min(c0 + i, sc.y - 1);
            own[i] = *(const f32x4*)(states + (kc * pl.H + h) * PN + e);
            last[i] = cs[(kc * pl.H + h) * pl.Q + pl.Q - 1];
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            if (c0 + i < sc.y) {
                const size_t kc = (size_t)sc.x + c0 + i;
                *(f32x4*)(states + (kc * pl.H + h) * PN + e) = st;
                st = __expf(last[i]) * st + own[i];
            }
        }
    }
    if (fin) *(f32x4*)(fin + off) = st;
}

// ------------------------------------------------------------------ chunk_scan
// Workgroup per (chunk k, head h, tile pt of 32 columns of P); it writes
//   y[t][p] = exp(cs_t) sum_n C[t][n] h_k[p][n]                      (state term)
//           + sum_{s<=t} (C_t . B_s) exp(cs_t - cs_s) dt_s x[s][p]   (causal intra-chunk term)
//           + D x[t][p]
// for the chunk's tokens t and the tile's columns p, with h_k the state
// entering the chunk (written by state_passing).
//
// Decay bookkeeping.  The chunk is cut into 32-token blocks j with start
// s_j = 32j - 1 and end e_j = 32j + 31 (cs_{-1} := 0).  The workgroup shares
// these fp32 tables in LDS:
//   wb[s]   = exp(cs_{e(s)} - cs_s) dt_s          weight of token s to its block end (<= dt_s)
//   gam[j]  = exp(cs_{e_j} - cs_{s_j})            decay across block j (<= 1)
//   ul[t]   = exp(cs_t - cs_{s(t)})               decay from the block start to t (<= 1)
//   ue[t]   = exp(cs_t - cs_{e(t)})               = ul[t] / gam[j] (>= 1)
//   fast[j] = decay across block j below kFastBlockDecay (so ue stays finite)
// Output block i (32 tokens, MFMA rows t; columns p) then is a Horner scheme
// over the blocks j <= i:
//   acc  = C_rows . h_k^T                        (state hi/lo pair from LDS)
//   acc  = gam[j] acc + (C.B^T)[t, block j] . (x wb)_j        for j = 0 .. i
//          (the diagonal block masked to s <= t)
//   acc *= ue[t]
// which leaves exp(cs_t) on the state term and exp(cs_t - cs_s) dt_s on every
// intra-chunk pair, with every factor applied <= 1 except ue on its own block
// (an underflow only ever drops a term below 1e-38 of dt x).  A block whose
// decay exceeds kFastBlockDecay stops the scheme before its diagonal, scales
// by ul[t] and adds its diagonal with exact per-element factors instead.
constexpr float kFastBlockDecay = 60.f;

struct ChunkTables {
    float* cs;   // [Q]
    float* dt;   // [Q]
    float* wb;   // [Q]
    float* ul;   // [Q]
    float* ue;   // [Q]
    float* gam;  // [8]
    int* fast;   // [8]
};

__host__ __device__ constexpr size_t tables_bytes(int Q) {
    return ((size_t)(5 * Q + 8) * sizeof(float) + 8 * sizeof(int) + 15) & ~(size_t)15;
}

__device__ inline ChunkTables carve_tables(char* base, int Q) {
    ChunkTables tb;
    tb.cs = (float*)base;
    tb.dt = tb.cs + Q;
    tb.wb = tb.dt + Q;
    tb.ul = tb.wb + Q;
    tb.ue = tb.ul + Q;
    tb.gam = tb.ue + Q;
    tb.fast = (int*)(tb.gam + 8);
    return tb;
}

template <int Q, int NTHR>
__device__ inline void build_tables(const ChunkTables& tb, const float* __restrict__ csk,
                                    const float* __restrict__ dtk, int tid) {
    for (int q = tid; q < Q; q += NTHR) {
        const float a = csk[q], d = dtk[q];
        const float ce = csk[q | 31];
        const int s = (q & ~31) - 1;
        const float c0 = s >= 0 ? csk[s] : 0.f;
        tb.cs[q] = a;
        tb.dt[q] = d;
        tb.wb[q] = __expf(ce - a) * d;
        tb.ul[q] = __expf(a - c0);
        tb.ue[q] = __expf(fminf(a - ce, kFastBlockDecay));
    }
    if (tid < Q / 32) {
        const float c0 = tid > 0 ? csk[32 * tid - 1] : 0.f;
        const float ce = csk[32 * tid + 31];
        tb.gam[tid] = __expf(ce - c0);
        tb.fast[tid] = (c0 - ce) < kFastBlockDecay ? 1 : 0;
    }
}

// hi/lo copy of the fp32 state rows p in [32pt, 32pt+32) as the B operand of
// the state term: sh[pl][n] (+ sl[pl][n] when split), pitch NS, zero past P
// and past N.
template <typename T, int NT, int NTHR>
__device__ inline void stage_state(const float* __restrict__ src, int P, int N, int pt, T* sh, T* sl,
                                   int NS, int tid) {
    typedef typename Tr<T>::v4 v4;
    constexpr int NQ = NT / 4;
    constexpr int U = 32 * NQ;
    f32x4 v[(U + NTHR - 1) / NTHR];
#pragma unroll
    for (int i = 0; i * NTHR < U; ++i) {
        const int u = i * NTHR + tid;
        const int r = u / NQ, n = 4 * (u % NQ);
        const int p = 32 * pt + r;
        const bool ok = (U % NTHR == 0 || u < U) && p < P && n < N;
        const f32x4 raw = *(const f32x4*)(src + (ok ? (size_t)p * N + n : 0));
        v[i] = ok ? raw : f32x4{};
    }
#pragma unroll
    for (int i = 0; i * NTHR < U; ++i) {
        const int u = i * NTHR + tid;
        if (U % NTHR != 0 && u >= U) break;
        const int r = u / NQ, n = 4 * (u % NQ);
        const v4 hi = Tr<T>::narrow4(v[i]);
        Tr<T>::st4raw(sh + r * NS + n, hi);
        if (Split<T>::on) Tr<T>::st4raw(sl + r * NS + n, Tr<T>::narrow4(v[i] - Tr<T>::widen4(hi)));
    }
}

template <typename T>
__host__ __device__ constexpr size_t chunk_scan_lds_bytes(int NT, int Q) {
    return tables_bytes(Q) + (size_t)32 * (Q + 8) * sizeof(T) +
           (size_t)(Split<T>::on ? 2 : 1) * 32 * (NT + 8) * sizeof(T);
}

__host__ __device__ constexpr int scan_waves(int NTI) { return NTI < 4 ? NTI : 4; }

template <typename T, typename TY>
struct ScanCtx {
    ChunkTables tb;
    const T* xh;     // (x wb)^T hi, pitch Q + 8
    const T* sh;     // entering state hi, pitch NT + 8
    const T* sl;     // entering state lo
    const T* cbk;    // C.B^T of the chunk, [Q][Q]
    const T* Cm;     // C
    const T* xcol;   // x at row 0, head h, column min(p, P-1)
    TY* ycol;        // y at row 0, head h, column p
    int64_t row0;
    int len, G, g, N, HP, pvalid, has_state;
    float Dh;
};

// One 32-token output block TI of the workgroup's tile, for the calling wave.
template <typename T, typename TY, int NT, int NTI, int TI>
__device__ __forceinline__ void scan_block(const ScanCtx<T, TY>& c) {
    constexpr bool SP = Split<T>::on;
    constexpr int Q = 32 * NTI, LP = Q + 8, NS = NT + 8;
    typedef typename Tr<T>::v8 v8;
    typedef typename Tr<T>::elem E;
    const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    const int ta = 32 * TI + col;  // this lane's A row
    // global operands first: C.B^T rows of the block, then x for the D x term
    v8 ga[TI + 1][2];
    const T* grow = c.cbk + (size_t)ta * Q + 8 * half;
#pragma unroll
    for (int kj = 0; kj <= TI; ++kj)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) ga[kj][ks] = Tr<T>::ld8(grow + 32 * kj + 16 * ks);
    float xd[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int t = min(32 * TI + acc_row(v, lane), c.len - 1);
        xd[v] = (float)c.xcol[(c.row0 + t) * c.HP];
    }
    f32x16 acc = {};
    if (c.has_state) {
        const T* crow = c.Cm + ((c.row0 + min(ta, c.len - 1)) * c.G + c.g) * c.N;
        const T* srow = c.sh + col * NS + 8 * half;
        const T* lrow = c.sl + col * NS + 8 * half;
        v8 ca[NT / 16];
#pragma unroll
        for (int s = 0; s < NT / 16; ++s) ca[s] = Tr<T>::ld8(crow + min(16 * s + 8 * half, c.N - 8));
#pragma unroll
        for (int s = 0; s < NT / 16; ++s) {
            mma16(acc, ca[s], Tr<T>::ld8(srow + 16 * s));
            if (SP) mma16(acc, ca[s], Tr<T>::ld8(lrow + 16 * s));
        }
    }
    const bool fast = c.tb.fast[TI] != 0;
    const T* xrow = c.xh + col * LP + 8 * half;
#pragma unroll
    for (int kj = 0; kj <= TI; ++kj) {
        if (kj < TI || fast) {
            acc *= c.tb.gam[kj];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                v8 a = ga[kj][ks];
                if (kj == TI) {
                    const int k0 = 32 * kj + 16 * ks + 8 * half;
#pragma unroll
                    for (int i = 0; i < 8; ++i) a[i] = (k0 + i <= ta) ? a[i] : (E)0;
                }
                mma16(acc, a, Tr<T>::ld8(xrow + 32 * kj + 16 * ks));
            }
        }
    }
    const float* scale = fast ? c.tb.ue : c.tb.ul;
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) {
        const f32x4 u = *(const f32x4*)(scale + 32 * TI + 8 * vg + 4 * half);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * vg + j] *= u[j];
    }
    if (!fast) {
        // decay across this block beyond the fast range: exact factors, raw x
        const float cst = c.tb.cs[ta];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int k0 = 32 * TI + 16 * ks + 8 * half;
            const f32x8 gv = Tr<T>::widen(ga[TI][ks]);
            f32x8 m;
            v8 xb;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int kk = k0 + i;
                const float e = __expf(fminf(cst - c.tb.cs[kk], 0.f)) * c.tb.dt[kk];
                m[i] = kk <= ta ? gv[i] * e : 0.f;
                xb[i] = c.xcol[(c.row0 + min(kk, c.len - 1)) * c.HP];
            }
            mma16(acc, Tr<T>::narrow(m), xb);
        }
    }
    // + D x; rows t of this block, column p
    if (c.pvalid) {
        TY* yb = c.ycol + (c.row0 + 32 * TI) * c.HP;
        if (32 * TI + 32 <= c.len) {
#pragma unroll
            for (int v = 0; v < 16; ++v) yb[(int64_t)acc_row(v, lane) * c.HP] = (TY)(acc[v] + c.Dh * xd[v]);
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (32 * TI + acc_row(v, lane) < c.len)
                    yb[(int64_t)acc_row(v, lane) * c.HP] = (TY)(acc[v] + c.Dh * xd[v]);
        }
    }
}

template <typename T, typename TY, int NT, int NTI>
__global__ __launch_bounds__(64 * scan_waves(NTI)) void ssd_chunk_scan_kernel(
    Plan pl, int per_xcd, int npt, const T* __restrict__ x, const float* __restrict__ cs,
    const float* __restrict__ dtc, const T* __restrict__ Cm, const T* __restrict__ cb,
    const float* __restrict__ D, const float* __restrict__ init, const float* __restrict__ states,
    TY* __restrict__ y) {
    extern __shared__ __align__(16) char smem[];
    constexpr int Q = 32 * NTI, LP = Q + 8, NS = NT + 8;
    constexpr int NTHR = 64 * scan_waves(NTI);
    const int64_t item = xcd_item(per_xcd);
    if (item >= (int64_t)pl.nchunk_ub * pl.H * npt) return;
    const int pt = (int)(item % npt);
    const int64_t kh = item / npt;
    const int h = (int)(kh % pl.H), k = (int)(kh / pl.H);
    const ChunkDesc cd = chunk_desc(pl, k);
    if (cd.seq < 0) return;
    const int P = pl.P, N = pl.N, H = pl.H, G = pl.G;
    const int tid = threadIdx.x;
    ScanCtx<T, TY> c;
    c.tb = carve_tables(smem, Q);
    T* xh = (T*)(smem + tables_bytes(Q));
    T* sh = xh + 32 * LP;
    T* sl = sh + 32 * NS;
    c.has_state = (cd.idx > 0 || init != nullptr) ? 1 : 0;
    build_tables<Q, NTHR>(c.tb, cs + ((size_t)k * H + h) * Q, dtc + ((size_t)k * H + h) * Q, tid);
    if (c.has_state)
        stage_state<T, NT, NTHR>(states + ((size_t)k * H + h) * P * N, P, N, pt, sh, sl, NS, tid);
    __syncthreads();
    stage_xw<T, false, Q, NTHR>(x, cd, H, P, h, pt, c.tb.wb, xh, nullptr, LP, tid);
    __syncthreads();
    const int wave = tid >> 6, col = tid & 31;
    const int p = 32 * pt + col;
    c.xh = xh;
    c.sh = sh;
    c.sl = sl;
    c.cbk = cb + ((size_t)k * G + (h / pl.hpg)) * Q * Q;
    c.Cm = Cm;
    c.HP = H * P;
    c.xcol = x + (size_t)h * P + min(p, P - 1);
    c.ycol = y + (size_t)h * P + p;
    c.row0 = cd.row0;
    c.len = cd.len;
    c.G = G;
    c.g = h / pl.hpg;
    c.N = N;
    c.pvalid = p < P;
    c.Dh = D[h];
    // causal work is balanced by pairing block w with block NTI-1-w
    if constexpr (NTI == 8) {
        switch (wave) {
            case 0: scan_block<T, TY, NT, NTI, 0>(c); scan_block<T, TY, NT, NTI, 7>(c); break;
            case 1: scan_block<T, TY, NT, NTI, 1>(c); scan_block<T, TY, NT, NTI, 6>(c); break;
            case 2: scan_block<T, TY, NT, NTI, 2>(c); scan_block<T, TY, NT, NTI, 5>(c); break;
            default: scan_block<T, TY, NT, NTI, 3>(c); scan_block<T, TY, NT, NTI, 4>(c); break;
        }
    } else if constexpr (NTI == 4) {
        switch (wave) {
            case 0: scan_block<T, TY, NT, NTI, 0>(c); break;
            case 1: scan_block<T, TY, NT, NTI, 1>(c); break;
            case 2: scan_block<T, TY, NT, NTI, 2>(c); break;
            default: scan_block<T, TY, NT, NTI, 3>(c); break;
        }
    } else if constexpr (NTI == 2) {
        if (wave == 0) scan_block<T, TY, NT, NTI, 0>(c);
        else scan_block<T, TY, NT, NTI, 1>(c);
    } else {
        scan_block<T, TY, NT, NTI, 0>(c);
    }
}

// ------------------------------------------------------------------ launch
template <typename F>
hipError_t allow_lds(F* fn, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, typename TY, int NT, int NTI>
hipError_t run_prefill(const Plan& pl, const Layout& lay, const ScanArgs& a, hipStream_t stream,
                       hipEvent_t* marks) {
    constexpr int Q = 32 * NTI;
    char* ws = a.ws;
    const T* x = (const T*)a.x;
    const T* B = (const T*)a.B;
    const T* C = (const T*)a.C;
    float* cs = (float*)(ws + lay.cs);
    float* dtc = (float*)(ws + lay.dtc);
    T* cbm = (T*)(ws + lay.cb);
    T* bt = (T*)(ws + lay.bt);
    float* states = (float*)(ws + lay.states);
    hipError_t err;
    auto mark = [&](int i) -> hipError_t { return marks ? hipEventRecord(marks[i], stream) : hipSuccess; };
    const int npt = (pl.P + 31) / 32;
    const int64_t nitems = (int64_t)pl.nchunk_ub * pl.H * npt;
    const int per_xcd = (int)((nitems + 7) / 8);
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
        hipLaunchKernelGGL(ssd_cb_kernel<T>, dim3(pl.nchunk_ub, pl.G, NTI), dim3(64), 0, stream, pl, NT, B,
                           C, cbm, bt);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(3)) != hipSuccess) return err;
    if (nitems > 0) {
        auto* k2 = ssd_chunk_state_kernel<T, NT, NTI>;
        const size_t lds = chunk_state_lds_bytes<T>(Q);
        if ((err = allow_lds(k2, lds)) != hipSuccess) return err;
        hipLaunchKernelGGL(k2, dim3(8 * per_xcd), dim3(64 * state_waves(NT)), lds, stream, pl, per_xcd, npt,
                           x, cs, dtc, bt, states);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(4)) != hipSuccess) return err;
    if (pl.nseq > 0) {
        const int nblk = (pl.P * pl.N / 4 + kThreads - 1) / kThreads;
        hipLaunchKernelGGL(ssd_state_passing_kernel, dim3((unsigned)((int64_t)pl.nseq * pl.H * nblk)),
                           dim3(kThreads), 0, stream, pl, nblk, cs, states, a.init, a.final_state);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(5)) != hipSuccess) return err;
    if (nitems > 0) {
        auto* k4 = ssd_chunk_scan_kernel<T, TY, NT, NTI>;
        const size_t lds = chunk_scan_lds_bytes<T>(NT, Q);
        if ((err = allow_lds(k4, lds)) != hipSuccess) return err;
        hipLaunchKernelGGL(k4, dim3(8 * per_xcd), dim3(64 * scan_waves(NTI)), lds, stream, pl, per_xcd, npt,
                           x, cs, dtc, C, cbm, a.D, a.init, states, (TY*)a.y);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(6)) != hipSuccess) return err;
    return hipSuccess;
}

template <typename T, typename TY>
hipError_t dispatch(const Plan& pl, const Layout& lay, const ScanArgs& a, hipStream_t s, hipEvent_t* marks) {
    const int NT = padded_dstate(pl.N);
    const int NTI = pl.Q / 32;
#define SSD_CASE(nt, nti) \
    if (NT == nt && NTI == nti) return run_prefill<T, TY, nt, nti>(pl, lay, a, s, marks);
    SSD_CASE(32, 1) SSD_CASE(32, 2) SSD_CASE(32, 4) SSD_CASE(32, 8)
    SSD_CASE(64, 1) SSD_CASE(64, 2) SSD_CASE(64, 4) SSD_CASE(64, 8)
    SSD_CASE(128, 1) SSD_CASE(128, 2) SSD_CASE(128, 4) SSD_CASE(128, 8)
    SSD_CASE(256, 1) SSD_CASE(256, 2) SSD_CASE(256, 4) SSD_CASE(256, 8)
#undef SSD_CASE
    return hipErrorInvalidValue;
}

}  // namespace

size_t prefill_lds_bytes(int dtype, int N, int Q) {
    const int NT = padded_dstate(N);
    if (dtype == 1) return std::max(chunk_state_lds_bytes<bf16_t>(Q), chunk_scan_lds_bytes<bf16_t>(NT, Q));
    return std::max(chunk_state_lds_bytes<float>(Q), chunk_scan_lds_bytes<float>(NT, Q));
}

hipError_t launch_prefill(const Plan& plan, const Layout& lay, const ScanArgs& a, hipStream_t stream,
                          hipEvent_t* marks) {
    if (a.dtype == 1) {
        if (a.y_f32) return dispatch<bf16_t, float>(plan, lay, a, stream, marks);
        return dispatch<bf16_t, bf16_t>(plan, lay, a, stream, marks);
    }
    if (a.y_f32) return dispatch<float, float>(plan, lay, a, stream, marks);
    return dispatch<float, bf16_t>(plan, lay, a, stream, marks);
}

}  // namespace ssd
