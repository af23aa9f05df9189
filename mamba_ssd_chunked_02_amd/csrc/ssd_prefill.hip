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
//   cumsum         cs, dt and the chunk-state weights per (chunk, head),
//                  wave64 DPP prefix scan
//   cb             C.B^T per (chunk, group) on MFMA, and B^T per chunk in
//                  MFMA fragment order
// then either (enough (sequence, head, tile) walks to fill the chip)
//   chunk_state_passing  per (sequence, head, 32-column tile of P): walks the
//                  sequence's chunks, accumulating each S_c by MFMA onto the
//                  decayed running state; writes every h_c and the final state
// or
//   chunk_state    S_c per (chunk, head slice, 32-column tile of P), MFMA
//   state_passing  sequential over the chunks of a sequence, parallel over
//                  (head, P, N); replaces S_c by h_c, writes final states
// and
//   chunk_scan     y per (chunk, head slice, 32-column tile of P), MFMA
// chunk_state and chunk_scan have no dependence between chunks, so every
// (chunk, head slice, tile) is an independent workgroup.  The contractions run
// on 32x32 MFMA tiles (bf16 inputs: 32x32x16 bf16; fp32 inputs: 32x32x2 f32),
// fp32 accumulation everywhere.
#include <algorithm>

#include "ssd_prefill_shared.h"

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
        int nc = 0, len = 0, row0 = 0;
        if (s < pl.nseq) {
            const int a = pl.cu[s], b = pl.cu[s + 1];
            const bool valid = a >= 0 && b >= a && (int64_t)b <= pl.T;
            len = valid ? b - a : 0;
            row0 = valid ? a : 0;
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
        if (s < pl.nseq) ((int4*)pl.seq_tab)[s] = make_int4(s_carry + s_a[tid] - nc, nc, row0, len);
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
    // the scan walk's sequence order: by chunk count, longest first (ties in
    // index order), so that its longest walks start first
    if (pl.seq_order) {
        __syncthreads();  // seq_tab complete (or cleared)
        if (pl.nseq <= kOrderMaxSeq) {
            if (tid < pl.nseq) s_a[tid] = nchunks > 0 ? ((const int4*)pl.seq_tab)[tid].y : 0;
            __syncthreads();
            if (tid < pl.nseq) {
                const int mine = s_a[tid];
                int rank = 0;
                for (int t = 0; t < pl.nseq; ++t) rank += (s_a[t] > mine || (s_a[t] == mine && t < tid)) ? 1 : 0;
                pl.seq_order[rank] = tid;
            }
        } else {
            for (int s = tid; s < pl.nseq; s += kThreads) pl.seq_order[s] = s;
        }
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
// grid (chunks, ceil(H/16)): the workgroup reads the chunk's dt for 16 heads
// as contiguous 64-byte row pieces into LDS (through the dt activation when
// one is given), then wave w scans heads w, w+4, w+8, w+12 of the block.  Per
// (chunk, head):
//   cs[q]  = sum_{s<=q} dt_s A_h inside the chunk; positions past the chunk
//            end repeat the last value (dt = 0 there)
//   dtc[q] = dt with zeros past the end
//   wst[q] = exp(cs[Q-1] - cs[q]) dt[q], each token's weight in the chunk
//            state (<= dt, 0 past the end); not written when wst is NULL
constexpr int kCumHeads = 16;

__global__ __launch_bounds__(kThreads) void ssd_cumsum_kernel(Plan pl, const float* __restrict__ dt,
                                                               const float* __restrict__ A,
                                                               float* __restrict__ cs,
                                                               float* __restrict__ dtc,
                                                               float* __restrict__ wst, DtAct act) {
    constexpr int SP = 256 + 4;  // LDS row pitch (floats): one row per head
    __shared__ __align__(16) float sdt[kCumHeads * SP];
    const int k = blockIdx.x;
    const ChunkDesc cd = uniform_desc(chunk_desc(pl, k));
    if (cd.seq < 0) return;
    const int Q = pl.Q, H = pl.H, h0 = blockIdx.y * kCumHeads;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // thread (token q = tid/16 + 16i, head h0 + tid%16): all of its loads go
    // out before any is used (indices clamped into the chunk, masked after)
    {
        constexpr int QS = kThreads / kCumHeads;  // token stride
        constexpr int PER = 256 / QS;             // tokens per thread for the largest chunk
        const int hh = tid % kCumHeads, q0 = tid / kCumHeads;
        const int hc = min(h0 + hh, H - 1);
        const bool hok = h0 + hh < H;
        float v[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) v[i] = dt[(cd.row0 + min(q0 + i * QS, cd.len - 1)) * H + hc];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = q0 + i * QS;
            if (q < Q) sdt[hh * SP + q] = (hok && q < cd.len) ? dt_activate(act, v[i], h0 + hh) : 0.f;
        }
    }
    __syncthreads();
    const int ppl = Q >= 64 ? Q / 64 : 1;  // consecutive positions per lane
    for (int hh = wave; hh < kCumHeads; hh += kThreads / 64) {
        const int h = h0 + hh;
        if (h >= H) break;
        const float a = A[h];
        float d[4];
        float own = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = lane * ppl + i;
            d[i] = (i < ppl && q < Q) ? sdt[hh * SP + q] : 0.f;
            own += d[i] * a;
        }
        float run = wave_inclusive_scan(own) - own;  // exclusive prefix of lane totals
        float c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            run += d[i] * a;
            c[i] = run;
        }
        // The sums past the chunk end add only zeros, but the lane totals
        // reach later lanes through the scan tree in another order, so they
        // can differ from cs[len-1] in the last bit; once |cs| is large
        // (a flushing decay) exp() turns that bit into a visible factor.
        // Every position past the end, and cs_last, therefore takes the
        // bits of cs[len-1] itself.
        const int il = (cd.len - 1) % ppl;
        const float mine = il == 0 ? c[0] : il == 1 ? c[1] : il == 2 ? c[2] : c[3];
        const float last = __shfl(mine, (cd.len - 1) / ppl);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane * ppl + i >= cd.len) c[i] = last;
        float* csr = cs + ((size_t)k * H + h) * Q;
        float* dtr = dtc + ((size_t)k * H + h) * Q;
        if (ppl == 4) {
            // 256-token chunks: four consecutive positions per lane, 16-byte stores
            const int q = 4 * lane;
            *(f32x4*)(csr + q) = f32x4{c[0], c[1], c[2], c[3]};
            *(f32x4*)(dtr + q) = f32x4{d[0], d[1], d[2], d[3]};
            if (wst)
                *(f32x4*)(wst + ((size_t)k * H + h) * Q + q) =
                    f32x4{__expf(last - c[0]) * d[0], __expf(last - c[1]) * d[1], __expf(last - c[2]) * d[2],
                          __expf(last - c[3]) * d[3]};
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = lane * ppl + i;
                if (i < ppl && q < Q) {
                    csr[q] = c[i];
                    dtr[q] = d[i];
                    if (wst) wst[((size_t)k * H + h) * Q + q] = __expf(last - c[i]) * d[i];
                }
            }
        }
    }
}

// ------------------------------------------------------------------ C.B^T
// grid (chunks, G, NTI (NTI + 1) / 2), one wave per causal 32 x 32 tile
// (ti, kj <= ti) of cb = C B^T, stored in the input dtype, the part the chunk
// scan reads; the diagonal tile's entries above the diagonal are zero, rows
// and columns past the chunk end are zero.  The diagonal tile's wave also
// writes tokens [32 ti, 32 ti + 32) of B^T in fragment order, rows n padded
// with zeros to NT.  Outputs leave through LDS as 16-byte rows.
template <typename T>
__host__ __device__ constexpr size_t cb_lds_bytes(int NT) {
    return (size_t)32 * (NT + 16 / sizeof(T)) * sizeof(T);
}

template <typename T, int NT>
__global__ __launch_bounds__(64) void ssd_cb_kernel(Plan pl, const T* __restrict__ B, const T* __restrict__ C,
                                                    T* __restrict__ cb, T* __restrict__ bt) {
    extern __shared__ __align__(16) char smem[];
    T* ls = (T*)smem;
    constexpr int EPC = 16 / sizeof(T);  // elements per 16 bytes
    const int k = blockIdx.x, g = blockIdx.y;
    int kj = blockIdx.z, ti = 0;
    while (kj > ti) {  // blockIdx.z = ti (ti + 1) / 2 + kj
        kj -= ti + 1;
        ++ti;
    }
    const ChunkDesc cd = uniform_desc(chunk_desc(pl, k));
    if (cd.seq < 0) return;
    const int Q = pl.Q, N = pl.N, G = pl.G;
    const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;
    typedef typename Tr<T>::v8 v8;
    const int t = 32 * ti + col, kk = 32 * kj + col;
    const bool tv = t < cd.len, kv = kk < cd.len;
    const T* crow = C + ((cd.row0 + (tv ? t : 0)) * G + g) * N;
    const T* brow = B + ((cd.row0 + (kv ? kk : 0)) * G + g) * N;
    v8 a[NT / 16], b[NT / 16];
#pragma unroll
    for (int s = 0; s < NT / 16; ++s) {
        const int n = 16 * s + 8 * half;
        a[s] = Tr<T>::ld8(crow + (n < N ? n : 0));
        b[s] = Tr<T>::ld8(brow + (n < N ? n : 0));
    }
#pragma unroll
    for (int s = 0; s < NT / 16; ++s) {
        const bool nv = 16 * s + 8 * half < N;
        if (!(tv && nv)) a[s] = v8{};
        if (!(kv && nv)) b[s] = v8{};
    }
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < NT / 16; ++s) mma16(acc, a[s], b[s]);
    // the tile through LDS (pitch 32 + EPC), then 16-byte rows; LDS
    // operations of one wave complete in order
    constexpr int TP = 32 + EPC;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int r = acc_row(v, lane);
        ls[r * TP + col] = (T)((kj < ti || col <= r) ? acc[v] : 0.f);
    }
    T* out = cb + ((size_t)k * G + g) * Q * Q + (size_t)(32 * ti) * Q + 32 * kj;
#pragma unroll
    for (int i = 0; i < 32 * 32 / EPC / 64; ++i) {
        const int c = i * 64 + lane, r = c / (32 / EPC), c0 = (c % (32 / EPC)) * EPC;
        *(u32x4*)(out + (size_t)r * Q + c0) = *(const u32x4*)(ls + r * TP + c0);
    }
    if (kj != ti) return;
    // B^T fragments of this block's tokens: this wave's B operand rows, into
    // LDS as [token][n] (pitch NT + EPC), read back transposed
    constexpr int BP = NT + EPC;
#pragma unroll
    for (int s = 0; s < NT / 16; ++s) Tr<T>::st8(ls + col * BP + 16 * s + 8 * half, b[s]);
    T* btk = bt + ((size_t)k * G + g) * NT * Q;
#pragma unroll
    for (int f = 0; f < 2 * (NT / 32); ++f) {
        const int nt = f >> 1, sl = f & 1;
        const int n = 32 * nt + col, t0 = 16 * sl + 8 * half;
        v8 bv;
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] = ls[(t0 + j) * BP + n];
        Tr<T>::st8(btk + bt_frag(Q, nt, 2 * ti + sl, lane), bv);
    }
}

// Whole-chunk variant, grid (chunks, G), four waves: the chunk's B rows are
// staged once in LDS ([token][n], pitch NT + EPC, zero past the chunk end and
// past N) and wave w computes the causal tiles of output blocks w and
// NTI-1-w (nine 32 x 32 tiles each for 256-token chunks), with its C rows in
// registers and the B operand read from LDS.  The products, their operand
// order and the stored values are those of ssd_cb_kernel; B^T fragments are
// read from the staged rows.  Used when the staged chunk fits in LDS.
template <typename T>
__host__ __device__ constexpr size_t cb_chunk_lds_bytes(int NT, int Q) {
    return (size_t)Q * (NT + 16 / sizeof(T)) * sizeof(T) + (size_t)4 * 32 * (32 + 16 / sizeof(T)) * sizeof(T);
}

template <typename T, int NT>
__global__ __launch_bounds__(256) void ssd_cb_chunk_kernel(Plan pl, const T* __restrict__ B, const T* __restrict__ C,
                                                          T* __restrict__ cb, T* __restrict__ bt) {
    extern __shared__ __align__(16) char smem[];
    constexpr int EPC = 16 / sizeof(T);
    constexpr int BP = NT + EPC, TP = 32 + EPC;
    typedef typename Tr<T>::v8 v8;
    const int k = blockIdx.x, g = blockIdx.y;
    const ChunkDesc cd = uniform_desc(chunk_desc(pl, k));
    if (cd.seq < 0) return;
    const int Q = pl.Q, N = pl.N, G = pl.G, NTI = Q / 32;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, half = lane >> 5, col = lane & 31;
    T* bs = (T*)smem;
    T* ls = bs + (size_t)Q * BP + wave * 32 * TP;
    // output blocks of this wave: w and NTI-1-w
    const int b0 = wave, b1 = NTI - 1 - wave;
    const bool do0 = b0 < NTI && b0 <= b1, do1 = b1 > b0;
    // C rows of both blocks, then the chunk's B rows: every load goes out first
    auto load_c = [&](int ti, v8 (&a)[NT / 16]) {
        const int t = 32 * ti + col;
        const T* crow = C + ((cd.row0 + (t < cd.len ? t : 0)) * G + g) * N;
#pragma unroll
        for (int s = 0; s < NT / 16; ++s) {
            const int n = 16 * s + 8 * half;
            a[s] = Tr<T>::ld8(crow + (n < N ? n : 0));
        }
#pragma unroll
        for (int s = 0; s < NT / 16; ++s)
            if (!(t < cd.len && 16 * s + 8 * half < N)) a[s] = v8{};
    };
    v8 a0[NT / 16], a1[NT / 16];
    if (do0) load_c(b0, a0);
    if (do1) load_c(b1, a1);
    {
        // piece c = 256 i + tid is 8 elements (token c / PR, n = 8 (c % PR));
        // batches of 8 loads go out before their LDS writes
        constexpr int PR = NT / 8;  // pieces per staged row; PR rounds of 256 cover 256 tokens
        constexpr int BATCH = PR < 8 ? PR : 8;
#pragma unroll
        for (int i0 = 0; i0 < PR; i0 += BATCH) {
            v8 v[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int c = 256 * (i0 + u) + tid, t = c / PR, n = 8 * (c % PR);
                const bool ok = t < cd.len && n < N;
                v[u] = Tr<T>::ld8(B + ((cd.row0 + (ok ? t : 0)) * G + g) * N + (ok ? n : 0));
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int c = 256 * (i0 + u) + tid, t = c / PR, n = 8 * (c % PR);
                if (t < Q) Tr<T>::st8(bs + t * BP + n, (t < cd.len && n < N) ? v[u] : v8{});
            }
        }
    }
    __syncthreads();
    auto tiles = [&](int ti, const v8 (&a)[NT / 16]) {
        for (int kj = 0; kj <= ti; ++kj) {
            const T* brow = bs + (32 * kj + col) * BP + 8 * half;
            f32x16 acc = {};
#pragma unroll
            for (int s = 0; s < NT / 16; ++s) mma16(acc, a[s], Tr<T>::ld8(brow + 16 * s));
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = acc_row(v, lane);
                const float e = acc[v];
                ls[r * TP + col] = (T)((kj < ti || col <= r) ? e : 0.f);
            }
            T* out = cb + ((size_t)k * G + g) * Q * Q + (size_t)(32 * ti) * Q + 32 * kj;
#pragma unroll
            for (int i = 0; i < 32 * 32 / EPC / 64; ++i) {
                const int c = i * 64 + lane, r = c / (32 / EPC), c0 = (c % (32 / EPC)) * EPC;
                *(u32x4*)(out + (size_t)r * Q + c0) = *(const u32x4*)(ls + r * TP + c0);
            }
        }
    };
    if (do0) tiles(b0, a0);
    if (do1) tiles(b1, a1);
    // B^T fragments: n-tiles wave, wave + 4, ... of every 16-token step
    T* btk = bt + ((size_t)k * G + g) * NT * Q;
    for (int nt = wave; nt < NT / 32; nt += 4) {
        const int n = 32 * nt + col;
        for (int st = 0; st < 2 * NTI; ++st) {
            const int t0 = 16 * st + 8 * half;
            v8 bv;
#pragma unroll
            for (int j = 0; j < 8; ++j) bv[j] = bs[(t0 + j) * BP + n];
            Tr<T>::st8(btk + bt_frag(Q, nt, st, lane), bv);
        }
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

// Per-wave LDS tile for the output transpose: 32 tokens x 32 columns fp32.
constexpr int kEpPitch = 36;
constexpr int kEpBytes = 32 * kEpPitch * 4;

// Staging of x for one (chunk, head, 32-column tile): a unit is 4 tokens x 8
// columns, loaded early into registers (XUnit), then scaled by per-token fp32
// weights (the cumsum kernel's wst, 0 past the chunk end) and written
// transposed to LDS:
//   xh[pl][k] (+ xl[pl][k]) = x[row0+k][h][32pt+pl] * w[k]     (pitch LP)
// zero past P; xl (the rounding residue) only when LO.
template <typename T>
struct XUnit {
    typename Tr<T>::v8 raw[4];
    f32x4 w4;  // weights of the unit's tokens
    int pb, k0;
    bool pok;
};

// Unit u covers column group pb and token group kb; 16 consecutive units share
// pb, so a wave's transposed LDS writes fall on distinct banks.
template <typename T, int Q>
__device__ inline void load_xunit(XUnit<T>& xu, __amdgpu_buffer_rsrc_t rx, const ChunkDesc& cd, int H, int P,
                                  int h, int pt, int u, const float* __restrict__ wsk) {
    constexpr int G16 = Q / 4 < 16 ? Q / 4 : 16;
    xu.pb = (u / G16) & 3;
    xu.k0 = 4 * (u % G16 + G16 * (u / (4 * G16)));
    const int pc = 32 * pt + 8 * xu.pb;
    xu.pok = pc < P;
    const int p0 = xu.pok ? pc : 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int kk = min(xu.k0 + r, cd.len - 1);
        xu.raw[r] = buffer_ld8<T>(rx, ((kk * H + h) * P + p0) * (int)sizeof(T));
    }
    xu.w4 = *(const f32x4*)(wsk + xu.k0);
}

// Column i of a 4-token x 8-column unit, weighted, into the transposed tiles.
template <typename T, bool LO>
__device__ inline void stage_column(const typename Tr<T>::v8 (&raw)[4], f32x4 w, int i, T* xh, T* xl, int off) {
    typedef typename Tr<T>::v4 v4;
    const f32x4 o = {(float)raw[0][i] * w[0], (float)raw[1][i] * w[1], (float)raw[2][i] * w[2],
                     (float)raw[3][i] * w[3]};
    const v4 hi = Tr<T>::narrow4(o);
    Tr<T>::st4raw(xh + off, hi);
    if (LO) Tr<T>::st4raw(xl + off, Tr<T>::narrow4(o - Tr<T>::widen4(hi)));
}

template <typename T, bool LO>
__device__ inline void store_xunit(const XUnit<T>& xu, T* xh, T* xl, int LP) {
    const f32x4 w = xu.pok ? xu.w4 : f32x4{};
#pragma unroll
    for (int i = 0; i < 8; ++i) stage_column<T, LO>(xu.raw, w, i, xh, xl, (8 * xu.pb + i) * LP + xu.k0);
}

// Work item of the MFMA kernels: (chunk k, group g, slice of hpw heads of the
// group, tile pt of 32 columns of P).  The group's per-chunk operands (B^T,
// C, C.B^T) are loaded once per workgroup and reused for every head of the
// slice; the per-head inputs of the next head are loaded while the current
// head computes.
struct Item {
    int k, g, pt, h0, nh;
};

__device__ inline bool decode_item(const Plan& pl, int per_xcd, int npt, int hpw, int nslice, Item& it) {
    const int64_t item = xcd_item(per_xcd);
    if (item >= (int64_t)pl.nchunk_ub * pl.G * nslice * npt) return false;
    it.pt = (int)(item % npt);
    int64_t r = item / npt;
    const int slice = (int)(r % nslice);
    r /= nslice;
    it.g = (int)(r % pl.G);
    it.k = (int)(r / pl.G);
    it.h0 = it.g * pl.hpg + slice * hpw;
    it.nh = min(hpw, pl.hpg - slice * hpw);
    return it.nh > 0;
}

// ------------------------------------------------------------------ chunk_state
// Workgroup per item; for each head h of the slice:
//   S_k[p][n] = sum_t exp(cs_last - cs_t) dt_t x[t][p] B[t][n]
// for p in the tile and every n < N, as a (32 x Q) . (Q x NT) MFMA product:
// A = (x w)^T from LDS (hi/lo pair when split), B = the B^T rows the cb
// kernel wrote, held in registers for the whole slice (one wave per 32-wide
// n-tile).  The weight w_t = exp(cs_last - cs_t) dt_t <= dt_t never overflows.
template <typename T>
__host__ __device__ constexpr size_t chunk_state_stage_bytes(int Q) {
    return (size_t)(Split<T>::on ? 2 : 1) * 32 * (Q + 8) * sizeof(T);
}

// staging tile, then one 32 x 32 fp32 output tile per wave (NT/32 waves)
template <typename T>
__host__ __device__ constexpr size_t chunk_state_lds_bytes(int NT, int Q) {
    return chunk_state_stage_bytes<T>(Q) + (size_t)(NT / 32) * 32 * 36 * 4;
}

template <typename T, int NT, int NTI>
__global__ __launch_bounds__(2 * NT, (Split<T>::on && NT >= 128) ? 3 : 1) void ssd_chunk_state_kernel(
    Plan pl, int per_xcd, int npt, int hpw, int nslice, const T* __restrict__ x, const float* __restrict__ wst,
    const T* __restrict__ bt, float* __restrict__ states) {
    extern __shared__ __align__(16) char smem[];
    constexpr bool SP = Split<T>::on;
    constexpr int Q = 32 * NTI, LP = Q + 8;
    constexpr int NTHR = 2 * NT;  // one wave per n-tile
    constexpr int UPT = (Q + NTHR - 1) / NTHR;
    typedef typename Tr<T>::v8 v8;
    Item it;
    if (!decode_item(pl, per_xcd, npt, hpw, nslice, it)) return;
    const ChunkDesc cd = uniform_desc(chunk_desc(pl, it.k));
    if (cd.seq < 0) return;
    const int P = pl.P, N = pl.N, H = pl.H, G = pl.G, pt = it.pt, k = it.k;
    const int tid = threadIdx.x;
    const int nt = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, half = lane >> 5, col = lane & 31;
    T* xh = (T*)smem;
    T* xl = xh + 32 * LP;
    float* ep = (float*)(smem + chunk_state_stage_bytes<T>(Q)) + nt * (kEpBytes / 4);
    v8 bf[Q / 16];
    const T* bfr = bt + ((size_t)k * G + it.g) * NT * Q + bt_frag(Q, nt, 0, lane);
#pragma unroll
    for (int s = 0; s < Q / 16; ++s) bf[s] = Tr<T>::ld8(bfr + 512 * s);
    XUnit<T> xu[UPT];
    const __amdgpu_buffer_rsrc_t rx = chunk_x_rsrc(x, cd, H, P);
    auto prefetch = [&](int h) {
        const float* wsk = wst + ((size_t)k * H + h) * Q;
#pragma unroll
        for (int i = 0; i < UPT; ++i)
            if (Q % NTHR == 0 || i * NTHR + tid < Q)
                load_xunit<T, Q>(xu[i], rx, cd, H, P, h, pt, i * NTHR + tid, wsk);
    };
    prefetch(it.h0);
    // the B^T fragments and the first head's inputs are needed at once; past
    // this point the loop's own loads are the only ones in flight
    __builtin_amdgcn_s_waitcnt(0);
    const T* arow = xh + col * LP + 8 * half;
    const T* lrow = xl + col * LP + 8 * half;
    const int hl = it.h0 + it.nh - 1;
    for (int i = 0; i < it.nh; ++i) {
        const int h = it.h0 + i;
#pragma unroll
        for (int u = 0; u < UPT; ++u)
            if (Q % NTHR == 0 || u * NTHR + tid < Q) store_xunit<T, SP>(xu[u], xh, xl, LP);
        __syncthreads();
        // unconditional (the last head repeats itself), so the wait counts
        // never cover a path without these loads
        prefetch(min(h + 1, hl));
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < Q / 16; ++s) {
            mma16(acc, Tr<T>::ld8(arow + 16 * s), bf[s]);
            if (SP) mma16(acc, Tr<T>::ld8(lrow + 16 * s), bf[s]);
        }
        // acc: row p = 32pt + acc_row(v), column n.  Out through the wave's
        // LDS tile as 16-byte rows; every lane stores, rows past P and
        // columns past N go beyond the descriptor's range and are dropped
#pragma unroll
        for (int v = 0; v < 16; ++v) ep[acc_row(v, lane) * kEpPitch + col] = acc[v];
        const __amdgpu_buffer_rsrc_t rs =
            buffer_rsrc(states + ((size_t)k * H + h) * P * N, (uint32_t)(P * N * sizeof(float)));
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int pr = (lane >> 3) + 8 * i4, c4 = 4 * (lane & 7);
            const f32x4 r = *(const f32x4*)(ep + pr * kEpPitch + c4);
            const bool ok = 32 * pt + pr < P && 32 * nt + c4 < N;
            buffer_store4<float>(r, rs, ok ? ((32 * pt + pr) * N + 32 * nt + c4) * 4 : kOutOfRange);
        }
        __syncthreads();  // the next head overwrites the LDS tile
    }
}

// ------------------------------------------------------------------ chunk_state with state passing
// Workgroup per (sequence s, head h, tile pt of 32 columns of P); it walks the
// sequence's chunks in order and keeps the running state in the MFMA
// accumulators (row p = 32pt + acc_row(v), column n as in chunk_state):
//   acc <- initial state (or 0)
//   per chunk k:  slot_k <- acc;   acc <- exp(cs_last,k) acc + S_k
// with S_k the chunk_state contraction accumulated straight onto the decayed
// state, and acc written as the final state at the end.  The slots then hold
// the states entering each chunk, as state_passing leaves them, without the
// S_k round trip through memory.  Each wave holds its n-tile's B^T fragments
// of the chunk in registers; the next chunk's x, weights and B^T are loaded
// while the current one computes.
template <typename T, int NT, int NTI>
__global__ __launch_bounds__(2 * NT, (Split<T>::on && NT >= 128) ? 3 : 1) void ssd_chunk_state_passing_kernel(
    Plan pl, int per_xcd, int npt, const T* __restrict__ x, const float* __restrict__ cs,
    const float* __restrict__ wst, const T* __restrict__ bt, float* __restrict__ states,
    const float* __restrict__ init, float* __restrict__ fin) {
    extern __shared__ __align__(16) char smem[];
    constexpr bool SP = Split<T>::on;
    constexpr int Q = 32 * NTI, LP = Q + 8;
    constexpr int NTHR = 2 * NT;  // one wave per n-tile
    constexpr int UPT = (Q + NTHR - 1) / NTHR;
    typedef typename Tr<T>::v8 v8;
    const int64_t item = xcd_item(per_xcd);
    if (item >= (int64_t)pl.nseq * pl.H * npt) return;
    const int pt = (int)(item % npt);
    const int h = (int)((item / npt) % pl.H);
    const int s = (int)(item / npt / pl.H);
    const int P = pl.P, N = pl.N, H = pl.H, G = pl.G, g = h / pl.hpg;
    const int tid = threadIdx.x;
    const int nt = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, half = lane >> 5, col = lane & 31;
    T* xh = (T*)smem;
    T* xl = xh + 32 * LP;
    float* ep = (float*)(smem + chunk_state_stage_bytes<T>(Q)) + nt * (kEpBytes / 4);
    const size_t hoff = ((size_t)s * H + h) * P * N;
    const uint32_t hbytes = (uint32_t)(P * N * sizeof(float));
    // 16-byte rows of the wave's 32 x 32 tile: row pr, columns c4 .. c4+3
    const int c4 = 4 * (lane & 7);
    auto row_off = [&](int i4) {
        const int pr = (lane >> 3) + 8 * i4;
        const bool ok = 32 * pt + pr < P && 32 * nt + c4 < N;
        return ok ? ((32 * pt + pr) * N + 32 * nt + c4) * 4 : kOutOfRange;
    };
    auto put_state = [&](const f32x16& acc, float* dst) {
#pragma unroll
        for (int v = 0; v < 16; ++v) ep[acc_row(v, lane) * kEpPitch + col] = acc[v];
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(dst, hbytes);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 r = *(const f32x4*)(ep + ((lane >> 3) + 8 * i4) * kEpPitch + c4);
            buffer_store4<float>(r, rs, row_off(i4));
        }
    };
    f32x16 acc = {};
    if (init) {
        // the initial state into the accumulator layout through the LDS tile
        const __amdgpu_buffer_rsrc_t ri = buffer_rsrc(init + hoff, hbytes);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(ri, row_off(i4), 0, 0);
            *(f32x4*)(ep + ((lane >> 3) + 8 * i4) * kEpPitch + c4) = __builtin_bit_cast(f32x4, r);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = ep[acc_row(v, lane) * kEpPitch + col];
    }
    const SeqExtent se = seq_extent(pl, s);
    const int nck = __builtin_amdgcn_readfirstlane(se.nchunks);
    if (nck > 0) {
        const int k0 = __builtin_amdgcn_readfirstlane(se.chunk0);
        const int slen = __builtin_amdgcn_readfirstlane(se.len);
        const int64_t srow = (int64_t)__builtin_amdgcn_readfirstlane((int)se.row0);
        auto desc = [&](int c) {
            ChunkDesc d;
            d.seq = s;
            d.idx = c;
            d.row0 = srow + (int64_t)c * Q;
            d.len = min(Q, slen - c * Q);
            return d;
        };
        // B^T fragments of the chunk: uniform base, one lane offset for every chunk
        const int boff = bt_frag(Q, nt, 0, lane) * (int)sizeof(T);
        v8 bf[Q / 16];
        auto load_b = [&](int k) {
            const __amdgpu_buffer_rsrc_t rb =
                buffer_rsrc(bt + ((size_t)k * G + g) * NT * Q, (uint32_t)(NT * Q * sizeof(T)));
#pragma unroll
            for (int i = 0; i < Q / 16; ++i) bf[i] = buffer_ld8<T>(rb, boff + 512 * i * (int)sizeof(T));
        };
        XUnit<T> xu[UPT];
        float clast = 0.f;
        auto prefetch = [&](int c) {
            const int k = k0 + c;
            const ChunkDesc d = desc(c);
            const __amdgpu_buffer_rsrc_t rx = chunk_x_rsrc(x, d, H, P);
            const float* wsk = wst + ((size_t)k * H + h) * Q;
#pragma unroll
            for (int i = 0; i < UPT; ++i)
                if (Q % NTHR == 0 || i * NTHR + tid < Q)
                    load_xunit<T, Q>(xu[i], rx, d, H, P, h, pt, i * NTHR + tid, wsk);
            clast = cs[((size_t)k * H + h) * Q + Q - 1];
        };
        load_b(k0);
        prefetch(0);
        // everything above is needed at once; past this point the loop's own
        // loads and stores are the only ones in flight
        __builtin_amdgcn_s_waitcnt(0);
        const T* arow = xh + col * LP + 8 * half;
        const T* lrow = xl + col * LP + 8 * half;
        for (int c = 0; c < nck; ++c) {
            const int k = k0 + c;
            const float dec = __expf(clast);
#pragma unroll
            for (int u = 0; u < UPT; ++u)
                if (Q % NTHR == 0 || u * NTHR + tid < Q) store_xunit<T, SP>(xu[u], xh, xl, LP);
            __syncthreads();
            // unconditional (the last chunk repeats itself), so the wait
            // counts never cover a path without these loads
            const int cn = min(c + 1, nck - 1);
            prefetch(cn);
            put_state(acc, states + ((size_t)k * H + h) * P * N);
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] *= dec;
#pragma unroll
            for (int i = 0; i < Q / 16; ++i) {
                mma16(acc, Tr<T>::ld8(arow + 16 * i), bf[i]);
                if (SP) mma16(acc, Tr<T>::ld8(lrow + 16 * i), bf[i]);
            }
            load_b(k0 + cn);
            __syncthreads();  // the next chunk overwrites the staging tile
        }
    }
    if (fin) put_state(acc, fin + hoff);
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
// entering the chunk (written by the state walk or by state_passing).
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

// Table entries of token q, computed from values loaded early (TabIn).
struct TabIn {
    float a, d, ce, c0;  // cs_q, dt_q, cs at the end and before the start of q's block
    float gc0, gce;      // block tid (tid < Q/32): cs before its start and at its end
};

template <int Q>
__device__ inline void load_tab(TabIn& ti, const float* __restrict__ csk, const float* __restrict__ dtk,
                                int tid) {
    const int q = tid < Q ? tid : Q - 1;
    ti.a = csk[q];
    ti.d = dtk[q];
    ti.ce = csk[q | 31];
    const int s = (q & ~31) - 1;
    ti.c0 = s >= 0 ? csk[s] : 0.f;
    const int j = tid < Q / 32 ? tid : 0;
    ti.gc0 = j > 0 ? csk[32 * j - 1] : 0.f;
    ti.gce = csk[32 * j + 31];
}

template <int Q>
__device__ inline void store_tab(const ChunkTables& tb, const TabIn& ti, int tid) {
    if (tid < Q) {
        tb.cs[tid] = ti.a;
        tb.dt[tid] = ti.d;
        tb.wb[tid] = __expf(ti.ce - ti.a) * ti.d;
        tb.ul[tid] = __expf(ti.a - ti.c0);
        tb.ue[tid] = __expf(fminf(ti.a - ti.ce, kFastBlockDecay));
    }
    if (tid < Q / 32) {
        tb.gam[tid] = __expf(ti.gce - ti.gc0);
        tb.fast[tid] = (ti.gc0 - ti.gce) < kFastBlockDecay ? 1 : 0;
    }
}

// Staging unit of the chunk scan: 2 tokens x 8 columns of x (one per thread
// of the workgroup), written as is to the row tile xr[t][p] (for the D x
// term) and, scaled by wb, transposed to the hi tile.  16 consecutive units
// share the column group, so a wave's transposed LDS writes fall on distinct
// banks.
template <typename T>
struct XPair {
    typename Tr<T>::v8 raw[2];
    float c0, c1, d0, d1, ce;
    int pb, k0;
    bool pok;
};

template <typename T>
__device__ inline void load_xpair(XPair<T>& xp, const T* __restrict__ x, const ChunkDesc& cd, int H, int P,
                                  int h, int pt, int u, const float* __restrict__ csk,
                                  const float* __restrict__ dtk) {
    xp.pb = (u >> 4) & 3;
    xp.k0 = 2 * ((u & 15) + 16 * (u >> 6));
    const int pc = 32 * pt + 8 * xp.pb;
    xp.pok = pc < P;
    const int p0 = xp.pok ? pc : 0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int kk = min(xp.k0 + r, cd.len - 1);
        xp.raw[r] = Tr<T>::ld8(x + ((cd.row0 + kk) * H + h) * P + p0);
    }
    xp.c0 = csk[xp.k0];
    xp.c1 = csk[xp.k0 + 1];
    xp.d0 = dtk[xp.k0];
    xp.d1 = dtk[xp.k0 + 1];
    xp.ce = csk[xp.k0 | 31];
}

template <typename T>
__device__ inline void store_xpair(const XPair<T>& xp, const ChunkDesc& cd, T* xh, int LP, T* xr, int XRP) {
    Tr<T>::st8(xr + xp.k0 * XRP + 8 * xp.pb, xp.raw[0]);
    Tr<T>::st8(xr + (xp.k0 + 1) * XRP + 8 * xp.pb, xp.raw[1]);
    const float w0 = (xp.pok && xp.k0 < cd.len) ? __expf(xp.ce - xp.c0) * xp.d0 : 0.f;
    const float w1 = (xp.pok && xp.k0 + 1 < cd.len) ? __expf(xp.ce - xp.c1) * xp.d1 : 0.f;
    const f32x8 f0 = Tr<T>::widen(xp.raw[0]) * w0;
    const f32x8 f1 = Tr<T>::widen(xp.raw[1]) * w1;
    typedef T t2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < 8; ++i) *(t2*)(xh + (8 * xp.pb + i) * LP + xp.k0) = t2{(T)f0[i], (T)f1[i]};
}

// hi/lo copy of the fp32 state rows p in [32pt, 32pt+32) as the B operand of
// the state term: sh[pl][n] (+ sl[pl][n] when split), pitch NS, zero past P
// and past N.  Loaded early (load_state_rows), written after (store_state_rows).
template <int NT, int NTHR>
struct StateRows {
    static constexpr int NQ = NT / 4;
    static constexpr int U = 32 * NQ;
    static constexpr int PER = (U + NTHR - 1) / NTHR;
    f32x4 v[PER];
};

// The loads only move data (addresses outside the tile are clamped in bounds);
// the zeroing happens when the rows are written to LDS, so no instruction
// between the load and its consumer needs the loaded value.
template <int NT, int NTHR>
__device__ inline void load_state_rows(StateRows<NT, NTHR>& sr, const float* __restrict__ src, int P, int N,
                                       int pt, int tid) {
    typedef StateRows<NT, NTHR> S;
#pragma unroll
    for (int i = 0; i < S::PER; ++i) {
        const int u = i * NTHR + tid;
        const int r = u / S::NQ, n = 4 * (u % S::NQ);
        const int p = 32 * pt + r;
        const bool ok = (S::U % NTHR == 0 || u < S::U) && p < P && n < N;
        sr.v[i] = *(const f32x4*)(src + (ok ? (size_t)p * N + n : 0));
    }
}

template <typename T, int NT, int NTHR>
__device__ inline void store_state_rows(const StateRows<NT, NTHR>& sr, T* sh, T* sl, int NS, int P, int N, int pt,
                                        int tid) {
    typedef typename Tr<T>::v4 v4;
    typedef StateRows<NT, NTHR> S;
#pragma unroll
    for (int i = 0; i < S::PER; ++i) {
        const int u = i * NTHR + tid;
        if (S::U % NTHR != 0 && u >= S::U) break;
        const int r = u / S::NQ, n = 4 * (u % S::NQ);
        const bool ok = 32 * pt + r < P && n < N;
        const f32x4 v = ok ? sr.v[i] : f32x4{};
        const v4 hi = Tr<T>::narrow4(v);
        Tr<T>::st4raw(sh + r * NS + n, hi);
        if (Split<T>::on) Tr<T>::st4raw(sl + r * NS + n, Tr<T>::narrow4(v - Tr<T>::widen4(hi)));
    }
}

// Row pitch (elements) of the raw x tile xr[t][p]: 32 columns plus 16 bytes.
template <typename T>
__host__ __device__ constexpr int xr_pitch() { return 32 + 16 / (int)sizeof(T); }

// One staging buffer: tables | (x wb)^T hi [32][Q+8] | state hi, lo [32][NT+8] | x [Q][xr_pitch]
template <typename T>
__host__ __device__ constexpr size_t chunk_scan_lds_bytes(int NT, int Q) {
    return tables_bytes(Q) + (size_t)32 * (Q + 8) * sizeof(T) +
           (size_t)(Split<T>::on ? 2 : 1) * 32 * (NT + 8) * sizeof(T) + (size_t)Q * xr_pitch<T>() * sizeof(T);
}

// Two staging buffers (stage head i+1 while head i computes) when they fit
// in LDS next to the per-wave output tiles.
template <typename T>
__host__ __device__ constexpr int chunk_scan_buffers(int NT, int Q) {
    return 2 * chunk_scan_lds_bytes<T>(NT, Q) + (Q / 32) * 32 * 36 * 4 <= 160 * 1024 ? 2 : 1;
}

template <typename T>
__host__ __device__ constexpr size_t chunk_scan_total_lds(int NT, int Q) {
    return chunk_scan_buffers<T>(NT, Q) * chunk_scan_lds_bytes<T>(NT, Q) + (size_t)(Q / 32) * 32 * 36 * 4;
}



// Per-wave operands of output block TI that do not depend on the head:
// C.B^T rows of the block (A operand of the intra-chunk term) and C rows (A
// operand of the state term).
template <typename T, int NT, int TI>
struct BlockOps {
    typename Tr<T>::v8 ga[TI + 1][2];
    typename Tr<T>::v8 ca[NT / 16];
};

// One head's output block TI for the calling wave.  xrow/srow/lrow point to
// this lane's row of the LDS tiles, xcol to this lane's column of the raw x
// tile xr (pitch XRP), ep to the wave's output tile.  yoff is the byte offset
// of (row 32 TI, head h, column 32 pt) from the chunk's first row of y; pcols
// the tile's columns inside P.  No global loads: the block reads LDS and
// registers only; its outputs leave through the LDS tile as 16-byte rows.
template <typename T, typename TY, int NT, int NTI, int TI>
__device__ __forceinline__ void scan_block(const BlockOps<T, NT, TI>& o, const ChunkTables& tb, const T* xrow,
                                           const T* srow, const T* lrow, const T* xcol, float* ep,
                                           bool has_state, __amdgpu_buffer_rsrc_t ry, int yoff, int HP, int len,
                                           int pcols, float Dh) {
    constexpr bool SP = Split<T>::on;
    constexpr int XRP = xr_pitch<T>();
    typedef typename Tr<T>::v8 v8;
    const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    const int ta = 32 * TI + col;  // this lane's A row
    // two independent accumulation chains, so their MFMAs and the Horner
    // scaling overlap: the state term (hi and lo) and the intra-chunk Horner
    // scheme, joined with the state term's decay exp(cs) at the scheme's end
    f32x16 sacc = {};
    if (has_state) {
#pragma unroll
        for (int s = 0; s < NT / 16; ++s) {
            mma16(sacc, o.ca[s], Tr<T>::ld8(srow + 16 * s));
            if (SP) mma16(sacc, o.ca[s], Tr<T>::ld8(lrow + 16 * s));
        }
    }
    const bool fast = tb.fast[TI] != 0;
    // the Horner scheme as two interleaved chains (even and odd blocks), each
    // stepping two blocks at a time with the product of their decays; the
    // chain that does not end at the last included block K takes gam[K]
    f32x16 ce = {}, co = {};
#pragma unroll
    for (int kj = 0; kj <= TI; ++kj) {
        if (kj < TI || fast) {
            f32x16& ch = (kj & 1) ? co : ce;
            if (kj >= 2) ch *= tb.gam[kj - 1] * tb.gam[kj];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mma16(ch, o.ga[kj][ks], Tr<T>::ld8(xrow + 32 * kj + 16 * ks));
        }
    }
    const int K = fast ? TI : TI - 1;  // last block in the scheme
    f32x16 acc;
    if (K < 1) {
        acc = ce;  // at most block 0 (K = -1: no block, ce is zero)
    } else {
        const float gk = tb.gam[K];
        if (K & 1) acc = co + gk * ce;
        else acc = ce + gk * co;
    }
    if (has_state) {
        // decay of the state term up to where the scheme stopped: the end of
        // block TI (fast) or the end of block TI-1
        const int e = fast ? 32 * TI + 31 : 32 * TI - 1;
        const float dec = e >= 0 ? __expf(tb.cs[e]) : 1.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] += dec * sacc[v];
    }
    const float* scale = fast ? tb.ue : tb.ul;
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) {
        const f32x4 u = *(const f32x4*)(scale + 32 * TI + 8 * vg + 4 * half);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * vg + j] *= u[j];
    }
    if (!fast) {
        // decay across this block beyond the fast range: exact factors, raw x
        // (the C.B^T tile is already zero above its diagonal)
        const float cst = tb.cs[ta];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int k0 = 32 * TI + 16 * ks + 8 * half;
            const f32x8 gv = Tr<T>::widen(o.ga[TI][ks]);
            f32x8 m;
            v8 xb;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int kk = k0 + i;
                m[i] = gv[i] * (__expf(fminf(cst - tb.cs[kk], 0.f)) * tb.dt[kk]);
                xb[i] = xcol[kk * XRP];
            }
            mma16(acc, Tr<T>::narrow(m), xb);
        }
    }
    // transpose through the wave's LDS tile: lane (column p) writes its 16
    // rows, then each lane reads 4 consecutive columns of one row; LDS
    // operations of one wave complete in order, so no barrier is needed
#pragma unroll
    for (int v = 0; v < 16; ++v) ep[acc_row(v, lane) * kEpPitch + col] = acc[v];
    const T* xr0 = xcol - col;  // raw x tile, row 0, column 0
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int tr = (lane >> 3) + 8 * it, c4 = 4 * (lane & 7);
        const f32x4 xv = Tr<T>::ld4(xr0 + (32 * TI + tr) * XRP + c4);
        const f32x4 r = *(const f32x4*)(ep + tr * kEpPitch + c4) + Dh * xv;
        // every lane stores: an output outside the chunk or past P gets an
        // offset beyond the descriptor's range, which the hardware drops;
        // no branch, so the wait counters stay exact for the next loads
        const bool ok = 32 * TI + tr < len && c4 < pcols;
        buffer_store4<TY>(r, ry, ok ? yoff + (tr * HP + c4) * (int)sizeof(TY) : kOutOfRange);
    }
}

// Wave w of the workgroup computes output block blk(w) of every head of the
// slice.  With 8 blocks the blocks are ordered so that waves w and w+4 (which
// the hardware places on the same SIMD) hold causal work that sums to 9
// block products.
__host__ __device__ constexpr int scan_block_of_wave(int NTI, int w) {
    return NTI == 8 ? (w < 4 ? w : 11 - w) : w;
}

// With 8 blocks, the four waves of blocks 0-3 (the least causal work) stage
// every head's LDS inputs on their own, so the waves of blocks 4-7, which set
// the pace, only compute; with fewer blocks every wave stages a share.
__host__ __device__ constexpr bool scan_stager(int NTI, int TI) { return NTI != 8 || TI < 4; }
__host__ __device__ constexpr int scan_stage_threads(int NTI) { return NTI == 8 ? 256 : 64 * NTI; }

template <typename T, typename TY, int NT, int NTI, int TI>
__device__ __forceinline__ void scan_wave(const Plan& pl, const Item& it, const ChunkDesc& cd, char* smem,
                                          const T* __restrict__ x, const float* __restrict__ cs,
                                          const float* __restrict__ dtc, const T* __restrict__ Cm,
                                          const T* __restrict__ cb, const float* __restrict__ D,
                                          const float* __restrict__ states, bool has_state, TY* __restrict__ y) {
    constexpr int Q = 32 * NTI, LP = Q + 8, NS = NT + 8;
    constexpr bool STAGER = scan_stager(NTI, TI);
    constexpr int NTHR = scan_stage_threads(NTI);  // threads that stage
    constexpr int XPT = 64 * NTI / NTHR;           // x units per staging thread
    const int P = pl.P, N = pl.N, H = pl.H, G = pl.G, k = it.k, pt = it.pt;
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
    // the group's operands of this wave's block, once for the whole slice
    BlockOps<T, NT, TI> o;
    {
        const int ta = 32 * TI + col;
        const T* grow = cb + ((size_t)k * G + it.g) * Q * Q + (size_t)ta * Q + 8 * half;
#pragma unroll
        for (int kj = 0; kj <= TI; ++kj)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) o.ga[kj][ks] = Tr<T>::ld8(grow + 32 * kj + 16 * ks);
        if (has_state) {
            const T* crow = Cm + ((cd.row0 + min(ta, cd.len - 1)) * G + it.g) * N;
#pragma unroll
            for (int s = 0; s < NT / 16; ++s) o.ca[s] = Tr<T>::ld8(crow + min(16 * s + 8 * half, N - 8));
        }
    }
    const int HP = H * P;
    const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(y + cd.row0 * HP, (uint32_t)(cd.len * HP * sizeof(TY)));
    // per-head inputs, loaded one head ahead by the staging waves
    TabIn tin;
    XPair<T> xp[XPT];
    StateRows<NT, NTHR> sr;
    auto prefetch = [&](int h) {
        const float* csk = cs + ((size_t)k * H + h) * Q;
        const float* dtk = dtc + ((size_t)k * H + h) * Q;
        load_tab<Q>(tin, csk, dtk, tid);
#pragma unroll
        for (int r = 0; r < XPT; ++r) load_xpair(xp[r], x, cd, H, P, h, pt, tid + r * NTHR, csk, dtk);
        load_state_rows<NT, NTHR>(sr, states + ((size_t)k * H + h) * P * N, P, N, pt, tid);
    };
    constexpr size_t BUF = chunk_scan_lds_bytes<T>(NT, Q);
    constexpr int XRP = xr_pitch<T>();
    // buffer b: tables | xh | sh | sl | xr
    auto tile = [&](int b, int which) -> T* {
        char* base = smem + b * BUF;
        T* xh = (T*)(base + tables_bytes(Q));
        T* sh = xh + 32 * LP;
        if (which == 0) return xh;
        if (which == 1) return sh;
        if (which == 2) return sh + 32 * NS;
        return sh + (Split<T>::on ? 2 : 1) * 32 * NS;
    };
    auto stage = [&](int b) {
        store_tab<Q>(carve_tables(smem + b * BUF, Q), tin, tid);
#pragma unroll
        for (int r = 0; r < XPT; ++r) store_xpair(xp[r], cd, tile(b, 0), LP, tile(b, 3), XRP);
        if (has_state) store_state_rows<T, NT, NTHR>(sr, tile(b, 1), tile(b, 2), NS, P, N, pt, tid);
    };
    float* ep = (float*)(smem + chunk_scan_buffers<T>(NT, Q) * BUF) + (tid >> 6) * (kEpBytes / 4);
    const int pcols = P - 32 * pt;
    auto compute = [&](int b, int h) {
        const int yoff = (32 * TI * HP + h * P + 32 * pt) * (int)sizeof(TY);
        scan_block<T, TY, NT, NTI, TI>(o, carve_tables(smem + b * BUF, Q), tile(b, 0) + col * LP + 8 * half,
                                       tile(b, 1) + col * NS + 8 * half, tile(b, 2) + col * NS + 8 * half,
                                       tile(b, 3) + col, ep, has_state, ry, yoff, HP, cd.len, pcols, D[h]);
    };
    if (STAGER) prefetch(it.h0);
    if constexpr (chunk_scan_buffers<T>(NT, Q) == 2) {
        // head i computes from buffer i%2 while head i+1 is staged into the
        // other one: one workgroup barrier per head
        // the loads of every iteration are issued unconditionally (past the
        // slice's last head they repeat it), so the compiler's wait counts
        // never have to cover a path without them
        const int hl = it.h0 + it.nh - 1;
        if (STAGER) stage(0);
        __syncthreads();
        // the block operands loaded before the loop are complete here; saying
        // so keeps their loads out of the loop's wait counts
        __builtin_amdgcn_s_waitcnt(0);
        if (STAGER) prefetch(min(it.h0 + 1, hl));
        for (int i = 0; i < it.nh; ++i) {
            const int h = it.h0 + i;
            compute(i & 1, h);
            if (STAGER) {
                stage((i + 1) & 1);
                prefetch(min(h + 2, hl));
            }
            __syncthreads();  // buffer i%2 is restaged at i+1; buffer (i+1)%2 is read at i+1
        }
    } else {
        const int hl = it.h0 + it.nh - 1;
        for (int i = 0; i < it.nh; ++i) {
            const int h = it.h0 + i;
            if (STAGER) stage(0);
            __syncthreads();
            if (STAGER) prefetch(min(h + 1, hl));
            compute(0, h);
            __syncthreads();  // the next head overwrites the LDS tiles
        }
    }
}

// Workgroup per item (chunk, group, head slice, 32-column tile), one wave per
// 32-token output block.  Per head: the decay tables, (x wb)^T and the
// entering state's hi/lo pair are staged in LDS (loaded while the previous
// head computed), then every wave computes its block.
template <typename T, typename TY, int NT, int NTI>
__global__ __launch_bounds__(64 * NTI) void ssd_chunk_scan_kernel(
    Plan pl, int per_xcd, int npt, int hpw, int nslice, const T* __restrict__ x, const float* __restrict__ cs,
    const float* __restrict__ dtc, const T* __restrict__ Cm, const T* __restrict__ cb,
    const float* __restrict__ D, const float* __restrict__ init, const float* __restrict__ states,
    TY* __restrict__ y) {
    extern __shared__ __align__(16) char smem[];
    Item it;
    if (!decode_item(pl, per_xcd, npt, hpw, nslice, it)) return;
    const ChunkDesc cd = uniform_desc(chunk_desc(pl, it.k));
    if (cd.seq < 0) return;
    const bool has_state = cd.idx > 0 || init != nullptr;
    // wave index as a scalar: each wave takes one branch below
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#define SSD_WAVE(w)                                                                                   \
    case w:                                                                                           \
        if constexpr (w < NTI)                                                                        \
            scan_wave<T, TY, NT, NTI, scan_block_of_wave(NTI, w)>(pl, it, cd, smem, x, cs, dtc, Cm, cb, D, \
                                                                  states, has_state, y);              \
        break;
    switch (wave) {
        SSD_WAVE(0) SSD_WAVE(1) SSD_WAVE(2) SSD_WAVE(3) SSD_WAVE(4) SSD_WAVE(5) SSD_WAVE(6) SSD_WAVE(7)
        default: break;
    }
#undef SSD_WAVE
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
    float* wst = (float*)(ws + lay.wst);
    T* cbm = (T*)(ws + lay.cb);
    T* bt = (T*)(ws + lay.bt);
    float* states = (float*)(ws + lay.states);
    hipError_t err;
    auto mark = [&](int i) -> hipError_t { return marks ? hipEventRecord(marks[i], stream) : hipSuccess; };
    const int npt = (pl.P + 31) / 32;
    // chunk_scan items: (chunk, group, slice of a.hpw heads, column tile)
    const int nslice = (pl.hpg + a.hpw - 1) / a.hpw;
    const int64_t nitems = (int64_t)pl.nchunk_ub * pl.G * nslice * npt;
    const int per_xcd = (int)((nitems + 7) / 8);
    if ((err = mark(0)) != hipSuccess) return err;
    if (!pl.dense && pl.nseq > 0) {
        hipLaunchKernelGGL(ssd_plan_kernel, dim3(1), dim3(kThreads), 0, stream, pl);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(1)) != hipSuccess) return err;
    if (pl.nchunk_ub > 0) {
        hipLaunchKernelGGL(ssd_cumsum_kernel, dim3(pl.nchunk_ub, (pl.H + kCumHeads - 1) / kCumHeads), dim3(kThreads), 0,
                           stream, pl, a.dt, a.A, cs, dtc, a.path == kPathScanWalk ? nullptr : wst, a.act);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(2)) != hipSuccess) return err;
    if (pl.nchunk_ub > 0) {
        // the whole-chunk form needs enough (chunk, group) pairs to fill the
        // chip; below that the tile-per-wave form's 36x more workgroups finish first
        if (cb_chunk_lds_bytes<T>(NT, Q) <= 160 * 1024 && (int64_t)pl.nchunk_ub * pl.G >= 256) {
            auto* k1 = ssd_cb_chunk_kernel<T, NT>;
            const size_t lds = cb_chunk_lds_bytes<T>(NT, Q);
            if ((err = allow_lds(k1, lds)) != hipSuccess) return err;
            hipLaunchKernelGGL(k1, dim3(pl.nchunk_ub, pl.G), dim3(256), lds, stream, pl, B, C, cbm, bt);
        } else {
            // few chunks, or a staged chunk that would not fit (fp32, dstate > 128, 256-token chunks)
            auto* k1 = ssd_cb_kernel<T, NT>;
            hipLaunchKernelGGL(k1, dim3(pl.nchunk_ub, pl.G, NTI * (NTI + 1) / 2), dim3(64), cb_lds_bytes<T>(NT),
                               stream, pl, B, C, cbm, bt);
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(3)) != hipSuccess) return err;
    if (a.path == kPathScanWalk) {
        // one launch: states, their passing and y, per (sequence, group, slice of units)
        if ((err = mark(4)) != hipSuccess) return err;
        if ((err = mark(5)) != hipSuccess) return err;
        if ((err = mark(6)) != hipSuccess) return err;
        WalkArgs wa;
        wa.x = a.x;
        wa.cs = cs;
        wa.dtc = dtc;
        wa.tail = (float*)(ws + lay.tail);
        wa.C = a.C;
        wa.cb = cbm;
        wa.bt = bt;
        wa.D = a.D;
        wa.init = a.init;
        wa.final_state = a.final_state;
        wa.y = a.y;
        wa.npt = npt;
        wa.nslice = a.walk_nslice;
        wa.nus = a.walk_nus;
        const int64_t nwalk = (int64_t)pl.nseq * pl.G * a.walk_nslice;
        walk_grid(nwalk, &wa.run, &wa.per_xcd);
        wa.y_f32 = a.y_f32;
        if ((err = launch_scan_walk(pl, wa, stream)) != hipSuccess) return err;
        return mark(7);
    }
    if (a.path == kPathStateWalk) {
        // one launch walks every sequence: chunk states and the passing between them
        const int64_t nfused = (int64_t)pl.nseq * pl.H * npt;
        const int fper_xcd = (int)((nfused + 7) / 8);
        if (nfused > 0) {
            auto* k2 = ssd_chunk_state_passing_kernel<T, NT, NTI>;
            const size_t lds = chunk_state_lds_bytes<T>(NT, Q);
            if ((err = allow_lds(k2, lds)) != hipSuccess) return err;
            hipLaunchKernelGGL(k2, dim3(8 * fper_xcd), dim3(2 * NT), lds, stream, pl, fper_xcd, npt, x, cs,
                               wst, bt, states, a.init, a.final_state);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        if ((err = mark(4)) != hipSuccess) return err;
    } else {
        // chunk_state items: the same, with slices of a.hpw_state heads
        const int nslice_s = (pl.hpg + a.hpw_state - 1) / a.hpw_state;
        const int64_t nitems_s = (int64_t)pl.nchunk_ub * pl.G * nslice_s * npt;
        const int per_xcd_s = (int)((nitems_s + 7) / 8);
        if (nitems_s > 0) {
            auto* k2 = ssd_chunk_state_kernel<T, NT, NTI>;
            const size_t lds = chunk_state_lds_bytes<T>(NT, Q);
            if ((err = allow_lds(k2, lds)) != hipSuccess) return err;
            hipLaunchKernelGGL(k2, dim3(8 * per_xcd_s), dim3(2 * NT), lds, stream, pl, per_xcd_s, npt,
                               a.hpw_state, nslice_s, x, wst, bt, states);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        if ((err = mark(4)) != hipSuccess) return err;
        if (pl.nseq > 0) {
            const int nblk = (pl.P * pl.N / 4 + kThreads - 1) / kThreads;
            hipLaunchKernelGGL(ssd_state_passing_kernel, dim3((unsigned)((int64_t)pl.nseq * pl.H * nblk)),
                               dim3(kThreads), 0, stream, pl, nblk, cs, states, a.init, a.final_state);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
    }
    if ((err = mark(5)) != hipSuccess) return err;
    if (nitems > 0) {
        auto* k4 = ssd_chunk_scan_kernel<T, TY, NT, NTI>;
        const size_t lds = chunk_scan_total_lds<T>(NT, Q);
        if ((err = allow_lds(k4, lds)) != hipSuccess) return err;
        hipLaunchKernelGGL(k4, dim3(8 * per_xcd), dim3(64 * NTI), lds, stream, pl, per_xcd, npt, a.hpw,
                           nslice, x, cs, dtc, C, cbm, a.D, a.init, states, (TY*)a.y);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(6)) != hipSuccess) return err;
    return mark(7);
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
    if (dtype == 1) return std::max(chunk_state_lds_bytes<bf16_t>(NT, Q), chunk_scan_total_lds<bf16_t>(NT, Q));
    return std::max(chunk_state_lds_bytes<float>(NT, Q), chunk_scan_total_lds<float>(NT, Q));
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
