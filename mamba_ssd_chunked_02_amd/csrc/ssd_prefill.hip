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
// last two are carried as hi/lo pairs (hi = rn(v), lo = rn(v - hi)) and
// contracted with two MFMAs where the state's precision depends on them (the
// state term of y and the state update), which keeps that error ~2^-16
// relative; the intra-chunk term uses the hi part only.  fp32 operands are not
// split.
template <typename T>
struct Split {
    static constexpr bool on = !__is_same(T, float);
};

// Workgroup layout of the chunk-walking kernels: one wave per 32-wide tile of
// the head dimension (NPT waves).  Wave pt owns columns p in [32pt, 32pt+32)
// of the state S (P x N) and of y, for every n and every token, so the state
// never leaves its registers: st[nt] is the 32x32 tile S^T[32nt.., 32pt..] in
// accumulator layout, i.e. register v of lane l holds
//   S[p = 32pt + l%32][n = 32nt + 8(v/4) + 4(l/32) + v%4].
//
// Decay bookkeeping.  The chunk is cut into 32-token blocks j with start
// s_j = 32j - 1 and end e_j = 32j + 31 (cs_{-1} := 0).  Per chunk the
// workgroup shares these fp32 tables in LDS:
//   wb[k]   = exp(cs_{e(k)} - cs_k) dt_k          weight of token k to its block end (<= dt_k)
//   gam[j]  = exp(cs_{e_j} - cs_{s_j})            decay across block j (<= 1)
//   ul[t]   = exp(cs_t - cs_{s(t)})               decay from the block start to t (<= 1)
//   ue[t]   = exp(cs_t - cs_{e(t)})               = ul[t] / gam[j] (>= 1)
//   fast[j] = decay across block j below kFastBlockDecay (so ue stays finite)
// Every factor exp(cs_t - cs_k) dt_k with k <= t then equals
//   ul[t] * (prod of gam over the blocks strictly between k's block and t's) * wb[k] / ...
// which both the output and the state update evaluate with a Horner scheme:
// one 16-register multiply per block, no per-element exponentials, and all
// factors <= 1 (an underflow only ever drops a term below 1e-38 of dt x).
constexpr float kFastBlockDecay = 60.f;

struct ChunkTables {
    float* csl;  // [Q]
    float* dtl;  // [Q]
    float* wb;   // [Q]
    float* ul;   // [Q]
    float* ue;   // [Q]
    float* gam;  // [8]
    int* fast;   // [8]
};

__host__ __device__ inline size_t tables_bytes(int Q) {
    return ((size_t)(5 * Q + 8) * sizeof(float) + 8 * sizeof(int) + 15) & ~(size_t)15;
}

__device__ inline ChunkTables carve_tables(char* base, int Q) {
    ChunkTables tb;
    tb.csl = (float*)base;
    tb.dtl = tb.csl + Q;
    tb.wb = tb.dtl + Q;
    tb.ul = tb.wb + Q;
    tb.ue = tb.ul + Q;
    tb.gam = tb.ue + Q;
    tb.fast = (int*)(tb.gam + 8);
    return tb;
}

// Fill the tables for one chunk of one head.  The tables are private to one
// wave (64 lanes fill them); LDS operations of one wave complete in order, so
// its lanes may read them right after without a workgroup barrier.
__device__ inline void build_tables(const ChunkTables& tb, const float* __restrict__ csk,
                                    const float* __restrict__ dtk, int Q, int lane) {
    for (int q = lane; q < Q; q += 64) {
        const float a = csk[q], d = dtk[q];
        const float ce = csk[q | 31];
        const int s = (q & ~31) - 1;
        const float cs0 = s >= 0 ? csk[s] : 0.f;
        tb.csl[q] = a;
        tb.dtl[q] = d;
        tb.wb[q] = __expf(ce - a) * d;
        tb.ul[q] = __expf(a - cs0);
        tb.ue[q] = __expf(fminf(a - ce, kFastBlockDecay));
    }
    if (lane < Q / 32) {
        const float cs0 = lane > 0 ? csk[32 * lane - 1] : 0.f;
        const float ce = csk[32 * lane + 31];
        tb.gam[lane] = __expf(ce - cs0);
        tb.fast[lane] = (cs0 - ce) < kFastBlockDecay ? 1 : 0;
    }
}

// Wave-private transposed copy of x * wb for the chunk's columns
// [32pt, 32pt+32) of head h: xh[pl][k] + xl[pl][k] = x[row0+k][h][32pt+pl] wb[k]
// (pitch LP; xl only when split), zero past the chunk end and past P.
// One unit = 8 tokens x 8 columns per lane and step.
template <typename T>
__device__ inline void stage_xw(const T* __restrict__ x, const ChunkDesc& cd, int H, int P, int h, int Q,
                                int pt, const float* wb, T* xh, T* xl, int LP, int lane) {
    typedef typename Tr<T>::v8 v8;
    constexpr int kUnits = 2;  // Q <= 256: (Q/8) * 4 units over 64 lanes
    const int nunits = (Q / 8) * 4;
    v8 raw[kUnits][8];
    // all loads first (addresses clamped in bounds, masked after), so the
    // wave waits for memory once
#pragma unroll
    for (int s = 0; s < kUnits; ++s) {
        const int u = lane + 64 * s;
        const int pb = u & 3, kb = u >> 2;
        const int p0 = min(32 * pt + 8 * pb, P - 8);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int kk = min(8 * kb + r, cd.len - 1);
            raw[s][r] = Tr<T>::ld8(x + ((cd.row0 + kk) * H + h) * P + p0);
        }
    }
#pragma unroll
    for (int s = 0; s < kUnits; ++s) {
        const int u = lane + 64 * s;
        if (u < nunits) {
            const int pb = u & 3, kb = u >> 2;
            const int k0 = 8 * kb;
            const bool pok = 32 * pt + 8 * pb < P;
            f32x8 f[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const bool ok = pok && (k0 + r < cd.len);
                f[r] = Tr<T>::widen(raw[s][r]) * (ok ? wb[k0 + r] : 0.f);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                f32x8 o;
#pragma unroll
                for (int r = 0; r < 8; ++r) o[r] = f[r][i];
                const v8 hi = Tr<T>::narrow(o);
                Tr<T>::st8(xh + (8 * pb + i) * LP + k0, hi);
                if (Split<T>::on) Tr<T>::st8(xl + (8 * pb + i) * LP + k0, Tr<T>::narrow(o - Tr<T>::widen(hi)));
            }
        }
    }
}

template <typename T, int NNT>
__device__ inline void load_bt_block(typename Tr<T>::v8 (&a)[2][NNT], const T* __restrict__ btk, int Q, int j,
                                     int col, int half) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt)
            a[ks][nt] = Tr<T>::ld8(btk + (size_t)(32 * nt + col) * Q + 32 * j + 16 * ks + 8 * half);
}

// One block of the Horner state update:  st <- gam_j st + B_j^T (x wb)_j.
template <typename T, int NNT>
__device__ inline void update_block(f32x16 (&st)[NNT], const typename Tr<T>::v8 (&a)[2][NNT], float gj,
                                    const T* xhrow, const T* xlrow, int j, int half) {
    typedef typename Tr<T>::v8 v8;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) st[nt] *= gj;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int kb = 32 * j + 16 * ks + 8 * half;
        const v8 bh = Tr<T>::ld8(xhrow + kb);
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) mma16(st[nt], a[ks][nt], bh);
        if (Split<T>::on) {
            const v8 bl = Tr<T>::ld8(xlrow + kb);
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) mma16(st[nt], a[ks][nt], bl);
        }
    }
}

// Horner state update over the chunk's 32-token blocks:
//   for each block j:  st <- gam[j] st + B_j^T (x wb)_j
// which gives exp(cs_last) S + sum_k exp(cs_last - cs_k) dt_k x_k (outer) B_k.
// B^T rows are padded with zeros to NT, so no bounds checks are needed.  The
// next block's B^T fragments load while the current block computes.
template <typename T, int NNT>
__device__ inline void state_update(f32x16 (&st)[NNT], const T* __restrict__ btk, int Q, const T* xhrow,
                                    const T* xlrow, const float* gam, int col, int half) {
    typedef typename Tr<T>::v8 v8;
    const int nti = Q / 32;
    v8 a[2][NNT];
    load_bt_block<T, NNT>(a, btk, Q, 0, col, half);
    for (int j = 0; j < nti; ++j) {
        const float gj = gam[j];
        v8 cur[2][NNT];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) cur[ks][nt] = a[ks][nt];
        if (j + 1 < nti) load_bt_block<T, NNT>(a, btk, Q, j + 1, col, half);
        update_block<T, NNT>(st, cur, gj, xhrow, xlrow, j, half);
    }
}

template <int NNT>
__device__ inline void load_state(f32x16 (&st)[NNT], const float* src, int P, int N, int p, int half) {
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) {
        st[nt] = f32x16{};
        if (src && p < P) {
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                const int n = 32 * nt + 8 * vg + 4 * half;
                if (n < N) {
                    const f32x4 v = *(const f32x4*)(src + (size_t)p * N + n);
                    st[nt][4 * vg] = v[0];
                    st[nt][4 * vg + 1] = v[1];
                    st[nt][4 * vg + 2] = v[2];
                    st[nt][4 * vg + 3] = v[3];
                }
            }
        }
    }
}

template <int NNT>
__device__ inline void store_state(const f32x16 (&st)[NNT], float* dst, int P, int N, int p, int half) {
    if (p >= P) return;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) {
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
            const int n = 32 * nt + 8 * vg + 4 * half;
            if (n < N)
                *(f32x4*)(dst + (size_t)p * N + n) =
                    f32x4{st[nt][4 * vg], st[nt][4 * vg + 1], st[nt][4 * vg + 2], st[nt][4 * vg + 3]};
        }
    }
}

// Grid order: item i of (segment-major) work runs as workgroup L with
// i = (L % 8) * per_xcd + L / 8.  Workgroups are dealt to the 8 XCDs round
// robin, so each XCD walks a contiguous range of items: the heads of one
// segment run together and share its chunks' C.B^T, C and B^T in that XCD's L2.
__device__ inline int xcd_item(int per_xcd) { return (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3); }

// LDS of one wave: its decay tables, then its x * wb tile (hi, and lo when split).
template <typename T>
__host__ __device__ inline size_t wave_lds_bytes(int Q) {
    return tables_bytes(Q) + (size_t)(Split<T>::on ? 2 : 1) * 32 * (Q + 8) * sizeof(T);
}
template <typename T>
__host__ __device__ inline size_t wave_kernel_lds_bytes(int NPT, int Q) {
    return (size_t)NPT * wave_lds_bytes<T>(Q);
}

// ------------------------------------------------------------------ chunk_state
// For every segment that is not the last of its sequence, the state that the
// segment alone produces from a zero state (the Horner update above, chunk by
// chunk).  The waves of a workgroup are independent.
template <typename T, int NPT, int NT>
__global__ __launch_bounds__(64 * NPT) void ssd_chunk_state_kernel(
    Plan pl, int per_xcd, const T* __restrict__ x, const float* __restrict__ cs,
    const float* __restrict__ dtc, const T* __restrict__ bt, float* __restrict__ sbuf) {
    extern __shared__ __align__(16) char smem[];
    constexpr int NNT = NT / 32;
    const int item = xcd_item(per_xcd);
    if (item >= pl.nseg_ub * pl.H) return;
    const int h = item % pl.H;
    const SegDesc sd = seg_desc(pl, item / pl.H);
    if (sd.seq < 0 || sd.last) return;
    const int Q = pl.Q, P = pl.P, N = pl.N, H = pl.H, G = pl.G;
    const int g = h / pl.hpg;
    const int LP = Q + 8;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    char* wl = smem + (size_t)wave * wave_lds_bytes<T>(Q);
    const ChunkTables tb = carve_tables(wl, Q);
    T* xh = (T*)(wl + tables_bytes(Q));
    T* xl = xh + 32 * LP;
    f32x16 st[NNT];
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) st[nt] = f32x16{};
    for (int c = 0; c < sd.nchunks; ++c) {
        const int kc = sd.chunk0 + c;
        const ChunkDesc cd = chunk_desc(pl, kc);
        build_tables(tb, cs + ((size_t)kc * H + h) * Q, dtc + ((size_t)kc * H + h) * Q, Q, lane);
        stage_xw<T>(x, cd, H, P, h, Q, wave, tb.wb, xh, xl, LP, lane);
        state_update<T, NNT>(st, bt + ((size_t)kc * G + g) * NT * Q, Q, xh + col * LP, xl + col * LP, tb.gam,
                             col, half);
    }
    store_state<NNT>(st, sbuf + ((size_t)sd.slot_out * H + h) * P * N, P, N, 32 * wave + col, half);
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
// For each chunk of the segment, in order (t, k tokens of the chunk):
//   y[t][p] = exp(cs_t) sum_n C[t][n] S[p][n]                          (state term)
//           + sum_{k<=t} (C_t . B_k) exp(cs_t - cs_k) dt_k x[k][p]      (causal intra-chunk term)
//           + D x[t][p]
//   S <- exp(cs_last) S + sum_k exp(cs_last - cs_k) dt_k x_k (outer) B_k  (carried to the next chunk)
// Output tile (32-token block ti, this wave's p-tile), MFMA rows t, columns p:
//   acc  = C_rows . S^T                 A = C (n in the state registers' order),
//                                       B = state hi/lo pair from registers
//   for blocks j < ti:  acc = gam[j] acc + cb[t, block j] . (x wb)_j
//   diagonal block:     acc = gam[ti] acc + mask(cb[t, block ti]) . (x wb)_ti
//   acc *= ue[t]                        (= exp(cs_t - cs_{e_ti}))
// which leaves exp(cs_t) on the state term and exp(cs_t - cs_k) dt_k on every
// intra-chunk pair.  A block with decay beyond kFastBlockDecay stops the
// Horner scheme before its diagonal, scales by ul[t] and adds its diagonal
// with exact per-element factors instead.  The operands of block ti+1 are
// loaded while block ti computes.
template <typename T, typename TY, int NPT, int NT>
__global__ __launch_bounds__(64 * NPT) void ssd_chunk_scan_kernel(
    Plan pl, int per_xcd, const T* __restrict__ x, const float* __restrict__ cs,
    const float* __restrict__ dtc, const T* __restrict__ Cm, const T* __restrict__ cb,
    const T* __restrict__ bt, const float* __restrict__ D, const float* __restrict__ init,
    const float* __restrict__ sbuf, TY* __restrict__ y, float* __restrict__ fin) {
    extern __shared__ __align__(16) char smem[];
    constexpr bool SP = Split<T>::on;
    constexpr int NNT = NT / 32;
    typedef typename Tr<T>::v8 v8;
    const int item = xcd_item(per_xcd);
    if (item >= pl.nseg_ub * pl.H) return;
    const int h = item % pl.H;
    const SegDesc sd = seg_desc(pl, item / pl.H);
    if (sd.seq < 0) return;
    const int Q = pl.Q, P = pl.P, N = pl.N, H = pl.H, G = pl.G;
    const int g = h / pl.hpg;
    const int LP = Q + 8;
    const int nti = Q / 32;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    const int p = 32 * wave + col;  // this lane's column of S and y
    char* wl = smem + (size_t)wave * wave_lds_bytes<T>(Q);
    const ChunkTables tb = carve_tables(wl, Q);
    T* xh = (T*)(wl + tables_bytes(Q));
    T* xl = xh + 32 * LP;
    const T* xhrow = xh + col * LP;
    const T* xlrow = xl + col * LP;
    const bool need_final = sd.last && fin != nullptr;
    const float Dh = D[h];
    const int HP = H * P;

    const float* src = nullptr;
    if (sd.slot_in >= 0) src = sbuf + ((size_t)sd.slot_in * H + h) * P * N;
    else if (init) src = init + ((size_t)sd.seq * H + h) * P * N;
    bool zero_state = (src == nullptr);
    f32x16 st[NNT];
    load_state<NNT>(st, src, P, N, p, half);
    // state operand of the state term: fragment (nt, m) = st[nt][8m .. 8m+7];
    // within a 16-wide step its element i of lane half hf is n = 16m + 8(i/4) + 4hf + i%4
    v8 sh[NNT][2], sl[NNT][2];
    auto split_state = [&]() {
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                f32x8 f;
#pragma unroll
                for (int j = 0; j < 8; ++j) f[j] = st[nt][8 * m + j];
                sh[nt][m] = Tr<T>::narrow(f);
                sl[nt][m] = SP ? Tr<T>::narrow(f - Tr<T>::widen(sh[nt][m])) : v8{};
            }
        }
    };
    split_state();

    for (int c = 0; c < sd.nchunks; ++c) {
        const int kc = sd.chunk0 + c;
        const ChunkDesc cd = chunk_desc(pl, kc);
        const bool update = (c + 1 < sd.nchunks) || need_final;
        build_tables(tb, cs + ((size_t)kc * H + h) * Q, dtc + ((size_t)kc * H + h) * Q, Q, lane);
        stage_xw<T>(x, cd, H, P, h, Q, wave, tb.wb, xh, xl, LP, lane);

        const T* cbk = cb + ((size_t)kc * G + g) * Q * Q;
        const T* btk = bt + ((size_t)kc * G + g) * NT * Q;
        // Operands of 32-token block ti for this lane's A row ta = 32 ti + col:
        // C row ta in the state registers' n order, cb row ta, B^T block ti.
        // Rows past the chunk end are clamped (their outputs are never stored).
        v8 ca[NNT][2], ga[8][2], ba[2][NNT];
        auto load_c = [&](int ti) {
            if (zero_state) return;
            const int ta = min(32 * ti + col, cd.len - 1);
            const T* crow = Cm + ((cd.row0 + ta) * G + g) * N;
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    // padding columns n >= N meet zero state rows; clamp to stay in bounds
                    const int n0 = 32 * nt + 16 * m + 4 * half;
                    const typename Tr<T>::v4 c0 = Tr<T>::ld4raw(crow + min(n0, N - 4));
                    const typename Tr<T>::v4 c1 = Tr<T>::ld4raw(crow + min(n0 + 8, N - 4));
                    ca[nt][m] = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
                }
        };
        auto load_g = [&](int ti) {
            const T* grow = cbk + (size_t)(32 * ti + col) * Q;
#pragma unroll
            for (int kj = 0; kj < 8; ++kj)
                if (kj <= ti) {
                    ga[kj][0] = Tr<T>::ld8(grow + 32 * kj + 8 * half);
                    ga[kj][1] = Tr<T>::ld8(grow + 32 * kj + 16 + 8 * half);
                }
        };
        load_c(0);
        if (update) load_bt_block<T, NNT>(ba, btk, Q, 0, col, half);
        const T* xcol = x + (size_t)h * P + min(p, P - 1);
        for (int ti = 0; ti < nti; ++ti) {
            const int ta = 32 * ti + col;
            // x at this lane's 16 output rows for the D x term (rows clamped)
            float xd[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = min(32 * ti + acc_row(v, lane), cd.len - 1);
                xd[v] = (float)xcol[(size_t)(cd.row0 + t) * HP];
            }
            load_g(ti);  // covered by the state-term and update MFMAs below
            f32x16 acc = {};
            if (!zero_state) {
#pragma unroll
                for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        mma16(acc, ca[nt][m], sh[nt][m]);
                        if (SP) mma16(acc, ca[nt][m], sl[nt][m]);
                    }
                if (ti + 1 < nti) load_c(ti + 1);
            }
            if (update) {
                // the chunk-start state operand (sh/sl) stays untouched until the chunk ends
                update_block<T, NNT>(st, ba, tb.gam[ti], xhrow, xlrow, ti, half);
                if (ti + 1 < nti) load_bt_block<T, NNT>(ba, btk, Q, ti + 1, col, half);
            }
            const bool fast = tb.fast[ti] != 0;
#pragma unroll
            for (int kj = 0; kj < 8; ++kj) {
                if (kj < ti || (kj == ti && fast)) {
                    acc *= tb.gam[kj];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        v8 a = ga[kj][ks];
                        if (kj == ti) {
                            const int k0 = 32 * kj + 16 * ks + 8 * half;
#pragma unroll
                            for (int i = 0; i < 8; ++i) a[i] = (k0 + i <= ta) ? a[i] : (typename Tr<T>::elem)0;
                        }
                        mma16(acc, a, Tr<T>::ld8(xhrow + 32 * kj + 16 * ks + 8 * half));
                    }
                }
            }
            const float* scale = fast ? tb.ue : tb.ul;
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                const f32x4 u = *(const f32x4*)(scale + 32 * ti + 8 * vg + 4 * half);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[4 * vg + j] *= u[j];
            }
            if (!fast) {
                // decay across this block beyond the fast range: exact factors, raw x
                const float cst = tb.csl[ta];
                const T* grow = cbk + (size_t)ta * Q;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int k0 = 32 * ti + 16 * ks + 8 * half;
                    const f32x8 gv = Tr<T>::widen(Tr<T>::ld8(grow + k0));
                    f32x8 m;
                    v8 xb;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int kk = k0 + i;
                        const float e = __expf(fminf(cst - tb.csl[kk], 0.f)) * tb.dtl[kk];
                        m[i] = kk <= ta ? gv[i] * e : 0.f;
                        const int kr = min(kk, cd.len - 1);
                        xb[i] = x[(cd.row0 + kr) * HP + h * P + min(p, P - 1)];
                    }
                    mma16(acc, Tr<T>::narrow(m), xb);
                }
            }
            // + D x; store rows t of this block, column p
            if (p < P) {
                TY* ycol = y + (size_t)(cd.row0 + 32 * ti) * HP + (size_t)h * P + p;
                if (32 * ti + 32 <= cd.len) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) ycol[(size_t)acc_row(v, lane) * HP] = (TY)(acc[v] + Dh * xd[v]);
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (32 * ti + acc_row(v, lane) < cd.len)
                            ycol[(size_t)acc_row(v, lane) * HP] = (TY)(acc[v] + Dh * xd[v]);
                }
            }
        }
        if (update) {
            split_state();
            zero_state = false;
        }
    }
    if (need_final) store_state<NNT>(st, fin + ((size_t)sd.seq * H + h) * P * N, P, N, p, half);
}

template <typename F>
hipError_t allow_lds(F* fn, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, int NPT, int NT>
hipError_t run_prefill(const Plan& pl, const Layout& lay, const ScanArgs& a, hipStream_t stream,
                       hipEvent_t* marks) {
    char* ws = a.ws;
    const T* x = (const T*)a.x;
    const T* B = (const T*)a.B;
    const T* C = (const T*)a.C;
    float* cs = (float*)(ws + lay.cs);
    float* dtc = (float*)(ws + lay.dtc);
    T* cbm = (T*)(ws + lay.cb);
    T* bt = (T*)(ws + lay.bt);
    float* sbuf = (float*)(ws + lay.sbuf);
    hipError_t err;
    auto mark = [&](int i) -> hipError_t { return marks ? hipEventRecord(marks[i], stream) : hipSuccess; };
    const int per_xcd = (int)(((int64_t)pl.nseg_ub * pl.H + 7) / 8);
    const size_t lds = wave_kernel_lds_bytes<T>(NPT, pl.Q);
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
                           pl, NT, B, C, cbm, bt);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(3)) != hipSuccess) return err;
    if (a.run_passing && pl.nseg_ub > 0 && pl.nslot_ub > 0) {
        auto* k2 = ssd_chunk_state_kernel<T, NPT, NT>;
        if ((err = allow_lds(k2, lds)) != hipSuccess) return err;
        hipLaunchKernelGGL(k2, dim3(8 * per_xcd), dim3(64 * NPT), lds, stream, pl, per_xcd, x, cs, dtc,
                           bt, sbuf);
        if ((err = hipGetLastError()) != hipSuccess) return err;
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
        if (a.y_f32) {
            auto* k4 = ssd_chunk_scan_kernel<T, float, NPT, NT>;
            if ((err = allow_lds(k4, lds)) != hipSuccess) return err;
            hipLaunchKernelGGL(k4, dim3(8 * per_xcd), dim3(64 * NPT), lds, stream, pl, per_xcd, x, cs, dtc, C,
                               cbm, bt, a.D, a.init, sbuf, (float*)a.y, a.final_state);
        } else {
            auto* k4 = ssd_chunk_scan_kernel<T, bf16_t, NPT, NT>;
            if ((err = allow_lds(k4, lds)) != hipSuccess) return err;
            hipLaunchKernelGGL(k4, dim3(8 * per_xcd), dim3(64 * NPT), lds, stream, pl, per_xcd, x, cs, dtc, C,
                               cbm, bt, a.D, a.init, sbuf, (bf16_t*)a.y, a.final_state);
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = mark(6)) != hipSuccess) return err;
    return hipSuccess;
}

template <typename T>
hipError_t dispatch_nt(const Plan& pl, const Layout& lay, const ScanArgs& a, hipStream_t s,
                       hipEvent_t* marks) {
    const int NPT = (pl.P + 31) / 32;
    const int NT = padded_dstate(pl.N);
#define SSD_CASE(npt, nt) \
    if (NPT == npt && NT == nt) return run_prefill<T, npt, nt>(pl, lay, a, s, marks);
    SSD_CASE(1, 32) SSD_CASE(1, 64) SSD_CASE(1, 128) SSD_CASE(1, 256)
    SSD_CASE(2, 32) SSD_CASE(2, 64) SSD_CASE(2, 128) SSD_CASE(2, 256)
    SSD_CASE(3, 32) SSD_CASE(3, 64) SSD_CASE(3, 128) SSD_CASE(3, 256)
    SSD_CASE(4, 32) SSD_CASE(4, 64) SSD_CASE(4, 128) SSD_CASE(4, 256)
#undef SSD_CASE
    return hipErrorInvalidValue;
}

}  // namespace

size_t chunk_scan_lds_bytes(int dtype, int P, int N, int Q) {
    (void)N;
    const int npt = (P + 31) / 32;
    return dtype == 1 ? wave_kernel_lds_bytes<bf16_t>(npt, Q) : wave_kernel_lds_bytes<float>(npt, Q);
}

hipError_t launch_prefill(const Plan& plan, const Layout& lay, const ScanArgs& a, hipStream_t stream,
                          hipEvent_t* marks) {
    if (a.dtype == 1) return dispatch_nt<bf16_t>(plan, lay, a, stream, marks);
    return dispatch_nt<float>(plan, lay, a, stream, marks);
}

}  // namespace ssd
