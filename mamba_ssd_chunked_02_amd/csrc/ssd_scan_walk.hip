// Fused chunked scan on gfx950: chunk states, the passing between chunks and
// the chunk outputs of one sequence in a single walk over its chunks, so the
// state entering each chunk never leaves the chip and x is read once.
//
// The computation is the chunked regrouping of the recurrence
//   S_t = exp(dt_t A) S_{t-1} + dt_t x_t (outer) B_t,   y_t = S_t C_t + D x_t
// ("Engineering hybrid state-space models", section 2: the duality
// Y = (M o CB^T) X over chunks of Q tokens; "Compiler-First State Space
// Duality...", abstract: fixed-size chunking, einsum-shaped contractions).
// Per chunk c with entering state h_c, inclusive decay sums cs inside the
// chunk and the chunk cut into 32-token blocks j:
//   y_t     = exp(cs_t) C_t h_c^T + sum_{s<=t} (C_t . B_s) exp(cs_t - cs_s) dt_s x_s + D x_t
//   h_{c+1} = Horner over the blocks: H <- gam_j H + sum_{s in j} wb_s x_s (outer) B_s,
//             starting from H = h_c, with gam_j = exp(decay across block j) <= 1
//             and wb_s = exp(cs_end(j) - cs_s) dt_s <= dt_s,
// so h_{c+1} = exp(cs_last) h_c + sum_s exp(cs_last - cs_s) dt_s x_s (outer) B_s.
// A chunk that decays by less than kWeakDecay over its whole length takes that
// last form directly (weakly decaying chunks): the weights go to the chunk's
// end, wc_s = exp(cs_last - cs_s) dt_s, the state is scaled once and the
// advance is a plain sum, and y's intra-chunk term is one unscaled sum
//   y_t = exp(cs_t - cs_last) (sum_{s<=t} (C_t . B_s) wc_s x_s + exp(cs_last) C_t h_c^T) + D x_t,
// whose row factor stays below exp(kWeakDecay).
// The state advance contracts x wb as a hi/lo bf16 pair, so that the state
// keeps the accuracy the final state needs.  A chunk whose sequence decays by
// kLoSkipDecay or more after it contributes to the final state only through
// that decay (below exp(-kLoSkipDecay)); its advance takes the hi half alone,
// the single rounding that y's intra-chunk term uses too.  A small kernel
// before the walk gives each (chunk, head) the decay still to come.
//
// Work item: one sequence, one group, and a slice of up to NU units, a unit
// being (head of the group, 32-column tile of P).  The workgroup walks the
// sequence's chunks in order and, inside a chunk, its units in order: one
// step per (chunk, unit).  Eight waves with two roles:
//   waves 0-3  output blocks w and 7-w of y: they hold the chunk's C.B^T rows
//              and C rows of their two blocks in registers for every unit of
//              the chunk, and read the unit's staged x and state from LDS;
//   waves 4-7  n-tile w-4 of every unit's state, kept in MFMA accumulators
//              across the whole walk (the transposed tile h^T[n][p]); per step
//              they advance the current unit's tile over the chunk, write the
//              next step's state as a hi/lo bf16 pair to LDS, stage the next
//              step's x and decay tables in LDS and load the step after that.
// LDS holds two staging buffers, two state buffers and the output waves'
// transpose tiles (159 KB); one barrier
// per step separates the step that reads a buffer from the one that refills
// it.  Only bf16 inputs, 256-token chunks and dstate in (64, 128] take this
// kernel; the host picks the separate kernels for everything else.
#include <type_traits>

#include "ssd_prefill_shared.h"

namespace ssd {

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kQ = 256;          // chunk length
constexpr int kNTI = kQ / 32;    // 32-token blocks per chunk
constexpr int kNT = 128;         // dstate rows, padded
constexpr int kLP = kQ + 8;      // token pitch (elements) of the transposed x tiles
constexpr int kNS = kNT + 8;     // n pitch (elements) of the state tiles
constexpr float kFastDecay = 60.f;  // same bound as the chunk scan's Horner scheme
constexpr float kWeakDecay = 60.f;  // whole-chunk decay below which the weights go to the chunk's end
constexpr float kLoSkipDecay = 8.f;  // decay after a chunk from which its advance drops the lo half
constexpr float kBlockSkipDecay = 16.f;  // decay to the chunk's end past which a block leaves the advance
constexpr float kStateSkipDecay = 16.f;  // decay since the chunk's start past which a block of y drops the state term

// One staging buffer: tables | (x wb)^T hi | (x wb)^T lo | x^T, the tiles
// [32 columns p][kLP tokens] in bf16.
constexpr size_t kTabBytes = (size_t)(4 * kQ + 16) * 4;
constexpr size_t kTileBytes = (size_t)32 * kLP * 2;
constexpr size_t kStageBytes = kTabBytes + 3 * kTileBytes;
// One state buffer: h hi, h lo as [32 columns p][kNS] bf16.
constexpr size_t kStateBytes = (size_t)2 * 32 * kNS * 2;
// Per output wave: a 32 x 32 fp32 tile that turns a block's accumulator
// layout into 16-byte row pieces for the y stores.
constexpr int kEpPitch = 36;
constexpr size_t kEpBytes = (size_t)32 * kEpPitch * 4;
constexpr size_t kWalkLds = 2 * kStageBytes + 2 * kStateBytes + 4 * kEpBytes;
static_assert(kWalkLds <= 160 * 1024, "scan walk LDS");

// A weakly decaying chunk (flag bit 1 of every fast[] entry) stores
// exp(cs_t - cs_last) in ue and exp(cs_last) in every gam entry; ul is not
// read then, and all its blocks are fast.  Flag bit 2 (every entry): the
// chunk's advance takes the hi half of x wb alone, and the lo tile is not
// written.
struct WalkTables {
    float* cs;   // [Q] cs_t
    float* dt;   // [Q] dt_t (0 past the chunk end)
    float* ul;   // [Q] exp(cs_t - cs before t's block)          (<= 1)
    float* ue;   // [Q] exp(min(cs_t - cs at t's block end, 60))   (>= 1)
    float* gam;  // [8] decay across each block                   (<= 1)
    int* fast;   // [8] bit 0: block decay below kFastDecay; bit 1: weakly decaying chunk;
                 //     bit 2: hi half alone in the advance; bit 3: the block decays by
                 //     kBlockSkipDecay or more before the chunk's end
};

__device__ inline WalkTables walk_tables(char* base) {
    WalkTables t;
    t.cs = (float*)base;
    t.dt = t.cs + kQ;
    t.ul = t.dt + kQ;
    t.ue = t.ul + kQ;
    t.gam = t.ue + kQ;
    t.fast = (int*)(t.gam + 8);
    return t;
}

struct WalkBufs {
    char* smem;
    __device__ char* stage(int b) const { return smem + b * kStageBytes; }
    __device__ bf16_t* xh(int b) const { return (bf16_t*)(stage(b) + kTabBytes); }
    __device__ bf16_t* xl(int b) const { return xh(b) + 32 * kLP; }
    __device__ bf16_t* xr(int b) const { return xl(b) + 32 * kLP; }
    __device__ bf16_t* sh(int b) const { return (bf16_t*)(smem + 2 * kStageBytes + b * kStateBytes); }
    __device__ bf16_t* sl(int b) const { return sh(b) + 32 * kNS; }
    __device__ float* ep(int w) const { return (float*)(smem + 2 * kStageBytes + 2 * kStateBytes + w * kEpBytes); }
};

// The walk of one workgroup: sequence s, group g, units [u0, u0 + nu) of the
// group's hpg * npt units (unit u: head g hpg + u / npt, column tile u % npt).
struct Walk {
    int s, g, u0, nu, npt;
    int chunk0, nck, len;  // first chunk, chunk count, tokens of the sequence
    int64_t row0;          // first token row of the sequence
    __device__ int head(const Plan& pl, int j) const { return g * pl.hpg + (u0 + j) / npt; }
    __device__ int tile(int j) const { return (u0 + j) % npt; }
    __device__ ChunkDesc chunk(int c) const {
        ChunkDesc d;
        d.seq = s;
        d.idx = c;
        d.row0 = row0 + (int64_t)c * kQ;
        d.len = min(kQ, len - c * kQ);
        return d;
    }
};

// Items are (pair, slice) with the slice fastest, a pair being (sequence,
// group) and the sequences in the order pl.seq_order gives (longest first,
// for a packed batch) or in index order.  Runs of `run` consecutive items
// share an XCD, so the walks of one pair read each chunk's C.B^T, C and B^T
// from one L2; the runs are dealt to the XCDs in turn, so the longest pairs
// start first, spread over the chip.  (Slice-major order, which spreads every
// XCD over all sequences, measured 6% slower.)
__device__ inline bool walk_of(const Plan& pl, int run, int npt, int nslice, int nus, Walk& w) {
    const int64_t l = blockIdx.x >> 3;
    const int64_t item = ((int64_t)(blockIdx.x & 7) + 8 * (l / run)) * run + l % run;
    if (item >= (int64_t)pl.nseq * pl.G * nslice) return false;
    const int slice = (int)(item % nslice);
    const int64_t r = item / nslice;
    w.g = (int)(r % pl.G);
    const int rank = (int)(r / pl.G);
    w.s = pl.seq_order ? __builtin_amdgcn_readfirstlane(pl.seq_order[rank]) : rank;
    w.npt = npt;
    w.u0 = slice * nus;
    w.nu = min(nus, pl.hpg * npt - w.u0);
    const SeqExtent se = seq_extent(pl, w.s);
    w.chunk0 = __builtin_amdgcn_readfirstlane(se.chunk0);
    w.nck = __builtin_amdgcn_readfirstlane(se.nchunks);
    w.len = __builtin_amdgcn_readfirstlane(se.len);
    w.row0 = (int64_t)__builtin_amdgcn_readfirstlane((int)se.row0);
    return w.nu > 0;
}

// hi = rn(v) and lo = rn(v - hi) of four fp32 values as bf16 pairs packed in
// 32-bit words (element 0 in the low half).  hi's fp32 value is read back from
// its bits (a shift or a mask) rather than converted a second time.
__device__ inline void split_hilo(const f32x4& v, u32x2& hi, u32x2& lo) {
    hi = __builtin_bit_cast(u32x2, Tr<bf16_t>::narrow4(v));
    const uint32_t h0 = hi[0], h1 = hi[1];
    const f32x4 hf = {__builtin_bit_cast(float, h0 << 16), __builtin_bit_cast(float, h0 & 0xffff0000u),
                      __builtin_bit_cast(float, h1 << 16), __builtin_bit_cast(float, h1 & 0xffff0000u)};
    lo = __builtin_bit_cast(u32x2, Tr<bf16_t>::narrow4(v - hf));
}

// s_waitcnt vmcnt(0) and vmcnt(4) with expcnt and lgkmcnt left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kWaitVmcnt4 = 0x0F74;

// ------------------------------------------------------------------ staging (waves 4-7)
// Thread tau of the 256 staging threads owns 4 consecutive tokens k0..k0+3
// and 8 columns 8 pb..8 pb+7 of the unit's tile: it loads 4 x 16 bytes of x
// plus the tokens' decay sums and steps, and writes the column-major tiles
// (4 tokens = 8 bytes per column).  The threads of pb = 0 also write the
// decay tables of their 4 tokens, and of their block when k0 starts one.
struct StageRegs {
    bf16x8 raw[4];
    f32x4 cs4, dt4;
    float ce, c0;  // cs at the end of the tokens' block, cs before its start
    float cl;      // cs at the chunk's last token (positions past the end hold it too)
    float after;   // decay from the chunk's end to its sequence's end
};

__device__ inline int stage_pb(int tau) { return (tau >> 4) & 3; }
__device__ inline int stage_k0(int tau) { return 4 * ((tau & 15) + 16 * (tau >> 6)); }

__device__ inline void stage_load(StageRegs& r, const Plan& pl, const Walk& w, int c, int j, const bf16_t* x,
                                  const float* cs, const float* dtc, const float* tail, int tau) {
    const ChunkDesc d = w.chunk(c);
    const int k = w.chunk0 + c, h = w.head(pl, j), pt = w.tile(j);
    const int H = pl.H, P = pl.P;
    const int pb = stage_pb(tau), k0 = stage_k0(tau);
    const int pc = 32 * pt + 8 * pb;
    const int p0 = pc < P ? pc : 0;
    const __amdgpu_buffer_rsrc_t rx = chunk_x_rsrc(x, d, H, P);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kk = min(k0 + i, d.len - 1);
        r.raw[i] = buffer_ld8<bf16_t>(rx, ((kk * H + h) * P + p0) * 2);
    }
    const float* csk = cs + ((size_t)k * H + h) * kQ;
    const float* dtk = dtc + ((size_t)k * H + h) * kQ;
    r.cs4 = *(const f32x4*)(csk + k0);
    r.dt4 = *(const f32x4*)(dtk + k0);
    r.ce = csk[k0 | 31];
    r.c0 = csk[max((k0 & ~31) - 1, 0)];
    const f32x2 t = *(const f32x2*)(tail + 2 * ((size_t)k * H + h));
    r.cl = t[0];
    r.after = t[1];
}

__device__ inline void stage_store(const StageRegs& r, const Plan& pl, const Walk& w, const WalkBufs& bufs, int c,
                                   int j, int b, int tau) {
    const ChunkDesc d = w.chunk(c);
    const int pb = stage_pb(tau), k0 = stage_k0(tau);
    const bool pok = 32 * w.tile(j) + 8 * pb < pl.P;
    const float c0 = k0 >= 32 ? r.c0 : 0.f;
    // every thread reads the same cs_last, so all take the same form
    const bool weak = -r.cl < kWeakDecay;
    const bool hi_only = r.after >= kLoSkipDecay;  // false for a NaN
    const float ref = weak ? r.cl : r.ce;
    float wb[4];
    bf16x8 xm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        wb[i] = pok ? __expf(ref - r.cs4[i]) * r.dt4[i] : 0.f;  // dt is 0 past the chunk end
        xm[i] = (pok && k0 + i < d.len) ? r.raw[i] : bf16x8{};
    }
    bf16_t* xh = bufs.xh(b) + (8 * pb) * kLP + k0;
    bf16_t* xl = bufs.xl(b) + (8 * pb) * kLP + k0;
    bf16_t* xr = bufs.xr(b) + (8 * pb) * kLP + k0;
#pragma unroll
    for (int col = 0; col < 8; ++col) {
        const f32x4 o = {(float)xm[0][col] * wb[0], (float)xm[1][col] * wb[1], (float)xm[2][col] * wb[2],
                         (float)xm[3][col] * wb[3]};
        if (hi_only) {
            *(u32x2*)(xh + col * kLP) = __builtin_bit_cast(u32x2, Tr<bf16_t>::narrow4(o));
        } else {
            u32x2 hi, lo;
            split_hilo(o, hi, lo);
            *(u32x2*)(xh + col * kLP) = hi;
            *(u32x2*)(xl + col * kLP) = lo;
        }
        Tr<bf16_t>::st4raw(xr + col * kLP, bf16x4{xm[0][col], xm[1][col], xm[2][col], xm[3][col]});
    }
    if (pb == 0) {
        const WalkTables tb = walk_tables(bufs.stage(b));
        *(f32x4*)(tb.cs + k0) = r.cs4;
        *(f32x4*)(tb.dt + k0) = r.dt4;
        f32x4 ul, ue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ul[i] = __expf(r.cs4[i] - c0);
            ue[i] = weak ? __expf(r.cs4[i] - r.cl) : __expf(fminf(r.cs4[i] - r.ce, kFastDecay));
        }
        *(f32x4*)(tb.ul + k0) = ul;
        *(f32x4*)(tb.ue + k0) = ue;
        if ((k0 & 31) == 0) {
            tb.gam[k0 >> 5] = weak ? __expf(r.cl) : __expf(r.ce - c0);
            tb.fast[k0 >> 5] = (weak ? 3 : (c0 - r.ce) < kFastDecay ? 1 : 0) | (hi_only ? 4 : 0) |
                               (r.ce - r.cl >= kBlockSkipDecay ? 8 : 0);
        }
    }
}

// ------------------------------------------------------------------ state tiles (waves 4-7)
// acc holds h^T[n][p] for n in n-tile nt (row 8 (v/4) + 4 half + v%4 of the
// tile) and p = 32 pt + lane%32.  Written to a state buffer as [p][n]
// hi/lo pairs: 4 consecutive n per lane and register group, 8 bytes each.
__device__ inline void put_state(const f32x16& acc, const WalkBufs& bufs, int b, int nt) {
    const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    bf16_t* sh = bufs.sh(b) + col * kNS + 32 * nt + 4 * half;
    bf16_t* sl = bufs.sl(b) + col * kNS + 32 * nt + 4 * half;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4 v = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        u32x2 hi, lo;
        split_hilo(v, hi, lo);
        *(u32x2*)(sh + 8 * q) = hi;
        *(u32x2*)(sl + 8 * q) = lo;
    }
}

// Byte offset of element (p, n) of a P x N state for the lane's accumulator
// register v, or an offset past the descriptor when (p, n) is padding.
__device__ inline int state_off(int v, int pt, int nt, int P, int N) {
    const int lane = threadIdx.x & 63;
    const int p = 32 * pt + (lane & 31);
    const int n = 32 * nt + acc_row(v, lane);
    return (p < P && n < N) ? (p * N + n) * 4 : kOutOfRange;
}

// One chunk of the state walk for the current unit: the Horner scheme over
// the 8 blocks, H <- gam_j H + X_j from H = h_c, X_j being block j's
// contribution with its weights taken to the block's end.  A = the chunk's
// B^T fragments (n-tile rows), B = the staged (x wb)^T hi and lo tiles.  The
// operands of block j + 1 are read from LDS while block j's MFMAs run (the
// scheduling barriers keep the reads ahead); the other wave on the SIMD fills
// the matrix core while this one scales H.  A weakly decaying chunk's staged
// weights already reach the chunk's end: H is scaled once, by exp(cs_last),
// and the blocks are a plain sum.
// LO: whether the lo half is contracted too; RUNTIME: take that from lo_rt
// instead, one loop with the choice inside.  The six-unit instance takes that
// form because its registers do not hold two copies of the loop, and the
// one-unit instance because it measured faster (every one of its steps
// switches chunks).
// JB0: the first block contracted.  The blocks before it decay by
// kBlockSkipDecay or more before the chunk's end, so their tokens reach the
// state scaled by less than exp(-kBlockSkipDecay) and are left out; the
// Horner scheme still applies their decays.
template <bool LO, bool RUNTIME, int JB0>
__device__ inline void walk_advance(f32x16& acc, const bf16x8 (&bf)[kQ / 16], const WalkBufs& bufs, int b,
                                    bool weak, bool lo_rt) {
    const bool lo_too = RUNTIME ? lo_rt : LO;
    const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    const WalkTables tb = walk_tables(bufs.stage(b));
    const bf16_t* hrow = bufs.xh(b) + col * kLP + 8 * half;
    const bf16_t* lrow = bufs.xl(b) + col * kLP + 8 * half;
    const f32x4 g0 = *(const f32x4*)tb.gam;
    const f32x4 g1 = *(const f32x4*)(tb.gam + 4);
    const float gm[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
    bf16x8 op[2][4];
    auto ld = [&](int jb, bf16x8 (&o)[4]) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            o[2 * ks] = Tr<bf16_t>::ld8(hrow + 16 * (2 * jb + ks));
            if (lo_too) o[2 * ks + 1] = Tr<bf16_t>::ld8(lrow + 16 * (2 * jb + ks));
        }
    };
    ld(JB0, op[JB0 & 1]);
    if (weak) {
        acc *= gm[0];
    } else if (JB0 > 0) {
        float g = gm[0];
#pragma unroll
        for (int jb = 1; jb < JB0; ++jb) g *= gm[jb];
        acc *= g;
    }
#pragma unroll
    for (int jb = JB0; jb < kNTI; ++jb) {
        if (jb + 1 < kNTI) ld(jb + 1, op[(jb + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        if (!weak) acc *= gm[jb];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            mma16(acc, bf[2 * jb + ks], op[jb & 1][2 * ks]);
            if (lo_too) mma16(acc, bf[2 * jb + ks], op[jb & 1][2 * ks + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int NU>
__device__ void walk_states(const Plan& pl, const Walk& w, const WalkBufs& bufs, const bf16_t* __restrict__ x,
                            const float* __restrict__ cs, const float* __restrict__ dtc,
                            const float* __restrict__ tail, const bf16_t* __restrict__ bt,
                            const float* __restrict__ init, float* __restrict__ fin) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int nt = __builtin_amdgcn_readfirstlane((tid >> 6) - 4);
    const int tau = tid - 256;
    const int P = pl.P, N = pl.N, H = pl.H, G = pl.G;
    const int nu = w.nu;
    const int total = w.nck * nu;
    f32x16 acc[NU];
#pragma unroll
    for (int j = 0; j < NU; ++j) {
        acc[j] = f32x16{};
        if (j < nu && init) {
            const int h = w.head(pl, j), pt = w.tile(j);
            const __amdgpu_buffer_rsrc_t ri =
                buffer_rsrc(init + ((size_t)w.s * H + h) * P * N, (uint32_t)(P * N * 4));
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[j][v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                          ri, state_off(v, pt, nt, P, N), 0, 0));
        }
    }
    bf16x8 bf[kQ / 16];
    const int boff = bt_frag(kQ, nt, 0, lane) * 2;
    auto load_bt = [&](int c) {
        const __amdgpu_buffer_rsrc_t rb =
            buffer_rsrc(bt + ((size_t)(w.chunk0 + c) * G + w.g) * kNT * kQ, (uint32_t)(kNT * kQ * 2));
#pragma unroll
        for (int s = 0; s < kQ / 16; ++s) bf[s] = buffer_ld8<bf16_t>(rb, boff + 512 * s * 2);
    };
    // staging registers: sr holds the next step's inputs (loaded a step
    // ago), sn receives the inputs of the step after it, loaded at the start
    // of a step so their latency spans the whole step
    StageRegs sr, sn;
    auto load_step = [&](StageRegs& r, int i) {  // i < total
        const int c = i / nu;
        stage_load(r, pl, w, c, i - c * nu, x, cs, dtc, tail, tau);
    };
    if (total > 0) {
        load_bt(0);
        load_step(sr, 0);
        stage_store(sr, pl, w, bufs, 0, 0, 0, tau);
        put_state(acc[0], bufs, 0, nt);
        load_step(sr, min(1, total - 1));
    }
    __syncthreads();
    for (int c = 0; c < w.nck; ++c) {
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            if (j < nu) {
                const int i = c * nu + j, b = i & 1;
                // unconditional (the last step repeats itself), so the wait
                // counts never cover a path without these loads
                load_step(sn, min(i + 2, total - 1));
                // the next step's unit is j + 1 of this chunk, whose state is
                // ready, or unit 0 of the next chunk, whose state is ready
                // once this step has advanced it (with one unit per
                // workgroup it is the unit advanced here)
                const bool more = i + 1 < total;
                const int cn = j + 1 < nu ? c : c + 1, jn = j + 1 < nu ? j + 1 : 0;
                if (more) {
                    if (j + 1 < nu) put_state(acc[(j + 1) % NU], bufs, b ^ 1, nt);
                    stage_store(sr, pl, w, bufs, cn, jn, b ^ 1, tau);
                }
                const int flags = __builtin_amdgcn_readfirstlane(walk_tables(bufs.stage(b)).fast[0]);
                const bool weak = (flags & 2) != 0, lo = (flags & 4) == 0;
                if constexpr (NU >= 6 || NU == 1) {
                    walk_advance<true, true, 0>(acc[j], bf, bufs, b, weak, lo);
                } else {
                    // leading blocks that leave the advance: four or none (one
                    // loop start per case; starts at every second block spilled
                    // more registers and measured no faster)
                    const int* fl = walk_tables(bufs.stage(b)).fast;
                    int skip = 0;
#pragma unroll
                    for (int jb = 0; jb < kNTI; ++jb)
                        skip += (__builtin_amdgcn_readfirstlane(fl[jb]) >> 3) & 1;  // the flags are monotone in jb
                    skip = skip >= 4 ? 4 : 0;
                    if (lo) {
                        if (skip == 0) walk_advance<true, false, 0>(acc[j], bf, bufs, b, weak, true);
                        else walk_advance<true, false, 4>(acc[j], bf, bufs, b, weak, true);
                    } else {
                        if (skip == 0) walk_advance<false, false, 0>(acc[j], bf, bufs, b, weak, false);
                        else walk_advance<false, false, 4>(acc[j], bf, bufs, b, weak, false);
                    }
                }
                if (more && j + 1 == nu) put_state(acc[0], bufs, b ^ 1, nt);
                // sn's loads, issued at the step's start, are waited for here
                // on every path.  Otherwise the copy into sr, placed after
                // the branch, waits on a count that must also hold on the
                // path without the B^T reload, which on the reload path
                // means waiting for most of those 16 younger loads.
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                if (j == nu - 1 && c + 1 < w.nck) load_bt(c + 1);
                sr = sn;
                __syncthreads();
            }
        }
    }
    if (fin) {
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            if (j < nu) {
                const int h = w.head(pl, j), pt = w.tile(j);
                const __amdgpu_buffer_rsrc_t rf =
                    buffer_rsrc(fin + ((size_t)w.s * H + h) * P * N, (uint32_t)(P * N * 4));
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    // the element goes through a scalar first: a bit cast of a
                    // vector element expression compiles to element 0
                    const float e = acc[j][v];
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, e), rf,
                                                          state_off(v, pt, nt, P, N), 0, 0);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ outputs (waves 0-3)
// Output block TI (tokens 32 TI .. 32 TI + 31, the tile's 32 columns) of one
// unit: the state term C_rows . h_c^T from the staged hi/lo state.  The intra-chunk
// term is the Horner scheme of the chunk scan: two chains over the blocks
// kj <= TI with the (C.B^T) rows ga as A and the staged (x wb)^T as B, the
// diagonal block inside the scheme when its decay is below kFastDecay (then
// scaled by ue), else added with exact per-element factors after scaling by
// ul.  y leaves through the wave's LDS tile as 16-byte row pieces.
template <typename TY, int TI, bool SKIP>
__device__ __forceinline__ void walk_block(const bf16x8 (&ga)[TI + 1][2], const bf16x8 (&ca)[kNT / 16],
                                           bool has_state, const bf16_t* shrow, const bf16_t* slrow,
                                           const WalkTables& tb, const bf16_t* xhrow, const bf16_t* xrrow,
                                           float* ep, __amdgpu_buffer_rsrc_t ry, int yb0, int rowb, int len,
                                           int pcols, float Dh) {
    const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    // the state term C_rows . h_c^T, a chain of its own: hi and lo, or hi
    // alone once the block's first token has decayed by kLoSkipDecay since
    // the chunk's start (every row of the term is then scaled by less than
    // exp(-kLoSkipDecay)), or none once it has decayed by kStateSkipDecay
    // (the term is then below the hi half's rounding at kLoSkipDecay), where
    // SKIP is set; a NaN keeps both halves
    f32x16 sacc = {};
    if (has_state) {
        const float cs0 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                        __builtin_bit_cast(int, tb.cs[32 * TI])));
        if (!(cs0 <= -kLoSkipDecay)) {
#pragma unroll
            for (int s = 0; s < kNT / 16; ++s) {
                mma16(sacc, ca[s], Tr<bf16_t>::ld8(shrow + 16 * s));
                mma16(sacc, ca[s], Tr<bf16_t>::ld8(slrow + 16 * s));
            }
        } else if (!SKIP || !(cs0 <= -kStateSkipDecay)) {
#pragma unroll
            for (int s = 0; s < kNT / 16; ++s) mma16(sacc, ca[s], Tr<bf16_t>::ld8(shrow + 16 * s));
        }
    }
    const int flags = __builtin_amdgcn_readfirstlane(tb.fast[TI]);
    // Every branch below leaves the sum in the chain of TI's parity (acc):
    // where the branches meet only acc is live, in the same registers on all
    // paths.
    f32x16 ce = {}, co = {};
    f32x16& acc = (TI & 1) ? co : ce;
    f32x16& other = (TI & 1) ? ce : co;
    auto scale_rows = [&](const float* scale) {
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
            const f32x4 u = *(const f32x4*)(scale + 32 * TI + 8 * vg + 4 * half);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[4 * vg + i] *= u[i];
        }
    };
    if (flags & 2) {
        // weakly decaying chunk: weights to the chunk's end, one unscaled
        // chain over the blocks kj <= TI (the C.B^T tiles are causal), the
        // state term scaled by exp(cs_last), rows by exp(cs_t - cs_last)
#pragma unroll
        for (int kj = 0; kj <= TI; ++kj)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mma16(acc, ga[kj][ks], Tr<bf16_t>::ld8(xhrow + 32 * kj + 16 * ks));
        if (has_state) acc += tb.gam[0] * sacc;
        scale_rows(tb.ue);
    } else {
        const bool fast = flags & 1;
        // blocks kj < TI: two chains (even and odd blocks), each stepping two
        // blocks at a time with the product of their decays
#pragma unroll
        for (int kj = 0; kj < TI; ++kj) {
            f32x16& ch = (kj & 1) ? co : ce;
            if (kj >= 2) ch *= tb.gam[kj - 1] * tb.gam[kj];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mma16(ch, ga[kj][ks], Tr<bf16_t>::ld8(xhrow + 32 * kj + 16 * ks));
        }
        // the chain that ends at the last included block K is complete; the other
        // one still takes the decay across block K.  K is TI (diagonal block in
        // the scheme) or TI - 1, so each branch knows both chains' roles.  Each
        // branch also adds the state term and applies its row scaling.
        if (fast) {
            // acc ends at TI - 2: across blocks TI - 1 and TI, then block TI
            if (TI >= 2) acc *= tb.gam[TI - 1] * tb.gam[TI];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mma16(acc, ga[TI][ks], Tr<bf16_t>::ld8(xhrow + 32 * TI + 16 * ks));
            if (TI >= 1) acc += tb.gam[TI] * other;
            if (has_state) acc += __expf(tb.cs[32 * TI + 31]) * sacc;
            scale_rows(tb.ue);
        } else {
            // K = TI - 1 ends other; acc (ends at TI - 2, or zero) takes block
            // K's decay.  TI = 1: other is block 0's chain, acc zero.
            if (TI >= 1) acc = other + tb.gam[TI - 1] * acc;
            if (has_state) acc += (TI > 0 ? __expf(tb.cs[32 * TI - 1]) : 1.f) * sacc;
            scale_rows(tb.ul);
            // the diagonal block with exact per-element factors
            const float cst = tb.cs[32 * TI + col];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int k0 = 32 * TI + 16 * ks + 8 * half;
                const f32x8 gv = Tr<bf16_t>::widen(ga[TI][ks]);
                f32x8 m;
#pragma unroll
                for (int i = 0; i < 8; ++i) m[i] = gv[i] * (__expf(fminf(cst - tb.cs[k0 + i], 0.f)) * tb.dt[k0 + i]);
                mma16(acc, Tr<bf16_t>::narrow(m), Tr<bf16_t>::ld8(xrrow + k0));
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4 xv = Tr<bf16_t>::ld4(xrrow + 32 * TI + 8 * q + 4 * half);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * q + i] += Dh * xv[i];
    }
    // through the wave's LDS tile: lane (column) writes its 16 rows, then
    // each lane reads 4 consecutive columns of one row (one wave: its LDS
    // operations complete in order); every lane stores, an output outside
    // the chunk or past P getting an offset beyond the descriptor
#pragma unroll
    for (int v = 0; v < 16; ++v) ep[acc_row(v, lane) * kEpPitch + col] = acc[v];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int tr = (lane >> 3) + 8 * it, c4 = 4 * (lane & 7);
        const f32x4 r = *(const f32x4*)(ep + tr * kEpPitch + c4);
        // the row bound and the offset as one lane term and a uniform one:
        // folded together, each row group's lane offset is loop-invariant,
        // gets hoisted, and the eight of them spill
        const int rows = __builtin_amdgcn_readfirstlane(len - 32 * TI - 8 * it);
        const int uoff = __builtin_amdgcn_readfirstlane((32 * TI + 8 * it) * rowb + yb0);
        const bool ok = (lane >> 3) < rows && c4 < pcols;
        buffer_store4<TY>(r, ry, ok ? (lane >> 3) * rowb + c4 * (int)sizeof(TY) + uoff : kOutOfRange);
    }
    __builtin_amdgcn_wave_barrier();
}

template <typename TY, int TA, int TB, bool SKIP>
__device__ void walk_outputs(const Plan& pl, const Walk& w, const WalkBufs& bufs, const bf16_t* __restrict__ Cm,
                             const bf16_t* __restrict__ cb, const float* __restrict__ D, bool has_init,
                             TY* __restrict__ y) {
    const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    const int H = pl.H, P = pl.P, N = pl.N, G = pl.G, HP = H * P;
    bf16x8 ga_a[TA + 1][2], ga_b[TB + 1][2], ca_a[kNT / 16], ca_b[kNT / 16];
    // the chunk's operands of one output block: its C.B^T rows (A of the
    // intra-chunk term) and C rows (A of the state term).  C goes through a
    // buffer over the chunk's rows (one 32-bit offset, the k-steps as
    // immediate offsets); columns n >= N (the padding of a dstate below 128)
    // are zeroed after the load.  That select waits for the loads, and the
    // wait covers the y stores issued before them, so it sits behind a
    // uniform branch that dstate 128 skips: there the loads are first used
    // in the next step.
    auto load_block = [&](int c, auto ti, auto& ga, bf16x8 (&ca)[kNT / 16]) {
        constexpr int TI = decltype(ti)::value;
        const ChunkDesc d = w.chunk(c);
        // buffers from the block's first row, so that the lane offsets are
        // the same for both blocks and every chunk
        const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(
            cb + (((size_t)(w.chunk0 + c) * G + w.g) * kQ + 32 * TI) * kQ, (uint32_t)(32 * kQ * 2));
        const int goff = (col * kQ + 8 * half) * 2;
#pragma unroll
        for (int kj = 0; kj <= TI; ++kj)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) ga[kj][ks] = buffer_ld8<bf16_t>(rg, goff + (32 * kj + 16 * ks) * 2);
        // C rows past the chunk's end read as zero (their y is not stored)
        // (the byte count through readfirstlane: computed on the vector
        // unit it would make the descriptor look divergent)
        const int cbytes = __builtin_amdgcn_readfirstlane(max(d.len - 32 * TI, 0) * G * N * 2);
        const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(Cm + (d.row0 + 32 * TI) * G * N, (uint32_t)cbytes);
        const int off = ((col * G + w.g) * N + 8 * half) * 2;
#pragma unroll
        for (int s = 0; s < kNT / 16; ++s) ca[s] = buffer_ld8<bf16_t>(rc, off + 32 * s);
        if (N < kNT) {
#pragma unroll
            for (int s = 0; s < kNT / 16; ++s)
                if (16 * s + 8 * half >= N) ca[s] = bf16x8{};
        }
    };
    using IA = std::integral_constant<int, TA>;
    using IB = std::integral_constant<int, TB>;
    if (w.nck > 0) {
        load_block(0, IA{}, ga_a, ca_a);
        load_block(0, IB{}, ga_b, ca_b);
    }
    __syncthreads();
    for (int c = 0; c < w.nck; ++c) {
        const ChunkDesc d = w.chunk(c);
        const bool has_state = c > 0 || has_init;
        const __amdgpu_buffer_rsrc_t ry =
            buffer_rsrc(y + d.row0 * HP, (uint32_t)((size_t)d.len * HP * sizeof(TY)));
        for (int j = 0; j < w.nu; ++j) {
            const int i = c * w.nu + j, b = i & 1;
            const int h = w.head(pl, j), pt = w.tile(j);
            const float Dh = D[h];
            const bf16_t* shrow = bufs.sh(b) + col * kNS + 8 * half;
            const bf16_t* slrow = bufs.sl(b) + col * kNS + 8 * half;
            const WalkTables tb = walk_tables(bufs.stage(b));
            const bf16_t* xhrow = bufs.xh(b) + col * kLP + 8 * half;
            const bf16_t* xrrow = bufs.xr(b) + col * kLP;
            const int pcols = P - 32 * pt;
            const int rowb = HP * (int)sizeof(TY);
            const int yb0 = (h * P + 32 * pt) * (int)sizeof(TY);
            float* ep = bufs.ep(threadIdx.x >> 6);
            // one block at a time: overlapping the two would need both blocks'
            // accumulators at once.  After the chunk's last unit each block's
            // registers are refilled with the next chunk's operands as soon as
            // the block is done, so the reload spreads over the step instead
            // of leaving together at its end.
            const bool reload = j == w.nu - 1 && c + 1 < w.nck;
            // Before each (conditional) reload, everything but the block's
            // own 4 y stores is waited for, on both paths: the other block's
            // operands, reloaded a block earlier, are then known to have
            // arrived.  Without it the wait before their first use has to
            // hold on the path without this reload too, and on the reload
            // path it then also waits for most of the younger reload loads.
            walk_block<TY, TA, SKIP>(ga_a, ca_a, has_state, shrow, slrow, tb, xhrow, xrrow, ep, ry, yb0, rowb, d.len,
                               pcols, Dh);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt4);
            if (reload) load_block(c + 1, IA{}, ga_a, ca_a);
            __builtin_amdgcn_sched_barrier(0);
            walk_block<TY, TB, SKIP>(ga_b, ca_b, has_state, shrow, slrow, tb, xhrow, xrrow, ep, ry, yb0, rowb, d.len,
                               pcols, Dh);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt4);
            if (reload) load_block(c + 1, IB{}, ga_b, ca_b);
            __syncthreads();
        }
    }
}

// Per (sequence, head), one wave: for each chunk, its cs_last and the decay
// from its end to the sequence's end (the sum of -cs_last over the later
// chunks), in windows of 64 chunks from the sequence's end, lane c of a
// window holding chunk base + c.  cs_last is copied bit for bit; the decay
// only decides whether the advance takes the lo half.
__global__ __launch_bounds__(256) void ssd_walk_tail_kernel(Plan pl, const float* __restrict__ cs,
                                                            float* __restrict__ tail) {
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= (int64_t)pl.nseq * pl.H) return;
    const int H = pl.H;
    const int s = (int)(pair / H), h = (int)(pair % H);
    const SeqExtent se = seq_extent(pl, s);
    float later = 0.f;  // decay of the chunks after the current window
    for (int end = se.nchunks; end > 0; end -= 64) {
        const int c = end - 64 + lane;
        const bool ok = c >= 0;
        const size_t k = (size_t)se.chunk0 + (ok ? c : 0);
        const float cl = ok ? cs[(k * H + h) * kQ + kQ - 1] : 0.f;
        const float v = -cl;
        const float incl = wave_inclusive_scan(v);  // the window's chunks up to c
        const float total = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
        if (ok) *(f32x2*)(tail + 2 * (k * H + h)) = f32x2{cl, later + (total - incl)};
        later += total;
    }
}

template <typename TY, int NU>
__global__ __launch_bounds__(512, 1) void ssd_scan_walk_kernel(
    Plan pl, int run, int npt, int nslice, int nus, const bf16_t* __restrict__ x, const float* __restrict__ cs,
    const float* __restrict__ dtc, const float* __restrict__ tail, const bf16_t* __restrict__ Cm,
    const bf16_t* __restrict__ cb,
    const bf16_t* __restrict__ bt, const float* __restrict__ D, const float* __restrict__ init,
    float* __restrict__ fin, TY* __restrict__ y) {
    extern __shared__ __align__(16) char smem[];
    Walk w;
    if (!walk_of(pl, run, npt, nslice, nus, w)) return;
    const WalkBufs bufs{smem};
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Output wave w takes blocks w and 7 - w.  With several units per
    // workgroup the larger block goes first: at a chunk switch its reload
    // then leaves first and has the most time to arrive, while the smaller
    // block's reload is needed only after the larger block's work in the next
    // step.  With one unit every step switches chunks, and the smaller block
    // goes first, so that the larger block's reload has the smaller block's
    // work, not its own, to hide behind.  The state term's skip in blocks
    // that have decayed by kStateSkipDecay follows the same split: it gains
    // with two or more units and measured slower with one.
    constexpr bool kLargeFirst = NU > 1;
    const bool has_init = init != nullptr;
    switch (wave) {
        case 0:
            walk_outputs<TY, kLargeFirst ? 7 : 0, kLargeFirst ? 0 : 7, kLargeFirst>(pl, w, bufs, Cm, cb, D, has_init, y);
            break;
        case 1:
            walk_outputs<TY, kLargeFirst ? 6 : 1, kLargeFirst ? 1 : 6, kLargeFirst>(pl, w, bufs, Cm, cb, D, has_init, y);
            break;
        case 2:
            walk_outputs<TY, kLargeFirst ? 5 : 2, kLargeFirst ? 2 : 5, kLargeFirst>(pl, w, bufs, Cm, cb, D, has_init, y);
            break;
        case 3:
            walk_outputs<TY, kLargeFirst ? 4 : 3, kLargeFirst ? 3 : 4, kLargeFirst>(pl, w, bufs, Cm, cb, D, has_init, y);
            break;
        default: walk_states<NU>(pl, w, bufs, x, cs, dtc, tail, bt, init, fin); break;
    }
}

template <typename TY, int NU>
hipError_t run_walk(const Plan& pl, const WalkArgs& a, hipStream_t stream) {
    auto* k = ssd_scan_walk_kernel<TY, NU>;
    hipError_t err = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWalkLds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k, dim3(8 * a.per_xcd), dim3(512), kWalkLds, stream, pl, a.run, a.npt, a.nslice, a.nus,
                       (const bf16_t*)a.x, a.cs, a.dtc, a.tail, (const bf16_t*)a.C, (const bf16_t*)a.cb,
                       (const bf16_t*)a.bt, a.D, a.init, a.final_state, (TY*)a.y);
    return hipGetLastError();
}

template <typename TY>
hipError_t dispatch_walk(const Plan& pl, const WalkArgs& a, hipStream_t stream) {
    switch (a.nus) {
        case 1: return run_walk<TY, 1>(pl, a, stream);
        case 2: return run_walk<TY, 2>(pl, a, stream);
        case 3: return run_walk<TY, 3>(pl, a, stream);
        case 4: return run_walk<TY, 4>(pl, a, stream);
        case 5: return run_walk<TY, 5>(pl, a, stream);
        case 6: return run_walk<TY, 6>(pl, a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool scan_walk_supported(int dtype, int N, int Q) { return dtype == 1 && Q == kQ && N > 64 && N <= kNT; }

size_t scan_walk_lds_bytes() { return kWalkLds; }

hipError_t launch_scan_walk(const Plan& pl, const WalkArgs& a, hipStream_t stream) {
    if (a.per_xcd <= 0) return hipSuccess;
    const int64_t pairs = (int64_t)pl.nseq * pl.H;
    hipLaunchKernelGGL(ssd_walk_tail_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, stream, pl, a.cs,
                       a.tail);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return a.y_f32 ? dispatch_walk<float>(pl, a, stream) : dispatch_walk<bf16_t>(pl, a, stream);
}

}  // namespace ssd
