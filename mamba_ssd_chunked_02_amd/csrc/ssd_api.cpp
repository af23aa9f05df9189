// Host side of the C ABI declared in include/ssd.h: argument validation (pure
// host code, before any launch), the chunk plan, the workspace carve and the
// kernel queueing.  Nothing here allocates, frees or synchronizes.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>

#include "ssd.h"
#include "ssd_internal.h"

#define SSD_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_detail[320] = "";

ssd_status fail(ssd_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return st;
}

ssd_status ok() {
    g_detail[0] = '\0';
    return SSD_OK;
}

}  // namespace

namespace ssd {

int32_t set_error_detail(int32_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return st;
}

}  // namespace ssd

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Alignment each pointer argument needs: dt, A, D and the dt bias are fp32
// vectors that every kernel reads one element at a time (4 bytes); every
// other tensor is read or written with 16-byte accesses.
struct PtrArg {
    const void* p;
    const char* name;
    bool required;
    int align;
};

ssd_status check_ptrs(const PtrArg* args, int n) {
    for (int i = 0; i < n; ++i) {
        const PtrArg& q = args[i];
        if (!q.p && q.required) {
            if (q.name[0] == 'w') return fail(SSD_ERR_WORKSPACE, "workspace is NULL");
            return fail(SSD_ERR_NULL, "%s is NULL", q.name);
        }
        if (q.p && ((uintptr_t)q.p & (uintptr_t)(q.align - 1)) != 0)
            return fail(SSD_ERR_ALIGN, "%s is not %d-byte aligned", q.name, q.align);
    }
    return SSD_OK;
}

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

constexpr size_t kMaxLds = 160 * 1024;  // LDS per CU on gfx950
constexpr int64_t kMaxGrid = ((int64_t)1 << 31) - 8;
// chunk-parallel chunk_state: ~8 workgroups per CU (three fit at once), at most 16 heads each
constexpr int64_t kStateWorkgroups = 2048;
constexpr int64_t kStateMaxHeads = 16;
// chunk_scan: one 8-wave workgroup fits per CU; one per CU, each walking as
// many heads as that allows (up to the whole group), amortizes the
// per-workgroup block operands and prologue best
constexpr int64_t kScanWorkgroups = 256;
constexpr int64_t kFusedMinWalks = 256;  // one per CU
// where the scan walk applies (bf16, chunk 256, dstate in (64, 128]) and a
// walk is the right shape, the library's own choice takes it: it moves
// about half the bytes of the state walk followed by chunk_scan
constexpr bool kAutoScanWalk = true;

struct Prepared {
    ssd::Plan plan;
    ssd::Layout lay;
    int32_t path;       // ssd::kPath*
    int32_t walk_nus;    // scan walk: units per workgroup
    int32_t walk_nslice; // scan walk: workgroups per (sequence, group)
};

// The scan walk's work split: each workgroup walks at most kWalkMaxUnits
// (head, column tile) units of one group, the group's units cut into equal
// slices.  A workgroup's chunk step takes about kWalkStepFixedUs + n
// kWalkStepUnitUs for n units: the output waves' per-chunk work and the
// operand reload are shared by the units.  Measured on the 2.7B-shaped layer
// (L8192 H80), one round of workgroups each: at batch 4, 6, 8 and 9 (216 to
// 256 busy CUs, 3 to 6 units) 14.2, 18.3, 22.5 and 26.0 us per chunk step,
// whose least-squares line is 2.34 + 3.98 n; at batch 2 (160 CUs, 2 units)
// 9.35 us, below the line, as fewer CUs share L2 and HBM.
constexpr int64_t kXcds = 8, kCusPerXcd = 32;
constexpr int64_t kWalkMaxUnits = 6;
constexpr double kWalkStepFixedUs = 2.34, kWalkStepUnitUs = 3.98;

// Sequences of equal length: one 8-wave workgroup fits per CU, so a launch
// runs in rounds of 32 workgroups per XCD; the split with the least rounds x
// step time wins, the one with more workgroups on a tie.
void walk_split(const ssd::Plan& pl, int32_t* nus, int32_t* nslice) {
    const int64_t npt = (pl.P + 31) / 32;
    const int64_t upg = (int64_t)pl.hpg * npt;
    const int64_t walks = (int64_t)pl.nseq * pl.G;
    double best = 0.0;
    for (int64_t n = 1; n <= std::min(kWalkMaxUnits, upg); ++n) {
        const int64_t ns = (upg + n - 1) / n, nu = (upg + ns - 1) / ns;
        const int64_t per_xcd = (walks * ns + kXcds - 1) / kXcds;
        const int64_t rounds = std::max<int64_t>(1, (per_xcd + kCusPerXcd - 1) / kCusPerXcd);
        const double cost = (double)rounds * (kWalkStepFixedUs + kWalkStepUnitUs * (double)nu);
        if (n == 1 || cost < best) {
            best = cost;
            *nslice = (int32_t)ns;
            *nus = (int32_t)nu;
        }
    }
}

// A packed batch whose lengths the host holds, with at most kOrderMaxSeq
// sequences: the walk starts its longest pairs first (the plan kernel orders
// the sequences by chunk count), so it takes about the longer of its longest
// walks and its total work spread over the CUs.  The split with the least
// such time wins.  The chunk-parallel kernels take about kChunkParallelNs per
// token, head and 8192 state elements (measured 0.26-0.27 ns on the grouped
// packed batch, on one 32K-token sequence and at the 2.7B shape) plus
// kChunkParallelFixedUs (their launches; 20-90 us measured on smaller
// batches); the library's choice walks when that is expected to be at least
// 10% faster.
constexpr double kChunkParallelNs = 0.265;
constexpr double kChunkParallelFixedUs = 40.0;
constexpr double kWalkMargin = 0.9;

struct PackedWalk {
    int32_t nus = 0, nslice = 0;
    double us = 0.0;
};

PackedWalk packed_walk(const ssd::Plan& pl, const int32_t* cu) {
    const int64_t npt = (pl.P + 31) / 32;
    const int64_t upg = (int64_t)pl.hpg * npt;
    int64_t total = 0, longest = 0, nlong = 0;
    for (int64_t s = 0; s < pl.nseq; ++s) {
        const int64_t nc = ((int64_t)cu[s + 1] - cu[s] + pl.Q - 1) / pl.Q;
        total += nc;
        if (nc > longest) longest = nc, nlong = 0;
        if (nc == longest) ++nlong;
    }
    PackedWalk best;
    const int64_t cus = kXcds * kCusPerXcd;
    for (int64_t n = 1; n <= std::min(kWalkMaxUnits, upg); ++n) {
        const int64_t ns = (upg + n - 1) / n, nu = (upg + ns - 1) / ns;
        const double step = kWalkStepFixedUs + kWalkStepUnitUs * (double)nu;
        // the longest sequences' workgroups start together, in rounds when
        // they outnumber the CUs
        const int64_t rounds = (nlong * pl.G * ns + cus - 1) / cus;
        const double crit = (double)(rounds * longest) * step;
        const double spread = (double)total * (double)(pl.G * ns) * step / (double)cus;
        const double us = std::max(crit, spread);
        if (n == 1 || us < best.us) {
            best.nus = (int32_t)nu;
            best.nslice = (int32_t)ns;
            best.us = us;
        }
    }
    return best;
}

double chunk_parallel_us(const ssd::Plan& pl) {
    return kChunkParallelNs * 1e-3 * (double)pl.T * pl.H * ((double)pl.P * pl.N / 8192.0) + kChunkParallelFixedUs;
}

// Heads of one group that a chunk_state / chunk_scan workgroup walks: the
// group's per-chunk operands are loaded once per workgroup, so more heads per
// workgroup means less L2 traffic and prologue, as long as about `target`
// workgroups remain.
int heads_per_workgroup(const ssd::Plan& pl, int64_t target, int64_t max_heads) {
    const int64_t npt = (pl.P + 31) / 32;
    const int64_t units = (int64_t)pl.nchunk_ub * pl.H * npt;
    int64_t hpw = units / target;
    hpw = std::max<int64_t>(1, std::min<int64_t>(hpw, std::min<int64_t>(max_heads, pl.hpg)));
    // equal slices: the fewest slices of at most hpw heads, then spread evenly
    const int64_t nslice = (pl.hpg + hpw - 1) / hpw;
    return (int)((pl.hpg + nslice - 1) / nslice);
}

// Chunk states and the passing between chunks in one launch when there are
// enough (sequence, head, column tile) walks to fill the chip: each walk is
// sequential over its sequence's chunks, so with few of them the separate
// kernels, parallel over chunks, finish first.  A walk also lasts as long as
// its sequence: when the host copy of a packed batch's offsets shows the
// longest sequence with more than 1.5 times the mean chunk count of the
// non-empty ones, the chunk-parallel kernels finish first too.
bool fuse_state_passing(const ssd::Plan& pl, const ssd_shape* sh) {
    const int64_t npt = (pl.P + 31) / 32;
    if ((int64_t)pl.nseq * pl.H * npt < kFusedMinWalks) return false;
    if (!pl.dense && sh->cu_seqlens_host) {
        const int32_t* cu = sh->cu_seqlens_host;
        int64_t total = 0, longest = 0, nonempty = 0;
        for (int64_t s = 0; s < pl.nseq; ++s) {
            const int64_t nc = ((int64_t)cu[s + 1] - cu[s] + pl.Q - 1) / pl.Q;
            total += nc;
            longest = std::max(longest, nc);
            nonempty += nc > 0;
        }
        if (nonempty > 0 && 2 * longest * nonempty > 3 * total) return false;
    }
    return true;
}

ssd_status check_head_dims(const ssd_shape* sh) {
    if (sh->dtype != SSD_F32 && sh->dtype != SSD_BF16)
        return fail(SSD_ERR_DTYPE, "dtype %d is neither SSD_F32 (0) nor SSD_BF16 (1)", sh->dtype);
    if (sh->ydtype != SSD_F32 && sh->ydtype != SSD_BF16)
        return fail(SSD_ERR_DTYPE, "ydtype %d is neither SSD_F32 (0) nor SSD_BF16 (1)", sh->ydtype);
    if (sh->reserved != 0) return fail(SSD_ERR_SHAPE, "reserved must be 0");
    if (sh->path < SSD_PATH_AUTO || sh->path > SSD_PATH_SCAN_WALK)
        return fail(SSD_ERR_VALUE, "path %d is not one of the SSD_PATH_* values", sh->path);
    if (sh->nheads < 1) return fail(SSD_ERR_SHAPE, "nheads must be >= 1 (got %d)", sh->nheads);
    if (sh->ngroups < 1 || sh->nheads % sh->ngroups != 0)
        return fail(SSD_ERR_SHAPE, "ngroups %d must be >= 1 and divide nheads %d", sh->ngroups,
                    sh->nheads);
    if (sh->headdim < 8 || sh->headdim > 128 || sh->headdim % 8 != 0)
        return fail(SSD_ERR_SHAPE, "headdim %d must be a multiple of 8 in [8, 128]", sh->headdim);
    if (sh->dstate < 8 || sh->dstate > 256 || sh->dstate % 8 != 0)
        return fail(SSD_ERR_SHAPE, "dstate %d must be a multiple of 8 in [8, 256]", sh->dstate);
    if (sh->batch < 0) return fail(SSD_ERR_SHAPE, "batch must be >= 0 (got %lld)", (long long)sh->batch);
    return SSD_OK;
}

ssd_status prepare(const ssd_shape* sh, int32_t chunk, Prepared* out) {
    if (!sh) return fail(SSD_ERR_NULL, "shape is NULL");
    ssd_status st = check_head_dims(sh);
    if (st != SSD_OK) return st;
    if (chunk != 32 && chunk != 64 && chunk != 128 && chunk != 256)
        return fail(SSD_ERR_CHUNK, "chunk %d is not one of 32, 64, 128, 256", chunk);
    if (sh->seqlen < 0) return fail(SSD_ERR_SHAPE, "seqlen must be >= 0");
    const bool packed = sh->cu_seqlens != nullptr;
    const int64_t nseq = sh->batch;
    const int64_t T = packed ? sh->seqlen : sh->batch * sh->seqlen;
    if (sh->batch > (1 << 24) || sh->seqlen > ((int64_t)1 << 30) || T > ((int64_t)1 << 30))
        return fail(SSD_ERR_SHAPE, "token count %lld exceeds the supported 2^30", (long long)T);
    if (T * sh->nheads * (int64_t)sh->headdim > ((int64_t)1 << 40))
        return fail(SSD_ERR_SHAPE, "tensor too large");
    if (packed && sh->cu_seqlens_host) {
        const int32_t* cu = sh->cu_seqlens_host;
        if (cu[0] != 0) return fail(SSD_ERR_SEQLENS, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
        for (int64_t s = 0; s < nseq; ++s)
            if (cu[s + 1] < cu[s])
                return fail(SSD_ERR_SEQLENS, "cu_seqlens decreases at %lld", (long long)s);
        if (cu[nseq] != T)
            return fail(SSD_ERR_SEQLENS, "cu_seqlens[batch] = %d differs from seqlen %lld", cu[nseq],
                        (long long)T);
    }
    if (!packed && sh->cu_seqlens_host)
        return fail(SSD_ERR_SHAPE, "cu_seqlens_host given without the device cu_seqlens");
    const size_t lds = ssd::prefill_lds_bytes(sh->dtype, sh->dstate, chunk);
    if (lds > kMaxLds)
        return fail(SSD_ERR_UNSUPPORTED,
                    "dstate %d, chunk %d and dtype %d need %zu bytes of LDS (> %zu); use a smaller chunk",
                    sh->dstate, chunk, sh->dtype, lds, kMaxLds);

    ssd::Plan& pl = out->plan;
    pl = ssd::Plan{};
    pl.H = sh->nheads;
    pl.P = sh->headdim;
    pl.N = sh->dstate;
    pl.G = sh->ngroups;
    pl.hpg = sh->nheads / sh->ngroups;
    pl.Q = chunk;
    pl.nseq = (int32_t)nseq;
    pl.dense = packed ? 0 : 1;
    pl.T = T;
    pl.cu = sh->cu_seqlens;
    int64_t nchunks;
    if (!packed) {
        pl.L = sh->seqlen;
        pl.cpseq = (int32_t)((sh->seqlen + chunk - 1) / chunk);
        nchunks = nseq * pl.cpseq;
    } else {
        pl.L = 0;
        // every sequence wastes less than one chunk
        nchunks = nseq == 0 ? 0 : (T + nseq * (int64_t)(chunk - 1)) / chunk;
    }
    const int64_t npt = (sh->headdim + 31) / 32;
    const int64_t nblk = ((int64_t)sh->headdim * sh->dstate / 4 + 255) / 256;
    if (nchunks * sh->nheads * npt > kMaxGrid || nseq * sh->nheads * nblk > kMaxGrid ||
        nseq * sh->nheads * npt > kMaxGrid ||
        (sh->nheads + 3) / 4 > 65535 || sh->ngroups > 65535)
        return fail(SSD_ERR_SHAPE, "problem too large for one launch grid");
    // one chunk of x or y is addressed with 32-bit byte offsets
    if ((int64_t)chunk * sh->nheads * sh->headdim * 4 >= ((int64_t)1 << 31))
        return fail(SSD_ERR_SHAPE, "nheads * headdim %lld too large", (long long)sh->nheads * sh->headdim);
    pl.nchunk_ub = (int32_t)nchunks;

    // kernel path: the caller's, or the library's choice
    const bool walk_ok = ssd::scan_walk_supported(sh->dtype, sh->dstate, chunk);
    if (sh->path == SSD_PATH_SCAN_WALK && !walk_ok)
        return fail(SSD_ERR_UNSUPPORTED,
                    "the scan walk needs bf16 inputs, 256-token chunks and dstate in (64, 128]");
    if (sh->path != SSD_PATH_AUTO) out->path = sh->path;
    else if (!fuse_state_passing(pl, sh)) out->path = ssd::kPathChunkParallel;
    else out->path = (walk_ok && kAutoScanWalk) ? ssd::kPathScanWalk : ssd::kPathStateWalk;
    walk_split(pl, &out->walk_nus, &out->walk_nslice);
    // a packed batch with its lengths on the host: the walk's split, and for
    // the library's choice whether to walk, from the longest-first estimate
    if (walk_ok && packed && sh->cu_seqlens_host && nseq <= ssd::kOrderMaxSeq &&
        (sh->path == SSD_PATH_AUTO || sh->path == SSD_PATH_SCAN_WALK)) {
        const PackedWalk pw = packed_walk(pl, sh->cu_seqlens_host);
        if (sh->path == SSD_PATH_SCAN_WALK || pw.us < kWalkMargin * chunk_parallel_us(pl)) {
            out->path = ssd::kPathScanWalk;
            out->walk_nus = pw.nus;
            out->walk_nslice = pw.nslice;
        } else {
            out->path = ssd::kPathChunkParallel;
        }
    }
    const bool scan_walk = out->path == ssd::kPathScanWalk;

    ssd::Layout& L = out->lay;
    const size_t es = sh->dtype == SSD_BF16 ? 2 : 4;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += up256(bytes);
        return at;
    };
    L.seq_tab = take(packed ? (size_t)nseq * 16 : 0);
    L.chunk_tab = take(packed ? (size_t)pl.nchunk_ub * 16 : 0);
    L.seq_order = take(packed && scan_walk ? (size_t)nseq * 4 : 0);
    L.cs = take((size_t)pl.nchunk_ub * pl.H * chunk * 4);
    L.dtc = take((size_t)pl.nchunk_ub * pl.H * chunk * 4);
    L.wst = take(scan_walk ? 0 : (size_t)pl.nchunk_ub * pl.H * chunk * 4);
    L.cb = take((size_t)pl.nchunk_ub * pl.G * chunk * chunk * es);
    L.bt = take((size_t)pl.nchunk_ub * pl.G * ssd::padded_dstate(pl.N) * chunk * es);
    L.states = take(scan_walk ? 0 : (size_t)pl.nchunk_ub * pl.H * pl.P * pl.N * 4);
    L.tail = take(scan_walk ? (size_t)pl.nchunk_ub * pl.H * 8 : 0);
    L.total = std::max<size_t>(off, 256);
    return SSD_OK;
}

}  // namespace

SSD_API const char* ssd_status_string(int32_t status) {
    switch (status) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL: return "a required pointer is NULL";
        case SSD_ERR_SHAPE: return "a size is out of range or inconsistent";
        case SSD_ERR_DTYPE: return "unknown dtype";
        case SSD_ERR_ALIGN: return "a tensor pointer is not aligned as required";
        case SSD_ERR_CHUNK: return "chunk must be 32, 64, 128 or 256";
        case SSD_ERR_WORKSPACE: return "workspace missing or too small";
        case SSD_ERR_HIP: return "HIP runtime error";
        case SSD_ERR_UNSUPPORTED: return "valid but unsupported configuration";
        case SSD_ERR_SEQLENS: return "cu_seqlens is not a valid offset list";
        case SSD_ERR_VALUE: return "a scalar argument is out of range";
        default: return "unknown status";
    }
}

SSD_API const char* ssd_last_error_detail(void) { return g_detail; }

SSD_API ssd_status ssd_chunked_scan_workspace_size(const ssd_shape* shape, int32_t chunk,
                                                   size_t* bytes) {
    if (!bytes) return fail(SSD_ERR_NULL, "bytes is NULL");
    Prepared pr;
    const ssd_status st = prepare(shape, chunk, &pr);
    if (st != SSD_OK) return st;
    *bytes = pr.lay.total;
    return ok();
}

namespace {

ssd_status scan_impl(const void* x, const float* dt, const float* A, const void* B, const void* C,
                     const float* D, int32_t chunk, const float* init_state, void* y,
                     float* final_state, const ssd_shape* shape, void* workspace,
                     size_t workspace_bytes, void* stream, hipEvent_t* marks,
                     int* path_out = nullptr, const ssd::DtAct* act = nullptr) {
    Prepared pr;
    ssd_status st = prepare(shape, chunk, &pr);
    if (st != SSD_OK) return st;
    const bool any_tokens = pr.plan.T > 0;
    const PtrArg ptrs[] = {{x, "x", any_tokens, 16},          {dt, "dt", any_tokens, 4},
                           {A, "A", true, 4},                 {B, "B", any_tokens, 16},
                           {C, "C", any_tokens, 16},          {D, "D", true, 4},
                           {y, "y", any_tokens, 16},          {init_state, "init_state", false, 16},
                           {final_state, "final_state", false, 16}, {workspace, "workspace", true, 16}};
    st = check_ptrs(ptrs, (int)(sizeof(ptrs) / sizeof(ptrs[0])));
    if (st != SSD_OK) return st;
    if (workspace_bytes < pr.lay.total)
        return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                    pr.lay.total);
    if (y && (y == x || y == B || y == C || y == (const void*)dt))
        return fail(SSD_ERR_SHAPE, "y aliases an input");
    ssd::ScanArgs a;
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.init = init_state;
    a.y = y;
    a.final_state = final_state;
    a.ws = (char*)workspace;
    a.dtype = shape->dtype;
    a.y_f32 = shape->ydtype == SSD_F32 ? 1 : 0;
    a.hpw = heads_per_workgroup(pr.plan, kScanWorkgroups, pr.plan.hpg);
    a.hpw_state = heads_per_workgroup(pr.plan, kStateWorkgroups, kStateMaxHeads);
    a.path = pr.path;
    a.walk_nus = pr.walk_nus;
    a.walk_nslice = pr.walk_nslice;
    a.act = act ? *act : ssd::DtAct{nullptr, 0.f, 0.f, 0};
    if (path_out) *path_out = a.path;
    pr.plan.seq_tab = (int32_t*)(a.ws + pr.lay.seq_tab);
    pr.plan.chunk_tab = (int32_t*)(a.ws + pr.lay.chunk_tab);
    pr.plan.seq_order = !pr.plan.dense && a.path == ssd::kPathScanWalk ? (int32_t*)(a.ws + pr.lay.seq_order) : nullptr;
    if (pr.plan.nseq == 0 && !marks) return ok();
    const hipError_t err = ssd::launch_prefill(pr.plan, pr.lay, a, (hipStream_t)stream, marks);
    if (err != hipSuccess)
        return fail(SSD_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return ok();
}

}  // namespace

SSD_API ssd_status ssd_chunked_scan(const void* x, const float* dt, const float* A, const void* B,
                                    const void* C, const float* D, int32_t chunk,
                                    const float* init_state, void* y, float* final_state,
                                    const ssd_shape* shape, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return scan_impl(x, dt, A, B, C, D, chunk, init_state, y, final_state, shape, workspace,
                     workspace_bytes, stream, nullptr);
}

SSD_API ssd_status ssd_chunked_scan_profiled(const void* x, const float* dt, const float* A,
                                             const void* B, const void* C, const float* D,
                                             int32_t chunk, const float* init_state, void* y,
                                             float* final_state, const ssd_shape* shape,
                                             void* workspace, size_t workspace_bytes, void* stream,
                                             float* stage_ms) {
    if (!stage_ms) return fail(SSD_ERR_NULL, "stage_ms is NULL");
    static_assert(SSD_PREFILL_STAGES == ssd::kPrefillStages, "stage count");
    constexpr int kMarks = SSD_PREFILL_STAGES + 1;
    hipEvent_t ev[kMarks] = {};
    hipError_t err = hipSuccess;
    int made = 0;
    for (; made < kMarks && err == hipSuccess; ++made) err = hipEventCreate(&ev[made]);
    ssd_status st = SSD_OK;
    if (err != hipSuccess) {
        st = fail(SSD_ERR_HIP, "hipEventCreate failed: %s", hipGetErrorString(err));
        --made;
    } else {
        int path = 0;
        st = scan_impl(x, dt, A, B, C, D, chunk, init_state, y, final_state, shape, workspace,
                       workspace_bytes, stream, ev, &path);
        if (st == SSD_OK) err = hipEventSynchronize(ev[kMarks - 1]);
        for (int i = 0; st == SSD_OK && err == hipSuccess && i < SSD_PREFILL_STAGES; ++i)
            err = hipEventElapsedTime(&stage_ms[i], ev[i], ev[i + 1]);
        // stages a path does not run read exactly 0 (their marks are back to back)
        if (st == SSD_OK && err == hipSuccess) {
            if (path == ssd::kPathStateWalk) stage_ms[4] = 0.f;  // inside chunk_state
            if (path == ssd::kPathScanWalk) stage_ms[3] = stage_ms[4] = stage_ms[5] = 0.f;
            if (path != ssd::kPathScanWalk) stage_ms[6] = 0.f;
        }
        if (st == SSD_OK && err != hipSuccess)
            st = fail(SSD_ERR_HIP, "event timing failed: %s", hipGetErrorString(err));
    }
    for (int i = 0; i < made; ++i) (void)hipEventDestroy(ev[i]);
    return st;
}

namespace {

// Validated copy of an activation argument.
ssd_status dt_act_of(const ssd_dt_activation* act, ssd::DtAct* out) {
    if (!act) return fail(SSD_ERR_NULL, "act is NULL");
    if (act->dt_bias && !aligned4(act->dt_bias)) return fail(SSD_ERR_ALIGN, "dt_bias is not 4-byte aligned");
    const float lo = act->dt_min, hi = act->dt_max;
    if (!(lo >= 0.f) || lo > 3.0e38f) return fail(SSD_ERR_VALUE, "dt_min %g must be finite and >= 0", (double)lo);
    if (!(hi >= lo)) return fail(SSD_ERR_VALUE, "dt_max %g must be >= dt_min %g", (double)hi, (double)lo);
    *out = ssd::DtAct{act->dt_bias, lo, hi, 1};
    return SSD_OK;
}

ssd_status decode_impl(float* state, const void* x, const float* dt, const float* A, const void* B,
                       const void* C, const float* D, void* y, const ssd_shape* shape, void* stream,
                       const ssd::DtAct* act);

}  // namespace

SSD_API ssd_status ssd_chunked_scan_dt_act(const void* x, const float* dt_raw, const float* A,
                                           const void* B, const void* C, const float* D, int32_t chunk,
                                           const float* init_state, void* y, float* final_state,
                                           const ssd_dt_activation* act, const ssd_shape* shape,
                                           void* workspace, size_t workspace_bytes, void* stream) {
    ssd::DtAct a;
    const ssd_status st = dt_act_of(act, &a);
    if (st != SSD_OK) return st;
    return scan_impl(x, dt_raw, A, B, C, D, chunk, init_state, y, final_state, shape, workspace,
                     workspace_bytes, stream, nullptr, nullptr, &a);
}

SSD_API ssd_status ssd_decode_step_dt_act(float* state, const void* x, const float* dt_raw, const float* A,
                                          const void* B, const void* C, const float* D, void* y,
                                          const ssd_dt_activation* act, const ssd_shape* shape,
                                          void* stream) {
    ssd::DtAct a;
    const ssd_status st = dt_act_of(act, &a);
    if (st != SSD_OK) return st;
    return decode_impl(state, x, dt_raw, A, B, C, D, y, shape, stream, &a);
}

SSD_API ssd_status ssd_decode_step(float* state, const void* x, const float* dt, const float* A,
                                   const void* B, const void* C, const float* D, void* y,
                                   const ssd_shape* shape, void* stream) {
    return decode_impl(state, x, dt, A, B, C, D, y, shape, stream, nullptr);
}

namespace {

// Argument checks shared by the decode entry points (one token per sequence).
ssd_status check_decode(const float* state, const void* x, const float* dt, const float* A, const void* B,
                        const void* C, const float* D, const void* y, const ssd_shape* shape) {
    if (!shape) return fail(SSD_ERR_NULL, "shape is NULL");
    ssd_status st = check_head_dims(shape);
    if (st != SSD_OK) return st;
    const bool any = shape->batch > 0;
    const PtrArg ptrs[] = {{state, "state", any, 16}, {x, "x", any, 16}, {dt, "dt", any, 4},
                           {A, "A", true, 4},          {B, "B", any, 16}, {C, "C", any, 16},
                           {D, "D", true, 4},          {y, "y", any, 16}};
    st = check_ptrs(ptrs, (int)(sizeof(ptrs) / sizeof(ptrs[0])));
    if (st != SSD_OK) return st;
    if (y && (y == x || y == B || y == C || y == (const void*)state))
        return fail(SSD_ERR_SHAPE, "y aliases an input");
    if (shape->batch * (int64_t)shape->nheads * shape->headdim > ((int64_t)1 << 40))
        return fail(SSD_ERR_SHAPE, "tensor too large");
    // one wave per (sequence, head) block, at least one per workgroup
    if (shape->batch * (int64_t)shape->nheads > kMaxGrid)
        return fail(SSD_ERR_SHAPE, "batch * nheads %lld too large for one launch grid",
                    (long long)(shape->batch * (int64_t)shape->nheads));
    return SSD_OK;
}

ssd_status decode_impl(float* state, const void* x, const float* dt, const float* A, const void* B,
                       const void* C, const float* D, void* y, const ssd_shape* shape, void* stream,
                       const ssd::DtAct* act) {
    const ssd_status st = check_decode(state, x, dt, A, B, C, D, y, shape);
    if (st != SSD_OK) return st;
    ssd::DecodeArgs a;
    a.state = state;
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.y = y;
    a.batch = shape->batch;
    a.H = shape->nheads;
    a.P = shape->headdim;
    a.N = shape->dstate;
    a.G = shape->ngroups;
    a.dtype = shape->dtype;
    a.y_f32 = shape->ydtype == SSD_F32 ? 1 : 0;
    a.act = act ? *act : ssd::DtAct{nullptr, 0.f, 0.f, 0};
    const hipError_t err = ssd::launch_decode(a, (hipStream_t)stream);
    if (err != hipSuccess)
        return fail(SSD_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return ok();
}

constexpr int32_t kMaxWindow = 16;

}  // namespace

SSD_API ssd_status ssd_decode_window_step(float* state, const void* x, const float* dt, const float* A,
                                          const void* B, const void* C, const float* D, void* y,
                                          int32_t window, int32_t t, int32_t flush,
                                          const ssd_dt_activation* act, const ssd_shape* shape,
                                          void* stream) {
    ssd::DtAct da{nullptr, 0.f, 0.f, 0};
    if (act) {
        const ssd_status sa = dt_act_of(act, &da);
        if (sa != SSD_OK) return sa;
    }
    if (window < 1 || window > kMaxWindow)
        return fail(SSD_ERR_VALUE, "window %d must be in [1, %d]", window, kMaxWindow);
    if (t < 0 || t >= window) return fail(SSD_ERR_VALUE, "t %d must be in [0, window %d)", t, window);
    if (flush != 0 && flush != 1) return fail(SSD_ERR_VALUE, "flush must be 0 or 1 (got %d)", flush);
    const ssd_status st = check_decode(state, x, dt, A, B, C, D, y, shape);
    if (st != SSD_OK) return st;
    if (shape->batch * (int64_t)window * shape->nheads * shape->headdim > ((int64_t)1 << 40))
        return fail(SSD_ERR_SHAPE, "tensor too large");
    ssd::WindowArgs a;
    a.state = state;
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.y = y;
    a.batch = shape->batch;
    a.H = shape->nheads;
    a.P = shape->headdim;
    a.N = shape->dstate;
    a.G = shape->ngroups;
    a.W = window;
    a.t = t;
    a.flush = flush;
    a.dtype = shape->dtype;
    a.y_f32 = shape->ydtype == SSD_F32 ? 1 : 0;
    a.act = da;
    const hipError_t err = ssd::launch_decode_window(a, (hipStream_t)stream);
    if (err != hipSuccess)
        return fail(SSD_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return ok();
}

// ------------------------------------------------------------------ conv1d
namespace {

constexpr int32_t kMaxConvChannels = 1 << 20;

ssd_status check_cu_host(const int32_t* cu, int64_t nseq, int64_t T) {
    if (cu[0] != 0) return fail(SSD_ERR_SEQLENS, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
    for (int64_t s = 0; s < nseq; ++s)
        if (cu[s + 1] < cu[s]) return fail(SSD_ERR_SEQLENS, "cu_seqlens decreases at %lld", (long long)s);
    if (cu[nseq] != T)
        return fail(SSD_ERR_SEQLENS, "cu_seqlens[batch] = %d differs from seqlen %lld", cu[nseq], (long long)T);
    return SSD_OK;
}

// Validates what the prefill and the step share and fills `a` (rows = T for
// the prefill, batch for the step).
ssd_status conv_prepare(const void* x, const float* weight, const float* bias, const ssd_conv_outputs* out,
                        const ssd_conv_shape* sh, bool step, ssd::ConvArgs* a) {
    if (!sh) return fail(SSD_ERR_NULL, "shape is NULL");
    if (!out) return fail(SSD_ERR_NULL, "out is NULL");
    if (sh->dtype != SSD_F32 && sh->dtype != SSD_BF16)
        return fail(SSD_ERR_DTYPE, "dtype %d is neither SSD_F32 (0) nor SSD_BF16 (1)", sh->dtype);
    if (sh->ydtype != SSD_F32 && sh->ydtype != SSD_BF16)
        return fail(SSD_ERR_DTYPE, "ydtype %d is neither SSD_F32 (0) nor SSD_BF16 (1)", sh->ydtype);
    if (sh->reserved != 0) return fail(SSD_ERR_SHAPE, "reserved must be 0");
    if (sh->activation != 0 && sh->activation != 1)
        return fail(SSD_ERR_VALUE, "activation %d is neither 0 (none) nor 1 (SiLU)", sh->activation);
    if (sh->channels < 8 || sh->channels > kMaxConvChannels || sh->channels % 8 != 0)
        return fail(SSD_ERR_SHAPE, "channels %d must be a multiple of 8 in [8, 2^20]", sh->channels);
    if (sh->width < 2 || sh->width > 4) return fail(SSD_ERR_SHAPE, "width %d must be in [2, 4]", sh->width);
    if (sh->batch < 0 || sh->batch > (1 << 24)) return fail(SSD_ERR_SHAPE, "batch must be in [0, 2^24]");
    const bool packed = !step && sh->cu_seqlens != nullptr;
    if (!step && sh->seqlen < 0) return fail(SSD_ERR_SHAPE, "seqlen must be >= 0");
    const int64_t rows = step ? sh->batch : packed ? sh->seqlen : sh->batch * sh->seqlen;
    if (rows > ((int64_t)1 << 31) || rows * (int64_t)sh->channels > ((int64_t)1 << 40))
        return fail(SSD_ERR_SHAPE, "tensor too large");
    if (!step) {
        if (!packed && sh->cu_seqlens_host)
            return fail(SSD_ERR_SHAPE, "cu_seqlens_host given without the device cu_seqlens");
        if (packed && sh->cu_seqlens_host) {
            const ssd_status st = check_cu_host(sh->cu_seqlens_host, sh->batch, rows);
            if (st != SSD_OK) return st;
        }
    }
    if (out->nparts < 1 || out->nparts > 3) return fail(SSD_ERR_SHAPE, "nparts %d must be 1, 2 or 3", out->nparts);
    int64_t sum = 0;
    for (int p = 0; p < 3; ++p) {
        if (p >= out->nparts) {
            if (out->channels[p] != 0 || out->out[p] != nullptr)
                return fail(SSD_ERR_SHAPE, "unused output part %d must be 0 / NULL", p);
            continue;
        }
        if (out->channels[p] < 8 || out->channels[p] % 8 != 0)
            return fail(SSD_ERR_SHAPE, "output part %d has %d channels (a positive multiple of 8 is needed)", p,
                        out->channels[p]);
        sum += out->channels[p];
        if (!out->out[p] && rows > 0) return fail(SSD_ERR_NULL, "output part %d is NULL", p);
        if (!aligned16(out->out[p])) return fail(SSD_ERR_ALIGN, "output part %d is not 16-byte aligned", p);
    }
    if (sum != sh->channels)
        return fail(SSD_ERR_SHAPE, "output parts hold %lld channels, not %d", (long long)sum, sh->channels);
    if (!weight) return fail(SSD_ERR_NULL, "weight is NULL");
    if (!x && rows > 0) return fail(SSD_ERR_NULL, "x is NULL");
    struct {
        const void* p;
        const char* name;
    } in[] = {{x, "x"}, {weight, "weight"}, {bias, "bias"}};
    for (auto& q : in)
        if (q.p && !aligned16(q.p)) return fail(SSD_ERR_ALIGN, "%s is not 16-byte aligned", q.name);
    for (int p = 0; p < out->nparts; ++p)
        for (auto& q : in)
            if (q.p && out->out[p] == q.p) return fail(SSD_ERR_SHAPE, "output part %d aliases %s", p, q.name);
    a->x = x;
    a->weight = weight;
    a->bias = bias;
    a->state_in = nullptr;
    a->state_out = nullptr;
    a->cu = packed ? sh->cu_seqlens : nullptr;
    for (int p = 0; p < 3; ++p) {
        a->out[p] = out->out[p];
        a->part_ch[p] = out->channels[p];
    }
    a->nparts = out->nparts;
    a->nseq = sh->batch;
    a->L = step ? 1 : (packed ? 0 : sh->seqlen);
    a->T = rows;
    a->C = sh->channels;
    a->K = sh->width;
    a->dtype = sh->dtype;
    a->y_f32 = sh->ydtype == SSD_F32 ? 1 : 0;
    a->silu = sh->activation;
    return SSD_OK;
}

bool aliases_output(const ssd_conv_outputs* out, const void* p) {
    for (int q = 0; q < out->nparts; ++q)
        if (p && out->out[q] == p) return true;
    return false;
}

}  // namespace

SSD_API ssd_status ssd_causal_conv1d(const void* x, const float* weight, const float* bias,
                                     const void* conv_state_in, void* conv_state_out,
                                     const ssd_conv_outputs* out, const ssd_conv_shape* shape, void* stream) {
    ssd::ConvArgs a;
    ssd_status st = conv_prepare(x, weight, bias, out, shape, false, &a);
    if (st != SSD_OK) return st;
    if (shape->cu_seqlens && shape->batch == 0 && a.T > 0)
        return fail(SSD_ERR_SHAPE, "packed rows without sequences");
    if (conv_state_in && !aligned16(conv_state_in)) return fail(SSD_ERR_ALIGN, "conv_state_in is not 16-byte aligned");
    if (conv_state_out && !aligned16(conv_state_out))
        return fail(SSD_ERR_ALIGN, "conv_state_out is not 16-byte aligned");
    if (aliases_output(out, conv_state_in) || aliases_output(out, conv_state_out))
        return fail(SSD_ERR_SHAPE, "an output part aliases a conv state");
    if (conv_state_out && (conv_state_out == x || conv_state_out == (const void*)weight ||
                           conv_state_out == (const void*)bias))
        return fail(SSD_ERR_SHAPE, "conv_state_out aliases an input");
    a.state_in = conv_state_in;
    a.state_out = conv_state_out;
    const hipError_t err = ssd::launch_conv1d(a, (hipStream_t)stream);
    if (err != hipSuccess) return fail(SSD_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return ok();
}

SSD_API ssd_status ssd_causal_conv1d_step(void* conv_state, const void* x, const float* weight, const float* bias,
                                          const ssd_conv_outputs* out, const ssd_conv_shape* shape,
                                          void* stream) {
    ssd::ConvArgs a;
    ssd_status st = conv_prepare(x, weight, bias, out, shape, true, &a);
    if (st != SSD_OK) return st;
    if (!conv_state && a.nseq > 0) return fail(SSD_ERR_NULL, "conv_state is NULL");
    if (!aligned16(conv_state)) return fail(SSD_ERR_ALIGN, "conv_state is not 16-byte aligned");
    if (aliases_output(out, conv_state) || (conv_state && (conv_state == x || conv_state == (const void*)weight ||
                                                          conv_state == (const void*)bias)))
        return fail(SSD_ERR_SHAPE, "conv_state aliases another argument");
    a.state_out = conv_state;
    const hipError_t err = ssd::launch_conv1d_step(a, (hipStream_t)stream);
    if (err != hipSuccess) return fail(SSD_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return ok();
}
