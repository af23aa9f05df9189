// Private declarations shared by the host ABI (ssd_api.cpp) and the kernel
// launchers (ssd_prefill.hip, ssd_decode.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace ssd {

// Everything a prefill kernel needs to map its grid index to tokens.  Built
// on the host; for a packed batch the tables are filled on the device by the
// plan kernel from the device copy of cu_seqlens.
//
// A *chunk* is <= Q consecutive tokens of one sequence (chunks restart at
// every sequence start).  Chunk-indexed launches cover nchunk_ub chunks; in a
// packed batch the entries past the real chunk count are marked empty.
struct Plan {
    int32_t H, P, N, G, hpg, Q;
    int32_t nseq;
    int32_t dense;     // 1: uniform batch, descriptors are arithmetic
    int64_t L;         // dense: tokens per sequence
    int64_t T;         // total token rows
    int32_t nchunk_ub; // grid bound of chunk-indexed launches (exact when dense)
    int32_t cpseq;     // dense: chunks per sequence
    const int32_t* cu; // packed: device cu_seqlens [nseq+1]
    int32_t* seq_tab;  // packed: per sequence {chunk0, nchunks, first row, tokens}
    int32_t* chunk_tab;// packed: per chunk {seq, row0, len, index in sequence}
    int32_t* seq_order;// packed scan walk: sequences by chunk count, longest first
                       // (filled by the plan kernel; NULL: in index order)
};

// The plan kernel orders the sequences by chunk count when there are at most
// this many (one workgroup ranks them); more keep their index order.
constexpr int32_t kOrderMaxSeq = 256;

// Byte offsets of the workspace regions (all 256-byte aligned).
struct Layout {
    size_t seq_tab, chunk_tab;  // int32 x4 entries
    size_t seq_order;           // int32 [nseq] (packed batches)
    size_t cs;      // f32 [nchunk_ub][H][Q]   inclusive sums of dt A within each chunk
    size_t dtc;     // f32 [nchunk_ub][H][Q]   dt per chunk and head, 0 past the chunk end
    size_t wst;     // f32 [nchunk_ub][H][Q]   exp(cs_last - cs) dt, each token's weight in the chunk state
                    //                         (not used by the scan walk: empty there)
    size_t cb;      // elem [nchunk_ub][G][Q][Q] C_t . B_k within each chunk
    size_t bt;      // elem [nchunk_ub][G][NT * Q] B transposed per chunk in MFMA fragment order, 0 past the end and N
    size_t states;  // f32 [nchunk_ub][H][P][N] chunk states, then the states entering each chunk
                    //                         (not used by the scan walk: empty there)
    size_t tail;    // f32 [nchunk_ub][H][2]   scan walk only: cs_last of each chunk and the decay
                    //                         from its end to its sequence's end
    size_t total;
};

// dt activation applied where dt enters the kernels (on = 0: dt used as given):
// dt = min(max(softplus(raw + bias[h]), lo), hi).
struct DtAct {
    const float* bias;  // [H] or NULL
    float lo, hi;
    int32_t on;
};

struct ScanArgs {
    const void* x;
    const float* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* init;
    void* y;
    float* final_state;
    char* ws;
    int32_t dtype;     // 0 f32, 1 bf16 (x, B, C)
    int32_t y_f32;     // 1: y is fp32, 0: y is bf16
    int32_t hpw;       // heads per workgroup of chunk_scan (within one group)
    int32_t hpw_state; // heads per workgroup of the chunk-parallel chunk_state
    int32_t path;      // kPathChunkParallel, kPathStateWalk or kPathScanWalk
    int32_t walk_nus;  // scan walk: units (head, column tile) per workgroup
    int32_t walk_nslice; // scan walk: workgroups per (sequence, group)
    DtAct act;
};

// How the prefill computes the chunk states, the passing between chunks and
// the outputs:
//   kPathChunkParallel  chunk_state, state_passing, chunk_scan: three launches,
//                       each parallel over chunks (the per-chunk states round
//                       trip through the workspace)
//   kPathStateWalk      one walk per (sequence, head, column tile) for the
//                       states and their passing, then chunk_scan
//   kPathScanWalk       one walk per (sequence, group, slice of units) that
//                       also writes y: no per-chunk state leaves the chip
//                       (bf16 inputs, 256-token chunks, dstate in (64, 128])
constexpr int32_t kPathChunkParallel = 1;
constexpr int32_t kPathStateWalk = 2;
constexpr int32_t kPathScanWalk = 3;

// Arguments of the scan walk launch.
struct WalkArgs {
    const void* x;
    const float* cs;
    const float* dtc;
    float* tail;  // [nchunk_ub][H][2], written by launch_walk_tails
    const void* C;
    const void* cb;
    const void* bt;
    const float* D;
    const float* init;
    float* final_state;
    void* y;
    int32_t per_xcd, run, npt, nslice, nus;  // per_xcd, run: walk_grid
    int32_t y_f32;
};

// Grid of a walk over `items` (pair, slice) items: runs of `run` consecutive
// items share an XCD, the runs dealt to the 8 XCDs in turn; per_xcd
// workgroups per XCD (some past the last item, which return at once).  Up to
// 256 items this is one contiguous range per XCD.
inline void walk_grid(int64_t items, int32_t* run, int32_t* per_xcd) {
    int64_t r = (items + 7) / 8;
    r = r < 1 ? 1 : (r > 32 ? 32 : r);
    const int64_t nruns = (items + r - 1) / r;
    *run = (int32_t)r;
    *per_xcd = (int32_t)(r * ((nruns + 7) / 8));
}

// Whether the scan walk kernel covers this dtype, dstate and chunk.
bool scan_walk_supported(int dtype, int N, int Q);

// LDS bytes per workgroup of the scan walk.
size_t scan_walk_lds_bytes();

// Queue the scan walk (after the cumsum and C.B^T kernels): first the
// per-(chunk, head) table a.tail from a.cs, then the walk.
hipError_t launch_scan_walk(const Plan& plan, const WalkArgs& a, hipStream_t stream);

struct DecodeArgs {
    float* state;
    const void* x;
    const float* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    void* y;
    int64_t batch;
    int32_t H, P, N, G;
    int32_t dtype;
    int32_t y_f32;
    DtAct act;
};

struct WindowArgs {
    float* state;      // S0, [batch, H, P, N]; rewritten on a flush step
    const void* x;     // [batch, W, H, P]
    const float* dt;   // [batch, W, H]
    const float* A;
    const void* B;     // [batch, W, G, N]
    const void* C;     // [batch, W, G, N]
    const float* D;
    void* y;           // [batch, H, P]
    int64_t batch;
    int32_t H, P, N, G;
    int32_t W, t, flush;
    int32_t dtype;
    int32_t y_f32;
    DtAct act;
};

struct ConvArgs {
    const void* x;           // [rows, C]
    const float* weight;     // [C, K]
    const float* bias;       // [C] or NULL
    const void* state_in;    // [nseq, K-1, C] or NULL
    void* state_out;         // [nseq, K-1, C] or NULL (the step: the state, in place)
    const int32_t* cu;       // device [nseq+1] or NULL (dense)
    void* out[3];            // output parts [rows, part_ch[p]]
    int32_t part_ch[3];
    int32_t nparts;
    int64_t nseq, L, T;      // sequences, dense length, total rows
    int32_t C, K;
    int32_t dtype, y_f32, silu;
};

// Sets the sentence ssd_last_error_detail() returns on this thread (for
// entry points outside ssd_api.cpp); returns st.
int32_t set_error_detail(int32_t st, const char* fmt, ...);

// dstate padded to the 32-row tiles the kernels use.
inline int padded_dstate(int N) { return N <= 32 ? 32 : N <= 64 ? 64 : N <= 128 ? 128 : 256; }

// LDS bytes per workgroup of the largest prefill kernel for this shape.
size_t prefill_lds_bytes(int dtype, int N, int Q);

// Queue the prefill kernels.  Returns hipSuccess or the launch error.
// When `marks` is non-NULL, an event is recorded before the first stage and
// after each of the seven stages (plan, cumsum, cb, chunk_state,
// state_passing, chunk_scan, scan_walk), eight events in all.  Stages a path
// does not run are empty: the state walk runs inside chunk_state, and the
// scan walk alone replaces chunk_state, state_passing and chunk_scan.
constexpr int kPrefillStages = 7;
hipError_t launch_prefill(const Plan& plan, const Layout& lay, const ScanArgs& a,
                          hipStream_t stream, hipEvent_t* marks = nullptr);

// Queue the decode kernel.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Queue the windowed decode kernel (window <= 16).
hipError_t launch_decode_window(const WindowArgs& a, hipStream_t stream);

// Queue the conv1d prefill (and the final-state pass when a.state_out is set).
hipError_t launch_conv1d(const ConvArgs& a, hipStream_t stream);

// Queue the conv1d decode step (state in a.state_out, updated in place).
hipError_t launch_conv1d_step(const ConvArgs& a, hipStream_t stream);

}  // namespace ssd
