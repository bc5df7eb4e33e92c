// ssd_plan.h -- host-side work decomposition of the fused scan, shared by the
// C ABI and its tests. Plain C++: no HIP calls.
//
// One workgroup walks the chunks of one (batch row, head, sequence segment,
// 64-wide slice of D, 64-row slice of N) in order, keeping its 64 x 64 block of
// the state on chip. With more than one N slice, each writes a partial y (the
// output sums over n) and a pass adds the slices up. When there
// are too few (batch, head) sequences to fill the GPU, each sequence is cut
// into P segments that the scan runs side by side, segment 0 from the initial
// state and the others from zero; each records its end state, its total
// log-decay and the log-decay at each of its chunk starts. A prefix pass then
// composes the states entering every segment (and the final state), and a
// fix-up pass adds each later segment's missing term, the entering state seen
// through the decay, Re(exp(Lambda_t) C_t H_in), to its outputs.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ssd {

constexpr int kThreads = 512;     // eight wave64s per workgroup
constexpr int kNPad = 64;         // state rows handled per workgroup (N padded)
constexpr int kDBlock = 64;       // state columns (D) per workgroup
constexpr int kTargetGroups = 256;  // one workgroup per compute unit of an MI355X
constexpr int kMaxBlock = 256;
// Input layouts of the forward scan.
constexpr int kLayoutC64 = 0;       // x, B_t, C_t complex64; dt float32
constexpr int kLayoutProj = 1;      // in_proj rows, float32
constexpr int kLayoutProjBf16 = 2;  // in_proj rows, bfloat16

// Kernel arguments. Complex arrays are interleaved (re, im) float pairs.
struct ScanParams {
    const float *x;           // (B, T, H, D) complex
    const float *A;           // (H) complex
    const float *Bt;          // (B, T, H, N) complex
    const float *Ct;          // (B, T, H, N) complex
    const float *dt;          // (B, T, H)
    const float *init_state;  // (B, H, N, D) complex or null
    float *y;                 // (B, T, H, D)
    float *final_state;       // (B, H, N, D) complex or null
    float *seg_state;         // (B, H, P, N, D) complex: segment end states (from the segment's
                              // own start); after the prefix pass slot p-1 holds the state
                              // entering segment p
    float *seg_logdecay;      // (B, H, P) complex, sum of softplus(dt)*A over a segment
    float *chunk_log;         // (B, H, nc) complex, that sum from the segment start to each
                              // chunk start
    float *y_part;            // (nnb, B, T, H, D): per-slice partial y when N > 64
    int B, T, H, N, D, Q;
    int nc;    // chunks per sequence
    int P;     // segments per sequence
    int spc;   // chunks per segment
    int ndb;   // 64-wide D slices
    int nnb;   // 64-row N slices
    int groups_per_seq;  // workgroups per sequence and D slice: the P segments
    int fix_groups;      // fix-up workgroups per (sequence, later segment, D slice)
    int64_t tok_stride;  // in_proj layout: floats between consecutive tokens' rows
};

struct Plan {
    int R = 0;     // padded chunk rows held by the kernel (16, 32 or 64)
    int nc = 0;
    int P = 1;
    int spc = 0;
    int ndb = 0;
    int nnb = 0;
    int fix_groups = 0;
    size_t seg_state_bytes = 0;
    size_t seg_decay_bytes = 0;
    size_t chunk_log_bytes = 0;
    size_t y_part_bytes = 0;
    size_t workspace_bytes = 0;
};

constexpr int kFixThreads = 256;        // four wave64s, one 16-column tile of D each
constexpr int kFixTargetGroups = 1024;  // fix-up workgroups to aim for (four per CU)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Tokens the kernel treats as one chunk: chunk_size itself up to 64; a longer
// chunk is evaluated as consecutive 64-token sub-chunks with the state passed
// between them, which is the same sum re-associated (the result does not depend
// on the chunk size beyond rounding) and keeps every block on chip.
constexpr int kMaxRows = 64;
inline int64_t block_rows(int64_t chunk_size) { return chunk_size < kMaxRows ? chunk_size : kMaxRows; }

// Sizes are assumed validated (positive, within the supported envelope).
inline Plan make_plan(int64_t B, int64_t T, int64_t H, int64_t N, int64_t D, int64_t chunk_size)
{
    Plan p;
    const int64_t Q = block_rows(chunk_size);
    p.R = Q <= 16 ? 16 : (Q <= 32 ? 32 : 64);
    p.nc = (int)((T + Q - 1) / Q);
    p.ndb = (int)((D + kDBlock - 1) / kDBlock);
    p.nnb = (int)((N + kNPad - 1) / kNPad);
    if (p.nc <= 0) {
        p.P = 1;
        p.spc = 0;
        return p;
    }
    int64_t seqs = B * H * p.ndb * p.nnb;
    int64_t want = (kTargetGroups + seqs - 1) / seqs;
    if (want < 1)
        want = 1;
    if (want > p.nc)
        want = p.nc;
    p.spc = (int)((p.nc + want - 1) / want);
    p.P = (p.nc + p.spc - 1) / p.spc;
    if (p.P > 1) {
        p.seg_state_bytes = align_up((size_t)B * H * p.P * N * D * 8, 256);
        p.seg_decay_bytes = align_up((size_t)B * H * p.P * 8, 256);
        p.chunk_log_bytes = align_up((size_t)B * H * p.nc * 8, 256);
        const int64_t units = B * H * (p.P - 1) * p.ndb;  // fix-up work units
        int64_t g = (kFixTargetGroups + units - 1) / units;
        p.fix_groups = (int)(g < p.spc ? g : p.spc);
    }
    if (p.nnb > 1)
        p.y_part_bytes = align_up((size_t)p.nnb * B * T * H * D * 4, 256);
    p.workspace_bytes = p.seg_state_bytes + p.seg_decay_bytes + p.chunk_log_bytes + p.y_part_bytes;
    return p;
}

}  // namespace ssd
