// kda_layout.hpp -- the prefill workspace layout, shared by the prefill kernels and the
// backward (which runs the prefill and then reads its chunk table).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace kda {

constexpr int kChunk = 64;

__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
__host__ __device__ constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------
// Workspace layout (all offsets 256-byte aligned):
//   chunk_off  int32 [num_seqs + 1]     first chunk of each sequence; [num_seqs] = count
//   seg_off    int32 [num_seqs + 1]     first segment of each sequence; [num_seqs] = count
//   table      int4  [max_chunks]       {sequence, first token, length, 0}
//   segtab     int4  [max_segs]         {sequence, first chunk, chunks, 2 k + last}
//   records    [max_chunks * H]         one per (chunk, head), granule order:
//     W, QG  [token block 4][dk granule GK][lane 64] x 16 B     rows t, k over dk
//     Kt     [dk block DK/16][token granule GT][lane 64] x 16 B rows c, k over tokens
//     Ut     [dv tile NT][token block 4][lane 64] x UB          accumulator layout
//     P      [token block 4][token granule GT][lane 64] x 16 B  rows t, k over tokens
//     exp(G_L) [DK] fp32
//   segment blocks [max_segs * H], fp32 row-major:
//     S_loc [DK][DV]   state after the segment from a zero state
//     Phi   [DK][DK]   the segment's transition (S_end = Phi S_start + S_loc)
//     S_start [DK][DV] state entering the segment
// A segment is up to seg_chunks consecutive chunks of one sequence: 16, doubled
// (up to 128) while the batch would give more than 256 (segment, head) pairs, i.e.
// about one segment workgroup per compute unit.  Small batches still spread over
// every CU; long ones get fewer, longer segments: a shorter sequential scan, and
// more of the work in each sequence's last segment, which the local pass skips.
// ---------------------------------------------------------------------------
__host__ __device__ inline int seg_chunks_for(int64_t total_tokens, int H) {
    int seg = 16;
    while (seg < 128 && total_tokens / kChunk / seg * H > 256) seg *= 2;
    return seg;
}

struct WsLayout {
    int64_t max_chunks, max_segs;
    int seg_chunks;
    size_t off_segoff, off_table, off_segtab, off_rec, rec_bytes, off_seg, seg_bytes, total;
    size_t o_w, o_q, o_kt, o_u, o_p, o_gl;
    size_t s_loc, s_phi, s_start;
    __host__ __device__ WsLayout(int num_seqs, int64_t total_tokens, int H, int dk, int dv, int e) {
        max_chunks = total_tokens / kChunk + num_seqs;
        seg_chunks = seg_chunks_for(total_tokens, H);
        max_segs = max_chunks / seg_chunks + num_seqs;
        off_segoff = align_up(sizeof(int32_t) * (num_seqs + 1), 256);
        off_table = off_segoff + align_up(sizeof(int32_t) * (num_seqs + 1), 256);
        off_segtab = off_table + align_up(sizeof(int32_t) * 4 * max_chunks, 256);
        off_rec = off_segtab + align_up(sizeof(int32_t) * 4 * max_segs, 256);
        o_w = 0;
        o_q = o_w + static_cast<size_t>(kChunk) * dk * e;
        o_kt = o_q + static_cast<size_t>(kChunk) * dk * e;
        o_u = o_kt + static_cast<size_t>(dk) * kChunk * e;
        o_p = o_u + static_cast<size_t>(kChunk) * dv * e;
        o_gl = o_p + static_cast<size_t>(kChunk) * kChunk * e;
        rec_bytes = align_up(o_gl + sizeof(float) * dk, 256);
        off_seg = off_rec + rec_bytes * static_cast<size_t>(max_chunks) * H;
        s_loc = 0;
        s_phi = s_loc + sizeof(float) * dk * dv;
        s_start = s_phi + sizeof(float) * dk * dk;
        seg_bytes = align_up(s_start + sizeof(float) * dk * dv, 256);
        total = off_seg + seg_bytes * static_cast<size_t>(max_segs) * H;
    }
};

}  // namespace kda
