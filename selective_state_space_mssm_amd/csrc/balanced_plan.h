// balanced_plan.h -- the cut of the balanced persistent schedule of the
// forward scan (and the backward pre-pass, the same kernel), as plain integer
// arithmetic shared by the kernel and the host (a CPU unit test compiles this
// header alone and walks every worker's segments).
//
// The work is the sequence of (channel block, 16-step tile) units in block
// order, nblk blocks of T tiles each.  Worker w of `workers` takes the units
// [U w / workers, U (w + 1) / workers), U = nblk T: equal contiguous ranges.
// The recurrence is sequential in time within a block, so a block split
// between two workers hands its state over: the earlier part publishes its
// end state, the later part waits for it.  A worker runs its segments in this
// order:
//   1. its range's last piece, if the range ends inside a block: it starts at
//      the block's first tile, so it depends on nobody; it publishes;
//   2. the blocks wholly inside its range;
//   3. its range's first piece, if the range starts inside a block: it waits
//      for the state the previous worker publishes in step 1.
// A worker only waits on the worker before it, which publishes before it
// waits on anyone, so every wait ends once the earlier workers have started
// (workgroups are dispatched in increasing order).  All of this needs every
// range to reach past the end of the block it starts in -- true when
// nblk >= workers, since a range then holds at least T units; the host only
// uses the schedule then (balanced_plan_ok).
#pragma once

#include <stdint.h>

namespace mssm {

// Where a segment's initial state comes from and what becomes of its final one.
enum BalancedFrom { kFromH0 = 0, kFromChunkCarry = 1, kFromPublished = 2 };
enum BalancedTo { kKeep = 0, kFinal = 1, kPublish = 2 };

struct BalancedRange {
    int b0, b1;           // blocks of the range's first and last unit
    int64_t t0, t1;       // first tile in b0; end tile (exclusive, 1..T) in b1
    int tail_piece;       // 1: the range ends inside b1 (segment 0 runs it and publishes)
    int full_first;       // first block wholly inside the range
    int nseg;             // segments of this worker
};

struct BalancedSegment {
    int blk;
    int64_t tile_begin, tile_end;  // tiles [tile_begin, tile_end) of block blk
    int from, to;                  // BalancedFrom, BalancedTo
};

__host__ __device__ inline bool balanced_plan_ok(int64_t nblk, int64_t workers) {
    return workers > 0 && nblk >= workers;
}

__host__ __device__ inline BalancedRange balanced_range(int64_t nblk, int64_t T, int64_t workers, int64_t w) {
    BalancedRange r;
    const int64_t U = nblk * T;
    const int64_t u0 = U * w / workers;
    const int64_t u1 = U * (w + 1) / workers;
    r.b0 = static_cast<int>(u0 / T);
    r.t0 = u0 - static_cast<int64_t>(r.b0) * T;
    r.b1 = static_cast<int>((u1 - 1) / T);
    r.t1 = u1 - static_cast<int64_t>(r.b1) * T;
    r.tail_piece = (r.b1 > r.b0 && r.t1 < T) ? 1 : 0;
    r.full_first = r.t0 == 0 ? r.b0 : r.b0 + 1;
    const int full_last = r.t1 == T ? r.b1 : r.b1 - 1;
    r.nseg = r.tail_piece + (full_last - r.full_first + 1) + (r.t0 > 0 ? 1 : 0);
    return r;
}

// Segment `sg` (0 <= sg < r.nseg) of a worker's range.
__host__ __device__ inline BalancedSegment balanced_segment(const BalancedRange& r, int64_t T, int sg) {
    BalancedSegment s;
    if (sg < r.tail_piece) {                          // last piece, ends inside block b1
        s.blk = r.b1; s.tile_begin = 0; s.tile_end = r.t1; s.from = kFromH0; s.to = kPublish;
    } else if (sg < r.nseg - (r.t0 > 0 ? 1 : 0)) {    // a whole block
        s.blk = r.full_first + (sg - r.tail_piece); s.tile_begin = 0; s.tile_end = T; s.from = kFromH0; s.to = kFinal;
    } else {                                          // first piece, starts inside block b0
        s.blk = r.b0; s.tile_begin = r.t0; s.tile_end = T; s.from = kFromPublished; s.to = kFinal;
    }
    return s;
}

}  // namespace mssm
