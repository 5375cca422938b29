// Index arithmetic of the equal-work segmentation of paged decode attention, used both by
// the host (grid size, workspace) and by the kernels (segment length, merge ranges), so that
// a host program can check it over random lengths without a GPU.
//
// Work units are 16-token chunks of (text, head group) runs («The KV Cache and
// PagedAttention» › "The Block Table": a text's tokens, in logical order, spread over
// blocks), numbered text-major, then run, then chunk. The units of a launch are cut into W
// contiguous segments of `seg` units, one per wavefront; a run whose units span several
// segments leaves one partial result per segment, and the merge combines them.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pagedkv {
namespace seg {

constexpr int kChunk = 16;  // tokens per work unit

// Units of a run over L attended tokens (an empty run still takes one unit, which
// produces its zero output).
__host__ __device__ inline int units_of(int L) { return L <= 0 ? 1 : (L + kChunk - 1) / kChunk; }

// Segments of a launch. units_bound: units at the host's bound on the context lengths.
// seg_units 0: `slots` segments (waves resident at once), fewer if there are fewer units;
// else enough segments of seg_units units for units_bound.
__host__ inline int64_t grid_segments(int64_t units_bound, int64_t slots, int64_t seg_units) {
  if (units_bound < 1) units_bound = 1;
  if (seg_units <= 0) return slots < units_bound ? slots : units_bound;
  return (units_bound + seg_units - 1) / seg_units;
}

// Segment length for `total` units over W segments: seg_fixed units when W of them cover
// every unit, else the smallest length that does. A context longer than the host's bound
// therefore lengthens the segments instead of leaving units past W * seg to no wave.
// At least 1.
__host__ __device__ inline int64_t segment_units(int64_t total, int64_t W, int64_t seg_fixed) {
  const int64_t fit = W > 0 ? (total + W - 1) / W : total;
  const int64_t s = seg_fixed > fit ? seg_fixed : fit;
  return s > 0 ? s : 1;
}

// Segments holding units [lo, hi) of a run (hi > lo): w0 .. w1, w1 clamped to W - 1.
__host__ __device__ inline void run_segments(int64_t lo, int64_t hi, int64_t seg, int64_t W,
                                             int64_t* w0, int64_t* w1) {
  int64_t a = lo / seg, b = (hi - 1) / seg;
  if (b > W - 1) b = W - 1;
  if (a > b) a = b;
  *w0 = a;
  *w1 = b;
}

// Which of a segment's two partial slots a run not finished inside it uses: 0 when the run
// starts at or before the segment's first unit (the segment's first run), else 1 (its last
// run, which starts inside the segment and goes on past it).
__host__ __device__ inline int partial_slot(int64_t run_lo, int64_t seg_lo) {
  return run_lo <= seg_lo ? 0 : 1;
}

// Whether a segment whose first unit lies `u` units into a run names that run to the merge:
// the run started in the segment before (0 < u <= seg), so a run split over several
// segments is named once, by the first segment boundary it crosses, and a run that starts
// at a segment's first unit is not split there.
__host__ __device__ inline bool names_split_run(int64_t u, int64_t seg) { return u > 0 && u <= seg; }

// Offset, in floats, of the partial of query head j (of a wave's gs heads) in slot `slot`
// of segment w; a record is stride floats (m, l, two pads, acc[head_dim]).
__host__ __device__ inline int64_t partial_offset(int64_t w, int slot, int j, int gs, int stride) {
  return ((w * 2 + slot) * gs + j) * (int64_t)stride;
}

}  // namespace seg
}  // namespace pagedkv
