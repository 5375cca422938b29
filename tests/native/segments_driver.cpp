// Host check of the decode's segmentation arithmetic (csrc/segments.hpp, the functions the
// kernels call) over random batches: every unit of a launch lies in exactly one segment
// below W, every run's merge range [w0, w1] is exactly the segments the run touches, no two
// runs write the same partial record, and every record lies inside the workspace.
//
//   segments_driver <seed> <cases> [old]
//
// "old" replaces the segment length by the fixed partition length whenever one is given
// (what the kernels did before a device-side length beyond the host's bound lengthened
// the segments), so that the test can show the check catches that mistake.
// Prints "ok <cases>" or the first failing case, and exits non-zero on a failure.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <random>
#include <vector>

#include "segments.hpp"

using namespace pagedkv::seg;

namespace {

constexpr int kThreads = 256;   // threads per workgroup of the partition kernel
constexpr int kWavesPerGroup = 4;
constexpr int kMaxGS = 8;

struct Case {
  int S, H, Hkv, GS, D, B, maxb, max_ctx, T, slots;
  std::vector<int> lens;
};

bool check(const Case& c, bool old, char* why, size_t n) {
  const int Gq = c.H / c.Hkv, R = c.Hkv * (Gq / c.GS);
  const int64_t capacity = (int64_t)c.maxb * c.B;
  // host: the grid from the bound on the lengths
  const int64_t units_bound = (int64_t)c.S * c.H * units_of(c.max_ctx);
  const int64_t W = grid_segments(units_bound, c.slots, c.T / kChunk);
  // device: the lengths as the kernels clamp them
  std::vector<int64_t> U(c.S), excl(c.S);
  int64_t total = 0;
  for (int s = 0; s < c.S; ++s) {
    int64_t L = c.lens[s] < 0 ? 0 : c.lens[s];
    if (L > capacity) L = capacity;
    U[s] = units_of((int)L);
    excl[s] = total;
    total += (int64_t)R * U[s];
  }
  const int64_t seg_fixed = c.T / kChunk;
  const int64_t seg = old ? (seg_fixed > 0 ? seg_fixed : (total + W - 1) / W)
                          : segment_units(total, W, seg_fixed);
  // every unit in exactly one segment below W (segments are disjoint by construction)
  int64_t covered = 0;
  for (int64_t w = 0; w < W; ++w) {
    const int64_t lo = w * seg, hi = lo + seg < total ? lo + seg : total;
    if (hi > lo) covered += hi - lo;
  }
  if (covered != total) {
    snprintf(why, n, "segments cover %lld of %lld units (W %lld, seg %lld)", (long long)covered,
             (long long)total, (long long)W, (long long)seg);
    return false;
  }
  // the workgroups' search for their waves' first units: thread ranges of ceil(S / 256)
  // texts, an exclusive scan of the range sums, a walk of the range holding each start
  const int per = (c.S + kThreads - 1) / kThreads;
  std::vector<int64_t> range_first(kThreads), range_units(kThreads);
  int64_t run = 0;
  for (int t = 0; t < kThreads; ++t) {
    const int lo = t * per < c.S ? t * per : c.S, hi = lo + per < c.S ? lo + per : c.S;
    range_first[t] = run;
    int64_t m = 0;
    for (int i = lo; i < hi; ++i) m += (int64_t)R * U[i];
    range_units[t] = m;
    run += m;
  }
  if (run != total) {
    snprintf(why, n, "range sums %lld != total %lld", (long long)run, (long long)total);
    return false;
  }
  for (int64_t w = 0; w < W; ++w) {
    const int64_t c0 = w * seg;
    if (c0 >= total) continue;
    int hits = 0, text = -1;
    int64_t off = -1;
    // the ranges holding c0: the last range starting at or before it, and any empty ranges
    // sharing that start (which hold nothing)
    const int last = (int)(std::upper_bound(range_first.begin(), range_first.end(), c0) -
                           range_first.begin()) - 1;
    for (int t = last; t >= 0 && range_first[t] == range_first[last]; --t) {
      if (!(c0 >= range_first[t] && c0 < range_first[t] + range_units[t])) continue;
      ++hits;
      int64_t e = range_first[t];
      const int lo = t * per, hi = lo + per < c.S ? lo + per : c.S;
      for (int i = lo; i < hi; ++i) {
        if (c0 < e + (int64_t)R * U[i]) {
          text = i;
          off = c0 - e;
          break;
        }
        e += (int64_t)R * U[i];
      }
    }
    if (hits != 1 || text < 0 || excl[text] + off != c0 || off >= (int64_t)R * U[text]) {
      snprintf(why, n, "segment %lld: start unit %lld found %d times (text %d, offset %lld)",
               (long long)w, (long long)c0, hits, text, (long long)off);
      return false;
    }
  }
  // runs: merge ranges, partial records
  const int64_t records = W * 2 * kMaxGS;  // partial records the workspace holds
  std::vector<int64_t> writer(records, -1);  // record -> run writing it
  for (int s = 0; s < c.S; ++s) {
    for (int r = 0; r < R; ++r) {
      const int64_t lo = excl[s] + (int64_t)r * U[s], hi = lo + U[s];
      int64_t w0, w1;
      run_segments(lo, hi, seg, W, &w0, &w1);
      const int64_t want0 = lo / seg, want1 = (hi - 1) / seg;
      if (w0 != want0 || w1 != want1 || w1 >= W) {
        snprintf(why, n, "run [%lld, %lld): merge range %lld..%lld, touches %lld..%lld, W %lld",
                 (long long)lo, (long long)hi, (long long)w0, (long long)w1,
                 (long long)want0, (long long)want1, (long long)W);
        return false;
      }
      if (w0 == w1) continue;  // finished inside one segment: no partials
      const int64_t run_id = (int64_t)s * R + r;
      for (int64_t w = w0; w <= w1; ++w) {
        // the partition kernel's slot (flush) and the merge's slot (read) of this record
        const int slot = partial_slot(lo, w * seg);
        for (int j = 0; j < c.GS; ++j) {
          const int64_t off = partial_offset(w, slot, j, c.GS, c.D + 4);
          if (off < 0 || off + c.D + 4 > records * (int64_t)(c.D + 4)) {
            snprintf(why, n, "record at %lld floats outside the workspace (%lld records)",
                     (long long)off, (long long)records);
            return false;
          }
          int64_t& who = writer[off / (c.D + 4)];
          if (who >= 0 && who != run_id) {
            snprintf(why, n, "segment %lld slot %d written by runs %lld and %lld", (long long)w,
                     slot, (long long)who, (long long)run_id);
            return false;
          }
          who = run_id;
        }
      }
    }
  }
  return true;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 3) {
    fprintf(stderr, "usage: %s seed cases [old]\n", argv[0]);
    return 2;
  }
  const unsigned seed = (unsigned)strtoul(argv[1], nullptr, 10);
  const int cases = atoi(argv[2]);
  const bool old = argc > 3 && strcmp(argv[3], "old") == 0;
  std::mt19937_64 rng(seed);
  auto pick = [&](int lo, int hi) { return (int)(lo + rng() % (uint64_t)(hi - lo + 1)); };
  char why[512];
  for (int k = 0; k < cases; ++k) {
    Case c;
    const int shape = pick(0, 3);
    c.S = shape == 0 ? pick(1, 8) : shape == 1 ? pick(1, 300) : shape == 2 ? pick(250, 3000)
                                                                          : pick(1, 40);
    const int gs_opts[4] = {1, 2, 4, 8};
    c.GS = gs_opts[pick(0, 3)];
    const int G = c.GS * pick(1, 2);
    c.Hkv = pick(1, 6);
    c.H = c.Hkv * G;
    c.D = pick(0, 1) ? 64 : 128;
    const int bs[4] = {4, 8, 16, 32};
    c.B = bs[pick(0, 3)];
    const int longest = shape == 3 ? pick(1, 40000) : pick(0, 2100);
    c.maxb = (longest + c.B - 1) / c.B + pick(0, 3);
    if (c.maxb < 1) c.maxb = 1;
    c.lens.resize(c.S);
    for (int s = 0; s < c.S; ++s) c.lens[s] = pick(0, 9) == 0 ? 0 : pick(0, longest);
    int mx = 0;
    for (int L : c.lens) mx = L > mx ? L : mx;
    // the host's bound: usually right, sometimes below the longest length on the device
    const int under = pick(0, 2) == 0;
    c.max_ctx = under ? pick(0, mx) : mx + pick(0, 64);
    c.T = pick(0, 2) == 0 ? 0 : kChunk * pick(1, 64);
    c.slots = kWavesPerGroup * (pick(0, 3) == 0 ? pick(1, 16) : 256);
    if (!check(c, old, why, sizeof why)) {
      printf("FAIL case %d: S %d H %d Hkv %d GS %d B %d max_ctx %d (longest %d) T %d: %s\n", k,
             c.S, c.H, c.Hkv, c.GS, c.B, c.max_ctx, mx, c.T, why);
      return 1;
    }
  }
  printf("ok %d\n", cases);
  return 0;
}
