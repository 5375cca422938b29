// Host check of the decode's segmentation arithmetic (csrc/segments.hpp, the functions the
// kernels call) over random batches: every unit of a launch lies in exactly one segment
// below W, every run's merge range [w0, w1] is exactly the segments the run touches, every
// run split over segments is named to the merge by exactly one segment boundary, no two
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
#include <random>
#include <vector>

#include "segments.hpp"

using namespace pagedkv::seg;

namespace {

constexpr int kLanes = 64;      // lanes of the wave that searches for its segment's start
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
  // each wave's search for its first unit: lane ranges of ceil(n / 64) of the n texts in
  // question, a scan of the range sums, the range holding the start; repeated inside that
  // range while it holds more than one text
  std::vector<int64_t> cum(c.S + 1, 0);  // units of the texts before each
  for (int s = 0; s < c.S; ++s) cum[s + 1] = cum[s] + (int64_t)R * U[s];
  {
    const int64_t run = cum[c.S];
    if (run != total) {
      snprintf(why, n, "range sums %lld != total %lld", (long long)run, (long long)total);
      return false;
    }
  }
  std::vector<int> named((size_t)c.S * R, 0);  // run -> boundaries naming it
  for (int64_t w = 0; w < W; ++w) {
    const int64_t c0 = w * seg;
    if (c0 >= total) continue;
    int lo = 0, cnt = c.S, text = -1, rounds = 0;
    int64_t base = 0, off = -1;
    for (;;) {
      ++rounds;
      const int per = (cnt + kLanes - 1) / kLanes;
      int hits = 0, hlo = -1, hhi = -1;
      int64_t hbase = 0, first = base;
      for (int t = 0; t < kLanes; ++t) {
        const int a = lo + (t * per < cnt ? t * per : cnt);
        const int b = lo + (t * per + per < cnt ? t * per + per : cnt);
        const int64_t m = cum[b] - cum[a];
        if (c0 >= first && c0 < first + m) {
          ++hits;
          hlo = a;
          hhi = b;
          hbase = first;
        }
        first += m;
      }
      if (hits != 1 || rounds > 8) {
        snprintf(why, n, "segment %lld: start unit %lld in %d ranges at round %d", (long long)w,
                 (long long)c0, hits, rounds);
        return false;
      }
      if (per == 1 || hhi - hlo <= 1) {
        text = hlo;
        off = c0 - hbase;
        break;
      }
      lo = hlo;
      cnt = hhi - hlo;
      base = hbase;
    }
    if (text < 0 || text >= c.S || excl[text] + off != c0 || off >= (int64_t)R * U[text]) {
      snprintf(why, n, "segment %lld: start unit %lld found in text %d at offset %lld",
               (long long)w, (long long)c0, text, (long long)off);
      return false;
    }
    // the run this segment boundary names to the merge (the partition wave's record)
    const int64_t r = off / U[text], u = off - r * U[text];
    if (names_split_run(u, seg)) ++named[(int64_t)text * R + r];
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
      const int64_t run_id = (int64_t)s * R + r;
      // a merge wave per boundary visits exactly the runs with partials, each once
      if (named[run_id] != (w0 == w1 ? 0 : 1)) {
        snprintf(why, n, "run [%lld, %lld) over segments %lld..%lld named by %d boundaries",
                 (long long)lo, (long long)hi, (long long)w0, (long long)w1, named[run_id]);
        return false;
      }
      if (w0 == w1) continue;  // finished inside one segment: no partials
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
    const int shape = pick(0, 4);
    c.S = shape == 0 ? pick(1, 8) : shape == 1 ? pick(1, 300) : shape == 2 ? pick(250, 3000)
          : shape == 3 ? pick(1, 40) : pick(4000, 20000);  // shape 4: three search rounds
    const int gs_opts[4] = {1, 2, 4, 8};
    c.GS = gs_opts[pick(0, 3)];
    const int G = c.GS * pick(1, 2);
    c.Hkv = pick(1, 6);
    c.H = c.Hkv * G;
    c.D = pick(0, 1) ? 64 : 128;
    const int bs[4] = {4, 8, 16, 32};
    c.B = bs[pick(0, 3)];
    const int longest = shape == 3 ? pick(1, 40000) : shape == 4 ? pick(0, 300) : pick(0, 2100);
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
