// Paged decode attention for gfx950.
//
// What is computed: «KV cache» › "How it works" — the new position's query is
// compared with every cached key of its text (its own included) and the softmax
// weights mix the values. «The KV Cache and PagedAttention» › "The Block Table" —
// the kernel follows each text's block table to its blocks, wherever they sit.
//
// How (design for MI355X; decode is bound by HBM bandwidth, so no MFMA):
//  * Work unit = one 16-token chunk of one (text, head). All units of the batch
//    are numbered text-major, head, chunk, and cut into equal contiguous
//    segments, one per wavefront ("split-context" with equal work per wave, so
//    any mix of lengths fills the 256 CUs evenly).
//  * Inside a wave, a K or V row of head_dim elements is read by LPR lanes with
//    16-byte loads; the wave covers RPW = 64 / LPR rows per load instruction, so
//    a block's rows stream as fully coalesced 1 KiB wave loads. The lanes of a
//    row form a group; the dot product is summed over the group with DPP.
//  * Each group keeps its own online softmax (running max m, sum l, weighted
//    values acc) in the exp2 domain; groups and waves are merged at the end of
//    a run. The loads of the next chunk are in flight while the current chunk
//    is computed (two register buffers).
//  * Block ids are wave-uniform per load instruction and come through the
//    scalar cache; the token index is clamped to the text's last token so no
//    unfilled place is read.
//  * A run (the chunks of one (text, head)) covered entirely by one wave is
//    finished in place; otherwise each wave covering part of it leaves a partial
//    (m, l, acc) and decode_merge combines a run's partials in segment order.
//    Merging inside this kernel by the last segment to arrive was measured
//    slower on the 7 x 2,048 OPT-13B step: with agent-scope release/acquire
//    fences (an L2 writeback and invalidate per partial) the launch doubled;
//    with device-coherent stores, a completion wait and a counter it still cost
//    more than this kernel plus the merge kernel. The kernel boundary gives the
//    merge its visibility for free. The order of every sum depends only on
//    logical positions, never on where blocks are placed.
#include "device.hpp"

#include <cmath>

namespace pagedkv {
namespace {

constexpr int kChunk = 16;                 // tokens per work unit
constexpr int kWavesPerGroup = 4;          // wavefronts per workgroup
constexpr int kThreads = 64 * kWavesPerGroup;
constexpr int kWavesPerCU = 4;             // auto grid: segments per CU (measured best of 4, 6, 8, 12, 16)
constexpr int kHdrBytes = 256;             // workspace header: total units, segment length

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Keys and values are read once per launch: non-temporal loads keep them from
// displacing the block tables, queries and partials in the caches (measured on
// the 7 x 2,048 OPT-13B step: 55 -> 48 us for the partition kernel).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const char* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__host__ __device__ __forceinline__ int units_of(int L) {
  return L <= 0 ? 1 : (L + kChunk - 1) / kChunk;
}

template <int DT, int D>
struct Geo {
  static constexpr int ELT = DT == PA_F32 ? 4 : 2;
  static constexpr int EPL = 16 / ELT;      // elements per lane per load
  static constexpr int LPR = D / EPL;       // lanes per row
  static constexpr int RPW = 64 / LPR;      // rows per wave load
  static constexpr int NLD = kChunk / RPW;  // load instructions per chunk and tensor
  static constexpr int PSTRIDE = D + 4;     // floats per partial: m, l, pad, pad, acc[D]
};

// Wave-uniform position in the unit numbering.
struct Cursor {
  int s, h, u;      // text, head, chunk within the run
  int U, L;         // chunks in the run, attended tokens (clamped to the table's capacity)
  int over;         // context_lens[s] exceeded the table's capacity
  int64_t excl;     // number of the first unit of text s
};

struct Ctx {
  int S, H, Hkv, group, maxb, num_blocks;
  int64_t capacity;  // max_blocks_per_seq * block_size
  const int32_t* __restrict__ ctx;
};

__device__ __forceinline__ void set_text(Cursor& c, const Ctx& x, int s) {
  c.s = s;
  int L = s < x.S ? x.ctx[s] : 0;
  if (L < 0) L = 0;
  c.over = L > x.capacity;
  if (c.over) L = (int)x.capacity;
  c.L = L;
  c.U = units_of(L);
}

__device__ __forceinline__ void advance(Cursor& c, const Ctx& x) {
  if (++c.u == c.U) {
    c.u = 0;
    if (++c.h == x.H) {
      c.h = 0;
      c.excl += (int64_t)x.H * c.U;
      set_text(c, x, c.s + 1);
    }
  }
}

template <int DT, int D>
struct Buf {
  uint4 k[Geo<DT, D>::NLD];
  uint4 v[Geo<DT, D>::NLD];
  uint4 q;
  bool bad;  // a table entry outside the pool, or a context longer than the table
};

template <int DT, int D>
struct State {
  float m, l;
  float acc[Geo<DT, D>::EPL];
  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int e = 0; e < Geo<DT, D>::EPL; ++e) acc[e] = 0.f;
  }
};

template <int DT, int D, int B>
__device__ __forceinline__ void load_chunk(Buf<DT, D>& b, const Cursor& c, const Ctx& x,
                                           const char* __restrict__ kc,
                                           const char* __restrict__ vc,
                                           const char* __restrict__ q,
                                           const int32_t* __restrict__ tables, int lane) {
  using G = Geo<DT, D>;
  constexpr int kRowBytes = D * G::ELT;
  constexpr int64_t kTileBytes = (int64_t)B * kRowBytes;  // one (block, kv head) tile
  const int g = lane / G::LPR, lp = lane % G::LPR;
  const int kvh = c.h / x.group;
  const int last = c.L > 0 ? c.L - 1 : 0;
  const int32_t* trow = tables + (int64_t)c.s * x.maxb;
  const int t_first = c.u * kChunk;
  b.bad = c.over;
  if constexpr (B >= kChunk) {
    // the whole chunk lies in one block: one scalar table lookup, a scalar tile base
    // and 32-bit lane offsets
    int blk = trow[t_first / B];
    const bool bad = (unsigned)blk >= (unsigned)x.num_blocks;
    b.bad |= bad;
    if (bad) blk = 0;  // read block 0 instead; the result is poisoned
    const int64_t tile = ((int64_t)blk * x.Hkv + kvh) * kTileBytes;
    const char* kb = kc + tile;
    const char* vb = vc + tile;
#pragma unroll
    for (int i = 0; i < G::NLD; ++i) {
      const int t = t_first + i * G::RPW + g;
      const int tc = t < last ? t : last;
      const uint32_t off = (uint32_t)(tc % B) * kRowBytes + lp * 16;
      b.k[i] = load_stream(kb + off);
      b.v[i] = load_stream(vb + off);
    }
  } else {
#pragma unroll
    for (int i = 0; i < G::NLD; ++i) {
      const int t = t_first + i * G::RPW + g;
      const int tc = t < last ? t : last;
      int blk;
      if constexpr (B >= G::RPW) {
        // the rows of one load instruction lie in one block: a scalar lookup
        const int t0 = min(t_first + i * G::RPW, last);
        blk = trow[t0 / B];
      } else {
        blk = trow[tc / B];
      }
      const bool bad = (unsigned)blk >= (unsigned)x.num_blocks;
      b.bad |= bad;
      if (bad) blk = 0;
      const int64_t off = ((int64_t)blk * x.Hkv + kvh) * kTileBytes +
                          (uint32_t)(tc % B) * kRowBytes + lp * 16;
      b.k[i] = load_stream(kc + off);
      b.v[i] = load_stream(vc + off);
    }
  }
  b.q = *reinterpret_cast<const uint4*>(q + ((int64_t)c.s * x.H + c.h) * kRowBytes + lp * 16);
}

template <int DT, int D>
__device__ __forceinline__ void compute_chunk(const Buf<DT, D>& b, const Cursor& c,
                                              State<DT, D>& st, float scale_log2, int lane) {
  using G = Geo<DT, D>;
  if (c.L == 0) return;  // nothing attended: the run's result is zeros
  const int g = lane / G::LPR;
  float qf[G::EPL];
  widen16<DT>(b.q, qf);
  float sc[G::NLD];
  float mc = -INFINITY;
#pragma unroll
  for (int i = 0; i < G::NLD; ++i) {
    float kf[G::EPL];
    widen16<DT>(b.k[i], kf);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < G::EPL; ++e) d = fmaf(qf[e], kf[e], d);
    d = group_sum<G::LPR>(d) * scale_log2;
    const int t = c.u * kChunk + i * G::RPW + g;
    if (t >= c.L) d = -INFINITY;
    sc[i] = d;
    mc = fmaxf(mc, d);
  }
  const float mn = fmaxf(st.m, mc);
  const float mu = mn == -INFINITY ? 0.f : mn;
  const float alpha = fast_exp2(st.m - mu);
  st.l *= alpha;
#pragma unroll
  for (int e = 0; e < G::EPL; ++e) st.acc[e] *= alpha;
#pragma unroll
  for (int i = 0; i < G::NLD; ++i) {
    const float p = fast_exp2(sc[i] - mu);
    st.l += p;
    float vf[G::EPL];
    widen16<DT>(b.v[i], vf);
#pragma unroll
    for (int e = 0; e < G::EPL; ++e) st.acc[e] = fmaf(p, vf[e], st.acc[e]);
  }
  st.m = mn;
  if (b.bad) {
#pragma unroll
    for (int e = 0; e < G::EPL; ++e) st.acc[e] = __builtin_nanf("");
  }
}

// Merge the row groups of a wave (fixed butterfly order); every lane ends with the result.
template <int DT, int D>
__device__ __forceinline__ void merge_groups(State<DT, D>& st) {
  using G = Geo<DT, D>;
#pragma unroll
  for (int off = G::LPR; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(st.m, off);
    const float l2 = __shfl_xor(st.l, off);
    const float mn = fmaxf(st.m, m2);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float a = fast_exp2(st.m - mu), b = fast_exp2(m2 - mu);
    st.l = st.l * a + l2 * b;
#pragma unroll
    for (int e = 0; e < G::EPL; ++e) {
      const float x2 = __shfl_xor(st.acc[e], off);
      st.acc[e] = st.acc[e] * a + x2 * b;
    }
    st.m = mn;
  }
}

// Output row of (s, h) from fp32 values, PER consecutive elements per lane.
template <int DT, int PER>
__device__ __forceinline__ void store_out(char* __restrict__ dst, const float* o) {
  if constexpr (DT == PA_F32) {
#pragma unroll
    for (int e = 0; e < PER; ++e) reinterpret_cast<float*>(dst)[e] = o[e];
  } else if constexpr (DT == PA_F16) {
#pragma unroll
    for (int e = 0; e < PER; ++e) reinterpret_cast<_Float16*>(dst)[e] = (_Float16)o[e];
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)bf16_bits_rne(o[e]);
  }
}

// Combine the partials of one run, left by segments w0..w1, in segment order.
// Segment w0 holds the run in its slot 1 unless the run starts exactly at w0's
// first unit (then it is w0's first run, slot 0); every later segment starts
// inside the run, so the run is its first run (slot 0).
// Combine the partials of one run, left by segments w0..w1, in segment order.
// Segment w0 holds the run in its slot 1 unless the run starts exactly at w0's
// first unit (then it is w0's first run, slot 0); every later segment starts
// inside the run, so the run is its first run (slot 0). The partials are read
// UNROLL at a time with all loads in flight, and combined with a running maximum
// (the same rescaling as the online softmax), so one pass over memory suffices.
template <int DT, int D>
__device__ __forceinline__ void merge_run(const float* __restrict__ partials, int64_t w0,
                                          int64_t w1, int64_t run_lo, int64_t seg,
                                          char* __restrict__ dst_row, int lane) {
  using G = Geo<DT, D>;
  constexpr int PER = D / 64;   // output elements per lane
  constexpr int UNROLL = 8;
  auto slot_of = [&](int64_t w) -> int64_t {
    return w * 2 + ((w == w0 && run_lo != w0 * seg) ? 1 : 0);
  };
  float M = -INFINITY, den = 0.f, num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
  for (int64_t w = w0; w <= w1; w += UNROLL) {
    float m[UNROLL], l[UNROLL], a[UNROLL][PER];
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      // past w1: an empty partial (weight 0) instead of a load
      m[j] = -INFINITY;
      l[j] = 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) a[j][e] = 0.f;
      if (w + j <= w1) {
        const float* p = partials + slot_of(w + j) * G::PSTRIDE;
        m[j] = p[0];
        l[j] = p[1];
#pragma unroll
        for (int e = 0; e < PER; ++e) a[j][e] = p[4 + lane * PER + e];
      }
    }
    float mg = M;
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) mg = fmaxf(mg, m[j]);
    const float mu = mg == -INFINITY ? 0.f : mg;
    const float r = fast_exp2(M - mu);
    den *= r;
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] *= r;
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {  // segment order
      const float f = fast_exp2(m[j] - mu);
      den += f * l[j];
#pragma unroll
      for (int e = 0; e < PER; ++e) num[e] += f * a[j][e];
    }
    M = mg;
  }
  float o[PER];
  const float inv = den > 0.f ? 1.f / den : 0.f;
  // 0 * num: NaN stays visible for a poisoned run
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = den > 0.f ? num[e] * inv : 0.f * num[e];
  store_out<DT, PER>(dst_row + lane * PER * G::ELT, o);
}

template <int DT, int D>
__device__ __forceinline__ void flush_run(State<DT, D>& st, const Cursor& c, int64_t seg_lo,
                                          int64_t seg_hi, int w, char* __restrict__ out,
                                          float* __restrict__ partials, int H, int lane) {
  using G = Geo<DT, D>;
  merge_groups<DT, D>(st);
  const int64_t run_lo = c.excl + (int64_t)c.h * c.U;
  const int64_t run_hi = run_lo + c.U;
  if (lane < G::LPR) {
    if (run_lo >= seg_lo && run_hi <= seg_hi) {
      // the whole run is in this segment: finish it here
      float o[G::EPL];
      const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
      // 0 * acc: zeros when nothing was attended, NaN for a poisoned run
#pragma unroll
      for (int e = 0; e < G::EPL; ++e) o[e] = st.l > 0.f ? st.acc[e] * inv : 0.f * st.acc[e];
      char* dst = out + (((int64_t)c.s * H + c.h) * D) * G::ELT + lane * 16;
      *reinterpret_cast<uint4*>(dst) = narrow16<DT>(o);
    } else {
      const int slot = run_lo <= seg_lo ? 0 : 1;
      float* p = partials + ((int64_t)w * 2 + slot) * G::PSTRIDE;
      if (lane == 0) {
        p[0] = st.m;
        p[1] = st.l;
      }
      float4* a4 = reinterpret_cast<float4*>(p + 4 + lane * G::EPL);
#pragma unroll
      for (int e = 0; e < G::EPL; e += 4)
        a4[e / 4] = make_float4(st.acc[e], st.acc[e + 1], st.acc[e + 2], st.acc[e + 3]);
    }
  }
  st.reset();
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Sum over the workgroup (every thread gets it).
__device__ __forceinline__ int64_t block_sum(int64_t x, int64_t* sh) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  const int wave = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[wave] = x;
  __syncthreads();
  int64_t t = 0;
#pragma unroll
  for (int j = 0; j < kWavesPerGroup; ++j) t += sh[j];
  return t;
}

template <int DT, int D, int B>
__global__ __launch_bounds__(kThreads) void decode_partition(
    char* __restrict__ out, const char* __restrict__ q, const char* __restrict__ kc,
    const char* __restrict__ vc, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ ctx, int S, int H, int Hkv, int maxb, int num_blocks, int W,
    int seg_fixed, float scale_log2, int64_t* __restrict__ hdr, int64_t* __restrict__ excl_out,
    float* __restrict__ partials) {
  __shared__ int64_t sh_red[kWavesPerGroup];
  __shared__ int sh_seq[kWavesPerGroup];
  __shared__ int64_t sh_off[kWavesPerGroup];
  __shared__ int64_t sh_excl[kWavesPerGroup];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t capacity = (int64_t)maxb * B;
  auto units_at = [&](int i) -> int64_t {
    int L = ctx[i];
    if (L < 0) L = 0;
    if (L > capacity) L = (int)capacity;
    return (int64_t)H * units_of(L);
  };

  // ---- locate each wave's segment: total units, then an exclusive scan ----
  int64_t local = 0;
  for (int i = tid; i < S; i += kThreads) local += units_at(i);
  const int64_t total = uniform64(block_sum(local, sh_red));
  const int64_t seg = seg_fixed > 0 ? seg_fixed : (total + W - 1) / W;
  if (blockIdx.x == 0 && tid == 0) {
    hdr[0] = total;
    hdr[1] = seg;
  }
  int64_t carry = 0;
  for (int base = 0; base < S; base += kThreads) {
    const int i = base + tid;
    const int64_t n = i < S ? units_at(i) : 0;
    int64_t incl = n;
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    __syncthreads();
    if (lane == 63) sh_red[wave] = incl;
    __syncthreads();
    int64_t before = 0, all = 0;
#pragma unroll
    for (int j = 0; j < kWavesPerGroup; ++j) {
      before += j < wave ? sh_red[j] : 0;
      all += sh_red[j];
    }
    const int64_t ex = carry + before + incl - n;
    if (i < S) {
      if (blockIdx.x == 0) excl_out[i] = ex;
#pragma unroll
      for (int j = 0; j < kWavesPerGroup; ++j) {
        const int64_t c0 = ((int64_t)blockIdx.x * kWavesPerGroup + j) * seg;
        if (c0 >= ex && c0 < ex + n) {
          sh_seq[j] = i;
          sh_off[j] = c0 - ex;
          sh_excl[j] = ex;
        }
      }
    }
    carry += all;
  }
  __syncthreads();

  const int w = blockIdx.x * kWavesPerGroup + wave;
  const int64_t seg_lo = (int64_t)w * seg;
  if (w >= W || seg_lo >= total) return;
  const int64_t seg_hi = seg_lo + seg < total ? seg_lo + seg : total;
  const int n = (int)(seg_hi - seg_lo);

  const Ctx x{S, H, Hkv, H / Hkv, maxb, num_blocks, capacity, ctx};
  Cursor cur;
  // values read from LDS are the same in every lane: keep them in scalar registers
  cur.excl = uniform64(sh_excl[wave]);
  set_text(cur, x, __builtin_amdgcn_readfirstlane(sh_seq[wave]));
  {
    const int64_t off = uniform64(sh_off[wave]);
    cur.h = (int)(off / cur.U);
    cur.u = (int)(off - (int64_t)cur.h * cur.U);
  }
  Cursor ld = cur;
  const float sl = scale_log2;

  State<DT, D> st;
  st.reset();
  Buf<DT, D> A, Bb;
  load_chunk<DT, D, B>(A, ld, x, kc, vc, q, tables, lane);
  advance(ld, x);

  auto finish = [&](int i) {
    // last chunk of the run, or of the segment
    if (cur.u == cur.U - 1 || i == n - 1)
      flush_run<DT, D>(st, cur, seg_lo, seg_hi, w, out, partials, H, lane);
    advance(cur, x);
  };

  int i = 0;
  while (i + 2 < n) {
    load_chunk<DT, D, B>(Bb, ld, x, kc, vc, q, tables, lane);
    advance(ld, x);
    compute_chunk<DT, D>(A, cur, st, sl, lane);
    finish(i);
    load_chunk<DT, D, B>(A, ld, x, kc, vc, q, tables, lane);
    advance(ld, x);
    compute_chunk<DT, D>(Bb, cur, st, sl, lane);
    finish(i + 1);
    i += 2;
  }
  if (i + 1 < n) {
    load_chunk<DT, D, B>(Bb, ld, x, kc, vc, q, tables, lane);
    compute_chunk<DT, D>(A, cur, st, sl, lane);
    finish(i);
    compute_chunk<DT, D>(Bb, cur, st, sl, lane);
    finish(i + 1);
  } else {
    compute_chunk<DT, D>(A, cur, st, sl, lane);
    finish(i);
  }
}

// Merge pass: one wave per (text, head); runs finished inside one segment return at once.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void decode_merge(
    char* __restrict__ out, const int32_t* __restrict__ ctx, int S, int H, int maxb, int bsz,
    const int64_t* __restrict__ hdr, const int64_t* __restrict__ excl,
    const float* __restrict__ partials) {
  using G = Geo<DT, D>;
  const int lane = threadIdx.x & 63;
  const int64_t pair =
      (int64_t)blockIdx.x * kWavesPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (pair >= (int64_t)S * H) return;
  const int s = (int)(pair / H), h = (int)(pair - (int64_t)s * H);
  int L = ctx[s];
  if (L < 0) L = 0;
  const int64_t capacity = (int64_t)maxb * bsz;
  if (L > capacity) L = (int)capacity;
  const int U = units_of(L);
  const int64_t seg = hdr[1];
  const int64_t lo = excl[s] + (int64_t)h * U, hi = lo + U;
  const int64_t w0 = lo / seg, w1 = (hi - 1) / seg;
  if (w0 == w1) return;
  merge_run<DT, D>(partials, w0, w1, lo, seg, out + pair * D * G::ELT, lane);
}

// ---- host side -------------------------------------------------------------

// Workspace: header (total units, segment length), int64 unit offset of each text [S],
// fp32 partials [W][2][D+4]. Written by decode_partition, read by decode_merge.
struct Layout {
  int64_t W;  // wavefronts (segments) in the grid
  size_t excl_off, part_off, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int layout(int32_t S, int32_t H, int32_t D, int32_t max_ctx, int32_t T, Layout* lay) {
  if (S < 1 || H < 1 || (D != 64 && D != 128) || max_ctx < 0 || T < 0 || T % kChunk != 0)
    return fail(PA_EINVAL, "bad workspace shape (num_seqs %d, num_heads %d, head_dim %d, "
                "max_context_len %d, partition_tokens %d)", S, H, D, max_ctx, T);
  const int64_t units_bound = (int64_t)S * H * units_of(max_ctx);
  int64_t W;
  if (T == 0) {
    int cus = 0;
    int rc = device_cus(&cus);
    if (rc != PA_OK) return rc;
    W = (int64_t)cus * kWavesPerCU;
    if (W > units_bound) W = units_bound;
  } else {
    const int64_t seg = T / kChunk;
    W = (units_bound + seg - 1) / seg;
  }
  if (W > 0x7fffffff / 2) return fail(PA_EINVAL, "too many segments");
  lay->W = W;
  lay->excl_off = kHdrBytes;
  lay->part_off = align256(lay->excl_off + sizeof(int64_t) * (size_t)S);
  lay->bytes = align256(lay->part_off + sizeof(float) * (size_t)W * 2 * (D + 4));
  return PA_OK;
}

template <int DT, int D, int B>
void launch(char* out, const char* q, const char* kc, const char* vc, const int32_t* tables,
            const int32_t* ctx, int S, int H, int Hkv, int maxb, int nb, int W, int seg_fixed,
            float sl, char* ws, const Layout& lay, hipStream_t st) {
  int64_t* hdr = reinterpret_cast<int64_t*>(ws);
  int64_t* excl = reinterpret_cast<int64_t*>(ws + lay.excl_off);
  float* part = reinterpret_cast<float*>(ws + lay.part_off);
  const int groups = (W + kWavesPerGroup - 1) / kWavesPerGroup;
  hipLaunchKernelGGL((decode_partition<DT, D, B>), dim3(groups), dim3(kThreads), 0, st, out, q,
                     kc, vc, tables, ctx, S, H, Hkv, maxb, nb, W, seg_fixed, sl, hdr, excl, part);
  const int64_t pairs = (int64_t)S * H;
  const int mgroups = (int)((pairs + kWavesPerGroup - 1) / kWavesPerGroup);
  hipLaunchKernelGGL((decode_merge<DT, D>), dim3(mgroups), dim3(kThreads), 0, st, out, ctx, S, H,
                     maxb, B, hdr, excl, part);
}

__global__ void zero_fill_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

template <int DT, int D>
bool dispatch_b(int B, char* out, const char* q, const char* kc, const char* vc,
                const int32_t* tables, const int32_t* ctx, int S, int H, int Hkv, int maxb,
                int nb, int W, int seg_fixed, float sl, char* ws, const Layout& lay,
                hipStream_t st) {
  switch (B) {
    case 4: launch<DT, D, 4>(out, q, kc, vc, tables, ctx, S, H, Hkv, maxb, nb, W, seg_fixed, sl, ws, lay, st); return true;
    case 8: launch<DT, D, 8>(out, q, kc, vc, tables, ctx, S, H, Hkv, maxb, nb, W, seg_fixed, sl, ws, lay, st); return true;
    case 16: launch<DT, D, 16>(out, q, kc, vc, tables, ctx, S, H, Hkv, maxb, nb, W, seg_fixed, sl, ws, lay, st); return true;
    case 32: launch<DT, D, 32>(out, q, kc, vc, tables, ctx, S, H, Hkv, maxb, nb, W, seg_fixed, sl, ws, lay, st); return true;
  }
  return false;
}

template <int DT>
bool dispatch_d(int D, int B, char* out, const char* q, const char* kc, const char* vc,
                const int32_t* tables, const int32_t* ctx, int S, int H, int Hkv, int maxb,
                int nb, int W, int seg_fixed, float sl, char* ws, const Layout& lay,
                hipStream_t st) {
  if (D == 64) return dispatch_b<DT, 64>(B, out, q, kc, vc, tables, ctx, S, H, Hkv, maxb, nb, W, seg_fixed, sl, ws, lay, st);
  if (D == 128) return dispatch_b<DT, 128>(B, out, q, kc, vc, tables, ctx, S, H, Hkv, maxb, nb, W, seg_fixed, sl, ws, lay, st);
  return false;
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" int pa_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return fail(PA_EINVAL, "null workspace");
  if (((uintptr_t)workspace & 3u) || (workspace_bytes & 3u))
    return fail(PA_EINVAL, "workspace must be 4-byte aligned and sized");
  const int64_t n = (int64_t)(workspace_bytes / 4);
  if (n == 0) return ok();
  const int64_t want = (n + 255) / 256;
  const int groups = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(zero_fill_kernel, dim3(groups), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t*)workspace, n);
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                            int32_t head_dim, int32_t max_context_len,
                                            int32_t partition_tokens) {
  Layout lay;
  if (layout(num_seqs, num_heads, head_dim, max_context_len, partition_tokens, &lay) != PA_OK)
    return 0;
  return lay.bytes;
}

extern "C" int pa_decode_attention(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_context_len,
                                   int32_t partition_tokens, float scale, int32_t dtype,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return fail(PA_EINVAL, "dtype %d is not PA_F32/PA_F16/PA_BF16", dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (block_size != 4 && block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PA_EUNSUPPORTED, "block_size %d (supported: 4, 8, 16, 32)", block_size);
  if (num_seqs < 1 || num_heads < 1 || num_kv_heads < 1 || num_blocks < 1 ||
      max_blocks_per_seq < 1)
    return fail(PA_EINVAL, "num_seqs, num_heads, num_kv_heads, num_blocks and "
                "max_blocks_per_seq must be >= 1");
  if (num_heads % num_kv_heads != 0)
    return fail(PA_EINVAL, "num_heads %d is not a multiple of num_kv_heads %d", num_heads,
                num_kv_heads);
  if (max_context_len < 0 || partition_tokens < 0 || partition_tokens % kChunk != 0)
    return fail(PA_EINVAL, "max_context_len must be >= 0 and partition_tokens a multiple of %d",
                kChunk);
  if (!std::isfinite(scale)) return fail(PA_EINVAL, "scale is not finite");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !workspace)
    return fail(PA_EINVAL, "null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(workspace))
    return fail(PA_EINVAL, "out, q, pools and workspace must be 16-byte aligned");
  if (((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u))
    return fail(PA_EINVAL, "tables and context_lens must be 4-byte aligned");
  Layout lay;
  int rc = layout(num_seqs, num_heads, head_dim, max_context_len, partition_tokens, &lay);
  if (rc != PA_OK) return rc;
  if (workspace_bytes < lay.bytes)
    return fail(PA_EINVAL, "workspace_bytes %zu < %zu required", workspace_bytes, lay.bytes);
  const int seg_fixed = partition_tokens / kChunk;
  const float sl = scale * 1.4426950408889634f;  // scale * log2(e): softmax in the exp2 domain
  bool done = false;
#define PA_ARGS head_dim, block_size, (char*)out, (const char*)q, (const char*)k_cache, \
      (const char*)v_cache, block_tables, context_lens, num_seqs, num_heads, num_kv_heads, \
      max_blocks_per_seq, num_blocks, (int)lay.W, seg_fixed, sl, (char*)workspace, lay, \
      (hipStream_t)stream
  if (dtype == PA_F32) done = dispatch_d<PA_F32>(PA_ARGS);
  else if (dtype == PA_F16) done = dispatch_d<PA_F16>(PA_ARGS);
  else done = dispatch_d<PA_BF16>(PA_ARGS);
#undef PA_ARGS
  if (!done) return fail(PA_EUNSUPPORTED, "no kernel for this shape");
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}
