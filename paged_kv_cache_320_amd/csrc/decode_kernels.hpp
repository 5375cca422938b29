// Paged decode attention for gfx950: kernels and their launch templates.
// decode_inst.hip instantiates them once per (key/value format, query format,
// head_dim), one compile unit each; the C entry points are in decode.hip.
//
// What is computed: «KV cache» › "How it works" — the new position's query is
// compared with every cached key of its text (its own included) and the softmax
// weights mix the values. «The KV Cache and PagedAttention» › "The Block Table" —
// the kernel follows each text's block table to its blocks, wherever they sit.
// › "What Came After": several query heads may share one set of keys and values.
//
// How (design for MI355X; decode is bound by HBM bandwidth, so no MFMA):
//  * A wave serves GS query heads that share one key/value head (GS = 1, 2, 4 or
//    8), so each key/value row is read from HBM once per GS heads. A "run" is
//    one text's chunks for one such head group.
//  * Work unit = one 16-token chunk of one run. All units of the batch are
//    numbered text-major, head group, chunk, and cut into equal contiguous
//    segments, one per wavefront ("split-context" with equal work per wave, so
//    any mix of lengths fills the 256 CUs evenly).
//  * Inside a wave, a K or V row of head_dim elements is read by LPR lanes with
//    16-byte loads; the wave covers RPW = 64 / LPR rows per load instruction, so
//    a block's rows stream as fully coalesced 1 KiB wave loads. The lanes of a
//    row form a group; each dot product is summed over the group with DPP.
//  * Each row group keeps its own online softmax (running max m, sum l, weighted
//    values acc) per query head in the exp2 domain; groups are merged at the end
//    of a run. The loads of the next chunk are in flight while the current chunk
//    is computed (two register buffers).
//  * E4M3 (8-bit) pools: keys and values are widened to fp32 in registers by
//    the hardware conversion; the key scale is folded into the score scale and
//    the value scale applied once to the output, so the hot loop is unchanged.
//  * Block ids are wave-uniform per load instruction and come through the
//    scalar cache; the token index is clamped to the text's last token so no
//    unfilled place is read.
//  * A run covered entirely by one wave is finished in place; otherwise each
//    wave covering part of it leaves a partial (m, l, acc) and decode_merge
//    combines a run's partials in segment order. Merging inside this kernel by
//    the last segment to arrive was measured slower on the 7 x 2,048 OPT-13B
//    step: with agent-scope release/acquire fences (an L2 writeback and
//    invalidate per partial) the launch doubled; with device-coherent stores, a
//    completion wait and a counter it still cost more than this kernel plus the
//    merge kernel. The kernel boundary gives the merge its visibility for free.
//    The order of every sum depends only on logical positions, never on where
//    blocks are placed.
//  * Fused new-token write (pa_decode_attention_write): the step's new key and value
//    rows are read straight from k_new / v_new for the last position (and written
//    into the cache by one run per key/value head, for later steps), so the separate
//    write kernel and its launch go away. No wave reads that place from the cache.
#pragma once

#include "device.hpp"
#include "segments.hpp"

#include <cmath>

namespace pagedkv {
namespace decode_impl {


using seg::kChunk;                 // tokens per work unit
using seg::units_of;
constexpr int kWavesPerGroup = 4;  // wavefronts per workgroup
constexpr int kThreads = 64 * kWavesPerGroup;
constexpr int kWavesPerCU = 4;     // auto grid: segments per CU (measured best of 4, 6, 8, 12, 16)
constexpr int kHdrBytes = 256;     // workspace header: total units, segment length
constexpr int kMaxGS = 8;          // query heads per wave, at most

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Keys and values are read once per launch: non-temporal loads keep them from
// displacing the block tables, queries and partials in the caches (measured on
// the 7 x 2,048 OPT-13B step: 55 -> 48 us for the partition kernel).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const char* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// KT: storage format of keys and values; QT: format of queries and outputs (the same
// except for E4M3 pools, whose queries and outputs are 16-bit).
template <int KT, int D>
struct Geo {
  static constexpr int ELT = elt_size<KT>();
  static constexpr int EPL = 16 / ELT;      // elements per lane per load
  static constexpr int LPR = D / EPL;       // lanes per row
  static constexpr int RPW = 64 / LPR;      // rows per wave load
  static constexpr int NLD = kChunk / RPW;  // load instructions per chunk and tensor
  static constexpr int PSTRIDE = D + 4;     // floats per partial: m, l, pad, pad, acc[D]
};

// Wave-uniform position in the unit numbering.
struct Cursor {
  int s, r, u;      // text, run (head group) within the text, chunk within the run
  int U, L;         // chunks in the run, attended tokens (clamped to the table's capacity)
  int toff;         // tokens skipped at the start of the text's table row (a block multiple)
  int over;         // context_lens[s] exceeded the table's capacity
  int64_t excl;     // number of the first unit of text s
  int vfirst, vcount;  // shared-prefix mode 1: text s is a group; its first member and count
  int fold;            // shared-prefix mode 2: fold_mask of text s
};

// Shared-prefix decode (pa_decode_attention_prefix) runs the kernels twice. Mode 1 runs over
// groups of texts whose tables begin with the same blocks: a group is one text of this
// batch, its queries those of its members, read from the real batch's q (query head c of
// key/value head k is member c / Gr's head k * Gr + c % Gr, Gr = heads / Hkv), and each
// member's (m, l, acc) over the shared blocks goes to its row of `state`
// [texts][heads][D + 4] instead of an output. Mode 2 runs over every text's own blocks,
// from start[s] on, and folds the text's state in before the output is formed. Mode 0:
// plain decode.
struct Prefix {
  const int32_t* __restrict__ start;   // mode 2: tokens skipped per text (block multiples)
  float* state;                        // modes 1, 2
  const int32_t* __restrict__ vfirst;  // mode 1: first member of each group
  const int32_t* __restrict__ vcount;  // mode 1: members of each group
  int heads;                           // mode 1: query heads per text of the real batch
  int mode;
  // mode 2 over two nested levels: the outer level's starts and states. A text folds in
  // the outer state where its outer start is past 0 and the `state` row (the inner level's,
  // or with one level the only one) where `start` is past the outer start (past 0 with one
  // level); rows that do not apply are never read, so neither array needs clearing.
  const int32_t* __restrict__ start0;
  const float* state0;
  // mode 1: texts of the real batch, its query heads per key/value head (Gr), members a
  // group holds at most, and for each column c < 8 of a key/value head its member
  // (colm >> 4c & 15) and head offset (colh >> 4c & 15)
  int seqs, gr, members, colm, colh;
};

// Mode 1: group s's first member and member count as the set-up wrote them, clamped into
// the real batch (every row the kernels touch through them stays inside it).
__device__ __forceinline__ void group_members(const Prefix& pf, int s, int& f, int& n) {
  int ff = pf.vfirst[s];
  ff = ff < 0 ? 0 : ff >= pf.seqs ? pf.seqs - 1 : ff;
  const int most = pf.members < pf.seqs - ff ? pf.members : pf.seqs - ff;
  const int nn = pf.vcount[s];
  n = nn < 0 ? 0 : nn > most ? most : nn;
  f = ff;
}

// Mode 1: the row of the real batch's q (text x heads + head) holding column col of key/value
// head kvh of a group whose members are vfirst .. vfirst + vcount - 1. A column past the
// members reads the first member's row: its results are never stored.
__device__ __forceinline__ int64_t group_q_row(const Prefix& pf, int vfirst, int vcount, int kvh,
                                               int col) {
  const int m = (pf.colm >> (4 * col)) & 15, ho = (pf.colh >> (4 * col)) & 15;
  return (int64_t)(vfirst + (m < vcount ? m : 0)) * pf.heads + kvh * pf.gr + ho;
}

// Mode 2: which state rows text s folds in (bit 0: the outer level's, bit 1: `state`'s).
__device__ __forceinline__ int fold_mask(const Prefix& pf, int s) {
  const int p1 = pf.start[s];
  const int p0 = pf.start0 ? pf.start0[s] : 0;
  return (p0 > 0 ? 1 : 0) | (p1 > p0 ? 2 : 0);
}

struct Ctx {
  int S, H, Hkv;
  int G;            // query heads per key/value head
  int NG;           // head groups per key/value head (G / GS)
  int R;            // runs per text (Hkv * NG)
  int maxb, num_blocks, bsz;
  int64_t capacity;  // max_blocks_per_seq * block_size
  const int32_t* __restrict__ ctx;
  Prefix pf;
};

// Tokens text s attends: its context length clamped into [0, capacity], less the tokens
// its start skips (rounded down to a block, at most all of them). toff: the tokens
// skipped, 0 when none is left to attend (so the row's first entry stays the one read).
__device__ __forceinline__ int attended_from(int L, const int32_t* __restrict__ start, int s,
                                             int64_t capacity, int bsz, int* toff, int* over) {
  if (L < 0) L = 0;
  *over = L > capacity;
  if (L > capacity) L = (int)capacity;
  int P = start ? start[s] : 0;
  P = P < 0 ? 0 : P > L ? L : P;
  P -= P % bsz;
  *toff = L - P > 0 ? P : 0;
  return L - P;
}

// The same for context length ctx[s].
__device__ __forceinline__ int attended_len(const int32_t* __restrict__ ctx,
                                            const int32_t* __restrict__ start, int s,
                                            int64_t capacity, int bsz, int* toff, int* over) {
  return attended_from(ctx[s], start, s, capacity, bsz, toff, over);
}

// Mode 1: the state row of query head hv of a group whose members are texts vfirst ..
// vfirst + vcount - 1, or null for a column past its members.
template <int D>
__device__ __forceinline__ float* prefix_state_row(const Prefix& pf, int Hkv, int G, int vfirst,
                                                   int vcount, int hv) {
  const int kvh = hv / G, c = hv - kvh * G;
  const int Gr = pf.heads / Hkv;
  const int m = c / Gr;
  if (m >= vcount) return nullptr;
  return pf.state + ((int64_t)(vfirst + m) * pf.heads + kvh * Gr + (c - m * Gr)) * (D + 4);
}

// The step's new rows, for the fused write: k_new / v_new [S][Hkv][D] in the pools'
// format, slots [S] (block * B + place), the pools to write.
struct NewRows {
  const char* __restrict__ k;
  const char* __restrict__ v;
  const int64_t* __restrict__ slots;
  char* kc;
  char* vc;
};

// (In shared-prefix mode 1 the group's members are read here, once per group, with its
// length: read where a run is finished they made the wave wait for every load in flight.)
// The cursor at text s, whose context length is raw (ctx[s], already read).
__device__ __forceinline__ void set_text_raw(Cursor& c, const Ctx& x, int s, int raw) {
  c.s = s;
  c.vfirst = c.vcount = 0;
  c.fold = 0;
  if (s < x.S) {
    c.L = attended_from(raw, x.pf.start, s, x.capacity, x.bsz, &c.toff, &c.over);
    if (x.pf.mode == 1) {
      int f, n;
      group_members(x.pf, s, f, n);
      c.vfirst = __builtin_amdgcn_readfirstlane(f);
      c.vcount = __builtin_amdgcn_readfirstlane(n);
    } else if (x.pf.mode == 2) {
      c.fold = __builtin_amdgcn_readfirstlane(fold_mask(x.pf, s));
    }
  } else {
    c.L = c.toff = c.over = 0;
  }
  c.U = units_of(c.L);
}

__device__ __forceinline__ void set_text(Cursor& c, const Ctx& x, int s) {
  set_text_raw(c, x, s, s < x.S ? x.ctx[s] : 0);
}

__device__ __forceinline__ void advance(Cursor& c, const Ctx& x) {
  if (++c.u == c.U) {
    c.u = 0;
    if (++c.r == x.R) {
      c.r = 0;
      c.excl += (int64_t)x.R * c.U;
      set_text(c, x, c.s + 1);
    }
  }
}

// Key/value head of run r, and the first of its GS query heads.
template <int GS>
__device__ __forceinline__ int kv_head_of(int r, const Ctx& x) {
  return GS == 1 ? r / x.G : r / x.NG;
}
template <int GS>
__device__ __forceinline__ int first_head_of(int r, const Ctx& x) {
  return GS == 1 ? r : (r / x.NG) * x.G + (r % x.NG) * GS;
}

// 16-byte pieces of QT per lane holding the lane's EPL query (or output) elements
template <int KT, int QT, int D>
constexpr int q_pieces() { return Geo<KT, D>::EPL * elt_size<QT>() / 16; }

template <int KT, int QT, int D, int GS>
struct Buf {
  uint4 k[Geo<KT, D>::NLD];
  uint4 v[Geo<KT, D>::NLD];
  uint4 q[GS][q_pieces<KT, QT, D>()];
  bool bad;  // a table entry outside the pool, or a context longer than the table
};

template <int KT, int D, int GS>
struct State {
  float m[GS], l[GS];
  float acc[GS][Geo<KT, D>::EPL];
  // shared-prefix mode 2: the text's states over its shared blocks (the outer level's,
  // then the inner or only level's), loaded with the run's last chunk so that folding
  // them in waits for no load issued later; empty where a level does not apply
  float fm[2][GS], fl[2][GS];
  float facc[2][GS][Geo<KT, D>::EPL];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int j = 0; j < GS; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.f;
#pragma unroll
      for (int e = 0; e < Geo<KT, D>::EPL; ++e) acc[j][e] = 0.f;
    }
  }
  __device__ __forceinline__ void reset_fold() {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int j = 0; j < GS; ++j) {
        fm[k][j] = -INFINITY;
        fl[k][j] = 0.f;
#pragma unroll
        for (int e = 0; e < Geo<KT, D>::EPL; ++e) facc[k][j][e] = 0.f;
      }
  }
};

template <int KT, int QT, int D, int B, int GS, bool FUSED>
__device__ __forceinline__ void load_chunk(Buf<KT, QT, D, GS>& b, const Cursor& c, const Ctx& x,
                                           const char* __restrict__ kc,
                                           const char* __restrict__ vc,
                                           const char* __restrict__ q,
                                           const int32_t* __restrict__ tables,
                                           const NewRows& nr, int lane) {
  using G = Geo<KT, D>;
  constexpr int kRowBytes = D * G::ELT;
  constexpr int64_t kTileBytes = (int64_t)B * kRowBytes;  // one (block, kv head) tile
  constexpr int QP = q_pieces<KT, QT, D>();
  constexpr int kQRowBytes = D * elt_size<QT>();
  const int g = lane / G::LPR, lp = lane % G::LPR;
  const int kvh = kv_head_of<GS>(c.r, x);
  const int last = c.L > 0 ? c.L - 1 : 0;
  const int32_t* trow = tables + (int64_t)c.s * x.maxb + c.toff / B;
  const int t_first = c.u * kChunk;
  // fused write: the last position's rows come from k_new / v_new
  const int64_t new_row = ((int64_t)c.s * x.Hkv + kvh) * kRowBytes + lp * 16;
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
      if constexpr (FUSED) {
        const bool fresh = tc == last;
        b.k[i] = load_stream(fresh ? nr.k + new_row : kb + off);
        b.v[i] = load_stream(fresh ? nr.v + new_row : vb + off);
      } else {
        b.k[i] = load_stream(kb + off);
        b.v[i] = load_stream(vb + off);
      }
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
      if constexpr (FUSED) {
        const bool fresh = tc == last;
        b.k[i] = load_stream(fresh ? nr.k + new_row : kc + off);
        b.v[i] = load_stream(fresh ? nr.v + new_row : vc + off);
      } else {
        b.k[i] = load_stream(kc + off);
        b.v[i] = load_stream(vc + off);
      }
    }
  }
  // the GS query rows (cache hits after the run's first chunk); in shared-prefix mode 1 each
  // column's row lies in its member's part of the real batch
  const int h0 = first_head_of<GS>(c.r, x);
  if (x.pf.mode == 1) {
#pragma unroll
    for (int j = 0; j < GS; ++j) {
      const char* qrow = q + group_q_row(x.pf, c.vfirst, c.vcount, kvh, h0 + j - kvh * x.G) *
                                 kQRowBytes + lp * QP * 16;
#pragma unroll
      for (int p = 0; p < QP; ++p)
        b.q[j][p] = *reinterpret_cast<const uint4*>(qrow + p * 16);
    }
  } else {
    const char* qrow = q + ((int64_t)c.s * x.H + h0) * kQRowBytes + lp * QP * 16;
#pragma unroll
    for (int j = 0; j < GS; ++j)
#pragma unroll
      for (int p = 0; p < QP; ++p)
        b.q[j][p] = *reinterpret_cast<const uint4*>(qrow + j * kQRowBytes + p * 16);
  }
}

// Fused write: when a writing run's last chunk is computed, the lanes holding the new
// position's rows (just loaded from k_new / v_new) store them into their place, if it is
// in the pool. The first run of each (text, key/value head) writes. The slot is read
// through the scalar cache (a restrict kernel argument): a vector load there would make
// the compiler wait for every load in flight, the next chunk's included.
template <int B, int GS>
__device__ __forceinline__ bool writes_new_row(const Cursor& c, const Ctx& x) {
  return c.L > 0 && c.u == c.U - 1 && (GS == 1 ? c.r % x.G : c.r % x.NG) == 0;
}
// One 16-byte piece of the new row of one pool (kv: nr.kc or nr.vc) at byte col.
template <int D, int ELT, int B, int GS>
__device__ __forceinline__ void store_new_piece_of(const NewRows& nr, char* __restrict__ kv,
                                                   const Cursor& c, const Ctx& x, int col,
                                                   const uint4& piece) {
  constexpr int kRowBytes = D * ELT;
  const int64_t slot = nr.slots[c.s];
  if (slot < 0 || slot >= (int64_t)x.num_blocks * B) return;
  const int kvh = kv_head_of<GS>(c.r, x);
  const int64_t row = ((slot / B) * x.Hkv + kvh) * B + slot % B;
  *reinterpret_cast<uint4*>(kv + row * kRowBytes + col) = piece;
}
template <int D, int ELT, int B, int GS>
__device__ __forceinline__ void store_new_piece(const NewRows& nr, const Cursor& c, const Ctx& x,
                                                int col, const uint4& k, const uint4& v) {
  constexpr int kRowBytes = D * ELT;
  const int64_t slot = nr.slots[c.s];
  if (slot < 0 || slot >= (int64_t)x.num_blocks * B) return;
  const int kvh = kv_head_of<GS>(c.r, x);
  const int64_t row = ((slot / B) * x.Hkv + kvh) * B + slot % B;
  *reinterpret_cast<uint4*>(nr.kc + row * kRowBytes + col) = k;
  *reinterpret_cast<uint4*>(nr.vc + row * kRowBytes + col) = v;
}

template <int KT, int QT, int D, int GS>
__device__ __forceinline__ void compute_chunk(const Buf<KT, QT, D, GS>& b, const Cursor& c,
                                              State<KT, D, GS>& st, float scale_log2, int lane) {
  using G = Geo<KT, D>;
  constexpr int QP = q_pieces<KT, QT, D>();
  if (c.L == 0) return;  // nothing attended: the run's result is zeros
  const int g = lane / G::LPR;
  float kf[G::NLD][G::EPL];
#pragma unroll
  for (int i = 0; i < G::NLD; ++i) widen16<KT>(b.k[i], kf[i]);
  float vf[G::NLD][G::EPL];
#pragma unroll
  for (int i = 0; i < G::NLD; ++i) widen16<KT>(b.v[i], vf[i]);
#pragma unroll
  for (int j = 0; j < GS; ++j) {
    float qf[G::EPL];
#pragma unroll
    for (int p = 0; p < QP; ++p) widen16<QT>(b.q[j][p], qf + p * (G::EPL / QP));
    float sc[G::NLD];
    float mc = -INFINITY;
#pragma unroll
    for (int i = 0; i < G::NLD; ++i) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < G::EPL; ++e) d = fmaf(qf[e], kf[i][e], d);
      d = group_sum<G::LPR>(d) * scale_log2;
      const int t = c.u * kChunk + i * G::RPW + g;
      if (t >= c.L) d = -INFINITY;
      sc[i] = d;
      mc = fmaxf(mc, d);
    }
    const float mn = fmaxf(st.m[j], mc);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(st.m[j] - mu);
    st.l[j] *= alpha;
#pragma unroll
    for (int e = 0; e < G::EPL; ++e) st.acc[j][e] *= alpha;
#pragma unroll
    for (int i = 0; i < G::NLD; ++i) {
      const float p = fast_exp2(sc[i] - mu);
      st.l[j] += p;
#pragma unroll
      for (int e = 0; e < G::EPL; ++e) st.acc[j][e] = fmaf(p, vf[i][e], st.acc[j][e]);
    }
    st.m[j] = mn;
    if (b.bad) {
#pragma unroll
      for (int e = 0; e < G::EPL; ++e) st.acc[j][e] = __builtin_nanf("");
    }
  }
}

// Merge the row groups of a wave (fixed butterfly order); every lane ends with the result.
template <int KT, int D, int GS>
__device__ __forceinline__ void merge_groups(State<KT, D, GS>& st) {
  using G = Geo<KT, D>;
#pragma unroll
  for (int j = 0; j < GS; ++j) {
#pragma unroll
    for (int off = G::LPR; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(st.m[j], off);
      const float l2 = __shfl_xor(st.l[j], off);
      const float mn = fmaxf(st.m[j], m2);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float a = fast_exp2(st.m[j] - mu), b = fast_exp2(m2 - mu);
      st.l[j] = st.l[j] * a + l2 * b;
#pragma unroll
      for (int e = 0; e < G::EPL; ++e) {
        const float x2 = __shfl_xor(st.acc[j][e], off);
        st.acc[j][e] = st.acc[j][e] * a + x2 * b;
      }
      st.m[j] = mn;
    }
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

// Partial record of query head j of segment w's slot (0: the segment's first run,
// 1: its last run).
template <int D, int GS>
__device__ __forceinline__ int64_t partial_index(int64_t w, int slot, int j) {
  return seg::partial_offset(w, slot, j, GS, D + 4);
}

template <int KT, int QT, int D, int GS>
__device__ __forceinline__ void flush_run(State<KT, D, GS>& st, const Cursor& c, const Ctx& x,
                                          int64_t seg_lo, int64_t seg_hi, int w,
                                          char* __restrict__ out, float* __restrict__ partials,
                                          float v_scale, int lane) {
  using G = Geo<KT, D>;
  constexpr int QP = q_pieces<KT, QT, D>();
  merge_groups<KT, D, GS>(st);
  const int64_t run_lo = c.excl + (int64_t)c.r * c.U;
  const int64_t run_hi = run_lo + c.U;
  const int h0 = first_head_of<GS>(c.r, x);
  if (lane < G::LPR) {
    if (run_lo >= seg_lo && run_hi <= seg_hi) {
      // the whole run is in this segment: finish it here
#pragma unroll
      for (int j = 0; j < GS; ++j) {
        if (x.pf.mode == 1) {
          // shared blocks: the member's state, unnormalized
          float* row = prefix_state_row<D>(x.pf, x.Hkv, x.G, c.vfirst, c.vcount, h0 + j);
          if (row) {
            if (lane == 0) {
              row[0] = st.m[j];
              row[1] = st.l[j];
            }
            float4* a4 = reinterpret_cast<float4*>(row + 4 + lane * G::EPL);
#pragma unroll
            for (int e = 0; e < G::EPL; e += 4)
              a4[e / 4] = make_float4(st.acc[j][e], st.acc[j][e + 1], st.acc[j][e + 2],
                                      st.acc[j][e + 3]);
          }
          continue;
        }
        if (x.pf.mode == 2) {
          // fold in the text's states over its shared blocks (prefetched by load_fold;
          // a level that does not apply is empty and weighs 0)
          const float M = fmaxf(st.m[j], fmaxf(st.fm[0][j], st.fm[1][j]));
          const float mu = M == -INFINITY ? 0.f : M;
          const float f = fast_exp2(st.m[j] - mu);
          const float fa = fast_exp2(st.fm[0][j] - mu), fb = fast_exp2(st.fm[1][j] - mu);
          st.l[j] = st.l[j] * f + st.fl[0][j] * fa + st.fl[1][j] * fb;
#pragma unroll
          for (int e = 0; e < G::EPL; ++e)
            st.acc[j][e] = st.acc[j][e] * f + st.facc[0][j][e] * fa + st.facc[1][j][e] * fb;
        }
        float o[G::EPL];
        const float inv = st.l[j] > 0.f ? v_scale / st.l[j] : 0.f;
        // 0 * acc: zeros when nothing was attended, NaN for a poisoned run
#pragma unroll
        for (int e = 0; e < G::EPL; ++e)
          o[e] = st.l[j] > 0.f ? st.acc[j][e] * inv : 0.f * st.acc[j][e];
        char* dst = out + ((int64_t)c.s * x.H + h0 + j) * D * elt_size<QT>() + lane * QP * 16;
#pragma unroll
        for (int p = 0; p < QP; ++p)
          reinterpret_cast<uint4*>(dst)[p] = narrow16<QT>(o + p * (G::EPL / QP));
      }
    } else {
      const int slot = seg::partial_slot(run_lo, seg_lo);
#pragma unroll
      for (int j = 0; j < GS; ++j) {
        float* p = partials + partial_index<D, GS>(w, slot, j);
        if (lane == 0) {
          p[0] = st.m[j];
          p[1] = st.l[j];
        }
        float4* a4 = reinterpret_cast<float4*>(p + 4 + lane * G::EPL);
#pragma unroll
        for (int e = 0; e < G::EPL; e += 4)
          a4[e / 4] = make_float4(st.acc[j][e], st.acc[j][e + 1], st.acc[j][e + 2], st.acc[j][e + 3]);
      }
    }
  }
  st.reset();
  if (x.pf.mode == 2) st.reset_fold();
}

// Mode 2: the offset (in floats, of the run's first query head; the GS rows follow it) of
// the state rows that flush_run folds in when the run whose last chunk the cursor c points
// at is finished within this segment and the text has a level to fold, else -1. 16- and
// 32-bit pools only (the shared-prefix call takes no E4M3 pools).
template <int KT, int QT, int D, int GS>
__device__ __forceinline__ int64_t fold_row(const Cursor& c, const Ctx& x, int64_t seg_lo,
                                            int64_t seg_hi) {
  if constexpr (KT != QT) {
    return -1;
  } else {
    if (x.pf.mode != 2 || c.fold == 0 || c.u != c.U - 1) return -1;
    const int64_t run_lo = c.excl + (int64_t)c.r * c.U;
    if (run_lo < seg_lo || run_lo + c.U > seg_hi) return -1;
    return ((int64_t)c.s * x.H + first_head_of<GS>(c.r, x)) * (D + 4);
  }
}

// Load the state rows the text folds (its fold mask) into st.fm / st.fl / st.facc (lane l
// holds the lane l % LPR slice, the slice the first row group's lanes fold in); the other
// set stays empty.
template <int KT, int D, int GS>
__device__ __forceinline__ void load_fold(State<KT, D, GS>& st, const Prefix& pf, int fold,
                                          int64_t off, int lane) {
  using G = Geo<KT, D>;
  const int lp = lane % G::LPR;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (!(fold >> k & 1)) continue;
    const float* row = (k == 0 ? pf.state0 : pf.state) + off;
#pragma unroll
    for (int j = 0; j < GS; ++j) {
      const float* r = row + j * (D + 4);
      const float2 ml = *reinterpret_cast<const float2*>(r);
      st.fm[k][j] = ml.x;
      st.fl[k][j] = ml.y;
#pragma unroll
      for (int e = 0; e < G::EPL; e += 4) {
        const float4 a = *reinterpret_cast<const float4*>(r + 4 + lp * G::EPL + e);
        st.facc[k][j][e] = a.x;
        st.facc[k][j][e + 1] = a.y;
        st.facc[k][j][e + 2] = a.z;
        st.facc[k][j][e + 3] = a.w;
      }
    }
  }
}

// This wave's segment of the unit numbering. Returns false when the wave has no units;
// otherwise sets the segment [seg_lo, seg_hi), the context and the cursor at the segment's
// first unit (all wave-uniform).
struct Segment {
  int w;
  int64_t seg_lo, seg_hi;
  int n;
  int64_t split_run;  // the run this segment's first boundary names to the merge, or -1
};

// One step of a wave scan: add the value that DPP control CTRL moves into each lane of the
// rows in ROWS (lanes without a source add 0), 64 bits as two halves with the carry.
template <int CTRL, int ROWS>
__device__ __forceinline__ void scan_step(uint32_t& lo, uint32_t& hi) {
  const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, CTRL, ROWS, 0xf, false);
  const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, CTRL, ROWS, 0xf, false);
  const uint32_t nl = lo + l2;
  hi = hi + h2 + (nl < lo ? 1u : 0u);
  lo = nl;
}

// Inclusive sum over lanes 0..lane of a wave, by DPP moves (no LDS): row shifts by 1, 2,
// 4, 8 within each row of 16 lanes, then lane 15 of each row into the next row, and lane 31
// into the upper two rows.
__device__ __forceinline__ int64_t wave_scan64(int64_t v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)((uint64_t)v >> 32);
  scan_step<0x111, 0xf>(lo, hi);  // row_shr:1
  scan_step<0x112, 0xf>(lo, hi);  // row_shr:2
  scan_step<0x114, 0xf>(lo, hi);  // row_shr:4
  scan_step<0x118, 0xf>(lo, hi);  // row_shr:8
  scan_step<0x142, 0xa>(lo, hi);  // row_bcast:15 into rows 1 and 3
  scan_step<0x143, 0xc>(lo, hi);  // row_bcast:31 into rows 2 and 3
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int src) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, src);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), src);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Every wave finds where its own segment starts from the texts' lengths: lane l takes a
// contiguous range of about S / 64 texts and sums their units (independent loads, all in
// flight), a wave-wide scan of the 64 range sums gives each range's first unit and the
// total, and a ballot names the lane whose range holds the wave's first unit. While that
// range holds more than one text, the wave splits it over its lanes the same way (a second
// round for S > 64, a third past 4,096). No barrier and no LDS: a wave starts loading keys
// and values as soon as its own lengths arrive (a workgroup-wide search with two barriers
// took 3.0 us from the first instruction to the first load on the 7 x 2,048 OPT-13B step,
// this one 2.2 us). Wave 0 of workgroup 0 also writes every text's first unit (excl_out)
// and the header (total units, segment length) for the merge, and a wave w < W whose
// segment is empty writes split_out[w] = -1; the others leave in sg.split_run the run (text
// x runs + run) that crosses into their segment from the segment before, or -1, for the
// kernel to store once its segment is done (a store ahead of the first loads delayed them). A run split over several segments is named once, by the first boundary it
// crosses, so a merge wave per boundary visits every split run once.
template <int B, int GS>
__device__ __forceinline__ bool start_segment(const int32_t* __restrict__ ctx, int S, int H,
                                              int Hkv, int maxb, int num_blocks, int W,
                                              int seg_fixed, const Prefix& pf,
                                              int64_t* __restrict__ hdr,
                                              int64_t* __restrict__ excl_out,
                                              int64_t* __restrict__ split_out, Segment& sg,
                                              Ctx& x, Cursor& cur) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t capacity = (int64_t)maxb * B;
  const int Gq = H / Hkv;
  const int R = Hkv * (Gq / GS);
  auto units_at = [&](int i) -> int64_t {
    int toff, over;
    return (int64_t)R * units_of(attended_len(ctx, pf.start, i, capacity, B, &toff, &over));
  };
  // lane's range of texts [r_lo, r_hi) of the n texts from lo, its units, and its first unit
  // (base + the units of the lower lanes' ranges)
  auto split = [&](int lo, int n, int64_t base, int& r_lo, int& r_hi, int64_t& mine,
                   int64_t& incl, int& first_raw) {
    const int per = (n + 63) / 64;
    r_lo = lo + (lane * per < n ? lane * per : n);
    r_hi = lo + (lane * per + per < n ? lane * per + per : n);
    first_raw = r_lo < r_hi ? ctx[r_lo] : 0;
    mine = 0;
    for (int i = r_lo; i < r_hi; ++i) mine += units_at(i);
    incl = wave_scan64(mine) + base;
    return per;
  };

  // ---- every text: the total, the segment length, the header ----
  int r_lo, r_hi, first_raw;
  int64_t mine, incl;
  int per = split(0, S, 0, r_lo, r_hi, mine, incl, first_raw);
  const int64_t total = readlane64(incl, 63);
  const int64_t seg = seg::segment_units(total, W, seg_fixed);
  if (blockIdx.x == 0 && wave == 0) {
    if (lane == 0) {
      hdr[0] = total;
      hdr[1] = seg;
    }
    int64_t e = incl - mine;
    for (int i = r_lo; i < r_hi; ++i) {
      excl_out[i] = e;
      e += units_at(i);
    }
  }

  sg.w = blockIdx.x * kWavesPerGroup + wave;
  sg.seg_lo = (int64_t)sg.w * seg;
  if (sg.w >= W) return false;
  if (sg.seg_lo >= total) {
    if (lane == 0) split_out[sg.w] = -1;
    return false;
  }
  sg.seg_hi = sg.seg_lo + seg < total ? sg.seg_lo + seg : total;
  sg.n = (int)(sg.seg_hi - sg.seg_lo);

  // ---- the text holding this wave's first unit: exactly one lane's range holds it ----
  const int64_t c0 = sg.seg_lo;
  int found, f_raw;
  int64_t f_excl;
  for (;;) {
    const uint64_t hit = __ballot(c0 >= incl - mine && c0 < incl);
    const int src = __builtin_amdgcn_readfirstlane(__builtin_ffsll((long long)hit) - 1);
    const int lo = __builtin_amdgcn_readlane(r_lo, src);
    const int hi = __builtin_amdgcn_readlane(r_hi, src);
    const int64_t base = readlane64(incl - mine, src);
    if (per == 1 || hi - lo <= 1) {  // (each round's n is below the last's: it ends)
      found = lo < S ? lo : S - 1;
      f_raw = __builtin_amdgcn_readlane(first_raw, src);
      f_excl = base;
      break;
    }
    per = split(lo, hi - lo, base, r_lo, r_hi, mine, incl, first_raw);
  }

  x = Ctx{S, H, Hkv, Gq, Gq / GS, R, maxb, num_blocks, B, capacity, ctx, pf};
  cur.excl = f_excl;
  set_text_raw(cur, x, found, f_raw);
  const int64_t off = c0 - f_excl;  // below R * U
  cur.r = off <= 0x7fffffff ? (int)off / cur.U : (int)(off / cur.U);
  cur.u = (int)(off - (int64_t)cur.r * cur.U);
  sg.split_run = seg::names_split_run(cur.u, seg) ? (int64_t)found * R + cur.r : -1;
  return true;
}

template <int KT, int QT, int D, int B, int GS, bool FUSED>
__global__ __launch_bounds__(kThreads) void decode_partition(
    char* __restrict__ out, const char* __restrict__ q, const char* __restrict__ kc,
    const char* __restrict__ vc, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ ctx, int S, int H, int Hkv, int maxb, int num_blocks, int W,
    int seg_fixed, float scale_log2, float v_scale, int64_t* __restrict__ hdr,
    int64_t* __restrict__ excl_out, float* __restrict__ partials,
    int64_t* __restrict__ split_out, NewRows nr_arg, const int64_t* __restrict__ new_slots,
    Prefix pf) {
  // the slots as a restrict argument: the compiler may then read them through the scalar
  // cache, which keeps the fused write's slot lookup out of the vector wait counts
  NewRows nr = nr_arg;
  nr.slots = new_slots;
  const int lane = threadIdx.x & 63;
  Segment sg;
  Ctx x;
  Cursor cur;
  if (!start_segment<B, GS>(ctx, S, H, Hkv, maxb, num_blocks, W, seg_fixed, pf, hdr, excl_out,
                            split_out, sg, x, cur))
    return;
  const int w = sg.w;
  const int64_t seg_lo = sg.seg_lo, seg_hi = sg.seg_hi;
  const int n = sg.n;
  const int64_t split_run = sg.split_run;
  Cursor ld = cur;
  const float sl = scale_log2;

  State<KT, D, GS> st;
  st.reset();
  st.reset_fold();
  Buf<KT, QT, D, GS> A, Bb;
  load_chunk<KT, QT, D, B, GS, FUSED>(A, ld, x, kc, vc, q, tables, nr, lane);
  {
    const int64_t fr = fold_row<KT, QT, D, GS>(ld, x, seg_lo, seg_hi);
    if (fr >= 0) load_fold<KT, D, GS>(st, x.pf, ld.fold, fr, lane);
  }
  advance(ld, x);

  auto compute = [&](const Buf<KT, QT, D, GS>& b) {
    compute_chunk<KT, QT, D, GS>(b, cur, st, sl, lane);
    if constexpr (FUSED) {
      using G = Geo<KT, D>;
      if (writes_new_row<B, GS>(cur, x)) {
        const int g = lane / G::LPR;
#pragma unroll
        for (int i = 0; i < G::NLD; ++i)
          if (cur.u * kChunk + i * G::RPW + g == cur.L - 1)
            store_new_piece<D, G::ELT, B, GS>(nr, cur, x, (lane % G::LPR) * 16, b.k[i], b.v[i]);
      }
    }
  };
  auto finish = [&](int i) {
    // last chunk of the run, or of the segment
    if (cur.u == cur.U - 1 || i == n - 1)
      flush_run<KT, QT, D, GS>(st, cur, x, seg_lo, seg_hi, w, out, partials, v_scale, lane);
    advance(cur, x);
  };

  if constexpr (KT == PA_FP8_E4M3) {
    // 8-bit pools: a chunk is half the bytes of a 16-bit one, so two chunks stay in flight
    // (three buffers) to keep as many bytes in flight per wave. (No fold rows and no fused
    // write here: neither takes 8-bit pools.)
    Buf<KT, QT, D, GS> C;
    if (n > 1) {
      load_chunk<KT, QT, D, B, GS, FUSED>(Bb, ld, x, kc, vc, q, tables, nr, lane);
      advance(ld, x);
    }
    int i = 0;
    while (i + 4 < n) {  // A: chunk i, Bb: chunk i + 1, both issued
      load_chunk<KT, QT, D, B, GS, FUSED>(C, ld, x, kc, vc, q, tables, nr, lane);
      advance(ld, x);
      compute(A);
      finish(i);
      load_chunk<KT, QT, D, B, GS, FUSED>(A, ld, x, kc, vc, q, tables, nr, lane);
      advance(ld, x);
      compute(Bb);
      finish(i + 1);
      load_chunk<KT, QT, D, B, GS, FUSED>(Bb, ld, x, kc, vc, q, tables, nr, lane);
      advance(ld, x);
      compute(C);
      finish(i + 2);
      i += 3;
    }
    const int r = n - i;  // 1 .. 4 chunks left; A holds chunk i, Bb chunk i + 1 (r >= 2)
    if (r >= 3) {
      load_chunk<KT, QT, D, B, GS, FUSED>(C, ld, x, kc, vc, q, tables, nr, lane);
      advance(ld, x);
    }
    compute(A);
    finish(i);
    if (r == 4) load_chunk<KT, QT, D, B, GS, FUSED>(A, ld, x, kc, vc, q, tables, nr, lane);
    if (r >= 2) {
      compute(Bb);
      finish(i + 1);
    }
    if (r >= 3) {
      compute(C);
      finish(i + 2);
    }
    if (r == 4) {
      compute(A);
      finish(i + 3);
    }
    if (lane == 0) split_out[w] = split_run;
    return;
  }
  // steady state: both loads unconditional, so the next chunk's loads stay in
  // flight while the current one is computed
  // (a chunk's fold row is loaded once the chunk before it has been finished, which
  // is when that chunk's own fold, if any, has been used)
  int i = 0;
  while (i + 2 < n) {
    load_chunk<KT, QT, D, B, GS, FUSED>(Bb, ld, x, kc, vc, q, tables, nr, lane);
    const int64_t fb = fold_row<KT, QT, D, GS>(ld, x, seg_lo, seg_hi);
    const int fbm = ld.fold;
    advance(ld, x);
    compute(A);
    finish(i);
    if (fb >= 0) load_fold<KT, D, GS>(st, x.pf, fbm, fb, lane);
    load_chunk<KT, QT, D, B, GS, FUSED>(A, ld, x, kc, vc, q, tables, nr, lane);
    const int64_t fa = fold_row<KT, QT, D, GS>(ld, x, seg_lo, seg_hi);
    const int fam = ld.fold;
    advance(ld, x);
    compute(Bb);
    finish(i + 1);
    if (fa >= 0) load_fold<KT, D, GS>(st, x.pf, fam, fa, lane);
    i += 2;
  }
  if (i + 1 < n) {
    load_chunk<KT, QT, D, B, GS, FUSED>(Bb, ld, x, kc, vc, q, tables, nr, lane);
    const int64_t fb = fold_row<KT, QT, D, GS>(ld, x, seg_lo, seg_hi);
    const int fbm = ld.fold;
    compute(A);
    finish(i);
    if (fb >= 0) load_fold<KT, D, GS>(st, x.pf, fbm, fb, lane);
    compute(Bb);
    finish(i + 1);
  } else {
    compute(A);
    finish(i);
  }
  if (lane == 0) split_out[w] = split_run;
}

// Combining the partials of one run, left by segments w0..w1, in segment order, for all GS
// query heads of the run at once: the wave's lanes form GS groups of CL = 64 / GS lanes,
// group j taking head j's D values, PE = D / CL per lane. Segment w0 holds the run in its
// slot 1 unless the run starts exactly at w0's first unit (then it is w0's first run, slot
// 0); every later segment starts inside the run, so the run is its first run (slot 0).
// The partials are read UNROLL at a time with all loads in flight.
//
// The records a merge step reads: UNROLL partials of one lane's head (m, l, its acc values).
template <int D, int GS>
struct MergeBatch {
  static constexpr int CL = 64 / GS;  // lanes per head
  static constexpr int PE = D / CL;   // values per lane
  static constexpr int UNROLL = PE >= 16 ? 4 : 8;
  float m[UNROLL], l[UNROLL], a[UNROLL][PE];
};

// Loads the partials of segments w .. min(w + UNROLL - 1, w1) of the run starting at run_lo
// (past w1: empty partials of weight 0).
template <int D, int GS>
__device__ __forceinline__ void load_batch(MergeBatch<D, GS>& b, const float* __restrict__ partials,
                                           int64_t w, int64_t w1, int64_t run_lo, int64_t seg,
                                           int lane) {
  using MB = MergeBatch<D, GS>;
  const int j = lane / MB::CL, c = lane % MB::CL;
#pragma unroll
  for (int k = 0; k < MB::UNROLL; ++k) {
    b.m[k] = -INFINITY;
    b.l[k] = 0.f;
#pragma unroll
    for (int e = 0; e < MB::PE; ++e) b.a[k][e] = 0.f;
    if (w + k <= w1) {
      const float* p =
          partials + partial_index<D, GS>(w + k, seg::partial_slot(run_lo, (w + k) * seg), j);
      b.m[k] = p[0];
      b.l[k] = p[1];
#pragma unroll
      for (int e = 0; e < MB::PE; ++e) b.a[k][e] = p[4 + c * MB::PE + e];
    }
  }
}

template <int D, int GS>
__device__ __forceinline__ void fold_batch(const MergeBatch<D, GS>& b, float& M, float& den,
                                           float* num) {
  using MB = MergeBatch<D, GS>;
  float mg = M;
#pragma unroll
  for (int k = 0; k < MB::UNROLL; ++k) mg = fmaxf(mg, b.m[k]);
  const float mu = mg == -INFINITY ? 0.f : mg;
  const float r = fast_exp2(M - mu);
  den *= r;
#pragma unroll
  for (int e = 0; e < MB::PE; ++e) num[e] *= r;
#pragma unroll
  for (int k = 0; k < MB::UNROLL; ++k) {  // segment order
    const float f = fast_exp2(b.m[k] - mu);
    den += f * b.l[k];
#pragma unroll
    for (int e = 0; e < MB::PE; ++e) num[e] += f * b.a[k][e];
  }
  M = mg;
}

// Writes a merged run: the state itself (state_dst, unnormalized) or the output row
// (dst_row; null with no state_dst: the lane's head writes nothing).
template <int QT, int D, int GS>
__device__ __forceinline__ void merge_finish(float M, float den, const float* num,
                                             float v_scale, char* __restrict__ dst_row,
                                             float* state_dst, int lane) {
  using MB = MergeBatch<D, GS>;
  constexpr int PE = MB::PE;
  const int c = lane % MB::CL;
  if (state_dst || !dst_row) {
    if (!state_dst) return;
    if (c == 0) {
      state_dst[0] = M;
      state_dst[1] = den;
    }
#pragma unroll
    for (int e = 0; e < PE; ++e) state_dst[4 + c * PE + e] = num[e];
    return;
  }
  float o[PE];
  const float inv = den > 0.f ? v_scale / den : 0.f;
  // 0 * num: NaN stays visible for a poisoned run
#pragma unroll
  for (int e = 0; e < PE; ++e) o[e] = den > 0.f ? num[e] * inv : 0.f * num[e];
  store_out<QT, PE>(dst_row + c * PE * elt_size<QT>(), o);
}

// Merges a run's partials w0 .. w1 (in segment order) into its output row, with one
// running maximum (the rescaling of the online softmax), in one pass. init / init2: states
// (m, l, pad, pad, acc[D]) of the lane's head that come first (null: none); state_dst: the
// merged state itself is written there instead of an output row (null: the lane's head
// writes nothing).
template <int QT, int D, int GS>
__device__ __forceinline__ void merge_run(const float* __restrict__ partials, int64_t w0,
                                          int64_t w1, int64_t run_lo, int64_t seg,
                                          float v_scale, char* __restrict__ dst_row, int lane,
                                          const float* init, float* state_dst,
                                          const float* init2) {
  using MB = MergeBatch<D, GS>;
  constexpr int PE = MB::PE;
  const int c = lane % MB::CL;
  float M = -INFINITY, den = 0.f, num[PE];
#pragma unroll
  for (int e = 0; e < PE; ++e) num[e] = 0.f;
  if (init) {
    M = init[0];
    den = init[1];
#pragma unroll
    for (int e = 0; e < PE; ++e) num[e] = init[4 + c * PE + e];
  }
  if (init2) {  // a second state (the inner level's), folded in as a partial would be
    const float m2 = init2[0], mg = fmaxf(M, m2);
    const float mu = mg == -INFINITY ? 0.f : mg;
    const float r = fast_exp2(M - mu), f = fast_exp2(m2 - mu);
    den = den * r + init2[1] * f;
#pragma unroll
    for (int e = 0; e < PE; ++e) num[e] = num[e] * r + init2[4 + c * PE + e] * f;
    M = mg;
  }
  for (int64_t w = w0; w <= w1; w += MB::UNROLL) {
    MB b;
    load_batch<D, GS>(b, partials, w, w1, run_lo, seg, lane);
    fold_batch<D, GS>(b, M, den, num);
  }
  merge_finish<QT, D, GS>(M, den, num, v_scale, dst_row, state_dst, lane);
}

// Merge pass: one wave per run (a text's head group of GS query heads), or per segment
// boundary when runs outnumber segments (decode_merge's split array), all GS heads at
// once; runs finished inside one segment return at once. W: segments of the partition
// launch (the merge range is clamped to it). (One wave per query head instead launched GS
// times the waves for the same partials. Taking the first unit and the segment length from
// the lengths themselves for small batches, instead of the header and offsets the partition
// kernel wrote, measured 0.6 us slower per op on the 7 x 2,048 OPT-13B step: loading the
// partials on a guess beside them, checked against them, is what saves the round trip.)
// The merge of run `run` (wave-uniform) of one pass.
template <int QT, int D, int GS>
__device__ __forceinline__ void merge_one_run(
    char* __restrict__ out, const int32_t* __restrict__ ctx, int S, int H, int Hkv, int maxb,
    int bsz, int W, float v_scale, const int64_t* __restrict__ hdr,
    const int64_t* __restrict__ excl, const float* __restrict__ partials, const Prefix& pf,
    int max_ctx, int seg_fixed, int64_t run) {
  const int lane = threadIdx.x & 63;
  const int Gq = H / Hkv, NG = Gq / GS, R = Hkv * NG;
  if (run >= (int64_t)S * R) return;
  const int s = (int)(run / R), r = (int)(run - (int64_t)s * R);
  const int64_t capacity = (int64_t)maxb * bsz;
  if (pf.mode == 0) {
    // The geometry if every text attends max_context_len tokens (a batch of equal lengths):
    // this run's partials are loaded on that guess at once, beside the lengths, header and
    // offsets that decide it, instead of after them (one memory round trip fewer), and
    // used only where the guess holds.
    const int Lg = max_ctx < 0 ? 0 : max_ctx > capacity ? (int)capacity : max_ctx;
    const int Ug = units_of(Lg);
    const int64_t segg = seg::segment_units((int64_t)S * R * Ug, W, seg_fixed);
    const int64_t log = ((int64_t)s * R + r) * Ug;
    int64_t gw0, gw1;
    seg::run_segments(log, log + Ug, segg, W, &gw0, &gw1);
    using MB = MergeBatch<D, GS>;
    MB b;
    load_batch<D, GS>(b, partials, gw0, gw1, log, segg, lane);
    int toff, over;
    const int L = attended_len(ctx, pf.start, s, capacity, bsz, &toff, &over);
    const int64_t seg = hdr[1];
    const int64_t lo = excl[s] + (int64_t)r * units_of(L);
    if (units_of(L) == Ug && seg == segg && lo == log) {
      if (gw0 == gw1) return;
      const int h = (r / NG) * Gq + (r % NG) * GS + lane / (64 / GS);
      float M = -INFINITY, den = 0.f, num[MB::PE];
#pragma unroll
      for (int e = 0; e < MB::PE; ++e) num[e] = 0.f;
      fold_batch<D, GS>(b, M, den, num);  // the same batches, in the same order, as merge_run
      for (int64_t w = gw0 + MB::UNROLL; w <= gw1; w += MB::UNROLL) {
        MB b2;
        load_batch<D, GS>(b2, partials, w, gw1, lo, seg, lane);
        fold_batch<D, GS>(b2, M, den, num);
      }
      merge_finish<QT, D, GS>(M, den, num, v_scale,
                              out + ((int64_t)s * H + h) * D * elt_size<QT>(), nullptr, lane);
      return;
    }
  }
  int toff, over;
  const int L = attended_len(ctx, pf.start, s, capacity, bsz, &toff, &over);
  const int U = units_of(L);
  const int64_t seg = hdr[1];
  const int64_t lo = excl[s] + (int64_t)r * U, hi = lo + U;
  int64_t w0, w1;
  seg::run_segments(lo, hi, seg, W, &w0, &w1);
  if (w0 == w1) return;
  const int h = (r / NG) * Gq + (r % NG) * GS + lane / (64 / GS);  // the lane's query head
  const int64_t pair = (int64_t)s * H + h;
  if (pf.mode == 1) {
    int f, n;
    group_members(pf, s, f, n);
    float* row = prefix_state_row<D>(pf, Hkv, Gq, f, n, h);
    merge_run<QT, D, GS>(partials, w0, w1, lo, seg, v_scale, nullptr, lane, nullptr, row,
                         nullptr);
    return;
  }
  // mode 2: the text's states over its shared blocks come first (the levels that apply)
  const int fold = pf.mode == 2 ? fold_mask(pf, s) : 0;
  const float* init = fold & 1 ? pf.state0 + pair * (D + 4) : nullptr;
  const float* init2 = fold & 2 ? pf.state + pair * (D + 4) : nullptr;
  merge_run<QT, D, GS>(partials, w0, w1, lo, seg, v_scale, out + pair * D * elt_size<QT>(),
                       lane, init, nullptr, init2);
}

// The run merge wave i takes: run i, or with `split` (batches with more runs than
// segments) the run that crosses segment boundary i, if any (-1: none).
__device__ __forceinline__ int64_t merge_run_of(const int64_t* __restrict__ split, int W,
                                                int64_t i) {
  if (!split) return i;
  return i < W ? split[i] : -1;
}

template <int QT, int D, int GS>
__global__ __launch_bounds__(kThreads) void decode_merge(
    char* __restrict__ out, const int32_t* __restrict__ ctx, int S, int H, int Hkv, int maxb,
    int bsz, int W, float v_scale, const int64_t* __restrict__ hdr,
    const int64_t* __restrict__ excl, const float* __restrict__ partials,
    const int64_t* __restrict__ split, Prefix pf, int max_ctx, int seg_fixed) {
  const int64_t run = merge_run_of(
      split, W,
      (int64_t)blockIdx.x * kWavesPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
  if (run < 0) return;
  merge_one_run<QT, D, GS>(out, ctx, S, H, Hkv, maxb, bsz, W, v_scale, hdr, excl, partials, pf,
                           max_ctx, seg_fixed, run);
}

// One shared-block level's pass as its merge reads it (shared-prefix mode 1: states out).
struct MergePass {
  const int32_t* ctx;  // the level's group lengths
  int S, H, maxb, W, max_ctx;
  const int64_t* hdr;
  const int64_t* excl;
  const float* partials;
  const int64_t* split;  // the split runs by segment boundary, or null: a wave per run
  Prefix pf;
  int groups;  // workgroups of this pass's merge
};

// The merges of both levels of the nested shared-block decode in one launch: workgroups
// below a.groups merge the outer level's runs, the rest the inner level's (each level's
// passes wrote their own partials, so both run after both passes).
template <int QT, int D, int GS0, int GS1>
__global__ __launch_bounds__(kThreads) void decode_merge_pair(MergePass a, MergePass b, int Hkv,
                                                              int bsz) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if ((int)blockIdx.x < a.groups) {
    const int64_t run = merge_run_of(a.split, a.W, (int64_t)blockIdx.x * kWavesPerGroup + w);
    if (run >= 0)
      merge_one_run<QT, D, GS0>(nullptr, a.ctx, a.S, a.H, Hkv, a.maxb, bsz, a.W, 1.0f, a.hdr,
                                a.excl, a.partials, a.pf, a.max_ctx, 0, run);
  } else {
    const int64_t run =
        merge_run_of(b.split, b.W, (int64_t)(blockIdx.x - a.groups) * kWavesPerGroup + w);
    if (run >= 0)
      merge_one_run<QT, D, GS1>(nullptr, b.ctx, b.S, b.H, Hkv, b.maxb, bsz, b.W, 1.0f, b.hdr,
                                b.excl, b.partials, b.pf, b.max_ctx, 0, run);
  }
}

// ---- shared key/value heads on the matrix cores --------------------------------
//
// With 8 (or 4) query heads per key/value head, every key and value row feeds 8 (4) dot
// products and as many weighted sums: 4-8 flop per byte, which the vector ALUs cannot sustain at
// HBM speed. Here a wave's GS = 8 (or 4) heads are the columns of 16x16 MFMA tiles:
//   S^T (16 tokens x heads) = K (16 tokens x 32 dims) . Q^T     v_mfma_f32_16x16x32
//   O^T (16 dims x heads)  += V^T (16 dims x 16 tokens) . P^T  v_mfma_f32_16x16x16
// Lane l (col = l % 16, grp = l / 16) loads 16 bytes of token col's key and value rows at
// dims 8 grp + 32 c, which is the K operand's layout as loaded; its S^T results are head
// col's scores for tokens 4 grp .. 4 grp + 3, which is the P^T operand's layout. The
// values go through the wave's own LDS rows once, for the transposing read that builds
// the V^T operand. Segmentation, partials and the merge are those of decode_partition.

template <int QT>
struct Mma16;

template <>
struct Mma16<PA_F16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f4 qk(v8 a, v8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f4 pv(v4 a, v4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){x, y}, h2));
  }
};

template <>
struct Mma16<PA_BF16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef short v4 __attribute__((ext_vector_type(4)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f4 qk(v8 a, v8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f4 pv(v4 a, v4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){x, y}, b2));
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct MmaBuf {
  uint4 k[D / 32];
  uint4 v[D / 32];
  bool bad;
};

template <int D>
struct MmaState {
  typedef float f4 __attribute__((ext_vector_type(4)));
  f4 o[D / 16];  // O^T tile mt: dims 16 mt + 4 grp + r, head col
  float m, l;    // head col's running maximum; sum over this lane's tokens
  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) o[mt] = f4{0.f, 0.f, 0.f, 0.f};
  }
};

template <int QT, int D, int B, int GS, bool FUSED>
__device__ __forceinline__ void load_chunk_mma(MmaBuf<D>& b, const Cursor& c, const Ctx& x,
                                               const char* __restrict__ kc,
                                               const char* __restrict__ vc,
                                               const int32_t* __restrict__ tables,
                                               const NewRows& nr, int lane) {
  constexpr int kRowBytes = D * 2;
  constexpr int64_t kTileBytes = (int64_t)B * kRowBytes;
  const int col = lane & 15, grp = lane >> 4;
  const int kvh = kv_head_of<GS>(c.r, x);
  const int last = c.L > 0 ? c.L - 1 : 0;
  const int32_t* trow = tables + (int64_t)c.s * x.maxb + c.toff / B;
  const int t = c.u * kChunk + col;
  const int tc = t < last ? t : last;
  int blk;
  if constexpr (B >= kChunk) {
    const int t0 = min(c.u * kChunk, last);  // the chunk lies in one block
    blk = trow[t0 / B];
  } else {
    blk = trow[tc / B];
  }
  const bool bad = (unsigned)blk >= (unsigned)x.num_blocks;
  b.bad = c.over || bad;
  if (bad) blk = 0;  // read block 0 instead; the result is poisoned
  const int64_t row = ((int64_t)blk * x.Hkv + kvh) * kTileBytes + (int64_t)(tc % B) * kRowBytes;
  // fused write: the last position's rows come from k_new / v_new
  const bool fresh = FUSED && tc == last;
  const char* ksrc = fresh ? nr.k + ((int64_t)c.s * x.Hkv + kvh) * kRowBytes : kc + row;
#pragma unroll
  for (int cc = 0; cc < D / 32; ++cc) b.k[cc] = load_stream(ksrc + (8 * grp + 32 * cc) * 2);
  // values go through LDS anyway (for the transposing read), so they are loaded whole rows
  // at a time: load cc takes rows kVRows cc + lane / kVLanes, 16 bytes each (the keys' MFMA
  // layout reads half of each 128-byte line per load)
  constexpr int kVLanes = kRowBytes / 16, kVRows = 64 / kVLanes;
  const int vr = lane / kVLanes, vp = lane % kVLanes;
  const char* vnew = nr.v + ((int64_t)c.s * x.Hkv + kvh) * kRowBytes + vp * 16;
#pragma unroll
  for (int cc = 0; cc < D / 32; ++cc) {
    const int tv = c.u * kChunk + kVRows * cc + vr;
    const int tvc = tv < last ? tv : last;
    int vblk = blk;
    if constexpr (B < kChunk) {
      vblk = trow[tvc / B];
      if ((unsigned)vblk >= (unsigned)x.num_blocks) {
        b.bad = true;
        vblk = 0;
      }
    }
    const char* vsrc = FUSED && tvc == last
                           ? vnew
                           : vc + ((int64_t)vblk * x.Hkv + kvh) * kTileBytes +
                                 (int64_t)(tvc % B) * kRowBytes + vp * 16;
    b.v[cc] = load_stream(vsrc);
  }
}

template <int QT, int D>
__device__ __forceinline__ void compute_chunk_mma(const MmaBuf<D>& b, const Cursor& c,
                                                  MmaState<D>& st,
                                                  const typename Mma16<QT>::v8* qv,
                                                  uint16_t* __restrict__ vrow, float scale_log2,
                                                  int lane) {
  using M = Mma16<QT>;
  typedef typename M::v8 v8;
  typedef typename M::v4 v4;
  typedef typename M::f4 f4;
  constexpr int VS = D + 16;  // LDS row: 8-bank shift per row for the transposing read
  if (c.L == 0) return;  // nothing attended: the run's result is zeros
  const int col = lane & 15, grp = lane >> 4;
  // values into this wave's LDS rows, read back transposed below (load cc holds rows
  // kVRows cc + lane / kVLanes, piece lane % kVLanes)
  constexpr int kVLanes = D * 2 / 16, kVRows = 64 / kVLanes;
#pragma unroll
  for (int cc = 0; cc < D / 32; ++cc)
    *reinterpret_cast<uint4*>(vrow + (kVRows * cc + lane / kVLanes) * VS +
                              8 * (lane % kVLanes)) = b.v[cc];
  f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cc = 0; cc < D / 32; ++cc) s = M::qk(__builtin_bit_cast(v8, b.k[cc]), qv[cc], s);
  float z[4];
  float cm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = c.u * kChunk + 4 * grp + r;
    z[r] = t < c.L ? s[r] * scale_log2 : -INFINITY;
    cm = fmaxf(cm, z[r]);
  }
  cm = fmaxf(cm, __shfl_xor(cm, 16));
  cm = fmaxf(cm, __shfl_xor(cm, 32));
  const float mn = fmaxf(st.m, cm);
  if (__any(mn > st.m)) {
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(st.m - mu);  // m = -inf: 0
    st.l *= alpha;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) st.o[mt] *= alpha;
    st.m = mn;
  }
  const float mu = st.m == -INFINITY ? 0.f : st.m;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    z[r] = fast_exp2(z[r] - mu);
    st.l += z[r];
  }
  const uint2 pw = make_uint2(M::pack2(z[0], z[1]), M::pack2(z[2], z[3]));
  const v4 pb = __builtin_bit_cast(v4, pw);
  // V^T operand of dims 16 mt + col: lane j of a 16-lane group addresses token
  // 4 grp + j / 4 at dims 16 mt + 4 (j % 4); the transposing read hands lane i the
  // 4 tokens at dim 16 mt + i
  const uint16_t* vsrc = vrow + (4 * grp + (col >> 2)) * VS + 4 * (col & 3);
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) {
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vsrc + 16 * mt));
    st.o[mt] = M::pv(__builtin_bit_cast(v4, a), pb, st.o[mt]);
  }
  if (b.bad) {
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) st.o[mt] = f4{1.f, 1.f, 1.f, 1.f} * __builtin_nanf("");
  }
}

template <int QT, int D, int GS>
__device__ __forceinline__ void flush_run_mma(MmaState<D>& st, const Cursor& c, const Ctx& x,
                                              int64_t seg_lo, int64_t seg_hi, int w,
                                              char* __restrict__ out, float* __restrict__ partials,
                                              float v_scale, int lane) {
  const int col = lane & 15, grp = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const int64_t run_lo = c.excl + (int64_t)c.r * c.U;
  const int64_t run_hi = run_lo + c.U;
  const int h0 = first_head_of<GS>(c.r, x);
  if (col < GS) {
    if (run_lo >= seg_lo && run_hi <= seg_hi && x.pf.mode == 1) {
      // shared blocks: the member's state, unnormalized
      float* row = prefix_state_row<D>(x.pf, x.Hkv, x.G, c.vfirst, c.vcount, h0 + col);
      if (row) {
        if (grp == 0) {
          row[0] = st.m;
          row[1] = l;
        }
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt)
          *reinterpret_cast<float4*>(row + 4 + 16 * mt + 4 * grp) =
              make_float4(st.o[mt][0], st.o[mt][1], st.o[mt][2], st.o[mt][3]);
      }
    } else if (run_lo >= seg_lo && run_hi <= seg_hi) {
      // the whole run is in this segment: finish it here
      if (x.pf.mode == 2) {
        // fold in the text's states over its shared blocks (the levels that apply)
        const int64_t off = ((int64_t)c.s * x.H + h0 + col) * (D + 4);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if (!(c.fold >> k & 1)) continue;
          const float* row = (k == 0 ? x.pf.state0 : x.pf.state) + off;
          const float ms = row[0], M = fmaxf(st.m, ms);
          const float mu = M == -INFINITY ? 0.f : M;
          const float fa = fast_exp2(st.m - mu), fb = fast_exp2(ms - mu);
          l = l * fa + row[1] * fb;
#pragma unroll
          for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              st.o[mt][r] = st.o[mt][r] * fa + row[4 + 16 * mt + 4 * grp + r] * fb;
          st.m = M;
        }
      }
      const float inv = l > 0.f ? v_scale / l : 0.f;
      char* dst = out + ((int64_t)c.s * x.H + h0 + col) * D * elt_size<QT>();
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        float o[4];
        // 0 * acc: zeros when nothing was attended, NaN for a poisoned run
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = l > 0.f ? st.o[mt][r] * inv : 0.f * st.o[mt][r];
        store_out<QT, 4>(dst + (16 * mt + 4 * grp) * elt_size<QT>(), o);
      }
    } else {
      const int slot = seg::partial_slot(run_lo, seg_lo);
      float* p = partials + partial_index<D, GS>(w, slot, col);
      if (grp == 0) {
        p[0] = st.m;
        p[1] = l;
      }
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt)
        *reinterpret_cast<float4*>(p + 4 + 16 * mt + 4 * grp) =
            make_float4(st.o[mt][0], st.o[mt][1], st.o[mt][2], st.o[mt][3]);
    }
  }
  st.reset();
}

template <int QT, int D, int B, int GS, bool FUSED>
__global__ __launch_bounds__(kThreads) void decode_partition_mma(
    char* __restrict__ out, const char* __restrict__ q, const char* __restrict__ kc,
    const char* __restrict__ vc, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ ctx, int S, int H, int Hkv, int maxb, int num_blocks, int W,
    int seg_fixed, float scale_log2, float v_scale, int64_t* __restrict__ hdr,
    int64_t* __restrict__ excl_out, float* __restrict__ partials,
    int64_t* __restrict__ split_out, NewRows nr_arg, const int64_t* __restrict__ new_slots,
    Prefix pf) {
  static_assert(GS == 4 || GS == 8, "4 or 8 query heads per wave");
  NewRows nr = nr_arg;
  nr.slots = new_slots;
  constexpr int VS = D + 16;
  using M = Mma16<QT>;
  typedef typename M::v8 v8;
  __shared__ __align__(16) uint16_t vlds[kWavesPerGroup][kChunk * VS];
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  Segment sg;
  Ctx x;
  Cursor cur;
  if (!start_segment<B, GS>(ctx, S, H, Hkv, maxb, num_blocks, W, seg_fixed, pf, hdr, excl_out,
                            split_out, sg, x, cur))
    return;
  const int w = sg.w;
  const int64_t seg_lo = sg.seg_lo, seg_hi = sg.seg_hi;
  const int n = sg.n;
  const int64_t split_run = sg.split_run;
  uint16_t* vrow = vlds[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];

  // Q^T operand of the run's 8 heads: lane holds q[h0 + col][8 grp + 32 c .. +7]; the
  // unused columns 8..15 are zero
  v8 qv[D / 32];
  int q_run = -1, q_text = -1;
  auto load_q = [&](const Cursor& c) {
    if (c.r == q_run && c.s == q_text) return;
    q_run = c.r;
    q_text = c.s;
    const int h = first_head_of<GS>(c.r, x) + (col & (GS - 1));
    const int kvh = kv_head_of<GS>(c.r, x);
    const char* qrow =
        q + (x.pf.mode == 1 ? group_q_row(x.pf, c.vfirst, c.vcount, kvh, h - kvh * x.G)
                            : (int64_t)c.s * x.H + h) * D * 2;
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc) {
      uint4 v = *reinterpret_cast<const uint4*>(qrow + (8 * grp + 32 * cc) * 2);
      if (col >= GS) v = make_uint4(0u, 0u, 0u, 0u);
      qv[cc] = __builtin_bit_cast(v8, v);
    }
  };

  Cursor ld = cur;
  MmaState<D> st;
  st.reset();
  MmaBuf<D> A, Bb;
  load_chunk_mma<QT, D, B, GS, FUSED>(A, ld, x, kc, vc, tables, nr, lane);
  advance(ld, x);

  auto step = [&](const MmaBuf<D>& b, int i) {
    load_q(cur);
    compute_chunk_mma<QT, D>(b, cur, st, qv, vrow, scale_log2, lane);
    if constexpr (FUSED) {
      if (writes_new_row<B, GS>(cur, x)) {
        const int at = cur.L - 1 - cur.u * kChunk;  // the new row's place in the chunk
        if (col == at) {
#pragma unroll
          for (int cc = 0; cc < D / 32; ++cc)
            store_new_piece_of<D, 2, B, GS>(nr, nr.kc, cur, x, (8 * grp + 32 * cc) * 2, b.k[cc]);
        }
        constexpr int kVLanes = D * 2 / 16, kVRows = 64 / kVLanes;
#pragma unroll
        for (int cc = 0; cc < D / 32; ++cc)
          if (kVRows * cc + lane / kVLanes == at)
            store_new_piece_of<D, 2, B, GS>(nr, nr.vc, cur, x, (lane % kVLanes) * 16, b.v[cc]);
      }
    }
    // last chunk of the run, or of the segment
    if (cur.u == cur.U - 1 || i == n - 1)
      flush_run_mma<QT, D, GS>(st, cur, x, seg_lo, seg_hi, w, out, partials, v_scale, lane);
    advance(cur, x);
  };

  // steady state: both loads unconditional, so the next chunk's loads stay in flight
  // while the current one is computed
  int i = 0;
  while (i + 2 < n) {
    load_chunk_mma<QT, D, B, GS, FUSED>(Bb, ld, x, kc, vc, tables, nr, lane);
    advance(ld, x);
    step(A, i);
    load_chunk_mma<QT, D, B, GS, FUSED>(A, ld, x, kc, vc, tables, nr, lane);
    advance(ld, x);
    step(Bb, i + 1);
    i += 2;
  }
  if (i + 1 < n) {
    load_chunk_mma<QT, D, B, GS, FUSED>(Bb, ld, x, kc, vc, tables, nr, lane);
    step(A, i);
    step(Bb, i + 1);
  } else {
    step(A, i);
  }
  if (lane == 0) split_out[w] = split_run;
}

// ---- launch ------------------------------------------------------------------

// Workspace: header (total units, segment length), int64 unit offset of each text [S],
// int64 split run of each segment boundary [W], fp32 partials [W][2][GS][D+4] (sized for
// GS = 8). Written by decode_partition, read by decode_merge.
struct Layout {
  int64_t W;  // wavefronts (segments) in the grid
  size_t excl_off, split_off, part_off, bytes;
};

// Merge waves of a pass with `runs` runs over W segments: one per run, or with more runs
// than segments one per segment boundary (only runs crossing a boundary have partials).
inline bool merge_by_boundary(int64_t runs, int64_t W) { return runs > W; }

struct Launch {
  char* out;
  const char* q;
  const char* kc;
  const char* vc;
  const int32_t* tables;
  const int32_t* ctx;
  int S, H, Hkv, maxb, nb, W, seg_fixed;
  int max_ctx;    // the caller's bound on the context lengths (the merge's guess)
  float sl;       // scale * k_scale * log2(e)
  float v_scale;
  char* ws;
  Layout lay;
  hipStream_t st;
  NewRows nr;  // fused new-token write when nr.k != nullptr
  Prefix pf;   // shared-prefix passes (mode 0: plain decode)
  bool defer_merge;  // partition only: the caller launches the merge
};

template <int KT, int QT, int D, int B, int GS, bool FUSED>
void launch_partition(const Launch& a, int64_t* hdr, int64_t* excl, float* part,
                      int64_t* split) {
  const int groups = (a.W + kWavesPerGroup - 1) / kWavesPerGroup;
  if constexpr ((GS == 4 || GS == 8) && KT == QT && (KT == PA_F16 || KT == PA_BF16))
    hipLaunchKernelGGL((decode_partition_mma<QT, D, B, GS, FUSED>), dim3(groups), dim3(kThreads),
                       0, a.st, a.out, a.q, a.kc, a.vc, a.tables, a.ctx, a.S, a.H, a.Hkv, a.maxb,
                       a.nb, a.W, a.seg_fixed, a.sl, a.v_scale, hdr, excl, part, split, a.nr,
                       a.nr.slots, a.pf);
  else
    hipLaunchKernelGGL((decode_partition<KT, QT, D, B, GS, FUSED>), dim3(groups), dim3(kThreads),
                       0, a.st, a.out, a.q, a.kc, a.vc, a.tables, a.ctx, a.S, a.H, a.Hkv, a.maxb,
                       a.nb, a.W, a.seg_fixed, a.sl, a.v_scale, hdr, excl, part, split, a.nr,
                       a.nr.slots, a.pf);
}

template <int KT, int QT, int D, int B, int GS>
bool launch(const Launch& a) {
  int64_t* hdr = reinterpret_cast<int64_t*>(a.ws);
  int64_t* excl = reinterpret_cast<int64_t*>(a.ws + a.lay.excl_off);
  float* part = reinterpret_cast<float*>(a.ws + a.lay.part_off);
  int64_t* split = reinterpret_cast<int64_t*>(a.ws + a.lay.split_off);
  if (a.nr.k) {
    // the fused write stores rows in the pools' own format: not for E4M3 pools, whose
    // new rows arrive in 16 bits and are quantized by pa_kv_write_fp8
    if constexpr (KT == QT) launch_partition<KT, QT, D, B, GS, true>(a, hdr, excl, part, split);
    else return false;
  } else {
    launch_partition<KT, QT, D, B, GS, false>(a, hdr, excl, part, split);
  }
  if (a.defer_merge) return true;
  const int64_t runs = (int64_t)a.S * (a.H / GS);
  const bool by_boundary = merge_by_boundary(runs, a.W);
  const int64_t mwaves = by_boundary ? a.W : runs;
  const int mgroups = (int)((mwaves + kWavesPerGroup - 1) / kWavesPerGroup);
  hipLaunchKernelGGL((decode_merge<QT, D, GS>), dim3(mgroups), dim3(kThreads), 0, a.st, a.out,
                     a.ctx, a.S, a.H, a.Hkv, a.maxb, B, a.W, a.v_scale, hdr, excl, part,
                     by_boundary ? split : (const int64_t*)nullptr, a.pf, a.max_ctx,
                     a.seg_fixed);
  return true;
}

template <int KT, int QT, int D, int B>
bool dispatch_gs(int GS, const Launch& a) {
  switch (GS) {
    case 1: return launch<KT, QT, D, B, 1>(a);
    case 2: return launch<KT, QT, D, B, 2>(a);
    case 4: return launch<KT, QT, D, B, 4>(a);
    case 8: return launch<KT, QT, D, B, 8>(a);
  }
  return false;
}

template <int KT, int QT, int D>
bool dispatch_b(int B, int GS, const Launch& a) {
  switch (B) {
    case 4: return dispatch_gs<KT, QT, D, 4>(GS, a);
    case 8: return dispatch_gs<KT, QT, D, 8>(GS, a);
    case 16: return dispatch_gs<KT, QT, D, 16>(GS, a);
    case 32: return dispatch_gs<KT, QT, D, 32>(GS, a);
  }
  return false;
}

template <int KT, int QT>
bool dispatch_d(int D, int B, int GS, const Launch& a) {
  if (D == 64) return dispatch_b<KT, QT, 64>(B, GS, a);
  if (D == 128) return dispatch_b<KT, QT, 128>(B, GS, a);
  return false;
}

}  // namespace decode_impl

// One instance per (key/value format, query/output format, head_dim), from decode_inst.hip.
#define PA_DECL_INST(kt, qt, d) \
  bool decode_launch_##kt##_##qt##_d##d(int B, int GS, const decode_impl::Launch& a);
PA_DECL_INST(PA_F32, PA_F32, 64)
PA_DECL_INST(PA_F32, PA_F32, 128)
PA_DECL_INST(PA_F16, PA_F16, 64)
PA_DECL_INST(PA_F16, PA_F16, 128)
PA_DECL_INST(PA_BF16, PA_BF16, 64)
PA_DECL_INST(PA_BF16, PA_BF16, 128)
PA_DECL_INST(PA_FP8_E4M3, PA_F16, 64)
PA_DECL_INST(PA_FP8_E4M3, PA_F16, 128)
PA_DECL_INST(PA_FP8_E4M3, PA_BF16, 64)
PA_DECL_INST(PA_FP8_E4M3, PA_BF16, 128)
#undef PA_DECL_INST

}  // namespace pagedkv
