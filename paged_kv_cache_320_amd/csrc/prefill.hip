// Prompt-phase (causal) attention over the paged cache on gfx950 matrix cores.
//
// What is computed: «The KV Cache and PagedAttention» › "One Token at a Time" — the
// prompt phase handles a text's whole prompt at once; each position's query attends
// the keys and values of every position up to and including its own (› "What It
// Does"; «KV cache» › "How it works"). The queries are the last n positions of a
// text, so a prompt may follow a cached prefix (› "What Came After") or recompute a
// text's cache in one go (› "When Memory Runs Out"). Keys and values, the prompt's
// own included, are read through the block table (› "The Block Table").
//
// How (design for MI355X): with up to thousands of queries per key this is a dense
// contraction, so both products run on the matrix cores (v_mfma_f32_32x32x16 for
// fp16 and bf16, fp32 accumulation).
//  * A workgroup of 4 waves takes 128 consecutive queries of one (text, head); wave w
//    holds queries 32w..32w+31 as the 32 columns of its MFMA tiles.
//  * Keys stream in tiles of 64 positions, double-buffered in LDS. gfx950's LDS DMA
//    (global_load_lds_dwordx4) moves each 16-byte piece of a tile's keys and values
//    from its block straight into LDS, without a trip through registers, while the
//    previous tile is being multiplied. Rows past the last position any query of the
//    workgroup needs repeat that position (finite, and given no weight).
//  * A DMA writes a wave's 64 pieces to 1 KiB of consecutive LDS, so conflict-free
//    operand reads come from an XOR swizzle of the 16-byte pieces within a row instead
//    of row padding.
//  * S^T = K Q^T puts keys on the rows and queries on the columns, so a lane holds
//    16 scores of one query and its partner lane (lane ^ 32) the other 16: the row
//    maximum and sum need one exchange between the pair, no wider reduction.
//  * Online softmax in the exp2 domain (scale * log2(e) folded in). The weights are
//    rounded to the input format and O^T += V^T P^T runs on MFMA; the order in which
//    each lane holds its scores is the order of the P^T operand's k index, so the
//    weights never leave their registers. V^T comes from the row-major value tile
//    through gfx950's transposing LDS read (two reads per MFMA operand).
//  * Waves whose queries all precede a key tile skip its arithmetic (causal skip);
//    the longest query tiles of a text are dispatched first.
#include "device.hpp"

#include <cmath>

namespace pagedkv {
namespace prefill_impl {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQRows = 32 * kWaves;  // queries per workgroup
constexpr int kKeys = 64;            // key positions per tile (two 32-key MFMA subtiles)
constexpr int kSub = kKeys / 32;     // 32-key subtiles per tile

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DT>
struct Mma;

template <>
struct Mma<PA_F16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static constexpr float kSlack = 8.f;  // log2 of the largest softmax weight held
  // two fp32 -> two fp16 in one word (round to nearest even), first in the low half
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){x, y}, h2));
  }
};

template <>
struct Mma<PA_BF16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static constexpr float kSlack = 0.f;
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){x, y}, b2));
  }
};

// Key position held in accumulator register r of a lane in half `half` (0: lanes 0-31,
// 1: lanes 32-63) of the 32x32 MFMA output, relative to the tile.
__device__ __forceinline__ int key_of(int r, int half) { return (r >> 2) * 8 + half * 4 + (r & 3); }

// LDS tile layout: key or value row r (of kKeys) holds D 16-bit elements as CPR = D / 8
// pieces of 16 bytes; logical piece c of row r sits in slot c ^ swz(r). LDS has 64 banks
// of 4 bytes, so a piece's bank group (of 16) is (r * CPR + slot) mod 16.
//  * Keys: a 16-lane key-operand read takes one piece p of rows r0 .. r0 + 15. With
//    swz(r) = r mod 16 (D = 128) or (r / 2) mod 8 (D = 64, where odd rows already sit
//    8 groups further) the 16 rows land in 16 distinct bank groups.
//  * Values: a 32-lane half of a transposing read takes pieces 4m .. 4m + 3 of rows
//    r0 .. r0 + 3 (r0 a multiple of 4). With swz(r) = 4 (r mod 4) (D = 128) or
//    4 ((r / 2) mod 2) (D = 64) the 4 rows take 4 disjoint groups of 4: 16 distinct.
template <int CPR>
__device__ __forceinline__ int swz_k(int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & 7); }
template <int CPR>
__device__ __forceinline__ int swz_v(int r) { return CPR == 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// A operand of O^T += V^T P^T for 32-key subtile st, 32-row tile mt and k-step kk: lane l
// needs V[key_of(8 kk + j, l / 32)][32 mt + l % 32] for j = 0..7. gfx950's
// ds_read_b64_tr_b16 reads, per group of 16 lanes, the 4 x 16-bit pieces that lane j of
// the group addresses and hands lane i element i % 4 of lane 4k + i / 4's piece as its
// value k. So lane j of a group addresses key (its value k = j / 4) at dims 4 (j % 4) ..
// +3 of the group's 16 dims, and lane i receives 4 keys at dim (group base) + i. Two
// reads give the 8 keys: 16 kk + 4 half + (0..3), then the same + 8.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Element offset, within a value tile, of the piece lane `lane` addresses for 32-row tile mt
// of subtile 0, k-step 0: the lane's key there is 4 (grp / 2) + j / 4, whose swizzle
// (depending on key mod 4, or (key / 2) mod 2 for D = 64) is the same for every subtile,
// k-step and the +8 key of the second read, which therefore only add (32 st + 16 kk [+ 8]) D
// elements. Computed once per lane (the per-read address then costs no arithmetic).
template <int D>
__device__ __forceinline__ int v_offset(int mt, int lane) {
  constexpr int CPR = D / 8;
  const int grp = lane >> 4, j = lane & 15;
  const int dim = 32 * mt + 16 * (grp & 1) + 4 * (j & 3);
  const int key = 4 * (grp >> 1) + (j >> 2);
  return key * D + (((dim >> 3) ^ swz_v<CPR>(key)) << 3) + (dim & 7);
}

// The two transposing reads of one A operand: keys `key0` and key0 + 8 relative to the
// lane's offset; the two 64-bit results are the operand's four words as they come.
template <int D>
__device__ __forceinline__ u32x4 vt_operand(const uint16_t* vs, int voff, int key0) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vs + voff + key0 * D));
  const s16x4 b =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vs + voff + (key0 + 8) * D));
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  return u32x4{ua.x, ua.y, ub.x, ub.y};
}

// gfx950 LDS DMA: each lane's 16 bytes from `src` land at lds + 16 * lane (lds must be
// the same for every lane of the wave).
__device__ __forceinline__ void dma16(const char* src, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

template <int DT, int D, int B>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(
    char* __restrict__ out, const char* __restrict__ q, const char* __restrict__ kc,
    const char* __restrict__ vc, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ ctx, const int32_t* __restrict__ q_start, int T, int H, int Hkv,
    int maxb, int num_blocks, int qtiles, int nwork, int round_robin, float scale_log2) {
  using M = Mma<DT>;
  typedef typename M::v8 v8;
  constexpr int CPR = D / 8;                     // 16-byte pieces per key row
  constexpr int NQ = D / 16;                     // MFMA k-steps of S^T
  constexpr int NM = D / 32;                     // 32-row tiles of O^T
  constexpr int NI = kKeys * CPR / 64 / kWaves;  // DMAs per wave, tensor and tile
  static_assert(NI * 64 * kWaves == kKeys * CPR, "tile copy must cover the tile exactly");
  // Two named buffers rather than one indexed array: the compiler then sees that the
  // next tile's DMA never writes what this tile's operand reads read, and does not make
  // those reads wait for it.
  __shared__ __align__(16) uint16_t k0[kKeys * D], k1[kKeys * D];  // two buffers: compute
  __shared__ __align__(16) uint16_t v0[kKeys * D], v1[kKeys * D];  // one tile, load the next

  __shared__ int bad_sh;

  // Work item = (text, head, query tile), a unit being a text's key/value head with the
  // Gr query heads it serves. Workgroups are dealt to the 8 XCDs in turn (workgroup b to
  // XCD b % 8), and each XCD walks its items in order (a unit's heads, each head's longest
  // query tiles first), so the heads sharing a key/value head run on one XCD, whose L2 then
  // serves their keys and values. Prompts of equal length: XCD x takes the x-th contiguous
  // eighth of the units. Unequal lengths (round_robin): unit u goes to XCD u % 8, so every
  // XCD gets an even share of every text's heads and no XCD holds the longest prompts
  // alone (on 64 prompts of 16-2,048 tokens the contiguous dealing left one XCD ~1.4x the
  // mean work).
  const int Gr = H / Hkv;
  const int per_unit = Gr * qtiles;
  const int units = nwork / per_unit;  // texts x key/value heads
  const int upx = (units + 7) >> 3;    // units per XCD
  const int rank = (int)(blockIdx.x >> 3);
  const int ui = rank / per_unit;
  const int x = (int)(blockIdx.x & 7);
  const int u = round_robin ? x + 8 * ui : x * upx + ui;
  if (ui >= upx || u >= units) return;
  const int rem = rank - ui * per_unit;
  // a head's query tiles longest first, in snake order over groups of four of the XCD's
  // workgroups (15 14 13 12, 8 9 10 11, 7 6 5 4, 0 1 2 3 for 16 tiles; heads of 4 tiles
  // alternate direction): an XCD starts its workgroups on its shader engines in turn, and
  // in plain descending order engine k would always get the k-th longest of every four
  // tiles (40 : 36 : 32 : 28 of the work for 16 tiles); this way each engine gets the same
  // share. Only where a unit's items come in whole groups of four (else plain order).
  int d = rem;
  if ((per_unit & 3) == 0 && ((rank >> 2) & 1)) d = (rem & ~3) + 3 - (rem & 3);
  const int qt0 = qtiles - 1 - d % qtiles;
  const int s = u / Hkv;
  const int kvh = u - s * Hkv;
  const int h = kvh * Gr + d / qtiles;
  const int r0 = q_start[s], r1 = q_start[s + 1];
  const int n = r1 - r0;
  if (r0 < 0 || r1 > T || n <= 0) return;  // no rows of `out` to write
  int L = ctx[s];
  const int64_t cap = (int64_t)maxb * B;
  const bool bad_shape = L < n || (int64_t)L > cap;
  if ((int64_t)L > cap) L = (int)cap;
  const int first = L - n;  // position of the text's first query

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int col = lane & 31, half = lane >> 5;
  const int32_t* trow = tables + (int64_t)s * maxb;
  if (tid == 0) bad_sh = 0;
  __syncthreads();  // cleared before any tile load can set it

  for (int qt = qt0; qt * kQRows < n; qt += qtiles) {
    const int row_lo = qt * kQRows;
    const int row_hi = min(n, row_lo + kQRows);
    const int kv_end = first + row_hi;           // positions [0, kv_end) are needed
    const int kv_lim = min(kv_end, L);
    const int wrow0 = row_lo + wave * 32;
    const bool wave_on = wrow0 < row_hi;
    const int wave_last = first + min(row_hi, wrow0 + 32) - 1;
    const int row = wrow0 + col;
    const bool row_ok = row < row_hi;
    const int pos = row_ok ? first + row : -1;   // -1 attends nothing

    // LDS element offsets of this lane's operand reads (fixed for the whole loop): key
    // operand of k-step c (subtile 1 adds 32 D), value operand of 32-row tile mt
    int koff[NQ], voff[NM];
#pragma unroll
    for (int c = 0; c < NQ; ++c) koff[c] = col * D + (((2 * c + half) ^ swz_k<CPR>(col)) * 8);
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) voff[mt] = v_offset<D>(mt, lane);

    // queries: lane holds q[row][16c + 8 half .. +7] for k-step c
    v8 qv[NQ];
    {
      const char* qp = q + ((int64_t)(r0 + (row_ok ? row : row_lo)) * H + h) * (D * 2);
#pragma unroll
      for (int c = 0; c < NQ; ++c) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row_ok) x = *(const u32x4*)(qp + (16 * c + 8 * half) * 2);
        qv[c] = __builtin_bit_cast(v8, x);
      }
    }
    f32x16 o[NM];
#pragma unroll
    for (int mt = 0; mt < NM; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[mt][r] = 0.f;
    float m = -INFINITY, l = 0.f;

    const int ntiles = kv_end > 0 ? (kv_end + kKeys - 1) / kKeys : 0;
    const int wave_first = first + wrow0;  // position of the wave's first query
    const int kv_last = max(kv_lim - 1, 0);
    // A wave moves rows 16 wave .. 16 wave + 15 of every tile. With block_size >= 16 they lie
    // in one block: one table entry per wave and tile (a scalar), and each lane's offset in
    // the (block, head) tile is fixed but for rows past the last needed position, which
    // re-read that position. Smaller blocks take one entry per lane and load.
    constexpr bool kWaveBlock = B >= 16;
    static_assert(NI * 64 == 16 * CPR, "a wave moves 16 rows of each tile");
    int tb[NI];
    int tbw = 0;
    auto load_table = [&](int kt) {
      if constexpr (kWaveBlock) {
        tbw = trow[min(kt * kKeys + 16 * wave, kv_last) / B];
      } else {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int row = ((wave * NI + j) * 64 + lane) / CPR;
          tb[j] = trow[min(kt * kKeys + row, kv_last) / B];
        }
      }
    };
    bool bad = false;
    auto dma = [&](int kt, uint16_t* kd, uint16_t* vd) {
      // every address first (the table entries arrived during the previous tile), so
      // no wait for a table entry falls between two tile loads
      const char* ksrc[NI];
      const char* vsrc[NI];
      if constexpr (kWaveBlock) {
        const int pos0 = kt * kKeys + 16 * wave;
        const bool out_of_pool = (unsigned)tbw >= (unsigned)num_blocks;
        bad |= out_of_pool && pos0 < kv_lim;
        const int64_t tile_off = ((int64_t)(out_of_pool ? 0 : tbw) * Hkv + kvh) * (B * D * 2);
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int r = (j * 64 + lane) / CPR, slot = (j * 64 + lane) % CPR;
          const int row = 16 * wave + r;
          const uint32_t in_tile = (uint32_t)(min(pos0 + r, kv_last) & (B - 1)) * (D * 2);
          ksrc[j] = kc + tile_off + (in_tile + (uint32_t)((slot ^ swz_k<CPR>(row)) * 16));
          vsrc[j] = vc + tile_off + (in_tile + (uint32_t)((slot ^ swz_v<CPR>(row)) * 16));
        }
      } else {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int chunk = (wave * NI + j) * 64 + lane;
          const int row = chunk / CPR, slot = chunk % CPR;
          const int kp = kt * kKeys + row;
          const bool out_of_pool = (unsigned)tb[j] >= (unsigned)num_blocks;
          bad |= out_of_pool && kp < kv_lim;
          const int blk = out_of_pool ? 0 : tb[j];
          const int64_t off = (((int64_t)blk * Hkv + kvh) * B + min(kp, kv_last) % B) * (D * 2);
          ksrc[j] = kc + off + ((slot ^ swz_k<CPR>(row)) * 16);
          vsrc[j] = vc + off + ((slot ^ swz_v<CPR>(row)) * 16);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        dma16(ksrc[j], kd + (wave * NI + j) * 512);
        dma16(vsrc[j], vd + (wave * NI + j) * 512);
      }
    };
    auto tile = [&](int kt, const uint16_t* kb, const uint16_t* vb, uint16_t* kn, uint16_t* vn) {
      dma(kt + 1, kn, vn);
      load_table(kt + 2);
      if (wave_on && kt * kKeys <= wave_last) {  // causal skip (wave-uniform)
        // S^T = K Q^T per 32-key subtile: A = 32 keys x 16 dims from LDS, B = the wave's
        // queries; the subtiles' products are independent, so they overlap
        // (the swizzle of row 32 st + col equals that of row col, so subtile st's pieces
        // sit 32 D elements after subtile 0's; the first product starts from zero)
        // The key operands of k-step c + 1 are read while the products of step c run, so
        // the LDS latency is not paid before every pair of products.
        f32x16 sacc[kSub];
        u32x4 ka[2][kSub];
#pragma unroll
        for (int st = 0; st < kSub; ++st) ka[0][st] = *(const u32x4*)(kb + koff[0] + 32 * st * D);
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
          if (c + 1 < NQ) {
#pragma unroll
            for (int st = 0; st < kSub; ++st)
              ka[(c + 1) & 1][st] = *(const u32x4*)(kb + koff[c + 1] + 32 * st * D);
          }
#pragma unroll
          for (int st = 0; st < kSub; ++st)
            sacc[st] = M::mfma(__builtin_bit_cast(v8, ka[c & 1][st]), qv[c],
                               c == 0 ? f32x16{} : sacc[st]);
        }
        // keep that order (the scheduler would otherwise sink each read next to its use):
        // the reads of steps 0 and 1, then per step its two products and the next reads
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kSub, 0);
#pragma unroll
        for (int c = 0; c + 2 < NQ; ++c) {
          __builtin_amdgcn_sched_group_barrier(0x008, kSub, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, kSub, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * kSub, 0);
        // raw scores (scale_log2 > 0 keeps their order); on a diagonal tile, keys after
        // a query's own position get no weight
        if (kt * kKeys + kKeys - 1 > wave_first) {
#pragma unroll
          for (int st = 0; st < kSub; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kt * kKeys + 32 * st + key_of(r, half) > pos) sacc[st][r] = -INFINITY;
        }
        float tmax = sacc[0][0];
#pragma unroll
        for (int st = 0; st < kSub; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[st][r]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * scale_log2;
        // fp16 weights: the reference maximum m moves only when a score exceeds it by
        // more than 2^8 (or on the first key), so weights stay below 256 and most tiles
        // skip the rescaling of the accumulators; any reference gives the same result
        // in exact arithmetic, since l and O are scaled alike. bf16 weights (8-bit
        // significand): m is the exact running maximum, so the largest weight is 1 and
        // exact, and rounding touches only the smaller ones.
        const bool move = tmax > m + M::kSlack;
        if (__any(move)) {
          const float m_new = move ? tmax : m;
          const float alpha = fast_exp2(m - m_new);  // m = -inf: 0
          l *= alpha;
#pragma unroll
          for (int mt = 0; mt < NM; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[mt][r] *= alpha;
          m = m_new;
        }
        const float m_use = m == -INFINITY ? 0.f : m;
        float psum = 0.f;
#pragma unroll
        for (int st = 0; st < kSub; ++st) {
          // V^T operands of this subtile first (rows d = 32 mt + col over its keys, through
          // the transposing LDS read), held back by a scheduling barrier so that they
          // arrive while the weights below are formed, instead of each read being sunk next
          // to its product
          u32x4 va[NM][2];
#pragma unroll
          for (int mt = 0; mt < NM; ++mt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
              va[mt][kk] = vt_operand<D>(vb, voff[mt], 32 * st + 16 * kk);
          __builtin_amdgcn_sched_barrier(0);
          // P^T operand of k-step kk: the lane's scores r = 8kk .. 8kk+7 (keys
          // 32 st + key_of(r, half))
          v8 pb[2];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            float z[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              z[j] = fast_exp2(__builtin_fmaf(sacc[st][8 * kk + j], scale_log2, -m_use));
              psum += z[j];
            }
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = M::pack2(z[2 * j], z[2 * j + 1]);
            pb[kk] = __builtin_bit_cast(v8, w);
          }
          // O^T += V^T P^T: A = V^T rows d = 32 mt + col over the same 8 keys per k-step
#pragma unroll
          for (int mt = 0; mt < NM; ++mt) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
              o[mt] = M::mfma(__builtin_bit_cast(v8, va[mt][kk]), pb[kk], o[mt]);
          }
        }
        l += psum;
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // the next tile is in LDS; this one is no longer read
    };
    load_table(0);
    dma(0, k0, v0);
    load_table(1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < ntiles; kt += 2) {
      tile(kt, k0, v0, k1, v1);
      if (kt + 1 < ntiles) tile(kt + 1, k1, v1, k0, v0);
    }
    if (bad) bad_sh = 1;
    __syncthreads();
    const float lt = l + __shfl_xor(l, 32);
    float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (bad_shape || bad_sh) inv = __builtin_nanf("");
    if (row_ok) {
      char* op = out + ((int64_t)(r0 + row) * H + h) * (D * 2);
#pragma unroll
      for (int mt = 0; mt < NM; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * mt + 8 * g + 4 * half;  // registers 4g..4g+3: dims d..d+3
          uint2 w;
          w.x = M::pack2(o[mt][4 * g] * inv, o[mt][4 * g + 1] * inv);
          w.y = M::pack2(o[mt][4 * g + 2] * inv, o[mt][4 * g + 3] * inv);
          *(uint2*)(op + d * 2) = w;
        }
    }
  }
}

struct Args {
  char* out;
  const char *q, *kc, *vc;
  const int32_t *tables, *ctx, *q_start;
  int S, T, H, Hkv, maxb, num_blocks, qtiles, nwork, round_robin;
  float scale_log2;
  hipStream_t st;
};

template <int DT, int D, int B>
void launch(const Args& a) {
  // 8 XCDs x the units each is dealt (ceil(units / 8)) x the items of a unit
  const int64_t per_unit = (int64_t)(a.H / a.Hkv) * a.qtiles;
  const int64_t units = (int64_t)a.S * a.Hkv;
  const dim3 grid((unsigned)(8 * ((units + 7) / 8) * per_unit)), block(kThreads);
  hipLaunchKernelGGL((prefill_kernel<DT, D, B>), grid, block, 0, a.st, a.out, a.q, a.kc, a.vc,
                     a.tables, a.ctx, a.q_start, a.T, a.H, a.Hkv, a.maxb, a.num_blocks,
                     a.qtiles, a.nwork, a.round_robin, a.scale_log2);
}

template <int DT, int D>
void launch_b(int B, const Args& a) {
  switch (B) {
    case 4: launch<DT, D, 4>(a); break;
    case 8: launch<DT, D, 8>(a); break;
    case 16: launch<DT, D, 16>(a); break;
    default: launch<DT, D, 32>(a); break;
  }
}

template <int DT>
void launch_d(int D, int B, const Args& a) {
  if (D == 64) launch_b<DT, 64>(B, a);
  else launch_b<DT, 128>(B, a);
}

}  // namespace prefill_impl
}  // namespace pagedkv

using namespace pagedkv;

extern "C" int pa_prefill_attention(void* out, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, const int32_t* q_start,
                                    int32_t num_seqs, int32_t num_rows, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, int32_t max_blocks_per_seq,
                                    int32_t max_q_len, float scale, int32_t dtype, void* stream) {
  using namespace prefill_impl;
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_EUNSUPPORTED, "prefill dtype %d (supported: PA_F16, PA_BF16)", dtype);
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
  if (num_heads > 65535) return fail(PA_EINVAL, "num_heads %d > 65535", num_heads);
  if (num_rows < 0 || max_q_len < 0) return fail(PA_EINVAL, "num_rows and max_q_len must be >= 0");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(PA_EINVAL, "scale must be finite and > 0");
  if (num_rows == 0 || max_q_len == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !q_start)
    return fail(PA_EINVAL, "null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_EINVAL, "out, q and pools must be 16-byte aligned");
  if (((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u) ||
      ((uintptr_t)q_start & 3u))
    return fail(PA_EINVAL, "tables, context_lens and q_start must be 4-byte aligned");
  const int64_t qtiles = ((int64_t)max_q_len + kQRows - 1) / kQRows;
  if (((int64_t)num_seqs * num_kv_heads + 7) * (num_heads / num_kv_heads) * qtiles > 0x7ffffff0LL)
    return fail(PA_EINVAL, "num_seqs * num_heads * ceil(max_q_len / %d) exceeds the grid",
                kQRows);
  const Args a{(char*)out, (const char*)q, (const char*)k_cache, (const char*)v_cache,
               block_tables, context_lens, q_start, num_seqs, num_rows, num_heads,
               num_kv_heads, max_blocks_per_seq, num_blocks, (int)qtiles,
               (int)(num_seqs * num_heads * qtiles),
               // every prompt max_q_len long exactly when the rows add up to that
               (int64_t)num_rows != (int64_t)num_seqs * max_q_len,
               scale * 1.4426950408889634f, (hipStream_t)stream};
  if (dtype == PA_F16) launch_d<PA_F16>(head_dim, block_size, a);
  else launch_d<PA_BF16>(head_dim, block_size, a);
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}
