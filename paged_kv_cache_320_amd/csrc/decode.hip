// C entry points of paged decode attention: argument checks, workspace layout and
// the choice of kernel instance. The kernels are in decode_kernels.hpp.
#include "decode_kernels.hpp"

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

namespace pagedkv {
namespace {

using decode_impl::kChunk;
using decode_impl::kHdrBytes;
using decode_impl::kMaxGS;
using decode_impl::kWavesPerCU;
using decode_impl::Launch;
using decode_impl::Layout;
using decode_impl::units_of;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// wpc: segments per compute unit of an auto grid (partition_tokens 0).
int layout(int32_t S, int32_t H, int32_t D, int32_t max_ctx, int32_t T, Layout* lay,
           int wpc = kWavesPerCU) {
  if (S < 1 || H < 1 || (D != 64 && D != 128) || max_ctx < 0 || T < 0 || T % kChunk != 0)
    return fail(PA_EINVAL, "bad workspace shape (num_seqs %d, num_heads %d, head_dim %d, "
                "max_context_len %d, partition_tokens %d)", S, H, D, max_ctx, T);
  // runs per text are at most H (one query head per wave), so this bounds every GS; a
  // device-side length beyond max_ctx lengthens the segments (seg::segment_units)
  const int64_t units_bound = (int64_t)S * H * units_of(max_ctx);
  int64_t slots = 0;
  if (T == 0) {
    int cus = 0;
    int rc = device_cus(&cus);
    if (rc != PA_OK) return rc;
    slots = (int64_t)cus * wpc;
  }
  const int64_t W = pagedkv::seg::grid_segments(units_bound, slots, T / kChunk);
  if (W > 0x7fffffff / 2) return fail(PA_EINVAL, "too many segments");
  lay->W = W;
  lay->excl_off = kHdrBytes;
  lay->split_off = align256(lay->excl_off + sizeof(int64_t) * (size_t)S);
  lay->part_off = align256(lay->split_off + sizeof(int64_t) * (size_t)W);
  lay->bytes = align256(lay->part_off + sizeof(float) * (size_t)W * 2 * kMaxGS * (D + 4));
  return PA_OK;
}

// Query heads served per wave: the largest of 8, 4, 2, 1 dividing num_heads / num_kv_heads.
int heads_per_wave(int G) {
  for (int gs = kMaxGS; gs > 1; gs /= 2)
    if (G % gs == 0) return gs;
  return 1;
}

__global__ void zero_fill_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
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

namespace {

// Shared checks and launch of the decode entry points. kv_dtype is the pools' format,
// q_dtype that of q and out.
int decode_common(void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                  int32_t partition_tokens, float scale, float k_scale, float v_scale,
                  int32_t kv_dtype, int32_t q_dtype, void* workspace, size_t workspace_bytes,
                  void* stream, const decode_impl::NewRows& nr = decode_impl::NewRows{},
                  const decode_impl::Prefix& pf = decode_impl::Prefix{},
                  int wpc = kWavesPerCU, bool defer_merge = false) {
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
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !(k_scale > 0.f) || !(v_scale > 0.f))
    return fail(PA_EINVAL, "k_scale and v_scale must be finite and > 0");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !workspace)
    return fail(PA_EINVAL, "null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(workspace))
    return fail(PA_EINVAL, "out, q, pools and workspace must be 16-byte aligned");
  if (((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u))
    return fail(PA_EINVAL, "tables and context_lens must be 4-byte aligned");
  Layout lay;
  int rc = layout(num_seqs, num_heads, head_dim, max_context_len, partition_tokens, &lay, wpc);
  if (rc != PA_OK) return rc;
  if (workspace_bytes < lay.bytes)
    return fail(PA_EINVAL, "workspace_bytes %zu < %zu required", workspace_bytes, lay.bytes);
  const Launch a{(char*)out, (const char*)q, (const char*)k_cache, (const char*)v_cache,
                 block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                 max_blocks_per_seq, num_blocks, (int)lay.W, partition_tokens / kChunk,
                 max_context_len,
                 // scale * k_scale * log2(e): scores in the exp2 domain, key scale folded in
                 scale * k_scale * 1.4426950408889634f, v_scale,
                 (char*)workspace, lay, (hipStream_t)stream, nr, pf, defer_merge};
  const int GS = heads_per_wave(num_heads / num_kv_heads);
  bool done = false;
  const bool d64 = head_dim == 64;
  const int B = block_size;
  if (kv_dtype == PA_FP8_E4M3 && q_dtype == PA_F16)
    done = d64 ? decode_launch_PA_FP8_E4M3_PA_F16_d64(B, GS, a)
               : decode_launch_PA_FP8_E4M3_PA_F16_d128(B, GS, a);
  else if (kv_dtype == PA_FP8_E4M3 && q_dtype == PA_BF16)
    done = d64 ? decode_launch_PA_FP8_E4M3_PA_BF16_d64(B, GS, a)
               : decode_launch_PA_FP8_E4M3_PA_BF16_d128(B, GS, a);
  else if (kv_dtype == PA_F32)
    done = d64 ? decode_launch_PA_F32_PA_F32_d64(B, GS, a) : decode_launch_PA_F32_PA_F32_d128(B, GS, a);
  else if (kv_dtype == PA_F16)
    done = d64 ? decode_launch_PA_F16_PA_F16_d64(B, GS, a) : decode_launch_PA_F16_PA_F16_d128(B, GS, a);
  else if (kv_dtype == PA_BF16)
    done = d64 ? decode_launch_PA_BF16_PA_BF16_d64(B, GS, a)
               : decode_launch_PA_BF16_PA_BF16_d128(B, GS, a);
  if (!done) return fail(PA_EUNSUPPORTED, "no kernel for this shape");
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}

}  // namespace

extern "C" int pa_decode_attention(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_context_len,
                                   int32_t partition_tokens, float scale, int32_t dtype,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return fail(PA_EINVAL, "dtype %d is not PA_F32/PA_F16/PA_BF16", dtype);
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, partition_tokens, scale, 1.0f, 1.0f, dtype, dtype,
                       workspace, workspace_bytes, stream);
}

extern "C" int pa_decode_attention_fp8(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       int32_t partition_tokens, float scale, float k_scale,
                                       float v_scale, int32_t q_dtype, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (q_dtype != PA_F16 && q_dtype != PA_BF16)
    return fail(PA_EUNSUPPORTED, "q_dtype %d: E4M3 pools take PA_F16 or PA_BF16 queries", q_dtype);
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, partition_tokens, scale, k_scale, v_scale, PA_FP8_E4M3,
                       q_dtype, workspace, workspace_bytes, stream);
}

namespace pagedkv {
namespace {

// Debug re-check of the fused write's promise: each text's slot (when inside the pool) is
// the place of its last attended position in its table, and no two texts share a slot.
int check_new_slots(const int64_t* slots, const int32_t* tables, const int32_t* ctx, int32_t S,
                    int32_t maxb, int32_t B, int32_t num_blocks, hipStream_t st) {
  int rc = check_slots(slots, S, (int64_t)num_blocks * B, st);
  if (rc != PA_OK) return rc;
  std::vector<int64_t> sl;
  std::vector<int32_t> tab, len;
  if ((rc = fetch(sl, slots, (size_t)S, st)) != PA_OK) return rc;
  if ((rc = fetch(tab, tables, (size_t)S * maxb, st)) != PA_OK) return rc;
  if ((rc = fetch(len, ctx, (size_t)S, st)) != PA_OK) return rc;
  for (int32_t s = 0; s < S; ++s) {
    if (sl[s] < 0 || sl[s] >= (int64_t)num_blocks * B || len[s] < 1) continue;
    const int64_t p = len[s] - 1;
    if (p / B >= maxb) continue;  // the decode poisons such a text
    const int64_t want = (int64_t)tab[(int64_t)s * maxb + p / B] * B + p % B;
    if (sl[s] != want)
      return fail(PA_EINVAL, "debug check: text %d writes slot %lld, but its last position "
                  "%lld sits at slot %lld of its table", s, (long long)sl[s], (long long)p,
                  (long long)want);
  }
  return PA_OK;
}

}  // namespace
}  // namespace pagedkv

extern "C" int pa_decode_attention_write(void* out, const void* q, void* k_cache, void* v_cache,
                                         const void* k_new, const void* v_new,
                                         const int64_t* slots, const int32_t* block_tables,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                         int32_t max_blocks_per_seq, int32_t max_context_len,
                                         int32_t partition_tokens, float scale, int32_t dtype,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return fail(PA_EINVAL, "dtype %d is not PA_F32/PA_F16/PA_BF16", dtype);
  if (!k_new || !v_new || !slots) return fail(PA_EINVAL, "null pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || ((uintptr_t)slots & 7u))
    return fail(PA_EINVAL, "k_new and v_new must be 16-byte aligned, slots 8-byte aligned");
  if (debug_checks() && block_tables && context_lens && num_seqs > 0 && max_blocks_per_seq > 0 &&
      num_blocks > 0 && block_size > 0) {
    const int rc = check_new_slots(slots, block_tables, context_lens, num_seqs,
                                   max_blocks_per_seq, block_size, num_blocks,
                                   (hipStream_t)stream);
    if (rc != PA_OK) return rc;
  }
  const decode_impl::NewRows nr{(const char*)k_new, (const char*)v_new, slots, (char*)k_cache,
                                (char*)v_cache};
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, partition_tokens, scale, 1.0f, 1.0f, dtype, dtype,
                       workspace, workspace_bytes, stream, nr);
}

// ---- decode with the library's own workspace ---------------------------------------
//
// For callers that cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc): the workspace is a file-scope device array, one
// copy per GPU, held until the process ends. Calls on one GPU share it.

namespace pagedkv {

constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kScratchDevices = 64;

// Workspace of pa_decode_attention_noalloc. Host code must not pass this name to a kernel
// (on the host it is only a stand-in for the symbol): scratch_address() gives the device
// address of the current GPU's copy.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex scratch_mu;
void* scratch_ptr[kScratchDevices];

// The current GPU's copy of `scratch`, looked up once per device with that device current.
int scratch_address(void** out) {
  int dev = 0;
  PA_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kScratchDevices)
    return fail(PA_EUNSUPPORTED, "device %d: the built-in workspace serves devices 0..%d", dev,
                kScratchDevices - 1);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    PA_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(PA_EHIP, "hipGetSymbolAddress gave a null address for the workspace");
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return PA_OK;
}

}  // namespace
}  // namespace pagedkv

extern "C" size_t pa_decode_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int pa_decode_attention_noalloc(void* out, const void* q, const void* k_cache,
                                           const void* v_cache, const int32_t* block_tables,
                                           const int32_t* context_lens, int32_t num_seqs,
                                           int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, int32_t max_blocks_per_seq,
                                           int32_t max_context_len, int32_t partition_tokens,
                                           float scale, int32_t dtype, void* stream) {
  if (!dtype_ok(dtype)) return fail(PA_EINVAL, "dtype %d is not PA_F32/PA_F16/PA_BF16", dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  Layout lay;
  int rc = layout(num_seqs, num_heads, head_dim, max_context_len, partition_tokens, &lay);
  if (rc != PA_OK) return rc;
  if (lay.bytes > kScratchBytes)
    return fail(PA_EINVAL, "this launch needs %zu bytes of workspace, more than the %zu of the "
                "built-in one (fewer texts, partition_tokens 0, or pa_decode_attention with a "
                "workspace)", lay.bytes, kScratchBytes);
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != PA_OK) return rc;
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, partition_tokens, scale, 1.0f, 1.0f, dtype, dtype, ws,
                       kScratchBytes, stream);
}

// ---- decode over shared prompt blocks --------------------------------------------
//
// Texts forked from one prompt (parallel sampling, beam search) hold the prompt's blocks
// in common, and a plain decode reads those blocks once per text. Here the shared blocks
// are read once per group: pass 1 attends every member's queries to the group's shared
// blocks at once (the members' heads as the query heads of one key/value head, up to 8)
// and keeps each member's (m, l, acc); pass 2 attends each text to its own blocks only
// and folds that state in. Softmax over the union of the two token sets is the same
// softmax, merged as the split-context partials are.

namespace pagedkv {
namespace {

constexpr int kPrefixCols = 8;  // query heads per key/value head in a shared-blocks pass, at most

// Workspace of the shared-prefix decode: the decode workspace (sized for the largest of the
// outer level's pass and the own pass), with two levels a second one for the inner level's
// pass (both levels' partials are merged in one launch after both passes), then per level the
// texts' states [S][H][D + 4] and starts [S], and the level's group arrays and table rows. The set-up writes the starts, group arrays, table rows and
// outer groups (the plan); the passes write the decode workspace and the states.
struct PrefixLevel {
  size_t state_off, start_off, vfirst_off, vcount_off, vctx_off, vtab_off;
  int maxbp;  // table entries per group (shared blocks at most)
};
struct PrefixLayout {
  size_t decode_bytes, bytes;
  size_t decode1_off, decode1_bytes;  // two levels: the inner level's decode workspace
  size_t gid_off;  // two levels: each text's outer group (-1: none) [S]
  int levels;
  PrefixLevel lv[2];
};

// Segments per compute unit of one pass of the shared-block decode, whose key/value heads
// each serve G query heads: the matrix-core kernel (4 or 8 query heads per wave, 16-bit
// formats) keeps 4; the vector kernel takes 16 for two heads a wave (a group's columns: the
// forked pairs' blocks, runs of ~17 chunks; 16 is the most that stay resident at 104
// VGPRs) and 8 otherwise (the texts' own blocks, runs of one or two chunks, where more
// segments mostly add partials). On the 32 x 8 sharing workload (bf16): 8 took the pairs'
// pass from 162 to 142 us and the own pass from 24 to 20 us; 16 for both took the op from
// 323-327 to 317-320 us (12: no change), and 8 again for the own pass to 312-315 us. (The
// matrix-core prompts pass went from 128 to 136 us with 8.)
int pass_waves(int G, int32_t elt) {
  const int gs = heads_per_wave(G);
  if (gs >= 4 && elt == 2) return kWavesPerCU;
  return gs == 2 ? 4 * kWavesPerCU : 2 * kWavesPerCU;
}

int prefix_layout(int32_t S, int32_t H, int32_t Hkv, int32_t D, int32_t max_ctx, int32_t levels,
                  const int32_t* V, const int32_t* max_prefix, const int32_t* cols, int32_t bsz,
                  int32_t elt, PrefixLayout* pl) {
  if (Hkv < 1 || H % Hkv != 0 || bsz < 1 || levels < 1 || levels > 2)
    return fail(PA_EINVAL, "bad shared-prefix shape (num_heads %d, num_kv_heads %d, "
                "block_size %d)", H, Hkv, bsz);
  for (int l = 0; l < levels; ++l)
    if (V[l] < 1 || max_prefix[l] < 0)
      return fail(PA_EINVAL, "bad shared-prefix groups (level %d: num_groups %d, "
                  "max_prefix_len %d)", l + 1, V[l], max_prefix[l]);
  Layout a;
  int rc = layout(S, H, D, max_ctx, 0, &a, pass_waves(H / Hkv, elt));
  if (rc != PA_OK) return rc;
  size_t need = a.bytes, need1 = 0;
  for (int l = 0; l < levels; ++l) {
    Layout b;
    rc = layout(V[l], Hkv * cols[l], D, max_prefix[l], 0, &b, pass_waves(cols[l], elt));
    if (rc != PA_OK) return rc;
    if (l == 1) need1 = b.bytes;
    else if (b.bytes > need) need = b.bytes;
  }
  size_t off = align256(need);
  pl->decode_bytes = off;
  pl->decode1_off = off;
  pl->decode1_bytes = align256(need1);
  off += pl->decode1_bytes;
  pl->levels = levels;
  for (int l = 0; l < levels; ++l) {
    PrefixLevel& v = pl->lv[l];
    v.maxbp = max_prefix[l] / bsz > 0 ? max_prefix[l] / bsz : 1;
    v.state_off = off;
    off = align256(off + sizeof(float) * (size_t)S * H * (D + 4));
    v.start_off = off;
    off = align256(off + sizeof(int32_t) * (size_t)S);
    v.vfirst_off = off;
    off = align256(off + sizeof(int32_t) * (size_t)V[l]);
    v.vcount_off = off;
    off = align256(off + sizeof(int32_t) * (size_t)V[l]);
    v.vctx_off = off;
    off = align256(off + sizeof(int32_t) * (size_t)V[l]);
    v.vtab_off = off;
    off = align256(off + sizeof(int32_t) * (size_t)V[l] * v.maxbp);
  }
  pl->gid_off = off;
  if (levels > 1) off = align256(off + sizeof(int32_t) * (size_t)S);
  pl->bytes = off;
  return PA_OK;
}

// No text skips a start at any level and none is in an outer group (b and gid: two levels
// only). The states are not cleared: a level's state row is read only where that level's
// start moved past the level before.
__global__ void prefix_clear_starts_kernel(int32_t* __restrict__ a, int32_t* __restrict__ b,
                                           int32_t* __restrict__ gid, int S) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < S; i += gridDim.x * blockDim.x) {
    a[i] = 0;
    if (b) b[i] = 0;
    if (gid) gid[i] = -1;
  }
}

// One workgroup per (group, key/value head): its members (clamped into the batch, at most
// 8 / (H / Hkv)), its shared length (at most every member's context less one token, so
// that each keeps its newest token, at most max_prefix, rounded down to a block) and, from
// the members' skipped start and the group's table row (its first member's, past the
// shared blocks zero). The members' lengths are read by one lane each and reduced across
// the wave.
// Two levels: the outer level records each member's group (gid_out); the inner level keeps
// its members up to the first whose outer group (base_gid) differs from its first member's.
__global__ void prefix_prep_kernel(const int32_t* __restrict__ vfirst_in,
                                   const int32_t* __restrict__ vcount_in,
                                   const int32_t* __restrict__ vprefix_in,
                                   const int32_t* __restrict__ ctx,
                                   const int32_t* __restrict__ tables, int S, int H, int Hkv,
                                   int maxb, int bsz, int max_prefix, int maxbp,
                                   int32_t* __restrict__ vfirst, int32_t* __restrict__ vcount,
                                   int32_t* __restrict__ vctx, int32_t* __restrict__ vtables,
                                   int32_t* __restrict__ start,
                                   const int32_t* __restrict__ base_start,
                                   int32_t* __restrict__ start_also, int cols,
                                   int32_t* __restrict__ gid_out,
                                   const int32_t* __restrict__ base_gid) {
  const int v = blockIdx.x;
  const int Gr = H / Hkv;
  __shared__ int sh[4];
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int f = vfirst_in[v];
    f = f < 0 ? 0 : f >= S ? S - 1 : f;
    int n = vcount_in[v];
    const int most = cols / Gr < S - f ? cols / Gr : S - f;
    n = n < 0 ? 0 : n > most ? most : n;
    const int64_t capacity = (int64_t)maxb * bsz;
    int64_t P = vprefix_in[v];
    if (P > max_prefix) P = max_prefix;
    // an inner level keeps its members up to the first whose outer group differs from the
    // first member's (members of different outer groups cannot share this level's blocks)
    if (base_gid && n > 1) {
      const bool other = lane < n && base_gid[f + lane] != base_gid[f];
      const uint64_t mask = __ballot(other);
      if (mask) n = __ffsll((unsigned long long)mask) - 1;
    }
    int64_t keep = INT32_MAX;  // the members' lengths less one, smallest
    if (lane < n) {
      int64_t L = ctx[f + lane];
      L = L < 0 ? 0 : L > capacity ? capacity : L;
      keep = L - 1;
    }
    for (int o = 32; o > 0; o >>= 1) {
      const int64_t other = __shfl_xor(keep, o);
      keep = other < keep ? other : keep;
    }
    if (P > keep) P = keep;
    if (P < 0 || n == 0) P = 0;
    P -= P % bsz;
    // an inner level starts where the first member's outer level ended
    const int P0 = base_start && n > 0 ? base_start[f] : 0;
    if (P < P0) P = P0;
    if (lane == 0) {
      sh[0] = f;
      sh[1] = n;
      sh[2] = (int)P;
      sh[3] = P0;
      vfirst[v] = f;
      vcount[v] = n;
      vctx[v] = (int)P - P0;
    }
  }
  __syncthreads();
  const int f = sh[0], n = sh[1], P = sh[2], P0 = sh[3];
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    start[f + i] = P;
    if (start_also) start_also[f + i] = P;
    if (gid_out) gid_out[f + i] = v;
  }
  const int nb = (P - P0) / bsz, b0 = P0 / bsz;
  for (int k = threadIdx.x; k < maxbp; k += blockDim.x)
    vtables[(int64_t)v * maxbp + k] = k < nb ? tables[(int64_t)f * maxb + b0 + k] : 0;
}

// ---- the set-up in one launch --------------------------------------------------------
// For batches of at most kSetupMax texts and kSetupMax groups per level the clear and the
// per-level set-ups above run as one kernel: workgroup 0 takes every text's starts and
// outer group from per-text membership arrays it builds in LDS (so no text's entries need
// clearing first, and no level waits for the one before it), and workgroup 1 + b takes
// group b of the outer level, then of the inner one: its geometry and its table row. Both
// compute a group's geometry with the same
// functions, as prefix_prep_kernel computes it; overlapping groups (refused by the debug
// check) resolve to the highest-numbered group.
constexpr int kSetupMax = 2048;

struct SetupLevel {
  const int32_t *first, *count, *prefix;  // the caller's groups
  int n, max_prefix, cols, maxbp;
  int32_t *vfirst, *vcount, *vctx, *vtab;  // the level's batch of groups
  int32_t* start;  // each text's start at this level
};

struct SetupArgs {
  SetupLevel lv[2];
  int levels;
  const int32_t* ctx;
  const int32_t* tables;
  int S, H, Hkv, maxb, bsz;
  int32_t* gid;  // two levels: each text's outer group (-1: none)
};

// Group v's first member, clamped into the batch, and its member count, clamped to the
// level's width and to the batch's end.
__device__ __forceinline__ void setup_members(const SetupLevel& g, int v, int S, int Gr, int& f,
                                              int& n) {
  int ff = g.first[v];
  ff = ff < 0 ? 0 : ff >= S ? S - 1 : ff;
  const int most = g.cols / Gr < S - ff ? g.cols / Gr : S - ff;
  const int c = g.count[v];
  n = c < 0 ? 0 : c > most ? most : c;
  f = ff;
}

// Shared length of a group with requested length `prefix`, n members whose attended
// lengths less one token have minimum `keep` (INT32_MAX for none), starting at P0: at most
// max_prefix and keep, rounded down to a block, not below P0.
__device__ __forceinline__ int setup_len_from(int64_t prefix, int max_prefix, int64_t keep, int n,
                                              int P0, int bsz) {
  int64_t P = prefix;
  if (P > max_prefix) P = max_prefix;
  if (P > keep) P = keep;
  if (P < 0 || n == 0) P = 0;
  P -= P % bsz;
  if (P < P0) P = P0;
  return (int)P;
}

// A member's attended length less one token (its length clamped into [0, capacity]).
__device__ __forceinline__ int64_t setup_keep(const SetupArgs& a, int t) {
  const int64_t capacity = (int64_t)a.maxb * a.bsz;
  int64_t L = a.ctx[t];
  L = L < 0 ? 0 : L > capacity ? capacity : L;
  return L - 1;
}

// The same for group v over its members f .. f + n - 1 (n <= kPrefixCols), one thread.
__device__ __forceinline__ int setup_shared_len(const SetupLevel& g, int v, int f, int n, int P0,
                                                const SetupArgs& a) {
  int64_t keep = INT32_MAX;
#pragma unroll
  for (int m = 0; m < kPrefixCols; ++m) {
    if (m < n) {
      const int64_t k = setup_keep(a, f + m);
      if (k < keep) keep = k;
    }
  }
  return setup_len_from(g.prefix[v], g.max_prefix, keep, n, P0, a.bsz);
}

// Minimum over the wave of x (64-bit).
__device__ __forceinline__ int64_t wave_min64(int64_t x) {
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t y = __shfl_xor(x, o);
    x = y < x ? y : x;
  }
  return x;
}

__global__ __launch_bounds__(256) void prefix_setup_kernel(SetupArgs a) {
  __shared__ int memb0[kSetupMax], memb1[kSetupMax], len0[kSetupMax], len1[kSetupMax];
  __shared__ int sh[4];
  const int S = a.S, Gr = a.H / a.Hkv;
  const SetupLevel& g0 = a.lv[0];
  if (blockIdx.x == 0) {
    // every text: the groups holding it, then its starts
    for (int t = threadIdx.x; t < S; t += blockDim.x) {
      memb0[t] = -1;
      memb1[t] = -1;
    }
    __syncthreads();
    for (int u = threadIdx.x; u < g0.n; u += blockDim.x) {
      int f, n;
      setup_members(g0, u, S, Gr, f, n);
      len0[u] = setup_shared_len(g0, u, f, n, 0, a);
      for (int m = 0; m < n; ++m) atomicMax(&memb0[f + m], u);
    }
    __syncthreads();
    if (a.levels > 1) {
      const SetupLevel& g1 = a.lv[1];
      for (int v = threadIdx.x; v < g1.n; v += blockDim.x) {
        int f, n;
        setup_members(g1, v, S, Gr, f, n);
        // members up to the first whose outer group differs from the first member's
        const int of = n > 0 ? memb0[f] : -1;
        for (int m = 1; m < n; ++m)
          if (memb0[f + m] != of) {
            n = m;
            break;
          }
        // the inner level starts where the first member's outer level ended
        const int P0 = n > 0 && of >= 0 ? len0[of] : 0;
        len1[v] = setup_shared_len(g1, v, f, n, P0, a);
        for (int m = 0; m < n; ++m) atomicMax(&memb1[f + m], v);
      }
      __syncthreads();
    }
    for (int t = threadIdx.x; t < S; t += blockDim.x) {
      const int u = memb0[t];
      const int st0 = u >= 0 ? len0[u] : 0;
      g0.start[t] = st0;
      if (a.levels > 1) {
        a.gid[t] = u;
        const int v = memb1[t];
        a.lv[1].start[t] = v >= 0 ? len1[v] : st0;
      }
    }
    return;
  }
  // group v of level l
  const int b = blockIdx.x - 1;
  const int l = b < g0.n ? 0 : 1;
  const int v = l == 0 ? b : b - g0.n;
  const SetupLevel& g = a.lv[l];
  if (threadIdx.x < 64) {
    // few dependent memory round trips: the descriptors (this group's and, for the inner
    // level, the outer groups' one per lane) at once, then every member's length one per
    // lane, reduced over the wave
    const int lane = threadIdx.x;
    int f, n;
    setup_members(g, v, S, Gr, f, n);
    const int64_t prefix = g.prefix[v];
    int P0 = 0;
    if (l == 1) {
      // each member's outer group: the highest outer group holding it, by ballots over the
      // outer groups, 64 at a time; the lane that holds its descriptor hands it over
      int og[kPrefixCols], ofo = 0, ono = 0;
#pragma unroll
      for (int m = 0; m < kPrefixCols; ++m) og[m] = -1;
      for (int u0 = 0; u0 < g0.n; u0 += 64) {
        const int u = u0 + lane;
        int fu = 0, nu = 0;
        if (u < g0.n) setup_members(g0, u, S, Gr, fu, nu);
#pragma unroll
        for (int m = 0; m < kPrefixCols; ++m) {
          const uint64_t hit = __ballot(m < n && f + m >= fu && f + m < fu + nu);
          if (hit) {
            const int src = 63 - __builtin_clzll(hit);
            og[m] = u0 + src;
            if (m == 0) {
              ofo = __shfl(fu, src);
              ono = __shfl(nu, src);
            }
          }
        }
      }
      for (int m = 1; m < n; ++m)
        if (og[m] != og[0]) {
          n = m;
          break;
        }
      if (n > 0 && og[0] >= 0) {
        const int64_t ko = wave_min64(lane < ono ? setup_keep(a, ofo + lane) : INT32_MAX);
        P0 = setup_len_from(g0.prefix[og[0]], g0.max_prefix, ko, ono, 0, a.bsz);
      }
    }
    const int64_t keep = wave_min64(lane < n ? setup_keep(a, f + lane) : INT32_MAX);
    const int P = setup_len_from(prefix, g.max_prefix, keep, n, P0, a.bsz);
    if (lane == 0) {
      sh[0] = f;
      sh[2] = P;
      sh[3] = P0;
      g.vfirst[v] = f;
      g.vcount[v] = n;
      g.vctx[v] = P - P0;
    }
  }
  __syncthreads();
  const int f = sh[0], P = sh[2], P0 = sh[3];
  const int nb = (P - P0) / a.bsz, b0 = P0 / a.bsz;
  for (int k = threadIdx.x; k < g.maxbp; k += blockDim.x)
    g.vtab[(int64_t)v * g.maxbp + k] = k < nb ? a.tables[(int64_t)f * a.maxb + b0 + k] : 0;
}

}  // namespace
}  // namespace pagedkv

namespace pagedkv {
namespace {

// One level of shared-prefix groups as the caller gives it.
struct GroupsIn {
  int32_t n;
  const int32_t *first, *count, *prefix;
  int32_t max_prefix;
  int32_t cols;  // query columns per key/value head in the level's pass (members x H / Hkv)
};

size_t prefix_bytes(int32_t S, int32_t H, int32_t Hkv, int32_t D, int32_t bsz, int32_t max_ctx,
                    int levels, const int32_t* V, const int32_t* maxp, const int32_t* cols,
                    int32_t dtype) {
  if (!dtype_ok(dtype)) return 0;
  PrefixLayout pl;
  if (prefix_layout(S, H, Hkv, D, max_ctx, levels, V, maxp, cols, bsz, elt_bytes(dtype), &pl) !=
      PA_OK)
    return 0;
  return pl.bytes;
}

// Query columns per key/value head for groups of up to `members` texts: the members' heads,
// rounded up to a head-group width the decode kernels take (1, 2, 4, 8); 0 if too many.
int32_t prefix_cols(int32_t members, int32_t H, int32_t Hkv) {
  if (Hkv < 1 || H % Hkv != 0 || members < 1) return 0;
  const int32_t need = members * (H / Hkv);
  for (int32_t c = 1; c <= kPrefixCols; c *= 2)
    if (c >= need) return c;
  return 0;
}

// Debug re-check of the share groups' promise, with the set-up kernel's own clamps: at
// each level no text is in two groups, and every member's table holds the same blocks as
// its group's first member's over the blocks the level reads once for the group.
int check_groups(int levels, const GroupsIn* g, const int32_t* ctx_d, const int32_t* tables_d,
                 int32_t S, int32_t H, int32_t Hkv, int32_t maxb, int32_t B, hipStream_t st) {
  std::vector<int32_t> ctx, tab;
  int rc;
  if ((rc = fetch(ctx, ctx_d, (size_t)S, st)) != PA_OK) return rc;
  if ((rc = fetch(tab, tables_d, (size_t)S * maxb, st)) != PA_OK) return rc;
  const int Gr = H / Hkv;
  const int64_t capacity = (int64_t)maxb * B;
  std::vector<int32_t> start_prev(S, 0), gid_prev(S, -1);
  for (int l = 0; l < levels; ++l) {
    std::vector<int32_t> first, count, prefix;
    if ((rc = fetch(first, g[l].first, (size_t)g[l].n, st)) != PA_OK) return rc;
    if ((rc = fetch(count, g[l].count, (size_t)g[l].n, st)) != PA_OK) return rc;
    if ((rc = fetch(prefix, g[l].prefix, (size_t)g[l].n, st)) != PA_OK) return rc;
    std::vector<int32_t> owner(S, -1), start(start_prev), gid(S, -1);
    for (int32_t v = 0; v < g[l].n; ++v) {
      const int32_t f = first[v] < 0 ? 0 : first[v] >= S ? S - 1 : first[v];
      const int32_t most = std::min(g[l].cols / Gr, S - f);
      int32_t n = count[v] < 0 ? 0 : count[v] > most ? most : count[v];
      if (l > 0)
        for (int32_t m = 1; m < n; ++m)
          if (gid_prev[f + m] != gid_prev[f]) {
            n = m;
            break;
          }
      int64_t P = std::min(prefix[v], g[l].max_prefix);
      int64_t keep = INT32_MAX;
      for (int32_t m = 0; m < n; ++m)
        keep = std::min(keep, std::min<int64_t>(std::max(ctx[f + m], 0), capacity) - 1);
      if (P > keep) P = keep;
      if (P < 0 || n == 0) P = 0;
      P -= P % B;
      const int64_t P0 = l > 0 && n > 0 ? start_prev[f] : 0;
      if (P < P0) P = P0;
      for (int32_t m = 0; m < n; ++m) {
        if (owner[f + m] >= 0)
          return fail(PA_EINVAL, "debug check: text %d is in groups %d and %d (level %d)", f + m,
                      owner[f + m], v, l + 1);
        owner[f + m] = v;
        start[f + m] = (int32_t)P;
        gid[f + m] = v;
        for (int64_t j = P0 / B; j < P / B; ++j)
          if (tab[(int64_t)(f + m) * maxb + j] != tab[(int64_t)f * maxb + j])
            return fail(PA_EINVAL, "debug check: group %d (level %d): text %d holds block %d "
                        "at logical block %lld, its first member %d holds block %d", v, l + 1,
                        f + m, tab[(int64_t)(f + m) * maxb + j], (long long)j, f,
                        tab[(int64_t)f * maxb + j]);
      }
    }
    start_prev.swap(start);
    gid_prev.swap(gid);
  }
  return PA_OK;
}

// The merges of both shared-block levels in one launch (decode_merge_pair), the outer
// level 8 heads a wave, the inner one GS1.
template <int QT, int D>
bool merge_pair_gs(int GS1, const decode_impl::MergePass& a, const decode_impl::MergePass& b,
                   int Hkv, int bsz, hipStream_t st) {
  using decode_impl::decode_merge_pair;
  const dim3 grid(a.groups + b.groups), block(decode_impl::kThreads);
  switch (GS1) {
    case 1: hipLaunchKernelGGL((decode_merge_pair<QT, D, 8, 1>), grid, block, 0, st, a, b, Hkv, bsz); return true;
    case 2: hipLaunchKernelGGL((decode_merge_pair<QT, D, 8, 2>), grid, block, 0, st, a, b, Hkv, bsz); return true;
    case 4: hipLaunchKernelGGL((decode_merge_pair<QT, D, 8, 4>), grid, block, 0, st, a, b, Hkv, bsz); return true;
    case 8: hipLaunchKernelGGL((decode_merge_pair<QT, D, 8, 8>), grid, block, 0, st, a, b, Hkv, bsz); return true;
  }
  return false;
}

bool merge_pair(int32_t dtype, int D, int GS1, const decode_impl::MergePass& a,
                const decode_impl::MergePass& b, int Hkv, int bsz, hipStream_t st) {
  const bool d64 = D == 64;
  if (dtype == PA_F32)
    return d64 ? merge_pair_gs<PA_F32, 64>(GS1, a, b, Hkv, bsz, st)
               : merge_pair_gs<PA_F32, 128>(GS1, a, b, Hkv, bsz, st);
  if (dtype == PA_F16)
    return d64 ? merge_pair_gs<PA_F16, 64>(GS1, a, b, Hkv, bsz, st)
               : merge_pair_gs<PA_F16, 128>(GS1, a, b, Hkv, bsz, st);
  if (dtype == PA_BF16)
    return d64 ? merge_pair_gs<PA_BF16, 64>(GS1, a, b, Hkv, bsz, st)
               : merge_pair_gs<PA_BF16, 128>(GS1, a, b, Hkv, bsz, st);
  return false;
}

// Checks that the set-up and the passes of the shared-prefix decode share, and the
// workspace layout they agree on.
int prefix_check(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                 int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
                 int levels, const GroupsIn* g, int32_t dtype, const void* workspace,
                 size_t workspace_bytes, PrefixLayout* pl) {
  if (!dtype_ok(dtype)) return fail(PA_EINVAL, "dtype %d is not PA_F32/PA_F16/PA_BF16", dtype);
  for (int l = 0; l < levels; ++l)
    if (g[l].n < 1) return fail(PA_EINVAL, "num_groups %d < 1 (level %d)", g[l].n, l + 1);
  if (num_kv_heads < 1 || num_heads % num_kv_heads != 0)
    return fail(PA_EINVAL, "num_heads %d is not a multiple of num_kv_heads %d", num_heads,
                num_kv_heads);
  if (num_heads / num_kv_heads > kPrefixCols)
    return fail(PA_EUNSUPPORTED, "%d query heads per key/value head (at most %d share a read)",
                num_heads / num_kv_heads, kPrefixCols);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (block_size != 4 && block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PA_EUNSUPPORTED, "block_size %d (supported: 4, 8, 16, 32)", block_size);
  if (!workspace) return fail(PA_EINVAL, "null pointer");
  if (!aligned16(workspace)) return fail(PA_EINVAL, "workspace must be 16-byte aligned");
  if (num_seqs < 1 || max_blocks_per_seq < 1 || max_context_len < 0)
    return fail(PA_EINVAL, "num_seqs and max_blocks_per_seq must be >= 1, max_context_len >= 0");
  const int32_t V[2] = {g[0].n, levels > 1 ? g[1].n : 0};
  const int32_t maxp[2] = {g[0].max_prefix, levels > 1 ? g[1].max_prefix : 0};
  const int32_t cols[2] = {g[0].cols, levels > 1 ? g[1].cols : 1};
  for (int l = 0; l < levels; ++l)
    if (cols[l] < num_heads / num_kv_heads || cols[l] > kPrefixCols)
      return fail(PA_EINVAL, "bad group width at level %d", l + 1);
  const int rc = prefix_layout(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                               levels, V, maxp, cols, block_size, elt_bytes(dtype), pl);
  if (rc != PA_OK) return rc;
  if (workspace_bytes < pl->bytes)
    return fail(PA_EINVAL, "workspace_bytes %zu < %zu required", workspace_bytes, pl->bytes);
  return PA_OK;
}

// The set-up of the shared-prefix decode (the plan): what the block tables, context lengths
// and groups alone decide, into the workspace. Every layer of a decode step attends with
// the same tables, lengths and groups, so one set-up serves all of them.
int prefix_plan(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t max_blocks_per_seq, int32_t max_context_len, int levels,
                const GroupsIn* g, int32_t dtype, void* workspace, size_t workspace_bytes,
                void* stream) {
  PrefixLayout pl;
  int rc = prefix_check(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, max_context_len, levels, g, dtype, workspace,
                        workspace_bytes, &pl);
  if (rc != PA_OK) return rc;
  for (int l = 0; l < levels; ++l) {
    if (!g[l].first || !g[l].count || !g[l].prefix) return fail(PA_EINVAL, "null pointer");
    if (((uintptr_t)g[l].first & 3u) || ((uintptr_t)g[l].count & 3u) ||
        ((uintptr_t)g[l].prefix & 3u))
      return fail(PA_EINVAL, "group arrays must be 4-byte aligned");
  }
  if (!block_tables || !context_lens) return fail(PA_EINVAL, "null pointer");
  if (((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u))
    return fail(PA_EINVAL, "tables and context_lens must be 4-byte aligned");
  char* ws = (char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  if (debug_checks()) {
    rc = check_groups(levels, g, context_lens, block_tables, num_seqs, num_heads, num_kv_heads,
                      max_blocks_per_seq, block_size, st);
    if (rc != PA_OK) return rc;
  }
  int32_t* start[2];
  for (int l = 0; l < levels; ++l) start[l] = (int32_t*)(ws + pl.lv[l].start_off);
  bool one_launch = num_seqs <= kSetupMax;
  for (int l = 0; l < levels; ++l) one_launch = one_launch && g[l].n <= kSetupMax;
  if (one_launch) {
    SetupArgs sa{};
    for (int l = 0; l < levels; ++l) {
      const PrefixLevel& v = pl.lv[l];
      sa.lv[l] = SetupLevel{g[l].first, g[l].count, g[l].prefix, g[l].n, g[l].max_prefix,
                            (int)g[l].cols, v.maxbp, (int32_t*)(ws + v.vfirst_off),
                            (int32_t*)(ws + v.vcount_off), (int32_t*)(ws + v.vctx_off),
                            (int32_t*)(ws + v.vtab_off), start[l]};
    }
    sa.levels = levels;
    sa.ctx = context_lens;
    sa.tables = block_tables;
    sa.S = num_seqs;
    sa.H = num_heads;
    sa.Hkv = num_kv_heads;
    sa.maxb = max_blocks_per_seq;
    sa.bsz = block_size;
    sa.gid = levels > 1 ? (int32_t*)(ws + pl.gid_off) : nullptr;
    const int groups = 1 + g[0].n + (levels > 1 ? g[1].n : 0);
    hipLaunchKernelGGL(prefix_setup_kernel, dim3(groups), dim3(256), 0, st, sa);
    PA_HIP_CHECK(hipGetLastError());
    return ok();
  }
  const int blocks = (num_seqs + 255) / 256;
  hipLaunchKernelGGL(prefix_clear_starts_kernel, dim3(blocks < 1024 ? blocks : 1024), dim3(256),
                     0, st, start[0], levels > 1 ? start[1] : (int32_t*)nullptr,
                     levels > 1 ? (int32_t*)(ws + pl.gid_off) : (int32_t*)nullptr, num_seqs);
  for (int l = 0; l < levels; ++l) {
    const PrefixLevel& v = pl.lv[l];
    hipLaunchKernelGGL(prefix_prep_kernel, dim3(g[l].n), dim3(256), 0, st, g[l].first,
                       g[l].count, g[l].prefix, context_lens, block_tables, num_seqs, num_heads,
                       num_kv_heads, max_blocks_per_seq, block_size, g[l].max_prefix, v.maxbp,
                       (int32_t*)(ws + v.vfirst_off), (int32_t*)(ws + v.vcount_off),
                       (int32_t*)(ws + v.vctx_off), (int32_t*)(ws + v.vtab_off), start[l],
                       l > 0 ? start[l - 1] : (const int32_t*)nullptr,
                       l + 1 < levels ? start[l + 1] : (int32_t*)nullptr, (int)g[l].cols,
                       l == 0 && levels > 1 ? (int32_t*)(ws + pl.gid_off) : (int32_t*)nullptr,
                       l > 0 ? (const int32_t*)(ws + pl.gid_off) : (const int32_t*)nullptr);
    PA_HIP_CHECK(hipGetLastError());
  }
  return ok();
}

// The passes of the shared-prefix decode over a workspace that prefix_plan filled: one pass
// per level over the groups' shared blocks (states out), then every text's own blocks with
// its states folded in (each level's where it applies). Only g[l].n, .max_prefix and .cols
// are read here. A workspace holding no plan for these shapes, tables, lengths and groups
// gives meaningless outputs, with every access still inside the batch, the pools and the
// workspace: the kernels clamp the plan's members, lengths and starts and bound its table
// entries as they do the caller's.
int prefix_run(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
               int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
               int levels, const GroupsIn* g, float scale, int32_t dtype, void* workspace,
               size_t workspace_bytes, void* stream,
               const decode_impl::NewRows& nr = decode_impl::NewRows{}) {
  PrefixLayout pl;
  int rc = prefix_check(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, max_context_len, levels, g, dtype, workspace,
                        workspace_bytes, &pl);
  if (rc != PA_OK) return rc;
  // the plain decode's checks (pointers, alignment) before anything is launched
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_EINVAL, "null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_EINVAL, "out, q, pools and workspace must be 16-byte aligned");
  if (num_blocks < 1) return fail(PA_EINVAL, "num_blocks must be >= 1");
  if (!std::isfinite(scale)) return fail(PA_EINVAL, "scale is not finite");
  char* ws = (char*)workspace;
  float* state[2];
  int32_t* start[2];
  for (int l = 0; l < levels; ++l) {
    state[l] = (float*)(ws + pl.lv[l].state_off);
    start[l] = (int32_t*)(ws + pl.lv[l].start_off);
  }
  const int Gr = num_heads / num_kv_heads;
  const int elt = elt_bytes(dtype);
  // With two levels (the outer one 8 heads a wave) the level passes write their partials to
  // their own decode workspaces and one launch merges both after both passes, instead of a
  // merge after each.
  const bool pair = levels == 2 && heads_per_wave(g[0].cols) == 8;
  decode_impl::MergePass mp[2];
  decode_impl::Prefix p1[2];
  for (int l = 0; l < levels; ++l) {
    const PrefixLevel& v = pl.lv[l];
    int colm = 0, colh = 0;
    for (int c = 0; c < g[l].cols; ++c) {
      colm |= (c / Gr) << (4 * c);
      colh |= (c % Gr) << (4 * c);
    }
    p1[l] = decode_impl::Prefix{nullptr, state[l], (const int32_t*)(ws + v.vfirst_off),
                                (const int32_t*)(ws + v.vcount_off), num_heads, 1, nullptr,
                                nullptr, num_seqs, Gr, g[l].cols / Gr, colm, colh};
    if (pair) {
      Layout lay;
      rc = layout(g[l].n, num_kv_heads * g[l].cols, head_dim, g[l].max_prefix, 0, &lay,
                  pass_waves(g[l].cols, elt));
      if (rc != PA_OK) return rc;
      const char* region = l == 1 ? ws + pl.decode1_off : ws;
      const int64_t runs = (int64_t)g[l].n * (num_kv_heads * g[l].cols / heads_per_wave(g[l].cols));
      const bool by_boundary = decode_impl::merge_by_boundary(runs, lay.W);
      const int64_t mwaves = by_boundary ? lay.W : runs;
      mp[l] = decode_impl::MergePass{(const int32_t*)(ws + v.vctx_off), g[l].n,
                                     num_kv_heads * g[l].cols, v.maxbp, (int)lay.W,
                                     g[l].max_prefix, (const int64_t*)region,
                                     (const int64_t*)(region + lay.excl_off),
                                     (const float*)(region + lay.part_off),
                                     by_boundary ? (const int64_t*)(region + lay.split_off)
                                                 : (const int64_t*)nullptr,
                                     p1[l],
                                     (int)((mwaves + decode_impl::kWavesPerGroup - 1) /
                                           decode_impl::kWavesPerGroup)};
    }
  }
  for (int l = 0; l < levels; ++l) {
    const PrefixLevel& v = pl.lv[l];
    char* region = l == 1 ? ws + pl.decode1_off : ws;
    const size_t region_bytes = l == 1 ? pl.decode1_bytes : pl.decode_bytes;
    rc = decode_common(out, q, k_cache, v_cache, (const int32_t*)(ws + v.vtab_off),
                       (const int32_t*)(ws + v.vctx_off), g[l].n, num_kv_heads * g[l].cols,
                       num_kv_heads, head_dim, block_size, num_blocks, v.maxbp, g[l].max_prefix,
                       0, scale, 1.0f, 1.0f, dtype, dtype, region, region_bytes, stream,
                       decode_impl::NewRows{}, p1[l], pass_waves(g[l].cols, elt), pair);
    if (rc != PA_OK) return rc;
  }
  if (pair) {
    if (!merge_pair(dtype, head_dim, heads_per_wave(g[1].cols), mp[0], mp[1], num_kv_heads,
                    block_size, (hipStream_t)stream))
      return fail(PA_EUNSUPPORTED, "no merge for this shape");
    PA_HIP_CHECK(hipGetLastError());
  }
  // with new rows, the own pass also stores them (a text's newest token lies in its own
  // blocks: every level leaves each member at least that token)
  const decode_impl::Prefix p2{start[levels - 1], state[levels - 1], nullptr, nullptr, num_heads,
                               2, levels > 1 ? start[0] : (const int32_t*)nullptr,
                               levels > 1 ? state[0] : (const float*)nullptr};
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, 0, scale, 1.0f, 1.0f, dtype, dtype, workspace,
                       pl.decode_bytes, stream, nr, p2, pass_waves(Gr, elt));
}

// The shared-prefix decode over one level of groups or two nested ones: the set-up, then
// the passes.
int prefix_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                  int levels, const GroupsIn* g, float scale, int32_t dtype, void* workspace,
                  size_t workspace_bytes, void* stream,
                  const decode_impl::NewRows& nr = decode_impl::NewRows{}) {
  // the passes' own checks first, so that nothing is launched for a call they refuse
  PrefixLayout pl;
  int rc = prefix_check(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, max_context_len, levels, g, dtype, workspace,
                        workspace_bytes, &pl);
  if (rc != PA_OK) return rc;
  if (!out || !q || !k_cache || !v_cache) return fail(PA_EINVAL, "null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_EINVAL, "out, q, pools and workspace must be 16-byte aligned");
  if (num_blocks < 1) return fail(PA_EINVAL, "num_blocks must be >= 1");
  if (!std::isfinite(scale)) return fail(PA_EINVAL, "scale is not finite");
  rc = prefix_plan(block_tables, context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                   block_size, max_blocks_per_seq, max_context_len, levels, g, dtype, workspace,
                   workspace_bytes, stream);
  if (rc != PA_OK) return rc;
  return prefix_run(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                    num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                    max_context_len, levels, g, scale, dtype, workspace, workspace_bytes, stream,
                    nr);
}

}  // namespace
}  // namespace pagedkv

extern "C" size_t pa_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                                   int32_t num_kv_heads, int32_t head_dim,
                                                   int32_t block_size, int32_t max_context_len,
                                                   int32_t num_groups, int32_t max_prefix_len,
                                                   int32_t dtype) {
  const int32_t V[1] = {num_groups}, maxp[1] = {max_prefix_len}, cols[1] = {kPrefixCols};
  return prefix_bytes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len, 1,
                      V, maxp, cols, dtype);
}

extern "C" size_t pa_decode_prefix2_workspace_bytes(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_context_len, int32_t num_groups, int32_t max_prefix_len,
    int32_t num_inner_groups, int32_t max_inner_prefix_len, int32_t inner_members,
    int32_t dtype) {
  const int32_t V[2] = {num_groups, num_inner_groups};
  const int32_t maxp[2] = {max_prefix_len, max_inner_prefix_len};
  const int32_t cols[2] = {kPrefixCols, prefix_cols(inner_members, num_heads, num_kv_heads)};
  if (cols[1] == 0) return 0;
  return prefix_bytes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len, 2,
                      V, maxp, cols, dtype);
}

extern "C" int pa_decode_attention_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_groups,
    const int32_t* group_first, const int32_t* group_count, const int32_t* group_prefix,
    int32_t max_prefix_len, float scale, int32_t dtype, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (!dtype_ok(dtype)) return fail(PA_EINVAL, "dtype %d is not PA_F32/PA_F16/PA_BF16", dtype);
  if (num_groups < 0) return fail(PA_EINVAL, "num_groups %d < 0", num_groups);
  if (num_groups == 0)
    return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                         num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                         max_blocks_per_seq, max_context_len, 0, scale, 1.0f, 1.0f, dtype, dtype,
                         workspace, workspace_bytes, stream);
  const GroupsIn g[1] = {{num_groups, group_first, group_count, group_prefix, max_prefix_len,
                          kPrefixCols}};
  return prefix_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, 1, g, scale, dtype, workspace, workspace_bytes, stream);
}

namespace {

// The two levels of the nested shared-block calls as the caller gives them (null arrays
// where a call reads only the counts and lengths).
int prefix2_levels(int32_t num_heads, int32_t num_kv_heads, int32_t num_groups,
                   const int32_t* group_first, const int32_t* group_count,
                   const int32_t* group_prefix, int32_t max_prefix_len, int32_t num_inner_groups,
                   const int32_t* inner_first, const int32_t* inner_count,
                   const int32_t* inner_prefix, int32_t max_inner_prefix_len,
                   int32_t inner_members, GroupsIn* g) {
  if (num_groups < 1 || num_inner_groups < 1)
    return fail(PA_EINVAL, "num_groups %d and num_inner_groups %d must be >= 1", num_groups,
                num_inner_groups);
  if (num_kv_heads < 1 || num_heads % num_kv_heads != 0)
    return fail(PA_EINVAL, "num_heads %d is not a multiple of num_kv_heads %d", num_heads,
                num_kv_heads);
  const int32_t icols = prefix_cols(inner_members, num_heads, num_kv_heads);
  if (icols == 0)
    return fail(inner_members < 1 ? PA_EINVAL : PA_EUNSUPPORTED,
                "inner_members %d: 1 .. %d with %d query heads per key/value head",
                inner_members, kPrefixCols / (num_heads / num_kv_heads),
                num_heads / num_kv_heads);
  g[0] = GroupsIn{num_groups, group_first, group_count, group_prefix, max_prefix_len,
                  kPrefixCols};
  g[1] = GroupsIn{num_inner_groups, inner_first, inner_count, inner_prefix, max_inner_prefix_len,
                  icols};
  return PA_OK;
}

// The new rows of a fused write, checked (nullptr rows: none, all three null).
int new_rows_of(const void* k_new, const void* v_new, const int64_t* slots, void* k_cache,
                void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                int32_t num_blocks, void* stream, bool optional, decode_impl::NewRows* nr) {
  *nr = decode_impl::NewRows{};
  if (optional && !k_new && !v_new && !slots) return PA_OK;
  if (!k_new || !v_new || !slots) return fail(PA_EINVAL, "null pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || ((uintptr_t)slots & 7u))
    return fail(PA_EINVAL, "k_new and v_new must be 16-byte aligned, slots 8-byte aligned");
  if (debug_checks() && block_tables && context_lens && num_seqs > 0 && max_blocks_per_seq > 0 &&
      num_blocks > 0 && block_size > 0) {
    const int rc = check_new_slots(slots, block_tables, context_lens, num_seqs,
                                   max_blocks_per_seq, block_size, num_blocks,
                                   (hipStream_t)stream);
    if (rc != PA_OK) return rc;
  }
  *nr = decode_impl::NewRows{(const char*)k_new, (const char*)v_new, slots, (char*)k_cache,
                             (char*)v_cache};
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_attention_prefix2(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_groups,
    const int32_t* group_first, const int32_t* group_count, const int32_t* group_prefix,
    int32_t max_prefix_len, int32_t num_inner_groups, const int32_t* inner_first,
    const int32_t* inner_count, const int32_t* inner_prefix, int32_t max_inner_prefix_len,
    int32_t inner_members, float scale, int32_t dtype, void* workspace, size_t workspace_bytes,
    void* stream) {
  GroupsIn g[2];
  const int rc = prefix2_levels(num_heads, num_kv_heads, num_groups, group_first, group_count,
                                group_prefix, max_prefix_len, num_inner_groups, inner_first,
                                inner_count, inner_prefix, max_inner_prefix_len, inner_members,
                                g);
  if (rc != PA_OK) return rc;
  return prefix_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, 2, g, scale, dtype, workspace, workspace_bytes, stream);
}

extern "C" int pa_decode_attention_prefix2_write(
    void* out, const void* q, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
    const int64_t* slots, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t num_groups, const int32_t* group_first, const int32_t* group_count,
    const int32_t* group_prefix, int32_t max_prefix_len, int32_t num_inner_groups,
    const int32_t* inner_first, const int32_t* inner_count, const int32_t* inner_prefix,
    int32_t max_inner_prefix_len, int32_t inner_members, float scale, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return fail(PA_EINVAL, "dtype %d is not PA_F32/PA_F16/PA_BF16", dtype);
  GroupsIn g[2];
  int rc = prefix2_levels(num_heads, num_kv_heads, num_groups, group_first, group_count,
                          group_prefix, max_prefix_len, num_inner_groups, inner_first,
                          inner_count, inner_prefix, max_inner_prefix_len, inner_members, g);
  if (rc != PA_OK) return rc;
  decode_impl::NewRows nr;
  rc = new_rows_of(k_new, v_new, slots, k_cache, v_cache, block_tables, context_lens, num_seqs,
                   max_blocks_per_seq, block_size, num_blocks, stream, false, &nr);
  if (rc != PA_OK) return rc;
  return prefix_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, 2, g, scale, dtype, workspace, workspace_bytes, stream,
                       nr);
}

extern "C" int pa_decode_prefix2_plan(
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_groups,
    const int32_t* group_first, const int32_t* group_count, const int32_t* group_prefix,
    int32_t max_prefix_len, int32_t num_inner_groups, const int32_t* inner_first,
    const int32_t* inner_count, const int32_t* inner_prefix, int32_t max_inner_prefix_len,
    int32_t inner_members, int32_t dtype, void* workspace, size_t workspace_bytes,
    void* stream) {
  GroupsIn g[2];
  const int rc = prefix2_levels(num_heads, num_kv_heads, num_groups, group_first, group_count,
                                group_prefix, max_prefix_len, num_inner_groups, inner_first,
                                inner_count, inner_prefix, max_inner_prefix_len, inner_members,
                                g);
  if (rc != PA_OK) return rc;
  return prefix_plan(block_tables, context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                     block_size, max_blocks_per_seq, max_context_len, 2, g, dtype, workspace,
                     workspace_bytes, stream);
}

extern "C" int pa_decode_attention_prefix2_run(
    void* out, const void* q, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
    const int64_t* slots, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t num_groups, int32_t max_prefix_len, int32_t num_inner_groups,
    int32_t max_inner_prefix_len, int32_t inner_members, float scale, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream) {
  GroupsIn g[2];
  int rc = prefix2_levels(num_heads, num_kv_heads, num_groups, nullptr, nullptr, nullptr,
                          max_prefix_len, num_inner_groups, nullptr, nullptr, nullptr,
                          max_inner_prefix_len, inner_members, g);
  if (rc != PA_OK) return rc;
  decode_impl::NewRows nr;
  rc = new_rows_of(k_new, v_new, slots, k_cache, v_cache, block_tables, context_lens, num_seqs,
                   max_blocks_per_seq, block_size, num_blocks, stream, true, &nr);
  if (rc != PA_OK) return rc;
  return prefix_run(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                    num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                    max_context_len, 2, g, scale, dtype, workspace, workspace_bytes, stream, nr);
}
