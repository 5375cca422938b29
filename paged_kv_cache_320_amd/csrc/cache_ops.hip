// Cache writes on the device: the new token's key/value write and the
// copy-on-write block copy. Both are pure 16-byte moves (bit-exact).
//
// «The KV Cache and PagedAttention» › "One Token at a Time": each step adds only
// the new token's key and value to the cache. › "Shared, Copied on Write": a
// shared block is copied whole before a sharer writes into it.
#include "device.hpp"

namespace pagedkv {
namespace {

constexpr int kThreads = 256;

// One thread moves 16 bytes of one (token, kv head) row for K and for V.
// rows = num_tokens * Hkv, row = D * elt bytes = lpr 16-byte pieces.
__global__ __launch_bounds__(kThreads) void kv_write_kernel(
    uint4* __restrict__ kc, uint4* __restrict__ vc, const uint4* __restrict__ kn,
    const uint4* __restrict__ vn, const int64_t* __restrict__ slots, int64_t pieces,
    int lpr, int hkv, int bsz, int64_t num_slots) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < pieces;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = i / lpr;          // token * hkv + head
    const int piece = (int)(i - row * lpr);
    const int64_t tok = row / hkv;
    const int head = (int)(row - tok * hkv);
    const int64_t slot = slots[tok];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / bsz;
    const int place = (int)(slot - blk * bsz);
    const int64_t dst = (((blk * hkv + head) * bsz + place) * lpr) + piece;
    kc[dst] = kn[i];
    vc[dst] = vn[i];
  }
}

// One thread moves 16 bytes of one block for K and for V.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    uint4* __restrict__ kc, uint4* __restrict__ vc, const int32_t* __restrict__ pairs,
    int64_t pieces_per_block, int64_t total, int num_blocks) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t p = i / pieces_per_block;
    const int64_t off = i - p * pieces_per_block;
    const int src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
    kc[(int64_t)dst * pieces_per_block + off] = kc[(int64_t)src * pieces_per_block + off];
    vc[(int64_t)dst * pieces_per_block + off] = vc[(int64_t)src * pieces_per_block + off];
  }
}

int check_shape(int32_t num_blocks, int32_t hkv, int32_t d, int32_t bsz, int32_t dtype) {
  if (!dtype_ok(dtype)) return fail(PA_EINVAL, "dtype %d is not PA_F32/PA_F16/PA_BF16", dtype);
  if (d != 64 && d != 128) return fail(PA_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", d);
  if (bsz != 4 && bsz != 8 && bsz != 16 && bsz != 32)
    return fail(PA_EUNSUPPORTED, "block_size %d (supported: 4, 8, 16, 32)", bsz);
  if (num_blocks < 1 || hkv < 1) return fail(PA_EINVAL, "num_blocks and num_kv_heads must be >= 1");
  return PA_OK;
}

int grid_for(int64_t pieces) {
  int cus = 0;
  if (device_cus(&cus) != PA_OK) cus = 256;
  int64_t want = (pieces + kThreads - 1) / kThreads;
  int64_t cap = (int64_t)cus * 16;
  return (int)(want < cap ? want : cap);
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" int pa_kv_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int64_t* slots, int32_t num_tokens, int32_t num_blocks,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t dtype, void* stream) {
  int rc = check_shape(num_blocks, num_kv_heads, head_dim, block_size, dtype);
  if (rc != PA_OK) return rc;
  if (num_tokens < 0) return fail(PA_EINVAL, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !slots) return fail(PA_EINVAL, "null pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PA_EINVAL, "pools and new rows must be 16-byte aligned");
  if (((uintptr_t)slots & 7u) != 0) return fail(PA_EINVAL, "slots must be 8-byte aligned");
  const int lpr = head_dim * elt_bytes(dtype) / 16;
  const int64_t pieces = (int64_t)num_tokens * num_kv_heads * lpr;
  hipLaunchKernelGGL(kv_write_kernel, dim3(grid_for(pieces)), dim3(kThreads), 0,
                     (hipStream_t)stream, (uint4*)k_cache, (uint4*)v_cache,
                     (const uint4*)k_new, (const uint4*)v_new, slots, pieces, lpr,
                     (int)num_kv_heads, (int)block_size, (int64_t)num_blocks * block_size);
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}

extern "C" int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t dtype,
                              void* stream) {
  int rc = check_shape(num_blocks, num_kv_heads, head_dim, block_size, dtype);
  if (rc != PA_OK) return rc;
  if (num_pairs < 0) return fail(PA_EINVAL, "num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !pairs) return fail(PA_EINVAL, "null pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache)) return fail(PA_EINVAL, "pools must be 16-byte aligned");
  if (((uintptr_t)pairs & 3u) != 0) return fail(PA_EINVAL, "pairs must be 4-byte aligned");
  const int64_t ppb = (int64_t)num_kv_heads * block_size * head_dim * elt_bytes(dtype) / 16;
  const int64_t total = ppb * num_pairs;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid_for(total)), dim3(kThreads), 0,
                     (hipStream_t)stream, (uint4*)k_cache, (uint4*)v_cache, pairs, ppb, total,
                     (int)num_blocks);
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}
