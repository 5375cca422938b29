// Cache writes on the device: the new token's key/value write and the
// copy-on-write block copy. Both are pure 16-byte moves (bit-exact).
//
// «The KV Cache and PagedAttention» › "One Token at a Time": each step adds only
// the new token's key and value to the cache. › "Shared, Copied on Write": a
// shared block is copied whole before a sharer writes into it. › "When Memory Runs
// Out": a text that gives way moves all its blocks to host memory and back (swap).
#include "device.hpp"

#include <cmath>

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

// Swap: one thread moves 16 bytes of one block for K and for V from the source pools to
// the destination pools (one side pinned host memory, read or written across the bus).
__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(
    uint4* __restrict__ dk, uint4* __restrict__ dv, const uint4* __restrict__ sk,
    const uint4* __restrict__ sv, const int32_t* __restrict__ pairs, int64_t pieces_per_block,
    int64_t total, int num_src, int num_dst) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t p = i / pieces_per_block;
    const int64_t off = i - p * pieces_per_block;
    const int src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= num_src || dst < 0 || dst >= num_dst) continue;
    const uint4 k = sk[(int64_t)src * pieces_per_block + off];
    const uint4 v = sv[(int64_t)src * pieces_per_block + off];
    dk[(int64_t)dst * pieces_per_block + off] = k;
    dv[(int64_t)dst * pieces_per_block + off] = v;
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

// Quantizing write into E4M3 pools: one thread turns 16 source values of one (token,
// kv head) row into 16 codes (16 bytes) for K and for V. rows = num_tokens * Hkv,
// row = D codes = lpr 16-byte pieces; SRC is the source element format.
template <int SRC>
__global__ __launch_bounds__(kThreads) void kv_write_fp8_kernel(
    uint4* __restrict__ kc, uint4* __restrict__ vc, const uint4* __restrict__ kn,
    const uint4* __restrict__ vn, const int64_t* __restrict__ slots, int64_t pieces, int lpr,
    int hkv, int bsz, int64_t num_slots, float k_inv, float v_inv) {
  constexpr int IN = 16 * elt_size<SRC>() / 16;  // 16-byte source pieces per 16 codes
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < pieces;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = i / lpr;
    const int piece = (int)(i - row * lpr);
    const int64_t tok = row / hkv;
    const int head = (int)(row - tok * hkv);
    const int64_t slot = slots[tok];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / bsz;
    const int place = (int)(slot - blk * bsz);
    const int64_t dst = (((blk * hkv + head) * bsz + place) * lpr) + piece;
    float kf[16], vf[16];
#pragma unroll
    for (int j = 0; j < IN; ++j) {
      widen16<SRC>(kn[i * IN + j], kf + j * (16 / IN));
      widen16<SRC>(vn[i * IN + j], vf + j * (16 / IN));
    }
    uint32_t kw[4], vw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kw[j] = vw[j] = 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        kw[j] |= e4m3_from_f32(kf[4 * j + b] * k_inv) << (8 * b);
        vw[j] |= e4m3_from_f32(vf[4 * j + b] * v_inv) << (8 * b);
      }
    }
    kc[dst] = make_uint4(kw[0], kw[1], kw[2], kw[3]);
    vc[dst] = make_uint4(vw[0], vw[1], vw[2], vw[3]);
  }
}

int check_shape(int32_t num_blocks, int32_t hkv, int32_t d, int32_t bsz, int32_t dtype) {
  if (!pool_dtype_ok(dtype))
    return fail(PA_EINVAL, "dtype %d is not PA_F32/PA_F16/PA_BF16/PA_FP8_E4M3", dtype);
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

extern "C" int pa_kv_write_fp8(void* k_cache, void* v_cache, const void* k_new,
                               const void* v_new, const int64_t* slots, int32_t num_tokens,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t src_dtype, float k_scale,
                               float v_scale, void* stream) {
  int rc = check_shape(num_blocks, num_kv_heads, head_dim, block_size, PA_FP8_E4M3);
  if (rc != PA_OK) return rc;
  if (!dtype_ok(src_dtype))
    return fail(PA_EINVAL, "src_dtype %d is not PA_F32/PA_F16/PA_BF16", src_dtype);
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_EINVAL, "scales must be finite and > 0");
  if (num_tokens < 0) return fail(PA_EINVAL, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !slots) return fail(PA_EINVAL, "null pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PA_EINVAL, "pools and new rows must be 16-byte aligned");
  if (((uintptr_t)slots & 7u) != 0) return fail(PA_EINVAL, "slots must be 8-byte aligned");
  if (debug_checks()) {
    rc = check_slots(slots, num_tokens, (int64_t)num_blocks * block_size, (hipStream_t)stream);
    if (rc != PA_OK) return rc;
  }
  const int lpr = head_dim / 16;  // 16 codes per piece
  const int64_t pieces = (int64_t)num_tokens * num_kv_heads * lpr;
  // the rounding of x / scale is decided as fp32(x) * fp32(1 / scale)
  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  const dim3 grid(grid_for(pieces)), block(kThreads);
  hipStream_t st = (hipStream_t)stream;
  if (src_dtype == PA_F32)
    hipLaunchKernelGGL(kv_write_fp8_kernel<PA_F32>, grid, block, 0, st, (uint4*)k_cache,
                       (uint4*)v_cache, (const uint4*)k_new, (const uint4*)v_new, slots, pieces,
                       lpr, (int)num_kv_heads, (int)block_size, num_slots, k_inv, v_inv);
  else if (src_dtype == PA_F16)
    hipLaunchKernelGGL(kv_write_fp8_kernel<PA_F16>, grid, block, 0, st, (uint4*)k_cache,
                       (uint4*)v_cache, (const uint4*)k_new, (const uint4*)v_new, slots, pieces,
                       lpr, (int)num_kv_heads, (int)block_size, num_slots, k_inv, v_inv);
  else
    hipLaunchKernelGGL(kv_write_fp8_kernel<PA_BF16>, grid, block, 0, st, (uint4*)k_cache,
                       (uint4*)v_cache, (const uint4*)k_new, (const uint4*)v_new, slots, pieces,
                       lpr, (int)num_kv_heads, (int)block_size, num_slots, k_inv, v_inv);
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}

extern "C" int pa_kv_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int64_t* slots, int32_t num_tokens, int32_t num_blocks,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t dtype, void* stream) {
  if (dtype == PA_FP8_E4M3)
    return fail(PA_EINVAL, "E4M3 pools are written with pa_kv_write_fp8");
  int rc = check_shape(num_blocks, num_kv_heads, head_dim, block_size, dtype);
  if (rc != PA_OK) return rc;
  if (num_tokens < 0) return fail(PA_EINVAL, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !slots) return fail(PA_EINVAL, "null pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PA_EINVAL, "pools and new rows must be 16-byte aligned");
  if (((uintptr_t)slots & 7u) != 0) return fail(PA_EINVAL, "slots must be 8-byte aligned");
  if (debug_checks()) {
    rc = check_slots(slots, num_tokens, (int64_t)num_blocks * block_size, (hipStream_t)stream);
    if (rc != PA_OK) return rc;
  }
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
  if (debug_checks()) {
    rc = check_pairs(pairs, num_pairs, num_blocks, (hipStream_t)stream);
    if (rc != PA_OK) return rc;
  }
  const int64_t ppb = (int64_t)num_kv_heads * block_size * head_dim * elt_bytes(dtype) / 16;
  const int64_t total = ppb * num_pairs;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid_for(total)), dim3(kThreads), 0,
                     (hipStream_t)stream, (uint4*)k_cache, (uint4*)v_cache, pairs, ppb, total,
                     (int)num_blocks);
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}

namespace {

// The address a kernel on the current device uses for p: device memory of this device,
// or pinned host memory (its device mapping). Anything else (pageable host memory,
// another device's memory, managed memory) is refused.
int device_view(const void* p, const char* name, const void** out) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return pagedkv::fail(PA_EINVAL, "%s is neither device memory nor pinned host memory", name);
  }
  int dev = 0;
  PA_HIP_CHECK(hipGetDevice(&dev));
  if (at.type == hipMemoryTypeDevice && !at.isManaged) {
    if (at.device != dev)
      return pagedkv::fail(PA_EINVAL, "%s is memory of device %d, not of the current device %d",
                           name, at.device, dev);
    *out = p;
    return PA_OK;
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer && !at.isManaged) {
    // the mapping may be reported for the allocation's start or for p itself
    const char* host = at.hostPointer ? (const char*)at.hostPointer : (const char*)p;
    *out = (const char*)at.devicePointer + ((const char*)p - host);
    return PA_OK;
  }
  return pagedkv::fail(PA_EINVAL, "%s is neither device memory nor pinned host memory", name);
}

}  // namespace

extern "C" int pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* pairs, int32_t num_pairs, int32_t num_src_blocks,
                              int32_t num_dst_blocks, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t dtype, void* stream) {
  using namespace pagedkv;
  int rc = check_shape(num_src_blocks, num_kv_heads, head_dim, block_size, dtype);
  if (rc != PA_OK) return rc;
  if (num_dst_blocks < 1) return fail(PA_EINVAL, "num_dst_blocks %d < 1", num_dst_blocks);
  if (num_pairs < 0) return fail(PA_EINVAL, "num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return ok();
  if (!dst_k || !dst_v || !src_k || !src_v || !pairs) return fail(PA_EINVAL, "null pointer");
  if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v))
    return fail(PA_EINVAL, "pools must be 16-byte aligned");
  if (((uintptr_t)pairs & 3u) != 0) return fail(PA_EINVAL, "pairs must be 4-byte aligned");
  const void *dk, *dv, *sk, *sv, *pp;
  if ((rc = device_view(dst_k, "dst_k", &dk)) != PA_OK) return rc;
  if ((rc = device_view(dst_v, "dst_v", &dv)) != PA_OK) return rc;
  if ((rc = device_view(src_k, "src_k", &sk)) != PA_OK) return rc;
  if ((rc = device_view(src_v, "src_v", &sv)) != PA_OK) return rc;
  if ((rc = device_view(pairs, "pairs", &pp)) != PA_OK) return rc;
  const int64_t ppb = (int64_t)num_kv_heads * block_size * head_dim * elt_bytes(dtype) / 16;
  const int64_t total = ppb * num_pairs;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(grid_for(total)), dim3(kThreads), 0,
                     (hipStream_t)stream, (uint4*)dk, (uint4*)dv, (const uint4*)sk,
                     (const uint4*)sv, (const int32_t*)pp, ppb, total, (int)num_src_blocks,
                     (int)num_dst_blocks);
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}
