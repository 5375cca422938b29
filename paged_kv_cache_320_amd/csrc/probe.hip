// Measurement helpers: the HBM read rate a plain streaming kernel reaches on this
// device (the practical ceiling next to the 8 TB/s specification), and a copy of
// known size used to calibrate the memory-traffic counters.
#include "device.hpp"

namespace pagedkv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;

// Each workgroup reads its own contiguous range in 16-byte pieces, kUnroll non-temporal
// loads in flight per lane (64 KiB per workgroup). Measured on this part: with 4 waves
// per CU this pattern reads ~7.1 TB/s, plain loads or 4 loads in flight ~6.2-6.3 TB/s.
// The range's last, partial group is issued at once too (lanes past the end re-read the
// range's last piece, not counted), so a range of any length keeps its loads in flight.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ buf,
                                                               int64_t pieces,
                                                               uint32_t* __restrict__ sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* p = reinterpret_cast<const u32x4*>(buf);
  const int64_t per = (pieces + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < pieces ? lo + per : pieces;
  int64_t i = lo + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kUnroll - 1) * kThreads < hi; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) v[j] = __builtin_nontemporal_load(p + i + j * kThreads);
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (lo < hi && i - threadIdx.x < hi) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t k = i + j * kThreads;
      v[j] = __builtin_nontemporal_load(p + (k < hi ? k : hi - 1));
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
      if (i + j * kThreads < hi) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t sh[kThreads / 64];
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x / 64] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = sh[0] ^ sh[1] ^ sh[2] ^ sh[3];
}

// Random-tile read: the tiles named by ids (whole tiles of TB bytes, 1 KiB wave loads),
// each wave a contiguous share of the list with 32 KiB in flight; ids are clamped into
// the buffer.
template <int TB>
__global__ __launch_bounds__(kThreads) void tile_read_kernel(const char* __restrict__ buf,
                                                             int64_t nbuf,
                                                             const int32_t* __restrict__ ids,
                                                             int64_t n, uint32_t* __restrict__ sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  constexpr int LPT = TB / 1024, TU = 32768 / TB;
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t wv = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t lo = n * wv / nw, hi = n * (wv + 1) / nw;
  auto tile_base = [&](int64_t t) {
    int64_t id = ids[t];
    id = id < 0 ? 0 : id >= nbuf ? nbuf - 1 : id;
    return reinterpret_cast<const u32x4*>(buf + id * TB);
  };
  auto tile = [&](int64_t t) { return tile_base(t) + lane; };
  uint32_t x = 0;
  int64_t t = lo;
  for (; t + TU <= hi; t += TU) {
    u32x4 v[TU][LPT];
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const u32x4* p = tile(t + u);
#pragma unroll
      for (int j = 0; j < LPT; ++j) v[u][j] = __builtin_nontemporal_load(p + 64 * j);
    }
#pragma unroll
    for (int u = 0; u < TU; ++u)
#pragma unroll
      for (int j = 0; j < LPT; ++j) x ^= v[u][j].x ^ v[u][j].y ^ v[u][j].z ^ v[u][j].w;
  }
  if (t < hi) {
    // the last, partial group with its loads in flight together; past hi every lane
    // reads the same 16 bytes (not counted)
    u32x4 v[TU][LPT];
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const bool real = t + u < hi;
      const u32x4* p = real ? tile(t + u) : tile_base(hi - 1);
#pragma unroll
      for (int j = 0; j < LPT; ++j) v[u][j] = __builtin_nontemporal_load(p + (real ? 64 * j : 0));
    }
#pragma unroll
    for (int u = 0; u < TU; ++u)
      if (t + u < hi) {
#pragma unroll
        for (int j = 0; j < LPT; ++j) x ^= v[u][j].x ^ v[u][j].y ^ v[u][j].z ^ v[u][j].w;
      }
  }
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t sh[kThreads / 64];
  if (lane == 0) sh[threadIdx.x / 64] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = sh[0] ^ sh[1] ^ sh[2] ^ sh[3];
}

__global__ __launch_bounds__(kThreads) void copy_kernel(uint4* __restrict__ dst,
                                                        const uint4* __restrict__ src,
                                                        int64_t pieces) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < pieces;
       i += (int64_t)gridDim.x * kThreads)
    dst[i] = src[i];
}

int probe_groups(int32_t waves_per_cu, int* groups) {
  int cus = 0;
  int rc = device_cus(&cus);
  if (rc != PA_OK) return rc;
  if (waves_per_cu <= 0) waves_per_cu = 4;
  *groups = cus * ((waves_per_cu + 3) / 4);
  return PA_OK;
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" size_t pa_probe_sink_bytes(int32_t waves_per_cu) {
  int groups = 0;
  if (probe_groups(waves_per_cu, &groups) != PA_OK) return 0;
  return (size_t)groups * sizeof(uint32_t);
}

extern "C" int pa_stream_read_probe(const void* buf, size_t bytes, void* sink,
                                    int32_t waves_per_cu, void* stream) {
  if (!buf || !sink) return fail(PA_EINVAL, "null pointer");
  if (bytes % 16 != 0 || !aligned16(buf)) return fail(PA_EINVAL, "bytes and buf must be 16-byte multiples");
  if (waves_per_cu < 0 || waves_per_cu > 32) return fail(PA_EINVAL, "waves_per_cu outside [0, 32]");
  int groups = 0;
  int rc = probe_groups(waves_per_cu, &groups);
  if (rc != PA_OK) return rc;
  hipLaunchKernelGGL(stream_read_kernel, dim3(groups), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint4*)buf, (int64_t)(bytes / 16), (uint32_t*)sink);
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}

extern "C" int pa_tile_read_probe(const void* buf, size_t buf_bytes, int32_t tile_bytes,
                                  const int32_t* tile_ids, int64_t n_ids, void* sink,
                                  void* stream) {
  if (!buf || !tile_ids || !sink) return fail(PA_EINVAL, "null pointer");
  if (tile_bytes != 2048 && tile_bytes != 4096 && tile_bytes != 8192 && tile_bytes != 16384)
    return fail(PA_EINVAL, "tile_bytes %d not 2048, 4096, 8192 or 16384", tile_bytes);
  if (!aligned16(buf) || buf_bytes < (size_t)tile_bytes || n_ids < 0)
    return fail(PA_EINVAL, "buf must be 16-byte aligned and hold a tile; n_ids >= 0");
  if (n_ids == 0) return ok();
  int groups = 0;
  int rc = probe_groups(4, &groups);
  if (rc != PA_OK) return rc;
  const int64_t nbuf = (int64_t)(buf_bytes / (size_t)tile_bytes);
  hipStream_t st = (hipStream_t)stream;
  const char* b = (const char*)buf;
  uint32_t* sk = (uint32_t*)sink;
  switch (tile_bytes) {
    case 2048: hipLaunchKernelGGL(tile_read_kernel<2048>, dim3(groups), dim3(kThreads), 0, st, b, nbuf, tile_ids, n_ids, sk); break;
    case 4096: hipLaunchKernelGGL(tile_read_kernel<4096>, dim3(groups), dim3(kThreads), 0, st, b, nbuf, tile_ids, n_ids, sk); break;
    case 8192: hipLaunchKernelGGL(tile_read_kernel<8192>, dim3(groups), dim3(kThreads), 0, st, b, nbuf, tile_ids, n_ids, sk); break;
    default: hipLaunchKernelGGL(tile_read_kernel<16384>, dim3(groups), dim3(kThreads), 0, st, b, nbuf, tile_ids, n_ids, sk); break;
  }
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}

extern "C" int pa_copy_probe(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src) return fail(PA_EINVAL, "null pointer");
  if (bytes % 16 != 0 || !aligned16(dst) || !aligned16(src))
    return fail(PA_EINVAL, "bytes, dst and src must be 16-byte multiples");
  int groups = 0;
  int rc = probe_groups(8, &groups);
  if (rc != PA_OK) return rc;
  hipLaunchKernelGGL(copy_kernel, dim3(groups), dim3(kThreads), 0, (hipStream_t)stream,
                     (uint4*)dst, (const uint4*)src, (int64_t)(bytes / 16));
  PA_HIP_CHECK(hipGetLastError());
  return ok();
}
