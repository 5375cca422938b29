// Measurement helpers: the HBM read rate a plain streaming kernel reaches on this
// device (the practical ceiling next to the 8 TB/s specification), and a copy of
// known size used to calibrate the memory-traffic counters.
#include "device.hpp"

namespace pagedkv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// Each thread reads 16-byte pieces with a grid-wide stride, kUnroll loads in flight.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ buf,
                                                               int64_t pieces,
                                                               uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kUnroll - 1) * stride < pieces; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) v[j] = buf[i + j * stride];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < pieces; i += stride) {
    const uint4 v = buf[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t sh[kThreads / 64];
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x / 64] = x;
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
  if (waves_per_cu <= 0) waves_per_cu = 8;
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
