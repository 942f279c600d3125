// Plain HBM streams for measurement: the achievable read, write and copy
// rates of the device, measured with code of this library (no vendor
// kernels), as the ceiling the HBM-bound kernels of the layer are read
// against.  Each workgroup of 256 threads moves 32 KB blocks: 8 independent
// 16-byte loads (or stores) per thread, lane-contiguous, so a wave's access
// is 1 KB of whole cache lines and every thread keeps 8 loads in flight;
// blocks are walked grid-stride.  The read stream folds what it loaded into
// one word per thread (written to `sink`, so the loads are not removed).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kProbeThreads = 256, kProbeUnroll = 8;
constexpr int64_t kBlock = (int64_t)kProbeThreads * kProbeUnroll * 16;  // 32 KB

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4_t* src, int64_t n16, uint32_t* sink) {
  const int64_t per = kBlock / 16;
  uint32_t acc = 0;
  for (int64_t b = blockIdx.x; b * per < n16; b += gridDim.x) {
    const int64_t base = b * per + threadIdx.x;
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) {
      const int64_t i = base + j * kProbeThreads;
      v[j] = i < n16 ? src[i] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kProbeThreads) void probe_write_kernel(u32x4_t* dst, int64_t n16) {
  const int64_t per = kBlock / 16;
  const u32x4_t v = {blockIdx.x, threadIdx.x, 0u, 0u};
  for (int64_t b = blockIdx.x; b * per < n16; b += gridDim.x) {
    const int64_t base = b * per + threadIdx.x;
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) {
      const int64_t i = base + j * kProbeThreads;
      if (i < n16) __builtin_nontemporal_store(v, dst + i);
    }
  }
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const u32x4_t* src, u32x4_t* dst, int64_t n16) {
  const int64_t per = kBlock / 16;
  for (int64_t b = blockIdx.x; b * per < n16; b += gridDim.x) {
    const int64_t base = b * per + threadIdx.x;
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) {
      const int64_t i = base + j * kProbeThreads;
      v[j] = i < n16 ? src[i] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) {
      const int64_t i = base + j * kProbeThreads;
      if (i < n16) __builtin_nontemporal_store(v[j], dst + i);
    }
  }
}

}  // namespace

int launch_probe(int kind, const void* src, void* dst, int64_t bytes, int wgs, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0 || wgs <= 0) return 0;
  if (kind == 0)
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)wgs), dim3(kProbeThreads), 0, stream, (const u32x4_t*)src, n16,
                       (uint32_t*)dst);
  else if (kind == 1)
    hipLaunchKernelGGL(probe_write_kernel, dim3((unsigned)wgs), dim3(kProbeThreads), 0, stream, (u32x4_t*)dst, n16);
  else
    hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)wgs), dim3(kProbeThreads), 0, stream, (const u32x4_t*)src,
                       (u32x4_t*)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace moe
