// Measurement probes of the benchmark (libda_probe.so): a plain streaming read and a plain
// copy. Not part of the attention library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "da_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per compute unit streams a contiguous share of the buffer, each thread
// keeping four 16-byte loads in flight (of the layouts tried on MI355X, the fastest
// plain streaming read: about 7.3 TB/s).
constexpr int kProbeThreads = 512, kProbeUnroll = 4;
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* src, size_t n16, float* sink) {
  const size_t b0 = n16 * blockIdx.x / gridDim.x, b1 = n16 * (blockIdx.x + 1) / gridDim.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = b0 + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < b1; i += kProbeUnroll * kProbeThreads) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < b1; i += kProbeThreads) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0 && x == 0x7fc00001u) sink[blockIdx.x] = 1.f;  // keeps the loads alive
}

__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* src, u32x4* dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

int da_read_probe(const void* src, size_t n_bytes, float* sink, void* stream) {
  if (!src || !sink || n_bytes == 0 || n_bytes % 16) return -1;
  const size_t n16 = n_bytes / 16;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  size_t blocks = cus < 1 ? 1 : (size_t)cus;
  if (blocks > 4096) blocks = 4096;
  if (blocks > n16) blocks = n16;
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int da_copy_probe(const void* src, void* dst, size_t n_bytes, void* stream) {
  if (!src || !dst || n_bytes == 0 || n_bytes % 16) return -1;
  const size_t n16 = n_bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  (void)hipGetLastError();
  hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                     (u32x4*)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
