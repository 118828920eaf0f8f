// A plain streaming read of a device buffer: the practical HBM ceiling that the decode kernels' fractions of the
// 8 TB/s peak are read against ("Where This Fits in the Inference Stack", "What Changes When KV Cache Is 4x
// Smaller": decode attention reads the whole cache from HBM each step, so the rate at which bytes stream in is
// its bound).
//
// Every lane reads 16-byte words with a grid stride, four loads in flight, folds them into one word and stores it
// only if it equals a value the data never makes it take (so the loads stay live): no other memory traffic.
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kStreamThreads = 512;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                                                     uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) + (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u && sink) sink[0] = acc;
}

}  // namespace

int launch_stream_read(const void *buf, int64_t bytes, int blocks, uint32_t *sink, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kStreamThreads), 0, stream, (const u32x4 *)buf,
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

}  // namespace tq
