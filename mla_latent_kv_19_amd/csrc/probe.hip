// HBM read-rate probe: the measurement the decode kernel's rate is set
// against, beside the published peak.  Not part of the attention path.
//
// Every thread reads 16-byte words grid-stride, eight loads in flight, and
// folds them into one word; the fold is stored only if it equals a magic
// value, so the loads cannot be elided and nothing is written in practice.
#include "mla_common.h"

namespace mla {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void hbm_read_probe_kernel(const u32x4* __restrict__ p, size_t n16,
                                                             uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[0] = 1u;
}

}  // namespace mla

// 512 work-groups of 256 threads (measured the fastest of 512..4096 for a
// 2.4 GB read on this part).
extern "C" hipError_t mla_launch_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                                hipStream_t stream) {
  const mla::u32x4* p = static_cast<const mla::u32x4*>(buf);
  size_t n16 = bytes / 16;
  void* args[] = {&p, &n16, &sink};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::hbm_read_probe_kernel), dim3(512),
                         dim3(256), args, 0, stream);
}
