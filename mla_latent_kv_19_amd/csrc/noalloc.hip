// Decode without any device allocation: split-KV attention followed by the
// log-sum-exp combine and W_UV, with the split partials kept in a buffer the
// library owns.
//
// The buffer is a file-scope device array of a fixed size, one copy per GPU
// the library runs on, held until the process ends.  Host code must never
// hand the array's name to a kernel or a copy: in host code that name is a
// host-side stand-in, not a device address.  Its device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// kept; the kernels then take it as an ordinary argument.
//
// Every call on one GPU shares that GPU's buffer, which keeps the last call's
// contents.  Nothing in it must start at zero (the attention kernel writes the
// partials and log-sum-exps of every (split, query row) pair the combine
// reads, empty splits included), but two calls that overlap on one GPU (on
// different streams, or from different host threads without ordering) race
// on it.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "mla.h"

extern "C" hipError_t mla_launch_decode_paged(const uint16_t* q_lat, const uint16_t* q_r,
                                              const uint16_t* kv, const int32_t* block_table,
                                              const int32_t* seq_lens, int B, int Tq, int max_blocks,
                                              float softmax_scale, int num_splits, float* part_o,
                                              float* part_lse, unsigned long long* clk,
                                              hipStream_t stream);
extern "C" hipError_t mla_launch_combine(const float* part_o, const float* part_lse,
                                         const uint16_t* w_uv, uint16_t* out, float* lse_out, int M,
                                         int S, hipStream_t stream);

namespace {

// (split, query row) pairs the buffer holds: one pair is a 128 x 512 fp32
// partial output (256 KiB) and 128 fp32 log-sum-exps.
constexpr size_t kPairs = MLA_NOALLOC_MAX_PAIRS;
constexpr size_t kPartOFloats = kPairs * 128 * 512;
constexpr size_t kPartLseFloats = kPairs * 128;
constexpr int kMaxDevices = 64;

}  // namespace

// 160 MiB of partial outputs followed by 320 KiB of log-sum-exps.
static __device__ __align__(256) float scratch[kPartOFloats + kPartLseFloats];

namespace {

std::mutex g_mutex;
float* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device

// Device address of this device's copy of `scratch` (looked up on the first
// call on the device, with it current), or null on a HIP error.
float* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || p == nullptr) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch[dev] = static_cast<float*>(p);
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" hipError_t mla_launch_decode_noalloc(const uint16_t* q_lat, const uint16_t* q_r,
                                                const uint16_t* kv, const int32_t* block_table,
                                                const int32_t* seq_lens, const uint16_t* w_uv,
                                                uint16_t* out, float* lse_out, int B, int Tq,
                                                int max_blocks, float softmax_scale,
                                                int num_splits, hipStream_t stream) {
  hipError_t err = hipSuccess;
  float* base = scratch_on_current_device(&err);
  if (base == nullptr) return err;
  float* part_o = base;
  float* part_lse = base + kPartOFloats;
  err = mla_launch_decode_paged(q_lat, q_r, kv, block_table, seq_lens, B, Tq, max_blocks,
                                softmax_scale, num_splits, part_o, part_lse, nullptr, stream);
  if (err != hipSuccess) return err;
  return mla_launch_combine(part_o, part_lse, w_uv, out, lse_out, B * Tq, num_splits, stream);
}
