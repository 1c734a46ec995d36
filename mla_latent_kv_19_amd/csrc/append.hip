// Cache append: the latent and rotary key of M new tokens, written into the
// paged cache.
//
// What it computes ("DeepSeek-V3" llm-vis explorer, boxes "KV latent
// compression" and "Rotary position embedding (RoPE)"; "Teardown:
// DeepSeek-V3", section 4: only c and k_R are cached): for token m with hidden
// state x_m, sequence b_m and position p_m,
//   [c_raw | k_raw] = W_kv x_m                       (d_model -> 512 + 64)
//   c   = c_raw / sqrt(mean(c_raw^2) + eps) * gamma   (RMSNorm over 512)
//   k_R = pairs (k_raw[2i], k_raw[2i+1]) rotated by p_m * theta^(-2i/64)
// stored as the cache row c | k_R of token p_m of sequence b_m.
//
// Two kernels (MI355X):
//   * the split-K projection of linear.hip (fp32 partial sums per K slice of
//     the 7168-wide hidden state into the workspace);
//   * append_finish_kernel: four waves per token sum the K slices (every
//     fourth each, all loads in flight), then one wave does the RMSNorm of the
//     latent (wave reduction), RoPE of the rotary part (angle reduced in
//     float64: positions reach 10^5 and more), bf16 rounding, the cache write.
#include <cmath>

#include "mla_common.h"

extern "C" int mla_linear_splits(int M, int N, int K);
extern "C" hipError_t mla_launch_linear_splitk(const uint16_t* x, const uint16_t* w, float* part,
                                               int M, int N, int K, int splits,
                                               hipStream_t stream);

namespace mla {

constexpr int kAppOut = 576;            // 512 latent + 64 rotary outputs
constexpr int kAppDc = 512;

__global__ __launch_bounds__(256) void append_finish_kernel(
    const float* __restrict__ part, const uint16_t* __restrict__ gamma,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ block_table, uint16_t* __restrict__ kv, int M, int splits,
    int max_blocks, float eps, double log_theta) {
  __shared__ float red[4][kAppOut];
  const int m = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // Output n = lane + 64j: j < 8 latent, j = 8 rotary value lane.  Wave w sums
  // slices w, w + 4, ..., eight of them per batch (all 72 loads in flight), so
  // up to 32 slices take one memory round trip; then wave 0 adds the four.
  float v[9];
#pragma unroll
  for (int j = 0; j < 9; ++j) v[j] = 0.f;
  for (int s0 = w; s0 < splits; s0 += 32) {
    float t[8][9];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sl = min(s0 + 4 * u, splits - 1);
      const float* p = part + ((size_t)sl * M + m) * kAppOut + lane;
#pragma unroll
      for (int j = 0; j < 9; ++j) t[u][j] = p[64 * j];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = s0 + 4 * u < splits;
#pragma unroll
      for (int j = 0; j < 9; ++j) v[j] += ok ? t[u][j] : 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < 9; ++j) red[w][lane + 64 * j] = v[j];
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int j = 0; j < 9; ++j)
    v[j] = (red[0][lane + 64 * j] + red[1][lane + 64 * j]) + (red[2][lane + 64 * j] + red[3][lane + 64 * j]);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float inv_rms = 1.f / sqrtf(ss / kAppDc + eps);

  // RoPE: lane = 2i (+1) holds element 2i (2i+1) of the rotary part.
  const int pos = positions[m];
  const int i = lane >> 1;
  const double ang = fmod((double)pos * exp(-(2.0 * i / 64.0) * log_theta), 6.283185307179586);
  const float cs = cosf((float)ang), sn = sinf((float)ang);
  const float other = __shfl_xor(v[8], 1);
  const float rot = (lane & 1) ? other * sn + v[8] * cs : v[8] * cs - other * sn;

  const int blk = block_table[(size_t)seq_idx[m] * max_blocks + (pos >> 6)];
  uint16_t* row = kv + ((size_t)blk * 64 + (pos & 63)) * kAppOut;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float g = __builtin_bit_cast(float, (uint32_t)gamma[lane + 64 * j] << 16);
    row[lane + 64 * j] = __builtin_bit_cast(uint16_t, (__bf16)(v[j] * inv_rms * g));
  }
  row[kAppDc + lane] = __builtin_bit_cast(uint16_t, (__bf16)rot);
}

}  // namespace mla

extern "C" hipError_t mla_launch_cache_append(const uint16_t* x, const uint16_t* w_kv,
                                              const uint16_t* gamma, const int32_t* seq_idx,
                                              const int32_t* positions, const int32_t* block_table,
                                              uint16_t* kv, float* workspace, int M, int d_model,
                                              int max_blocks, float eps, float theta,
                                              hipStream_t stream) {
  const int splits = mla_linear_splits(M, mla::kAppOut, d_model);
  {
    const hipError_t e = mla_launch_linear_splitk(x, w_kv, workspace, M, mla::kAppOut, d_model,
                                                  splits, stream);
    if (e != hipSuccess) return e;
  }
  int s = splits;
  double log_theta = std::log((double)theta);
  void* args[] = {&workspace, &gamma, &seq_idx, &positions, &block_table, &kv, &M, &s,
                  &max_blocks, &eps, &log_theta};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::append_finish_kernel), dim3(M),
                         dim3(256), args, 0, stream);
}
