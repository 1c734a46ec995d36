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
//   * append_gemm_kernel: one wave per (64 tokens, 64 outputs, K slice); A
//     (hidden states) and B (weight rows, the layer's [out, in] layout) are
//     both k-contiguous, so each MFMA 32x32x16 operand is one 16-byte load
//     per lane straight from global memory, four k-steps in flight; fp32
//     partial sums per K slice go to the workspace.  The K split is chosen so
//     that a handful of decode tokens still spreads the 8 MB weight over the
//     whole chip.
//   * append_finish_kernel: one wave per token: sums the K slices, RMSNorm of
//     the latent (wave reduction), RoPE of the rotary part (angle reduced in
//     float64: positions reach 10^5 and more), bf16 rounding, the cache write.
#include <cmath>

#include "mla_common.h"

namespace mla {

constexpr int kAppOut = 576;            // 512 latent + 64 rotary outputs
constexpr int kAppDc = 512;
constexpr int kAppNTiles = kAppOut / 64;

__global__ __launch_bounds__(64) void append_gemm_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w,
                                                         float* __restrict__ part, int M,
                                                         int d_model, int ksteps_per_split) {
  const int n_tile = blockIdx.x % kAppNTiles;
  const int m_tile = (blockIdx.x / kAppNTiles) % ((M + 63) / 64);
  const int split = blockIdx.x / (kAppNTiles * ((M + 63) / 64));
  const int lane = threadIdx.x, half = lane >> 5, l32 = lane & 31;
  const int ks0 = split * ksteps_per_split;
  const int ks1 = min(d_model / 16, ks0 + ksteps_per_split);

  // Operand rows: tokens m0 + 32tb + l32 (clamped into range; never stored
  // past M), outputs n0 + 32ob + l32; 8 consecutive k at 16ks + 8*half.
  const int m0 = m_tile * 64, n0 = n_tile * 64;
  const uint16_t* arow[2];
  const uint16_t* brow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    arow[t] = x + (size_t)min(m0 + 32 * t + l32, M - 1) * d_model + 8 * half;
    brow[t] = w + (size_t)(n0 + 32 * t + l32) * d_model + 8 * half;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  // Operands of k-step ks: a[0..1], b[0..1]; five register stages, four
  // k-steps of loads in flight (a K slice is often only 8 k-steps long, so
  // latency, not bandwidth, sets its time).
  constexpr int kStages = 5, kAhead = 4;
  bf16x8 op[kStages][4];
  auto load = [&](int stage, int ks) {
    op[stage][0] = ld_global_bf16x8(arow[0] + 16 * ks);
    op[stage][1] = ld_global_bf16x8(arow[1] + 16 * ks);
    op[stage][2] = ld_global_bf16x8(brow[0] + 16 * ks);
    op[stage][3] = ld_global_bf16x8(brow[1] + 16 * ks);
  };
  const int n = ks1 - ks0;
#pragma unroll
  for (int u = 0; u < kAhead; ++u)
    if (u < n) load(u, ks0 + u);
  for (int j = 0; j < n; j += kStages) {
#pragma unroll
    for (int u = 0; u < kStages; ++u) {
      if (j + u < n) {
        if (j + u + kAhead < n) load((u + kAhead) % kStages, ks0 + j + u + kAhead);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(op[u][a], op[u][2 + b], acc[a][b]);
      }
    }
  }

  // acc[a][b][r]: token m0 + 32a + 8(r/4) + 4*half + r%4, output n0 + 32b + l32.
  float* dst = part + (size_t)split * M * kAppOut;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 32 * a + 8 * (r >> 2) + 4 * half + (r & 3);
      if (m < M) {
#pragma unroll
        for (int b = 0; b < 2; ++b) dst[(size_t)m * kAppOut + n0 + 32 * b + l32] = acc[a][b][r];
      }
    }
}

__global__ __launch_bounds__(64) void append_finish_kernel(
    const float* __restrict__ part, const uint16_t* __restrict__ gamma,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ block_table, uint16_t* __restrict__ kv, int M, int splits,
    int max_blocks, float eps, double log_theta) {
  const int m = blockIdx.x;
  const int lane = threadIdx.x;
  // Output n = lane + 64j: j < 8 latent, j = 8 rotary value lane.
  float v[9];
#pragma unroll
  for (int j = 0; j < 9; ++j) v[j] = 0.f;
  // Slices in groups of 8, so that 72 loads are in flight at once.
  int s = 0;
  for (; s + 8 <= splits; s += 8) {
    float t[8][9];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* p = part + ((size_t)(s + u) * M + m) * kAppOut + lane;
#pragma unroll
      for (int j = 0; j < 9; ++j) t[u][j] = p[64 * j];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int j = 0; j < 9; ++j) v[j] += t[u][j];
  }
  for (; s < splits; ++s) {
    const float* p = part + ((size_t)s * M + m) * kAppOut + lane;
#pragma unroll
    for (int j = 0; j < 9; ++j) v[j] += p[64 * j];
  }
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

// K split for M tokens: enough work-groups to cover the chip (~512 waves).
extern "C" int mla_append_splits(int M, int d_model) {
  const int m_tiles = (M + 63) / 64;
  const int ksteps = d_model / 16;
  int s = (512 + m_tiles * mla::kAppNTiles - 1) / (m_tiles * mla::kAppNTiles);
  s = s < 1 ? 1 : (s > ksteps ? ksteps : s);
  const int per = (ksteps + s - 1) / s;
  return (ksteps + per - 1) / per;
}

extern "C" hipError_t mla_launch_cache_append(const uint16_t* x, const uint16_t* w_kv,
                                              const uint16_t* gamma, const int32_t* seq_idx,
                                              const int32_t* positions, const int32_t* block_table,
                                              uint16_t* kv, float* workspace, int M, int d_model,
                                              int max_blocks, float eps, float theta,
                                              hipStream_t stream) {
  const int splits = mla_append_splits(M, d_model);
  const int ksteps = d_model / 16;
  int per = (ksteps + splits - 1) / splits;
  const int m_tiles = (M + 63) / 64;
  {
    void* args[] = {&x, &w_kv, &workspace, &M, &d_model, &per};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&mla::append_gemm_kernel),
                                         dim3(m_tiles * mla::kAppNTiles * splits), dim3(64), args,
                                         0, stream);
    if (e != hipSuccess) return e;
  }
  int s = splits;
  double log_theta = std::log((double)theta);
  void* args[] = {&workspace, &gamma, &seq_idx, &positions, &block_table, &kv, &M, &s,
                  &max_blocks, &eps, &log_theta};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::append_finish_kernel), dim3(M),
                         dim3(64), args, 0, stream);
}
