// Split-K projection y = x W^T for the small-M (decode) and medium-M shapes of
// the attention block's linear layers ("Teardown: DeepSeek-V3", section 4,
// table of attention weights: W_DQ 7168 -> 1536, W_UQ 1536 -> 128 x (128+64),
// W_DKV and W_KR 7168 -> 512+64, W_O 128 x 128 -> 7168).
//
//   part[s, m, n] = sum over k in K slice s of x[m, k] * w[n, k]
//
// x is [M, K] and w is a linear layer's [N, K] weight, both bf16 and
// k-contiguous, so every MFMA 32x32x16 operand is one 16-byte load per lane
// straight from global memory: one wave per (64 rows, 64 outputs, K slice),
// four k-steps of loads in flight.  The K split is chosen so that about 512
// waves cover the chip even for a single decode batch, which streams each
// weight once at HBM rate; the callers' finish kernels sum the slices.
#include "mla_common.h"

namespace mla {

__global__ __launch_bounds__(64) void linear_splitk_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w,
                                                           float* __restrict__ part, int M, int N,
                                                           int K, int ksteps_per_split) {
  const int n_tiles = N / 64, m_tiles = (M + 63) / 64;
  const int n_tile = blockIdx.x % n_tiles;
  const int m_tile = (blockIdx.x / n_tiles) % m_tiles;
  const int split = blockIdx.x / (n_tiles * m_tiles);
  const int lane = threadIdx.x, half = lane >> 5, l32 = lane & 31;
  const int ks0 = split * ksteps_per_split;
  const int ks1 = min(K / 16, ks0 + ksteps_per_split);

  // Operand rows: rows m0 + 32t + l32 (clamped into range; never stored past
  // M), outputs n0 + 32t + l32; 8 consecutive k at 16ks + 8*half.
  const int m0 = m_tile * 64, n0 = n_tile * 64;
  const uint16_t* arow[2];
  const uint16_t* brow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    arow[t] = x + (size_t)min(m0 + 32 * t + l32, M - 1) * K + 8 * half;
    brow[t] = w + (size_t)(n0 + 32 * t + l32) * K + 8 * half;
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

  // acc[a][b][r]: row m0 + 32a + 8(r/4) + 4*half + r%4, output n0 + 32b + l32.
  float* dst = part + (size_t)split * M * N;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 32 * a + 8 * (r >> 2) + 4 * half + (r & 3);
      if (m < M) {
#pragma unroll
        for (int b = 0; b < 2; ++b) dst[(size_t)m * N + n0 + 32 * b + l32] = acc[a][b][r];
      }
    }
}

}  // namespace mla

// K slices for an [M, K] x [N, K]^T product: about 512 waves in total, at
// least one k-step (16 values) per slice.  N must be a multiple of 64.
extern "C" int mla_linear_splits(int M, int N, int K) {
  const int tiles = ((M + 63) / 64) * (N / 64);
  const int ksteps = K / 16;
  int s = (512 + tiles - 1) / tiles;
  s = s < 1 ? 1 : (s > ksteps ? ksteps : s);
  const int per = (ksteps + s - 1) / s;
  return (ksteps + per - 1) / per;
}

extern "C" hipError_t mla_launch_linear_splitk(const uint16_t* x, const uint16_t* w, float* part,
                                               int M, int N, int K, int splits,
                                               hipStream_t stream) {
  const int ksteps = K / 16;
  int per = (ksteps + splits - 1) / splits;
  void* args[] = {&x, &w, &part, &M, &N, &K, &per};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::linear_splitk_kernel),
                         dim3(((M + 63) / 64) * (N / 64) * splits), dim3(64), args, 0, stream);
}
