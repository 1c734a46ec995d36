// Split-K projection y = x W^T for the small-M (decode) and medium-M shapes of
// the attention block's linear layers ("Teardown: DeepSeek-V3", section 4,
// table of attention weights: W_DQ 7168 -> 1536, W_UQ 1536 -> 128 x (128+64),
// W_DKV and W_KR 7168 -> 512+64, W_O 128 x 128 -> 7168).
//
//   part[s, m, n] = sum over k in K slice s of x[m, k] * w[n, k]
//
// x is [M, K] and w is a linear layer's [N, K] weight, both bf16 and
// k-contiguous.  Three kernels, one output contract (the callers' finish
// kernels sum the slices):
//  * linear_stream_kernel, M <= 64 (a decode batch), K a multiple of 64: the
//    weight is the traffic.  A work-group of 4 waves takes 256 outputs and a
//    K slice; chunks of 64 k of the weight rows (256 x 128 B) and of x
//    (64 x 128 B) stream into a 3-stage LDS ring with direct-to-LDS loads, each
//    load instruction covering 8 rows x 128 contiguous bytes, and the MFMA
//    operands are read from LDS (chunk swizzle: conflict-free).
//  * linear_tile_kernel, M > 64 with N a multiple of 192 and K of 64 (a
//    prefill chunk): MFMA-bound.  A work-group of 4 waves (2 x 2) takes a
//    128 x 192 output tile and a K slice; 64-k chunks of the x and weight
//    rows (16 + 24 KB) go through the same kind of 3-stage LDS ring, each wave
//    computing 64 x 96 outputs (6 MFMA blocks per k-step from 5 operand reads).
//  * linear_splitk_kernel otherwise: one wave per (64 rows, 64 outputs, K
//    slice), every MFMA 32x32x16 operand one 16-byte load per lane straight
//    from global memory, four k-steps of loads in flight.
// The K split is chosen so that a few hundred work-groups cover the chip even
// for a single decode batch.
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

constexpr int kLsThreads = 256;                          // 4 waves
constexpr int kLsN = 256;                                // outputs per work-group
constexpr int kLsKc = 64;                                // k per chunk
constexpr int kLsStages = 3;
constexpr int kLsWBytes = kLsN * kLsKc * 2;              // 32768
constexpr int kLsXBytes = 64 * kLsKc * 2;                // 8192
constexpr int kLsStageBytes = kLsWBytes + kLsXBytes;     // 40960
constexpr int kLsWLoads = kLsWBytes / 16 / kLsThreads;   // 8 per thread per chunk
constexpr int kLsXLoads = kLsXBytes / 16 / kLsThreads;   // 2
constexpr int kLsLoads = kLsWLoads + kLsXLoads;          // 10
static_assert(kLsWLoads * 16 * kLsThreads == kLsWBytes && kLsXLoads * 16 * kLsThreads == kLsXBytes,
              "chunk split");

// A chunk row is 8 sixteen-byte pieces (128 B); piece c of row r sits at
// position c ^ ((r >> 1) & 7), so the 16 rows that a 16-lane group of an
// operand read touches fall on 16 distinct 4-bank groups.
__device__ __forceinline__ int ls_swz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(kLsThreads, 1) void linear_stream_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ part,
    int M, int N, int K, int chunks_per_split) {
  extern __shared__ __attribute__((aligned(16))) unsigned char ls_smem[];
  lds_u8* smem = to_lds(ls_smem);
  const int n_tiles = (N + kLsN - 1) / kLsN;
  const int n0 = (blockIdx.x % n_tiles) * kLsN;
  const int split = blockIdx.x / n_tiles;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = split * chunks_per_split;
  const int nch = min(K / kLsKc, c0 + chunks_per_split) - c0;

  // Load sources, fixed but for the chunk's k offset: slot = it * 256 + tid
  // fills LDS bytes [16 slot, 16 slot + 16) of its region: row slot / 8,
  // position slot % 8, which holds piece (slot % 8) ^ ls_swz(row).  Rows past
  // N or M read a valid row (their results are never stored).
  const uint16_t* wsrc[kLsWLoads];
  const uint16_t* xsrc[kLsXLoads];
#pragma unroll
  for (int it = 0; it < kLsWLoads; ++it) {
    const int slot = it * kLsThreads + tid, r = slot >> 3;
    wsrc[it] = w + (size_t)min(n0 + r, N - 1) * K + (((slot & 7) ^ ls_swz(r)) * 8) + (size_t)c0 * kLsKc;
  }
#pragma unroll
  for (int it = 0; it < kLsXLoads; ++it) {
    const int slot = it * kLsThreads + tid, r = slot >> 3;
    xsrc[it] = x + (size_t)min(r, M - 1) * K + (((slot & 7) ^ ls_swz(r)) * 8) + (size_t)c0 * kLsKc;
  }
  auto issue = [&](int ci) {
    lds_u8* st = smem + (ci % kLsStages) * kLsStageBytes + (tid & ~63) * 16;
#pragma unroll
    for (int it = 0; it < kLsWLoads; ++it)
      g2lds16_opaque(wsrc[it] + ci * kLsKc, st + it * kLsThreads * 16);
#pragma unroll
    for (int it = 0; it < kLsXLoads; ++it)
      g2lds16_opaque(xsrc[it] + ci * kLsKc, st + kLsWBytes + it * kLsThreads * 16);
  };

  // Operand reads: x rows 32a + l32 (A), weight rows 64 wave + 32t + l32 (B);
  // k-step ks of a chunk is piece 2ks + half of the row.
  int xoff[2], woff[2], xsw[2], wsw[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int xr = 32 * t + l32, wr = 64 * wave + 32 * t + l32;
    xoff[t] = kLsWBytes + xr * 128;
    woff[t] = wr * 128;
    xsw[t] = ls_swz(xr);
    wsw[t] = ls_swz(wr);
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  issue(0);
  if (nch > 1) issue(1);
  for (int ci = 0; ci < nch; ++ci) {
    // Chunk ci has landed for every thread; every wave is done with chunk
    // ci-1, whose stage then takes chunk ci+2.
    if (ci + 1 < nch) wait_vmcnt<kLsLoads>(); else wait_vmcnt<0>();
    lds_barrier();
    if (ci + 2 < nch) issue(ci + 2);
    const lds_u8* st = smem + (ci % kLsStages) * kLsStageBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int pc = 2 * ks + half;
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = ld_lds_bf16x8(st + xoff[t] + ((pc ^ xsw[t]) * 16));
        bv[t] = ld_lds_bf16x8(st + woff[t] + ((pc ^ wsw[t]) * 16));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(av[a], bv[b], acc[a][b]);
    }
  }

  // acc[a][b][r]: row 32a + 8(r/4) + 4*half + r%4, output n0 + 64 wave + 32b + l32.
  float* dst = part + (size_t)split * M * N;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int n = n0 + 64 * wave + 32 * b + l32;
    if (n >= N) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * a + 8 * (r >> 2) + 4 * half + (r & 3);
        if (m < M) dst[(size_t)m * N + n] = acc[a][b][r];
      }
  }
}


constexpr int kLtBM = 128, kLtBN = 192;
constexpr int kLtXBytes = kLtBM * kLsKc * 2;             // 16384
constexpr int kLtWBytes = kLtBN * kLsKc * 2;             // 24576
constexpr int kLtStageBytes = kLtXBytes + kLtWBytes;     // 40960
constexpr int kLtXLoads = kLtXBytes / 16 / kLsThreads;   // 4 per thread per chunk
constexpr int kLtWLoads = kLtWBytes / 16 / kLsThreads;   // 6
constexpr int kLtLoads = kLtXLoads + kLtWLoads;          // 10
static_assert(kLtXLoads * 16 * kLsThreads == kLtXBytes && kLtWLoads * 16 * kLsThreads == kLtWBytes,
              "tile chunk split");

__global__ __launch_bounds__(kLsThreads, 1) void linear_tile_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ part,
    int M, int N, int K, int chunks_per_split) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lt_smem[];
  lds_u8* smem = to_lds(lt_smem);
  const int n_tiles = N / kLtBN, m_tiles = (M + kLtBM - 1) / kLtBM;
  const int n0 = (blockIdx.x % n_tiles) * kLtBN;
  const int m0 = ((blockIdx.x / n_tiles) % m_tiles) * kLtBM;
  const int split = blockIdx.x / (n_tiles * m_tiles);
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;       // rows 64 wm.., outputs 96 wn..
  const int c0 = split * chunks_per_split;
  const int nch = min(K / kLsKc, c0 + chunks_per_split) - c0;

  // Load sources as in linear_stream_kernel (rows past M read a valid row;
  // their results are never stored).
  const uint16_t* xsrc[kLtXLoads];
  const uint16_t* wsrc[kLtWLoads];
#pragma unroll
  for (int it = 0; it < kLtXLoads; ++it) {
    const int slot = it * kLsThreads + tid, r = slot >> 3;
    xsrc[it] = x + (size_t)min(m0 + r, M - 1) * K + (((slot & 7) ^ ls_swz(r)) * 8) + (size_t)c0 * kLsKc;
  }
#pragma unroll
  for (int it = 0; it < kLtWLoads; ++it) {
    const int slot = it * kLsThreads + tid, r = slot >> 3;
    wsrc[it] = w + (size_t)(n0 + r) * K + (((slot & 7) ^ ls_swz(r)) * 8) + (size_t)c0 * kLsKc;
  }
  auto issue = [&](int ci) {
    lds_u8* st = smem + (ci % kLsStages) * kLtStageBytes + (tid & ~63) * 16;
#pragma unroll
    for (int it = 0; it < kLtXLoads; ++it)
      g2lds16_opaque(xsrc[it] + ci * kLsKc, st + it * kLsThreads * 16);
#pragma unroll
    for (int it = 0; it < kLtWLoads; ++it)
      g2lds16_opaque(wsrc[it] + ci * kLsKc, st + kLtXBytes + it * kLsThreads * 16);
  };

  // Operand reads: x rows 64 wm + 32a + l32 (A), weight rows 96 wn + 32b + l32 (B).
  int xoff[2], xsw[2], woff[3], wsw[3];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int r = 64 * wm + 32 * a + l32;
    xoff[a] = r * 128;
    xsw[a] = ls_swz(r);
  }
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const int r = 96 * wn + 32 * b + l32;
    woff[b] = kLtXBytes + r * 128;
    wsw[b] = ls_swz(r);
  }
  f32x16 acc[2][3];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 3; ++b) acc[a][b] = f32x16{};

  issue(0);
  if (nch > 1) issue(1);
  for (int ci = 0; ci < nch; ++ci) {
    // Chunk ci has landed for every thread; every wave is done with chunk
    // ci-1, whose stage then takes chunk ci+2.
    if (ci + 1 < nch) wait_vmcnt<kLtLoads>(); else wait_vmcnt<0>();
    lds_barrier();
    if (ci + 2 < nch) issue(ci + 2);
    const lds_u8* st = smem + (ci % kLsStages) * kLtStageBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int pc = 2 * ks + half;
      bf16x8 av[2], bv[3];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = ld_lds_bf16x8(st + xoff[a] + ((pc ^ xsw[a]) * 16));
#pragma unroll
      for (int b = 0; b < 3; ++b) bv[b] = ld_lds_bf16x8(st + woff[b] + ((pc ^ wsw[b]) * 16));
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) acc[a][b] = mfma32(av[a], bv[b], acc[a][b]);
    }
  }

  // acc[a][b][r]: row m0 + 64 wm + 32a + 8(r/4) + 4*half + r%4,
  // output n0 + 96 wn + 32b + l32.
  float* dst = part + (size_t)split * M * N;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 64 * wm + 32 * a + 8 * (r >> 2) + 4 * half + (r & 3);
      if (m < M) {
#pragma unroll
        for (int b = 0; b < 3; ++b) dst[(size_t)m * N + n0 + 96 * wn + 32 * b + l32] = acc[a][b][r];
      }
    }
}
}  // namespace mla

// Which kernel takes an [M, K] x [N, K]^T product.
static bool use_stream(int M, int N, int K) {
  return M >= 1 && M <= 64 && K % mla::kLsKc == 0 && N % 64 == 0;
}
static bool use_tile(int M, int N, int K) {
  return M > 64 && K % mla::kLsKc == 0 && N % mla::kLtBN == 0;
}

// K slices for an [M, K] x [N, K]^T product.  Tile kernel: about 192
// work-groups, at least 8 chunks per slice.  Streaming kernel: at most 256
// work-groups (one round), at least 4 chunks (256 k) per slice.  Split-K kernel: about
// 512 waves, at least one k-step (16 values) per slice.  N must be a multiple
// of 64.
extern "C" int mla_linear_splits(int M, int N, int K) {
  if (use_tile(M, N, K)) {
    // About 192 work-groups (fewer K slices beat more work-groups here: the
    // slices' partial sums are traffic too), at least 8 chunks (512 k) per slice.
    const int tiles = (N / mla::kLtBN) * ((M + mla::kLtBM - 1) / mla::kLtBM);
    const int chunks = K / mla::kLsKc;
    int s = (192 + tiles - 1) / tiles;
    const int smax = (chunks + 7) / 8;
    s = s < 1 ? 1 : (s > smax ? smax : s);
    const int per = (chunks + s - 1) / s;
    return (chunks + per - 1) / per;
  }
  if (use_stream(M, N, K)) {
    // At most one round of work-groups on the 256 compute units (one per CU:
    // the ring takes 120 KB of LDS): a partial second round leaves most CUs
    // idle while it runs (W_O 64 x 16384 -> 7168: 9 slices 51 us, 14 slices
    // 60 us; W_UQ 1536 -> 24576: 2 slices 22 us, 4 slices 26 us).
    const int tiles = (N + mla::kLsN - 1) / mla::kLsN;
    const int chunks = K / mla::kLsKc;
    int s = 256 / tiles;
    const int smax = (chunks + 3) / 4;
    s = s < 1 ? 1 : (s > smax ? smax : s);
    const int per = (chunks + s - 1) / s;
    return (chunks + per - 1) / per;
  }
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
  if (use_tile(M, N, K)) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&mla::linear_tile_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize, mla::kLsStages * mla::kLtStageBytes);
    if (attr != hipSuccess) return attr;
    const int chunks = K / mla::kLsKc;
    int per = (chunks + splits - 1) / splits;
    void* args[] = {&x, &w, &part, &M, &N, &K, &per};
    const int tiles = (N / mla::kLtBN) * ((M + mla::kLtBM - 1) / mla::kLtBM);
    return hipLaunchKernel(reinterpret_cast<const void*>(&mla::linear_tile_kernel),
                           dim3(tiles * splits), dim3(mla::kLsThreads), args,
                           mla::kLsStages * mla::kLtStageBytes, stream);
  }
  if (use_stream(M, N, K)) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&mla::linear_stream_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize, mla::kLsStages * mla::kLsStageBytes);
    if (attr != hipSuccess) return attr;
    const int chunks = K / mla::kLsKc;
    int per = (chunks + splits - 1) / splits;
    void* args[] = {&x, &w, &part, &M, &N, &K, &per};
    const int n_tiles = (N + mla::kLsN - 1) / mla::kLsN;
    return hipLaunchKernel(reinterpret_cast<const void*>(&mla::linear_stream_kernel),
                           dim3(n_tiles * splits), dim3(mla::kLsThreads), args,
                           mla::kLsStages * mla::kLsStageBytes, stream);
  }
  const int ksteps = K / 16;
  int per = (ksteps + splits - 1) / splits;
  void* args[] = {&x, &w, &part, &M, &N, &K, &per};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::linear_splitk_kernel),
                         dim3(((M + 63) / 64) * (N / 64) * splits), dim3(64), args, 0, stream);
}
