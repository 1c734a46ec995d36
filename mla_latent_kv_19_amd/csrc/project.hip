// The attention block's projections around the latent attention.
//
// Query side ("DeepSeek-V3" llm-vis explorer, "Query low-rank projection" and
// "Rotary position embedding (RoPE)"; "Teardown: DeepSeek-V3", section 4,
// c_q = W_DQ h and q_C = W_UQ c_q with W_UQ 1536 -> 128 x (128 + 64)):
//   c_q  = W_DQ x                       (7168 -> 1536)
//   c_q' = RMSNorm(c_q) * gamma_q
//   per head h: [q_C | q_R'] = (W_UQ c_q')[192h .. 192h + 191]   (128 | 64)
//   q_R  = q_R' with pairs (2i, 2i+1) rotated by pos * theta^(-2i/64)
// Output side ("Output projection": the 128 value heads, concatenated, are
// mapped back to the 7168-wide residual stream, no bias):
//   y = W_O o                           (128 x 128 -> 7168)
//
// Each product is the split-K projection of linear.hip; the kernels here sum
// its K slices and apply what follows the product: RMSNorm, the per-head split
// and RoPE (64 lanes per head), or a plain bf16 rounding.  RMSNorm's per-row
// factor commutes with the second product, so it is applied after it:
//   W_UQ (gamma * c_q / rms) = (W_UQ (gamma * c_q)) / rms,
// and the sum over c_q's K slices runs as one wave per 256 columns, writing
// bf16(gamma * c_q) and the block's sum of squares; the split + RoPE kernel
// then scales by 1 / rms of its row.
#include <cmath>

#include "mla_common.h"

extern "C" int mla_linear_splits(int M, int N, int K);
extern "C" hipError_t mla_launch_linear_splitk(const uint16_t* x, const uint16_t* w, float* part,
                                               int M, int N, int K, int splits,
                                               hipStream_t stream);

namespace mla {

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// One wave per (row m, 256 columns): c = sum_s part[s, m, n] over the K
// slices (16-byte loads, 16 slices in flight per lane), cq[m, n] =
// bf16(gamma[n] * c) and ssq[m, blk] = sum over the block's columns of c^2.
// N is a multiple of 256.
__global__ __launch_bounds__(64) void qnorm_sum_kernel(const float* __restrict__ part, int splits,
                                                       int M, int N,
                                                       const uint16_t* __restrict__ gamma,
                                                       uint16_t* __restrict__ cq,
                                                       float* __restrict__ ssq) {
  const int nb = N / 256;
  const int m = blockIdx.x / nb, blk = blockIdx.x - m * nb;
  const int n = blk * 256 + 4 * threadIdx.x;
  const size_t stride = (size_t)M * N;
  const float* p = part + (size_t)m * N + n;
  float4 c = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < splits; s0 += 16) {
    float4 t[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      t[u] = (s0 + u < splits) ? *reinterpret_cast<const float4*>(p + (size_t)(s0 + u) * stride)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      c.x += t[u].x;
      c.y += t[u].y;
      c.z += t[u].z;
      c.w += t[u].w;
    }
  }
  bf16x4 o;
  o[0] = (__bf16)(c.x * bf16_to_f32(gamma[n]));
  o[1] = (__bf16)(c.y * bf16_to_f32(gamma[n + 1]));
  o[2] = (__bf16)(c.z * bf16_to_f32(gamma[n + 2]));
  o[3] = (__bf16)(c.w * bf16_to_f32(gamma[n + 3]));
  *reinterpret_cast<bf16x4*>(cq + (size_t)m * N + n) = o;
  float q = c.x * c.x + c.y * c.y + c.z * c.z + c.w * c.w;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) q += __shfl_xor(q, off);
  if (threadIdx.x == 0) ssq[blockIdx.x] = q;
}

// Per (row m, head h): 64 lanes.  Lane l sums columns 192h + l and 192h + 64 + l
// (content query) and 192h + 128 + l (rotary query, rotated with its pair
// partner l ^ 1), then scales by the row's 1 / rms (from the nb block sums of
// squares of c_q, over q_rank values).  Work-group = 4 heads of one row.
__global__ __launch_bounds__(256) void qsplit_rope_kernel(
    const float* __restrict__ part, int splits, int M, int H, const int32_t* __restrict__ positions,
    double log_theta, const float* __restrict__ ssq, int nb, int q_rank, float eps,
    uint16_t* __restrict__ q_c, uint16_t* __restrict__ q_r) {
  const int m = blockIdx.x / (H / 4);
  const int h = (blockIdx.x % (H / 4)) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int N = H * 192;
  float a = 0.f, b = 0.f, r = 0.f;
#pragma unroll 4
  for (int s = 0; s < splits; ++s) {
    const float* p = part + ((size_t)s * M + m) * N + 192 * h + lane;
    a += p[0];
    b += p[64];
    r += p[128];
  }
  float ss = 0.f;
  for (int k = 0; k < nb; ++k) ss += ssq[m * nb + k];
  const float inv_rms = 1.f / sqrtf(ss / q_rank + eps);
  a *= inv_rms;
  b *= inv_rms;
  r *= inv_rms;
  const int pos = positions[m];
  const int i = lane >> 1;
  const double ang = fmod((double)pos * exp(-(2.0 * i / 64.0) * log_theta), 6.283185307179586);
  const float cs = cosf((float)ang), sn = sinf((float)ang);
  const float other = __shfl_xor(r, 1);
  const float rot = (lane & 1) ? other * sn + r * cs : r * cs - other * sn;
  uint16_t* qc = q_c + ((size_t)m * H + h) * 128;
  qc[lane] = f32_to_bf16(a);
  qc[64 + lane] = f32_to_bf16(b);
  q_r[((size_t)m * H + h) * 64 + lane] = f32_to_bf16(rot);
}

// out[i] = bf16(sum_s part[s, i]) over M*N values, four per thread.
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ part,
                                                         int splits, size_t total,
                                                         uint16_t* __restrict__ out) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= total) return;
  // Eight slices per batch, all loads in flight (clamped index, then a select:
  // one load per iteration would make every slice its own round trip).
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float4 t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      t[u] = *reinterpret_cast<const float4*>(part + (size_t)min(s0 + u, splits - 1) * total + i);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = s0 + u < splits;
      acc.x += ok ? t[u].x : 0.f;
      acc.y += ok ? t[u].y : 0.f;
      acc.z += ok ? t[u].z : 0.f;
      acc.w += ok ? t[u].w : 0.f;
    }
  }
  bf16x4 o;
  o[0] = (__bf16)acc.x;
  o[1] = (__bf16)acc.y;
  o[2] = (__bf16)acc.z;
  o[3] = (__bf16)acc.w;
  *reinterpret_cast<bf16x4*>(out + i) = o;
}

}  // namespace mla

// Workspace layout of the query projection: gamma * c_q (bf16 [M, q_rank]),
// the block sums of squares (fp32 [M, q_rank / 256]), each rounded up to 256
// bytes, then the K-slice partials of whichever product is running (the
// first product's are consumed before the second's are written).
static size_t qp_cq_bytes(int M, int q_rank) { return (((size_t)M * q_rank * 2) + 255) / 256 * 256; }
static size_t qp_ssq_bytes(int M, int q_rank) { return (((size_t)M * (q_rank / 256) * 4) + 255) / 256 * 256; }
extern "C" size_t mla_query_project_ws(int M, int d_model, int q_rank, int H) {
  const size_t cq = qp_cq_bytes(M, q_rank) + qp_ssq_bytes(M, q_rank);
  const size_t p1 = (size_t)mla_linear_splits(M, q_rank, d_model) * M * q_rank * 4;
  const size_t p2 = (size_t)mla_linear_splits(M, H * 192, q_rank) * M * H * 192 * 4;
  return cq + (p1 > p2 ? p1 : p2);
}

extern "C" hipError_t mla_launch_query_project(const uint16_t* x, const uint16_t* w_dq,
                                               const uint16_t* gamma_q, const uint16_t* w_uq,
                                               const int32_t* positions, uint16_t* q_c,
                                               uint16_t* q_r, void* workspace, int M, int d_model,
                                               int q_rank, int H, float eps, float theta,
                                               hipStream_t stream) {
  uint16_t* cq = static_cast<uint16_t*>(workspace);
  float* ssq = reinterpret_cast<float*>(static_cast<char*>(workspace) + qp_cq_bytes(M, q_rank));
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + qp_cq_bytes(M, q_rank) +
                                         qp_ssq_bytes(M, q_rank));
  int s1 = mla_linear_splits(M, q_rank, d_model);
  hipError_t e = mla_launch_linear_splitk(x, w_dq, part, M, q_rank, d_model, s1, stream);
  if (e != hipSuccess) return e;
  int nb = q_rank / 256;
  {
    void* args[] = {&part, &s1, &M, &q_rank, &gamma_q, &cq, &ssq};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&mla::qnorm_sum_kernel), dim3(M * nb),
                        dim3(64), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  const int n2 = H * 192;
  int s2 = mla_linear_splits(M, n2, q_rank);
  e = mla_launch_linear_splitk(cq, w_uq, part, M, n2, q_rank, s2, stream);
  if (e != hipSuccess) return e;
  double log_theta = std::log((double)theta);
  void* args[] = {&part, &s2, &M, &H, &positions, &log_theta, &ssq, &nb, &q_rank, &eps, &q_c, &q_r};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::qsplit_rope_kernel),
                         dim3(M * (H / 4)), dim3(256), args, 0, stream);
}

extern "C" size_t mla_output_project_ws(int M, int d_in, int d_out) {
  return (size_t)mla_linear_splits(M, d_out, d_in) * M * d_out * 4;
}

extern "C" hipError_t mla_launch_output_project(const uint16_t* o, const uint16_t* w_o,
                                                uint16_t* y, void* workspace, int M, int d_in,
                                                int d_out, hipStream_t stream) {
  float* part = static_cast<float*>(workspace);
  int s = mla_linear_splits(M, d_out, d_in);
  hipError_t e = mla_launch_linear_splitk(o, w_o, part, M, d_out, d_in, s, stream);
  if (e != hipSuccess) return e;
  size_t total = (size_t)M * d_out;
  void* args[] = {&part, &s, &total, &y};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::sum_slices_kernel),
                         dim3((unsigned)((total / 4 + 255) / 256)), dim3(256), args, 0, stream);
}
