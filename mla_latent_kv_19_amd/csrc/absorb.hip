// q-absorption: q_lat[m, h, :] = q_C[m, h, :] . W_UK[h]   (128 -> 512 per head).
//
// "DeepSeek-V3" (llm-vis explorer), box "KV latent compression": the key
// up-projection is absorbed into the query, q^T (W_uk c) = (W_uk^T q)^T c, so
// scores can be taken directly against the cached latent.  W_UK[h] is stored
// [d_h = 128 rows i][d_c = 512 columns j]; q_lat[j] = sum_i q_C[i] W_UK[h][i][j].
//
// This is a weight-streaming product (16.8 MB of W_UK per call, a few query
// rows): one work-group per (head, 128-column block of j) stages its 32 KB
// slice of W_UK once in LDS, keeps it in registers as the A operand of
// q_lat^T = W_UK[h]^T . q_C^T (transposed LDS reads give the 8-consecutive-i
// operand layout), and streams all query rows through it in blocks of 32.
#include "mla_common.h"

namespace mla {

constexpr int kAbsThreads = 256;
constexpr int kAbsPitch = 128 + 32;   // bf16 per LDS row (320 B: rows 16 banks apart, so the
                                      // 4 rows of a transposed read hit disjoint banks)

__global__ __launch_bounds__(kAbsThreads) void absorb_q_kernel(const uint16_t* __restrict__ q_c,
                                                               const uint16_t* __restrict__ w_uk,
                                                               uint16_t* __restrict__ q_lat, int M) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[128 * kAbsPitch];
  const int h = blockIdx.x >> 2;
  const int jblk = blockIdx.x & 3;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wave = tid >> 6;

  // Query operands of a block of 32 rows (lane: row m0 + l32, 8 consecutive i).
  // q_c through an empty asm: loads from a const __restrict__ argument count as
  // invariant, and the compiler then sinks the first block's loads past the
  // weight staging below (to their first use), serialising the two round trips.
  typedef __attribute__((address_space(1))) const bf16x8 gbl_bf16x8;
  const uint16_t* q_src = q_c;
  asm volatile("" : "+s"(q_src));
  auto load_q = [&](int m0, bf16x8 (&bq)[8]) {
    const int m = m0 + l32;
    const uint16_t* src = q_src + ((size_t)min(m, M - 1) * 128 + h) * 128 + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) bq[ks] = *(gbl_bf16x8*)(src + 16 * ks);
  };
  // The first block's queries are loaded before the weight slice is staged, so
  // the two loads overlap.
  bf16x8 bq[8];
  load_q(0, bq);

  // Stage W_UK[h][0:128][128*jblk : +128]: 128 rows x 256 B = 2048 16-byte chunks.
  const uint16_t* wsrc = w_uk + (size_t)h * 128 * 512 + jblk * 128;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int chunk = k * kAbsThreads + tid;
    const int i = chunk >> 4, c = chunk & 15;
    *reinterpret_cast<uint4*>(&wt[i * kAbsPitch + c * 8]) =
        *reinterpret_cast<const uint4*>(wsrc + (size_t)i * 512 + c * 8);
  }
  __syncthreads();

  // A operands (W^T, rows j = 32*wave + l32, k = i): two transposed reads per
  // k-step.  Group g = lane/16: rows i0 + 8*(g/2) + q/4 (+4), columns
  // 32*wave + 16*(g%2) + 4*(q%4).
  const int q16 = lane & 15;
  const int colhalf = (lane >> 4) & 1;
  const lds_u8* tbase = to_lds(wt) +
                        ((8 * half + (q16 >> 2)) * kAbsPitch + 32 * wave + 16 * colhalf + 4 * (q16 & 3)) * 2;
  bf16x8 a[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const bf16x4 lo = ld_lds_tr(tbase + (16 * ks) * kAbsPitch * 2);
    const bf16x4 hi = ld_lds_tr(tbase + (16 * ks + 4) * kAbsPitch * 2);
    a[ks] = cat(lo, hi);
  }

  for (int m0 = 0; m0 < M; m0 += 32) {
    // Next block's queries in flight during this block's product.
    bf16x8 bn[8];
    if (m0 + 32 < M) load_q(m0 + 32, bn);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) acc = mfma32(a[ks], bq[ks], acc);
    // acc[r]: j = 32*wave + 8*(r/4) + 4*half + r%4, m = m0 + l32.
    const int m = m0 + l32;
    if (m < M) {
      uint16_t* dst = q_lat + ((size_t)m * 128 + h) * 512 + jblk * 128 + 32 * wave + 4 * half;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * g + e];
        *reinterpret_cast<bf16x4*>(dst + 8 * g) = v;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) bq[ks] = bn[ks];
  }
}

}  // namespace mla

extern "C" hipError_t mla_launch_absorb_q(const uint16_t* q_c, const uint16_t* w_uk, uint16_t* q_lat,
                                          int M, hipStream_t stream) {
  void* args[] = {&q_c, &w_uk, &q_lat, &M};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::absorb_q_kernel), dim3(128 * 4),
                         dim3(mla::kAbsThreads), args, 0, stream);
}
