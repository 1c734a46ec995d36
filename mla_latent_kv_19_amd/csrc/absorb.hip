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
//
// Every global access is a whole row piece: a query row q_C[m, h, :] is 256
// contiguous bytes, read by 16 lanes, and the block's 256-byte piece of a
// q_lat row likewise; both pass through LDS to and from the MFMA layouts
// (lane = row, 8 consecutive values), which read or write only 32 bytes of a
// row per lane pair and would touch 32 cache lines per instruction.  The rows
// of 128 queries (four blocks) are loaded in one round trip, 32 bytes of
// registers per row and lane group.
#include "mla_common.h"

namespace mla {

constexpr int kAbsThreads = 256;
constexpr int kAbsPitch = 128 + 32;   // bf16 per W LDS row (320 B: rows 16 banks apart, so the
                                      // 4 rows of a transposed read hit disjoint banks)
constexpr int kRowPitch = 128 + 8;    // bf16 per query / output LDS row (272 B: 16 consecutive
                                      // rows read at one column hit 16 distinct 4-bank groups)
constexpr int kGroupRows = 128;       // query rows in flight together

__global__ __launch_bounds__(kAbsThreads) void absorb_q_kernel(const uint16_t* __restrict__ q_c,
                                                               const uint16_t* __restrict__ w_uk,
                                                               uint16_t* __restrict__ q_lat, int M) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[128 * kAbsPitch];
  __shared__ __attribute__((aligned(16))) uint16_t qs[32 * kRowPitch];   // one block of query rows
  __shared__ __attribute__((aligned(16))) uint16_t os[32 * kRowPitch];   // one block of q_lat pieces
  const int h = blockIdx.x >> 2;
  const int jblk = blockIdx.x & 3;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wave = tid >> 6;

  // Query rows g0 .. g0+127 (clamped to M - 1): thread tid holds 16-byte
  // chunk tid % 16 of rows g0 + 16 k + tid / 16, k = 0..7; block b of 32 rows
  // is in k = 2b, 2b + 1.  q_c through an empty asm: loads from a const
  // __restrict__ argument count as invariant, and the compiler then sinks the
  // first group's loads past the weight staging below (to their first use),
  // serialising the two round trips.
  const uint16_t* q_src = q_c;
  asm volatile("" : "+s"(q_src));
  const int rc = tid & 15, rr = tid >> 4;
  // Named chunks, not an array: an array indexed by the block loop is kept in
  // scratch memory.
  struct QRows {
    uint4 k0, k1, k2, k3, k4, k5, k6, k7;
  } qv;
  auto q_chunk = [&](int g0, int k) {
    const int m = min(g0 + 16 * k + rr, M - 1);
    return *reinterpret_cast<const uint4*>(q_src + ((size_t)m * 128 + h) * 128 + rc * 8);
  };
  auto load_group = [&](int g0) {
    qv.k0 = q_chunk(g0, 0); qv.k1 = q_chunk(g0, 1); qv.k2 = q_chunk(g0, 2); qv.k3 = q_chunk(g0, 3);
    qv.k4 = q_chunk(g0, 4); qv.k5 = q_chunk(g0, 5); qv.k6 = q_chunk(g0, 6); qv.k7 = q_chunk(g0, 7);
  };
  load_group(0);

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

  for (int g0 = 0; g0 < M; g0 += kGroupRows) {
#pragma unroll
    for (int bk = 0; bk < kGroupRows / 32; ++bk) {
      const int m0 = g0 + 32 * bk;
      if (m0 >= M) continue;                           // uniform: every thread skips
      // The block's query rows into LDS (the previous block's operand reads
      // and output reads are done: the barrier at the end of its iteration).
      const uint4 lo = bk == 0 ? qv.k0 : bk == 1 ? qv.k2 : bk == 2 ? qv.k4 : qv.k6;
      const uint4 hi = bk == 0 ? qv.k1 : bk == 1 ? qv.k3 : bk == 2 ? qv.k5 : qv.k7;
      *reinterpret_cast<uint4*>(&qs[rr * kRowPitch + rc * 8]) = lo;
      *reinterpret_cast<uint4*>(&qs[(16 + rr) * kRowPitch + rc * 8]) = hi;
      __syncthreads();
      // B operands: lane = row l32, i = 16 ks + 8 half .. +7.
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        acc = mfma32(a[ks], *reinterpret_cast<const bf16x8*>(&qs[l32 * kRowPitch + 16 * ks + 8 * half]), acc);
      // acc[r]: j = 32*wave + 8*(r/4) + 4*half + r%4 (of the block's 128), m = m0 + l32.
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * g + e];
        *reinterpret_cast<bf16x4*>(&os[l32 * kRowPitch + 32 * wave + 8 * g + 4 * half]) = v;
      }
      __syncthreads();
      // Row pieces out: thread tid writes chunk tid % 16 of rows tid / 16 and
      // 16 + tid / 16.
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int r = 16 * k + rr, m = m0 + r;
        if (m < M)
          *reinterpret_cast<uint4*>(q_lat + ((size_t)m * 128 + h) * 512 + jblk * 128 + rc * 8) =
              *reinterpret_cast<const uint4*>(&os[r * kRowPitch + rc * 8]);
      }
      __syncthreads();
    }
    if (g0 + kGroupRows < M) load_group(g0 + kGroupRows);
  }
}

}  // namespace mla

extern "C" hipError_t mla_launch_absorb_q(const uint16_t* q_c, const uint16_t* w_uk, uint16_t* q_lat,
                                          int M, hipStream_t stream) {
  void* args[] = {&q_c, &w_uk, &q_lat, &M};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::absorb_q_kernel), dim3(128 * 4),
                         dim3(mla::kAbsThreads), args, 0, stream);
}
