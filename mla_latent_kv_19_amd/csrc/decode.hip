// Split-KV flash decode over the paged latent cache (absorbed form).
//
// What it computes ("Teardown: DeepSeek-V3", section 4; "DeepSeek-V3" llm-vis
// explorer, "KV latent compression" and "Scaled dot-product attention"):
// for every sequence b, query i and head h, over the tokens t of one split of
// the sequence's pages that the query may see (t <= L_b - Tq + i),
//   s_t   = (q_lat[b,i,h] . c_t + q_R[b,i,h] . k_R,t) * scale
//   o_s   = sum_t softmax(s)_t c_t            (512 wide, fp32)
//   lse_s = ln sum_t exp(s_t)
// with the softmax renormalised online, one 64-token page at a time.
//
// Work decomposition (MI355X: 256 CUs, 64-wide waves, 160 KB LDS per CU):
//   * one work-group of 4 waves per (sequence, split, query); the 128 heads
//     share each cached row, so a page is loaded once into LDS and used by all
//     128 heads: wave w owns heads 32w .. 32w+31;
//   * each wave keeps its 32 queries (576 wide, bf16) in registers as the B
//     operand and its output O^T (512 x 32 heads, fp32) in 256 accumulator
//     registers;
//   * per 32-token slice: S^T[32 tok x 32 heads] = K[32 x 576] . Q^T
//     (36 MFMA 32x32x16, K read from LDS with 16-byte reads), online softmax in
//     registers (lane = head), then O^T[512 x 32] += V^T[512 x 32 tok] . P^T
//     (32 MFMA; V^T read from the same LDS tile with transposed reads, P^T taken
//     straight from the score registers: no shuffles);
//   * pages stream global -> LDS with 16-byte direct-to-LDS loads, double
//     buffered: page n+1 is in flight while page n is multiplied.
#include "mla_common.h"

namespace mla {

constexpr int kDecThreads = 256;
constexpr int kTok = 64;                       // tokens per cache block
constexpr int kRowVals = 576;                  // 512 latent + 64 rotary
constexpr int kRowBytes = kRowVals * 2;        // 1152
constexpr int kChunks = kRowBytes / 16;        // 72 sixteen-byte chunks per row
constexpr int kPageBytes = kTok * kRowBytes;   // 73728
constexpr int kLoadsPerThread = kPageBytes / 16 / kDecThreads;  // 18
constexpr int kDecLdsBytes = 2 * kPageBytes;   // double buffer

static_assert(kLoadsPerThread * 16 * kDecThreads == kPageBytes, "page must split evenly");

// Lazy renormalisation threshold (log2 units): unnormalised weights stay <= 2^8.
constexpr float kLazy = 8.f;

// LDS placement of chunk c of token row t: the low three bits of the chunk
// index are XORed with a per-row pattern so that both the 16-byte row reads of
// the score product (8 rows, same chunk) and the transposed reads of the value
// product (4 rows x 2 adjacent chunks) hit distinct banks.
__device__ __forceinline__ int row_swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }
__device__ __forceinline__ int chunk_off(int t, int c) {
  return (t * kChunks + (c ^ row_swz(t))) * 16;
}

// All 256 threads: copy one 64-token page into an LDS buffer.  Thread tid
// fills LDS slots it*256 + tid; each slot's source chunk is chosen so that the
// slot order realises chunk_off().
__device__ __forceinline__ void issue_page(const uint16_t* page, lds_u8* buf, int tid) {
  // Recompute the slot addresses per page instead of keeping 18 of them live
  // across the loop (the register file is nearly full).
  asm volatile("" : "+v"(tid));
  const char* g = reinterpret_cast<const char*>(page);
  lds_u8* wave_base = buf + (tid & ~63) * 16;
#pragma unroll
  for (int it = 0; it < kLoadsPerThread; ++it) {
    const int slot = it * kDecThreads + tid;
    const int t = slot / kChunks;
    const int p = slot - t * kChunks;
    const int c = p ^ row_swz(t);
    g2lds16(g + t * kRowBytes + c * 16, wave_base + it * kDecThreads * 16);
  }
}

__global__ __launch_bounds__(kDecThreads, 1) void decode_paged_kernel(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ q_r,
    const uint16_t* __restrict__ kv, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int B, int Tq, int max_blocks, float scale_log2,
    int num_splits, int num_units, float* __restrict__ part_o, float* __restrict__ part_lse) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dec_smem[];
  lds_u8* smem = to_lds(dec_smem);

  // Work-group -> (unit = (sequence, split), query).  Consecutive ids go to
  // different XCDs; the Tq work-groups of one unit get ids 8 apart so they
  // land on the same XCD and share its L2 for the unit's pages.
  const int wg = blockIdx.x;
  const int k8 = wg >> 3;
  const int qi = k8 % Tq;
  const int unit = (k8 / Tq) * 8 + (wg & 7);
  if (unit >= num_units) return;
  const int b = unit / num_splits;
  const int split = unit - b * num_splits;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wave = tid >> 6;
  const int head = wave * 32 + l32;

  const int L = seq_lens[b];
  const int n_pages = (L + kTok - 1) / kTok;
  const int per = (n_pages + num_splits - 1) / num_splits;
  const int p0 = min(n_pages, split * per);
  const int n_vis = L - Tq + qi + 1;                  // keys this query sees
  const int p1 = min(min(n_pages, p0 + per), (n_vis + kTok - 1) / kTok);
  const int count = p1 - p0;

  const size_t row = (size_t)(b * Tq + qi) * 128 + head;   // query row index (H = 128)
  float* o_dst = part_o + ((size_t)split * B * Tq * 128 + row) * 512;
  float* lse_dst = part_lse + (size_t)split * B * Tq * 128 + row;

  if (count <= 0) {
    // Nothing visible in this split: o = 0, lse = -inf.
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4*>(o_dst + cb * 32 + 8 * a + 4 * half) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (half == 0) *lse_dst = -INFINITY;
    return;
  }

  const int32_t* table = block_table + (size_t)b * max_blocks;
  issue_page(kv + (size_t)table[p0] * (kTok * kRowVals), smem, tid);

  // Queries as B operands: k-step kk covers dims 16kk .. 16kk+15 of [q_lat; q_R].
  bf16x8 qreg[36];
  {
    const uint16_t* ql = q_lat + row * 512 + 8 * half;
    const uint16_t* qr = q_r + row * 64 + 8 * half;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) qreg[kk] = ld_global_bf16x8(ql + 16 * kk);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qreg[32 + kk] = ld_global_bf16x8(qr + 16 * kk);
  }

  f32x16 acc[16];
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) acc[cb] = f32x16{};
  float m_ref = -INFINITY;   // exponent reference (<= running max + 0), log2 units
  float l_run = 0.f;         // this lane's share of sum 2^(x - m_ref)

  // Per-lane LDS offsets.
  // Score product: lane reads token (l32) of the slice, chunk 2kk + half.
  const int sq = row_swz(l32);
  const int qk_base = l32 * kRowBytes;
  // Transposed value reads: group g = lane/16 (g/2 = half, g%2 = column half),
  // q = lane%16 supplies row 4*half + q/4 (+8 for the second read), columns
  // 16*(g%2) + 4*(q%4) .. +3 of the 32-column block.
  const int q16 = lane & 15;
  const int colhalf = (lane >> 4) & 1;
  const int tr_row = 4 * half + (q16 >> 2);
  const int st = row_swz(tr_row);
  const int tr_base = tr_row * kRowBytes + (q16 & 1) * 8;
  const int tr_c0 = (2 * colhalf + ((q16 & 3) >> 1)) ^ st;        // even column blocks
  const int tr_c1 = (4 + 2 * colhalf + ((q16 & 3) >> 1)) ^ st;    // odd column blocks

  for (int i = 0; i < count; ++i) {
    lds_u8* cur = smem + (i & 1) * kPageBytes;
    // One barrier per page: after it, page i has landed for every wave and
    // every wave has finished page i-1, whose buffer then takes page i+1.
    wait_vmcnt<0>();
    lds_barrier();
    if (i + 1 < count)
      issue_page(kv + (size_t)table[p0 + i + 1] * (kTok * kRowVals),
                 smem + ((i + 1) & 1) * kPageBytes, tid);

    const int pg = p0 + i;
    const int valid = L - pg * kTok;                // rows of this page inside the sequence
    if (valid < kTok) {
      // Rows past the sequence end may hold anything (NaN): zero them so that
      // 0-weight tokens contribute exactly 0 to the value product.
      for (int off = valid * kRowBytes + tid * 16; off < kPageBytes; off += kDecThreads * 16)
        st_lds_zero16(cur + off);
      lds_barrier();
    }

#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const lds_u8* slice = cur + tb * 32 * kRowBytes;
      // Score product with the accumulator pinned to VGPRs (the 256 AGPRs hold
      // the output accumulators); see mfma32_vgpr.
      f32x16 s;
#pragma unroll
      for (int kk = 0; kk < 36; ++kk) {
        const int c = 8 * (kk >> 2) + ((2 * (kk & 3) + half) ^ sq);
        const bf16x8 kop = ld_lds_bf16x8(slice + qk_base + c * 16);
        if (kk == 0)
          s = mfma32_vgpr_first(kop, qreg[kk]);
        else
          mfma32_vgpr_acc(s, kop, qreg[kk]);
      }
      mfma_vgpr_settle(s);
      // s[r] is token tok0 + 8*(r/4) + r%4 of this slice for head `head`.
      const int tok0 = pg * kTok + tb * 32 + 4 * half;
      float x[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = tok0 + 8 * (r >> 2) + (r & 3);
        x[r] = (t < n_vis) ? s[r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // Lazy renormalisation: the exponent reference m_ref only moves when the
      // slice maximum exceeds it by more than kLazy (so p <= 2^kLazy); the
      // accumulators are rescaled only then, and not at all on the first
      // visible slice, when they are still zero.
      const bool move = mx > m_ref + kLazy;
      if (__any(move && m_ref != -INFINITY)) {
        const float alpha = move ? fast_exp2(m_ref - mx) : 1.f;
        l_run *= alpha;
        agpr_scale_begin();
#pragma unroll
        for (int cb = 0; cb < 16; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) MLA_AGPR_SCALE(acc[cb][r], alpha);
        agpr_scale_end();
      }
      if (move) m_ref = mx;
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      bf16x8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(x[r] - m_use);
        l_run += p;
        pb[r >> 3][r & 7] = (__bf16)p;
      }
      // O^T += V^T . P^T over the slice's two 16-token k-steps.
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const lds_u8* vrow = slice + (16 * kt) * kRowBytes + tr_base;
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) {
          const int coff = (8 * (cb >> 1) + ((cb & 1) ? tr_c1 : tr_c0)) * 16;
          const bf16x4 lo = ld_lds_tr(vrow + coff);
          const bf16x4 hi = ld_lds_tr(vrow + 8 * kRowBytes + coff);
          acc[cb] = mfma32(cat(lo, hi), pb[kt], acc[cb]);
        }
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<float4*>(o_dst + cb * 32 + 8 * a + 4 * half) =
          make_float4(acc[cb][4 * a] * inv, acc[cb][4 * a + 1] * inv, acc[cb][4 * a + 2] * inv,
                      acc[cb][4 * a + 3] * inv);
  if (half == 0) *lse_dst = (l_tot > 0.f) ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
}

}  // namespace mla

extern "C" hipError_t mla_launch_decode_paged(
    const uint16_t* q_lat, const uint16_t* q_r, const uint16_t* kv, const int32_t* block_table,
    const int32_t* seq_lens, int B, int Tq, int max_blocks, float softmax_scale, int num_splits,
    float* part_o, float* part_lse, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&mla::decode_paged_kernel),
      hipFuncAttributeMaxDynamicSharedMemorySize, mla::kDecLdsBytes);
  if (attr != hipSuccess) return attr;
  const int num_units = B * num_splits;
  const int grid = ((num_units + 7) / 8) * 8 * Tq;
  float scale_log2 = softmax_scale * mla::kLog2e;
  void* args[] = {&q_lat, &q_r, &kv, &block_table, &seq_lens, &B, &Tq, &max_blocks,
                  &scale_log2, &num_splits, const_cast<int*>(&num_units), &part_o, &part_lse};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::decode_paged_kernel), dim3(grid),
                         dim3(mla::kDecThreads), args, mla::kDecLdsBytes, stream);
}
