// Log-sum-exp merge of the decode splits, then the W_UV up-projection.
//
// "DeepSeek-V3" (llm-vis explorer), box "Scaled dot-product attention": the
// key blocks are renormalised online, which gives the same result as one
// softmax; here that renormalisation is applied once across splits:
//   lse = ln sum_s e^{lse_s},  o_lat = sum_s e^{lse_s - lse} o_s.
// "Output projection" box / "Teardown: DeepSeek-V3" section 4: the value
// up-projection v = W_UV c folds into the output side, so
//   out[m, h, d] = sum_j o_lat[m, h, j] W_UV[h][j][d]      (512 -> 128)
//
// One work-group per (head, block of 32 query rows).  The merged o_lat rows are
// kept in LDS as a bf16 hi/lo pair (o = hi + lo to about 16 bits), so the
// bf16 MFMA product carries nearly fp32 accuracy of o_lat at twice the (tiny)
// matrix work.  W_UV[h] is staged through LDS in 128-row slices and read with
// transposed reads to form the 8-consecutive-j operand layout.  The split merge
// skips row groups that lie past M; when a block holds at most eight rows, the
// two halves of the work-group take alternate splits of the same rows and add
// their fp32 partial sums in LDS, so few-row decode does not leave half idle.
#include "mla_common.h"

namespace mla {

constexpr int kCmbThreads = 256;
constexpr int kOPitch = 512 + 8;     // bf16 per o_lat LDS row (1040 B)
constexpr int kWPitch = 128 + 32;    // bf16 per W_UV LDS row (320 B: rows 16 banks apart,
                                     // so the 4 rows of a transposed read hit disjoint banks)

__global__ __launch_bounds__(kCmbThreads) void combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ out, float* __restrict__ lse_out,
    int M, int S) {
  extern __shared__ __attribute__((aligned(16))) unsigned char cmb_smem[];
  uint16_t* o_hi = reinterpret_cast<uint16_t*>(cmb_smem);             // [32][kOPitch]
  uint16_t* o_lo = o_hi + 32 * kOPitch;                               // [32][kOPitch]
  uint16_t* wt = o_lo + 32 * kOPitch;                                 // [128][kWPitch]
  float* wts = reinterpret_cast<float*>(wt + 128 * kWPitch);          // [S][32]

  const int h = blockIdx.x % 128;
  const int m0 = (blockIdx.x / 128) * 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wave = tid >> 6;
  const size_t split_stride = (size_t)M * 128;   // rows of one split

  // W_UV[h] rows 128jc .. 128jc+127 (slice jc: 128 x 16 sixteen-byte chunks),
  // staged through registers, three slices deep: slice 0 is loaded first (it
  // overlaps the split merge below), slices 1 and 2 right after the merge,
  // slice 3 once slice 0 is in LDS (slices 0 and 3 in w0, 1 in w1, 2 in w2).
  const uint16_t* wsrc = w_uv + (size_t)h * 512 * 128;
  // Eight named chunks (not an array, which the compiler would keep in
  // scratch memory).
  struct WSlice {
    uint4 c0, c1, c2, c3, c4, c5, c6, c7;
  };
  auto w_src = [&](int jc, int k) {
    const int c = k * kCmbThreads + tid;
    return *reinterpret_cast<const uint4*>(wsrc + (size_t)(jc * 128 + (c >> 4)) * 128 + (c & 15) * 8);
  };
  auto w_dst = [&](int k) -> uint4& {
    const int c = k * kCmbThreads + tid;
    return *reinterpret_cast<uint4*>(&wt[(c >> 4) * kWPitch + (c & 15) * 8]);
  };
  auto load_w = [&](int jc, WSlice& d) {
    d.c0 = w_src(jc, 0); d.c1 = w_src(jc, 1); d.c2 = w_src(jc, 2); d.c3 = w_src(jc, 3);
    d.c4 = w_src(jc, 4); d.c5 = w_src(jc, 5); d.c6 = w_src(jc, 6); d.c7 = w_src(jc, 7);
  };
  auto store_w = [&](const WSlice& d) {
    w_dst(0) = d.c0; w_dst(1) = d.c1; w_dst(2) = d.c2; w_dst(3) = d.c3;
    w_dst(4) = d.c4; w_dst(5) = d.c5; w_dst(6) = d.c6; w_dst(7) = d.c7;
  };
  WSlice w0, w1, w2;

  // 1. Split weights per row.  All threads load the split log-sum-exps (four
  // each, unconditionally from clamped addresses), then the first W_UV slice is
  // put in flight, then the log-sum-exps go to LDS (wts has at least 1024
  // slots, so the stores need no test and the loads cannot be moved into one)
  // and one thread per row normalises them: one memory round trip for up to
  // 32 splits.
  const int n_l = S * 32;
  float lv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + k * kCmbThreads;
    const int sp = min(i >> 5, S - 1), m = min(m0 + (i & 31), M - 1);
    lv[k] = part_lse[sp * split_stride + (size_t)m * 128 + h];
  }
  load_w(0, w0);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + k * kCmbThreads;
    wts[i] = (i < n_l && m0 + (i & 31) < M) ? lv[k] : -INFINITY;
  }
  for (int i = tid + 4 * kCmbThreads; i < n_l; i += kCmbThreads) {
    const int sp = i >> 5, r = i & 31;
    wts[i] = (m0 + r < M) ? part_lse[sp * split_stride + (size_t)(m0 + r) * 128 + h] : -INFINITY;
  }
  __syncthreads();
  if (tid < 32) {
    const int m = m0 + tid;
    float mx = -INFINITY;
    for (int sp = 0; sp < S; ++sp) mx = fmaxf(mx, wts[sp * 32 + tid]);
    float z = 0.f;
    if (mx != -INFINITY)
      for (int sp = 0; sp < S; ++sp) {
        const float w = __expf(wts[sp * 32 + tid] - mx);
        wts[sp * 32 + tid] = w;
        z += w;
      }
    const float inv = (z > 0.f) ? 1.f / z : 0.f;
    for (int sp = 0; sp < S; ++sp) wts[sp * 32 + tid] = (mx != -INFINITY) ? wts[sp * 32 + tid] * inv : 0.f;
    if (lse_out != nullptr && m < M)
      lse_out[(size_t)m * 128 + h] = (mx != -INFINITY) ? mx + __logf(z) : -INFINITY;
  }
  __syncthreads();

  // 2. o_lat rows: thread handles columns 4*(tid%128) .. +3 of eight
  // consecutive rows, r0 .. r0+7 with r0 = 8*(tid/128) (+16 in the second
  // iteration), so that the partials of eight rows and two splits are in flight
  // together.  A group of eight rows with none below M is skipped (uniform per
  // pair of waves): its LDS rows only feed output rows >= M, which are never
  // written.  When the block has at most eight rows below M, both pairs of
  // waves work on them, each on every second split, and their fp32 sums meet
  // in the (not yet used) W_UV staging area.  A split of weight 0 (empty,
  // whose partial may hold anything) is dropped by a select, not a branch.
  {
    const int cq = tid & 127, hh = tid >> 7;
    const bool pair = M - m0 <= 8;                      // uniform over the work-group
    float* scratch = reinterpret_cast<float*>(wt);      // [2][8][512] when pair
    auto store_hilo = [&](int r, float4 v) {
      const float ov[4] = {v.x, v.y, v.z, v.w};
      bf16x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = (__bf16)ov[e];
        lo[e] = (__bf16)(ov[e] - (float)hi[e]);
      }
      *reinterpret_cast<bf16x4*>(&o_hi[r * kOPitch + 4 * cq]) = hi;
      *reinterpret_cast<bf16x4*>(&o_lo[r * kOPitch + 4 * cq]) = lo;
    };
#pragma unroll 1
    for (int it = 0; it < 2; ++it) {
      const int r0 = pair ? 0 : hh * 8 + 16 * it;
      if (pair ? it > 0 : m0 + r0 >= M) continue;
      const int s_first = pair ? hh : 0, s_step = pair ? 2 : 1;
      float4 o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 2
      for (int s = s_first; s < S; s += s_step) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int m = min(m0 + r0 + u, M - 1);
          v[u] = *reinterpret_cast<const float4*>(part_o + (s * split_stride + (size_t)m * 128 + h) * 512 +
                                                  4 * cq);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float w = (m0 + r0 + u < M) ? wts[s * 32 + r0 + u] : 0.f;
          const bool use = w != 0.f;
          o[u].x += use ? w * v[u].x : 0.f;
          o[u].y += use ? w * v[u].y : 0.f;
          o[u].z += use ? w * v[u].z : 0.f;
          o[u].w += use ? w * v[u].w : 0.f;
        }
      }
      if (pair) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          *reinterpret_cast<float4*>(&scratch[(hh * 8 + u) * 512 + 4 * cq]) = o[u];
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) store_hilo(r0 + u, o[u]);
      }
    }
    if (pair) {
      __syncthreads();
      if (hh == 0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float4 a0 = *reinterpret_cast<const float4*>(&scratch[u * 512 + 4 * cq]);
          const float4 a1 = *reinterpret_cast<const float4*>(&scratch[(8 + u) * 512 + 4 * cq]);
          store_hilo(u, make_float4(a0.x + a1.x, a0.y + a1.y, a0.z + a1.z, a0.w + a1.w));
        }
      }
    }
  }

  // 3. out[32 rows x 128] = o_lat . W_UV[h]; wave w owns columns 32w .. 32w+31.
  const int q16 = lane & 15;
  const int colhalf = (lane >> 4) & 1;
  const lds_u8* trb = to_lds(wt) +
                      ((8 * half + (q16 >> 2)) * kWPitch + 32 * wave + 16 * colhalf + 4 * (q16 & 3)) * 2;
  const lds_u8* ahb = to_lds(o_hi) + (l32 * kOPitch + 8 * half) * 2;
  const lds_u8* alb = to_lds(o_lo) + (l32 * kOPitch + 8 * half) * 2;
  load_w(1, w1);
  load_w(2, w2);
  f32x16 acc = {};
  auto product = [&](int jc) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x4 blo = ld_lds_tr(trb + (16 * ks) * kWPitch * 2);
      const bf16x4 bhi = ld_lds_tr(trb + (16 * ks + 4) * kWPitch * 2);
      const bf16x8 bw = cat(blo, bhi);
      const int koff = (jc * 128 + 16 * ks) * 2;
      acc = mfma32(ld_lds_bf16x8(ahb + koff), bw, acc);
      acc = mfma32(ld_lds_bf16x8(alb + koff), bw, acc);
    }
  };
  // Each slice: every wave is done with the previous one, then it goes to LDS.
  __syncthreads();
  store_w(w0);
  __syncthreads();
  load_w(3, w0);
  product(0);
  __syncthreads();
  store_w(w1);
  __syncthreads();
  product(1);
  __syncthreads();
  store_w(w2);
  __syncthreads();
  product(2);
  __syncthreads();
  store_w(w0);
  __syncthreads();
  product(3);
  // acc[r]: row m0 + 8*(r/4) + 4*half + r%4, column 32*wave + l32.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (m < M) {
      const __bf16 v = (__bf16)acc[r];
      out[((size_t)m * 128 + h) * 128 + 32 * wave + l32] = __builtin_bit_cast(uint16_t, v);
    }
  }
}

size_t combine_lds_bytes(int S) {
  return (size_t)(2 * 32 * kOPitch + 128 * kWPitch) * 2 + (size_t)(S > 32 ? S : 32) * 32 * 4;
}

}  // namespace mla

extern "C" hipError_t mla_launch_combine(const float* part_o, const float* part_lse,
                                         const uint16_t* w_uv, uint16_t* out, float* lse_out, int M,
                                         int S, hipStream_t stream) {
  const size_t lds = mla::combine_lds_bytes(S);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&mla::combine_kernel),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)mla::combine_lds_bytes(256));
  if (attr != hipSuccess) return attr;
  const int grid = 128 * ((M + 31) / 32);
  void* args[] = {&part_o, &part_lse, &w_uv, &out, &lse_out, &M, &S};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::combine_kernel), dim3(grid),
                         dim3(mla::kCmbThreads), args, lds, stream);
}
