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
// One work-group per (head, block of 32 query rows; 16 when there are at most
// 32 rows, so that 17-32 rows still fill 256 work-groups).  The merged o_lat rows are
// kept in LDS as a bf16 hi/lo pair (o = hi + lo to about 16 bits), so the
// bf16 MFMA product carries nearly fp32 accuracy of o_lat at twice the (tiny)
// matrix work.  W_UV[h] is staged through LDS in 128-row slices and read with
// transposed reads to form the 8-consecutive-j operand layout.  The split merge
// skips row groups that lie past M; when a block holds at most eight rows, the
// row groups of the work-group take alternate splits of the same rows and add
// their fp32 partial sums in LDS, so few-row decode does not leave them idle;
// a block of one row (up to 32 splits) puts all its partials in flight with
// the log-sum-exps, one round trip for the whole merge.
//
// Two forms.  Up to 64 rows (at most 256 work-groups: one round on the chip)
// the merge covers all 512 latent columns at once (~109 KB of LDS, one
// work-group per compute unit).  Past that the work-group runs two passes of
// 256 columns (merge, then the matching 256 rows of W_UV), ~78 KB of LDS, so
// that two share a compute unit and one's memory round trips overlap the
// other's work: 128 rows 30 -> 24 us, 512 rows 80 -> 55 us; at 32 rows and
// fewer the single pass is 1-2 us faster.
#include "mla_common.h"

namespace mla {

constexpr int kCmbThreads = 256;
constexpr int kWPitch = 128 + 32;    // bf16 per W_UV LDS row (320 B: rows 16 banks apart,
                                     // so the 4 rows of a transposed read hit disjoint banks)
constexpr int kLseLoads = 5;         // split log-sum-exps per thread in the first round trip
constexpr int kWtsMin = kLseLoads * kCmbThreads;   // weight slots always present (40 splits)

// LDS of one form: merged rows (hi and lo), one W_UV slice, split weights.
constexpr size_t combine_lds(int passes, int S) {
  return (size_t)(2 * 32 * (512 / passes + 8) + 128 * kWPitch) * 2 +
         (size_t)(S * 32 > kWtsMin ? S * 32 : kWtsMin) * 4 + 16;
}
static_assert(combine_lds(2, 40) <= 80 * 1024, "two-pass form: two work-groups per compute unit");

template <int kPasses>
__global__ __launch_bounds__(kCmbThreads) void combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ out, float* __restrict__ lse_out,
    int M, int S, int rb) {
  constexpr int kOCols = 512 / kPasses;              // latent columns per pass
  constexpr int kOPitch = kOCols + 8;                // bf16 per o_lat LDS row
  constexpr int kRowLanes = kOCols / 4;              // threads per merged row (4 columns each)
  constexpr int kGroups = kCmbThreads / kRowLanes;   // groups of eight rows merged at once
  constexpr int kIters = 32 / (8 * kGroups);         // rounds of row groups per pass
  constexpr int kSlices = 4 / kPasses;               // W_UV slices per pass
  static_assert(kGroups * 8 * kOCols * 4 <= 128 * kWPitch * 2, "pair-form scratch inside the W_UV area");
  extern __shared__ __attribute__((aligned(16))) unsigned char cmb_smem[];
  uint16_t* o_hi = reinterpret_cast<uint16_t*>(cmb_smem);             // [32][kOPitch]
  uint16_t* o_lo = o_hi + 32 * kOPitch;                               // [32][kOPitch]
  uint16_t* wt = o_lo + 32 * kOPitch;                                 // [128][kWPitch]
  float* wts = reinterpret_cast<float*>(wt + 128 * kWPitch);          // [S][32]
  int* s_end_lds = reinterpret_cast<int*>(wts + (S * 32 > kWtsMin ? S * 32 : kWtsMin));  // 1 + last split of weight > 0

  const int h = blockIdx.x % 128;
  const int m0 = (blockIdx.x / 128) * rb;
  const int m_end = min(M, m0 + rb);             // rows of this block: m0 .. m_end-1
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

  // 1. Split weights per row.  All threads load the split log-sum-exps (five
  // each, unconditionally from clamped addresses), then the first W_UV slice is
  // put in flight, then the log-sum-exps go to LDS (wts has at least
  // kWtsMin slots, so the stores need no test and the loads cannot be moved
  // into one) and one thread per row normalises them: one memory round trip
  // for up to 40 splits.  The same threads find the last split of non-zero
  // weight over the block's rows; step 2 stops there.
  const int cq = tid % kRowLanes, grp = tid / kRowLanes;
  const int n_l = S * 32;
  float lv[kLseLoads];
#pragma unroll
  for (int k = 0; k < kLseLoads; ++k) {
    const int i = tid + k * kCmbThreads;
    const int sp = min(i >> 5, S - 1), m = min(m0 + (i & 31), m_end - 1);
    lv[k] = part_lse[sp * split_stride + (size_t)m * 128 + h];
  }
  // A block of one row (single pass, at most 32 splits): the partials of all
  // its splits go in flight here, behind the log-sum-exps and ahead of the
  // W_UV slices, so that the merge waits one memory round trip instead of one
  // per two splits.  Thread (grp, cq) takes splits grp, grp + kGroups, ...
  constexpr int kOneRowLoads = 32 / kGroups;
  const bool one_row = kPasses == 1 && m_end - m0 == 1 && S <= 32;   // uniform
  float4 pv[kOneRowLoads];
  if constexpr (kPasses == 1) {
    if (one_row) {
#pragma unroll
      for (int k = 0; k < kOneRowLoads; ++k) {
        const int sp = min(grp + kGroups * k, S - 1);
        pv[k] = *reinterpret_cast<const float4*>(part_o + (sp * split_stride + (size_t)m0 * 128 + h) * 512 + 4 * cq);
      }
    }
  }
  load_w(0, w0);
  if constexpr (kPasses == 2) {
    load_w(1, w1);
  } else if (one_row) {
    load_w(1, w1);
    load_w(2, w2);
  }
#pragma unroll
  for (int k = 0; k < kLseLoads; ++k) {
    const int i = tid + k * kCmbThreads;
    wts[i] = (i < n_l && m0 + (i & 31) < m_end) ? lv[k] : -INFINITY;
  }
  for (int i = tid + kLseLoads * kCmbThreads; i < n_l; i += kCmbThreads) {
    const int sp = i >> 5, r = i & 31;
    wts[i] = (m0 + r < m_end) ? part_lse[sp * split_stride + (size_t)(m0 + r) * 128 + h] : -INFINITY;
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
    int last = -1;
    for (int sp = 0; sp < S; ++sp) {
      const float w = (mx != -INFINITY) ? wts[sp * 32 + tid] * inv : 0.f;
      wts[sp * 32 + tid] = w;
      if (w != 0.f) last = sp;
    }
#pragma unroll
    for (int d = 16; d > 0; d >>= 1) last = max(last, __shfl_xor(last, d, 32));
    if (tid == 0) *s_end_lds = last + 1;
    if (lse_out != nullptr && m < m_end)
      lse_out[(size_t)m * 128 + h] = (mx != -INFINITY) ? mx + __logf(z) : -INFINITY;
  }
  __syncthreads();

  // 2. o_lat rows, pass p: columns kOCols p .. +kOCols-1.  Thread handles
  // columns 4*(tid % kRowLanes) .. +3 (a row's pass columns are one contiguous
  // read across kRowLanes threads) of eight consecutive rows, r0 .. r0+7 with
  // r0 = 8*(tid / kRowLanes) (+8 kGroups in later rounds), so that the
  // partials of eight rows and two splits are in flight together.  A group of
  // eight rows with none inside the block (m0 .. m_end-1) is skipped (uniform
  // per row group): its LDS rows only feed output rows past the block, which
  // are never written.  When the block has at most eight rows, every row group
  // works on them, each on
  // every kGroups-th split, and their fp32 sums meet in the (then unused) W_UV
  // staging area.  Splits past the block's last one of non-zero weight are not
  // visited; a split of weight 0 before it (empty: lse = -inf, its partial
  // never written) is read and dropped by a select, not a branch, which keeps
  // the loads of eight rows and two splits in flight together (reading split
  // 0's row in its place, or testing the weight first, measured slower).
  const bool pair = m_end - m0 <= 8;                      // uniform over the work-group
  float* scratch = reinterpret_cast<float*>(wt);      // [kGroups][8][kOCols] when pair
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
  auto merge = [&](int p) {
#pragma unroll 1
    for (int it = 0; it < kIters; ++it) {
      const int r0 = pair ? 0 : grp * 8 + 8 * kGroups * it;
      if (pair ? it > 0 : m0 + r0 >= m_end) continue;
      const int s_first = pair ? grp : 0, s_step = pair ? kGroups : 1;
      const int s_stop = *s_end_lds;
      float4 o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (one_row) {
        // The partials loaded in step 1 (row 0; the other seven stay zero).
#pragma unroll
        for (int k = 0; k < kOneRowLoads; ++k) {
          const int sp = grp + kGroups * k;
          const float w = (sp < s_stop) ? wts[sp * 32] : 0.f;
          const bool use = w != 0.f;
          o[0].x += use ? w * pv[k].x : 0.f;
          o[0].y += use ? w * pv[k].y : 0.f;
          o[0].z += use ? w * pv[k].z : 0.f;
          o[0].w += use ? w * pv[k].w : 0.f;
        }
      }
#pragma unroll 2
      for (int s = one_row ? s_stop : s_first; s < s_stop; s += s_step) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int m = min(m0 + r0 + u, m_end - 1);
          v[u] = *reinterpret_cast<const float4*>(part_o + (s * split_stride + (size_t)m * 128 + h) * 512 +
                                                  kOCols * p + 4 * cq);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float w = (m0 + r0 + u < m_end) ? wts[s * 32 + r0 + u] : 0.f;
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
          *reinterpret_cast<float4*>(&scratch[(grp * 8 + u) * kOCols + 4 * cq]) = o[u];
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) store_hilo(r0 + u, o[u]);
      }
    }
    // The pass's merged rows are in LDS for every wave (with few rows, after
    // the row groups' sums are added).
    if (pair) {
      __syncthreads();
      if (grp == 0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float4 a = *reinterpret_cast<const float4*>(&scratch[u * kOCols + 4 * cq]);
#pragma unroll
          for (int g2 = 1; g2 < kGroups; ++g2) {
            const float4 c = *reinterpret_cast<const float4*>(&scratch[(8 * g2 + u) * kOCols + 4 * cq]);
            a = make_float4(a.x + c.x, a.y + c.y, a.z + c.z, a.w + c.w);
          }
          store_hilo(u, a);
        }
      }
    }
  };

  // 3. out[32 rows x 128] = o_lat . W_UV[h]; wave w owns columns 32w .. 32w+31.
  const int q16 = lane & 15;
  const int colhalf = (lane >> 4) & 1;
  const lds_u8* trb = to_lds(wt) +
                      ((8 * half + (q16 >> 2)) * kWPitch + 32 * wave + 16 * colhalf + 4 * (q16 & 3)) * 2;
  const lds_u8* ahb = to_lds(o_hi) + (l32 * kOPitch + 8 * half) * 2;
  const lds_u8* alb = to_lds(o_lo) + (l32 * kOPitch + 8 * half) * 2;
  f32x16 acc = {};
  // Slice jc of W_UV[h] (in LDS) against its 128 columns of the pass's rows.
  auto product = [&](int jc) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x4 blo = ld_lds_tr(trb + (16 * ks) * kWPitch * 2);
      const bf16x4 bhi = ld_lds_tr(trb + (16 * ks + 4) * kWPitch * 2);
      const bf16x8 bw = cat(blo, bhi);
      const int koff = ((jc % kSlices) * 128 + 16 * ks) * 2;
      acc = mfma32(ld_lds_bf16x8(ahb + koff), bw, acc);
      acc = mfma32(ld_lds_bf16x8(alb + koff), bw, acc);
    }
  };
  // A slice goes to LDS once every wave is done with the previous one (and
  // with a pair-form scratch there).
  if constexpr (kPasses == 1) {
    // Slices 0 (since step 1), 1 and 2 in registers, 3 once slice 0 is in LDS.
    merge(0);
    if (!one_row) {
      load_w(1, w1);
      load_w(2, w2);
    }
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
  } else {
    // Slices 0 and 1 in registers since step 1; 2 and 3 follow them.
    merge(0);
    __syncthreads();
    store_w(w0);
    __syncthreads();
    load_w(2, w0);
    product(0);
    __syncthreads();
    store_w(w1);
    __syncthreads();
    load_w(3, w1);
    product(1);
    __syncthreads();
    merge(1);                       // overwrites the merged rows (and slice 1 with few rows)
    __syncthreads();
    store_w(w0);
    __syncthreads();
    product(2);
    __syncthreads();
    store_w(w1);
    __syncthreads();
    product(3);
  }
  // acc[r]: row m0 + 8*(r/4) + 4*half + r%4, column 32*wave + l32.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (m < m_end) {
      const __bf16 v = (__bf16)acc[r];
      out[((size_t)m * 128 + h) * 128 + 32 * wave + l32] = __builtin_bit_cast(uint16_t, v);
    }
  }
}

}  // namespace mla

extern "C" hipError_t mla_launch_combine(const float* part_o, const float* part_lse,
                                         const uint16_t* w_uv, uint16_t* out, float* lse_out, int M,
                                         int S, hipStream_t stream) {
  static const hipError_t attr1 = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&mla::combine_kernel<1>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)mla::combine_lds(1, 256));
  static const hipError_t attr2 = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&mla::combine_kernel<2>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)mla::combine_lds(2, 256));
  if (attr1 != hipSuccess) return attr1;
  if (attr2 != hipSuccess) return attr2;
  // One form per call: a single pass while the grid fits one round of one
  // work-group per compute unit (M <= 64), two passes beyond.
  const int passes = M > 64 ? 2 : 1;
  int rb = M <= 32 ? 16 : 32;
  const int grid = 128 * ((M + rb - 1) / rb);
  void* args[] = {&part_o, &part_lse, &w_uv, &out, &lse_out, &M, &S, &rb};
  const void* fn = passes == 2 ? reinterpret_cast<const void*>(&mla::combine_kernel<2>)
                               : reinterpret_cast<const void*>(&mla::combine_kernel<1>);
  return hipLaunchKernel(fn, dim3(grid), dim3(mla::kCmbThreads), args, mla::combine_lds(passes, S), stream);
}
