// Causal MLA prefill in the un-absorbed form.
//
// "Teardown: DeepSeek-V3", section 4: per head the keys are [W_UK c; k_R]
// (128 + 64 values, k_R shared by all heads) and the values W_UV c (128);
// scores are scaled by 1/sqrt(128 + 64).  "DeepSeek-V3" (llm-vis explorer),
// "Scaled dot-product attention": causal mask (position i sees keys <= i) and
// online renormalisation over key blocks.
//
// For T queries per sequence the un-absorbed form needs 2.8x fewer FLOPs than
// attending in the 576-wide latent space, so prefill rebuilds per-head keys and
// values once and runs a flash-attention kernel over them:
//
//   prefill_kv_kernel   K_C[b,h,t,:] = W_UK[h] c_t          (bf16, [B,H,Lpad,128])
//                       V^T[b,h,:,t] = (c_t W_UV[h])^T      (bf16, tile-major
//                                        [B,H,Lpad/64,128,64], keys permuted in 16s)
//   prefill_attn_kernel out[b,i,h,:] = softmax(q . k * scale, causal) V
//
// Work decomposition (MI355X):
//   * reconstruction: one work-group of 8 waves per (sequence, head, 256
//     positions); the 256x512 latent block is an MFMA operand read straight
//     from the paged cache, W_UK[h] and W_UV[h] are staged through LDS in
//     64-row slices; the outputs leave through LDS as whole 16-byte chunks of
//     contiguous rows (a 256-position block of K_C and four 64-key V^T tiles
//     are each one contiguous 64 KB range);
//   * attention: one work-group of 8 waves (2 per SIMD) per (sequence, head,
//     256 queries), wave w owning 32 queries; 64-key tiles ([K_C | k_R] and
//     V^T) stream into LDS with direct-to-LDS loads through a 3-stage ring; S^T = K Q^T and
//     O^T += V^T P^T run on MFMA 32x32x16 with P^T taken straight from the
//     score registers; query blocks are dispatched longest (most keys) first.
#include "mla_common.h"

namespace mla {

constexpr int kPfThreads = 512;                   // 8 waves
constexpr int kPfPos = 256;                       // cached positions per work-group

// ---------------------------------------------------------------------------
// Key order inside V^T rows.  P^T comes out of the score product with lane
// half hh holding keys {4hh..4hh+3, 8+4hh..8+4hh+3} of each 16-key step; V^T
// is stored with each 16-key group in that order so the matching A operand is
// one contiguous 16-byte read.  pos(t) for t in a group: [0-3, 8-11, 4-7, 12-15].
// ---------------------------------------------------------------------------
__device__ __forceinline__ int vt_pos(int t) {
  const int u = t & 15;
  const int q = u >> 2;                       // which 4-key quarter
  const int pq = ((q & 1) << 1) | (q >> 1);   // quarters 0,1,2,3 -> slots 0,2,1,3
  return (t & ~15) | (pq << 2) | (u & 3);
}

// ===========================================================================
// Reconstruction
// ===========================================================================
constexpr int kWkPitch = 64 + 8;     // bf16 per W_UK LDS row (144 B)
constexpr int kWvPitch = 128 + 32;   // bf16 per W_UV LDS row (320 B: rows 16 banks apart,
                                     // so the 4 rows of a transposed read hit disjoint banks)
constexpr int kWkSlice = 128 * kWkPitch;   // bf16 per W_UK slice buffer
constexpr int kWvSlice = 64 * kWvPitch;    // bf16 per W_UV slice buffer

// LDS: the two weight-slice buffers (76 KB), reused after the products for the
// output staging (a 256-position K_C block and four V^T tiles, 128 KB).
constexpr int kKvWBytes = 2 * (kWkSlice + kWvSlice) * 2;
constexpr int kKvLdsBytes = 2 * kPfPos * 128 * 2;
static_assert(kKvWBytes <= kKvLdsBytes && kKvLdsBytes <= 160 * 1024, "reconstruction LDS");

// One work-group of 8 waves (two per SIMD) per 256 positions: the 256 KB of
// W_UK[h] and W_UV[h] a work-group streams through LDS serve 256 positions.
// The weight slices are double buffered through registers.
__global__ __launch_bounds__(kPfThreads, 1) void prefill_kv_kernel(
    const uint16_t* __restrict__ kv, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ w_uk,
    const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ ws_k, uint16_t* __restrict__ ws_vt,
    int max_blocks, int n_tblk) {
  extern __shared__ __attribute__((aligned(16))) unsigned char kv_smem[];
  uint16_t* wk = reinterpret_cast<uint16_t*>(kv_smem);   // [i][j slice] x 2
  uint16_t* wv = wk + 2 * kWkSlice;                      // [j slice][d] x 2

  const int tblk = blockIdx.x % n_tblk;
  const int h = (blockIdx.x / n_tblk) % 128;
  const int b = blockIdx.x / (n_tblk * 128);
  // Unvalidated caller metadata: keep every block-table read inside the row.
  const int L = min(seq_lens[b], max_blocks * 64);
  const int t0 = tblk * kPfPos;
  if (t0 >= L) return;
  const int Lpad = max_blocks * 64;

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, l32 = lane & 31, wave = tid >> 6;
  const int q16 = lane & 15, colhalf = (lane >> 4) & 1;

  // A operand rows: token t = t0 + 32*wave + l32 of sequence b.
  const int t_row = t0 + 32 * wave + l32;
  const int t_clamped = min(t_row, L - 1);     // rows past L are masked at the store
  const uint16_t* crow = kv + ((size_t)block_table[(size_t)b * max_blocks + (t_clamped >> 6)] * 64 +
                               (t_clamped & 63)) * 576 + 8 * half;

  f32x16 acc_k[4], acc_v[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) { acc_k[n] = f32x16{}; acc_v[n] = f32x16{}; }

  const uint16_t* wuk = w_uk + (size_t)h * 128 * 512;
  const uint16_t* wuv = w_uv + (size_t)h * 512 * 128;
  // W_UK as the A operand of K_C^T (rows i, k = j): lane reads row i = 32n + l32,
  // 8 consecutive j at 16*ks + 8*half.  The latent block is then the B operand
  // (columns = positions), so each lane ends up holding 4 consecutive dims of
  // one position, as it does for V^T.
  const int wk_rd = (l32 * kWkPitch + 8 * half) * 2;
  // B operand for V (W_UV: k = j, n = d) by transposed reads: group g = lane/16
  // supplies rows j = 16*ks + 8*(g/2) + q/4 (+4), columns 32n + 16*(g%2) + 4*(q%4).
  const int wv_rd = ((8 * half + (q16 >> 2)) * kWvPitch + 16 * colhalf + 4 * (q16 & 3)) * 2;

  // Slice jc (j = 64jc .. 64jc+63) of both weights: 4 sixteen-byte chunks per
  // thread, global -> registers -> LDS.  Thread chunk k: W_UK row (ch / 8),
  // W_UV row (ch / 16), ch = 512k + tid.
  const uint16_t* wk_src[2];
  const uint16_t* wv_src[2];
  int wk_dst[2], wv_dst[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int ch = k * kPfThreads + tid;
    wk_src[k] = wuk + (size_t)(ch >> 3) * 512 + (ch & 7) * 8;
    wv_src[k] = wuv + (size_t)(ch >> 4) * 128 + (ch & 15) * 8;
    wk_dst[k] = (ch >> 3) * kWkPitch + (ch & 7) * 8;
    wv_dst[k] = (ch >> 4) * kWvPitch + (ch & 15) * 8;
  }
  uint4 sk0, sk1, sv0, sv1;
#define MLA_PF_LOAD_SLICE(jc)                                                       \
  do {                                                                              \
    sk0 = *reinterpret_cast<const uint4*>(wk_src[0] + 64 * (jc));                   \
    sk1 = *reinterpret_cast<const uint4*>(wk_src[1] + 64 * (jc));                   \
    sv0 = *reinterpret_cast<const uint4*>(wv_src[0] + (size_t)64 * 128 * (jc));     \
    sv1 = *reinterpret_cast<const uint4*>(wv_src[1] + (size_t)64 * 128 * (jc));     \
  } while (0)
#define MLA_PF_STORE_SLICE(buf)                                                     \
  do {                                                                              \
    uint16_t* wkb = wk + (buf) * kWkSlice;                                          \
    uint16_t* wvb = wv + (buf) * kWvSlice;                                          \
    *reinterpret_cast<uint4*>(wkb + wk_dst[0]) = sk0;                               \
    *reinterpret_cast<uint4*>(wkb + wk_dst[1]) = sk1;                               \
    *reinterpret_cast<uint4*>(wvb + wv_dst[0]) = sv0;                               \
    *reinterpret_cast<uint4*>(wvb + wv_dst[1]) = sv1;                               \
  } while (0)

  bf16x8 a[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) a[ks] = ld_global_bf16x8(crow + 16 * ks);
  MLA_PF_LOAD_SLICE(0);
  MLA_PF_STORE_SLICE(0);
#pragma unroll
  for (int jc = 0; jc < 8; ++jc) {
    // The next slice's weights and latent operands are in flight meanwhile.
    bf16x8 an[4];
    if (jc + 1 < 8) {
      MLA_PF_LOAD_SLICE(jc + 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) an[ks] = ld_global_bf16x8(crow + 64 * (jc + 1) + 16 * ks);
    }
    __syncthreads();                             // slice jc visible in buffer jc % 2
    const lds_u8* wk_l = to_lds(wk + (jc & 1) * kWkSlice) + wk_rd;
    const lds_u8* wv_l = to_lds(wv + (jc & 1) * kWvSlice) + wv_rd;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bf16x8 bk = ld_lds_bf16x8(wk_l + (32 * n * kWkPitch + 16 * ks) * 2);
        acc_k[n] = mfma32(bk, a[ks], acc_k[n]);
        const bf16x4 lo = ld_lds_tr(wv_l + ((16 * ks) * kWvPitch + 32 * n) * 2);
        const bf16x4 hi = ld_lds_tr(wv_l + ((16 * ks + 4) * kWvPitch + 32 * n) * 2);
        acc_v[n] = mfma32(a[ks], cat(lo, hi), acc_v[n]);
      }
    }
    if (jc + 1 < 8) {
      // Buffer (jc+1) % 2 was last read in iteration jc-1, before this
      // iteration's barrier.
      MLA_PF_STORE_SLICE((jc + 1) & 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) a[ks] = an[ks];
    }
  }
#undef MLA_PF_LOAD_SLICE
#undef MLA_PF_STORE_SLICE

  // acc_k[n][r]: dim 32n + 8*(r/4) + 4*half + r%4 of position t0 + 32*wave + l32;
  // acc_v[n][r]: dim 32n + l32 of position t0 + 32*wave + 8*(r/4) + 4*half + r%4.
  // Positions at or past L are written as zeros.  Both go to LDS as 8-byte
  // pieces (the weight buffers are free once every wave is past this barrier):
  //   K block  [128 positions][16 chunks of 8 dims], chunk c at c ^ (pos & 15);
  //   V^T      [2 tiles][128 dims][8 chunks of 8 keys], chunk c at c ^ ((d >> 1) & 7),
  //            keys in vt_pos() order inside each 16-key group.
  __syncthreads();
  lds_u8* kst = to_lds(kv_smem);                       // 64 KB K_C block
  lds_u8* vst = to_lds(kv_smem) + kPfPos * 256;        // four 16 KB V^T tiles
  {
    const int pk = 32 * wave + l32;            // this lane's K position in the block
    const bool k_ok = t0 + pk < L;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 kk;
#pragma unroll
        for (int e = 0; e < 4; ++e) kk[e] = (__bf16)(k_ok ? acc_k[n][4 * g + e] : 0.f);
        const int c = (4 * n + g) ^ (pk & 15);
        *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(kst + pk * 256 + c * 16 +
                                                                     half * 8) = kk;
      }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int pv = 32 * wave + 8 * g + 4 * half;      // first of 4 consecutive positions
      const int u = vt_pos(pv & 63);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int d = 32 * n + l32;
        bf16x4 vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = (__bf16)(t0 + pv + e < L ? acc_v[n][4 * g + e] : 0.f);
        const int c = (u >> 3) ^ ((d >> 1) & 7);
        *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(
            vst + (pv >> 6) * 16384 + d * 128 + c * 16 + (u & 7) * 2) = vv;
      }
    }
  }
  __syncthreads();
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  // 4096 chunks of each output per work-group, 8 per thread.  Positions past
  // Lpad (the last 256-block may overhang by up to three 64-key tiles) are not
  // stored.
  uint16_t* kdst = ws_k + ((size_t)(b * 128 + h) * Lpad + t0) * 128;
  uint16_t* vdst = ws_vt + ((size_t)(b * 128 + h) * Lpad + t0) * 128;   // tile t0 / 64
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = k * kPfThreads + tid;
    const int r = q >> 4, c = q & 15;
    if (t0 + r < Lpad)
      *reinterpret_cast<u32x4*>(kdst + r * 128 + c * 8) =
          *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(kst + r * 256 +
                                                                             (c ^ (r & 15)) * 16);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = k * kPfThreads + tid;
    const int tile = q >> 10, d = (q >> 3) & 127, c = q & 7;
    if (t0 + 64 * tile < Lpad)
      *reinterpret_cast<u32x4*>(vdst + (tile * 128 + d) * 64 + c * 8) =
          *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
              vst + tile * 16384 + d * 128 + (c ^ ((d >> 1) & 7)) * 16);
  }
}

// ===========================================================================
// Attention
// ===========================================================================
constexpr int kKeyTile = 64;
constexpr int kKRowChunks = 24;                         // 192 bf16 = 24 x 16 B
constexpr int kKTileBytes = kKeyTile * kKRowChunks * 16;  // 24576
constexpr int kVRowChunks = kKeyTile * 2 / 16;          // 8 chunks of 8 keys
constexpr int kVTileBytes = 128 * kVRowChunks * 16;     // 16384
constexpr int kStageBytes = kKTileBytes + kVTileBytes;  // 40960
constexpr int kAttnThreads = 512;                       // 8 waves, 2 per SIMD
constexpr int kQBlock = 256;                            // queries per work-group
constexpr int kRingStages = 3;                          // key tiles: 1 in use, 2 in flight
constexpr int kPfLdsBytes = kRingStages * kStageBytes;  // 122880
constexpr int kKSlotsPerThread = kKeyTile * kKRowChunks / kAttnThreads;   // 3
constexpr int kVSlotsPerThread = 128 * kVRowChunks / kAttnThreads;        // 2
constexpr int kTileLoadsPerThread = kKSlotsPerThread + kVSlotsPerThread;  // 5
static_assert(kKSlotsPerThread * kAttnThreads == kKeyTile * kKRowChunks, "K tile split");
static_assert(kVSlotsPerThread * kAttnThreads == 128 * kVRowChunks, "V tile split");
static_assert(kPfLdsBytes <= 160 * 1024, "LDS budget");

// Chunk placement (same scheme as the decode page): XOR of the low 3 bits of
// the chunk index, so 16 consecutive rows reading one chunk hit 16 distinct
// 4-bank groups of the 64-bank LDS.
__device__ __forceinline__ int k_swz(int key) {
  return (((key >> 1) & 1) << 2) | (((key >> 2) & 1) << 1) | ((key >> 3) & 1);
}
__device__ __forceinline__ int v_swz(int d) { return (d >> 1) & 7; }

// All 512 threads: one 64-key tile ([K_C | k_R] rows and the V^T columns)
// into an LDS stage with 16-byte direct-to-LDS loads (5 per thread).  Measured
// here, the builtin form beats the opaque one: with two waves per SIMD the
// compiler's serialised LDS waits cost less than the operand reads it
// otherwise schedules.
__device__ __forceinline__ void issue_kv_tile(const uint16_t* kc_src,   // ws_k row of key k0
                                              const uint16_t* kr_page,  // cache block of keys k0..
                                              const uint16_t* vt_src,   // V^T tile of keys k0..
                                              lds_u8* stage, int tid) {
  lds_u8* kdst = stage + (tid & ~63) * 16;
#pragma unroll
  for (int it = 0; it < kKSlotsPerThread; ++it) {
    const int slot = it * kAttnThreads + tid;
    const int key = slot / kKRowChunks;
    const int p = slot - key * kKRowChunks;
    const int c = p ^ k_swz(key);
    const void* src = (c < 16) ? static_cast<const void*>(kc_src + (size_t)key * 128 + c * 8)
                               : static_cast<const void*>(kr_page + (size_t)key * 576 + 512 + (c - 16) * 8);
    g2lds16(src, kdst + it * kAttnThreads * 16);
  }
  lds_u8* vdst = stage + kKTileBytes + (tid & ~63) * 16;
#pragma unroll
  for (int it = 0; it < kVSlotsPerThread; ++it) {
    const int slot = it * kAttnThreads + tid;
    const int d = slot >> 3;
    const int c = (slot & 7) ^ v_swz(d);
    g2lds16(vt_src + d * 64 + c * 8, vdst + it * kAttnThreads * 16);
  }
}

__global__ __launch_bounds__(kAttnThreads, 1) void prefill_attn_kernel(
    const uint16_t* __restrict__ q_c, const uint16_t* __restrict__ q_r,
    const uint16_t* __restrict__ kv, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ ws_k,
    const uint16_t* __restrict__ ws_vt, uint16_t* __restrict__ out, int B, int T, int max_blocks,
    int n_qblk, float scale_log2) {
  extern __shared__ __attribute__((aligned(16))) unsigned char pf_smem[];
  lds_u8* smem = to_lds(pf_smem);

  // Longest query blocks first: consecutive ids walk (sequence, head) for the
  // last query block, then the one before, ...
  const int per_q = B * 128;
  const int qblk = n_qblk - 1 - (int)(blockIdx.x / per_q);
  const int bh = blockIdx.x % per_q;
  const int b = bh / 128, h = bh % 128;
  // Unvalidated caller metadata: clamp into [T, max_blocks * 64] (T fits: the
  // host checks it) so that no key index leaves the workspace or the table row.
  const int L = min(max(seq_lens[b], T), max_blocks * 64);
  const int Lpad = max_blocks * 64;

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, l32 = lane & 31, wave = tid >> 6;

  // This lane's query: index i (0..T-1), position L - T + i.
  const int qi = qblk * kQBlock + 32 * wave + l32;
  const bool q_ok = qi < T;
  const int qpos = L - T + qi;
  // Keys needed by the work-group: up to the position of its last valid query.
  const int last_q = min(T - 1, qblk * kQBlock + kQBlock - 1);
  const int n_keys = L - T + last_q + 1;
  const int n_tiles = (n_keys + kKeyTile - 1) / kKeyTile;
  // Position of this wave's first query if all 32 of its queries exist, else
  // -1 (then every tile takes the masked path); last key any of its queries
  // sees (-1: the wave has no query), past which it skips a tile.
  const int wave_q0 = qblk * kQBlock + 32 * wave;
  const int wave_qmin = (wave_q0 + 31 < T) ? L - T + wave_q0 : -1;
  const int wave_kmax = (wave_q0 < T) ? L - T + min(T - 1, wave_q0 + 31) : -1;

  // Q^T as B operands: k-step ks covers dims 16ks .. of [q_C (128); q_R (64)].
  bf16x8 qreg[12];
  {
    const size_t row = ((size_t)b * T + (q_ok ? qi : 0)) * 128 + h;
    const uint16_t* qc = q_c + row * 128 + 8 * half;
    const uint16_t* qr = q_r + row * 64 + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = q_ok ? ld_global_bf16x8(qc + 16 * ks) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qreg[8 + ks] = q_ok ? ld_global_bf16x8(qr + 16 * ks) : bf16x8{};
  }

  const uint16_t* kc_base = ws_k + ((size_t)(b * 128 + h) * Lpad) * 128;
  const uint16_t* vt_base = ws_vt + ((size_t)(b * 128 + h) * 128) * Lpad;   // 64-key tiles of 8192
  const int32_t* table = block_table + (size_t)b * max_blocks;

  auto issue = [&](int tile, lds_u8* stage) {
    const int k0 = tile * kKeyTile;
    issue_kv_tile(kc_base + (size_t)k0 * 128, kv + (size_t)table[k0 >> 6] * 64 * 576, vt_base + (size_t)k0 * 128,
                  stage, tid);
  };
  issue(0, smem);
  if (n_tiles > 1) issue(1, smem + kStageBytes);

  f32x16 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;

  // Per-lane LDS read offsets within a stage.  The swizzle leaves four
  // distinct lane offsets per operand kind; the rest of each address is an
  // immediate.  K: key row l32 (+32 for the second half of the tile), k-step
  // ks = 4q + r reads chunk 8q + ((2r + half) ^ k_swz(l32)).  V^T: row d =
  // 32n + l32, 16-key step k reads chunk (2k + half) ^ v_swz(l32).
  int koff[4], voff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    koff[r] = l32 * kKRowChunks * 16 + (((2 * r + half) ^ k_swz(l32)) * 16);
    voff[r] = kKTileBytes + l32 * kVRowChunks * 16 + (((2 * r + half) ^ v_swz(l32)) * 16);
  }

  for (int i = 0; i < n_tiles; ++i) {
    lds_u8* cur = smem + (i % kRingStages) * kStageBytes;
    // Tile i has landed for every wave; every wave is done with tile i-1,
    // whose stage then takes tile i+2.
    if (i + 1 < n_tiles) wait_vmcnt<kTileLoadsPerThread>(); else wait_vmcnt<0>();
    lds_barrier();
    if (i + 2 < n_tiles) issue(i + 2, smem + ((i + 2) % kRingStages) * kStageBytes);

    const int k0 = i * kKeyTile;
    if (k0 > wave_kmax) continue;               // no query of this wave sees the tile
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) {
        const lds_u8* kp = cur + koff[ks & 3] + kt * 32 * kKRowChunks * 16 + (ks >> 2) * 128;
        s[kt] = mfma32(ld_lds_bf16x8(kp), qreg[ks], s[kt]);
      }
    }
    // s[kt][r]: key k0 + 32kt + 8*(r/4) + 4*half + r%4, query qi.
    // Raw scores; the scale (> 0) is applied inside the exponent below, so the
    // maximum can be taken first.  Only tiles that reach past the wave's first
    // query position need the per-element causal mask.
    float x[32];
    float mx = -INFINITY;
    if (k0 + kKeyTile - 1 <= wave_qmin) {
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        x[r] = s[r >> 4][r & 15];
        mx = fmaxf(mx, x[r]);
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = q_ok && key <= qpos && key < L;
          x[16 * kt + r] = vis ? s[kt][r] : -INFINITY;
          mx = fmaxf(mx, x[16 * kt + r]);
        }
    }
    mx = pair32_max(mx) * scale_log2;     // over lanes l, l^32 (one query's keys); log2 units
    const bool move = mx > m_ref + 8.f;
    if (move) {
      const float alpha = (m_ref == -INFINITY) ? 0.f : fast_exp2(m_ref - mx);
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[n] *= alpha;
      m_ref = mx;
    }
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    bf16x8 pb[4];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const float p = fast_exp2(fmaf(x[r], scale_log2, -m_use));
      l_run += p;
      pb[r >> 3][r & 7] = (__bf16)p;
    }
    // O^T[128 d x 32 q] += V^T[128 x 16 keys] . P^T over four 16-key steps.
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bf16x8 av = ld_lds_bf16x8(cur + voff[kstep] + 32 * n * kVRowChunks * 16);
        acc[n] = mfma32(av, pb[kstep], acc[n]);
      }
    }
  }

  const float l_tot = pair32_sum(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (q_ok) {
    uint16_t* dst = out + (((size_t)b * T + qi) * 128 + h) * 128;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[n][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(dst + 32 * n + 8 * g + 4 * half) = v;
      }
  }
}

}  // namespace mla

extern "C" hipError_t mla_launch_prefill(const uint16_t* q_c, const uint16_t* q_r, const uint16_t* kv,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         const uint16_t* w_uk, const uint16_t* w_uv, uint16_t* out,
                                         void* workspace, int B, int T, int max_blocks,
                                         float softmax_scale, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&mla::prefill_attn_kernel),
      hipFuncAttributeMaxDynamicSharedMemorySize, mla::kPfLdsBytes);
  if (attr != hipSuccess) return attr;
  const size_t Lpad = (size_t)max_blocks * 64;
  uint16_t* ws_k = static_cast<uint16_t*>(workspace);
  uint16_t* ws_vt = ws_k + (size_t)B * 128 * Lpad * 128;
  int n_tblk = (int)((Lpad + mla::kPfPos - 1) / mla::kPfPos);
  {
    static const hipError_t kv_attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&mla::prefill_kv_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize, mla::kKvLdsBytes);
    if (kv_attr != hipSuccess) return kv_attr;
    void* args[] = {&kv, &block_table, &seq_lens, &w_uk, &w_uv, &ws_k, &ws_vt, &max_blocks, &n_tblk};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&mla::prefill_kv_kernel),
                                         dim3(B * 128 * n_tblk), dim3(mla::kPfThreads), args,
                                         mla::kKvLdsBytes, stream);
    if (e != hipSuccess) return e;
  }
  int n_qblk = (T + mla::kQBlock - 1) / mla::kQBlock;
  float scale_log2 = softmax_scale * mla::kLog2e;
  void* args[] = {&q_c, &q_r, &kv, &block_table, &seq_lens, &ws_k, &ws_vt, &out,
                  &B, &T, &max_blocks, &n_qblk, &scale_log2};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::prefill_attn_kernel),
                         dim3(B * 128 * n_qblk), dim3(mla::kAttnThreads), args, mla::kPfLdsBytes,
                         stream);
}

