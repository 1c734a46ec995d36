// Split-KV flash decode over the paged latent cache (absorbed form).
//
// What it computes ("Teardown: DeepSeek-V3", section 4; "DeepSeek-V3" llm-vis
// explorer, "KV latent compression" and "Scaled dot-product attention"):
// for every sequence b, query i and head h, over the tokens t of one split of
// the sequence's pages that the query may see (t <= L_b - Tq + i),
//   s_t   = (q_lat[b,i,h] . c_t + q_R[b,i,h] . k_R,t) * scale
//   o_s   = sum_t softmax(s)_t c_t            (512 wide, fp32)
//   lse_s = ln sum_t exp(s_t)
// with the softmax renormalised online, 32 tokens at a time.
//
// Work decomposition (MI355X: 256 CUs, 64-wide waves, 160 KB LDS per CU):
//   * one work-group of 4 waves per (sequence, split, query); the 128 heads
//     share each cached row, so a tile is loaded once into LDS and used by all
//     128 heads: wave w owns heads 32w .. 32w+31;
//   * each wave keeps its 32 latent queries (512 wide, bf16) in 128 VGPRs as the
//     B operand (the 64-wide rotary queries of all heads sit in LDS) and its
//     output O^T (512 x 32 heads, fp32) in the 256 AGPRs;
//   * per 32-token tile: S^T[32 tok x 32 heads] = K[32 x 576] . Q^T as one
//     chain of 36 MFMA 32x32x16, online softmax in registers (lane = head), then O^T[512 x 32] += V^T[512 x 32 tok] . P^T
//     (32 MFMA; V^T read from the same LDS tile with transposed reads, P^T is the
//     score registers reinterpreted: no shuffles);
//   * software pipeline: the score MFMAs of tile n, then the value MFMAs of
//     tile n-1 with the softmax of tile n issued in pieces between them;
//   * tiles stream global -> LDS with 16-byte direct-to-LDS loads through a ring
//     of 4 stages (2 in flight while 2 are being multiplied), one barrier per
//     tile; wave w loads rows 8w .. 8w+7 of a tile, in 9 pieces spread over the
//     score MFMAs of the tile two ahead, with scalar addresses only;
//   * the score mask runs only on the (at most two) tiles that reach past the
//     query's last visible key; the loop over all other tiles has no mask and
//     no per-load test.
#include <type_traits>

#include "mla_common.h"

namespace mla {

constexpr int kDecThreads = 256;
constexpr int kTok = 64;                        // tokens per cache block
constexpr int kRowVals = 576;                   // 512 latent + 64 rotary
constexpr int kRowBytes = kRowVals * 2;         // 1152
constexpr int kChunks = kRowBytes / 16;         // 72 sixteen-byte chunks per row
constexpr int kTileTok = 32;                    // tokens per pipeline stage
constexpr int kTileBytes = kTileTok * kRowBytes;                 // 36864
constexpr int kRing = 4;                        // stages in the LDS ring
constexpr int kLoadsPerThread = kTileBytes / 16 / kDecThreads;  // 9
constexpr int kQrBytes = 128 * 64 * 2;          // rotary queries of the 128 heads
constexpr int kDecLdsBytes = kRing * kTileBytes + kQrBytes;      // 163840

static_assert(kLoadsPerThread * 16 * kDecThreads == kTileBytes, "tile must split evenly");
static_assert(kDecLdsBytes <= 160 * 1024, "LDS budget");

// Lazy renormalisation threshold (log2 units): unnormalised weights stay <= 2^8.
constexpr float kLazy = 8.f;

// The nine loads of the tile two ahead are issued one every fourth score
// MFMA (after k-steps 1, 5, ..., 33): piece index, or -1.
__host__ __device__ constexpr int qk_piece(int kk) { return (kk & 3) == 1 ? (kk >> 2) : -1; }
static_assert(qk_piece(33) == 8 && qk_piece(35) == -1, "nine pieces over 36 k-steps");

// LDS layout of a 32-row tile.  The tile is cut into 4 x 9 blocks of 8 rows x
// 8 sixteen-byte chunks (1 KB each, block (t/8, c/8) at (t/8)*9 + c/8); inside a
// block, row t%8 holds its 8 chunks with the chunk index XORed by bits 1..3 of
// the row.  On the 64-bank LDS both access patterns are conflict-free: 16
// consecutive rows reading one chunk (score operand, 16 lanes per cycle) and 4
// consecutive rows x 4 adjacent chunks (transposed value reads, 32 lanes per
// cycle).  One 64-lane direct-to-LDS load fills exactly one block.
__device__ __forceinline__ int row_swz(int t) {
  return (((t >> 1) & 1) << 2) | (((t >> 2) & 1) << 1) | ((t >> 3) & 1);
}
constexpr int kBlkBytes = 1024;                 // 8 rows x 8 chunks
constexpr int kRowGrpBytes = 9 * kBlkBytes;     // 8 rows x 72 chunks

// Byte offset of (row t, chunk c) inside a tile.
__device__ __forceinline__ int tile_off(int t, int c) {
  return (t >> 3) * kRowGrpBytes + (c >> 3) * kBlkBytes + (t & 7) * 128 + ((c & 7) ^ row_swz(t)) * 16;
}

// Copy of a 32-row tile into an LDS stage: wave w loads row group w (rows
// 8w .. 8w+7, the 9 blocks (w, 0..8) of 1 KB) in 9 pieces.  Lane j of piece IT
// loads row 8w + j/8, chunk 8 IT + ((j%8) ^ swizzle); its byte offset inside the
// row group (voff) depends only on the lane and the parity of w, so the
// per-tile address work is scalar: the row group's global address is one SGPR
// pair (gw) and each piece adds 128 IT bytes as the instruction's immediate
// offset.  That offset is added to the LDS destination as well (M0 + offset +
// 16 x lane), so M0 = stage_w + 1024 IT - 128 IT puts piece IT at block IT.
// The load is inline asm with M0 set here: as a builtin it is a FLAT
// instruction that may write LDS, after which the compiler makes every later
// LDS wait lgkmcnt(0) and serialises the operand reads issued ahead; the
// hardware counts it in vmcnt only, which the kernel waits on explicitly.
template <int IT>
__device__ __forceinline__ void load_piece(const char* gw, int voff, lds_u8* stage_w) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned>(reinterpret_cast<uintptr_t>(stage_w)));
  const uintptr_t a = reinterpret_cast<uintptr_t>(gw);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32));
  const unsigned long long sb = (static_cast<unsigned long long>(hi) << 32) | lo;
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%4"
               :
               : "v"(voff), "s"(sb), "s"(m0), "n"(IT * (kBlkBytes - 128)), "n"(IT * 128)
               : "m0");
}
// Piece `it` (a compile-time constant at every call site once unrolled).
__device__ __forceinline__ void issue_piece(int it, const char* gw, int voff, lds_u8* stage_w) {
  switch (it) {
    case 0: load_piece<0>(gw, voff, stage_w); break;
    case 1: load_piece<1>(gw, voff, stage_w); break;
    case 2: load_piece<2>(gw, voff, stage_w); break;
    case 3: load_piece<3>(gw, voff, stage_w); break;
    case 4: load_piece<4>(gw, voff, stage_w); break;
    case 5: load_piece<5>(gw, voff, stage_w); break;
    case 6: load_piece<6>(gw, voff, stage_w); break;
    case 7: load_piece<7>(gw, voff, stage_w); break;
    default: load_piece<8>(gw, voff, stage_w); break;
  }
}
static_assert(kLoadsPerThread == 9 && kDecThreads / 64 * 8 == kTileTok, "one row group per wave, 9 pieces");

__global__ __launch_bounds__(kDecThreads, 1) void decode_paged_kernel(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ q_r,
    const uint16_t* __restrict__ kv, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int B, int Tq, int max_blocks, float scale_log2,
    int num_splits, int num_units, float* __restrict__ part_o, float* __restrict__ part_lse) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dec_smem[];
  lds_u8* smem = to_lds(dec_smem);
  lds_u8* qr_lds = smem + kRing * kTileBytes;

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int head = wave * 32 + l32;
  // Source offset of this lane's 16 bytes inside its wave's row group: row
  // lane/8, chunk (lane%8) ^ row_swz(row), where bit 0 of the swizzle is the
  // parity of the row group (= wave).
  int voff;
  {
    const int f = (((lane >> 4) & 1) << 2) | (((lane >> 5) & 1) << 1) | (wave & 1);
    voff = (lane >> 3) * kRowBytes + ((lane & 7) ^ f) * 16;
  }

  const int L = seq_lens[b];
  const int n_pages = (L + kTok - 1) / kTok;
  const int per = (n_pages + num_splits - 1) / num_splits;
  const int p0 = min(n_pages, split * per);
  const int n_vis = L - Tq + qi + 1;                  // keys this query sees
  const int T0 = p0 * kTok;                           // first token of the split
  const int T1 = min(min(n_pages, p0 + per) * kTok, n_vis);
  const int ntiles = (T1 > T0) ? (T1 - T0 + kTileTok - 1) / kTileTok : 0;

  const size_t qrow = (size_t)(b * Tq + qi) * 128;          // first row of this query's heads
  const size_t row = qrow + head;
  float* o_dst = part_o + ((size_t)split * B * Tq * 128 + row) * 512;
  float* lse_dst = part_lse + (size_t)split * B * Tq * 128 + row;

  if (ntiles == 0) {
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
  auto tile_rows = [&](int n) {
    const int t = T0 + n * kTileTok;                  // a tile never crosses a cache block
    return kv + ((size_t)table[t >> 6] * kTok + (t & (kTok - 1))) * kRowVals;
  };

  // Start-up loads, in this order so that one round trip brings what the first
  // score product needs: the latent queries (registers), tile 0, the rotary
  // queries (staged in LDS: waiting for them also waits for everything issued
  // before, vmcnt being in order), then tile 1, which streams in behind.
  // Latent queries as B operands: k-step kk covers dims 16kk .. 16kk+15.
  bf16x8 qreg[32];
  {
    const uint16_t* ql = q_lat + row * 512 + 8 * half;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) qreg[kk] = ld_global_bf16x8(ql + 16 * kk);
  }

  {
    const char* g0 = reinterpret_cast<const char*>(tile_rows(0)) + wave * 8 * kRowBytes;
#pragma unroll
    for (int it = 0; it < kLoadsPerThread; ++it) issue_piece(it, g0, voff, smem + wave * kRowGrpBytes);
  }
  // Rotary queries of all 128 heads -> LDS, [head][64] with the 8 chunks of a
  // row XOR-swizzled by bits 1..3 of the head (16 consecutive heads reading one
  // chunk then hit distinct banks).
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int id = k * kDecThreads + tid;
    const int h = id >> 3, c = id & 7;
    const uint4 v = *reinterpret_cast<const uint4*>(q_r + (qrow + h) * 64 + c * 8);
    st_lds16(qr_lds + (h * 8 + (c ^ ((h >> 1) & 7))) * 16, v);
  }

  if (ntiles > 1) {
    const char* g1 = reinterpret_cast<const char*>(tile_rows(1)) + wave * 8 * kRowBytes;
#pragma unroll
    for (int it = 0; it < kLoadsPerThread; ++it)
      issue_piece(it, g1, voff, smem + kTileBytes + wave * kRowGrpBytes);
  }

  f32x16 acc[16];
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) acc[cb] = f32x16{};
  agpr_settle16(acc);
  float m_ref = -INFINITY;   // exponent reference, log2 units
  float l_run = 0.f;         // this lane's share of sum 2^(x - m_ref)

  // Per-lane LDS offsets.
  // Score operand: lane reads tile row l32, chunk 2kk + half.
  const int sq = row_swz(l32);
  const int qk_base = (l32 >> 3) * kRowGrpBytes + (l32 & 7) * 128;
  const lds_u8* qr_rd = qr_lds + head * 128;
  const int qr_s = (head >> 1) & 7;
  // Transposed value reads: group g = lane/16 (g/2 = half, g%2 = column half),
  // q = lane%16 supplies tile row 16kt + 8rd + 4*half + q/4, columns
  // 32cb + 16*(g%2) + 4*(q%4) .. +3.
  const int q16 = lane & 15;
  const int colhalf = (lane >> 4) & 1;
  const int tr_row = 4 * half + (q16 >> 2);                     // row within its 8-row group
  const int tr_base = tr_row * 128 + (q16 & 1) * 8;
  const int tr_cc = 2 * colhalf + ((q16 & 3) >> 1);             // chunk within 4 of the block
  const int st0 = row_swz(tr_row), st1 = row_swz(tr_row + 8);
  const int tr_e0 = (tr_cc ^ st0) * 16, tr_o0 = ((4 + tr_cc) ^ st0) * 16;   // even / odd cb, rd = 0
  const int tr_e1 = (tr_cc ^ st1) * 16, tr_o1 = ((4 + tr_cc) ^ st1) * 16;   // rd = 1

  // ---- pipeline stages -----------------------------------------------------
  // Tile n+2, loaded in pieces between the score MFMAs of tile n: a burst of
  // nine direct-to-LDS loads per wave would stall the wave at issue while the
  // address unit drains the other waves' loads.
  struct Next {
    const char* g;       // this wave's row group of tile n+2, or null
    lds_u8* stage;       // its LDS destination
  };
  auto top = [&](int n, Next& nx) {
    // Tile n has landed for every wave, every wave is done with tile n-2, whose
    // stage then takes tile n+2.
    if (n + 1 < ntiles) wait_vmcnt<kLoadsPerThread>(); else wait_vmcnt<0>();
    lds_barrier();
    nx.g = nullptr;
    if (n + 2 < ntiles) {
      nx.g = reinterpret_cast<const char*>(tile_rows(n + 2)) + wave * 8 * kRowBytes;
      nx.stage = smem + ((n + 2) % kRing) * kTileBytes + wave * kRowGrpBytes;
    }
    const int valid = L - (T0 + n * kTileTok);        // rows of tile n inside the sequence
    if (valid < kTileTok) {
      // Rows past the sequence end may hold anything (NaN): zero them so that
      // 0-weight tokens contribute exactly 0 to the value product.  They are
      // read by the value product one barrier later.
      lds_u8* stage = smem + (n % kRing) * kTileBytes;
      for (int idx = tid; idx < (kTileTok - valid) * kChunks; idx += kDecThreads) {
        const int t = valid + idx / kChunks;
        st_lds_zero16(stage + tile_off(t, idx % kChunks));
      }
    }
  };

  // Score operand (tile row l32, chunk 2kk + half) and rotary query (k-step 32 + j).
  auto ld_k = [&](const lds_u8* rd, int kk) {
    return ld_lds_bf16x8(rd + (kk >> 2) * kBlkBytes + ((2 * (kk & 3) + half) ^ sq) * 16);
  };
  auto ld_qr = [&](int j) { return ld_lds_bf16x8(qr_rd + ((2 * j + half) ^ qr_s) * 16); };
  // Value operand m = 16kt + cb: V^T rows 32cb.., tokens 16kt + {4h..4h+3, 8+4h..}.
  auto ld_v = [&](const lds_u8* stage, int m) {
    const int kt = m >> 4, cb = m & 15;
    const lds_u8* vrow = stage + 2 * kt * kRowGrpBytes + tr_base + (cb >> 1) * kBlkBytes;
    const bf16x4 lo = ld_lds_tr(vrow + ((cb & 1) ? tr_o0 : tr_e0));
    const bf16x4 hi = ld_lds_tr(vrow + kRowGrpBytes + ((cb & 1) ? tr_o1 : tr_e1));
    return cat(lo, hi);
  };

  // Online softmax of one tile (scores sp, lane = head, 16 tokens per lane) cut
  // into 32 small steps, one after each MFMA of the value product.  A wave
  // issues in order, so a step never waits on a result of the same step: a
  // transcendental's result is consumed at least one MFMA later.
  //   0-7    mask rows past the query's limit (lim), running maximum
  //   8-11   maximum over the lane pair, exponent reference (lazy rescale)
  //   12-27  the 16 exponentials; the sum lags one step
  //   28-31  last sum term, bf16 packing of P, running sum l_run
  struct Softmax {
    float x[16];
    float mx = -INFINITY, m_use = 0.f, sum = 0.f, mxs = 0.f, arg = 0.f;
    bool move = false;
  };
  auto sm_step = [&](auto MASK, int k, int lim, Softmax& st, const f32x16& sp, bf16x8 (&pb)[2], float& alpha,
                     bool& resc) {
    if (k < 8) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 2 * k + e;
        if constexpr (decltype(MASK)::value) st.x[r] = (8 * (r >> 2) + (r & 3) < lim) ? sp[r] : -INFINITY;
        else st.x[r] = sp[r];
        st.mx = fmaxf(st.mx, st.x[r]);
      }
    } else if (k == 8) {
      // maximum over lanes l and l^32 (the two halves of one head's tokens)
      st.mx = pair32_max(st.mx);
    } else if (k == 9) {
      st.mxs = st.mx * scale_log2;                 // log2 units
      st.move = st.mxs > m_ref + kLazy;
    } else if (k == 10) {
      resc = st.move && m_ref != -INFINITY;       // accumulators are still zero otherwise
      st.arg = m_ref - st.mxs;
    } else if (k == 11) {
      alpha = resc ? fast_exp2(st.arg) : 1.f;
      if (st.move) m_ref = st.mxs;
      st.m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    } else if (k < 28) {
      const int r = k - 12;
      st.x[r] = fast_exp2(fmaf(st.x[r], scale_log2, -st.m_use));
      if (r > 0) st.sum += st.x[r - 1];
    } else {
      const int j = k - 28;
      if (j == 0) st.sum += st.x[15];
#pragma unroll
      for (int e = 0; e < 4; ++e) pb[j >> 1][4 * (j & 1) + e] = (__bf16)st.x[4 * j + e];
      if (j == 3) l_run = l_run * alpha + st.sum;
    }
  };
  auto tile_lim = [&](int n) { return n_vis - (T0 + n * kTileTok + 4 * half); };

  // Score product of tile n, one MFMA chain over the 36 k-steps, with the nine
  // loads of tile n+2 spread over it (LD: the caller knows there is a tile
  // n+2, so the loads are issued without a test).  sched_barrier
  // fences pin the order: the LDS reads stay 4 k-steps ahead of their MFMA.
  // The MFMAs are compiler builtins (VGPR form), so the compiler inserts every
  // wait state their results need.  Operands rotate through 6 registers: the
  // load issued after MFMA kk refills the one MFMA kk-2 used.
  auto scores = [&](auto LD, int n, const Next& nx, f32x16& sn) {
    const lds_u8* rd = smem + (n % kRing) * kTileBytes + qk_base;
    bf16x8 kb[6], qrb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kb[j] = ld_k(rd, j);
    f32x16 ae = {};
#pragma unroll
    for (int kk = 0; kk < 36; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 qop = (kk < 32) ? qreg[kk] : qrb[kk - 32];
      ae = mfma32(kb[kk % 6], qop, ae);
      if (kk + 4 < 36) kb[(kk + 4) % 6] = ld_k(rd, kk + 4);
      if (kk >= 28 && kk < 32) qrb[kk - 28] = ld_qr(kk - 28);
      if (qk_piece(kk) >= 0 && (decltype(LD)::value || nx.g != nullptr))
        issue_piece(qk_piece(kk), nx.g, voff, nx.stage);
    }
    __builtin_amdgcn_sched_barrier(0);
    sn = ae;
  };

  // Rare rescale, then O^T += V^T . P^T for tile n (32 MFMAs, value operands
  // read 3 ahead with transposed LDS reads and rotating through 5 registers).
  // With a next tile (scores sp), its softmax runs in pieces between the value
  // MFMAs and leaves P, alpha and the rescale flag for the next call in
  // pb2 / alpha2 / resc2.
  auto rescale_and_pv = [&](auto MASK, int n, bf16x8 (&pb)[2], float alpha, bool resc, bool with_sm,
                            const f32x16& sp, bf16x8 (&pb2)[2], float& alpha2, bool& resc2) {
    valu_to_mfma_settle(pb[0], pb[1]);
    if (__any(resc)) {
      agpr_settle16(acc);
#pragma unroll
      for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) MLA_AGPR_SCALE(acc[cb][r], alpha);
      agpr_settle16(acc);
    }
    const lds_u8* stage = smem + (n % kRing) * kTileBytes;
    const int lim = tile_lim(n + 1);
    Softmax st;
    alpha2 = 1.f;
    resc2 = false;
    bf16x8 vb[5];
#pragma unroll
    for (int j = 0; j < 3; ++j) vb[j] = ld_v(stage, j);
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                   : "+a"(acc[m & 15]) : "v"(vb[m % 5]), "v"(pb[m >> 4]));
      if (m + 3 < 32) vb[(m + 3) % 5] = ld_v(stage, m + 3);
      if (with_sm) sm_step(MASK, m, lim, st, sp, pb2, alpha2, resc2);
    }
  };

  // ---- prologue: scores and softmax of tile 0 ----
  bf16x8 pb[2];
  float alpha = 1.f;
  bool resc = false;
  {
    f32x16 s0;
    Next nx;
    top(0, nx);
    scores(std::false_type{}, 0, nx, s0);
    Softmax st;
#pragma unroll
    for (int k = 0; k < 32; ++k) sm_step(std::true_type{}, k, tile_lim(0), st, s0, pb, alpha, resc);
  }
  // ---- steady state: scores(n), then values(n-1) with softmax(n) ----
  // The softmax of tile n runs in iteration n.  Tiles below n_full are visible
  // to the query in full (no score mask); below n_ld there is also a tile n+2
  // to load.  The remaining (at most two) iterations run the general form.
  const int n_full = min(ntiles, (n_vis - T0) / kTileTok);
  const int n_ld = min(n_full, ntiles - 2);
  int n = 1;
  for (; n < n_ld; ++n) {
    Next nx;
    top(n, nx);
    f32x16 sn;
    scores(std::true_type{}, n, nx, sn);
    bf16x8 pb2[2];
    float alpha2;
    bool resc2;
    rescale_and_pv(std::false_type{}, n - 1, pb, alpha, resc, true, sn, pb2, alpha2, resc2);
    pb[0] = pb2[0];
    pb[1] = pb2[1];
    alpha = alpha2;
    resc = resc2;
  }
  for (; n < ntiles; ++n) {
    Next nx;
    top(n, nx);
    f32x16 sn;
    scores(std::false_type{}, n, nx, sn);
    bf16x8 pb2[2];
    float alpha2;
    bool resc2;
    rescale_and_pv(std::true_type{}, n - 1, pb, alpha, resc, true, sn, pb2, alpha2, resc2);
    pb[0] = pb2[0];
    pb[1] = pb2[1];
    alpha = alpha2;
    resc = resc2;
  }
  {
    bf16x8 pd[2];
    float ad;
    bool rd;
    rescale_and_pv(std::false_type{}, ntiles - 1, pb, alpha, resc, false, f32x16{}, pd, ad, rd);
  }

  agpr_settle16(acc);
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
