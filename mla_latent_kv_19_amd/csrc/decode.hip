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
//   * one work-group of 4 waves per (unit of work, query); the 128 heads
//     share each cached row, so a tile is loaded once into LDS and used by all
//     128 heads: wave w owns heads 32w .. 32w+31;
//   * from 64 query rows on, units are token-balanced across the batch,
//     planned on the device from seq_lens: the sequences' pages are laid end
//     to end, each sequence charged kPieceCost extra pages for its start-up
//     and write-out, and the line is cut into equal chunks, one per unit (at
//     most the work-groups the chip holds at once).  A unit may cover the end
//     of one sequence and the start of the next: it runs one piece per
//     sequence, each written to the sequence's next partial slot.  Chunks are
//     at least long enough that no sequence needs more than num_splits slots.
//     Smaller batches cut each sequence into num_splits equal ranges (no scan
//     of the lengths before the first load); num_splits = 1 attends each
//     sequence whole;
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
#include <algorithm>
#include <atomic>
#include <climits>
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
constexpr int kQStageBytes = 32 * 512;          // one wave's half query rows (start-up staging)

static_assert(kLoadsPerThread * 16 * kDecThreads == kTileBytes, "tile must split evenly");
static_assert(kDecLdsBytes <= 160 * 1024, "LDS budget");
static_assert(4 * kQStageBytes <= 2 * kTileBytes, "query staging inside stages 2 and 3");
static_assert(4 * 32 * (256 + 4) * 4 <= kRing * kTileBytes, "epilogue transpose area inside the ring");

// Lazy renormalisation threshold (log2 units): unnormalised weights stay <= 2^8.
constexpr float kLazy = 8.f;

// Fixed cost of one piece (load of the queries, pipeline fill, write-out of
// the partial, and the partial's share of the combine), in pages of attention
// work, for the token-balanced split: a piece costs about as much as five to
// six pages at decode clocks, and a chunk of at most kPieceCost + 1 never
// holds two pieces (that takes a page, a sequence start and another page).  Batches whose sequences all have the same page
// count are cut without it, so that chunks fall on sequence boundaries.
constexpr int kPieceCost = 6;
// Query rows (B * Tq) from which the split is token-balanced.
constexpr int kBalanceMinRows = 64;

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
// One 16-byte direct-to-LDS load per lane: lane j's bytes land at
// dst + 16 j; the source is sbase + voff (sbase wave-uniform, voff per lane).
__device__ __forceinline__ void dma16(const char* sbase, unsigned voff, lds_u8* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned>(reinterpret_cast<uintptr_t>(dst)));
  const uintptr_t a = reinterpret_cast<uintptr_t>(sbase);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32));
  const unsigned long long sb = (static_cast<unsigned long long>(hi) << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(m0)
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

// Wave-wide reductions and scan used by the split planning (results in every
// lane).
__device__ __forceinline__ unsigned wave_incl_scan_u32(unsigned x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const unsigned y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}
__device__ __forceinline__ unsigned wave_sum_u32(unsigned x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x += __shfl_xor(x, d);
  return x;
}
__device__ __forceinline__ int wave_max_i32(int x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x = max(x, __shfl_xor(x, d));
  return x;
}
__device__ __forceinline__ int wave_min_i32(int x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x = min(x, __shfl_xor(x, d));
  return x;
}

__global__ __launch_bounds__(kDecThreads, 1) void decode_paged_kernel(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ q_r,
    const uint16_t* __restrict__ kv, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int B, int Tq, int max_blocks, float scale_log2,
    int num_splits, int plan, int num_units, float* __restrict__ part_o, float* __restrict__ part_lse,
    unsigned long long* __restrict__ clk) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dec_smem[];
  // Measurement only (clk is null in normal use): shader-clock cycles and
  // 100 MHz real-time ticks of this work-group, summed into clk[0] / clk[1].
  unsigned long long c0 = 0, r0 = 0;
  if (clk != nullptr) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  lds_u8* smem = to_lds(dec_smem);
  lds_u8* qr_lds = smem + kRing * kTileBytes;

  // Work-group -> (unit, query).  Consecutive ids go to different XCDs; the
  // Tq work-groups of one unit get ids 8 apart so they land on the same XCD
  // and share its L2 for the unit's pages.
  const int wg = blockIdx.x;
  const int k8 = wg >> 3;
  const int qi = k8 % Tq;
  const int unit = (k8 / Tq) * 8 + (wg & 7);
  if (unit >= num_units) return;

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

  // seq_lens is caller metadata that is not validated on the host: each
  // length is clamped into [Tq, max_blocks * 64] so that no block-table read
  // leaves its row.
  const int len_cap = max_blocks * kTok;
  auto seq_len = [&](int bb) { return min(max(seq_lens[bb], Tq), len_cap); };
  const size_t slot_stride = (size_t)B * Tq * 128;   // floats of part_lse per slot

  // One piece: tokens [64 pg_lo, 64 pg_hi) of sequence b (length L), written
  // to partial slot `slot`; `last` marks the sequence's last piece, which also
  // marks the slots after it as empty.
  auto run_piece = [&](int b, int L, int pg_lo, int pg_hi, int slot, bool last) {
    const int n_vis = L - Tq + qi + 1;                  // keys this query sees
    const int T0 = pg_lo * kTok;                        // first token of the piece
    const int T1 = min(pg_hi * kTok, n_vis);
    const int ntiles = (T1 > T0) ? (T1 - T0 + kTileTok - 1) / kTileTok : 0;

    const size_t qrow = (size_t)(b * Tq + qi) * 128;          // first row of this query's heads
    // Per-lane addresses are a uniform base plus a 32-bit lane offset: a
    // 64-bit per-lane pointer would stay live across the pieces (and spill).
    float* lse_row = part_lse + (size_t)slot * slot_stride + qrow;    // [head]
    if (last && half == 0)
      for (int s2 = slot + 1; s2 < num_splits; ++s2) part_lse[(size_t)s2 * slot_stride + qrow + head] = -INFINITY;

    if (ntiles == 0) {
      // Nothing visible in this piece: lse = -inf, which the combine reads as
      // weight 0 without reading the partial output.
      if (half == 0) lse_row[head] = -INFINITY;
      return;
    }

    const int32_t* table = block_table + (size_t)b * max_blocks;
    auto tile_rows = [&](int n) {
      const int t = T0 + n * kTileTok;                  // a tile never crosses a cache block
      return kv + ((size_t)table[t >> 6] * kTok + (t & (kTok - 1))) * kRowVals;
    };

    // Start-up loads.  The latent queries (B operands: k-step kk covers dims
    // 16kk .. 16kk+15, lane = head) are staged through LDS as whole row pieces:
    // loaded straight into registers, every instruction would read 32 bytes
    // from each of 32 head rows (32 cache lines), and the 128 KB of queries
    // took ~1k line requests per wave.  Stages 2 and 3 of the ring are free
    // until tile 2's loads (after the first tile barrier), room for half the
    // queries: round 0 brings dims 0..255 of the wave's 32 rows, round 1 dims
    // 256..511, each 16 direct-to-LDS loads of two 512-byte row halves, their
    // 16-byte chunks XOR-swizzled by the row's low 4 bits (the operand reads,
    // 16 rows at one chunk, then hit distinct banks).  Order: round 0, tile 0,
    // the rotary queries (registers -> LDS), round 0 read out, then round 1 and
    // tile 1 together; the first tile's wait covers round 1, which is read out
    // before its barrier (tile 2's loads overwrite the staging area after it).
    bf16x8 qreg[32];
    lds_u8* q_stage = smem + 2 * kTileBytes + wave * kQStageBytes;
    const char* q_rows = reinterpret_cast<const char*>(q_lat + (qrow + 32 * wave) * 512);
    // The per-lane source offsets depend only on the lane: computed from a
    // register the compiler cannot see is the lane id, so that they are not
    // hoisted out of the loop over pieces and kept alive (spilled) across it.
    auto issue_q_round = [&](int rnd) {
      int ln;
      asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = 2 * j + (ln >> 5);                  // row of this lane's chunk
        const int c = (ln & 31) ^ (r & 15);               // source chunk of LDS slot ln & 31
        dma16(q_rows, static_cast<unsigned>(r * 1024 + rnd * 512 + c * 16), q_stage + j * 1024);
      }
    };
    auto read_q_round = [&](int rnd) {
      int ln;
      asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane) : "memory");
      const int r = ln & 31, h = ln >> 5;
#pragma unroll
      for (int k = 0; k < 16; ++k)
        qreg[16 * rnd + k] = ld_lds_bf16x8(q_stage + r * 512 + (((2 * k + h) ^ (r & 15)) * 16));
    };
    issue_q_round(0);

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

    // Round 0 has landed (it precedes everything still outstanding): read it
    // out, then refill the staging area with round 1.
    wait_vmcnt<0>();
    read_q_round(0);
    __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    issue_q_round(1);

    if (ntiles > 1) {
      const char* g1 = reinterpret_cast<const char*>(tile_rows(1)) + wave * 8 * kRowBytes;
#pragma unroll
      for (int it = 0; it < kLoadsPerThread; ++it)
        issue_piece(it, g1, voff, smem + kTileBytes + wave * kRowGrpBytes);
    }

    // Zeroed from a register the compiler cannot see is zero: a constant
    // initialisation would be hoisted out of the loop over pieces, and its
    // 256 zeros kept alive (spilled) across the whole piece.
    float zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    f32x16 acc[16];
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][r] = zero;
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
    auto top = [&](auto FIRST, int n, Next& nx) {
      // Page of tile n+2: a scalar load issued now, so that the wait of the
      // barrier below covers it (issued after the barrier, its wait stalled the
      // start of the score product of every wave).
      const int pg2 = (n + 2 < ntiles) ? table[(T0 + (n + 2) * kTileTok) >> 6] : 0;
      // This wave's rows of tile n have landed (its own direct-to-LDS loads).
      if (n + 1 < ntiles) wait_vmcnt<kLoadsPerThread>(); else wait_vmcnt<0>();
      // First tile: query round 1 (issued before tile 1) has landed too; read
      // it out before the barrier, after which tile 2 overwrites the area.
      if constexpr (decltype(FIRST)::value) read_q_round(1);
      const int valid = L - (T0 + n * kTileTok);        // rows of tile n inside the sequence
      if (valid < 8 * wave + 8) {
        // Rows past the sequence end may hold anything (NaN): each wave zeroes
        // the ones of its own row group (its loads of them are complete) so
        // that 0-weight tokens contribute exactly 0 to the value product; the
        // barrier below publishes the zeroes before any wave reads the tile.
        // Nobody reads this stage's previous tile any more: its value product
        // ended before the barrier of iteration n - 2.
        lds_u8* stage = smem + (n % kRing) * kTileBytes;
        for (int idx = lane; idx < 8 * kChunks; idx += 64) {
          const int t = 8 * wave + idx / kChunks;
          if (t >= valid) st_lds_zero16(stage + tile_off(t, idx % kChunks));
        }
      }
      // Tile n is complete for every wave, every wave is done with tile n-2,
      // whose stage then takes tile n+2.
      lds_barrier();
      nx.g = nullptr;
      if (n + 2 < ntiles) {
        nx.g = reinterpret_cast<const char*>(
                   kv + ((size_t)pg2 * kTok + ((T0 + (n + 2) * kTileTok) & (kTok - 1))) * kRowVals) +
               wave * 8 * kRowBytes;
        nx.stage = smem + ((n + 2) % kRing) * kTileBytes + wave * kRowGrpBytes;
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
    // read 3 ahead with transposed LDS reads and rotating through 5 registers;
    // the two token halves of one accumulator block are multiplied back to
    // back, ~2 % fewer cycles than 16 blocks apart).
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
      // m -> (cb = m >> 1, token half kt = m & 1): the two k-steps of one
      // accumulator back to back.
      for (int j = 0; j < 3; ++j) vb[j] = ld_v(stage, ((j & 1) << 4) | (j >> 1));
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(acc[m >> 1]) : "v"(vb[m % 5]), "v"(pb[m & 1]));
        if (m + 3 < 32) vb[(m + 3) % 5] = ld_v(stage, (((m + 3) & 1) << 4) | ((m + 3) >> 1));
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
      top(std::true_type{}, 0, nx);
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
      top(std::false_type{}, n, nx);
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
      top(std::false_type{}, n, nx);
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
    // Partial o_s out through LDS: lane = head holds 4-column pieces of its
    // head's row, so stored directly every instruction would touch 32 rows; the
    // wave writes its O^T into a [32 heads][256 + 4] fp32 area of the (now idle)
    // ring and reads it back a head row at a time, so every global store is one
    // contiguous 1 KB.  Two rounds of 256 columns; each wave uses its own area.
    constexpr int kOPitchF = 256 + 4;                  // floats per row: conflict-free writes
    lds_barrier();                                     // every wave is done with the ring
    lds_u8* o_lds = smem + wave * 32 * kOPitchF * 4;
    float* o_row0 = part_o + ((size_t)slot * slot_stride + qrow + wave * 32) * 512;
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd) {
#pragma unroll
      for (int c8 = 0; c8 < 8; ++c8)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int cb = 8 * rnd + c8;
          const f32x4 v = {acc[cb][4 * a] * inv, acc[cb][4 * a + 1] * inv, acc[cb][4 * a + 2] * inv,
                           acc[cb][4 * a + 3] * inv};
          *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(
              o_lds + (l32 * kOPitchF + c8 * 32 + 8 * a + 4 * half) * 4) = v;
        }
#pragma unroll 4
      for (int h = 0; h < 32; ++h) {
        const f32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
            o_lds + (h * kOPitchF + 4 * lane) * 4);
        *reinterpret_cast<f32x4*>(o_row0 + (size_t)h * 512 + 256 * rnd + 4 * lane) = v;
      }
    }
    if (half == 0) lse_row[head] = (l_tot > 0.f) ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  };

  // ---- this unit's pieces ----
  // Plan 0 (one slot per sequence): a unit is a whole sequence.
  // Plan 1 (per-sequence equal split): unit = (sequence b, split j); b's
  // pages are cut into num_splits ranges of ceil(pages_b / num_splits), the
  // trailing ones possibly empty; split j goes to slot j.
  // Plan 2 (token-balanced): every wave scans seq_lens (64 sequences per
  // step): the total cost tot (pages, plus kPieceCost per sequence unless all
  // have the same page count), then
  // chunk = max(ceil(tot / num_units), ceil(longest / (num_splits - 1))) and
  // unit u covers cost positions [u chunk, (u + 1) chunk).  Sequence b's pages
  // sit at [q_b, q_b + pages_b), q_b = (cost of the sequences before it) +
  // its own start-up cost; its piece in unit u goes to slot u - q_b / chunk.
  // A sequence of p pages meets at most floor((p - 1) / chunk) + 2 units,
  // which the second term of chunk keeps <= num_splits; the unit holding a
  // sequence's last piece marks its later slots empty.
  int chunk = 1, u_lo = 0, u_hi = 0, extra = 0;
  int lv = 0;          // plan 2: lengths of the current 64 sequences, one per lane
  if (plan == 2) {
    // The host guarantees B * (max_blocks + kPieceCost) <= INT_MAX, so every
    // cost position fits an int.
    int tot = 0, pmax = 0, pmin = INT_MAX;
    for (int c = 0; c < B; c += 64) {
      const int bb = c + lane;
      const int lc = (bb < B) ? seq_len(bb) : 0;
      if (c == 0) lv = lc;                            // kept for the first step below
      const int pv = (lc + kTok - 1) / kTok;
      tot += static_cast<int>(wave_sum_u32(static_cast<unsigned>(pv)));
      pmax = max(pmax, wave_max_i32(pv));
      pmin = min(pmin, wave_min_i32((bb < B) ? pv : INT_MAX));
    }
    extra = (pmin == pmax) ? 0 : kPieceCost;
    tot += B * extra;
    chunk = max((tot + num_units - 1) / num_units, (pmax + num_splits - 2) / (num_splits - 1));
    if (unit >= (tot + chunk - 1) / chunk) return;    // past the last chunk
    u_lo = unit * chunk;
    u_hi = (tot - u_lo > chunk) ? u_lo + chunk : tot;
  }
  // Scan state of plan 2: chunk of sequences c, the pieces of this unit in it
  // still to run (mask), the lengths (lv) and cost positions relative to carry
  // (qrel) of its 64 sequences, one per lane.
  int c = -64, carry = 0, chunk_cost = 0, qrel = 0;
  unsigned long long mask = 0;
  bool first = true;
  for (;;) {
    int b, L, pg_lo, pg_hi, slot, last = 0;
    if (plan != 2) {
      if (!first) break;
      b = (plan == 0) ? unit : unit / num_splits;
      slot = unit - b * num_splits;
      L = seq_len(b);
      const int n_pages = (L + kTok - 1) / kTok;
      const int per = (n_pages + num_splits - 1) / num_splits;
      pg_lo = min(n_pages, slot * per);
      pg_hi = min(n_pages, pg_lo + per);
    } else {
      while (mask == 0) {
        if (c >= 0) carry += chunk_cost;
        c += 64;
        if (c >= B || carry >= u_hi) break;
        const int bb = c + lane;
        if (c > 0) lv = (bb < B) ? seq_len(bb) : 0;
        const int pv = (lv + kTok - 1) / kTok;
        const int cost = (bb < B) ? pv + extra : 0;
        const int incl = static_cast<int>(wave_incl_scan_u32(static_cast<unsigned>(cost)));
        qrel = incl - cost + extra;
        chunk_cost = __builtin_amdgcn_readlane(incl, 63);
        const int qv = carry + qrel;
        mask = __ballot(bb < B && qv + pv > u_lo && qv < u_hi);
      }
      if (mask == 0) break;
      const int i = __builtin_ctzll(mask);
      mask &= mask - 1;
      b = c + i;
      L = __builtin_amdgcn_readlane(lv, i);
      const int n_pages = (L + kTok - 1) / kTok;
      const int q0 = carry + __builtin_amdgcn_readlane(qrel, i);
      pg_lo = max(u_lo, q0) - q0;
      pg_hi = min(u_hi, q0 + n_pages) - q0;
      slot = unit - q0 / chunk;
      last = (q0 + n_pages - 1) / chunk == unit;
    }
    // The previous piece's write-out read the ring: every wave is done with
    // it before this piece's loads land there.
    if (!first) lds_barrier();
    first = false;
    run_piece(__builtin_amdgcn_readfirstlane(b), __builtin_amdgcn_readfirstlane(L),
              __builtin_amdgcn_readfirstlane(pg_lo), __builtin_amdgcn_readfirstlane(pg_hi),
              __builtin_amdgcn_readfirstlane(slot), __builtin_amdgcn_readfirstlane(last) != 0);
  }
  if (clk != nullptr && tid == 0) {
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    atomicAdd(clk, c1 - c0);
    atomicAdd(clk + 1, r1 - r0);
  }
}

// Compute units and accelerator complex dies (XCDs) of the current device,
// cached per device.  Consecutive work-group ids go to different XCDs.
hipError_t device_cu_count(int* cus, int* xcds) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached_cus[kMaxDevices], cached_xcds[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int n = cached_cus[dev].load(std::memory_order_relaxed);
  int x = cached_xcds[dev].load(std::memory_order_relaxed);
  if (n <= 0 || x <= 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n <= 0) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x <= 0 ||
        n % x != 0)
      x = 1;
    cached_cus[dev].store(n, std::memory_order_relaxed);
    cached_xcds[dev].store(x, std::memory_order_relaxed);
  }
  *cus = n;
  *xcds = x;
  return hipSuccess;
}

}  // namespace mla

extern "C" hipError_t mla_launch_decode_paged(
    const uint16_t* q_lat, const uint16_t* q_r, const uint16_t* kv, const int32_t* block_table,
    const int32_t* seq_lens, int B, int Tq, int max_blocks, float softmax_scale, int num_splits,
    float* part_o, float* part_lse, unsigned long long* clk, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&mla::decode_paged_kernel),
      hipFuncAttributeMaxDynamicSharedMemorySize, mla::kDecLdsBytes);
  if (attr != hipSuccess) return attr;
  // One slot per sequence: one unit per sequence (plan 0).  Fewer than 64
  // query rows: one unit per (sequence, split) (plan 1, no scan of the
  // lengths: the lowest start-up latency).  Otherwise the token-balanced plan
  // 2 with as many units as the chip holds work-groups at once, but no more
  // than B * num_splits, the most pieces the slots can take (the plan's chunk
  // length adapts to the count).  Work-group ids go round-robin over the
  // XCDs and the Tq work-groups of a unit share one, so each XCD gets
  // floor(its compute units / Tq) units: with cus / Tq units, for Tq = 5 on
  // 8 XCDs of 32, three would get 35 work-groups and run a second round.
  int plan = (num_splits == 1) ? 0 : ((long)B * Tq < mla::kBalanceMinRows ? 1 : 2);
  int num_units = (plan == 1) ? B * num_splits : B;
  if (plan == 2) {
    int cus = 0, xcds = 1;
    const hipError_t e = mla::device_cu_count(&cus, &xcds);
    if (e != hipSuccess) return e;
    const long per_xcd = cus / xcds;
    const long resident = per_xcd >= Tq ? xcds * (per_xcd / Tq) : cus / Tq;
    num_units = static_cast<int>(std::max(1L, std::min(resident, (long)B * num_splits)));
  }
  const int grid = ((num_units + 7) / 8) * 8 * Tq;
  float scale_log2 = softmax_scale * mla::kLog2e;
  void* args[] = {&q_lat, &q_r, &kv, &block_table, &seq_lens, &B, &Tq, &max_blocks,
                  &scale_log2, &num_splits, &plan, &num_units, &part_o, &part_lse, &clk};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla::decode_paged_kernel), dim3(grid),
                         dim3(mla::kDecThreads), args, mla::kDecLdsBytes, stream);
}
