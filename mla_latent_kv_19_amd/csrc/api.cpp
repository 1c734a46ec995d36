// Host side of the C ABI declared in include/mla.h: argument checks, launch
// geometry and status mapping.  Kernels live in the .hip files; this file
// only validates and dispatches.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "mla.h"

extern "C" hipError_t mla_launch_absorb_q(const uint16_t* q_c, const uint16_t* w_uk, uint16_t* q_lat,
                                          int M, hipStream_t stream);
extern "C" hipError_t mla_launch_decode_paged(const uint16_t* q_lat, const uint16_t* q_r,
                                              const uint16_t* kv, const int32_t* block_table,
                                              const int32_t* seq_lens, int B, int Tq, int max_blocks,
                                              float softmax_scale, int num_splits, float* part_o,
                                              float* part_lse, unsigned long long* clk,
                                              hipStream_t stream);
extern "C" hipError_t mla_launch_combine(const float* part_o, const float* part_lse,
                                         const uint16_t* w_uv, uint16_t* out, float* lse_out, int M,
                                         int S, hipStream_t stream);
extern "C" hipError_t mla_launch_prefill(const uint16_t* q_c, const uint16_t* q_r,
                                         const uint16_t* kv, const int32_t* block_table,
                                         const int32_t* seq_lens, const uint16_t* w_uk,
                                         const uint16_t* w_uv, uint16_t* out, void* workspace,
                                         int B, int T, int max_blocks, float softmax_scale,
                                         hipStream_t stream);

extern "C" hipError_t mla_launch_decode_noalloc(const uint16_t* q_lat, const uint16_t* q_r,
                                                const uint16_t* kv, const int32_t* block_table,
                                                const int32_t* seq_lens, const uint16_t* w_uv,
                                                uint16_t* out, float* lse_out, int B, int Tq,
                                                int max_blocks, float softmax_scale,
                                                int num_splits, hipStream_t stream);
extern "C" hipError_t mla_launch_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                                hipStream_t stream);
extern "C" int mla_linear_splits(int M, int N, int K);
extern "C" hipError_t mla_launch_cache_append(const uint16_t* x, const uint16_t* w_kv,
                                              const uint16_t* gamma, const int32_t* seq_idx,
                                              const int32_t* positions, const int32_t* block_table,
                                              uint16_t* kv, float* workspace, int M, int d_model,
                                              int max_blocks, float eps, float theta,
                                              hipStream_t stream);

extern "C" size_t mla_query_project_ws(int M, int d_model, int q_rank, int H);
extern "C" hipError_t mla_launch_query_project(const uint16_t* x, const uint16_t* w_dq,
                                               const uint16_t* gamma_q, const uint16_t* w_uq,
                                               const int32_t* positions, uint16_t* q_c,
                                               uint16_t* q_r, void* workspace, int M, int d_model,
                                               int q_rank, int H, float eps, float theta,
                                               hipStream_t stream);
extern "C" size_t mla_output_project_ws(int M, int d_in, int d_out);
extern "C" hipError_t mla_launch_output_project(const uint16_t* o, const uint16_t* w_o,
                                                uint16_t* y, void* workspace, int M, int d_in,
                                                int d_out, hipStream_t stream);

namespace {

// The one shape family the kernels are written for (DeepSeek-V3's MLA dims).
constexpr int kH = 128, kDC = 512, kDR = 64, kDH = 128, kDV = 128, kBlock = 64;
constexpr int kMaxTq = 8;             // query tokens per sequence in one decode call
constexpr int kMaxRows = 65536;
constexpr int kMaxAppendRows = 1 << 20;    // new tokens per cache-append call

int status_of(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  if (e == hipErrorNotSupported) return MLA_ERR_UNSUPPORTED;
  return MLA_ERR_HIP;
}

bool finite_positive(float x) { return std::isfinite(x) && x > 0.f; }

// Decode metadata sizes the kernels' int arithmetic holds: Tq keys fit the
// table row, a row's token count max_blocks * block_size fits an int, and so
// does the split plan's total cost, B * (max_blocks + 6) pages (6: the
// plan's per-sequence cost; the block table then has fewer than 2^31
// entries).
bool plan_fits(int B, int Tq, int max_blocks_per_seq, int block_size) {
  const long row_tokens = (long)max_blocks_per_seq * block_size;
  return (long)Tq <= row_tokens && row_tokens <= INT_MAX &&
         (long)B * ((long)max_blocks_per_seq + 6) <= INT_MAX;
}

}  // namespace

extern "C" {

const char* mla_strerror(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK: success";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: null pointer, non-positive size or bad workspace/splits";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: shape outside H=128, d_c=512, d_r=64, d_h=d_v=128, block 64, Tq<=8";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: the HIP runtime rejected a kernel launch";
    case MLA_ERR_NOALLOC_LIMIT:
      return "MLA_ERR_NOALLOC_LIMIT: num_splits * B * Tq exceeds the library-owned partial buffer "
             "of mla_decode_noalloc (MLA_NOALLOC_MAX_PAIRS)";
    default: return "unknown mla status";
  }
}

int mla_version(void) { return 100; }

int mla_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return MLA_ERR_INVALID_ARG;
  return status_of(mla_launch_hbm_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

int mla_absorb_q(const uint16_t* q_c, const uint16_t* w_uk, uint16_t* q_lat, int M, int H, int d_h,
                 int d_c, void* stream) {
  if (!q_c || !w_uk || !q_lat || M <= 0 || H <= 0 || d_h <= 0 || d_c <= 0 || M > kMaxRows)
    return MLA_ERR_INVALID_ARG;
  if (H != kH || d_h != kDH || d_c != kDC) return MLA_ERR_UNSUPPORTED;
  return status_of(mla_launch_absorb_q(q_c, w_uk, q_lat, M, static_cast<hipStream_t>(stream)));
}

namespace {
int decode_paged_checked(const uint16_t* q_lat, const uint16_t* q_r, const uint16_t* kv_cache,
                         const int32_t* block_table, const int32_t* seq_lens, int B, int Tq, int H,
                         int d_c, int d_r, int num_blocks, int block_size, int max_blocks_per_seq,
                         float softmax_scale, int num_splits, float* part_o, float* part_lse,
                         unsigned long long* clk, void* stream) {
  if (!q_lat || !q_r || !kv_cache || !block_table || !seq_lens || !part_o || !part_lse)
    return MLA_ERR_INVALID_ARG;
  if (B <= 0 || Tq <= 0 || H <= 0 || d_c <= 0 || d_r <= 0 || num_blocks <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || !finite_positive(softmax_scale) || num_splits < 1 ||
      num_splits > MLA_MAX_SPLITS || (long)B * Tq > kMaxRows)
    return MLA_ERR_INVALID_ARG;
  if (H != kH || d_c != kDC || d_r != kDR || block_size != kBlock || Tq > kMaxTq)
    return MLA_ERR_UNSUPPORTED;
  if (!plan_fits(B, Tq, max_blocks_per_seq, block_size)) return MLA_ERR_INVALID_ARG;
  return status_of(mla_launch_decode_paged(q_lat, q_r, kv_cache, block_table, seq_lens, B, Tq,
                                           max_blocks_per_seq, softmax_scale, num_splits, part_o,
                                           part_lse, clk, static_cast<hipStream_t>(stream)));
}
}  // namespace

int mla_decode_paged(const uint16_t* q_lat, const uint16_t* q_r, const uint16_t* kv_cache,
                     const int32_t* block_table, const int32_t* seq_lens, int B, int Tq, int H,
                     int d_c, int d_r, int num_blocks, int block_size, int max_blocks_per_seq,
                     float softmax_scale, int num_splits, float* part_o, float* part_lse,
                     void* stream) {
  return decode_paged_checked(q_lat, q_r, kv_cache, block_table, seq_lens, B, Tq, H, d_c, d_r,
                              num_blocks, block_size, max_blocks_per_seq, softmax_scale,
                              num_splits, part_o, part_lse, nullptr, stream);
}

int mla_decode_paged_clocked(const uint16_t* q_lat, const uint16_t* q_r, const uint16_t* kv_cache,
                             const int32_t* block_table, const int32_t* seq_lens, int B, int Tq,
                             int H, int d_c, int d_r, int num_blocks, int block_size,
                             int max_blocks_per_seq, float softmax_scale, int num_splits,
                             float* part_o, float* part_lse, uint64_t* clock_sums, void* stream) {
  if (!clock_sums || (reinterpret_cast<uintptr_t>(clock_sums) & 7) != 0) return MLA_ERR_INVALID_ARG;
  return decode_paged_checked(q_lat, q_r, kv_cache, block_table, seq_lens, B, Tq, H, d_c, d_r,
                              num_blocks, block_size, max_blocks_per_seq, softmax_scale,
                              num_splits, part_o, part_lse,
                              reinterpret_cast<unsigned long long*>(clock_sums), stream);
}

int mla_combine(const float* part_o, const float* part_lse, const uint16_t* w_uv, uint16_t* out,
                float* lse_out, int B, int Tq, int H, int d_c, int d_v, int num_splits,
                void* stream) {
  if (!part_o || !part_lse || !w_uv || !out || B <= 0 || Tq <= 0 || H <= 0 || d_c <= 0 ||
      d_v <= 0 || num_splits < 1 || num_splits > MLA_MAX_SPLITS || (long)B * Tq > kMaxRows)
    return MLA_ERR_INVALID_ARG;
  if (H != kH || d_c != kDC || d_v != kDV) return MLA_ERR_UNSUPPORTED;
  // The partial rows [S, B, Tq, H, d_c] are (split, query row) pairs: the
  // merge and the up-projection see the B * Tq query rows alike.
  return status_of(mla_launch_combine(part_o, part_lse, w_uv, out, lse_out, B * Tq, num_splits,
                                      static_cast<hipStream_t>(stream)));
}

int mla_decode_noalloc(const uint16_t* q_lat, const uint16_t* q_r, const uint16_t* kv_cache,
                       const int32_t* block_table, const int32_t* seq_lens, const uint16_t* w_uv,
                       uint16_t* out, float* lse_out, int B, int Tq, int H, int d_c, int d_r,
                       int d_v, int num_blocks, int block_size, int max_blocks_per_seq,
                       float softmax_scale, int num_splits, void* stream) {
  if (!q_lat || !q_r || !kv_cache || !block_table || !seq_lens || !w_uv || !out)
    return MLA_ERR_INVALID_ARG;
  if (B <= 0 || Tq <= 0 || H <= 0 || d_c <= 0 || d_r <= 0 || d_v <= 0 || num_blocks <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || !finite_positive(softmax_scale) ||
      num_splits < 1 || num_splits > MLA_MAX_SPLITS || (long)B * Tq > kMaxRows)
    return MLA_ERR_INVALID_ARG;
  if (H != kH || d_c != kDC || d_r != kDR || d_v != kDV || block_size != kBlock || Tq > kMaxTq)
    return MLA_ERR_UNSUPPORTED;
  if (!plan_fits(B, Tq, max_blocks_per_seq, block_size)) return MLA_ERR_INVALID_ARG;
  if ((long)num_splits * B * Tq > MLA_NOALLOC_MAX_PAIRS) return MLA_ERR_NOALLOC_LIMIT;
  return status_of(mla_launch_decode_noalloc(q_lat, q_r, kv_cache, block_table, seq_lens, w_uv,
                                             out, lse_out, B, Tq, max_blocks_per_seq,
                                             softmax_scale, num_splits,
                                             static_cast<hipStream_t>(stream)));
}

size_t mla_decode_workspace_bytes(int B, int Tq, int H, int d_c, int num_splits) {
  const size_t o = mla_decode_part_o_bytes(B, Tq, H, d_c, num_splits);
  const size_t l = mla_decode_part_lse_bytes(B, Tq, H, num_splits);
  if (o == 0 || l == 0) return 0;
  return (o + 255) / 256 * 256 + l;
}

size_t mla_decode_part_o_bytes(int B, int Tq, int H, int d_c, int num_splits) {
  if (B <= 0 || Tq <= 0 || H <= 0 || d_c <= 0 || num_splits <= 0) return 0;
  return (size_t)num_splits * B * Tq * H * d_c * sizeof(float);
}

size_t mla_decode_part_lse_bytes(int B, int Tq, int H, int num_splits) {
  if (B <= 0 || Tq <= 0 || H <= 0 || num_splits <= 0) return 0;
  return (size_t)num_splits * B * Tq * H * sizeof(float);
}

size_t mla_prefill_workspace_bytes(long total_kv_tokens, int H, int d_h, int d_v) {
  if (total_kv_tokens <= 0 || H <= 0 || d_h <= 0 || d_v <= 0) return 0;
  // Rebuilt content keys and values for every addressable cache slot:
  // bf16 [B, H, max_blocks * block_size, d_h + d_v].
  return (size_t)total_kv_tokens * H * (d_h + d_v) * 2;
}

int mla_prefill(const uint16_t* q_c, const uint16_t* q_r, const uint16_t* kv_cache,
                const int32_t* block_table, const int32_t* seq_lens, const uint16_t* w_uk,
                const uint16_t* w_uv, uint16_t* out, void* workspace, size_t workspace_bytes, int B,
                int T, int H, int d_c, int d_r, int d_h, int d_v, int num_blocks, int block_size,
                int max_blocks_per_seq, float softmax_scale, void* stream) {
  if (!q_c || !q_r || !kv_cache || !block_table || !seq_lens || !w_uk || !w_uv || !out ||
      !workspace)
    return MLA_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || H <= 0 || d_c <= 0 || d_r <= 0 || d_h <= 0 || d_v <= 0 ||
      num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 ||
      !finite_positive(softmax_scale) || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return MLA_ERR_INVALID_ARG;
  if (H != kH || d_c != kDC || d_r != kDR || d_h != kDH || d_v != kDV || block_size != kBlock)
    return MLA_ERR_UNSUPPORTED;
  if ((long)T > (long)max_blocks_per_seq * block_size) return MLA_ERR_INVALID_ARG;
  if (workspace_bytes <
      mla_prefill_workspace_bytes((long)B * max_blocks_per_seq * block_size, H, d_h, d_v))
    return MLA_ERR_INVALID_ARG;
  return status_of(mla_launch_prefill(q_c, q_r, kv_cache, block_table, seq_lens, w_uk, w_uv, out,
                                      workspace, B, T, max_blocks_per_seq, softmax_scale,
                                      static_cast<hipStream_t>(stream)));
}

size_t mla_cache_append_workspace_bytes(int M, int d_model) {
  if (M <= 0 || d_model <= 0 || d_model % 16 != 0 || M > kMaxAppendRows) return 0;
  return (size_t)mla_linear_splits(M, kDC + kDR, d_model) * M * (kDC + kDR) * sizeof(float);
}

int mla_cache_append(const uint16_t* x, const uint16_t* w_kv, const uint16_t* gamma,
                     const int32_t* seq_idx, const int32_t* positions, const int32_t* block_table,
                     uint16_t* kv_cache, void* workspace, size_t workspace_bytes, int M,
                     int d_model, int d_c, int d_r, int num_blocks, int block_size,
                     int max_blocks_per_seq, float eps, float rope_theta, void* stream) {
  if (!x || !w_kv || !gamma || !seq_idx || !positions || !block_table || !kv_cache || !workspace)
    return MLA_ERR_INVALID_ARG;
  if (M <= 0 || M > kMaxAppendRows || d_model <= 0 || d_c <= 0 || d_r <= 0 || num_blocks <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || !std::isfinite(eps) || eps < 0.f ||
      !finite_positive(rope_theta) || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return MLA_ERR_INVALID_ARG;
  if (d_c != kDC || d_r != kDR || block_size != kBlock || d_model % 16 != 0)
    return MLA_ERR_UNSUPPORTED;
  if (workspace_bytes < mla_cache_append_workspace_bytes(M, d_model)) return MLA_ERR_INVALID_ARG;
  return status_of(mla_launch_cache_append(x, w_kv, gamma, seq_idx, positions, block_table, kv_cache,
                                           static_cast<float*>(workspace), M, d_model,
                                           max_blocks_per_seq, eps, rope_theta,
                                           static_cast<hipStream_t>(stream)));
}

size_t mla_query_project_workspace_bytes(int M, int d_model, int q_rank) {
  if (M <= 0 || M > kMaxAppendRows || d_model <= 0 || d_model % 16 != 0 || q_rank <= 0 ||
      q_rank % 256 != 0 || q_rank > 4096)
    return 0;
  return mla_query_project_ws(M, d_model, q_rank, kH);
}

int mla_query_project(const uint16_t* x, const uint16_t* w_dq, const uint16_t* gamma_q,
                      const uint16_t* w_uq, const int32_t* positions, uint16_t* q_c, uint16_t* q_r,
                      void* workspace, size_t workspace_bytes, int M, int d_model, int q_rank,
                      int H, int d_h, int d_r, float eps, float rope_theta, void* stream) {
  if (!x || !w_dq || !gamma_q || !w_uq || !positions || !q_c || !q_r || !workspace)
    return MLA_ERR_INVALID_ARG;
  if (M <= 0 || M > kMaxAppendRows || d_model <= 0 || q_rank <= 0 || H <= 0 || d_h <= 0 ||
      d_r <= 0 || !std::isfinite(eps) || eps < 0.f || !finite_positive(rope_theta) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return MLA_ERR_INVALID_ARG;
  if (H != kH || d_h != kDH || d_r != kDR || d_model % 16 != 0 || q_rank % 256 != 0 ||
      q_rank > 4096)
    return MLA_ERR_UNSUPPORTED;
  if (workspace_bytes < mla_query_project_ws(M, d_model, q_rank, H)) return MLA_ERR_INVALID_ARG;
  return status_of(mla_launch_query_project(x, w_dq, gamma_q, w_uq, positions, q_c, q_r, workspace,
                                            M, d_model, q_rank, H, eps, rope_theta,
                                            static_cast<hipStream_t>(stream)));
}

size_t mla_output_project_workspace_bytes(int M, int d_in, int d_out) {
  if (M <= 0 || M > kMaxAppendRows || d_in <= 0 || d_in % 16 != 0 || d_out <= 0 ||
      d_out % 64 != 0)
    return 0;
  return mla_output_project_ws(M, d_in, d_out);
}

int mla_output_project(const uint16_t* o, const uint16_t* w_o, uint16_t* y, void* workspace,
                       size_t workspace_bytes, int M, int d_in, int d_out, void* stream) {
  if (!o || !w_o || !y || !workspace) return MLA_ERR_INVALID_ARG;
  if (M <= 0 || M > kMaxAppendRows || d_in <= 0 || d_out <= 0 ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0 ||
      (reinterpret_cast<uintptr_t>(y) & 7) != 0)
    return MLA_ERR_INVALID_ARG;
  if (d_in % 16 != 0 || d_out % 64 != 0) return MLA_ERR_UNSUPPORTED;
  if (workspace_bytes < mla_output_project_ws(M, d_in, d_out)) return MLA_ERR_INVALID_ARG;
  return status_of(mla_launch_output_project(o, w_o, y, workspace, M, d_in, d_out,
                                             static_cast<hipStream_t>(stream)));
}

int mla_decode_num_splits(int B, int Tq, int H, int max_seq_len, int block_size, int num_cus) {
  if (B <= 0 || Tq <= 0 || H <= 0 || max_seq_len <= 0 || block_size <= 0 || num_cus <= 0) return 0;
  const long groups = (long)B * (((long)Tq * H + 127) / 128);    // work-groups per unit of work
  const long pages = (max_seq_len + block_size - 1) / block_size;
  // Four or more rounds of whole sequences balance by themselves (the
  // hardware starts each as a compute unit frees up), and a single block
  // cannot be cut.  With two rounds the token-balanced plan is faster: B = 64,
  // Tq = 8, L ~ U[4096, 8192] on MI355X 0.811 ms per step with 3 slots against
  // 0.878 ms whole.
  if (groups >= 4L * num_cus || pages == 1) return 1;
  // c splits per sequence fill the chip about once.  Below 64 query rows the
  // decode cuts each sequence into num_splits equal ranges: c.  From 64 rows
  // on it balances the batch's tokens: 2c (room for sequences up to twice the
  // mean length), plus one for a chunk that straddles two sequences, where
  // that is at most 40 (the slots the combine reads in one round trip), else
  // c + 1.
  const long c = (num_cus + groups - 1) / groups;
  long s = (c < pages ? c : pages);
  if (B * (long)Tq >= 64) {
    const long s2 = (2 * c < pages ? 2 * c : pages) + 1;
    s = (s2 <= 40) ? s2 : s + 1;
  }
  if (s > MLA_MAX_SPLITS) s = MLA_MAX_SPLITS;
  return (int)s;
}

}  // extern "C"
