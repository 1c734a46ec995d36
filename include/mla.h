/*
 * mla.h -- C ABI of libmla.so: multi-head latent attention (MLA) over the
 * latent KV cache, hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources named by page title and section):
 *   "Teardown: DeepSeek-V3", section 4 "Multi-head latent attention":
 *     per token the cache holds the content latent c (d_c = 512) and one
 *     rotary key k_R (d_r = 64) shared by all heads; per head h the content
 *     key is k_C = W_UK c (d_h = 128), the value is v = W_UV c (d_v = 128);
 *     query [q_C; q_R] and key [k_C; k_R] are scored with scale
 *     1/sqrt(128 + 64); W_UK folds into the query at inference.
 *   "DeepSeek-V3" (llm-vis explorer), boxes "KV latent compression" (cache
 *     row = latent then rotary key; q^T (W_uk c) = (W_uk^T q)^T c; the value
 *     up-projection folds into the output side) and "Scaled dot-product
 *     attention" (softmax(q k^T * scale) v, causal mask, online
 *     renormalisation over key blocks).
 *
 * Decode runs in the absorbed form:
 *   mla_absorb_q      q_lat[m,h,:] = q_C[m,h,:] . W_UK[h]            (512 wide)
 *   mla_decode_paged  per split s of each sequence's pages:
 *                     s_t = (q_lat . c_t + q_R . k_R,t) * scale,
 *                     o_s = sum_t softmax(s)_t c_t,  lse_s = ln sum_t e^{s_t}
 *   mla_combine       o_lat = sum_s e^{lse_s - lse} o_s,  lse = ln sum_s e^{lse_s},
 *                     out[m,h,:] = o_lat . W_UV[h]                   (128 wide)
 * Prefill runs in the un-absorbed form (keys and values rebuilt per head).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or synchronises; each call only enqueues
 *     kernels on `stream` (a hipStream_t passed as void*; NULL = null stream)
 *     and returns.
 *   - Tensors are dense, row-major, contiguous.  bf16 values are passed as
 *     uint16_t bit patterns; fp32 as float; indices as int32_t.
 *   - Weight index order: w_uk is [H, d_h, d_c] with w_uk[h,i,j] multiplying
 *     c[j] into k_C[i]; w_uv is [H, d_c, d_v] with w_uv[h,j,d] multiplying
 *     c[j] into v[d].
 *   - Cache: kv_cache is [num_blocks, block_size, d_c + d_r]; a row is c then
 *     k_R.  block_table[b, p] names the block holding tokens
 *     [p*block_size, (p+1)*block_size) of sequence b.
 *   - seq_lens[b] = L_b counts every cached token of sequence b INCLUDING the
 *     Tq (or T) query tokens, which are already in the cache.  Query i of a
 *     sequence sits at position L_b - Tq + i and sees tokens 0 .. L_b - Tq + i.
 *   - Supported shapes: H = 128, d_c = 512, d_r = 64, d_h = d_v = 128,
 *     block_size = 64, 1 <= Tq <= 8 for decode (one token, or a token and up
 *     to 7 speculative drafts verified together).  Other values return
 *     MLA_ERR_UNSUPPORTED.  NULL pointers, non-positive sizes, a too-small
 *     workspace or num_splits outside [1, MLA_MAX_SPLITS] return
 *     MLA_ERR_INVALID_ARG.  A HIP launch error returns MLA_ERR_HIP.
 *   - Device-resident metadata (seq_lens, block_table) is NOT validated (that
 *     would need a synchronisation).  Preconditions: Tq <= L_b <=
 *     max_blocks_per_seq * block_size; 0 <= block_table[b,p] < num_blocks for
 *     p < ceil(L_b / block_size); no block shared between sequences.  Entries
 *     past a sequence's last block, rows past L_b in its last block and unused
 *     blocks may hold anything (NaN included): they never reach an output.
 *   - A query row that sees no key in a split gets o_s = 0 and lse_s = -inf.
 *   - No mutable global state: calls on different streams may run
 *     concurrently.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,
  MLA_ERR_UNSUPPORTED = 2,
  MLA_ERR_HIP = 3,
  MLA_ERR_NOALLOC_LIMIT = 4
};

/* Largest num_splits accepted by mla_decode_paged / mla_combine. */
#define MLA_MAX_SPLITS 256

/* Most (split, query row) pairs, num_splits * B * Tq, that mla_decode_noalloc
 * keeps in its library-owned buffer (160 MiB + 320 KiB per GPU: a decode step of
 * 64 sequences with the 9 slots mla_decode_num_splits suggests fits). */
#define MLA_NOALLOC_MAX_PAIRS 640

/* Static string describing a status code (never NULL). */
const char* mla_strerror(int status);

/* Version of this ABI (major * 10000 + minor * 100 + patch). */
int mla_version(void);

/*
 * q-absorption.  Source: "DeepSeek-V3" (llm-vis explorer), box "KV latent
 * compression" (q^T (W_uk c) = (W_uk^T q)^T c: the key up-projection folds
 * into the query); "Teardown: DeepSeek-V3", section 4 (W_UK of each head maps
 * the 512-wide latent to the 128-wide content key).
 *   q_lat[m, h, j] = sum_i q_c[m, h, i] * w_uk[h, i, j]     (fp32 accumulate)
 * q_c   bf16 [M, H, d_h]   (M = B * Tq query rows), read only
 * w_uk  bf16 [H, d_h, d_c], read only
 * q_lat bf16 [M, H, d_c]   written, rounded to nearest even
 * M may be any value in [1, 65536].  Errors: MLA_ERR_INVALID_ARG for NULL
 * pointers or M outside that range, MLA_ERR_UNSUPPORTED for other dims.
 */
int mla_absorb_q(const uint16_t* q_c, const uint16_t* w_uk, uint16_t* q_lat,
                 int M, int H, int d_h, int d_c, void* stream);

/*
 * Split-KV flash decode over the paged latent cache: scores, online softmax,
 * causal mask and the per-split partials of the absorbed form.  Source:
 * "Teardown: DeepSeek-V3", section 4 (score = [q_C; q_R] . [k_C; k_R] /
 * sqrt(128 + 64), k_R shared by the heads, only c and k_R cached);
 * "DeepSeek-V3" (llm-vis explorer), boxes "KV latent compression" (the
 * absorbed query scores the cached latent directly) and "Scaled dot-product
 * attention" (softmax(q k^T * scale) v with the causal mask, renormalised
 * online block by block).
 * q_lat  bf16 [B, Tq, H, d_c]   from mla_absorb_q, read only
 * q_r    bf16 [B, Tq, H, d_r]   rotary part of the query, already rotated
 * kv_cache, block_table, seq_lens as described above (read only)
 * softmax_scale: score scale (1/sqrt(192) for DeepSeek-V3's dims), finite > 0
 * num_splits S in [1, MLA_MAX_SPLITS]: partial slots per (sequence, query).
 *   S = 1: each sequence is attended whole, slot 0.
 *   S > 1 and B * Tq < 64: each sequence's ceil(L_b / block_size) blocks are
 *   cut into S contiguous ranges of ceil(blocks / S) blocks, range j in slot
 *   j (trailing ranges may be empty).
 *   S > 1 and B * Tq >= 64: the split is token-balanced over the batch,
 *   planned on the device from seq_lens: the sequences' blocks are laid end
 *   to end (each sequence charged 6 blocks more for its fixed per-split cost,
 *   unless all sequences have the same block count) and cut into equal
 *   chunks, as many as the device holds work-groups at once (XCDs x
 *   floor(compute units per XCD / Tq), at most B * S), but no shorter than
 *   ceil(longest / (S - 1))
 *   blocks, so that each sequence meets at most S chunks.  Sequence b's part
 *   of chunk u goes to slot u - (chunk of its first block); its slots past
 *   the last are empty.
 * part_o   fp32 [S, B, Tq, H, d_c]  written for non-empty slots: o_s,
 *          normalised within its slot; rows of empty slots are not written
 * part_lse fp32 [S, B, Tq, H]       written for every slot:
 *          ln sum_{t in slot} e^{s_t}, -inf for an empty slot
 * (both may be carved from one buffer of mla_decode_workspace_bytes bytes).
 * Errors: MLA_ERR_INVALID_ARG for NULL pointers, non-positive sizes, a
 * non-finite or non-positive scale, S out of range, B * Tq > 65536,
 * Tq > max_blocks_per_seq * block_size, a row of more than 2^31 - 1 tokens
 * or B * (max_blocks_per_seq + 6) > 2^31 - 1; MLA_ERR_UNSUPPORTED for other
 * dims.
 */
int mla_decode_paged(const uint16_t* q_lat, const uint16_t* q_r,
                     const uint16_t* kv_cache, const int32_t* block_table,
                     const int32_t* seq_lens,
                     int B, int Tq, int H, int d_c, int d_r,
                     int num_blocks, int block_size, int max_blocks_per_seq,
                     float softmax_scale, int num_splits,
                     float* part_o, float* part_lse, void* stream);

/*
 * Log-sum-exp merge of the splits, then the W_UV up-projection.  Source:
 * "DeepSeek-V3" (llm-vis explorer), box "Scaled dot-product attention" (the
 * online renormalisation across key blocks, applied here across splits) and
 * box "Output projection" (the value up-projection folds into the output
 * side); "Teardown: DeepSeek-V3", section 4 (v_C = W_UV c).
 * part_o, part_lse as written by mla_decode_paged for the same B, Tq and
 *         num_splits (read only; the part_o row of a slot whose lse is -inf
 *         is not read and may hold anything)
 * w_uv    bf16 [H, d_c, d_v], read only
 * out     bf16 [B, Tq, H, d_v]   written
 * lse_out fp32 [B, Tq, H] or NULL: ln sum over all splits (natural log)
 * A row whose splits are all empty gets out = 0 and lse = -inf.  Errors as
 * for mla_decode_paged (B * Tq > 65536 is MLA_ERR_INVALID_ARG).
 */
int mla_combine(const float* part_o, const float* part_lse, const uint16_t* w_uv,
                uint16_t* out, float* lse_out,
                int B, int Tq, int H, int d_c, int d_v, int num_splits, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one
 * mla_decode_paged followed by one mla_combine (same kernels, same results
 * bit for bit), with part_o and part_lse kept in a buffer the library owns
 * instead of caller workspace.  Allocates nothing: the buffer is a static
 * device array of MLA_NOALLOC_MAX_PAIRS (split, query row) pairs, 160 MiB +
 * 320 KiB, one per GPU the library runs on, held until the process ends; its
 * device address is looked up once per device on the first call there.
 * Arguments as for mla_decode_paged and mla_combine (out bf16 [B, Tq, H, d_v],
 * lse_out fp32 [B, Tq, H] or NULL).  Every call on one GPU shares that GPU's
 * buffer: calls that overlap on one GPU (different streams, or host threads
 * without ordering) race and must not be issued.  Errors as for those two
 * entry points, plus MLA_ERR_NOALLOC_LIMIT when num_splits * B * Tq exceeds
 * MLA_NOALLOC_MAX_PAIRS.
 */
int mla_decode_noalloc(const uint16_t* q_lat, const uint16_t* q_r,
                       const uint16_t* kv_cache, const int32_t* block_table,
                       const int32_t* seq_lens, const uint16_t* w_uv,
                       uint16_t* out, float* lse_out,
                       int B, int Tq, int H, int d_c, int d_r, int d_v,
                       int num_blocks, int block_size, int max_blocks_per_seq,
                       float softmax_scale, int num_splits, void* stream);

/*
 * Causal prefill in the un-absorbed form.  Source: "Teardown: DeepSeek-V3",
 * section 4 (k_C = W_UK c, v_C = W_UV c per head, keys [k_C; k_R] and queries
 * [q_C; q_R] of 192 values, scale 1/sqrt(192)); "DeepSeek-V3" (llm-vis
 * explorer), box "Scaled dot-product attention" (causal mask: position i sees
 * positions <= i).  Per head, keys (192 wide) and values (128 wide) are
 * rebuilt from the cache into `workspace`, then softmax(q k^T * scale) v runs
 * with the causal mask.
 * q_c  bf16 [B, T, H, d_h], q_r bf16 [B, T, H, d_r]: queries of the LAST T
 *      positions of each sequence (positions L_b - T .. L_b - 1), read only
 * kv_cache, block_table, seq_lens as described above (T <= L_b), read only
 * w_uk, w_uv as above; out bf16 [B, T, H, d_v] written
 * workspace: caller-owned device scratch of at least
 *      mla_prefill_workspace_bytes(B * max_blocks_per_seq * block_size, H, d_h, d_v)
 *      bytes, 256-byte aligned; its contents on entry do not matter.
 * Errors: MLA_ERR_INVALID_ARG for NULL pointers, non-positive sizes, a bad
 * scale, a misaligned or too small workspace or T > max_blocks_per_seq *
 * block_size; MLA_ERR_UNSUPPORTED for other dims.
 */
int mla_prefill(const uint16_t* q_c, const uint16_t* q_r,
                const uint16_t* kv_cache, const int32_t* block_table,
                const int32_t* seq_lens,
                const uint16_t* w_uk, const uint16_t* w_uv, uint16_t* out,
                void* workspace, size_t workspace_bytes,
                int B, int T, int H, int d_c, int d_r, int d_h, int d_v,
                int num_blocks, int block_size, int max_blocks_per_seq,
                float softmax_scale, void* stream);

/*
 * Cache append ("DeepSeek-V3" llm-vis explorer, boxes "KV latent compression"
 * and "Rotary position embedding (RoPE)"): for each of M new tokens m, with
 * hidden state x[m], sequence seq_idx[m] and position positions[m],
 *   [c_raw | k_raw] = w_kv x[m]                      (d_model -> d_c + d_r)
 *   c   = c_raw / sqrt(mean(c_raw^2) + eps) * gamma   (RMSNorm over d_c)
 *   k_R = (k_raw[2i], k_raw[2i+1]) rotated by positions[m] * theta^(-2i/d_r)
 * is written as the cache row c | k_R of that token: block
 * block_table[seq_idx[m], positions[m] / block_size], row
 * positions[m] % block_size.  Only those M rows are written.
 * x       bf16 [M, d_model]
 * w_kv    bf16 [d_c + d_r, d_model]   (a linear layer's [out, in] weight)
 * gamma   bf16 [d_c]                  RMSNorm gain
 * seq_idx, positions  int32 [M]      device arrays, not validated (a sync):
 *         0 <= seq_idx < (rows of block_table), 0 <= positions <
 *         max_blocks_per_seq * block_size, the block named for the position
 *         in range; two tokens of one call must not share a cache row.
 * kv_cache  as described above; rows written in bf16, rounded to nearest even
 * workspace fp32, at least mla_cache_append_workspace_bytes(M, d_model) bytes,
 *         256-byte aligned: the K-sliced partial products.
 * Supported: d_c = 512, d_r = 64, block_size = 64, d_model a multiple of 16
 * (7168 in DeepSeek-V3).  theta > 0 (10000 in DeepSeek-V3), eps >= 0.
 */
int mla_cache_append(const uint16_t* x, const uint16_t* w_kv, const uint16_t* gamma,
                     const int32_t* seq_idx, const int32_t* positions,
                     const int32_t* block_table, uint16_t* kv_cache,
                     void* workspace, size_t workspace_bytes,
                     int M, int d_model, int d_c, int d_r, int num_blocks, int block_size,
                     int max_blocks_per_seq, float eps, float rope_theta, void* stream);

/* Workspace bytes mla_cache_append needs for M tokens (0 on invalid args). */
size_t mla_cache_append_workspace_bytes(int M, int d_model);

/*
 * Query side ("DeepSeek-V3" llm-vis explorer, "Query low-rank projection";
 * "Teardown: DeepSeek-V3", section 4, c_q = W_DQ h, q_C = W_UQ c_q): for each
 * of M tokens with hidden state x[m] at position positions[m],
 *   c_q = w_dq x[m]  (d_model -> q_rank), c_q' = RMSNorm(c_q) * gamma_q,
 *   per head h: [q_C | q_R'] = (w_uq c_q')[192h .. 192h + 191]  (d_h | d_r),
 *   q_R = q_R' with pairs (2i, 2i+1) rotated by positions[m] * theta^(-2i/d_r).
 * x bf16 [M, d_model]; w_dq bf16 [q_rank, d_model]; gamma_q bf16 [q_rank];
 * w_uq bf16 [H * (d_h + d_r), q_rank]; positions int32 [M] (device, >= 0);
 * q_c bf16 [M, H, d_h] and q_r bf16 [M, H, d_r] out (the inputs of
 * mla_absorb_q and mla_decode_paged).  RMSNorm's per-row factor is applied
 * after the second product (it commutes with it): gamma_q * c_q is rounded to
 * bf16 between the two products and the fp32 result of the second is scaled
 * by 1 / sqrt(mean(c_q^2) + eps).  workspace: mla_query_project_workspace_bytes(M, d_model,
 * q_rank) bytes, 256-byte aligned.
 * Supported: H = 128, d_h = 128, d_r = 64, d_model a multiple of 16, q_rank a
 * multiple of 256 up to 4096 (7168 and 1536 in DeepSeek-V3).
 */
int mla_query_project(const uint16_t* x, const uint16_t* w_dq, const uint16_t* gamma_q,
                      const uint16_t* w_uq, const int32_t* positions,
                      uint16_t* q_c, uint16_t* q_r, void* workspace, size_t workspace_bytes,
                      int M, int d_model, int q_rank, int H, int d_h, int d_r,
                      float eps, float rope_theta, void* stream);
size_t mla_query_project_workspace_bytes(int M, int d_model, int q_rank);

/*
 * Output projection ("DeepSeek-V3" llm-vis explorer, "Output projection": the
 * concatenated value heads mapped back to the residual stream, no bias):
 *   y[m] = w_o o[m]
 * o bf16 [M, d_in] (mla_combine's out viewed as [M, H * d_v]); w_o bf16
 * [d_out, d_in]; y bf16 [M, d_out] out, 8-byte aligned.  workspace:
 * mla_output_project_workspace_bytes(M, d_in, d_out) bytes, 256-byte aligned.
 * Supported: d_in a multiple of 16, d_out a multiple of 64 (16384 -> 7168 in
 * DeepSeek-V3).
 */
int mla_output_project(const uint16_t* o, const uint16_t* w_o, uint16_t* y,
                       void* workspace, size_t workspace_bytes,
                       int M, int d_in, int d_out, void* stream);
size_t mla_output_project_workspace_bytes(int M, int d_in, int d_out);

/*
 * Workspace of one decode step: part_o then part_lse in one buffer, part_lse
 * starting at mla_decode_part_o_bytes(...) rounded up to 256 bytes.  Returns
 * the total (0 on non-positive arguments).
 */
size_t mla_decode_workspace_bytes(int B, int Tq, int H, int d_c, int num_splits);
/* Bytes of part_o and of part_lse alone (0 on non-positive arguments). */
size_t mla_decode_part_o_bytes(int B, int Tq, int H, int d_c, int num_splits);
size_t mla_decode_part_lse_bytes(int B, int Tq, int H, int num_splits);

/*
 * Workspace bytes mla_prefill needs: rebuilt bf16 content keys and values of
 * every cache slot the block table can address, total_kv_tokens =
 * B * max_blocks_per_seq * block_size (0 on non-positive arguments).
 */
size_t mla_prefill_workspace_bytes(long total_kv_tokens, int H, int d_h, int d_v);

/*
 * Suggested num_splits (partial slots) for a decode step.  With at least
 * four rounds of work-groups in whole sequences (B * Tq >= 4 num_cus), or
 * sequences of one block, it is 1.
 * Otherwise, with c = ceil(num_cus / (B * Tq)) splits per sequence (capped
 * at the longest sequence's block count) filling the compute units about
 * once: c for B * Tq < 64 (equal ranges per sequence); from B * Tq = 64 on
 * (token-balanced chunks), 2c + 1 (room for sequences up to twice the mean
 * length, plus a chunk that straddles two sequences) where that is at most
 * 40, the slots the combine reads in one round trip, else c + 1; at most
 * MLA_MAX_SPLITS.  Host-only arithmetic; returns 0 on invalid arguments.
 */
int mla_decode_num_splits(int B, int Tq, int H, int max_seq_len, int block_size,
                          int num_cus);

/*
 * Measurement utility, not part of the attention path: reads `bytes` of
 * device memory at `buf` once, grid-stride with 16-byte loads from every
 * compute unit, and folds them into one word that is written to `*sink`
 * (device memory, 4 bytes) only if it equals a magic value, so the reads
 * cannot be elided.  Timed around a cold call, it gives the HBM read rate
 * this part delivers to a plain read, which the decode kernel's rate is
 * reported against beside the published peak.  `buf` must be 16-byte
 * aligned and `bytes` a positive multiple of 16: MLA_ERR_INVALID_ARG
 * otherwise.
 */
int mla_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * Measurement utility, not part of the attention path: mla_decode_paged
 * (same kernel, same arguments and results) that also ADDS to clock_sums
 * (device uint64[2], 8-byte aligned, not cleared by the call) the sum over
 * its work-groups of shader-clock cycles (clock_sums[0]) and of 100 MHz
 * real-time ticks (clock_sums[1]) from each work-group's start to its end.
 * 0.1 GHz * clock_sums[0] / clock_sums[1] is the average shader clock the
 * kernel ran at; the bench sets its matrix-unit floor against it.  NULL or a
 * misaligned clock_sums returns MLA_ERR_INVALID_ARG; otherwise as
 * mla_decode_paged.
 */
int mla_decode_paged_clocked(const uint16_t* q_lat, const uint16_t* q_r,
                             const uint16_t* kv_cache, const int32_t* block_table,
                             const int32_t* seq_lens,
                             int B, int Tq, int H, int d_c, int d_r,
                             int num_blocks, int block_size, int max_blocks_per_seq,
                             float softmax_scale, int num_splits,
                             float* part_o, float* part_lse, uint64_t* clock_sums, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
