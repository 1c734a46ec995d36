"""Plain fp64 reference for appending new tokens to the latent KV cache.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the product path.

Sources, by page title:

* "DeepSeek-V3" (ainfra.dev llm-vis explorer), box "KV latent compression":
  the down-projection kv_down maps each token's hidden state (d_model = 7168)
  to 512 + 64 values, split([512, 64]); the 512-wide latent goes through
  kv_norm = RMSNorm(512) and the 64-wide part through RoPE at the token's
  position; the pair (latent, rotated key) is what the cache holds.
* Same page, box "Rotary position embedding (RoPE)": inverse frequencies
  1 / theta^(2i / d) for i = 0 .. d/2 - 1 with theta = 10000, and consecutive
  pairs (x[2i], x[2i+1]) rotated by the angle pos * inv_freq[i].
* "Teardown: DeepSeek-V3", section 4: only c and k_R are cached.

Readings where the pages are silent:

* Same page, box "RMSNorm": y = x / sqrt(mean(x^2) + eps) * g with a learned
  per-feature gain g and eps = 0.000001, the reduction done in fp32 in bf16
  models.  The box describes the 7168-wide norms; kv_norm = RMSNorm(512) is
  the same module over the 512 latent values, so the same formula and eps
  apply.  Here the reduction is exact (float64), eps defaults to the printed
  value and stays an argument.
* The pages mention a YaRN x40 frequency remap without defining it; it is
  not applied here (plain RoPE as printed).
* Angles are computed exactly (float64) rather than in the framework's
  default float32 of the printed snippet.

All arithmetic is float64 on the exact values handed in.  Nothing here rounds.
"""

import numpy as np

# eps of the explorer's "RMSNorm" box (printed as 0.000001).
RMS_EPS = 1e-6
# theta of the explorer's "Rotary position embedding (RoPE)" box.
ROPE_THETA = 10000.0


def kv_down(x, w_kv):
    """[M, d_model] x [d_c + d_r, d_model] (a linear layer's weight) -> [M, d_c + d_r]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_kv, dtype=np.float64).T


def rms_norm(c, gamma, eps=RMS_EPS):
    """RMSNorm over the last axis: c / sqrt(mean(c^2) + eps) * gamma ("RMSNorm" box)."""
    c = np.asarray(c, dtype=np.float64)
    rms = np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps)
    return c / rms * np.asarray(gamma, dtype=np.float64)


def rope_inv_freq(d_r, theta=ROPE_THETA):
    """1 / theta^(2i / d_r) for i = 0 .. d_r/2 - 1."""
    return 1.0 / (float(theta) ** (np.arange(0, d_r, 2, dtype=np.float64) / d_r))


def apply_rope(k, pos, theta=ROPE_THETA):
    """Rotate consecutive pairs of the last axis of k ([..., d_r]) by pos * inv_freq.

    ``pos`` broadcasts against the leading axes of k.
    """
    k = np.asarray(k, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(k.shape[-1], theta)
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = k[..., 0::2], k[..., 1::2]
    out = np.empty_like(k)
    out[..., 0::2] = x1 * cos - x2 * sin
    out[..., 1::2] = x1 * sin + x2 * cos
    return out


def cache_rows(x, w_kv, gamma, positions, eps=RMS_EPS, theta=ROPE_THETA, d_c=512):
    """The cache rows [M, d_c + d_r] of M new tokens: RMSNorm(latent) | RoPE(key)."""
    y = kv_down(x, w_kv)
    c = rms_norm(y[:, :d_c], gamma, eps)
    k_r = apply_rope(y[:, d_c:], positions, theta)
    return np.concatenate([c, k_r], axis=1)


def cache_append(x, w_kv, gamma, seq_idx, positions, block_table, kv_cache, eps=RMS_EPS,
                 theta=ROPE_THETA, d_c=512):
    """Write the rows of M new tokens into a copy of the paged cache.

    Token m belongs to sequence seq_idx[m] at position positions[m]; its row
    goes to block block_table[seq_idx[m], positions[m] // block_size], row
    positions[m] % block_size.  Returns (new cache as float64, rows [M, 576]).
    """
    rows = cache_rows(x, w_kv, gamma, positions, eps, theta, d_c)
    out = np.array(kv_cache, dtype=np.float64, copy=True)
    block_size = out.shape[1]
    for m, (b, p) in enumerate(zip(np.asarray(seq_idx), np.asarray(positions))):
        blk = int(block_table[int(b), int(p) // block_size])
        if not 0 <= blk < out.shape[0]:
            raise ValueError("block table entry out of range for an appended token")
        out[blk, int(p) % block_size] = rows[m]
    return out, rows
