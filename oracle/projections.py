"""Plain fp64 reference for the projections around the latent attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the product path.

Sources, by page title:

* "Teardown: DeepSeek-V3", section 4: c_q = W_DQ h and q_C = W_UQ c_q, with
  W_DQ 7168 -> 1536 and W_UQ 1536 -> 128 x (128 + 64) (the 64 per head being
  the rotary query); W_O 128 x 128 -> 7168.
* "DeepSeek-V3" (ainfra.dev llm-vis explorer), "Query low-rank projection":
  q = q_up(q_norm(q_down(x))) with q_norm = RMSNorm(1536); "Rotary position
  embedding (RoPE)": the rotation of consecutive pairs; "Output projection":
  the 128 value heads concatenated and mapped to 7168 with no bias.

Readings where the pages are silent: the per-head 192 outputs of W_UQ are the
content part (128) then the rotary part (64), the order of [q_C; q_R];
RMSNorm and RoPE as in ``oracle.cache_append`` (the explorer's RMSNorm box
with eps = 1e-6, no YaRN remap, exact angles).

All arithmetic is float64 on the exact values handed in.  Nothing here rounds.
"""

import numpy as np

from .cache_append import RMS_EPS, ROPE_THETA, apply_rope, rms_norm


def query_project(x, w_dq, gamma_q, w_uq, positions, eps=RMS_EPS, theta=ROPE_THETA, n_heads=128,
                  d_h=128, d_r=64):
    """(q_c [M, H, d_h], q_r [M, H, d_r]) of M tokens: c_q = W_DQ x, RMSNorm with
    gain gamma_q, q = W_UQ c_q split per head into [q_C; q_R'], q_R' rotated at
    the token's position."""
    c_q = np.asarray(x, dtype=np.float64) @ np.asarray(w_dq, dtype=np.float64).T
    c_q = rms_norm(c_q, gamma_q, eps)
    q = (c_q @ np.asarray(w_uq, dtype=np.float64).T).reshape(len(c_q), n_heads, d_h + d_r)
    q_c = q[..., :d_h]
    q_r = apply_rope(q[..., d_h:], np.asarray(positions)[:, None], theta)
    return q_c, q_r


def output_project(o, w_o):
    """y [M, d_out] = o [M, d_in] W_O^T (w_o is a linear layer's [d_out, d_in] weight)."""
    return np.asarray(o, dtype=np.float64) @ np.asarray(w_o, dtype=np.float64).T
