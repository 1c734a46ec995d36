"""fp64 CPU oracle for multi-head latent attention over the latent KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product path (the
HIP library and its Python binding) never imports it, and this package imports
nothing from the product path.

Every function here works on float64 numpy arrays holding the exact values of
the (bf16) inputs and does no rounding of its own.  Sources, by page title:

* "Teardown: DeepSeek-V3", section 4 "Multi-head latent attention": the
  equations c = W_DKV h, k_C = W_UK c, v_C = W_UV c, q = [q_C; q_R],
  k = [k_C; k_R], score scale 1/sqrt(128 + 64), only c and k_R cached; the
  table of attention weight shapes; the remark that the key up-projection
  folds into the query.
* "DeepSeek-V3" (ainfra.dev llm-vis explorer), boxes "Multi-Head Latent
  Attention (MLA)" and "KV latent compression" (the cache row is
  split([512, 64]) = latent then rope key; the absorption identity
  q^T (W_uk c) = (W_uk^T q)^T c) and "Scaled dot-product attention"
  (softmax(q k^T / sqrt(d)) v, causal mask "position i sees <= i", online
  renormalisation gives the same result).

Pin status (what fixes each function other than itself):

* ``attend_unabsorbed`` -- hand case with closed-form values, SDPA library
  cross-check, special cases (one token, zero query, a dominant score),
  permutation invariance.
* ``attend_absorbed`` -- equal to ``attend_unabsorbed`` to 1e-12 (absorption
  identity), plus the same hand case.
* ``absorb_q`` -- q_lat . c == q_C . (W_UK c) on random inputs.
* ``up_project`` -- (sum_t p_t c_t) W_UV == sum_t p_t (W_UV^T c_t).
* ``combine_partials`` -- combining attention over a partition of the keys
  reproduces attention over all keys (online renormalisation), and the
  all-empty convention.
* ``split_partial`` -- the same partition property.

Cache append (``oracle.cache_append``): kv_down, RMSNorm, RoPE and the paged
write of new tokens ("DeepSeek-V3" llm-vis explorer, boxes "KV latent
compression" and "Rotary position embedding (RoPE)").  Pins: RoPE hand cases
with closed forms, the inverse frequencies, position 0, pair norms, relative
position and composition identities; RMSNorm hand cases, scale invariance and
unit RMS; kv_down against brute force and coordinate-selecting weights; the
split order and the page placement worked out by hand.

Projections (``oracle.projections``): the query side (W_DQ, RMSNorm, W_UQ,
per-head split, RoPE of the rotary query) and the output projection W_O
("Teardown: DeepSeek-V3" section 4; explorer "Query low-rank projection" and
"Output projection").  Pins: a hand case through every step with closed-form
values, position independence of q_C, position 0 leaving q_R unrotated, the
per-head split order, brute force for W_O on tiny inputs.

No function is "parity unpinned".
"""

from . import cache_append, projections  # noqa: F401
from .mla_oracle import (  # noqa: F401
    absorb_q,
    attend_absorbed,
    attend_unabsorbed,
    combine_partials,
    decode,
    gather_rows,
    prefill,
    split_partial,
    up_project,
)
