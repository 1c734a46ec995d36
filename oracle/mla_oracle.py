"""Plain fp64 reference for multi-head latent attention (MLA) over the latent cache.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the product path.

Notation follows "Teardown: DeepSeek-V3", section 4 "Multi-head latent
attention": per token the cache holds the content latent c (d_c = 512 values)
and the shared rotary key k_R (d_r = 64 values); per head h the content key is
k_C = W_UK[h] c (d_h = 128 values) and the value is v_C = W_UV c (d_v = 128
values); each head's query and key are [q_C; q_R] and [k_C; k_R] and the score
is their dot product times 1/sqrt(d_h + d_r).

Index reading of the weights (the pages write the products as matrix times
vector and give the weight table only as "512 -> 128 x (128 + 128)"):

* ``w_uk`` has shape [H, d_h, d_c]; w_uk[h, i, j] multiplies c[j] into
  k_C[i], i.e. w_uk[h] is the matrix W_UK of head h as written.
* ``w_uv`` has shape [H, d_c, d_v]; w_uv[h, j, d] multiplies c[j] into v[d],
  i.e. w_uv[h] stores head h's W_UV transposed (latent index first).

Cache layout: ``kv_cache`` is [num_blocks, block_size, d_c + d_r]; a row is
c followed by k_R, the split([512, 64]) order of the "KV latent compression"
box of "DeepSeek-V3" (llm-vis explorer).  ``block_table[b, p]`` is the physical
block holding tokens [p * block_size, (p + 1) * block_size) of sequence b.

Causality ("Scaled dot-product attention" box: position i sees <= i): a
sequence with ``seq_len`` L cached tokens, L counting the Tq query tokens
themselves (the new token is appended before attention, as in the MLA box's
forward), has its query i at position L - Tq + i; that query sees tokens
0 .. L - Tq + i.

All arithmetic is float64 on the exact values handed in.  Nothing here rounds.
"""

import numpy as np

# Heads processed per numpy matmul in the un-absorbed form (memory bound only).
_HEAD_CHUNK = 16


def gather_rows(kv_cache, table_row, n_tokens):
    """Rows 0 .. n_tokens-1 of one sequence, read through its block table.

    Returns a float64 array [n_tokens, d_c + d_r]: logical token t lives in
    block table_row[t // block_size], row t % block_size.
    """
    block_size = kv_cache.shape[1]
    t = np.arange(n_tokens)
    blocks = np.asarray(table_row)[t // block_size]
    if n_tokens and (blocks.min() < 0 or blocks.max() >= kv_cache.shape[0]):
        raise ValueError("block table entry out of range for a used page")
    return np.asarray(kv_cache[blocks, t % block_size], dtype=np.float64)


def _visible(seq_len, tq):
    """Number of keys visible to each of the tq queries (causal, see module doc)."""
    if not tq <= seq_len:
        raise ValueError("seq_len must count the query tokens (tq <= seq_len)")
    return [seq_len - tq + i + 1 for i in range(tq)]


def _softmax_and_lse(s):
    """Explicit softmax of a score vector and the natural log of sum(exp(s))."""
    m = s.max()
    e = np.exp(s - m)
    total = e.sum()
    return e / total, m + np.log(total)


def attend_unabsorbed(q_c, q_r, c, k_r, w_uk, w_uv, scale, n_visible):
    """MLA attention in the form the pages write it, keys and values materialised.

    q_c [Tq, Hs, d_h], q_r [Tq, Hs, d_r]: the queries of Hs heads.
    c [L, d_c], k_r [L, d_r]: the sequence's cached latent and rotary key.
    w_uk [Hs, d_h, d_c], w_uv [Hs, d_c, d_v]: the same Hs heads' weights.
    n_visible: per query, how many leading tokens it attends to.

    Per head: k_C,t = W_UK c_t and v_t = W_UV c_t for every token (section 4
    equations of "Teardown: DeepSeek-V3"), k_t = [k_C,t; k_R,t] with k_R shared
    by all heads, q = [q_C; q_R], s_t = (q . k_t) * scale over the visible
    tokens, p = softmax(s), out = sum_t p_t v_t ("Scaled dot-product
    attention" box of the llm-vis explorer).

    Returns (out [Tq, Hs, d_v], lse [Tq, Hs]) with lse = ln sum_t exp(s_t).
    """
    tq, hs, _ = q_c.shape
    d_v = w_uv.shape[2]
    out = np.zeros((tq, hs, d_v))
    lse = np.zeros((tq, hs))
    for h0 in range(0, hs, _HEAD_CHUNK):
        h1 = min(hs, h0 + _HEAD_CHUNK)
        # k_C[h, t, i] = sum_j W_UK[h, i, j] c[t, j]
        k_c = np.matmul(c[None, :, :], np.transpose(w_uk[h0:h1], (0, 2, 1)))
        # v[h, t, d] = sum_j c[t, j] W_UV[h, j, d]
        v = np.matmul(c[None, :, :], w_uv[h0:h1])
        for h in range(h0, h1):
            k = np.concatenate([k_c[h - h0], k_r], axis=1)  # [L, d_h + d_r]
            for i in range(tq):
                n = n_visible[i]
                q = np.concatenate([q_c[i, h], q_r[i, h]])
                s = (k[:n] @ q) * scale
                p, lse[i, h] = _softmax_and_lse(s)
                out[i, h] = p @ v[h - h0, :n]
    return out, lse


def absorb_q(q_c, w_uk):
    """Fold W_UK into the query: q_lat[..., h, j] = sum_i q_c[..., h, i] w_uk[h, i, j].

    This is (W_UK^T q_C), the left side of q^T (W_uk c) = (W_uk^T q)^T c in the
    "KV latent compression" box; shape [..., H, d_c].
    """
    return np.einsum("...hi,hij->...hj", q_c, w_uk)


def up_project(o_lat, w_uv):
    """Apply W_UV after attention: out[..., h, d] = sum_j o_lat[..., h, j] w_uv[h, j, d].

    With o_lat = sum_t p_t c_t this equals sum_t p_t (W_UV c_t), the value
    side of the absorbed form ("Output projection" box: the value
    up-projection folds into the output side).
    """
    return np.einsum("...hj,hjd->...hd", o_lat, w_uv)


def attend_absorbed(q_c, q_r, c, k_r, w_uk, w_uv, scale, n_visible):
    """The same attention computed in latent space (the absorbed form).

    q_lat = W_UK^T q_C; s_t = (q_lat . c_t + q_R . k_R,t) * scale;
    o_lat = sum_t p_t c_t; out = o_lat W_UV.  Same arguments and returns as
    ``attend_unabsorbed``; kept as separate code so that the two can be
    compared.
    """
    tq, hs, _ = q_c.shape
    q_lat = absorb_q(q_c, w_uk)  # [Tq, Hs, d_c]
    scores = (np.einsum("ihj,tj->iht", q_lat, c)
              + np.einsum("ihr,tr->iht", q_r, k_r)) * scale
    o_lat = np.zeros((tq, hs, c.shape[1]))
    lse = np.zeros((tq, hs))
    for i in range(tq):
        n = n_visible[i]
        s = scores[i, :, :n]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        o_lat[i] = (e / z) @ c[:n]
        lse[i] = (m + np.log(z))[:, 0]
    return up_project(o_lat, w_uv), lse


def split_partial(q_lat, q_r, c, k_r, scale, t_begin, t_end, n_visible):
    """Attention restricted to tokens [t_begin, t_end), in latent space.

    For each query row: the keys it may see inside the range, s_t as in the
    absorbed form, and returns (o_s [Tq, Hs, d_c], lse_s [Tq, Hs]) with
    o_s = sum p_t c_t normalised within the range and lse_s = ln sum exp(s_t).
    A row that sees no key in the range gets o_s = 0 and lse_s = -inf.
    """
    tq, hs, d_c = q_lat.shape
    o = np.zeros((tq, hs, d_c))
    lse = np.full((tq, hs), -np.inf)
    for i in range(tq):
        hi = min(t_end, n_visible[i])
        if hi <= t_begin:
            continue
        cc = c[t_begin:hi]
        s = (q_lat[i] @ cc.T + q_r[i] @ k_r[t_begin:hi].T) * scale  # [Hs, n]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        o[i] = (e / z) @ cc
        lse[i] = (m + np.log(z))[:, 0]
    return o, lse


def combine_partials(part_o, part_lse, w_uv=None):
    """Merge per-split results by their log-sum-exp, then optionally apply W_UV.

    part_o [S, ..., H, d_c] (each split's normalised latent output) and
    part_lse [S, ..., H] (each split's ln sum exp of its scores).
    lse = ln sum_s exp(lse_s); o_lat = sum_s exp(lse_s - lse) o_s.  This is the
    online renormalisation of the "Scaled dot-product attention" box done once
    across splits.  Splits with lse_s = -inf carry no weight; a row whose
    splits are all empty gets o_lat = 0 and lse = -inf.

    Returns (out, lse): out is up_project(o_lat, w_uv) when w_uv is given,
    else o_lat.
    """
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    m = part_lse.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(part_lse), np.exp(part_lse - m_safe), 0.0)
    z = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, z, 1.0)), -np.inf)
    wn = np.where(finite, w / np.where(finite, z, 1.0), 0.0)
    o_lat = np.einsum("s...,s...j->...j", wn, np.where(wn[..., None] > 0, part_o, 0.0))
    if w_uv is None:
        return o_lat, lse
    return up_project(o_lat, w_uv), lse


def decode(q_c, q_r, kv_cache, block_table, seq_lens, w_uk, w_uv, scale,
           batches=None, heads=None, form="unabsorbed"):
    """Paged MLA decode over the latent cache.

    q_c [B, Tq, H, d_h], q_r [B, Tq, H, d_r] (q_R already rotated),
    kv_cache [num_blocks, block_size, d_c + d_r], block_table [B, max_blocks],
    seq_lens [B] (counting the Tq query tokens), w_uk [H, d_h, d_c],
    w_uv [H, d_c, d_v].  ``batches`` / ``heads`` select a subset of sequences
    and heads (default all).  ``form`` is "unabsorbed" (the definition) or
    "absorbed".

    Returns (out [nb, Tq, nh, d_v], lse [nb, Tq, nh]) in float64.
    """
    n_seq, tq, n_heads, _ = q_c.shape
    d_c = w_uk.shape[2]
    batches = list(range(n_seq)) if batches is None else list(batches)
    heads = list(range(n_heads)) if heads is None else list(heads)
    attend = {"unabsorbed": attend_unabsorbed, "absorbed": attend_absorbed}[form]
    out = np.zeros((len(batches), tq, len(heads), w_uv.shape[2]))
    lse = np.zeros((len(batches), tq, len(heads)))
    for k, b in enumerate(batches):
        seq_len = int(seq_lens[b])
        rows = gather_rows(kv_cache, block_table[b], seq_len)
        c, k_r = rows[:, :d_c], rows[:, d_c:]
        out[k], lse[k] = attend(
            np.asarray(q_c[b][:, heads], dtype=np.float64),
            np.asarray(q_r[b][:, heads], dtype=np.float64),
            c, k_r,
            np.asarray(w_uk[heads], dtype=np.float64),
            np.asarray(w_uv[heads], dtype=np.float64),
            scale, _visible(seq_len, tq))
    return out, lse


def prefill(q_c, q_r, kv_cache, block_table, seq_lens, w_uk, w_uv, scale,
            batches=None, heads=None, form="unabsorbed"):
    """Causal prefill: T query tokens per sequence, the last T positions.

    q_c [B, T, H, d_h] holds the queries of positions L - T .. L - 1 of each
    sequence (L = seq_lens[b]); query i sees tokens 0 .. L - T + i.  With
    T == L this is ordinary causal self-attention over the whole sequence.
    The computation is exactly that of ``decode`` with Tq = T.
    """
    return decode(q_c, q_r, kv_cache, block_table, seq_lens, w_uk, w_uv, scale,
                  batches=batches, heads=heads, form=form)
