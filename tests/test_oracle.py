"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these tests compares the oracle with itself: each checks it against a
closed form derived by hand, a library routine, an identity the pages state, a
special case with a known answer, or a printed number.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Hand case: 2 heads, latent of 2, content head dim 1, rotary dim 1, 3 tokens.
#   c   = [[1,0],[0,1],[1,1]],  k_R = [0, 0, -1]
#   W_UK[0] = [[1,0]], W_UK[1] = [[0,1]]   (d_h x d_c)
#   W_UV[0] = [[2],[3]], W_UV[1] = [[1],[-1]]   (d_c x d_v, latent index first)
#   q_C = [[1],[2]], q_R = [[0],[1]]
# Head 0: k_C = (1,0,1), v = (2,3,5), scores (1,0,1)        -> (7e+3)/(2e+1)
# Head 1: k_C = (0,1,1), v = (1,-1,0), scores 2*(0,1,1)+(0,0,-1) = (0,2,1)
#                                                          -> (1-e^2)/(1+e+e^2)
# ---------------------------------------------------------------------------

def _hand(tq=1, scale=1.0):
    c = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    k_r = np.array([[0.0], [0.0], [-1.0]])
    kv = np.concatenate([c, k_r], axis=1)[None]          # one block of 3 rows
    w_uk = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])        # [2, 1, 2]
    w_uv = np.array([[[2.0], [3.0]], [[1.0], [-1.0]]])   # [2, 2, 1]
    q_c1 = np.array([[1.0], [2.0]])
    q_r1 = np.array([[0.0], [1.0]])
    q_c = np.stack([q_c1] * tq)[None]                    # [1, tq, 2, 1]
    q_r = np.stack([q_r1] * tq)[None]
    table = np.array([[0]], dtype=np.int32)
    lens = np.array([3], dtype=np.int32)
    return q_c, q_r, kv, table, lens, w_uk, w_uv, scale


E = math.e


@pytest.mark.parametrize("form", ["unabsorbed", "absorbed"])
def test_hand_case_single_query(form):
    out, lse = oracle.decode(*_hand(), form=form)
    assert out.shape == (1, 1, 2, 1)
    assert out[0, 0, 0, 0] == pytest.approx((7 * E + 3) / (2 * E + 1), rel=1e-14)
    assert out[0, 0, 1, 0] == pytest.approx((1 - E**2) / (1 + E + E**2), rel=1e-14)
    assert lse[0, 0, 0] == pytest.approx(math.log(2 * E + 1), rel=1e-14)
    assert lse[0, 0, 1] == pytest.approx(math.log(1 + E + E**2), rel=1e-14)
    assert out[0, 0, 0, 0] == pytest.approx(3.4223187982515184, rel=1e-14)
    assert out[0, 0, 1, 0] == pytest.approx(-0.5752103826044414, rel=1e-14)


@pytest.mark.parametrize("form", ["unabsorbed", "absorbed"])
def test_hand_case_two_queries_causal(form):
    # Query 0 sits at position L-2 = 1 and sees tokens 0 and 1 only.
    out, _ = oracle.decode(*_hand(tq=2), form=form)
    assert out[0, 0, 0, 0] == pytest.approx((2 * E + 3) / (E + 1), rel=1e-14)
    assert out[0, 0, 1, 0] == pytest.approx(-math.tanh(1.0), rel=1e-14)
    # Query 1 sees all three tokens: same as the single-query case.
    assert out[0, 1, 0, 0] == pytest.approx((7 * E + 3) / (2 * E + 1), rel=1e-14)
    assert out[0, 1, 1, 0] == pytest.approx((1 - E**2) / (1 + E + E**2), rel=1e-14)


@pytest.mark.parametrize("form", ["unabsorbed", "absorbed"])
def test_hand_case_three_queries_causal(form):
    # Tq = L = 3 (a token and two drafts): query i sits at position i.
    out, lse = oracle.decode(*_hand(tq=3), form=form)
    # Query 0 sees token 0 alone: its value, v = 2 (head 0) and 1 (head 1), lse = its score.
    assert out[0, 0, 0, 0] == pytest.approx(2.0, rel=1e-15)
    assert out[0, 0, 1, 0] == pytest.approx(1.0, rel=1e-15)
    assert lse[0, 0, 0] == pytest.approx(1.0, rel=1e-15)
    assert lse[0, 0, 1] == pytest.approx(0.0, abs=1e-15)
    # Query 1 sees tokens 0 and 1, query 2 all three.
    assert out[0, 1, 0, 0] == pytest.approx((2 * E + 3) / (E + 1), rel=1e-14)
    assert out[0, 1, 1, 0] == pytest.approx(-math.tanh(1.0), rel=1e-14)
    assert out[0, 2, 0, 0] == pytest.approx((7 * E + 3) / (2 * E + 1), rel=1e-14)
    assert out[0, 2, 1, 0] == pytest.approx((1 - E**2) / (1 + E + E**2), rel=1e-14)


@pytest.mark.parametrize("form", ["unabsorbed", "absorbed"])
def test_hand_case_scaled(form):
    x = math.exp(1 / math.sqrt(2))
    out, _ = oracle.decode(*_hand(scale=1 / math.sqrt(2)), form=form)
    assert out[0, 0, 0, 0] == pytest.approx((7 * x + 3) / (2 * x + 1), rel=1e-14)
    assert out[0, 0, 1, 0] == pytest.approx((1 - x * x) / (1 + x + x * x), rel=1e-14)


# ---------------------------------------------------------------------------
# Random inputs with the real per-head dims but few heads.
# ---------------------------------------------------------------------------

def _random_case(rng, n_seq=3, tq=1, heads=3, d_c=512, d_r=64, d_h=128, d_v=128,
                 block_size=16, lens=(1, 37, 50), spare=3, w_std=512 ** -0.5):
    lens = np.array(lens[:n_seq], dtype=np.int32)
    pages = [(int(n) + block_size - 1) // block_size for n in lens]
    num_blocks = sum(pages) + spare
    perm = rng.permutation(num_blocks)
    table = np.full((n_seq, max(pages)), -1, dtype=np.int32)
    kv = np.full((num_blocks, block_size, d_c + d_r), np.nan)
    start = 0
    for b, p in enumerate(pages):
        table[b, :p] = perm[start:start + p]
        start += p
        rows = rng.standard_normal((int(lens[b]), d_c + d_r))
        for t in range(int(lens[b])):
            kv[table[b, t // block_size], t % block_size] = rows[t]
    q_c = rng.standard_normal((n_seq, tq, heads, d_h))
    q_r = rng.standard_normal((n_seq, tq, heads, d_r))
    w_uk = rng.standard_normal((heads, d_h, d_c)) * w_std
    w_uv = rng.standard_normal((heads, d_c, d_v)) * w_std
    return q_c, q_r, kv, table, lens, w_uk, w_uv, 1 / math.sqrt(d_h + d_r)


@pytest.mark.parametrize("tq,lens", [(1, (1, 37, 50)), (2, (2, 33, 64)), (5, (5, 17, 40))])
def test_absorbed_equals_unabsorbed(tq, lens):
    """Absorption identity q^T (W_uk c) = (W_uk^T q)^T c, end to end, to 1e-12."""
    rng = np.random.default_rng(11 + tq)
    args = _random_case(rng, tq=tq, lens=lens)
    out_u, lse_u = oracle.decode(*args, form="unabsorbed")
    out_a, lse_a = oracle.decode(*args, form="absorbed")
    rel = np.linalg.norm(out_a - out_u) / np.linalg.norm(out_u)
    assert rel <= 1e-12
    np.testing.assert_allclose(lse_a, lse_u, rtol=1e-12, atol=0)


def test_absorbed_equals_unabsorbed_medium():
    rng = np.random.default_rng(5)
    args = _random_case(rng, n_seq=2, heads=16, lens=(300, 513), block_size=64)
    out_u, _ = oracle.decode(*args, form="unabsorbed")
    out_a, _ = oracle.decode(*args, form="absorbed")
    assert np.max(np.abs(out_a - out_u)) / np.max(np.abs(out_u)) <= 1e-12


def test_absorb_q_identity():
    """q_lat . c == q_C . (W_UK c) for every head and token."""
    rng = np.random.default_rng(3)
    q_c = rng.standard_normal((4, 5, 128))
    w_uk = rng.standard_normal((5, 128, 512))
    c = rng.standard_normal((7, 512))
    q_lat = oracle.absorb_q(q_c, w_uk)
    assert q_lat.shape == (4, 5, 512)
    lhs = np.einsum("mhj,tj->mht", q_lat, c)
    k_c = np.stack([[w_uk[h] @ c[t] for t in range(7)] for h in range(5)])  # [h, t, i]
    rhs = np.stack([[[q_c[m, h] @ k_c[h, t] for t in range(7)] for h in range(5)]
                    for m in range(4)])
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def test_up_project_identity():
    """(sum_t p_t c_t) W_UV == sum_t p_t (W_UV^T c_t)."""
    rng = np.random.default_rng(4)
    c = rng.standard_normal((9, 512))
    p = rng.random((3, 9))
    p /= p.sum(axis=1, keepdims=True)
    w_uv = rng.standard_normal((3, 512, 128))
    o_lat = p @ c                                          # [3 heads, 512]
    out = oracle.up_project(o_lat[None], w_uv)[0]          # [3, 128]
    ref = np.stack([sum(p[h, t] * (w_uv[h].T @ c[t]) for t in range(9)) for h in range(3)])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_softmax_weights_sum_to_one():
    """A value that is 1 for every token makes the output the softmax row sum."""
    rng = np.random.default_rng(8)
    q_c, q_r, kv, table, lens, w_uk, w_uv, scale = _random_case(rng, lens=(1, 37, 50))
    # Latent column 0 is set to 1 for every token and W_UV reads only that column.
    kv[..., 0] = np.where(np.isnan(kv[..., 1]), np.nan, 1.0)
    w_uv = np.zeros_like(w_uv)
    w_uv[:, 0, :] = 1.0
    for form in ("unabsorbed", "absorbed"):
        out, _ = oracle.decode(q_c * 4, q_r * 4, kv, table, lens, w_uk, w_uv, scale, form=form)
        assert np.max(np.abs(out - 1.0)) <= 1e-15 * 64


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(9)
    q_c, q_r, kv, table, lens, w_uk, w_uv, scale = _random_case(rng, lens=(1, 1, 1))
    out, lse = oracle.decode(q_c, q_r, kv, table, lens, w_uk, w_uv, scale)
    for b in range(3):
        c0 = kv[table[b, 0], 0, :512]
        for h in range(3):
            np.testing.assert_allclose(out[b, 0, h], c0 @ w_uv[h], rtol=1e-13, atol=1e-13)
            s = (q_c[b, 0, h] @ (w_uk[h] @ c0) + q_r[b, 0, h] @ kv[table[b, 0], 0, 512:]) * scale
            assert lse[b, 0, h] == pytest.approx(s, rel=1e-12, abs=1e-12)


def test_zero_query_gives_mean_value():
    rng = np.random.default_rng(10)
    q_c, q_r, kv, table, lens, w_uk, w_uv, scale = _random_case(rng)
    out, lse = oracle.decode(q_c * 0, q_r * 0, kv, table, lens, w_uk, w_uv, scale)
    for b in range(3):
        n = int(lens[b])
        rows = np.stack([kv[table[b, t // 16], t % 16, :512] for t in range(n)])
        for h in range(3):
            np.testing.assert_allclose(out[b, 0, h], (rows @ w_uv[h]).mean(axis=0),
                                       rtol=1e-12, atol=1e-12)
            assert lse[b, 0, h] == pytest.approx(math.log(n), abs=1e-12)


def test_dominant_score_selects_its_token():
    """A key aligned with a huge query makes the output that token's value."""
    rng = np.random.default_rng(12)
    q_c, q_r, kv, table, lens, w_uk, w_uv, scale = _random_case(rng, lens=(20, 20, 20))
    b, h, t_star = 1, 2, 13
    q_c[:] = 0.0
    q_r[:] = 0.0
    q_r[b, 0, h, 0] = 1e4
    for t in range(20):
        kv[table[b, t // 16], t % 16, 512:] = 0.0
    kv[table[b, t_star // 16], t_star % 16, 512] = 1.0
    out, _ = oracle.decode(q_c, q_r, kv, table, lens, w_uk, w_uv, scale, batches=[b], heads=[h])
    c_star = kv[table[b, t_star // 16], t_star % 16, :512]
    np.testing.assert_allclose(out[0, 0, 0], c_star @ w_uv[h], rtol=1e-12, atol=1e-12)


def test_page_permutation_invariance():
    """Moving pages to other physical blocks (and fixing the table) changes nothing."""
    rng = np.random.default_rng(13)
    q_c, q_r, kv, table, lens, w_uk, w_uv, scale = _random_case(rng, tq=2, lens=(2, 37, 50))
    out0, lse0 = oracle.decode(q_c, q_r, kv, table, lens, w_uk, w_uv, scale)
    perm = rng.permutation(kv.shape[0])
    kv2 = np.empty_like(kv)
    kv2[perm] = kv
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
    out1, lse1 = oracle.decode(q_c, q_r, kv2, table2, lens, w_uk, w_uv, scale)
    np.testing.assert_array_equal(out0, out1)
    np.testing.assert_array_equal(lse0, lse1)


def test_matches_torch_sdpa_fp64():
    """Library cross-check: per head, torch's scaled_dot_product_attention in fp64."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(14)
    tq = 3
    q_c, q_r, kv, table, lens, w_uk, w_uv, scale = _random_case(rng, tq=tq, lens=(3, 37, 50))
    out, _ = oracle.decode(q_c, q_r, kv, table, lens, w_uk, w_uv, scale)
    for b in range(3):
        n = int(lens[b])
        rows = np.stack([kv[table[b, t // 16], t % 16] for t in range(n)])
        c, k_r = torch.from_numpy(rows[:, :512]), torch.from_numpy(rows[:, 512:])
        k = torch.cat([torch.einsum("hij,tj->hti", torch.from_numpy(w_uk), c),
                       k_r.expand(3, n, 64)], dim=-1)                  # [H, n, 192]
        v = torch.einsum("tj,hjd->htd", c, torch.from_numpy(w_uv))    # [H, n, 128]
        q = torch.cat([torch.from_numpy(q_c[b]), torch.from_numpy(q_r[b])], dim=-1)  # [tq, H, 192]
        q = q.permute(1, 0, 2)                                          # [H, tq, 192]
        pos = torch.arange(tq)[:, None] + (n - tq)
        mask = torch.arange(n)[None, :] <= pos                          # [tq, n]
        ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(out[b].transpose(1, 0, 2), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_prefill_rows_equal_decode_prefixes():
    """Causal prefill row t equals single-query decode over tokens 0..t."""
    rng = np.random.default_rng(15)
    T = 40
    q_c, q_r, kv, table, lens, w_uk, w_uv, scale = _random_case(
        rng, n_seq=1, tq=T, heads=2, lens=(T,))
    out_p, lse_p = oracle.prefill(q_c, q_r, kv, table, lens, w_uk, w_uv, scale)
    for t in (0, 1, 17, T - 1):
        out_d, lse_d = oracle.decode(q_c[:, t:t + 1], q_r[:, t:t + 1], kv, table,
                                     np.array([t + 1], dtype=np.int32), w_uk, w_uv, scale)
        np.testing.assert_allclose(out_p[:, t], out_d[:, 0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse_p[:, t], lse_d[:, 0], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("cuts", [(0, 50), (0, 1, 50), (0, 16, 32, 48, 50), (0, 7, 7, 30, 50)])
def test_combine_over_key_partition_equals_full(cuts):
    """Online renormalisation: merging per-range results reproduces full attention."""
    rng = np.random.default_rng(16)
    tq = 2
    q_c, q_r, kv, table, lens, w_uk, w_uv, scale = _random_case(
        rng, n_seq=1, tq=tq, lens=(50,))
    out, lse = oracle.decode(q_c, q_r, kv, table, lens, w_uk, w_uv, scale)
    rows = oracle.gather_rows(kv, table[0], 50)
    c, k_r = rows[:, :512], rows[:, 512:]
    q_lat = oracle.absorb_q(q_c[0], w_uk)
    vis = [50 - tq + i + 1 for i in range(tq)]
    parts = [oracle.split_partial(q_lat, q_r[0], c, k_r, scale, a, b, vis)
             for a, b in zip(cuts[:-1], cuts[1:])]
    part_o = np.stack([p[0] for p in parts])
    part_lse = np.stack([p[1] for p in parts])
    out_c, lse_c = oracle.combine_partials(part_o, part_lse, w_uv)
    np.testing.assert_allclose(out_c, out[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse_c, lse[0], rtol=1e-12, atol=1e-12)


def test_combine_empty_rows():
    part_o = np.full((3, 2, 4, 8), np.nan)
    part_lse = np.full((3, 2, 4), -np.inf)
    part_o[1, 0] = 2.0
    part_lse[1, 0] = 0.5
    o, lse = oracle.combine_partials(part_o, part_lse)
    np.testing.assert_array_equal(o[0], 2.0)
    np.testing.assert_array_equal(lse[0], 0.5)
    np.testing.assert_array_equal(o[1], 0.0)
    assert np.all(np.isneginf(lse[1]))


def test_combine_two_splits_closed_form():
    """Two splits with lse a and b: weights e^a/(e^a+e^b) and e^b/(e^a+e^b)."""
    part_o = np.array([[[[1.0, 0.0]]], [[[0.0, 1.0]]]])   # [S=2, M=1, H=1, 2]
    part_lse = np.array([[[math.log(3.0)]], [[math.log(1.0)]]])
    o, lse = oracle.combine_partials(part_o, part_lse)
    np.testing.assert_allclose(o[0, 0], [0.75, 0.25], rtol=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(4.0), rel=1e-15)


# ---------------------------------------------------------------------------
# The pins must be able to fail: plausible mistakes, planted on the CPU, are
# caught by the closed forms above.
# ---------------------------------------------------------------------------

def _hand_head_values(q_c, q_r, kv, table, lens, w_uk, w_uv, scale, tq=1):
    return oracle.decode(q_c, q_r, kv, table, lens, w_uk, w_uv, scale)[0]


def test_planted_mistakes_are_caught():
    q_c, q_r, kv, table, lens, w_uk, w_uv, scale = _hand()
    want0 = (7 * E + 3) / (2 * E + 1)
    want1 = (1 - E**2) / (1 + E + E**2)
    # Dropped rotary term: k_R zeroed.
    kv_no_rope = kv.copy()
    kv_no_rope[..., 2] = 0.0
    got = _hand_head_values(q_c, q_r, kv_no_rope, table, lens, w_uk, w_uv, scale)
    assert abs(got[0, 0, 1, 0] - want1) > 1e-3
    # Sign error on the rotary term.
    got = _hand_head_values(q_c, -q_r, kv, table, lens, w_uk, w_uv, scale)
    assert abs(got[0, 0, 1, 0] - want1) > 1e-3
    # Heads swapped in W_UK (a wrong head index).
    got = _hand_head_values(q_c, q_r, kv, table, lens, w_uk[::-1].copy(), w_uv, scale)
    assert abs(got[0, 0, 0, 0] - want0) > 1e-3
    # Latent index reversed in W_UV (a transposed / misread operand).
    got = _hand_head_values(q_c, q_r, kv, table, lens, w_uk, w_uv[:, ::-1].copy(), scale)
    assert abs(got[0, 0, 0, 0] - want0) > 1e-3
    # Scale by 1/sqrt(576) instead of 1/sqrt(192) changes the scaled hand case.
    x = math.exp(1 / math.sqrt(2))
    got = _hand_head_values(q_c, q_r, kv, table, lens, w_uk, w_uv, 1 / math.sqrt(6))
    assert abs(got[0, 0, 0, 0] - (7 * x + 3) / (2 * x + 1)) > 1e-3
    # Causal mask off for MTP query 0: it would see token 2 as well.
    q2 = _hand(tq=2)
    got = oracle.decode(*q2)[0]
    assert abs(got[0, 0, 0, 0] - want0) > 1e-3


# ---------------------------------------------------------------------------
# Printed numbers.
# ---------------------------------------------------------------------------

def test_printed_sizes():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)
    row = facts["cached_values_per_token_per_layer"]
    assert row["parts"]["latent"] + row["parts"]["rotary_key"] == row["value"] == 576
    dims = facts["attention_dims"]
    assert dims["content_key_value_size"] + dims["rotary_size"] == \
        facts["score_scale_denominator_sqrt_of"]["value"] == 192
    layers = facts["layers"]["value"]
    per_token = row["value"] * layers * 2                               # bf16
    assert round(per_token / 1000, 1) == facts["cache_kb_per_token_all_layers"]["value"]
    mem = facts["cache_gb_per_131072_tokens"]
    assert round(per_token * 131072 / 1e9, 1) == mem["value"]
    full = dims["heads"] * (192 + 128) * 2 * layers * 131072 / 1e9
    assert round(full) == mem["full_kv_gb"]
    assert round(dims["heads"] * (192 + 128) / 576) == mem["saving_factor"]
    params = dims["kv_latent"] * dims["heads"] * (128 + 128)
    assert round(params / 1e6, 1) == facts["w_uk_plus_w_uv_params_millions"]["value"]
    assert 4096 * 40 == facts["max_positions"]["value"]
    # One layer of a 163,840-token sequence is about 189 MB of latent cache.
    assert round(163840 * 576 * 2 / 1e6) == 189
