"""Pins of the cache-append oracle (kv_down -> RMSNorm | RoPE -> paged write).

Each test checks the oracle against something other than itself: a hand case
with a closed form, an identity rotations or norms must satisfy, brute force
on a tiny input, or a placement worked out by hand.
"""

import math

import numpy as np
import pytest

from oracle import cache_append as ca


def test_rope_hand_cases():
    # d_r = 2: one pair, inv_freq = [1]: a rotation by pos radians.
    np.testing.assert_allclose(ca.apply_rope([1.0, 0.0], 1, 10000.0),
                               [math.cos(1.0), math.sin(1.0)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(ca.apply_rope([0.0, 1.0], 2, 10000.0),
                               [-math.sin(2.0), math.cos(2.0)], rtol=0, atol=1e-15)
    # d_r = 4, theta = 16: inv_freq = [1, 1/4]; pair 1 of (0, 0, 2, 0) at pos 2 turns by 1/2.
    np.testing.assert_allclose(ca.apply_rope([0.0, 0.0, 2.0, 0.0], 2, 16.0),
                               [0.0, 0.0, 2 * math.cos(0.5), 2 * math.sin(0.5)], atol=1e-15)


def test_rope_inverse_frequencies():
    inv = ca.rope_inv_freq(64, 10000.0)
    assert inv.shape == (32,)
    assert inv[0] == 1.0
    assert inv[1] == pytest.approx(math.exp(-math.log(10000.0) / 32), rel=1e-15)
    assert inv[31] == pytest.approx(10000.0 ** (-62 / 64), rel=1e-14)
    assert np.all(np.diff(inv) < 0)


def test_rope_rotation_properties():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    # Position 0 is the identity; each pair keeps its length.
    np.testing.assert_array_equal(ca.apply_rope(q, 0, 10000.0), q)
    r = ca.apply_rope(q, 12345, 10000.0)
    np.testing.assert_allclose(r[0::2] ** 2 + r[1::2] ** 2, q[0::2] ** 2 + q[1::2] ** 2, rtol=1e-12)
    # Scores depend on the relative position only; rotations compose.
    for m, n in [(7, 3), (1000, 999), (163839, 5)]:
        lhs = ca.apply_rope(q, m, 10000.0) @ ca.apply_rope(k, n, 10000.0)
        rhs = ca.apply_rope(q, m - n, 10000.0) @ k
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9)
    np.testing.assert_allclose(ca.apply_rope(ca.apply_rope(q, 40, 10000.0), 2, 10000.0),
                               ca.apply_rope(q, 42, 10000.0), rtol=1e-12, atol=1e-12)


def test_rms_norm_hand_case_and_invariances():
    # (3, 4): mean square 12.5.
    np.testing.assert_allclose(ca.rms_norm([3.0, 4.0], [1.0, 1.0], 0.0),
                               [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15)
    np.testing.assert_allclose(ca.rms_norm([3.0, 4.0], [2.0, -1.0], 0.0),
                               [6 / math.sqrt(12.5), -4 / math.sqrt(12.5)], rtol=1e-15)
    # eps keeps a zero vector at zero; with eps the hand case shifts by it.
    np.testing.assert_array_equal(ca.rms_norm([0.0, 0.0], [1.0, 1.0], 1e-6), [0.0, 0.0])
    np.testing.assert_allclose(ca.rms_norm([3.0, 4.0], [1.0, 1.0], 0.5),
                               [3 / math.sqrt(13.0), 4 / math.sqrt(13.0)], rtol=1e-15)
    rng = np.random.default_rng(4)
    x = rng.standard_normal(512)
    y = ca.rms_norm(x, np.ones(512), 0.0)
    assert np.sqrt(np.mean(y * y)) == pytest.approx(1.0, rel=1e-14)
    np.testing.assert_allclose(ca.rms_norm(5.0 * x, np.ones(512), 0.0), y, rtol=1e-13)


def test_kv_down_against_brute_force():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 7))
    w = rng.standard_normal((5, 7))
    got = ca.kv_down(x, w)
    for m in range(3):
        for o in range(5):
            assert got[m, o] == pytest.approx(sum(x[m, j] * w[o, j] for j in range(7)), rel=1e-13)
    # A weight of unit rows picks coordinates.
    sel = np.eye(7)[[6, 0, 3]]
    np.testing.assert_array_equal(ca.kv_down(x, sel), x[:, [6, 0, 3]])


def test_cache_rows_split_order():
    # d_model = 4, d_c = 2, d_r = 2: outputs 0,1 are the latent, 2,3 the rotary key.
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    w = np.eye(4)[[0, 1, 2, 3]]
    rows = ca.cache_rows(x, w, gamma=[1.0, 1.0], positions=[1], eps=0.0, theta=10000.0, d_c=2)
    np.testing.assert_allclose(rows[0, :2], [1 / math.sqrt(2.5), 2 / math.sqrt(2.5)], rtol=1e-15)
    np.testing.assert_allclose(rows[0, 2:], [3 * math.cos(1) - 4 * math.sin(1),
                                             3 * math.sin(1) + 4 * math.cos(1)], rtol=1e-14)


def test_cache_append_placement():
    # Two sequences, block size 4; sequence 0 owns blocks [2, 0], sequence 1 [1].
    kv = np.full((3, 4, 4), np.nan)
    table = np.array([[2, 0], [1, -1]], dtype=np.int32)
    x = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0], [0, 0, 1.0, 0]])
    w = np.eye(4)
    out, rows = ca.cache_append(x, w, [1.0, 1.0], seq_idx=[0, 1, 0], positions=[5, 2, 0],
                                block_table=table, kv_cache=kv, eps=1e-6, theta=10000.0, d_c=2)
    np.testing.assert_array_equal(out[0, 1], rows[0])      # seq 0, pos 5 -> block 0, row 1
    np.testing.assert_array_equal(out[1, 2], rows[1])      # seq 1, pos 2 -> block 1, row 2
    np.testing.assert_array_equal(out[2, 0], rows[2])      # seq 0, pos 0 -> block 2, row 0
    written = {(0, 1), (1, 2), (2, 0)}
    for blk in range(3):
        for r in range(4):
            if (blk, r) not in written:
                assert np.all(np.isnan(out[blk, r]))
    # The input cache is left as it was.
    assert np.all(np.isnan(kv))


# --- projections around the attention ----------------------------------------

from oracle import projections as pj  # noqa: E402


def test_query_project_hand_case():
    # d_model 2, q_rank 2, one head with d_h = 1 and d_r = 2 (outputs: [q_C | q_R0, q_R1]).
    x = np.array([[3.0, 4.0]])
    w_dq = np.eye(2)                                   # c_q = (3, 4), RMS = sqrt(12.5)
    gamma = np.array([1.0, 2.0])                       # c_q' = (3, 8) / sqrt(12.5)
    w_uq = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    s = math.sqrt(12.5)
    q_c, q_r = pj.query_project(x, w_dq, gamma, w_uq, positions=[1], eps=0.0, theta=10000.0,
                                n_heads=1, d_h=1, d_r=2)
    assert q_c[0, 0, 0] == pytest.approx(3 / s, rel=1e-15)
    # Rotary pair (8/s, 11/s) turned by 1 radian (d_r = 2: inv_freq = 1).
    a, b = 8 / s, 11 / s
    np.testing.assert_allclose(q_r[0, 0], [a * math.cos(1) - b * math.sin(1),
                                           a * math.sin(1) + b * math.cos(1)], rtol=1e-14)


def test_query_project_structure():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 32))
    w_dq = rng.standard_normal((16, 32))
    gamma = 1 + 0.1 * rng.standard_normal(16)
    w_uq = rng.standard_normal((4 * (8 + 4), 16))
    args = dict(eps=1e-6, theta=10000.0, n_heads=4, d_h=8, d_r=4)
    qc0, qr0 = pj.query_project(x, w_dq, gamma, w_uq, positions=[0, 0, 0], **args)
    qc1, qr1 = pj.query_project(x, w_dq, gamma, w_uq, positions=[5, 900, 77777], **args)
    np.testing.assert_array_equal(qc0, qc1)             # the content query has no position
    # Position 0: the rotary query is the raw product's last 4 outputs of each head.
    cq = ca.rms_norm(x @ w_dq.T, gamma, 1e-6)
    raw = (cq @ w_uq.T).reshape(3, 4, 12)
    np.testing.assert_allclose(qr0, raw[..., 8:], rtol=1e-13)
    np.testing.assert_allclose(qc0, raw[..., :8], rtol=1e-13)
    np.testing.assert_allclose(qr1[1], ca.apply_rope(raw[1, :, 8:], 900, 10000.0), rtol=1e-12)


def test_output_project_against_brute_force():
    rng = np.random.default_rng(7)
    o = rng.standard_normal((2, 6))
    w_o = rng.standard_normal((3, 6))
    got = pj.output_project(o, w_o)
    for m in range(2):
        for d in range(3):
            assert got[m, d] == pytest.approx(sum(o[m, j] * w_o[d, j] for j in range(6)), rel=1e-13)


def test_printed_rmsnorm_eps_and_rope_theta():
    """The oracle's and the binding's defaults are the values the pages print:
    eps of the explorer's "RMSNorm" box and theta of its RoPE box
    (tests/golden/page_facts.json)."""
    import inspect
    import json
    import os

    from oracle import projections as pj

    with open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")) as f:
        facts = json.load(f)
    eps, theta = facts["rmsnorm_eps"]["value"], facts["rope_theta"]["value"]
    assert float(facts["rmsnorm_eps"]["printed"]) == eps
    assert ca.RMS_EPS == eps and ca.ROPE_THETA == theta
    for fn in (ca.rms_norm, ca.cache_rows, ca.cache_append, pj.query_project):
        params = inspect.signature(fn).parameters
        assert params["eps"].default == eps, fn.__name__
    for fn in (ca.rope_inv_freq, ca.apply_rope, ca.cache_rows, ca.cache_append, pj.query_project):
        assert inspect.signature(fn).parameters["theta"].default == theta, fn.__name__
    # The binding's defaults (read from its source: importing it needs torch only).
    from mla_latent_kv_19_amd import api
    for fn in (api.cache_append, api.query_project):
        params = inspect.signature(fn).parameters
        assert params["eps"].default == eps and params["rope_theta"].default == theta, fn.__name__
    # The printed formula with eps: a vector of mean square 1e-6 is scaled by 1/sqrt(2e-6).
    x = np.full(512, 1e-3)
    np.testing.assert_allclose(ca.rms_norm(x, np.ones(512)), x / math.sqrt(2e-6), rtol=1e-14)
