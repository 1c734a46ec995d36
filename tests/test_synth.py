"""CPU checks of the seeded input generator."""

import numpy as np
import pytest

from mla_latent_kv_19_amd import synth


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e38, 1e-40],
                 dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0).
    assert back[0] == 1.0 and back[1] == 1.0
    # 1 + 3*2^-8 ties between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert back[2] == np.float32(1.0 + 2**-6)
    assert back[3] == 1.0
    assert back[4] == -2.5
    # Against a float64 reference rounding of random values.
    rng = np.random.default_rng(0)
    v = rng.standard_normal(100000).astype(np.float32)
    got = synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(v))
    err = np.abs(got - v.astype(np.float64))
    assert np.all(err <= np.abs(v) * 2.0**-8 + 1e-45)


def test_deterministic_and_regenerable():
    wl = synth.small_workload(batch=4, len_lo=1, len_hi=200, seed=3)
    a = synth.make_inputs(wl)
    b = synth.make_inputs(wl)
    for name in ("q_c", "q_r", "kv_cache", "block_table", "seq_lens", "w_uk", "w_uv"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    # One sequence regenerated alone matches its rows in the paged cache.
    bs = wl.block_size
    for s in range(wl.batch):
        n = int(a.seq_lens[s])
        rows = synth.sequence_rows(wl, s, n)
        for t in (0, n // 2, n - 1):
            np.testing.assert_array_equal(a.kv_cache[a.block_table[s, t // bs], t % bs], rows[t])


def test_block_table_is_injective_and_poisoned():
    wl = synth.small_workload(batch=6, len_lo=1, len_hi=500, seed=4)
    inp = synth.make_inputs(wl)
    bs = wl.block_size
    used = []
    for s in range(wl.batch):
        n = int(inp.seq_lens[s])
        p = (n + bs - 1) // bs
        assert np.all(inp.block_table[s, :p] >= 0)
        assert np.all(inp.block_table[s, p:] == -1)
        used.extend(inp.block_table[s, :p].tolist())
        tail = n % bs
        if tail:
            assert np.all(inp.kv_cache[inp.block_table[s, p - 1], tail:] == synth.BF16_NAN)
    assert len(used) == len(set(used)), "a page is shared between sequences"
    spare = sorted(set(range(inp.kv_cache.shape[0])) - set(used))
    assert len(spare) >= 1
    assert np.all(inp.kv_cache[spare] == synth.BF16_NAN)


def test_contiguous_workload_has_identity_table():
    wl = synth.WORKLOADS["single"]
    table, num_blocks = synth.block_table_for(wl, np.array([1024], dtype=np.int32))
    np.testing.assert_array_equal(table[0], np.arange(16))
    assert num_blocks == 16


def test_distributions_and_logit_variance():
    wl = synth.small_workload(batch=2, len_lo=256, len_hi=256, seed=5)
    inp = synth.make_inputs(wl)
    q_c = inp.values("q_c")
    w_uk = inp.values("w_uk")
    assert abs(q_c.std() - 1.0) < 0.02
    assert abs(w_uk.std() - 512 ** -0.5) < 0.002
    # The scaled logit (q_C . W_UK c + q_R . k_R) / sqrt(192) has variance ~1.
    kv = inp.values("kv_cache")
    rows = kv[inp.block_table[0, :4]].reshape(-1, 576)
    c, k_r = rows[:, :512], rows[:, 512:]
    q_r = inp.values("q_r")
    logits = (np.einsum("hi,hij,tj->ht", q_c[0, 0], w_uk, c)
              + q_r[0, 0] @ k_r.T) * wl.scale
    assert 0.85 < logits.var() < 1.15


def test_named_workloads():
    w = synth.WORKLOADS
    assert (w["headline"].batch, w["headline"].len_lo, w["headline"].tq) == (64, 32768, 1)
    assert (w["mtp"].tq, w["mtp"].len_lo, w["mtp"].len_hi) == (2, 4096, 8192)
    assert (w["verify5"].tq, w["verify8"].tq, w["verify8"].batch) == (5, 8, 64)
    assert w["long"].len_lo == 163840
    assert w["prefill"].tq == w["prefill"].len_lo == 4096
    assert w["single"].scale == pytest.approx(192 ** -0.5)
    lens = synth.seq_lens_for(w["batched"])
    assert lens.min() >= 1 and lens.max() <= 4096 and len(lens) == 32
