"""Shared pieces of the GPU parity tests: move seeded inputs to the device,
run the HIP path through the binding, and compare with the fp64 oracle."""

import numpy as np
import torch

import oracle
from mla_latent_kv_19_amd import api, synth

# Parity bar: max-abs error and relative L2 error against the fp64 oracle.
MAX_ABS = 2e-2
REL_L2 = 5e-3


def to_dev(bits, dtype=torch.bfloat16):
    """uint16 bf16 bit patterns -> device tensor of that dtype (bit-exact)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(dtype).cuda()


def to_dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


class DevInputs:
    def __init__(self, inp):
        self.inp = inp
        self.q_c = to_dev(inp.q_c)
        self.q_r = to_dev(inp.q_r)
        self.kv = to_dev(inp.kv_cache)
        self.table = to_dev_i32(inp.block_table)
        self.lens = to_dev_i32(inp.seq_lens)
        self.w_uk = to_dev(inp.w_uk)
        self.w_uv = to_dev(inp.w_uv)


def bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_decode(dev, splits=None, want_lse=True):
    wl = dev.inp.wl
    if splits is None:
        splits = api.num_splits(wl.batch, wl.tq, int(dev.inp.seq_lens.max()))
    res = api.decode_step(dev.q_c, dev.q_r, dev.kv, dev.table, dev.lens, dev.w_uk, dev.w_uv,
                          wl.scale, splits=splits, want_lse=want_lse)
    torch.cuda.synchronize()
    return res


def oracle_decode(inp, batches=None, heads=None, form="unabsorbed"):
    return oracle.decode(inp.values("q_c"), inp.values("q_r"), inp.values("kv_cache"),
                         inp.block_table, inp.seq_lens, inp.values("w_uk"), inp.values("w_uv"),
                         inp.wl.scale, batches=batches, heads=heads, form=form)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    max_abs = float(np.max(np.abs(got - ref))) if got.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return max_abs, rel


def assert_parity(got, ref, what, max_abs=MAX_ABS, rel_l2=REL_L2):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    e_abs, e_rel = errors(got, ref)
    print(f"[parity] {what}: max_abs={e_abs:.3e} rel_l2={e_rel:.3e}", flush=True)
    assert e_abs <= max_abs and e_rel <= rel_l2, (
        f"{what}: max_abs {e_abs:.3e} (bar {max_abs}) rel_l2 {e_rel:.3e} (bar {rel_l2})")


def make(wl, seq_lens=None):
    return synth.make_inputs(wl, seq_lens=seq_lens)


def plant_dominant_keys(inp, keys, scale=40.0, seed=7):
    """Make key t of sequence b dominate every score that sees it, for each
    (b, t) in `keys`: all heads and queries of sequence b get the same rotary
    query u (N(0, 1), 64 wide) and token t's rotary key becomes scale * u, so
    its score exceeds the others by about scale * 64 / sqrt(192) (natural
    units).  Edits the bf16 bit arrays of `inp` in place."""
    rng = np.random.default_rng(seed)
    for b, t in keys:
        u = rng.standard_normal(64).astype(np.float32)
        inp.q_r[b] = synth.f32_to_bf16_bits(u)
        blk = inp.block_table[b, t // 64]
        inp.kv_cache[blk, t % 64, 512:576] = synth.f32_to_bf16_bits(np.float32(scale) * u)
    return inp


def plant_rescale_jump(inp, b, n_old, n_new, jump=6.0, seed=11):
    """Sequence b: latent queries q_C = 0 and rotary keys 0 for every token
    except n_new tokens starting at n_old, so all other scores are exactly 0;
    those n_new tokens get rotary key s * u (rotary query u for every head and
    query) with s chosen so that their score is about `jump` (natural units).
    With jump = 6 (8.7 in log2 units) the running maximum moves past a 2^8
    lazy-rescale threshold once, while the n_old earlier tokens keep a large
    share of the softmax mass (n_old against n_new * e^jump), so the rescale of
    what was accumulated before the jump decides the output.  Edits `inp` in
    place."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(64).astype(np.float32)
    ub = synth.f32_to_bf16_bits(u)
    uf = synth.bf16_bits_to_f64(ub)
    s = jump / (float(uf @ uf) * inp.wl.scale)
    inp.q_c[b] = 0
    inp.q_r[b] = ub
    L = int(inp.seq_lens[b])
    kb = synth.f32_to_bf16_bits(np.float32(s) * u)
    for t in range(L):
        blk = inp.block_table[b, t // 64]
        inp.kv_cache[blk, t % 64, 512:576] = kb if n_old <= t < n_old + n_new else 0
    return inp
