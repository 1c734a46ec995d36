"""Seeded synthetic inputs for MLA decode and prefill.

This module only draws and lays out inputs; it holds none of the attention
arithmetic.  Both the HIP path (through the Python binding) and the fp64
oracle consume what it produces, so it imports neither of them.

Recipe (shapes and distributions follow the workloads the pages' model
implies: 128 heads, content latent 512, rotary key 64, content head dim 128,
value head dim 128):

* Random streams: ``numpy.random.SeedSequence(seed).spawn`` gives independent
  streams for sequence lengths, the block table, q_C, q_R, W_UK, W_UV and one
  stream per sequence for its cached rows, so any one sequence can be
  regenerated alone.
* Activations q_C, q_R, c, k_R are N(0, 1); the up-projection weights W_UK and
  W_UV are N(0, 1/512) (variance 1/512).  Values are drawn in float32 and
  rounded to bfloat16 with round-to-nearest-even.  Every consumer gets the
  same bf16 bit patterns (uint16).
* Paged cache: pages of ``block_size`` tokens, rows of d_c + d_r values
  (latent first, then rotary key).  The pool holds every sequence's pages
  plus ``spare_frac`` spare pages; a seeded permutation assigns physical
  pages, so no page is shared between sequences.  Block-table entries past a
  sequence's last page are -1.  Rows past a sequence's length in its last
  page, and all spare pages, hold bf16 NaN so that a kernel reading them
  cannot go unnoticed.
"""

from dataclasses import dataclass, field

import numpy as np

BF16_NAN = 0x7FC0


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact float32 values of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits):
    """Exact float64 values of bf16 bit patterns."""
    return bf16_bits_to_f32(bits).astype(np.float64)


class Bf16View:
    """Read-only float64 view of a bf16 bit array, decoded on indexing.

    Lets a float64 consumer gather a few rows of a multi-GB bf16 cache without
    converting the whole cache.
    """

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, idx):
        return bf16_bits_to_f64(self.bits[idx])


@dataclass(frozen=True)
class Workload:
    """One synthetic decode or prefill workload."""

    name: str
    batch: int
    tq: int                 # query tokens per sequence (T for prefill)
    len_lo: int             # sequence length range, inclusive, counting the tq queries
    len_hi: int
    seed: int
    paged: bool = True      # False: identity block table (contiguous cache)
    heads: int = 128
    d_c: int = 512
    d_r: int = 64
    d_h: int = 128
    d_v: int = 128
    block_size: int = 64
    spare_frac: float = 0.10
    poison: bool = True
    prefill: bool = False
    note: str = ""

    @property
    def scale(self):
        """Score scale stated for these workloads: 1/sqrt(d_h + d_r)."""
        return float(1.0 / np.sqrt(self.d_h + self.d_r))

    @property
    def row_width(self):
        return self.d_c + self.d_r


# The named workloads.  Seeds are 1000 + the workload's number.
WORKLOADS = {
    "single": Workload("single", batch=1, tq=1, len_lo=1024, len_hi=1024, seed=1001,
                       paged=False, poison=False,
                       note="B=1 decode, L=1024, contiguous cache"),
    "batched": Workload("batched", batch=32, tq=1, len_lo=1, len_hi=4096, seed=1002,
                        note="B=32 paged decode, L ~ U[1, 4096]"),
    "mtp": Workload("mtp", batch=64, tq=2, len_lo=4096, len_hi=8192, seed=1003,
                    note="B=64 two-query causal decode, L ~ U[4096, 8192]"),
    "long": Workload("long", batch=8, tq=1, len_lo=163840, len_hi=163840, seed=1004,
                     note="B=8 decode, L=163,840 (4096 x 40)"),
    "prefill": Workload("prefill", batch=1, tq=4096, len_lo=4096, len_hi=4096, seed=1005,
                        paged=False, poison=False, prefill=True,
                        note="causal prefill, T=4096"),
    "headline": Workload("headline", batch=64, tq=1, len_lo=32768, len_hi=32768, seed=1006,
                         note="B=64 paged decode, L=32,768"),
    # Wider speculative verification: a token plus 4 or 7 drafts per sequence,
    # the MTP workload's batch and lengths otherwise.
    "verify5": Workload("verify5", batch=64, tq=5, len_lo=4096, len_hi=8192, seed=1007,
                        note="B=64 five-query causal verify, L ~ U[4096, 8192]"),
    "verify8": Workload("verify8", batch=64, tq=8, len_lo=4096, len_hi=8192, seed=1008,
                        note="B=64 eight-query causal verify, L ~ U[4096, 8192]"),
}


@dataclass
class Inputs:
    """bf16 bit patterns (uint16) and int32 metadata for one workload."""

    wl: Workload
    q_c: np.ndarray          # [B, Tq, H, d_h]
    q_r: np.ndarray          # [B, Tq, H, d_r]
    kv_cache: np.ndarray     # [num_blocks, block_size, d_c + d_r]
    block_table: np.ndarray  # int32 [B, max_blocks]
    seq_lens: np.ndarray     # int32 [B]
    w_uk: np.ndarray         # [H, d_h, d_c]
    w_uv: np.ndarray         # [H, d_c, d_v]
    extra: dict = field(default_factory=dict)

    def values(self, name):
        """float64 values of one bf16 input (kv_cache is returned as a lazy view)."""
        bits = getattr(self, name)
        if name == "kv_cache":
            return Bf16View(bits)
        return bf16_bits_to_f64(bits)


def _streams(seed):
    names = ["lens", "table", "q_c", "q_r", "w_uk", "w_uv", "rows"]
    return dict(zip(names, np.random.SeedSequence(seed).spawn(len(names))))


def _normal_bf16(seq, shape, std=1.0):
    rng = np.random.Generator(np.random.PCG64(seq))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def seq_lens_for(wl):
    """The workload's int32 sequence lengths."""
    if wl.len_lo == wl.len_hi:
        return np.full(wl.batch, wl.len_lo, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(_streams(wl.seed)["lens"]))
    return rng.integers(wl.len_lo, wl.len_hi + 1, size=wl.batch).astype(np.int32)


def sequence_rows(wl, b, seq_len):
    """Cached rows (bf16 bits [seq_len, d_c + d_r]) of sequence b, from its own stream."""
    seq = _streams(wl.seed)["rows"].spawn(wl.batch)[b]
    return _normal_bf16(seq, (seq_len, wl.row_width))


def weights_for(wl):
    """(w_uk [H, d_h, d_c], w_uv [H, d_c, d_v]) bf16 bits, N(0, 1/512)."""
    s = _streams(wl.seed)
    std = 1.0 / np.sqrt(512.0)
    w_uk = _normal_bf16(s["w_uk"], (wl.heads, wl.d_h, wl.d_c), std)
    w_uv = _normal_bf16(s["w_uv"], (wl.heads, wl.d_c, wl.d_v), std)
    return w_uk, w_uv


def queries_for(wl):
    """(q_c [B, Tq, H, d_h], q_r [B, Tq, H, d_r]) bf16 bits, N(0, 1)."""
    s = _streams(wl.seed)
    q_c = _normal_bf16(s["q_c"], (wl.batch, wl.tq, wl.heads, wl.d_h))
    q_r = _normal_bf16(s["q_r"], (wl.batch, wl.tq, wl.heads, wl.d_r))
    return q_c, q_r


def block_table_for(wl, seq_lens):
    """(block_table int32 [B, max_blocks], num_blocks) for the given lengths."""
    bs = wl.block_size
    pages = [(int(n) + bs - 1) // bs for n in seq_lens]
    max_blocks = max(1, max(pages))
    total = sum(pages)
    table = np.full((wl.batch, max_blocks), -1, dtype=np.int32)
    if not wl.paged:
        num_blocks = max(1, total)
        start = 0
        for b, p in enumerate(pages):
            table[b, :p] = np.arange(start, start + p, dtype=np.int32)
            start += p
        return table, num_blocks
    num_blocks = total + int(np.ceil(wl.spare_frac * total))
    rng = np.random.Generator(np.random.PCG64(_streams(wl.seed)["table"]))
    perm = rng.permutation(num_blocks).astype(np.int32)
    start = 0
    for b, p in enumerate(pages):
        table[b, :p] = perm[start:start + p]
        start += p
    return table, max(1, num_blocks)


def make_inputs(wl, seq_lens=None):
    """All inputs of a workload.  ``seq_lens`` overrides the drawn lengths."""
    lens = seq_lens_for(wl) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    if lens.shape != (wl.batch,):
        raise ValueError("seq_lens must have one entry per sequence")
    if (lens < wl.tq).any():
        raise ValueError("every sequence must hold at least its tq query tokens")
    table, num_blocks = block_table_for(wl, lens)
    bs = wl.block_size
    fill = BF16_NAN if wl.poison else 0
    kv = np.full((num_blocks, bs, wl.row_width), fill, dtype=np.uint16)
    for b in range(wl.batch):
        n = int(lens[b])
        rows = sequence_rows(wl, b, n)
        full, tail = divmod(n, bs)
        if full:
            kv[table[b, :full]] = rows[: full * bs].reshape(full, bs, wl.row_width)
        if tail:
            kv[table[b, full], :tail] = rows[full * bs:]
    q_c, q_r = queries_for(wl)
    w_uk, w_uv = weights_for(wl)
    return Inputs(wl, q_c, q_r, kv, table, lens, w_uk, w_uv)


def small_workload(name="small", batch=3, tq=1, len_lo=1, len_hi=300, seed=7, **kw):
    """A reduced-size workload with the full per-head dims, for quick parity checks."""
    return Workload(name, batch=batch, tq=tq, len_lo=len_lo, len_hi=len_hi, seed=seed, **kw)


@dataclass
class AppendInputs:
    """Inputs of one cache append (bf16 bit arrays and int32 index arrays)."""

    x: np.ndarray            # [M, d_model]
    w_kv: np.ndarray         # [d_c + d_r, d_model]
    gamma: np.ndarray        # [d_c]
    seq_idx: np.ndarray      # [M]
    positions: np.ndarray    # [M]
    block_table: np.ndarray  # [n_seq, max_blocks]
    kv_cache: np.ndarray     # [num_blocks, block_size, d_c + d_r], bf16 NaN everywhere


def append_inputs(m, d_model=7168, n_seq=4, max_pos=163840, seed=2001, block_size=64,
                  d_c=512, d_r=64, spare_frac=0.1):
    """M new tokens spread over n_seq sequences at distinct positions below max_pos.

    Hidden states are N(0, 1); the kv_down weight is N(0, 1/d_model) so each
    projected value is about N(0, 1); the RMSNorm gain is 1 + N(0, 0.1^2).
    Every sequence owns ceil(max_pos / block_size) pages of a pool with spare
    pages, assigned by a seeded permutation; the cache starts as bf16 NaN, so
    any row the append does not own stays NaN.
    """
    names = ["x", "w", "gamma", "seq", "pos", "table"]
    s = dict(zip(names, np.random.SeedSequence(seed).spawn(len(names))))
    x = _normal_bf16(s["x"], (m, d_model))
    w_kv = _normal_bf16(s["w"], (d_c + d_r, d_model), 1.0 / np.sqrt(d_model))
    g = np.random.Generator(np.random.PCG64(s["gamma"]))
    gamma = f32_to_bf16_bits(1.0 + 0.1 * g.standard_normal(d_c, dtype=np.float32))
    rng = np.random.Generator(np.random.PCG64(s["seq"]))
    seq_idx = rng.integers(0, n_seq, size=m).astype(np.int32)
    rng = np.random.Generator(np.random.PCG64(s["pos"]))
    positions = np.empty(m, dtype=np.int32)
    for b in range(n_seq):
        idx = np.nonzero(seq_idx == b)[0]
        positions[idx] = rng.choice(max_pos, size=idx.size, replace=False)
    pages = (max_pos + block_size - 1) // block_size
    total = n_seq * pages
    num_blocks = total + int(np.ceil(spare_frac * total))
    rng = np.random.Generator(np.random.PCG64(s["table"]))
    table = rng.permutation(num_blocks)[:total].astype(np.int32).reshape(n_seq, pages)
    kv = np.full((num_blocks, block_size, d_c + d_r), BF16_NAN, dtype=np.uint16)
    return AppendInputs(x, w_kv, gamma, seq_idx, positions, table, kv)


def query_inputs(m, d_model=7168, q_rank=1536, heads=128, d_h=128, d_r=64, max_pos=163840,
                 seed=2401):
    """(x, w_dq, gamma_q, w_uq, positions) for the query projection of m tokens.

    x N(0, 1); w_dq N(0, 1/d_model) and w_uq N(0, 1/q_rank), so each product's
    outputs are about N(0, 1); gamma_q 1 + N(0, 0.1^2); positions uniform
    below max_pos.  bf16 bit arrays and int32 positions.
    """
    s = dict(zip(["x", "dq", "g", "uq", "pos"], np.random.SeedSequence(seed).spawn(5)))
    x = _normal_bf16(s["x"], (m, d_model))
    w_dq = _normal_bf16(s["dq"], (q_rank, d_model), 1.0 / np.sqrt(d_model))
    g = np.random.Generator(np.random.PCG64(s["g"]))
    gamma_q = f32_to_bf16_bits(1.0 + 0.1 * g.standard_normal(q_rank, dtype=np.float32))
    w_uq = _normal_bf16(s["uq"], (heads * (d_h + d_r), q_rank), 1.0 / np.sqrt(q_rank))
    rng = np.random.Generator(np.random.PCG64(s["pos"]))
    positions = rng.integers(0, max_pos, size=m).astype(np.int32)
    return x, w_dq, gamma_q, w_uq, positions


def output_inputs(m, d_in=128 * 128, d_out=7168, seed=2501):
    """(o, w_o): head outputs N(0, 1) and W_O N(0, 1/d_in), bf16 bit arrays."""
    s = np.random.SeedSequence(seed).spawn(2)
    return _normal_bf16(s[0], (m, d_in)), _normal_bf16(s[1], (d_out, d_in), 1.0 / np.sqrt(d_in))
