"""CPU tests of the binding's debug-mode check of the paged-cache metadata
(block table and sequence lengths): the preconditions the C ABI documents but
cannot check without a synchronisation."""

import numpy as np
import pytest

api = pytest.importorskip("mla_latent_kv_19_amd.api")
from mla_latent_kv_19_amd import synth  # noqa: E402


def _good():
    # Three sequences, 64-token blocks, a pool of 10 blocks.
    table = np.array([[3, 7, -1], [0, -1, -1], [9, 2, 5]], dtype=np.int32)
    lens = np.array([100, 64, 129], dtype=np.int32)
    return table, lens


def test_valid_metadata_passes():
    table, lens = _good()
    api.check_paged_metadata(table, lens, num_blocks=10, n_query=1)
    api.check_paged_metadata(table, lens, num_blocks=10, n_query=64)


def test_seeded_workloads_pass():
    """The generator's block tables (a seeded permutation of the pool, one
    owner per block) meet every precondition at the bench and parity shapes."""
    for name in ("single", "batched", "mtp", "verify5", "verify8", "long", "headline", "prefill"):
        wl = synth.WORKLOADS[name]
        lens = synth.seq_lens_for(wl)
        table, num_blocks = synth.block_table_for(wl, lens)
        api.check_paged_metadata(table, lens, num_blocks, wl.tq)


@pytest.mark.parametrize("edit,needle", [
    (lambda t, l: l.__setitem__(1, 0), "outside [1, 192]"),            # shorter than Tq
    (lambda t, l: l.__setitem__(2, 193), "outside [1, 192]"),          # past the table row
    (lambda t, l: t.__setitem__((0, 1), -1), "block id -1"),           # used page unmapped
    (lambda t, l: t.__setitem__((2, 2), 10), "block id 10"),           # id past the pool
    (lambda t, l: t.__setitem__((1, 0), 7), "block 7 is used more than once"),   # shared page
    (lambda t, l: t.__setitem__((2, 1), 9), "block 9 is used more than once"),   # aliased page
])
def test_each_violation_is_named(edit, needle):
    table, lens = _good()
    edit(table, lens)
    with pytest.raises(ValueError, match=needle.replace("[", r"\[").replace("]", r"\]")):
        api.check_paged_metadata(table, lens, num_blocks=10, n_query=1)


def test_entries_past_the_used_pages_are_ignored():
    table, lens = _good()
    table[1, 1:] = [12345, 7]           # past sequence 1's single page: never read
    api.check_paged_metadata(table, lens, num_blocks=10, n_query=1)


def test_query_count_bound():
    table, lens = _good()
    with pytest.raises(ValueError, match="sequence 1"):
        api.check_paged_metadata(table, lens, num_blocks=10, n_query=65)


def test_debug_switch():
    prev = api.set_debug(True)
    try:
        assert api.debug_enabled()
        assert api.set_debug(False) is True
        assert not api.debug_enabled()
    finally:
        api.set_debug(prev)
