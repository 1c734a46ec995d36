"""The no-allocation decode (mla_decode_noalloc, partials in the library's own
device buffer) against mla_decode_paged + mla_combine with caller workspace,
through the C ABI: two calls in a row, the second smaller, each bit-identical
to the workspace path (same kernels) and within the parity bar of the fp64
oracle; the size limit is rejected on the host."""

import numpy as np
import pytest
import torch

from gpu_helpers import DevInputs, assert_parity, bf16_to_f64, make, oracle_decode
from mla_latent_kv_19_amd import api, synth

pytestmark = pytest.mark.gpu


def _workspace_path(dev, splits):
    q_lat = api.absorb_q(dev.q_c, dev.w_uk)
    part_o, part_lse = api.decode_paged(q_lat, dev.q_r, dev.kv, dev.table, dev.lens,
                                        dev.inp.wl.scale, splits)
    out, lse = api.combine(part_o, part_lse, dev.w_uv, want_lse=True)
    return q_lat, out, lse


def _noalloc_path(dev, q_lat, splits):
    b, tq = q_lat.shape[0], q_lat.shape[1]
    out = torch.empty((b, tq, 128, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, tq, 128), dtype=torch.float32, device="cuda")
    api.decode_noalloc(q_lat, dev.q_r, dev.kv, dev.table, dev.lens, dev.w_uv, dev.inp.wl.scale,
                       splits, out, lse)
    return out, lse


@pytest.mark.parametrize("first,second", [
    ((16, 2, 1, 1500, 8), (3, 1, 1, 200, 3)),       # (batch, tq, len_lo, len_hi, splits)
    ((64, 1, 1, 2048, 10), (5, 2, 2, 700, 16)),     # the buffer's full size (640 pairs), then a smaller call
])
def test_noalloc_matches_workspace_path(first, second):
    for k, (batch, tq, lo, hi, splits) in enumerate((first, second)):
        print(f"[case] noalloc call {k}: B={batch} Tq={tq} L=[{lo},{hi}] splits={splits}",
              flush=True)
        wl = synth.small_workload(batch=batch, tq=tq, len_lo=max(lo, tq), len_hi=hi,
                                  seed=3100 + 7 * k + batch)
        inp = make(wl)
        dev = DevInputs(inp)
        q_lat, ref_out, ref_lse = _workspace_path(dev, splits)
        out, lse = _noalloc_path(dev, q_lat, splits)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse, ref_lse)
        got = bf16_to_f64(out)
        picks = sorted({0, batch // 2, batch - 1})
        ref, _ = oracle_decode(inp, batches=picks, form="absorbed")
        assert_parity(got[picks], ref, f"noalloc call {k}")


def test_noalloc_limit_is_rejected():
    print("[case] noalloc limit", flush=True)
    wl = synth.small_workload(batch=65, tq=1, len_lo=1, len_hi=100, seed=3150)
    dev = DevInputs(make(wl))
    q_lat = api.absorb_q(dev.q_c, dev.w_uk)
    out = torch.empty((65, 1, 128, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.MLAError, match="NOALLOC_LIMIT"):
        api.decode_noalloc(q_lat, dev.q_r, dev.kv, dev.table, dev.lens, dev.w_uv, wl.scale, 10, out)
