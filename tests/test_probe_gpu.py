"""The HBM read probe through the C ABI: it reads the whole buffer and writes
nothing (the sink stays as it was unless the fold hits the magic value)."""

import pytest
import torch

from mla_latent_kv_19_amd import api

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 64 << 20])
def test_read_probe_runs_and_leaves_sink(nbytes):
    print(f"[case] read probe {nbytes} bytes", flush=True)
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    api.hbm_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
