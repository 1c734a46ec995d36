"""The decode step (absorb -> paged decode -> combine) captured in a HIP graph:
every replay, with eager work and synchronisations between replays, matches the
eager result bit for bit (the kernels clear nothing through memset nodes)."""

import numpy as np
import pytest
import torch

from gpu_helpers import DevInputs, make
from mla_latent_kv_19_amd import api, synth

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager():
    print("[case] decode step in a graph", flush=True)
    wl = synth.small_workload(batch=6, tq=2, len_lo=2, len_hi=900, seed=2801)
    inp = make(wl)
    dev = DevInputs(inp)
    B, Tq = wl.batch, wl.tq
    splits = 3
    q_lat = torch.empty((B, Tq, 128, 512), dtype=torch.bfloat16, device="cuda")
    part_o = torch.empty((splits, B, Tq, 128, 512), dtype=torch.float32, device="cuda")
    part_lse = torch.empty((splits, B, Tq, 128), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Tq, 128, 128), dtype=torch.bfloat16, device="cuda")

    def step():
        api.absorb_q(dev.q_c, dev.w_uk, out=q_lat)
        api.decode_paged(q_lat, dev.q_r, dev.kv, dev.table, dev.lens, wl.scale, splits, part_o,
                         part_lse)
        api.combine(part_o, part_lse, dev.w_uv, out=out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # eager run on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()                              # eager work between replays
        part_o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
