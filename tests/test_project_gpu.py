"""GPU parity of the query and output projections around the latent attention
against the fp64 oracle, through the C ABI, and of one whole attention-block
decode step (hidden state in, residual-stream update out)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_parity, bf16_to_f64, make, to_dev, to_dev_i32
from mla_latent_kv_19_amd import api, synth

pytestmark = pytest.mark.gpu
f64 = synth.bf16_bits_to_f64


@pytest.mark.parametrize("m", [1, 64, 300])
def test_query_project(m):
    print(f"[case] query projection m={m}", flush=True)
    x, w_dq, g, w_uq, pos = synth.query_inputs(m, seed=2410 + m)
    q_c, q_r = api.query_project(to_dev(x), to_dev(w_dq), to_dev(g), to_dev(w_uq), to_dev_i32(pos))
    torch.cuda.synchronize()
    ref_c, ref_r = oracle.projections.query_project(f64(x), f64(w_dq), f64(g), f64(w_uq), pos,
                                                    1e-6, 10000.0)
    assert_parity(bf16_to_f64(q_c), ref_c, f"q_C m={m}")
    assert_parity(bf16_to_f64(q_r), ref_r, f"q_R m={m}")


@pytest.mark.parametrize("m", [1, 64, 200])
def test_output_project(m):
    print(f"[case] output projection m={m}", flush=True)
    o, w_o = synth.output_inputs(m, seed=2510 + m)
    y = api.output_project(to_dev(o), to_dev(w_o))
    torch.cuda.synchronize()
    assert_parity(bf16_to_f64(y), oracle.projections.output_project(f64(o), f64(w_o)),
                  f"W_O m={m}")


@pytest.mark.parametrize("m,d_in,d_out", [
    (3, 80, 128),       # K not a multiple of 64: direct-load split-K kernel
    (64, 64, 320),      # streaming kernel, one 64-k chunk, a partly used 256-output tile
    (65, 64, 192),      # tile kernel, one chunk, a ragged 128-row tile
    (130, 448, 384),    # tile kernel, 7 chunks, two output tiles
    (100, 96, 128),     # M > 64, N not a multiple of 192: split-K kernel
])
def test_output_project_kernel_paths(m, d_in, d_out):
    """Each of the three projection kernels (and their edges) against the oracle."""
    print(f"[case] output projection m={m} d_in={d_in} d_out={d_out}", flush=True)
    o, w_o = synth.output_inputs(m, d_in=d_in, d_out=d_out, seed=2520 + m)
    y = api.output_project(to_dev(o), to_dev(w_o))
    torch.cuda.synchronize()
    assert_parity(bf16_to_f64(y), oracle.projections.output_project(f64(o), f64(w_o)),
                  f"W_O m={m} {d_in}->{d_out}")


def test_attention_block_decode_step():
    """x -> query projection -> absorb -> paged decode -> combine -> W_O, four
    sequences, against the oracle chain (un-absorbed attention in fp64).  The
    GPU rounds q_C, q_R and the head outputs to bf16 between stages; the
    oracle chain is exact."""
    print("[case] attention block decode step", flush=True)
    wl = synth.small_workload(batch=4, tq=1, len_lo=50, len_hi=400, seed=2601)
    inp = make(wl)
    B = wl.batch
    x, w_dq, g, w_uq, _ = synth.query_inputs(B, seed=2602)
    pos = (inp.seq_lens - 1).astype(np.int32)                  # the new token's position
    o_in, w_o = synth.output_inputs(1, seed=2603)
    q_c, q_r = api.query_project(to_dev(x), to_dev(w_dq), to_dev(g), to_dev(w_uq), to_dev_i32(pos))
    out = api.decode_step(q_c.view(B, 1, 128, 128), q_r.view(B, 1, 128, 64), to_dev(inp.kv_cache),
                          to_dev_i32(inp.block_table), to_dev_i32(inp.seq_lens),
                          to_dev(inp.w_uk), to_dev(inp.w_uv), wl.scale, splits=2)
    y = api.output_project(out.view(B, 128 * 128), to_dev(w_o))
    torch.cuda.synchronize()
    rc, rr = oracle.projections.query_project(f64(x), f64(w_dq), f64(g), f64(w_uq), pos,
                                              1e-6, 10000.0)
    att, _ = oracle.decode(rc[:, None], rr[:, None], inp.values("kv_cache"), inp.block_table,
                           inp.seq_lens, inp.values("w_uk"), inp.values("w_uv"), wl.scale)
    ref = oracle.projections.output_project(att.reshape(B, 128 * 128), f64(w_o))
    assert_parity(bf16_to_f64(y), ref, "attention block decode step")
