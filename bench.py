"""Benchmark of the MLA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]

A step is one full decode pass over one batch: q-absorption (W_UK folded into
the query), split-KV attention over the paged latent cache, log-sum-exp
combine and the W_UV up-projection.  Inputs are seeded synthetic data with
the shapes of the pages' model (128 heads, latent 512 + rotary 64, content
head 128) and are resident in HBM before timing starts.  Each timed step is
bracketed by its own HIP events; a 512 MiB read before each step (outside
the events) leaves no cache state from the previous step.  ms_per_step is the
mean over the timed steps, with p10 / p50 / p90 alongside.  The default 30
warm-up steps let the clock settle after the start of sustained load (a
transient in which the same launch runs up to ~1.5x slower).

Prints one JSON line: whole-job throughput in KV-tokens/s, the dominant
kernel's roofline position (algorithmic bytes / measured launch time against
the 8 TB/s HBM peak), and the fp64 CPU oracle timed on a bounded sample on
this host.
"""

import argparse
import hashlib
import json
import os
import re
import struct
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode KV-tokens/s and TFLOP/s (+% HBM/MFMA roofline), B=64 ctx 32K, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA peak
# Dense bf16 matrix work the chip retires per shader clock: 256 CUs x 4 SIMDs,
# each a v_mfma_f32_32x32x16_bf16 (32768 FLOP) every 32 clocks (2.52 PFLOP/s
# at 2.4 GHz, the published peak).
BF16_FLOP_PER_CLOCK = 256 * 4 * 32768 / 32
ROW_BYTES = 576 * 2            # one cached token: latent 512 + rotary key 64, bf16
FLOP_PER_TOKEN_QUERY = 128 * 2 * (576 + 512)   # scores + value product, all heads
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_paged_headline_traffic.json")
FLUSH_BYTES = 512 << 20


class _Flush:
    """Evicts the 4 MB L2s and the 256 MB Infinity Cache before a timed call by
    reading 512 MiB (a sum over a zero buffer).  A write would do it too, but
    it leaves dirty lines whose write-back then competes with the timed
    kernel's reads: measured here, a 235 MB read runs at 2.8 TB/s after a
    512 MiB write and at 5.5 TB/s after a 512 MiB read."""

    def __init__(self):
        import torch
        self.buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.sink = None

    def __call__(self):
        self.sink = self.buf.sum()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 30 warm-up steps (~20 ms of sustained load): the GPU's clock management
    # settles only after a transient in which the same decode launch runs up to
    # ~1.5x slower; timing 60 steps then averages over its remaining swings.
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--splits", type=int, default=0, help="0 = library heuristic")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="counter-collection mode: K decode steps plus a 1 GiB device copy "
                         "(the byte-count calibration for HBM counters), nothing else")
    ap.add_argument("--profile-all", action="store_true",
                    help="with --profile: also K calls of each secondary workload (prefill, "
                         "cache append, projections)")
    return ap.parse_args()


def _elf_sections(d):
    shoff = struct.unpack_from("<Q", d, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", d, 0x3A)
    secs = []
    for i in range(shnum):
        name, typ, _, addr, off, size, link, _, _, _ = struct.unpack_from("<IIQQQQIIQQ", d, shoff + i * shentsize)
        secs.append({"name": name, "typ": typ, "addr": addr, "off": off, "size": size, "link": link})
    st = secs[shstrndx]
    for sec in secs:
        b = d[st["off"] + sec["name"]:]
        sec["sname"] = b[:b.index(b"\0")].decode()
    return secs


def kernel_code_hash(lib_path, pattern=r"decode_paged_kernel"):
    """sha256 (16 hex digits) of the gfx950 machine code of the kernel whose
    symbol matches `pattern`, read from the code object bundled in the library:
    it changes when the kernel's instructions change and not with comments."""
    d = open(lib_path, "rb").read()
    fat = [x for x in _elf_sections(d) if x["sname"] == ".hip_fatbin"][0]
    blob = d[fat["off"]:fat["off"] + fat["size"]]
    for m in re.finditer(b"__CLANG_OFFLOAD_BUNDLE__", blob):
        b0 = m.start()
        n = struct.unpack_from("<Q", blob, b0 + 24)[0]
        p = b0 + 32
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", blob, p)
            triple = blob[p + 24:p + 24 + tl].decode()
            p += 24 + tl
            if "gfx950" not in triple:
                continue
            co = blob[b0 + off:b0 + off + size]
            secs = _elf_sections(co)
            text = [x for x in secs if x["sname"] == ".text"][0]
            for sec in secs:
                if sec["typ"] != 2:                          # SHT_SYMTAB
                    continue
                strs = secs[sec["link"]]
                for k in range(sec["size"] // 24):
                    st_name, st_info, _, _, st_value, st_size = struct.unpack_from(
                        "<IBBHQQ", co, sec["off"] + k * 24)
                    nb = co[strs["off"] + st_name:]
                    name = nb[:nb.index(b"\0")].decode()
                    if (st_info & 0xF) == 2 and re.search(pattern, name):
                        o = text["off"] + (st_value - text["addr"])
                        return hashlib.sha256(co[o:o + st_size]).hexdigest()[:16]
    return None


def measured_traffic(lib_path):
    """HBM bytes per launch from the committed rocprofv3 counters, reported only
    while the decode kernel's machine code is the one they were taken on."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("kernel_code_sha") != kernel_code_hash(lib_path):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, inp_meta, budget_s):
    """The fp64 oracle (un-absorbed form) on a bounded sample of the workload.

    The sample is whole sequences (all heads) regenerated from their seeded
    streams, as many as fit the time budget (at least one), timed with
    perf_counter around the oracle calls only.
    """
    import oracle
    from mla_latent_kv_19_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    q_c, q_r = synth.queries_for(wl)
    w_uk, w_uv = (synth.bf16_bits_to_f64(w) for w in synth.weights_for(wl))
    spent, tokens, n_seq = 0.0, 0, 0
    for b in range(wl.batch):
        L = int(inp_meta["seq_lens"][b])
        rows = synth.bf16_bits_to_f64(synth.sequence_rows(wl, b, L))
        n_blk = (L + wl.block_size - 1) // wl.block_size
        kv = np.zeros((n_blk * wl.block_size, rows.shape[1]))
        kv[:L] = rows
        kv = kv.reshape(n_blk, wl.block_size, rows.shape[1])
        table = np.arange(n_blk, dtype=np.int32)[None]
        t0 = time.perf_counter()
        oracle.decode(synth.bf16_bits_to_f64(q_c[b:b + 1]), synth.bf16_bits_to_f64(q_r[b:b + 1]),
                      kv, table, np.array([L], dtype=np.int32), w_uk, w_uv, wl.scale)
        spent += time.perf_counter() - t0
        tokens += L
        n_seq += 1
        if spent * (n_seq + 1) / n_seq > budget_s:
            break
    total = int(np.sum(inp_meta["seq_lens"]))
    return {"value": tokens / spent, "unit": "KV-tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n_seq} of {wl.batch} sequences (all {wl.heads} heads, "
                      f"{tokens} KV tokens), un-absorbed fp64 numpy oracle, {spent:.1f} s",
            "extrapolated_full_config_s": total * spent / tokens}


def _timed_cold(fn, steps, warmup):
    """Mean ms of fn() over `steps` calls, each timed alone (HIP events on the
    current stream) after a 512 MiB read that evicts L2 and the MALL, so the
    weights a call streams come from HBM."""
    import torch
    for _ in range(warmup):
        fn()
    flush = _Flush()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    del flush
    return float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))


def read_probe(nbytes, reps=5):
    """Measured HBM read rate on this machine: the library's read probe over a
    buffer of `nbytes` (the decode kernel's KV stream size), each call cold,
    mean GB/s over `reps` calls."""
    import torch
    from mla_latent_kv_19_amd import api
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ms = _timed_cold(lambda: api.hbm_read_probe(buf, sink), reps, 1)
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def bench_prefill(steps, warmup):
    """Causal prefill, T = L = 4096, B = 1 (reconstruction + attention), on MFMA."""
    import torch
    from mla_latent_kv_19_amd import api, synth
    wl = synth.WORKLOADS["prefill"]
    inp = synth.make_inputs(wl)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q_c, q_r, kv = dev(inp.q_c), dev(inp.q_r), dev(inp.kv_cache)
    table = torch.from_numpy(inp.block_table).cuda()
    lens = torch.from_numpy(inp.seq_lens).cuda()
    w_uk, w_uv = dev(inp.w_uk), dev(inp.w_uv)
    T = wl.tq
    out = torch.empty((1, T, 128, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(api.prefill_workspace_bytes(1, table.shape[1]), dtype=torch.uint8,
                     device="cuda")

    def run():
        api.prefill(q_c, q_r, kv, table, lens, w_uk, w_uv, wl.scale, out=out, workspace=ws)

    ms = _timed_cold(run, steps, warmup)
    pairs = T * (T + 1) // 2
    flops = pairs * 128 * 2 * (192 + 128) + T * 128 * 512 * 256 * 2
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": f"{wl.name}: {wl.note}", "ms": ms, "tokens_per_s": T / (ms * 1e-3),
            "tflops": tflops, "bound": "mfma", "peak_tflops": BF16_PEAK_TFLOPS,
            "frac": tflops / BF16_PEAK_TFLOPS, "algorithmic_flop": flops}


def bench_decode_configs(steps, warmup):
    """The other decode workloads (single sequence, batched ragged, two-,
    five- and eight-token verify, long context): one full step each (absorb,
    split-KV attention,
    combine), cold-timed, placed against its binding roofline by arithmetic
    intensity.  Algorithmic bytes: KV rows + W_UK + W_UV + queries + outputs;
    FLOP: attention over every (query, visible key) pair + absorb + W_UV."""
    import torch
    from mla_latent_kv_19_amd import api, synth

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    res = {}
    for name in ("single", "batched", "mtp", "verify5", "verify8", "long"):
        wl = synth.WORKLOADS[name]
        inp = synth.make_inputs(wl)
        B, Tq = wl.batch, wl.tq
        lens = inp.seq_lens.astype(np.int64)
        q_c, q_r, kv = dev(inp.q_c), dev(inp.q_r), dev(inp.kv_cache)
        table = torch.from_numpy(inp.block_table).cuda()
        lens_d = torch.from_numpy(inp.seq_lens).cuda()
        w_uk, w_uv = dev(inp.w_uk), dev(inp.w_uv)
        del inp
        splits = api.num_splits(B, Tq, int(lens.max()))
        q_lat = torch.empty((B, Tq, 128, 512), dtype=torch.bfloat16, device="cuda")
        part_o = torch.empty((splits, B, Tq, 128, 512), dtype=torch.float32, device="cuda")
        part_lse = torch.empty((splits, B, Tq, 128), dtype=torch.float32, device="cuda")
        out = torch.empty((B, Tq, 128, 128), dtype=torch.bfloat16, device="cuda")

        def step():
            api.absorb_q(q_c, w_uk, out=q_lat)
            api.decode_paged(q_lat, q_r, kv, table, lens_d, wl.scale, splits, part_o, part_lse)
            api.combine(part_o, part_lse, w_uv, out=out)

        ms = _timed_cold(step, steps, warmup)
        rows = int(lens.sum())
        attended = int(sum(int(L) - Tq + i + 1 for L in lens for i in range(Tq)))
        nq = B * Tq
        nbytes = rows * ROW_BYTES + 2 * 128 * 128 * 512 * 2 + nq * 128 * (192 + 128) * 2
        flops = attended * FLOP_PER_TOKEN_QUERY + 2 * nq * 128 * 2 * 128 * 512
        secs = ms * 1e-3
        bound = "hbm" if flops / nbytes < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
        frac = (nbytes / secs / 1e9 / HBM_PEAK_GBS if bound == "hbm"
                else flops / secs / 1e12 / BF16_PEAK_TFLOPS)
        res[name] = {"workload": f"{wl.name}: {wl.note}", "splits": splits, "ms": ms,
                     "kv_tokens_per_s": rows / secs, "attended_per_s": attended / secs,
                     "gbs": nbytes / secs / 1e9, "tflops": flops / secs / 1e12,
                     "bound": bound, "frac": frac, "algorithmic_bytes": nbytes,
                     "algorithmic_flop": flops}
        del q_c, q_r, kv, table, lens_d, w_uk, w_uv, q_lat, part_o, part_lse, out
        torch.cuda.empty_cache()
    return res


def bench_append(steps, warmup):
    """Cache append (kv_down 7168 -> 576, RMSNorm, RoPE, paged write) for the
    64 new tokens of one decode step and for a 4096-token prefill chunk."""
    import torch
    from mla_latent_kv_19_amd import api, synth

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    res = {}
    for m, n_seq, max_pos in ((64, 64, 128), (4096, 1, 4096)):
        a = synth.append_inputs(m, n_seq=n_seq, max_pos=max_pos, seed=2300 + m)
        x, w, g, kv = dev(a.x), dev(a.w_kv), dev(a.gamma), dev(a.kv_cache)
        seq = torch.from_numpy(a.seq_idx).cuda()
        pos = torch.from_numpy(a.positions).cuda()
        table = torch.from_numpy(a.block_table).cuda()
        ws = torch.empty(api.cache_append_workspace_bytes(m, 7168), dtype=torch.uint8,
                         device="cuda")

        def run():
            api.cache_append(x, w, g, seq, pos, table, kv, workspace=ws)

        ms = _timed_cold(run, steps, warmup)
        flop = 2.0 * m * 7168 * 576
        hbm = 576 * 7168 * 2 + m * 7168 * 2 + m * 576 * 2 + 512 * 2      # weight, x, rows, gain
        res[f"tokens_{m}"] = {"ms": ms, "tflops": flop / (ms * 1e-3) / 1e12,
                              "gbs": hbm / (ms * 1e-3) / 1e9,
                              "bound": "hbm" if m <= 256 else "mfma",
                              "frac": (hbm / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS) if m <= 256
                              else (flop / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS)}
    return res


def bench_projections(steps, warmup):
    """Query projection (W_DQ, RMSNorm, W_UQ, RoPE) and output projection (W_O)
    for the 64 tokens of one decode step: weight-streaming, HBM-bound."""
    import torch
    from mla_latent_kv_19_amd import api, synth

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    def timed(fn):
        return _timed_cold(fn, steps, warmup)

    m = 64
    x, w_dq, g, w_uq, pos = synth.query_inputs(m, seed=2700)
    x, w_dq, g, w_uq = dev(x), dev(w_dq), dev(g), dev(w_uq)
    pos = torch.from_numpy(pos).cuda()
    q_c = torch.empty((m, 128, 128), dtype=torch.bfloat16, device="cuda")
    q_r = torch.empty((m, 128, 64), dtype=torch.bfloat16, device="cuda")
    ws_q = torch.empty(api.load().mla_query_project_workspace_bytes(m, 7168, 1536),
                       dtype=torch.uint8, device="cuda")
    ms_q = timed(lambda: api.query_project(x, w_dq, g, w_uq, pos, q_c=q_c, q_r=q_r, workspace=ws_q))
    bytes_q = (1536 * 7168 + 128 * 192 * 1536 + m * 7168 + m * 128 * 192) * 2
    o, w_o = synth.output_inputs(m, seed=2701)
    o, w_o = dev(o), dev(w_o)
    y = torch.empty((m, 7168), dtype=torch.bfloat16, device="cuda")
    ws_o = torch.empty(api.load().mla_output_project_workspace_bytes(m, 16384, 7168),
                       dtype=torch.uint8, device="cuda")
    ms_o = timed(lambda: api.output_project(o, w_o, y=y, workspace=ws_o))
    bytes_o = (7168 * 16384 + m * 16384 + m * 7168) * 2
    out = {}
    for name, ms, b in (("query_project_64", ms_q, bytes_q), ("output_project_64", ms_o, bytes_o)):
        gbs = b / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "gbs": gbs, "bound": "hbm", "frac": gbs / HBM_PEAK_GBS,
                     "algorithmic_bytes": b}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the decode path has no multi-GPU component).", file=sys.stderr)
        sys.exit(2)
    import torch
    from mla_latent_kv_19_amd import api, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    api.load()
    wl = synth.WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    inp = synth.make_inputs(wl)
    gen_s = time.perf_counter() - t_gen

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q_c, q_r = dev(inp.q_c), dev(inp.q_r)
    kv = dev(inp.kv_cache)
    table = torch.from_numpy(inp.block_table).cuda()
    lens = torch.from_numpy(inp.seq_lens).cuda()
    w_uk, w_uv = dev(inp.w_uk), dev(inp.w_uv)
    B, Tq = wl.batch, wl.tq
    max_len = int(inp.seq_lens.max())
    splits = args.splits or api.num_splits(B, Tq, max_len)
    q_lat = torch.empty((B, Tq, 128, 512), dtype=torch.bfloat16, device="cuda")
    part_o = torch.empty((splits, B, Tq, 128, 512), dtype=torch.float32, device="cuda")
    part_lse = torch.empty((splits, B, Tq, 128), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Tq, 128, 128), dtype=torch.bfloat16, device="cuda")
    meta = {"seq_lens": inp.seq_lens}
    kv_tokens = int(inp.seq_lens.astype(np.int64).sum())
    del inp

    def step():
        api.absorb_q(q_c, w_uk, out=q_lat)
        api.decode_paged(q_lat, q_r, kv, table, lens, wl.scale, splits, part_o, part_lse)
        api.combine(part_o, part_lse, w_uv, out=out)

    if args.profile:
        for _ in range(args.warmup + args.steps):
            step()
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        if args.profile_all:
            bench_prefill(args.steps, args.warmup)
            bench_append(args.steps, args.warmup)
            bench_projections(args.steps, args.warmup)
            torch.cuda.synchronize()
        print(json.dumps({"profile": True, "steps": args.warmup + args.steps,
                          "kv_bytes_per_decode": kv_tokens * ROW_BYTES, "copy_bytes": 1 << 30,
                          "secondary": bool(args.profile_all)}))
        return

    for _ in range(args.warmup):
        step()
    # Timed steps: HIP events around each step; before each, outside the events,
    # a 512 MiB read evicts the 4 MB L2s and the 256 MB Infinity Cache, so no
    # step finds the previous step's weights or queries on chip.
    flush = _Flush()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for a, b in evs:
        flush()
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_step = float(step_ms.mean())
    del flush

    # The same step captured once in a HIP graph and replayed: one launch per
    # step instead of three host calls, so the host cannot leave the GPU idle
    # between kernels.  Same flush before each replay, outside the events.
    graph_ms = None
    try:
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            step()
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        flush = _Flush()
        for _ in range(args.warmup):
            graph.replay()
        gevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in gevs:
            flush()
            a.record()
            graph.replay()
            b.record()
        torch.cuda.synchronize()
        graph_ms = np.array([a.elapsed_time(b) for a, b in gevs])
        del flush, graph
    except RuntimeError as exc:          # capture unsupported: report eager only
        print(f"graph capture skipped: {exc}", file=sys.stderr)

    # Per-kernel launch durations, events on the stream the kernels run on,
    # each launch after the same cache-evicting read as the steps.
    kflush = _Flush()

    def time_kernel(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            kflush()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    n_k = max(5, args.steps)
    t_absorb = time_kernel(lambda: api.absorb_q(q_c, w_uk, out=q_lat), n_k)
    t_decode = time_kernel(lambda: api.decode_paged(q_lat, q_r, kv, table, lens, wl.scale, splits,
                                                    part_o, part_lse), n_k)
    t_combine = time_kernel(lambda: api.combine(part_o, part_lse, w_uv, out=out), n_k)
    # The shader clock the decode kernel runs at: the same kernel through the
    # library's clocked entry point (each work-group's clock cycles and 100 MHz
    # ticks, summed on the device), same flush before each launch.
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    t_clocked = time_kernel(lambda: api.decode_paged_clocked(q_lat, q_r, kv, table, lens, wl.scale,
                                                            splits, part_o, part_lse, clk), n_k)
    cyc, ticks = (int(v) for v in clk.cpu())
    clock_ghz = 0.1 * cyc / ticks if ticks else None
    del kflush

    kv_bytes = kv_tokens * ROW_BYTES
    weight_bytes = 2 * 128 * 128 * 512 * 2
    q_bytes = B * Tq * 128 * (128 + 64) * 2
    out_bytes = B * Tq * 128 * 128 * 2
    step_bytes = kv_bytes + weight_bytes + q_bytes + out_bytes
    flops = kv_tokens * Tq * FLOP_PER_TOKEN_QUERY + 2 * B * Tq * 128 * 2 * 128 * 512
    value = kv_tokens / (ms_step * 1e-3)
    decode_flops = kv_tokens * Tq * FLOP_PER_TOKEN_QUERY
    mfma_floor_us = (decode_flops / (BF16_FLOP_PER_CLOCK * clock_ghz * 1e9) * 1e6
                     if clock_ghz else None)
    achieved = kv_bytes / (t_decode * 1e-3) / 1e9
    traffic = measured_traffic(api.library_path())
    probe_gbs = read_probe(kv_bytes)
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_step_p10_p50_p90": [float(np.percentile(step_ms, q)) for q in (10, 50, 90)],
        "ms_per_step_graph": None if graph_ms is None else float(graph_ms.mean()),
        "ms_step_graph_p10_p50_p90": None if graph_ms is None else
        [float(np.percentile(graph_ms, q)) for q in (10, 50, 90)],
        "flush_between_steps_bytes": FLUSH_BYTES,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.note}", "batch": B, "query_tokens": Tq,
                   "seq_len": max_len, "heads": 128, "latent": 512, "rope": 64, "head_dim": 128,
                   "block_size": 64, "splits": splits, "kv_tokens": kv_tokens},
        "tflops": flops / (ms_step * 1e-3) / 1e12,
        "step_hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "step_mfma_frac": flops / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "kernels_ms": {"absorb_q": t_absorb, "decode_paged": t_decode, "combine": t_combine},
        "roofline": {
            "kernel": "decode_paged_kernel",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
            "mfma_tflops": decode_flops / (t_decode * 1e-3) / 1e12,
            "clock_ghz": clock_ghz,
            "clocked_launch_ms": t_clocked,
            "mfma_floor_us_at_clock": mfma_floor_us,
            "mfma_frac_at_clock": (mfma_floor_us / (t_clocked * 1e3)) if mfma_floor_us else None,
            "read_probe_gbs": probe_gbs,
            "frac_of_read_probe": achieved / probe_gbs,
        },
        "wall_s": wall,
        "input_gen_s": gen_s,
    }
    res["decode_configs"] = bench_decode_configs(max(5, args.steps // 4), 3)
    res["prefill"] = bench_prefill(max(3, args.steps // 4), 2)
    res["cache_append"] = bench_append(max(5, args.steps // 2), 3)
    res["projections"] = bench_projections(max(5, args.steps // 2), 3)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, meta, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
