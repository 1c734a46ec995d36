"""Thin torch binding over libmla.so.

Every function here only checks shapes, dtypes and devices, then passes raw
device pointers and the current HIP stream to the C ABI (include/mla.h).  All
arithmetic runs in the library's HIP kernels; nothing here computes, and there
is no fallback: if the library is missing or a call fails, an exception is
raised.

bf16 tensors are torch.bfloat16 (bit-identical to the ABI's uint16 patterns).
"""

import ctypes
import os

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")
_lib = None

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_HIP = 0, 1, 2, 3
MLA_ERR_NOALLOC_LIMIT = 4
MLA_MAX_SPLITS = 256
MLA_NOALLOC_MAX_PAIRS = 640

# Shapes the kernels are written for.
H, D_C, D_R, D_H, D_V, BLOCK = 128, 512, 64, 128, 128, 64

EXPORTED = (
    "mla_strerror", "mla_version", "mla_absorb_q", "mla_decode_paged", "mla_combine",
    "mla_prefill", "mla_decode_workspace_bytes", "mla_decode_part_o_bytes",
    "mla_decode_part_lse_bytes",
    "mla_prefill_workspace_bytes", "mla_decode_num_splits", "mla_cache_append",
    "mla_cache_append_workspace_bytes", "mla_query_project", "mla_query_project_workspace_bytes",
    "mla_output_project", "mla_output_project_workspace_bytes", "mla_hbm_read_probe",
    "mla_decode_noalloc", "mla_decode_paged_clocked",
)


# Debug mode: host checks of the device-resident metadata (block table and
# sequence lengths) before each call that reads it.  They copy the metadata to
# the host, a synchronisation, so they are off unless MLA_DEBUG is set (or
# set_debug(True) is called).
_debug = os.environ.get("MLA_DEBUG", "0") not in ("", "0")


def set_debug(on):
    """Turn the host-side metadata checks on or off; returns the previous setting."""
    global _debug
    prev, _debug = _debug, bool(on)
    return prev


def debug_enabled():
    return _debug


def check_paged_metadata(block_table, seq_lens, num_blocks, n_query, block_size=BLOCK):
    """Host check of the preconditions the library documents but cannot check
    without a synchronisation ("Teardown: DeepSeek-V3", section 12: the latent
    cache of one tenant must stay isolated from another's):

    * n_query <= L_b <= max_blocks * block_size for every sequence b
      (n_query = Tq in decode, T in prefill: the query tokens are cached);
    * 0 <= block_table[b, p] < num_blocks for every page p < ceil(L_b / block_size)
      a sequence uses;
    * no physical block is used twice (by two sequences, or twice by one).

    Accepts numpy arrays or torch tensors on any device (device tensors are
    copied to the host).  Raises ValueError naming the first violation.
    """
    def host(a):
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
        return np.asarray(a)

    table = host(block_table)
    lens = host(seq_lens)
    if table.ndim != 2 or lens.ndim != 1 or table.shape[0] != lens.shape[0]:
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    cap = table.shape[1] * block_size
    bad = np.nonzero((lens < n_query) | (lens > cap))[0]
    if bad.size:
        b = int(bad[0])
        raise ValueError(f"sequence {b}: seq_len {int(lens[b])} outside [{n_query}, {cap}] "
                         f"(query tokens .. max_blocks_per_seq * block_size)")
    pages = (lens.astype(np.int64) + block_size - 1) // block_size
    used = np.arange(table.shape[1])[None, :] < pages[:, None]
    ids = table.astype(np.int64)[used]
    owner = np.nonzero(used)[0]
    out = np.nonzero((ids < 0) | (ids >= num_blocks))[0]
    if out.size:
        k = int(out[0])
        raise ValueError(f"sequence {int(owner[k])}: block id {int(ids[k])} of a used page "
                         f"outside [0, {num_blocks})")
    uniq, first, counts = np.unique(ids, return_index=True, return_counts=True)
    if np.any(counts > 1):
        blk = int(uniq[np.argmax(counts > 1)])
        seqs = sorted({int(o) for o in owner[ids == blk]})
        raise ValueError(f"block {blk} is used more than once (sequences {seqs}): "
                         f"a page may belong to one sequence position only")


class MLAError(RuntimeError):
    """A non-zero status from libmla.so."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {strerror(status)}")


def library_path():
    return _LIB_PATH


def load():
    """Load libmla.so (once) and declare the ABI's argument types."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m mla_latent_kv_19_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.mla_strerror.argtypes, lib.mla_strerror.restype = [I], ctypes.c_char_p
    lib.mla_version.argtypes, lib.mla_version.restype = [], I
    lib.mla_absorb_q.argtypes = [P, P, P, I, I, I, I, P]
    lib.mla_decode_paged.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, P, P]
    lib.mla_combine.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P]
    lib.mla_prefill.argtypes = [P, P, P, P, P, P, P, P, P, Z, I, I, I, I, I, I, I, I, I, I, F, P]
    lib.mla_decode_paged_clocked.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, P, P, P]
    lib.mla_decode_paged_clocked.restype = I
    lib.mla_decode_noalloc.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, P]
    for fn in ("mla_absorb_q", "mla_decode_paged", "mla_combine", "mla_prefill",
               "mla_decode_noalloc"):
        getattr(lib, fn).restype = I
    lib.mla_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.mla_decode_workspace_bytes.restype = Z
    lib.mla_decode_part_o_bytes.argtypes, lib.mla_decode_part_o_bytes.restype = [I, I, I, I, I], Z
    lib.mla_decode_part_lse_bytes.argtypes, lib.mla_decode_part_lse_bytes.restype = [I, I, I, I], Z
    lib.mla_prefill_workspace_bytes.argtypes = [ctypes.c_long, I, I, I]
    lib.mla_prefill_workspace_bytes.restype = Z
    lib.mla_decode_num_splits.argtypes, lib.mla_decode_num_splits.restype = [I, I, I, I, I, I], I
    lib.mla_cache_append.argtypes = [P, P, P, P, P, P, P, P, Z, I, I, I, I, I, I, I, F, F, P]
    lib.mla_cache_append.restype = I
    lib.mla_cache_append_workspace_bytes.argtypes = [I, I]
    lib.mla_cache_append_workspace_bytes.restype = Z
    lib.mla_query_project.argtypes = [P, P, P, P, P, P, P, P, Z, I, I, I, I, I, I, F, F, P]
    lib.mla_query_project.restype = I
    lib.mla_query_project_workspace_bytes.argtypes = [I, I, I]
    lib.mla_query_project_workspace_bytes.restype = Z
    lib.mla_output_project.argtypes = [P, P, P, P, Z, I, I, I, P]
    lib.mla_hbm_read_probe.argtypes = [P, Z, P, P]
    lib.mla_output_project.restype = I
    lib.mla_output_project_workspace_bytes.argtypes = [I, I, I]
    lib.mla_output_project_workspace_bytes.restype = Z
    _lib = lib
    return lib


def strerror(status):
    return load().mla_strerror(int(status)).decode()


def _check(fn, status):
    if status != MLA_OK:
        raise MLAError(fn, status)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {devs}")
    return devs.pop()


def num_splits(batch, tq, max_seq_len, num_cus=None):
    """Split count that covers the GPU's compute units about once."""
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    s = load().mla_decode_num_splits(batch, tq, H, max_seq_len, BLOCK, num_cus)
    if s <= 0:
        raise ValueError("invalid arguments to mla_decode_num_splits")
    return s


def hbm_read_probe(buf, sink=None):
    """One read pass over the device tensor `buf` (16-byte aligned, a multiple of
    16 bytes long) with the library's HBM read probe; returns the 4-byte sink."""
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    dev = _same_device(buf, sink)
    _check("mla_hbm_read_probe", load().mla_hbm_read_probe(_ptr(buf), nbytes, _ptr(sink),
                                                            _stream(dev)))
    return sink


def absorb_q(q_c, w_uk, out=None):
    """q_lat[m, h, :] = q_c[m, h, :] @ w_uk[h]; q_c [..., H, 128] -> [..., H, 512] bf16."""
    lead = q_c.shape[:-2]
    m = 1
    for d in lead:
        m *= d
    _need(q_c, "q_c", torch.bfloat16, (*lead, H, D_H))
    _need(w_uk, "w_uk", torch.bfloat16, (H, D_H, D_C))
    if out is None:
        out = torch.empty((*lead, H, D_C), dtype=torch.bfloat16, device=q_c.device)
    _need(out, "out", torch.bfloat16, (*lead, H, D_C))
    dev = _same_device(q_c, w_uk, out)
    _check("mla_absorb_q", load().mla_absorb_q(_ptr(q_c), _ptr(w_uk), _ptr(out), m, H, D_H, D_C,
                                                _stream(dev)))
    return out


def decode_paged(q_lat, q_r, kv_cache, block_table, seq_lens, softmax_scale, splits,
                 part_o=None, part_lse=None):
    """Split-KV decode; returns (part_o [S,B,Tq,H,512] fp32, part_lse [S,B,Tq,H] fp32)."""
    b, tq = q_lat.shape[0], q_lat.shape[1]
    _need(q_lat, "q_lat", torch.bfloat16, (b, tq, H, D_C))
    _need(q_r, "q_r", torch.bfloat16, (b, tq, H, D_R))
    if kv_cache.dim() != 3 or kv_cache.shape[1:] != (BLOCK, D_C + D_R):
        raise ValueError(f"kv_cache must be [num_blocks, {BLOCK}, {D_C + D_R}]")
    _need(kv_cache, "kv_cache", torch.bfloat16)
    if block_table.dim() != 2 or block_table.shape[0] != b:
        raise ValueError("block_table must be [B, max_blocks]")
    _need(block_table, "block_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32, (b,))
    if part_o is None:
        part_o = torch.empty((splits, b, tq, H, D_C), dtype=torch.float32, device=q_lat.device)
    if part_lse is None:
        part_lse = torch.empty((splits, b, tq, H), dtype=torch.float32, device=q_lat.device)
    _need(part_o, "part_o", torch.float32, (splits, b, tq, H, D_C))
    _need(part_lse, "part_lse", torch.float32, (splits, b, tq, H))
    dev = _same_device(q_lat, q_r, kv_cache, block_table, seq_lens, part_o, part_lse)
    if _debug:
        check_paged_metadata(block_table, seq_lens, kv_cache.shape[0], tq)
    _check("mla_decode_paged", load().mla_decode_paged(
        _ptr(q_lat), _ptr(q_r), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
        b, tq, H, D_C, D_R, kv_cache.shape[0], BLOCK, block_table.shape[1],
        ctypes.c_float(softmax_scale), splits, _ptr(part_o), _ptr(part_lse), _stream(dev)))
    return part_o, part_lse


def decode_paged_clocked(q_lat, q_r, kv_cache, block_table, seq_lens, softmax_scale, splits,
                         part_o, part_lse, clock_sums):
    """decode_paged (same kernel) that also adds its work-groups' shader-clock
    cycles and 100 MHz ticks to clock_sums (int64 [2] on the device)."""
    b, tq = q_lat.shape[0], q_lat.shape[1]
    _need(clock_sums, "clock_sums", torch.int64, (2,))
    _need(part_o, "part_o", torch.float32, (splits, b, tq, H, D_C))
    _need(part_lse, "part_lse", torch.float32, (splits, b, tq, H))
    dev = _same_device(q_lat, q_r, kv_cache, block_table, seq_lens, part_o, part_lse, clock_sums)
    _check("mla_decode_paged_clocked", load().mla_decode_paged_clocked(
        _ptr(q_lat), _ptr(q_r), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
        b, tq, H, D_C, D_R, kv_cache.shape[0], BLOCK, block_table.shape[1],
        ctypes.c_float(softmax_scale), splits, _ptr(part_o), _ptr(part_lse), _ptr(clock_sums),
        _stream(dev)))
    return clock_sums


def combine(part_o, part_lse, w_uv, out=None, lse_out=None, want_lse=False):
    """Merge splits and apply W_UV; returns out [B,Tq,H,128] bf16 (and lse [B,Tq,H] fp32)."""
    s, b, tq = part_o.shape[0], part_o.shape[1], part_o.shape[2]
    _need(part_o, "part_o", torch.float32, (s, b, tq, H, D_C))
    _need(part_lse, "part_lse", torch.float32, (s, b, tq, H))
    _need(w_uv, "w_uv", torch.bfloat16, (H, D_C, D_V))
    if out is None:
        out = torch.empty((b, tq, H, D_V), dtype=torch.bfloat16, device=part_o.device)
    _need(out, "out", torch.bfloat16, (b, tq, H, D_V))
    if want_lse and lse_out is None:
        lse_out = torch.empty((b, tq, H), dtype=torch.float32, device=part_o.device)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, (b, tq, H))
    dev = _same_device(part_o, part_lse, w_uv, out, lse_out)
    _check("mla_combine", load().mla_combine(
        _ptr(part_o), _ptr(part_lse), _ptr(w_uv), _ptr(out), _ptr(lse_out),
        b, tq, H, D_C, D_V, s, _stream(dev)))
    return (out, lse_out) if lse_out is not None else out


def decode_noalloc(q_lat, q_r, kv_cache, block_table, seq_lens, w_uv, softmax_scale, splits,
                   out, lse_out=None):
    """mla_decode_paged + mla_combine with the split partials in the library's
    own device buffer (no allocation by the library; `out` and `lse_out` are
    the caller's).  Requires splits * B * Tq <= MLA_NOALLOC_MAX_PAIRS."""
    b, tq = q_lat.shape[0], q_lat.shape[1]
    _need(q_lat, "q_lat", torch.bfloat16, (b, tq, H, D_C))
    _need(q_r, "q_r", torch.bfloat16, (b, tq, H, D_R))
    if kv_cache.dim() != 3 or kv_cache.shape[1:] != (BLOCK, D_C + D_R):
        raise ValueError(f"kv_cache must be [num_blocks, {BLOCK}, {D_C + D_R}]")
    _need(kv_cache, "kv_cache", torch.bfloat16)
    if block_table.dim() != 2 or block_table.shape[0] != b:
        raise ValueError("block_table must be [B, max_blocks]")
    _need(block_table, "block_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32, (b,))
    _need(w_uv, "w_uv", torch.bfloat16, (H, D_C, D_V))
    _need(out, "out", torch.bfloat16, (b, tq, H, D_V))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, (b, tq, H))
    dev = _same_device(q_lat, q_r, kv_cache, block_table, seq_lens, w_uv, out, lse_out)
    if _debug:
        check_paged_metadata(block_table, seq_lens, kv_cache.shape[0], tq)
    _check("mla_decode_noalloc", load().mla_decode_noalloc(
        _ptr(q_lat), _ptr(q_r), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens), _ptr(w_uv),
        _ptr(out), _ptr(lse_out), b, tq, H, D_C, D_R, D_V, kv_cache.shape[0], BLOCK,
        block_table.shape[1], ctypes.c_float(softmax_scale), splits, _stream(dev)))
    return out


def decode_step(q_c, q_r, kv_cache, block_table, seq_lens, w_uk, w_uv, softmax_scale,
                splits=None, max_seq_len=None, want_lse=False, workspace=None):
    """One full decode step: absorb -> split-KV attention -> combine + W_UV.

    q_c [B, Tq, H, 128], q_r [B, Tq, H, 64] bf16.  ``max_seq_len`` (a host
    int) picks the split count when ``splits`` is not given; it avoids reading
    seq_lens back from the device.  ``workspace`` may hold preallocated
    (q_lat, part_o, part_lse) tensors.
    """
    b, tq = q_c.shape[0], q_c.shape[1]
    if splits is None:
        if max_seq_len is None:
            max_seq_len = block_table.shape[1] * BLOCK
        splits = num_splits(b, tq, max_seq_len)
    if workspace is None:
        q_lat = absorb_q(q_c, w_uk)
        part_o = part_lse = None
    else:
        q_lat, part_o, part_lse = workspace
        absorb_q(q_c, w_uk, out=q_lat)
    part_o, part_lse = decode_paged(q_lat, q_r, kv_cache, block_table, seq_lens, softmax_scale,
                                    splits, part_o, part_lse)
    return combine(part_o, part_lse, w_uv, want_lse=want_lse)


def prefill_workspace_bytes(batch, max_blocks_per_seq):
    return load().mla_prefill_workspace_bytes(batch * max_blocks_per_seq * BLOCK, H, D_H, D_V)


def decode_workspace_bytes(batch, tq, splits):
    """Bytes of one buffer holding part_o then part_lse (see decode_workspace)."""
    return load().mla_decode_workspace_bytes(batch, tq, H, D_C, splits)


def decode_workspace(batch, tq, splits, device=None):
    """(part_o [S,B,Tq,H,512], part_lse [S,B,Tq,H]) fp32 views of one device
    buffer laid out as mla_decode_workspace_bytes describes."""
    nbytes = decode_workspace_bytes(batch, tq, splits)
    if nbytes <= 0:
        raise ValueError("invalid decode workspace shape")
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device=device or "cuda")
    n_o = splits * batch * tq * H * D_C
    off = (n_o * 4 + 255) // 256 * 64
    part_o = buf[:n_o].view(splits, batch, tq, H, D_C)
    part_lse = buf[off:off + splits * batch * tq * H].view(splits, batch, tq, H)
    return part_o, part_lse


def prefill(q_c, q_r, kv_cache, block_table, seq_lens, w_uk, w_uv, softmax_scale,
            out=None, workspace=None):
    """Causal prefill over the cache; q for the last T positions of each sequence."""
    b, t = q_c.shape[0], q_c.shape[1]
    _need(q_c, "q_c", torch.bfloat16, (b, t, H, D_H))
    _need(q_r, "q_r", torch.bfloat16, (b, t, H, D_R))
    _need(kv_cache, "kv_cache", torch.bfloat16)
    _need(block_table, "block_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32, (b,))
    _need(w_uk, "w_uk", torch.bfloat16, (H, D_H, D_C))
    _need(w_uv, "w_uv", torch.bfloat16, (H, D_C, D_V))
    if out is None:
        out = torch.empty((b, t, H, D_V), dtype=torch.bfloat16, device=q_c.device)
    _need(out, "out", torch.bfloat16, (b, t, H, D_V))
    nbytes = prefill_workspace_bytes(b, block_table.shape[1])
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q_c.device)
    if workspace.numel() < nbytes:
        raise ValueError(f"prefill workspace needs {nbytes} bytes")
    dev = _same_device(q_c, q_r, kv_cache, block_table, seq_lens, w_uk, w_uv, out, workspace)
    if _debug:
        check_paged_metadata(block_table, seq_lens, kv_cache.shape[0], t)
    _check("mla_prefill", load().mla_prefill(
        _ptr(q_c), _ptr(q_r), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
        _ptr(w_uk), _ptr(w_uv), _ptr(out), _ptr(workspace), workspace.numel(),
        b, t, H, D_C, D_R, D_H, D_V, kv_cache.shape[0], BLOCK, block_table.shape[1],
        ctypes.c_float(softmax_scale), _stream(dev)))
    return out


def cache_append_workspace_bytes(m, d_model):
    return load().mla_cache_append_workspace_bytes(m, d_model)


def cache_append(x, w_kv, gamma, seq_idx, positions, block_table, kv_cache, eps=1e-6,
                 rope_theta=10000.0, workspace=None):
    """Write the cache rows (RMSNorm(latent) | RoPE(rotary key)) of M new tokens.

    x [M, d_model] bf16, w_kv [576, d_model] bf16, gamma [512] bf16, seq_idx and
    positions [M] int32; kv_cache is updated in place.
    """
    m, d_model = x.shape
    _need(x, "x", torch.bfloat16)
    _need(w_kv, "w_kv", torch.bfloat16, (D_C + D_R, d_model))
    _need(gamma, "gamma", torch.bfloat16, (D_C,))
    _need(seq_idx, "seq_idx", torch.int32, (m,))
    _need(positions, "positions", torch.int32, (m,))
    _need(block_table, "block_table", torch.int32)
    _need(kv_cache, "kv_cache", torch.bfloat16)
    nbytes = cache_append_workspace_bytes(m, d_model)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    if workspace.numel() < nbytes:
        raise ValueError(f"cache append workspace needs {nbytes} bytes")
    dev = _same_device(x, w_kv, gamma, seq_idx, positions, block_table, kv_cache, workspace)
    _check("mla_cache_append", load().mla_cache_append(
        _ptr(x), _ptr(w_kv), _ptr(gamma), _ptr(seq_idx), _ptr(positions), _ptr(block_table),
        _ptr(kv_cache), _ptr(workspace), workspace.numel(), m, d_model, D_C, D_R,
        kv_cache.shape[0], BLOCK, block_table.shape[1], ctypes.c_float(eps),
        ctypes.c_float(rope_theta), _stream(dev)))
    return kv_cache


def query_project(x, w_dq, gamma_q, w_uq, positions, eps=1e-6, rope_theta=10000.0,
                  q_c=None, q_r=None, workspace=None):
    """(q_c [M, H, 128], q_r [M, H, 64]) bf16 of M tokens: W_DQ, RMSNorm, W_UQ, RoPE."""
    m, d_model = x.shape
    q_rank = w_dq.shape[0]
    _need(x, "x", torch.bfloat16)
    _need(w_dq, "w_dq", torch.bfloat16, (q_rank, d_model))
    _need(gamma_q, "gamma_q", torch.bfloat16, (q_rank,))
    _need(w_uq, "w_uq", torch.bfloat16, (H * (D_H + D_R), q_rank))
    _need(positions, "positions", torch.int32, (m,))
    if q_c is None:
        q_c = torch.empty((m, H, D_H), dtype=torch.bfloat16, device=x.device)
    if q_r is None:
        q_r = torch.empty((m, H, D_R), dtype=torch.bfloat16, device=x.device)
    _need(q_c, "q_c", torch.bfloat16, (m, H, D_H))
    _need(q_r, "q_r", torch.bfloat16, (m, H, D_R))
    nbytes = load().mla_query_project_workspace_bytes(m, d_model, q_rank)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    if workspace.numel() < nbytes:
        raise ValueError(f"query projection workspace needs {nbytes} bytes")
    dev = _same_device(x, w_dq, gamma_q, w_uq, positions, q_c, q_r, workspace)
    _check("mla_query_project", load().mla_query_project(
        _ptr(x), _ptr(w_dq), _ptr(gamma_q), _ptr(w_uq), _ptr(positions), _ptr(q_c), _ptr(q_r),
        _ptr(workspace), workspace.numel(), m, d_model, q_rank, H, D_H, D_R, ctypes.c_float(eps),
        ctypes.c_float(rope_theta), _stream(dev)))
    return q_c, q_r


def output_project(o, w_o, y=None, workspace=None):
    """y [M, d_out] bf16 = o [M, d_in] W_O^T."""
    m, d_in = o.shape
    d_out = w_o.shape[0]
    _need(o, "o", torch.bfloat16)
    _need(w_o, "w_o", torch.bfloat16, (d_out, d_in))
    if y is None:
        y = torch.empty((m, d_out), dtype=torch.bfloat16, device=o.device)
    _need(y, "y", torch.bfloat16, (m, d_out))
    nbytes = load().mla_output_project_workspace_bytes(m, d_in, d_out)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=o.device)
    if workspace.numel() < nbytes:
        raise ValueError(f"output projection workspace needs {nbytes} bytes")
    dev = _same_device(o, w_o, y, workspace)
    _check("mla_output_project", load().mla_output_project(
        _ptr(o), _ptr(w_o), _ptr(y), _ptr(workspace), workspace.numel(), m, d_in, d_out,
        _stream(dev)))
    return y
