"""Python binding of the lnf4 C ABI (include/lnf4.h): same names, argument marshalling only.

Every entry point forwards to liblnf4.so through ctypes.  Tensors are passed as raw
device (or pinned host) addresses; streams as hipStream_t handles taken from
``torch.cuda.Stream``.  A non-zero status raises :class:`LNF4Error` with the library's
message.  Nothing here computes: all work runs in the HIP kernels of liblnf4.so, and a
missing library is an error (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LNF4_LIB") or os.path.join(_HERE, "liblnf4.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "lnf4.h")

LNF4_OK = 0
LNF4_EINVAL = -1
LNF4_ESHAPE = -2
LNF4_EALIGN = -3
LNF4_EHIP = -4
LNF4_ESTATE = -5
FMT_NF4 = 0
FMT_BF16 = 1
MAX_RANK = 64
MAX_GROUP = 8
EV_COPY, EV_STEP, EV_SLOT_COPY, EV_SLOT_WAIT = 0, 1, 2, 3
STREAM_RING, STREAM_RESIDENT, STREAM_REUSE = 0, 1, 2

_ERRNAMES = {LNF4_EINVAL: "EINVAL", LNF4_ESHAPE: "ESHAPE", LNF4_EALIGN: "EALIGN", LNF4_EHIP: "EHIP",
             LNF4_ESTATE: "ESTATE"}


class LNF4Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERRNAMES.get(code, code)}: {msg}")
        self.code = code


class lnf4_weight(ctypes.Structure):
    _fields_ = [("fmt", c_int32), ("data", c_void_p), ("absmax", c_void_p), ("out_f", c_int64),
                ("in_f", c_int64), ("blocksize", c_int32)]


class lnf4_proj(ctypes.Structure):
    _fields_ = [("W", lnf4_weight), ("A", c_void_p), ("B", c_void_p), ("r", c_int32), ("scale", c_float),
                ("y", c_void_p), ("u", c_void_p), ("dy", c_void_p), ("dA", c_void_p), ("dB", c_void_p)]


class lnf4_stream_event(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("call", c_int32), ("j", c_int32), ("layer", c_int32), ("buffer", c_int32),
                ("wait", c_int32)]

    def astuple(self):
        return (self.kind, self.call, self.j, self.layer, self.buffer, self.wait)


_lib = None


def _declare(L):
    vp, i32, i64, sz, f32 = c_void_p, c_int32, c_int64, c_size_t, c_float
    sig = {
        "lnf4_last_error": (c_char_p, []),
        "lnf4_version": (c_char_p, []),
        "lnf4_nf4_table": (i32, [POINTER(c_float)]),
        "nf4_dequant": (i32, [vp, vp, i64, i32, vp, vp]),
        "nf4_quantize": (i32, [vp, i64, i32, vp, vp, vp]),
        "lora_linear_fwd": (i32, [POINTER(lnf4_weight), vp, i64, vp, vp, i32, f32, vp, vp, vp]),
        "lora_linear_bwd_workspace": (sz, [i64, i64, i64, i32]),
        "lora_linear_bwd": (i32, [POINTER(lnf4_weight), vp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, i32, vp,
                                  sz, vp]),
        "lora_linear_bwd_noalloc": (i32, [POINTER(lnf4_weight), vp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, i32,
                                          vp]),
        "lora_group_fwd": (i32, [POINTER(lnf4_proj), i32, vp, i64, i32, vp]),
        "lora_group_fwd_workspace": (sz, [POINTER(lnf4_proj), i32, i64]),
        "lora_group_fwd_ws": (i32, [POINTER(lnf4_proj), i32, vp, i64, i32, vp, sz, vp]),
        "lora_group_bwd_workspace": (sz, [POINTER(lnf4_proj), i32, i64]),
        "lora_group_bwd": (i32, [POINTER(lnf4_proj), i32, vp, i64, vp, i32, vp, sz, vp]),
        "lnf4_shard_layout": (i32, [i32, POINTER(c_int64), POINTER(c_int64), i32, POINTER(c_int64),
                                    POINTER(c_int64)]),
        "lnf4_embed_gather": (i32, [vp, i64, i64, vp, i64, vp, vp]),
        "lnf4_cross_entropy": (i32, [vp, i64, i64, vp, f32, vp, i64, vp, vp, vp]),
        "lnf4_sequence_sums": (i32, [vp, i32, i64, vp, vp]),
        "lnf4_dpo_loss": (i32, [vp, vp, i32, f32, vp, vp, vp]),
        "lnf4_rmsnorm_fwd": (i32, [vp, i64, i64, vp, f32, vp, vp, vp]),
        "lnf4_rmsnorm_bwd": (i32, [vp, i64, i64, vp, vp, vp, vp, vp, vp]),
        "lnf4_rope_table": (i32, [i64, i32, ctypes.c_double, vp, vp]),
        "lnf4_rope": (i32, [vp, i64, i32, i32, i64, vp, i32, vp]),
        "lnf4_swiglu_fwd": (i32, [vp, vp, i64, vp, vp]),
        "lnf4_swiglu_bwd": (i32, [vp, vp, vp, i64, vp, vp, vp]),
        "lnf4_add": (i32, [vp, vp, i64, vp, vp]),
        "lnf4_attn_fwd": (i32, [vp, vp, vp, i64, i32, i32, i32, i64, vp, vp, vp]),
        "lnf4_attn_bwd": (i32, [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i64, vp, vp, vp, vp, sz, vp]),
        "lnf4_attn_bwd_workspace": (sz, [i64, i32, i32, i32]),
        "stream_compute_stream": (i32, [i32, POINTER(c_void_p)]),
        "stream_copy_stream": (i32, [i32, POINTER(c_void_p)]),
        "stream_create": (i32, [POINTER(c_void_p), POINTER(c_size_t), i32, POINTER(c_void_p), sz, i32,
                                POINTER(c_int32), i32, i32, vp, vp, sz, POINTER(c_void_p)]),
        "stream_layer_step": (i32, [vp, i32, vp, POINTER(c_void_p)]),
        "stream_slot_load": (i32, [vp, i32, vp]),
        "stream_slot_load_part": (i32, [vp, i32, i32, i32, vp]),
        "stream_slot_wait": (i32, [vp, vp, POINTER(c_void_p)]),
        "stream_reset": (i32, [vp, vp]),
        "stream_log": (i32, [vp, POINTER(lnf4_stream_event), i32, POINTER(c_int32)]),
        "stream_bytes_copied": (i32, [vp, POINTER(c_int64)]),
        "stream_create_disk": (i32, [ctypes.c_char_p, POINTER(c_int64), i32, POINTER(c_void_p), sz, i32,
                                     POINTER(c_void_p), POINTER(c_size_t), i32, POINTER(c_void_p), sz, i32,
                                     POINTER(c_int32), i32, vp, vp, sz, POINTER(c_void_p)]),
        "stream_disk_stats": (i32, [vp, POINTER(c_int64), POINTER(ctypes.c_double)]),
        "stream_destroy": (i32, [vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded liblnf4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c \"import __graft_entry__ as g; "
                               f"g.build()\"` (hipcc, gfx950)")
        # torch brings its own HIP runtime; loading it first makes the library bind to that
        # same runtime (one HIP runtime per process), whatever the caller imported first
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/lnf4.h declares."""
    txt = open(HEADER_PATH).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]*)\s*\(", txt, flags=re.M)
    return sorted(set(n for n in names if n not in ("typedef",)))


# ------------------------------------------------------------------ marshalling helpers
def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc: int):
    if rc != LNF4_OK:
        raise LNF4Error(rc, lib().lnf4_last_error().decode())
    return rc


def lnf4_last_error() -> str:
    return lib().lnf4_last_error().decode()


def lnf4_version() -> str:
    return lib().lnf4_version().decode()


def lnf4_nf4_table():
    out = (c_float * 16)()
    _check(lib().lnf4_nf4_table(out))
    return [out[i] for i in range(16)]


def nf4_dequant(codes, absmax, n_elems: int, blocksize: int, out_bf16, stream=None):
    _check(lib().nf4_dequant(_ptr(codes), _ptr(absmax), n_elems, blocksize, _ptr(out_bf16), _stream(stream)))


def nf4_quantize(w, n_elems: int, blocksize: int, codes, absmax, stream=None):
    _check(lib().nf4_quantize(_ptr(w), n_elems, blocksize, _ptr(codes), _ptr(absmax), _stream(stream)))


def make_weight(fmt: int, data, absmax, out_f: int, in_f: int, blocksize: int = 64) -> lnf4_weight:
    return lnf4_weight(fmt, _ptr(data), _ptr(absmax), out_f, in_f, blocksize)


def lora_linear_fwd(W: lnf4_weight, x, T: int, A, B, r: int, scale: float, y, u, stream=None):
    _check(lib().lora_linear_fwd(ctypes.byref(W), _ptr(x), T, _ptr(A), _ptr(B), r, scale, _ptr(y), _ptr(u),
                                 _stream(stream)))


def lora_linear_bwd_workspace(T: int, out_f: int, in_f: int, r: int) -> int:
    return int(lib().lora_linear_bwd_workspace(T, out_f, in_f, r))


def lora_linear_bwd(W: lnf4_weight, x, dy, T: int, A, B, r: int, scale: float, u_saved, dx, dA, dB,
                    accumulate: int, workspace, ws_bytes: int, stream=None):
    _check(lib().lora_linear_bwd(ctypes.byref(W), _ptr(x), _ptr(dy), T, _ptr(A), _ptr(B), r, scale, _ptr(u_saved),
                                 _ptr(dx), _ptr(dA), _ptr(dB), accumulate, _ptr(workspace), ws_bytes,
                                 _stream(stream)))


def lora_linear_bwd_noalloc(W: lnf4_weight, x, dy, T: int, A, B, r: int, scale: float, u_saved, dx, dA, dB,
                            accumulate: int, stream=None):
    """lora_linear_bwd with the library's fixed scratch as its workspace (allocates nothing)."""
    _check(lib().lora_linear_bwd_noalloc(ctypes.byref(W), _ptr(x), _ptr(dy), T, _ptr(A), _ptr(B), r, scale,
                                         _ptr(u_saved), _ptr(dx), _ptr(dA), _ptr(dB), accumulate, _stream(stream)))


def make_proj(W: lnf4_weight, A=None, B=None, r: int = 0, scale: float = 0.0, y=None, u=None, dy=None, dA=None,
              dB=None) -> lnf4_proj:
    return lnf4_proj(W, _ptr(A), _ptr(B), r, scale, _ptr(y), _ptr(u), _ptr(dy), _ptr(dA), _ptr(dB))


def _proj_array(projs):
    arr = (lnf4_proj * len(projs))(*projs)
    return arr, len(projs)


def lora_group_fwd(projs, x, T: int, adapters_enabled: int = 1, stream=None):
    arr, n = _proj_array(projs)
    _check(lib().lora_group_fwd(arr, n, _ptr(x), T, adapters_enabled, _stream(stream)))


def lora_group_fwd_workspace(projs, T: int) -> int:
    arr, n = _proj_array(projs)
    return int(lib().lora_group_fwd_workspace(arr, n, T))


def lora_group_fwd_ws(projs, x, T: int, adapters_enabled: int, workspace, ws_bytes: int, stream=None):
    arr, n = _proj_array(projs)
    _check(lib().lora_group_fwd_ws(arr, n, _ptr(x), T, adapters_enabled, _ptr(workspace), ws_bytes,
                                   _stream(stream)))


def lora_group_bwd_workspace(projs, T: int) -> int:
    arr, n = _proj_array(projs)
    return int(lib().lora_group_bwd_workspace(arr, n, T))


def lora_group_bwd(projs, x, T: int, dx, accumulate: int, workspace, ws_bytes: int, stream=None):
    arr, n = _proj_array(projs)
    _check(lib().lora_group_bwd(arr, n, _ptr(x), T, _ptr(dx), accumulate, _ptr(workspace), ws_bytes,
                                _stream(stream)))


def lnf4_shard_layout(out_f, in_f, fmt: int):
    n = len(out_f)
    o = (c_int64 * n)(*out_f)
    i = (c_int64 * n)(*in_f)
    offs = (c_int64 * (2 * n))()
    total = c_int64()
    _check(lib().lnf4_shard_layout(n, o, i, fmt, offs, ctypes.byref(total)))
    return [offs[k] for k in range(2 * n)], total.value


# ------------------------------------------------------------------ output side
def lnf4_embed_gather(table, vocab: int, hidden: int, ids, T: int, out, stream=None):
    _check(lib().lnf4_embed_gather(_ptr(table), vocab, hidden, _ptr(ids), T, _ptr(out), _stream(stream)))


def lnf4_cross_entropy(logits, T: int, vocab: int, labels, grad_scale: float, seq_scale, rows_per_scale: int, logp,
                       dlogits, stream=None):
    _check(lib().lnf4_cross_entropy(_ptr(logits), T, vocab, _ptr(labels), grad_scale, _ptr(seq_scale),
                                    rows_per_scale, _ptr(logp), _ptr(dlogits), _stream(stream)))


def lnf4_sequence_sums(x, n_seq: int, seq_len: int, sums, stream=None):
    _check(lib().lnf4_sequence_sums(_ptr(x), n_seq, seq_len, _ptr(sums), _stream(stream)))


def lnf4_dpo_loss(pol_sums, ref_sums, n_pairs: int, beta: float, loss, coef, stream=None):
    _check(lib().lnf4_dpo_loss(_ptr(pol_sums), _ptr(ref_sums), n_pairs, beta, _ptr(loss), _ptr(coef),
                               _stream(stream)))


# ------------------------------------------------------------------ decoder-layer glue
def lnf4_rmsnorm_fwd(x, T: int, H: int, g, eps: float, y, rstd, stream=None):
    _check(lib().lnf4_rmsnorm_fwd(_ptr(x), T, H, _ptr(g), eps, _ptr(y), _ptr(rstd), _stream(stream)))


def lnf4_rmsnorm_bwd(x, T: int, H: int, g, rstd, dy, dres, dx, stream=None):
    _check(lib().lnf4_rmsnorm_bwd(_ptr(x), T, H, _ptr(g), _ptr(rstd), _ptr(dy), _ptr(dres), _ptr(dx),
                                  _stream(stream)))


def lnf4_rope_table(seq_len: int, head_dim: int, base: float, table, stream=None):
    _check(lib().lnf4_rope_table(seq_len, head_dim, base, _ptr(table), _stream(stream)))


def lnf4_rope(x, T: int, n_heads: int, head_dim: int, seq_len: int, table, inverse: int, stream=None):
    _check(lib().lnf4_rope(_ptr(x), T, n_heads, head_dim, seq_len, _ptr(table), inverse, _stream(stream)))


def lnf4_swiglu_fwd(g, u, n: int, s, stream=None):
    _check(lib().lnf4_swiglu_fwd(_ptr(g), _ptr(u), n, _ptr(s), _stream(stream)))


def lnf4_swiglu_bwd(g, u, ds, n: int, dg, du, stream=None):
    _check(lib().lnf4_swiglu_bwd(_ptr(g), _ptr(u), _ptr(ds), n, _ptr(dg), _ptr(du), _stream(stream)))


def lnf4_add(a, b, n: int, out, stream=None):
    _check(lib().lnf4_add(_ptr(a), _ptr(b), n, _ptr(out), _stream(stream)))


def lnf4_attn_fwd(q, k, v, T: int, n_heads: int, n_kv: int, head_dim: int, seq_len: int, o, lse, stream=None):
    _check(lib().lnf4_attn_fwd(_ptr(q), _ptr(k), _ptr(v), T, n_heads, n_kv, head_dim, seq_len, _ptr(o), _ptr(lse),
                               _stream(stream)))


def lnf4_attn_bwd_workspace(T: int, n_heads: int, n_kv: int, head_dim: int) -> int:
    return int(lib().lnf4_attn_bwd_workspace(T, n_heads, n_kv, head_dim))


def lnf4_attn_bwd(q, k, v, o, lse, dout, T: int, n_heads: int, n_kv: int, head_dim: int, seq_len: int, dq, dk, dv,
                  workspace, ws_bytes: int, stream=None):
    _check(lib().lnf4_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), T, n_heads, n_kv,
                               head_dim, seq_len, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                               _stream(stream)))


# ------------------------------------------------------------------ layer stream
_compute_streams = {}
_copy_streams = {}


def stream_compute_stream(device=None):
    """The library's compute stream of `device` (default: the current device) as a torch
    stream: a hardware queue of its own, so a copy stream never shares its queue; ordered
    with the null stream like a default-flag stream.  The same stream on every call."""
    import torch
    if isinstance(device, int):
        idx = device
    else:
        d = torch.device(device or "cuda")
        idx = d.index if d.index is not None else torch.cuda.current_device()
    s = _compute_streams.get(idx)
    if s is None:
        h = c_void_p()
        _check(lib().stream_compute_stream(idx, ctypes.byref(h)))
        s = torch.cuda.ExternalStream(h.value, device=torch.device("cuda", idx))
        _compute_streams[idx] = s
    return s


def stream_copy_stream(device=None):
    """The library's copy stream of `device` as a torch stream: like the compute stream, a
    hardware queue of its own, ordered with the null stream.  The same stream on every call."""
    import torch
    if isinstance(device, int):
        idx = device
    else:
        d = torch.device(device or "cuda")
        idx = d.index if d.index is not None else torch.cuda.current_device()
    s = _copy_streams.get(idx)
    if s is None:
        h = c_void_p()
        _check(lib().stream_copy_stream(idx, ctypes.byref(h)))
        s = torch.cuda.ExternalStream(h.value, device=torch.device("cuda", idx))
        _copy_streams[idx] = s
    return s


def stream_create(host_shards, shard_bytes, dev_bufs, buf_bytes: int, schedule, mode: int, copy_stream,
                  slot_buf=None, slot_bytes: int = 0):
    n = len(host_shards)
    hs = (c_void_p * n)(*[_ptr(h) for h in host_shards])
    sb = (c_size_t * n)(*shard_bytes)
    nb = len(dev_bufs)
    db = (c_void_p * nb)(*[_ptr(d) for d in dev_bufs])
    sc = (c_int32 * len(schedule))(*schedule)
    out = c_void_p()
    _check(lib().stream_create(hs, sb, n, db, buf_bytes, nb, sc, len(schedule), mode, _stream(copy_stream),
                               _ptr(slot_buf), slot_bytes, ctypes.byref(out)))
    return out.value


def stream_create_disk(path: str, file_offsets, stage_bufs, stage_bytes: int, shard_bytes, dev_bufs,
                       buf_bytes: int, schedule, copy_stream, host_shards=None, drop_cache: bool = False,
                       slot_buf=None, slot_bytes: int = 0):
    """Ring-mode layer stream whose layer shards are read from `path` through the pinned
    staging buffers (the read-ahead depth is len(stage_bufs)); see stream_create_disk in
    include/lnf4.h."""
    n = len(shard_bytes)
    fo = (c_int64 * n)(*file_offsets)
    ns = len(stage_bufs)
    stg = (c_void_p * ns)(*[_ptr(b) for b in stage_bufs])
    hs = None if host_shards is None else (c_void_p * n)(*[_ptr(h) for h in host_shards])
    sb = (c_size_t * n)(*shard_bytes)
    nb = len(dev_bufs)
    db = (c_void_p * nb)(*[_ptr(d) for d in dev_bufs])
    sc = (c_int32 * len(schedule))(*schedule)
    out = c_void_p()
    _check(lib().stream_create_disk(os.fsencode(path), fo, int(drop_cache), stg, stage_bytes, ns, hs, sb, n, db,
                                    buf_bytes, nb, sc, len(schedule), _stream(copy_stream), _ptr(slot_buf),
                                    slot_bytes, ctypes.byref(out)))
    return out.value


def stream_disk_stats(st):
    """(bytes read from the file, seconds the reader spent in reads)."""
    b, t = c_int64(), ctypes.c_double()
    _check(lib().stream_disk_stats(st, ctypes.byref(b), ctypes.byref(t)))
    return b.value, t.value


def stream_layer_step(st, k: int, compute=None) -> int:
    p = c_void_p()
    _check(lib().stream_layer_step(st, k, _stream(compute), ctypes.byref(p)))
    return p.value


def stream_slot_load(st, shard: int, compute=None):
    _check(lib().stream_slot_load(st, shard, _stream(compute)))


def stream_slot_load_part(st, shard: int, part: int, n_parts: int, compute=None):
    _check(lib().stream_slot_load_part(st, shard, part, n_parts, _stream(compute)))


def stream_slot_wait(st, compute=None) -> int:
    p = c_void_p()
    _check(lib().stream_slot_wait(st, _stream(compute), ctypes.byref(p)))
    return p.value


def stream_reset(st, compute=None):
    _check(lib().stream_reset(st, _stream(compute)))


def stream_log(st, cap: int = 1 << 16):
    ev = (lnf4_stream_event * cap)()
    n = c_int32()
    _check(lib().stream_log(st, ev, cap, ctypes.byref(n)))
    return [ev[i].astuple() for i in range(n.value)]


def stream_bytes_copied(st) -> int:
    b = c_int64()
    _check(lib().stream_bytes_copied(st, ctypes.byref(b)))
    return b.value


def stream_destroy(st):
    _check(lib().stream_destroy(st))
