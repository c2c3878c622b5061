"""Lossless BF16 codec for MI355X: exponent reuse across iterations (CIERA)
plus the sigma-windowed 3-bit exponent code (ZipCCL), in hand-written HIP.

This package is a thin binding over the C ABI in ``include/ciera.h``
(``libciera.so``, built in-tree by ``build.py``).  Every step of the codec
runs in the HIP kernels; the binding only checks tensor types and passes
device pointers, sizes and the current HIP stream.  PyTorch supplies device
memory and streams and nothing else.  If the library is not built, every
entry point raises: there is no fallback.

Same names as the C ABI::

    zip3_max_encoded_size(n)              ciera_max_encoded_size(n, B)
    zip3_workspace_size(n)                ciera_workspace_size(n, B)
    zip3_encode(x, out, ws, out_size, e0_override=-1, stream=None, plan_groups=0)
    zip3_decode(inp, in_size, y, ws, stream=None)
    zip3_encode_e0(x, e0_src, out, ws, out_size, e0_offset=0, stream=None)
    ciera_encode(x, B, prev_exp, out, ws, out_size, e0_override=-1, stream=None, plan_groups=0)
    ciera_encode_e0(x, B, prev_exp, e0_src, out, ws, out_size, e0_offset=0, stream=None)
    zip3_encode_spec(x, hint_src, out, ws, out_size, hint_offset=0, stream=None)   (one read of x if the hinted window is right)
    ciera_encode_spec(x, B, prev_exp, hint_src, out, ws, out_size, hint_offset=0, stream=None)
    ciera_encode_hashed(x, B, hash_cache, out, ws, out_size, stream=None)
    ciera_hash_cache_size(n, B)
    zip3_encode_rans / zip3_decode_rans / ciera_encode_rans / ciera_decode_rans   (rANS-coded exponents)
    rans_max_encoded_size(n, B), rans_workspace_size(n, B)
    ciera_decode(inp, in_size, y, B, prev_exp, ws, stream=None)
    zip3_decode_batch(inps, in_sizes, ys, ws, stream=None)     (several streams of one n, one launch)
    ciera_decode_batch(inps, in_sizes, ys, B, prev_exps, ws, stream=None)
    decode_batch_workspace_size(n, k)
    ciera_read_error(ws, stream=None)
    ciera_time_kernels(pairs)             (profiling: per-kernel start/stop events)
    ciera_set_wait_limit(polls)           (test hook: bound of the waits between workgroups)
    ciera_encode_noalloc(x, B, prev_exp, out, out_size, stream=None)   (no workspace: allocates nothing)

``x``/``y`` are CUDA(HIP) tensors of dtype bfloat16, int16 or uint16 holding
the BF16 patterns; ``out``/``inp``/``ws``/``prev_exp`` are uint8 tensors and
``out_size`` a one-element int64/uint64 tensor, all on the same device.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "CieraError", "library_path", "load_library",
    "zip3_max_encoded_size", "ciera_max_encoded_size", "zip3_workspace_size", "ciera_workspace_size",
    "zip3_encode", "zip3_decode", "ciera_encode", "ciera_decode", "ciera_read_error", "ciera_status_string",
    "zip3_encode_e0", "ciera_encode_e0", "ciera_encode_hashed", "ciera_hash_cache_size",
    "rans_max_encoded_size", "rans_workspace_size", "zip3_encode_rans", "zip3_decode_rans", "ciera_encode_rans",
    "ciera_decode_rans",
    "bind", "ciera_time_kernels", "ciera_set_wait_limit", "ciera_encode_noalloc", "NOALLOC_MAX_N",
    "decode_batch_workspace_size", "zip3_decode_batch", "ciera_decode_batch", "DECODE_BATCH_MAX",
    "zip3_encode_spec", "ciera_encode_spec",
    "CHUNK",
]

CHUNK = 65536
NOALLOC_MAX_N = 1 << 27
DECODE_BATCH_MAX = 16
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libciera.so")
_lib = None

STATUS_NAMES = {0: "CIERA_OK", 1: "CIERA_ERR_ARG", 2: "CIERA_ERR_CAPACITY", 3: "CIERA_ERR_WORKSPACE",
                4: "CIERA_ERR_HIP", 5: "CIERA_ERR_FORMAT", 6: "CIERA_ERR_INTERNAL"}
STATUS_CODES = {name: code for code, name in STATUS_NAMES.items()}


class CieraError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load ``libciera.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "or python -m lossless_bf16_tensor_exp_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    u64, u32, vp, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
    for name, args in [("zip3_max_encoded_size", [u64]), ("ciera_max_encoded_size", [u64, u32]),
                       ("zip3_workspace_size", [u64]), ("ciera_workspace_size", [u64, u32]),
                       ("ciera_hash_cache_size", [u64, u32]), ("rans_max_encoded_size", [u64, u32]),
                       ("rans_workspace_size", [u64, u32])]:
        f = getattr(lib, name)
        f.argtypes, f.restype = args, u64
    sigs = {
        "zip3_encode": [vp, u64, vp, u64, vp, u64, vp, vp],
        "zip3_encode_ex": [vp, u64, vp, u64, vp, u64, vp, i32, u32, vp],
        "zip3_encode_e0": [vp, u64, vp, vp, u64, vp, u64, vp, vp],
        "ciera_encode_e0": [vp, u64, u32, vp, vp, vp, u64, vp, u64, vp, vp],
        "zip3_encode_spec": [vp, u64, vp, vp, u64, vp, u64, vp, vp],
        "ciera_encode_spec": [vp, u64, u32, vp, vp, vp, u64, vp, u64, vp, vp],
        "zip3_decode": [vp, u64, vp, u64, vp, u64, vp],
        "ciera_encode": [vp, u64, u32, vp, vp, u64, vp, u64, vp, vp],
        "ciera_encode_ex": [vp, u64, u32, vp, vp, u64, vp, u64, vp, i32, u32, vp],
        "ciera_decode": [vp, u64, vp, u64, u32, vp, vp, u64, vp],
        "ciera_encode_hashed": [vp, u64, u32, vp, vp, u64, vp, u64, vp, vp],
        "zip3_encode_rans": [vp, u64, vp, u64, vp, u64, vp, vp],
        "zip3_decode_rans": [vp, u64, vp, u64, vp, u64, vp],
        "ciera_encode_rans": [vp, u64, u32, vp, vp, u64, vp, u64, vp, vp],
        "ciera_decode_rans": [vp, u64, vp, u64, u32, vp, vp, u64, vp],
        "ciera_read_error": [vp, vp],
        "ciera_time_kernels": [ctypes.POINTER(vp), u32],
        "ciera_encode_noalloc": [vp, u64, u32, vp, vp, u64, vp, vp],
    }
    for name, args in sigs.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = args, i32
    pvp, pu64 = ctypes.POINTER(vp), ctypes.POINTER(u64)
    lib.decode_batch_workspace_size.argtypes, lib.decode_batch_workspace_size.restype = [u64, u32], u64
    lib.zip3_decode_batch.argtypes, lib.zip3_decode_batch.restype = [u32, pvp, pu64, pvp, u64, vp, u64, vp], i32
    lib.ciera_decode_batch.argtypes = [u32, pvp, pu64, pvp, u64, u32, pvp, vp, u64, vp]
    lib.ciera_decode_batch.restype = i32
    lib.ciera_status_string.argtypes, lib.ciera_status_string.restype = [i32], ctypes.c_char_p
    lib.ciera_set_wait_limit.argtypes, lib.ciera_set_wait_limit.restype = [u32], u32
    _lib = lib
    return lib


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else None


def _check_values(x, name):
    torch = _torch()
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold BF16 patterns (bfloat16/int16/uint16), got {x.dtype}")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def _check_bytes(t, name, min_len=0):
    torch = _torch()
    if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous uint8 device tensor")
    if t.numel() < min_len:
        raise ValueError(f"{name} holds {t.numel()} bytes, needs {min_len}")


def _check_size_slot(t):
    torch = _torch()
    if t.dtype not in (torch.int64, torch.uint64) or t.numel() < 1 or not t.is_cuda:
        raise ValueError("out_size must be a one-element int64/uint64 device tensor")


def _raise(st, what):
    if st != 0:
        raise CieraError(st, what)


def zip3_max_encoded_size(n: int) -> int:
    return load_library().zip3_max_encoded_size(n)


def ciera_max_encoded_size(n: int, B: int) -> int:
    return load_library().ciera_max_encoded_size(n, B)


def zip3_workspace_size(n: int) -> int:
    return load_library().zip3_workspace_size(n)


def ciera_workspace_size(n: int, B: int) -> int:
    return load_library().ciera_workspace_size(n, B)


def ciera_status_string(status: int) -> str:
    return load_library().ciera_status_string(status).decode()


def zip3_encode(x, out, ws, out_size, e0_override: int = -1, stream=None, plan_groups: int = 0) -> None:
    lib = load_library()
    _check_values(x, "x")
    _check_bytes(out, "out")
    _check_bytes(ws, "ws")
    _check_size_slot(out_size)
    st = lib.zip3_encode_ex(_ptr(x), x.numel(), _ptr(out), out.numel(), _ptr(ws), ws.numel(),
                            ctypes.c_void_p(out_size.data_ptr()), e0_override, plan_groups, _stream(stream))
    _raise(st, "zip3_encode")


def zip3_encode_e0(x, e0_src, out, ws, out_size, e0_offset: int = 0, stream=None) -> None:
    """zip3 encode reading x once, with the window base taken from byte
    ``e0_offset`` of the uint8 device tensor ``e0_src`` (for instance byte 7,
    the window base, of the previous iteration's stream)."""
    lib = load_library()
    _check_values(x, "x")
    _check_bytes(e0_src, "e0_src", e0_offset + 1)
    _check_bytes(out, "out")
    _check_bytes(ws, "ws")
    _check_size_slot(out_size)
    st = lib.zip3_encode_e0(_ptr(x), x.numel(), ctypes.c_void_p(e0_src.data_ptr() + e0_offset), _ptr(out),
                            out.numel(), _ptr(ws), ws.numel(), ctypes.c_void_p(out_size.data_ptr()), _stream(stream))
    _raise(st, "zip3_encode_e0")


def zip3_decode(inp, in_size: int, y, ws, stream=None) -> None:
    lib = load_library()
    _check_bytes(inp, "inp", in_size)
    _check_values(y, "y")
    _check_bytes(ws, "ws")
    st = lib.zip3_decode(_ptr(inp), in_size, _ptr(y), y.numel(), _ptr(ws), ws.numel(), _stream(stream))
    _raise(st, "zip3_decode")


def ciera_encode(x, B: int, prev_exp, out, ws, out_size, e0_override: int = -1, stream=None,
                 plan_groups: int = 0) -> None:
    lib = load_library()
    _check_values(x, "x")
    _check_bytes(prev_exp, "prev_exp", x.numel())
    _check_bytes(out, "out")
    _check_bytes(ws, "ws")
    _check_size_slot(out_size)
    st = lib.ciera_encode_ex(_ptr(x), x.numel(), B, _ptr(prev_exp), _ptr(out), out.numel(), _ptr(ws),
                             ws.numel(), ctypes.c_void_p(out_size.data_ptr()), e0_override, plan_groups,
                             _stream(stream))
    _raise(st, "ciera_encode")


def ciera_encode_noalloc(x, B: int, prev_exp, out, out_size, stream=None) -> None:
    """ciera_encode with its workspace in the library's own device array
    (nothing is allocated; n <= NOALLOC_MAX_N; calls on one GPU must not
    overlap)."""
    lib = load_library()
    _check_values(x, "x")
    _check_bytes(prev_exp, "prev_exp", x.numel())
    _check_bytes(out, "out")
    _check_size_slot(out_size)
    st = lib.ciera_encode_noalloc(_ptr(x), x.numel(), B, _ptr(prev_exp), _ptr(out), out.numel(),
                                  ctypes.c_void_p(out_size.data_ptr()), _stream(stream))
    _raise(st, "ciera_encode_noalloc")


def ciera_encode_e0(x, B: int, prev_exp, e0_src, out, ws, out_size, e0_offset: int = 0, stream=None) -> None:
    """ciera encode reading x and the sender cache once, with the window base
    taken from byte ``e0_offset`` of the uint8 device tensor ``e0_src``."""
    lib = load_library()
    _check_values(x, "x")
    _check_bytes(prev_exp, "prev_exp", x.numel())
    _check_bytes(e0_src, "e0_src", e0_offset + 1)
    _check_bytes(out, "out")
    _check_bytes(ws, "ws")
    _check_size_slot(out_size)
    st = lib.ciera_encode_e0(_ptr(x), x.numel(), B, _ptr(prev_exp), ctypes.c_void_p(e0_src.data_ptr() + e0_offset),
                             _ptr(out), out.numel(), _ptr(ws), ws.numel(), ctypes.c_void_p(out_size.data_ptr()),
                             _stream(stream))
    _raise(st, "ciera_encode_e0")


def zip3_encode_spec(x, hint_src, out, ws, out_size, hint_offset: int = 0, stream=None) -> None:
    """zip3_encode's stream, reading x once when the window base hinted by
    byte ``hint_offset`` of the uint8 device tensor ``hint_src`` (e.g. byte 7
    of the previous iteration's stream) is the one x's sigma gives."""
    lib = load_library()
    _check_values(x, "x")
    _check_bytes(hint_src, "hint_src", hint_offset + 1)
    _check_bytes(out, "out")
    _check_bytes(ws, "ws")
    _check_size_slot(out_size)
    st = lib.zip3_encode_spec(_ptr(x), x.numel(), ctypes.c_void_p(hint_src.data_ptr() + hint_offset), _ptr(out),
                              out.numel(), _ptr(ws), ws.numel(), ctypes.c_void_p(out_size.data_ptr()), _stream(stream))
    _raise(st, "zip3_encode_spec")


def ciera_encode_spec(x, B: int, prev_exp, hint_src, out, ws, out_size, hint_offset: int = 0, stream=None) -> None:
    """ciera_encode's stream and cache update, reading x and the sender cache
    once when the hinted window base (byte ``hint_offset`` of ``hint_src``)
    is the one x's sigma gives."""
    lib = load_library()
    _check_values(x, "x")
    _check_bytes(prev_exp, "prev_exp", x.numel())
    _check_bytes(hint_src, "hint_src", hint_offset + 1)
    _check_bytes(out, "out")
    _check_bytes(ws, "ws")
    _check_size_slot(out_size)
    st = lib.ciera_encode_spec(_ptr(x), x.numel(), B, _ptr(prev_exp), ctypes.c_void_p(hint_src.data_ptr() + hint_offset),
                               _ptr(out), out.numel(), _ptr(ws), ws.numel(), ctypes.c_void_p(out_size.data_ptr()),
                               _stream(stream))
    _raise(st, "ciera_encode_spec")


def ciera_hash_cache_size(n: int, B: int) -> int:
    return load_library().ciera_hash_cache_size(n, B)


def ciera_encode_hashed(x, B: int, hash_cache, out, ws, out_size, stream=None) -> None:
    """ciera encode with the block-hash sender state (uint8 tensor of
    ciera_hash_cache_size(n, B) bytes, zeroed before the first iteration)."""
    lib = load_library()
    _check_values(x, "x")
    _check_bytes(hash_cache, "hash_cache", ciera_hash_cache_size(x.numel(), B))
    _check_bytes(out, "out")
    _check_bytes(ws, "ws")
    _check_size_slot(out_size)
    st = lib.ciera_encode_hashed(_ptr(x), x.numel(), B, _ptr(hash_cache), _ptr(out), out.numel(), _ptr(ws),
                                 ws.numel(), ctypes.c_void_p(out_size.data_ptr()), _stream(stream))
    _raise(st, "ciera_encode_hashed")


def rans_max_encoded_size(n: int, B: int = 0) -> int:
    return load_library().rans_max_encoded_size(n, B)


def rans_workspace_size(n: int, B: int = 0) -> int:
    return load_library().rans_workspace_size(n, B)


def zip3_encode_rans(x, out, ws, out_size, stream=None) -> None:
    lib = load_library()
    _check_values(x, "x")
    _check_bytes(out, "out")
    _check_bytes(ws, "ws")
    _check_size_slot(out_size)
    st = lib.zip3_encode_rans(_ptr(x), x.numel(), _ptr(out), out.numel(), _ptr(ws), ws.numel(),
                              ctypes.c_void_p(out_size.data_ptr()), _stream(stream))
    _raise(st, "zip3_encode_rans")


def zip3_decode_rans(inp, in_size: int, y, ws, stream=None) -> None:
    lib = load_library()
    _check_bytes(inp, "inp", in_size)
    _check_values(y, "y")
    _check_bytes(ws, "ws")
    st = lib.zip3_decode_rans(_ptr(inp), in_size, _ptr(y), y.numel(), _ptr(ws), ws.numel(), _stream(stream))
    _raise(st, "zip3_decode_rans")


def ciera_encode_rans(x, B: int, prev_exp, out, ws, out_size, stream=None) -> None:
    lib = load_library()
    _check_values(x, "x")
    _check_bytes(prev_exp, "prev_exp", x.numel())
    _check_bytes(out, "out")
    _check_bytes(ws, "ws")
    _check_size_slot(out_size)
    st = lib.ciera_encode_rans(_ptr(x), x.numel(), B, _ptr(prev_exp), _ptr(out), out.numel(), _ptr(ws), ws.numel(),
                               ctypes.c_void_p(out_size.data_ptr()), _stream(stream))
    _raise(st, "ciera_encode_rans")


def ciera_decode_rans(inp, in_size: int, y, B: int, prev_exp, ws, stream=None) -> None:
    lib = load_library()
    _check_bytes(inp, "inp", in_size)
    _check_values(y, "y")
    _check_bytes(prev_exp, "prev_exp", y.numel())
    _check_bytes(ws, "ws")
    st = lib.ciera_decode_rans(_ptr(inp), in_size, _ptr(y), y.numel(), B, _ptr(prev_exp), _ptr(ws), ws.numel(),
                               _stream(stream))
    _raise(st, "ciera_decode_rans")


def ciera_decode(inp, in_size: int, y, B: int, prev_exp, ws, stream=None) -> None:
    lib = load_library()
    _check_bytes(inp, "inp", in_size)
    _check_values(y, "y")
    _check_bytes(prev_exp, "prev_exp", y.numel())
    _check_bytes(ws, "ws")
    st = lib.ciera_decode(_ptr(inp), in_size, _ptr(y), y.numel(), B, _ptr(prev_exp), _ptr(ws), ws.numel(),
                          _stream(stream))
    _raise(st, "ciera_decode")


def decode_batch_workspace_size(n: int, k: int) -> int:
    return load_library().decode_batch_workspace_size(n, k)


def _batch_arrays(inps, in_sizes, ys, prev_exps=None):
    """Host arrays of device pointers and sizes for the batch decodes."""
    k = len(inps)
    if not (len(in_sizes) == len(ys) == k) or (prev_exps is not None and len(prev_exps) != k):
        raise ValueError("one input size, output (and cache) per stream")
    if not 1 <= k <= DECODE_BATCH_MAX:
        raise ValueError(f"1 to {DECODE_BATCH_MAX} streams per batch, got {k}")
    n = ys[0].numel()
    for i in range(k):
        _check_bytes(inps[i], f"inps[{i}]", in_sizes[i])
        _check_values(ys[i], f"ys[{i}]")
        if ys[i].numel() != n:
            raise ValueError("every output of a batch holds the same number of values")
        if prev_exps is not None:
            _check_bytes(prev_exps[i], f"prev_exps[{i}]", n)
    arr = ctypes.c_void_p * k
    ins = arr(*[inp.data_ptr() for inp in inps])
    sizes = (ctypes.c_uint64 * k)(*in_sizes)
    outs = arr(*[y.data_ptr() if n else None for y in ys])
    caches = arr(*[c.data_ptr() if n else None for c in prev_exps]) if prev_exps is not None else None
    return k, n, ins, sizes, outs, caches


def zip3_decode_batch(inps, in_sizes, ys, ws, stream=None) -> None:
    """Decode len(inps) zip3 streams of the same n in one launch: stream i
    (in_sizes[i] bytes of inps[i]) into ys[i]."""
    lib = load_library()
    k, n, ins, sizes, outs, _ = _batch_arrays(inps, in_sizes, ys)
    _check_bytes(ws, "ws")
    st = lib.zip3_decode_batch(k, ins, sizes, outs, n, _ptr(ws), ws.numel(), _stream(stream))
    _raise(st, "zip3_decode_batch")


def ciera_decode_batch(inps, in_sizes, ys, B: int, prev_exps, ws, stream=None) -> None:
    """Decode len(inps) ciera streams of the same n and B in one launch:
    stream i against receiver cache prev_exps[i] (updated in place) into
    ys[i]."""
    lib = load_library()
    k, n, ins, sizes, outs, caches = _batch_arrays(inps, in_sizes, ys, prev_exps)
    _check_bytes(ws, "ws")
    st = lib.ciera_decode_batch(k, ins, sizes, outs, n, B, caches, _ptr(ws), ws.numel(), _stream(stream))
    _raise(st, "ciera_decode_batch")


def bind(name: str, *args, stream=None):
    """Pre-marshal one entry point's arguments and return a zero-argument
    callable that only makes the C call (for tight launch loops and
    benchmarks).  ``args`` are the tensors and integers in the C order,
    without the stream; tensors become device pointers, integers stay."""
    lib = load_library()
    fn = getattr(lib, name)
    cargs = []
    for a in args:
        if hasattr(a, "data_ptr"):
            cargs.append(ctypes.c_void_p(a.data_ptr()) if a.numel() else None)
        else:
            cargs.append(a)
    cargs.append(_stream(stream))

    def call():
        st = fn(*cargs)
        if st != 0:
            raise CieraError(st, name)
    return call


def ciera_read_error(ws, stream=None) -> int:
    """Synchronise the stream and return the device-side status word."""
    _check_bytes(ws, "ws")
    return load_library().ciera_read_error(_ptr(ws), _stream(stream))


def ciera_time_kernels(pairs, stream=None) -> None:
    """Queue (start, stop) ``torch.cuda.Event(enable_timing=True)`` pairs: the
    next ``len(pairs)`` kernel launches of this thread each record one pair at
    the kernel's own start and end.  Events not yet backed by a HIP event are
    recorded once on ``stream`` first so that their handles exist."""
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    handles = []
    for a, b in pairs:
        for e in (a, b):
            if not e.cuda_event:
                e.record(s)
            handles.append(e.cuda_event)
    arr = (ctypes.c_void_p * len(handles))(*handles)
    _raise(load_library().ciera_time_kernels(arr, len(pairs)), "ciera_time_kernels")


def ciera_set_wait_limit(polls: int) -> int:
    """Test hook: polls after which the next calls' waits on other workgroups
    give up (0 restores the default).  Returns the previous bound."""
    return int(load_library().ciera_set_wait_limit(polls))
