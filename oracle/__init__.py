"""CPU oracle for the lossless BF16 codec -- TEST INFRASTRUCTURE ONLY.

A thin ctypes/numpy wrapper around ``ciera_oracle.c``: plain scalar C that
encodes and decodes one value at a time, in element order.  It defines what
the HIP library must produce byte for byte.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package; the product library never does.

Parity pins (see the tests under ``tests/``): exhaustive round trips over all
65,536 BF16 bit patterns, the ZipCCL digest's Figure 2 binade shares and
97.5 % window share, the optimum u = 0.0172 and x_opt = log2(sigma) - 5.36
(ZipCCL research digest, section 3.1), the block reuse law (1-c)^B (CIERA
page, section 2), the closed-form stream size, exact-rational variance on
small inputs, a second, independent pure-Python encoder, and, for the block
hash of the hash sender, SplitMix64's published output sequence.  The byte layout
itself is a reading of the pages (they print no encoded bytes); it is pinned
by the size identity and by that second implementation only.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ciera_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libciera_oracle.so")

OK, ERR_ARG, ERR_CAPACITY, ERR_FORMAT, ERR_NOMEM = 0, 1, 2, 5, 6
CHUNK = 65536

_lib = None


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"oracle {what} failed with status {status}")
        self.status = status


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libciera_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
               "-ffp-contract=off", "-pthread", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    u64, u32, vp, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = ctypes.c_double
    lib.orc_exponent_sums.argtypes = [vp, u64, vp, vp, ctypes.POINTER(u64)]
    lib.orc_exponent_sums.restype = None
    lib.orc_window_base_exact.argtypes = [vp, vp, u64]
    lib.orc_window_base_exact.restype = i32
    lib.orc_window_base.argtypes = [ctypes.c_double, u64]
    lib.orc_window_base.restype = i32
    lib.orc_choose_e0.argtypes = [vp, u64]
    lib.orc_choose_e0.restype = i32
    lib.orc_max_encoded_size.argtypes = [u64, u32]
    lib.orc_max_encoded_size.restype = u64
    lib.orc_encode.argtypes = [vp, u64, u32, vp, i32, vp, u64, ctypes.POINTER(u64), vp]
    lib.orc_encode.restype = i32
    lib.orc_decode.argtypes = [vp, u64, vp, u64, u32, vp]
    lib.orc_decode.restype = i32
    lib.orc_encode_mt.argtypes = [vp, u64, u32, vp, i32, vp, u64, ctypes.POINTER(u64), vp, i32]
    lib.orc_encode_mt.restype = i32
    lib.orc_decode_mt.argtypes = [vp, u64, vp, u64, u32, vp, i32]
    lib.orc_decode_mt.restype = i32
    lib.orc_splitmix64_next.argtypes = [ctypes.POINTER(u64)]
    lib.orc_splitmix64_next.restype = u64
    lib.orc_block_hashes.argtypes = [vp, u64, u32, vp]
    lib.orc_block_hashes.restype = None
    lib.orc_rans_freqs.argtypes = [vp, vp]
    lib.orc_rans_freqs.restype = None
    lib.orc_rans_max_encoded_size.argtypes = [u64, u32]
    lib.orc_rans_max_encoded_size.restype = u64
    lib.orc_encode_rans.argtypes = [vp, u64, u32, vp, vp, u64, ctypes.POINTER(u64), vp]
    lib.orc_encode_rans.restype = i32
    lib.orc_decode_rans.argtypes = [vp, u64, vp, u64, u32, vp]
    lib.orc_decode_rans.restype = i32
    _lib = lib
    return lib


def _u16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("BF16 data must be passed as a uint16 bit-pattern array")
    return x.reshape(-1)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a.size else None


def bf16_value(bits: int) -> float:
    return _load().orc_bf16_value(bits)


def exponent_sums(x) -> tuple[np.ndarray, np.ndarray, int]:
    """Per exponent field E (256 entries): the sum of the signed integer
    significands M and of M^2 over the finite values (a value is
    M * 2^(max(E, 1) - 134)), and the number of finite values."""
    x = _u16(x)
    a = np.zeros(256, dtype=np.int64)
    b = np.zeros(256, dtype=np.uint64)
    nf = ctypes.c_uint64()
    _load().orc_exponent_sums(_ptr(x), x.size, _ptr(a), _ptr(b), ctypes.byref(nf))
    return a, b, nf.value


def exact_moments(x) -> tuple[int, Fraction, Fraction]:
    """(finite count, exact sum of the finite values, exact sum of their
    squares), from the oracle's integer sums."""
    a, b, nf = exponent_sums(x)
    s1 = sum(int(a[e]) << (max(e, 1) - 1) for e in range(255))
    s2 = sum(int(b[e]) << (2 * max(e, 1) - 2) for e in range(255))
    return nf, Fraction(s1, 1 << 133), Fraction(s2, 1 << 266)


def variance(x) -> tuple[Fraction, int]:
    """(exact sample variance of the finite values, number of finite values);
    0 when fewer than two values are finite."""
    nf, s1, s2 = exact_moments(x)
    if nf < 2:
        return Fraction(0), nf
    return (nf * s2 - s1 * s1) / (nf * (nf - 1)), nf


def window_base(var: float, nfinite: int) -> int:
    return _load().orc_window_base(var, nfinite)


def choose_e0(x) -> int:
    x = _u16(x)
    return _load().orc_choose_e0(_ptr(x), x.size)


def window_base_exact(a, b, nf: int) -> int:
    """Window base from per-exponent significand sums (see exponent_sums)."""
    a = np.ascontiguousarray(a, dtype=np.int64)
    b = np.ascontiguousarray(b, dtype=np.uint64)
    assert a.size == 256 and b.size == 256
    return _load().orc_window_base_exact(_ptr(a), _ptr(b), nf)


def max_encoded_size(n: int, B: int = 0) -> int:
    return _load().orc_max_encoded_size(n, B)


def encode(x, B: int = 0, cache: np.ndarray | None = None, e0_override: int = -1, threads: int = 0):
    """Encode ``x`` (uint16 BF16 patterns).  ``B = 0`` is zip3 mode; otherwise
    ciera mode with block size ``B`` and the sender cache ``cache`` (uint8,
    len(x), updated in place).  ``threads`` > 0 runs the chunk-parallel
    driver on that many threads (same bytes).  Returns (stream bytes as uint8
    array, {"E0", "changed_blocks", "escapes"})."""
    x = _u16(x)
    n = x.size
    if B:
        if cache is None or cache.dtype != np.uint8 or cache.size != n or not cache.flags.c_contiguous:
            raise ValueError("ciera mode needs a contiguous uint8 cache of len(x)")
    cap = max_encoded_size(n, B)
    out = np.zeros(cap, dtype=np.uint8)
    size = ctypes.c_uint64()
    stats = np.zeros(3, dtype=np.uint64)
    if threads > 0:
        st = _load().orc_encode_mt(_ptr(x), n, B, _ptr(cache) if B else None, e0_override,
                                   _ptr(out), cap, ctypes.byref(size), _ptr(stats), threads)
    else:
        st = _load().orc_encode(_ptr(x), n, B, _ptr(cache) if B else None, e0_override,
                                _ptr(out), cap, ctypes.byref(size), _ptr(stats))
    if st != OK:
        raise OracleError(st, "encode")
    return out[: size.value].copy(), {"E0": int(stats[0]), "changed_blocks": int(stats[1]),
                                      "escapes": int(stats[2])}


def decode(stream, n: int, B: int = 0, cache: np.ndarray | None = None, threads: int = 0) -> np.ndarray:
    """Decode a stream back to n uint16 BF16 patterns (ciera mode updates
    ``cache`` in place); ``threads`` > 0 decodes chunks on that many threads."""
    stream = np.ascontiguousarray(stream, dtype=np.uint8).reshape(-1)
    y = np.zeros(n, dtype=np.uint16)
    if B:
        if cache is None or cache.dtype != np.uint8 or cache.size != n or not cache.flags.c_contiguous:
            raise ValueError("ciera mode needs a contiguous uint8 cache of n bytes")
    if threads > 0:
        st = _load().orc_decode_mt(_ptr(stream), stream.size, _ptr(y), n, B, _ptr(cache) if B else None, threads)
    else:
        st = _load().orc_decode(_ptr(stream), stream.size, _ptr(y), n, B, _ptr(cache) if B else None)
    if st != OK:
        raise OracleError(st, "decode")
    return y


def splitmix64(seed: int, count: int) -> list[int]:
    """The first ``count`` outputs of a SplitMix64 generator seeded with ``seed``."""
    st = ctypes.c_uint64(seed)
    return [int(_load().orc_splitmix64_next(ctypes.byref(st))) for _ in range(count)]


def block_hashes(x, B: int) -> np.ndarray:
    """The two 64-bit hashes of every block of B values of ``x``'s exponent
    fields: a uint64 array of shape (ceil(len(x) / B), 2)."""
    x = _u16(x)
    nb = -(-x.size // B)
    out = np.zeros((nb, 2), dtype=np.uint64)
    _load().orc_block_hashes(_ptr(x), x.size, B, _ptr(out))
    return out


def rans_freqs(hist) -> np.ndarray:
    """The normalised rANS frequencies (sum 4096) of a 256-bin histogram."""
    h = np.ascontiguousarray(hist, dtype=np.uint32).reshape(-1)
    assert h.size == 256
    f = np.zeros(256, dtype=np.uint16)
    _load().orc_rans_freqs(_ptr(h), _ptr(f))
    return f


def rans_max_encoded_size(n: int, B: int = 0) -> int:
    return _load().orc_rans_max_encoded_size(n, B)


def encode_rans(x, B: int = 0, cache: np.ndarray | None = None):
    """rANS-mode encode (B = 0: zip3 + rANS; else ciera + rANS, ``cache``
    updated in place).  Returns (stream, {"changed_blocks", "coded"})."""
    x = _u16(x)
    n = x.size
    if B:
        if cache is None or cache.dtype != np.uint8 or cache.size != n or not cache.flags.c_contiguous:
            raise ValueError("ciera mode needs a contiguous uint8 cache of len(x)")
    cap = rans_max_encoded_size(n, B)
    out = np.zeros(cap, dtype=np.uint8)
    size = ctypes.c_uint64()
    stats = np.zeros(2, dtype=np.uint64)
    st = _load().orc_encode_rans(_ptr(x), n, B, _ptr(cache) if B else None, _ptr(out), cap, ctypes.byref(size),
                                 _ptr(stats))
    if st != OK:
        raise OracleError(st, "encode_rans")
    return out[: size.value].copy(), {"changed_blocks": int(stats[0]), "coded": int(stats[1])}


def decode_rans(stream, n: int, B: int = 0, cache: np.ndarray | None = None) -> np.ndarray:
    stream = np.ascontiguousarray(stream, dtype=np.uint8).reshape(-1)
    y = np.zeros(n, dtype=np.uint16)
    if B:
        if cache is None or cache.dtype != np.uint8 or cache.size != n or not cache.flags.c_contiguous:
            raise ValueError("ciera mode needs a contiguous uint8 cache of n bytes")
    st = _load().orc_decode_rans(_ptr(stream), stream.size, _ptr(y), n, B, _ptr(cache) if B else None)
    if st != OK:
        raise OracleError(st, "decode_rans")
    return y


def zip3_encode(x, e0_override: int = -1):
    return encode(x, 0, None, e0_override)


def zip3_decode(stream, n: int) -> np.ndarray:
    return decode(stream, n, 0, None)


def ciera_encode(x, B: int, cache: np.ndarray, e0_override: int = -1):
    return encode(x, B, cache, e0_override)


def ciera_decode(stream, n: int, B: int, cache: np.ndarray) -> np.ndarray:
    return decode(stream, n, B, cache)
