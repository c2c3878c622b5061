"""The C-ABI library loads, exports every symbol include/ciera.h declares, and
its host-side logic (size queries, argument checks) behaves; no GPU needed."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import lossless_bf16_tensor_exp_amd as ciera
    if not os.path.exists(ciera.library_path()):
        from lossless_bf16_tensor_exp_amd import build
        build.build()
    return ciera.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "ciera.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for f in ("zip3_encode", "zip3_decode", "ciera_encode", "ciera_decode"):
        assert f in names
    assert len(names) >= 12


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


@pytest.mark.parametrize("B", [0, 64, 128, 512, 65536])
def test_size_queries_match_the_oracle(lib, B):
    for n in [0, 1, 7, 8, 100, 65535, 65536, 65537, 10 ** 6, 3 * 65536 + 5, 104891392, 10 ** 9]:
        want = oracle.max_encoded_size(n, B)
        got = lib.zip3_max_encoded_size(n) if B == 0 else lib.ciera_max_encoded_size(n, B)
        assert got == want, (n, B)
        ws = lib.zip3_workspace_size(n) if B == 0 else lib.ciera_workspace_size(n, B)
        assert ws >= 256 and ws % 256 == 0


def test_invalid_sizes_and_blocks(lib):
    assert lib.ciera_max_encoded_size(1000, 100) == 0
    assert lib.ciera_max_encoded_size(1000, 32) == 0
    assert lib.ciera_max_encoded_size(1000, 131072) == 0
    assert lib.zip3_max_encoded_size((1 << 40) + 1) == 0
    assert lib.ciera_workspace_size(1000, 48) == 0


def test_argument_errors_return_before_any_launch(lib):
    # every case fails a host-side check, so no HIP call is made
    big = (1 << 40) + 1
    p = ctypes.c_void_p(16 * 1024)  # never dereferenced
    assert lib.zip3_encode(p, big, p, 1 << 50, p, 1 << 30, p, None) == 1
    assert lib.zip3_encode(None, 10, p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.zip3_encode(p, 10, p, 10, p, 1 << 20, p, None) == 2
    assert lib.zip3_encode(p, 10, p, 1 << 20, p, 10, p, None) == 3
    assert lib.ciera_encode(p, 10, 100, p, p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.ciera_encode(p, 10, 0, p, p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.zip3_encode_ex(p, 10, p, 1 << 20, p, 1 << 20, p, 250, 0, None) == 1
    assert lib.ciera_decode(p, 1 << 20, p, 10, 96, p, p, 1 << 20, None) == 1
    assert lib.zip3_decode(ctypes.c_void_p(16 * 1024 + 8), 1 << 20, p, 10, p, 1 << 20, None) == 1
    assert lib.ciera_read_error(None, None) == 1
    assert lib.zip3_encode_e0(p, 10, None, p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.zip3_encode_e0(p, 10, p, p, 10, p, 1 << 20, p, None) == 2
    # ciera_encode_e0(x, n, B, cache, e0, out, cap, ws, ws_bytes, out_size, stream)
    assert lib.ciera_encode_e0(p, 10, 0, p, p, p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.ciera_encode_e0(p, 10, 96, p, p, p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.ciera_encode_e0(p, 10, 64, p, None, p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.ciera_encode_e0(p, 10, 64, None, p, p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.ciera_encode_e0(p, 10, 64, ctypes.c_void_p(16 * 1024 + 8), p, p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.ciera_encode_e0(p, (1 << 39) + 1, 64, p, p, p, 1 << 50, p, 1 << 40, p, None) == 1
    assert lib.ciera_encode_e0(p, 10, 64, p, p, p, 10, p, 1 << 20, p, None) == 2
    assert lib.ciera_encode_e0(p, 10, 64, p, p, p, 1 << 20, p, 10, p, None) == 3
    assert lib.ciera_encode_hashed(p, 10, 64, None, p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.ciera_encode_hashed(p, 10, 0, p, p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.ciera_encode_hashed(p, 10, 64, ctypes.c_void_p(16 * 1024 + 8), p, 1 << 20, p, 1 << 20, p, None) == 1
    assert lib.ciera_encode_hashed(p, 10, 64, p, p, 10, p, 1 << 20, p, None) == 2
    assert lib.ciera_hash_cache_size(1000, 64) == 16 * 16
    assert lib.ciera_hash_cache_size(1000, 48) == 0
    assert lib.zip3_encode_rans(p, 10, p, 10, p, 1 << 30, p, None) == 2
    assert lib.zip3_encode_rans(p, 10, p, 1 << 20, p, 10, p, None) == 3
    assert lib.ciera_encode_rans(p, 10, 0, p, p, 1 << 20, p, 1 << 30, p, None) == 1
    assert lib.ciera_encode_rans(p, 10, 96, p, p, 1 << 20, p, 1 << 30, p, None) == 1
    assert lib.ciera_decode_rans(p, 1 << 20, p, 10, 0, p, p, 1 << 20, None) == 1
    assert lib.zip3_decode_rans(ctypes.c_void_p(16 * 1024 + 8), 1 << 20, p, 10, p, 1 << 20, None) == 1
    assert lib.rans_max_encoded_size(1000, 48) == 0 and lib.rans_max_encoded_size(0, 0) == 256
    assert lib.ciera_time_kernels(None, 1) == 1
    assert lib.ciera_time_kernels(None, 0) == 0


def test_batch_decode_sizes_and_argument_errors(lib):
    # one status word per workgroup of every stream after the 256-byte
    # control block: a 2^20-value stream has 16 chunks x 4 parts x 4 slices
    # workgroups, a 2^26-value one 1024 chunks x 4 parts
    assert lib.decode_batch_workspace_size(1 << 20, 3) == 256 + 4 * 3 * 256
    assert lib.decode_batch_workspace_size(1 << 26, 2) == 256 + 4 * 2 * 4096
    assert lib.decode_batch_workspace_size(0, 1) == 512
    assert lib.decode_batch_workspace_size(10, 0) == 0
    assert lib.decode_batch_workspace_size(10, 17) == 0
    assert lib.decode_batch_workspace_size(1 << 39, 3) == 0  # k n above 2^40
    # every case fails a host-side check, so no HIP call is made
    two = (ctypes.c_void_p * 2)(16 * 1024, 32 * 1024)
    mis = (ctypes.c_void_p * 2)(16 * 1024, 32 * 1024 + 8)
    nul = (ctypes.c_void_p * 2)(16 * 1024, None)
    sizes = (ctypes.c_uint64 * 2)(1 << 20, 1 << 20)
    p = ctypes.c_void_p(64 * 1024)
    ws = 1 << 20
    assert lib.zip3_decode_batch(0, two, sizes, two, 10, p, ws, None) == 1
    assert lib.zip3_decode_batch(17, two, sizes, two, 10, p, ws, None) == 1
    assert lib.zip3_decode_batch(2, None, sizes, two, 10, p, ws, None) == 1
    assert lib.zip3_decode_batch(2, two, None, two, 10, p, ws, None) == 1
    assert lib.zip3_decode_batch(2, mis, sizes, two, 10, p, ws, None) == 1
    assert lib.zip3_decode_batch(2, two, sizes, mis, 10, p, ws, None) == 1
    assert lib.zip3_decode_batch(2, two, sizes, nul, 10, p, ws, None) == 1
    assert lib.zip3_decode_batch(2, two, sizes, two, 10, ctypes.c_void_p(64 * 1024 + 8), ws, None) == 1
    assert lib.zip3_decode_batch(2, two, sizes, two, 1 << 40, p, 1 << 40, None) == 1
    assert lib.zip3_decode_batch(2, two, sizes, two, 10, p, 16, None) == 3
    assert lib.ciera_decode_batch(2, two, sizes, two, 10, 0, two, p, ws, None) == 1
    assert lib.ciera_decode_batch(2, two, sizes, two, 10, 96, two, p, ws, None) == 1
    assert lib.ciera_decode_batch(2, two, sizes, two, 10, 64, None, p, ws, None) == 1
    assert lib.ciera_decode_batch(2, two, sizes, two, 10, 64, mis, p, ws, None) == 1
    assert lib.ciera_decode_batch(2, two, sizes, two, 10, 64, two, p, 16, None) == 3


def test_status_strings(lib):
    assert lib.ciera_status_string(0) == b"ok"
    assert lib.ciera_status_string(5) == b"malformed stream"
    assert lib.ciera_status_string(99) == b"unknown status"
