"""Buffer owners for the C ABI: allocate the stream, workspace, size slot and
exponent caches once with torch, then call the library on them.

Allocation happens only in the constructors; ``encode``/``decode`` only pass
pointers.
"""
from __future__ import annotations

import torch

from . import (CieraError, ciera_decode, ciera_encode, ciera_encode_e0, ciera_encode_spec, ciera_max_encoded_size,
               ciera_read_error, ciera_workspace_size, zip3_decode, zip3_encode, zip3_encode_e0, zip3_encode_spec,
               zip3_max_encoded_size, zip3_workspace_size)


class Zip3Codec:
    """3-bit exponent code only (no cross-iteration state)."""

    def __init__(self, n: int, device="cuda"):
        self.n = n
        self.capacity = zip3_max_encoded_size(n)
        self.out = torch.empty(self.capacity, dtype=torch.uint8, device=device)
        self.ws = torch.empty(zip3_workspace_size(n), dtype=torch.uint8, device=device)
        self.size = torch.zeros(1, dtype=torch.int64, device=device)

    def encode(self, x, e0_override: int = -1, stream=None):
        zip3_encode(x, self.out, self.ws, self.size, e0_override, stream)

    def encode_e0(self, x, stream=None):
        """Single-read encode with the window base of the previous stream in
        ``out`` (its header byte 7, read on the device before it is
        rewritten); the previous call must have been an encode."""
        zip3_encode_e0(x, self.out, self.out, self.ws, self.size, 7, stream)

    def encode_spec(self, x, stream=None):
        """``encode``'s stream, with x read once when the previous stream's
        window base (its header byte 7 in ``out``) is still the one x's sigma
        gives; the previous call must have been an encode."""
        zip3_encode_spec(x, self.out, self.out, self.ws, self.size, 7, stream)

    def decode(self, stream_bytes, in_size: int, y, stream=None):
        zip3_decode(stream_bytes, in_size, y, self.ws, stream)

    def nbytes(self) -> int:
        return int(self.size.item())

    def error(self, stream=None) -> int:
        return ciera_read_error(self.ws, stream)


class CieraCodec:
    """Exponent reuse with block size B plus the 3-bit code; keeps a sender
    and a receiver exponent cache (both start at zero)."""

    def __init__(self, n: int, B: int, device="cuda"):
        self.n, self.B = n, B
        self.capacity = ciera_max_encoded_size(n, B)
        if self.capacity == 0:
            raise ValueError(f"invalid block size {B}")
        self.out = torch.empty(self.capacity, dtype=torch.uint8, device=device)
        self.ws = torch.empty(ciera_workspace_size(n, B), dtype=torch.uint8, device=device)
        self.ws_dec = torch.empty(ciera_workspace_size(n, B), dtype=torch.uint8, device=device)
        self.size = torch.zeros(1, dtype=torch.int64, device=device)
        self.send_cache = torch.zeros(max(n, 1), dtype=torch.uint8, device=device)
        self.recv_cache = torch.zeros(max(n, 1), dtype=torch.uint8, device=device)

    def encode(self, x, e0_override: int = -1, stream=None):
        ciera_encode(x, self.B, self.send_cache, self.out, self.ws, self.size, e0_override, stream)

    def encode_e0(self, x, stream=None):
        """Single-read encode (x and the sender cache read once) with the
        window base of the previous stream in ``out`` (its header byte 7,
        read on the device before it is rewritten); the previous call must
        have been an encode."""
        ciera_encode_e0(x, self.B, self.send_cache, self.out, self.out, self.ws, self.size, 7, stream)

    def encode_spec(self, x, stream=None):
        """``encode``'s stream and cache update, with x and the sender cache
        read once when the previous stream's window base (its header byte 7
        in ``out``) is still the one x's sigma gives; the previous call must
        have been an encode."""
        ciera_encode_spec(x, self.B, self.send_cache, self.out, self.out, self.ws, self.size, 7, stream)

    def decode(self, stream_bytes, in_size: int, y, stream=None):
        ciera_decode(stream_bytes, in_size, y, self.B, self.recv_cache, self.ws_dec, stream)

    def nbytes(self) -> int:
        return int(self.size.item())

    def error(self, stream=None) -> int:
        """Device status of the last encode."""
        return ciera_read_error(self.ws, stream)

    def decode_error(self, stream=None) -> int:
        """Device status of the last decode."""
        return ciera_read_error(self.ws_dec, stream)


# One-shot calls: allocate the stream and workspace with torch, run one
# encode or decode on the current stream, and return the result.  Reading the
# compressed size back synchronizes the stream; the classes above keep their
# buffers and do not.

def _raise_device_error(ws, what: str) -> None:
    st = ciera_read_error(ws)
    if st:
        raise CieraError(st, what)


def zip3_encode_tensor(x):
    """3-bit code of the BF16 values x (a CUDA tensor, read as raw 16-bit
    patterns).  Returns (stream bytes, size)."""
    n = x.numel()
    out = torch.empty(zip3_max_encoded_size(n), dtype=torch.uint8, device=x.device)
    ws = torch.empty(zip3_workspace_size(n), dtype=torch.uint8, device=x.device)
    size = torch.zeros(1, dtype=torch.int64, device=x.device)
    zip3_encode(x, out, ws, size)
    _raise_device_error(ws, "zip3_encode")
    k = int(size.item())
    return out[:k], k


def zip3_decode_tensor(stream_bytes, n: int):
    """Inverse of zip3_encode_tensor: the n values as an int16 tensor of raw patterns."""
    y = torch.empty(n, dtype=torch.int16, device=stream_bytes.device)
    ws = torch.empty(zip3_workspace_size(n), dtype=torch.uint8, device=stream_bytes.device)
    zip3_decode(stream_bytes, stream_bytes.numel(), y, ws)
    _raise_device_error(ws, "zip3_decode")
    return y


def ciera_encode_tensor(x, B: int, prev_exp):
    """Exponent reuse against the sender cache prev_exp (n bytes, updated in
    place) plus the 3-bit code.  Returns (stream bytes, size)."""
    n = x.numel()
    cap = ciera_max_encoded_size(n, B)
    if cap == 0:
        raise ValueError(f"invalid block size {B}")
    out = torch.empty(cap, dtype=torch.uint8, device=x.device)
    ws = torch.empty(ciera_workspace_size(n, B), dtype=torch.uint8, device=x.device)
    size = torch.zeros(1, dtype=torch.int64, device=x.device)
    ciera_encode(x, B, prev_exp, out, ws, size)
    _raise_device_error(ws, "ciera_encode")
    k = int(size.item())
    return out[:k], k


def ciera_decode_tensor(stream_bytes, n: int, B: int, prev_exp):
    """Inverse of ciera_encode_tensor against the receiver cache prev_exp
    (updated in place)."""
    y = torch.empty(n, dtype=torch.int16, device=stream_bytes.device)
    ws = torch.empty(ciera_workspace_size(n, B), dtype=torch.uint8, device=stream_bytes.device)
    ciera_decode(stream_bytes, stream_bytes.numel(), y, B, prev_exp, ws)
    _raise_device_error(ws, "ciera_decode")
    return y
