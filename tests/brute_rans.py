"""A second, independent encoder for the rANS stream modes (zip3 + rANS and
ciera + rANS), in plain Python, written from the format description and not
from the oracle's C: per part (16384 values) the coded exponents, a
frequency table normalised to 4096, 64 interleaved rANS states with 16-bit
renormalisation, payload = header, table, flushed states, then the emitted
words step by step.  Slow; for small inputs only."""
from __future__ import annotations

import struct

import numpy as np

M, L, LANES, PART, CHUNK = 4096, 1 << 16, 64, 16384, 65536


def pad128(v):
    return -(-v // 128) * 128


def norm_freqs(hist):
    m = sum(hist)
    d = sum(1 for h in hist if h)
    f = [0] * 256
    if m == 0:
        return f
    for s, h in enumerate(hist):
        if h:
            f[s] = max(1, h * (M - d) // m)
    top = max(range(256), key=lambda s: (hist[s], -s))
    f[top] += M - sum(f)
    return f


def part_payload(sym):
    if not sym:
        return b""
    hist = [0] * 256
    for s in sym:
        hist[s] += 1
    f = norm_freqs(hist)
    cum = [sum(f[:s]) for s in range(256)]
    present = [s for s in range(256) if f[s]]
    lo, hi = present[0], present[-1]
    steps = -(-len(sym) // LANES)
    x = [L] * LANES
    groups = [[] for _ in range(steps)]
    for t in reversed(range(steps)):
        for lane in range(LANES):
            i = t * LANES + lane
            if i >= len(sym):
                break
            s = sym[i]
            if x[lane] >= f[s] << 20:
                groups[t].append(x[lane] & 0xFFFF)
                x[lane] >>= 16
            x[lane] = (x[lane] // f[s]) * M + x[lane] % f[s] + cum[s]
    words = []
    for v in x:
        words += [v & 0xFFFF, v >> 16]
    for g in groups:
        words += g
    out = bytes([lo, hi, 0, 0]) + struct.pack("<I", len(words))
    out += b"".join(struct.pack("<H", f[s]) for s in range(lo, hi + 1))
    out += b"".join(struct.pack("<H", w) for w in words)
    return out


def encode(x, B=0, cache=None):
    """Stream bytes for uint16 BF16 patterns x (B = 0: zip3 + rANS)."""
    x = [int(v) for v in np.asarray(x, dtype=np.uint16)]
    n = len(x)
    e = [(v >> 7) & 0xFF for v in x]
    nchunks = -(-n // CHUNK)
    nparts = 4 * nchunks
    changed = []
    if B:
        nb = -(-n // B)
        changed = [any(e[i] != int(cache[i]) for i in range(b * B, min(n, (b + 1) * B))) for b in range(nb)]
    sm_pos = 128 + pad128(8 * (nparts + 1))
    bm_pos = sm_pos + pad128(n)
    pos = bm_pos + (128 * nchunks if B else 0)
    body = bytearray(pos)
    for i, v in enumerate(x):
        body[sm_pos + i] = ((v >> 15) << 7) | (v & 0x7F)
    if B:
        for c in range(nchunks):
            for j in range(CHUNK // B):
                if c * CHUNK + j * B < n and changed[c * (CHUNK // B) + j]:
                    body[bm_pos + 128 * c + (j >> 3)] |= 1 << (j & 7)
    table = []
    coded = 0
    for p in range(nparts):
        table.append(pos)
        sym = [e[i] for i in range(p * PART, min(n, (p + 1) * PART)) if not B or changed[i // B]]
        coded += len(sym)
        pay = part_payload(sym)
        body += pay + bytes(pad128(len(pay)) - len(pay))
        pos += pad128(len(pay))
    table.append(pos)
    for k, t in enumerate(table):
        body[128 + 8 * k:136 + 8 * k] = struct.pack("<Q", t)
    hd = (b"CIER" if B else b"ZIP3") + struct.pack("<HBB", 1, 3 if B else 2, 0)
    hd += struct.pack("<QIIQQQQ", n, B, CHUNK, nchunks, pos, sum(changed), coded)
    body[:len(hd)] = hd
    return np.frombuffer(bytes(body), dtype=np.uint8)
