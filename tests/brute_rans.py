"""A second, independent encoder for the rANS stream modes (zip3 + rANS and
ciera + rANS), in plain Python, written from the format description and not
from the oracle's C: per chunk (65536 values) one frequency table over its
coded exponents, normalised to 4096; per part (16384 values) 64 interleaved
rANS states with 16-bit renormalisation over the part's coded exponents;
chunk payload = header with the parts' word counts, table, then each part's
flushed states and emitted words step by step.  Slow; for small inputs
only."""
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


def coded_stream(sym, f, cum):
    """One part's 16-bit words: 64 interleaved states coding sym with the
    table (f, cum), last step first; then the flushed states and the words
    each step emitted, steps in decoding order."""
    if not sym:
        return []
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
    return words


def chunk_payload(parts):
    """Payload of one chunk from its four parts' symbol lists: one table
    over all of them, then each part's stream."""
    allsym = [s for part in parts for s in part]
    if not allsym:
        return b""
    hist = [0] * 256
    for s in allsym:
        hist[s] += 1
    f = norm_freqs(hist)
    cum = [sum(f[:s]) for s in range(256)]
    present = [s for s in range(256) if f[s]]
    lo, hi = present[0], present[-1]
    streams = [coded_stream(part, f, cum) for part in parts]
    out = bytes([lo, hi, 0, 0]) + struct.pack("<4H", *[len(w) for w in streams])
    out += b"".join(struct.pack("<H", f[s]) for s in range(lo, hi + 1))
    for w in streams:
        out += b"".join(struct.pack("<H", v) for v in w)
    return out


def encode(x, B=0, cache=None):
    """Stream bytes for uint16 BF16 patterns x (B = 0: zip3 + rANS)."""
    x = [int(v) for v in np.asarray(x, dtype=np.uint16)]
    n = len(x)
    e = [(v >> 7) & 0xFF for v in x]
    nchunks = -(-n // CHUNK)
    changed = []
    if B:
        nb = -(-n // B)
        changed = [any(e[i] != int(cache[i]) for i in range(b * B, min(n, (b + 1) * B))) for b in range(nb)]
    sm_pos = 128 + pad128(8 * (nchunks + 1))
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
    for c in range(nchunks):
        table.append(pos)
        parts = []
        for h in range(4):
            lo_v = c * CHUNK + h * PART
            parts.append([e[i] for i in range(lo_v, min(n, lo_v + PART)) if not B or changed[i // B]])
        coded += sum(len(q) for q in parts)
        pay = chunk_payload(parts)
        body += pay + bytes(pad128(len(pay)) - len(pay))
        pos += pad128(len(pay))
    table.append(pos)
    for k, t in enumerate(table):
        body[128 + 8 * k:136 + 8 * k] = struct.pack("<Q", t)
    hd = (b"CIER" if B else b"ZIP3") + struct.pack("<HBB", 2, 3 if B else 2, 0)
    hd += struct.pack("<QIIQQQQ", n, B, CHUNK, nchunks, pos, sum(changed), coded)
    body[:len(hd)] = hd
    return np.frombuffer(bytes(body), dtype=np.uint8)
