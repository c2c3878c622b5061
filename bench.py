#!/usr/bin/env python3
"""Codec benchmark: GB/s of BF16 input through encode + decode on one MI355X.

A step is one pass of the whole codec over one synthetic tensor already
resident in HBM: encode (variance/change pass, window plan, pack) and decode.
Default workload: the largest one, the 1e9-value stress buffer (mixed
N(0, 0.02) / Student-t / constant regions with +-0, subnormals, Inf and NaN
payloads, 1 % exponent flips between two iterations; exponent reuse with
B = 512 plus the 3-bit code).  The reuse workloads' steps alternate between
two consecutive iterations, so the caches always hold the previous one.

Prints one JSON line.  ``value`` = 2 n K / (wall time of K steps), in GB/s of
BF16 input (1 GB = 1e9 bytes).  A second pass of the same K steps times every
kernel with HIP events recorded at the kernel's own start and end;
``roofline`` describes the streaming kernel with the longest average
duration.  In the back-to-back steps, work that one call leaves in the
256 MB MALL (decode's output lines, still to be written back) is paid by the
next call, so a third pass, ``isolated``, times encode alone and decode alone
with the MALL swept by a 1 GiB read before every call.

Checks in the same run: the stream of the timed encode is compared byte for
byte with the CPU oracle's for the same input and cache (``bit_exact_vs_oracle``;
the run exits with status 1 when it differs), and the decoded tensor with the
input.  ``cpu_baseline`` times that oracle on the host's cores: one thread,
and chunk-parallel on all of them (the same bytes).  ``configs`` repeats the
isolated measurement, the oracle check and both oracle legs for the other
workloads (1: a 2^20-value shard, 2: the 64 Mi-value gradient tensor, 3: the
OLMoE-like shard at B = 64 and 1024, 4: the DeepSeek-like chain's last
iteration).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# VALU issue peak of MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane
# instructions per second (a wave64 instruction occupies a 16-lane SIMD for 4
# cycles): 614.4 G wave instructions/s.
VALU_PEAK_WAVE_INSTR_PER_S = 256 * 4 * 2.4e9 / 4
WORKLOAD_NAMES = {
    1: "shard 1,048,576 BF16 ~N(0,0.02), iter t = iter t-1 + N(0,1e-4); exponent reuse B={B} + 3-bit code",
    2: "gradient 67,108,864 BF16 ~N(0,1e-3) + 0.1% Student-t(3); 3-bit code only, 128-B chunks",
    3: "OLMoE-like layer shard W=4, 104,891,392 BF16 ~N(0,0.02), ~0.3% exponent flips; exponent reuse B={B}",
    4: "DeepSeek-MoE-like layer shard W=8, 71,368,704 BF16 ~N(0,0.015), 0.5% flips in 20% of blocks; B={B}",
    5: "stress 1e9 BF16 mixed N/t/constant + specials, 1% flips; exponent reuse B={B}",
}
DEFAULT_B = {1: 256, 2: 0, 3: 64, 4: 128, 5: 512}
# the encode's kernels, in launch order, then the decode's; a tensor of at most
# SELF_PLAN_CHUNKS chunks is planned inside k_write (two launches)
ENC_KERNELS = ["k_stats", "k_sums", "k_plan", "k_write"]
ENC_KERNELS_SMALL = ["k_stats", "k_write"]
SELF_PLAN_CHUNKS = 16
DEC_KERNELS = ["k_decode"]
# the speculative encode's launches (tensors of more than SELF_PLAN_CHUNKS chunks)
SPEC_KERNELS = ["k_prep1", "k_write1", "k_sums", "k_check", "k_stats", "k_plan", "k_write"]
STREAMING = ["k_stats", "k_write", "k_decode"]


def source_hash() -> str:
    with open(os.path.join(ROOT, "lossless_bf16_tensor_exp_amd", "csrc", "ciera.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def host_threads() -> int:
    """Threads for the all-core oracle leg: the host's CPUs, at most 16 (a
    one-GPU share of the box)."""
    return max(1, min(16, os.cpu_count() or 1))


class _Offset:
    """A device pointer into a tensor at a byte offset, for ciera.bind."""

    def __init__(self, t, off):
        self.t, self.off = t, off

    def data_ptr(self):
        return self.t.data_ptr() + self.off

    def numel(self):
        return self.t.numel() - self.off


def measured_bandwidth(torch, dev, nbytes=2 << 30, reps=5):
    """Practical HBM bandwidth in the same run: a streaming copy-like kernel
    (reads and writes nbytes) and a read-only reduction (reads nbytes), each
    the best of reps, in GB/s of bytes moved."""
    a = torch.full((nbytes // 4,), 1, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    af = torch.ones((nbytes // 4,), dtype=torch.float32, device=dev)
    r = torch.empty((), dtype=torch.float32, device=dev)

    def best(fn):
        t = []
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            t.append(e0.elapsed_time(e1))
        return min(t[1:]) * 1e-3

    copy = 2 * nbytes / best(lambda: torch.bitwise_not(a, out=b)) / 1e9
    read = nbytes / best(lambda: torch.sum(af, dim=0, out=r)) / 1e9
    del a, b, af
    return copy, read


def changed_values(prev, cur, B):
    """Values in blocks whose exponents changed between two iterations."""
    import numpy as np
    n = prev.size
    nb = -(-n // B)
    diff = ((prev ^ cur) & 0x7F80) != 0
    pad = np.zeros(nb * B, dtype=bool)
    pad[:n] = diff
    blk = pad.reshape(nb, B).any(axis=1)
    sizes = np.full(nb, B, dtype=np.int64)
    sizes[-1] = n - (nb - 1) * B
    return int(sizes[blk].sum())


def _profile_record(kind: str, kernel: str, workload: int, B: int):
    """A per-launch figure for kernel on (workload, B) from the ```json blocks
    of the ``*{kind}*.md`` summaries in profiles/, if taken on the current
    kernel source (else None)."""
    import glob
    import re
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*{kind}*.md"))):
        with open(path) as f:
            text = f.read()
        for block in re.findall(r"```json\n(.*?)```", text, flags=re.S):
            rec = json.loads(block)
            if rec.get("source_hash") != source_hash():
                continue
            hit = rec.get("kernels", {}).get(f"{kernel}/w{workload}/B{B}")
            if hit is not None:
                return hit
    return None


def load_valu(kernel: str, workload: int, B: int):
    """VALU wave instructions per launch (rocprofv3 SQ_INSTS_VALU, a device
    total) from the instruction summaries in profiles/."""
    return _profile_record("valu", kernel, workload, B)


def load_traffic(kernel: str, workload: int, B: int):
    """Counter-derived HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled
    by a copy kernel of known size) from the traffic summaries in profiles/."""
    return _profile_record("traffic", kernel, workload, B)


def alu_roofline(kernel: str, key: str, workload: int, B: int, ms: float):
    """The kernel against the VALU issue peak: its counted VALU instructions
    per launch over its average duration (null without a counter record)."""
    v = load_valu(key, workload, B)
    if v is None:
        return {"kernel": kernel, "bound": "alu", "achieved": None, "peak": VALU_PEAK_WAVE_INSTR_PER_S / 1e9,
                "unit": "G VALU wave instr/s", "frac": None}
    a = v / (ms * 1e-3)
    return {"kernel": kernel, "bound": "alu", "achieved": round(a / 1e9, 1), "peak": VALU_PEAK_WAVE_INSTR_PER_S / 1e9,
            "unit": "G VALU wave instr/s", "frac": round(a / VALU_PEAK_WAVE_INSTR_PER_S, 4),
            "valu_instr_per_launch": v, "avg_launch_ms": round(ms, 5)}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Gpu:
    """The device, stream, MALL sweep and isolated-call timer shared by the
    measurements."""

    def __init__(self, torch, ciera, K):
        self.torch, self.ciera, self.K = torch, ciera, K
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream()
        self.sweep = torch.ones(1 << 28, dtype=torch.float32, device=self.dev)
        self.sweep_out = torch.empty((), dtype=torch.float32, device=self.dev)

    def isolated(self, call, restore=None):
        """K + 1 calls, each preceded (outside its events) by restore() and a
        1 GiB read that leaves only clean lines in the MALL; the first call
        is a warm-up.  Returns (median ms, min ms)."""
        torch = self.torch
        marks = []
        for _ in range(self.K + 1):
            if restore is not None:
                restore()
            torch.sum(self.sweep, dim=0, out=self.sweep_out)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(self.stream)
            call()
            b.record(self.stream)
            marks.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in marks[1:])
        return ms[len(ms) // 2], ms[0]


def oracle_legs(oracle, np, x, B, prev_exps, threads):
    """The CPU oracle on one input: one thread and `threads` threads, encode
    then decode, each timed.  Returns (stream, timings dict)."""
    res = {}
    streams = []
    for leg, nt in (("single", 0), ("all_cores", threads)):
        cache = prev_exps.copy() if B else None
        t = time.perf_counter()
        s, _ = oracle.encode(x, B, cache, threads=nt)
        t_enc = time.perf_counter() - t
        rcache = prev_exps.copy() if B else None
        t = time.perf_counter()
        y = oracle.decode(s, x.size, B, rcache, threads=nt)
        t_dec = time.perf_counter() - t
        if not np.array_equal(y, x):
            raise AssertionError(f"the oracle's own round trip failed ({leg})")
        res[leg] = {"threads": max(1, nt), "encode_s": round(t_enc, 3), "decode_s": round(t_dec, 3),
                    "encode_GBps": round(2 * x.size / t_enc / 1e9, 4),
                    "decode_GBps": round(2 * x.size / t_dec / 1e9, 4),
                    "GBps": round(2 * x.size / (t_enc + t_dec) / 1e9, 4)}
        streams.append(s)
    if streams[0].tobytes() != streams[1].tobytes():
        raise AssertionError("the chunk-parallel oracle wrote other bytes than the single-threaded one")
    return streams[0], res


def stream_stats(s, n):
    """Header fields of a stream: window base, changed blocks, escapes."""
    import numpy as np
    hd = s[:56].view(np.uint64)
    return {"E0": int(s[7]), "changed_blocks": int(hd[5]), "escapes": int(hd[6])}


# Shard-sized tensors also time the batch decode of BATCH_PEERS streams (the
# W - 1 = 3 peer shards a rank of a 4-way sharded all-gather receives).
BATCH_MAX_N = 1 << 22
BATCH_PEERS = 3


def measure_decode_batch(gpu, out, sz, n, B, pristine, xd, single_ms):
    """BATCH_PEERS copies of one stream decoded in one batch call (each into
    its own output, against its own receiver cache), timed like the isolated
    calls, against BATCH_PEERS single decodes."""
    torch, ciera = gpu.torch, gpu.ciera
    k = BATCH_PEERS
    ys = [torch.empty(n, dtype=torch.int16, device=gpu.dev) for _ in range(k)]
    caches = [pristine.clone() for _ in range(k)] if B else None
    ws = torch.empty(ciera.decode_batch_workspace_size(n, k), dtype=torch.uint8, device=gpu.dev)
    inps, sizes = [out] * k, [sz] * k
    if B:
        call = lambda: ciera.ciera_decode_batch(inps, sizes, ys, B, caches, ws, stream=gpu.stream)  # noqa: E731
        restore = lambda: [c.copy_(pristine) for c in caches]  # noqa: E731
    else:
        call = lambda: ciera.zip3_decode_batch(inps, sizes, ys, ws, stream=gpu.stream)  # noqa: E731
        restore = None
    ms, ms_min = gpu.isolated(call, restore)
    ok = ciera.ciera_read_error(ws) == 0 and all(bool(torch.equal(y, xd)) for y in ys)
    return {"streams": k, "ms": round(ms, 5), "min_ms": round(ms_min, 5),
            "GBps": round(2 * n * k / (ms * 1e-3) / 1e9, 1),
            "speedup_vs_single_decodes": round(k * single_ms / ms, 3), "roundtrip_ok": ok}


def measure_config(gpu, oracle, np, wl, workload, B_pick, threads):
    """One workload's isolated encode and decode on the GPU, its stream
    against the oracle's, and both oracle legs."""
    torch, ciera = gpu.torch, gpu.ciera
    t0 = time.time()
    d = wl.WORKLOADS[workload]()
    iters, mode = d["iters"], d["mode"]
    B = 0 if mode == "zip3" else B_pick
    x = iters[-1]
    prev = ((iters[-2] >> 7) & 0xFF).astype(np.uint8) if len(iters) >= 2 else None
    n = x.size
    log(f"config {workload} B={B} n={n} generated in {time.time() - t0:.1f}s")
    dev = gpu.dev
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    if mode == "zip3":
        cap, wsz = ciera.zip3_max_encoded_size(n), ciera.zip3_workspace_size(n)
    else:
        cap, wsz = ciera.ciera_max_encoded_size(n, B), ciera.ciera_workspace_size(n, B)
    out = torch.empty(cap, dtype=torch.uint8, device=dev)
    ws_e = torch.empty(wsz, dtype=torch.uint8, device=dev)
    ws_d = torch.empty(wsz, dtype=torch.uint8, device=dev)
    size = torch.zeros(1, dtype=torch.int64, device=dev)
    y = torch.empty(n, dtype=torch.int16, device=dev)
    pristine = send = recv = None
    if mode != "zip3":
        pristine = torch.from_numpy(prev).to(dev)
        send, recv = pristine.clone(), pristine.clone()
        enc = ciera.bind("ciera_encode", xd, n, B, send, out, cap, ws_e, wsz, size, stream=gpu.stream)
    else:
        enc = ciera.bind("zip3_encode", xd, n, out, cap, ws_e, wsz, size, stream=gpu.stream)
    if send is not None:
        send.copy_(pristine)
    enc()
    torch.cuda.synchronize()
    assert ciera.ciera_read_error(ws_e) == 0
    sz = int(size.item())
    if mode == "zip3":
        dec = ciera.bind("zip3_decode", out, sz, y, n, ws_d, wsz, stream=gpu.stream)
    else:
        dec = ciera.bind("ciera_decode", out, sz, y, n, B, recv, ws_d, wsz, stream=gpu.stream)
    restore_s = (lambda: send.copy_(pristine)) if send is not None else None
    e_ms, e_min = gpu.isolated(enc, restore_s)
    d_ms, d_min = gpu.isolated(dec, (lambda: recv.copy_(pristine)) if recv is not None else None)
    assert ciera.ciera_read_error(ws_e) == 0 and ciera.ciera_read_error(ws_d) == 0
    roundtrip = bool(torch.equal(y, xd))
    batch = measure_decode_batch(gpu, out, sz, n, B, pristine, xd, d_ms) if n <= BATCH_MAX_N else None
    spec = None
    if -(-n // 65536) > SELF_PLAN_CHUNKS:
        # the speculative encode hinted by this stream's window byte (a right
        # hint), into its own buffer: its time and its stream against this one
        out_s = torch.empty(cap, dtype=torch.uint8, device=dev)
        size_s = torch.zeros(1, dtype=torch.int64, device=dev)
        hint = out[7:8].clone()
        if mode == "zip3":
            enc_s = ciera.bind("zip3_encode_spec", xd, n, hint, out_s, cap, ws_e, wsz, size_s, stream=gpu.stream)
        else:
            enc_s = ciera.bind("ciera_encode_spec", xd, n, B, send, hint, out_s, cap, ws_e, wsz, size_s,
                               stream=gpu.stream)
        s_ms, s_min = gpu.isolated(enc_s, restore_s)
        ok = ciera.ciera_read_error(ws_e) == 0 and int(size_s.item()) == sz and bool(torch.equal(out_s[:sz], out[:sz]))
        spec = {"encode_ms": round(s_ms, 5), "encode_min_ms": round(s_min, 5),
                "encode_GBps": round(2 * n / (s_ms * 1e-3) / 1e9, 1), "speedup_vs_two_pass": round(e_ms / s_ms, 3),
                "stream_equal_to_full_encode": ok}
        del out_s
    g_stream = out[:sz].cpu().numpy()
    o_stream, legs = oracle_legs(oracle, np, x, B, prev, threads)
    exact = g_stream.tobytes() == o_stream.tobytes()
    ch = changed_values(iters[-2], x, B) if mode != "zip3" else 0
    in_bytes = 2 * n
    alg_enc = in_bytes + (n + ch if mode != "zip3" else 0) + in_bytes + sz
    alg_dec = sz + in_bytes + (n if mode != "zip3" else 0)
    st = stream_stats(g_stream, n)
    nb = -(-n // B) if B else 0
    res = {"workload": WORKLOAD_NAMES[workload].format(B=B), "n": n, "B": B, "mode": mode,
           "encode_ms": round(e_ms, 5), "encode_min_ms": round(e_min, 5),
           "encode_GBps": round(in_bytes / (e_ms * 1e-3) / 1e9, 1),
           "encode_algorithmic_bytes": alg_enc,
           "decode_ms": round(d_ms, 5), "decode_min_ms": round(d_min, 5),
           "decode_GBps": round(in_bytes / (d_ms * 1e-3) / 1e9, 1),
           "decode_algorithmic_bytes": alg_dec,
           "compression_ratio": round(in_bytes / sz, 4), "stream_bytes": sz,
           "E0": st["E0"], "escape_pct": round(100.0 * st["escapes"] / max(1, n), 3),
           "reuse_pct": round(100.0 * (1 - st["changed_blocks"] / nb), 2) if nb else None,
           "bit_exact_vs_oracle": exact, "roundtrip_ok": roundtrip, "oracle": legs}
    if batch is not None:
        res["decode_batch"] = batch
    if spec is not None:
        res["speculative_encode"] = spec
    del out, ws_e, ws_d, y, xd, send, recv, pristine
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=5, choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--block", type=int, default=None, help="block size B for the reuse workloads")
    ap.add_argument("--configs", default="auto",
                    help="extra workloads to measure isolated, as w or w:B, comma-separated; 'auto' = "
                         "1,2,3:64,3:1024,4 with the default workload, none otherwise; '' = none")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle legs and the oracle check")
    ap.add_argument("--verify", action="store_true", help="check the last step's round trip on the device")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after timing, run a plain elementwise kernel that reads and writes MIB MiB each "
                         "(reference dispatch for calibrating hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the codec codes one rank's shard on its own GPU; there is no multi-GPU path)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import lossless_bf16_tensor_exp_amd as ciera
    from lossless_bf16_tensor_exp_amd import workloads as wl

    if not os.path.exists(ciera.library_path()):
        from lossless_bf16_tensor_exp_amd import build as hip_build
        hip_build.build()
    ciera.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    gpu = Gpu(torch, ciera, args.steps)
    dev = gpu.dev
    K = args.steps

    t0 = time.time()
    d = wl.WORKLOADS[args.workload]()
    iters = d["iters"]
    mode = d["mode"]
    B = 0 if mode == "zip3" else (args.block or d["B"][0])
    n = iters[0].size
    log(f"workload {args.workload} n={n} B={B} generated in {time.time() - t0:.1f}s")

    # the two tensors a step alternates between (zip3: one tensor)
    pair = [iters[-2], iters[-1]] if len(iters) >= 2 else [iters[0], iters[0]]
    del d, iters
    xs = [torch.from_numpy(a.view(np.int16)).to(dev) for a in pair]
    y = torch.empty(n, dtype=torch.int16, device=dev)
    if mode == "zip3":
        cap, wsz = ciera.zip3_max_encoded_size(n), ciera.zip3_workspace_size(n)
    else:
        cap, wsz = ciera.ciera_max_encoded_size(n, B), ciera.ciera_workspace_size(n, B)
    out = torch.empty(cap, dtype=torch.uint8, device=dev)
    ws_e = torch.empty(wsz, dtype=torch.uint8, device=dev)
    ws_d = torch.empty(wsz, dtype=torch.uint8, device=dev)
    size = torch.zeros(1, dtype=torch.int64, device=dev)
    send = recv = e_prev = None
    if mode != "zip3":
        e_prev = torch.from_numpy(((pair[0] >> 7) & 0xFF).astype(np.uint8)).to(dev)
        send, recv = e_prev.clone(), e_prev.clone()
    stream = gpu.stream

    # Pre-bound C calls (argument marshalling done once, outside the timing).
    if mode == "zip3":
        enc = [ciera.bind("zip3_encode", xs[k], n, out, cap, ws_e, wsz, size, stream=stream) for k in (0, 1)]
    else:
        enc = [ciera.bind("ciera_encode", xs[k], n, B, send, out, cap, ws_e, wsz, size, stream=stream)
               for k in (0, 1)]

    def dec_for(in_size):
        if mode == "zip3":
            return ciera.bind("zip3_decode", out, in_size, y, n, ws_d, wsz, stream=stream)
        return ciera.bind("ciera_decode", out, in_size, y, n, B, recv, ws_d, wsz, stream=stream)

    # Stream sizes per input are fixed, so decode takes the size learned in
    # the first steps without a host sync inside the timed loops.  Step s
    # encodes input (s+1) % 2 against caches holding the other input.
    sizes, dec = {}, {}
    order = [1, 0] if mode != "zip3" else [0, 0]
    for k in order:
        enc[k]()
        torch.cuda.synchronize()
        sizes[k] = int(size.item())
        dec[k] = dec_for(sizes[k])
        dec[k]()
        torch.cuda.synchronize()
        assert ciera.ciera_read_error(ws_e) == 0 and ciera.ciera_read_error(ws_d) == 0

    def step(s):
        k = (s + 1) % 2 if mode != "zip3" else 0
        enc[k]()
        dec[k]()

    for w in range(2 * args.warmup):
        step(w)
    torch.cuda.synchronize()

    # Pass 1, the headline number: K steps back to back, nothing between them.
    log(f"pass 1: {K} steps back to back")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(K):
        step(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    # Pass 2, the same K steps with every kernel timed by HIP events that the
    # runtime records at the kernel's own start and end (hipExtLaunchKernel);
    # a step launches encode's four kernels, then decode's one.
    enc_names = ENC_KERNELS_SMALL if -(-n // 65536) <= SELF_PLAN_CHUNKS else ENC_KERNELS
    names = enc_names + DEC_KERNELS
    ne = len(enc_names)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
          for _ in range(K)]
    ciera.ciera_time_kernels([pair_ for row in ev for pair_ in row], stream=stream)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for s in range(K):
        k = (K + s + 1) % 2 if mode != "zip3" else 0  # continues the alternation of pass 1
        enc[k]()
        dec[k]()
    torch.cuda.synchronize()
    wall2 = time.perf_counter() - t2
    ciera.ciera_time_kernels([])
    kern_ms = {nm: sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(K)) / K for i, nm in enumerate(names)}
    enc_ms = [ev[s][0][0].elapsed_time(ev[s][ne - 1][1]) for s in range(K)]  # k_stats start .. k_write end
    dec_ms = [ev[s][ne][0].elapsed_time(ev[s][ne][1]) for s in range(K)]
    assert ciera.ciera_read_error(ws_e) == 0 and ciera.ciera_read_error(ws_d) == 0
    if args.verify:
        klast = (2 * K) % 2 if mode != "zip3" else 0  # input of the last step, index 2K-1
        assert torch.equal(y, xs[klast]), "round trip failed"

    # Graph replay: the same steps captured once in a HIP graph (two steps
    # for the reuse workloads, so the caches keep alternating) and replayed;
    # no host launch work per step.
    log("graph replay")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            cap_stream = torch.cuda.current_stream()
            order_g = [1, 0] if mode != "zip3" else [0]
            for k in order_g:
                if mode == "zip3":
                    ciera.zip3_encode(xs[k], out, ws_e, size, stream=cap_stream)
                    ciera.zip3_decode(out, sizes[k], y, ws_d, stream=cap_stream)
                else:
                    ciera.ciera_encode(xs[k], B, send, out, ws_e, size, stream=cap_stream)
                    ciera.ciera_decode(out, sizes[k], y, B, recv, ws_d, stream=cap_stream)
    steps_g = 2 if mode != "zip3" else 1
    reps_g = max(1, K // steps_g)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    tg = time.perf_counter()
    for _ in range(reps_g):
        g.replay()
    torch.cuda.synchronize()
    wall_g = time.perf_counter() - tg
    assert ciera.ciera_read_error(ws_e) == 0 and ciera.ciera_read_error(ws_d) == 0
    graph = {"steps": reps_g * steps_g, "ms_per_step": round(wall_g * 1e3 / (reps_g * steps_g), 4),
             "GBps": round(2 * n * reps_g * steps_g / wall_g / 1e9, 2)}
    del g

    # Pass 3: each direction on its own, K calls each (the ciera caches
    # restored from a pristine copy and the MALL swept before every call,
    # outside the events).  Encode takes the step input of pass 1 against
    # the other input's exponents; decode takes the stream that encode wrote.
    log("pass 3: isolated encode and decode")
    k_iso = 1 if mode != "zip3" else 0
    restore_s = (lambda: send.copy_(e_prev)) if send is not None else None
    restore_r = (lambda: recv.copy_(e_prev)) if recv is not None else None
    enc_iso, enc_iso_min = gpu.isolated(enc[k_iso], restore_s)
    g_stream = out[:sizes[k_iso]].cpu().numpy()  # the timed encode's stream, for the oracle check
    dec_iso, dec_iso_min = gpu.isolated(dec[k_iso], restore_r)
    assert ciera.ciera_read_error(ws_e) == 0 and ciera.ciera_read_error(ws_d) == 0
    iso_roundtrip = bool(torch.equal(y, xs[k_iso]))
    batch = (measure_decode_batch(gpu, out, sizes[k_iso], n, B, e_prev, xs[k_iso], dec_iso)
             if n <= BATCH_MAX_N else None)
    # The floor of this method: one launch of a one-element fill, timed the
    # same way (launch and event overhead, part of every isolated time).
    one = torch.zeros(1, device=gpu.dev)
    floor_ms, floor_min = gpu.isolated(lambda: one.zero_())

    # Single-read encode, timed like pass 3: the window base is byte 7 of the
    # stream the full encode of the same input just wrote (read on the
    # device); x (and the sender cache) are read once (a tensor of at most
    # SELF_PLAN_CHUNKS chunks takes the self-planned two-launch encode with
    # that window instead).  Its stream must equal the full encode's.  Then
    # its kernels once more with events.
    log("single-read encode")
    out1 = torch.empty(cap, dtype=torch.uint8, device=dev)
    size1 = torch.zeros(1, dtype=torch.int64, device=dev)
    ws1 = torch.empty(wsz, dtype=torch.uint8, device=dev)
    if mode == "zip3":
        enc1 = ciera.bind("zip3_encode_e0", xs[k_iso], n, _Offset(out, 7), out1, cap, ws1, wsz, size1,
                          stream=stream)
    else:
        enc1 = ciera.bind("ciera_encode_e0", xs[k_iso], n, B, send, _Offset(out, 7), out1, cap, ws1, wsz, size1,
                          stream=stream)
    sr_iso, sr_iso_min = gpu.isolated(enc1, restore_s)
    assert ciera.ciera_read_error(ws1) == 0
    sz_sr = int(size1.item())
    sr_same = sz_sr == sizes[k_iso] and bool(torch.equal(out1[:sz_sr], out[:sz_sr]))
    ev1 = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2)]
           for _ in range(K)]
    ciera.ciera_time_kernels([pr for row in ev1 for pr in row], stream=stream)
    for _ in range(K):
        if restore_s is not None:
            restore_s()
        torch.sum(gpu.sweep, dim=0, out=gpu.sweep_out)
        enc1()
    torch.cuda.synchronize()
    ciera.ciera_time_kernels([])
    assert ciera.ciera_read_error(ws1) == 0
    sr_small = -(-n // 65536) <= SELF_PLAN_CHUNKS
    sr_names = ENC_KERNELS_SMALL if sr_small else ["k_prep1", "k_write1"]
    prep_ms = sum(ev1[s][0][0].elapsed_time(ev1[s][0][1]) for s in range(K)) / K
    write1_ms = sum(ev1[s][1][0].elapsed_time(ev1[s][1][1]) for s in range(K)) / K
    del out1, ws1

    # Speculative encode (tensors of more than SELF_PLAN_CHUNKS chunks): the
    # regular encode's stream and cache from one read of x when the hinted
    # window base is the one the variance gives.  Timed like pass 3 with a
    # right hint (byte 7 of the regular encode's stream of the same input) and
    # with one a binade off (the fallback), each stream compared with the
    # regular encode's; its kernels once more with events; then K steps back
    # to back like pass 1, each encode hinted by the byte 7 that the previous
    # step left in the output buffer it writes.
    spec_leg = None
    if -(-n // 65536) > SELF_PLAN_CHUNKS:
        log("speculative encode")
        out_s = torch.empty(cap, dtype=torch.uint8, device=dev)
        size_s = torch.zeros(1, dtype=torch.int64, device=dev)
        e0_right = int(out[7].item())
        wrong = torch.tensor([e0_right + 1 if e0_right < 249 else e0_right - 1], dtype=torch.uint8, device=dev)

        def spec_call(xk, hint, dst, sz_t):
            if mode == "zip3":
                return ciera.bind("zip3_encode_spec", xk, n, hint, dst, cap, ws_e, wsz, sz_t, stream=stream)
            return ciera.bind("ciera_encode_spec", xk, n, B, send, hint, dst, cap, ws_e, wsz, sz_t, stream=stream)

        def same_stream():
            sz = int(size_s.item())
            return sz == sizes[k_iso] and bool(torch.equal(out_s[:sz], out[:sz]))

        right_call = spec_call(xs[k_iso], _Offset(out, 7), out_s, size_s)
        sp_ms, sp_min = gpu.isolated(right_call, restore_s)
        assert ciera.ciera_read_error(ws_e) == 0
        sp_same = same_stream()
        evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in SPEC_KERNELS] for _ in range(K)]
        ciera.ciera_time_kernels([pr for row in evs for pr in row], stream=stream)
        for _ in range(K):
            if restore_s is not None:
                restore_s()
            torch.sum(gpu.sweep, dim=0, out=gpu.sweep_out)
            right_call()
        torch.cuda.synchronize()
        ciera.ciera_time_kernels([])
        sk = {nm: round(sum(evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(K)) / K, 5)
              for j, nm in enumerate(SPEC_KERNELS)}
        sw_ms, sw_min = gpu.isolated(spec_call(xs[k_iso], wrong, out_s, size_s), restore_s)
        assert ciera.ciera_read_error(ws_e) == 0
        sw_same = same_stream()
        # the steps write out_s (which now holds the regular encode's stream
        # of xs[k_iso], so its byte 7 is a right first hint) and decode it;
        # out keeps that stream for the hash sender's comparison below
        enc_sp = [spec_call(xs[k], _Offset(out_s, 7), out_s, size_s) for k in (0, 1)]
        if mode == "zip3":
            dec_sp = {k: ciera.bind("zip3_decode", out_s, sizes[k], y, n, ws_d, wsz, stream=stream) for k in sizes}
        else:
            dec_sp = {k: ciera.bind("ciera_decode", out_s, sizes[k], y, n, B, recv, ws_d, wsz, stream=stream)
                      for k in sizes}
        if send is not None:
            send.copy_(e_prev)
            recv.copy_(e_prev)

        def step_spec(s_):
            k = (s_ + 1) % 2 if mode != "zip3" else 0
            enc_sp[k]()
            dec_sp[k]()

        for w in range(2 * args.warmup):
            step_spec(w)
        torch.cuda.synchronize()
        t_sp = time.perf_counter()
        for s_ in range(K):
            step_spec(s_)
        torch.cuda.synchronize()
        wall_sp = time.perf_counter() - t_sp
        assert ciera.ciera_read_error(ws_e) == 0 and ciera.ciera_read_error(ws_d) == 0
        klast = K % 2 if mode != "zip3" else 0  # input of the last step, index K-1
        sp_roundtrip = bool(torch.equal(y, xs[klast]))
        spec_leg = {"isolated_ms": round(sp_ms, 5), "isolated_min_ms": round(sp_min, 5),
                "isolated_GBps": round(2 * n / (sp_ms * 1e-3) / 1e9, 2),
                "speedup_vs_two_pass_isolated": round(enc_iso / sp_ms, 3),
                "stream_equal_to_full_encode": sp_same,
                "kernels": sk,
                "wrong_hint_ms": round(sw_ms, 5), "wrong_hint_stream_equal_to_full_encode": sw_same,
                "steps": K, "ms_per_step": round(wall_sp * 1e3 / K, 4),
                "GBps": round(2 * n * K / wall_sp / 1e9, 2), "step_roundtrip_ok": sp_roundtrip,
                "path": "k_prep1 + k_write1 with the variance sums, k_sums, k_check; k_stats, k_plan, k_write "
                        "return at once on a right hint and encode again on a wrong one"}
        del out_s, enc_sp, dec_sp

    # Hash sender (ciera workloads): the same encode with two 64-bit hashes
    # per block as the sender state.  Its starting cache (the hashes of the
    # other input's exponents) comes from one hashed encode of that input
    # from a zeroed cache; timed like pass 3, and its stream compared with
    # the exact sender's.
    hashed = None
    changed_vals = changed_values(pair[0], pair[1], B) if mode != "zip3" else 0
    if mode != "zip3":
        log("hash sender")
        hsz = ciera.ciera_hash_cache_size(n, B)
        h_pristine = torch.zeros(hsz, dtype=torch.uint8, device=dev)
        h_cache = torch.empty_like(h_pristine)
        out_h = torch.empty(cap, dtype=torch.uint8, device=dev)
        size_h = torch.zeros(1, dtype=torch.int64, device=dev)
        ciera.ciera_encode_hashed(xs[1 - k_iso], B, h_pristine, out_h, ws_e, size_h)
        enc_h = ciera.bind("ciera_encode_hashed", xs[k_iso], n, B, h_cache, out_h, cap, ws_e, wsz, size_h,
                           stream=stream)
        h_ms, h_min = gpu.isolated(enc_h, lambda: h_cache.copy_(h_pristine))
        # the same calls once more with each kernel timed
        evk = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in enc_names]
               for _ in range(K)]
        ciera.ciera_time_kernels([pr for row in evk for pr in row], stream=stream)
        for i in range(K):
            h_cache.copy_(h_pristine)
            torch.sum(gpu.sweep, dim=0, out=gpu.sweep_out)
            enc_h()
        torch.cuda.synchronize()
        ciera.ciera_time_kernels([])
        assert ciera.ciera_read_error(ws_e) == 0
        szh = int(size_h.item())
        same = szh == sizes[k_iso] and bool(torch.equal(out_h[:szh], out[:szh]))
        hk = {nm: sum(evk[i][j][0].elapsed_time(evk[i][j][1]) for i in range(K)) / K
              for j, nm in enumerate(enc_names)}
        alg_h = 2 * n + hsz + 16 * (changed_vals // B) + 2 * n + sizes[k_iso]
        hashed = {"encode_ms": round(h_ms, 5), "encode_min_ms": round(h_min, 5),
                  "encode_GBps": round(2 * n / (h_ms * 1e-3) / 1e9, 2),
                  "cache_bytes": hsz, "blocks": -(-n // B), "stream_equal_to_exact_sender": same,
                  "encode_algorithmic_bytes": alg_h,
                  "kernels": {nm: round(v, 5) for nm, v in hk.items()},
                  # its k_stats hashes every exponent word twice: VALU-bound
                  "alu_roofline": alu_roofline("k_stats<true, true, 1u>", "k_stats_hash", args.workload, B,
                                               hk["k_stats"])}
        del h_pristine, h_cache, out_h

    # rANS modes: the same input and caches, the coded exponents range-ANS
    # coded instead of the 3-bit code; encode and decode timed like pass 3,
    # each kernel once more with events; the round trip checked on the GPU.
    log("rANS modes")
    rcap, rwsz = ciera.rans_max_encoded_size(n, B), ciera.rans_workspace_size(n, B)
    out_r = torch.empty(rcap, dtype=torch.uint8, device=dev)
    ws_r = torch.empty(rwsz, dtype=torch.uint8, device=dev)
    size_r = torch.zeros(1, dtype=torch.int64, device=dev)
    y_r = torch.empty_like(y)
    if mode == "zip3":
        enc_r = ciera.bind("zip3_encode_rans", xs[k_iso], n, out_r, rcap, ws_r, rwsz, size_r, stream=stream)
    else:
        enc_r = ciera.bind("ciera_encode_rans", xs[k_iso], n, B, send, out_r, rcap, ws_r, rwsz, size_r, stream=stream)
    if restore_s is not None:
        restore_s()
    enc_r()
    torch.cuda.synchronize()
    assert ciera.ciera_read_error(ws_r) == 0
    szr = int(size_r.item())
    if mode == "zip3":
        dec_r = ciera.bind("zip3_decode_rans", out_r, szr, y_r, n, ws_d, wsz, stream=stream)
    else:
        dec_r = ciera.bind("ciera_decode_rans", out_r, szr, y_r, n, B, recv, ws_d, wsz, stream=stream)
    r_enc, r_enc_min = gpu.isolated(enc_r, restore_s)
    r_dec, r_dec_min = gpu.isolated(dec_r, restore_r)
    assert ciera.ciera_read_error(ws_r) == 0 and ciera.ciera_read_error(ws_d) == 0
    r_ok = bool(torch.equal(y_r, xs[k_iso]))
    evr = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
           for _ in range(K)]
    ciera.ciera_time_kernels([pr for row in evr for pr in row], stream=stream)
    for i in range(K):
        if restore_s is not None:
            restore_s()
            restore_r()
        torch.sum(gpu.sweep, dim=0, out=gpu.sweep_out)
        enc_r()
        dec_r()
    torch.cuda.synchronize()
    ciera.ciera_time_kernels([])
    rk = [sum(evr[i][j][0].elapsed_time(evr[i][j][1]) for i in range(K)) / K for j in range(4)]
    rans = {"encode_ms": round(r_enc, 5), "encode_min_ms": round(r_enc_min, 5),
            "decode_ms": round(r_dec, 5), "decode_min_ms": round(r_dec_min, 5),
            "stream_bytes": szr, "roundtrip_ok": r_ok,
            "compression_ratio": round(2 * n / szr, 4),
            "encode_GBps": round(2 * n / (r_enc * 1e-3) / 1e9, 2),
            "decode_GBps": round(2 * n / (r_dec * 1e-3) / 1e9, 2),
            "kernels": {"k_stats": round(rk[0], 5), "k_rans_enc": round(rk[1], 5), "k_rans_finish": round(rk[2], 5),
                        "k_rans_dec": round(rk[3], 5)},
            # the coders are bound by their dependent steps, not by HBM:
            # their VALU issue rate against the chip's
            "alu_roofline": [alu_roofline("k_rans_enc", "k_rans_enc", args.workload, B, rk[1]),
                             alu_roofline("k_rans_dec", "k_rans_dec", args.workload, B, rk[3])]}
    del out_r, ws_r, y_r

    if args.copy_probe:
        a = torch.full((args.copy_probe << 19,), 3, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.bitwise_not(a, out=b)
        torch.cuda.synchronize()
        del a, b
    del out, ws_e, ws_d, y, xs, send, recv, e_prev
    torch.cuda.empty_cache()
    bw_copy, bw_read = measured_bandwidth(torch, dev)

    in_bytes = 2 * n
    value = in_bytes * K / wall / 1e9
    enc_avg = sum(enc_ms) / K
    dec_avg = sum(dec_ms) / K
    stream_bytes = sizes[k_iso]
    ratio = in_bytes / stream_bytes

    # Algorithmic bytes per launch of each streaming kernel: what the method
    # must move.  k_stats reads x (+ the sender cache, and rewrites the
    # exponents of changed blocks); k_write reads x and writes the stream;
    # k_decode reads the stream and writes y (+ the receiver cache: read for
    # unchanged blocks, written for changed ones, n bytes in total).
    alg = {
        "k_stats": in_bytes + (n + changed_vals if mode != "zip3" else 0),
        "k_write": in_bytes + stream_bytes,
        "k_decode": stream_bytes + in_bytes + (n if mode != "zip3" else 0),
    }
    dom = max(STREAMING, key=lambda nm: kern_ms[nm])
    dom_gbps = alg[dom] / (kern_ms[dom] * 1e-3) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic(dom, args.workload, B),
                "algorithmic_bytes_per_launch": alg[dom], "avg_launch_ms": round(kern_ms[dom], 5),
                "frac_of_measured_copy": round(dom_gbps / bw_copy, 4)}
    kernels = {nm: {"avg_ms": round(kern_ms[nm], 5)} for nm in names}
    for nm, by in alg.items():
        kernels[nm]["algorithmic_bytes"] = by
        kernels[nm]["GBps"] = round(by / (kern_ms[nm] * 1e-3) / 1e9, 1)
        kernels[nm]["frac_of_hbm_peak"] = round(by / (kern_ms[nm] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)

    alg_enc = alg["k_stats"] + alg["k_write"]
    alg_dec = alg["k_decode"]
    iso = {"method": "each call alone, MALL swept by a 1 GiB read before it; median (min) of K calls",
           "encode_ms": round(enc_iso, 5), "encode_min_ms": round(enc_iso_min, 5),
           "encode_GBps": round(in_bytes / (enc_iso * 1e-3) / 1e9, 2),
           "encode_algorithmic_bytes": alg_enc,
           "encode_frac_of_hbm_peak": round(alg_enc / (enc_iso * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "encode_frac_of_measured_copy": round(alg_enc / (enc_iso * 1e-3) / 1e9 / bw_copy, 4),
           "decode_ms": round(dec_iso, 5), "decode_min_ms": round(dec_iso_min, 5),
           "decode_GBps": round(in_bytes / (dec_iso * 1e-3) / 1e9, 2),
           "decode_algorithmic_bytes": alg_dec,
           "decode_frac_of_hbm_peak": round(alg_dec / (dec_iso * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "decode_frac_of_measured_copy": round(alg_dec / (dec_iso * 1e-3) / 1e9 / bw_copy, 4),
           "decode_roundtrip_ok": iso_roundtrip,
           "floor_ms": round(floor_ms, 5), "floor_min_ms": round(floor_min, 5),
           "floor_what": "one launch of a one-element fill timed the same way"}
    # The same fractions with the bytes the HBM counters saw (FETCH_SIZE +
    # WRITE_SIZE per launch, from the traffic summaries taken on this kernel
    # source), null where no such record exists.
    cnt = {nm: load_traffic(nm, args.workload, B) for nm in enc_names + DEC_KERNELS}
    if all(cnt[nm] is not None for nm in STREAMING):
        c_enc = sum(cnt[nm] or 0 for nm in enc_names)
        iso["encode_counted_bytes"] = c_enc
        iso["encode_frac_counted"] = round(c_enc / (enc_iso * 1e-3) / 1e9 / bw_copy, 4)
        iso["decode_counted_bytes"] = cnt["k_decode"]
        iso["decode_frac_counted"] = round(cnt["k_decode"] / (dec_iso * 1e-3) / 1e9 / bw_copy, 4)
    else:
        iso["encode_frac_counted"] = iso["decode_frac_counted"] = None

    # single-read: x once [+ the cache, read, and its changed values rewritten] + the stream
    # (a small tensor's two-launch path: the full encode's bytes)
    alg_sr = alg_enc if sr_small else in_bytes + (n + changed_vals if mode != "zip3" else 0) + stream_bytes
    alg_w1 = alg["k_write"] if sr_small else alg_sr
    single = {"isolated_ms": round(sr_iso, 5), "isolated_min_ms": round(sr_iso_min, 5),
              "isolated_GBps": round(in_bytes / (sr_iso * 1e-3) / 1e9, 2),
              "isolated_algorithmic_bytes": alg_sr,
              "isolated_frac_of_hbm_peak": round(alg_sr / (sr_iso * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
              "isolated_frac_of_measured_copy": round(alg_sr / (sr_iso * 1e-3) / 1e9 / bw_copy, 4),
              "isolated_stream_equal_to_full_encode": sr_same,
              "speedup_vs_two_pass_isolated": round(enc_iso / sr_iso, 3),
              "path": ("self-planned two-launch encode with the given window (at most %d chunks)" % SELF_PLAN_CHUNKS
                       if sr_small else "k_prep1 + k_write1, one read of x"),
              "kernels": {sr_names[0]: {"avg_ms": round(prep_ms, 5)},
                          sr_names[1]: {"avg_ms": round(write1_ms, 5), "algorithmic_bytes": alg_w1,
                                        "GBps": round(alg_w1 / (write1_ms * 1e-3) / 1e9, 1),
                                        "frac_of_hbm_peak": round(alg_w1 / (write1_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                                                  4)}}}
    if hashed is not None:
        hashed["encode_frac_of_measured_copy"] = round(hashed["encode_algorithmic_bytes"] /
                                                       (hashed["encode_ms"] * 1e-3) / 1e9 / bw_copy, 4)

    # The CPU oracle: the timed encode's stream against the oracle's (same
    # input, same cache), then the oracle timed on one thread and on all the
    # host's cores.
    cpu = None
    exact = None
    threads = host_threads()
    if not args.no_cpu_baseline:
        import oracle
        log(f"oracle: single thread and {threads} threads on the full tensor")
        prev = ((pair[0] >> 7) & 0xFF).astype(np.uint8) if mode != "zip3" else None
        o_stream, legs = oracle_legs(oracle, np, pair[k_iso], B, prev, threads)
        exact = g_stream.tobytes() == o_stream.tobytes()
        a = legs["all_cores"]
        cpu = {"value": a["GBps"], "unit": "GB/s", "cores": a["threads"], "kind": "oracle",
               "sample": f"the full {n}-value tensor, one encode + one decode: the scalar C oracle's "
                         f"chunk-parallel driver on {a['threads']} threads (single_thread: the same on one)",
               "encode_GBps": a["encode_GBps"], "decode_GBps": a["decode_GBps"],
               "single_thread": legs["single"], "host_cpus": os.cpu_count()}
        del o_stream
    del g_stream

    configs = []
    spec = args.configs
    if spec == "auto":
        spec = "1,2,3:64,3:1024,4" if args.workload == 5 and not args.no_cpu_baseline else ""
    if spec:
        import oracle
        for item in spec.split(","):
            w, _, b = item.partition(":")
            w = int(w)
            c = measure_config(gpu, oracle, np, wl, w, int(b) if b else DEFAULT_B[w], threads)
            c["encode_frac_of_measured_copy"] = round(c["encode_algorithmic_bytes"] / (c["encode_ms"] * 1e-3) / 1e9 /
                                                      bw_copy, 4)
            c["decode_frac_of_measured_copy"] = round(c["decode_algorithmic_bytes"] / (c["decode_ms"] * 1e-3) / 1e9 /
                                                      bw_copy, 4)
            configs.append(c)

    line = {
        "metric": "codec encode/decode GB/s of BF16 input (% HBM roofline) + compression ratio",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload].format(B=B), "n": n, "B": B, "mode": mode},
        "bit_exact_vs_oracle": exact,
        "encode_GBps": round(in_bytes / (enc_avg * 1e-3) / 1e9, 2),
        "decode_GBps": round(in_bytes / (dec_avg * 1e-3) / 1e9, 2),
        "encode_ms": round(enc_avg, 5),
        "decode_ms": round(dec_avg, 5),
        "compression_ratio": round(ratio, 4),
        "stream_bytes": stream_bytes,
        "pass2_ms_per_step": round(wall2 * 1e3 / K, 4),
        "kernels": kernels,
        "graph_replay": graph,
        "isolated": iso,
        **({"decode_batch": batch} if batch is not None else {}),
        "hash_sender": hashed,
        "rans": rans,
        "single_read_encode": single,
        "speculative_encode": spec_leg,
        "bw_measured_GBps": {"copy": round(bw_copy, 1), "read": round(bw_read, 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "configs": configs,
        "source_hash": source_hash(),
    }
    print(json.dumps(line), flush=True)
    batches = [b for b in [batch] + [c.get("decode_batch") for c in configs] if b is not None]
    spec_bad = spec_leg is not None and not (spec_leg["stream_equal_to_full_encode"] and spec_leg["step_roundtrip_ok"]
                                             and spec_leg["wrong_hint_stream_equal_to_full_encode"])
    spec_bad = spec_bad or any(not c["speculative_encode"]["stream_equal_to_full_encode"]
                               for c in configs if "speculative_encode" in c)
    # the other modes' streams: the hash sender's equals the exact sender's,
    # the single-read encode's the full encode's, the rANS round trip holds
    modes_bad = ((hashed is not None and not hashed["stream_equal_to_exact_sender"])
                 or not sr_same or not rans["roundtrip_ok"])
    bad = (exact is False or not iso_roundtrip or spec_bad or modes_bad or any(not b["roundtrip_ok"] for b in batches)
           or any(not c["bit_exact_vs_oracle"] or not c["roundtrip_ok"] for c in configs))
    if bad:
        log("FAILED: a GPU stream differs from the oracle's or from the regular encode's, or a round trip failed")
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
