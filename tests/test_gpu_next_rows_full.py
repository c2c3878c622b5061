"""Full-size oracle parity of the next rows on the workloads their other
tests do not reach: the single-read encode (ciera_encode_e0) on the
DeepSeek-like ten-iteration chain and on the 10^9-value stress buffer, the
hash sender on the stress buffer, and the rANS modes on the 2^20-value
shard, the DeepSeek-like chain and the stress buffer.  Each compares the
stream bytes, the caches (or the hash cache) and the decoded values with
the oracle's (CIERA page, section 3.1: exponent reuse with a block-hash
sender and ANS-coded changed exponents; ZipCCL digest, section 3.1: the
3-bit code)."""
import numpy as np
import pytest

import oracle
from gpu_util import (check_encode_e0_ciera, check_encode_hashed, check_rans, check_roundtrip, exps,
                      gpu_decode_rans, gpu_encode_e0_ciera, gpu_encode_rans, require_gpu, say)
from lossless_bf16_tensor_exp_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def stress():
    d = wl.workload5()
    return d["iters"][0], d["iters"][1], d["B"][0]


def test_single_read_deepseek_like_chain():
    """Ten iterations, each window base taken on the device from byte 7 of
    the previous iteration's stream (the first from the oracle's window of
    x0), caches persistent on both sides."""
    d = wl.workload4()
    it = d["iters"]
    B = d["B"][0]
    say(f"single-read deepseek-like chain n={it[0].size} B={B}")
    send = np.zeros(it[0].size, dtype=np.uint8)
    recv = send.copy()
    e0 = oracle.choose_e0(it[0])
    for t, x in enumerate(it):
        s = check_encode_e0_ciera(x, B, send, e0)
        recv = check_roundtrip(s, x, B, recv)
        send = exps(x)
        e0 = int(s[7])
        say(f"  iter {t} E0={e0}")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_single_read_stress_billion(stress):
    x0, x1, B = stress
    e0 = oracle.choose_e0(x1)
    say(f"single-read stress n={x1.size} B={B} E0={e0}")
    s = check_encode_e0_ciera(x1, B, exps(x0), e0)
    check_roundtrip(s, x1, B, exps(x0))
    # the window of the previous iteration, read from a stream on the device
    prev_e0 = oracle.choose_e0(x0)
    src = torch.tensor([0] * 7 + [prev_e0], dtype=torch.uint8, device="cuda")
    g, st, gc = gpu_encode_e0_ciera(x1, B, exps(x0), src, e0_offset=7)
    assert st == 0
    o_cache = exps(x0)
    o, _ = oracle.encode(x1, B, o_cache, prev_e0, threads=16)
    assert g.tobytes() == o.tobytes() and np.array_equal(gc, o_cache)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_hash_sender_stress_billion(stress):
    x0, x1, B = stress
    say(f"hash sender stress n={x1.size} B={B}")
    check_encode_hashed(x1, B, exps(x0))


def test_rans_shard_iteration():
    d = wl.workload1()
    x0, x1 = d["iters"]
    B = d["B"][0]
    say(f"rans shard n={x0.size} B={B}")
    check_rans(x0, B, np.zeros(x0.size, dtype=np.uint8))
    s = check_rans(x1, B, exps(x0))
    say(f"  rANS ratio {2 * x1.size / s.size:.4f}")


def test_rans_deepseek_like_chain():
    d = wl.workload4()
    it = d["iters"]
    B = d["B"][0]
    say(f"rans deepseek-like chain n={it[0].size} B={B}")
    send = np.zeros(it[0].size, dtype=np.uint8)
    for t, x in enumerate(it):
        s = check_rans(x, B, send)
        send = exps(x)
        say(f"  iter {t} ratio {2 * x.size / s.size:.4f}")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_rans_stress_billion(stress):
    x0, x1, B = stress
    say(f"rans stress n={x1.size} B={B}")
    g, gc = gpu_encode_rans(x1, B, exps(x0))
    oc = exps(x0)
    o, _ = oracle.encode_rans(x1, B, oc)
    assert g.tobytes() == o.tobytes(), "rANS stream differs from the oracle's"
    assert np.array_equal(gc, oc)
    y, rc, st = gpu_decode_rans(g, x1.size, B, exps(x0))
    assert st == 0 and np.array_equal(y, x1) and np.array_equal(rc, exps(x1))
    say(f"  rANS ratio {2 * x1.size / g.size:.4f}")
