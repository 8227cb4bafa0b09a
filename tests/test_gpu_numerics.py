"""The decoder's float32 numerics on the GPU, bit for bit against the oracle.

The decoder and the oracle implement one written operation sequence each for
exp on [-80, 0] (Cody & Waite reduction, degree-7 Taylor polynomial), log1p on
[0, 1] (2 atanh(x / (2 + x)) series) and logsumexp (max + log1p(exp(min -
max)), the correction dropped below -80).  The parity tests demand scores that
are bitwise equal to the oracle's, which holds only if the two sequences agree
on every input the decode can produce.  Here every float32 of [-80, 0] (exp)
and of [0, 1] (log1p, and the quotient x / (2 + x) that the device computes
without a division) is run through the device code (tests/probe_hip, compiled
from the decoder's own header with the decoder's flags) and compared with the
oracle's C functions and with the IEEE quotient; logsumexp is compared on
seeded pairs that cover its special cases."""
import os

import numpy as np
import pytest
import torch

import oracle
import probe_hip

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26
THREADS = max(1, min(16, os.cpu_count() or 1))


def f32bits(x):
    return int(np.array([x], np.float32).view(np.uint32)[0])


# every float of the domain, as a range of bit patterns (inclusive)
DOMAINS = {
    "exp": (0, f32bits(-0.0), f32bits(-80.0)),      # -0.0 .. -80.0 (magnitudes increase)
    "log1p": (1, f32bits(0.0), f32bits(1.0)),
    "quot": (2, f32bits(0.0), f32bits(1.0)),
}


def run_gpu(op, first, n, out, a=None, b=None):
    st = torch.cuda.current_stream().cuda_stream
    rc = probe_hip.lib().math_probe(op, first, n, None if a is None else a.data_ptr(),
                                    None if b is None else b.data_ptr(), out.data_ptr(), st)
    assert rc == 0, rc


@pytest.mark.parametrize("name", list(DOMAINS))
def test_every_float_of_the_domain_is_bitwise_equal(oracle_lib, name):
    op, lo, hi = DOMAINS[name]
    total = hi - lo + 1
    print(f"[case] numerics {name}: {total} floats", flush=True)
    out = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    bad = 0
    first_bad = None
    for start in range(lo, hi + 1, CHUNK):
        n = min(CHUNK, hi + 1 - start)
        run_gpu(op, start, n, out)
        gpu = out[:n].cpu().numpy().view(np.uint32)
        cpu = oracle.math_sweep(op, start, n, threads=THREADS).view(np.uint32)
        diff = np.nonzero(gpu != cpu)[0]
        if diff.size:
            bad += diff.size
            if first_bad is None:
                i = int(diff[0])
                x = np.array([start + i], np.uint32).view(np.float32)[0]
                first_bad = (float(x), hex(int(gpu[i])), hex(int(cpu[i])))
    assert bad == 0, f"{name}: {bad} of {total} floats differ; first (x, gpu, oracle) {first_bad}"


def lse_pairs(n, seed=0):
    rng = np.random.default_rng(seed)
    m = -np.abs(rng.normal(0.0, 300.0, n)).astype(np.float32)
    d = -(rng.random(n) * 100.0).astype(np.float32)             # differences in [-100, 0]
    a = m
    b = (m + d).astype(np.float32)
    swap = rng.random(n) < 0.5
    a, b = np.where(swap, b, a), np.where(swap, a, b)
    neg = np.float32(-np.finfo(np.float32).max)
    k = n // 16
    # special cases: NEG on either side or both, equal operands, signed zeros,
    # differences at and just past -80, scores near the bottom of the range
    a[:k], b[:k] = neg, m[:k]
    a[k:2 * k], b[k:2 * k] = m[k:2 * k], neg
    a[2 * k:3 * k], b[2 * k:3 * k] = neg, neg
    a[3 * k:4 * k], b[3 * k:4 * k] = m[3 * k:4 * k], m[3 * k:4 * k]
    a[4 * k:5 * k], b[4 * k:5 * k] = np.float32(0.0), np.float32(-0.0)
    e = (m[5 * k:6 * k] - np.float32(80.0)).astype(np.float32)
    a[5 * k:6 * k], b[5 * k:6 * k] = m[5 * k:6 * k], e
    e2 = np.nextafter(e, np.float32(-np.inf)).astype(np.float32)
    a[6 * k:7 * k], b[6 * k:7 * k] = e2, m[6 * k:7 * k]
    a[7 * k:8 * k] = (neg * np.float32(0.999) + m[7 * k:8 * k]).astype(np.float32)
    return a.astype(np.float32), b.astype(np.float32)


def test_lse_is_bitwise_equal(oracle_lib):
    n = 1 << 24
    a, b = lse_pairs(n)
    print(f"[case] numerics lse: {n} pairs", flush=True)
    ad, bd = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    run_gpu(3, 0, n, out, ad, bd)
    gpu = out.cpu().numpy()
    cpu = oracle.math_sweep(3, 0, n, a, b, threads=THREADS)
    diff = np.nonzero(gpu.view(np.uint32) != cpu.view(np.uint32))[0]
    assert diff.size == 0, (f"{diff.size} pairs differ; first: a={a[diff[0]]!r} b={b[diff[0]]!r} "
                            f"gpu={gpu[diff[0]]!r} oracle={cpu[diff[0]]!r}")
    # and the identities the decode relies on hold on the GPU too
    neg = np.float32(-np.finfo(np.float32).max)
    assert (gpu[:n // 16] == b[:n // 16]).all()                     # lse(NEG, x) == x
    assert (gpu[2 * (n // 16):3 * (n // 16)] == neg).all()          # lse(NEG, NEG) == NEG
