"""Seeded random configurations against the oracle: beam, vocabulary, blank id,
threshold, storage, page size, frame lengths and streaming chunkings drawn
from one generator, so that combinations no hand-written case covers are
exercised.  Every case prints its parameters before it runs.  The number of
cases can be raised with CTCPB_RANDOM_CASES (offline; a tenth of it for
streaming) for a longer sweep."""
import os

import numpy as np
import pytest
import torch

import ctc_prefix_beam_amd as cpb
import oracle
import synth
from gpu_util import assert_parity, gpu_offline

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    W = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 24, 31, 32, 40, 77, 128]))
    V = int(rng.choice([2, 3, 7, 29, 64, 100, 257, 640, 1500]))
    B = int(rng.integers(1, 5))
    T = int(rng.integers(1, 70))
    blank = int(rng.integers(0, V)) if rng.random() < 0.3 else 0
    theta = float(rng.choice([1.0, 0.99, 0.9, 0.6, 0.0]))
    paged = bool(rng.random() < 0.5)
    ps = int(rng.choice([4, 8, 16, 64]))
    N = int(rng.integers(1, W + 1))
    mol = int(rng.choice([0, 3, T]))
    p_blank = float(rng.choice([0.1, 0.5, 0.8]))
    return dict(W=W, V=V, B=B, T=T, blank=blank, theta=theta, paged=paged, ps=ps, N=N, mol=mol,
                p_blank=p_blank, seed=seed)


N_OFFLINE = int(os.environ.get("CTCPB_RANDOM_CASES", "48"))
N_STREAMING = max(16, N_OFFLINE // 10)


@pytest.mark.parametrize("seed", range(N_OFFLINE))
def test_random_offline(seed):
    c = draw(seed)
    print(f"[case] random offline {c}", flush=True)
    lp, _ = synth.peaky(c["B"], c["T"], c["V"], seed=2000 + seed, p_blank=c["p_blank"],
                        blank=c["blank"])
    lens = np.random.default_rng(3000 + seed).integers(0, c["T"] + 1, size=c["B"]).astype(np.int32)
    got = gpu_offline(lp, lens, c["W"], c["N"], c["blank"], c["theta"], c["mol"], c["paged"],
                      c["ps"])
    ref = oracle.decode(lp, lens, c["W"], c["N"], c["blank"], c["theta"], c["mol"])
    assert_parity(got, ref, what=f"random {seed}")


@pytest.mark.parametrize("seed", range(N_STREAMING))
def test_random_streaming(seed):
    c = draw(100 + seed)
    W = c["W"]   # beams above 32 run on the wide decoder, streaming too
    N = min(c["N"], W)
    T = max(c["T"], 2)
    print(f"[case] random streaming {c}", flush=True)
    lp, _ = synth.peaky(c["B"], T, c["V"], seed=4000 + seed, p_blank=c["p_blank"],
                        blank=c["blank"])
    rng = np.random.default_rng(5000 + seed)
    mask = (rng.random((c["B"], T)) < 0.75).astype(np.uint8) if seed % 2 else None
    cuts = sorted(set(rng.integers(1, T, size=3).tolist()))
    bounds = [0] + cuts + [T]
    # the state sized for the session (the default 4096-token capacity with small
    # pages needs more LDS than a CU has for paged metadata)
    cfg = cpb.DecoderConfig(beam=W, nbest=N, blank_id=c["blank"], max_out_len=T, capacity=T,
                            paged=c["paged"], page_size=c["ps"])
    pool = cpb.StreamPool(cfg, c["V"], c["B"])
    x = torch.from_numpy(lp).cuda()
    m = torch.from_numpy(mask).cuda() if mask is not None else None
    for a, b in zip(bounds[:-1], bounds[1:]):
        pool.chunk(x[:, a:b], is_speech=None if m is None else m[:, a:b].contiguous())
    t, l, s = pool.read()
    st = pool.row_stats().cpu().numpy()
    torch.cuda.synchronize()
    assert (st[:, 2] == 0).all()
    got = (t.cpu().numpy(), l.cpu().numpy(), s.cpu().numpy())
    outs = []
    for r in range(c["B"]):
        so = oracle.Stream(W, c["V"], c["blank"], capacity=T)
        for a, b in zip(bounds[:-1], bounds[1:]):
            so.feed(lp[r, a:b], None if mask is None else mask[r, a:b])
        outs.append(so.read(N, T))
    ref = tuple(np.stack([o[i] for o in outs]) for i in range(3))
    assert_parity(got, ref, what=f"random stream {seed}")
