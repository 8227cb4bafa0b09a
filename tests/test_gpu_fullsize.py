"""The five workloads at full size, in the launch configuration the benchmark
times (one call for the whole batch / all streams): sampled rows against the
oracle, every row against the cross-path identities (flat = paged, streaming
= offline)."""
import numpy as np
import pytest
import torch

import ctc_prefix_beam_amd as cpb
import oracle
import synth
from gpu_util import assert_parity, gpu_offline

pytestmark = pytest.mark.gpu


def sampled_oracle(lp_dev, lens, rows, wl, mol):
    lp = lp_dev[rows].cpu().numpy()
    return oracle.decode(lp, lens[rows], wl.beam, wl.nbest, 0, wl.threshold, mol)


def subset(got, rows):
    return tuple(g[rows] for g in got)


def test_bpe256_full_all_rows():
    wl = synth.WORKLOADS["bpe256"]
    lp, lens = wl.make(0)
    print(f"[case] bpe256 full B={wl.B}", flush=True)
    got = gpu_offline(lp, lens, wl.beam, wl.nbest, 0, wl.threshold, wl.max_out_len)
    ref = oracle.decode(lp, lens, wl.beam, wl.nbest, 0, wl.threshold, wl.max_out_len)
    assert_parity(got, ref, what="bpe256")


def test_bpe1024_full_sampled():
    wl = synth.WORKLOADS["bpe1024"]
    x, lens = wl.make_device(0, "cuda")
    print(f"[case] bpe1024 full B={wl.B} T={wl.T}", flush=True)
    got = gpu_offline(x, lens, wl.beam, wl.nbest, 0, wl.threshold, wl.max_out_len)
    rows = [0, 17, 42, 63]
    ref = sampled_oracle(x, lens, rows, wl, wl.max_out_len)
    assert_parity(subset(got, rows), ref, what="bpe1024")
    paged = gpu_offline(x, lens, wl.beam, wl.nbest, 0, wl.threshold, wl.max_out_len, paged=True)
    for a, b in zip(got, paged):
        assert np.array_equal(a, b)


def test_vocab5000_full_sampled_flat_and_paged():
    wl = synth.WORKLOADS["vocab5000"]
    x, lens = wl.make_device(0, "cuda")
    print(f"[case] vocab5000 full B={wl.B} T={wl.T} V={wl.V}", flush=True)
    paged = gpu_offline(x, lens, wl.beam, wl.nbest, 0, wl.threshold, wl.max_out_len, paged=True)
    flat = gpu_offline(x, lens, wl.beam, wl.nbest, 0, wl.threshold, wl.max_out_len)
    for a, b in zip(flat, paged):
        assert np.array_equal(a, b)
    rows = [77]
    ref = sampled_oracle(x, lens, rows, wl, wl.max_out_len)
    assert_parity(subset(paged, rows), ref, what="vocab5000")
    # best paths are longer than the 512-token output: lengths report the full count
    assert (paged[1][:, 0] > wl.max_out_len).all()


def test_stream512_full_sampled():
    wl = synth.WORKLOADS["stream512"]
    x, _ = wl.make_device(0, "cuda")
    print(f"[case] stream512 full S={wl.B} chunks={wl.T // wl.chunk}", flush=True)
    pool = cpb.StreamPool(cpb.DecoderConfig(beam=wl.beam, nbest=wl.nbest, max_out_len=wl.T),
                          wl.V, wl.B)
    for a in range(0, wl.T, wl.chunk):
        pool.chunk(x[:, a:a + wl.chunk])
    t, l, s = pool.read()
    torch.cuda.synchronize()
    got = (t.cpu().numpy(), l.cpu().numpy(), s.cpu().numpy())
    rows = [0, 255]
    lp = x[rows].cpu().numpy()
    outs = []
    for i in range(len(rows)):
        st = oracle.Stream(wl.beam, wl.V, 0, 4096)
        for a in range(0, wl.T, wl.chunk):
            st.feed(lp[i, a:a + wl.chunk])
        outs.append(st.read(wl.nbest, wl.T))
    ref = tuple(np.stack([o[i] for o in outs]) for i in range(3))
    assert_parity(subset(got, rows), ref, what="stream512")
    off = gpu_offline(x, np.full(wl.B, wl.T, np.int32), wl.beam, wl.nbest, 0, 1.0, wl.T)
    for a, b in zip(got, off):
        assert np.array_equal(a, b)
