"""Beams of 33..128 slots (the wide offline decoder) against the oracle, through
the C ABI: tokens and lengths exact, scores within 1e-4 (bitwise where the
hypotheses coincide)."""
import numpy as np
import pytest

import ctc_prefix_beam_amd as cpb
import oracle
import synth
from gpu_util import assert_parity, gpu_offline

pytestmark = pytest.mark.gpu


def run_both(lp, lens, W, N, threshold=1.0, blank=0, max_out_len=None, what=""):
    T = lp.shape[1]
    mol = T if max_out_len is None else max_out_len
    print(f"[case] wide {what} B={lp.shape[0]} T={T} V={lp.shape[2]} W={W}", flush=True)
    got = gpu_offline(lp, lens, W, N, blank, threshold, mol)
    ref = oracle.decode(lp, lens, W, N, blank, threshold, mol)
    assert_parity(got, ref, what=what)
    return got


@pytest.mark.parametrize("W", [33, 48, 64, 100, 128])
def test_wide_beams(W):
    lp, lens = synth.peaky(3, 60, 300, seed=70 + W, p_blank=0.5)
    run_both(lp, lens, W, W, what=f"W{W}")


@pytest.mark.parametrize("W,theta", [(40, 0.9), (128, 0.95)])
def test_wide_beams_with_frame_skipping(W, theta):
    lp, lens = synth.peaky(3, 80, 200, seed=80 + W, p_blank=0.6)
    nsel = [len(oracle.select_frames(lp[b], lens[b], 0, theta)) for b in range(3)]
    assert min(nsel) < 80
    run_both(lp, lens, W, 16, threshold=theta, what=f"skip W{W}")


def test_wide_beams_narrow_vocabulary_and_ragged_rows():
    # fewer labels than slots: dead slots stay dead; ragged and empty rows
    lp, _ = synth.peaky(4, 50, 20, seed=90, p_blank=0.4)
    lens = np.array([50, 0, 17, 1], np.int32)
    run_both(lp, lens, 64, 64, what="narrow vocab")


def test_wide_beams_flat_and_uniform_frames():
    # flat posteriors (beams far from beam order) and exact ties
    lp, lens = synth.peaky(3, 40, 150, seed=91, p_blank=0.1, blank_bias=0.0, token_bias=0.0)
    flat = np.full(150, np.log(0.999 / 149), np.float32)
    flat[0] = np.float32(np.log(0.001))
    lp[:, ::3] = flat
    run_both(lp, lens, 96, 32, what="flat/uniform")


def test_wide_beams_blank_not_zero_truncation_and_repeat():
    lp, lens = synth.peaky(2, 70, 40, seed=92, p_blank=0.5, blank=39)
    a = run_both(lp, lens, 50, 10, blank=39, max_out_len=5, what="blank39")
    b = gpu_offline(lp, lens, 50, 10, 39, 1.0, 5)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_wide_beams_larger_vocabulary():
    lp, lens = synth.peaky(2, 120, 1024, seed=93, p_blank=0.7)
    run_both(lp, lens, 64, 64, what="V1024")
    st = gpu_offline.last_stats
    assert (st[:, 0] == 120).all() and (st[:, 2] == 0).all()


def test_wide_beam_bpe1024_full_size_sampled():
    # the bpe1024 inputs at full size (B=64, T=875, ragged) with beam 64, in the
    # launch the benchmark times; rows sampled against the oracle
    wl = synth.WORKLOADS["bpe1024"]
    x, lens = wl.make_device(0, "cuda")
    W = 64
    print(f"[case] wide bpe1024 full B={wl.B} T={wl.T} W={W}", flush=True)
    got = gpu_offline(x, lens, W, W, 0, wl.threshold, wl.max_out_len)
    rows = [5, 40]
    lp = x[rows].cpu().numpy()
    ref = oracle.decode(lp, lens[rows], W, W, 0, wl.threshold, wl.max_out_len)
    assert_parity(tuple(g[rows] for g in got), ref, what="wide bpe1024")
