"""Parity of the HIP decoder (through the C ABI) with the CPU oracle on the
same seeded inputs: tokens and lengths bit-exact, scores within 1e-4 (and in
practice bit-identical), at sizes the oracle finishes in seconds."""
import numpy as np
import pytest
import torch

import ctc_prefix_beam_amd as cpb
import oracle
import synth
from gpu_util import assert_parity, gpu_offline

pytestmark = pytest.mark.gpu


def run_both(lp, lens, beam, nbest, blank=0, threshold=1.0, max_out_len=None, paged=False,
             page_size=16, what=""):
    T = lp.shape[1]
    mol = T if max_out_len is None else max_out_len
    print(f"[case] {what} B={lp.shape[0]} T={T} V={lp.shape[2]} W={beam} paged={paged}",
          flush=True)
    got = gpu_offline(lp, lens, beam, nbest, blank, threshold, mol, paged, page_size)
    ref = oracle.decode(lp, lens, beam, nbest, blank, threshold, mol)
    assert_parity(got, ref, what=what)
    return got, ref


@pytest.mark.parametrize("paged", [False, True])
def test_tiny(paged):
    lp, lens = synth.peaky(10, 50, 29, seed=0, p_blank=0.65)
    run_both(lp, lens, 4, 4, paged=paged, what="tiny")


@pytest.mark.parametrize("paged", [False, True])
def test_bpe256_cut(paged):
    wl = synth.WORKLOADS["bpe256"]
    lp, lens = wl.make(1, B=4, T=200)
    run_both(lp, lens, 8, 8, 0, 0.999, 200, paged, what="bpe256")


@pytest.mark.parametrize("paged", [False, True])
def test_bpe1024_ragged(paged):
    lp, lens = synth.peaky(4, 300, 1024, seed=2, p_blank=0.7, token_bias=(3.0, 8.0),
                           lengths=(100, 300), nan_tail=True)
    run_both(lp, lens, 16, 16, 0, 0.999, 256, paged, what="bpe1024")


@pytest.mark.parametrize("paged", [False, True])
def test_vocab5000_cut(paged):
    lp, lens = synth.peaky(2, 80, 5000, seed=3, p_blank=0.55, p_low=0.2)
    run_both(lp, lens, 32, 32, 0, 0.999, 64, paged, what="vocab5000")


def test_frame_skipping_active():
    # strong blank frames so that a threshold of 0.9 really skips frames
    lp, lens = synth.peaky(6, 120, 40, seed=5, p_blank=0.6, blank_bias=12.0)
    nsel = [len(oracle.select_frames(lp[b], lens[b], 0, 0.9)) for b in range(6)]
    assert min(nsel) < 100
    for paged in (False, True):
        run_both(lp, lens, 6, 6, 0, 0.9, 120, paged, what="skip")


@pytest.mark.parametrize("W,V", [(1, 29), (2, 2), (4, 2), (16, 20), (32, 40), (3, 5)])
def test_beam_vocab_corners(W, V):
    lp, lens = synth.peaky(3, 40, V, seed=W * 100 + V, p_blank=0.5)
    run_both(lp, lens, W, W, what=f"W{W}V{V}")


@pytest.mark.parametrize("W,paged", [(8, False), (16, True), (32, False)])
def test_flat_posteriors(W, paged):
    # no blank or token peaks (plain Gaussian logits): in about a third of the
    # steps the beams' best candidates leave beam order or second candidates
    # compete, and the step takes the sorting network and the selection fallbacks
    lp, lens = synth.peaky(3, 60, 300, seed=40 + W, p_blank=0.1, blank_bias=0.0, token_bias=0.0)
    run_both(lp, lens, W, W, paged=paged, what=f"flat W{W}")


def uniform_frames(B, T, V, seed, frac):
    """Peaky frames, a fraction `frac` of them replaced by frames in which every
    non-blank label has the same log-probability."""
    lp, lens = synth.peaky(B, T, V, seed=seed, p_blank=0.5)
    rng = np.random.default_rng(seed + 1)
    pick = rng.random((B, T)) < frac
    flat = np.full(V, np.log(0.999 / (V - 1)), np.float32)   # blank below every label
    flat[0] = np.float32(np.log(0.001))
    lp[pick] = flat
    return lp, lens


@pytest.mark.parametrize("W,paged", [(8, False), (32, True)])
def test_exact_selection_on_uniform_frames(W, paged):
    # labels past the ranked list tie with ranked ones, so the pruned candidate
    # set cannot be shown to hold the top W: the full beam x vocabulary
    # selection decides those steps (its log-probs come from the frame in
    # global memory, the slot having been handed back at the top of the step)
    lp, lens = uniform_frames(3, 50, 120, seed=60 + W, frac=0.3)
    run_both(lp, lens, W, W, paged=paged, what=f"uniform W{W}")
    fb = int(gpu_offline.last_stats[:, cpb.STAT_FIELDS.index("fallbacks")].sum())
    assert fb > 0, "no step took the full selection"


def test_blank_not_zero_and_truncation():
    lp, lens = synth.peaky(3, 70, 33, seed=8, p_blank=0.5, blank=32)
    run_both(lp, lens, 5, 3, blank=32, max_out_len=6, what="blank32")
    run_both(lp, lens, 5, 5, blank=32, max_out_len=0, what="mol0")


def test_empty_rows_and_thresholds():
    lp, _ = synth.peaky(4, 30, 12, seed=9)
    lens = np.array([0, 30, 7, 1], np.int32)
    for thr in (0.0, -1.0, 0.5, 1.0, 2.0):
        run_both(lp, lens, 4, 4, 0, thr, 30, what=f"thr{thr}")


def test_noncontiguous_rows():
    lp, lens = synth.peaky(3, 40, 64, seed=10)
    big = np.full((3, 50, 80), np.nan, np.float32)
    big[:, :40, :64] = lp
    x = torch.from_numpy(big)[:, :40, :64]          # stride_b = 4000, stride_t = 80
    got = gpu_offline(x, lens, 6, 6, 0, 1.0, 40)
    ref = oracle.decode(lp, lens, 6, 6, 0, 1.0, 40)
    assert_parity(got, ref, what="strided")


def test_flat_equals_paged_and_page_sizes():
    lp, lens = synth.peaky(4, 150, 300, seed=11, p_blank=0.5)
    base = gpu_offline(lp, lens, 12, 12, 0, 1.0, 150)
    for ps in (4, 8, 16, 64):
        other = gpu_offline(lp, lens, 12, 12, 0, 1.0, 150, paged=True, page_size=ps)
        for a, b in zip(base, other):
            assert np.array_equal(a, b), ps


def test_repeat_runs_are_bitwise_identical():
    lp, lens = synth.peaky(8, 200, 700, seed=12, p_blank=0.5, p_low=0.3)
    first = gpu_offline(lp, lens, 24, 24, 0, 1.0, 200, paged=True)
    for _ in range(3):
        again = gpu_offline(lp, lens, 24, 24, 0, 1.0, 200, paged=True)
        for a, b in zip(first, again):
            assert np.array_equal(a, b)


def test_offline_decode_replayed_from_a_captured_graph():
    # frame selection + decode captured once (workspace and outputs allocated
    # beforehand), replayed with eager work in between: every replay equals
    # the eager decode and the oracle
    lp, lens = synth.peaky(4, 120, 300, seed=97, p_blank=0.6)
    print("[case] offline graph B=4 T=120 V=300 W=8", flush=True)
    dec = cpb.OfflineDecoder(cpb.DecoderConfig(beam=8, nbest=8, blank_threshold=0.9,
                                               max_out_len=120))
    x = torch.from_numpy(lp).cuda()
    ld = torch.from_numpy(lens).cuda()
    out = dec.decode(x, ld)
    eager = tuple(t.cpu().numpy().copy() for t in out)
    assert_parity(eager, oracle.decode(lp, lens, 8, 8, 0, 0.9, 120), what="graph eager")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dec.decode(x, ld, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in out:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, eager):
            assert np.array_equal(a.cpu().numpy(), b), rep


def test_bounded_page_pool():
    # pages come from a pool of num_pages per row.  The high-water mark a
    # decode reports per row is exactly what that row needs: a row whose mark
    # fits the pool decodes as with the default pool, a row whose mark does
    # not runs out, which sets its status bit 0 (its outputs are then
    # unspecified) and leaves the other rows untouched
    lp, lens = synth.peaky(6, 240, 300, seed=98, p_blank=0.4)
    lens[:] = [240, 200, 160, 120, 80, 40]
    print("[case] bounded pool B=6 T=240 V=300 W=16 ps=8", flush=True)
    # a pool the caller sizes (here the default's size, given explicitly)
    # follows the page's allocator exactly; the default pool appends in place
    # where only the source row also holds the page, which needs fewer pages
    loose = gpu_offline(lp, lens, 16, 16, 0, 1.0, 240, paged=True, page_size=8)
    loose_high = gpu_offline.last_stats[:, 3].copy()
    full = gpu_offline(lp, lens, 16, 16, 0, 1.0, 240, paged=True, page_size=8,
                       num_pages=16 * (240 // 8 + 1))
    high = gpu_offline.last_stats[:, 3].copy()
    assert (loose_high <= high).all()
    assert all(np.array_equal(a, b) for a, b in zip(loose, full))
    assert (gpu_offline.last_stats[:, 2] == 0).all()
    assert_parity(full, oracle.decode(lp, lens, 16, 16, 0, 1.0, 240), what="bounded pool")
    # the marks are those of the page's allocator as the oracle models it
    # (sec. 3.4.5 fork / copy-on-write, sec. 4.2 alloc_page)
    assert list(high) == list(oracle.decode_pages(lp, lens, 16, page_size=8)[:, 0])
    assert high.min() < high.max()
    npages = int(np.median(high))
    fits = high <= npages
    assert fits.any() and (~fits).any()
    got = gpu_offline(lp, lens, 16, 16, 0, 1.0, 240, paged=True, page_size=8, num_pages=npages,
                      check_status=False)
    st = gpu_offline.last_stats
    assert np.array_equal(st[:, 2] & 1, (~fits).astype(st.dtype))
    dry = oracle.decode_pages(lp, lens, 16, page_size=8, num_pages=npages)[:, 1]
    assert np.array_equal(st[:, 2] & 1, dry.astype(st.dtype))
    for b in np.nonzero(fits)[0]:
        for a, e in zip(got, full):
            assert np.array_equal(a[b], e[b])
    # a pool of exactly the largest mark is enough for every row
    got = gpu_offline(lp, lens, 16, 16, 0, 1.0, 240, paged=True, page_size=8,
                      num_pages=int(high.max()))
    assert (gpu_offline.last_stats[:, 2] == 0).all()
    assert np.array_equal(gpu_offline.last_stats[:, 3], high)
    for a, e in zip(got, full):
        assert np.array_equal(a, e)


@pytest.mark.parametrize("W,ps,theta", [(1, 4, 1.0), (2, 8, 0.9), (4, 4, 1.0), (10, 16, 0.9),
                                         (32, 64, 1.0), (32, 4, 0.95)])
def test_page_counts_equal_the_page_allocator(W, ps, theta):
    # pages in use at most per row (paged storage, beams up to 32) against the
    # oracle's model of the page's allocator, and the same rows running dry in
    # a pool one page short of the largest mark
    lp, lens = synth.peaky(4, 150, 200, seed=160 + W + ps, p_blank=0.5, lengths=(40, 150))
    print(f"[case] page counts W={W} ps={ps} theta={theta}", flush=True)
    got = gpu_offline(lp, lens, W, W, 0, theta, 150, paged=True, page_size=ps,
                      num_pages=W * (-(-150 // ps) + 1))
    high = gpu_offline.last_stats[:, 3].copy()
    model = oracle.decode_pages(lp, lens, W, threshold=theta, page_size=ps)
    assert list(high) == list(model[:, 0])
    assert_parity(got, oracle.decode(lp, lens, W, W, 0, theta, 150), what="page counts")
    n = int(high.max()) - 1
    gpu_offline(lp, lens, W, W, 0, theta, 150, paged=True, page_size=ps, num_pages=n,
                check_status=False)
    dry = oracle.decode_pages(lp, lens, W, threshold=theta, page_size=ps, num_pages=n)[:, 1]
    assert list(gpu_offline.last_stats[:, 2] & 1) == list(dry) and dry.any()


def test_exact_selection_every_step_at_vocab5000():
    # frames uniform over every label (the blank included) at beam 32, V =
    # 5000: candidates tie across the list boundary, so the ranked list cannot
    # bound the unlisted labels and the full beam x vocabulary selection
    # decides the steps; the oracle decides what is right
    B, T, V, W = 2, 40, 5000, 32
    lp, lens = synth.peaky(B, T, V, seed=61, p_blank=0.5)
    lp[:, 1:] = np.float32(np.log(1.0 / V))   # frame 0 peaky (distinct per row), then uniform
    print(f"[case] uniform every step B={B} T={T} V={V} W={W}", flush=True)
    got = gpu_offline(lp, lens, W, W, 0, 1.0, T)
    fb = gpu_offline.last_stats[:, cpb.STAT_FIELDS.index("fallbacks")]
    assert_parity(got, oracle.decode(lp, lens, W, W, 0, 1.0, T), what="uniform every step")
    assert (fb >= T // 4).all(), fb        # about a third of the steps


@pytest.mark.parametrize("beam,V,n_tied,paged", [(2, 8, 4, False), (2, 8, 4, True), (3, 10, 5, False),
                                                 (4, 12, 6, False), (8, 24, 12, False)])
def test_rounding_ties_across_the_checked_candidates(beam, V, n_tied, paged):
    # extensions whose sums round to one score rank by id, not by log-prob:
    # the tie runs past the candidates each beam sends to the sort, so only a
    # score-level bound on the ones left out keeps the selection exact
    lp = synth.rounding_ties(V=V, n_tied=n_tied)
    got, ref = run_both(lp, np.array([2], np.int32), beam, beam, paged=paged, what="rounding ties")
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
