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


# ------------------------------------------------- streaming, beams 33..128 --
def oracle_streams(lp, W, capacity, cuts, nbest, mol, masks=None, starts=None):
    outs = []
    for s in range(lp.shape[0]):
        st = oracle.Stream(W, lp.shape[2], 0, capacity)
        for i, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
            m = None if masks is None else masks[s, a:b]
            sf = None if (starts is None or i > 0) else int(starts[s])
            st.feed(lp[s, a:b], m, sf)
        outs.append(st.read(nbest, mol))
    return tuple(np.stack([o[i] for o in outs]) for i in range(3))


def pool_read(pool, rows=None):
    import torch
    t, l, s = pool.read(rows)
    st = pool.row_stats().cpu().numpy()
    torch.cuda.synchronize()
    assert (st[:, 2] == 0).all()
    return t.cpu().numpy(), l.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("W,cuts", [(40, [0, 16, 32, 48, 64, 80]), (64, [0, 1, 17, 40, 41, 80]),
                                    (128, [0, 30, 80])])
def test_wide_beams_streaming_equals_oracle_and_offline(W, cuts):
    import torch
    S, T, V = 4, 80, 200
    lp, _ = synth.peaky(S, T, V, seed=90 + W, p_blank=0.55)
    print(f"[case] wide stream W={W} S={S} T={T} V={V} cuts={cuts}", flush=True)
    pool = cpb.StreamPool(cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T), V, S)
    x = torch.from_numpy(lp).cuda()
    fresh = pool_read(pool)
    assert (fresh[1] == 0).all() and (fresh[2][:, 0] == 0).all()
    for a, b in zip(cuts[:-1], cuts[1:]):
        pool.chunk(x[:, a:b])
        if a == cuts[1]:
            # read midway: non-mutating, and equal to the oracle there
            mid = pool_read(pool)
            assert_parity(mid, oracle_streams(lp, W, 4096, cuts[:3], W, T), what="wide mid")
    got = pool_read(pool)
    assert_parity(got, oracle_streams(lp, W, 4096, cuts, W, T), what=f"wide stream W{W}")
    off = gpu_offline(lp, np.full(S, T, np.int32), W, W, 0, 1.0, T)
    for g, o in zip(got, off):
        assert np.array_equal(g, o)


def test_wide_beams_streaming_mask_start_frames_capacity_and_reset():
    import torch
    S, T, V, W, CH, CAP = 4, 64, 120, 48, 16, 40
    lp, _ = synth.peaky(S, T, V, seed=97, p_blank=0.5)
    mask = (np.random.default_rng(98).random((S, T)) < 0.75).astype(np.uint8)
    mask[1, :20] = 0                 # first decoded frame > 0: seeded under the gap rule
    start = np.array([0, 3, 50, 9], np.int32)
    print(f"[case] wide stream mask W={W} cap={CAP}", flush=True)
    pool = cpb.StreamPool(cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T, capacity=CAP), V, S)
    x = torch.from_numpy(lp).cuda()
    m = torch.from_numpy(mask).cuda()
    rows = torch.tensor([2, 0, 3, 1], dtype=torch.int32, device="cuda")
    perm = [2, 0, 3, 1]   # chunk row i continues stream perm[i]
    for a in range(0, T, CH):
        sf = torch.from_numpy(start[perm]).cuda() if a == 0 else None
        pool.chunk(x[perm, a:a + CH], rows=rows, is_speech=m[perm, a:a + CH].contiguous(),
                   start_frame=sf)
    got = pool_read(pool)
    ref = oracle_streams(lp, W, CAP, list(range(0, T + 1, CH)), W, T, masks=mask, starts=start)
    assert_parity(got, ref, what="wide stream mask")
    st = pool.row_stats().cpu().numpy()
    assert list(st[:, 0]) == [min(CAP, int(mask[s].sum())) for s in range(S)]
    assert list(st[:, 1]) == list(start + T)
    # reset stream 1 and feed it stream 3's frames, unmasked
    one = torch.tensor([1], dtype=torch.int32, device="cuda")
    pool.reset(one)
    for a in range(0, T, CH):
        pool.chunk(x[[3], a:a + CH], rows=one)
    t, l, s = pool.read(one)
    ref = oracle_streams(lp[[3]], W, CAP, list(range(0, T + 1, CH)), W, T)
    assert_parity((t.cpu().numpy(), l.cpu().numpy(), s.cpu().numpy()), ref, what="wide reset")


def test_wide_beams_per_frame_step():
    import torch
    S, T, V, W = 3, 30, 60, 36
    lp, _ = synth.peaky(S, T, V, seed=99)
    idx = (np.cumsum(np.random.default_rng(100).integers(1, 4, size=(S, T)), axis=1) - 1).astype(
        np.int32)
    pool = cpb.StreamPool(cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T), V, S)
    x = torch.from_numpy(lp).cuda()
    fi = torch.from_numpy(idx).cuda()
    for t in range(T):
        pool.step(x[:, t], frame_index=fi[:, t].contiguous())
    got = pool_read(pool)
    outs = []
    for s in range(S):
        st = oracle.Stream(W, V, 0)
        for t in range(T):
            st.step_at(lp[s, t], int(idx[s, t]))
        outs.append(st.read(W, T))
    assert_parity(got, tuple(np.stack([o[i] for o in outs]) for i in range(3)), what="wide step")


# ------------------------------------------------- paged storage, 33..128 --
@pytest.mark.parametrize("W,ps", [(33, 4), (64, 16), (100, 8), (128, 64)])
def test_wide_beams_paged_equals_oracle_and_flat(W, ps):
    # pages of 4..64 tokens (page boundaries every few labels with 4), prefix
    # sharing by reference counts and copy-on-write; ragged and empty rows
    lp, _ = synth.peaky(4, 90, 250, seed=110 + W, p_blank=0.45)
    lens = np.array([90, 0, 61, 1], np.int32)
    print(f"[case] wide paged W={W} page_size={ps}", flush=True)
    got = gpu_offline(lp, lens, W, W, 0, 1.0, 90, paged=True, page_size=ps)
    high = gpu_offline.last_stats[:, 3]
    assert_parity(got, oracle.decode(lp, lens, W, W, 0, 1.0, 90), what=f"wide paged W{W}")
    flat = gpu_offline(lp, lens, W, W, 0, 1.0, 90)
    assert all(np.array_equal(a, b) for a, b in zip(got, flat))
    # pages in use at most: the page's allocator as the oracle models it
    # (sec. 3.4.5 / 4.2), never more than the default pool W (ceil(T / ps) + 1)
    model = oracle.decode_pages(lp, lens, W, page_size=ps)
    assert list(high) == list(model[:, 0]) and (model[:, 1] == 0).all()
    assert high[1] == 0 and 0 < high[0] <= W * ((90 + ps - 1) // ps + 1)


def test_wide_beams_paged_skips_and_truncation():
    lp, lens = synth.peaky(3, 80, 200, seed=120, p_blank=0.6)
    print("[case] wide paged skips", flush=True)
    got = gpu_offline(lp, lens, 72, 12, 0, 0.9, 7, paged=True, page_size=8)
    assert_parity(got, oracle.decode(lp, lens, 72, 12, 0, 0.9, 7), what="wide paged skips")


def test_wide_beams_paged_bounded_pool():
    # a pool equal to a row's reported high-water mark decodes it exactly; one
    # page less flags the row (status bit 0) and leaves the other rows as they were
    lp, lens = synth.peaky(3, 70, 120, seed=121, p_blank=0.5)
    W = 48
    print("[case] wide paged bounded pool", flush=True)
    full = gpu_offline(lp, lens, W, W, 0, 1.0, 70, paged=True, page_size=4)
    high = gpu_offline.last_stats[:, 3].copy()
    tight = int(high.max())
    got = gpu_offline(lp, lens, W, W, 0, 1.0, 70, paged=True, page_size=4, num_pages=tight)
    assert (gpu_offline.last_stats[:, 2] == 0).all()
    assert all(np.array_equal(a, b) for a, b in zip(got, full))
    short = gpu_offline(lp, lens, W, W, 0, 1.0, 70, paged=True, page_size=4,
                        num_pages=tight - 1, check_status=False)
    st = gpu_offline.last_stats
    # the oracle's model of the page's allocator: same high-water marks, and
    # the same rows run dry in the smaller pool
    assert list(high) == list(oracle.decode_pages(lp, lens, W, page_size=4)[:, 0])
    dry = oracle.decode_pages(lp, lens, W, page_size=4, num_pages=tight - 1)[:, 1]
    assert list(st[:, 2] & 1) == list(dry)
    for r in range(3):
        if high[r] > tight - 1:
            assert st[r, 2] & 1, (r, high[r])
        else:
            assert st[r, 2] == 0
            assert all(np.array_equal(a[r], b[r]) for a, b in zip(short, full))


@pytest.mark.parametrize("W,cuts,ps", [(40, [0, 16, 32, 48, 64, 80], 4), (128, [0, 1, 30, 80], 16)])
def test_wide_beams_paged_streaming(W, cuts, ps):
    import torch
    S, T, V = 4, 80, 200
    lp, _ = synth.peaky(S, T, V, seed=130 + W, p_blank=0.55)
    print(f"[case] wide paged stream W={W} ps={ps} cuts={cuts}", flush=True)
    pool = cpb.StreamPool(cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T, paged=True,
                                            page_size=ps), V, S)
    x = torch.from_numpy(lp).cuda()
    for a, b in zip(cuts[:-1], cuts[1:]):
        pool.chunk(x[:, a:b])
    got = pool_read(pool)
    assert_parity(got, oracle_streams(lp, W, 4096, cuts, W, T), what=f"wide paged stream W{W}")
    # pages in use at most, against the oracle's model along the same chunks
    high = pool.row_stats().cpu().numpy()[:, 3]
    for s_ in range(S):
        st = oracle.Stream(W, V, 0, 4096, page_size=ps)
        for a, b in zip(cuts[:-1], cuts[1:]):
            st.feed(lp[s_, a:b])
        assert st.pages()[0] == high[s_] and st.pages()[1] == 0
    off = gpu_offline(lp, np.full(S, T, np.int32), W, W, 0, 1.0, T, paged=True, page_size=ps)
    for g, o in zip(got, off):
        assert np.array_equal(g, o)
    # reset stream 2 and decode stream 0's frames in it again
    two = torch.tensor([2], dtype=torch.int32, device="cuda")
    pool.reset(two)
    for a, b in zip(cuts[:-1], cuts[1:]):
        pool.chunk(x[[0], a:b], rows=two)
    t, l, s = pool.read(two)
    assert np.array_equal(t.cpu().numpy()[0], got[0][0])
    assert np.array_equal(s.cpu().numpy()[0], got[2][0])
