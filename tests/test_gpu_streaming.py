"""Streaming decode on the GPU (stream_init / stream_chunk / read_state /
stream_reset through the C ABI) against the oracle's streaming decode and
against the GPU's own offline decode of the concatenated frames."""
import numpy as np
import pytest
import torch

import ctc_prefix_beam_amd as cpb
import oracle
import synth
from gpu_util import assert_parity, gpu_offline

pytestmark = pytest.mark.gpu


def oracle_streams(lp, beam, capacity, chunk, nbest, mol):
    S = lp.shape[0]
    outs = []
    for s in range(S):
        st = oracle.Stream(beam, lp.shape[2], 0, capacity)
        for a in range(0, lp.shape[1], chunk):
            st.feed(lp[s, a:a + chunk])
        outs.append(st.read(nbest, mol))
    return tuple(np.stack([o[i] for o in outs]) for i in range(3))


def read(pool, rows=None):
    t, l, s = pool.read(rows)
    st = pool.row_stats().cpu().numpy()
    torch.cuda.synchronize()
    assert (st[:, 2] == 0).all(), f"stream status bits set: {np.unique(st[:, 2])}"
    return t.cpu().numpy(), l.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("paged", [False, True])
def test_chunks_equal_oracle_stream_and_offline(paged):
    S, T, V, W, CH = 6, 96, 512, 10, 16
    lp, _ = synth.peaky(S, T, V, seed=21, p_blank=0.65)
    print(f"[case] stream S={S} T={T} V={V} W={W} paged={paged}", flush=True)
    cfg = cpb.DecoderConfig(beam=W, nbest=W, capacity=4096, max_out_len=T, paged=paged)
    pool = cpb.StreamPool(cfg, V, S)
    x = torch.from_numpy(lp).cuda()
    for a in range(0, T, CH):
        pool.chunk(x[:, a:a + CH])
    got = read(pool)
    ref = oracle_streams(lp, W, 4096, CH, W, T)
    assert_parity(got, ref, what="stream")
    off = gpu_offline(lp, np.full(S, T, np.int32), W, W, 0, 1.0, T, paged=paged)
    for a, b in zip(got, off):
        assert np.array_equal(a, b)


def test_uniform_frames_take_the_exact_selection():
    # frames whose non-blank labels all share one log-probability force the
    # full beam x vocabulary selection, which reads the chunk's frame from
    # global memory
    S, T, V, W, CH = 4, 64, 96, 12, 16
    lp, _ = synth.peaky(S, T, V, seed=23, p_blank=0.5)
    pick = np.random.default_rng(24).random((S, T)) < 0.3
    flat = np.full(V, np.log(0.999 / (V - 1)), np.float32)   # blank below every label
    flat[0] = np.float32(np.log(0.001))
    lp[pick] = flat
    print(f"[case] stream uniform S={S} T={T} V={V} W={W}", flush=True)
    cfg = cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T)
    pool = cpb.StreamPool(cfg, V, S)
    x = torch.from_numpy(lp).cuda()
    for a in range(0, T, CH):
        pool.chunk(x[:, a:a + CH])
    got = read(pool)
    st = pool.row_stats().cpu().numpy()
    assert st[:, cpb.STAT_FIELDS.index("fallbacks")].sum() > 0, "no step took the full selection"
    assert_parity(got, oracle_streams(lp, W, 4096, CH, W, T), what="stream uniform")


def test_read_is_non_mutating_and_midway_results():
    S, T, V, W, CH = 3, 64, 100, 8, 16
    lp, _ = synth.peaky(S, T, V, seed=22)
    cfg = cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T)
    pool = cpb.StreamPool(cfg, V, S)
    x = torch.from_numpy(lp).cuda()
    fresh = read(pool)
    assert (fresh[1] == 0).all() and (fresh[2][:, 0] == 0).all()
    assert (fresh[2][:, 1:] == -np.finfo(np.float32).max).all()
    for a in range(0, 32, CH):
        pool.chunk(x[:, a:a + CH])
    mid1, mid2 = read(pool), read(pool)
    for a, b in zip(mid1, mid2):
        assert np.array_equal(a, b)
    assert_parity(mid1, oracle_streams(lp[:, :32], W, 4096, CH, W, T), what="mid")
    for a in range(32, T, CH):
        pool.chunk(x[:, a:a + CH])
    assert_parity(read(pool), oracle_streams(lp, W, 4096, CH, W, T), what="end")


def test_row_subsets_reset_and_capacity():
    S, T, V, W = 5, 48, 64, 6
    lp, _ = synth.peaky(S, T, V, seed=23)
    cfg = cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T, capacity=40)
    pool = cpb.StreamPool(cfg, V, S)
    x = torch.from_numpy(lp).cuda()
    rows = torch.tensor([3, 0], dtype=torch.int32, device="cuda")
    # only streams 3 and 0 advance; chunk row i feeds stream rows[i]
    for a in range(0, T, 16):
        pool.chunk(x[[3, 0], a:a + 16], rows=rows)
    got = read(pool)
    ref = oracle_streams(lp[[0, 3]], W, 40, 16, W, T)   # capacity 40 < 48 frames
    assert_parity(tuple(g[[0, 3]] for g in got), ref, what="subset")
    assert (got[1][[1, 2, 4]] == 0).all()               # untouched streams still fresh
    # reset stream 3 and feed it stream 1's frames
    pool.reset(torch.tensor([3], dtype=torch.int32, device="cuda"))
    for a in range(0, T, 16):
        pool.chunk(x[[1], a:a + 16], rows=torch.tensor([3], dtype=torch.int32, device="cuda"))
    got = read(pool, torch.tensor([3, 0], dtype=torch.int32, device="cuda"))
    ref = oracle_streams(lp[[1, 0]], W, 40, 16, W, T)
    assert_parity(got, ref, what="reset")


def test_uneven_chunks_equal_single_chunk():
    S, T, V, W = 4, 75, 200, 12
    lp, _ = synth.peaky(S, T, V, seed=24, p_low=0.2)
    x = torch.from_numpy(lp).cuda()
    outs = []
    for cuts in ([0, 75], [0, 1, 2, 17, 40, 41, 75], list(range(0, 76, 5))):
        pool = cpb.StreamPool(cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T), V, S)
        for a, b in zip(cuts[:-1], cuts[1:]):
            pool.chunk(x[:, a:b])
        outs.append(read(pool))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


# ------------------------------------ speech mask and caller frame indices --
def oracle_masked(lp, mask, W, capacity, chunk, nbest, mol, start=None):
    outs, frames = [], []
    for s in range(lp.shape[0]):
        st = oracle.Stream(W, lp.shape[2], 0, capacity)
        for a in range(0, lp.shape[1], chunk):
            sf = None if (start is None or a > 0) else int(start[s])
            st.feed(lp[s, a:a + chunk], None if mask is None else mask[s, a:a + chunk], sf)
        outs.append(st.read(nbest, mol))
        frames.append(st.frames)
    return tuple(np.stack([o[i] for o in outs]) for i in range(3)), frames


@pytest.mark.parametrize("paged", [False, True])
def test_speech_mask_equals_oracle(paged):
    S, T, V, W, CH = 6, 64, 96, 8, 16
    lp, _ = synth.peaky(S, T, V, seed=41, p_blank=0.6)
    rng = np.random.default_rng(42)
    mask = (rng.random((S, T)) < 0.7).astype(np.uint8)
    mask[1] = 0                       # a stream that decodes nothing
    mask[2, :20] = 0                  # first decoded frame > 0: seeded under the gap rule
    print(f"[case] stream mask S={S} T={T} V={V} W={W} paged={paged}", flush=True)
    cfg = cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T, paged=paged)
    pool = cpb.StreamPool(cfg, V, S)
    x = torch.from_numpy(lp).cuda()
    m = torch.from_numpy(mask).cuda()
    for a in range(0, T, CH):
        pool.chunk(x[:, a:a + CH], is_speech=m[:, a:a + CH].contiguous())
    got = read(pool)
    ref, frames = oracle_masked(lp, mask, W, 4096, CH, W, T)
    assert_parity(got, ref, what="stream mask")
    st = pool.row_stats().cpu().numpy()
    assert list(st[:, 0]) == list(mask.sum(1))          # steps decoded
    assert list(st[:, 1]) == frames == [T] * S          # frames given


def test_mask_from_threshold_equals_offline():
    # the page's recipe: a mask computed from the blank log-prob against the
    # threshold turns the stream into the offline decode of that selection
    S, T, V, W, theta = 4, 80, 64, 6, 0.9
    lp, _ = synth.peaky(S, T, V, seed=43, p_blank=0.6)
    mask = np.zeros((S, T), np.uint8)
    for s in range(S):
        mask[s, oracle.select_frames(lp[s], T, 0, theta)] = 1
    assert 0 < mask.sum() < S * T
    print(f"[case] stream threshold mask S={S} T={T} V={V} W={W}", flush=True)
    cfg = cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T)
    pool = cpb.StreamPool(cfg, V, S)
    x = torch.from_numpy(lp).cuda()
    m = torch.from_numpy(mask).cuda()
    for a in range(0, T, 16):
        pool.chunk(x[:, a:a + 16], is_speech=m[:, a:a + 16].contiguous())
    got = read(pool)
    off = gpu_offline(lp, np.full(S, T, np.int32), W, W, 0, theta, T)
    for a, b in zip(got, off):
        assert np.array_equal(a, b)
    assert_parity(got, oracle.decode(lp, np.full(S, T), W, W, 0, theta, T), what="thr mask")


@pytest.mark.parametrize("paged", [False, True])
def test_per_frame_step_with_frame_index(paged):
    S, T, V, W = 3, 40, 50, 5
    lp, _ = synth.peaky(S, T, V, seed=44)
    rng = np.random.default_rng(45)
    # per stream, increasing frame numbers with gaps of 1..3
    idx = np.cumsum(rng.integers(1, 4, size=(S, T)), axis=1).astype(np.int32) - 1
    print(f"[case] stream step S={S} T={T} V={V} W={W} paged={paged}", flush=True)
    cfg = cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T, paged=paged)
    pool = cpb.StreamPool(cfg, V, S)
    x = torch.from_numpy(lp).cuda()
    fi = torch.from_numpy(idx).cuda()
    for t in range(T):
        pool.step(x[:, t], frame_index=fi[:, t].contiguous())
    got = read(pool)
    outs = []
    for s in range(S):
        st = oracle.Stream(W, V, 0)
        for t in range(T):
            st.step_at(lp[s, t], int(idx[s, t]))
        outs.append(st.read(W, T))
    ref = tuple(np.stack([o[i] for o in outs]) for i in range(3))
    assert_parity(got, ref, what="step")
    st = pool.row_stats().cpu().numpy()
    assert list(st[:, 1]) == list(idx[:, -1] + 1)


def test_start_frame_capacity_and_row_subsets():
    S, T, V, W, CH, CAP = 4, 48, 40, 4, 16, 30
    lp, _ = synth.peaky(S, T, V, seed=46)
    mask = (np.random.default_rng(47).random((S, T)) < 0.8).astype(np.uint8)
    start = np.array([0, 5, 100, 7], np.int32)
    print(f"[case] stream start frames S={S} T={T} V={V} W={W} cap={CAP}", flush=True)
    cfg = cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T, capacity=CAP)
    pool = cpb.StreamPool(cfg, V, S)
    x = torch.from_numpy(lp).cuda()
    m = torch.from_numpy(mask).cuda()
    rows = torch.tensor([2, 0, 3, 1], dtype=torch.int32, device="cuda")
    perm = [2, 0, 3, 1]   # chunk row i continues stream perm[i]
    for a in range(0, T, CH):
        sf = torch.from_numpy(start[perm]).cuda() if a == 0 else None
        pool.chunk(x[perm, a:a + CH], rows=rows, is_speech=m[perm, a:a + CH].contiguous(),
                   start_frame=sf)
    got = read(pool)
    ref, frames = oracle_masked(lp, mask, W, CAP, CH, W, T, start=start)
    assert_parity(got, ref, what="start frames")
    st = pool.row_stats().cpu().numpy()
    assert list(st[:, 0]) == [min(CAP, int(mask[s].sum())) for s in range(S)]
    assert list(st[:, 1]) == frames == list(start + T)


def test_chunks_replayed_from_a_captured_graph():
    # reset + four chunk calls captured once into a HIP graph (no host sync and
    # no allocation inside the calls), replayed several times with eager work
    # and synchronisations in between: every replay equals the eager decode
    S, T, V, W, CH = 8, 64, 512, 10, 16
    lp, _ = synth.peaky(S, T, V, seed=26, p_blank=0.65)
    print(f"[case] stream graph S={S} T={T} V={V} W={W}", flush=True)
    cfg = cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T, capacity=T)
    pool = cpb.StreamPool(cfg, V, S)
    x = torch.from_numpy(lp).cuda()
    chunks = [x[:, a:a + CH].contiguous() for a in range(0, T, CH)]
    for c in chunks:
        pool.chunk(c)
    eager = read(pool)
    assert_parity(eager, oracle_streams(lp, W, T, CH, W, T), what="graph eager")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pool.reset()
            for c in chunks:
                pool.chunk(c)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        pool.reset()                       # eager work between replays
        junk = torch.ones(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = read(pool)
        for a, b in zip(got, eager):
            assert np.array_equal(a, b), rep
        assert float(junk) == float(1 << 20)


def test_bounded_page_pool_streams():
    # streams with a page pool below the default: a stream whose high-water
    # mark (row_stats [3], reported by the unbounded run) fits decodes exactly
    # as before, a stream that needs more sets status bit 0; a reset clears it
    S, T, V, W, CH = 6, 160, 300, 12, 16
    lp, _ = synth.peaky(S, T, V, seed=33, p_blank=0.4)
    print(f"[case] stream bounded pool S={S} T={T} V={V} W={W} ps=8", flush=True)
    x = torch.from_numpy(lp).cuda()

    def run(num_pages):
        cfg = cpb.DecoderConfig(beam=W, nbest=W, capacity=T, max_out_len=T, paged=True,
                                page_size=8, num_pages=num_pages)
        pool = cpb.StreamPool(cfg, V, S)
        for a in range(0, T, CH):
            pool.chunk(x[:, a:a + CH])
        t, l, s = pool.read()
        st = pool.row_stats().cpu().numpy()
        return pool, (t.cpu().numpy(), l.cpu().numpy(), s.cpu().numpy()), st

    # the pool sized explicitly (the default's size) follows the page's
    # allocator, whose marks are the pools that decode each stream exactly
    _, full, st = run(W * (-(-T // 8) + 1))
    assert (st[:, 2] == 0).all()
    assert_parity(full, oracle_streams(lp, W, T, CH, W, T), what="stream pool")
    high = st[:, 3].copy()
    for s_ in range(S):
        ost = oracle.Stream(W, V, 0, T, page_size=8)
        for a in range(0, T, CH):
            ost.feed(lp[s_, a:a + CH])
        assert ost.pages()[0] == high[s_]
    npages = int(np.median(high))
    fits = high <= npages
    assert fits.any() and (~fits).any(), high
    pool, got, st = run(npages)
    assert np.array_equal(st[:, 2] & 1, (~fits).astype(st.dtype))
    for b in np.nonzero(fits)[0]:
        for a, e in zip(got, full):
            assert np.array_equal(a[b], e[b])
    # the flagged streams start again, on their own, and their first chunk
    # decodes as in an unbounded pool
    idx = [int(i) for i in np.nonzero(~fits)[0]]
    bad = torch.tensor(idx, dtype=torch.int32, device="cuda")
    pool.reset(bad)
    pool.chunk(x[idx, :CH], rows=bad)
    st = pool.row_stats().cpu().numpy()
    assert (st[:, 2] == 0).all()
    t, l, s = pool.read(bad)
    ref = oracle_streams(lp[np.nonzero(~fits)[0], :CH], W, T, CH, W, T)
    assert_parity((t.cpu().numpy(), l.cpu().numpy(), s.cpu().numpy()), ref, what="after reset")


@pytest.mark.parametrize("paged", [False, True])
def test_masked_chunks_take_the_exact_selection_from_the_flagged_frame(paged):
    # frames whose non-blank labels all share one log-probability force the
    # full beam x vocabulary selection, which reads the decoded frame's row
    # from global memory.  With a speech mask, the step that decodes the f-th
    # flagged frame of a chunk must read that frame's row, not chunk row f:
    # masked frames sit before uniform ones in every chunk
    S, T, V, W, CH = 4, 64, 96, 12, 16
    lp, _ = synth.peaky(S, T, V, seed=27, p_blank=0.5)
    rng = np.random.default_rng(28)
    flat = np.full(V, np.log(0.999 / (V - 1)), np.float32)   # blank below every label
    flat[0] = np.float32(np.log(0.001))
    mask = np.ones((S, T), np.uint8)
    for a in range(0, T, CH):
        mask[:, a:a + 3] = 0                                  # three masked frames first
        pick = rng.random((S, CH - 3)) < 0.4
        for s in range(S):
            for j in np.nonzero(pick[s])[0]:
                lp[s, a + 3 + j] = flat
    print(f"[case] stream masked uniform S={S} T={T} V={V} W={W} paged={paged}", flush=True)
    cfg = cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T, paged=paged)
    pool = cpb.StreamPool(cfg, V, S)
    x = torch.from_numpy(lp).cuda()
    m = torch.from_numpy(mask).cuda()
    for a in range(0, T, CH):
        pool.chunk(x[:, a:a + CH], is_speech=m[:, a:a + CH].contiguous())
    got = read(pool)
    st = pool.row_stats().cpu().numpy()
    assert st[:, cpb.STAT_FIELDS.index("fallbacks")].sum() > 0, "no step took the full selection"
    ref, _ = oracle_masked(lp, mask, W, 4096, CH, W, T)
    assert_parity(got, ref, what="stream masked uniform")


def test_long_streams_with_reordering_beams_and_uneven_chunks():
    # ambiguous frames make the beams change lineage often, so the flat store
    # copies rows on many steps; uneven chunks move the chunk boundaries (where
    # the store's lineage and common-prefix bounds are saved and reloaded)
    # across every phase of its 16-step prefix advance; one stream is reset
    # halfway and restarted on another stream's frames
    S, T, V, W = 6, 320, 64, 10
    lp, _ = synth.peaky(S, T, V, seed=41, p_blank=0.5, token_bias=(0.5, 3.0), p_low=0.3)
    sched = [5, 11, 3, 16, 7, 1, 9, 13, 2, 17]
    cuts, a = [], 0
    while a < T:
        b = min(T, a + sched[len(cuts) % len(sched)])
        cuts.append((a, b))
        a = b
    print(f"[case] long streams S={S} T={T} V={V} W={W} chunks={len(cuts)}", flush=True)
    cfg = cpb.DecoderConfig(beam=W, nbest=W, capacity=4096, max_out_len=T)
    pool = cpb.StreamPool(cfg, V, S)
    x = torch.from_numpy(lp).cuda()
    half = len(cuts) // 2
    for i, (a, b) in enumerate(cuts):
        if i == half:
            pool.reset(torch.tensor([2], dtype=torch.int32, device="cuda"))
        pool.chunk(x[:, a:b])
    got = read(pool)
    # stream 2 decoded frames [cuts[half][0], T) only
    t0 = cuts[half][0]
    refs = []
    for s in range(S):
        st = oracle.Stream(W, V, 0, 4096)
        for i, (a, b) in enumerate(cuts):
            if s == 2 and i < half:
                continue
            st.feed(lp[s, a:b])
        refs.append(st.read(W, T))
    ref = tuple(np.stack([r[i] for r in refs]) for i in range(3))
    assert_parity(got, ref, what="long streams")
    keep = [s for s in range(S) if s != 2]
    off = gpu_offline(lp[keep], np.full(len(keep), T, np.int32), W, W, 0, 1.0, T)
    for g, o in zip(got, off):
        assert np.array_equal(g[keep], o)
    off2 = gpu_offline(np.ascontiguousarray(lp[2:3, t0:]), np.array([T - t0], np.int32), W, W, 0,
                       1.0, T)
    for g, o in zip(got, off2):
        assert np.array_equal(g[2:3], o)
