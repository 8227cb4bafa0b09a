"""Pins of the CPU oracle against facts outside the oracle itself.

- brute force: with a beam wide enough to keep every prefix and no frame
  skipping, prefix beam search is exact, so its scores must equal the log-sum
  over all alignments that collapse to each prefix (enumerated here in fp64);
- torch's CPU ``ctc_loss`` (the textbook CTC forward recursion, fp64): equal
  to the exact posteriors above, and an upper bound of every pruned score;
- closed forms at T = 1 (step-0 seeding, the empty slot, dead slots, ties);
- the page's stated edge cases (empty rows, thresholds 0 and 1, truncation);
- a hand-worked frame-skip case (tests/golden/gap_two_skips.json);
- invariants on the five workloads' generators;
- the numerics against libm in fp64.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NEG = -np.finfo(np.float32).max


# ---------------------------------------------------------------- helpers --
def collapse(path, blank=0):
    out, prev = [], None
    for c in path:
        if c != prev and c != blank:
            out.append(c)
        prev = c
    return tuple(out)


def brute_force(lp, blank=0):
    """{prefix: log P(prefix | x)} by enumerating every alignment (fp64)."""
    T, V = lp.shape
    lp64 = lp.astype(np.float64)
    acc = {}
    for path in itertools.product(range(V), repeat=T):
        s = float(sum(lp64[t, c] for t, c in enumerate(path)))
        key = collapse(path, blank)
        acc[key] = np.logaddexp(acc[key], s) if key in acc else s
    return acc


def ctc_logp(lp, target, blank=0):
    """log P(target | x) from torch's CTC forward (CPU, fp64)."""
    T = lp.shape[0]
    x = torch.from_numpy(lp.astype(np.float64)).unsqueeze(1)
    tgt = torch.tensor(list(target), dtype=torch.long)
    loss = torch.nn.functional.ctc_loss(x, tgt, torch.tensor([T]), torch.tensor([len(target)]),
                                        blank=blank, reduction="sum", zero_infinity=False)
    return -float(loss)


def live_hyps(toks, lengths, scores):
    out = []
    for r in range(len(lengths)):
        if scores[r] > NEG:
            out.append((tuple(int(t) for t in toks[r, :lengths[r]]), float(scores[r])))
    return out


def f32log(p):
    return np.log(np.asarray(p, np.float64)).astype(np.float32)


# -------------------------------------------------------------- numerics --
def test_exp_matches_libm(oracle_lib):
    xs = np.concatenate([np.linspace(-80.0, 0.0, 20001), -np.logspace(-8, 1.9, 2001), [0.0]])
    worst = 0.0
    for x in xs.astype(np.float32):
        got = oracle_lib.exp(float(x))
        ref = math.exp(float(x))
        worst = max(worst, abs(got - ref) / ref)
    assert worst < 4e-7, worst  # a few ulp of float32


def test_log1p_matches_libm(oracle_lib):
    xs = np.concatenate([np.linspace(0.0, 1.0, 20001), np.logspace(-30, 0, 2001)])
    worst = 0.0
    for x in xs.astype(np.float32):
        got = oracle_lib.log1p(float(x))
        ref = math.log1p(float(x))
        if ref > 0:
            worst = max(worst, abs(got - ref) / ref)
        else:
            assert got == 0.0
    assert worst < 4e-7, worst


def test_lse_identities(oracle_lib):
    lse = oracle_lib.lse
    rng = np.random.default_rng(0)
    for a in rng.uniform(-5000, 0, 200).astype(np.float32):
        assert lse(float(a), NEG) == float(a)  # NEG is the identity
        assert lse(NEG, float(a)) == float(a)
        b = float(np.float32(a - rng.uniform(0, 90)))
        assert lse(float(a), b) == lse(b, float(a))  # symmetric
        ref = np.logaddexp(np.float64(a), np.float64(b))
        assert abs(lse(float(a), b) - ref) <= 4 * np.spacing(np.float32(abs(ref))) + 1e-7
    assert lse(NEG, NEG) == NEG
    assert lse(0.0, 0.0) == pytest.approx(math.log(2.0), abs=1e-7)


# ------------------------------------------------------ frame selection --
def test_select_boundaries(oracle_lib):
    lp, _ = synth.peaky(1, 40, 7, seed=3, p_blank=0.5, blank_bias=9.0)
    row = lp[0]
    assert list(oracle_lib.select_frames(row, 40, 0, 1.0)) == list(range(40))
    assert list(oracle_lib.select_frames(row, 40, 0, 1.5)) == list(range(40))
    assert len(oracle_lib.select_frames(row, 40, 0, 0.0)) == 0
    assert len(oracle_lib.select_frames(row, 40, 0, -1.0)) == 0
    assert list(oracle_lib.select_frames(row, 17, 0, 1.0)) == list(range(17))  # length bound
    thr = 0.9
    log_thr = np.float32(math.log(float(np.float32(thr))))  # threshold crosses as float32
    expect = [t for t in range(40) if row[t, 0] < log_thr]
    assert list(oracle_lib.select_frames(row, 40, 0, thr)) == expect
    # strict comparison: a blank log-prob exactly at log(threshold) is kept out
    row2 = row.copy()
    row2[5, 0] = log_thr
    assert 5 not in oracle_lib.select_frames(row2, 40, 0, thr)
    row2[5, 0] = np.nextafter(log_thr, np.float32(-np.inf))
    assert 5 in oracle_lib.select_frames(row2, 40, 0, thr)


# ------------------------------------------------------------ brute force --
@pytest.mark.parametrize("T,V,seed", [(1, 3, 0), (2, 3, 1), (3, 3, 2), (4, 3, 3), (5, 3, 4),
                                      (6, 3, 5), (3, 4, 6), (4, 4, 7), (5, 4, 8), (4, 5, 9)])
def test_unpruned_equals_brute_force(oracle_lib, T, V, seed):
    lp, lens = synth.peaky(1, T, V, seed=seed, p_blank=0.5, blank_bias=1.0, token_bias=1.5,
                           repeat_p=0.5)
    exact = brute_force(lp[0])
    W = len(exact) + V  # wide enough to keep every prefix
    toks, L, S = oracle_lib.decode(lp, lens, W, W, 0, 1.0, T)
    got = live_hyps(toks[0], L[0], S[0])
    assert len(got) == len(exact)
    assert {h for h, _ in got} == set(exact)
    for h, s in got:
        assert s == pytest.approx(exact[h], abs=2e-5), h
    # scores are reported in non-increasing order
    assert all(got[i][1] >= got[i + 1][1] for i in range(len(got) - 1))
    # the posteriors of all prefixes sum to one
    assert np.logaddexp.reduce([s for _, s in got]) == pytest.approx(0.0, abs=2e-5)


def test_unpruned_equals_ctc_forward(oracle_lib):
    lp, lens = synth.peaky(1, 6, 3, seed=11, p_blank=0.4, blank_bias=1.0, token_bias=1.0)
    W = 200
    toks, L, S = oracle_lib.decode(lp, lens, W, W, 0, 1.0, 6)
    for h, s in live_hyps(toks[0], L[0], S[0]):
        assert s == pytest.approx(ctc_logp(lp[0], h), abs=2e-5)


@pytest.mark.parametrize("name,T,W", [("tiny", 50, 4), ("bpe256", 120, 8), ("stream512", 80, 10),
                                      ("bpe1024", 60, 16)])
def test_pruned_scores_bounded_by_ctc_forward(oracle_lib, name, T, W):
    wl = synth.WORKLOADS[name]
    gen = dict(wl.gen)
    gen.pop("lengths", None)
    gen.pop("nan_tail", None)
    lp, lens = synth.peaky(2, T, wl.V, seed=5, **gen)
    toks, L, S = oracle_lib.decode(lp, lens, W, W, 0, 1.0, T)
    for b in range(2):
        hyps = live_hyps(toks[b], L[b], S[b])
        assert len(hyps) == W
        for h, s in hyps:
            exact = ctc_logp(lp[b], h)
            # a beam-restricted alignment sum never exceeds the full sum
            assert s <= exact + 1e-5 * abs(exact) + 1e-4, (h, s, exact)
        # the 1-best of a peaky input keeps most of its exact posterior
        assert hyps[0][1] >= ctc_logp(lp[b], hyps[0][0]) - 0.5


# --------------------------------------------------------- closed forms --
def test_single_frame_seeding(oracle_lib):
    # T = 1: the top-(W-1) non-blank tokens by (lp desc, id asc) at their lp,
    # plus the empty prefix at lp[blank]; reported by (score desc, slot asc).
    lp = f32log([[0.30, 0.10, 0.25, 0.10, 0.05, 0.20]])[None]  # ties: ids 1 and 3
    toks, L, S = oracle_lib.decode(lp, [1], 4, 4, 0, 1.0, 1)
    got = live_hyps(toks[0], L[0], S[0])
    assert [h for h, _ in got] == [(), (2,), (5,), (1,)]
    assert [s for _, s in got] == [float(lp[0, 0, c]) for c in (0, 2, 5, 1)]


def test_single_frame_beam_one(oracle_lib):
    # beam 1 has no empty slot: the best non-blank token is kept (sec. 3.3)
    lp = f32log([[0.90, 0.04, 0.06]])[None]
    toks, L, S = oracle_lib.decode(lp, [1], 1, 1, 0, 1.0, 1)
    assert live_hyps(toks[0], L[0], S[0]) == [((2,), float(lp[0, 0, 2]))]


def test_dead_slots_when_vocab_is_narrow(oracle_lib):
    # V - 1 < W - 1: slots without a token stay dead (score NEG, length 0)
    lp = f32log([[0.7, 0.3], [0.6, 0.4]])[None]
    toks, L, S = oracle_lib.decode(lp, [2], 4, 4, 0, 1.0, 2)
    hyps = live_hyps(toks[0], L[0], S[0])
    exact = brute_force(lp[0])
    assert {h for h, _ in hyps} == set(exact)
    assert list(S[0, len(hyps):]) == [NEG] * (4 - len(hyps))
    assert list(L[0, len(hyps):]) == [0] * (4 - len(hyps))
    assert (toks[0, len(hyps):] == -1).all()


def test_empty_rows(oracle_lib):
    # sec. 13: zero-length rows and rows with every frame skipped hold the
    # empty hypothesis at 0.0, other slots at NEG with length 0
    lp, _ = synth.peaky(2, 10, 5, seed=1)
    for lens, thr in (([0, 0], 0.98), ([10, 10], 0.0), ([10, 10], -3.0)):
        toks, L, S = oracle_lib.decode(lp, lens, 3, 3, 0, thr, 10)
        assert (L == 0).all()
        assert (S[:, 0] == 0.0).all() and (S[:, 1:] == NEG).all()
        assert (toks == -1).all()


def test_truncation_keeps_full_length(oracle_lib):
    lp, lens = synth.peaky(1, 60, 12, seed=2, p_blank=0.3)
    full = oracle_lib.decode(lp, lens, 5, 5, 0, 1.0, 60)
    cut = oracle_lib.decode(lp, lens, 5, 5, 0, 1.0, 7)
    assert (full[1] == cut[1]).all() and (full[2] == cut[2]).all()
    assert (full[1][0] > 7).all()
    assert (cut[0] == full[0][:, :, :7]).all()


def test_gap_golden(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "gap_two_skips.json")))
    lp = f32log(g["probs"])[None]
    T = lp.shape[1]
    sel = oracle_lib.select_frames(lp[0], T, g["blank"], g["threshold"])
    assert list(sel) == [0, 2, 3]
    toks, L, S = oracle_lib.decode(lp, [T], g["beam"], g["nbest"], g["blank"], g["threshold"], T)
    hyps = live_hyps(toks[0], L[0], S[0])
    assert [list(h) for h, _ in hyps] == g["expected_tokens"]
    assert list(L[0]) == g["expected_lengths"]
    for (_, s), p in zip(hyps, g["expected_scores_log"]):
        assert s == pytest.approx(math.log(p), abs=1e-6)


def test_gap_leading_skip_golden(oracle_lib):
    # step 0 after skipped leading frames seeds the labels' mass into the
    # blank-ending part (sec. 3.3 need_add_blank); the next frame repeats the
    # first label, which only the blank-ending part can extend
    g = json.load(open(os.path.join(GOLDEN, "gap_leading_skip.json")))
    lp = f32log(g["probs"])
    T = lp.shape[0]
    assert list(oracle_lib.select_frames(lp, T, g["blank"], g["threshold"])) == [1, 2]
    toks, L, S = oracle_lib.decode(lp[None], [T], g["beam"], g["nbest"], g["blank"],
                                   g["threshold"], T)
    hyps = live_hyps(toks[0], L[0], S[0])
    assert [list(h) for h, _ in hyps] == g["expected_tokens"]
    assert list(L[0]) == g["expected_lengths"]
    for (_, s), p in zip(hyps, g["expected_scores_log"]):
        assert s == pytest.approx(math.log(p), abs=1e-6)
    # the same selection as a masked stream and as frames numbered 1, 2
    st = oracle_lib.Stream(g["beam"], g["vocab"], g["blank"])
    st.feed(lp, is_speech=[0, 1, 1])
    assert [list(h) for h, _ in live_hyps(*st.read(g["nbest"], T))] == g["expected_tokens"]
    st = oracle_lib.Stream(g["beam"], g["vocab"], g["blank"])
    st.step_at(lp[1], 1)
    st.step_at(lp[2], 2)
    t2, l2, s2 = st.read(g["nbest"], T)
    assert (t2 == toks[0]).all() and (l2 == L[0]).all() and (s2 == S[0]).all()


@pytest.mark.parametrize("case", [0, 1])
def test_final_tie_golden(oracle_lib, case):
    # exactly tied final scores: the order is (score desc, slot asc), the
    # slots of a step being in (key desc, flat id asc) order
    g = json.load(open(os.path.join(GOLDEN, "final_tie.json")))["cases"][case]
    lp = f32log(g["probs"])
    T = lp.shape[0]
    toks, L, S = oracle_lib.decode(lp[None], [T], g["beam"], g["nbest"], g["blank"],
                                   g["threshold"], T)
    hyps = live_hyps(toks[0], L[0], S[0])
    assert [list(h) for h, _ in hyps] == g["expected_tokens"]
    assert list(L[0]) == g["expected_lengths"]
    for (_, s), p in zip(hyps, g["expected_scores_log"]):
        assert s == pytest.approx(math.log(p), abs=1e-6)
    assert S[0, 0] == S[0, 1]          # the tie is exact in float32


def brute_force_masked(lp, allowed, blank=0):
    """{prefix: log P} over the alignments whose frame t emits a label of
    allowed[t] (fp64, -inf log-probs excluded by construction)."""
    lp64 = lp.astype(np.float64)
    acc = {}
    for path in itertools.product(*allowed):
        s = float(sum(lp64[t, c] for t, c in enumerate(path)))
        key = collapse(path, blank)
        acc[key] = np.logaddexp(acc[key], s) if key in acc else s
    return acc


@pytest.mark.parametrize("seed", range(8))
def test_gap_rule_equals_certain_blank_frames(oracle_lib, seed):
    # The gap rule (sec. 3.3 step 0, sec. 3.4 collapse before the tables and
    # blank-slot rule, sec. 3.4.5 winners' reset) is what a frame that is
    # blank with probability one does to every beam: (pb, pnb) becomes
    # (logsumexp(pb, pnb), NEG) and nothing else survives.  So a decode that
    # skips frames equals, when nothing is pruned, the exact posteriors of the
    # selected frames with a certain-blank frame before (after step 0) and
    # after each frame that follows a gap.  Pinned by enumeration.
    V, T, theta = 3, 8, 0.9
    lp, _ = synth.peaky(1, T, V, seed=200 + seed, p_blank=0.6, blank_bias=3.5,
                        token_bias=1.5, repeat_p=0.5)
    sel = list(oracle_lib.select_frames(lp[0], T, 0, theta))
    assert 0 < len(sel) < T
    frames, allowed = [], []
    blank_only, every = [0], list(range(V))
    for s, t in enumerate(sel):
        gap = t > 0 if s == 0 else t > sel[s - 1] + 1
        if gap and s > 0:
            frames.append(np.zeros(V, np.float32))
            allowed.append(blank_only)
        frames.append(lp[0, t])
        allowed.append(every)
        if gap:
            frames.append(np.zeros(V, np.float32))
            allowed.append(blank_only)
    exact = brute_force_masked(np.stack(frames), allowed)
    W = len(exact) + V
    toks, L, S = oracle_lib.decode(lp, [T], W, W, 0, theta, T)
    got = live_hyps(toks[0], L[0], S[0])
    assert {h for h, _ in got} == set(exact)
    for h, sc in got:
        assert sc == pytest.approx(exact[h], abs=2e-5), h
    assert np.logaddexp.reduce([sc for _, sc in got]) == pytest.approx(0.0, abs=2e-5)


# -------------------------------------------------------------- invariants --
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_invariants_on_workload_generators(oracle_lib, name):
    wl = synth.WORKLOADS[name]
    T = min(wl.T, 120)
    gen = dict(wl.gen)
    if "lengths" in gen:
        gen["lengths"] = (T // 2, T)
    lp, lens = synth.peaky(2, T, wl.V, seed=7, **gen)
    toks, L, S = oracle_lib.decode(lp, lens, wl.beam, wl.nbest, 0, wl.threshold, T)
    for b in range(2):
        nsel = len(oracle_lib.select_frames(lp[b], lens[b], 0, wl.threshold))
        hyps = live_hyps(toks[b], L[b], S[b])
        assert len(hyps) == wl.nbest
        assert len({h for h, _ in hyps}) == len(hyps)                 # distinct
        assert all(hyps[i][1] >= hyps[i + 1][1] for i in range(len(hyps) - 1))
        for h, _ in hyps:
            assert all(0 < c < wl.V for c in h)                       # blank-free, in range
            assert len(h) <= nsel
        assert np.logaddexp.reduce([s for _, s in hyps]) <= 1e-5      # total mass <= 1
        for n in {len(h) for h, _ in hyps}:
            assert np.logaddexp.reduce([s for h, s in hyps if len(h) == n]) <= 1e-5


def test_streaming_equals_offline(oracle_lib):
    lp, lens = synth.peaky(1, 70, 9, seed=4)
    off = oracle_lib.decode(lp, lens, 6, 6, 0, 1.0, 70)
    st = oracle_lib.Stream(6, 9, 0, capacity=4096)
    for a in range(0, 70, 16):
        st.feed(lp[0, a:a + 16])
    t, l, s = st.read(6, 70)
    assert (t == off[0][0]).all() and (l == off[1][0]).all() and (s == off[2][0]).all()


def test_streaming_capacity_saturates(oracle_lib):
    lp, lens = synth.peaky(1, 40, 9, seed=4)
    st = oracle_lib.Stream(4, 9, 0, capacity=25)
    assert st.feed(lp[0, :16]) == 16
    assert st.feed(lp[0, 16:]) == 25  # frames past the capacity are ignored
    off = oracle_lib.decode(lp, [25], 4, 4, 0, 1.0, 40)
    t, l, s = st.read(4, 40)
    assert (t == off[0][0]).all() and (s == off[2][0]).all()


def test_fresh_stream_reads_empty(oracle_lib):
    st = oracle_lib.Stream(3, 5, 0)
    t, l, s = st.read(3, 4)
    assert list(l) == [0, 0, 0] and s[0] == 0.0 and (s[1:] == NEG).all() and (t == -1).all()


# ------------------------------------------- streaming with a speech mask --
# The page's is_speech_mask (sec. 9, 12): a frame marked 0 bypasses the
# decoder; the next decoded frame carries the gap through its frame index.
def test_masked_stream_gap_golden(oracle_lib):
    # the hand-worked frame-skip case, its skipped frame given as a 0 flag
    g = json.load(open(os.path.join(GOLDEN, "gap_two_skips.json")))
    lp = f32log(g["probs"])
    st = oracle_lib.Stream(g["beam"], g["vocab"], g["blank"])
    st.feed(lp[:2], is_speech=[1, 0])
    st.feed(lp[2:], is_speech=[1, 1])
    assert st.step == 3 and st.frames == 4
    toks, L, S = st.read(g["nbest"], 4)
    hyps = live_hyps(toks, L, S)
    assert [list(h) for h, _ in hyps] == g["expected_tokens"]
    for (_, s), p in zip(hyps, g["expected_scores_log"]):
        assert s == pytest.approx(math.log(p), abs=1e-6)


def test_masked_stream_gap_golden_by_frame_index(oracle_lib):
    # the same case through the per-frame step with the caller's frame index
    g = json.load(open(os.path.join(GOLDEN, "gap_two_skips.json")))
    lp = f32log(g["probs"])
    st = oracle_lib.Stream(g["beam"], g["vocab"], g["blank"])
    for t in (0, 2, 3):
        st.step_at(lp[t], t)
    toks, L, S = st.read(g["nbest"], 4)
    assert [list(h) for h, _ in live_hyps(toks, L, S)] == g["expected_tokens"]


@pytest.mark.parametrize("theta,chunk", [(0.9, 7), (0.99, 16), (0.5, 5)])
def test_masked_stream_equals_offline_selection(oracle_lib, theta, chunk):
    # a mask computed as the offline filter (blank lp below log(theta), sec.
    # 3.5) must give the offline decode of that selection, bit for bit
    lp, lens = synth.peaky(3, 90, 13, seed=31, p_blank=0.6)
    off = oracle_lib.decode(lp, lens, 5, 5, 0, theta, 90)
    for b in range(3):
        sel = oracle_lib.select_frames(lp[b], 90, 0, theta)
        mask = np.zeros(90, np.uint8)
        mask[sel] = 1
        assert 0 < mask.sum() < 90
        st = oracle_lib.Stream(5, 13, 0)
        for a in range(0, 90, chunk):
            st.feed(lp[b, a:a + chunk], is_speech=mask[a:a + chunk])
        assert st.step == len(sel) and st.frames == 90
        t, l, s = st.read(5, 90)
        assert (t == off[0][b]).all() and (l == off[1][b]).all() and (s == off[2][b]).all()


def test_mask_of_ones_and_frame_indices_match_plain_feed(oracle_lib):
    lp, _ = synth.peaky(1, 48, 11, seed=32)
    plain = oracle_lib.Stream(4, 11, 0)
    ones = oracle_lib.Stream(4, 11, 0)
    steps = oracle_lib.Stream(4, 11, 0)
    for a in range(0, 48, 16):
        plain.feed(lp[0, a:a + 16])
        ones.feed(lp[0, a:a + 16], is_speech=np.ones(16, np.uint8))
    for t in range(48):
        steps.step_at(lp[0, t], t)
    ref = plain.read(4, 48)
    for other in (ones, steps):
        got = other.read(4, 48)
        assert all((x == y).all() for x, y in zip(got, ref))
        assert other.frames == 48


def test_start_frame_equals_masked_gap(oracle_lib):
    # a chunk fed from frame 20 after frames 0..15 is the same stream as one
    # whose frames 16..19 were marked 0
    lp, _ = synth.peaky(1, 36, 9, seed=33)
    a = oracle_lib.Stream(4, 9, 0)
    a.feed(lp[0, :16])
    a.feed(lp[0, 16:], start_frame=20)
    assert a.frames == 40 and a.step == 36
    b = oracle_lib.Stream(4, 9, 0)
    b.feed(lp[0, :16])
    b.feed(np.concatenate([np.zeros((4, 9), np.float32), lp[0, 16:]]),
           is_speech=np.r_[np.zeros(4), np.ones(20)].astype(np.uint8))
    assert b.frames == 40 and b.step == 36
    assert all((x == y).all() for x, y in zip(a.read(4, 36), b.read(4, 36)))
    # and it differs from the gap-free stream (the gap rule took effect)
    c = oracle_lib.Stream(4, 9, 0)
    c.feed(lp[0])
    assert not all((x == y).all() for x, y in zip(a.read(4, 36), c.read(4, 36)))


def test_all_zero_mask_decodes_nothing(oracle_lib):
    lp, _ = synth.peaky(1, 20, 7, seed=34)
    st = oracle_lib.Stream(3, 7, 0)
    st.feed(lp[0, :10], is_speech=np.zeros(10, np.uint8))
    assert st.step == 0 and st.frames == 10
    fresh = oracle_lib.Stream(3, 7, 0).read(3, 5)
    assert all((x == y).all() for x, y in zip(st.read(3, 5), fresh))
    # the first decoded frame then has index 10 > 0: seeded under the gap rule
    st.feed(lp[0, 10:])
    ref = oracle_lib.Stream(3, 7, 0)
    for t in range(10, 20):
        ref.step_at(lp[0, t], t)
    assert all((x == y).all() for x, y in zip(st.read(3, 10), ref.read(3, 10)))


# ------------------------------------------------------------ space slot --
# The space slot (sec. 3.4.1 skips the space label; sec. 3.4.2 scores it as
# lp[space] + logsumexp(pb, pnb) for every beam): a space frame always emits
# a new space token, so a beam ending in the space label has no stay term.
def collapse_space(path, blank, space):
    out, prev = [], None
    for c in path:
        if c == blank:
            pass
        elif c == space or c != prev:
            out.append(c)
        prev = c
    return tuple(out)


def brute_force_space(lp, blank, space):
    T, V = lp.shape
    lp64 = lp.astype(np.float64)
    acc = {}
    for path in itertools.product(range(V), repeat=T):
        s = float(sum(lp64[t, c] for t, c in enumerate(path)))
        key = collapse_space(path, blank, space)
        acc[key] = np.logaddexp(acc[key], s) if key in acc else s
    return acc


@pytest.mark.parametrize("T,V,space,seed", [(4, 3, 2, 0), (5, 4, 3, 1), (6, 3, 1, 2), (5, 4, 1, 3),
                                            (6, 4, 2, 4)])
def test_space_slot_unpruned_equals_brute_force(oracle_lib, T, V, space, seed):
    # token bias on the space label too, so that runs of space frames occur
    lp, lens = synth.peaky(1, T, V, seed=300 + seed, p_blank=0.4, blank_bias=1.0, token_bias=1.5,
                           repeat_p=0.6)
    exact = brute_force_space(lp[0], 0, space)
    W = len(exact) + V
    toks, L, S = oracle_lib.decode(lp, lens, W, W, 0, 1.0, T, space=space)
    got = live_hyps(toks[0], L[0], S[0])
    assert {h for h, _ in got} == set(exact)
    for h, sc in got:
        assert sc == pytest.approx(exact[h], abs=2e-5), h
    assert np.logaddexp.reduce([sc for _, sc in got]) == pytest.approx(0.0, abs=2e-5)
    # repeated spaces do occur among the hypotheses
    assert any(space in h and any(a == b == space for a, b in zip(h, h[1:])) for h, _ in got)


def test_space_slot_disabled_forms(oracle_lib):
    # -1 and the blank label mean no space slot (sec. 3.4.2: space_id >= 0 and
    # != blank_id)
    lp, lens = synth.peaky(3, 40, 9, seed=310, p_blank=0.5)
    base = oracle_lib.decode(lp, lens, 6, 6, 0, 1.0, 40)
    for sp in (-1, 0):
        other = oracle_lib.decode(lp, lens, 6, 6, 0, 1.0, 40, space=sp)
        for a, b in zip(base, other):
            assert (a == b).all()
    # and a space label that never reaches a beam changes nothing: label 8
    # made improbable in every frame
    lp2 = lp.copy()
    lp2[:, :, 8] = np.float32(-60.0)
    plain = oracle_lib.decode(lp2, lens, 6, 6, 0, 1.0, 40)
    sp = oracle_lib.decode(lp2, lens, 6, 6, 0, 1.0, 40, space=8)
    for a, b in zip(plain, sp):
        assert (a == b).all()


def test_space_slot_golden(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "space_slot.json")))
    lp = f32log(g["probs"])
    T = lp.shape[0]
    toks, L, S = oracle_lib.decode(lp[None], [T], g["beam"], g["nbest"], g["blank"],
                                   g["threshold"], T, space=g["space"])
    hyps = live_hyps(toks[0], L[0], S[0])
    assert [list(h) for h, _ in hyps] == g["expected_tokens"]
    for (_, s), p in zip(hyps, g["expected_scores_log"]):
        assert s == pytest.approx(math.log(p), abs=1e-6)
    # streaming gives the same (the space slot is part of every step)
    st = oracle_lib.Stream(g["beam"], g["vocab"], g["blank"], space=g["space"])
    st.feed(lp)
    t2, l2, s2 = st.read(g["nbest"], T)
    assert (t2 == toks[0]).all() and (l2 == L[0]).all() and (s2 == S[0]).all()


# ------------------------------------------------- paged page accounting --
def test_page_model_hand_worked(oracle_lib):
    # sec. 3.4.5 / 4.2 allocator on hand-chosen winners (tests/golden/page_model.json)
    oracle = oracle_lib
    g = json.load(open(os.path.join(GOLDEN, "page_model.json")))
    used, summary = oracle.page_model_run(g["beam"], g["page_size"], g["cap"], g["nseed"],
                                          g["src"], g["lab"], g["blank"])
    assert list(used) == g["used"]
    assert list(summary) == g["summary"]
    for pool in (4, 3):
        _, s = oracle.page_model_run(g["beam"], g["page_size"], g["cap"], g["nseed"], g["src"],
                                     g["lab"], g["blank"], num_pages=pool)
        assert list(s) == g[f"pool_{pool}"], pool


@pytest.mark.parametrize("W,ps", [(4, 4), (10, 16), (33, 8)])
def test_page_model_bounds_and_exact_pool(oracle_lib, W, ps):
    # the page's sizing claim (sec. 4.2): a row never needs more than
    # beam * (ceil(T / page_size) + 1) pages; pops take freed pages before the
    # bump pointer, so a pool of exactly the high-water mark never runs dry
    # and one page less does
    oracle = oracle_lib
    lp, lens = synth.peaky(4, 60, 30, seed=140 + W, p_blank=0.4)
    st = oracle.decode_pages(lp, lens, W, page_size=ps)
    bound = W * (-(-60 // ps) + 1)
    assert (st[:, 0] <= bound).all() and (st[:, 1] == 0).all() and (st[:, 0] > 0).all()
    for b in range(4):
        h = int(st[b, 0])
        ok = oracle.decode_pages(lp[b:b + 1], lens[b:b + 1], W, page_size=ps, num_pages=h)
        short = oracle.decode_pages(lp[b:b + 1], lens[b:b + 1], W, page_size=ps, num_pages=h - 1)
        assert ok[0, 1] == 0 and ok[0, 0] == h
        assert short[0, 1] == 1 and short[0, 2] >= 0


def test_page_model_stream_equals_offline(oracle_lib):
    # the accounting along a stream fed in chunks is that of the offline decode
    oracle = oracle_lib
    lp, lens = synth.peaky(1, 50, 20, seed=150, p_blank=0.5)
    st = oracle.Stream(12, 20, 0, capacity=50, page_size=4)
    for a in range(0, 50, 7):
        st.feed(lp[0, a:a + 7])
    off = oracle.decode_pages(lp, lens, 12, page_size=4)
    assert st.pages() == tuple(int(v) for v in off[0])


def test_rounding_ties_rank_by_id(oracle_lib):
    # frame 1 extends the empty prefix (score -1000) by labels 4, 5, 6 (log-prob
    # -1.0 and the next floats below it) and 2 (the float below those): every
    # sum rounds to -1001.0, so the candidates tie and rank by id, label 2
    # first, although it ranks last by log-probability.  The best two are [2]
    # and [4]; the prefix [1] (-1000.5) extends to -1001.5 at best.
    lp = synth.rounding_ties()
    assert {float(np.float32(-1000.0) + lp[0, 1, c]) for c in (2, 4, 5, 6)} == {-1001.0}
    t, l, s = oracle_lib.decode(lp, np.array([2], np.int32), 2, 2, 0, 1.0, 2)
    assert t[0, :, 0].tolist() == [2, 4] and l[0].tolist() == [1, 1]
    assert s[0].tolist() == [-1001.0, -1001.0]
