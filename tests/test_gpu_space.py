"""The space slot (sec. 3.4.1 / 3.4.2, config space_id) on the GPU against the
oracle: offline with flat and paged tokens, streaming, the exact beam x vocab
selection, wide beams; a space label equal to the blank means no slot."""
import numpy as np
import pytest
import torch

import ctc_prefix_beam_amd as cpb
import oracle
import synth
from gpu_util import assert_parity

pytestmark = pytest.mark.gpu


def with_space_runs(B, T, V, space, seed, frac=0.35, bias=5.0, **kw):
    """Peaky frames; a fraction of them gets a peak on the space label (so
    that runs of space frames occur), renormalised in float64."""
    lp, lens = synth.peaky(B, T, V, seed=seed, **kw)
    rng = np.random.default_rng(seed + 1000)
    pick = rng.random((B, T)) < frac
    z = lp.astype(np.float64)
    z[pick, space] += bias
    m = z.max(axis=2, keepdims=True)
    z = z - (m + np.log(np.exp(z - m).sum(axis=2, keepdims=True)))
    return z.astype(np.float32), lens


def gpu_decode(lp, lens, W, thr, mol, space, paged=False):
    dec = cpb.OfflineDecoder(cpb.DecoderConfig(beam=W, nbest=W, blank_threshold=thr,
                                               max_out_len=mol, paged=paged, space_id=space))
    t, l, s = dec.decode(torch.from_numpy(lp).cuda(), torch.from_numpy(lens).cuda())
    st = dec.row_stats().cpu().numpy()
    torch.cuda.synchronize()
    assert (st[:, 2] == 0).all()
    gpu_decode.stats = st
    return t.cpu().numpy(), l.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("W,V,space,paged,thr", [(4, 29, 3, False, 1.0), (8, 40, 39, True, 1.0),
                                                 (16, 300, 1, False, 0.9), (32, 120, 7, True, 1.0),
                                                 (10, 512, 500, False, 1.0), (1, 12, 2, False, 1.0)])
def test_space_slot_offline(W, V, space, paged, thr):
    lp, lens = with_space_runs(4, 80, V, space, seed=W * 7 + V, p_blank=0.5, lengths=(40, 80))
    print(f"[case] space offline W={W} V={V} space={space} paged={paged}", flush=True)
    got = gpu_decode(lp, lens, W, thr, 80, space, paged)
    ref = oracle.decode(lp, lens, W, W, 0, thr, 80, space=space)
    assert_parity(got, ref, what=f"space W{W}")
    # the decode differs from the one without a space slot
    plain = oracle.decode(lp, lens, W, W, 0, thr, 80)
    assert any(not np.array_equal(a, b) for a, b in zip(ref, plain))


def test_space_equal_to_blank_means_none():
    lp, lens = synth.peaky(3, 60, 50, seed=71, p_blank=0.5)
    a = gpu_decode(lp, lens, 8, 1.0, 60, 0)
    b = gpu_decode(lp, lens, 8, 1.0, 60, -1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert_parity(a, oracle.decode(lp, lens, 8, 8, 0, 1.0, 60), what="space=blank")


def test_space_slot_exact_selection():
    # frames with every non-blank label at one log-probability force the full
    # beam x vocabulary selection, where a beam ending in the space label
    # extends by it as by any other label
    lp, lens = with_space_runs(3, 60, 96, 5, seed=72, p_blank=0.5)
    pick = np.random.default_rng(73).random((3, 60)) < 0.25
    flat = np.full(96, np.log(0.999 / 95), np.float32)
    flat[0] = np.float32(np.log(0.001))
    lp[pick] = flat
    got = gpu_decode(lp, lens, 12, 1.0, 60, 5)
    assert gpu_decode.stats[:, cpb.STAT_FIELDS.index("fallbacks")].sum() > 0
    assert_parity(got, oracle.decode(lp, lens, 12, 12, 0, 1.0, 60, space=5), what="space fallback")


@pytest.mark.parametrize("paged", [False, True])
def test_space_slot_streaming(paged):
    S, T, V, W, CH, space = 5, 96, 200, 10, 16, 11
    lp, _ = with_space_runs(S, T, V, space, seed=74, p_blank=0.55)
    print(f"[case] space stream S={S} T={T} V={V} W={W} paged={paged}", flush=True)
    pool = cpb.StreamPool(cpb.DecoderConfig(beam=W, nbest=W, max_out_len=T, paged=paged,
                                            space_id=space), V, S)
    x = torch.from_numpy(lp).cuda()
    for a in range(0, T, CH):
        pool.chunk(x[:, a:a + CH])
    t, l, s = pool.read()
    torch.cuda.synchronize()
    got = (t.cpu().numpy(), l.cpu().numpy(), s.cpu().numpy())
    outs = []
    for i in range(S):
        st = oracle.Stream(W, V, 0, 4096, space=space)
        for a in range(0, T, CH):
            st.feed(lp[i, a:a + CH])
        outs.append(st.read(W, T))
    ref = tuple(np.stack([o[i] for o in outs]) for i in range(3))
    assert_parity(got, ref, what="space stream")


@pytest.mark.parametrize("W", [40, 64])
def test_space_slot_wide_beams(W):
    lp, lens = with_space_runs(3, 70, 150, 9, seed=75 + W, p_blank=0.5)
    print(f"[case] space wide W={W}", flush=True)
    got = gpu_decode(lp, lens, W, 1.0, 70, 9)
    assert_parity(got, oracle.decode(lp, lens, W, W, 0, 1.0, 70, space=9), what=f"space wide {W}")
