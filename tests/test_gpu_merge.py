"""The merge's exact token comparison on the GPU.

The decoder tracks which beam is another's prefix minus its last label
structurally (from how the winners were formed).  The one case that the
structure cannot decide is a beam whose parent prefix was not live in the
previous step and is re-created in this step by extending its own parent; the
decoder then looks the new prefix up by a hash and confirms it with an exact
token comparison (row_stats [5] counts them).  These inputs make that happen:
the oracle's beam sets, read after every step, say in which steps and rows,
and the GPU must count at least as many comparisons there and still match the
oracle."""
import numpy as np
import pytest

import ctc_prefix_beam_amd as cpb
import oracle
import synth
from gpu_util import assert_parity, gpu_offline

pytestmark = pytest.mark.gpu


def recreated_parents(lp, W):
    """Steps in which a live prefix h (two labels or more) stays live while
    h[:-1], not live before the step, becomes live in it (oracle beam sets)."""
    T, V = lp.shape
    st = oracle.Stream(W, V, 0, T)
    prev, n = set(), 0
    for t in range(T):
        st.feed(lp[t:t + 1])
        toks, L, S = st.read(W, T)
        cur = {tuple(toks[r, :L[r]]) for r in range(W) if S[r] > -3e38}
        n += sum(1 for h in cur if len(h) >= 2 and h in prev and h[:-1] not in prev
                 and h[:-1] in cur)
        prev = cur
    return n


@pytest.mark.parametrize("W,paged", [(4, False), (6, True), (3, False), (40, False), (36, True)])
def test_recreated_parent_prefixes_are_compared_exactly(W, paged):
    B, T, V = 40, 60, 3
    rows = [synth.peaky(1, T, V, seed=s, p_blank=0.3, blank_bias=1.0, token_bias=1.0,
                        repeat_p=0.5)[0][0] for s in range(B)]
    lp = np.stack(rows)
    lens = np.full(B, T, np.int32)
    events = np.array([recreated_parents(lp[b], W) for b in range(B)])
    assert events.sum() > 0
    print(f"[case] merge compare B={B} T={T} V={V} W={W} paged={paged} events={events.sum()}",
          flush=True)
    got = gpu_offline(lp, lens, W, W, 0, 1.0, T, paged=paged)
    verifies = gpu_offline.last_stats[:, cpb.STAT_FIELDS.index("verifies")]
    assert_parity(got, oracle.decode(lp, lens, W, W, 0, 1.0, T), what=f"merge W{W}")
    assert (verifies >= events).all(), (verifies, events)
    assert verifies.sum() > 0
