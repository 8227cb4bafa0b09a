"""Helpers of the GPU parity tests: run the HIP decoder and the oracle on the
same seeded inputs and compare them."""
import numpy as np
import torch

import ctc_prefix_beam_amd as cpb
import oracle

TOL = 1e-4  # absolute, log domain
DEAD = -3.0e38  # scores at or below this are dead slots (-FLT_MAX)


def gpu_offline(lp, lens, beam, nbest, blank, threshold, max_out_len, paged=False, page_size=16,
                num_pages=0, device="cuda", check_status=True):
    dec = cpb.OfflineDecoder(cpb.DecoderConfig(beam=beam, nbest=nbest, blank_id=blank,
                                               blank_threshold=threshold,
                                               max_out_len=max_out_len, paged=paged,
                                               page_size=page_size, num_pages=num_pages))
    x = lp if isinstance(lp, torch.Tensor) else torch.from_numpy(lp)
    t, l, s = dec.decode(x.to(device), torch.as_tensor(lens, dtype=torch.int32).to(device))
    stats = dec.row_stats().cpu().numpy()
    torch.cuda.synchronize()
    assert not check_status or (stats[:, 2] == 0).all(), f"row status bits set: {np.unique(stats[:, 2])}"
    gpu_offline.last_stats = stats   # per-row counters of the call (cpb.STAT_FIELDS)
    return t.cpu().numpy(), l.cpu().numpy(), s.cpu().numpy()


def tie_groups(scores, tol=TOL):
    """Ranks of one row grouped into runs whose consecutive oracle scores lie
    within `tol` of each other (scores are in descending order)."""
    groups, cur = [], [0]
    for n in range(1, len(scores)):
        if abs(float(scores[n]) - float(scores[n - 1])) <= tol:
            cur.append(n)
        else:
            groups.append(cur)
            cur = [n]
    groups.append(cur)
    return groups


def assert_parity(got, ref, rows=None, exact=True, what=""):
    """Tokens and lengths bit-exact per rank; scores within TOL (bit-exact if
    `exact` wherever the rank holds the oracle's hypothesis).  Ranks whose
    oracle scores lie within TOL of each other (a near-tie group) may hold
    their hypotheses in any order, but the group's GPU hypotheses must be a
    permutation of the oracle's.  A group that reaches the last reported rank
    may continue past the N-best cut, so there the GPU may report another
    hypothesis of the tie: its hypotheses need only be distinct (among those
    that fit the output width)."""
    gt, gl, gs = got
    rt, rl, rs = ref
    B, N = rl.shape
    rows = range(B) if rows is None else rows

    def hyp(t, l, b, n):
        return (int(l[b, n]), tuple(int(v) for v in t[b, n]))

    for i, b in enumerate(rows):
        for grp in tie_groups(rs[b]):
            mine = [hyp(gt, gl, i, n) for n in grp]
            theirs = [hyp(rt, rl, b, n) for n in grp]
            for n in grp:
                assert abs(float(gs[i, n]) - float(rs[b, n])) <= TOL, (
                    f"{what} row {b} rank {n}: score {gs[i, n]!r} vs {rs[b, n]!r}")
                if exact and hyp(gt, gl, i, n) == hyp(rt, rl, b, n):
                    assert gs[i, n] == rs[b, n], (
                        f"{what} row {b} rank {n}: score {gs[i, n]!r} vs {rs[b, n]!r} not bitwise")
            if len(grp) == 1:
                n = grp[0]
                assert mine[0] == theirs[0], (
                    f"{what} row {b} rank {n}: gpu len {gl[i, n]} score {gs[i, n]!r} vs oracle "
                    f"len {rl[b, n]} score {rs[b, n]!r}; first tokens gpu {gt[i, n, :8]} "
                    f"oracle {rt[b, n, :8]}")
            elif grp[-1] == N - 1 and rs[b, N - 1] > DEAD:
                # (hypotheses longer than the output width are compared by
                # their reported prefix only, which two of them may share)
                mol = gt.shape[2]
                live = [h for h, n in zip(mine, grp) if gs[i, n] > DEAD and h[0] <= mol]
                assert len(set(live)) == len(live), (
                    f"{what} row {b} ranks {grp}: duplicated hypothesis in a tie at the cut")
            else:
                assert sorted(mine) == sorted(theirs), (
                    f"{what} row {b} ranks {grp}: tie group is not a permutation of the "
                    f"oracle's hypotheses")
