"""Helpers of the GPU parity tests: run the HIP decoder and the oracle on the
same seeded inputs and compare them."""
import numpy as np
import torch

import ctc_prefix_beam_amd as cpb
import oracle

TOL = 1e-4  # absolute, log domain


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


def assert_parity(got, ref, rows=None, exact=True, what=""):
    """Tokens and lengths bit-exact per rank; scores within TOL (bit-exact if
    `exact`).  Two ranks whose oracle scores lie within TOL of each other may
    hold their hypotheses in either order."""
    gt, gl, gs = got
    rt, rl, rs = ref
    B, N = rl.shape
    rows = range(B) if rows is None else rows
    for i, b in enumerate(rows):
        for n in range(N):
            same = (gl[i, n] == rl[b, n] and np.array_equal(gt[i, n], rt[b, n]))
            if not same:
                near = [m for m in range(N) if m != n and abs(rs[b, m] - rs[b, n]) <= TOL]
                swapped = any(gl[i, n] == rl[b, m] and np.array_equal(gt[i, n], rt[b, m])
                              for m in near)
                assert swapped, (f"{what} row {b} rank {n}: gpu len {gl[i, n]} score "
                                 f"{gs[i, n]!r} vs oracle len {rl[b, n]} score {rs[b, n]!r}; "
                                 f"first tokens gpu {gt[i, n, :8]} oracle {rt[b, n, :8]}")
            assert abs(float(gs[i, n]) - float(rs[b, n])) <= TOL, (
                f"{what} row {b} rank {n}: score {gs[i, n]!r} vs {rs[b, n]!r}")
            if exact and same:
                assert gs[i, n] == rs[b, n], (
                    f"{what} row {b} rank {n}: score {gs[i, n]!r} vs {rs[b, n]!r} not bitwise")
