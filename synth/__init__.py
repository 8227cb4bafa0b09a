"""Seeded synthetic CTC posteriors ("peaky" log_prob tensors).

This module only draws inputs.  It holds none of the decoder's arithmetic and
is shared by the tests, the smoke check and the benchmark, so that the HIP
decoder and the CPU oracle always see the same bits.

Recipe (one frame t of row b, all draws from ``numpy.random.default_rng(seed)``
in the order stated in ``peaky``): logits z ~ N(0, 1) over the vocabulary; with
probability ``p_blank`` the frame is blank-dominant and the blank logit gets
``blank_bias``; otherwise one non-blank token gets ``token_bias`` - with
probability 0.3 it repeats the row's previous peaked token, else it is uniform
over the non-blank ids.  A fraction ``p_low`` of frames is low-confidence: its
peak bias is 2 instead.  log_prob = z - logsumexp(z) in float64, rounded once
to float32.  Frames at or past a row's length can be filled with NaN, which a
correct decoder never reads.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def peaky(B: int, T: int, V: int, seed: int, p_blank: float = 0.65,
          blank_bias: float = 8.0, token_bias=6.0, p_low: float = 0.0,
          low_bias: float = 2.0, lengths=None, nan_tail: bool = False,
          blank: int = 0, repeat_p: float = 0.3, dtype=np.float32):
    """Return (log_prob[B, T, V] float32, lengths[B] int32).

    ``token_bias`` is a number, or a (lo, hi) pair for a per-frame uniform
    draw.  ``lengths`` is None (all T), an int array, or a (lo, hi) pair for
    a per-row uniform integer draw in [lo, hi].
    """
    rng = np.random.default_rng(seed)
    if lengths is None:
        lens = np.full(B, T, np.int32)
    elif isinstance(lengths, tuple):
        lens = rng.integers(lengths[0], lengths[1] + 1, size=B).astype(np.int32)
    else:
        lens = np.asarray(lengths, np.int32)
    out = np.empty((B, T, V), dtype)
    nonblank = np.array([c for c in range(V) if c != blank], np.int64)
    for b in range(B):
        z = rng.standard_normal((T, V))
        low = rng.random(T) < p_low
        is_blank = rng.random(T) < p_blank
        u = rng.random(T)
        rand_tok = nonblank[rng.integers(0, V - 1, size=T)]
        if isinstance(token_bias, tuple):
            tb = rng.uniform(token_bias[0], token_bias[1], size=T)
        else:
            tb = np.full(T, float(token_bias))
        tok = np.empty(T, np.int64)
        prev = -1
        for t in range(T):
            if is_blank[t]:
                tok[t] = blank
            else:
                tok[t] = prev if (prev >= 0 and u[t] < repeat_p) else rand_tok[t]
                prev = tok[t]
        bias = np.where(low, low_bias, np.where(is_blank, blank_bias, tb))
        z[np.arange(T), tok] += bias
        m = z.max(axis=1, keepdims=True)
        lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))
        out[b] = (z - lse).astype(dtype)
        if nan_tail and lens[b] < T:
            out[b, lens[b]:] = np.nan
    return out, lens


def peaky_device(B: int, T: int, V: int, seed: int, device, p_blank: float = 0.65,
                 blank_bias: float = 8.0, token_bias=6.0, p_low: float = 0.0,
                 low_bias: float = 2.0, lengths=None, nan_tail: bool = False,
                 blank: int = 0, repeat_p: float = 0.3, rows_per_chunk: int = 8):
    """Same recipe as ``peaky`` for large tensors: the per-frame choices are
    drawn with numpy, the logits with a seeded torch generator on `device`
    (float64), so the tensor never exists on the host.  Returns (log_prob
    torch float32 on device, lengths numpy int32).  Its bits differ from
    ``peaky`` with the same seed (another generator), not its distribution."""
    import torch
    rng = np.random.default_rng(seed)
    if lengths is None:
        lens = np.full(B, T, np.int32)
    elif isinstance(lengths, tuple):
        lens = rng.integers(lengths[0], lengths[1] + 1, size=B).astype(np.int32)
    else:
        lens = np.asarray(lengths, np.int32)
    nonblank = np.array([c for c in range(V) if c != blank], np.int64)
    low = rng.random((B, T)) < p_low
    is_blank = rng.random((B, T)) < p_blank
    u = rng.random((B, T))
    rand_tok = nonblank[rng.integers(0, V - 1, size=(B, T))]
    if isinstance(token_bias, tuple):
        tb = rng.uniform(token_bias[0], token_bias[1], size=(B, T))
    else:
        tb = np.full((B, T), float(token_bias))
    tok = np.empty((B, T), np.int64)
    prev = np.full(B, -1, np.int64)
    for t in range(T):
        pick = np.where((prev >= 0) & (u[:, t] < repeat_p), prev, rand_tok[:, t])
        tok[:, t] = np.where(is_blank[:, t], blank, pick)
        prev = np.where(is_blank[:, t], prev, pick)
    bias = np.where(low, low_bias, np.where(is_blank, blank_bias, tb))
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = torch.empty((B, T, V), dtype=torch.float32, device=device)
    for b0 in range(0, B, rows_per_chunk):
        b1 = min(B, b0 + rows_per_chunk)
        z = torch.randn((b1 - b0, T, V), generator=gen, device=device, dtype=torch.float64)
        idx = torch.from_numpy(tok[b0:b1]).to(device).unsqueeze(-1)
        z.scatter_add_(2, idx, torch.from_numpy(bias[b0:b1]).to(device).unsqueeze(-1))
        out[b0:b1] = (z - torch.logsumexp(z, dim=2, keepdim=True)).to(torch.float32)
        del z
    if nan_tail:
        for b in range(B):
            if lens[b] < T:
                out[b, lens[b]:] = float("nan")
    return out, lens


def rounding_ties(V: int = 8, n_tied: int = 4, dtype=np.float32):
    """Two frames (log_prob[1, 2, V]) built so that the second frame's best
    extensions of the first frame's best prefix all round to one score.

    Frame 0 makes the empty prefix score -1000 and the prefix [1] score
    -1000.5.  In frame 1, labels 4, 5, 6, ... get -1.0 and the next floats
    below it, and label 2 the float below those (n_tied labels in all): added
    to -1000 (spacing 2^-14 there) they all give -1001.0.  So the label that
    ranks last by log-probability has the smallest id among the tied
    extensions.  Every other entry is far below.
    """
    lp = np.full((1, 2, V), -3000.0, dtype)
    lp[0, 0, 0] = -1000.0
    lp[0, 0, 1] = -1000.5
    lp[0, 1, :] = -100.0 - np.arange(V, dtype=dtype)
    x = np.float32(-1.0)
    for c in list(range(4, 4 + n_tied - 1)) + [2]:
        lp[0, 1, c] = x
        x = np.nextafter(x, np.float32(-np.inf))
    lp[0, 1, 0] = -60.0
    return lp


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    V: int
    beam: int
    nbest: int
    threshold: float
    max_out_len: int
    gen: dict = field(default_factory=dict)
    streaming: bool = False
    chunk: int = 0
    paged: bool = False

    def make(self, seed: int, B: int | None = None, T: int | None = None):
        """Inputs of this workload (optionally with fewer rows or frames)."""
        return peaky(B or self.B, T or self.T, self.V, seed, **self.gen)

    def make_device(self, seed: int, device, B: int | None = None, T: int | None = None):
        """Full-size inputs drawn directly on `device` (see peaky_device)."""
        return peaky_device(B or self.B, T or self.T, self.V, seed, device, **self.gen)


# The five workloads: shapes, decode settings and generator parameters.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 50, 29, 4, 4, 1.0, 50, dict(p_blank=0.65)),
    "bpe256": Workload("bpe256", 16, 500, 256, 8, 8, 0.999, 200, dict(p_blank=0.6)),
    "bpe1024": Workload("bpe1024", 64, 875, 1024, 16, 16, 0.999, 256,
                        dict(p_blank=0.7, token_bias=(3.0, 8.0), lengths=(300, 875),
                             nan_tail=True)),
    "stream512": Workload("stream512", 256, 1024, 512, 10, 10, 1.0, 4096,
                          dict(p_blank=0.65), streaming=True, chunk=16),
    "vocab5000": Workload("vocab5000", 128, 1500, 5000, 32, 32, 0.999, 512,
                          dict(p_blank=0.55, p_low=0.2), paged=True),
}
