"""CPU reference ("oracle") of batched CTC prefix beam search.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The decoder
library (``ctc_prefix_beam_amd``) never imports, loads or calls it, and the two
share no code.

The arithmetic lives in ``ctc_oracle.c`` (plain C, float32, following the page
"GPU CTC Prefix Beam Search Decoder", sections 3.1-3.7, 8 and 13); this module
only builds it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ctc_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

# One rounding per written operation: no contraction, no fast-math.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-builtin-expf", "-Wall", "-Wextra", "-Wno-unused-parameter"]

NEG = -np.finfo(np.float32).max


def build(force: bool = True) -> str:
    """Compile liboracle.so next to its source (gcc, host only)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        f32, i32, i64, p = ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        L.oracle_exp.restype = f32
        L.oracle_exp.argtypes = [f32]
        L.oracle_log1p.restype = f32
        L.oracle_log1p.argtypes = [f32]
        L.oracle_lse.restype = f32
        L.oracle_lse.argtypes = [f32, f32]
        L.oracle_math_sweep.restype = None
        L.oracle_math_sweep.argtypes = [i32, ctypes.c_uint32, i64, p, p, p]
        L.oracle_log_threshold.restype = f32
        L.oracle_log_threshold.argtypes = [f32]
        L.oracle_select_frames.restype = i32
        L.oracle_select_frames.argtypes = [p, i64, i32, i32, f32, p]
        L.oracle_decode.restype = i32
        L.oracle_decode.argtypes = [p, i64, i64, i32, i32, p, i32, i32, i32, i32, f32, i32,
                                    p, p, p]
        L.oracle_decode_sp.restype = i32
        L.oracle_decode_sp.argtypes = [p, i64, i64, i32, i32, p, i32, i32, i32, i32, f32, i32,
                                       p, p, p, i32]
        L.oracle_stream_new.restype = p
        L.oracle_stream_new.argtypes = [i32, i32, i32, i32]
        L.oracle_stream_new_sp.restype = p
        L.oracle_stream_new_sp.argtypes = [i32, i32, i32, i32, i32]
        L.oracle_stream_free.restype = None
        L.oracle_stream_free.argtypes = [p]
        L.oracle_stream_reset.restype = None
        L.oracle_stream_reset.argtypes = [p]
        L.oracle_stream_feed.restype = i32
        L.oracle_stream_feed.argtypes = [p, p, i64, i32]
        L.oracle_stream_feed_ex.restype = i32
        L.oracle_stream_feed_ex.argtypes = [p, p, i64, i32, p, i32]
        L.oracle_stream_frame_count.restype = i32
        L.oracle_stream_frame_count.argtypes = [p]
        L.oracle_stream_step_count.restype = i32
        L.oracle_stream_step_count.argtypes = [p]
        L.oracle_stream_read.restype = None
        L.oracle_stream_read.argtypes = [p, i32, i32, p, p, p]
        L.oracle_stream_new_paged.restype = p
        L.oracle_stream_new_paged.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.oracle_stream_pages.restype = None
        L.oracle_stream_pages.argtypes = [p, p]
        L.oracle_decode_pages.restype = i32
        L.oracle_decode_pages.argtypes = [p, i64, i64, i32, i32, p, i32, i32, i32, f32, i32,
                                          i32, i32, p]
        L.oracle_page_model_run.restype = i32
        L.oracle_page_model_run.argtypes = [i32, i32, i32, i32, i32, i32, i32, p, p, p, p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def exp(x: float) -> float:
    return lib().oracle_exp(float(x))


def log1p(x: float) -> float:
    return lib().oracle_log1p(float(x))


def lse(a: float, b: float) -> float:
    return lib().oracle_lse(float(a), float(b))


def math_sweep(op: int, first_bits: int, n: int, a=None, b=None, threads: int = 1) -> np.ndarray:
    """The oracle's exp (op 0), log1p (op 1) or x / (2 + x) (op 2) of the n
    floats whose bit patterns start at first_bits, or lse(a, b) (op 3), as a
    float32 array.  Runs on `threads` threads (ctypes releases the GIL)."""
    out = np.empty(n, np.float32)
    if op == 3:
        a = np.ascontiguousarray(a, np.float32)
        b = np.ascontiguousarray(b, np.float32)
        assert a.shape == b.shape == (n,)

    def part(lo, hi):
        pa = None if op != 3 else a[lo:hi].ctypes.data_as(ctypes.c_void_p)
        pb = None if op != 3 else b[lo:hi].ctypes.data_as(ctypes.c_void_p)
        lib().oracle_math_sweep(op, (first_bits + lo) & 0xffffffff, hi - lo, pa, pb,
                                out[lo:hi].ctypes.data_as(ctypes.c_void_p))

    if threads <= 1 or n < 1 << 16:
        part(0, n)
    else:
        from concurrent.futures import ThreadPoolExecutor
        step = -(-n // threads)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda lo: part(lo, min(n, lo + step)), range(0, n, step)))
    return out


def select_frames(lp_row: np.ndarray, length: int, blank: int, threshold: float) -> np.ndarray:
    lp_row = np.ascontiguousarray(lp_row, dtype=np.float32)
    T, V = lp_row.shape
    sel = np.zeros(max(T, 1), np.int32)
    n = lib().oracle_select_frames(_ptr(lp_row), V, int(length), int(blank),
                                   float(threshold), _ptr(sel))
    return sel[:n].copy()


def decode(log_prob: np.ndarray, seq_lengths, beam: int, nbest: int | None = None,
           blank: int = 0, threshold: float = 1.0, max_out_len: int | None = None,
           space: int = -1):
    """Offline decode (`space`: the space label of the space slot, -1 none).
    Returns (tokens[B,N,max_out_len] -1 padded, lengths[B,N], scores[B,N])."""
    log_prob = np.ascontiguousarray(log_prob, dtype=np.float32)
    B, T, V = log_prob.shape
    nbest = beam if nbest is None else nbest
    max_out_len = T if max_out_len is None else max_out_len
    lens = np.ascontiguousarray(seq_lengths, dtype=np.int32)
    assert lens.shape == (B,)
    toks = np.full((B, nbest, max(max_out_len, 0)), -1, np.int32)
    lengths = np.zeros((B, nbest), np.int32)
    scores = np.zeros((B, nbest), np.float32)
    rc = lib().oracle_decode_sp(_ptr(log_prob), T * V, V, B, T, _ptr(lens), beam, nbest, V,
                                blank, float(threshold), max_out_len, _ptr(toks),
                                _ptr(lengths), _ptr(scores), int(space))
    if rc != 0:
        raise ValueError("oracle_decode: invalid argument")
    return toks, lengths, scores


def decode_pages(log_prob: np.ndarray, seq_lengths, beam: int, blank: int = 0,
                 threshold: float = 1.0, space: int = -1, page_size: int = 16,
                 num_pages: int = 0) -> np.ndarray:
    """The paged variant's page accounting along offline decodes (the page's
    allocator, sec. 3.4.5 / 4.2): int32 [B, 3] = most pages in use at once, 1
    if a pop found nothing, the step of the first such pop (-1)."""
    log_prob = np.ascontiguousarray(log_prob, dtype=np.float32)
    B, T, V = log_prob.shape
    lens = np.ascontiguousarray(seq_lengths, dtype=np.int32)
    out = np.zeros((B, 3), np.int32)
    rc = lib().oracle_decode_pages(_ptr(log_prob), T * V, V, B, T, _ptr(lens), beam, V, blank,
                                   float(threshold), int(space), page_size, num_pages, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_decode_pages: invalid argument")
    return out


def page_model_run(beam: int, page_size: int, cap: int, nseed: int, src, lab, blank: int = 0,
                   num_pages: int = 0):
    """The page model alone on given winners: src / lab [nsteps][beam] for
    steps 1..nsteps (source slot, -1 dead; label).  Returns (pages in use
    after each step [nsteps + 1], (high, failed, first failing step))."""
    src = np.ascontiguousarray(src, dtype=np.int32).reshape(-1, beam)
    lab = np.ascontiguousarray(lab, dtype=np.int32).reshape(-1, beam)
    n = src.shape[0]
    used = np.zeros(n + 1, np.int32)
    out = np.zeros(3, np.int32)
    rc = lib().oracle_page_model_run(beam, page_size, num_pages, cap, blank, nseed, n,
                                     _ptr(src), _ptr(lab), _ptr(used), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_page_model_run: invalid argument")
    return used, tuple(int(v) for v in out)


class Stream:
    """One streaming decode: frames fed in chunks, optionally gated by a
    speech mask (0 = skip the frame) and numbered from a caller-given frame
    index.  With page_size, it also counts pages as the paged variant's
    allocator would (pages())."""

    def __init__(self, beam: int, vocab: int, blank: int = 0, capacity: int = 4096,
                 space: int = -1, page_size: int | None = None, num_pages: int = 0):
        self.beam, self.vocab = beam, vocab
        if page_size is None:
            self._h = lib().oracle_stream_new_sp(beam, vocab, blank, capacity, space)
        else:
            self._h = lib().oracle_stream_new_paged(beam, vocab, blank, capacity, space,
                                                    page_size, num_pages)
        if not self._h:
            raise ValueError("oracle_stream_new: invalid argument")

    def pages(self):
        """(most pages in use at once, 1 if a pop found nothing, first such step)."""
        out = np.zeros(3, np.int32)
        lib().oracle_stream_pages(self._h, _ptr(out))
        return tuple(int(v) for v in out)

    def feed(self, frames: np.ndarray, is_speech=None, start_frame: int | None = None) -> int:
        """Chunk frame f is frame number start + f (start = start_frame, or the
        frames given so far); it is decoded unless is_speech[f] == 0."""
        frames = np.ascontiguousarray(frames, dtype=np.float32)
        n, V = frames.shape
        assert V == self.vocab
        if is_speech is None and start_frame is None:
            return lib().oracle_stream_feed(self._h, _ptr(frames), V, n)
        mask = None
        if is_speech is not None:
            mask = np.ascontiguousarray(is_speech, dtype=np.uint8)
            assert mask.shape == (n,)
        start = -1 if start_frame is None else int(start_frame)
        assert start_frame is None or start >= 0
        return lib().oracle_stream_feed_ex(self._h, _ptr(frames), V, n,
                                           None if mask is None else _ptr(mask), start)

    def step_at(self, frame: np.ndarray, frame_index: int) -> int:
        """One frame decoded as frame number frame_index (the page's per-frame
        step with the caller's actual frame index)."""
        return self.feed(np.asarray(frame, np.float32).reshape(1, -1), None, frame_index)

    @property
    def frames(self) -> int:
        return lib().oracle_stream_frame_count(self._h)

    @property
    def step(self) -> int:
        return lib().oracle_stream_step_count(self._h)

    def reset(self):
        lib().oracle_stream_reset(self._h)

    def read(self, nbest: int | None = None, max_out_len: int = 4096):
        nbest = self.beam if nbest is None else nbest
        toks = np.full((nbest, max_out_len), -1, np.int32)
        lengths = np.zeros(nbest, np.int32)
        scores = np.zeros(nbest, np.float32)
        lib().oracle_stream_read(self._h, nbest, max_out_len, _ptr(toks), _ptr(lengths),
                                 _ptr(scores))
        return toks, lengths, scores

    def close(self):
        if self._h:
            lib().oracle_stream_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def decode_parallel(log_prob, seq_lengths, beam, nbest=None, blank=0, threshold=1.0,
                    max_out_len=None, processes: int = 1, space: int = -1):
    """Rows spread over `processes` threads of this process (rows are
    independent, each decode is single-threaded C and ctypes releases the
    GIL).  Same results as ``decode``."""
    if processes <= 1:
        return decode(log_prob, seq_lengths, beam, nbest, blank, threshold, max_out_len, space)
    from concurrent.futures import ThreadPoolExecutor
    B = log_prob.shape[0]
    nbest = beam if nbest is None else nbest
    max_out_len = log_prob.shape[1] if max_out_len is None else max_out_len
    lens = np.asarray(seq_lengths, np.int32)

    def one(b):
        return decode(log_prob[b:b + 1], lens[b:b + 1], beam, nbest, blank, threshold,
                      max_out_len, space)

    with ThreadPoolExecutor(processes) as ex:
        parts = list(ex.map(one, range(B)))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]),
            np.concatenate([p[2] for p in parts]))
