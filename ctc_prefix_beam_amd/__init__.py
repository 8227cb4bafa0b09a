"""Batched CTC prefix beam search on AMD Instinct MI355X (gfx950).

Thin Python binding of ``libctcpb.so`` (C ABI in ``include/ctcpb.h``).  This
module only marshals arguments: every step of the decode runs in the library's
HIP kernels.  PyTorch provides device memory and the current HIP stream.  If
the library is missing the calls raise; there is no CPU fallback.

The method and its options follow the page "GPU CTC Prefix Beam Search
Decoder" (OASR documentation), sections 9-11: an offline batch decode and a
streaming init / chunk / read-state lifecycle.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libctcpb.so")

FLAT, PAGED = 0, 1
EXPORTS = ("ctcpb_workspace_size", "ctcpb_decode_offline", "ctcpb_state_size",
           "ctcpb_stream_init", "ctcpb_stream_reset", "ctcpb_stream_chunk",
           "ctcpb_stream_chunk_ex", "ctcpb_stream_step", "ctcpb_read_state",
           "ctcpb_row_stats", "ctcpb_decode_offline_noalloc", "ctcpb_last_error",
           "ctcpb_version")
NOALLOC_SCRATCH_BYTES = 64 << 20   # CTCPB_NOALLOC_SCRATCH_BYTES
STAT_FIELDS = ("frames", "selected", "status", "pages_high", "fallbacks", "verifies", "common_prefix",
               "shared_pages")


class CtcpbConfig(ctypes.Structure):
    _fields_ = [("beam", ctypes.c_int32), ("nbest", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("blank_id", ctypes.c_int32), ("blank_threshold", ctypes.c_float),
                ("max_out_len", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("storage", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("space_id", ctypes.c_int32)]


@dataclass
class DecoderConfig:
    """Decoder options (the page's GpuDecoderConfig, sec. 10-11)."""
    beam: int = 10
    nbest: int | None = None
    blank_id: int = 0
    blank_threshold: float = 0.98
    max_out_len: int | None = None
    capacity: int = 0
    paged: bool = False
    page_size: int = 16
    num_pages: int = 0
    space_id: int = -1     # label of the space slot (sec. 3.4.2), -1 none

    def c_struct(self, vocab: int, max_out_len: int) -> CtcpbConfig:
        return CtcpbConfig(self.beam, self.nbest or self.beam, vocab, self.blank_id,
                           float(self.blank_threshold), max_out_len, self.capacity,
                           PAGED if self.paged else FLAT, self.page_size, self.num_pages,
                           self.space_id)


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with ctc_prefix_beam_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cfgp = ctypes.POINTER(CtcpbConfig)
        L.ctcpb_workspace_size.argtypes = [cfgp, i32, i32, ctypes.POINTER(sz)]
        L.ctcpb_decode_offline.argtypes = [cfgp, p, i64, i64, i32, i32, p, p, sz, p, p, p, p]
        L.ctcpb_state_size.argtypes = [cfgp, i32, ctypes.POINTER(sz)]
        L.ctcpb_stream_init.argtypes = [cfgp, p, sz, i32, p]
        L.ctcpb_stream_reset.argtypes = [cfgp, p, sz, i32, p, i32, p]
        L.ctcpb_stream_chunk.argtypes = [cfgp, p, sz, i32, p, i64, i64, i32, p, i32, p]
        L.ctcpb_stream_chunk_ex.argtypes = [cfgp, p, sz, i32, p, i64, i64, i32, p, p, p, i32, p]
        L.ctcpb_stream_step.argtypes = [cfgp, p, sz, i32, p, i64, p, p, i32, p]
        L.ctcpb_read_state.argtypes = [cfgp, p, sz, i32, p, i32, p, p, p, p]
        L.ctcpb_row_stats.argtypes = [cfgp, p, sz, i32, i32, p, p]
        L.ctcpb_decode_offline_noalloc.argtypes = [cfgp, p, i64, i64, i32, i32, p, p, p, p, p]
        for name in EXPORTS[:-2]:  # all but the two string getters
            getattr(L, name).restype = ctypes.c_int
        L.ctcpb_last_error.restype = ctypes.c_char_p
        L.ctcpb_last_error.argtypes = []
        L.ctcpb_version.restype = ctypes.c_char_p
        L.ctcpb_version.argtypes = []
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        msg = lib().ctcpb_last_error().decode()
        if rc == 1:
            raise ValueError(msg)
        raise RuntimeError(f"ctcpb error {rc}: {msg}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check_dev(t, device, name, dtype=None, shape=None, contiguous=False):
    """Raise ValueError unless `t` is a GPU tensor on `device` (and of the given
    dtype, shape and layout): the library hands raw device pointers to its
    kernels, so a host tensor or one on another GPU must never reach it."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device}, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_size(cfg: DecoderConfig, vocab: int, batch: int, max_T: int,
                   max_out_len: int | None = None) -> int:
    out = ctypes.c_size_t()
    c = cfg.c_struct(vocab, max_T if max_out_len is None else max_out_len)
    _check(lib().ctcpb_workspace_size(ctypes.byref(c), batch, max_T, ctypes.byref(out)))
    return out.value


def state_size(cfg: DecoderConfig, vocab: int, num_streams: int) -> int:
    out = ctypes.c_size_t()
    c = cfg.c_struct(vocab, cfg.max_out_len or 0)
    _check(lib().ctcpb_state_size(ctypes.byref(c), num_streams, ctypes.byref(out)))
    return out.value


class OfflineDecoder:
    """Offline batch decode (sec. 3.7).  Holds a reusable device workspace."""

    def __init__(self, cfg: DecoderConfig):
        self.cfg = cfg
        self.workspace = None

    def decode(self, log_prob: torch.Tensor, seq_lengths: torch.Tensor, out=None, stream=None):
        """log_prob: (B, T, V) float32 on the GPU, unit stride over V;
        seq_lengths: (B,) int32 on the GPU.  Returns (tokens (B, N, max_out_len)
        int32, lengths (B, N) int32, scores (B, N) float32) on the GPU."""
        if not isinstance(log_prob, torch.Tensor) or not log_prob.is_cuda:
            raise ValueError("log_prob must be a GPU tensor")
        dev = log_prob.device
        if log_prob.dtype != torch.float32 or log_prob.dim() != 3:
            raise ValueError("log_prob must be a 3-D float32 GPU tensor")
        if log_prob.stride(2) != 1:
            raise ValueError("log_prob must have unit stride over the vocabulary")
        B, T, V = log_prob.shape
        _check_dev(seq_lengths, dev, "seq_lengths", torch.int32, (B,), contiguous=True)
        if self.workspace is not None and self.workspace.device != dev:
            self.workspace = None   # a decoder reused on another GPU gets a new workspace
        cfg = self.cfg
        N = cfg.nbest or cfg.beam
        mol = T if cfg.max_out_len is None else cfg.max_out_len
        c = cfg.c_struct(V, mol)
        need = ctypes.c_size_t()
        _check(lib().ctcpb_workspace_size(ctypes.byref(c), B, T, ctypes.byref(need)))
        if self.workspace is None or self.workspace.numel() < need.value:
            self.workspace = torch.empty(max(need.value, 1), dtype=torch.uint8,
                                         device=log_prob.device)
        if out is None:
            out = (torch.empty((B, N, mol), dtype=torch.int32, device=log_prob.device),
                   torch.empty((B, N), dtype=torch.int32, device=log_prob.device),
                   torch.empty((B, N), dtype=torch.float32, device=log_prob.device))
        toks, lens, scores = out
        _check_dev(toks, dev, "out tokens", torch.int32, (B, N, mol), contiguous=True)
        _check_dev(lens, dev, "out lengths", torch.int32, (B, N), contiguous=True)
        _check_dev(scores, dev, "out scores", torch.float32, (B, N), contiguous=True)
        _check(lib().ctcpb_decode_offline(
            ctypes.byref(c), _ptr(log_prob), log_prob.stride(0), log_prob.stride(1), B, T,
            _ptr(seq_lengths), _ptr(self.workspace), self.workspace.numel(), _ptr(toks),
            _ptr(lens), _ptr(scores), _stream(stream)))
        self._last = (c, B, T)
        return toks, lens, scores

    def row_stats(self, stream=None) -> torch.Tensor:
        """Per-row counters of the last decode, int32 (B, 8): see STAT_FIELDS."""
        c, B, T = self._last
        out = torch.empty((B, 8), dtype=torch.int32, device=self.workspace.device)
        _check(lib().ctcpb_row_stats(ctypes.byref(c), _ptr(self.workspace), self.workspace.numel(),
                                     B, T, _ptr(out), _stream(stream)))
        return out


def decode_offline_noalloc(cfg: DecoderConfig, log_prob: torch.Tensor,
                           seq_lengths: torch.Tensor, out, stream=None):
    """ctcpb_decode_offline_noalloc: the offline decode with the library's
    fixed device scratch as its workspace (no allocation by the library or
    here).  `out` = (tokens (B, N, max_out_len) int32, lengths (B, N) int32,
    scores (B, N) float32), preallocated on log_prob's GPU.  Calls that may
    overlap on one GPU must be ordered by the caller (they share the scratch)."""
    if not isinstance(log_prob, torch.Tensor) or not log_prob.is_cuda:
        raise ValueError("log_prob must be a GPU tensor")
    dev = log_prob.device
    if log_prob.dtype != torch.float32 or log_prob.dim() != 3 or log_prob.stride(2) != 1:
        raise ValueError("log_prob must be a 3-D float32 tensor with unit stride over V")
    B, T, V = log_prob.shape
    _check_dev(seq_lengths, dev, "seq_lengths", torch.int32, (B,), contiguous=True)
    N = cfg.nbest or cfg.beam
    toks, lens, scores = out
    mol = toks.shape[2] if toks.dim() == 3 else -1
    _check_dev(toks, dev, "out tokens", torch.int32, (B, N, mol), contiguous=True)
    _check_dev(lens, dev, "out lengths", torch.int32, (B, N), contiguous=True)
    _check_dev(scores, dev, "out scores", torch.float32, (B, N), contiguous=True)
    c = cfg.c_struct(V, mol)
    _check(lib().ctcpb_decode_offline_noalloc(
        ctypes.byref(c), _ptr(log_prob), log_prob.stride(0), log_prob.stride(1), B, T,
        _ptr(seq_lengths), _ptr(toks), _ptr(lens), _ptr(scores), _stream(stream)))
    return toks, lens, scores


def decode_offline(log_prob, seq_lengths, **kw):
    """One-shot offline decode; keyword arguments are DecoderConfig fields."""
    return OfflineDecoder(DecoderConfig(**kw)).decode(log_prob, seq_lengths)


class StreamPool:
    """A device-resident state blob of `num_streams` independent streams
    (sec. 8): init, chunk after chunk, read the N best at any time."""

    def __init__(self, cfg: DecoderConfig, vocab: int, num_streams: int, device="cuda",
                 stream=None):
        self.cfg, self.vocab, self.num_streams = cfg, vocab, num_streams
        self.max_out_len = cfg.max_out_len if cfg.max_out_len is not None else (
            cfg.capacity or 4096)
        self.c = cfg.c_struct(vocab, self.max_out_len)
        need = ctypes.c_size_t()
        _check(lib().ctcpb_state_size(ctypes.byref(self.c), num_streams, ctypes.byref(need)))
        self.state = torch.empty(max(need.value, 1), dtype=torch.uint8, device=device)
        self.nbytes = need.value
        _check(lib().ctcpb_stream_init(ctypes.byref(self.c), _ptr(self.state), self.nbytes,
                                       num_streams, _stream(stream)))

    def _rows(self, rows, n=None):
        if rows is not None:
            _check_dev(rows, self.state.device, "rows", torch.int32, contiguous=True)
            if rows.dim() != 1 or (n is not None and rows.numel() != n):
                raise ValueError("rows must be a 1-D int32 tensor with one entry per row")
        return rows

    def reset(self, rows: torch.Tensor | None = None, stream=None):
        self._rows(rows)
        n = self.num_streams if rows is None else rows.numel()
        _check(lib().ctcpb_stream_reset(ctypes.byref(self.c), _ptr(self.state), self.nbytes,
                                        self.num_streams, _ptr(rows), n, _stream(stream)))

    def chunk(self, log_prob_chunk: torch.Tensor, rows: torch.Tensor | None = None, stream=None,
              is_speech: torch.Tensor | None = None, start_frame: torch.Tensor | None = None):
        """log_prob_chunk: (n_rows, chunk_T, V) float32 on the GPU; row i
        continues stream rows[i] (default: stream i).  is_speech: optional
        (n_rows, chunk_T) uint8 on the GPU, 0 = skip the frame; start_frame:
        optional (n_rows,) int32 on the GPU, the number of each row's first
        frame (default: the stream's own frame count)."""
        _check_dev(log_prob_chunk, self.state.device, "log_prob_chunk", torch.float32)
        if log_prob_chunk.dim() != 3:
            raise ValueError("log_prob_chunk must be a 3-D float32 tensor")
        if log_prob_chunk.stride(2) != 1:
            raise ValueError("log_prob_chunk must have unit stride over the vocabulary")
        n, T, V = log_prob_chunk.shape
        if V != self.vocab:
            raise ValueError("vocabulary size differs from the pool's")
        self._rows(rows, n)
        if is_speech is not None:
            _check_dev(is_speech, self.state.device, "is_speech", torch.uint8, (n, T),
                       contiguous=True)
        if start_frame is not None:
            _check_dev(start_frame, self.state.device, "start_frame", torch.int32, (n,),
                       contiguous=True)
        if is_speech is None and start_frame is None:
            _check(lib().ctcpb_stream_chunk(
                ctypes.byref(self.c), _ptr(self.state), self.nbytes, self.num_streams,
                _ptr(log_prob_chunk), log_prob_chunk.stride(0), log_prob_chunk.stride(1), T,
                _ptr(rows), n, _stream(stream)))
        else:
            _check(lib().ctcpb_stream_chunk_ex(
                ctypes.byref(self.c), _ptr(self.state), self.nbytes, self.num_streams,
                _ptr(log_prob_chunk), log_prob_chunk.stride(0), log_prob_chunk.stride(1), T,
                _ptr(is_speech), _ptr(start_frame), _ptr(rows), n, _stream(stream)))

    def step(self, log_prob_frame: torch.Tensor, frame_index: torch.Tensor | None = None,
             rows: torch.Tensor | None = None, stream=None):
        """One frame per row: log_prob_frame (n_rows, V) float32 on the GPU,
        decoded as frame number frame_index[i] (int32 on the GPU; default: the
        stream's own frame count) of stream rows[i]."""
        _check_dev(log_prob_frame, self.state.device, "log_prob_frame", torch.float32)
        if log_prob_frame.dim() != 2:
            raise ValueError("log_prob_frame must be a 2-D float32 tensor")
        if log_prob_frame.stride(1) != 1:
            raise ValueError("log_prob_frame must have unit stride over the vocabulary")
        n, V = log_prob_frame.shape
        if V != self.vocab:
            raise ValueError("vocabulary size differs from the pool's")
        self._rows(rows, n)
        if frame_index is not None:
            _check_dev(frame_index, self.state.device, "frame_index", torch.int32, (n,),
                       contiguous=True)
        _check(lib().ctcpb_stream_step(
            ctypes.byref(self.c), _ptr(self.state), self.nbytes, self.num_streams,
            _ptr(log_prob_frame), log_prob_frame.stride(0), _ptr(frame_index), _ptr(rows), n,
            _stream(stream)))

    def row_stats(self, stream=None) -> torch.Tensor:
        """Per-stream counters, int32 (num_streams, 8): see STAT_FIELDS."""
        out = torch.empty((self.num_streams, 8), dtype=torch.int32, device=self.state.device)
        _check(lib().ctcpb_row_stats(ctypes.byref(self.c), _ptr(self.state), self.nbytes,
                                     self.num_streams, 0, _ptr(out), _stream(stream)))
        return out

    def read(self, rows: torch.Tensor | None = None, stream=None):
        self._rows(rows)
        n = self.num_streams if rows is None else rows.numel()
        N = self.cfg.nbest or self.cfg.beam
        dev = self.state.device
        toks = torch.empty((n, N, self.max_out_len), dtype=torch.int32, device=dev)
        lens = torch.empty((n, N), dtype=torch.int32, device=dev)
        scores = torch.empty((n, N), dtype=torch.float32, device=dev)
        _check(lib().ctcpb_read_state(ctypes.byref(self.c), _ptr(self.state), self.nbytes,
                                      self.num_streams, _ptr(rows), n, _ptr(toks), _ptr(lens),
                                      _ptr(scores), _stream(stream)))
        return toks, lens, scores
