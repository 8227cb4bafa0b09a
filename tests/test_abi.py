"""Host-side checks of libctcpb.so that need no GPU: every symbol declared in
include/ctcpb.h is exported, the size queries are consistent, and every
validation path returns its documented status before touching the device."""
import ctypes
import os
import re

import pytest

import ctc_prefix_beam_amd as cpb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ctcpb.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(cpb.LIB_PATH):
        from ctc_prefix_beam_amd import build
        build.build()
    return cpb.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ctcpb_\w+)\s*\(", text, re.M)))


def cfg(**kw):
    base = dict(beam=8, nbest=8, vocab=256, blank_id=0, blank_threshold=0.999, max_out_len=200,
                capacity=0, storage=0, page_size=16, num_pages=0, space_id=-1)
    base.update(kw)
    return cpb.CtcpbConfig(**base)


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(cpb.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n
    assert L.ctcpb_version().decode().startswith("ctcpb")


def ws(L, c, B, T):
    out = ctypes.c_size_t()
    rc = L.ctcpb_workspace_size(ctypes.byref(c), B, T, ctypes.byref(out))
    return rc, out.value


def ss(L, c, S):
    out = ctypes.c_size_t()
    rc = L.ctcpb_state_size(ctypes.byref(c), S, ctypes.byref(out))
    return rc, out.value


def test_size_queries(L):
    rc, one = ws(L, cfg(), 1, 500)
    assert rc == 0 and one > 0 and one % 256 == 0
    rc, sixteen = ws(L, cfg(), 16, 500)
    assert rc == 0 and sixteen == 16 * one                     # rows are independent regions
    assert ws(L, cfg(), 16, 1000)[1] > sixteen                 # grows with the frame count
    assert ws(L, cfg(), 0, 500) == (0, 0)
    rc, flat = ss(L, cfg(vocab=512, beam=10, nbest=10), 256)
    rc2, paged = ss(L, cfg(vocab=512, beam=10, nbest=10, storage=1), 256)
    assert rc == rc2 == 0 and flat > 0 and paged > 0
    # capacity 0 means the default 4096 tokens per stream
    assert ss(L, cfg(capacity=0), 3)[1] == ss(L, cfg(capacity=4096), 3)[1]


@pytest.mark.parametrize("kw,code", [
    (dict(beam=0), 1), (dict(beam=129), 1),
    (dict(nbest=0), 1), (dict(nbest=9), 1), (dict(vocab=1), 1), (dict(vocab=20000), 3),
    (dict(blank_id=-1), 1), (dict(blank_id=256), 1), (dict(max_out_len=-1), 1),
    (dict(storage=2), 1), (dict(storage=1, page_size=3), 1), (dict(storage=1, page_size=65), 1),
    (dict(storage=1, page_size=6), 1), (dict(storage=1, page_size=12), 1),
    (dict(num_pages=-1), 1), (dict(capacity=-5), 1), (dict(blank_threshold=float("nan")), 1),
    (dict(space_id=256), 1),
])
def test_config_validation(L, kw, code):
    rc, _ = ws(L, cfg(**kw), 2, 10)
    assert rc == code
    assert L.ctcpb_last_error().decode() != ""
    assert ws(L, cfg(), 2, 10)[0] == 0
    assert L.ctcpb_last_error().decode() == ""


def test_decode_argument_errors_need_no_device(L):
    c = cfg()
    p = ctypes.c_void_p(256)  # never dereferenced: every case fails on the host
    n = ctypes.c_void_p(None)
    # NULL pointers
    assert L.ctcpb_decode_offline(ctypes.byref(c), n, 500 * 256, 256, 2, 500, p, p, 1 << 30,
                                  p, p, p, n) == 1
    # stride_t smaller than the vocabulary
    assert L.ctcpb_decode_offline(ctypes.byref(c), p, 500 * 256, 100, 2, 500, p, p, 1 << 30,
                                  p, p, p, n) == 1
    # workspace too small
    need = ws(L, c, 2, 500)[1]
    assert L.ctcpb_decode_offline(ctypes.byref(c), p, 500 * 256, 256, 2, 500, p, p, need - 1,
                                  p, p, p, n) == 2
    # empty batch: nothing to do
    assert L.ctcpb_decode_offline(ctypes.byref(c), n, 0, 256, 0, 500, n, n, 0, n, n, n, n) == 0
    # LDS budget: a very wide vocabulary with paged metadata does not fit a CU
    # (the size query says so too)
    big = cfg(vocab=16384, beam=32, nbest=32, storage=1, page_size=4, max_out_len=8)
    assert ws(L, big, 1, 20000)[0] == 3
    assert L.ctcpb_decode_offline(ctypes.byref(big), p, 20000 * 16384, 16384, 1, 20000, p, p,
                                  1 << 62, p, p, p, n) == 3


# The vocabulary limits ctcpb_config.vocab documents: (beam, storage, frames,
# largest V that fits one CU).  Checked through the size queries, which make
# the decoder's own LDS check and launch nothing.
DOCUMENTED_LIMITS = [(8, 0, 1500, 14616), (16, 0, 1500, 14540), (32, 0, 1500, 14232),
                     (8, 1, 1500, 13756), (16, 1, 1500, 12896), (32, 1, 1500, 11180),
                     (32, 1, 4096, 5996)]


@pytest.mark.parametrize("beam,storage,T,vmax", DOCUMENTED_LIMITS)
def test_documented_vocabulary_limits(L, beam, storage, T, vmax):
    def c(V):
        return cfg(beam=beam, nbest=min(beam, 8), vocab=V, storage=storage, max_out_len=512,
                   capacity=T)
    assert ws(L, c(vmax), 1, T)[0] == 0
    assert ws(L, c(vmax + 1), 1, T)[0] == 3
    # a stream's capacity plays the part of max_T
    assert ss(L, c(vmax), 1)[0] == 0
    assert ss(L, c(vmax + 1), 1)[0] == 3
    # beams above 32 (the wide decoder) fit every vocabulary
    assert ws(L, cfg(beam=64, nbest=8, vocab=16384, storage=storage), 1, T)[0] == 0


def test_wide_beams_flat_and_paged(L):
    # beams of 33..128 run on the wide decoder (flat or paged tokens), offline
    # and streaming; its kept beam state makes a stream's region larger
    assert ws(L, cfg(beam=128, nbest=128), 2, 100)[0] == 0
    rc, paged = ws(L, cfg(beam=128, nbest=128, storage=1), 2, 100)
    assert rc == 0 and paged > 0
    rc, wide = ss(L, cfg(beam=64, nbest=8), 4)
    assert rc == 0 and wide > ss(L, cfg(beam=32, nbest=8), 4)[1]
    assert ss(L, cfg(beam=64, nbest=8, storage=1), 4)[0] == 0


def test_stream_argument_errors_need_no_device(L):
    c = cfg(vocab=512, beam=10, nbest=10)
    p = ctypes.c_void_p(256)
    n = ctypes.c_void_p(None)
    need = ss(L, c, 4)[1]
    assert L.ctcpb_stream_init(ctypes.byref(c), p, need - 1, 4, n) == 2
    assert L.ctcpb_stream_reset(ctypes.byref(c), p, need, 4, n, 5, n) == 1
    assert L.ctcpb_stream_chunk(ctypes.byref(c), p, need, 4, p, 16 * 512, 512, 16, n, 5, n) == 1
    assert L.ctcpb_stream_chunk(ctypes.byref(c), p, need, 4, p, 16 * 512, 100, 16, n, 4, n) == 1
    assert L.ctcpb_stream_chunk(ctypes.byref(c), p, need, 4, p, 16 * 512, 512, -1, n, 4, n) == 1
    assert L.ctcpb_stream_chunk(ctypes.byref(c), p, need, 4, p, 16 * 512, 512, 0, n, 4, n) == 0
    # the gated / indexed variants validate the same way
    assert L.ctcpb_stream_chunk_ex(ctypes.byref(c), p, need, 4, p, 16 * 512, 512, 16, p, p, n, 5,
                                   n) == 1
    assert L.ctcpb_stream_chunk_ex(ctypes.byref(c), p, need - 1, 4, p, 16 * 512, 512, 16, p, n,
                                   n, 4, n) == 2
    assert L.ctcpb_stream_chunk_ex(ctypes.byref(c), p, need, 4, n, 16 * 512, 512, 16, p, n, n, 4,
                                   n) == 1
    assert L.ctcpb_stream_chunk_ex(ctypes.byref(c), p, need, 4, p, 16 * 512, 512, 0, p, p, n, 4,
                                   n) == 0
    assert L.ctcpb_stream_step(ctypes.byref(c), p, need, 4, p, 512, p, n, 5, n) == 1
    assert L.ctcpb_stream_step(ctypes.byref(c), p, need - 1, 4, p, 512, p, n, 4, n) == 2
    assert L.ctcpb_stream_step(ctypes.byref(c), n, need, 4, p, 512, p, n, 4, n) == 1
    assert L.ctcpb_read_state(ctypes.byref(c), p, need - 1, 4, n, 4, p, p, p, n) == 2
    assert L.ctcpb_read_state(ctypes.byref(c), n, need, 4, n, 4, p, p, p, n) == 1


def test_python_wrapper_raises():
    with pytest.raises(ValueError):
        cpb.workspace_size(cpb.DecoderConfig(beam=0), 256, 2, 10)
    with pytest.raises(RuntimeError):
        cpb.workspace_size(cpb.DecoderConfig(beam=8), 20000, 2, 10)
