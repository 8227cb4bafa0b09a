"""ctcpb_decode_offline_noalloc through the C ABI: the offline decode with the
library's fixed device scratch as its workspace must give exactly what
ctcpb_decode_offline gives with a caller workspace, on consecutive calls
(the second smaller than the first, so stale scratch contents from the first
call are present), and refuse a decode that does not fit its scratch."""
import ctypes

import numpy as np
import pytest
import torch

import ctc_prefix_beam_amd as cpb
import oracle
import synth
from gpu_util import assert_parity

pytestmark = pytest.mark.gpu


def with_workspace(cfg, x, lens_d):
    dec = cpb.OfflineDecoder(cfg)
    out = dec.decode(x, lens_d)
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in out)


def no_alloc(cfg, x, lens_d, N, mol):
    B, T, V = x.shape
    dev = x.device
    out = (torch.full((B, N, mol), 7, dtype=torch.int32, device=dev),
           torch.full((B, N), 7, dtype=torch.int32, device=dev),
           torch.full((B, N), 7.0, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    c = cfg.c_struct(V, mol)
    rc = cpb.lib().ctcpb_decode_offline_noalloc(
        ctypes.byref(c), ctypes.c_void_p(x.data_ptr()), x.stride(0), x.stride(1), B, T,
        ctypes.c_void_p(lens_d.data_ptr()), ctypes.c_void_p(out[0].data_ptr()),
        ctypes.c_void_p(out[1].data_ptr()), ctypes.c_void_p(out[2].data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, cpb.lib().ctcpb_last_error().decode()
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in out)


CASES = [
    # (B, T, V, beam, threshold, max_out_len, paged, seed, num_pages): the first
    # call fills much of the scratch, the next ones are smaller and read over
    # stale contents (a pool the caller sizes, and beams above 32, included)
    (24, 400, 1024, 16, 0.999, 256, True, 1, 0),
    (5, 150, 1024, 16, 0.9, 150, True, 2, 0),
    (12, 300, 300, 32, 1.0, 300, False, 3, 0),
    (6, 120, 200, 48, 1.0, 120, True, 5, 0),
    (4, 100, 200, 8, 0.95, 100, True, 6, 8 * (100 // 16 + 2)),
    (2, 60, 40, 4, 0.9, 60, False, 4, 0),
]


def test_no_alloc_equals_workspace_decode_at_full_size_then_smaller():
    # vocab5000 at full size with flat token lists: about 50 MB of the 64 MiB
    # scratch, then the smaller cases below over its stale contents
    wl = synth.WORKLOADS["vocab5000"]
    x, lens = wl.make_device(0, "cuda")
    lens_d = torch.from_numpy(lens).cuda()
    cfg = cpb.DecoderConfig(beam=wl.beam, nbest=wl.nbest, blank_threshold=wl.threshold,
                            max_out_len=wl.max_out_len)
    assert cpb.workspace_size(cfg, wl.V, wl.B, wl.T, wl.max_out_len) > 40 << 20
    print(f"[case] no-alloc vocab5000 flat B={wl.B} T={wl.T}", flush=True)
    ref = with_workspace(cfg, x, lens_d)
    got = no_alloc(cfg, x, lens_d, wl.nbest, wl.max_out_len)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
    del x
    torch.cuda.empty_cache()
    for B, T, V, W, thr, mol, paged, seed, npages in CASES:
        print(f"[case] no-alloc B={B} T={T} V={V} W={W} paged={paged} num_pages={npages}",
              flush=True)
        lp, lens = synth.peaky(B, T, V, seed=seed, p_blank=0.6, lengths=(T // 2, T))
        x = torch.from_numpy(lp).cuda()
        lens_d = torch.from_numpy(lens).cuda()
        cfg = cpb.DecoderConfig(beam=W, nbest=W, blank_threshold=thr, max_out_len=mol,
                                paged=paged, num_pages=npages)
        ref = with_workspace(cfg, x, lens_d)
        got = no_alloc(cfg, x, lens_d, W, mol)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)
        if B * T * V <= 2_000_000:
            assert_parity(got, oracle.decode(lp, lens, W, W, 0, thr, mol), what="no-alloc")


def test_no_alloc_refuses_a_decode_larger_than_its_scratch():
    # vocab5000-sized rows with flat token lists: 200 rows need more than the
    # scratch; refused before anything is enqueued (outputs untouched)
    cfg = cpb.DecoderConfig(beam=32, nbest=32, blank_threshold=0.999, max_out_len=8)
    need = cpb.workspace_size(cfg, 5000, 200, 1500, 8)
    assert need > cpb.NOALLOC_SCRATCH_BYTES
    c = cfg.c_struct(5000, 8)
    x = torch.zeros(4, dtype=torch.float32, device="cuda")
    out = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(x.data_ptr())
    rc = cpb.lib().ctcpb_decode_offline_noalloc(ctypes.byref(c), p, 1500 * 5000, 5000, 200,
                                                1500, ctypes.c_void_p(out.data_ptr()), p, p, p,
                                                None)
    assert rc == 2
    assert "scratch" in cpb.lib().ctcpb_last_error().decode()
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 7).all()
