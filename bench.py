#!/usr/bin/env python3
"""Benchmark of the MI355X CTC prefix beam search decoder.

Headline: decoded frames per second (B*T per second) of the offline decode of
the large-vocabulary workload (B=128 utterances x T=1500 frames, V=5000,
beam 32, 32-best, blank threshold 0.999, 512-token outputs, paged token
storage), one GPU, inputs resident in HBM before the timed region.  A step is
one ctcpb_decode_offline call over the whole batch (frame filter + decode).
Also reported on the same line: the roofline of the decode kernel, the CPU
oracle's throughput on a bounded sample (one thread and the host's cores),
the other offline workloads (tiny, bpe256, bpe1024, vocab5000 with flat
storage) with their roofline fractions, per-chunk latency of 256 concurrent
streams (V=512, beam 10, 16-frame chunks) at capacity 1024 and 4096, and
beams of 64 and 128.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, vendor figure
PMC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_vocab5000_pmc.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha():
    """Identity of the built decoder (hash of libctcpb.so): the stored HBM
    counter figures are used only while the library they were taken on is the
    one being timed."""
    import ctc_prefix_beam_amd as cpb
    return hashlib.sha256(open(cpb.LIB_PATH, "rb").read()).hexdigest()[:16]


def algorithmic_bytes_per_frame(V, W):
    # the frame's log-probabilities read once, plus the beam state of every
    # slot read and written (pb, pnb, score, last label, length: 20 B) and one
    # 4-byte token append
    return 4 * V + 44 * W


def time_offline(dec, x, lens_d, out, steps, warmup):
    import torch
    for _ in range(warmup):
        dec.decode(x, lens_d, out=out)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        dec.decode(x, lens_d, out=out)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = [a.elapsed_time(b) for a, b in evs]
    return wall, kernel_ms


def host_threads():
    """Threads the oracle may use: the cores this process may run on, at most
    16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(x, lens, wl, seconds):
    """The oracle as it stands on a bounded sample of the same workload: first
    on one thread (the first frames of one row), then one row per thread on
    the host's cores (the first frames of `threads` rows), each sized to about
    `seconds` of work."""
    import numpy as np

    import oracle
    oracle.build(force=False)
    threads = host_threads()
    # a quick probe on a few frames sizes the samples
    probe_T = min(60, wl.T)
    lp1 = x[0:1, :probe_T].cpu().numpy()
    t = time.perf_counter()
    oracle.decode(lp1, np.array([probe_T], np.int32), wl.beam, wl.nbest, 0, wl.threshold,
                  wl.max_out_len)
    per_frame = (time.perf_counter() - t) / probe_T
    T = int(min(wl.T, max(probe_T, seconds / max(per_frame, 1e-9))))

    # one thread, one row
    lp = x[0:1, :T].cpu().numpy()
    ln = np.minimum(lens[0:1], T).astype(np.int32)
    t = time.perf_counter()
    oracle.decode(lp, ln, wl.beam, wl.nbest, 0, wl.threshold, wl.max_out_len)
    wall1 = time.perf_counter() - t
    one = {"value": round(float(T / wall1), 1), "unit": "decoded frames/s", "cores": 1,
           "sample": f"row 0 x first {T} frames of {wl.name} ({wall1:.1f} s)"}

    rows = list(range(threads))
    lp = x[rows, :T].cpu().numpy()
    ln = np.minimum(lens[rows], T).astype(np.int32)
    t = time.perf_counter()
    oracle.decode_parallel(lp, ln, wl.beam, wl.nbest, 0, wl.threshold, wl.max_out_len,
                           processes=threads)
    wall = time.perf_counter() - t
    return {"value": round(float(len(rows) * T / wall), 1), "unit": "decoded frames/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} rows x first {T} frames of {wl.name}, one single-threaded "
                      f"oracle decode per row on {threads} threads ({wall:.1f} s)",
            "host_cpu_count": os.cpu_count(), "one_core": one}


SPACER_CYCLES = 1_000_000   # GPU clock cycles of the spin kernel before a timed chunk


def streaming_latency(reps=3, seed=0, mask_theta=None, capacity=None):
    """256 streams, 64 chunks of 16 frames: per-chunk latency of one
    ctcpb_stream_chunk call advancing every stream (device time by HIP events
    around the chunk's GPU work, the host's enqueue hidden behind a spin kernel;
    host time from the Python call to completion, in separate passes).  `capacity` is the frames (and
    tokens) a stream can hold: the session's 1024, or the page's default 4096
    (whose flat token lists no longer fit on chip).  With mask_theta, each
    chunk is gated by a speech mask computed once on the GPU as blank log-prob
    < log(mask_theta) (frames flagged 0 are skipped)."""
    import numpy as np
    import torch

    import ctc_prefix_beam_amd as cpb
    import synth
    wl = synth.WORKLOADS["stream512"]
    x, _ = wl.make_device(seed, "cuda")
    cap = wl.T if capacity is None else capacity
    pool = cpb.StreamPool(cpb.DecoderConfig(beam=wl.beam, nbest=wl.nbest, max_out_len=wl.T,
                                            capacity=cap), wl.V, wl.B)
    mask = None
    if mask_theta is not None:
        mask = (x[:, :, 0] < float(np.float32(np.log(mask_theta)))).to(torch.uint8)
        masks = [mask[:, a:a + wl.chunk].contiguous() for a in range(0, wl.T, wl.chunk)]
    dev_ms, host_ms = [], []
    for rep in range(2 * reps + 1):
        # passes alternate: device time, then host time (the first pass is a warm-up)
        spaced = rep % 2 == 1
        pool.reset()
        torch.cuda.synchronize()
        for ci, a in enumerate(range(0, wl.T, wl.chunk)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if spaced:
                # a spin kernel keeps the GPU busy while the host enqueues the
                # events and the chunk, so that the events bracket the chunk's
                # GPU work only (not the binding's host-side argument handling)
                torch.cuda._sleep(SPACER_CYCLES)
            t = time.perf_counter()
            e0.record()
            pool.chunk(x[:, a:a + wl.chunk], is_speech=None if mask is None else masks[ci])
            e1.record()
            torch.cuda.synchronize()
            if rep > 0 and spaced:
                dev_ms.append(e0.elapsed_time(e1))
            elif rep > 0:
                host_ms.append((time.perf_counter() - t) * 1e3)
    d = np.array(dev_ms)
    h = np.array(host_ms)
    if mask is not None:
        frac = float(mask.float().mean())
        return {"mask": f"blank log-prob < log({mask_theta}), computed once on the GPU",
                "speech_fraction": round(frac, 4),
                "p50_chunk_ms": round(float(np.percentile(d, 50)), 4),
                "p90_chunk_ms": round(float(np.percentile(d, 90)), 4),
                "decoded_frames_per_s": round(float(wl.B * wl.chunk * frac / (d.mean() / 1e3)), 1),
                "chunks_timed": int(d.size)}
    return {"workload": f"stream512: 256 streams, V=512, beam 10, 16-frame chunks, 64 chunks, "
                        f"capacity {cap}",
            "p50_chunk_ms": round(float(np.percentile(d, 50)), 4),
            "p90_chunk_ms": round(float(np.percentile(d, 90)), 4),
            "p99_chunk_ms": round(float(np.percentile(d, 99)), 4),
            "p50_host_chunk_ms": round(float(np.percentile(h, 50)), 4),
            "device_timing": f"HIP events around the chunk, behind a {SPACER_CYCLES}-cycle spin "
                             "kernel (host enqueue excluded); host: Python call to completion",
            "frames_per_s": round(float(wl.B * wl.chunk / (d.mean() / 1e3)), 1),
            "launches_per_chunk": 1,
            "chunks_timed": int(d.size)}


def wide_beams():
    """Beams above 32 (the wide offline decoder, flat tokens) on the bpe1024
    inputs (B=64, T=875, V=1024, ragged lengths), beam 64 and 128."""
    import numpy as np
    import torch

    import ctc_prefix_beam_amd as cpb
    import synth
    wl = synth.WORKLOADS["bpe1024"]
    x, lens = wl.make_device(0, "cuda")
    lens_d = torch.from_numpy(lens).cuda()
    res = {"workload": "bpe1024 inputs: B=64 T=875 V=1024 ragged 300..875, threshold 0.999, "
                       "flat tokens"}
    for W in (64, 128):
        dec = cpb.OfflineDecoder(cpb.DecoderConfig(beam=W, nbest=W,
                                                   blank_threshold=wl.threshold,
                                                   max_out_len=wl.max_out_len))
        out = dec.decode(x, lens_d)
        wall, kms = time_offline(dec, x, lens_d, out, 3, 1)
        st = dec.row_stats().cpu().numpy()
        steps = int(st[:, 0].sum())
        ms = float(np.mean(kms))
        alg = steps * algorithmic_bytes_per_frame(wl.V, W)
        res[f"beam{W}"] = {"ms_per_decode": round(ms, 3),
                           "frames_per_s": round(wl.B * wl.T / (ms / 1e3), 1),
                           "decoded_frames_per_s": round(steps / (ms / 1e3), 1),
                           "us_per_step": round(ms * 1e3 / max(1, int(st[:, 0].max())), 2),
                           "hbm_frac": round(alg / (ms / 1e3) / 8.0e12, 5)}
    del x
    return res


def other_workloads():
    """The other offline workloads (flat token lists, as configured) and
    vocab5000 with flat storage beside the paged headline: one decode per
    step, timed with HIP events, with each one's roofline fraction."""
    import numpy as np
    import torch

    import ctc_prefix_beam_amd as cpb
    import synth
    res = {}
    for name, paged, steps in (("tiny", False, 20), ("bpe256", False, 10), ("bpe1024", False, 10),
                               ("vocab5000", False, 5)):
        wl = synth.WORKLOADS[name]
        x, lens = wl.make_device(0, "cuda")
        lens_d = torch.from_numpy(lens).cuda()
        dec = cpb.OfflineDecoder(cpb.DecoderConfig(beam=wl.beam, nbest=wl.nbest,
                                                   blank_threshold=wl.threshold,
                                                   max_out_len=wl.max_out_len, paged=paged))
        out = dec.decode(x, lens_d)
        wall, kms = time_offline(dec, x, lens_d, out, steps, 2)
        st = dec.row_stats().cpu().numpy()
        sel = int(st[:, 1].sum())
        ms = float(np.mean(kms))
        alg = sel * algorithmic_bytes_per_frame(wl.V, wl.beam)
        key = name + ("_paged" if paged else "_flat")
        res[key] = {"shape": f"B={wl.B} T={wl.T} V={wl.V} beam={wl.beam}",
                    "ms_per_decode": round(ms, 4),
                    "frames_per_s": round(wl.B * wl.T / (ms / 1e3), 1),
                    "valid_frames_per_s": round(float(np.sum(lens)) / (ms / 1e3), 1),
                    "selected_frames": sel,
                    "hbm_frac": round(alg / (ms / 1e3) / (PEAK_HBM_GBS * 1e9), 5),
                    "us_per_step": round(ms * 1e3 / max(1, int(st[:, 0].max())), 3),
                    "fallback_steps": int(st[:, 4].sum()),
                    "workspace_bytes": int(dec.workspace.numel())}
        del x
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="vocab5000")
    ap.add_argument("--storage", choices=["paged", "flat"], default="paged")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other workloads, streaming latency and wide beams")
    ap.add_argument("--with-copy", action="store_true",
                    help="after the timed decodes, run a plain streaming kernel of known size "
                         "twice (1 GiB read, 1 GiB written, 16-byte accesses per lane) to "
                         "calibrate the HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decoder shards by utterance/stream with no "
              f"exchange between GPUs, and this benchmark measures one GPU's share (got --gpus "
              f"{args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ctc_prefix_beam_amd as cpb
    import synth

    torch.cuda.set_device(0)

    wl = synth.WORKLOADS[args.workload]
    paged = args.storage == "paged"
    log(f"[bench] generating {wl.name} inputs on the GPU: B={wl.B} T={wl.T} V={wl.V}")
    x, lens = wl.make_device(0, "cuda")
    lens_d = torch.from_numpy(lens).cuda()
    cfg = cpb.DecoderConfig(beam=wl.beam, nbest=wl.nbest, blank_threshold=wl.threshold,
                            max_out_len=wl.max_out_len, paged=paged)
    dec = cpb.OfflineDecoder(cfg)
    out = dec.decode(x, lens_d)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} decodes after {args.warmup} warm-up")
    wall, kernel_ms = time_offline(dec, x, lens_d, out, args.steps, args.warmup)
    stats = dec.row_stats().cpu().numpy()
    selected = int(stats[:, 1].sum())
    frames = wl.B * wl.T
    value = frames * args.steps / wall
    launch_ms = float(np.mean(kernel_ms))
    bytes_per_launch = selected * algorithmic_bytes_per_frame(wl.V, wl.beam)
    achieved = bytes_per_launch / (launch_ms / 1e3) / 1e9
    traffic = None
    if os.path.exists(PMC_FILE):
        pmc = json.load(open(PMC_FILE))
        if pmc.get("kernel_sha") == kernel_sha() and pmc.get("storage") == args.storage:
            traffic = int(pmc["hbm_bytes_per_launch"])
    ws_bytes = int(dec.workspace.numel())
    pages_high = int(stats[:, 3].max()) if paged else None
    result = {
        "metric": "decoded frames/sec (B*T/s) offline + p50 streaming chunk latency; % HBM peak",
        "value": round(value, 1),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.B} T={wl.T} V={wl.V} beam={wl.beam} "
                               f"nbest={wl.nbest} threshold={wl.threshold} "
                               f"max_out_len={wl.max_out_len} storage={args.storage}",
                   "global_batch": wl.B, "seq_len": wl.T, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic,
                     "kernel": "decode_kernel (+ select_kernel, timed together per call)",
                     "algorithmic_bytes_per_launch": int(bytes_per_launch),
                     "launch_ms": round(launch_ms, 4)},
        "decode": {"selected_frames": selected, "fallback_steps": int(stats[:, 4].sum()),
                   "launches_per_decoded_frame": round(2 / max(selected, 1), 8),
                   "merge_verifications": int(stats[:, 5].sum()),
                   "workspace_bytes": ws_bytes, "paged_pages_high_per_row": pages_high,
                   "kernel_sha": kernel_sha()},
    }
    if paged:
        # token storage per row (f32-sized tokens): the two flat lists of every
        # slot at full capacity, the default page pool (the bound that cannot
        # run out), the pages this decode's busiest row held at most with the
        # default pool (in-place appends where only the source row also holds
        # the page), and the pool the page's allocator needs on the same decode
        # (a pool given explicitly, of the default's size, follows it exactly;
        # that mark is the smallest pool that decodes the row)
        ps = cfg.page_size or 16
        flat_b = 2 * wl.beam * wl.T * 4
        npool = wl.beam * (-(-wl.T // ps) + 1)
        pool_b = npool * ps * 4
        high_b = pages_high * ps * 4
        exact = cpb.OfflineDecoder(cpb.DecoderConfig(
            beam=wl.beam, nbest=wl.nbest, blank_threshold=wl.threshold,
            max_out_len=wl.max_out_len, paged=True, num_pages=npool))
        exact.decode(x, lens_d)
        rule_high = int(exact.row_stats().cpu().numpy()[:, 3].max())
        del exact
        rule_b = rule_high * ps * 4
        result["decode"]["token_store_bytes_per_row"] = {
            "flat_lists": flat_b, "paged_default_pool": pool_b, "paged_high_water": high_b,
            "flat_over_high_water": round(flat_b / max(high_b, 1), 2),
            "paged_high_water_page_allocator": rule_b,
            "flat_over_page_allocator": round(flat_b / max(rule_b, 1), 2)}
    if args.with_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        a.fill_(1.0)
        c = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(2):
            torch.add(a, 1.0, out=c)   # vectorised elementwise kernel: 16 B per lane
        torch.cuda.synchronize()
        result["copy_calibration"] = {"bytes_each_way": a.numel() * 4, "copies": 2}
        del a, c
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(x, lens, wl, args.cpu_seconds)
    del x
    torch.cuda.empty_cache()
    if not args.no_extras:
        log("[bench] other workloads (tiny, bpe256, bpe1024, vocab5000 flat)")
        result["workloads"] = other_workloads()
        log("[bench] streaming latency, 256 streams, capacity 1024")
        result["streaming"] = streaming_latency()
        log("[bench] streaming latency, capacity 4096")
        result["streaming"]["capacity_4096"] = streaming_latency(capacity=4096)
        log("[bench] streaming latency with a speech mask")
        result["streaming"]["speech_masked"] = streaming_latency(mask_theta=0.7)
        log("[bench] wide beams (64, 128)")
        result["wide_beams"] = wide_beams()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
