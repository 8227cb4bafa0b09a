"""Per-phase cycle counters of the decode kernel (a diagnostics build).

``build()`` compiles ``libctcpb_phase.so``: the same library with
``-DCTCPB_PHASE_PROF``, whose decode kernel reads the shader clock at phase
boundaries and leaves the sums in the workspace header of every row.  The
counters perturb the timing a little (each mark waits for the wave's
outstanding LDS operations); they show where a step's cycles go, not the
product's speed.

    python -m ctc_prefix_beam_amd.diagnostics vocab5000:paged bpe1024:flat

prints one JSON line per workload: the beam wave's cycles per step by phase,
the producers' ranking and waiting cycles per frame (and the ranking's own
phases), the store wave's work and waiting per step (paged: its sub-phases).
This module must run in a process of its own: it points the binding at the
diagnostics library before the library is first loaded.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libctcpb_phase.so")

# beam-wave phase slots of the counters (header words 32.. as 64-bit sums)
BEAM_PHASES = {0: "wait_ready", 1: "pre", 9: "lse_and_candidates", 3: "order_or_sort",
               4: "exact_or_gather", 5: "outside_bound", 6: "update", 7: "publish"}
STORE_PHASES = {2: "tail", 8: "fork", 10: "append", 11: "shared_pages"}
RANK_PHASES = ["clear", "group_maxima", "threshold", "groups", "gather", "rank", "restore"]


def build() -> str:
    from .build import FLAGS, SRC
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    proc = subprocess.run([hipcc, *FLAGS, "-DCTCPB_PHASE_PROF", SRC, "-o", tmp],
                          capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stdout + proc.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def profile(name: str, paged: bool, seed: int = 0) -> dict:
    import numpy as np
    import torch

    import ctc_prefix_beam_amd as cpb
    import synth
    wl = synth.WORKLOADS[name]
    x, lens = wl.make_device(seed, "cuda")
    B = x.shape[0]
    lens_d = torch.from_numpy(lens).cuda()
    dec = cpb.OfflineDecoder(cpb.DecoderConfig(beam=wl.beam, nbest=wl.nbest,
                                               blank_threshold=wl.threshold,
                                               max_out_len=wl.max_out_len, paged=paged))
    for _ in range(2):
        dec.decode(x, lens_d)
    dec.workspace.zero_()   # the producer and store counters are added to
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    dec.decode(x, lens_d)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    rb = dec.workspace.numel() // B
    lay = dec.workspace[: B * rb].view(B, rb)[:, 256:256 + 16].contiguous().cpu().numpy()
    ldr = lay.view(np.uint64).astype(np.float64)   # loader counters (beam arrays region)
    hdr = dec.workspace[: B * rb].view(B, rb)[:, :256].contiguous().cpu().numpy()
    h32 = hdr.view(np.int32)[:, :64]
    h64 = hdr.view(np.uint64)[:, :32].astype(np.float64)
    steps = float(h32[:, 0].sum())
    prof, rprof, extra = h64[:, 16:28], h64[:, 8:16], h64[:, 28:32]
    beam = {v: round(prof[:, i].sum() / steps) for i, v in BEAM_PHASES.items()}
    beam["total"] = sum(beam.values())
    out = {"workload": name, "storage": "paged" if paged else "flat",
           "ms_per_decode": round(ms, 4), "steps_per_row": int(h32[:, 0].max()),
           "us_per_step": round(ms * 1e3 / max(1, int(h32[:, 0].max())), 3),
           "beam_wave_cycles_per_step": beam,
           "producer_cycles_per_frame": {"rank": round(extra[:, 1].sum() / steps),
                                         "wait": round(extra[:, 0].sum() / steps)},
           "rank_phases_per_frame": {v: round(rprof[:, i].sum() / steps)
                                     for i, v in enumerate(RANK_PHASES)},
           "loader_cycles_per_frame": {"wait_for_slot": round(ldr[:, 0].sum() / steps),
                                       "load": round(ldr[:, 1].sum() / steps)},
           "store_wave_cycles_per_step": {"work": round(extra[:, 3].sum() / steps),
                                          "wait": round(extra[:, 2].sum() / steps)},
           "shader_clock_ghz_est": round(beam["total"] / (ms * 1e6 / max(1, h32[:, 0].max())), 3)}
    if paged:
        out["store_wave_cycles_per_step"]["paged_parts"] = {
            v: round(prof[:, i].sum() / steps) for i, v in STORE_PHASES.items()}
    del x
    torch.cuda.empty_cache()
    return out


def main(argv):
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run ctc_prefix_beam_amd.diagnostics.build()")
    sys.path.insert(0, ROOT)
    import ctc_prefix_beam_amd as cpb
    cpb.LIB_PATH = LIB_PATH   # before the library is first loaded
    for arg in argv or ["vocab5000:paged"]:
        name, storage = arg.split(":")
        print(json.dumps(profile(name, storage == "paged")), flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
