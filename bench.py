"""Benchmark of one CSA layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only prefill|decode|hca|compress|next|peaks]
                    [--no-cpu-baseline] [--calibrate-copy]

One step is one CSA prefill layer at n = 8192 (64 heads, c = 512, m = 4,
k = 512, window 128, indexer 64 x 128, bf16): the main-entry compressor, the
indexer-key compressor, indexer scoring + top-k, and the main attention, all
on device-resident synthetic inputs.  The JSON line reports prefill tokens/s
as `value`, the attention kernel's MFMA roofline fraction from HIP-event
timings, and the CPU oracle's rate on a bounded sample.  Secondary lines in
the same JSON object: 1M-context decode (8 sequences, microseconds per step),
the HCA prefill layer (n = 131072), the compressor sweep (n = 65536), and
what a plain library copy and bf16 GEMM reach on the same GPU, beside the
published peaks.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA prefill tokens/s @n=8192 (% MFMA roofline); 1M-ctx decode µs/step"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


class KernelTimer:
    """HIP-event timing of named launches on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []
        self.total = {}
        self.count = {}

    def run(self, name, fn):
        a, b = _events(self.torch)
        a.record()
        r = fn()
        b.record()
        self.pending.append((name, a, b))
        return r

    def collect(self):
        self.torch.cuda.synchronize()
        for name, a, b in self.pending:
            self.total[name] = self.total.get(name, 0.0) + a.elapsed_time(b)
            self.count[name] = self.count.get(name, 0) + 1
        self.pending = []

    def avg_us(self, name):
        return 1000.0 * self.total[name] / self.count[name]


def prewarm(torch, fn, seconds=0.3):
    """Run fn untimed for at least `seconds` of GPU time so that the clocks
    reach their steady state before the warm-up and timed steps."""
    t0 = time.perf_counter()
    while True:
        fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def timed_steps(torch, fn, steps):
    """Time `steps` calls of fn: a HIP event on the stream before the first
    and after each one, synchronised on both sides.  Returns (median of the
    per-step event intervals in ms, wall-clock mean in ms)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = 1000.0 * (time.perf_counter() - t0) / steps
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    mid = len(per) // 2
    med = per[mid] if len(per) % 2 else 0.5 * (per[mid - 1] + per[mid])
    return med, wall


# --------------------------------------------------------------- prefill ----

def prefill_pairs(n, m, k, n_win):
    """(selected, window) query-entry pairs of a causal CSA prefill."""
    sel = sum(min(k, (t + 1) // m) for t in range(n))
    win = sum(min(t + 1, n_win) for t in range(n))
    return sel, win


def run_prefill(args, torch, L, synth):
    p = dict(synth.PREFILL)
    d = synth.prefill_inputs(device="cuda")
    n, m, k, nw, nh, c, nI, cI = p["n"], p["m"], p["k"], p["n_win"], p["n_h"], p["c"], p["n_hI"], p["c_I"]
    ne = n // m
    lib = L.load_library()
    st = torch.cuda.current_stream().cuda_stream
    Cc = torch.empty((1, ne, c), dtype=torch.bfloat16, device="cuda")
    KI = torch.empty((1, ne, cI), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((1, n, k), dtype=torch.int32, device="cuda")
    out = torch.empty((1, n, nh, c), dtype=torch.bfloat16, device="cuda")
    ws_bytes = lib.csa_index_topk_workspace_size(1, n, ne, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    P = lambda t: t.data_ptr()

    def comp_main():
        return lib.csa_compress(P(d["Ca"]), P(d["Cb"]), P(d["Za"]), P(d["Zb"]), P(d["Ba"]), P(d["Bb"]),
                                None, None, 1, n, c, m, 1, 1, P(Cc), 0, st)

    def comp_index():
        return lib.csa_compress(P(d["ICa"]), P(d["ICb"]), P(d["IZa"]), P(d["IZb"]), P(d["IBa"]),
                                P(d["IBb"]), None, None, 1, n, cI, m, 1, 1, P(KI), 0, st)

    def index_topk():
        return lib.csa_index_topk(P(d["qI"]), P(d["w"]), P(KI), 0, 1, n, 0, ne, nI, cI, m, k, 1, P(idx),
                                  None, P(ws), ws_bytes, st)

    def attend():
        return lib.csa_attend(P(d["q"]), P(Cc), 0, P(idx), P(d["kv_raw"]), 0, 0, P(d["sink"]), 1, n, 0, ne,
                              n, nh, c, k, m, nw, d["scale"], 1, None, 0, P(out), st)

    stages = [("compress_main", comp_main), ("compress_index_keys", comp_index),
              ("index_topk", index_topk), ("attend", attend)]

    def step(timer=None):
        for name, fn in stages:
            rc = timer.run(name, fn) if timer else fn()
            if rc != 0:
                raise RuntimeError(f"{name} failed: {L.strerror(rc)}")

    prewarm(torch, step)
    for _ in range(args.warmup):
        step()
    # K steps: median of the per-step HIP-event intervals (and the wall mean)
    ms, ms_wall = timed_steps(torch, step, args.steps)
    # per-kernel HIP-event timings over a second pass of K steps
    timer = KernelTimer(torch)
    for _ in range(args.steps):
        step(timer)
    timer.collect()
    stage_us = {name: timer.avg_us(name) for name, _ in stages}

    if args.core:
        return {"ms_per_step": ms, "ms_per_step_wall": ms_wall, "stage_us": stage_us}

    # The FP4 indexer at this shape: the step's queries and keys quantised to
    # MXFP4 before timing, the index + top-k timed like the stages (the step
    # above keeps the bf16 indexer: the library has no quantising compressor).
    qc, qs = synth.to_mxfp4(d["qI"])
    kc, ks = synth.to_mxfp4(KI)

    def index_mx():
        return lib.csa_index_topk_mxfp4(P(qc), P(qs), P(d["w"]), P(kc), P(ks), 0, 1, n, 0, ne, nI, cI, m, k,
                                        P(idx), None, P(ws), ws_bytes, st)

    timer4 = KernelTimer(torch)
    for _ in range(2):
        index_mx()
    for _ in range(args.steps):
        if timer4.run("index_topk_mxfp4", index_mx) != 0:
            raise RuntimeError("mxfp4 index failed")
    timer4.collect()
    index_mx_us = timer4.avg_us("index_topk_mxfp4")

    # the E4M3 indexer at this shape (codes converted before timing)
    qI8 = d["qI"].to(torch.float8_e4m3fn)
    KI8 = KI.to(torch.float8_e4m3fn)

    def index_f8():
        return lib.csa_index_topk(P(qI8), P(d["w"]), P(KI8), 0, 1, n, 0, ne, nI, cI, m, k, 2, P(idx), None, P(ws),
                                  ws_bytes, st)

    for _ in range(2):
        index_f8()
    for _ in range(args.steps):
        if timer4.run("index_topk_fp8", index_f8) != 0:
            raise RuntimeError("fp8 index failed")
    timer4.collect()
    index_f8_us = timer4.avg_us("index_topk_fp8")
    del qI8, KI8

    # A whole step with the FP4 indexer: the library encodes the key
    # compressor's bf16 output and the step's bf16 indexer queries to MXFP4
    # inside the step, then indexes over the codes.
    def quant_keys():
        return lib.csa_quantize_mxfp4(P(KI), cI, ne, cI, 1, P(kc), cI // 2, P(ks), cI // 32, st)

    def quant_queries():
        return lib.csa_quantize_mxfp4(P(d["qI"]), cI, n * nI, cI, 1, P(qc), cI // 2, P(qs), cI // 32, st)

    stages4 = [("compress_main", comp_main), ("compress_index_keys", comp_index), ("quantize_keys", quant_keys),
               ("quantize_queries", quant_queries), ("index_topk_mxfp4", index_mx), ("attend", attend)]

    def step4():
        for name, fn in stages4:
            if fn() != 0:
                raise RuntimeError(f"{name} failed")

    for _ in range(args.warmup):
        step4()
    ms4, _ = timed_steps(torch, step4, args.steps)
    del qc, qs, kc, ks

    # A whole step with the normalisation and partial RoPE around the core
    # attention: compressed entries (at m * s), window rows and query heads are
    # RMS-normalised and rotated on their last 64 dims, and the output is
    # turned back by -t in place.  Gains are seeded synthetic values.
    _, gq = synth.norm_rope_inputs(1, 1, c, seed=46, device="cuda")
    _, gk = synth.norm_rope_inputs(1, 1, c, seed=47, device="cuda")
    qn = torch.empty_like(d["q"])
    Cn = torch.empty_like(Cc)
    Rn = torch.empty_like(d["kv_raw"])
    eps, rd, base = 1e-6, 64, 10000.0

    def norm_entries():
        return lib.csa_norm_rope(P(Cc), c, P(Cn), c, P(gk), eps, ne, 1, c, rd, base, 0, m, 1, st)

    def norm_window_rows():
        return lib.csa_norm_rope(P(d["kv_raw"]), c, P(Rn), c, P(gk), eps, n, 1, c, rd, base, 0, 1, 1, st)

    def norm_queries():
        return lib.csa_norm_rope(P(d["q"]), nh * c, P(qn), nh * c, P(gq), eps, n, nh, c, rd, base, 0, 1, 1, st)

    def attend_normed():
        return lib.csa_attend(P(qn), P(Cn), 0, P(idx), P(Rn), 0, 0, P(d["sink"]), 1, n, 0, ne, n, nh, c, k, m, nw,
                              d["scale"], 1, None, 0, P(out), st)

    def rotate_output():
        return lib.csa_norm_rope(P(out), nh * c, P(out), nh * c, None, 0.0, n, nh, c, rd, base, 0, -1, 1, st)

    stagesR = [("compress_main", comp_main), ("compress_index_keys", comp_index),
               ("norm_rope_entries", norm_entries), ("norm_rope_window_rows", norm_window_rows),
               ("norm_rope_queries", norm_queries), ("index_topk", index_topk), ("attend", attend_normed),
               ("rotate_output", rotate_output)]

    def stepR(timer=None):
        for name, fn in stagesR:
            rc = timer.run(name, fn) if timer else fn()
            if rc != 0:
                raise RuntimeError(f"{name} failed: {L.strerror(rc)}")

    for _ in range(args.warmup):
        stepR()
    msR, _ = timed_steps(torch, stepR, args.steps)
    timerR = KernelTimer(torch)
    for _ in range(args.steps):
        stepR(timerR)
    timerR.collect()

    # The same step with the query norm and rotation done in the attention's
    # Q load and the output's -t rotation in its epilogue (csa_attend_norm_rope):
    # the separate query and output passes are gone.
    def attend_fused():
        return lib.csa_attend_norm_rope(P(d["q"]), P(gq), eps, rd, base, P(Cn), 0, P(idx), P(Rn), 0, 0,
                                        P(d["sink"]), 1, n, 0, ne, n, nh, c, k, m, nw, d["scale"], 1, None, 0,
                                        P(out), st)

    stagesF = [("compress_main", comp_main), ("compress_index_keys", comp_index),
               ("norm_rope_entries", norm_entries), ("norm_rope_window_rows", norm_window_rows),
               ("index_topk", index_topk), ("attend_norm_rope", attend_fused)]

    def stepF(timer=None):
        for name, fn in stagesF:
            rc = timer.run(name, fn) if timer else fn()
            if rc != 0:
                raise RuntimeError(f"{name} failed: {L.strerror(rc)}")

    for _ in range(args.warmup):
        stepF()
    msF, _ = timed_steps(torch, stepF, args.steps)
    timerF = KernelTimer(torch)
    for _ in range(args.steps):
        stepF(timerF)
    timerF.collect()
    fused_step = {"ms_per_step": msF, "tokens_per_s": n / (msF / 1000.0),
                  "stages": [name for name, _ in stagesF],
                  "stage_us": {name: timerF.avg_us(name) for name, _ in stagesF}}
    nq_bytes = 2 * n * nh * c * 2            # query heads read and written once
    rot_bytes = 2 * n * nh * rd * 2          # rotated output dims read and written
    nr_us = {name: timerR.avg_us(name) for name, _ in stagesR if name.startswith(("norm", "rotate"))}
    norm_rope_step = {
        "ms_per_step": msR, "tokens_per_s": n / (msR / 1000.0), "stages": [name for name, _ in stagesR],
        "stage_us": nr_us,
        "queries_gbs": nq_bytes / (nr_us["norm_rope_queries"] * 1e-6) / 1e9,
        "queries_hbm_frac": nq_bytes / (nr_us["norm_rope_queries"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "rotate_output_gbs": rot_bytes / (nr_us["rotate_output"] * 1e-6) / 1e9,
        "gains": "seeded synthetic (1 + N(0, 0.1^2) per dim); eps 1e-6, RoPE base 10000 on the last 64 dims",
        "fused_queries": fused_step,
    }
    del qn, Cn, Rn

    # The grouped output projection of the step's attention output at the
    # Flash shape (g = 8 groups of 8 heads, d_g = 1024, d = 4096), seeded
    # synthetic weights: two bf16 MFMA products, timed together.
    g_, dg_, dm_ = 8, 1024, 4096
    _, WG, WO = synth.out_proj_inputs(1, nh, c, g_, dg_, dm_, seed=48, device="cuda")
    mid = torch.empty((n, g_ * dg_), dtype=torch.bfloat16, device="cuda")
    proj = torch.empty((n, dm_), dtype=torch.bfloat16, device="cuda")

    def out_proj():
        return lib.csa_grouped_out_proj(P(out), P(WG), P(WO), n, nh, c, g_, dg_, dm_, 1, P(mid), P(proj), st)

    timerP = KernelTimer(torch)
    for _ in range(5):
        out_proj()
    for _ in range(args.steps):
        if timerP.run("grouped_out_proj", out_proj) != 0:
            raise RuntimeError("grouped output projection failed")
    timerP.collect()
    proj_us = timerP.avg_us("grouped_out_proj")
    proj_flop = 2 * n * (nh * c) * dg_ + 2 * n * (g_ * dg_) * dm_
    out_proj_rec = {"us": proj_us, "flop": proj_flop, "tflops": proj_flop / (proj_us * 1e-6) / 1e12,
                    "mfma_frac": proj_flop / (proj_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                    "shape": "n=8192, 64 heads x 512 -> 8 groups x 1024 -> 4096, bf16",
                    "weights": "seeded synthetic, N(0,1)/sqrt(fan-in)"}
    del WG, WO, mid, proj

    sel, win = prefill_pairs(n, m, k, nw)
    flop_attend = (sel + win) * 4 * nh * c
    vis_pairs = sum(min((t + 1) // m, ne) for t in range(n))
    flop_index = vis_pairs * 2 * nI * cI
    att_tflops = flop_attend / (stage_us["attend"] * 1e-6) / 1e12
    return {
        "ms_per_step": ms,
        "ms_per_step_wall": ms_wall,
        "tokens_per_s": n / (ms / 1000.0),
        "stage_us": stage_us,
        "flop_attend": flop_attend,
        "flop_index": flop_index,
        "attend_tflops": att_tflops,
        "index_tflops": flop_index / (stage_us["index_topk"] * 1e-6) / 1e12,
        "index_topk_mxfp4_us": index_mx_us,
        "index_topk_fp8_us": index_f8_us,
        "norm_rope_step": norm_rope_step,
        "out_proj": out_proj_rec,
        "mxfp4_step": {"ms_per_step": ms4, "tokens_per_s": n / (ms4 / 1000.0),
                       "stages": [name for name, _ in stages4],
                       "queries": "bf16 indexer queries and keys encoded to MXFP4 inside the step"},
        "step_tflops": (flop_attend + flop_index) / (ms * 1e-3) / 1e12,
        "inputs": d,
    }


# ---------------------------------------------------------------- decode ----

def run_decode(args, torch, L, synth):
    d = synth.decode_inputs(device="cuda")
    p = d["params"]
    b, hist, m, nh, c, nw, nI, cI, k, steps = (p["b"], p["history"], p["m"], p["n_h"], p["c"], p["n_win"],
                                               p["n_hI"], p["c_I"], p["k"], p["steps"])
    lib = L.load_library()
    st = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    ne0 = d["n_comp0"]
    cap = d["Ccomp"].shape[1]
    # The new token's rows are placed where the producing projection writes
    # them: stream rows in the block tails [b, m, width] at slot t % m, the
    # raw row in the window buffer.  The timed steps cover one block
    # (t = history .. history + m - 1), so every slot is written once, before
    # the timed region, and each step reads its inputs in place.
    assert steps == m, "the timed decode steps cover exactly one block"
    tails = {key: torch.empty((b, m, c if key[0] != "I" else cI), dtype=torch.bfloat16, device="cuda")
             for key in ("Ca", "Cb", "Za", "Zb", "ICa", "ICb", "IZa", "IZb")}
    for i in range(steps):
        j = (hist + i) % m
        for key in tails:
            tails[key][:, j].copy_(d["tok"][key][i])
        d["window"][:, nw + i].copy_(d["tok"]["Ca"][i])
    idx = torch.empty((b, 1, k), dtype=torch.int32, device="cuda")
    out = torch.empty((b, 1, nh, c), dtype=torch.bfloat16, device="cuda")
    wsI_bytes = lib.csa_index_topk_workspace_size(b, 1, ne0 + steps, k)
    wsI = torch.empty(wsI_bytes, dtype=torch.uint8, device="cuda")
    wsA_bytes = max(lib.csa_attend_workspace_size(b, 1, hist + s, ne0 + 1, nh, c, k, m, nw, 1)
                    for s in range(steps))
    wsA = torch.empty(max(wsA_bytes, 256), dtype=torch.uint8, device="cuda")
    win = d["window"]
    raw_pos0 = d["window_pos0"]

    def one_step(i):
        t = hist + i
        if (t + 1) % m == 0:
            # the block is complete: emit one entry of each compressed cache
            # from the block and the previous block's stream-b state
            e = (t + 1) // m - 1
            rc = lib.csa_compress(P(tails["Ca"]), P(tails["Cb"]), P(tails["Za"]), P(tails["Zb"]), P(d["Ba"]),
                                  P(d["Bb"]), P(d["prev_Cb"]), P(d["prev_Zb"]), b, m, c, m, 1, 1,
                                  d["Ccomp"][:, e].data_ptr(), cap * c, st)
            rc |= lib.csa_compress(P(tails["ICa"]), P(tails["ICb"]), P(tails["IZa"]), P(tails["IZb"]),
                                   P(d["IBa"]), P(d["IBb"]), P(d["prev_ICb"]), P(d["prev_IZb"]), b, m, cI, m,
                                   1, 1, d["KIcomp"][:, e].data_ptr(), cap * cI, st)
            if rc != 0:
                raise RuntimeError("decode compress failed")
        n_comp = (t + 1) // m
        rc = lib.csa_index_topk(P(d["qI"][i]), P(d["w"][i]), P(d["KIcomp"]), cap * cI, b, 1, t, n_comp, nI,
                                cI, m, k, 1, P(idx), None, P(wsI), wsI_bytes, st)
        if rc != 0:
            raise RuntimeError(f"decode index failed: {L.strerror(rc)}")
        rc = lib.csa_attend(P(d["q"][i]), P(d["Ccomp"]), cap * c, P(idx), P(win), (nw + steps) * c, raw_pos0,
                            P(d["sink"]), b, 1, t, n_comp, nw + steps, nh, c, k, m, nw, d["scale"], 1,
                            P(wsA), wsA.numel(), P(out), st)
        if rc != 0:
            raise RuntimeError(f"decode attend failed: {L.strerror(rc)}")

    reps = max(1, args.decode_reps)
    for _ in range(20):   # untimed, also brings the clocks to their steady state
        for i in range(steps):
            one_step(i)
    torch.cuda.synchronize()
    a, bb = _events(torch)
    a.record()
    for _ in range(reps):
        for i in range(steps):
            one_step(i)
    bb.record()
    torch.cuda.synchronize()
    us = 1000.0 * a.elapsed_time(bb) / (reps * steps)
    key_bytes = b * ne0 * cI * 2
    gathered = b * (k + nw) * c * 2
    small = b * (nh * c * 2 * 2 + nI * cI * 2 + nI * 4 + k * 4)
    step_bytes = key_bytes + gathered + small
    res = {"us_per_step": us, "bytes_per_step": step_bytes,
           "hbm_gbs": step_bytes / (us * 1e-6) / 1e9, "b": b, "history": hist, "k": k}
    if args.core:
        return res

    # The low-precision indexer: the same state with the indexer keys and
    # queries as E4M3 codes (converted before timing), over the first
    # steps - 1 steps of the block, which complete no entry, so that every
    # timed kernel is the library's (index + top-k, attention).
    KI8 = d["KIcomp"].to(torch.float8_e4m3fn)
    qI8 = d["qI"].to(torch.float8_e4m3fn)

    def step8(i):
        t = hist + i
        n_comp = (t + 1) // m
        rc = lib.csa_index_topk(P(qI8[i]), P(d["w"][i]), P(KI8), cap * cI, b, 1, t, n_comp, nI, cI, m, k, 2,
                                P(idx), None, P(wsI), wsI_bytes, st)
        rc |= lib.csa_attend(P(d["q"][i]), P(d["Ccomp"]), cap * c, P(idx), P(win), (nw + steps) * c, raw_pos0,
                             P(d["sink"]), b, 1, t, n_comp, nw + steps, nh, c, k, m, nw, d["scale"], 1,
                             P(wsA), wsA.numel(), P(out), st)
        if rc != 0:
            raise RuntimeError("fp8 decode step failed")

    n8 = steps - 1
    for i in range(n8):
        step8(i)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        for i in range(n8):
            step8(i)
    bb.record()
    torch.cuda.synchronize()
    us8 = 1000.0 * a.elapsed_time(bb) / (reps * n8)
    bytes8 = b * ne0 * cI + gathered + b * (nh * c * 2 * 2 + nI * cI + nI * 4 + k * 4)
    res["fp8_indexer"] = {"us_per_step": us8, "bytes_per_step": bytes8,
                          "hbm_gbs": bytes8 / (us8 * 1e-6) / 1e9,
                          "steps": f"the {n8} steps of a block that complete no entry"}
    del KI8

    # The FP4 indexer (OCP MXFP4 codes and block scales): the key cache is
    # encoded once before timing (the history), the step's indexer query is
    # given as MXFP4 codes, and the block-completing step encodes its new key
    # entry into the FP4 cache in place with the library's encoder.  All
    # steps of the block are timed.
    KIc, KIs = synth.to_mxfp4(d["KIcomp"])
    qIq = [synth.to_mxfp4(d["qI"][i]) for i in range(steps)]
    knew = torch.empty((b, 1, cI), dtype=torch.bfloat16, device="cuda")

    def step4(i):
        t = hist + i
        rc = 0
        if (t + 1) % m == 0:
            e = (t + 1) // m - 1
            rc |= lib.csa_compress(P(tails["Ca"]), P(tails["Cb"]), P(tails["Za"]), P(tails["Zb"]), P(d["Ba"]),
                                   P(d["Bb"]), P(d["prev_Cb"]), P(d["prev_Zb"]), b, m, c, m, 1, 1,
                                   d["Ccomp"][:, e].data_ptr(), cap * c, st)
            rc |= lib.csa_compress(P(tails["ICa"]), P(tails["ICb"]), P(tails["IZa"]), P(tails["IZb"]),
                                   P(d["IBa"]), P(d["IBb"]), P(d["prev_ICb"]), P(d["prev_IZb"]), b, m, cI, m,
                                   1, 1, P(knew), cI, st)
            rc |= lib.csa_quantize_mxfp4(P(knew), cI, b, cI, 1, KIc[:, e].data_ptr(), cap * (cI // 2),
                                         KIs[:, e].data_ptr(), cap * (cI // 32), st)
        n_comp = (t + 1) // m
        rc |= lib.csa_index_topk_mxfp4(P(qIq[i][0]), P(qIq[i][1]), P(d["w"][i]), P(KIc), P(KIs), cap, b, 1, t,
                                       n_comp, nI, cI, m, k, P(idx), None, P(wsI), wsI_bytes, st)
        rc |= lib.csa_attend(P(d["q"][i]), P(d["Ccomp"]), cap * c, P(idx), P(win), (nw + steps) * c, raw_pos0,
                             P(d["sink"]), b, 1, t, n_comp, nw + steps, nh, c, k, m, nw, d["scale"], 1,
                             P(wsA), wsA.numel(), P(out), st)
        if rc != 0:
            raise RuntimeError("mxfp4 decode step failed")

    for i in range(steps):
        step4(i)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        for i in range(steps):
            step4(i)
    bb.record()
    torch.cuda.synchronize()
    us4 = 1000.0 * a.elapsed_time(bb) / (reps * steps)
    bytes4 = b * ne0 * (cI // 2 + cI // 32) + gathered + b * (nh * c * 2 * 2 + nI * (cI // 2 + cI // 32) + nI * 4
                                                             + k * 4)
    res["mxfp4_indexer"] = {"us_per_step": us4, "bytes_per_step": bytes4,
                            "hbm_gbs": bytes4 / (us4 * 1e-6) / 1e9,
                            "steps": f"all {steps} steps of a block; the last appends one entry to each cache, "
                                     "the key entry encoded to MXFP4 in place"}
    return res


# ------------------------------------------------------------------- HCA ----

def run_hca(args, torch, L, synth):
    d = synth.hca_inputs(device="cuda")
    p = d["params"]
    n, mp, nh, c, nw = p["n"], p["m_prime"], p["n_h"], p["c"], p["n_win"]
    lib = L.load_library()
    st = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    Cc = torch.empty((1, n // mp, c), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(d["q"])
    need = lib.hca_layer_workspace_size(1, n, nh, c, mp, nw, 1)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")

    def step():
        rc = lib.hca_layer(P(d["C"]), P(d["Z"]), P(d["B"]), P(d["q"]), P(d["kv_raw"]), P(d["sink"]), 1, n, c,
                           mp, nh, nw, d["scale"], 1, P(Cc), P(ws), ws.numel(), P(out), st)
        if rc != 0:
            raise RuntimeError(f"hca_layer failed: {L.strerror(rc)}")

    for _ in range(2):   # untimed
        step()
    torch.cuda.synchronize()
    a, b = _events(torch)
    iters = max(1, args.hca_iters)
    a.record()
    for _ in range(iters):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    ne = n // mp
    pairs = sum(min((t + 1) // mp, ne) + min(t + 1, nw) for t in range(n))
    flop = pairs * 4 * nh * c

    # The attention alone, plain and with the query norm and rotation fused
    # in (hca_attend_norm_rope; seeded synthetic gain, eps 1e-6, RoPE base
    # 10000 on the last 64 dims), on the layer's compressed entries.
    _, gq = synth.norm_rope_inputs(1, 1, c, seed=49, device="cuda")
    wsA = lib.hca_attend_workspace_size(1, n, 0, ne, nh, c, mp, nw, 1)
    wsAt = torch.empty(max(wsA, 256), dtype=torch.uint8, device="cuda")

    def attend_plain():
        return lib.hca_attend(P(d["q"]), P(Cc), 0, P(d["kv_raw"]), 0, 0, P(d["sink"]), 1, n, 0, ne, n, nh, c, mp,
                              nw, d["scale"], 1, P(wsAt), wsAt.numel(), P(out), st)

    def attend_fused():
        return lib.hca_attend_norm_rope(P(d["q"]), P(gq), 1e-6, 64, 10000.0, P(Cc), 0, P(d["kv_raw"]), 0, 0,
                                        P(d["sink"]), 1, n, 0, ne, n, nh, c, mp, nw, d["scale"], 1, P(wsAt),
                                        wsAt.numel(), P(out), st)

    att_ms = {}
    for name, fn in (("attend", attend_plain), ("attend_norm_rope", attend_fused)):
        if fn() != 0:
            raise RuntimeError(f"hca {name} failed")
        torch.cuda.synchronize()
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        att_ms[name] = a.elapsed_time(b) / iters
    del d, out
    torch.cuda.empty_cache()
    return {"ms_per_layer": ms, "tokens_per_s": n / (ms * 1e-3), "tflops": flop / (ms * 1e-3) / 1e12,
            "mfma_frac": flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "flop": flop,
            "attend_ms": att_ms["attend"], "attend_norm_rope_ms": att_ms["attend_norm_rope"]}


def run_hca_decode(args, torch, L, synth):
    """HCA attention at the 1M-context decode shape: 8 sequences, each with
    8192 completed HCA entries (m' = 128) and a 128-row window, one query."""
    d = synth.hca_decode_inputs(device="cuda")
    p = d["params"]
    b, ne, c, nh, mp, nw, t = p["b"], p["n_comp"], p["c"], p["n_h"], p["m_prime"], p["n_win"], p["t"]
    Cc, win, q, sink = d["Ccomp"], d["window"], d["q"], d["sink"]
    lib = L.load_library()
    st = torch.cuda.current_stream().cuda_stream
    P = lambda t_: t_.data_ptr()
    out = torch.empty_like(q)
    wsb = max(lib.hca_attend_workspace_size(b, 1, t, ne, nh, c, mp, nw, 1), 256)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def call():
        rc = lib.hca_attend(P(q), P(Cc), ne * c, P(win), nw * c, t - nw + 1, P(sink), b, 1, t, ne, nw, nh, c, mp,
                            nw, 1.0 / math.sqrt(c), 1, P(ws), wsb, P(out), st)
        if rc != 0:
            raise RuntimeError(f"hca_attend failed: {L.strerror(rc)}")

    for _ in range(50):   # untimed
        call()
    torch.cuda.synchronize()
    a, bb = _events(torch)
    iters = 100
    a.record()
    for _ in range(iters):
        call()
    bb.record()
    torch.cuda.synchronize()
    us = 1000.0 * a.elapsed_time(bb) / iters
    nbytes = b * (ne + nw) * c * 2 + b * nh * c * 2 * 2
    return {"us_per_call": us, "bytes": nbytes, "hbm_gbs": nbytes / (us * 1e-6) / 1e9, "b": b, "entries": ne,
            "n_win": nw}


# ----------------------------------- paged decode, backward, FP8 KV, BF16 ----

def _event_us(torch, fn, iters, warm=3):
    # clocks to their steady state first (see prewarm), then a few more calls
    prewarm(torch, fn, 0.2)
    for _ in range(warm):
        fn()
    a, b = _events(torch)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    return 1000.0 * a.elapsed_time(b) / iters


def _recall(torch, ref, got, n_comp):
    """Mean over rows of the share of ref's selected entries that got also
    selected (rows with no selection are left out)."""
    rows = ref.shape[0]
    mask = torch.zeros((rows, n_comp + 1), dtype=torch.bool, device=ref.device)
    mask.scatter_(1, torch.where(ref >= 0, ref, n_comp).long(), True)
    mask[:, n_comp] = False
    hit = torch.gather(mask, 1, torch.where(got >= 0, got, n_comp).long()) & (got >= 0)
    n_ref = (ref >= 0).sum(1)
    ok = n_ref > 0
    return float((hit.sum(1)[ok].double() / n_ref[ok].double()).mean())


def run_paged_decode(args, torch, L, synth):
    """1M-context decode of 8 requests through the paged heterogeneous
    cache: per step, each request's token is appended (state update; CSA
    entry and key on block completion), then indexer + top-k, CSA attention
    and HCA attention; blocks are scattered over the pool."""
    b, hist, c, cI, m, mp, nw, nh, nI, k = 8, 1 << 20, 512, 128, 4, 128, 128, 64, 64, 512
    blocks_per_req = hist // 128 + 1
    n_blocks = b * blocks_per_req
    cache = L.PagedCache(n_blocks, b, blocks_per_req, c, cI, m, mp, nw, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    pv = cache.blocks.view(n_blocks, cache.block_bytes // 2)
    pv[:, : 32 * c].normal_(0.0, 1.0 / math.sqrt(c), generator=g)
    pv[:, 32 * c: 32 * (c + cI)].normal_(0.0, 1.0 / math.sqrt(cI), generator=g)
    pv[:, 32 * (c + cI):].normal_(0.0, 1.0 / math.sqrt(c), generator=g)
    cache.state.normal_(0.0, 1.0 / math.sqrt(c), generator=g)
    perm = torch.randperm(n_blocks, device="cuda", generator=g).to(torch.int32)
    cache.table.copy_(perm.view(b, blocks_per_req))
    sc = lambda *s_, d=c: (torch.randn(s_, device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
    biases = {"Ba": sc(m, c), "Bb": sc(m, c), "IBa": sc(m, cI, d=cI), "IBb": sc(m, cI, d=cI), "B_h": sc(mp, c)}
    steps = 4
    toks = [{x: sc(b, c) for x in ("Ca", "Cb", "Za", "Zb", "C_h", "Z_h")} for _ in range(steps)]
    for tk in toks:
        tk.update({x: sc(b, cI, d=cI) for x in ("ICa", "ICb", "IZa", "IZb")})
    q = [sc(b, nh, c) for _ in range(steps)]
    qI = [sc(b, nI, cI, d=cI) for _ in range(steps)]
    w = [torch.nn.functional.softplus(torch.randn((b, nI), device="cuda", generator=g)) for _ in range(steps)]
    sink = torch.randn(nh, device="cuda", generator=g)
    pos = [torch.full((b,), hist + i, dtype=torch.int64, device="cuda") for i in range(steps)]
    lib = L.load_library()
    n_comp_max = (hist + steps) // m
    n_hca_max = (hist + steps) // mp
    wsI = torch.empty(lib.csa_index_topk_workspace_size(b, 1, n_comp_max, k), dtype=torch.uint8, device="cuda")
    wsA = torch.empty(max(lib.csa_paged_attend_workspace_size(b, nh, k, nw), 256), dtype=torch.uint8, device="cuda")
    wsH = torch.empty(max(lib.hca_paged_attend_workspace_size(b, nh, n_hca_max, nw), 256), dtype=torch.uint8,
                      device="cuda")
    idx = torch.empty((b, k), dtype=torch.int32, device="cuda")
    out = torch.empty((b, nh, c), dtype=torch.bfloat16, device="cuda")
    hout = torch.empty_like(out)

    def step(i):
        L.csa_paged_append(cache, pos[i], toks[i], biases)
        L.csa_paged_index_topk(cache, qI[i], w[i], pos[i], n_comp_max, k, idx=idx, workspace=wsI)
        L.csa_paged_attend(cache, q[i], idx, sink, pos[i], n_comp_max, out=out, workspace=wsA)
        L.hca_paged_attend(cache, q[i], sink, pos[i], n_hca_max, out=hout, workspace=wsH)

    for _ in range(10):
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    us = _event_us(torch, lambda: [step(i) for i in range(steps)], 5, warm=0) / steps
    key_bytes = b * (hist // m) * cI * 2
    hca_bytes = b * (hist // mp) * c * 2
    return {"us_per_step": us, "b": b, "history": hist, "k": k, "blocks": n_blocks,
            "block_bytes": cache.block_bytes, "state_bytes_per_request": cache.state_bytes,
            "stages": "append (state + compression on block completion), CSA index + top-k, CSA attention, "
                      "HCA attention, all through the block table",
            "hbm_bytes_per_step": key_bytes + hca_bytes + b * (k + 2 * nw) * c * 2,
            "hbm_gbs": (key_bytes + hca_bytes + b * (k + 2 * nw) * c * 2) / (us * 1e-6) / 1e9}


def run_backward(args, torch, L, synth):
    """CSA attention backward at the prefill head shape (n = 4096, k = 512,
    window 128, 64 heads, c = 512) and the overlapped compressor backward at
    n = 65536, c = 512."""
    n, m, k, nw = 4096, 4, 512, 128
    d = synth.prefill_inputs(n=n, device="cuda", k=k)
    nh, c = d["params"]["n_h"], d["params"]["c"]
    Cc = L.csa_compress(*(d[x] for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    KI = L.csa_compress(*(d[x] for x in ("ICa", "ICb", "IZa", "IZb", "IBa", "IBb")), m)
    idx = L.csa_index_topk(d["qI"], d["w"], KI, 0, m, k)
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    dout = (torch.randn(d["q"].shape, device="cuda", generator=g) / math.sqrt(c)).to(torch.bfloat16)
    lib = L.load_library()
    ws = torch.empty(lib.csa_attend_backward_workspace_size(1, n, nh, c, k, nw), dtype=torch.uint8, device="cuda")
    f = dict(dtype=torch.float32, device="cuda")
    grads = (torch.empty((1, n, nh, c), **f), torch.empty((1, n // m, c), **f), torch.empty((1, n, c), **f),
             torch.empty(nh, **f))
    call = lambda: L.csa_attend_backward(d["q"], Cc, idx, d["kv_raw"], d["sink"], dout, 0, m, nw, d["scale"],
                                         grads=grads, workspace=ws)
    us = _event_us(torch, call, 3, warm=1)
    sel, win = prefill_pairs(n, m, k, nw)
    flop = (sel + win) * nh * 10 * c      # q.e, g.e, dq, and both roles of de: 10 c flops per (pair, head)
    # every slot's entry contribution is written and read back once (float32)
    contrib_bytes = n * (k + nw) * c * 4 * 2
    tf = flop / (us * 1e-6) / 1e12
    res = {"csa_attend_backward": {"us": us, "n": n, "k": k, "flop": flop, "tflops": tf,
                                   "mfma_bf16_frac": tf / PEAK_BF16_TFLOPS,
                                   "contrib_bytes": contrib_bytes,
                                   "bound": "mfma (bf16 products of exact bf16 inputs, float32 accumulation; "
                                            "p and dl as bf16 high part + remainder) and the float32 contribution "
                                            "traffic"}}
    del d, dout, ws, grads
    cd = synth.compress_inputs(True, device="cuda")
    nc, cc, mc = synth.COMPRESS["n"], synth.COMPRESS["c"], cd["m"]
    dCc = torch.randn((1, nc // mc, cc), device="cuda", generator=g)
    callc = lambda: L.csa_compress_backward(cd["Ca"], cd["Cb"], cd["Za"], cd["Zb"], cd["Ba"], cd["Bb"], mc, dCc)
    usc = _event_us(torch, callc, 5, warm=2)
    nbytes = 4 * nc * cc * 2 + (nc // mc) * cc * 4 + 4 * nc * cc * 4
    res["compress_backward"] = {"us": usc, "n": nc, "bytes": nbytes, "gbs": nbytes / (usc * 1e-6) / 1e9,
                                "hbm_frac": nbytes / (usc * 1e-6) / 1e9 / PEAK_HBM_GBS}
    return res


def run_fp8kv_and_bf16_scores(args, torch, L, synth):
    """Attention over FP8-stored entries (prefill n = 8192; decode 8 x 2^18
    entries) and the selection on BF16 index scores: time and recall against
    the float32-score selection."""
    res = {}
    n, m, k, nw = 8192, 4, 512, 128
    d = synth.prefill_inputs(device="cuda")
    Cc = L.csa_compress(*(d[x] for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m)
    KI = L.csa_compress(*(d[x] for x in ("ICa", "ICb", "IZa", "IZb", "IBa", "IBb")), m)
    idx = L.csa_index_topk(d["qI"], d["w"], KI, 0, m, k)
    idx16 = L.csa_index_topk(d["qI"], d["w"], KI, 0, m, k, bf16_scores=True)
    lib = L.load_library()
    wsI = torch.empty(lib.csa_index_topk_workspace_size(1, n, n // m, k), dtype=torch.uint8, device="cuda")
    us32 = _event_us(torch, lambda: L.csa_index_topk(d["qI"], d["w"], KI, 0, m, k, idx=idx, workspace=wsI), 10)
    us16 = _event_us(torch, lambda: L.csa_index_topk(d["qI"], d["w"], KI, 0, m, k, idx=idx16, workspace=wsI,
                                                     bf16_scores=True), 10)
    res["bf16_scores_prefill"] = {"recall": _recall(torch, idx[0], idx16[0], n // m), "index_topk_us": us16,
                                  "index_topk_fp32_scores_us": us32}
    codes, rope, scale = L.csa_quantize_kv_fp8(Cc)
    out = torch.empty_like(d["q"])
    wsF = torch.empty(lib.csa_attend_fp8kv_workspace_size(1, n, 0, n // m, 64, 512, k, m, nw), dtype=torch.uint8,
                      device="cuda")
    usq = _event_us(torch, lambda: L.csa_quantize_kv_fp8(Cc), 10)
    usa = _event_us(torch, lambda: L.csa_attend_fp8kv(d["q"], codes, rope, scale, idx, d["kv_raw"], d["sink"], 0, m,
                                                       nw, out=out, workspace=wsF), 5)
    res["fp8_kv_prefill"] = {"attend_us": usa, "quantize_entries_us": usq, "entries": n // m,
                             "entry_bytes": 448 + 128 + 4,
                             "note": "every entry decoded to bf16 in the workspace, then the bf16 MFMA attention"}
    del d, out, wsF, wsI
    dd = synth.decode_inputs(device="cuda")
    p = dd["params"]
    b, hist, nh, c, cI, nI = p["b"], p["history"], p["n_h"], p["c"], p["c_I"], p["n_hI"]
    ne = dd["n_comp0"]
    t = hist
    cap = dd["Ccomp"].shape[1]
    i32 = L.csa_index_topk(dd["qI"][0], dd["w"][0], dd["KIcomp"], t, m, k, n_comp=ne)
    i16 = L.csa_index_topk(dd["qI"][0], dd["w"][0], dd["KIcomp"], t, m, k, n_comp=ne, bf16_scores=True)
    res["bf16_scores_decode"] = {"recall": _recall(torch, i32[:, 0], i16[:, 0], ne), "b": b, "candidates": ne}
    codes, rope, scale = L.csa_quantize_kv_fp8(dd["Ccomp"])
    dout = torch.empty_like(dd["q"][0])
    need = lib.csa_attend_fp8kv_workspace_size(b, 1, t, ne, nh, c, k, m, nw)
    wsD = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    win = dd["window"]
    usd = _event_us(torch, lambda: L.csa_attend_fp8kv(dd["q"][0], codes, rope, scale, i32, win, dd["sink"], t, m, nw,
                                                       raw_pos0=dd["window_pos0"], n_comp=ne, out=dout, workspace=wsD),
                    20, warm=5)
    wsB = torch.empty(max(lib.csa_attend_workspace_size(b, 1, t, ne, nh, c, k, m, nw, 1), 256), dtype=torch.uint8,
                      device="cuda")
    usb = _event_us(torch, lambda: L.csa_attend(dd["q"][0], dd["Ccomp"], i32, win, dd["sink"], t, m, nw,
                                                 raw_pos0=dd["window_pos0"], n_comp=ne, out=dout, workspace=wsB),
                    20, warm=5)
    res["fp8_kv_decode"] = {"attend_us": usd, "bf16_attend_us": usb, "b": b, "entries": ne,
                            "cache_bytes": b * ne * (448 + 128 + 4), "bf16_cache_bytes": b * ne * c * 2,
                            "note": "the selected entries decoded to bf16, then the bf16 decode attention"}
    return res


# ------------------------------------------------------------ compressor ----

def run_compress(args, torch, L, synth):
    lib = L.load_library()
    st = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    res = {}
    for overlap in (True, False):
        d = synth.compress_inputs(overlap, device="cuda")
        m = d["m"]
        n, c = synth.COMPRESS["n"], synth.COMPRESS["c"]
        out = torch.empty((1, n // m, c), dtype=torch.bfloat16, device="cuda")
        if overlap:
            call = lambda: lib.csa_compress(P(d["Ca"]), P(d["Cb"]), P(d["Za"]), P(d["Zb"]), P(d["Ba"]), P(d["Bb"]),
                                            None, None, 1, n, c, m, 1, 1, P(out), 0, st)
            nbytes = 4 * n * c * 2 + 2 * m * c * 2 + (n // m) * c * 2
        else:
            call = lambda: lib.csa_compress(P(d["C"]), None, P(d["Z"]), None, P(d["B"]), None, None, None, 1, n,
                                            c, m, 0, 1, P(out), 0, st)
            nbytes = 2 * n * c * 2 + m * c * 2 + (n // m) * c * 2
        for _ in range(200):   # untimed, also brings the clocks to their steady state
            call()
        torch.cuda.synchronize()
        a, b = _events(torch)
        iters = 200
        a.record()
        for _ in range(iters):
            call()
        b.record()
        torch.cuda.synchronize()
        us = 1000.0 * a.elapsed_time(b) / iters
        res["overlap_m4" if overlap else "pool_m128"] = {
            "us": us, "bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    return res


# ---------------------------------------------------------- CPU baseline ----

def cpu_baseline(prefill_inputs, torch, n_queries):
    """The oracle, as it stands, on a bounded sample of the same prefill:
    both compressors over all 8192 tokens, then indexer + top-k + attention
    for `n_queries` query rows spread over the sequence.  The rate is
    extrapolated to all 8192 queries."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info()}))
    except Exception:  # pragma: no cover
        threads, blas = os.cpu_count(), "unknown"
    d = {key: v.detach().to("cpu", torch.float64).numpy() for key, v in prefill_inputs.items()
         if isinstance(v, torch.Tensor) and key not in ("q", "qI", "w")}
    p = prefill_inputs["params"]
    n, m, k, nw = p["n"], p["m"], p["k"], p["n_win"]
    rows = np.linspace(0, n - 1, n_queries).astype(np.int64)
    rsel = torch.tensor(rows, device=prefill_inputs["q"].device)
    q = prefill_inputs["q"][rsel].to("cpu", torch.float64).numpy()
    qI = prefill_inputs["qI"][rsel].to("cpu", torch.float64).numpy()
    w = prefill_inputs["w"][rsel].to("cpu", torch.float64).numpy()
    t0 = time.perf_counter()
    Cc = O.compress_overlap(d["Ca"], d["Cb"], d["Za"], d["Zb"], d["Ba"], d["Bb"], m)
    KI = O.compress_overlap(d["ICa"], d["ICb"], d["IZa"], d["IZb"], d["IBa"], d["IBb"], m)
    t1 = time.perf_counter()
    idx, _ = O.index_topk(qI, w, KI, rows, m, k)
    O.csa_attend(q, Cc, idx, d["Ca"], 0, d["sink"], rows, nw, prefill_inputs["scale"], m)
    t2 = time.perf_counter()
    full = (t1 - t0) + (t2 - t1) * n / n_queries
    return {"value": n / full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"float64 NumPy oracle ({blas}): both compressors over all {n} tokens "
                       f"({t1 - t0:.2f} s) + indexer/top-k/attention for {n_queries} evenly spaced "
                       f"queries ({t2 - t1:.2f} s), extrapolated to {n} queries"),
            "seconds": t2 - t0}


def calibrate_copy(torch):
    """A plain elementwise copy of known size (1 GiB read, 1 GiB written),
    for scaling the HBM byte counters."""
    nbytes = 1 << 30
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 3}))


def run_achievable_peaks(args, torch):
    """What plain library work reaches on this GPU beside the published
    peaks: an elementwise copy of 1 GiB (1 GiB read and 1 GiB written per
    call) and a square bf16 GEMM (torch.mm, 8192^3, both operands
    contiguous, float32 accumulation).  Context for the roofline fractions,
    which stay against the published peaks."""
    nbytes = 1 << 30
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    us_copy = _event_us(torch, lambda: torch.mul(a, 1.0, out=b), 20)
    del a, b
    nm = 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    x = torch.randn((nm, nm), device="cuda", generator=g).to(torch.bfloat16)
    y = torch.randn((nm, nm), device="cuda", generator=g).to(torch.bfloat16)
    z = torch.empty((nm, nm), dtype=torch.bfloat16, device="cuda")
    us_mm = _event_us(torch, lambda: torch.mm(x, y, out=z), 20)
    del x, y, z
    gbs = 2 * nbytes / (us_copy * 1e-6) / 1e9
    tf = 2 * nm ** 3 / (us_mm * 1e-6) / 1e12
    return {"hbm_copy_gbs": gbs, "hbm_copy_frac": gbs / PEAK_HBM_GBS,
            "bf16_gemm_tflops": tf, "bf16_gemm_frac": tf / PEAK_BF16_TFLOPS,
            "copy": "torch elementwise copy, 1 GiB read + 1 GiB written per call",
            "gemm": "torch.mm, 8192 x 8192 x 8192 bf16, contiguous operands"}


# ------------------------------------------------------- HBM traffic ----

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_ds_csa_prefill_n8192_hbm_traffic.json")
ATTEND_SOURCES = [os.path.join(ROOT, "long_context_compressed_csa_amd", "csrc", f)
                  for f in ("attend.hip", "common.hpp")]


def _sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _pmc_mean(csv_dir, counter, name_regex, grid=None):
    """Mean of one counter over the dispatches whose kernel name matches (and
    whose grid has `grid` threads, when given)."""
    import csv
    import glob
    import re
    vals = []
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter and re.search(name_regex, row["Kernel_Name"]) and \
                        (grid is None or int(row["Grid_Size"]) == grid):
                    vals.append(float(row["Counter_Value"]))
    if not vals:
        raise RuntimeError(f"no {counter} samples for /{name_regex}/ under {csv_dir}")
    return sum(vals) / len(vals), len(vals)


def traffic_summary(pmc_dir, commands):
    """Per-launch HBM bytes of the prefill attention kernel from four counter
    runs (prefill FETCH_SIZE, prefill WRITE_SIZE, copy FETCH_SIZE, copy
    WRITE_SIZE, each in KiB per dispatch, in PMC_DIR/prefill-fetch,
    prefill-write, copy-FETCH_SIZE, copy-WRITE_SIZE), every counter scaled by
    what it reads for the 1 GiB copy."""
    att = r"attend_ds<0, 0, 0, 0>"
    grid = 8192 * 256   # the n = 8192 prefill launch: one 256-thread workgroup per query
    cp = "vectorized_elementwise_kernel<4, at::native::AUnary"
    f_att, nf = _pmc_mean(os.path.join(pmc_dir, "prefill-fetch"), "FETCH_SIZE", att, grid)
    w_att, nw = _pmc_mean(os.path.join(pmc_dir, "prefill-write"), "WRITE_SIZE", att, grid)
    f_cp, _ = _pmc_mean(os.path.join(pmc_dir, "copy-FETCH_SIZE"), "FETCH_SIZE", cp)
    w_cp, _ = _pmc_mean(os.path.join(pmc_dir, "copy-WRITE_SIZE"), "WRITE_SIZE", cp)
    copy_bytes = float(1 << 30)
    f_scale = copy_bytes / (f_cp * 1024.0)
    w_scale = copy_bytes / (w_cp * 1024.0)
    read_b = f_att * 1024.0 * f_scale
    write_b = w_att * 1024.0 * w_scale
    rec = {
        "kernel": "attend_ds<0,0,0,0> (csa_attend), CSA prefill n=8192, n_h=64, c=512, k=512, n_win=128",
        "attend_sources_sha256": _sources_sha256(ATTEND_SOURCES),
        "fetch_kib_per_dispatch": f_att, "write_kib_per_dispatch": w_att,
        "dispatches": {"fetch": nf, "write": nw},
        "copy_fetch_kib": f_cp, "copy_write_kib": w_cp, "copy_bytes_each_way": copy_bytes,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "read_bytes_per_launch": read_b, "write_bytes_per_launch": write_b,
        "traffic_bytes_per_launch": read_b + write_b,
        "commands": commands,
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def recorded_traffic():
    """The recorded per-launch HBM bytes, or None when there is no record or
    the attention sources have changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("attend_sources_sha256") != _sources_sha256(ATTEND_SOURCES):
        return None
    return rec.get("traffic_bytes_per_launch")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps before the timed ones; about 50 prefill steps bring the GPU clocks to "
                         "their steady state (dispatch times fall by about a fifth over the first 25)")
    ap.add_argument("--only", choices=["prefill", "decode", "hca", "compress", "next", "peaks"], default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-queries", type=int, default=8192)
    ap.add_argument("--decode-reps", type=int, default=10)
    ap.add_argument("--hca-iters", type=int, default=3)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--core", action="store_true",
                    help="with --only: time only the workload's main step (for profiler runs), no secondary lines")
    ap.add_argument("--traffic-summary", metavar="PMC_DIR", default=None,
                    help="summarise counter runs under PMC_DIR/{attend_fetch,attend_write,copy_fetch,"
                         "copy_write} into the traffic record under profiles/ (no GPU needed)")
    ap.add_argument("--traffic-commands", default="", help="the commands that made PMC_DIR, for the record")
    a = ap.parse_args(argv)
    if a.traffic_summary:
        traffic_summary(a.traffic_summary, a.traffic_commands)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: this library has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import long_context_compressed_csa_amd as L
    from long_context_compressed_csa_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    L.load_library()
    if a.calibrate_copy:
        calibrate_copy(torch)
        return
    extras = {}
    pre = None
    if a.only in (None, "prefill"):
        print("[bench] prefill", file=sys.stderr, flush=True)
        pre = run_prefill(a, torch, L, synth)
    if a.only in (None, "decode"):
        print("[bench] decode", file=sys.stderr, flush=True)
        extras["decode_1m"] = run_decode(a, torch, L, synth)
    if a.only in (None, "hca"):
        print("[bench] hca", file=sys.stderr, flush=True)
        extras["hca_prefill"] = run_hca(a, torch, L, synth)
        extras["hca_decode_1m"] = run_hca_decode(a, torch, L, synth)
    if a.only in (None, "compress"):
        print("[bench] compress", file=sys.stderr, flush=True)
        extras["compressor"] = run_compress(a, torch, L, synth)
    if a.only in (None, "next") and not a.core:
        print("[bench] paged decode", file=sys.stderr, flush=True)
        extras["paged_decode_1m"] = run_paged_decode(a, torch, L, synth)
        torch.cuda.empty_cache()
        print("[bench] backward", file=sys.stderr, flush=True)
        extras["backward"] = run_backward(a, torch, L, synth)
        torch.cuda.empty_cache()
        print("[bench] fp8 kv, bf16 scores", file=sys.stderr, flush=True)
        extras.update(run_fp8kv_and_bf16_scores(a, torch, L, synth))
        torch.cuda.empty_cache()
    if a.only in (None, "peaks") and not a.core:
        print("[bench] achievable peaks", file=sys.stderr, flush=True)
        extras["achievable_peaks"] = run_achievable_peaks(a, torch)
        torch.cuda.empty_cache()
    if pre is None or a.core:
        if pre is not None:
            extras["prefill"] = {k: v for k, v in pre.items() if k != "inputs"}
        print(json.dumps({"extras": extras}))
        return
    cpu = None
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(pre["inputs"], torch, a.cpu_queries)
    att_us = pre["stage_us"]["attend"]
    line = {
        "metric": METRIC,
        "value": pre["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": pre["ms_per_step"],
        "ms_per_step_wall_mean": pre["ms_per_step_wall"],
        "timing": "ms_per_step is the median of the K per-step HIP-event intervals (after 0.3 s of untimed "
                  "steps for the clocks and W warm-up steps); the wall-clock mean of the same K steps is "
                  "ms_per_step_wall_mean",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs at the layer's shapes; no trained weights)",
        "config": {"workload": "CSA prefill layer, n=8192, n_h=64, c=512, m=4, k=512, n_win=128, "
                               "indexer 64x128, bf16, causal",
                   "global_batch": 1, "seq_len": 8192},
        "roofline": {"bound": "mfma", "kernel": "attend_ds (csa_attend)",
                     "achieved": pre["attend_tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": pre["attend_tflops"] / PEAK_BF16_TFLOPS, "traffic": recorded_traffic(),
                     "flop_per_launch": pre["flop_attend"], "avg_launch_us": att_us},
        "cpu_baseline": cpu,
        "stage_us": pre["stage_us"],
        "step_mfma_frac": pre["step_tflops"] / PEAK_BF16_TFLOPS,
        "index_tflops": pre["index_tflops"],
        "index_topk_mxfp4_us": pre["index_topk_mxfp4_us"],
        "index_topk_fp8_us": pre["index_topk_fp8_us"],
        "prefill_mxfp4_indexer": pre["mxfp4_step"],
        "prefill_norm_rope": pre["norm_rope_step"],
        "grouped_out_proj": pre["out_proj"],
    }
    if "decode_1m" in extras:
        line["decode_us_per_step"] = extras["decode_1m"]["us_per_step"]
    line["extras"] = extras
    print(json.dumps(line))


if __name__ == "__main__":
    main()
