#!/usr/bin/env python3
"""Benchmark of one DFlash drafting round on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload q32] [--temperature T]

A step is one pass of the whole hot path over one batch: fuse the target
features of the rows accepted last round (1-16 rows per sequence, a seeded
schedule), inject them into every layer's context K/V, run the drafter forward
on [anchor, MASK x 15] with the fused argmax and greedy accept against seeded
target tokens, and take the bonus token as the next anchor (written in place).
With --temperature T > 0 the round drafts by sampling instead: the forward
writes the draft's fp32 logits, the candidates are drawn from softmax(logits/T)
and verified against seeded target logits by speculative rejection sampling
(residual resampling on rejection); the emitted token becomes the anchor.
Inputs are resident in HBM before the timed region. The context grows by the
appended rows every step, as in decoding; the reported context range covers
the whole run.

The default workload is the Qwen3-8B-shaped drafter at batch 32 with ragged
contexts of 512-8192 positions (the largest single-GPU configuration, where the
projections are matrix-core bound); a shorter batch-1 leg (context 2048, the
same drafter) follows it in the same process and is reported under "batch1".

Prints one JSON line: throughput in drafted block-tokens/s (batch * 16 per
step), the dominant kernel against its roofline (timed live with HIP events on
the library's stream), the attention kernel's HBM rate and the projections'
aggregate and per-class MFMA rates against the datasheet peaks and against
peaks measured in the same process (a 1 GiB device copy; an MFMA loop), the
whole step against its roofline, and the CPU oracle timed on this host on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "drafted block-tokens/sec (5-layer, block 16) + % HBM/MFMA roofline"


def measured_traffic(workload: str, kernel_class: str):
    """HBM bytes per launch from the counter record committed under profiles/
    for this workload and kernel class (FETCH_SIZE and WRITE_SIZE passes, each
    scaled by a 1 GiB copy), or None when there is none or when one of the
    kernel sources it lists has changed since the counters were taken."""
    import glob
    import hashlib
    import re
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for block in re.findall(r"```json\n(.*?)```", open(path).read(), flags=re.S):
            try:
                rec = json.loads(block)
            except ValueError:
                continue
            if rec.get("workload") != workload or rec.get("kernel_class") != kernel_class:
                continue
            for src, digest in rec.get("sources_sha256", {}).items():
                fp = os.path.join(ROOT, src)
                if not os.path.exists(fp) or hashlib.sha256(open(fp, "rb").read()).hexdigest() != digest:
                    return None
            return rec.get("traffic_bytes_per_launch")
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="q32", choices=["q1", "q32", "q4l", "l16", "train"],
                    help="train: the training-pattern attention of packed blocks alone "
                         "(its own metric; the drafting workloads time whole rounds)")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: draft by sampling softmax(logits / T) and verify by speculative "
                         "rejection sampling against seeded target logits (0: greedy)")
    ap.add_argument("--block", type=int, default=0,
                    help="drafter variant: block size B (default: the workload's, 16)")
    ap.add_argument("--layers", type=int, default=0,
                    help="drafter variant: number of draft layers (default: the workload's, 5)")
    ap.add_argument("--window", type=int, default=0,
                    help="drafter variant: every layer a sliding-window layer of this many keys")
    ap.add_argument("--graph", action="store_true",
                    help="also time the device-resident round (accept, fuse the block, inject "
                         "the accepted rows, draft) eagerly and as one replayed HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one 1 GiB device copy before timing (HBM counter calibration)")
    ap.add_argument("--no-batch1", action="store_true",
                    help="skip the batch-1 leg that follows the default batch-32 workload")
    ap.add_argument("--batch1-steps", type=int, default=30)
    return ap.parse_args()


def main() -> int:
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {a.gpus} is not supported "
              "(the drafter pass needs no exchange between GPUs).", file=sys.stderr)
        return 2
    import torch
    from block_diffusion_drafter_amd import binding as B
    from synth import WORKLOADS
    from synth import inputs as I
    from synth import torch_io

    if not torch.cuda.is_available():
        print("no GPU visible: bench.py needs an MI355X", file=sys.stderr)
        return 1
    if a.workload == "train":
        return bench_packed(a)
    W = WORKLOADS[a.workload]
    variant = {}
    if a.block:
        variant["block_size"] = a.block
    if a.layers:
        variant["n_layers"] = a.layers
    if a.window:
        variant["sliding_window"] = a.window
        variant["sliding_layers"] = tuple(range(a.layers or W.model.n_layers))

    def with_variant(w):
        if not variant:
            return w
        import dataclasses
        return dataclasses.replace(w, model=w.model.with_(**variant))

    W = with_variant(W)
    cfg = W.model
    host = I.Weights(cfg, W.seeds["weights"])
    model = B.DraftModel(cfg, torch_io.weights_to_device(host))

    if a.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out, leg = run_rounds(a, W, model, a.steps, a.warmup, headline=True)
    peaks = measured_peaks(B)
    attach_measured_peaks(out, peaks)

    # the batch-1 leg: same drafter, context 2048, after the headline
    if a.workload == "q32" and not a.no_batch1 and a.temperature == 0:
        W1 = with_variant(WORKLOADS["q1"])
        b1, _ = run_rounds(a, W1, model, a.batch1_steps, a.warmup, headline=False)
        attach_measured_peaks(b1, peaks)
        out["batch1"] = b1

    if a.graph:
        out["round_graph"] = time_round_graph(a, B, I, torch_io, W, model, leg["cache"], leg["ws"],
                                              leg["anchor"], leg["drafts"], leg["acc"],
                                              leg["status"])

    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W, host, leg["ctx_lens"], leg["n_new"], leg["feats"],
                                           a.cpu_seconds)

    print(json.dumps(out), flush=True)
    return 0


GEMM_CLASSES = ("gemm_f32out", "gemm_resid", "gemm_swiglu", "lm_head")


def measured_peaks(B) -> dict:
    """Peaks measured in this process on this chip: a 1 GiB device-to-device
    copy (read + write bytes per second) and the library's MFMA calibration
    loop (every matrix core busy with bf16 16x16x32 MFMAs and nothing else)."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(3):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 3 * 2 * (1 << 30) / (c0.elapsed_time(c1) / 1e3) / 1e9
    del src, dst
    n_wg, iters = 1024, 8000
    sink = torch.empty(n_wg * 8, dtype=torch.float32, device="cuda")
    B.probe_mfma_bf16(n_wg, iters // 4, sink)  # warm-up
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0.record()
    fl = sum(B.probe_mfma_bf16(n_wg, iters, sink) for _ in range(3))
    m1.record()
    torch.cuda.synchronize()
    mfma_tfl = fl / (m0.elapsed_time(m1) / 1e3) / 1e12
    return {"hbm_copy_GBps": round(copy_gbs, 1), "mfma_bf16_loop_TFLOPs": round(mfma_tfl, 1),
            "mfma_loop": f"{n_wg} workgroups x 8 waves x {iters} iterations x 8 MFMAs, 3 launches"}


def attach_measured_peaks(out: dict, peaks: dict) -> None:
    """Fractions of the measured peaks beside the datasheet ones."""
    out["measured_peaks"] = peaks
    roof = out["roofline"]
    if roof["bound"] == "hbm":
        roof["frac_of_measured_copy"] = round(roof["achieved"] / peaks["hbm_copy_GBps"], 4)
    else:
        roof["frac_of_measured_mfma_loop"] = round(roof["achieved"] /
                                                   peaks["mfma_bf16_loop_TFLOPs"], 4)
    for k in ("attention", "gemm"):
        e = roof.get(k)
        if not e:
            continue
        if e["unit"] == "GB/s":
            e["frac_of_measured_copy"] = round(e["achieved"] / peaks["hbm_copy_GBps"], 4)
        else:
            e["frac_of_measured_mfma_loop"] = round(e["achieved"] / peaks["mfma_bf16_loop_TFLOPs"], 4)
            for c in e.get("classes", {}).values():
                c["frac_of_measured_mfma_loop"] = round(c["TFLOPs"] / peaks["mfma_bf16_loop_TFLOPs"], 4)


def run_rounds(a, W, model, steps: int, warmup: int, headline: bool):
    """Prefill W's contexts, then time `steps` drafting rounds (after `warmup`).
    Returns the JSON record of the workload and the buffers the later legs use."""
    import torch
    from block_diffusion_drafter_amd import binding as B
    from synth import inputs as I
    from synth import torch_io

    cfg = W.model
    b, Bk, d = W.batch, cfg.block_size, cfg.hidden
    ctx_lens = I.ctx_lengths(W)
    max_new = cfg.block_size  # a round appends a + 1 <= B rows
    n_prof = max(3, min(10, steps))
    n_dist, n_cold = (min(steps, 20), min(steps, 10)) if headline else (0, 0)
    total_steps = (warmup + n_prof + steps + n_dist + n_cold +
                   (2 * (warmup + steps) if a.graph and headline else 0))
    cap = int(((int(ctx_lens.max()) + max_new * total_steps + Bk + 31) // 32) * 32)
    print(f"[bench] workload {W.name}: batch {b}, ctx {int(ctx_lens.min())}-{int(ctx_lens.max())}, "
          f"capacity {cap}", file=sys.stderr, flush=True)
    dt = model.dtype

    # ---- prefill (untimed): the context the rounds draft against -------------
    chunk_rows = 8192
    ws = model.new_workspace(b, cap, max(chunk_rows, b * max_new))
    cache = model.new_cache(b, cap)
    for s in range(b):
        for lo in range(0, int(ctx_lens[s]), chunk_rows):
            n = min(chunk_rows, int(ctx_lens[s]) - lo)
            feats = I.target_hiddens(cfg, n, seed=W.seeds["hiddens"], tag=f"prefill.{s}.{lo}")
            fd = [torch_io.to_device(f) for f in feats]
            ctx = torch.empty((n, d), dtype=dt, device="cuda")
            model.ctx_project(fd, ctx, ws)
            counts = np.zeros(b, np.int32)
            counts[s] = n
            cu = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
            model.ctx_kv_append(cache, ctx, cu, ws)
    torch.cuda.synchronize()

    # ---- per-round inputs (resident before timing) ----------------------------
    rng = np.random.Generator(np.random.PCG64(W.seeds["round_base"]))
    n_new = rng.integers(1, max_new + 1, size=b).astype(np.int32)
    n_tok = int(n_new.sum())
    feats = I.target_hiddens(cfg, n_tok, seed=W.seeds["round_base"], tag="round")
    feats_d = [torch_io.to_device(f) for f in feats]
    cu_new = torch.from_numpy(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)).cuda()
    ctx_new = torch.empty((n_tok, d), dtype=dt, device="cuda")
    anchor = torch.from_numpy(I.anchors(cfg, b, seed=W.seeds["targets"])).cuda()
    targets = torch.from_numpy(I.uniform_tokens(cfg, (b, Bk), W.seeds["targets"], "bench")).cuda()
    drafts = torch.empty((b, Bk - 1), dtype=torch.int32, device="cuda")
    acc = torch.empty(b, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    T = a.temperature
    if T > 0:
        # the draft's logits at the masked slots, the target's at the B block
        # positions (seeded stand-ins for the target's verify pass)
        V, m = cfg.vocab, Bk - 1
        logits = torch.empty((b, m, V), dtype=torch.float32, device="cuda")
        t_logits = torch.from_numpy(
            I.normal(W.seeds["targets"], "bench.target_logits", (b, Bk, V), 2.0, False)
            .reshape(b, Bk, V)).cuda()
        samp_ws = B.sampling_workspace(b, Bk, V)
        out_tok = torch.empty(b, dtype=torch.int32, device="cuda")
        logq = torch.empty(b * m, dtype=torch.float32, device="cuda")
    rnd = [0]

    def step():
        model.ctx_project(feats_d, ctx_new, ws)
        model.ctx_kv_append(cache, ctx_new, cu_new, ws, status)
        if T > 0:
            # sample the candidates from the draft's laws, verify them against
            # the target's; the emitted token is written over the anchor
            model.draft_forward(cache, anchor, drafts, ws, logits=logits, dev_status=status)
            B.sample_drafts(logits.view(b * m, V), T, 1234, rnd[0], drafts.view(-1), samp_ws,
                            logq=logq)
            B.verify_sampled(drafts, logits, t_logits, T, 1234, rnd[0], acc, out_tok, samp_ws,
                             anchor_out=anchor, draft_logq=logq)
            rnd[0] += 1
            return
        # the bonus token is written over the anchor: next round's anchor
        model.draft_forward(cache, anchor, drafts, ws, target_tokens=targets, accept_len=acc,
                            bonus=anchor, dev_status=status)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    assert status.item() == 0, f"device status {status.item()}"

    es = 2 if cfg.dtype == "bf16" else 4
    L, hd, Hkv, Hq = cfg.n_layers, cfg.head_dim, cfg.n_kv_heads, cfg.n_heads

    def read_profile(n_steps, ctx_before):
        """Per-class totals; attention bytes/flops from the context each step saw:
        step i attends over ctx_before + (i+1)*n_new + B keys per sequence."""
        prof = B.profiler_read()
        B.profiler_reset()
        keys = sum(float((ctx_before + (i + 1) * n_new + Bk).sum()) for i in range(n_steps))
        per_step = prof["attention"]["launches"] / max(n_steps, 1)
        prof["attention"]["bytes"] = keys * Hkv * hd * es * 2 * per_step   # K and V of every key
        prof["attention"]["flops"] = keys * Hq * Bk * hd * 4 * per_step
        return prof

    # ---- breakdown pass (untimed for the headline): every kernel bracketed ----
    ctx0 = cache.ctx_len.cpu().numpy().astype(np.int64)
    B.profiler_start(100000)
    for _ in range(n_prof):
        step()
    torch.cuda.synchronize()
    B.profiler_stop()
    prof_all = read_profile(n_prof, ctx0)
    ctx1 = cache.ctx_len.cpu().numpy().astype(np.int64)
    dom_name = max((k for k in prof_all if prof_all[k]["launches"]),
                   key=lambda k: prof_all[k]["ms"])

    # ---- timed region: only the dominant kernel class carries events --------
    B.profiler_start(100000, classes=[dom_name])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    B.profiler_stop()
    ms_step = e0.elapsed_time(e1) / steps
    dom = read_profile(steps, ctx1)[dom_name]
    assert status.item() == 0, f"device status {status.item()}"
    value = b * Bk / (ms_step / 1e3)

    # ---- after the headline: per-step spread, then steps with the 256 MB MALL
    # flushed by a 1 GiB read-modify-write before each ----------------------------
    def timed_steps(n, before=None):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for s0, s1 in ev:
            if before is not None:
                before()
            s0.record()
            step()
            s1.record()
        torch.cuda.synchronize()
        return sorted(s0.elapsed_time(s1) for s0, s1 in ev)

    if headline:
        spread = timed_steps(n_dist)
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cold = timed_steps(n_cold, before=lambda: scratch.add_(1))
        del scratch

    # KV append alone (the round's new rows: the stacked context K/V projection
    # of every layer, then norm/RoPE and the scatter into the cache); ctx_len
    # is put back after each call, so the same positions are rewritten.
    saved_len = cache.ctx_len.clone()
    for _ in range(2):  # untimed warm-up calls
        model.ctx_kv_append(cache, ctx_new, cu_new, ws, status)
        cache.ctx_len.copy_(saved_len)
    n_app = 10
    app_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_app)]
    # A short append (batch 1: two launches, ~30 us) is quicker than the host
    # takes to issue it; the stream spins first so that all calls are queued
    # before the first runs and each event pair brackets device time only.
    torch.cuda.synchronize()
    torch.cuda._sleep(20_000_000)
    for s0, s1 in app_ev:
        s0.record()
        model.ctx_kv_append(cache, ctx_new, cu_new, ws, status)
        s1.record()
        cache.ctx_len.copy_(saved_len)
    torch.cuda.synchronize()
    app_ms = float(np.median([s0.elapsed_time(s1) for s0, s1 in app_ev]))
    kvw = L * 2 * Hkv * hd
    app_bytes = (kvw * d * es              # K/V projection weights of every layer
                 + n_tok * d * es           # the new context rows
                 + n_tok * kvw * es)        # K/V rows scattered into the cache
    kv_append = {"ms": round(app_ms, 5), "rows": n_tok, "algorithmic_bytes": int(app_bytes),
                 "GBps": round(app_bytes / (app_ms / 1e3) / 1e9, 1),
                 "frac_of_hbm_peak": round(app_bytes / (app_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                 "traffic": measured_traffic(W.name, "kv_append")}
    ctx_end = cache.ctx_len.cpu().numpy().astype(np.int64)
    assert status.item() == 0, f"device status {status.item()}"

    def pct(v, q):
        return round(float(np.percentile(np.asarray(v), q)), 5)

    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    t_dom = dom["ms"] / 1e3
    gbs = dom["bytes"] / t_dom / 1e9
    tfl = dom["flops"] / t_dom / 1e12
    if dom["flops"] / max(dom["bytes"], 1.0) <= ridge:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tfl, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tfl / BF16_PEAK_TFLOPS, 4)}
    roof.update({"traffic": measured_traffic(W.name, dom_name), "kernel_class": dom_name,
                 "launches_per_step": dom["launches"] // steps,
                 "ms_per_launch": round(dom["ms"] / dom["launches"], 5),
                 "algorithmic_bytes_per_launch": dom["bytes"] / dom["launches"],
                 "algorithmic_flops_per_launch": dom["flops"] / dom["launches"],
                 "timing": f"HIP events around every launch of the class in the timed region "
                           f"({steps} steps)"})
    # The attention kernel against HBM, and the projections against the MFMA
    # peak (aggregate and per class), from the breakdown pass.
    att = prof_all["attention"]
    if att["launches"]:
        ag = att["bytes"] / (att["ms"] / 1e3) / 1e9
        roof["attention"] = {"achieved": round(ag, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(ag / HBM_PEAK_GBS, 4),
                             "traffic": measured_traffic(W.name, "attention"),
                             "ms_per_launch": round(att["ms"] / att["launches"], 5),
                             "timing": f"breakdown pass, every launch event-bracketed "
                                       f"({n_prof} steps)"}
    g_fl = sum(prof_all[c]["flops"] for c in GEMM_CLASSES)
    g_ms = sum(prof_all[c]["ms"] for c in GEMM_CLASSES)
    if g_ms > 0:
        gt = g_fl / (g_ms / 1e3) / 1e12
        classes = {c: {"TFLOPs": round(prof_all[c]["flops"] / (prof_all[c]["ms"] / 1e3) / 1e12, 1),
                       "frac": round(prof_all[c]["flops"] / (prof_all[c]["ms"] / 1e3) / 1e12 /
                                     BF16_PEAK_TFLOPS, 4),
                       "ms_per_step": round(prof_all[c]["ms"] / n_prof, 5),
                       "gflop_per_step": round(prof_all[c]["flops"] / n_prof / 1e9, 2)}
                   for c in GEMM_CLASSES if prof_all[c]["ms"] > 0}
        roof["gemm"] = {"achieved": round(gt, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(gt / BF16_PEAK_TFLOPS, 4), "classes": classes,
                        "timing": f"breakdown pass, every launch event-bracketed ({n_prof} steps); "
                                  "flops 2*M*N*K of the rows actually drafted (no padding)"}

    # whole step against its roofline: sum over kernels of max(bytes/BW, flops/peak)
    t_roof = sum(max(e["bytes"] / (HBM_PEAK_GBS * 1e9), e["flops"] / (BF16_PEAK_TFLOPS * 1e12))
                 for e in prof_all.values() if e["launches"]) / n_prof
    kernels = {k: {"launches_per_step": e["launches"] // n_prof,
                   "ms_per_step": round(e["ms"] / n_prof, 5),
                   "GBps": round(e["bytes"] / (e["ms"] / 1e3) / 1e9, 1) if e["bytes"] else None}
               for k, e in prof_all.items() if e["launches"]}

    out = {
        "metric": METRIC if (L, Bk) == (5, 16) else
        f"drafted block-tokens/sec ({L}-layer, block {Bk}) + % HBM/MFMA roofline",
        "value": round(value, 1), "unit": "block-tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic: seeded random-init drafter N(0,0.02^2), N(0,1) target hidden states",
        "config": {"workload": W.name, "batch": b, "block": Bk, "layers": L,
                   "ctx_len": [int(ctx_lens.min()), int(ctx_end.max())],
                   "new_rows_per_round": int(n_tok), "hidden": d, "heads": [Hq, Hkv],
                   "intermediate": cfg.intermediate, "vocab": cfg.vocab,
                   "decoding": f"sampled, temperature {T}" if T > 0 else "greedy",
                   "sliding_window": cfg.sliding_window or None,
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "step_roofline": {"t_roof_ms": round(t_roof * 1e3, 5),
                          "frac": round(t_roof * 1e3 / ms_step, 4),
                          "peaks": {"hbm_GBps": HBM_PEAK_GBS, "bf16_TFLOPs": BF16_PEAK_TFLOPS}},
        "kernels_event_bracketed": kernels,
        "wall_s_timed": round(wall, 4),
        "drafted_tokens_per_s": round(b * (Bk - 1) / (ms_step / 1e3), 1),
        "kv_append": kv_append,
    }
    if headline:
        out["ms_per_step_spread"] = {"steps": n_dist, "p10": pct(spread, 10),
                                     "p50": pct(spread, 50), "p90": pct(spread, 90)}
        out["ms_per_step_cold_mall"] = {"steps": n_cold, "p50": pct(cold, 50),
                                        "note": "1 GiB read-modify-write before each step, "
                                                "outside its events"}
    leg = dict(cache=cache, ws=ws, anchor=anchor, drafts=drafts, acc=acc, status=status,
               ctx_lens=ctx_lens, n_new=n_new, feats=feats)
    return out, leg


def time_round_graph(a, B, I, torch_io, W, model, cache, ws, anchor, drafts, acc, status):
    """The device-resident round (accept the verified block, fuse the features
    of all its B positions, inject the accepted rows, draft the next block):
    the four calls made one by one, then the same round captured once as a HIP
    graph and replayed. The synthetic target tokens are fixed, so the accept
    lengths (and with them the rows injected) come from the device."""
    import torch
    cfg = W.model
    b, Bk = W.batch, cfg.block_size
    feats = [torch_io.to_device(f) for f in
             I.target_hiddens(cfg, b * Bk, seed=W.seeds["round_base"], tag="block")]
    targets = torch.from_numpy(I.uniform_tokens(cfg, (b, Bk), W.seeds["targets"], "graph")).cuda()
    ctx = torch.empty((b * Bk, cfg.hidden), dtype=model.dtype, device="cuda")

    def eager():
        B.accept(drafts, targets, Bk, acc, anchor)
        model.ctx_project(feats, ctx, ws)
        model.ctx_kv_append_accepted(cache, ctx, acc, ws, status)
        model.draft_forward(cache, anchor, drafts, ws, dev_status=status)

    g = B.RoundGraph(model, cache, feats, targets, drafts, acc, anchor, ctx, ws, None, status)
    res = {}
    for name, fn in (("eager", eager), ("graph", g.replay)):
        for _ in range(a.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(a.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[f"ms_per_round_{name}"] = round(e0.elapsed_time(e1) / a.steps, 5)
    g.close()
    assert status.item() == 0, f"device status {status.item()}"
    res["block_tokens_per_s_graph"] = round(b * Bk / (res["ms_per_round_graph"] / 1e3), 1)
    res["rows_fused_per_round"] = b * Bk
    return res


def blas_facts() -> dict:
    """The BLAS NumPy runs on: vendor (from NumPy's build configuration) and the
    threads it uses (threadpoolctl)."""
    facts = {}
    try:
        cfg = np.show_config(mode="dicts")
        facts["vendor"] = cfg["Build Dependencies"]["blas"].get("name")
        facts["version"] = cfg["Build Dependencies"]["blas"].get("version")
    except Exception as e:  # numpy without the dict mode
        facts["vendor"] = f"unknown ({type(e).__name__})"
    try:
        import threadpoolctl
        pools = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            facts["threads"] = pools[0].get("num_threads")
            facts["internal_api"] = pools[0].get("internal_api")
    except Exception as e:
        facts["threads"] = f"unknown ({type(e).__name__})"
    return facts


def cpu_baseline(W, host, ctx_lens, n_new, feats, budget_s):
    """The CPU oracle as it stands on one sequence of the same round: fuse +
    inject its new rows, run the drafter forward and accept. Timed twice: with
    the oracle's arithmetic in float32 (the reported value) and in float64
    (its parity precision), each on about half of budget_s. The sequence's
    existing context K/V is a seeded synthetic cache state (setup, untimed).
    Reported in block-tokens/s."""
    from oracle import dflash_oracle as O
    from synth import inputs as I
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cfg = W.model
    c0 = int(ctx_lens[0])
    n0 = int(n_new[0])
    anchor = I.anchors(cfg, 1, seed=W.seeds["targets"])
    targets = I.uniform_tokens(cfg, (1, cfg.block_size), W.seeds["targets"], "bench")
    st = I.cache_state(cfg, [c0], seed=W.seeds["hiddens"] + 100)
    res = {}
    for dt, name in ((np.float32, "fp32"), (np.float64, "fp64")):
        # weights and cache in the compute type up front (setup, untimed)
        ow = {n: host.get(n).f32().astype(dt) for n in host.names()}
        if cfg.tied_embeddings:
            ow["lm_head"] = ow["embed"]
        cache = O.SeqCache([st[l][0][0].f32().astype(dt) for l in range(cfg.n_layers)],
                           [st[l][0][1].f32().astype(dt) for l in range(cfg.n_layers)])
        f0 = [f.f32()[:n0].astype(dt) for f in feats]
        rounds, t_used = 0, 0.0
        with O.compute_dtype(dt):
            while rounds < 1 or (t_used < budget_s / 2 and rounds < 20):
                t0 = time.perf_counter()
                ctx = O.ctx_project(f0, ow["fc"], ow["fc_norm"], cfg.rms_eps)
                new = O.prefill_cache(ctx, c0, ow, cfg)
                r = O.draft_forward(cfg, ow, [cache.append(new)], anchor)
                O.accept(r.drafts, targets)
                t_used += time.perf_counter() - t0
                rounds += 1
        res[name] = (rounds, t_used)
        del ow, cache
    r32, t32 = res["fp32"]
    r64, t64 = res["fp64"]
    return {"value": round(cfg.block_size * r32 / t32, 3), "unit": "block-tokens/s",
            "cores": cores, "kind": "oracle", "blas": blas_facts(),
            "fp64_value": round(cfg.block_size * r64 / t64, 3),
            "sample": f"1 sequence of {W.name} (ctx {c0}, {n0} new rows) per round: fusion, "
                      f"K/V injection, forward, accept; NumPy oracle with its arithmetic in "
                      f"float32: {r32} round(s) in {t32:.1f} s (value); in float64 (its parity "
                      f"precision): {r64} round(s) in {t64:.1f} s (fp64_value)"}


def bench_packed(a) -> int:
    """Training-pattern attention of packed blocks, every draft layer once per
    step: 4 sequences of 4096 positions of Qwen3-8B-shaped context (fused +
    injected by the library from seeded features), 512 anchors per sequence
    drawn over the response (positions 512..4096), block 16. The kernel reads
    each block's context prefix (mostly from L2: the blocks of a sequence share
    it) and its own 16 keys."""
    import torch
    from block_diffusion_drafter_amd import binding as B
    from synth import QWEN3_8B_SHAPED
    from synth import inputs as I
    from synth import torch_io

    cfg = QWEN3_8B_SHAPED
    n_seq, ctx_len, nb, prompt = 4, 4096, 512, 512
    Bk, L, Hq, Hkv, hd = cfg.block_size, cfg.n_layers, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    name = f"packed-blocks-qwen3-8b-shaped-{n_seq}x{ctx_len}-{nb}anchors"
    print(f"[bench] workload {name}", file=sys.stderr, flush=True)
    host = I.Weights(cfg, 0)
    model = B.DraftModel(cfg, torch_io.weights_to_device(host))
    cap = ((ctx_len + Bk + 31) // 32) * 32
    ws = model.new_workspace(n_seq, cap, 8192)
    cache = model.new_cache(n_seq, cap)
    for s in range(n_seq):
        for lo in range(0, ctx_len, 4096):
            n = min(4096, ctx_len - lo)
            fd = [torch_io.to_device(f) for f in I.target_hiddens(cfg, n, seed=1, tag=f"train.{s}.{lo}")]
            ctx = torch.empty((n, cfg.hidden), dtype=model.dtype, device="cuda")
            model.ctx_project(fd, ctx, ws)
            counts = np.zeros(n_seq, np.int32)
            counts[s] = n
            cu = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
            model.ctx_kv_append(cache, ctx, cu, ws)
    anchors = np.stack([I.training_anchors(ctx_len, nb, prompt, seed=6, tag=f"bench{s}")
                        for s in range(n_seq)])
    qh, kh, vh = I.packed_block_qkv(cfg, n_seq * nb, seed=5, tag="bench")
    q = torch_io.to_device(qh).view(n_seq, nb, Bk, Hq, hd)
    kb = torch_io.to_device(kh).view(n_seq, nb, Bk, Hkv, hd)
    vb = torch_io.to_device(vh).view(n_seq, nb, Bk, Hkv, hd)
    out = torch.empty_like(q)
    anc = torch.from_numpy(anchors).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step():
        for l in range(L):
            model.packed_block_attention(cache, l, anc, q, kb, vb, out, status)

    if a.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(a.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    assert status.item() == 0, f"device status {status.item()}"
    ms = e0.elapsed_time(e1) / a.steps
    keys = anchors.astype(np.int64) + Bk                          # keys per block
    flops = float(4 * hd * Hq * Bk * keys.sum()) * L              # QK^T and PV per step
    ctx_bytes = float(keys.sum()) * 2 * Hkv * hd * 2 * L           # K/V rows each block reads
    uniq = (n_seq * ctx_len * 2 * Hkv * hd * 2 + q.numel() * 2 * 2 + 2 * kb.numel() * 2) * L
    t = ms / 1e3
    res = {
        "metric": "packed-block attention block-tokens/sec (training pattern, 5 layers, block 16)",
        "value": round(n_seq * nb * Bk / t, 1), "unit": "block-tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic: seeded drafter, N(0,1) target features, N(0,1) block q/k/v",
        "config": {"workload": name, "sequences": n_seq, "ctx_len": ctx_len,
                   "anchors_per_seq": nb, "block": Bk, "layers": L, "heads": [Hq, Hkv],
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(flops / t / 1e12, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(name, "attention_packed"),
                     "kernel_class": "attention_packed",
                     "context_rows_streamed_TBps": round(ctx_bytes / t / 1e12, 2),
                     "unique_hbm_bytes_per_step": int(uniq),
                     "hbm_frac_of_unique_bytes": round(uniq / t / 1e12 / (HBM_PEAK_GBS / 1e3), 4)},
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_packed(cfg, host, anchors, qh, kh, vh, ctx_len, a.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline_packed(cfg, host, anchors, qh, kh, vh, ctx_len, budget_s):
    """The training-pattern oracle (fp64 NumPy) on blocks of sequence 0, layer
    0, one block at a time until the budget is spent; the context K/V of that
    sequence through the oracle's own fusion and projection (setup, untimed)."""
    from oracle import dflash_oracle as O
    from oracle import training as TR
    from synth import inputs as I
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    ow = {n: host.get(n).f32() for n in ("fc", "fc_norm", "layers.0.wk", "layers.0.wv",
                                         "layers.0.k_norm")}
    feats = [f.f32() for f in I.target_hiddens(cfg, ctx_len, seed=1, tag="train.0.0")]
    ctx = O.ctx_project(feats, ow["fc"], ow["fc_norm"], cfg.rms_eps)
    k, v = O.context_kv(ctx, np.arange(ctx_len), O.layer_weights(ow, 0), cfg)
    Bk, nb = cfg.block_size, anchors.shape[1]
    q = qh.f32().reshape(-1, Bk, cfg.n_heads, cfg.head_dim)
    kb = kh.f32().reshape(-1, Bk, cfg.n_kv_heads, cfg.head_dim)
    vb = vh.f32().reshape(-1, Bk, cfg.n_kv_heads, cfg.head_dim)
    done, t_used = 0, 0.0
    while done < nb and (done < 1 or t_used < budget_s):
        t0 = time.perf_counter()
        TR.packed_block_attention(q[done:done + 1], kb[done:done + 1], vb[done:done + 1], k, v,
                                  anchors[0, done:done + 1], cfg.n_heads // cfg.n_kv_heads)
        t_used += time.perf_counter() - t0
        done += 1
    return {"value": round(Bk * done / t_used / cfg.n_layers, 3), "unit": "block-tokens/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{done} block(s) of sequence 0 at layer 0 (anchors {int(anchors[0, 0])}.."
                      f"{int(anchors[0, done - 1])}), fp64 NumPy, {t_used:.1f} s; scaled to "
                      f"{cfg.n_layers} layers per step"}


if __name__ == "__main__":
    sys.exit(main())
