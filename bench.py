#!/usr/bin/env python3
"""Benchmark of the MoE dispatch -> expert FFN -> combine path on one MI355X.

A step is one pass of the whole path (plan, dispatch, expert FFN, combine) over
one batch of synthetic input already resident in HBM. Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload zipf_skew]

Default workload: zipf_skew (T=16384, H=4096, I=1536, 128 experts, K=8, tile
128, Zipf(1.2)-biased routing, bf16), the largest of the five workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense MFMA, bf16
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense MFMA, fp8
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


FFN_SOURCES = ("ffn.hip", "ffn_sq.hip", "ffn_sq.h")


def kernel_source_hash() -> str:
    """Hash of the FFN kernel sources, comments and blank lines left out: counter readings
    in profiles/ are valid only for the code they were taken on."""
    import re

    code = []
    for name in FFN_SOURCES:
        p = os.path.join(ROOT, "combine_moe_dispatch_02_amd", "csrc", name)
        code += [re.sub(r"//.*$", "", ln).rstrip() for ln in open(p).read().splitlines()]
    return hashlib.sha256("\n".join(ln for ln in code if ln).encode()).hexdigest()[:16]


def read_traffic(workload: str, src_hash: str):
    """HBM bytes per FFN call from the committed counter summary, if it matches this source."""
    p = os.path.join(ROOT, "profiles", f"ffn_traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    if d.get("ffn_source_sha256_16") != src_hash:
        return None
    return d.get("hbm_bytes_per_ffn_call")


def algorithmic_work(cfg, idx_np):
    """Per-step algorithmic work, real rows only (padding excluded)."""
    import numpy as np

    local = (idx_np >= cfg.expert_begin) & (idx_np < cfg.expert_begin + cfg.num_local_experts)
    N = int(local.sum())                        # local pairs
    T_act = int(local.any(axis=1).sum())        # tokens with at least one local pair
    H, I, K, T = cfg.H, cfg.I, cfg.K, cfg.T
    # bytes per element with scales: bf16 2; fp8 e4m3 + fp32 per 1x128 group (activations) or
    # per 128x128 block (weights); mxfp4 e4m3 + E8M0 per 1x32 (activations), e2m1 + E8M0 per 1x32
    pool_b = {"bf16": 2, "fp8": 1 + 4 / 128, "mxfp4": 1 + 1 / 32}[cfg.dtype]
    w_b = {"bf16": 2, "fp8": 1 + 4 / (128 * 128), "mxfp4": 0.5 + 1 / 32}[cfg.dtype]
    return {
        "pairs": N,
        "ffn_flops": 6.0 * N * H * I,
        # least HBM traffic of the FFN: every local weight once, the pool rows read,
        # h written and read back, y written
        "ffn_bytes": cfg.num_local_experts * 3 * H * I * w_b + N * H * pool_b + 2 * N * I * pool_b + N * H * 2,
        "dispatch_bytes": T_act * H * 2 + N * H * pool_b,
        "combine_bytes": N * H * 2 + T * H * 2 + T * K * 8,
    }


def cpu_baseline(inp, max_tokens: int, target_s: float = 15.0, gpu_out=None):
    """The oracle as it stands, timed on the first tokens of the same workload: probes on 64 and
    256 tokens size the sample to about ``target_s`` seconds of CPU work (at most ``max_tokens``).
    With ``gpu_out`` (the layer's output on the GPU), also the max-normwise relative error of
    those tokens against the oracle."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    # two probes: the oracle's time is a fixed part (the experts' weights in float64) plus a
    # part per token, so a straight line through two sample sizes sizes the run
    probes = []
    for m in (min(64, max_tokens), min(256, max_tokens)):
        t0 = time.perf_counter()
        oracle.moe_layer(inp, tokens=np.arange(m))
        probes.append((m, time.perf_counter() - t0))
    (m0, p0), (m1, p1) = probes
    per_tok = max((p1 - p0) / max(m1 - m0, 1), 1e-6)
    fixed = max(p0 - m0 * per_tok, 0.0)
    n = int(max(64, min(max_tokens, (target_s - fixed) / per_tok)))
    # larger samples run faster per token (bigger matrix products), so a sample that finishes
    # in under half the target is grown once by the ratio and timed again
    sized = f"sized by probes of {m0} and {m1} tokens: {p0:.1f} and {p1:.1f} s"
    for attempt in range(2):
        toks = np.arange(n)
        t0 = time.perf_counter()
        ref = oracle.moe_layer(inp, tokens=toks)
        dt = time.perf_counter() - t0
        if attempt == 1 or dt >= 0.5 * target_s or n >= max_tokens:
            break
        sized += f"; {n} tokens took {dt:.1f} s"
        n = int(min(max_tokens, n * target_s / max(dt, 1e-3)))
    out = {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"tokens 0..{n - 1} of the workload (all their pairs), float64 NumPy oracle incl. "
                     f"weight dequantisation, {dt:.1f} s ({sized})"}
    if gpu_out is not None:
        got = oracle.bf16_to_f64(gpu_out[:n].cpu())
        out["gpu_max_norm_rel_err"] = float(oracle.max_norm_rel_err(got, ref.out))
    return out


def measured_peaks(dev):
    """The device's own rates beside the spec peaks: a bf16 MFMA loop and streaming read /
    write / copy kernels of the library (moe_calibrate_*), timed with HIP events."""
    import ctypes

    import torch

    import combine_moe_dispatch_02_amd as moe
    from combine_moe_dispatch_02_amd import _abi

    lib = _abi.load()
    cus = moe.device_cu_count()
    s = torch.cuda.current_stream()
    sp = ctypes.c_void_p(s.cuda_stream)
    sink = torch.empty(cus * 8 * 512, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=3):
        fn()
        best = 1e9
        for _ in range(reps):
            e0.record(s)
            fn()
            e1.record(s)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        return best

    iters = 20000
    t = timed(lambda: _abi.check("moe_calibrate_mfma", lib.moe_calibrate_mfma(
        iters, ctypes.c_void_p(sink.data_ptr()), cus, sp)))
    mfma = cus * 8 * iters * 16 * 16384 / t / 1e12
    nbytes = 2 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    a.fill_(1)
    rates = {}
    for mode, name, factor in ((0, "read", 1), (1, "write", 1), (2, "copy", 2)):
        t = timed(lambda: _abi.check("moe_calibrate_stream", lib.moe_calibrate_stream(
            ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), nbytes, mode,
            ctypes.c_void_p(sink.data_ptr()), cus * 8, sp)))
        rates[name] = factor * nbytes / t / 1e9
    del a, b
    return {"mfma_bf16_loop_TFLOPs": round(mfma, 1), "spec_bf16_TFLOPs": PEAK_BF16_TFLOPS,
            "hbm_read_GBps": round(rates["read"], 1), "hbm_write_GBps": round(rates["write"], 1),
            "hbm_copy_GBps": round(rates["copy"], 1), "spec_hbm_GBps": PEAK_HBM_GBS,
            "method": f"bf16 MFMA loop on {cus} CUs x 8 waves; one grid-stride pass over 2 GiB "
                      f"(copy counts read + write bytes); best of 3, HIP events"}


def routing_stats(layer, cfg):
    """Realised routing of the step: pairs per local expert and the pool it makes."""
    c = layer.plan.counts.cpu().numpy().astype(float)
    return {"max_count": int(c.max()), "mean_count": round(float(c.mean()), 1),
            "max_over_mean": round(float(c.max() / max(c.mean(), 1e-9)), 2),
            "empty_experts": int((c == 0).sum()), "tiles": int(layer.plan.num_tiles.item()),
            "pool_rows": int(layer.plan.offsets[-1].item())}


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    import re
    import subprocess
    try:
        out = subprocess.run(["c++filt", name], capture_output=True, text=True).stdout.strip()
        name = out or name
    except OSError:
        pass
    return re.sub(r"moe::|\(moe::\w+\)|void |at::native::", "", name)[:70]


def summarize_profiles(workload, trace_dir, fetch_dir, write_dir, out_dir, commands, train=False):
    """rocprofv3 CSV output -> profiles/moe_layer_<workload>.txt and the FFN traffic JSON
    (training runs: profiles/moe_train_<workload>.txt only).

    FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by what they read for the
    three 1 GiB device-to-device copies of --copy-calibration."""
    import collections

    stats = _read_csv(os.path.join(trace_dir, "run_kernel_stats.csv"))
    per = {}
    for d, cname in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rows = [r for r in _read_csv(os.path.join(d, "run_counter_collection.csv")) if r["Counter_Name"] == cname]
        copies = sorted((float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]),
                        reverse=True)
        scale = (1 << 20) / (sum(copies[:3]) / 3)  # KiB of a 1 GiB copy -> bytes factor
        # the 256 MiB copies, where the run made them (a reading near a quarter of the 1 GiB
        # one): the factor should not depend on the size
        quarter = sum(copies[:3]) / 12
        small = [c for c in copies[3:] if abs(c - quarter) < 0.2 * quarter][:3]
        scale_small = (1 << 18) / (sum(small) / len(small)) if len(small) == 3 else None
        agg = collections.defaultdict(list)
        for r in rows:
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]) * 1024 * scale)
        per[cname] = ({k: sum(v) / len(v) for k, v in agg.items()}, scale, scale_small)
    ffn = [r for r in stats if "ffn_" in r["Name"]]
    ffn_ns = sum(float(r["AverageNs"]) for r in ffn)
    fetch = sum(v for k, v in per["FETCH_SIZE"][0].items() if "ffn_" in k)
    write = sum(v for k, v in per["WRITE_SIZE"][0].items() if "ffn_" in k)
    title = "MoE layer training step (forward keeping G + backward)" if train else "MoE layer"
    lines = [f"# rocprofv3 summary: {title}, workload {workload}", "",
             "Commands (from the repository root on one MI355X):"]
    lines += [f"  {c}" for c in commands]
    lines += ["", f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} "
              f"{'fetch_MB':>10s} {'write_MB':>10s}"]
    for r in stats:
        n = r["Name"]
        fv = per["FETCH_SIZE"][0].get(n)
        wv = per["WRITE_SIZE"][0].get(n)
        lines.append(f"{_short(n):70s} {r['Calls']:>6s} {float(r['AverageNs'])/1e3:10.1f} "
                     f"{float(r['MinNs'])/1e3:10.1f} {float(r['MaxNs'])/1e3:10.1f} "
                     f"{(fv or 0)/1e6:10.1f} {(wv or 0)/1e6:10.1f}")
    def _sc(c):
        s1, s2 = per[c][1], per[c][2]
        return f"x{s1:.3f}" + (f" (256 MiB copy: x{s2:.3f})" if s2 else "")
    lines += ["", f"fetch_MB / write_MB: FETCH_SIZE / WRITE_SIZE, the bytes the L2 requested from / wrote to the",
              f"memory fabric (L2 misses; Infinity Cache hits included), scaled to bytes by what the counters",
              f"read for a device copy of known size: FETCH_SIZE {_sc('FETCH_SIZE')} of the KiB reading "
              f"(1 GiB copy), WRITE_SIZE {_sc('WRITE_SIZE')}."]
    os.makedirs(out_dir, exist_ok=True)
    if train:
        lines += ["The training step's kernels, by template: ffn_big_kernel<..., GEMM_A=true, ...> is the",
                  "forward GEMM A keeping G; <..., GEMM_A=false, ..., EPI=1, ...> the backward GEMM Y (data,",
                  "SwiGLU backward in its epilogue); <..., GEMM_A=false, ..., EPI=0, ...> both the forward",
                  "GEMM Y and the backward GEMM A (data), averaged together; wgrad_kernel both weight-gradient",
                  "GEMMs (dW2, then dW1), averaged together."]
        txt = os.path.join(out_dir, f"moe_train_{workload}.txt")
        with open(txt, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(txt)
        return
    lines.append(f"expert FFN (all ffn_ kernels of one call): {ffn_ns/1e3:.1f} us, "
                 f"L2-miss fetch {fetch/1e9:.3f} GB + write {write/1e9:.3f} GB per call")
    txt = os.path.join(out_dir, f"moe_layer_{workload}.txt")
    with open(txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    js = os.path.join(out_dir, f"ffn_traffic_{workload}.json")
    with open(js, "w") as f:
        json.dump({"workload": workload, "ffn_source_sha256_16": kernel_source_hash(),
                   "hbm_bytes_per_ffn_call": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
                   "ffn_avg_us": ffn_ns / 1e3, "fetch_scale": per["FETCH_SIZE"][1],
                   "write_scale": per["WRITE_SIZE"][1], "fetch_scale_256MiB": per["FETCH_SIZE"][2],
                   "write_scale_256MiB": per["WRITE_SIZE"][2],
                   "counts": "FETCH_SIZE / WRITE_SIZE: L2-to-memory-fabric bytes (Infinity Cache hits included)",
                   "commands": commands}, f, indent=1)
    print(txt)
    print(js)


def train_bench(args, cfg):
    """Training step = forward (plan, dispatch, FFN keeping G, combine) + backward (combine
    backward, backward grouped GEMMs Y and A with their weight gradients, dispatch backward)."""
    import torch

    import combine_moe_dispatch_02_amd as moe
    from synth import make_dout, make_inputs

    if cfg.dtype != "bf16":
        raise SystemExit("--train runs the bf16 workloads")
    log(f"[bench] generating {cfg.name} inputs (training)")
    inp = make_inputs(cfg, pin_memory=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x, idx, w = inp.x.to(dev), inp.topk_idx.to(dev), inp.topk_weights.to(dev)
    dout = make_dout(cfg, inp.seed).to(dev)
    layer = moe.StreamMoE(cfg.T, cfg.H, cfg.I, cfg.K, cfg.num_local_experts, expert_begin=cfg.expert_begin,
                          tile=cfg.tile, dtype="bf16", train=True)
    w1d, w2d = inp.w1.to(dev), inp.w2.to(dev)
    w1, w2, _, _ = layer.prepare_weights(w1d, w2d)
    w1t, w2t = layer.prepare_backward_weights(w1d, w2d)
    del w1d, w2d
    torch.cuda.synchronize()
    work = algorithmic_work(cfg, inp.topk_idx.numpy())

    streams = moe.make_streams() if args.streams else None

    def step():
        layer.forward(x, idx, w, w1, w2, streams=streams)
        return layer.backward(dout, w, w1t, w2t, streams=streams)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if moe.moe_get_error(layer.ws) != 0:
        raise RuntimeError("device error during warmup")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # stages on the stream the calls run on
    s = torch.cuda.current_stream()
    names = ["plan", "dispatch", "ffn_train", "combine", "combine_backward", "ffn_backward", "dispatch_backward"]
    acc = dict.fromkeys(names, 0.0)
    dw1 = torch.empty(cfg.num_local_experts, 2 * cfg.I, cfg.H, dtype=torch.bfloat16, device=dev)
    dw2 = torch.empty(cfg.num_local_experts, cfg.H, cfg.I, dtype=torch.bfloat16, device=dev)
    evs = []
    for _ in range(args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        ep = layer.next_epoch()
        ev[0].record(s)
        moe.moe_plan(idx, layer.plan, layer.ws, s); ev[1].record(s)
        moe.moe_dispatch(x, layer.plan, layer.pool, None, ep, layer.ws, "bf16", s); ev[2].record(s)
        moe.moe_expert_ffn_train(layer.plan, layer.pool, w1, w2, ep, layer.ws, layer.y_pool, layer.g_pool,
                                 layer.cfg, s); ev[3].record(s)
        moe.moe_combine(layer.y_pool, w, layer.plan, layer.out, s); ev[4].record(s)
        eb = layer.next_epoch()
        moe.moe_combine_backward(dout, w, layer.y_pool, layer.plan, layer.y_pool, layer.dw, eb, layer.ws, s)
        ev[5].record(s)
        moe.moe_expert_ffn_backward(layer.plan, layer.pool, layer.y_pool, layer.g_pool, w1t, w2t, eb, layer.ws,
                                    layer.dx_pool, dw1, dw2, layer.cfg, s); ev[6].record(s)
        moe.moe_dispatch_backward(layer.dx_pool, layer.plan, layer.dx, s); ev[7].record(s)
        evs.append(ev)
    torch.cuda.synchronize()
    if moe.moe_get_error(layer.ws) != 0:
        raise RuntimeError("device error during timing")
    for ev in evs:
        for i, k in enumerate(names):
            acc[k] += ev[i].elapsed_time(ev[i + 1]) / len(evs)
    bwd_flops = 2 * work["ffn_flops"]          # data and weight gradients of both GEMMs
    bwd_tflops = bwd_flops / (acc["ffn_backward"] * 1e-3) / 1e12
    result = {
        "metric": "MoE layer training step tokens/s (forward + backward); backward grouped GEMMs % MFMA peak",
        "value": round(cfg.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "experts": cfg.num_experts,
                   "local_experts": cfg.num_local_experts, "K": cfg.K, "tile": cfg.tile, "routing": cfg.routing,
                   "pairs": work["pairs"], "mode": "training step (forward keeping G + backward)",
                   "streams": "two (comm + compute)" if args.streams else "one"},
        "roofline": {"bound": "mfma", "kernel": "backward grouped GEMMs (dgrad + wgrad of A and Y)",
                     "achieved": round(bwd_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "stages_ms": {k: round(v, 4) for k, v in acc.items()},
        "ffn_train_TFLOPs": round(work["ffn_flops"] / (acc["ffn_train"] * 1e-3) / 1e12, 1),
        "ffn_backward_TFLOPs": round(bwd_tflops, 1),
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def summarize_counters(workload, pmc_dirs, out_dir, commands):
    """rocprofv3 --pmc CSV output (one directory per counter pass) -> the per-kernel counter
    averages of the GEMM kernels with the rates read from them, in
    profiles/ffn_counters_<workload>.txt."""
    import collections

    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in pmc_dirs:
        for r in _read_csv(os.path.join(d, "run_counter_collection.csv")):
            vals[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = [f"# rocprofv3 counters: GEMM kernels, workload {workload}", "",
             "Commands (from the repository root on one MI355X):"]
    lines += [f"  {c}" for c in commands]
    lines += ["", "Values are per dispatch, averaged over the run's dispatches, summed over XCDs and CUs.",
              "GRBM_GUI_ACTIVE sums the 8 XCDs (cycles = GRBM_GUI_ACTIVE / 8); 1024 SIMDs, 256 CUs.", ""]
    for k, cs in vals.items():
        if not any(s in k for s in ("ffn_", "wgrad")):
            continue
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        lines.append(_short(k))
        for c in sorted(avg):
            lines.append(f"  {c:30s} {avg[c]:.4g}")
        cyc = avg.get("GRBM_GUI_ACTIVE", 0) / 8
        notes = []
        if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            notes.append(f"MFMA busy {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.1%} of SIMD cycles")
        if "SQ_WAIT_INST_ANY" in avg and avg.get("SQ_WAVE_CYCLES"):
            notes.append(f"waves waiting {avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.1%} of wave cycles")
        if cyc and "SQ_LDS_BANK_CONFLICT" in avg:
            notes.append(f"LDS bank-conflict cycles {avg['SQ_LDS_BANK_CONFLICT'] / (cyc * 256):.1%} of CU cycles")
        if "TCC_HIT" in avg and "TCC_MISS" in avg:
            notes.append(f"L2 hit rate {avg['TCC_HIT'] / (avg['TCC_HIT'] + avg['TCC_MISS']):.1%}")
        if cyc and "TCP_PENDING_STALL_CYCLES" in avg:
            notes.append(f"TCP pending-stall {avg['TCP_PENDING_STALL_CYCLES'] / (cyc * 256):.1%} of CU cycles")
        if cyc and "TA_BUSY_avr" in avg:
            notes.append(f"TA busy {avg['TA_BUSY_avr'] / cyc:.1%}")
        if notes:
            lines.append("  -> " + "; ".join(notes))
        lines.append("")
    os.makedirs(out_dir, exist_ok=True)
    txt = os.path.join(out_dir, f"ffn_counters_{workload}.txt")
    with open(txt, "w") as f:
        f.write("\n".join(lines))
    print(txt)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="zipf_skew")
    ap.add_argument("--streams", action="store_true", help="dispatch/combine and FFN on two streams")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured in a HIP graph (one stream)")
    ap.add_argument("--train", action="store_true",
                    help="time a training step: the forward (keeping G) plus the backward pass (bf16 workloads)")
    ap.add_argument("--combine-on-completion", action="store_true",
                    help="GEMM Y's workgroups combine each token once its tiles are done (no separate combine)")
    ap.add_argument("--block-n", type=int, default=0, help="tile config override: N block (0 = auto)")
    ap.add_argument("--gemm-wgs", type=int, default=0, help="tile config override: GEMM grid (0 = auto)")
    ap.add_argument("--unit-order", type=int, default=0, help="tile config override: unit walk (0 = auto)")
    ap.add_argument("--unit-rows", type=int, default=0,
                    help="tile config override: rows per GEMM work unit (0 = auto, 128, 256)")
    ap.add_argument("--dispatch-cus", type=int, default=0,
                    help="tile config override: CUs GEMM A leaves to a concurrent dispatch (0 = auto)")
    ap.add_argument("--a-stages", type=int, default=0,
                    help="tile config override: pool-row pipeline depth of the big-tile GEMMs (0 = auto, 2, 4)")
    ap.add_argument("--cpu-sample", type=int, default=16384,
                    help="most tokens of the oracle CPU baseline, sized to about 15 s of CPU work (0 = skip)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured MFMA / HBM peaks")
    ap.add_argument("--flush-steps", type=int, default=5,
                    help="steps also timed one by one after a 512 MiB write (the last-level cache "
                         "flushed); 0 = skip")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run three 1 GiB device-to-device copies (a known-size reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 CSV output and exit (no GPU)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="write profiles/ffn_counters_<workload>.txt from rocprofv3 --pmc CSV output and "
                         "exit (no GPU)")
    ap.add_argument("--profile-commands", default="", help="';'-separated commands recorded in the summary")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.workload, args.summarize_counters, os.path.join(ROOT, "profiles"),
                           [c.strip() for c in args.profile_commands.split(";") if c.strip()])
        return
    if args.summarize_profiles:
        summarize_profiles(args.workload, *args.summarize_profiles, os.path.join(ROOT, "profiles"),
                           [c.strip() for c in args.profile_commands.split(";") if c.strip()], train=args.train)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this single-GPU "
              f"path (no sharding across GPUs is built).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import combine_moe_dispatch_02_amd as moe
    from synth import config_by_name, make_inputs

    cfg = config_by_name(args.workload)
    if args.copy_calibration:
        # three 1 GiB copies, then three 256 MiB ones: two known sizes for the byte counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for n in (1 << 30, 1 << 28):
            for _ in range(3):
                dst[:n].copy_(src[:n])
        torch.cuda.synchronize()
        del src, dst
    if args.train:
        train_bench(args, cfg)
        return
    fp8 = cfg.dtype == "fp8"
    log(f"[bench] generating {cfg.name} inputs")
    inp = make_inputs(cfg, pin_memory=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = inp.x.to(dev, non_blocking=True)
    idx = inp.topk_idx.to(dev)
    w = inp.topk_weights.to(dev)
    if fp8 or cfg.dtype == "mxfp4":
        w1, w2 = inp.w1.view(torch.uint8).to(dev), inp.w2.view(torch.uint8).to(dev)
        w1s, w2s = inp.w1_scale.to(dev), inp.w2_scale.to(dev)
    else:
        w1, w2, w1s, w2s = inp.w1.to(dev), inp.w2.to(dev), None, None
    torch.cuda.synchronize()
    tcfg = None
    if args.block_n or args.gemm_wgs or args.unit_order or args.a_stages or args.unit_rows or args.dispatch_cus:
        tcfg = moe.TileConfig(args.block_n, args.gemm_wgs, 0, args.unit_order, 0, args.a_stages,
                              args.dispatch_cus, args.unit_rows)
    layer = moe.StreamMoE(cfg.T, cfg.H, cfg.I, cfg.K, cfg.num_local_experts,
                          expert_begin=cfg.expert_begin, tile=cfg.tile, dtype=cfg.dtype, cfg=tcfg,
                          combine_on_completion=args.combine_on_completion)
    # weight preprocessing at load time (not part of a step): MFMA fragment order when used
    w1, w2, w1s, w2s = layer.prepare_weights(w1, w2, w1s, w2s)
    torch.cuda.synchronize()
    work = algorithmic_work(cfg, inp.topk_idx.numpy())
    streams = moe.make_streams() if args.streams else None

    def step():
        return layer.forward(x, idx, w, w1, w2, w1s, w2s, streams)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rc = moe.moe_get_error(layer.ws)
    if rc != 0:
        raise RuntimeError(f"device error {rc} during warmup")
    if args.graph:
        # one step captured in a HIP graph (the same launches, replayed without the host)
        if streams is not None:
            raise SystemExit("--graph runs the one-stream step")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()

        def step():  # noqa: F811
            graph.replay()

        step()
        torch.cuda.synchronize()

    # whole-step timing: K steps bracketed by synchronisation
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    e_start.record()
    for _ in range(args.steps):
        step()
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e_start.elapsed_time(e_end) / args.steps

    # per-stage timing on the stream the kernels run on (single stream here)
    s = torch.cuda.current_stream()
    stage_ms = {"plan": 0.0, "dispatch": 0.0, "ffn": 0.0, "combine": 0.0}
    evs = []
    for _ in range(args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        epoch = layer.next_epoch()
        ev[0].record(s)
        moe.moe_plan(idx, layer.plan, layer.ws, s)
        ev[1].record(s)
        moe.moe_dispatch(x, layer.plan, layer.pool, layer.pool_s, epoch, layer.ws, cfg.dtype, s)
        ev[2].record(s)
        if args.combine_on_completion:
            # one call: the FFN with the combine inside GEMM Y (reported under "ffn"; combine 0)
            moe.moe_expert_ffn_combine(layer.plan, layer.pool, layer.pool_s, w1, w1s, w2, w2s, epoch,
                                       layer.ws, layer.y_pool, w, layer.out, cfg.dtype, layer.cfg, s)
            ev[3].record(s)
        else:
            moe.moe_expert_ffn(layer.plan, layer.pool, layer.pool_s, w1, w1s, w2, w2s, epoch, layer.ws,
                               layer.y_pool, cfg.dtype, layer.cfg, s)
            ev[3].record(s)
            moe.moe_combine(layer.y_pool, w, layer.plan, layer.out, s)
        ev[4].record(s)
        evs.append(ev)
    torch.cuda.synchronize()
    rc = moe.moe_get_error(layer.ws)
    if rc != 0:
        raise RuntimeError(f"device error {rc} during timing")
    for ev in evs:
        for i, k in enumerate(stage_ms):
            stage_ms[k] += ev[i].elapsed_time(ev[i + 1]) / len(evs)

    # the same steps with the last-level cache (256 MB) flushed before each: a 512 MiB write
    flushed = None
    if args.flush_steps > 0 and not args.graph:
        import ctypes

        from combine_moe_dispatch_02_amd import _abi
        junk = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        lib = _abi.load()
        f_ms = []
        for _ in range(args.flush_steps):
            _abi.check("moe_calibrate_stream", lib.moe_calibrate_stream(
                None, ctypes.c_void_p(junk.data_ptr()), junk.numel(), 1, None, 2048,
                ctypes.c_void_p(s.cuda_stream)))
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(s)
            step()
            a1.record(s)
            torch.cuda.synchronize()
            f_ms.append(a0.elapsed_time(a1))
        del junk
        f = sorted(f_ms)[len(f_ms) // 2]
        flushed = {"ms_per_step": round(f, 4), "value": round(cfg.T / (f * 1e-3), 1),
                   "steps": args.flush_steps, "how": "median of single steps, each after a 512 MiB write"}

    tokens_s = cfg.T / (ms_step * 1e-3)
    ffn_tflops = work["ffn_flops"] / (stage_ms["ffn"] * 1e-3) / 1e12
    ffn_gbs = work["ffn_bytes"] / (stage_ms["ffn"] * 1e-3) / 1e9
    # mxfp4 multiplies e2m1 weights by e4m3 activations: the scaled MFMA runs at the
    # rate of its wider operand, fp8
    peak = PEAK_FP8_TFLOPS if cfg.dtype in ("fp8", "mxfp4") else PEAK_BF16_TFLOPS
    # the FFN's bound: MFMA unless streaming its least traffic takes longer at HBM peak
    hbm_bound = work["ffn_bytes"] / (PEAK_HBM_GBS * 1e9) > work["ffn_flops"] / (peak * 1e12)
    disp_gbs = work["dispatch_bytes"] / (stage_ms["dispatch"] * 1e-3) / 1e9
    comb_gbs = (work["combine_bytes"] / (stage_ms["combine"] * 1e-3) / 1e9
                if not args.combine_on_completion else None)
    src_hash = kernel_source_hash()
    traffic = read_traffic(cfg.name, src_hash)
    result = {
        "metric": "MoE layer tokens/s; grouped-GEMM % MFMA peak; dispatch/combine HBM GB/s",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8", "mxfp4": "mxfp4 (e2m1 x e4m3)"}[cfg.dtype],
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I,
                   "experts": cfg.num_experts, "local_experts": cfg.num_local_experts, "K": cfg.K,
                   "tile": cfg.tile, "routing": cfg.routing, "pairs": work["pairs"],
                   "pool_rows": int(layer.plan.offsets[-1].item()),
                   "streams": "two (comm + compute)" if args.streams else "one",
                   "launch": "HIP graph replay" if args.graph else "eager",
                   "combine": ("on completion, inside GEMM Y (stage 'ffn' includes it)"
                               if args.combine_on_completion else "kernel after the FFN"),
                   "weights": "MFMA-tiled (permuted once at load time)" if layer.tiled else "row-major"},
        "roofline": ({"bound": "hbm", "kernel": "expert FFN (grouped GEMM A + Y)",
                      "achieved": round(ffn_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(ffn_gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
                     if hbm_bound else
                     {"bound": "mfma", "kernel": "expert FFN (grouped GEMM A + Y)",
                      "achieved": round(ffn_tflops, 1), "peak": peak, "unit": "TFLOP/s",
                      "frac": round(ffn_tflops / peak, 4), "traffic": traffic}),
        "ffn_TFLOPs": round(ffn_tflops, 1),
        "ffn_GBps_least_traffic": round(ffn_gbs, 1),
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "dispatch_GBps": round(disp_gbs, 1),
        "combine_GBps": round(comb_gbs, 1) if comb_gbs is not None else None,
        "dispatch_combine_frac_hbm": round(
            (work["dispatch_bytes"] + work["combine_bytes"])
            / ((stage_ms["dispatch"] + stage_ms["combine"]) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        if not args.combine_on_completion else None,
        "wall_s_timed": round(wall, 3),
        "mall_flushed": flushed,
        "routing": routing_stats(layer, cfg),
    }
    if not args.no_peaks:
        log("[bench] measured peaks")
        pk = measured_peaks(dev)
        result["measured_peaks"] = pk
        r = result["roofline"]
        if r["unit"] == "TFLOP/s" and cfg.dtype == "bf16":
            r["frac_of_measured_mfma_loop"] = round(r["achieved"] / pk["mfma_bf16_loop_TFLOPs"], 4)
        dc_rate = result["dispatch_combine_frac_hbm"]
        if dc_rate is not None:
            # dispatch writes about eight times what it reads, combine the reverse: the copy
            # rate is the streaming limit for that mix
            result["dispatch_combine_frac_of_measured_copy"] = round(
                dc_rate * PEAK_HBM_GBS / pk["hbm_copy_GBps"], 4)
    if args.cpu_sample > 0:
        log(f"[bench] oracle CPU baseline (at most {args.cpu_sample} tokens)")
        torch.cuda.synchronize()
        result["cpu_baseline"] = cpu_baseline(inp, min(args.cpu_sample, cfg.T), gpu_out=layer.out)
        result["oracle_max_norm_rel_err"] = result["cpu_baseline"].pop("gpu_max_norm_rel_err", None)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
