"""Benchmark of the nanochat GPT forward on one MI355X through libnc.so.

One step = the whole hot path over one batch: prefill of B x T prompt tokens with fp32
logits at every position, then greedy decode steps (argmax fed back).  Default line: the d20
bf16 model (20 layers, d=1280, 10x128 query heads, one K/V head, MLP 5120, vocab 65536),
prefill 32 x 2048 (the pages' 32 rows of 2048 tokens per GPU) and 128 decode steps of 64
rows at context 2048, seeded N(0, 0.02) weights and uniform random token ids.  Beside it, on
the same JSON line, the two stress runs of the other configs, each graded against its own
roof: "d26" (prefill 16 x 2048, the prefill products against the bf16 MFMA peak) and "d30"
(256 decode steps of 128 rows at context lengths uniform in [256, 2048], the decode
attention graded alone against HBM bandwidth).  Decode contexts that differ from the
prefill batch are built outside the timed steps.

Other workloads run alone with --workload (d12: prefill 8 x 2048 then 256 decode steps of
the same rows; d26; d30; tiny; d20-gqa with 5 K/V heads; d20-sssl with an SSSL pattern of
512-key sliding windows; d20-blocks with the later version's learned blocks; d12-sample
with sampled decode picks, temperature 1 and top-50, uniforms drawn before timing).

    python bench.py [--steps K] [--warmup W]
                    [--workload d20|d12|d26|d30|d20-gqa|d20-sssl|d20-blocks|d12-sample|tiny]
                    [--no-extra] [--no-cpu] [--no-roofline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="d20")
    p.add_argument("--no-extra", action="store_true",
                   help="default line only: skip the d26 prefill and d30 decode runs beside it")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--decode-steps", type=int, default=None,
                   help="override the workload's decode steps (short runs under a profiler)")
    p.add_argument("--no-roofline", action="store_true", help="skip the kernel-timing pass")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def cpu_baseline(shape, weights, wl, budget_s, windows=None, extras=None):
    """Time the fp64 oracle on the host on a bounded sample of the same workload.

    Sample: one row; prefill of min(T, 2048) tokens, then greedy decode steps until the
    time budget is spent.  The per-phase rates are combined with the workload's own mix of
    prefill and decode tokens into one tokens/s figure."""
    from oracle import OracleModel
    cores = len(os.sched_getaffinity(0))  # host cores this process may run on
    blas = {"vendor": "unknown", "threads": None}
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = {"vendor": f"{info[0].get('internal_api')} {info[0].get('version')}",
                    "threads": int(info[0].get("num_threads", 1))}
    except Exception:  # noqa: BLE001
        pass
    from dense_decoder_only_bf16_amd.inputs import make_tokens
    orc = OracleModel(shape, weights, windows=windows, extras=extras)
    t_pre = min(wl.prefill_len or wl.decode_context, 2048)  # decode-only: its context
    prompt = make_tokens(shape.vocab, 1, t_pre, seed=1)
    t0 = time.perf_counter()
    logits, cache = orc.prefill(prompt, max_seq=t_pre + 64, logits_at=[t_pre - 1])
    t1 = time.perf_counter()
    pre_rate = t_pre / (t1 - t0)
    tok = np.argmax(logits[:, 0], -1)
    steps = 0
    t2 = time.perf_counter()
    while steps < 64 and (steps < 2 or time.perf_counter() - t2 < budget_s / 2):
        tok = np.argmax(orc.decode_step(cache, tok), -1)
        steps += 1
    t3 = time.perf_counter()
    dec_rate = steps / (t3 - t2)
    n_pre = wl.prefill_batch * wl.prefill_len
    n_dec = wl.decode_batch * wl.decode_steps
    value = (n_pre + n_dec) / (n_pre / pre_rate + (n_dec / dec_rate if n_dec else 0.0))
    return {"value": round(value, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "blas": blas,
            "sample": (f"fp64 numpy oracle, 1 row: prefill {t_pre} tokens ({t1 - t0:.1f} s, "
                       f"{pre_rate:.1f} tok/s) + {steps} greedy decode steps at context "
                       f"{t_pre} ({t3 - t2:.1f} s, {dec_rate:.2f} tok/s); combined with the "
                       f"workload's mix of {n_pre} prefill and {n_dec} decode tokens"),
            "prefill_tokens_per_s": round(pre_rate, 2), "decode_tokens_per_s": round(dec_rate, 3)}


HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6  # MI355X dense bf16 matrix peak (256 CUs x 4096 flop/clk x 2.4 GHz)
FP32_VEC_PEAK_TFS = 157.3    # MI355X fp32 (the tiny fp32 model's products)

CLASSES = (  # (timing class, name, bound); classes without a launch in the workload are skipped
    ("NC_KC_DECODE_GEMM", "decode_gemm", "hbm"),
    ("NC_KC_DECODE_ATTN", "decode_attn", "hbm"),
    ("NC_KC_PREFILL_GEMM", "prefill_gemm", "mfma"),
    ("NC_KC_PREFILL_ATTN", "prefill_attn", "mfma"),
)
KERNEL_NAMES = {"decode_gemm": "dec_gemm_wide_kernel + dec_reduce4_kernel / dec_gemm_kernel (decode projections)",
                "decode_attn": "attn_decode_kernel (decode attention)",
                "prefill_gemm": "gemm_bf16_kernel / gemm_bf16_comp_kernel (prefill projections)",
                "prefill_attn": "attn_prefill_kernel"}


# HBM-side bytes per launch of a kernel class, from two rocprofv3 counter passes
# (FETCH_SIZE, WRITE_SIZE) scaled by a plain-copy calibration, valid only for the kernel
# sources they were taken with (hash of the listed files); otherwise the report says null.
TRAFFIC = {
    ("d20", "prefill_gemm"): {"bytes_per_launch": 2.5033e+09, "profile": "profiles/d20_pmc_traffic.md",
                             "sources": ('csrc/gemm.hip', 'csrc/common.h', 'csrc/kernels.h'),
                             "sha": "706ed5f8bdd703e1"},
    ("d20", "decode_gemm"): {"bytes_per_launch": 2.0450e+07, "profile": "profiles/d20_pmc_traffic.md",
                             "sources": ('csrc/gemv.hip', 'csrc/rowops.hip', 'csrc/finish.h', 'csrc/common.h', 'csrc/kernels.h'),
                             "sha": "b2c8f44f8b37a5e7"},
    ("d20", "decode_attn"): {"bytes_per_launch": 7.2363e+07, "profile": "profiles/d20_pmc_traffic.md",
                             "sources": ('csrc/attention.hip', 'csrc/common.h', 'csrc/kernels.h'),
                             "sha": "04f7d6c2a87f0269"},
    ("d26", "prefill_gemm"): {"bytes_per_launch": 1.7559e+09, "profile": "profiles/d26_prefill_pmc.md",
                             "sources": ('csrc/gemm.hip', 'csrc/common.h', 'csrc/kernels.h'),
                             "sha": "706ed5f8bdd703e1"},
    ("d30", "decode_attn"): {"bytes_per_launch": 8.5874e+07, "profile": "profiles/d30_decode_pmc_traffic.md",
                             "sources": ('csrc/attention.hip', 'csrc/common.h', 'csrc/kernels.h'),
                             "sha": "04f7d6c2a87f0269"},
    ("d30", "decode_gemm"): {"bytes_per_launch": 4.7364e+07, "profile": "profiles/d30_decode_pmc_traffic.md",
                             "sources": ('csrc/gemv.hip', 'csrc/rowops.hip', 'csrc/finish.h', 'csrc/common.h', 'csrc/kernels.h'),
                             "sha": "b2c8f44f8b37a5e7"},
}


def measured_traffic(workload, name):
    import hashlib
    t = TRAFFIC.get((workload, name))
    if not t:
        return None
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dense_decoder_only_bf16_amd")
    for f in t["sources"]:
        with open(os.path.join(base, f), "rb") as fh:
            h.update(fh.read())
    return t["bytes_per_launch"] if h.hexdigest()[:16] == t["sha"] else None


def roofline(nc, one_step, dtype, workload, classes=None, grade=None):
    """Kernel timing pass: one more full step per kernel class with the library's timing
    mode on (every kernel of the class launched with dispatch-stamped start/stop events on
    its stream; decode launches eager instead of graph replays).  Reports, per class, the
    launches, the average kernel time per launch and the algorithmic GB/s and TFLOP/s.  The
    roofline object is the class `grade` names, or else the class with the largest total
    kernel time."""
    import torch
    res = {}
    for cname, name, bound in CLASSES:
        if classes is not None and name not in classes:
            continue
        nc.nc_timing_enable(getattr(nc, cname))
        one_step(per_decode_step=nc.nc_timing_read)
        torch.cuda.synchronize()
        launches, ms, byts, flops = nc.nc_timing_read()
        if launches == 0:
            continue
        res[name] = {"launches": int(launches), "ms_total": round(ms, 3),
                     "avg_us": round(1000.0 * ms / launches, 3),
                     "GB_per_s": round(byts / (ms * 1e-3) / 1e9, 1),
                     "TFLOP_per_s": round(flops / (ms * 1e-3) / 1e12, 2),
                     "bytes_per_launch": byts / launches, "flops_per_launch": flops / launches,
                     "bound": bound}
    nc.nc_timing_enable(nc.NC_KC_NONE)
    for r in res.values():  # every class against its own roof
        if r["bound"] == "hbm":
            r["frac"] = round(r["GB_per_s"] / HBM_PEAK_GBS, 4)
        else:
            peak = MFMA_BF16_PEAK_TFS if dtype == "bf16" else FP32_VEC_PEAK_TFS
            r["frac"] = round(r["TFLOP_per_s"] / peak, 4)
    dom = grade if grade in res else max(res, key=lambda k: res[k]["ms_total"])
    r = res[dom]
    if r["bound"] == "hbm":
        ach, peak, unit = r["GB_per_s"], HBM_PEAK_GBS, "GB/s"
    else:
        ach, unit = r["TFLOP_per_s"], "TFLOP/s"
        peak = MFMA_BF16_PEAK_TFS if dtype == "bf16" else FP32_VEC_PEAK_TFS
    roof = {"kernel": KERNEL_NAMES[dom], "class": dom, "bound": r["bound"], "achieved": ach,
            "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
            "traffic": measured_traffic(workload, dom),
            "bytes_per_launch": r["bytes_per_launch"],
            "avg_launch_us": r["avg_us"], "launches": r["launches"]}
    return roof, res


def copy_calibration(mib):
    """One plain device-to-device copy of `mib` MiB (torch's copy kernel): the reference
    dispatch whose FETCH_SIZE / WRITE_SIZE counters scale the kernels' counter readings."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4}), flush=True)


def progress(msg):
    """A progress line on stderr (stdout carries only the JSON result)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def run_workload(name, args, cpu=True, roof_classes=None, grade=None):
    """Time one workload: warmup steps, then exactly args.steps steps bracketed by device
    synchronisation; then the kernel-timing pass and, if asked, the oracle on the host.
    Returns the report dict of this workload (its value = its tokens per second)."""
    import torch

    from dense_decoder_only_bf16_amd import nc
    from dense_decoder_only_bf16_amd.inputs import (WORKLOADS, canonical_list, make_extras,
                                                    make_lens, make_tokens, make_weights)

    wl = WORKLOADS[name]
    shape = wl.shape
    Bp, T = wl.prefill_batch, wl.prefill_len
    Bd, steps = wl.decode_batch, wl.decode_steps
    if args.decode_steps is not None and steps:
        steps = args.decode_steps
    shared = Bp > 0 and Bd == Bp  # decode continues the prefilled rows
    progress(f"{name}: drawing weights")
    weights = make_weights(shape, seed=0)
    windows = (nc.layer_windows(wl.window_pattern, shape.n_layer, wl.short_window)
               if wl.window_pattern else None)
    extras = make_extras(shape, seed=wl.extras_seed) if wl.extras_seed >= 0 else None
    model = nc.Model(shape, canonical_list(weights), max_seq=shape.max_seq, windows=windows,
                     extras=extras)
    if not cpu:
        del weights
    stream = torch.cuda.current_stream()
    V = shape.vocab

    kv_p = logits = tokens = None
    if Bp:
        kv_p = model.new_kv(Bp, T + (steps if shared else 0))
        tokens = torch.from_numpy(make_tokens(V, Bp, T, seed=1)).cuda()
        logits = torch.empty((Bp, T, V), device="cuda", dtype=torch.float32)
    kv_d = dlog = tok = ctx = first = None
    if steps:
        dlog = torch.empty((Bd, V), device="cuda", dtype=torch.float32)
        tok = torch.zeros(Bd, device="cuda", dtype=torch.int32)
        if shared:
            kv_d = kv_p
        else:  # decode context built once, outside the timed steps: prefill without logits,
            # then per-row lengths; every step re-truncates to them (exact, by causality)
            C = wl.decode_context
            kv_d = model.new_kv(Bd, C + steps)
            kv_d.prefill(torch.from_numpy(make_tokens(V, Bd, C, seed=1)).cuda(), None, stream)
            ctx = (make_lens(Bd, 256, C, seed=2) if wl.mixed_lengths
                   else np.full(Bd, C, dtype=np.int32))
            kv_d.set_lens(ctx)
            first = torch.from_numpy(make_tokens(V, 1, Bd, seed=3)[0]).cuda()
    zeros = np.zeros(max(Bp, 1), dtype=np.int32)
    u_all = None
    if steps and wl.temperature > 0:  # one uniform per row and step, drawn untimed
        u_all = torch.from_numpy(np.random.default_rng(4).random((steps, Bd)).astype(np.float32)).cuda()

    def one_step(ev=None, per_decode_step=None):
        if ev:
            ev[0].record(stream)
        if Bp:
            kv_p.set_lens(zeros[:Bp])
            kv_p.prefill(tokens, logits, stream)
            if shared:  # greedy pick from each row's last prompt position
                for b in range(Bp):
                    nc.nc_argmax(logits[b, T - 1], 1, V, tok[b:b + 1], stream)
        if ev:
            ev[1].record(stream)
        if steps:
            if not shared:
                kv_d.set_lens(ctx)
                tok.copy_(first)
            for s in range(steps):
                if u_all is None:  # decode step and greedy pick in one graph
                    kv_d.decode_greedy(tok, dlog, tok, stream)
                else:
                    kv_d.decode(tok, dlog, stream)
                    nc.nc_sample(dlog, Bd, V, wl.temperature, wl.top_k, u_all[s], tok, stream)
                if per_decode_step:
                    per_decode_step()
        if ev:
            ev[2].record(stream)

    progress(f"{name}: model on the GPU, {args.warmup} warmup steps")
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    progress(f"{name}: {args.steps} timed steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    dec_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    ms_per_step = wall * 1000.0 / args.steps
    n_pre, n_dec = Bp * T, Bd * steps
    kvh = f"{shape.n_kv_head} K/V head" + ("s" if shape.n_kv_head > 1 else "")
    win = (f", windows {wl.window_pattern} with {wl.short_window}-key short windows"
           if wl.window_pattern else "")
    if extras is not None:
        win += (f", value embeddings on layers {sorted(extras['ve'])}, residual lambdas, smear, "
                f"backout at layer {extras['backout_layer']}")
    desc = (f"{name} ({shape.n_layer} layers, d {shape.d_model}, {shape.n_head}x"
            f"{shape.head_dim} query heads, {kvh}, MLP {shape.d_ff}, vocab {V}, "
            f"{shape.dtype}{win}):")
    if Bp:
        desc += f" prefill {Bp}x{T} with fp32 logits at every position"
    if steps:
        ctxd = ("the prefilled rows" if shared else
                (f"context lengths U{{256..{wl.decode_context}}} (built untimed)" if wl.mixed_lengths
                 else f"context {wl.decode_context} (built untimed)"))
        pick = (f"sampled (temperature {wl.temperature}, top-{wl.top_k})" if wl.temperature > 0
                else "greedy")
        desc += (", then" if Bp else "") + f" {steps} {pick} decode steps of {Bd} rows from {ctxd}"
    out = {"value": round((n_pre + n_dec) / (ms_per_step / 1000.0), 1), "unit": "tokens/s",
           "ms_per_step": round(ms_per_step, 3),
           "config": {"workload": desc, "prefill_batch": Bp, "prefill_len": T,
                      "decode_batch": Bd, "decode_steps": steps}}
    if Bp:
        out["prefill_ms"] = round(pre_ms, 3)
        out["prefill_tokens_per_s"] = round(n_pre / (pre_ms / 1000.0), 1)
    if steps:
        out["decode_ms"] = round(dec_ms, 3)
        out["decode_tokens_per_s"] = round(n_dec / (dec_ms / 1000.0), 1)
    if not args.no_roofline:
        progress(f"{name}: kernel-timing pass")
        out["roofline"], out["kernels"] = roofline(nc, one_step, shape.dtype, name,
                                                   roof_classes, grade)
    if cpu and not args.no_cpu:
        progress(f"{name}: oracle on the host cores")
        out["cpu_baseline"] = cpu_baseline(shape, weights, wl, args.cpu_seconds, windows, extras)
    for kv in {id(k): k for k in (kv_p, kv_d) if k is not None}.values():
        kv.close()
    model.close()
    del logits, dlog, tokens
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# Runs reported beside the default line: (workload, kernel classes timed, class graded).
EXTRA = (("d26", ("prefill_gemm", "prefill_attn"), "prefill_gemm"),
         ("d30", ("decode_attn", "decode_gemm"), "decode_attn"))


def main():
    args = parse()
    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(batch rows are independent, so more GPUs would each run their own rows).",
              file=sys.stderr)
        sys.exit(2)
    from dense_decoder_only_bf16_amd.inputs import WORKLOADS
    if args.workload not in WORKLOADS:
        print(f"unknown workload {args.workload}; one of {sorted(WORKLOADS)}", file=sys.stderr)
        sys.exit(2)
    from dense_decoder_only_bf16_amd import nc

    main_run = run_workload(args.workload, args)
    out = {
        "metric": "prefill tokens/s + decode tokens/s (1 GPU); % MFMA peak / % HBM BW",
        "value": main_run.pop("value"),
        "unit": main_run.pop("unit"),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": main_run.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": WORKLOADS[args.workload].shape.dtype, "data": "synthetic",
        "config": main_run.pop("config"),
    }
    cpu = main_run.pop("cpu_baseline", None)
    out.update(main_run)
    if args.workload == "d20" and not args.no_extra:
        for name, classes, grade in EXTRA:
            r = run_workload(name, args, cpu=False, roof_classes=classes, grade=grade)
            r["graded"] = grade
            out[name] = r
        # the two targets side by side: prefill products vs MFMA peak, decode attention vs HBM
        targets = {}
        for name, cls, need in (("d20", "prefill_gemm", 0.60), ("d26", "prefill_gemm", 0.60),
                                ("d20", "decode_attn", 0.70), ("d30", "decode_attn", 0.70)):
            k = (out if name == "d20" else out.get(name, {})).get("kernels", {}).get(cls)
            if k:
                targets[f"{name}_{cls}"] = {"frac": k["frac"], "target": need}
        out["targets"] = targets
    if not args.no_roofline:
        # what this GPU sustains with plain kernels, beside the published peaks
        rnd = nc.nc_diag_mfma_rate(True)
        const = nc.nc_diag_mfma_rate(False)
        hbm = nc.nc_diag_hbm_read_rate()
        out["sustained"] = {
            "mfma_bf16_random_operands_tflops": round(rnd, 1),
            "mfma_bf16_constant_operands_tflops": round(const, 1),
            "hbm_read_stream_tbps": round(hbm, 3),
            "roofline_frac_of_sustained": round(
                out["roofline"]["achieved"] / (rnd if out["roofline"]["unit"] == "TFLOP/s" else hbm * 1000.0), 4),
        }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
