"""Benchmark of the nanochat GPT forward on one MI355X through libnc.so.

One step = the whole hot path over one batch: prefill of B x T prompt tokens with fp32
logits at every position, then `decode_steps` greedy decode steps (argmax fed back), on the
d12 bf16 model (12 layers, d=768, 6x128 heads, one K/V head, MLP 3072, vocab 65536) with
seeded N(0, 0.02) weights and uniform random token ids.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload d12|d20|d30|tiny] [--no-cpu]
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
    p.add_argument("--workload", default="d12")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    return p.parse_args()


def cpu_baseline(shape, weights, wl, budget_s):
    """Time the fp64 oracle on the host on a bounded sample of the same workload.

    Sample: one row; prefill of min(T, 2048) tokens, then greedy decode steps until the
    time budget is spent.  The per-phase rates are combined with the workload's own mix of
    prefill and decode tokens into one tokens/s figure."""
    from oracle import OracleModel
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    from dense_decoder_only_bf16_amd.inputs import make_tokens
    orc = OracleModel(shape, weights)
    t_pre = min(wl.prefill_len, 2048)
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
    value = (n_pre + n_dec) / (n_pre / pre_rate + n_dec / dec_rate)
    return {"value": round(value, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 numpy oracle, 1 row: prefill {t_pre} tokens ({t1 - t0:.1f} s, "
                       f"{pre_rate:.1f} tok/s) + {steps} greedy decode steps at context "
                       f"{t_pre} ({t3 - t2:.1f} s, {dec_rate:.2f} tok/s); combined with the "
                       f"workload's mix of {n_pre} prefill and {n_dec} decode tokens"),
            "prefill_tokens_per_s": round(pre_rate, 2), "decode_tokens_per_s": round(dec_rate, 3)}


HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6  # MI355X dense bf16 matrix peak


def roofline(nc, one_step, steps, stream):
    """Time the decode and prefill projection kernels with HIP events around every launch
    (library timing mode; graph event nodes for decode) over one more full step, and report
    the roofline of the one that takes longer.  Decode projections are HBM-bound (bytes:
    weights + activations + outputs, each once); prefill projections are MFMA-bound."""
    import torch
    res = {}
    for cls, name in ((nc.NC_KC_DECODE_GEMM, "decode_gemm"), (nc.NC_KC_PREFILL_GEMM, "prefill_gemm")):
        nc.nc_timing_enable(cls)
        one_step(per_step=lambda: nc.nc_timing_read())
        torch.cuda.synchronize()
        launches, ms, byts, flops = nc.nc_timing_read()
        res[name] = {"launches": int(launches), "ms_total": round(ms, 3),
                     "avg_us": round(1000.0 * ms / max(launches, 1), 3),
                     "GB_per_s": round(byts / (ms * 1e-3) / 1e9, 1) if ms > 0 else None,
                     "TFLOP_per_s": round(flops / (ms * 1e-3) / 1e12, 1) if ms > 0 else None}
    nc.nc_timing_enable(nc.NC_KC_NONE)
    dom = max(res, key=lambda k: res[k]["ms_total"])
    r = res[dom]
    if dom == "decode_gemm":
        roof = {"kernel": "dec_gemm_kernel (decode projections)", "bound": "hbm",
                "achieved": r["GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(r["GB_per_s"] / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        roof = {"kernel": "gemm_bf16_kernel (prefill projections)", "bound": "mfma",
                "achieved": r["TFLOP_per_s"], "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(r["TFLOP_per_s"] / MFMA_BF16_PEAK_TFS, 4), "traffic": None}
    return roof, res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(batch rows are independent, so more GPUs would each run their own rows).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from dense_decoder_only_bf16_amd import nc
    from dense_decoder_only_bf16_amd.inputs import WORKLOADS, canonical_list, make_tokens, make_weights

    wl = WORKLOADS[args.workload]
    shape = wl.shape
    if wl.prefill_batch == 0 or wl.decode_steps == 0 or wl.decode_batch != wl.prefill_batch:
        print("bench.py times workloads that prefill and then decode the same batch "
              "(tiny, d12)", file=sys.stderr)
        sys.exit(2)
    B, T, steps = wl.prefill_batch, wl.prefill_len, wl.decode_steps
    max_seq = T + steps
    weights = make_weights(shape, seed=0)
    model = nc.Model(shape, canonical_list(weights), max_seq=shape.max_seq)
    kv = model.new_kv(B, max_seq)
    stream = torch.cuda.current_stream()
    tokens = torch.from_numpy(make_tokens(shape.vocab, B, T, seed=1)).cuda()
    logits = torch.empty((B, T, shape.vocab), device="cuda", dtype=torch.float32)
    dlog = torch.empty((B, shape.vocab), device="cuda", dtype=torch.float32)
    tok = torch.empty(B, device="cuda", dtype=torch.int32)
    zeros = np.zeros(B, dtype=np.int32)

    def one_step(ev=None, per_step=None):
        kv.set_lens(zeros)
        if ev:
            ev[0].record(stream)
        kv.prefill(tokens, logits, stream)
        for b in range(B):  # greedy pick from each row's last prompt position
            nc.nc_argmax(logits[b, T - 1], 1, shape.vocab, tok[b:b + 1], stream)
        if ev:
            ev[1].record(stream)
        for _ in range(steps):
            kv.decode(tok, dlog, stream)
            nc.nc_argmax(dlog, B, shape.vocab, tok, stream)
            if per_step:
                per_step()
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
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
    n_tok = B * T + B * steps
    out = {
        "metric": "prefill tokens/s + decode tokens/s (1 GPU); % MFMA peak / % HBM BW",
        "value": round(n_tok / (ms_per_step / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": shape.dtype, "data": "synthetic",
        "config": {"workload": (f"{args.workload} ({shape.n_layer} layers, d {shape.d_model}, "
                                f"{shape.n_head}x{shape.head_dim} query heads, 1 K/V head, MLP "
                                f"{shape.d_ff}, vocab {shape.vocab}, {shape.dtype}): prefill "
                                f"{B}x{T} with fp32 logits at every position, then {steps} "
                                f"greedy decode steps of {B} rows"),
                   "batch": B, "prefill_len": T, "decode_steps": steps},
        "prefill_ms": round(pre_ms, 3), "decode_ms": round(dec_ms, 3),
        "prefill_tokens_per_s": round(B * T / (pre_ms / 1000.0), 1),
        "decode_tokens_per_s": round(B * steps / (dec_ms / 1000.0), 1),
    }
    out["roofline"], out["kernels"] = roofline(nc, one_step, steps, stream)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(shape, weights, wl, args.cpu_seconds)
    kv.close()
    model.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
