#!/usr/bin/env python3
"""Throughput of the DFlash drafter's hot path on one MI355X.

A step is one pass of the whole hot path over one batch: the context append of the rows
a propose round commits (fc + hidden_norm, per-layer K/V with k_norm + RoPE, page
allocation and writeback; `--append-rows`, default 16 = a fully accepted gamma=16 block)
followed by one gamma=16 block forward (embedding, every layer, final norm, lm_head +
argmax). Workload: the 8-layer, hidden-2048, GQA 32:4, head_dim-128, ff-6144,
vocab-151936 drafter with 5 taps of hidden 2048, one sequence whose context is
prefilled (untimed) with 4096 rows of N(0,1) hidden states; weights N(0,0.02) bf16
from seed. Inputs are resident in HBM before the timed region.

Prints one JSON line on stdout: blocks/s (value, from a timed region of plain launches),
tokens/s, the roofline of the dominant kernel class (its launches bracketed by
dispatch-attached HIP events over a second timed region of the same length, since the
events themselves slow the step), a per-class breakdown, a 16-sequence batched line, and
the CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "drafted γ=16 blocks/sec at batch 1 and 16; achieved HBM GB/s vs peak"
WORKLOAD = "qwen3-L8-h2048-ctx4096-b1"
WORKLOAD_B16 = "qwen3-L8-h2048-b16-ctx512to8192"
WORKLOAD_LONG = "qwen3-L8-h2048-b32-ctx8192to32768-append2048"
WORKLOAD_WIDE = "wide-L5-h5376-yarn-swa2048-ctx16384-b1"
WORKLOAD_TINY = "tiny-L2-h256-ctx64-b1"
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_bytes(m, M, fp8=False):
    """Algorithmic HBM bytes of the forward's weight-streaming GEMMs for M block rows:
    each weight byte once (FP8: one byte a weight and a 4-byte scale a row), the bf16
    activation in, the fp32 result out."""
    h, hd, nh, nkv, ff = m["hidden"], m["head_dim"], m["num_q_heads"], m["num_kv_heads"], m["intermediate"]
    qd, kvd = nh * hd, nkv * hd
    shapes = [(qd + 2 * kvd, h), (h, qd), (2 * ff, h), (h, ff)]
    wb = (lambda N, K: N * K + 4 * N) if fp8 else (lambda N, K: N * K * 2)
    per_layer = sum(wb(N, K) + M * K * 2 + M * N * 4 for N, K in shapes)
    return per_layer * m["num_layers"]


# HBM bytes per launch of the forward's layer GEMMs (k_gemm_split, mean over
# the QKV, O, gate/up and down shapes), from `rocprofv3 --pmc FETCH_SIZE` and
# `--pmc WRITE_SIZE` runs of `bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-batch16
# --no-longctx --no-fp8 --no-dspark --no-dflash2 --no-wide`, scaled by what the same counters read for
# 20 plain 256 MiB device copies (`bench.py --calibrate-copy 256`: FETCH_SIZE 0.500 of the
# bytes read, WRITE_SIZE 1.000 of the bytes written). Valid only for the kernel source they
# were taken on.
TRAFFIC = {
    "gemm": dict(source="block_diffusion_draft_02_amd/csrc/k_gemm.hip",
                 sha256="44617ab29dc69c5bc9f5e49c4970ef7a25b300b0908646e0415cdde03a2ab183",
                 fetch_bytes=30.19e6, write_bytes=3.540e6),
}


def measured_traffic(kind):
    import hashlib
    t = TRAFFIC.get(kind)
    if t is None:
        return None
    try:
        with open(os.path.join(ROOT, t["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != t["sha256"]:
                return None
    except OSError:
        return None
    return int(t["fetch_bytes"] + t["write_bytes"])


def gemm_weight_elems(m):
    h, hd, nh, nkv, ff = m["hidden"], m["head_dim"], m["num_q_heads"], m["num_kv_heads"], m["intermediate"]
    qd, kvd = nh * hd, nkv * hd
    return ((qd + 2 * kvd) * h + h * qd + 2 * ff * h + h * ff) * m["num_layers"]


def markov_bytes(m, n_bands, gamma):
    """Algorithmic bytes of a DSpark chain: per drafted row, W2 [V, R] bf16 once for all
    bands, each band's logits row read and W1 row gathered."""
    V, R = m["vocab"], m["markov_rank"]
    return (gamma - 1) * (V * R * 2 + n_bands * (V * 4 + R * 2))


def lmhead_bytes(m, M, fp8=False):
    w = m["vocab"] * (m["hidden"] + 4) if fp8 else m["vocab"] * m["hidden"] * 2
    return w + M * m["hidden"] * 2


def attn_bytes(m, kv_lens, gamma):
    """K and V bytes the layers read: per band, the keys visible to the block (every key, C +
    gamma, in full-attention layers; in sliding layers the keys within the window of block
    row 0, min(C, W - 1) context keys + gamma, with default positions), both halves, all kv
    heads."""
    kvd = m["num_kv_heads"] * m["head_dim"]
    win = int(m.get("sliding_window") or 0)
    sl = m.get("layer_sliding") or [False] * m["num_layers"]
    keys = 0
    for l in range(m["num_layers"]):
        for c in kv_lens:
            keys += (min(c, win - 1) if (win and sl[l]) else c) + gamma
    return keys * kvd * 2 * 2


def forward_bytes(m, kv_lens, gamma):
    """Algorithmic bytes of one forward: every weight once (layers, lm_head, the touched
    embedding rows) and the K/V of every visible key, per layer."""
    h, hd, nh, nkv, ff = m["hidden"], m["head_dim"], m["num_q_heads"], m["num_kv_heads"], m["intermediate"]
    qd, kvd = nh * hd, nkv * hd
    layer_w = ((qd + 2 * kvd) * h + h * qd + 2 * ff * h + h * ff) * 2 + (2 * h + 2 * hd) * 2
    return (layer_w * m["num_layers"] + m["vocab"] * h * 2 + h * 2
            + attn_bytes(m, kv_lens, gamma) + len(kv_lens) * 2 * h * 2)


def append_bytes(m, n):
    h, kvd, L = m["hidden"], m["num_kv_heads"] * m["head_dim"], m["num_layers"]
    return (h * m["num_taps"] * m["target_hidden"] * 2 + L * 2 * kvd * h * 2
            + n * m["num_taps"] * m["target_hidden"] * 2 + n * L * 2 * kvd * 2)


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"]), info[0].get("internal_api", "blas")
    except Exception:
        pass
    return len(os.sched_getaffinity(0)), "unknown"


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_steps(step, budget_s, n_max):
    """Run step(i) until budget_s seconds of it have run (at least once, at most n_max)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        step(n)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= n_max:
            return n, el


def cpu_baseline_config(name, m, W, dtype, budget_s, a, gamma, H_app=None):
    """The oracle as it stands on this host for one workload and precision: an untimed prefill
    of the workload's contexts (seeded draws) and weight widening, then timed steps. A step is
    what the GPU line times: an `a`-row context append per sequence (the batched append for
    the 16-band workload) and one gamma-block forward over every sequence; for the long-context
    workload, one sequence's 2048-row append and its block forward."""
    import numpy as np

    import synth
    from oracle import dflash_oracle as O
    w = synth.workload(name)
    seed, nb = w["seed"], w["batch"]
    lens = synth.gen_ctx_lengths(w["ctx"][0], w["ctx"][1], nb, seed)
    t_setup = time.perf_counter()
    if name == WORKLOAD_LONG:
        nb = 1   # one sequence of the workload, labelled per sequence
    max_seq = int(lens[:nb].max()) + 64 * a + 2048 + gamma + 16
    eng = O.Engine(m, W, max_seq, nb, dtype=dtype)
    for s in range(nb):
        for c, r0 in enumerate(range(0, int(lens[s]), 2048)):
            eng.ctx_kv_append(s, synth.gen_hidden(m, seed, min(2048, int(lens[s]) - r0), 1000 * s + c))
    for n_, _, _ in synth.weight_specs(m):
        if n_ != "embed_tokens":
            eng.d.w(n_)
    setup_s = time.perf_counter() - t_setup
    seqs = list(range(nb))
    bonus = synth.gen_bonus(m, seed, 64 * nb, index=5)
    if name == WORKLOAD_LONG:
        Hl = synth.gen_hidden(m, seed, w["append"], 999)

        def step(i):
            eng.ctx_kv_append(0, Hl)
            eng.block_forward([0], [int(bonus[i])], gamma=gamma)
        n, el = _oracle_steps(step, budget_s, 1)
        unit, value = "sequences/s", n / el
        what = (f"one sequence of the workload (context {int(lens[0])}): its 2048-row append and one block "
                f"forward per step")
    else:
        Hs = synth.gen_hidden(m, seed, 64 * nb * a, 7)

        def step(i):
            rows = Hs[i * nb * a:(i + 1) * nb * a]
            if nb > 1:
                eng.ctx_kv_append_batch(seqs, [a] * nb, rows)
            else:
                eng.ctx_kv_append(0, rows)
            eng.block_forward(seqs, [int(b) for b in bonus[i * nb:(i + 1) * nb]], gamma=gamma)
        n, el = _oracle_steps(step, budget_s, 64)
        unit, value = "blocks/s", n * nb / el
        what = f"{n} steps ({a}-row append per sequence + one {nb}-band gamma={gamma} forward)"
    return dict(workload=name, dtype=np.dtype(dtype).name, value=round(value, 4), unit=unit, steps=n,
                seconds=round(el, 3), setup_seconds=round(setup_s, 1), sample=what)


def run_cpu_baseline(configs, budget_s, a, gamma):
    """The oracle on every workload in float64 (its parity mode) and float32; `configs` maps a
    workload name to (model, weights). The headline entry is the batch-1 workload in float64."""
    import numpy as np
    thr, api = blas_threads()
    entries = []
    for name, (m, W) in configs.items():
        for dt in (np.float64, np.float32):
            e = cpu_baseline_config(name, m, W, dt, budget_s, a, gamma)
            log(f"[bench] cpu oracle {name} {e['dtype']}: {e['value']} {e['unit']} "
                f"({e['seconds']} s timed, {e['setup_seconds']} s setup)")
            entries.append(e)
    head = next(e for e in entries if e["workload"] == WORKLOAD and e["dtype"] == "float64")
    return dict(value=head["value"], unit="blocks/s", cores=thr, kind="oracle",
                sample=f"{head['sample']} of {WORKLOAD} after an untimed prefill of its context and weight "
                       f"widening; numpy float64, BLAS={api} on {thr} threads; host CPU: {cpu_model()}",
                seconds=head["seconds"], by_config=entries)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--append-rows", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="timed budget of the oracle baseline, per workload and precision")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-quick", action="store_true", help="oracle baseline on the batch-1 workload only")
    ap.add_argument("--no-wide", action="store_true", help="skip the wide-drafter line")
    ap.add_argument("--no-batch16", action="store_true")
    ap.add_argument("--no-longctx", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 E4M3 weight-only lines")
    ap.add_argument("--no-dspark", action="store_true", help="skip the DSpark Markov-head lines")
    ap.add_argument("--no-dflash2", action="store_true", help="skip the DFlash2 lines")
    ap.add_argument("--longctx-only", action="store_true",
                    help="only run the 32-sequence long-context section and print its JSON (for counter runs)")
    ap.add_argument("--batch16-only", action="store_true",
                    help="only run the 16-sequence batched section and print its JSON (for counter runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 20 plain device-to-device copies of MIB MiB (the reference for "
                         "scaling the HBM traffic counters) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 20}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path would shard data-parallel over sequences, each GPU serving its own bands)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from block_diffusion_draft_02_amd import binding as B

    dev = torch.device("cuda:0")
    w = synth.workload(WORKLOAD)
    m = w["model_cfg"]
    gamma = m["gamma_max"]
    a = args.append_rows
    ctx = w["ctx"][0]
    total = args.warmup + 2 * args.steps + 8
    t = time.perf_counter()
    W = synth.gen_weights(m, w["seed"])
    H_ctx = synth.gen_hidden(m, w["seed"], ctx, 0)
    H_steps = synth.gen_hidden(m, w["seed"], total * a, 1)
    bonus = synth.gen_bonus(m, w["seed"], total)
    log(f"[bench] inputs generated in {time.perf_counter() - t:.1f}s")

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    Wd = {k: to_dev(v) for k, v in W.items()}
    if args.longctx_only:
        print(json.dumps(bench_longctx(m, Wd, gamma, B, torch, np, synth, to_dev)), flush=True)
        return
    if args.batch16_only:
        print(json.dumps(bench_batch16(m, Wd, gamma, a, args, B, torch, np, synth, to_dev)), flush=True)
        return
    max_seq = ctx + total * a + gamma + 16
    d = B.Drafter(m, Wd, max_seq, 1)
    d.dflash_ctx_kv_append(0, to_dev(H_ctx))
    Hs = to_dev(H_steps)
    toks = torch.empty((1, gamma - 1), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    step_i = [0]

    def step():
        i = step_i[0]
        d.dflash_ctx_kv_append(0, Hs[i * a:(i + 1) * a])
        d.dflash_block_forward([0], [int(bonus[i])], toks, gamma=gamma)
        step_i[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-class breakdown on a few untimed steps (every launch bracketed by events)
    d.dflash_timing(list(B.K_CLASSES))
    nb = 4
    for _ in range(nb):
        step()
    torch.cuda.synchronize()
    br = d.dflash_timing_read()
    d.dflash_timing([])
    breakdown = {k: dict(ms_per_step=v[0] / nb, launches_per_step=v[1] / nb) for k, v in br.items() if v[1]}
    dominant = max(breakdown, key=lambda k: breakdown[k]["ms_per_step"])
    log("[bench] breakdown (ms/step): " + ", ".join(f"{k}={v['ms_per_step']:.4f}" for k, v in breakdown.items()))

    # the timed region: plain launches, nothing bracketed
    kv0 = d.dflash_seq_info(0)[0]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    el = t1 - t0
    ms_step = el / args.steps * 1e3
    blocks = args.steps / el
    M = gamma
    mean_kv = kv0 + a * (args.steps + 1) / 2

    # the roofline pass: the same number of steps right after, every launch bracketed by
    # dispatch-attached HIP events on the launch stream (bracketing only the dominant class
    # would slow exactly those launches); the dominant class's average is the roofline's
    kv1 = d.dflash_seq_info(0)[0]
    d.dflash_timing(list(B.K_CLASSES))
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    dom = d.dflash_timing_read()[dominant]
    d.dflash_timing([])
    mean_kv1 = kv1 + a * (args.steps + 1) / 2
    dom_bytes_step = {"gemm": gemm_bytes(m, M), "lmhead": lmhead_bytes(m, M),
                      "attn": attn_bytes(m, [mean_kv1], gamma)}.get(dominant)
    roofline = None
    if dom_bytes_step is not None and dom[1]:
        launches_per_step = dom[1] / args.steps
        avg_ms = dom[0] / dom[1]
        per_launch = dom_bytes_step / launches_per_step
        achieved = per_launch / (avg_ms * 1e-3) / 1e9
        roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(dominant),
                        kernel_class=dominant,
                        avg_launch_us=round(avg_ms * 1e3, 3), launches_per_step=launches_per_step,
                        algorithmic_bytes_per_launch=int(per_launch),
                        pass_ms_per_step=round((t3 - t2) / args.steps * 1e3, 4))
    step_bytes = forward_bytes(m, [mean_kv], gamma) + append_bytes(m, a)
    log(f"[bench] {blocks:.1f} blocks/s, {ms_step:.3f} ms/step, whole-step {step_bytes / (ms_step * 1e-3) / 1e9:.0f} GB/s")

    out = {
        "metric": METRIC, "value": round(blocks, 2), "unit": "blocks/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": 1, "ctx": ctx, "gamma": gamma,
                   "append_rows_per_step": a, "layers": m["num_layers"], "hidden": m["hidden"],
                   "vocab": m["vocab"]},
        "tokens_per_s": round(blocks * (gamma - 1), 1),
        "step_algorithmic_bytes": int(step_bytes),
        "step_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "roofline": roofline,
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in breakdown.items()},
    }
    d.close()

    if not args.no_batch16:
        out["batch16"] = bench_batch16(m, Wd, gamma, a, args, B, torch, np, synth, to_dev)
    if not args.no_longctx:
        out["longctx"] = bench_longctx(m, Wd, gamma, B, torch, np, synth, to_dev)
    if not args.no_fp8:
        mf = dict(m, weight_format="fp8")
        out["fp8"] = dict(batch1=bench_variant_b1(mf, "fp8", Wd, H_ctx, H_steps, bonus, a, gamma, args, B, torch,
                                                  to_dev))
        if not args.no_batch16:
            out["fp8"]["batch16"] = bench_batch16(mf, Wd, gamma, a, args, B, torch, np, synth, to_dev)
    if not args.no_dspark:
        # the same trunk with a rank-256 Markov head (its two tables drawn from the same seed)
        md = synth.model("qwen3-L8-h2048-dspark")
        Wdd = dict(Wd, **{k: to_dev(synth.gen_weight(md, w["seed"], k)) for k in ("markov_w1", "markov_w2")})
        out["dspark"] = dict(batch1=bench_variant_b1(md, "dspark", Wdd, H_ctx, H_steps, bonus, a, gamma, args, B,
                                                     torch, to_dev))
        if not args.no_batch16:
            out["dspark"]["batch16"] = bench_batch16(md, Wdd, gamma, a, args, B, torch, np, synth, to_dev)
        del Wdd
    if not args.no_dflash2:
        # the same trunk with DFlash2's convs and candidate selector (their tensors drawn from
        # the same seed)
        m2 = synth.model("qwen3-L8-h2048-dflash2")
        extra = [n for n, _, _ in synth.weight_specs(m2) if "_conv_" in n or n.startswith("selector")]
        Wd2 = dict(Wd, **{k: to_dev(synth.gen_weight(m2, w["seed"], k)) for k in extra})
        out["dflash2"] = dict(batch1=bench_variant_b1(m2, "dflash2", Wd2, H_ctx, H_steps, bonus, a, gamma, args, B,
                                                      torch, to_dev))
        if not args.no_batch16:
            out["dflash2"]["batch16"] = bench_batch16(m2, Wd2, gamma, a, args, B, torch, np, synth, to_dev)
        del Wd2

    W_wide = None
    if not args.no_wide:
        del Wd
        out["wide"], W_wide = bench_wide(a, args, B, torch, np, synth, to_dev)
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        configs = {WORKLOAD_TINY: None, WORKLOAD: (m, W), WORKLOAD_B16: (m, W), WORKLOAD_LONG: (m, W)}
        mt = synth.model("tiny-L2-h256")
        configs[WORKLOAD_TINY] = (mt, synth.gen_weights(mt, synth.workload(WORKLOAD_TINY)["seed"]))
        if W_wide is not None:
            configs[WORKLOAD_WIDE] = (synth.model("wide-L5-h5376-yarn-swa2048"), W_wide)
        if args.cpu_quick:
            configs = {WORKLOAD: configs[WORKLOAD]}
        out["cpu_baseline"] = run_cpu_baseline(configs, args.cpu_seconds, a, gamma)
    print(json.dumps(out), flush=True)


def bench_variant_b1(mv, label, Wd, H_ctx, H_steps, bonus, a, gamma, args, B, torch, to_dev):
    """The batch-1 step of a variant of the drafter (`mv`: the model with FP8 E4M3 trunk
    weights, a DSpark Markov head, or DFlash2's convs and selector): the same inputs, plain
    launches timed, then one
    pass with every launch bracketed for the per-class times and the stream rates of the
    classes the variant changes."""
    steps = args.steps
    total = args.warmup + 2 * steps + 8
    ctx = H_ctx.shape[0]
    d = B.Drafter(mv, Wd, ctx + total * a + gamma + 16, 1)
    d.dflash_ctx_kv_append(0, to_dev(H_ctx))
    Hs = to_dev(H_steps)
    toks = torch.empty((1, gamma - 1), dtype=torch.int32, device="cuda:0")
    step_i = [0]

    def step():
        i = step_i[0]
        d.dflash_ctx_kv_append(0, Hs[i * a:(i + 1) * a])
        d.dflash_block_forward([0], [int(bonus[i])], toks, gamma=gamma)
        step_i[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    d.dflash_timing(list(B.K_CLASSES))
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    br = d.dflash_timing_read()
    d.dflash_timing([])
    d.close()
    blocks = steps / el
    ms = {k: v[0] / steps for k, v in br.items() if v[1]}
    fp8 = mv.get("weight_format") == "fp8"
    streams = []
    if fp8:
        streams += [("gemm", gemm_bytes(mv, gamma, fp8=True)), ("lmhead", lmhead_bytes(mv, gamma, fp8=True))]
    if mv.get("markov_rank", 0):
        streams.append(("markov", markov_bytes(mv, 1, gamma)))
    rates = {}
    for k, nbytes in streams:
        if k in ms:
            rates[k] = dict(algorithmic_bytes_per_step=int(nbytes), gbs=round(nbytes / (ms[k] * 1e-3) / 1e9, 1),
                            frac=round(nbytes / (ms[k] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    if "markov" in br and br["markov"][1]:
        rates["markov"]["avg_launch_us"] = round(br["markov"][0] / br["markov"][1] * 1e3, 3)
    log(f"[bench] {label} batch1: {blocks:.1f} blocks/s, {el / steps * 1e3:.3f} ms/step; "
        + ", ".join(f"{k} {v['gbs']:.0f} GB/s" for k, v in rates.items()))
    return dict(workload=WORKLOAD, variant=label, value=round(blocks, 2), unit="blocks/s",
                steps=steps, ms_per_step=round(el / steps * 1e3, 4), tokens_per_s=round(blocks * (gamma - 1), 1),
                kernels_ms_per_step={k: round(v, 4) for k, v in ms.items()}, streams=rates,
                timing="value from plain launches; per-class times from a second, bracketed pass")


def bench_batch16(m, Wd, gamma, a, args, B, torch, np, synth, to_dev):
    """16 sequences with contexts U[512, 8192] on a shared pool with permuted pages; a step
    appends `a` rows to every sequence in one batched append (the batched context
    precompute) and runs one 16-band forward. Same weights as the batch-1 line (the shapes,
    not the draws, set the cost). Also times the batched append alone against the same rows
    appended sequence by sequence."""
    w = synth.workload(WORKLOAD_B16)
    nb = w["batch"]
    dev = torch.device("cuda:0")
    lens = synth.gen_ctx_lengths(w["ctx"][0], w["ctx"][1], nb, w["seed"])
    steps = max(5, args.steps // 2)
    # warmup, the plain timed steps, then as many bracketed by events for the breakdown
    total = args.warmup + 2 * steps
    app_reps = 10
    max_seq = int(lens.max()) + (total + 2 * app_reps) * a + gamma + 16
    per_seq = -(-(max_seq + gamma + 1) // 16)
    order = synth.gen_page_order(per_seq * nb, w["seed"])
    d = B.Drafter(m, Wd, max_seq, nb, page_order=order)
    for s in range(nb):
        d.dflash_ctx_kv_append(s, to_dev(synth.gen_hidden(m, w["seed"], int(lens[s]), s)))
    # per step, the rows of all sequences one after another (as the batched call takes them)
    Hb = to_dev(synth.gen_hidden(m, w["seed"], (total + 2 * app_reps) * nb * a, 100))
    bonus = synth.gen_bonus(m, w["seed"], nb * total)
    toks = torch.empty((nb, gamma - 1), dtype=torch.int32, device=dev)
    seqs = list(range(nb))
    batched = nb * a <= 256

    def append(i, per_seq_loop=False):
        rows = Hb[i * nb * a:(i + 1) * nb * a]
        if batched and not per_seq_loop:
            d.dflash_ctx_kv_append_batch(seqs, [a] * nb, rows)
        else:
            for j, s in enumerate(seqs):
                d.dflash_ctx_kv_append(s, rows[j * a:(j + 1) * a])

    def step(i):
        append(i)
        d.dflash_block_forward(seqs, bonus[i * nb:(i + 1) * nb], toks, gamma=gamma)

    for i in range(args.warmup):
        step(i)
    # the rate from plain launches (events attached to launches slow them down), the per-class
    # breakdown from a second pass of as many steps with every launch class bracketed
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    d.dflash_timing(list(B.K_CLASSES))
    t0 = time.perf_counter()
    for i in range(steps):
        step(args.warmup + steps + i)
    torch.cuda.synchronize()
    el_br = time.perf_counter() - t0
    br = d.dflash_timing_read()
    d.dflash_timing([])
    # the append alone: one batched call against the sequence-by-sequence loop, same rows
    app = {}
    for mode, first in (("batched", total), ("per_seq", total + app_reps)):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for r in range(app_reps):
            append(first + r, per_seq_loop=(mode == "per_seq"))
        torch.cuda.synchronize()
        app[mode] = (time.perf_counter() - t1) / app_reps * 1e3
    d.close()
    blocks = nb * steps / el
    wbytes = 1 if m.get("weight_format") == "fp8" else 2
    variant = ("fp8" if wbytes == 1 else "dspark" if m.get("markov_rank", 0) else
               "dflash2" if m.get("selector_rank", 0) else "bf16")
    log(f"[bench] batch16 ({variant}): {blocks:.1f} blocks/s, {el / steps * 1e3:.3f} ms/step; append of {nb}x{a} rows: "
        f"batched {app['batched']:.3f} ms, per sequence {app['per_seq']:.3f} ms")
    gemm_ms = br["gemm"][0] / steps
    M = nb * gamma
    gemm_flop = 2 * M * gemm_weight_elems(m)
    gemm_stats = dict(rows=M, flop_per_step=gemm_flop, ms_per_step=round(gemm_ms, 4),
                      tflops=round(gemm_flop / (gemm_ms * 1e-3) / 1e12, 1),
                      mfma_frac=round(gemm_flop / (gemm_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                      weight_gbs=round(gemm_weight_elems(m) * wbytes / (gemm_ms * 1e-3) / 1e9, 1))
    extra = {}
    if m.get("markov_rank", 0) and br.get("markov", (0, 0))[1]:
        mk_ms = br["markov"][0] / steps
        mk_b = markov_bytes(m, nb, gamma)
        extra["markov"] = dict(ms_per_step=round(mk_ms, 4), algorithmic_bytes_per_step=int(mk_b),
                               gbs=round(mk_b / (mk_ms * 1e-3) / 1e9, 1),
                               avg_launch_us=round(br["markov"][0] / br["markov"][1] * 1e3, 3))
    return dict(workload=WORKLOAD_B16, variant=variant, value=round(blocks, 2), unit="blocks/s", steps=steps,
                ms_per_step=round(el / steps * 1e3, 4), tokens_per_s=round(blocks * (gamma - 1), 1),
                bracketed_ms_per_step=round(el_br / steps * 1e3, 4), ctx_lengths=[int(x) for x in lens],
                timing="value from plain launches; per-class times from a second pass with every launch class "
                       "bracketed by events",
                append=dict(rows=nb * a, form="one batched call" if batched else "per sequence",
                            batched_ms=round(app["batched"], 4), per_seq_loop_ms=round(app["per_seq"], 4),
                            timing="wall clock, 10 calls, nothing bracketed"),
                layer_gemms=gemm_stats,
                kernels_ms_per_step={k: round(v[0] / steps, 4) for k, v in br.items() if v[1]}, **extra)


def bench_longctx(m, Wd, gamma, B, torch, np, synth, to_dev):
    """32 sequences with contexts U{8192..32768} on a pool of permuted pages (prefilled
    untimed from four reused seeded 2048-row chunks: the shapes, not the draws, set the
    cost); timed: the 2048-row append of every sequence (MFMA-bound) and the 32-band block
    forward (attention-bound), with the attention launches bracketed by events."""
    w = synth.workload(WORKLOAD_LONG)
    nb, app_rows = w["batch"], w["append"]
    dev = torch.device("cuda:0")
    lens = synth.gen_ctx_lengths(w["ctx"][0], w["ctx"][1], nb, w["seed"])
    per_seq = -(-(w["max_seq_len"] + gamma + 1) // 16)
    d = B.Drafter(m, Wd, w["max_seq_len"], nb, page_order=synth.gen_page_order(per_seq * nb, w["seed"]))
    chunks = [to_dev(synth.gen_hidden(m, w["seed"], 2048, 1000 + i)) for i in range(4)]
    t = time.perf_counter()
    for s in range(nb):
        for c, r0 in enumerate(range(0, int(lens[s]), 2048)):
            d.dflash_ctx_kv_append(s, chunks[c % 4][:min(2048, int(lens[s]) - r0)])
    torch.cuda.synchronize()
    log(f"[bench] longctx: prefilled {int(lens.sum())} rows in {time.perf_counter() - t:.1f}s")
    tail = to_dev(synth.gen_hidden(m, w["seed"], app_rows, 999))
    t0 = time.perf_counter()
    for s in range(nb):
        d.dflash_ctx_kv_append(s, tail)
    torch.cuda.synchronize()
    app_s = time.perf_counter() - t0
    kvd = m["num_kv_heads"] * m["head_dim"]
    app_flop = nb * 2 * app_rows * (m["num_taps"] * m["target_hidden"] * m["hidden"]
                                     + m["hidden"] * m["num_layers"] * 2 * kvd)
    toks = torch.empty((nb, gamma - 1), dtype=torch.int32, device=dev)
    bonus = synth.gen_bonus(m, w["seed"], nb)
    seqs = list(range(nb))
    d.dflash_block_forward(seqs, bonus, toks, gamma=gamma)
    torch.cuda.synchronize()
    reps = 10
    t0 = time.perf_counter()
    for _ in range(reps):
        d.dflash_block_forward(seqs, bonus, toks, gamma=gamma)
    torch.cuda.synchronize()
    fwd_s = (time.perf_counter() - t0) / reps
    d.dflash_timing(["attn"])
    for _ in range(reps):
        d.dflash_block_forward(seqs, bonus, toks, gamma=gamma)
    torch.cuda.synchronize()
    attn = d.dflash_timing_read()["attn"]
    d.dflash_timing([])
    d.close()
    kv_lens = [int(c) + app_rows for c in lens]
    kv_bytes = attn_bytes(m, kv_lens, gamma)
    attn_ms = attn[0] / reps
    attn_gbs = kv_bytes / (attn_ms * 1e-3) / 1e9
    log(f"[bench] longctx: append {app_flop / app_s / 1e12:.0f} TFLOP/s, forward {nb / fwd_s:.0f} blocks/s, "
        f"attention {attn_gbs:.0f} GB/s")
    return dict(workload=WORKLOAD_LONG, appended_rows_per_seq=app_rows, ctx_lengths=[int(x) for x in lens],
                append=dict(seconds=round(app_s, 5), flop=app_flop, tflops=round(app_flop / app_s / 1e12, 1),
                            mfma_frac=round(app_flop / app_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                            timing="wall clock around the 32 appends (one sample: each append advances kv_len)"),
                forward=dict(ms=round(fwd_s * 1e3, 4), blocks_per_s=round(nb / fwd_s, 2),
                             tokens_per_s=round(nb * (gamma - 1) / fwd_s, 1)),
                attention=dict(bound="hbm", kv_bytes_per_forward=int(kv_bytes), ms_per_forward=round(attn_ms, 4),
                               launches_per_forward=attn[1] / reps, achieved=round(attn_gbs, 1),
                               peak=HBM_PEAK_GBS, unit="GB/s", frac=round(attn_gbs / HBM_PEAK_GBS, 4)))


def bench_wide(a, args, B, torch, np, synth, to_dev):
    """The wide drafter (5 layers, hidden 5376, GQA 64:8, ff 10752, vocab 262144, YaRN, window
    2048 on layers 0-3) at batch 1 on a 16384-row context (prefilled untimed): a step is an
    `a`-row append and one block forward. Plain launches give blocks/s; a second pass with every
    launch bracketed by events gives the per-class times and the weight-stream rates of the
    layer GEMMs and the 2.8 GB lm_head, and the attention's K/V bytes per second."""
    w = synth.workload(WORKLOAD_WIDE)
    m, seed = w["model_cfg"], w["seed"]
    gamma = m["gamma_max"]
    t = time.perf_counter()
    W = synth.gen_weights(m, seed)
    Wd = {k: to_dev(v) for k, v in W.items()}
    ctx = w["ctx"][0]
    steps = max(5, args.steps // 2)
    total = args.warmup + 2 * steps
    d = B.Drafter(m, Wd, ctx + total * a + gamma + 16, 1)
    for c, r0 in enumerate(range(0, ctx, 2048)):
        d.dflash_ctx_kv_append(0, to_dev(synth.gen_hidden(m, seed, min(2048, ctx - r0), c)))
    Hs = to_dev(synth.gen_hidden(m, seed, total * a, 100))
    bonus = synth.gen_bonus(m, seed, total)
    toks = torch.empty((1, gamma - 1), dtype=torch.int32, device="cuda:0")
    torch.cuda.synchronize()
    log(f"[bench] wide: weights and {ctx}-row prefill in {time.perf_counter() - t:.1f}s")
    step_i = [0]

    def step():
        i = step_i[0]
        d.dflash_ctx_kv_append(0, Hs[i * a:(i + 1) * a])
        d.dflash_block_forward([0], [int(bonus[i])], toks, gamma=gamma)
        step_i[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kv0 = d.dflash_seq_info(0)[0]
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    kv1 = d.dflash_seq_info(0)[0]
    d.dflash_timing(list(B.K_CLASSES))
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    br = d.dflash_timing_read()
    d.dflash_timing([])
    d.close()
    ms = {k: v[0] / steps for k, v in br.items() if v[1]}
    blocks = steps / el
    mean_kv = (kv0 + kv1) / 2 + a / 2
    rates = {}
    for k, nbytes in (("gemm", gemm_bytes(m, gamma)), ("lmhead", lmhead_bytes(m, gamma)),
                      ("attn", attn_bytes(m, [mean_kv], gamma))):
        if k in ms:
            g = nbytes / (ms[k] * 1e-3) / 1e9
            rates[k] = dict(algorithmic_bytes_per_step=int(nbytes), ms_per_step=round(ms[k], 4), gbs=round(g, 1),
                            frac=round(g / HBM_PEAK_GBS, 4),
                            avg_launch_us=round(br[k][0] / br[k][1] * 1e3, 3), launches_per_step=br[k][1] / steps)
    step_bytes = forward_bytes(m, [mean_kv], gamma) + append_bytes(m, a)
    log(f"[bench] wide batch1: {blocks:.1f} blocks/s, {el / steps * 1e3:.3f} ms/step; "
        + ", ".join(f"{k} {v['gbs']:.0f} GB/s" for k, v in rates.items()))
    return dict(workload=WORKLOAD_WIDE, value=round(blocks, 2), unit="blocks/s", steps=steps,
                ms_per_step=round(el / steps * 1e3, 4), tokens_per_s=round(blocks * (gamma - 1), 1),
                step_algorithmic_bytes=int(step_bytes),
                step_gbs=round(step_bytes / (el / steps) / 1e9, 1), streams=rates,
                kernels_ms_per_step={k: round(v, 4) for k, v in ms.items()},
                timing="value from plain launches; per-class times from a second, bracketed pass"), W


if __name__ == "__main__":
    main()
