#!/usr/bin/env python3
"""Benchmark of quantization-aware attention (forward + straight-through
backward) on one MI355X.

A step is one pass of the whole hot path over the DiT image joint-attention
batch (B1 H24 N4608 D128 bf16, P fake-quant e4m3): the forward (scores,
online softmax, P fake quant, O and O_hp, log-sum-exp) and the backward
(Delta, dQ, dK/dV).  Inputs are seeded synthetic tensors already resident in
HBM; outputs and workspaces are allocated once, outside the timed region.

Prints one JSON line (rank 0):
  value     credited TFLOP/s: 16 W / step time, W = B H Nq Nkv D
            (forward: QK^T, P^V, P_hp V; backward: S, dP, dV, dQ, dK;
            recomputation in the split backward is not credited)
  roofline  the slowest kernel of the step, timed with HIP events on the
            stream it runs on, against the bf16 dense MFMA peak
  cpu_baseline  the float64 oracle on a bounded sample (six of the 24 heads by
            default) on the host cores, scaled to TFLOP/s
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "QAT attn fwd+bwd TFLOP/s, B1 H24 N4608 D128 bf16; % of MFMA peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dit_image")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--kv-chunks", type=int, default=1,
                    help="chunked-KV mode: the step as C forwards over equal KV chunks (multiples of 64 keys) + "
                         "qat_attn_merge, and C chunk backwards + qat_attn_sum of the dQ parts")
    ap.add_argument("--cpu-heads", type=int, default=6, help="heads in the oracle sample (0: skip)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (calibrates HBM byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a --copy-mib run "
                         "into profiles/hbm_traffic_<workload>.json and exit (no GPU needed)")
    return ap.parse_args()


# stage label -> kernels that implement it (the forward has a ping-pong kernel
# for value inputs and a separate one for fp8 V; the dK/dV stage adds a small
# merge kernel when it splits its last key blocks over query ranges)
KERNEL_TAGS = {
    "fwd_kernel": ("fwd_pp_kernel", "fwd_f8v_kernel"),
    "delta_kernel": ("delta_kernel",),
    "dq_kernel": ("dq_kernel",),
    "dkdv_kernel": ("dkdv_pair_kernel", "dkdv_merge_kernel"),
    "token_quant_kernel": ("token_quant_kernel", "kmean_partial_kernel", "kmean_final_kernel", "shift_rows_kernel"),
}


def stage_of(kernel_name: str):
    for tag, names in KERNEL_TAGS.items():
        if any(f"qat::{n}<" in kernel_name for n in names):
            return tag
    return None


def summarize_pmc(fetch_csv: str, write_csv: str, workload: str, copy_mib: int):
    """Per-launch HBM bytes of each kernel from FETCH_SIZE / WRITE_SIZE (KiB
    per dispatch), each scaled by what the same counter reads for the plain
    copy of copy_mib MiB in the same run (known: copy_mib MiB read and
    written)."""
    import csv
    from collections import defaultdict

    def load(path, counter):
        # bytes per stage call: the mean over dispatches of each kernel,
        # summed over the kernels of the stage
        per = defaultdict(lambda: defaultdict(list))
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            tag = stage_of(name)
            if "copyBuffer" in name:
                tag = "copy"
            if tag:
                per[tag][name.split("<")[0]].append(float(r["Counter_Value"]) * 1024.0)
        return {t: sum(sum(v) / len(v) for v in ks.values()) for t, ks in per.items()}

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    known = float(copy_mib << 20)
    ff, wf = known / fetch["copy"], known / write["copy"]
    from quantization_aware_attention_amd import workloads as W
    w = W.WORKLOADS[workload]
    e = 2                      # bytes per element of Q, K, dO, O, O_hp, dQ, dK, dV
    ev = 1 if w.v_fp8 else 2   # V: e5m2 codes with fp8 V (plus its [B, H, D] fp32 scale)
    BH = w.B * w.H
    vsc = BH * w.D * 4 if w.v_fp8 else 0
    alg = {
        "fwd_kernel": BH * (w.Nq * w.D * e + w.Nkv * w.D * (e + ev)) + vsc + BH * w.Nq * (2 * w.D * e + 4),
        "delta_kernel": BH * w.Nq * (2 * w.D * e + 4),
        # the step's dQ call also reads O_hp (it forms Delta; Delta is written instead of read)
        "dq_kernel": BH * (3 * w.Nq * w.D * e + w.Nkv * w.D * (e + ev) + 8 * w.Nq) + vsc + BH * w.Nq * w.D * e,
        "dkdv_kernel": BH * (2 * w.Nq * w.D * e + w.Nkv * w.D * (e + ev) + 8 * w.Nq) + vsc + 2 * BH * w.Nkv * w.D * e,
    }
    out = {"workload": workload, "source_hash": kernel_source_hash(),
           "calibration": {"copy_bytes": known, "fetch_counter_bytes": fetch["copy"],
                           "write_counter_bytes": write["copy"], "fetch_factor": ff, "write_factor": wf},
           "kernels": {}}
    for t in fetch:
        if t == "copy" or t not in write:
            continue
        fb, wb = fetch[t] * ff, write[t] * wf
        out["kernels"][t] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
                             "algorithmic_bytes": alg.get(t)}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"hbm_traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def kernel_source_hash() -> str:
    """Hash of the HIP sources with comments and blank lines left out; HBM
    counter readings are valid only for the kernels they were taken on (an
    edit of a comment does not change a kernel)."""
    import hashlib
    import re
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quantization_aware_attention_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(root)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            text = open(os.path.join(root, name), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)   # block comments (none sit inside strings here)
            code = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
            h.update(name.encode())
            h.update("\n".join(line for line in code if line).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str = "dit_image"):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/hbm_traffic_<workload>.json), or None when the summary is
    missing or was taken on different kernel sources."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, args.copy_mib or 512)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the kernel runs on one "
              "GPU's share of the heads); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantization_aware_attention_amd import ops
    from quantization_aware_attention_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[w.dtype]

    inp = W.make_inputs(w)
    def up(name):
        return torch.from_numpy(inp[name + "_bits"].view(np.int16)).view(tdt).to(dev)
    q, k, v, do = up("q"), up("k"), up("v"), up("do")
    flags = ops.QAT_P_QUANT | (ops.QAT_P_E5M2 if w.p_fmt == "e5m2" else 0)
    flags |= ops.QAT_QKV_QUANT if w.qkv_quant else 0
    flags |= ops.QAT_SMOOTH_K if w.smooth_k else 0
    v_scale = None
    if w.v_fp8:
        flags |= ops.QAT_V_FP8_E5M2
        v, v_scale = ops.quant_v_fp8(v)
    dims = ops.dims_of(q, k)
    o, o_hp = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device=dev, dtype=torch.float32)
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    dv = torch.empty(k.shape, device=dev, dtype=tdt)
    ws_f = torch.empty(max(256, ops.workspace_bytes(dims, flags, 0)), device=dev, dtype=torch.uint8)
    ws_b = torch.empty(max(256, ops.workspace_bytes(dims, flags, 1)), device=dev, dtype=torch.uint8)

    def fwd():
        ops.attn_fwd(q, k, v, w.sm_scale, w.causal, flags, v_scale=v_scale, out=(o, o_hp, lse), workspace=ws_f)

    def bwd(stages=ops.QAT_BWD_ALL):
        ops.attn_bwd(q, k, v, o_hp, lse, do, w.sm_scale, w.causal, flags, v_scale=v_scale,
                     out=(dq, dk, dv), workspace=ws_b, stages=stages)

    def step():
        fwd()
        bwd()

    C = args.kv_chunks
    if C > 1:   # chunked-KV mode (non-causal, plain value inputs): per-chunk buffers outside the timed region
        if w.causal or w.v_fp8 or w.qkv_quant or w.smooth_k or (w.Nkv // C) % 64 or w.Nkv % C:
            print("--kv-chunks needs a non-causal workload with plain inputs and Nkv/C a multiple of 64",
                  file=sys.stderr)
            sys.exit(2)
        n = w.Nkv // C
        kc = [k[:, :, i * n:(i + 1) * n].contiguous() for i in range(C)]
        vc = [v[:, :, i * n:(i + 1) * n].contiguous() for i in range(C)]
        outs = [(torch.empty_like(q), torch.empty_like(q), torch.empty_like(lse)) for _ in range(C)]
        gouts = [(torch.empty_like(q), torch.empty_like(kc[0]), torch.empty_like(vc[0])) for _ in range(C)]
        cdims = ops.dims_of(q, kc[0])
        ws_fc = torch.empty(max(256, ops.workspace_bytes(cdims, flags, 0)), device=dev, dtype=torch.uint8)
        ws_bc = torch.empty(max(256, ops.workspace_bytes(cdims, flags, 1)), device=dev, dtype=torch.uint8)

        def fwd():
            for i in range(C):
                ops.attn_fwd(q, kc[i], vc[i], w.sm_scale, False, flags, out=outs[i], workspace=ws_fc)
            ops.attn_merge([t[0] for t in outs], [t[1] for t in outs], [t[2] for t in outs], out=(o, o_hp, lse))

        def bwd_chunked():
            for i in range(C):
                ops.attn_bwd(q, kc[i], vc[i], o_hp, lse, do, w.sm_scale, False, flags, out=gouts[i],
                             workspace=ws_bc)
            ops.attn_sum([t[0] for t in gouts], out=dq)

        def step():
            fwd()
            bwd_chunked()

    stream = torch.cuda.current_stream()
    Wn = w.B * w.H * w.Nq * w.Nkv * w.D
    if w.causal:
        Wn = Wn * (w.Nq + 1) / (2 * w.Nq)
    credited = 16.0 * Wn

    # The diagnostic measurements (per call, per kernel, host enqueue rate)
    # run first: they are not the headline, and they bring the chip to the
    # clock it holds under sustained load, which a few warm-up steps alone do
    # not reach (the first tens of milliseconds of work run slower).

    # ---- median and minimum per call of the forward, the backward (from the
    # saved forward outputs) and the whole step, one event pair per call
    def per_call(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        return {"median": round(ts[len(ts) // 2], 4), "min": round(ts[0], 4)}

    # about 100 ms of steps first, so that the first diagnostic calls do not
    # run on the cold clock either
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    for _ in range(min(100, int(0.1 / max(time.perf_counter() - t0, 1e-4)))):
        step()
    torch.cuda.synchronize()

    split_ms = {"fwd": per_call(fwd, max(args.steps, 20)),
                "bwd": per_call(bwd if C == 1 else bwd_chunked, max(args.steps, 20)),
                "step": per_call(step, max(args.steps, 20))}
    # host time to enqueue the timed loop's steps (no synchronisation inside):
    # tells a host-bound timed window from a GPU-bound one
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    host_ms = (time.perf_counter() - h0) * 1e3 / args.steps
    torch.cuda.synchronize()

    # ---- per-stage durations (each call below launches one kernel, and the
    # dK/dV stage at most one more: the merge of split key blocks)
    kernels = {
        "fwd_kernel": (fwd, 6.0 * Wn),
        "delta_kernel": (lambda: bwd(ops.QAT_BWD_DELTA), None),
        "dq_kernel": (lambda: bwd(ops.QAT_BWD_DQ), 2.0 * Wn),
        "dkdv_kernel": (lambda: bwd(ops.QAT_BWD_DKDV), 8.0 * Wn),
    }
    if w.qkv_quant or w.smooth_k:
        # the forward call also runs the K smoothing / Q/K/V pre-pass: time that stage alone
        kernels = {n: kv for n, kv in kernels.items() if n != "fwd_kernel"}
        kernels["token_quant_kernel"] = (lambda: bwd(ops.QAT_BWD_PREPARE), None)
    kernel_ms = {}
    for name, (fn, _) in kernels.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # one whole step queued ahead keeps the GPU busy while the host enqueues
        # the timed calls, so a short kernel is timed back to back and not at
        # the host's launch rate
        step()
        e0.record(stream)
        for _ in range(args.kernel_reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        kernel_ms[name] = e0.elapsed_time(e1) / args.kernel_reps

    # ---- the headline: W warm-up steps, then exactly K timed steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    value = credited / (ms_step * 1e-3) / 1e12

    dom = max((n for n in kernels if kernels[n][1] is not None), key=lambda n: kernel_ms[n])
    dom_tflops = kernels[dom][1] / (kernel_ms[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(dom_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom_tflops / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(dom, w.name), "kernel": dom,
                "kernel_ms": {n: round(t, 4) for n, t in kernel_ms.items()}}
    # HBM-bound stages: algorithmic bytes (each tensor once) per call / duration
    e = 2
    BH = w.B * w.H
    hbm_bytes = {"delta_kernel": BH * w.Nq * (2 * w.D * e + 4)}
    prep_bytes = 0
    if w.smooth_k:    # read K for its mean; without Q/K/V quant also read K, write K - mean
        prep_bytes += BH * w.Nkv * w.D * e * (1 if w.qkv_quant else 3)
    if w.qkv_quant:   # read Q, K, V; write the Q, K code values, V^ and the Q, K scales
        prep_bytes += BH * (2 * (w.Nq + 2 * w.Nkv) * w.D * e + 4 * (w.Nq + w.Nkv))
    if prep_bytes:
        hbm_bytes["token_quant_kernel"] = prep_bytes
    roofline["hbm_stages_gbps"] = {n: round(b / (kernel_ms[n] * 1e-3) / 1e9, 1) for n, b in hbm_bytes.items()
                                   if n in kernel_ms}

    # ---- plain copy of a known size (counter calibration runs)
    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # ---- float64 oracle on a bounded sample of the same workload
    cpu = None
    if args.cpu_heads > 0:
        from threadpoolctl import threadpool_info

        from oracle import qat_attention as oracle
        nh = min(args.cpu_heads, w.B * w.H)
        sample = W.make_inputs(w, heads=nh)
        v_codes = vs = None
        if w.v_fp8:
            v_codes, vs = oracle.quantize_v_channels(sample["v"], "e5m2")
        kw = dict(causal=w.causal, p_fmt=w.p_fmt, qkv_quant=w.qkv_quant, v_codes=v_codes, v_scale=vs,
                  smooth_k=w.smooth_k, dtype=w.dtype)
        c0 = time.perf_counter()
        oracle.attention_forward(sample["q"], sample["k"], sample["v"], w.sm_scale, **kw)
        c1 = time.perf_counter()
        oracle.attention_backward(sample["q"], sample["k"], sample["v"], sample["do"], w.sm_scale, **kw)
        c2 = time.perf_counter()
        # the threads the oracle ran on: NumPy's BLAS pool (its matrix products
        # are where the time goes; everything else is single-threaded)
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        share = nh / (w.B * w.H)
        cpu = {"value": round(credited * share / (c2 - c0) / 1e12, 6), "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle",
               "sample": f"{nh} of {w.B * w.H} heads, forward + backward, float64 NumPy, {c2 - c0:.1f} s",
               "host_cpu_count": os.cpu_count(), "blas_threads": threads,
               "fwd_s": round(c1 - c0, 3), "bwd_s": round(c2 - c1, 3),
               "fwd_tflops": round(6.0 * Wn * share / (c1 - c0) / 1e12, 6),
               "bwd_tflops": round(10.0 * Wn * share / (c2 - c1) / 1e12, 6)}

    fa_conv = 14.0 * Wn / (ms_step * 1e-3) / 1e12
    # forward, backward and step throughput from the per-call medians
    # (credited 6W, 10W, 16W) and their share of the bf16 dense peak
    passes = {}
    for name, flop in (("fwd", 6.0 * Wn), ("bwd", 10.0 * Wn), ("step", 16.0 * Wn)):
        tf = flop / (split_ms[name]["median"] * 1e-3) / 1e12
        passes[name] = {"tflops": round(tf, 2), "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
    extra = {}
    if w.v_fp8:
        # the quantized P^V runs on the fp8 MFMA (twice the bf16 rate): the
        # step's time at a blended peak, and the forward's HBM rate (V 1 B/elt)
        t_peak = (14.0 * Wn / PEAK_BF16_TFLOPS + 2.0 * Wn / PEAK_FP8_TFLOPS) / 1e12
        extra["pct_of_blended_peak"] = round(100 * t_peak / (ms_step * 1e-3), 2)
        fwd_bytes = w.B * w.H * (w.Nq * w.D * 2 + w.Nkv * w.D * 2 + w.Nkv * w.D + 2 * w.Nq * w.D * 2 + 4 * w.Nq)
        extra["fwd_hbm_gbps"] = round(fwd_bytes / (split_ms["fwd"]["median"] * 1e-3) / 1e9, 1)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B{w.B} H{w.H} Nq{w.Nq} Nkv{w.Nkv} D{w.D} {w.dtype}, "
                               f"{'causal' if w.causal else 'non-causal'}, P fake-quant {w.p_fmt}"
                               f"{', K smoothed' if w.smooth_k else ''}"
                               f"{', Q/K/V fake-quant e4m3' if w.qkv_quant else ''}"
                               f"{', V e5m2' if w.v_fp8 else ''}",
                   "credited_flop_per_step": credited, "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "fa_convention_tflops": round(fa_conv, 2), "call_ms": split_ms, "per_pass": passes,
                   "host_enqueue_ms_per_step": round(host_ms, 4),
                   **({"kv_chunks": C} if C > 1 else {}), **extra},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
