"""Benchmark of the sparse-MoE layer forward on one MI355X.

One step = one full layer forward (router, top-k, permutation, grouped
gate/up and down GEMMs with the shared expert, combine) over one batch of
synthetic tokens, inputs already resident in HBM.  The default workload is
the full-shape decode layer (T = 64 tokens, hidden 4096, 288 experts top-8,
intermediate 1280, shared expert); the full-shape prefill layer (T = 8192)
is measured beside it and reported under "prefill".

Each step reads the routed weights of another copy of the layer (weight
copies rotate), as consecutive MoE layers of a model would, so the 256 MB
last-level cache does not serve one step's expert weights from the last.

Prints one JSON line.  The pages this layer comes from publish model
configuration only and no throughput numbers, so vs_baseline is null.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--config decode]
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

METRIC = "MoE-layer tokens/s at T=64/8192 (4096→1280, 288e top-8); % of MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
NOTE = "the pages publish model configuration only, no throughput numbers"


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode",
                    choices=["decode", "prefill", "skewed", "long", "tiny"])
    ap.add_argument("--weight-copies", type=int, default=4)
    ap.add_argument("--no-secondary", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    return ap.parse_args()


def counts(wl, U):
    """Algorithmic FLOPs and HBM bytes of one layer forward (U = experts with
    at least one pair) and of the gate/up kernel."""
    H, E, I, Is, T, P = wl.H, wl.E, wl.I, wl.Is, wl.T, wl.P
    flop_router = 2.0 * T * H * E
    flop_experts = 6.0 * P * H * I + 6.0 * T * H * Is
    bytes_layer = U * 3.0 * H * I * 2 + 3.0 * H * Is * 2 + E * H * 4 + E * 4 + T * H * 2 * 2
    gu_bytes = (U * 2.0 * H * I + 2.0 * H * Is) * 2 + T * H * 2
    gu_flop = 4.0 * P * H * I + 4.0 * T * H * Is
    return dict(flop_router=flop_router, flop_experts=flop_experts, bytes_layer=bytes_layer,
                gateup_bytes=gu_bytes, gateup_flop=gu_flop)


def traffic_for(kernel, workload):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "sparse_moe_layer_fp32_amd", "csrc", "experts.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    ent = rec.get(f"{kernel}:{workload}")
    if not ent or ent.get("source_sha256") != sha:
        return None
    return ent.get("bytes_per_launch")


def measure(wl, moe, synth, experts_host, copies, steps, warmup):
    import numpy as np
    import torch

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    x = dev(synth.gen_x(wl))
    rw_h, rb_h, _ = synth.gen_router(wl)
    rw, rb = dev(rw_h), dev(rb_h)
    cfg = moe.make_config(wl.T, wl.H, wl.E, wl.k, wl.I, wl.Is, wl.routed_scaling,
                          wl.renormalize, wl.limit, wl.limit_shared)
    ws = moe.alloc_workspace(cfg)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")

    def step(i, events=None):
        c = copies[i % len(copies)]
        if events is None:
            moe.moe_forward(cfg, x, rw, rb, *c, y, ids, w, ws)
        else:
            moe.moe_forward_timed(cfg, x, rw, rb, *c, y, ids, w, ws, events=events)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps

    # Per-kernel durations: the same steps again with HIP events recorded on
    # the launch stream between the kernels.
    nst = moe.MOE_NUM_STAGES
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    stage_ms = {name: sum(e[s].elapsed_time(e[s + 1]) for e in evs) / steps
                for s, name in enumerate(moe.STAGES)}

    ids_h = ids.cpu().numpy()
    hist = np.bincount(ids_h.ravel(), minlength=wl.E)
    U = int(np.count_nonzero(hist))
    c = counts(wl, U)
    t = ms * 1e-3
    gu_t = stage_ms["gateup"] * 1e-3
    out = dict(
        ms_per_step=ms,
        tokens_per_s=wl.T / t,
        tflops=(c["flop_router"] + c["flop_experts"]) / t * 1e-12,
        gbs=c["bytes_layer"] / t * 1e-9,
        frac_mfma=(c["flop_router"] + c["flop_experts"]) / t * 1e-12 / BF16_PEAK_TFLOPS,
        frac_hbm=c["bytes_layer"] / t * 1e-9 / HBM_PEAK_GBS,
        stage_ms={k: round(v, 5) for k, v in stage_ms.items()},
        experts_used=U,
        tokens_per_expert=dict(min=int(hist.min()), median=float(np.median(hist)),
                               max=int(hist.max())),
        hot16_share=float(np.sort(hist)[::-1][:16].sum() / hist.sum()),
        gateup=dict(ms=stage_ms["gateup"], gbs=c["gateup_bytes"] / gu_t * 1e-9,
                    tflops=c["gateup_flop"] / gu_t * 1e-12, bytes=c["gateup_bytes"],
                    flop=c["gateup_flop"]),
    )
    del ws
    return out, ids_h


def roofline(wl, res, bound):
    g = res["gateup"]
    if bound == "hbm":
        tr = traffic_for("gateup_kernel", wl.name)
        return dict(kernel="gateup_kernel", bound="hbm", achieved=round(g["gbs"], 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(g["gbs"] / HBM_PEAK_GBS, 4),
                    traffic=tr, algorithmic_bytes_per_launch=g["bytes"],
                    avg_launch_ms=round(g["ms"], 5))
    tr = traffic_for("gateup_kernel", wl.name)
    return dict(kernel="gateup_kernel", bound="mfma", achieved=round(g["tflops"], 1),
                peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=round(g["tflops"] / BF16_PEAK_TFLOPS, 4),
                traffic=tr, algorithmic_flop_per_launch=g["flop"], avg_launch_ms=round(g["ms"], 5))


def cpu_baseline(wl, inp):
    import oracle
    threads = oracle.default_threads()
    cfg = oracle.cfg_of(wl)
    t0 = time.perf_counter()
    oracle.forward(cfg, inp, threads=threads)
    dt = time.perf_counter() - t0
    return dict(value=round(wl.T / dt, 3), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"all {wl.T} tokens of the {wl.name} workload (double-precision "
                       f"per-token oracle, {dt:.1f} s wall)")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this build has no "
              "multi-GPU path; the layer would shard by tokens or by experts, see DESIGN.md",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import sparse_moe_layer_fp32_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.load_library()
    wl = synth.WORKLOADS[args.config]
    log(f"[bench] generating inputs for {wl.name} (T={wl.T})")
    experts_host = synth.gen_experts(wl)

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)

    base = [dev(a) for a in experts_host]
    ncopy = max(1, args.weight_copies if wl.name != "tiny" else 1)
    copies = [tuple(base)]
    for _ in range(ncopy - 1):
        copies.append(tuple(t.clone() for t in base))
    torch.cuda.synchronize()
    log(f"[bench] {ncopy} weight copies resident; timing {args.steps} steps")
    res, _ = measure(wl, moe, synth, experts_host, copies, args.steps, args.warmup)
    log(f"[bench] {wl.name}: {res['ms_per_step']:.4f} ms/step, stages {res['stage_ms']}")

    bound = "hbm" if wl.name in ("decode", "tiny") else "mfma"
    rec = dict(metric=METRIC, value=round(res["tokens_per_s"], 1), unit="tokens/s", n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=round(res["ms_per_step"], 5),
               higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
               data="synthetic",
               config=dict(workload=wl.name, tokens=wl.T, hidden=wl.H, experts=wl.E, top_k=wl.k,
                           inter=wl.I, inter_shared=wl.Is, swiglu_limit=wl.limit,
                           weight_copies=ncopy, seed=wl.seed, parallelism="single GPU"),
               roofline=roofline(wl, res, bound),
               layer=dict(tflops=round(res["tflops"], 2), gbs=round(res["gbs"], 1),
                          frac_mfma=round(res["frac_mfma"], 4), frac_hbm=round(res["frac_hbm"], 4),
                          stage_ms=res["stage_ms"], experts_used=res["experts_used"],
                          tokens_per_expert=res["tokens_per_expert"],
                          hot16_share=round(res["hot16_share"], 3)),
               note=NOTE)

    if wl.name == "decode" and not args.no_secondary:
        pw = synth.WORKLOADS["prefill"]
        log("[bench] prefill T=8192")
        pres, _ = measure(pw, moe, synth, experts_host, copies[:2], max(5, args.steps // 5),
                          max(2, args.warmup // 2))
        rec["prefill"] = dict(tokens_per_s=round(pres["tokens_per_s"], 1),
                              ms_per_step=round(pres["ms_per_step"], 5),
                              tflops=round(pres["tflops"], 2),
                              frac_mfma=round(pres["frac_mfma"], 4),
                              roofline=roofline(pw, pres, "mfma"), stage_ms=pres["stage_ms"],
                              experts_used=pres["experts_used"])
        log(f"[bench] prefill: {pres['ms_per_step']:.4f} ms/step, stages {pres['stage_ms']}")

    if not args.no_cpu and wl.name in ("decode", "tiny"):
        log("[bench] CPU oracle baseline")
        inp = synth.make_inputs(wl, experts=experts_host)
        rec["cpu_baseline"] = cpu_baseline(wl, inp)
    gp = torch.cuda.get_device_properties(0)
    rec["device"] = dict(name=gp.name, arch=getattr(gp, "gcnArchName", ""),
                         compute_units=gp.multi_processor_count)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
