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
import re
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
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the second workloads (Step-3 MoE shape, dense FFN)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES five times (to scale HBM "
                         "traffic counters) and exit")
    ap.add_argument("--summarize-profiles", default="", metavar="DIR",
                    help="write profiles/*.md and profiles/traffic.json from the rocprofv3 "
                         "outputs of PROFILE_COMMANDS under DIR, and exit (no GPU needed)")
    return ap.parse_args()


# Commands whose outputs --summarize-profiles reads (DIR = its argument).
PROFILE_COMMANDS = {
    "kt_decode": "rocprofv3 --kernel-trace --stats --output-format csv -d DIR/kt_decode -o run -- "
                 "python3 bench.py --config decode --steps 20 --warmup 5 --no-cpu --no-secondary",
    "kt_prefill": "rocprofv3 --kernel-trace --stats --output-format csv -d DIR/kt_prefill -o run -- "
                  "python3 bench.py --config prefill --steps 10 --warmup 3 --no-cpu --weight-copies 2",
    "pmc_fetch_decode": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/pmc_fetch_decode -o run -- "
                        "python3 bench.py --config decode --steps 4 --warmup 1 --no-cpu --no-secondary",
    "pmc_write_decode": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/pmc_write_decode -o run -- "
                        "python3 bench.py --config decode --steps 4 --warmup 1 --no-cpu --no-secondary",
    "pmc_fetch_prefill": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/pmc_fetch_prefill -o run -- "
                         "python3 bench.py --config prefill --steps 2 --warmup 1 --no-cpu --weight-copies 1",
    "pmc_write_prefill": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/pmc_write_prefill -o run -- "
                         "python3 bench.py --config prefill --steps 2 --warmup 1 --no-cpu --weight-copies 1",
    "pmc_fetch_copy": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/pmc_fetch_copy -o run -- "
                      "python3 bench.py --copy-calibration 1073741824",
    "pmc_write_copy": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/pmc_write_copy -o run -- "
                      "python3 bench.py --copy-calibration 1073741824",
}
# The sources each kernel is built from (its file and the headers it includes).
_EXPERT_SRC = ("experts.hip", "expert_tile.h", "common.h", "kernels.h")
_ROUTER_SRC = ("router.hip", "router_ops.h", "common.h", "kernels.h")
_PERMUTE_SRC = ("permute.hip", "permute_ops.h", "common.h", "kernels.h")
KERNEL_SOURCES = {"expert_gemm": _EXPERT_SRC, "combine_kernel": _EXPERT_SRC,
                  "router_gemm_kernel": _ROUTER_SRC, "topk_kernel": _ROUTER_SRC,
                  "topk_block_kernel": _ROUTER_SRC, "router_split_kernel": _ROUTER_SRC,
                  "permute_small_kernel": _PERMUTE_SRC, "rank_kernel": _PERMUTE_SRC,
                  "scan_kernel": _PERMUTE_SRC, "scatter_kernel": _PERMUTE_SRC}


def _short(name):
    name = name.replace("moe::(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].strip()


def _src_sha(fnames):
    """SHA-256 over the given kernel sources, in order."""
    h = hashlib.sha256()
    for fname in fnames:
        with open(os.path.join(ROOT, "sparse_moe_layer_fp32_amd", "csrc", fname), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def summarize_profiles(d):
    """Turn rocprofv3 CSV outputs under d (made by PROFILE_COMMANDS) into the
    text summaries under profiles/ and profiles/traffic.json."""
    import csv
    import collections
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    for wl in ("decode", "prefill"):
        path = os.path.join(d, f"kt_{wl}", "run_kernel_stats.csv")
        rows = list(csv.DictReader(open(path)))
        lines = [f"# Kernel durations, {wl} workload (rocprofv3 kernel trace)", "",
                 "Command (from /tmp with TMPDIR=/tmp; DIR = an output directory):", "",
                 "```", PROFILE_COMMANDS[f"kt_{wl}"], "```", "",
                 "| Kernel | Calls | Average us | Min us | Max us | Share |",
                 "|---|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f}% |")
        lines += ["", "`__amd_rocclr_copyBuffer` is the benchmark's own weight-copy setup, outside "
                  "the timed region.", ""]
        with open(os.path.join(out_dir, f"kernels_{wl}.md"), "w") as f:
            f.write("\n".join(lines))

    def per_kernel(name):
        agg = collections.defaultdict(list)
        for r in csv.DictReader(open(os.path.join(d, name, "run_counter_collection.csv"))):
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in agg.items()}

    copy_fetch = per_kernel("pmc_fetch_copy")["__amd_rocclr_copyBuffer"]
    copy_write = per_kernel("pmc_write_copy")["__amd_rocclr_copyBuffer"]
    cal_bytes = 1073741824
    f_fetch = cal_bytes / (copy_fetch * 1024)   # bytes per reported KiB unit
    f_write = cal_bytes / (copy_write * 1024)
    traffic = {"calibration": {"copy_bytes": cal_bytes, "fetch_kib": copy_fetch,
                               "write_kib": copy_write, "fetch_factor": f_fetch,
                               "write_factor": f_write}}
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Each counter ran alone.  Scale: a plain 1 GiB device copy "
             f"(`__amd_rocclr_copyBuffer`) reads FETCH_SIZE = {copy_fetch:.0f} KiB and "
             f"WRITE_SIZE = {copy_write:.0f} KiB, so bytes = FETCH_SIZE x 1024 x {f_fetch:.3f} "
             f"and WRITE_SIZE x 1024 x {f_write:.3f}.", "", "Commands (from /tmp with TMPDIR=/tmp):", "", "```"]
    lines += [PROFILE_COMMANDS[k] for k in PROFILE_COMMANDS if k.startswith("pmc_")]
    lines += ["```", "", "| Workload | Kernel | Read MB/launch | Written MB/launch |", "|---|---|---|---|"]
    for wl in ("decode", "prefill"):
        fe = per_kernel(f"pmc_fetch_{wl}")
        wr = per_kernel(f"pmc_write_{wl}")
        for k in sorted(fe, key=lambda k: -fe[k]):
            if "moe::" not in k:
                continue
            rb = fe[k] * 1024 * f_fetch
            wb = wr.get(k, 0.0) * 1024 * f_write
            lines.append(f"| {wl} | `{_short(k)}` | {rb / 1e6:.1f} | {wb / 1e6:.1f} |")
            short = _short(k)
            base = short.split("<")[0]
            mode = re.match(r"expert_gemm(?:_persistent)?<(\d)", short)
            key = ("gateup_kernel" if mode and mode.group(1) == "0" else
                   "down_kernel" if mode and mode.group(1) == "1" else base)
            traffic[f"{key}:{wl}"] = {"kernel": short, "read_bytes": rb, "write_bytes": wb,
                                      "bytes_per_launch": rb + wb,
                                      "source_sha256": _src_sha(KERNEL_SOURCES.get(base, _EXPERT_SRC))}
    with open(os.path.join(out_dir, "hbm_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(out_dir, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    print(f"wrote {out_dir}")


def copy_calibration(nbytes):
    """Five plain device-to-device copies of nbytes: the reference for the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 5}))


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
    ent = rec.get(f"{kernel}:{workload}")
    if not ent or ent.get("source_sha256") != _src_sha(_EXPERT_SRC):
        return None  # counters were taken on another version of the kernel
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
    rw, rb = dev(rw_h), (dev(rb_h) if wl.use_bias else None)
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


def measure_single_launch(wl, moe, synth, copies, steps, warmup, ms_multi):
    """moe_forward_fused (the whole layer in one launch) on the same inputs and
    weight copies as the multi-launch measurement; its output is checked equal,
    bit for bit, to moe_forward's on the first copy."""
    import numpy as np
    import torch

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    x = dev(synth.gen_x(wl))
    rw_h, rb_h, _ = synth.gen_router(wl)
    rw, rb = dev(rw_h), (dev(rb_h) if wl.use_bias else None)
    cfg = moe.make_config(wl.T, wl.H, wl.E, wl.k, wl.I, wl.Is, wl.routed_scaling,
                          wl.renormalize, wl.limit, wl.limit_shared)
    ws = moe.alloc_workspace(cfg)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    y_ref = torch.empty_like(y)
    moe.moe_forward(cfg, x, rw, rb, *copies[0], y_ref, None, None, ws)
    moe.moe_forward_fused(cfg, x, rw, rb, *copies[0], y, None, None, ws)
    torch.cuda.synchronize()
    identical = bool(torch.equal(y.view(torch.int16), y_ref.view(torch.int16)))
    for i in range(warmup):
        moe.moe_forward_fused(cfg, x, rw, rb, *copies[i % len(copies)], y, None, None, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.moe_forward_fused(cfg, x, rw, rb, *copies[i % len(copies)], y, None, None, ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del ws
    return dict(ms_per_step=round(ms, 5), tokens_per_s=round(wl.T / (ms * 1e-3), 1),
                vs_multi_launch=round(ms_multi / ms, 3), identical_to_multi_launch=identical)


def measure_fp8(wl, moe, synth, copies8, shared, steps, warmup):
    """moe_forward_fp8 (routed experts as e4m3 codes + row scales) on the
    workload's inputs, the copies of the FP8 weights rotated per step."""
    import numpy as np
    import torch

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    x = dev(synth.gen_x(wl))
    rw_h, rb_h, _ = synth.gen_router(wl)
    rw, rb = dev(rw_h), (dev(rb_h) if wl.use_bias else None)
    cfg = moe.make_config(wl.T, wl.H, wl.E, wl.k, wl.I, wl.Is, wl.routed_scaling,
                          wl.renormalize, wl.limit, wl.limit_shared)
    ws = moe.alloc_workspace(cfg)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")

    def step(i):
        moe.moe_forward_fp8(cfg, x, rw, rb, *copies8[i % len(copies8)], *shared, y, ids, w, ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    U = int(np.count_nonzero(np.bincount(ids.cpu().numpy().ravel(), minlength=wl.E)))
    H, I, Is, T, E, P = wl.H, wl.I, wl.Is, wl.T, wl.E, wl.P
    nbytes = U * (3.0 * H * I + 4.0 * (2 * I + H)) + 3.0 * H * Is * 2 + E * H * 4 + T * H * 2 * 2
    flop = 2.0 * T * H * E + 6.0 * P * H * I + 6.0 * T * H * Is
    t = ms * 1e-3
    return dict(ms_per_step=round(ms, 5), tokens_per_s=round(T / t, 1),
                gbs=round(nbytes / t * 1e-9, 1), frac_hbm=round(nbytes / t * 1e-9 / HBM_PEAK_GBS, 4),
                tflops=round(flop / t * 1e-12, 2),
                frac_mfma=round(flop / t * 1e-12 / BF16_PEAK_TFLOPS, 4), experts_used=U,
                algorithmic_bytes=nbytes)


def measure_dense(wl, moe, synth, steps, warmup):
    """The dense SwiGLU FFN (moe_dense_forward) on its workload: ms/step and
    the MFMA rate of its 6*T*H*I FLOPs."""
    import numpy as np
    import torch

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    inp = synth.make_inputs(wl)
    x, wg, wu, wd = dev(inp.x), dev(inp.ws_gate), dev(inp.ws_up), dev(inp.ws_down)
    cfg = moe.make_dense_config(wl.T, wl.H, wl.Is, wl.limit_shared)
    ws = moe.alloc_dense_workspace(cfg)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    for _ in range(warmup):
        moe.moe_dense_forward(cfg, x, wg, wu, wd, y, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        moe.moe_dense_forward(cfg, x, wg, wu, wd, y, ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    flop = 6.0 * wl.T * wl.H * wl.Is
    tf = flop / (ms * 1e-3) * 1e-12
    return dict(tokens=wl.T, hidden=wl.H, inter=wl.Is, ms_per_step=round(ms, 5),
                tokens_per_s=round(wl.T / (ms * 1e-3), 1), tflops=round(tf, 2),
                frac_mfma=round(tf / BF16_PEAK_TFLOPS, 4))


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
    """The oracle on the whole decode batch, repeated until at least 10 s of
    CPU time have passed (capped at 30 s)."""
    import oracle
    threads = oracle.default_threads()
    cfg = oracle.cfg_of(wl)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(cfg, inp, threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or dt * (reps + 1) / reps > 30.0:
            break
    return dict(value=round(reps * wl.T / dt, 3), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{reps} passes over all {wl.T} tokens of the {wl.name} workload "
                       f"(double-precision per-token oracle, {dt:.1f} s wall)")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): there is no "
              "multi-GPU path; the layer would shard by tokens (each GPU a full replica) or "
              "by experts (an all-to-all of the routed pairs)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
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

    if wl.name == "decode" and not args.no_secondary and not args.no_extra:
        # Second workloads on the same kernels: the predecessor Step-3's MoE shape and the
        # dense SwiGLU FFN of the first layers.
        rec["workloads"] = {}
        # The same decode step in one launch (moe_forward_fused)
        rec["workloads"]["decode_single_launch"] = measure_single_launch(
            wl, moe, synth, copies, args.steps, args.warmup, res["ms_per_step"])
        log(f"[bench] decode single launch: "
            f"{rec['workloads']['decode_single_launch']['ms_per_step']:.4f} ms/step")
        sw = synth.WORKLOADS["step3"]
        log(f"[bench] step3 T={sw.T} (H {sw.H}, E {sw.E}, k {sw.k}, I {sw.I})")
        s_host = synth.gen_experts(sw)
        s_dev = [tuple(dev(a) for a in s_host)]
        del s_host
        sres, _ = measure(sw, moe, synth, None, s_dev, 10, 3)
        rec["workloads"]["step3"] = dict(
            tokens=sw.T, hidden=sw.H, experts=sw.E, top_k=sw.k, inter=sw.I, inter_shared=sw.Is,
            ms_per_step=round(sres["ms_per_step"], 5), tokens_per_s=round(sres["tokens_per_s"], 1),
            tflops=round(sres["tflops"], 2), frac_mfma=round(sres["frac_mfma"], 4),
            experts_used=sres["experts_used"], stage_ms=sres["stage_ms"])
        log(f"[bench] step3: {sres['ms_per_step']:.4f} ms/step")
        del s_dev
        torch.cuda.empty_cache()
        # FP8 (e4m3) routed-expert weights on the decode and prefill workloads
        log("[bench] fp8 experts: decode and prefill")
        f8 = synth.gen_experts_fp8(wl)

        def dev8(a):
            return torch.from_numpy(np.ascontiguousarray(a)).cuda()

        c8 = [tuple(dev8(a) for a in (f8.w8_gate, f8.w8_up, f8.w8_down, f8.s_gate, f8.s_up,
                                      f8.s_down))]
        for _ in range(ncopy - 1):
            c8.append(tuple(t.clone() for t in c8[0]))
        del f8
        shared = tuple(copies[0][3:6])
        rec["workloads"]["decode_fp8"] = measure_fp8(wl, moe, synth, c8, shared, args.steps,
                                                     args.warmup)
        log(f"[bench] decode fp8: {rec['workloads']['decode_fp8']['ms_per_step']:.4f} ms/step")
        rec["workloads"]["prefill_fp8"] = measure_fp8(synth.WORKLOADS["prefill"], moe, synth,
                                                      c8[:2], shared, 10, 3)
        log(f"[bench] prefill fp8: {rec['workloads']['prefill_fp8']['ms_per_step']:.4f} ms/step")
        del c8
        torch.cuda.empty_cache()
        dw = synth.WORKLOADS["dense"]
        log(f"[bench] dense FFN T={dw.T} I={dw.Is}")
        rec["workloads"]["dense_ffn"] = measure_dense(dw, moe, synth, 10, 3)
        log(f"[bench] dense: {rec['workloads']['dense_ffn']['ms_per_step']:.4f} ms/step")

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
