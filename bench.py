"""Benchmark of the SMOE routed-expert MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--copies C]
    python bench.py --workload quantise_qwen235b_expert_q4   (the GPU quantiser)
    python bench.py --workload qwen235b_q4_b1_offload_direct  (experts in host memory)

A step is one full forward of the layer (route, group, gate/up + SwiGLU, down,
combine; a stack of layers for the stacked workload) on synthetic inputs that
are resident in HBM before timing starts. Expert banks are replicated into C
distinct copies and consecutive steps rotate through them (and through
distinct router logits), so the working set of the timed loop is far larger
than the 256 MB Infinity Cache and every step reads its experts from HBM.

Prints one JSON line (metric, value = tokens/s, roofline of the dominant
kernel, CPU-oracle baseline on a bounded sample).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (% of peak), Qwen3-235B-shape Q4"
HBM_PEAK_GBPS = 8000.0
# dense fp16 matrix-core peak (the prefill-sized stages multiply fp16 pairs)
MFMA_F16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="qwen235b_q4_b1")
    ap.add_argument("--copies", type=int, default=0,
                    help="distinct expert-bank copies to rotate through (0 = auto)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--trace-launches", type=int, default=400,
                    help="forwards per kernel in the per-launch timing pass (0 = skip)")
    ap.add_argument("--offload-slots", type=int, default=-1,
                    help="host-offload workloads: device cache slots (0 = direct reads; "
                         "-1 = the workload's default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for {args.gpus}); "
              "sharding is described in the design notes but not implemented", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.workload in QUANTISE_WORKLOADS:
        bench_quantise(args)
        return
    if args.workload in OFFLOAD_WORKLOADS:
        bench_offload(args)
        return
    import numpy as np
    import torch
    import synth
    import quantised_moe_expert_amd as smoe

    W = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    s_handle = stream.cuda_stream
    lay = smoe.smoe_expert_layout_of(W.d_model, W.ffn_dim, W.bits, smoe.SMOE_SCALE_F32)
    stride = lay.padded_size
    raw = lay.raw_size
    stack = W.n_layers > 1
    copies = args.copies or (W.n_layers if stack else (16 if W.n_tokens == 1 else 8))
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def make_bank(E, ffn, layout, stride_):
        """E experts at `stride_`: uniform code bytes, lognormal fp32 scales,
        zero padding; offsets from the library's layout query."""
        bank = smoe.aligned_buffer(E * stride_, device=dev).view(E, stride_)
        bank.random_(0, 256, generator=gen)
        for t in (layout.gate, layout.up, layout.down):
            sc = bank[:, t.scales_offset: t.scales_offset + t.scales_bytes].view(torch.float32)
            sc.copy_(torch.empty(sc.shape, device=dev).log_normal_(
                math.log(0.02), 0.5, generator=gen))
        bank[:, layout.raw_size:] = 0
        return bank

    banks, handles = [], []
    shared_blobs = []
    for c in range(copies):
        bank = make_bank(W.num_experts, W.ffn_dim, lay, stride)
        sh = None
        sh_bytes = 0
        if W.shared_ffn_dim:
            sl = smoe.smoe_expert_layout_of(W.d_model, W.shared_ffn_dim, W.bits,
                                            smoe.SMOE_SCALE_F32)
            sh = make_bank(1, W.shared_ffn_dim, sl, sl.padded_size).reshape(-1)
            sh_bytes = sh.numel()
            shared_blobs.append(sh)
        desc = smoe.make_desc(W.d_model, W.ffn_dim, W.num_experts, W.bits, stride,
                              smoe.SMOE_SCALE_F32, W.shared_ffn_dim)
        handles.append(smoe.smoe_load_blobs(desc, bank.data_ptr(), bank.numel(),
                                            sh.data_ptr() if sh is not None else 0, sh_bytes))
        banks.append(bank)
    T, E, k = W.n_tokens, W.num_experts, W.top_k
    n_logit_sets = 64
    lg_sets = torch.randn((n_logit_sets, W.n_layers, T, E), device=dev, generator=gen)
    if W.x_dtype == "bf16":
        x = torch.randn((T, W.d_model), device=dev, generator=gen).to(torch.bfloat16)
        x_dt = smoe.SMOE_DTYPE_BF16
    else:
        x = torch.randn((T, W.d_model), device=dev, generator=gen)
        x_dt = smoe.SMOE_DTYPE_F32
    h_state = torch.randn((T, W.d_model), device=dev, generator=gen) if stack else None
    out = torch.empty((T, W.d_model), dtype=torch.float32, device=dev)
    nws = smoe.smoe_workspace_bytes(handles[0], T, k)
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)

    # unique experts each step reads (algorithmic bytes); uniq0: layer 0 only
    top = torch.topk(lg_sets, k, dim=-1).indices  # [S, L, T, k]
    uniq, uniq0 = [], []
    for s in range(n_logit_sets):
        uniq.append(sum(int(torch.unique(top[s, l]).numel()) for l in range(W.n_layers)))
        uniq0.append(int(torch.unique(top[s, 0]).numel()))
    shared_raw = 0
    if W.shared_ffn_dim:
        shared_raw = smoe.smoe_expert_layout_of(W.d_model, W.shared_ffn_dim, W.bits,
                                                smoe.SMOE_SCALE_F32).raw_size
    act_bytes = W.n_layers * (T * W.d_model * (2 if W.x_dtype == "bf16" else 4)
                              + T * E * 4 + T * W.d_model * 4)

    def step(i):
        c = i % copies
        s = i % n_logit_sets
        if stack:
            smoe.smoe_decode_step(handles, h_state.data_ptr(), lg_sets[s].data_ptr(), T, k,
                                  W.norm_topk_prob, 1e-6, ws.data_ptr(), nws, s_handle)
        else:
            smoe.smoe_moe_forward(handles[c], x.data_ptr(), x_dt, lg_sets[s, 0].data_ptr(), T, k,
                                  W.norm_topk_prob, out.data_ptr(), 0, 0, ws.data_ptr(), nws,
                                  s_handle)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if stack:
        h_state.normal_(generator=gen)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    tokens_per_s = T / (ms * 1e-3)
    bytes_per_step = []
    for i in range(args.steps):
        s = (args.warmup + i) % n_logit_sets
        bytes_per_step.append(uniq[s] * raw + W.n_layers * shared_raw + act_bytes)
    alg_bytes = sum(bytes_per_step) / len(bytes_per_step)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    pairs = T * k * W.n_layers
    avg_unique = sum(uniq[(args.warmup + i) % n_logit_sets] for i in range(args.steps)) / args.steps

    # per-launch timing of the two expert kernels: HIP events recorded by the
    # library immediately around the launch, on the launch's stream, one pair
    # per forward, in a pass of its own after the timed loop
    single = T == 1 and not W.shared_ffn_dim
    x_bytes = T * W.d_model * (2 if W.x_dtype == "bf16" else 4)
    gu_raw = sum(t.codes_bytes + t.scales_bytes for t in (lay.gate, lay.up))
    dn_raw = lay.down.codes_bytes + lay.down.scales_bytes
    # a shared expert whose ffn is a multiple of the routed ffn runs inside the
    # routed launches (as shared_ffn / ffn more slots of all T tokens) unless
    # the call takes the K-sliced stages (24 or more pairs per slot on average)
    nsh, sh_gu, sh_dn = 0, 0, 0
    if W.shared_ffn_dim and W.shared_ffn_dim % W.ffn_dim == 0:
        q = W.shared_ffn_dim // W.ffn_dim
        if q <= 16 and (T * k + q * T) // (min(T * k, E) + q) < 24:
            nsh = q
            sl = smoe.smoe_expert_layout_of(W.d_model, W.shared_ffn_dim, W.bits,
                                            smoe.SMOE_SCALE_F32)
            sh_gu = sum(t.codes_bytes + t.scales_bytes for t in (sl.gate, sl.up))
            sh_dn = sl.down.codes_bytes + sl.down.scales_bytes
    h_bytes = (T * k + nsh * T) * W.ffn_dim * 4
    start = args.warmup + args.steps
    # does this layer have a separate down-projection launch?
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    eb.record(stream)
    torch.cuda.synchronize()
    smoe.smoe_trace_kernel(smoe.SMOE_KERNEL_DOWN, int(ea.cuda_event), int(eb.cuda_event))
    step(start)
    torch.cuda.synchronize()
    separate_down = smoe.smoe_trace_kernel(smoe.SMOE_KERNEL_NONE) == 0
    start += 1
    out_b = T * W.d_model * 4 * (2 if stack else 1)  # read-modify-write in a stack
    kern = {}
    if args.trace_launches > 0:
        passes = [("gate_up", smoe.SMOE_KERNEL_GATE_UP)]
        if separate_down:
            passes.append(("down", smoe.SMOE_KERNEL_DOWN))
        for name, kid in passes:
            n = args.trace_launches
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
            for a, b in evs:  # creates the events
                a.record(stream)
                b.record(stream)
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(evs):
                smoe.smoe_trace_kernel(kid, int(a.cuda_event), int(b.cuda_event))
                step(start + i)
            torch.cuda.synchronize()
            smoe.smoe_trace_kernel(smoe.SMOE_KERNEL_NONE)
            dts = [a.elapsed_time(b) * 1e-3 for a, b in evs]  # s
            u = [uniq0[(start + i) % n_logit_sets] for i in range(n)]
            if name == "gate_up":
                byts = [ui * gu_raw + sh_gu + x_bytes + T * E * 4 + h_bytes for ui in u]
            else:
                # the grouped down stage writes one row per pair for the
                # combine; the one-token and 1-4-token stages write out
                y_b = out_b if T <= 4 else (T * k + nsh * T) * W.d_model * 4
                byts = [ui * dn_raw + h_bytes + out_b if single else
                        ui * dn_raw + sh_dn + h_bytes + y_b
                        for ui in u]
            mean_dt = sum(dts) / n
            mean_b = sum(byts) / n
            kern[name] = {"mean_us": mean_dt * 1e6, "median_us": sorted(dts)[n // 2] * 1e6,
                          "bytes": mean_b, "GBps": mean_b / mean_dt / 1e9}
            start += n
    if single:
        names = {"gate_up": "k_dec_gate_up (routing + gate/up + SwiGLU)",
                 "down": "k_dec_down (down projection + weighted combine)"}
    elif T <= 4:
        names = {"gate_up": "k_sb_gate_up (routing + grouping + gate/up + SwiGLU)",
                 "down": "k_sb_down (down projection + weighted combine)"}
    else:
        names = {"gate_up": "k_gate_up (grouped gate/up + SwiGLU over the routed pairs)",
                 "down": "k_down (grouped down projection)"}
    dom = kern.get("gate_up")
    traffic = committed_traffic(W.name, "gate_up" if single else
                                ("gate_up_small" if T <= 4 else "gate_up_grouped"))
    # the gate/up launch's contraction: two flops per weight per routed pair
    # (one layer per launch); the roofline is whichever peak bounds it first
    gu_flops = (T * k + nsh * T) * 4 * W.d_model * W.ffn_dim
    roof = {"bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": None}
    if dom:
        dt = dom["mean_us"] * 1e-6
        hbm_frac = dom["bytes"] / dt / 1e9 / HBM_PEAK_GBPS
        mfma_frac = gu_flops / dt / 1e12 / MFMA_F16_PEAK_TFLOPS
        if mfma_frac > hbm_frac:
            roof.update(bound="mfma", achieved=round(gu_flops / dt / 1e12, 1),
                        peak=MFMA_F16_PEAK_TFLOPS, unit="TFLOP/s", frac=round(mfma_frac, 4))
        else:
            roof.update(achieved=round(dom["GBps"], 1), frac=round(hbm_frac, 4))
        roof.update(hbm_frac=round(hbm_frac, 4), mfma_frac=round(mfma_frac, 4))
    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": W.name, "d_model": W.d_model, "ffn_dim": W.ffn_dim,
            "num_experts": E, "top_k": k, "n_tokens": T, "bits": W.bits,
            "group_size": 64, "scale_dtype": "f32", "x_dtype": W.x_dtype,
            "norm_topk_prob": W.norm_topk_prob, "shared_ffn_dim": W.shared_ffn_dim,
            "n_layers": W.n_layers, "bank_copies_rotated": copies,
        },
        "hbm_GBps": round(achieved, 1),
        "pct_of_hbm_peak": round(100 * achieved / HBM_PEAK_GBPS, 2),
        "expert_reads_per_s": round(avg_unique / (ms * 1e-3), 1),
        "pairs_per_s": round(pairs / (ms * 1e-3), 1),
        "wall_s_timed": round(t_wall, 3),
        "algorithmic_bytes_per_step": int(alg_bytes),
        "roofline": {
            "bound": roof["bound"],
            "kernel": names["gate_up"],
            "achieved": roof["achieved"],
            "peak": roof["peak"],
            "unit": roof["unit"],
            "frac": roof["frac"],
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(dom["bytes"]) if dom else None,
            "algorithmic_flops_per_launch": gu_flops,
            "hbm_frac": roof.get("hbm_frac"),
            "mfma_frac": roof.get("mfma_frac"),
            "launch_us_mean": round(dom["mean_us"], 3) if dom else None,
            "launch_us_median": round(dom["median_us"], 3) if dom else None,
            "launches_timed": args.trace_launches,
        },
        "kernels": {names[n]: {"launch_us_mean": round(v["mean_us"], 3),
                               "algorithmic_bytes_per_launch": int(v["bytes"]),
                               "GBps": round(v["GBps"], 1)} for n, v in kern.items()},
    }
    if dom and args.trace_launches > 0:
        sizes = [int(dom["bytes"]), int(alg_bytes)]
        if "down" in kern:
            sizes.append(int(kern["down"]["bytes"]))
        ceil = stream_ceiling(sizes, args.trace_launches)
        c_gu = ceil[sizes[0] // 16 * 16]
        c_step = ceil[sizes[1] // 16 * 16]
        sc = {
            "method": "libsmoe_stream.so read kernel, event pair per launch, best of "
                      "normal/non-temporal loads x 256-2048 workgroups, windows rotated "
                      "over 2 GiB",
            "gate_up_bytes": sizes[0], "gate_up_us": round(c_gu, 3),
            "step_bytes_one_launch": sizes[1], "step_one_launch_us": round(c_step, 3),
        }
        result["roofline"]["stream_ceiling_us"] = round(c_gu, 3)
        result["roofline"]["pct_of_stream_ceiling"] = round(100 * c_gu / dom["mean_us"], 2)
        if "down" in kern:
            c_dn = ceil[sizes[2] // 16 * 16]
            sc.update(down_bytes=sizes[2], down_us=round(c_dn, 3),
                      down_pct_of_stream_ceiling=round(100 * c_dn / kern["down"]["mean_us"], 2))
        result["stream_ceiling"] = sc
        result["pct_of_stream_ceiling"] = round(100 * c_step / (ms * 1e3), 2)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, W, banks[0], stride, lg_sets[0, 0], x,
                                              shared_blobs[0] if shared_blobs else None)
    print(json.dumps(result), flush=True)
    for h in handles:
        smoe.smoe_free(h)


# GPU quantiser ("SMOE Quantisation", L2-MSE Scale Optimiser): one expert's
# three projections (gate and up [ffn, d], down [d, ffn]) per step.
QUANTISE_WORKLOADS = {
    "quantise_qwen235b_expert_q4": (4096, 1536, 4, "f16"),
    "quantise_qwen235b_expert_q2": (4096, 1536, 2, "f16"),
}
# fp64 operations of the squared-error search per weight: for each of the 64
# candidates, encode (divide, multiply, add, round, two clamp compares) and
# score (subtract, divide, multiply, subtract, multiply, add)
QUANT_OPS_PER_WEIGHT = 64 * 12
# fp64 vector issue: 256 CUs x 64 lanes per clock x 2.4 GHz, one operation
# per lane per clock (78.6 TFLOP/s counts a fused multiply-add as two)
FP64_OPS_PEAK_T = 256 * 64 * 2.4e9 / 1e12


def bench_quantise(args):
    """Quantiser throughput: K steps, each quantising one expert (three
    launches, fp32 weights resident in HBM, codes and scales written into an
    expert blob); per-launch HIP events on the launch stream."""
    import numpy as np
    import torch
    import synth
    import quantised_moe_expert_amd as smoe

    d, ffn, bits, sdt = QUANTISE_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    sd = smoe.SMOE_SCALE_F16 if sdt == "f16" else smoe.SMOE_SCALE_F32
    lay = smoe.smoe_expert_layout_of(d, ffn, bits, sd)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    tensors = [lay.gate, lay.up, lay.down]
    copies = 4
    ws = []
    for _ in range(copies):  # N(0, 0.02^2) weights, 1 % of them x10
        per = []
        for t in tensors:
            w = torch.randn(t.rows * t.cols, device=dev, generator=gen) * 0.02
            m = torch.rand(w.shape, device=dev, generator=gen) < 0.01
            per.append(torch.where(m, w * 10, w))
        ws.append(per)
    blob = torch.zeros(lay.padded_size, dtype=torch.uint8, device=dev)
    n_w = sum(t.rows * t.cols for t in tensors)

    def step(i, evs=None):
        for j, (t, w) in enumerate(zip(tensors, ws[i % copies])):
            if evs is not None:
                evs[j][0].record(stream)
            smoe.smoe_quantise(w.data_ptr(), w.numel(), bits, sd, blob.data_ptr() + t.codes_offset,
                               blob.data_ptr() + t.scales_offset, sh)
            if evs is not None:
                evs[j][1].record(stream)

    steps = min(args.steps, 200)
    for i in range(min(args.warmup, 10)):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n_l = 60
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(3)] for _ in range(n_l)]
    for i in range(n_l):
        step(i, evs[i])
    torch.cuda.synchronize()
    launch_s = sum(a.elapsed_time(b) for ev in evs for a, b in ev) * 1e-3 / (3 * n_l)
    per_launch_ops = (n_w / 3) * QUANT_OPS_PER_WEIGHT
    achieved = per_launch_ops / launch_s / 1e12
    result = {
        "metric": "quantised weights/s (GPU squared-error scale search, Qwen3-235B-shape expert)",
        "value": round(n_w / (ms * 1e-3), 1),
        "unit": "weights/s",
        "n_gpus": 1, "steps": steps, "warmup": min(args.warmup, 10),
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": args.workload, "d_model": d, "ffn_dim": ffn, "bits": bits,
                   "scale_dtype": sdt, "group_size": 64, "weights_per_step": n_w},
        "experts_per_s": round(1e3 / ms, 2),
        "roofline": {
            "bound": "alu", "kernel": "k_quantise (one wave per group, one lane per candidate)",
            "achieved": round(achieved, 3), "peak": round(FP64_OPS_PEAK_T, 2),
            "unit": "Tops/s (fp64 vector operations)", "frac": round(achieved / FP64_OPS_PEAK_T, 4),
            "traffic": None, "algorithmic_ops_per_launch": int(per_launch_ops),
            "launch_us_mean": round(launch_s * 1e6, 3), "launches_timed": 3 * n_l,
        },
    }
    if not args.no_cpu_baseline:
        import oracle as O
        from threadpoolctl import threadpool_info
        w0 = ws[0][0].cpu().numpy()
        t0 = time.perf_counter()
        n_g = 0
        while time.perf_counter() - t0 < args.cpu_baseline_seconds and n_g < w0.size // 64:
            O.mse_grid_scale(w0[n_g * 64:(n_g + 1) * 64], bits, sdt)
            n_g += 1
        dt = time.perf_counter() - t0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        result["cpu_baseline"] = {
            "value": round(n_g * 64 / dt, 1), "unit": "weights/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n_g} groups of the gate tensor through the oracle's scale search, "
                      f"{dt:.1f} s, host cpu_count={os.cpu_count()}"}
    print(json.dumps(result), flush=True)


# Host offload: the one-token Qwen3-235B-shape Q4 layer with its 128 experts in
# pinned host memory (1.36 GB), new routing every step; (workload, default
# cache slots): 0 = the kernels read the experts over PCIe, > 0 = an LRU
# device cache of that many blobs, misses copied by DMA.
OFFLOAD_WORKLOADS = {
    "qwen235b_q4_b1_offload_direct": 0,
    "qwen235b_q4_b1_offload_cache32": 32,
}
# PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 coding
PCIE_PEAK_GBPS = 32 * 16 * 128 / 130 / 8


def bench_offload(args):
    import torch
    import synth
    import quantised_moe_expert_amd as smoe

    W = synth.WORKLOADS["qwen235b_q4_b1"]
    slots = OFFLOAD_WORKLOADS[args.workload] if args.offload_slots < 0 else args.offload_slots
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    lay = smoe.smoe_expert_layout_of(W.d_model, W.ffn_dim, W.bits, smoe.SMOE_SCALE_F32)
    stride, raw, E, k = lay.padded_size, lay.raw_size, W.num_experts, W.top_k
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    host = smoe.aligned_buffer(E * stride, pin_memory=True).view(E, stride)
    for e in range(E):  # uniform code bytes, lognormal fp32 scales, zero padding
        b = torch.randint(0, 256, (stride,), dtype=torch.uint8, device=dev, generator=gen)
        for t in (lay.gate, lay.up, lay.down):
            sc = b[t.scales_offset: t.scales_offset + t.scales_bytes].view(torch.float32)
            sc.copy_(torch.empty(sc.shape, device=dev).log_normal_(math.log(0.02), 0.5,
                                                                   generator=gen))
        b[raw:] = 0
        host[e].copy_(b)
    torch.cuda.synchronize()
    cache = smoe.aligned_buffer(max(slots, 1) * stride, device=dev)
    table = torch.zeros(E, dtype=torch.int64, device=dev)
    desc = smoe.make_desc(W.d_model, W.ffn_dim, E, W.bits, stride, smoe.SMOE_SCALE_F32)
    off = smoe.smoe_offload_create(desc, host.data_ptr(), host.numel(), 0, 0,
                                   cache.data_ptr() if slots else 0, slots * stride,
                                   table.data_ptr())
    n_sets = 64
    lg = torch.randn((n_sets, 1, E), device=dev, generator=gen)
    x = torch.randn((1, W.d_model), device=dev, generator=gen).to(torch.bfloat16)
    out = torch.empty((1, W.d_model), dtype=torch.float32, device=dev)
    nws = smoe.smoe_offload_workspace_bytes(off, 1, k)
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)

    def step(i):
        smoe.smoe_offload_forward(off, x.data_ptr(), smoe.SMOE_DTYPE_BF16, lg[i % n_sets].data_ptr(),
                                  1, k, True, out.data_ptr(), 0, 0, ws.data_ptr(), nws, sh)

    steps = min(args.steps, 500)
    warm = min(args.warmup, 50)
    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    st0 = smoe.smoe_offload_get_stats(off)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(warm + i)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    st1 = smoe.smoe_offload_get_stats(off)
    ms = e0.elapsed_time(e1) / steps
    # bytes over PCIe per step: every selected expert (direct) or the misses
    # (copied) plus the experts read directly for want of a slot
    if slots == 0:
        pcie_bytes = k * raw
    else:
        pcie_bytes = ((st1.bytes_fetched - st0.bytes_fetched)
                      + (st1.direct - st0.direct) * raw) / steps
    achieved = pcie_bytes / (ms * 1e-3) / 1e9
    # a plain 256 MiB pinned host -> device copy: what the link gives a DMA
    src = torch.empty(1 << 28, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    for _ in range(2):
        dst.copy_(src, non_blocking=True)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src, non_blocking=True)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 5 * (1 << 28) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    hits = st1.hits - st0.hits
    fetched = st1.fetched - st0.fetched
    result = {
        "metric": "MoE-layer tokens/s with the routed experts in host memory (PCIe GB/s)",
        "value": round(1e3 / ms, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": args.workload, "d_model": W.d_model, "ffn_dim": W.ffn_dim,
                   "num_experts": E, "top_k": k, "n_tokens": 1, "bits": W.bits,
                   "scale_dtype": "f32", "cache_slots": slots,
                   "host_bank_bytes": E * stride},
        "pcie_bytes_per_step": int(pcie_bytes),
        "cache_hit_rate": round(hits / max(1, hits + fetched + (st1.direct - st0.direct)), 4),
        "copy_GBps_measured": round(copy_gbps, 2),
        "wall_s_timed": round(t_wall, 3),
        "roofline": {
            "bound": "pcie", "kernel": "whole forward (host-to-device traffic)",
            "achieved": round(achieved, 2), "peak": round(PCIE_PEAK_GBPS, 2), "unit": "GB/s",
            "frac": round(achieved / PCIE_PEAK_GBPS, 4), "traffic": None,
        },
    }
    print(json.dumps(result), flush=True)
    smoe.smoe_offload_free(off)


KERNEL_SOURCES = {
    "gate_up": ("smoe_decode.hpp", "smoe_decode_args.hpp", "smoe_device.hpp"),
    "gate_up_small": ("smoe_small.hpp", "smoe_small_args.hpp", "smoe_decode.hpp",
                      "smoe_decode_args.hpp", "smoe_device.hpp"),
    "gate_up_grouped": ("smoe_gemm.hpp", "smoe_gemv_args.hpp", "smoe_device.hpp"),
}


def kernel_sources_digest(kernel: str) -> str:
    """sha256 over the device sources of a kernel, so a committed counter
    reading can be matched to the code it was taken on."""
    import hashlib
    d = os.path.join(ROOT, "quantised_moe_expert_amd", "csrc")
    hsh = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(d, f), "rb") as fh:
            hsh.update(f.encode() + b"\0" + fh.read())
    return hsh.hexdigest()[:16]


def committed_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (profiles/traffic.txt: FETCH_SIZE + WRITE_SIZE per dispatch, scaled
    by the plain-copy calibration), or None when there is none for this
    workload and kernel or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    digest = kernel_sources_digest(kernel)
    with open(path) as fh:
        for line in fh:
            f = line.split()
            if len(f) == 4 and f[0] == workload and f[1] == kernel and f[2] == digest:
                return float(f[3])
    return None


def stream_ceiling(sizes, trace_n):
    """Streaming-read ceiling for each byte count in `sizes`: the mean launch
    time of libsmoe_stream.so's plain read kernel over that many bytes, timed
    exactly as the layer kernels are (an event pair around each launch on the
    launch stream), the best over normal / non-temporal loads and 256 to 2048
    workgroups. Every launch reads a different window of a 2 GiB buffer, so
    nothing is served from the 256 MB Infinity Cache. Returns {bytes: us}."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "quantised_moe_expert_amd", "libsmoe_stream.so"))
    lib.smoe_stream_read.restype = ctypes.c_int
    lib.smoe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    big = max(int(b) for b in sizes)
    pool = torch.ones(max(2 << 30, 4 * big + (1 << 20)), dtype=torch.uint8, device=dev)
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    n = max(trace_n, 20)
    out = {}
    for nbytes in sizes:
        nbytes = int(nbytes) // 16 * 16
        span = (nbytes + 16383) // 16384 * 16384
        windows = (pool.numel() - span) // span
        best = None
        for nt in (0, 1):
            for nwg in (256, 512, 1024, 2048):
                evs = [(torch.cuda.Event(enable_timing=True),
                        torch.cuda.Event(enable_timing=True)) for _ in range(n)]
                for j in range(-8, n):  # eight untimed launches first
                    src = pool.data_ptr() + (j % windows) * span
                    if j >= 0:
                        evs[j][0].record(stream)
                    rc = lib.smoe_stream_read(src, nbytes, sink.data_ptr(), nwg, nt,
                                              stream.cuda_stream)
                    if rc:
                        raise RuntimeError(f"smoe_stream_read failed ({rc})")
                    if j >= 0:
                        evs[j][1].record(stream)
                torch.cuda.synchronize()
                us = sum(a.elapsed_time(b) for a, b in evs) / n * 1e3
                if best is None or us < best:
                    best = us
        out[nbytes] = best
    del pool
    return out


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, five times: under rocprofv3
    --pmc its FETCH_SIZE / WRITE_SIZE per dispatch, divided by 1 GiB, are the
    counters' scale factors."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4, "copies": 5}), flush=True)


def cpu_baseline(args, W, bank, stride, logits, x, shared_blob):
    """The oracle, as it stands, on host cores: repeated single-layer forwards
    of the same workload (tokens of the first logit set, first bank copy) for
    about --cpu-baseline-seconds with every core the BLAS pool uses, then as
    long again on one thread."""
    import numpy as np
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits

    lg = logits.float().cpu().numpy()
    xs = x.float().cpu().numpy()
    T, k = W.n_tokens, W.top_k
    # only the selected experts are copied to the host
    sel = sorted({e for t in range(T) for e in O.route(lg[t], k, W.norm_topk_prob)[0]})
    blobs = {e: bank[e].cpu().numpy() for e in sel}
    sh = shared_blob.cpu().numpy() if shared_blob is not None else None
    layer = O.OracleLayer(W.d_model, W.ffn_dim, W.num_experts, W.bits, None, stride,
                          "f32", W.shared_ffn_dim, sh, expert_blobs=blobs)

    def leg():
        t0 = time.perf_counter()
        n_tok = 0
        while True:
            layer.drop_cache()
            for t in range(T):
                O.moe_forward(layer, xs[t:t + 1], lg[t:t + 1], k, W.norm_topk_prob)
                n_tok += 1
                if time.perf_counter() - t0 > args.cpu_baseline_seconds:
                    break
            if time.perf_counter() - t0 > args.cpu_baseline_seconds:
                break
        return n_tok, time.perf_counter() - t0

    n_tok, dt = leg()
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    with threadpool_limits(limits=1):
        n1, dt1 = leg()
    return {
        "value": round(n_tok / dt, 4),
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{n_tok} token forwards of one {W.name} layer (experts dequantised "
                   f"from the blob bytes per forward), {dt:.1f} s, "
                   f"host cpu_count={os.cpu_count()}"),
        "single_thread": {"value": round(n1 / dt1, 4), "unit": "tokens/s", "cores": 1,
                          "sample": f"{n1} token forwards, {dt1:.1f} s, BLAS pool limited "
                                    "to one thread"},
    }


if __name__ == "__main__":
    main()
