"""Throughput of the W4 mixture-of-experts layer on one MI355X.

``python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]``

One step is one whole layer (router when the workload has one, top-k
routing, histogram / scan / scatter / block map, the two grouped W4 GEMMs
with SwiGLU, and the combine) over one batch of T synthetic tokens, enqueued
by ``moe_ffn_forward`` on one stream.  Each step is timed two ways, eager
(the host enqueues every step's kernels, running ahead of the GPU) and as a
replay of a HIP graph captured once per weight copy / logit set; ``value``
uses the faster (``config.launch``), and both are in the line
(``--no-graph`` times eager launches only).
Inputs are resident in HBM before timing starts.  Weights are rotated over enough device copies of the
layer (>= 1 GiB in total) that every step reads its experts cold from HBM
rather than from the 256 MB Infinity Cache; decode workloads also rotate
over a pool of independent logit sets, so the touched experts change every
step.

Prints one JSON line.  ``value`` is tokens/s = T * K / (elapsed of the K
timed steps).  ``roofline`` is for the kernel with the largest average
duration among the stages that stream the layer's bulk data (the two
grouped GEMMs and the combine), from its algorithmic bytes (or flops) per
launch and its average duration between the stage events
recorded on its own stream (``moe_ffn_forward_timed``) over a second,
eager pass of the same steps.  ``cpu_baseline`` times
the CPU oracle on a bounded sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4 MoE-layer tokens/s at T=512 & 8192 prefill, T=1/8 decode; % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 MFMA
ROTATE_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_t512")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no HIP graph replays)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle sample")
    ap.add_argument("--ablation", choices=["host_blockmap", "unfused"], default=None,
                    help="also time the layer with the block map built on the host (a stream "
                         "synchronisation and copies mid-layer), against the same layer eager")
    ap.add_argument("--io", action="store_true",
                    help="also time the layer with the steps around it (moe_ffn_forward_io: "
                         "RMSNorm in front, bf16 residual sum behind), against the layer alone")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one plain device copy of 256 MiB, the reference "
                         "kernel for scaling HBM byte counters")
    return ap.parse_args()


# ------------------------------------------------------------------ work --
def expert_bytes(lay) -> dict:
    """Packed bytes per expert of each bank: codes (4 bits each) + bf16
    scale and bias per group."""
    H, I, G = lay.H, lay.I, lay.G
    bank = lambda N, K: N * K // 2 + 2 * 2 * N * K // G
    return {"gate_up": 2 * bank(lay.I, lay.H), "down": bank(lay.H, lay.I)}


def algorithmic(lay, touched: int) -> dict:
    """Bytes each single-kernel stage must move at minimum given its inputs
    and outputs, and its flops.  P = T * k pairs."""
    T, H, I, E, k = lay.T, lay.H, lay.I, lay.E, lay.k
    P = T * k
    eb = expert_bytes(lay)
    yb = 4 if T <= 8 else 3  # weighted expert outputs: fp32 (GEMV path) or packed 24-bit
    return {
        # x (fp16 operand copy) read + touched experts' gate and up banks + h fp16 written
        "gate_up": dict(bytes=touched * eb["gate_up"] + T * H * 2 + P * I * 2,
                        flops=4 * P * H * I),
        # h read + touched experts' down bank + weighted y_sorted written
        "down": dict(bytes=touched * eb["down"] + P * I * 2 + P * H * yb, flops=2 * P * H * I),
        # y_sorted read + pair_slot read + y written
        "combine": dict(bytes=P * H * yb + P * 4 + T * H * 4, flops=P * H),
        # x bf16 read + fp16 copy written, logits (or router weight) read,
        # ids / weights written
        "route": dict(bytes=T * H * 2 * 2 + (E * H * 2 + T * E * 4 if lay.router_weight is not None
                                            else T * E * 4) + P * 8,
                      flops=2 * T * H * E if lay.router_weight is not None else 0),
        # ids read, sorted_pairs / pair_slot written
        "build_blocks": dict(bytes=P * 4 * 3, flops=0),
    }


def layer_work(lay, touched: int) -> dict:
    """The whole layer's algorithmic flops and bytes: touched experts'
    packed weights, x, the logits or router weight, and y."""
    T, H, I, E, k = lay.T, lay.H, lay.I, lay.E, lay.k
    eb = expert_bytes(lay)
    flops = 6 * T * k * H * I + (2 * T * H * E if lay.router_weight is not None else 0)
    byts = touched * (eb["gate_up"] + eb["down"]) + T * H * 2 + T * H * 4
    byts += E * H * 2 if lay.router_weight is not None else T * E * 4
    return dict(flops=flops, bytes=byts)


# ---------------------------------------------------------- traffic file --
def kernel_source_digest(stage: str = "gate_up") -> str:
    """Digest of the sources the stage's kernels are built from (the grouped
    GEMM kernels, or the decode-attention kernels)."""
    h = hashlib.sha256()
    files = (("quantized_moe_top_amd/csrc/attn.hip",) if stage == "attention" else
             ("quantized_moe_top_amd/csrc/gemm.hip", "quantized_moe_top_amd/csrc/gemv.hip"))
    for rel in files + ("quantized_moe_top_amd/csrc/internal.h",):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch of `stage` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy kernel's reading), or
    None when there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_digest") != kernel_source_digest(stage):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ main --
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is "
              "measured at one GPU's share and nothing here uses a second GPU.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_moe_top_amd import _lib, api, synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    _lib.load()  # raises when the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    name = args.workload
    if name in synth.ATTN_WORKLOADS:
        return bench_attention(args, name, dev)
    log(f"[bench] drawing workload {name}")
    host = synth.make_layer(name)
    # the banks are packed once into the kernels' layout (load time, untimed)
    lay = api.pack_layer(host.to(dev))
    torch.cuda.synchronize()
    T, E, k = lay.T, lay.E, lay.k

    # weight copies for cold reads
    nbytes = lambda b: (b.words.numel() + b.sb.numel()) * 4
    per_copy = nbytes(lay.gate) + nbytes(lay.up) + nbytes(lay.down) + \
        (lay.router_weight.numel() * 2 if lay.router_weight is not None else 0)
    R = max(1, -(-ROTATE_BYTES // per_copy))
    copies = [lay]
    for _ in range(R - 1):
        gate, up, down = (dataclasses.replace(b, words=b.words.clone(), sb=b.sb.clone())
                          for b in (lay.gate, lay.up, lay.down))
        wr = lay.router_weight.clone() if lay.router_weight is not None else None
        copies.append(dataclasses.replace(lay, gate=gate, up=up, down=down, router_weight=wr))
    logit_pool = None
    if lay.logits is not None and T <= 8:
        logit_pool = [lay.logits] + list(synth.decode_logits_pool(T, E, 63, seed=1000 + T).to(dev))
    log(f"[bench] {R} weight copies of {per_copy / 2**20:.1f} MiB; "
        f"logit sets {len(logit_pool) if logit_pool else 1}")

    y = torch.empty((T, lay.H), dtype=torch.float32, device=dev)
    wsb = api.ffn_workspace_bytes(lay)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    nst = _lib.MOE_NUM_STAGES

    def step(i, evs=None, info=False):
        c = copies[i % R]
        lg = logit_pool[i % len(logit_pool)] if logit_pool else None
        return api.ffn_forward(c, logits=lg, y=y, workspace=ws, stage_events=evs, info=info)

    # touched experts per step (for the algorithmic byte counts): routing is
    # identical for every copy; decode rotates logit sets
    touched = []
    for i in range(len(logit_pool) if logit_pool else 1):
        _, inf = step(i, info=True)
        touched.append(int((inf["counts"] > 0).sum().item()))
    torch.cuda.synchronize()

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graphs = None
    if not args.no_graph:
        # one graph per (weight copy, logit set) that the steps use
        n_graphs = len(logit_pool) if logit_pool else R
        graphs = []
        for i in range(n_graphs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(min(args.warmup, n_graphs) or 1):
            graphs[i % n_graphs].replay()
        torch.cuda.synchronize()

    def timed(run):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(K):
            run(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end), time.perf_counter() - t0

    # Two ways to launch the same layer on one stream: eager (the host
    # enqueues every kernel of every step, running ahead of the GPU) and HIP
    # graph replay (one launch per step; each replay has a fixed cost of its
    # own, see launch_floor_us).  Both are timed and the faster is reported:
    # eager wins when a step's GPU time hides the host's enqueueing (prefill),
    # replay when it does not (decode).
    log(f"[bench] timing {K} steps eager" + ("" if graphs is None else " and by graph replay"))
    eager_plain_ms, eager_wall = timed(lambda i: step(i))
    graph_ms = None
    if graphs is not None:
        graph_ms, graph_wall = timed(lambda i: graphs[i % len(graphs)].replay())
    if graph_ms is not None and graph_ms < eager_plain_ms:
        elapsed_ms, wall, launch = graph_ms, graph_wall, "hip_graph"
    else:
        elapsed_ms, wall, launch = eager_plain_ms, eager_wall, "eager"
    ms_per_step = elapsed_ms / K
    value = T * K / (elapsed_ms / 1e3)

    # launch floor: the same number of steps replaying a graph of one
    # one-element fill kernel (what a step of the layer costs at the very
    # least per kernel it launches)
    floor = torch.zeros(1, device=dev)
    gf = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gf):
        floor.fill_(1.0)
    gf.replay()
    floor_ms, _ = timed(lambda i: gf.replay())
    launch_floor_us = floor_ms / K * 1e3

    # per-stage durations: an eager pass of the same steps with events
    # recorded between the stages on the layer's stream
    ev = [api.stage_events(nst + 1) for _ in range(K)]
    eager_ms, _ = timed(lambda i: step(i, ev[i]))
    stage_ms = np.array([[ev[i][s].elapsed_time(ev[i][s + 1]) for s in range(nst)] for i in range(K)])
    stage_us = {st: round(float(stage_ms[:, j].mean()) * 1e3, 3) for j, st in enumerate(_lib.STAGES)}
    log(f"[bench] {ms_per_step * 1e3:.2f} us/step ({launch}; wall {wall / K * 1e6:.2f}; eager "
        f"{eager_plain_ms / K * 1e3:.2f}, graph {graph_ms / K * 1e3 if graph_ms else float('nan'):.2f}); "
        f"eager with stage events {eager_ms / K * 1e3:.2f} us/step; stages us {stage_us}")

    # roofline of the dominant single-kernel stage
    mean_touched = float(np.mean([touched[i % len(touched)] for i in range(K)]))
    alg = algorithmic(lay, 0)
    alg_t = {s: dict(bytes=algorithmic(lay, 1)[s]["bytes"] - alg[s]["bytes"], flops=alg[s]["flops"])
             for s in alg}  # bytes per touched expert
    # the stages that stream the layer's bulk data; routing and the block map
    # move a few KB per token (at decode sizes a single workgroup: latency,
    # not bandwidth) and are reported in stage_us only
    bulk = ["gate_up", "down", "combine"]
    dom = max(bulk, key=lambda s: stage_us[s])
    dur_s = stage_us[dom] * 1e-6
    byts = alg[dom]["bytes"] + mean_touched * alg_t[dom]["bytes"]
    flops = alg[dom]["flops"]
    hbm_time = byts / (HBM_PEAK_GBS * 1e9)
    mfma_time = flops / (MFMA_FP16_PEAK_TFLOPS * 1e12)
    if hbm_time >= mfma_time:
        achieved, peak, unit, bound = byts / dur_s / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    else:
        achieved, peak, unit, bound = flops / dur_s / 1e12, MFMA_FP16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    traffic = measured_traffic(name, dom)
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom,
                "algorithmic_bytes": int(byts), "algorithmic_flops": int(flops),
                "avg_launch_us": stage_us[dom]}
    lw = layer_work(lay, 0)
    lw_t = layer_work(lay, 1)["bytes"] - lw["bytes"]
    lbytes = lw["bytes"] + mean_touched * lw_t
    t_step = ms_per_step * 1e-3
    layer_roof = {"hbm_frac": round(lbytes / t_step / (HBM_PEAK_GBS * 1e9), 4),
                  "mfma_frac": round(lw["flops"] / t_step / (MFMA_FP16_PEAK_TFLOPS * 1e12), 4),
                  "bytes": int(lbytes), "flops": int(lw["flops"]), "touched_experts": mean_touched}

    ablations = None
    if args.ablation == "host_blockmap" and api.host_blockmap_ints(lay) > 0:
        # both eager (the host variant cannot be captured): the same kernels,
        # with and without the mid-layer round trip
        hb = torch.empty(api.host_blockmap_ints(lay), dtype=torch.int32, pin_memory=True)

        def step_host(i):
            c = copies[i % R]
            lg = logit_pool[i % len(logit_pool)] if logit_pool else None
            return api.ffn_forward(c, logits=lg, y=y, workspace=ws, host_blockmap=hb)

        for i in range(args.warmup):
            step_host(i)
        plain_ms, _ = timed(lambda i: step(i))
        host_ms, _ = timed(step_host)
        ablations = {"host_blockmap": {
            "ms_per_step": round(host_ms / K, 6),
            "eager_single_submission_ms_per_step": round(plain_ms / K, 6),
            "graph_single_submission_ms_per_step": round(graph_ms / K, 6) if graph_ms else None,
            "single_submission_speedup_eager": round(host_ms / plain_ms, 3)}}
        log(f"[bench] host block map: {host_ms / K * 1e3:.2f} us/step vs eager {plain_ms / K * 1e3:.2f} "
            f"and graph {ms_per_step * 1e3:.2f}")

    io_res = None
    if args.io:
        # the same steps plus RMSNorm in front and out = bf16(residual + y)
        # behind, eager, against the layer alone eager
        gio = torch.Generator().manual_seed(7)
        gamma = (torch.rand(lay.H, generator=gio) + 0.5).to(torch.bfloat16).to(dev)
        resid = torch.randn(T, lay.H, generator=gio).to(torch.bfloat16).to(dev)
        out_bf = torch.empty(T, lay.H, dtype=torch.bfloat16, device=dev)
        ws_io = torch.empty(api.ffn_io_workspace_bytes(lay), dtype=torch.uint8, device=dev)

        def step_io(i):
            c = copies[i % R]
            lg = logit_pool[i % len(logit_pool)] if logit_pool else None
            return api.ffn_forward(c, logits=lg, y=y, workspace=ws_io, norm_weight=gamma,
                                   residual=resid, out=out_bf)

        for i in range(args.warmup):
            step_io(i)
        plain_ms, _ = timed(lambda i: step(i))
        io_ms, _ = timed(step_io)
        io_res = {"ms_per_step": round(io_ms / K, 6), "eager_layer_ms_per_step": round(plain_ms / K, 6),
                  "added_us_per_step": round((io_ms - plain_ms) / K * 1e3, 3),
                  "tokens_per_s": round(T * K / (io_ms / 1e3), 1)}
        log(f"[bench] with RMSNorm + residual: {io_ms / K * 1e3:.2f} us/step vs layer alone "
            f"{plain_ms / K * 1e3:.2f}")

    if args.ablation == "unfused" and api.unfused_bytes(lay) > 0:
        # every step expands all experts' weights to fp16 in HBM, then the
        # grouped GEMMs stream those: eager, against the fused layer eager
        ex = torch.empty(api.unfused_bytes(lay), dtype=torch.uint8, device=dev)

        def step_unfused(i):
            c = copies[i % R]
            lg = logit_pool[i % len(logit_pool)] if logit_pool else None
            return api.ffn_forward(c, logits=lg, y=y, workspace=ws, expanded=ex)

        for i in range(args.warmup):
            step_unfused(i)
        plain_ms, _ = timed(lambda i: step(i))
        unf_ms, _ = timed(step_unfused)
        ablations = dict(ablations or {})
        ablations["unfused"] = {
            "ms_per_step": round(unf_ms / K, 6),
            "eager_fused_ms_per_step": round(plain_ms / K, 6),
            "fused_speedup": round(unf_ms / plain_ms, 3)}
        log(f"[bench] unfused dequant: {unf_ms / K * 1e3:.2f} us/step vs fused {plain_ms / K * 1e3:.2f}")

    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 268435456 bytes read and written")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": name, "T": T, "H": lay.H, "I": lay.I, "E": E, "top_k": k,
                   "group_size": lay.G, "router": "weight" if lay.router_weight is not None else "logits",
                   "weight_copies": R, "block_m": api.ffn_block_m(lay), "launch": launch},
        "roofline": roofline, "layer_roofline": layer_roof, "stage_us": stage_us,
        "eager_ms_per_step": round(eager_plain_ms / K, 6),
        "graph_ms_per_step": round(graph_ms / K, 6) if graph_ms else None,
        "eager_with_stage_events_ms_per_step": round(eager_ms / K, 6),
        "launch_floor_us": round(launch_floor_us, 3),
        "cpu_baseline": cpu,
    }
    if ablations:
        out["ablations"] = ablations
    if io_res:
        out["io"] = io_res
    print(json.dumps(out), flush=True)


def bench_attention(args, name: str, dev) -> None:
    """The second workload: one decode-attention step (one query token per
    sequence against its block-paged KV cache) per step, the cache rotated
    over copies that together exceed 1 GiB, so every step reads it from
    HBM.  Prints the same JSON line shape as the layer workloads."""
    import numpy as np
    import torch

    from quantized_moe_top_amd import api, synth

    host = synth.make_attention_workload(name)
    case = host.to(dev)
    B, Hq, D = case.q.shape
    NB, Hkv, BLK, _ = case.kcache.shape
    kv_bytes = 2 * int(host.lens.sum()) * Hkv * D * 2  # keys and values read once
    R = max(1, -(-ROTATE_BYTES // (2 * case.kcache.numel() * 2)))
    copies = [case] + [synth.AttnCase(name, case.q, case.kcache.clone(), case.vcache.clone(), case.table,
                                      case.lens, BLK) for _ in range(R - 1)]
    max_len = int(host.lens.max())
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, int(api._L().moe_decode_attention_workspace_bytes(B, Hq, Hkv, max_len))),
                     dtype=torch.uint8, device=dev)
    step = lambda i: api.decode_attention(copies[i % R], out=out, workspace=ws, max_len=max_len)
    log(f"[bench] {name}: B={B} context {max_len} Hq={Hq} Hkv={Hkv} D={D} block={BLK}; "
        f"{kv_bytes / 2**20:.1f} MiB of K and V per step, {R} copies")
    for i in range(args.warmup):
        step(i)
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 268435456 bytes read and written")
    byts = kv_bytes + B * Hq * D * (2 + 4)
    achieved = byts / (ms * 1e-3) / 1e9
    line = {
        "metric": "decode attention tokens/s (one query token per sequence, block-paged KV cache)",
        "value": round(B / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "B": B, "context": max_len, "Hq": Hq, "Hkv": Hkv, "D": D,
                   "block": BLK, "launch": "eager"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(name, "attention"),
                     "kernel": "attention", "launches": "attn_split_kernel + attn_combine_kernel (one step)",
                     "algorithmic_bytes": int(byts), "avg_launch_us": round(ms * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        t0 = time.perf_counter()
        reps = 0
        while True:
            orc.decode_attention(host.q, host.kcache, host.vcache, host.table, host.lens)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds or reps >= 20:
                break
        dt = (time.perf_counter() - t0) / reps
        line["cpu_baseline"] = {"value": round(B / dt, 3), "unit": "tokens/s", "cores": orc.num_threads(),
                                "kind": "oracle", "sample": f"{reps} whole steps, {reps * dt:.1f} s"}
    print(json.dumps(line), flush=True)


def cpu_baseline(host, min_seconds: float) -> dict:
    """The CPU oracle on the host cores: the whole layer on a sample of the
    tokens (all of them when T <= 512), with routing over every token;
    repeated until `min_seconds` of work.  Scaled to whole-layer tokens/s."""
    import numpy as np

    import oracle

    orc = oracle.get()
    T = host.T
    n = min(T, 512)
    tokens = np.linspace(0, T - 1, n).round().astype(np.int32) if n < T else np.arange(T, dtype=np.int32)
    log(f"[bench] cpu baseline: oracle on {n} of {T} tokens, {orc.num_threads()} threads")
    t_route = t_ffn = 0.0
    reps = 0
    while True:
        t0 = time.perf_counter()
        logits = (orc.router_logits(host.x, host.router_weight) if host.router_weight is not None
                  else np.ascontiguousarray(host.logits.numpy()))
        ids, w = orc.route(logits, host.k)
        orc.build_blocks(ids, host.E, 64)
        t1 = time.perf_counter()
        orc.ffn(host.x, ids, w, host.gate, host.up, host.down, host.G, tokens=tokens)
        t2 = time.perf_counter()
        t_route += t1 - t0
        t_ffn += t2 - t1
        reps += 1
        if t_route + t_ffn >= min_seconds or reps >= 50:
            break
    per_layer = t_route / reps + (t_ffn / reps) * T / n
    return {"value": round(T / per_layer, 2), "unit": "tokens/s", "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"{reps} x (routing of all {T} tokens + layer output of {n} tokens); "
                      f"{t_route + t_ffn:.1f} s of CPU work, scaled to the whole layer"}


if __name__ == "__main__":
    main()
