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
    ap.add_argument("--no-targets", action="store_true",
                    help="skip the decode and large-prefill workloads reported beside prefill_t512")
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
    # weighted expert outputs: fp32 (GEMV path), or int16 mantissas with an
    # exponent byte per 16 values
    yb = 4 if T <= 8 else 2 + 1 / 16
    return {
        # x (fp16 operand copy) read + touched experts' gate and up banks + h fp16 written
        "gate_up": dict(bytes=touched * eb["gate_up"] + T * H * 2 + P * I * 2,
                        flops=4 * P * H * I),
        # h read + touched experts' down bank + weighted y_sorted written
        "down": dict(bytes=touched * eb["down"] + P * I * 2 + int(P * H * yb), flops=2 * P * H * I),
        # y_sorted read + pair_slot read + y written
        "combine": dict(bytes=int(P * H * yb) + P * 4 + T * H * 4, flops=P * H),
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


# ------------------------------------------------------------ trace file --
def trace_average_us(workload: str, role_prefix: str):
    """Average duration (us) of the kernel whose role starts with
    `role_prefix` in the committed kernel-trace summary
    profiles/kernels_<workload>.md, or None when there is none or the
    kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}.md")
    if not os.path.exists(path):
        return None
    digest, avg = None, None
    with open(path) as f:
        for line in f:
            if line.startswith("source_digest"):
                digest = line.split("=", 1)[1].strip()
            cells = [c.strip() for c in line.split("|")]
            if len(cells) > 6 and cells[2].startswith(role_prefix) and avg is None:
                try:
                    avg = float(cells[5])
                except ValueError:
                    pass
    if digest != kernel_source_digest("gate_up"):
        return None
    return avg


ROLE_OF_STAGE = {"gate_up": "S6", "down": "S7", "combine": "S8"}
# at decode sizes the routing runs inside the gate/up launch and the combine
# inside the down launch
ROLE_OF_STAGE_DECODE = {"gate_up": "S1-S6", "down": "S7-S8", "combine": "S7-S8"}


# -------------------------------------------------------------- workloads --
class Case:
    """A workload's device-resident inputs: the packed layer(s) rotated over
    enough copies (>= 1 GiB of weights in total) that every step reads its
    experts cold from HBM, and for decode sizes a pool of logit sets, so the
    touched experts change every step.  The long-context workload rotates
    its four independently seeded layers (weights and activations)."""

    def __init__(self, name, dev):
        import torch

        from quantized_moe_top_amd import api, synth

        self.name = name
        n_layers = synth.WORKLOADS[name].get("layers", 1)
        self.hosts = [synth.make_layer(name, i) for i in range(n_layers)]
        base = [api.pack_layer(h.to(dev)) for h in self.hosts]
        torch.cuda.synchronize()
        lay = base[0]
        self.lay = lay
        nbytes = lambda b: (b.words.numel() + b.sb.numel()) * 4
        per_copy = nbytes(lay.gate) + nbytes(lay.up) + nbytes(lay.down) + \
            (lay.router_weight.numel() * 2 if lay.router_weight is not None else 0)
        self.per_copy = per_copy
        R = max(len(base), -(-ROTATE_BYTES // per_copy))
        copies = list(base)
        while len(copies) < R:
            src = base[len(copies) % len(base)]
            gate, up, down = (dataclasses.replace(b, words=b.words.clone(), sb=b.sb.clone())
                              for b in (src.gate, src.up, src.down))
            wr = src.router_weight.clone() if src.router_weight is not None else None
            copies.append(dataclasses.replace(src, gate=gate, up=up, down=down, router_weight=wr))
        self.copies = copies
        self.R = R
        self.logit_pool = None
        if lay.logits is not None and lay.T <= 8:
            self.logit_pool = [lay.logits] + list(
                synth.decode_logits_pool(lay.T, lay.E, 63, seed=1000 + lay.T).to(dev))
        self.y = torch.empty((lay.T, lay.H), dtype=torch.float32, device=dev)
        wsb = max(api.ffn_workspace_bytes(c) for c in copies)
        self.ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        # touched experts per step (routing is identical for every copy of
        # one layer; decode rotates logit sets)
        self.touched = []
        for i in range(self.n_variants()):
            _, inf = self.step(i, info=True)
            self.touched.append(int((inf["counts"] > 0).sum().item()))
        torch.cuda.synchronize()

    def n_variants(self):
        return len(self.logit_pool) if self.logit_pool else len(self.hosts)

    def step(self, i, evs=None, info=False):
        from quantized_moe_top_amd import api
        c = self.copies[i % self.R]
        lg = self.logit_pool[i % len(self.logit_pool)] if self.logit_pool else None
        return api.ffn_forward(c, logits=lg, y=self.y, workspace=self.ws, stage_events=evs, info=info)

    def mean_touched(self, K):
        if self.logit_pool:
            return float(sum(self.touched[i % len(self.touched)] for i in range(K)) / K)
        return float(sum(self.touched[(i % self.R) % len(self.hosts)] for i in range(K)) / K)


def time_steps(run, K, repeats=3):
    """Median over `repeats` runs of K back-to-back steps between two events
    (ms for the K steps), and the host wall time of that run."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = []
    for _ in range(repeats):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(K):
            run(i)
        end.record()
        torch.cuda.synchronize()
        res.append((start.elapsed_time(end), time.perf_counter() - t0))
    res.sort()
    return res[len(res) // 2]


def measure(case, K, warmup, graph=True, repeats=3):
    """Eager launches and HIP graph replays of the same steps, each the
    median of `repeats` timed runs; returns both and the faster."""
    import torch
    for i in range(warmup):
        case.step(i)
    torch.cuda.synchronize()
    graphs = None
    if graph:
        # one graph per (weight copy, logit set) that the steps use
        n_graphs = len(case.logit_pool) if case.logit_pool else case.R
        graphs = []
        for i in range(n_graphs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                case.step(i)
            graphs.append(g)
        for i in range(max(min(warmup, n_graphs), 1)):
            graphs[i % n_graphs].replay()
        torch.cuda.synchronize()
    eager_ms, eager_wall = time_steps(lambda i: case.step(i), K, repeats)
    graph_ms = graph_wall = None
    if graphs is not None:
        graph_ms, graph_wall = time_steps(lambda i: graphs[i % len(graphs)].replay(), K, repeats)
    if graph_ms is not None and graph_ms < eager_ms:
        best = (graph_ms, graph_wall, "hip_graph")
    else:
        best = (eager_ms, eager_wall, "eager")
    del graphs
    return {"eager_ms": eager_ms, "graph_ms": graph_ms, "best_ms": best[0], "wall_s": best[1],
            "launch": best[2]}


def stage_times(case, K):
    """Per-stage averages (us) from an eager pass of the same steps with an
    event recorded on the layer's stream at every stage boundary."""
    import numpy as np
    import torch

    from quantized_moe_top_amd import _lib, api
    nst = _lib.MOE_NUM_STAGES
    ev = [api.stage_events(nst + 1) for _ in range(K)]
    ms, _ = time_steps(lambda i: case.step(i, ev[i]), K, repeats=1)
    stage_ms = np.array([[ev[i][s].elapsed_time(ev[i][s + 1]) for s in range(nst)] for i in range(K)])
    return ms, {st: round(float(stage_ms[:, j].mean()) * 1e3, 3) for j, st in enumerate(_lib.STAGES)}


def layer_fractions(lay, touched, ms_per_step):
    lw = layer_work(lay, 0)
    lw_t = layer_work(lay, 1)["bytes"] - lw["bytes"]
    lbytes = lw["bytes"] + touched * lw_t
    t_step = ms_per_step * 1e-3
    return {"hbm_frac": round(lbytes / t_step / (HBM_PEAK_GBS * 1e9), 4),
            "mfma_frac": round(lw["flops"] / t_step / (MFMA_FP16_PEAK_TFLOPS * 1e12), 4),
            "bytes": int(lbytes), "flops": int(lw["flops"]), "touched_experts": touched}


def launch_floors(dev, K):
    """What one launch costs at the least on this stream: K eager launches
    of a one-element fill kernel, and K replays of a graph holding one."""
    import torch
    floor = torch.zeros(1, device=dev)
    for _ in range(10):
        floor.fill_(1.0)
    eager_ms, _ = time_steps(lambda i: floor.fill_(1.0), K)
    gf = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gf):
        floor.fill_(1.0)
    gf.replay()
    graph_ms, _ = time_steps(lambda i: gf.replay(), K)
    return round(eager_ms / K * 1e3, 3), round(graph_ms / K * 1e3, 3)


# Workloads the bench line reports beside the headline one (the targets:
# decode T=1 and T=8 at >= 60% of HBM, prefill T >= 8192 at >= 50% of the
# dense fp16/bf16 MFMA peak), with the steps timed per run.
TARGETS = {"decode_t1": 200, "decode_t8": 200, "imbalanced_t8192": 20, "longctx_t32768": 20}


def target_line(name, dev, steps, warmup):
    import torch
    log(f"[bench] target workload {name}: drawing and packing")
    case = Case(name, dev)
    m = measure(case, steps, warmup)
    ms = m["best_ms"] / steps
    _, st = stage_times(case, steps)
    lay = case.lay
    out = {"ms_per_step": round(ms, 6), "tokens_per_s": round(lay.T / (ms * 1e-3), 1),
           "launch": m["launch"], "eager_ms_per_step": round(m["eager_ms"] / steps, 6),
           "graph_ms_per_step": round(m["graph_ms"] / steps, 6) if m["graph_ms"] else None,
           "steps": steps, "weight_copies": case.R, "layers_rotated": len(case.hosts),
           "layer_roofline": layer_fractions(lay, case.mean_touched(steps), ms), "stage_us": st}
    log(f"[bench] {name}: {ms * 1e3:.2f} us/step ({m['launch']}), layer fractions "
        f"{out['layer_roofline']['mfma_frac']} MFMA / {out['layer_roofline']['hbm_frac']} HBM; stages {st}")
    del case
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


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
    case = Case(name, dev)
    lay, host = case.lay, case.hosts[0]
    T, E, k = lay.T, lay.E, lay.k
    R = case.R
    log(f"[bench] {R} weight copies of {case.per_copy / 2**20:.1f} MiB; "
        f"logit sets {len(case.logit_pool) if case.logit_pool else 1}; layers {len(case.hosts)}")
    y, ws, step = case.y, case.ws, case.step
    copies, logit_pool = case.copies, case.logit_pool

    K = args.steps
    log(f"[bench] timing {K} steps eager" + ("" if args.no_graph else " and by graph replay") +
        ", median of 3 runs each")
    m = measure(case, K, args.warmup, graph=not args.no_graph)
    elapsed_ms, wall, launch = m["best_ms"], m["wall_s"], m["launch"]
    eager_plain_ms, graph_ms = m["eager_ms"], m["graph_ms"]
    ms_per_step = elapsed_ms / K
    value = T * K / (elapsed_ms / 1e3)

    floor_eager_us, floor_graph_us = launch_floors(dev, K)

    # per-stage durations: an eager pass of the same steps with events
    # recorded between the stages on the layer's stream
    eager_ms, stage_us = stage_times(case, K)
    log(f"[bench] {ms_per_step * 1e3:.2f} us/step ({launch}; wall {wall / K * 1e6:.2f}; eager "
        f"{eager_plain_ms / K * 1e3:.2f}, graph {graph_ms / K * 1e3 if graph_ms else float('nan'):.2f}); "
        f"eager with stage events {eager_ms / K * 1e3:.2f} us/step; stages us {stage_us}")

    # roofline of the dominant single-kernel stage
    mean_touched = case.mean_touched(K)
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
        work, peak, unit, bound, scale = byts, HBM_PEAK_GBS, "GB/s", "hbm", 1e9
    else:
        work, peak, unit, bound, scale = flops, MFMA_FP16_PEAK_TFLOPS, "TFLOP/s", "mfma", 1e12
    achieved = work / dur_s / scale
    traffic = measured_traffic(name, dom)
    trace_us = trace_average_us(name, (ROLE_OF_STAGE_DECODE if T <= 8 else ROLE_OF_STAGE)[dom])
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom,
                "algorithmic_bytes": int(byts), "algorithmic_flops": int(flops),
                "avg_launch_us": stage_us[dom],
                # the same kernel's average from the committed rocprofv3
                # trace (profiles/kernels_<workload>.md), and the fraction it gives
                "trace_avg_us": trace_us,
                "frac_from_trace": round(work / (trace_us * 1e-6) / scale / peak, 4) if trace_us else None}
    layer_roof = layer_fractions(lay, mean_touched, ms_per_step)

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
        plain_ms, _ = time_steps(lambda i: step(i), K)
        host_ms, _ = time_steps(step_host, K)
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
        plain_ms, _ = time_steps(lambda i: step(i), K)
        io_ms, _ = time_steps(step_io, K)
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
        plain_ms, _ = time_steps(lambda i: step(i), K)
        unf_ms, _ = time_steps(step_unfused, K)
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

    del case, copies, y, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    targets = None
    if not args.no_targets and name == "prefill_t512":
        targets = {}
        for tname, tsteps in TARGETS.items():
            targets[tname] = target_line(tname, dev, tsteps, min(args.warmup, 10))

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
                   "weight_copies": R, "block_m": api.ffn_block_m(lay), "launch": launch,
                   "timing": "median of 3 runs of the timed steps, eager and graph replay each"},
        "roofline": roofline, "layer_roofline": layer_roof, "stage_us": stage_us,
        "eager_ms_per_step": round(eager_plain_ms / K, 6),
        "graph_ms_per_step": round(graph_ms / K, 6) if graph_ms else None,
        "eager_with_stage_events_ms_per_step": round(eager_ms / K, 6),
        "launch_floor_us": {"eager_fill_kernel": floor_eager_us, "graph_replay_of_fill": floor_graph_us},
        "targets": targets,
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(host, min_seconds: float) -> dict:
    """The CPU oracle on the host cores: the whole layer on a sample of the
    tokens (all of them when T <= 512), with routing over every token.  Three
    timed passes, each repeated until `min_seconds` / 3 of work; the median
    pass is scaled to whole-layer tokens/s."""
    import numpy as np

    import oracle

    orc = oracle.get()
    T = host.T
    n = min(T, 512)
    tokens = np.linspace(0, T - 1, n).round().astype(np.int32) if n < T else np.arange(T, dtype=np.int32)
    log(f"[bench] cpu baseline: oracle on {n} of {T} tokens, {orc.num_threads()} threads")
    passes = []
    total = 0.0
    for _ in range(3):
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
            if t_route + t_ffn >= min_seconds / 3 or reps >= 50:
                break
        total += t_route + t_ffn
        passes.append(t_route / reps + (t_ffn / reps) * T / n)
    per_layer = sorted(passes)[1]
    return {"value": round(T / per_layer, 2), "unit": "tokens/s", "cores": orc.num_threads(),
            "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(), "kind": "oracle",
            "passes_tokens_per_s": [round(T / p, 2) for p in passes],
            "sample": f"median of 3 passes, each routing all {T} tokens and computing the layer output "
                      f"of {n} tokens (repeated to >= {min_seconds / 3:.1f} s); {total:.1f} s of CPU "
                      f"work in all, scaled to the whole layer"}


if __name__ == "__main__":
    main()
