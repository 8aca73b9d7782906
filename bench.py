"""Benchmark of the SDM layer forward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
copy-on-init of the tables from M0, product-key addressing of the keys (W write slots)
and queries (R read slots), and the sparse gated-delta recurrence over all tokens. The
step is issued through the library's C ABI calls: sdm_address_init for the keys and for
the queries, each carrying half of the table initialisation from M0 in the same launch
(the addressing kernel is bound by its vector ALU and leaves the memory pipe idle), then
the recurrence (the call sdm_forward makes), so that the recurrence kernel can be timed
on its own with HIP events on the stream it runs on.

Prints one JSON line. ``value`` is layer tokens/s (B*T tokens per step) with all inputs
resident in HBM before timing starts. ``roofline`` describes the recurrence kernel
(HBM-bound): algorithmic bytes per launch / its average event-timed duration, against
MI355X's 8 TB/s. ``cpu_baseline`` times the float64 CPU oracle on a bounded sample.

With --decay the step runs the whole-table decay variant instead (decay state reset with
the table every step; the recurrence call then includes the log-decay scan and the decay
pass).

With --backward the step is a training step of the layer: addressing of keys and queries
(carrying the table initialisation as above), the recurrence with its log of pre-update rows, the memory-efficient backward of
the recurrence (which restores M0 in place) and the addressing backward for keys and
queries, from a synthetic output gradient. ``roofline`` then describes the recurrence
backward call (preparation pass and reverse walk) and ``value`` counts layer tokens per
training step.

With --chunked the recurrence runs in its chunkwise two-phase form (64-token chunks: the
preparation kernel over every chunk in parallel, then the apply kernel over the chunks in
order); ``roofline`` describes that call, priced with the recurrence's algorithmic bytes.
Without a mode flag the recurrence runs in the form sdm_forward takes for the shape
(sdm_forward_uses_chunkwise: the chunkwise form for a float32 table with at least 32 units,
else the pipeline); --pipeline forces the pipelined recurrence.

With --epilogue the step is the calls on either side of the recurrence: the gates from their
pre-activations, the output normalisation and gate, and the head mixing (d_model =
--d-model, default H*d_v); the fused sdm_output_project is timed beside them and checked
equal. ``roofline`` describes the head mixing (bf16 MFMA, against 2.5 PFLOP/s).

The decode workload (T = 1) times consecutive fused decode steps captured as a HIP graph.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--decay | --backward | --chunked | --pipeline | --epilogue [--d-model D]]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sdm_inputs as SI  # noqa: E402

HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "layer_8b_long"
METRIC = "SDM layer tokens/s on 1 MI355X; gather/scatter HBM GB/s vs peak"
METRIC_BACKWARD = "SDM layer training tokens/s (forward with log + backward) on 1 MI355X; backward HBM GB/s vs peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def recurrence_bytes_per_token_head(sh: SI.Shape) -> int:
    """Algorithmic HBM bytes of the recurrence per (batch, head, token): W rows gathered and
    W rows written back, R rows gathered (d_v values each, table dtype), v_t read, o_t
    written (float32), alpha_t and beta_t read."""
    mem = 2 if sh.mem_dtype == "bf16" else 4
    inb = 2 if sh.in_dtype == "bf16" else 4
    return (2 * sh.W + sh.R) * sh.d_v * mem + sh.d_v * inb + sh.d_v * 4 + 8


def backward_bytes_per_token_head(sh: SI.Shape) -> int:
    """Algorithmic HBM bytes of the recurrence backward per (batch, head, token): the W
    logged rows, the W + R rows of G read and written (float32), the R read rows and W
    restored rows of the table, go_t read and dv_t written (float32), v_t read, the weight,
    alpha and beta gradients written and the slot lists, weights and gates read."""
    mem = 2 if sh.mem_dtype == "bf16" else 4
    inb = 2 if sh.in_dtype == "bf16" else 4
    rows = sh.W * sh.d_v * mem + 2 * (sh.W + sh.R) * sh.d_v * 4 + sh.R * sh.d_v * mem + sh.W * sh.d_v * mem
    return rows + 8 * sh.d_v + sh.d_v * inb + 4 * (sh.W + sh.R + 2) + 8 * (sh.W + sh.R) + 8


RECURRENCE_SOURCES = ("sdm_dataflow.hip", "sdm_device.hpp")
CHUNKED_SOURCES = ("sdm_chunked.hip", "sdm_device.hpp")
BACKWARD_SOURCES = ("sdm_backward.hip", "sdm_device.hpp")
DECAY_SOURCES = ("sdm_decay.hip", "sdm_dataflow.hip", "sdm_device.hpp")
DECODE_SOURCES = ("sdm_decode.hip", "sdm_select.hpp", "sdm_device.hpp")


def kernel_source_hash(kind: str = "recurrence") -> str:
    """Hash of the sources of the recurrence kernels (dependency pass and pipeline), with
    kind="chunked" of the chunkwise kernels (preparation and apply), with kind="backward" of
    the recurrence backward (preparation and walk), with kind="decay" of the whole-table
    decay recurrence (decay passes, dependency pass and pipeline)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_memory_linear_amd", "csrc")
    srcs = {"chunked": CHUNKED_SOURCES, "backward": BACKWARD_SOURCES, "decay": DECAY_SOURCES,
            "decode": DECODE_SOURCES}.get(kind, RECURRENCE_SOURCES)
    for f in srcs:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str, kind: str = "recurrence"):
    """HBM bytes per launch of the measured kernel (kind "recurrence", "chunked", "backward"
    or "decay") from the committed counter summary, if it was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kind}_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash(kind):
        return None
    return d.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- CPU baseline
def _oracle_unit(args):
    """Worker: the oracle on one unit over the first T_s tokens (all columns)."""
    name, b, h, T_s = args
    import oracle.sdm_oracle as O
    sh = SI.WORKLOADS[name]
    inp = _oracle_unit.inp
    sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
    t0 = time.perf_counter()
    O.forward_unit(SI.widen(inp["q"][b, h, :T_s], sh.in_dtype), SI.widen(inp["k"][b, h, :T_s], sh.in_dtype),
                   SI.widen(inp["v"][b, h, :T_s], sh.in_dtype), inp["alpha"][b, h, :T_s].astype(np.float64),
                   inp["beta"][b, h, :T_s].astype(np.float64), sk[0], sk[1], SI.widen(inp["M0"][h], sh.mem_dtype),
                   sh.kappa, sh.W, sh.R, sh.mem_dtype)
    return time.perf_counter() - t0


def cpu_baseline(name: str, inp, budget_s: float = 15.0):
    import multiprocessing as mp
    sh = SI.WORKLOADS[name]
    units = [(b, h) for b in range(sh.B) for h in range(sh.H)]
    ncpu = len(os.sched_getaffinity(0))
    P = max(1, min(16, ncpu, len(units)))
    _oracle_unit.inp = inp
    # calibrate on a short prefix in this process (one unit)
    T_cal = min(sh.T, 128)
    dt = _oracle_unit((name, 0, 0, T_cal))
    per_tok = dt / T_cal
    T_s = int(max(64, min(sh.T, budget_s / max(per_tok, 1e-9))))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(P) as pool:
        pool.map(_oracle_unit, [(name, b, h, T_s) for (b, h) in units[:P]])
    wall = time.perf_counter() - t0
    token_heads_per_s = P * T_s / wall
    return {
        "value": token_heads_per_s / sh.H,
        "unit": "tokens/s",
        "cores": P,
        "kind": "oracle",
        "sample": f"{P} (batch, head) units x first {T_s} tokens of {name}, float64 numpy oracle "
                  f"(addressing + recurrence), one process per unit; layer tokens/s = unit-tokens/s / H",
    }


# ----------------------------------------------------------------------------- GPU run
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(SI.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decay", action="store_true", help="whole-table decay variant")
    ap.add_argument("--backward", action="store_true", help="training step: forward with log and backward")
    ap.add_argument("--chunked", action="store_true", help="forward with the chunkwise two-phase recurrence")
    ap.add_argument("--pipeline", action="store_true", help="forward with the pipelined recurrence")
    ap.add_argument("--epilogue", action="store_true",
                    help="the steps around the recurrence: gates, output gate fused into the head mixing")
    ap.add_argument("--d-model", type=int, default=0, help="head mixing output width (default H*d_v)")
    args = ap.parse_args()
    if args.decay + args.backward + args.chunked + args.pipeline + args.epilogue > 1:
        print("--decay, --backward, --chunked, --pipeline and --epilogue are separate modes", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this path has no multi-GPU mode); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_memory_linear_amd as S

    sh = SI.WORKLOADS[args.workload]
    if sh.T == 1:
        return bench_decode(args, sh)
    if args.epilogue:
        return bench_epilogue(args, sh)
    if args.decay or args.backward or args.chunked or args.pipeline:
        args.no_cpu_baseline = True  # the oracle baseline times the default forward
    log(f"[bench] generating {sh.name} inputs")
    t0 = time.time()
    inp = SI.make_inputs(sh)
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")
    cpu = None
    if not args.no_cpu_baseline:
        # before the GPU is touched: the oracle workers are forked from this process
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(sh.name, inp)
        log(f"[bench] oracle {cpu['value']:.1f} tokens/s on {cpu['cores']} cores")

    def dev(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    q, k, v = (dev(inp[n], sh.in_dtype) for n in ("q", "k", "v"))
    subkeys = dev(inp["subkeys"], sh.in_dtype)
    alpha, beta = dev(inp["alpha"], "f32"), dev(inp["beta"], "f32")
    M0 = dev(inp["M0"], sh.mem_dtype)
    mdt = torch.bfloat16 if sh.mem_dtype == "bf16" else torch.float32
    M = torch.empty((sh.B, sh.H, sh.N, sh.d_v), dtype=mdt, device="cuda")
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    shape = S.make_shape(sh.B, sh.H, sh.T, sh.N, sh.d_k, sh.d_v, sh.kappa, sh.W, sh.R, sh.in_dtype, sh.mem_dtype)
    ws = torch.empty((S.workspace_bytes_decay if args.decay else S.workspace_bytes)(shape), dtype=torch.uint8,
                     device="cuda")
    if args.decay:
        lam = torch.empty((sh.B, sh.H, sh.N), dtype=torch.float64, device="cuda")
        lrun = torch.empty((sh.B, sh.H), dtype=torch.float64, device="cuda")
    widx = torch.empty((sh.B, sh.H, sh.T, sh.W), dtype=torch.int32, device="cuda")
    wgt = torch.empty((sh.B, sh.H, sh.T, sh.W), dtype=torch.float32, device="cuda")
    ridx = torch.empty((sh.B, sh.H, sh.T, sh.R), dtype=torch.int32, device="cuda")
    rgt = torch.empty((sh.B, sh.H, sh.T, sh.R), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    # the recurrence form sdm_forward takes for this shape, unless a mode flag fixes it
    if not (args.decay or args.backward or args.pipeline) and S.forward_uses_chunkwise(shape):
        args.chunked = True
        log("[bench] sdm_forward runs the chunkwise form for this shape")
    if args.chunked:
        cws = torch.empty(S.workspace_bytes_chunked(shape), dtype=torch.uint8, device="cuda")
    if args.backward:
        s_ = int(round(sh.N ** 0.5))
        xlog = torch.empty((sh.B, sh.H, sh.T, sh.W, sh.d_v), dtype=mdt, device="cuda")
        go = torch.randn((sh.B, sh.H, sh.T, sh.d_v), device="cuda",
                         generator=torch.Generator("cuda").manual_seed(11))
        G = torch.empty((sh.B, sh.H, sh.N, sh.d_v), dtype=torch.float32, device="cuda")
        dv = torch.empty_like(go)
        dal = torch.empty((sh.B, sh.H, sh.T), dtype=torch.float32, device="cuda")
        dbe = torch.empty_like(dal)
        dwg = torch.empty_like(wgt)
        drg = torch.empty_like(rgt)
        dq = torch.empty((sh.B, sh.H, sh.T, sh.d_k), dtype=torch.float32, device="cuda")
        dk = torch.empty_like(dq)
        dsub = torch.empty((sh.H, 2, s_, sh.d_k // 2), dtype=torch.float32, device="cuda")
        bws = torch.empty(S.backward_workspace_bytes(shape), dtype=torch.uint8, device="cuda")

    def train_step(ev=None):
        S.address_init(shape, k, subkeys, sh.W, widx, wgt, M0, M, 0, 2)
        S.address_init(shape, q, subkeys, sh.R, ridx, rgt, M0, M, 1, 2)
        S.recurrent_log(shape, widx, wgt, ridx, rgt, v, alpha, beta, M, o, xlog, ws)
        G.zero_()
        dsub.zero_()
        if ev is not None:
            ev[0].record(stream)
        S.recurrent_backward(shape, widx, wgt, ridx, rgt, v, alpha, beta, M, xlog, go, G, dv, dal, dbe, dwg, drg,
                             bws)
        if ev is not None:
            ev[1].record(stream)
        S.address_backward(shape, k, subkeys, sh.W, widx, wgt, dwg, dk, dsub)
        S.address_backward(shape, q, subkeys, sh.R, ridx, rgt, drg, dq, dsub)

    def step(ev=None):
        if args.backward:
            return train_step(ev)
        if args.decay:
            S.decay_state_init(shape, lam, lrun)
        S.address_init(shape, k, subkeys, sh.W, widx, wgt, M0, M, 0, 2)
        S.address_init(shape, q, subkeys, sh.R, ridx, rgt, M0, M, 1, 2)
        if ev is not None:
            ev[0].record(stream)
        if args.decay:
            S.recurrent_decay(shape, widx, wgt, ridx, rgt, v, alpha, beta, M, lam, lrun, o, ws)
        elif args.chunked:
            S.recurrent_chunked(shape, widx, wgt, ridx, rgt, v, alpha, beta, M, o, cws)
        else:
            S.recurrent(shape, widx, wgt, ridx, rgt, v, alpha, beta, M, o, ws)
        if ev is not None:
            ev[1].record(stream)

    # one plain copy-on-init before the warm-up, outside the timed steps: a copy kernel of known
    # size (M0 read once, B copies written) that HBM counter summaries calibrate against
    S.init_from_M0(shape, M0, M)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    rec_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    tokens = sh.B * sh.T
    value = tokens / (ms_step / 1e3)
    per_th = backward_bytes_per_token_head(sh) if args.backward else recurrence_bytes_per_token_head(sh)
    launch_bytes = per_th * sh.B * sh.H * sh.T
    achieved = launch_bytes / (rec_ms / 1e3) / 1e9
    log(f"[bench] {ms_step:.3f} ms/step, {'backward' if args.backward else 'recurrence'} {rec_ms:.3f} ms, "
        f"{achieved:.1f} GB/s")
    if args.backward:
        assert S.workspace_error(bws) == 0, "a workgroup of the backward gave up waiting"

    traffic = traffic_from_profile(sh.name, "chunked" if args.chunked else "backward" if args.backward else
                                   "decay" if args.decay else "recurrence")
    out = {
        "metric": (METRIC_BACKWARD if args.backward else METRIC),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sh.in_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": sh.name, "B": sh.B, "H": sh.H, "T": sh.T, "N": sh.N, "d_k": sh.d_k, "d_v": sh.d_v,
                   "kappa": sh.kappa, "W": sh.W, "R": sh.R, "in_dtype": sh.in_dtype, "mem_dtype": sh.mem_dtype,
                   "arith": "fp32", **({"decay": "whole table"} if args.decay else {}),
                   **({"step": "forward with log + backward"} if args.backward else {}),
                   **({"recurrence": "chunkwise two-phase, 64-token chunks"} if args.chunked else {})},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": ("recurrence backward" if args.backward else
                                "chunkwise recurrence (prep + apply)" if args.chunked else "recurrence"),
                     "ms_per_launch": rec_ms, "bytes_per_launch": launch_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_epilogue(args, sh):
    """The steps on either side of the recurrence at a workload's shape: gates from their
    pre-activations, the output normalisation and gate (sdm_output_gate) and the head mixing
    (sdm_head_mix). One step = those three calls over all B*T tokens (the faster output path
    at every shape measured); the fused sdm_output_project, which needs no bf16 x buffer, is
    timed beside them and checked equal bit for bit. Inputs: the seeded epilogue inputs of
    the workload and a seeded standard normal o in place of the recurrence's output (the
    cost does not depend on its values)."""
    import torch
    import sparse_memory_linear_amd as S

    d_model = args.d_model or sh.H * sh.d_v
    log(f"[bench] epilogue: {sh.name}, d_model {d_model}")
    ep = SI.make_epilogue_inputs(sh, d_model=d_model)
    rng = np.random.default_rng([sh.seed, 11])
    o_host = rng.standard_normal((sh.B, sh.H, sh.T, sh.d_v), dtype=np.float32)

    def dev(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    shape = S.make_shape(sh.B, sh.H, sh.T, sh.N, sh.d_k, sh.d_v, sh.kappa, sh.W, sh.R, sh.in_dtype, sh.mem_dtype)
    o = dev(o_host, "f32")
    del o_host
    z, w, Wo = dev(ep["z"], sh.in_dtype), dev(ep["w"], "f32"), dev(ep["Wo"], "bf16")
    a, b, A_log, dt_bias = (dev(ep[k], "f32") for k in ("a", "b", "A_log", "dt_bias"))
    M, K = sh.B * sh.T, sh.H * sh.d_v
    alpha = torch.empty((sh.B, sh.H, sh.T), dtype=torch.float32, device="cuda")
    beta = torch.empty_like(alpha)
    x = torch.empty((sh.B, sh.T, sh.H, sh.d_v), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, d_model), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y)
    calls = {
        "gates": lambda: S.gates(shape, a, b, A_log, dt_bias, alpha, beta),
        "output_project": lambda: S.output_project(shape, o, z, w, 1e-5, Wo, d_model, y),
        "output_gate": lambda: S.output_gate(shape, o, z, w, 1e-5, x),
        "head_mix": lambda: S.head_mix(x, Wo, y2, M, K, d_model),
    }
    for _ in range(max(1, args.warmup)):
        for f in calls.values():
            f()
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "fused and two-call outputs differ"
    times = {k: [] for k in calls}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for k, f in calls.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            times[k].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    med = {k: sorted(a_.elapsed_time(b_) for a_, b_ in v)[len(v) // 2] for k, v in times.items()}
    step_ms = med["gates"] + med["output_gate"] + med["head_mix"]
    ib = 2 if sh.in_dtype == "bf16" else 4
    proj_bytes = M * K * (4 + ib) + M * d_model * 4 + d_model * K * 2
    flops = 2.0 * M * K * d_model
    achieved = flops / (med["head_mix"] / 1e3) / 1e12
    log(f"[bench] epilogue: gates {med['gates']:.3f} ms, output gate {med['output_gate']:.3f} ms, head mixing "
        f"{med['head_mix']:.3f} ms ({achieved:.0f} TFLOP/s); fused output_project {med['output_project']:.3f} ms")
    out = {
        "metric": "SDM layer epilogue tokens/s (gates, output gate, head mixing) on 1 MI355X",
        "value": M / (step_ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": sh.name, "B": sh.B, "H": sh.H, "T": sh.T, "d_v": sh.d_v, "d_model": d_model,
                   "in_dtype": sh.in_dtype, "gates_ms": med["gates"], "output_gate_ms": med["output_gate"],
                   "head_mix_ms": med["head_mix"], "output_project_ms": med["output_project"],
                   "output_project_gbs": proj_bytes / (med["output_project"] / 1e3) / 1e9},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": achieved / 2500.0, "traffic": None, "kernel": "head_mix (bf16 MFMA)",
                     "ms_per_launch": med["head_mix"], "flops_per_launch": flops},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def _prefill_tokens(args):
    """Worker: the prefill tokens of one decode sequence."""
    name, b = args
    return b, SI.make_prefill(SI.WORKLOADS[name], b)


def _oracle_decode(args):
    """Worker: the oracle's decode step on one head's table, over nsteps bank tokens of
    sequence b; returns the wall time."""
    import oracle.sdm_oracle as O
    name, b, h, nsteps = args
    sh = SI.WORKLOADS[name]
    p, bank = _oracle_decode.params, _oracle_decode.bank
    sk = SI.widen(p["subkeys"][h], sh.in_dtype)
    M = SI.widen(p["M0"][h], sh.mem_dtype)
    t0 = time.perf_counter()
    for i in range(nsteps):
        _, M, _ = O.decode_step_unit(M, SI.widen(bank["q"][i, b, h, 0], sh.in_dtype),
                                     SI.widen(bank["k"][i, b, h, 0], sh.in_dtype),
                                     SI.widen(bank["v"][i, b, h, 0], sh.in_dtype), float(bank["alpha"][i, b, h, 0]),
                                     float(bank["beta"][i, b, h, 0]), sk[0], sk[1], sh.kappa, sh.W, sh.R,
                                     sh.mem_dtype)
    return time.perf_counter() - t0


def bench_decode(args, sh):
    """Decode workload: each step is one fused decode step over all B sequences (tables
    pre-filled by a 4096-token prefill through the forward), fed the next token of a bank
    of distinct tokens, so every step addresses fresh rows. The timed steps run as a serving
    loop would: n consecutive steps captured once as a HIP graph and replayed, so that the
    host's per-call cost (Python, argument checks, launch) does not sit between steps; the
    step time is the replay's event time / n and tokens/s = B / step time. The same steps
    launched one host call at a time are timed too (median event latency, reported beside)."""
    import multiprocessing as mp

    n = max(args.steps, 100)
    log(f"[bench] decode: token bank of {n + args.warmup} steps x {sh.B} sequences")
    params = SI.make_inputs(sh)
    bank = SI.make_decode_bank(sh, 3 * n + args.warmup)  # warmup, eager steps, graph warm-up, timed graph
    P = max(1, min(16, len(os.sched_getaffinity(0))))
    cpu = None
    _oracle_decode.params, _oracle_decode.bank = params, bank
    if args.no_cpu_baseline:
        # no worker processes: a run under a profiler whose preloaded library has already
        # initialised the GPU must not fork
        pre = {}
        for b in range(sh.B):
            pre[b] = _prefill_tokens((sh.name, b))[1]
            if b % 16 == 15:
                log(f"[bench] decode: prefill tokens of {b + 1}/{sh.B} sequences")
    else:
        # before the GPU is touched: prefill tokens and the oracle baseline in forked workers
        with mp.get_context("fork").Pool(P) as pool:
            log(f"[bench] decode: prefill tokens of {sh.B} sequences in {P} workers")
            pre = dict(pool.map(_prefill_tokens, [(sh.name, b) for b in range(sh.B)]))
            dt = _oracle_decode((sh.name, 0, 0, 2)) / 2
            steps = int(max(2, min(n, 15.0 / max(dt, 1e-6))))
            units = [(b % sh.B, b % sh.H) for b in range(P)]
            t0 = time.perf_counter()
            pool.map(_oracle_decode, [(sh.name, b, h, steps) for (b, h) in units])
            wall = time.perf_counter() - t0
            cpu = {"value": P * steps / wall / sh.H, "unit": "tokens/s", "cores": P, "kind": "oracle",
                   "sample": f"{P} (sequence, head) tables x {steps} consecutive bank tokens, float64 numpy oracle "
                             f"decode step (addressing + write + read) from M0, one process per table; tokens/s = "
                             f"table-steps/s / H"}
            log(f"[bench] oracle decode {cpu['value']:.1f} tokens/s on {P} cores")

    import torch
    import sparse_memory_linear_amd as S

    def dev(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    log(f"[bench] decode: building {sh.B}x{sh.H} tables")
    subkeys = dev(params["subkeys"], sh.in_dtype)
    M0 = dev(params["M0"], sh.mem_dtype)
    mdt = torch.bfloat16 if sh.mem_dtype == "bf16" else torch.float32
    M = torch.empty((sh.B, sh.H, sh.N, sh.d_v), dtype=mdt, device="cuda")
    s1 = S.make_shape(sh.B, sh.H, 1, sh.N, sh.d_k, sh.d_v, sh.kappa, sh.W, sh.R, sh.in_dtype, sh.mem_dtype)
    S.init_from_M0(s1, M0, M)
    Tp = sh.prefill
    sp = S.make_shape(1, sh.H, Tp, sh.N, sh.d_k, sh.d_v, sh.kappa, sh.W, sh.R, sh.in_dtype, sh.mem_dtype)
    ws = torch.empty(S.workspace_bytes(sp), dtype=torch.uint8, device="cuda")
    o_pre = torch.empty((1, sh.H, Tp, sh.d_v), dtype=torch.float32, device="cuda")
    for b in range(sh.B):
        t = {k: dev(pre[b][k], sh.in_dtype if k in ("q", "k", "v") else "f32") for k in ("q", "k", "v", "alpha",
                                                                                       "beta")}
        S.forward(sp, t["q"], t["k"], t["v"], t["alpha"], t["beta"], subkeys, M[b:b + 1], o_pre, ws)
    del pre
    bq, bk, bv = (dev(bank[k], sh.in_dtype) for k in ("q", "k", "v"))
    ba, bb = dev(bank["alpha"], "f32"), dev(bank["beta"], "f32")
    torch.cuda.synchronize()
    o = torch.empty((sh.B, sh.H, 1, sh.d_v), dtype=torch.float32, device="cuda")
    for i in range(args.warmup):
        S.decode_step(s1, bq[i], bk[i], bv[i], ba[i], bb[i], subkeys, M, o)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    t0 = time.perf_counter()
    for j in range(n):
        i = args.warmup + j
        ev[j][0].record()
        S.decode_step(s1, bq[i], bk[i], bv[i], ba[i], bb[i], subkeys, M, o)
        ev[j][1].record()
    torch.cuda.synchronize()
    lat = sorted(a.elapsed_time(b) for a, b in ev)

    # the next 2n tokens as two captured graphs of n steps: the first replay warms the graph
    # launch path, the second is timed
    graphs = []
    for part in (1, 2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(n):
                i = args.warmup + part * n + j
                S.decode_step(s1, bq[i], bk[i], bv[i], ba[i], bb[i], subkeys, M, o)
        graphs.append(g)
    torch.cuda.synchronize()
    graphs[0].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    graphs[1].replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / n
    per_th = recurrence_bytes_per_token_head(sh) + 2 * sh.d_k * (2 if sh.in_dtype == "bf16" else 4)
    launch_bytes = per_th * sh.B * sh.H
    achieved = launch_bytes / (ms / 1e3) / 1e9
    log(f"[bench] decode: {ms * 1e3:.1f} us per step in a graph of {n} steps ({achieved:.0f} GB/s algorithmic); "
        f"one host call per step: median {lat[n // 2] * 1e3:.1f} us (min {lat[0] * 1e3:.1f}, max {lat[-1] * 1e3:.1f})")
    out = {
        "metric": METRIC, "value": sh.B / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": n,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / n, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": sh.mem_dtype, "data": "synthetic",
        "config": {"workload": sh.name, "B": sh.B, "H": sh.H, "T": 1, "N": sh.N, "d_k": sh.d_k, "d_v": sh.d_v,
                   "kappa": sh.kappa, "W": sh.W, "R": sh.R, "in_dtype": sh.in_dtype, "mem_dtype": sh.mem_dtype,
                   "arith": "fp32", "prefill": Tp, "token_bank": 3 * n + args.warmup,
                   "timing": f"{n} consecutive steps captured as one HIP graph, replayed once (event time / {n})",
                   "step_ms_graph": ms, "eager_latency_ms_median": lat[n // 2], "eager_latency_ms_min": lat[0],
                   "eager_latency_ms_max": lat[-1]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_profile(sh.name, "decode"),
                     "kernel": "decode", "ms_per_launch": ms, "bytes_per_launch": launch_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
