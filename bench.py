#!/usr/bin/env python3
"""Benchmark of the MHLA forward pass (libmhla) on one MI355X.

One step = one full forward (block_kv_summary -> mix_summaries -> query_apply,
or the fused path) over one batch of seeded synthetic inputs already resident
in HBM.  Several input/output sets are rotated so that the 256 MB Infinity
Cache cannot serve the inputs of a step from the previous one.

Prints ONE JSON line: tokens/s over the timed steps, achieved algorithmic HBM
bandwidth of the whole path, a roofline entry for the dominant kernel (its
algorithmic bytes over its average duration, timed with HIP events on the
launch stream), and the float64 CPU oracle timed on the host as a baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MHLA fwd tokens/s + achieved HBM GB/s (% peak), N=65536 H=6 d=64 bf16"
# Sources of the forward kernels each path runs; a stored traffic summary is
# used only while the hash over its path's sources is unchanged.
_FWD = ("kernels_bf16.hip", "bf16_shared.h", "common.h", "mhla_api.cpp", "launch.h")
KERNEL_SOURCES = {
    "3kernel": _FWD,
    "fused": _FWD,
    "causal": _FWD + ("kernels_causal_bf16.hip",),
    "layer": _FWD + ("kernels_layer_bf16.hip",),
}
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak
MFMA_PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
MALL_BYTES = 256 << 20          # Infinity Cache


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload index (2 = the metric's workload)")
    ap.add_argument("--path", choices=["3kernel", "fused", "causal"], default="3kernel",
                    help="causal: the causal chunkwise form; without --block the chunks are the grid's raster rows")
    ap.add_argument("--stream-chunks", type=int, default=0,
                    help="with --path causal: stream the sequence through mhla_causal_stream in calls of this "
                         "many chunks (one step = the whole sequence)")
    ap.add_argument("--w", choices=["gaussian", "local", "identity", "ones", "linear", "cos", "exp", "gaussian-dmax"],
                    default="gaussian")
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0: enough to exceed 2x the MALL)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--out", default="", help="also write the JSON line to this file")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dq, dk, dv, dW) instead of the forward (bf16, d <= 64)")
    ap.add_argument("--layer", action="store_true",
                    help="time the whole layer around the core (mhla_layer_forward) instead")
    ap.add_argument("--phi", choices=["elu", "relu"], default="relu",
                    help="--layer: feature map (relu + eps as in the module's code, or elu + 1)")
    ap.add_argument("--qk-norm", action="store_true", help="--layer: RMSNorm on q and k")
    ap.add_argument("--block", default="", help="override the block extents, e.g. 32x32 (token-level head count sweeps)")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch size")
    ap.add_argument("--heads", type=int, default=0, help="override the workload's head count")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (10 times): the reference "
                         "for scaling the HBM byte counters of a profiler run")
    return ap.parse_args()


def kernel_source_sha(path: str = "3kernel"):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[path]:
        with open(os.path.join(ROOT, "token_level_head_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, path: str = "3kernel"):
    """Per-dispatch HBM bytes of each kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE, WRITE_SIZE scaled by a plain copy of known size), or {}
    if there is none for this workload or the kernel sources changed since."""
    fname = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(fname):
        return {}
    vals = {}
    for line in open(fname):
        line = line.strip()
        if not line or line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_sha(path):
        return {}
    fs, ws = float(vals["fetch_scale"]), float(vals["write_scale"])
    out = {}
    for k, v in vals.items():
        if k.endswith(" fetch_kib"):
            name = k[: -len(" fetch_kib")]
            w = float(vals.get(name + " write_kib", 0.0))
            out[name] = int(float(v) * 1024 * fs + w * 1024 * ws)
    return out


def measured_mfma(workload: str, path: str = "3kernel"):
    """MFMA flops per dispatch of each kernel (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) from the
    committed rocprofv3 counter summary, or {} (as measured_traffic)."""
    fname = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(fname):
        return {}
    vals = {}
    for line in open(fname):
        line = line.strip()
        if line and not line.startswith("#") and ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_sha(path):
        return {}
    return {k[: -len(" mfma_flops")]: float(v) for k, v in vals.items() if k.endswith(" mfma_flops")}


def kernel_bytes(p, ws_elem):
    """Algorithmic HBM bytes per launch of each kernel (compulsory reads + writes)."""
    B, N, H, d, M = p.batch, p.n_tokens, p.heads, p.head_dim, p.n_blocks
    e = p.elem_bytes
    P = B * H
    tensor = B * N * H * d * e
    sz = P * M * (d * d + d) * ws_elem
    st = P * M * d * d * ws_elem
    zt = P * M * d * 4
    w = M * M * 4
    return {
        "block_kv_summary": 2 * tensor + sz,
        "mix_summaries": sz + w + st + zt,
        "query_apply": tensor + st + zt + tensor,
        "query_apply_fused": tensor + sz + w + tensor,   # every summary read at least once
        "query_apply_causal": 3 * tensor + st + zt + tensor,   # q, k, v of the chunk once, mixtures, out
    }


class HipEvents:
    """HIP events created with hipEventDisableSystemFence, through the HIP runtime."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.made = []

    def create(self) -> int:
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.ct.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0 or not e.value:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.made.append(e.value)
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        x = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(x), self.ct.c_void_p(a), self.ct.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(x.value)

    def destroy_all(self):
        for e in self.made:
            self.hip.hipEventDestroy(self.ct.c_void_p(e))
        self.made = []


def host_cpu():
    """Host cores this process may run on, and the CPU model from /proc/cpuinfo."""
    ncpu = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return ncpu, model


def time_cpu(fn, max_runs=3, single_over_s=10.0):
    """Best wall time of up to max_runs calls (one call if it takes longer than single_over_s)."""
    best, runs = None, 0
    while runs < max_runs:
        t = time.perf_counter()
        r = fn()
        dt = time.perf_counter() - t
        runs += 1
        best = dt if best is None else min(best, dt)
        if dt > single_over_s:
            break
    return best, runs, r


def measure_copy(torch, nbytes, reps=20):
    """A plain device-to-device copy of nbytes (read nbytes, write nbytes) on
    the current stream, rotating over enough buffer pairs that the Infinity
    Cache cannot serve a copy's source from an earlier one.  Returns
    (microseconds per copy, GB/s of bytes read plus written)."""
    sets = max(2, int(np.ceil(2 * MALL_BYTES / (2 * nbytes))) + 1)
    bufs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda"),
             torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(sets)]
    for src, _ in bufs:
        src.fill_(1)
    stream = torch.cuda.current_stream()
    for i in range(3):
        bufs[i % sets][1].copy_(bufs[i % sets][0])
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(reps):
        dst, src = bufs[i % sets][1], bufs[i % sets][0]
        dst.copy_(src)
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / reps
    del bufs
    torch.cuda.empty_cache()
    return us, 2 * nbytes / (us * 1e-6) / 1e9


def backward_bytes(p, general=False, causal=False):
    """Algorithmic HBM bytes of each backward stage (compulsory reads + writes).
    The MFMA paths keep the summaries and their gradients as bf16 records (the
    causal one also passes each token's 1 / den and dden, two fp32 values, from
    the query side to the key/value side, and each pair's in-chunk dW[i, i]
    terms); the general kernels use fp32 records of d*d + d values, and their
    causal form passes each token's dnum (d fp32) and dden (fp32)."""
    B, N, H, d, M = p.batch, p.n_tokens, p.heads, p.head_dim, p.n_blocks
    tensor = B * N * H * d * p.elem_bytes
    P = B * H
    w = M * M * 4
    if causal and not general:
        rec = P * M * (d * d + d) * 2
        st = P * M * d * d * 2
        zt = P * M * d * 4
        tok = B * N * H * 8
        return {
            "recompute (summary + causal mix)": 2 * tensor + rec + rec + w + st + zt,
            "query side": 4 * tensor + st + zt + tensor + rec + tok + P * M * 4,
            "mix_transposed + dW partials": rec + w + st + zt + 2 * rec,
            "key/value side + dW reduce": 4 * tensor + tok + st + zt + 2 * tensor + P * M * 4 + w,
        }
    if general or causal:
        rec = P * M * (d * d + d) * 4
        tok = B * N * H * (d + 1) * 4 if causal else 0
        return {
            "recompute (summary + mix)": 2 * tensor + rec + rec + w + rec,
            "query side": (4 if causal else 2) * tensor + rec + tensor + rec + tok,
            "mix_transposed + dW partials": rec + w + rec + 2 * rec,
            ("key/value side + dW reduce" if causal else "key/value side"):
                (3 if causal else 2) * tensor + rec + 2 * tensor + tok + (P * M * 4 + w if causal else 0),
        }
    rec = P * M * (d * d + d) * 2      # summaries, or their gradients, as bf16 records
    st = P * M * d * d * 2
    zt = P * M * d * 4
    return {
        "recompute (block_kv_summary + mix)": 2 * tensor + rec + rec + w + st + zt,
        "bwd_query": 2 * tensor + st + zt + tensor + rec,
        "mix_transposed + dW partials": rec + w + st + zt + 2 * rec,
        "bwd_kv + dW reduce": 2 * tensor + st + zt + 2 * tensor + w,
    }   # (the reduce runs in the dW stage instead when the partials are many)


def bench_backward(args, p, torch, mh, synth):
    """One step = one mhla_backward call (recompute of the forward summaries,
    query side, transposed mixing and dW, key/value side) on synthetic inputs
    and a synthetic upstream gradient resident in HBM."""
    tensor_bytes = p.batch * p.n_tokens * p.heads * p.head_dim * p.elem_bytes
    sets = args.sets or max(2, int(np.ceil(2 * MALL_BYTES / (7 * tensor_bytes))))

    def dev(x):
        if p.dtype == synth.BF16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    data, host0 = [], None
    for s in range(sets):
        q, k, v, W = synth.make_inputs(p, seed=(args.config, s) if s else args.config, w_kind=args.w)
        rng = np.random.default_rng(1000 + s)
        g = rng.standard_normal(q.shape).astype(np.float32)
        g = synth.bf16_bits(g) if p.dtype == synth.BF16 else g
        t = [dev(x) for x in (q, k, v, g)]
        outs = [torch.empty_like(t[0]) for _ in range(3)]
        dW = torch.empty(p.n_blocks, p.n_blocks, dtype=torch.float32, device="cuda")
        data.append((t[0], t[1], t[2], torch.from_numpy(W).cuda(), t[3], outs[0], outs[1], outs[2], dW))
        if s == 0:
            host0 = (q, k, v, W, g)
    gr = mh.make_grid(p.batch, p.heads, p.head_dim, mh.MHLA_BF16 if p.dtype == synth.BF16 else mh.MHLA_F32,
                      p.grid, p.eps)
    bl = mh.make_block(p.block)
    causal = args.path == "causal"
    # matrix-core kernels: bf16 with d <= 64 (causal: chunks whole, i.e. at most
    # one sub-chunk per chunk in the forward)
    general = not (p.dtype == synth.BF16 and p.head_dim <= 64)
    if causal and not general:
        split = next((b for b in p.block if b > 1), 1)   # the axis sub-chunks would split
        general = split % 2 == 0 and p.block_tokens >= 512 and p.n_blocks * 2 <= 256
    wsize = mh.mhla_causal_backward_workspace_bytes if causal else mh.mhla_backward_workspace_bytes
    call = mh.mhla_causal_backward if causal else mh.mhla_backward
    ws_bytes = wsize(gr, bl)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i, events=None):
        q, k, v, W, g, dq, dk, dv, dW = data[i % sets]
        st = call(q, k, v, W, g, gr, bl, dq, dk, dv, dW, ws, ws_bytes, events, stream)
        if st != mh.MHLA_OK:
            raise mh.MhlaError(st, call.__name__)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    hev = HipEvents()
    evs = [[hev.create() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    stage_ms = np.array([[hev.elapsed_ms(r[j], r[j + 1]) for j in range(4)] for r in evs]).mean(axis=0)
    hev.destroy_all()
    kb = backward_bytes(p, general, causal)
    stages = {}
    for j, (name, nbytes) in enumerate(kb.items()):
        gbps = nbytes / (stage_ms[j] * 1e-3) / 1e9
        stages[name] = {"avg_us": round(float(stage_ms[j]) * 1e3, 2), "alg_bytes": int(nbytes),
                        "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    dom = max(stages, key=lambda n: stages[n]["avg_us"])
    U = 7 * tensor_bytes + 8 * p.n_blocks ** 2      # read q, k, v, dout, W; write dq, dk, dv, dW
    cpu = None
    if not args.no_cpu:
        import oracle
        q, k, v, W, g = host0
        ncpu = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        t = time.perf_counter()
        if causal:
            oracle.backward_causal(q, k, v, W, g, p.grid, p.block, eps=p.eps)
            used = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
            what = ("float64 causal chunkwise gradients in numpy (matrix products on the BLAS threads, "
                    "the rest on one thread)")
        else:
            _, used = oracle.backward(q, k, v, W, g, p.grid, p.block, eps=p.eps, threads=ncpu,
                                      return_threads=True)
            what = "float64 blockwise gradients, one thread per pair"
        dt_cpu = time.perf_counter() - t
        cpu = {"value": round(p.batch * p.n_tokens / dt_cpu, 1), "unit": "tokens/s", "cores": used,
               "kind": "oracle", "seconds": round(dt_cpu, 3),
               "sample": f"the full workload ({p.batch * p.heads} (b,h) pairs), {what}"}
    line = {
        "metric": f"MHLA {'causal ' if causal else ''}bwd tokens/s (dq, dk, dv, dW) + achieved HBM GB/s", "value":
            round(p.batch * p.n_tokens / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if p.dtype == synth.BF16 else "f32", "data": "synthetic",
        "config": {"workload": f"{p.name}: B={p.batch} H={p.heads} d={p.head_dim} grid={list(p.grid)} "
                               f"blocks={list(p.block)} N={p.n_tokens} M={p.n_blocks}",
                   "pass": "causal backward" if causal else "backward", "kernels": "general" if general else "mfma",
                   "input_sets": sets, "parallelism": "none (1 GPU)"},
        "path_hbm_gbps": round(U / (ms_step * 1e-3) / 1e9, 1),
        "path_hbm_frac": round(U / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "path_alg_bytes": U,
        "kernels": stages,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": stages[dom]["gbps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": stages[dom]["frac"], "traffic": None,
                     "avg_us": stages[dom]["avg_us"], "alg_bytes": stages[dom]["alg_bytes"]},
        "cpu_baseline": cpu,
    }
    s = json.dumps(line)
    print(s, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(s + "\n")


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def layer_costs(p, qk_norm: bool, lepe: bool):
    """Algorithmic HBM bytes and flops of each stage of the layer (compulsory
    reads + writes of that stage; bf16 activations)."""
    R, C = p.batch * p.n_tokens, p.heads * p.head_dim
    act = R * C * 2
    core = sum(kernel_bytes(p, p.elem_bytes)[k] for k in ("block_kv_summary", "mix_summaries", "query_apply"))
    return {
        "qkv projection": (act + 3 * C * C * 2 + 3 * act + (4 * act if qk_norm else 0), 2 * R * C * 3 * C),
        "core": (core, 0),
        "lepe": ((3 * act + C * 26 * 4) if lepe else 0, 2 * 25 * R * C if lepe else 0),
        "output projection": (2 * act + C * C * 2, 2 * R * C * C),
    }


def bench_layer(args, p, torch, mh, synth):
    """One step = one mhla_layer_forward call (LayerNorm + QKV projection, the
    core, LePE, output projection) on seeded inputs resident in HBM."""
    if p.dtype != synth.BF16:
        print("the layer is bf16", file=sys.stderr)
        sys.exit(1)
    lepe = len(p.grid) == 2
    phi = mh.MHLA_PHI_RELU_EPS if args.phi == "relu" else mh.MHLA_PHI_ELU1
    R, C = p.batch * p.n_tokens, p.heads * p.head_dim
    sets = args.sets or max(2, int(np.ceil(2 * MALL_BYTES / (6 * R * C * 2))))

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    data, host0 = [], None
    for s in range(sets):
        x, P, W = synth.make_layer_inputs(p, seed=(args.config, s) if s else args.config, lepe=lepe,
                                          qk_norm=args.qk_norm)
        params = {}
        for name, val in P.items():
            if val is not None:
                params[name] = dev(val) if name.startswith("w_") else \
                    torch.from_numpy(np.ascontiguousarray(val, dtype=np.float32)).cuda()
        data.append((dev(x), torch.from_numpy(W).cuda(), params, torch.empty(R, C, dtype=torch.bfloat16,
                                                                            device="cuda").view(p.batch, p.n_tokens, C)))
        if s == 0:
            host0 = (x, P, W)
    gr = mh.make_grid(p.batch, p.heads, p.head_dim, mh.MHLA_BF16, p.grid, p.eps)
    bl = mh.make_block(p.block)
    ws_bytes = mh.mhla_layer_workspace_bytes(gr, bl)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i, events=None):
        x, W, params, y = data[i % sets]
        st = mh.mhla_layer_forward(x, W, gr, bl, params, y, ws, ws_bytes, phi=phi, stage_events=events,
                                   stream=stream)
        if st != mh.MHLA_OK:
            raise mh.MhlaError(st, "mhla_layer_forward")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    hev = HipEvents()
    evs = [[hev.create() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    stage_ms = np.array([[hev.elapsed_ms(r[j], r[j + 1]) for j in range(4)] for r in evs]).mean(axis=0)
    hev.destroy_all()
    stages = {}
    for j, (name, (nbytes, flops)) in enumerate(layer_costs(p, args.qk_norm, lepe).items()):
        t = stage_ms[j] * 1e-3
        gbps = nbytes / t / 1e9
        tflops = flops / t / 1e12
        stages[name] = {"avg_us": round(float(stage_ms[j]) * 1e3, 2), "alg_bytes": int(nbytes), "flops": int(flops),
                        "gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                        "tflops": round(tflops, 1), "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    traffic = measured_traffic(p.name + "-layer", "layer") if (not args.qk_norm and args.phi == "relu"
                                                                and not args.batch and not args.heads) else {}
    for n in stages:
        stages[n]["traffic"] = traffic.get(n)
    dom = max(stages, key=lambda n: stages[n]["avg_us"])
    d = stages[dom]
    if d["mfma_frac"] > d["hbm_frac"]:
        roof = {"bound": "mfma", "achieved": d["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": d["mfma_frac"]}
    else:
        roof = {"bound": "hbm", "achieved": d["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": d["hbm_frac"]}
    roof.update({"kernel": dom, "traffic": traffic.get(dom), "avg_us": d["avg_us"], "alg_bytes": d["alg_bytes"]})
    # compulsory bytes of the whole layer: x, y, the weights and W
    U = 2 * R * C * 2 + 4 * C * C * 2 + p.n_blocks ** 2 * 4
    cpu = None
    if not args.no_cpu:
        from oracle import layer as oracle_layer
        x, P, W = host0
        t = time.perf_counter()
        oracle_layer.layer_forward(x, W, p.grid, p.block, p.heads, P, eps=p.eps,
                                   kind=oracle_layer.PHI_RELU_EPS if args.phi == "relu" else oracle_layer.PHI_ELU1)
        dt_cpu = time.perf_counter() - t
        blas = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
        cpu = {"value": round(R / dt_cpu, 1), "unit": "tokens/s", "cores": blas, "kind": "oracle",
               "seconds": round(dt_cpu, 3),
               "sample": "the full workload, float64 numpy layer oracle (matrix products on the BLAS threads, "
                         "the rest on one thread)"}
    line = {
        "metric": "MHLA layer fwd tokens/s (LayerNorm, QKV projection, core, LePE, output projection)",
        "value": round(R / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{p.name} layer: B={p.batch} H={p.heads} d={p.head_dim} C={C} grid={list(p.grid)} "
                               f"blocks={list(p.block)} N={p.n_tokens} M={p.n_blocks}",
                   "phi": args.phi, "qk_norm": bool(args.qk_norm), "lepe": lepe, "input_sets": sets,
                   "parallelism": "none (1 GPU)"},
        "path_hbm_gbps": round(U / (ms_step * 1e-3) / 1e9, 1),
        "path_hbm_frac": round(U / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "path_alg_bytes": U,
        "kernels": stages,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    s = json.dumps(line)
    print(s, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(s + "\n")


def bench_stream(args, p, torch, mh, synth):
    """Stateful causal execution: one step streams the whole sequence (chunks =
    the grid's raster rows) through mhla_causal_stream in calls of
    --stream-chunks chunks, carrying the fp32 state of chunk summaries."""
    C = args.stream_chunks
    if len(p.grid) != 2 or p.block[1] != p.grid[1]:
        raise SystemExit("--stream-chunks needs a 2D grid whose chunks are whole raster rows")
    R = p.block[0]                    # raster rows per chunk
    rows = p.grid[0] // R             # chunks in the sequence
    if rows % C:
        raise SystemExit("--stream-chunks must divide the number of chunks")
    ncall = rows // C
    T = R * p.grid[1]                 # tokens per chunk
    dt = mh.MHLA_BF16 if p.dtype == synth.BF16 else mh.MHLA_F32

    def dev(x):
        if p.dtype == synth.BF16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    q, k, v, W = synth.make_inputs(p, seed=args.config, w_kind=args.w)
    n = C * T
    # per-call inputs and outputs, contiguous, resident before the timed region
    calls = []
    for c in range(ncall):
        sl = slice(c * n, (c + 1) * n)
        qs, ks, vs = (dev(np.ascontiguousarray(x[:, sl])) for x in (q, k, v))
        calls.append((qs, ks, vs, torch.empty_like(qs)))
    Wd = torch.from_numpy(W).cuda()
    g = mh.make_grid(p.batch, p.heads, p.head_dim, dt, (C * R, p.grid[1]), p.eps)
    b = mh.make_block((R, p.grid[1]))
    g_all = mh.make_grid(p.batch, p.heads, p.head_dim, dt, p.grid, p.eps)
    state = torch.empty(mh.mhla_causal_state_bytes(g_all, b, rows) // 4, dtype=torch.float32, device="cuda")
    wsb = mh.mhla_causal_stream_workspace_bytes(g, b)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def step():
        for c, (qs, ks, vs, out) in enumerate(calls):
            st = mh.mhla_causal_stream(qs, ks, vs, Wd, g, b, c * C, state, rows, out, ws, wsb)
            if st != mh.MHLA_OK:
                raise mh.MhlaError(st, "mhla_causal_stream")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    tensor_bytes = p.batch * p.n_tokens * p.heads * p.head_dim * p.elem_bytes
    U = 4 * tensor_bytes + 4 * p.n_blocks ** 2
    cpu = None
    if not args.no_cpu:
        import oracle
        ncpu = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        t = time.perf_counter()
        oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps, threads=ncpu)
        dt_cpu = time.perf_counter() - t
        cpu = {"value": round(p.batch * p.n_tokens / dt_cpu, 1), "unit": "tokens/s",
               "cores": min(ncpu, p.batch * p.heads), "kind": "oracle", "seconds": round(dt_cpu, 3),
               "sample": f"the full workload in one call ({p.batch * p.heads} (b,h) pairs, {p.n_tokens} tokens), "
                         "float64 causal chunkwise oracle, one thread per pair"}
    line = {
        "metric": "MHLA causal streaming tokens/s", "value": round(p.batch * p.n_tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if p.dtype == synth.BF16 else "f32", "data": "synthetic",
        "config": {"workload": f"{p.name}: B={p.batch} H={p.heads} d={p.head_dim} N={p.n_tokens}, "
                               f"{rows} chunks of {T} tokens streamed in {ncall} calls of {C} chunks",
                   "path": "causal stream", "w": args.w, "parallelism": "none (1 GPU)"},
        "path_hbm_gbps": round(U / (ms_step * 1e-3) / 1e9, 1), "path_alg_bytes": U,
        "ms_per_call": round(ms_step / ncall, 5),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the (b, h) pairs are "
              "independent, so more GPUs would each run their own share of them).", file=sys.stderr)
        sys.exit(2)

    import torch
    import token_level_head_block_amd as mh
    from token_level_head_block_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_mib:
        n = args.copy_mib << 20
        x = torch.empty(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(10):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "dispatches": 10}), flush=True)
        return
    mh.lib()   # fail loudly if the HIP library is missing

    p = synth.CONFIGS[args.config]
    if args.batch or args.heads:
        p = p.with_(batch=args.batch or p.batch, heads=args.heads or p.heads)
    if args.block:
        p = p.with_(block=tuple(int(x) for x in args.block.lower().split("x")))
    elif args.path == "causal":
        # contiguous chunks: one raster row of the grid each
        p = p.with_(name=p.name + "-causal-rows", block=(1,) * (len(p.grid) - 1) + (p.grid[-1],))
    if args.backward:
        bench_backward(args, p, torch, mh, synth)
        return
    if args.layer:
        bench_layer(args, p, torch, mh, synth)
        return
    if args.stream_chunks:
        if args.path != "causal":
            raise SystemExit("--stream-chunks streams the causal form: add --path causal")
        bench_stream(args, p, torch, mh, synth)
        return
    path = {"3kernel": mh.MHLA_PATH_3KERNEL, "fused": mh.MHLA_PATH_FUSED, "causal": mh.MHLA_PATH_CAUSAL}[args.path]
    tensor_bytes = p.batch * p.n_tokens * p.heads * p.head_dim * p.elem_bytes
    per_set = 4 * tensor_bytes
    sets = args.sets or max(2, int(np.ceil(2 * MALL_BYTES / per_set)))
    dt = torch.bfloat16 if p.dtype == synth.BF16 else torch.float32

    def dev(x):
        if p.dtype == synth.BF16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    data = []
    for s in range(sets):
        q, k, v, W = synth.make_inputs(p, seed=(args.config, s) if s else args.config, w_kind=args.w)
        data.append((dev(q), dev(k), dev(v), torch.from_numpy(W).cuda(), torch.empty(q.shape, dtype=dt, device="cuda")))
        if s == 0:
            host0 = (q, k, v, W)
    g = mh.make_grid(p.batch, p.heads, p.head_dim, mh.MHLA_BF16 if p.dtype == synth.BF16 else mh.MHLA_F32,
                     p.grid, p.eps)
    b = mh.make_block(p.block)
    ws_bytes = mh.mhla_workspace_bytes(g, b)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i, events=None):
        q, k, v, W, out = data[i % sets]
        st = mh.mhla_forward_ex(q, k, v, W, g, b, out, ws, ws_bytes, path, events, stream)
        if st != mh.MHLA_OK:
            raise mh.MhlaError(st, "mhla_forward_ex")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` forward passes
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    tokens_per_s = p.batch * p.n_tokens / (ms_step * 1e-3)
    U = 4 * tensor_bytes + 4 * p.n_blocks ** 2
    path_gbps = U / (ms_step * 1e-3) / 1e9

    # ---- per-kernel attribution: stage events on the launch stream, same loop.
    # The events skip the system-scope fence (cache write-back) that a default
    # event performs when it completes, so they cost almost nothing between
    # kernels and agree with rocprofv3's kernel durations.
    nstage = args.steps
    hev = HipEvents()
    evs = [[hev.create() for _ in range(4)] for _ in range(nstage)]
    torch.cuda.synchronize()
    for i in range(nstage):
        step(i, evs[i])
    torch.cuda.synchronize()
    stage_ms = np.array([[hev.elapsed_ms(row[j], row[j + 1]) for j in range(3)] for row in evs])
    hev.destroy_all()
    avg = stage_ms.mean(axis=0)
    st_plan, plan = mh.mhla_launch_plan(g, b, path)
    if st_plan != mh.MHLA_OK:
        raise mh.MhlaError(st_plan, "mhla_launch_plan")
    names = plan if len(plan) == 3 else [plan[0], "(none)", plan[1]]
    ws_elem = p.elem_bytes
    kb = kernel_bytes(p, ws_elem)
    kernels = {}
    for j, n in enumerate(names):
        if n == "(none)":
            continue
        gbps = kb[n] / (avg[j] * 1e-3) / 1e9
        kernels[n] = {"avg_us": round(float(avg[j]) * 1e3, 2), "alg_bytes": int(kb[n]),
                      "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    dom = max(kernels, key=lambda n: kernels[n]["avg_us"])
    traffic = measured_traffic(p.name, args.path) if (args.path != "fused" and args.w == "gaussian"
                                           and not args.batch and not args.heads and not args.block) else {}
    mfma = measured_mfma(p.name, args.path) if (args.path != "fused" and args.w == "gaussian"
                                                 and not args.batch and not args.heads and not args.block) else {}
    for n in kernels:
        kernels[n]["traffic"] = traffic.get(n)
        # matrix-core use: counter flops of one dispatch over its event-timed duration, against
        # the dense bf16 peak
        f = mfma.get(n)
        tf = f / (kernels[n]["avg_us"] * 1e-6) / 1e12 if f else None
        kernels[n]["mfma_tflops"] = round(tf, 1) if tf else None
        kernels[n]["mfma_util"] = round(tf / MFMA_PEAK_BF16_TFLOPS, 4) if tf else None
    roofline = {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["gbps"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": kernels[dom]["frac"], "traffic": traffic.get(dom),
                "avg_us": kernels[dom]["avg_us"], "alg_bytes": kernels[dom]["alg_bytes"]}

    # ---- a plain device copy of the path's compulsory bytes, in the same run
    copy_us, copy_gbps = measure_copy(torch, U)

    # ---- CPU baseline: the float64 oracle on the host cores
    cpu = None
    if not args.no_cpu:
        import oracle
        q, k, v, W = host0
        ncpu, model = host_cpu()
        if args.path == "causal":
            dt_cpu, runs, _ = time_cpu(lambda: oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps,
                                                                     threads=ncpu))
            used = min(ncpu, p.batch * p.heads)   # the causal oracle runs one thread per (b, h) pair at most
            how = "causal chunkwise oracle, one thread per (b, h) pair"
        else:
            dt_cpu, runs, r = time_cpu(lambda: oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps,
                                                              threads=ncpu, return_threads=True))
            used = r[1]
            how = "blockwise oracle, threads over (pair, block) units"
        cpu = {"value": round(p.batch * p.n_tokens / dt_cpu, 1), "unit": "tokens/s", "cores": used,
               "kind": "oracle", "seconds": round(dt_cpu, 3), "host_cores": ncpu, "cpu_model": model,
               "sample": f"the full workload ({p.batch * p.heads} (b,h) pairs, {p.n_tokens} tokens), "
                         f"float64 {how}, best of {runs} runs"}

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if p.dtype == synth.BF16 else "f32", "data": "synthetic",
        "precision": (("q, k, v, out bf16; summaries [S|z] as bf16 records; fp32 accumulation; W (fp32 input) "
                       + {"causal": "as bf16 high and low parts in the mixing, mixed S bf16 and z fp32",
                          "fused": "applied in fp32 inside the apply, mixed S staged as bf16"}.get(
                           args.path, "rounded to bf16 for the mixing product, mixed S bf16 and z fp32"))
                      if p.dtype == synth.BF16 else "fp32 throughout"),
        "config": {"workload": f"{p.name}: B={p.batch} H={p.heads} d={p.head_dim} grid={list(p.grid)} "
                               f"blocks={list(p.block)} N={p.n_tokens} M={p.n_blocks}",
                   "path": args.path, "w": args.w, "input_sets": sets, "parallelism": "none (1 GPU)"},
        "path_hbm_gbps": round(path_gbps, 1), "path_hbm_frac": round(path_gbps / HBM_PEAK_GBPS, 4),
        "path_alg_bytes": U,
        "copy": {"bytes": U, "us": round(copy_us, 2), "gbps": round(copy_gbps, 1),
                 "frac_of_peak": round(copy_gbps / HBM_PEAK_GBPS, 4),
                 "what": "device-to-device copy of the path's compulsory byte count (read and written), "
                         "rotating buffers, same process"},
        "copy_gbps": round(copy_gbps, 1), "frac_of_copy": round(path_gbps / copy_gbps, 4),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    s = json.dumps(line)
    print(s, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
