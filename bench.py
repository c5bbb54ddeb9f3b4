"""Benchmark of the MoE experts step on one MI355X.

A step is one full experts pass (align, GEMM1 + activation, GEMM2, combine;
for the pre-grouped layout: segment tables, GEMM1, GEMM2, zero tail) over one
batch of synthetic, seeded input resident in HBM. Prints one JSON line.

The metric has two halves: bf16 prefill TFLOP/s and MXFP4 decode weight-stream
GB/s. The default run (--workload all) measures four workloads one after the
other and puts the headline on the largest, the fine-grained prefill layer
(T=8192, H=7168, I=2048, E=256 resident experts, top-8, Zipf-skewed load);
the Mixtral-shaped prefill, the MXFP4 decode step, the pre-grouped layout
and the MXFP4-weight prefill with MXFP8 activations (the decode layer's
shapes at 8192 tokens, on the block-scaled MFMA, roofline against the fp8
peak) go into the same line under "configs", each with its step time,
value, roofline and CPU-oracle baseline.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|NAME]
                  [--no-cpu-baseline] [--calib-copy] [--router] [--act-fmt bf16|mxfp8]
                  [--weight-copies N]

The K timed steps of a workload run twice after the warm-up: first with
hipEvents that the library records between its launches on the benchmark's
stream (the *_timed entry points), which give the per-kernel times (stage_ms,
the roofline's kernel time), then with no instrumentation: that pass's
wall-clock time gives ms_per_step and value. Decode steps rotate over several
copies of the weights (--weight-copies, default 4, 6.8 GB in all), so that
the 256 MB Infinity Cache cannot serve one step's weights to the next.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (MXFP8 x MXFP4 block-scaled MFMAs run at this rate)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
STAGES = ("align", "gemm1", "gemm2", "combine")
METRIC = "MoE experts TFLOP/s (bf16 prefill) + weight-stream GB/s (MXFP4 decode), 1 GPU"
HEADLINE = "fine_grained_prefill"
NESTED = ("mixtral_prefill", "mxfp4_decode", "pregrouped", "mxfp4_prefill")
DECODE_MIN_STEPS = 200      # a 0.2 ms step: fewer steps let the timed region's ends show


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed steps of the headline workload (decode workloads time at least "
                         f"{DECODE_MIN_STEPS}, reported in their own 'steps')")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    help="'all' (headline fine_grained_prefill plus nested configs) or one workload name")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None,
                    help="tokens (rows) of the oracle's sample; default per workload")
    ap.add_argument("--print-source-hash", action="store_true")
    ap.add_argument("--router", action="store_true",
                    help="run the router (moe_route, Renormalize) on the workload's logits inside each step")
    ap.add_argument("--act-fmt", default=None, choices=("bf16", "mxfp8"),
                    help="activation format of the GEMM inputs (mxfp8: MXFP4-weight workloads only); "
                         "default: the workload's own")
    ap.add_argument("--weight-copies", type=int, default=4,
                    help="MXFP4 decode: copies of the weights the steps rotate over")
    ap.add_argument("--row-layout", action="store_true",
                    help="keep the weights in their canonical layout instead of the kernels' layouts made once "
                         "before the timed steps (moe_bf16_pack_weights, moe_mx_pack_weights)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device copy (HBM counter calibration under rocprofv3 --pmc)")
    return ap.parse_args()


# Oracle sample per workload (tokens, or rows of the pre-grouped layout):
# about 2-8 s of float64 BLAS work on 16 host threads each.
CPU_SAMPLE = {"fine_grained_prefill": 512, "mixtral_prefill": 1024, "mxfp4_decode": 32, "pregrouped": 1024,
              "tiny": 64, "mxfp4_prefill": 16}


def is_decode(wl) -> bool:
    """MXFP4 workloads with at most 32 routed rows per expert: the weight
    stream is the metric (GB/s); everything else is a prefill (TFLOP/s)."""
    return wl.wfmt == "mxfp4" and wl.T * wl.k <= 32 * wl.E


def timed_passes(step, K, hev, n_ev, extra=None):
    """K steps with n_ev events per step (and one more per step when extra is
    set), then K steps with no events, whose wall-clock time is the step time
    (an event record between two launches leaves a gap on the stream: about
    14 us per decode step of 0.22 ms). Returns (ms_per_step, instrumented
    ms_per_step, events, extra events)."""
    import torch
    evs = [hev.create(n_ev) for _ in range(K)]
    xevs = hev.create(K) if extra else [None] * K
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, evs[i], xevs[i])
    torch.cuda.synchronize()
    instr = (time.perf_counter() - t0) * 1e3 / K
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    plain = (time.perf_counter() - t0) * 1e3 / K
    return plain, instr, evs, xevs


class HipEvents:
    """Minimal hipEvent_t plumbing through ctypes (timing only)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream.cuda_stream)) == 0

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        assert rc == 0, rc
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def kernel_source_hash(kind: str) -> str:
    """sha256 of the sources a GEMM1 kernel is built from (bf16: the prefill
    GEMM, with the align that leaves the cold segments out of its tiles and
    the cold-segment kernel beside it; mxfp4: the decode GEMM; mx_prefill: the
    block-scaled prefill GEMM)."""
    import hashlib
    h = hashlib.sha256()
    files = {"bf16": ("common.hpp", "align.hpp", "gemm_bf16.hpp", "gemm_cold.hpp"), "mxfp4": ("common.hpp", "gemm_skinny.hpp"),
             "mx_prefill": ("common.hpp", "gemm_bf16.hpp", "gemm_mx.hpp")}[kind]
    for f in files:
        with open(os.path.join(ROOT, "mixture_experts_expert_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(name: str, wfmt: str):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 counter summary
    profiles/gemm1_<name>_counters.txt: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter read for a 1 GiB device
    copy. None when there is no summary or the GEMM sources changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", f"gemm1_{name}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash(wfmt):
        return None
    copy_bytes = float(kv["copy_bytes"])
    f_scale = copy_bytes / (float(kv["copy_fetch_kib"]) * 1024.0)
    w_scale = copy_bytes / (float(kv["copy_write_kib"]) * 1024.0)
    return (float(kv["gemm1_fetch_kib"]) * 1024.0 * f_scale + float(kv["gemm1_write_kib"]) * 1024.0 * w_scale)


def touched_weight_bytes(wl, ids):
    import numpy as np
    n = len(np.unique(ids[(ids >= 0) & (ids < wl.E)]))
    per = 3 * wl.H * wl.I * (0.5 + 1.0 / 32 if wl.wfmt == "mxfp4" else 2.0)
    return n, n * per


def cpu_threads():
    """(threads the oracle's BLAS runs on, CPUs this process may use, CPUs of the host)."""
    import threadpoolctl
    info = threadpoolctl.threadpool_info()
    blas = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count() or 1
    return int(blas), int(aff), int(os.cpu_count() or 1)


def cpu_baseline(wl, x, ids, w, W, S, n_tokens, act_fmt="bf16"):
    """The CPU oracle, as it is, on the first n_tokens tokens of the workload
    (with the experts they touch, renumbered, copied to the host)."""
    import numpy as np
    import torch
    import oracle
    import synth
    n_tokens = min(n_tokens, wl.T)
    ids_s = ids[:n_tokens]
    touched = sorted({int(e) for e in ids_s.ravel() if 0 <= e < wl.E})
    remap = np.full(wl.E, -1, dtype=np.int32)
    remap[touched] = np.arange(len(touched), dtype=np.int32)
    ids_c = np.where((ids_s >= 0) & (ids_s < wl.E), remap[np.clip(ids_s, 0, wl.E - 1)], -1).astype(np.int32)
    xs = synth.bf16_to_f32(x[:n_tokens])
    sel = torch.as_tensor(touched, device=x.device)
    if wl.wfmt == "mxfp4":
        Wh = [(W[i].index_select(0, sel).cpu().numpy(), S[i].index_select(0, sel).cpu().numpy()) for i in range(3)]
    else:
        Wh = [synth.bf16_to_f32(W[i].index_select(0, sel)) for i in range(3)]
    kw = dict(act=wl.act, alpha=wl.alpha, beta=wl.beta, limit=wl.limit, act_fmt=act_fmt)
    blas, aff, host = cpu_threads()
    t0 = time.perf_counter()
    oracle.experts_forward(xs, ids_c, w[:n_tokens], *Wh, **kw)
    dt = time.perf_counter() - t0
    slots = int(np.sum(ids_c >= 0))
    if is_decode(wl):
        value = len(touched) * 3 * wl.H * wl.I * (0.5 + 1 / 32) / dt / 1e9
        unit = "GB/s"
    else:
        value = 6.0 * slots * wl.H * wl.I / dt / 1e12
        unit = "TFLOP/s"
    return {"value": round(value, 4), "unit": unit, "cores": blas, "kind": "oracle",
            "sample": f"first {n_tokens} of {wl.T} tokens ({slots} routed slots, {len(touched)} experts) of "
                      f"{wl.name}, float64 numpy on {blas} BLAS threads, {dt:.1f} s",
            "cpus_available": aff, "host_cpus": host}


def cpu_baseline_pregrouped(wl, x, cu, rw, W, n_rows):
    """The float64 oracle on rows [0, n_rows) of the pre-grouped layout (the
    segments they fall in, with their weights copied to the host)."""
    import numpy as np
    import torch
    import oracle
    import synth
    segs = [g for g in range(len(cu)) if (cu[g - 1] if g else 0) < n_rows and cu[g] > (cu[g - 1] if g else 0)]
    sub_cu = np.minimum(np.array([cu[g] for g in segs]), n_rows)
    xs = synth.bf16_to_f32(x[:n_rows])
    sel = torch.as_tensor(segs, device=x.device)
    Wh = [synth.bf16_to_f32(t.index_select(0, sel)) for t in W]
    blas, aff, host = cpu_threads()
    t0 = time.perf_counter()
    oracle.pregrouped_forward(xs, sub_cu, rw[:n_rows], *Wh)
    dt = time.perf_counter() - t0
    flops = 6.0 * n_rows * wl.H * wl.I
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": blas, "kind": "oracle",
            "sample": f"first {n_rows} of {wl.T} rows ({len(segs)} segments) of {wl.name}, float64 numpy on "
                      f"{blas} BLAS threads, {dt:.1f} s",
            "cpus_available": aff, "host_cpus": host}


def _calib_copy(dev):
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    del a, b


def run_pregrouped(args, wl, dev, K):
    """The pre-grouped entry (rows already contiguous per weight row, caller's
    cu_seqlens) on the pre-grouped workload: GEMM1, GEMM2 and the zero tail."""
    import numpy as np
    import torch
    import synth
    from mixture_experts_expert_02_amd import binding as B
    print(f"[bench] workload {wl.name}: NvS={wl.T} H={wl.H} I={wl.I} segments={wl.E}", file=sys.stderr, flush=True)
    lengths, source = synth.make_pregrouped_layout(wl)
    cu = np.cumsum(lengths).astype(np.int32)
    x = synth.make_x(wl, device=dev)
    W = synth.make_bf16_weights(wl, device=dev, source=source)
    rw = synth.make_route_weights_nvs(wl)
    cu_d, rw_d = torch.from_numpy(cu).to(dev), torch.from_numpy(rw).to(dev)
    p = B.problem(wl.T, wl.H, wl.I, wl.E, 1, wl.wfmt, wl.act, wl.alpha, wl.beta, wl.limit)
    packed = None
    if wl.wfmt == "bf16" and not args.row_layout:
        # the prefill kernels' operand-block weight layout, made once before the
        # timed steps (flashinfer_moe_ep page, process_weights_after_loading)
        packed = B.bf16_pack_weights(p, *W)
        torch.cuda.synchronize()
        p.bf16_packed = packed.data_ptr()
    ws = B.alloc_workspace(B.moe_experts_grouped_workspace_bytes(p), dev)
    out = torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    hev = HipEvents()

    def step(i, evs=(), _unused=None):
        rc = B.moe_experts_forward_grouped_timed(p, x, cu_d, rw_d, *W, None, None, None, out, ws, list(evs),
                                                 stream=stream)
        if rc != 0:
            raise B.MoeError(rc, "moe_experts_forward_grouped_timed")

    for i in range(args.warmup):
        step(i)
    if args.calib_copy:
        _calib_copy(dev)
    torch.cuda.synchronize()
    ms_per_step, instr_ms, evs, _ = timed_passes(step, K, hev, 5)
    stages = ("prep", "gemm1", "gemm2", "zero_tail")
    avg = {s: float(np.mean([hev.elapsed_ms(e[j], e[j + 1]) for e in evs])) for j, s in enumerate(stages)}
    step_ms = float(np.mean([hev.elapsed_ms(e[0], e[4]) for e in evs]))
    for e in evs:
        hev.destroy(e)
    M = int(cu[-1])
    n_touched = int(np.sum(lengths > 0))
    value = 6.0 * M * wl.H * wl.I / (ms_per_step * 1e-3) / 1e12
    achieved = 4.0 * M * wl.H * wl.I / (avg["gemm1"] * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": counter_traffic(wl.name, wl.wfmt),
            "kernel": "gemm1 (gate+up, bf16)",
            "algorithmic_bytes": n_touched * 2 * wl.I * wl.H * 2 + M * wl.H * 2 + M * wl.I * 2}
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "steps": K,
        "ms_per_step": round(ms_per_step, 4), "dtype": "bf16",
        "config": {"workload": wl.name, "NvS": wl.T, "H": wl.H, "I": wl.I, "segments": wl.E, "weights": wl.wfmt,
                   "activation": wl.act, "routed_rows": M, "touched_experts": n_touched,
                   **({"weight_layout": "packed once before the timed steps (moe_bf16_pack_weights)"}
                      if packed is not None else {})},
        "stage_ms": {s: round(v, 4) for s, v in avg.items()},
        "event_ms_per_step": round(step_ms, 4),
        "instrumented_ms_per_step": round(instr_ms, 4),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] {wl.name}: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        n = args.cpu_sample_tokens or CPU_SAMPLE[wl.name]
        res["cpu_baseline"] = cpu_baseline_pregrouped(wl, x, cu, rw, W, n)
    return res


def run_token_major(args, wl, dev, K, act_fmt):
    import numpy as np
    import torch
    import synth
    from mixture_experts_expert_02_amd import binding as B
    print(f"[bench] workload {wl.name}: T={wl.T} H={wl.H} I={wl.I} E={wl.E} k={wl.k} {wl.wfmt}", file=sys.stderr,
          flush=True)
    ids, w = synth.make_routing(wl)
    ids_d, w_d = torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)
    x = synth.make_x(wl, device=dev)
    if wl.wfmt == "mxfp4":
        (cg, sg), (cu, su), (cd, sd) = synth.make_mxfp4_weights(wl, device=dev)
        W, S = (cg, cu, cd), (sg, su, sd)
        copies = max(1, args.weight_copies) if is_decode(wl) else 1
    else:
        W, S = synth.make_bf16_weights(wl, device=dev), (None, None, None)
        copies = 1
    # copy 0 is the generated tensors; the others are clones at other addresses
    sets = [(W, S)] + [(tuple(t.clone() for t in W), tuple(t.clone() for t in S) if S[0] is not None else S)
                       for _ in range(copies - 1)]
    p = B.problem(wl.T, wl.H, wl.I, wl.E, wl.k, wl.wfmt, wl.act, wl.alpha, wl.beta, wl.limit, act_fmt=act_fmt)
    packs = None
    if not args.row_layout:
        # the kernels' weight layouts, made once per weight copy before the
        # timed steps (flashinfer_moe_ep page, process_weights_after_loading):
        # MXFP4 for the prefill GEMMs and the decode kernels' codes, bf16 for
        # the tiled and cold-segment prefill GEMMs
        if wl.wfmt == "mxfp4":
            packs = [B.mx_pack_weights(p, *Wc, *Sc) for Wc, Sc in sets]
        else:
            packs = [B.bf16_pack_weights(p, *W)]
        torch.cuda.synchronize()

    def set_packed(i):
        if packs is not None:
            if wl.wfmt == "mxfp4":
                p.mx_packed = packs[i % len(packs)].data_ptr()
            else:
                p.bf16_packed = packs[i % len(packs)].data_ptr()

    set_packed(0)
    ws = B.alloc_workspace(B.moe_experts_workspace_bytes(p), dev)
    out = torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    hev = HipEvents()

    if args.router:
        # the workload's ids and weights are this same Renormalize routing of these logits
        logits_d = torch.from_numpy(synth.make_logits(wl)).to(dev)
        rp = B.route_problem(wl.T, wl.E, wl.k, "renormalize")

    def step(i, evs=(), rev=None):
        Wi, Si = sets[i % copies]
        set_packed(i)
        if args.router:
            if rev is not None:
                hev.record(rev, stream)
            rc = B.moe_route(rp, logits_d, None, ids_d, w_d, stream=stream)
            if rc != 0:
                raise B.MoeError(rc, "moe_route")
        rc = B.moe_experts_forward_timed(p, x, ids_d, w_d, *Wi, *Si, out, ws, list(evs), stream=stream)
        if rc != 0:
            raise B.MoeError(rc, "moe_experts_forward_timed")

    for i in range(args.warmup):
        step(i)
    if args.calib_copy:
        _calib_copy(dev)
    torch.cuda.synchronize()

    ms_per_step, instr_ms, evs, revs = timed_passes(step, K, hev, 5, extra=args.router)
    stage_ms = {s: [] for s in (("router",) if args.router else ()) + STAGES}
    for e, r in zip(evs, revs):
        for j, s in enumerate(STAGES):
            stage_ms[s].append(hev.elapsed_ms(e[j], e[j + 1]))
        if args.router:
            stage_ms["router"].append(hev.elapsed_ms(r, e[0]))
    step_ms = [hev.elapsed_ms(r if args.router else e[0], e[4]) for e, r in zip(evs, revs)]
    for e in evs:
        hev.destroy(e)
    if args.router:
        hev.destroy(revs)

    M = wl.T * wl.k
    n_touched, wbytes = touched_weight_bytes(wl, ids)
    avg = {s: float(np.mean(v)) for s, v in stage_ms.items()}
    lay = B.moe_experts_workspace_layout(p)
    single = bool(lay.single_launch)
    if single:  # GEMM1, GEMM2 and the combine share one launch after the align
        avg = {"align": avg["align"], "gemm1+gemm2+combine": avg["gemm1"] + avg["gemm2"] + avg["combine"],
               **({"router": avg["router"]} if "router" in avg else {})}
    if lay.mx_tiled:  # the token rows' quantization and the scale blocks run before GEMM1
        avg = {("align+quant+prep" if s == "align" else s): v for s, v in avg.items()}
        unit = "TFLOP/s"
        value = wl.flops / (ms_per_step * 1e-3) / 1e12
        g1_flops = 4.0 * M * wl.H * wl.I
        achieved = g1_flops / (avg["gemm1"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": counter_traffic(wl.name, "mx_prefill"),
                "kernel": "gemm1 (gate+up, MXFP4 weights x MXFP8 activations, v_mfma_scale_f32_32x32x64_f8f6f4)",
                "algorithmic_bytes": int(n_touched * 2 * wl.I * wl.H * (0.5 + 1 / 32) + wl.T * wl.H * (1 + 1 / 32)
                                         + M * wl.I * (1 + 1 / 32))}
    elif wl.wfmt == "bf16":
        unit = "TFLOP/s"
        value = wl.flops / (ms_per_step * 1e-3) / 1e12
        g1_flops = 4.0 * M * wl.H * wl.I
        achieved = g1_flops / (avg["gemm1"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": counter_traffic(wl.name, wl.wfmt),
                "kernel": "gemm1 (gate+up, bf16)",
                "algorithmic_bytes": n_touched * 2 * wl.I * wl.H * 2 + M * wl.H * 2 + M * wl.I * 2}
    else:
        unit = "GB/s"
        value = (wbytes + 2 * wl.T * wl.H * 2) / (ms_per_step * 1e-3) / 1e9
        tag = wl.name + ("" if act_fmt == "bf16" else "_" + act_fmt)
        if single:
            k_bytes = wbytes + 2 * wl.T * wl.H * 2
            achieved = k_bytes / (avg["gemm1+gemm2+combine"] * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": counter_traffic(tag, wl.wfmt),
                    "kernel": "k_decode_fused (GEMM1 + GEMM2 + combine, one launch, MXFP4)",
                    "algorithmic_bytes": k_bytes}
        else:
            g1_bytes = n_touched * 2 * wl.H * wl.I * (0.5 + 1 / 32)
            achieved = g1_bytes / (avg["gemm1"] * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": counter_traffic(tag, wl.wfmt),
                    "kernel": "gemm1 (gate+up, MXFP4)", "algorithmic_bytes": g1_bytes}
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "steps": K,
        "ms_per_step": round(ms_per_step, 4),
        "dtype": "bf16" if wl.wfmt == "bf16" else f"mxfp4-weights/{act_fmt}-act",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "top_k": wl.k,
                   "weights": wl.wfmt, "activation": wl.act, "routed_rows": M, "touched_experts": n_touched,
                   **({"weight_copies": copies} if copies > 1 else {}),
                   **({"activations": act_fmt} if act_fmt != "bf16" else {}),
                   **({"weight_layout": "packed once before the timed steps ("
                                        + ("moe_mx_pack_weights)" if wl.wfmt == "mxfp4" else "moe_bf16_pack_weights)")}
                      if packs is not None else {})},
        "stage_ms": {s: round(v, 4) for s, v in avg.items()},
        "event_ms_per_step": round(float(np.mean(step_ms)), 4),
        "instrumented_ms_per_step": round(instr_ms, 4),
        "roofline": roof,
    }
    if args.router:
        rbytes = wl.T * wl.E * 4 + wl.T * wl.k * 8
        gbs = rbytes / (avg["router"] * 1e-3) / 1e9
        res["config"]["router"] = "renormalize"
        res["router"] = {"kernel": "k_route (Renormalize)", "us": round(avg["router"] * 1e3, 2),
                         "algorithmic_bytes": rbytes, "achieved": round(gbs, 1), "unit": "GB/s",
                         "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4), "bound": "hbm"}
    if not args.no_cpu_baseline:
        print(f"[bench] {wl.name}: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        n = args.cpu_sample_tokens or CPU_SAMPLE.get(wl.name, 1024)
        res["cpu_baseline"] = cpu_baseline(wl, x, ids, w, W, S, n, act_fmt)
    return res


def run_one(args, name, dev, K):
    import gc
    import torch
    import synth
    wl = synth.workload(name)
    if is_decode(wl):
        K = max(K, DECODE_MIN_STEPS)
    act_fmt = (args.act_fmt or wl.act_fmt) if wl.wfmt == "mxfp4" else "bf16"
    res = run_pregrouped(args, wl, dev, K) if wl.pregrouped else run_token_major(args, wl, dev, K, act_fmt)
    gc.collect()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.print_source_hash:
        import synth
        wl = synth.WORKLOADS[args.workload]
        print(kernel_source_hash("mx_prefill" if wl.act_fmt == "mxfp8" and not is_decode(wl) else wl.wfmt))
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the experts step "
              f"holds every expert on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    from mixture_experts_expert_02_amd import binding as B

    B.lib()  # fail loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    names = [HEADLINE, *NESTED] if args.workload == "all" else [args.workload]
    for n in names:
        if n not in synth.WORKLOADS:
            print(f"bench.py: unknown workload {n!r}", file=sys.stderr)
            sys.exit(2)
    if args.act_fmt not in (None, "bf16") and all(synth.WORKLOADS[n].wfmt != "mxfp4" for n in names):
        print(f"bench.py: --act-fmt {args.act_fmt} needs an MXFP4-weight workload", file=sys.stderr)
        sys.exit(2)
    results = {}
    for n in names:
        results[n] = run_one(args, n, dev, args.steps)
        r = results[n]
        print(f"[bench] {n}: {r['value']} {r['unit']}, {r['ms_per_step']} ms/step, "
              f"roofline frac {r['roofline']['frac']}", file=sys.stderr, flush=True)
    head = results[names[0]]
    line = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1, "steps": head["steps"],
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic",
        "config": head["config"],
        **{k: v for k, v in head.items() if k not in ("metric", "value", "unit", "steps", "ms_per_step", "dtype",
                                                     "config")},
    }
    if len(names) > 1:
        line["configs"] = {n: results[n] for n in names[1:]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
