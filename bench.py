#!/usr/bin/env python3
"""Throughput of the low-bit routed-expert MoE layer on one MI355X.

One step = the whole layer on one batch: moe_route -> moe_permute -> moe_expert_ffn (its
stages: prepare, FC1 + SwiGLU, FC2) -> moe_combine, on synthetic seeded inputs that are
already resident in HBM.  Default workload: the decode layer (384 experts, top-8, hidden
4096, intermediate 2048, 2-bit codebook weights with group-32 bf16 scales, Zipf-skewed
routing) at T = 64 tokens.

Every step is timed with HIP events on the stream the kernels run on; the last-level
caches are flushed between steps (outside the events) by *reading* a 1 GiB buffer, so the
expert weights come from HBM.  (A write flush would leave the 256 MB last-level cache full of
dirty lines whose write-back then competes with the timed kernels: a measurement artefact.)
Steps are timed twice: launched eagerly (each FFN stage between its own pair of events, which
gives the per-kernel times), and as one HIP graph capturing the step, replayed -- the way a
serving loop runs the decode step; `value` comes from the graph replays, checked to give the
eager result bit for bit.  The FC1 kernel (2/3 of the weight bytes and flops) is the dominant
kernel: its algorithmic bytes (decode: packed weights of the experts that received tokens, x
read once, h written once) or flops (prefill) divided by its event-timed duration give
`roofline.achieved`.

Prints one JSON line.  `--gpus` above 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
GEMM_MIN_TOKENS = 128          # the library runs the grouped-GEMM kernels from this batch size
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published
METRIC = "MoE-layer tokens/sec + weight HBM GB/s (decode) / MFMA % (prefill)"
CSRC = os.path.join(ROOT, "bit_moe_expert_top_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def csrc_digest() -> str:
    """sha256 over the kernel sources: a measured HBM-traffic figure is valid only for these."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel, from a committed counter summary under
    profiles/ (a line `bench-traffic: {json}`), if it was taken on the current sources."""
    if not os.path.isdir(PROFILES):
        return None
    digest = csrc_digest()
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        with open(os.path.join(PROFILES, name)) as f:
            for line in f:
                if line.startswith("bench-traffic:"):
                    rec = json.loads(line[len("bench-traffic:"):])
                    if rec.get("workload") == workload and rec.get("csrc_sha256") == digest:
                        return rec["bytes_per_launch"]
    return None


def weight_bytes_per_expert(sp: dict, which: int, fmt: str | None = None) -> int:
    """Packed bytes (codes + scales) of one expert's W1 (which=1) or W2 (which=2), in the
    layer's low-bit format or in `fmt` ("w2", "w3", "mxfp4")."""
    H, I = sp["H"], sp["I"]
    n = 2 * I * H if which == 1 else H * I
    fmt = fmt or sp["fmt"]
    if fmt == "w2":
        return n // 4 + (n // 32) * 2
    if fmt == "mxfp4":
        return n // 2 + n // 32
    return n * 3 // 8 + n // 64


def cpu_baseline(sp, batch, T, n_tok):
    """The oracle, as it stands, on the first n_tok tokens of the same batch."""
    import numpy as np

    from oracle import moe as OM
    import moegen

    logits, x = batch["logits"][:n_tok], batch["x"][:n_tok]
    ids, _ = OM.route(logits, sp["k"])
    used = sorted(set(ids.reshape(-1).tolist()))
    # only the experts the sample routes to are materialised for the oracle
    arrays = {}
    for e in used:
        for key, a in moegen.expert(sp, e).items():
            arrays.setdefault(key, {})[e] = a
    full = {key: np.zeros((sp["E"],) + next(iter(d.values())).shape, next(iter(d.values())).dtype)
            for key, d in arrays.items()}
    for key, d in arrays.items():
        for e, a in d.items():
            full[key][e] = a
    lay = OM.Layer(sp["fmt"], full)
    # the same sample again until about 10 s of CPU work have been timed (at most 8 passes)
    passes = 0
    t0 = time.perf_counter()
    while True:
        OM.layer_forward(lay, logits, x, sp["k"])
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or passes >= 8:
            break
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    try:  # the threads numpy's BLAS used for the matmuls
        from threadpoolctl import threadpool_info

        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        blas_threads = max((i.get("num_threads") or 0) for i in blas) if blas else None
    except ImportError:
        blas_threads = None
    return {"value": passes * n_tok / dt, "unit": "tokens/s", "cores": cores, "blas_threads": blas_threads,
            "kind": "oracle",
            "sample": f"first {n_tok} of the {T} tokens ({len(used)} experts), numpy fp64, {passes} passes "
                      f"in {dt:.1f} s"}


def setup_layer(name: str):
    import numpy as np  # noqa: F401

    import moegen
    from bit_moe_expert_top_amd import _lib as L

    sp = moegen.spec(name)
    print(f"[bench] generating layer {name} (E={sp['E']} k={sp['k']} H={sp['H']} I={sp['I']} {sp['fmt']})",
          file=sys.stderr, flush=True)
    arrays = moegen.weights(sp)
    flags = L.MOE_FLAG_HOT_RESIDUAL if sp["hot_mode"] == "residual" else 0
    dw = L.DeviceWeights({"w2": 1, "w3": 2}[sp["fmt"]], sp["E"], sp["H"], sp["I"], arrays, flags=flags)
    return sp, dw


def measure(sp: dict, dw, T: int, steps: int, warmup: int, flush_between: bool = True,
            batch_invariant: bool = False) -> dict:
    """Time `steps` layer steps on T tokens; returns the bench record (without cpu_baseline)."""
    import numpy as np
    import torch

    import moegen
    from bit_moe_expert_top_amd import _lib as L

    k, E, H, I = sp["k"], sp["E"], sp["H"], sp["I"]
    batch = moegen.batch(sp, T)
    dev = torch.device("cuda")
    logits = torch.from_numpy(batch["logits"]).to(dev)
    x = torch.from_numpy(batch["x"].view(np.int16)).to(dev)
    R = T * k
    i32 = dict(dtype=torch.int32, device=dev)
    ids = torch.empty((T, k), **i32)
    gw = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    perm, inv = torch.empty(R, **i32), torch.empty(R, **i32)
    ws_p = torch.empty(max(1, L.moe_permute_ws_bytes(T, k, E)), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(max(1, L.moe_expert_ffn_ws_bytes(dw, T, k)), dtype=torch.uint8, device=dev)
    y = torch.empty((R, H), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    n_stages = L.moe_expert_ffn_num_stages(dw, T, k, ws_f.numel())
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB, read to evict caches
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # with a hot set, the hot experts' preparation and MXFP4 -> FP8 conversion run on a second
    # stream, concurrent with the low-bit stages
    side = torch.cuda.Stream() if sp["n_hot"] > 0 else None

    # decode-sized batches: routing, grouping and the FFN's preparation (stage 0) in one call
    # (one launch up to 16 tokens, two above)
    front = side is None and T * k <= L.FRONT_MAX_ROWS

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        if front:
            if evs:
                evs[1].record(stream)
            L.moe_route_permute_prepare(dw, logits, x, k, ws_f, out=(ids, gw, counts, offsets, perm, inv))
            if evs:
                evs[2].record(stream)
        else:
            L.moe_route(logits, k, ids, gw)
            L.moe_permute(ids, E, ws=ws_p, out=(counts, offsets, perm, inv))
        stage_evs = {s: (evs[1 + 2 * s], evs[2 + 2 * s]) for s in range(n_stages)} if evs else None
        if side is not None:
            L.moe_expert_ffn_two_streams(dw, x, k, counts, offsets, perm, y, ws_f, side, stage_evs)
        else:
            for s in range(1 if front else 0, n_stages):
                if evs:
                    evs[1 + 2 * s].record(stream)
                L.moe_expert_ffn_stage(dw, x, k, counts, offsets, perm, y, ws_f, s)
                if evs:
                    evs[2 + 2 * s].record(stream)
        L.moe_combine(y, inv, gw, out_fp32=False, out=out)
        if evs:
            evs[-1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    n_active = int((counts > 0).sum().item())
    print(f"[bench] T={T}: {n_active} experts active; timing {steps} steps", file=sys.stderr, flush=True)

    all_evs = [[ev() for _ in range(2 + 2 * n_stages)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush_between:
            flush.sum()
        step(all_evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the same step captured once in a HIP graph and replayed (the decode step of a serving
    # loop is graph-captured): no per-kernel launch gaps; caches flushed between replays too
    graph_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        gev = [(ev(), ev()) for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            if flush_between:
                flush.sum()
            gev[i][0].record(stream)
            g.replay()
            gev[i][1].record(stream)
        torch.cuda.synchronize()
        graph_ms = [a.elapsed_time(b) for a, b in gev]
        # the replayed layer must produce the eager result
        out_graph = out.clone()
        step()
        torch.cuda.synchronize()
        if not torch.equal(out_graph, out):
            raise RuntimeError("graph replay differs from the eager step")
    except RuntimeError as e:  # capture unsupported: report the eager number only
        print(f"[bench] graph replay skipped: {e}", file=sys.stderr, flush=True)
        graph_ms = None

    step_ms = [e[0].elapsed_time(e[-1]) for e in all_evs]
    stage_ms = [[e[1 + 2 * s].elapsed_time(e[2 + 2 * s]) for e in all_evs] for s in range(n_stages)]
    eager_ms = float(np.mean(step_ms))
    ms = float(np.mean(graph_ms)) if graph_ms else eager_ms
    # low-bit stages: 1 FC1 streaming, 2 FC1 grouped GEMM, 3 FC2 streaming, 4 FC2 grouped GEMM;
    # with a hot set: 5 hot prepare, then per batch of hot experts 3 stages (convert, FP8 FC1,
    # FP8 FC2)
    fc1_ms = float(np.mean(stage_ms[1]) + np.mean(stage_ms[2]))
    fc2_ms = float(np.mean(stage_ms[3]) + np.mean(stage_ms[4]))
    hot_batches = (n_stages - 6) // 3 if sp["n_hot"] > 0 else 0
    conv_ms = sum(float(np.mean(stage_ms[6 + 3 * b])) for b in range(hot_batches))
    hot_fc1_ms = sum(float(np.mean(stage_ms[7 + 3 * b])) for b in range(hot_batches))
    hot_fc2_ms = sum(float(np.mean(stage_ms[8 + 3 * b])) for b in range(hot_batches))
    hot = torch.zeros(E, dtype=torch.bool, device=dev)
    if sp["n_hot"] > 0:
        hot[torch.from_numpy(moegen.hot_ids(sp)).long().to(dev)] = True
    n_hot_active = int(((counts > 0) & hot).sum().item())
    n_cold_active = n_active - n_hot_active
    hot_rows = int(counts[hot].sum().item())
    residual = sp["hot_mode"] == "residual"  # hot experts: 2-bit codes + an MXFP4 residual, both read
    hot_b = {which: weight_bytes_per_expert(sp, which, "mxfp4") + (weight_bytes_per_expert(sp, which) if residual else 0)
             for which in (1, 2)}
    w1b = n_cold_active * weight_bytes_per_expert(sp, 1) + n_hot_active * hot_b[1]
    w2b = n_cold_active * weight_bytes_per_expert(sp, 2) + n_hot_active * hot_b[2]
    gemm = T >= GEMM_MIN_TOKENS and not batch_invariant  # the invariant mode streams every group
    workload = f"{sp['name']} MoE layer E={E} top-{k} H={H} I={I} {sp['fmt']} T={T}"
    if sp["n_hot"] > 0:
        workload += (f" ({sp['n_hot']} hot experts with an mxfp4 residual)" if residual
                     else f" ({sp['n_hot']} hot experts mxfp4->fp8)")
    if batch_invariant:
        workload += " batch-invariant mode"
    if hot_batches > 0 and hot_rows > 0:
        # hot experts carry most rows: their FP8 FC1 (+ SwiGLU + MXFP8 of h) is the dominant
        # kernel; algorithmic flops = 2 * rows * (2I) * H over the hot experts' rows
        f = 2.0 * hot_rows * (2 * I) * H
        roof_ms = hot_fc1_ms / hot_batches
        achieved = f / hot_batches / (roof_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "moe_expert_ffn hot FP8 FC1 + SwiGLU + MXFP8 of h (fp8_gemm_kernel<1, MODE>)",
                "achieved": achieved, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / FP8_PEAK_TFLOPS, "alg_flops_per_launch": f / hot_batches, "hot_rows": hot_rows}
    elif gemm:
        # prefill-sized: FC1 of the groups above 32 rows is the grouped GEMM (stage 2);
        # algorithmic flops = 2 * rows * (2I) * H over the rows of those groups
        gemm_rows = int(counts[(counts > 32) & ~hot].sum().item())
        fc1_flops = 2.0 * gemm_rows * (2 * I) * H
        roof_ms = float(np.mean(stage_ms[2]))
        achieved = fc1_flops / (roof_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "moe_expert_ffn stage 2: FC1 + SwiGLU grouped GEMM (gemm_kernel<W2Fmt, 1, 2, 8>)",
                "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS, "alg_flops_per_launch": fc1_flops, "gemm_rows": gemm_rows}
    else:
        # decode-sized: FC1 streams the packed W1 bytes of every expert that received a
        # token, reads x once and writes h once
        fc1_bytes = w1b + T * H * 2 + R * I * 2
        roof_ms = float(np.mean(stage_ms[1]))  # the streaming kernel (stage 2 launches nothing)
        achieved = fc1_bytes / (roof_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "moe_expert_ffn stage 1: FC1 + SwiGLU weight streaming (stream_kernel<"
                + ("W3Fmt" if sp["fmt"] == "w3" else "W2Fmt") + ", 1, G, " + ("true" if residual else "false") + ">)",
                "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "alg_bytes_per_launch": fc1_bytes}
    roof["traffic"] = measured_traffic(workload)
    roof["avg_launch_ms"] = roof_ms
    all_flops = 2.0 * R * 3 * I * H
    # the whole layer against its roofline: t_roof = max(flops_bf16 / P_bf16 + flops_fp8 / P_fp8,
    # algorithmic bytes / HBM peak), with the bytes = packed weights of the experts that received
    # rows + logits + x + out (bf16)
    f_fp8 = 0.0 if residual else 2.0 * hot_rows * 3 * I * H
    f_bf16 = all_flops - f_fp8
    t_mfma = (f_bf16 / (BF16_PEAK_TFLOPS * 1e12) + f_fp8 / (FP8_PEAK_TFLOPS * 1e12)) * 1e3
    layer_bytes = w1b + w2b + T * E * 4 + T * H * 2 + T * H * 2
    t_hbm = layer_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
    layer_roof = {"bound": "mfma" if t_mfma > t_hbm else "hbm", "t_roof_ms": max(t_mfma, t_hbm),
                  "t_mfma_ms": t_mfma, "t_hbm_ms": t_hbm, "flops": all_flops, "alg_bytes": layer_bytes,
                  "frac": max(t_mfma, t_hbm) / ms}
    return {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded; uniform {sp['fmt']} codes and scales, N(0,1) bf16 x, Zipf s=1.1 router logits)",
        "config": {"workload": workload, "tokens": T, "experts_active": n_active,
                   "cache_flush_between_steps": flush_between, "batch_invariant": batch_invariant},
        "roofline": roof,
        "layer_roofline": layer_roof,
        "step_timing": "HIP graph replay" if graph_ms else "eager launches",
        "ms_per_step_eager": eager_ms,
        "hot_convert_overlapped": side is not None,
        "front_call": front,  # moe_route_permute_prepare instead of route + permute + stage 0
        "stages_ms": {"route+permute+prepare+combine (eager; stage sum for one stream)": eager_ms - fc1_ms - fc2_ms - conv_ms - hot_fc1_ms - hot_fc2_ms,
                      "fc1": fc1_ms, "fc2": fc2_ms, "hot_convert": conv_ms, "hot_fc1": hot_fc1_ms, "hot_fc2": hot_fc2_ms},
        "ffn_stage_ms": [float(np.mean(v)) for v in stage_ms],
        "weight_GBps_fc1_fc2": (w1b + w2b) / ((fc1_ms + fc2_ms + hot_fc1_ms + hot_fc2_ms) * 1e-3) / 1e9,
        "ffn_TFLOPs_fc1_fc2": all_flops / ((fc1_ms + fc2_ms + hot_fc1_ms + hot_fc2_ms) * 1e-3) / 1e12,
        "ms_per_step_min": float(np.min(graph_ms or step_ms)),
        "ms_per_step_median": float(np.median(graph_ms or step_ms)),
        "wall_s_timed_loop_incl_flush": wall,
    }


def extra_measurement(name: str, T: int, steps: int, warmup: int) -> dict:
    """A second workload in the same run (its own layer, freed afterwards): the prefill half of
    the metric (grouped-GEMM MFMA fraction) and the mixed layer (FP8 MFMA fraction)."""
    import gc

    import torch

    sp, dw = setup_layer(name)
    r = measure(sp, dw, T, steps, warmup)
    del dw
    gc.collect()
    torch.cuda.empty_cache()
    return {"workload": r["config"]["workload"], "value": r["value"], "unit": r["unit"],
            "ms_per_step": r["ms_per_step"], "steps": steps, "warmup": warmup,
            "experts_active": r["config"]["experts_active"], "roofline": r["roofline"],
            "layer_roofline": r["layer_roofline"], "stages_ms": r["stages_ms"],
            "step_timing": r["step_timing"]}


def measure_quantize(steps: int, warmup: int, flush_between: bool = True) -> dict:
    """Time the quantisers (fp32 weights -> 2-bit codebook, -> MXFP4) on the W1 matrices of 8
    experts of the decode/prefill shape: [8 * 4096][4096] fp32 (512 MiB), resident in HBM.
    Both kernels read each weight once: bound = HBM, algorithmic bytes = 4 per weight in plus
    the packed bytes out."""
    import numpy as np
    import torch

    from bit_moe_expert_top_amd import _lib as L

    rows, K = 8 * 4096, 4096
    n = rows * K
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    w = torch.randn((rows, K), generator=g, device="cuda", dtype=torch.float32) * 0.02
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for name, f, out_b in (("w2", L.moe_quantize_w2, 2.0 / 8 + 2.0 / 32), ("mxfp4", L.moe_quantize_mxfp4, 0.5 + 1.0 / 32)):
        for _ in range(warmup):
            f(w)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            if flush_between:
                flush.sum()
            a.record(stream)
            f(w)
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        res[name] = {"ms": ms, "weights_per_s": n / (ms * 1e-3), "GBps": n * (4 + out_b) / (ms * 1e-3) / 1e9}
    r = res["w2"]
    workload = f"quantise W1 of 8 experts: f32[{rows}][{K}]"
    return {
        "metric": "quantiser weights/s (fp32 -> 2-bit codebook + bf16 group-32 scales)",
        "value": r["weights_per_s"], "unit": "weights/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": r["ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (N(0, 0.02^2) fp32 weights, seeded torch generator)",
        "config": {"workload": workload, "cache_flush_between_steps": flush_between},
        "roofline": {"bound": "hbm", "kernel": "quantize_w2_kernel", "achieved": r["GBps"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": r["GBps"] / HBM_PEAK_GBS, "traffic": measured_traffic(workload),
                     "alg_bytes_per_launch": n * (4 + 2.0 / 8 + 2.0 / 32), "avg_launch_ms": r["ms"]},
        "mxfp4": res["mxfp4"],
    }


def copy_calibration(mib: int):
    """A plain device copy of known size (mib MiB read, mib MiB written), run after the timed
    region so that one counter run sees both it and the timed kernels: FETCH_SIZE and
    WRITE_SIZE of this copy scale the same counters of the other kernels to bytes."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {mib} MiB read + {mib} MiB written", file=sys.stderr, flush=True)


def measure_tier(sp: dict, arrays: dict, T: int, n_slots: int, steps: int, warmup: int,
                 pipelined: bool = False) -> dict:
    """The layer with its experts in pinned host memory and n_slots of them on the GPU (an LRU
    cache): every step is a new batch of T tokens, so misses are copied host -> device inside the
    timed step (which also synchronises once, for the plan).  Wall-clock time per step."""
    import numpy as np
    import torch

    import moegen
    from bit_moe_expert_top_amd import _lib as L

    k = sp["k"]
    tl = L.TieredLayer({"w2": 1, "w3": 2}[sp["fmt"]], sp["E"], sp["H"], sp["I"], arrays, n_slots)
    pool = moegen.batch(sp, (steps + warmup) * T)
    lg = torch.from_numpy(pool["logits"]).cuda()
    x = torch.from_numpy(pool["x"].view(np.int16)).cuda()
    per_expert = weight_bytes_per_expert(sp, 1) + weight_bytes_per_expert(sp, 2)
    stream = torch.cuda.current_stream()
    if pipelined:
        tl.forward_pipelined([(lg[i * T:(i + 1) * T], x[i * T:(i + 1) * T]) for i in range(warmup)], k)
    else:
        for i in range(warmup):
            tl.forward(lg[i * T:(i + 1) * T], x[i * T:(i + 1) * T], k)
    torch.cuda.synchronize()
    loaded0 = tl.loaded
    ms, load_ms, routed = [], [], 0
    orig_load = L.moe_tier_load

    def timed_load(*a):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        orig_load(*a)
        e1.record(stream)
        load_ms.append((e0, e1))

    if pipelined:
        # the copies of step i+1 overlap the FFN of step i (second stream); one timed sequence
        batches = [(lg[i * T:(i + 1) * T], x[i * T:(i + 1) * T]) for i in range(warmup, warmup + steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        outs = tl.forward_pipelined(batches, k)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        ms = [wall_ms / steps] * steps
        routed = sum(int((torch.bincount(o["ids"].view(-1).long(), minlength=sp["E"]) > 0).sum().item()) for o in outs)
    L.moe_tier_load = timed_load
    try:
        for i in (range(0) if pipelined else range(warmup, warmup + steps)):
            t0 = time.perf_counter()
            r = tl.forward(lg[i * T:(i + 1) * T], x[i * T:(i + 1) * T], k)
            torch.cuda.synchronize()
            ms.append((time.perf_counter() - t0) * 1e3)
            routed += int((r["counts"] > 0).sum().item())
    finally:
        L.moe_tier_load = orig_load
    loads = tl.loaded - loaded0
    copy_ms = float(sum(a.elapsed_time(b) for a, b in load_ms)) if not pipelined else 0.0
    step_ms = float(np.mean(ms))
    return {
        "metric": METRIC, "value": T / (step_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded), a new batch every step",
        "config": {"workload": f"{sp['name']} MoE layer E={sp['E']} top-{k} H={sp['H']} I={sp['I']} {sp['fmt']} "
                               f"T={T}, experts in pinned host RAM, {n_slots} GPU slots (LRU)"
                               + (", copies of step i+1 overlapped with step i" if pipelined else ""), "tokens": T},
        "tier": {"slots": n_slots, "experts_used_per_step": routed / steps, "loads_per_step": loads / steps,
                 "hit_rate": 1.0 - loads / max(1, routed), "h2d_bytes_per_step": loads * per_expert / steps,
                 "h2d_ms_per_step": copy_ms / steps if not pipelined else None,
                 "h2d_GBps": loads * per_expert / (copy_ms * 1e-3) / 1e9 if copy_ms > 0 else None},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layer", default="decode",
                    help="decode | prefill | mixed | residual | w3 | tiny | quantize (the quantisers, not a layer)")
    ap.add_argument("--T", type=int, default=64)
    ap.add_argument("--no-flush", action="store_true", help="do not flush caches between steps")
    ap.add_argument("--tier-slots", type=int, default=0,
                    help="keep the experts in pinned host RAM with this many GPU slots (LRU); 0 = all resident")
    ap.add_argument("--tier-pipeline", action="store_true",
                    help="with --tier-slots: overlap the copies of step i+1 with the FFN of step i")
    ap.add_argument("--batch-invariant", action="store_true",
                    help="run the layer in its batch-invariant mode (same bits for a token at any T)")
    ap.add_argument("--cpu-tokens", type=int, default=64, help="tokens of the oracle's timed sample (0 = skip)")
    ap.add_argument("--extras", default="prefill,mixed",
                    help="with the default decode T=64 run, also measure these workloads in the same run "
                         "(prefill = T 8192, mixed = T 4096; empty = none)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after timing, run a plain copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this MoE layer path runs on one GPU; --gpus above 1 is not supported "
              "(an expert-parallel split over several GPUs is not built)", file=sys.stderr)
        sys.exit(2)
    if args.layer == "quantize":
        res = measure_quantize(args.steps, args.warmup, not args.no_flush)
        if args.copy_calib_mib > 0:
            copy_calibration(args.copy_calib_mib)
        print(json.dumps(res), flush=True)
        return
    if args.tier_slots > 0:
        import moegen

        sp = moegen.spec(args.layer)
        print(json.dumps(measure_tier(sp, moegen.weights(sp), args.T, args.tier_slots, args.steps, args.warmup,
                                      args.tier_pipeline)), flush=True)
        return
    sp, dw = setup_layer(args.layer)
    dw.set_batch_invariant(args.batch_invariant)
    res = measure(sp, dw, args.T, args.steps, args.warmup, not args.no_flush, args.batch_invariant)
    if args.copy_calib_mib > 0:
        copy_calibration(args.copy_calib_mib)
    extras = [e for e in args.extras.split(",") if e] if (args.layer == "decode" and args.T == 64
                                                          and not args.batch_invariant) else []
    if extras:
        import gc

        import torch

        del dw
        gc.collect()
        torch.cuda.empty_cache()
        sizes = {"prefill": 8192, "mixed": 4096}
        for name in extras:
            res[name] = extra_measurement(name, sizes[name], min(args.steps, 10), min(args.warmup, 3))
    if args.cpu_tokens > 0:
        import moegen

        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(sp, moegen.batch(sp, args.T), args.T, min(args.cpu_tokens, args.T))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
