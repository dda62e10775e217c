"""Benchmark of the batch-invariant MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--T T]

A step is one moe_layer_forward (routing, permutation, gate/up SwiGLU GEMM,
down GEMM, combine) over one batch of seeded synthetic tokens whose inputs are
already resident in HBM.  The default workload is the small bf16 layer
(T=512, D=1024, E=64 routed + 1 shared expert, top-6 sigmoid routing, expert
inter dim 512).  Several replicas of the expert weights are rotated across
steps so that the 256 MB last-level cache cannot hold the weights between
steps.

Prints ONE JSON line with throughput (tokens/s), the roofline of the dominant
kernel (the gate/up SwiGLU GEMM) measured with HIP events recorded between the
stages of every timed step, and the CPU oracle timed on the host.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (FP4 x FP8 runs at the FP8 rate)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "gate_up_gemm_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=2, help="layer recipe (1..5), default 2")
    p.add_argument("--T", type=int, default=None, help="override the batch size")
    p.add_argument("--replicas", type=int, default=0, help="weight replicas (0 = auto)")
    p.add_argument("--w4a8", action="store_true",
                   help="MXFP4 routed experts on MXFP8 activations (FP4 x FP8 MFMA)")
    p.add_argument("--glu", choices=("swiglu", "clamp", "situ"), default="swiglu",
                   help="gated activation of the expert FFNs (clamped SwiGLU, SiTU-GLU)")
    p.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                          "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                   help="turn rocprofv3 --pmc counter CSVs (FETCH_SIZE run, WRITE_SIZE run, and "
                        "the same two counters over --copy-calibration) into the gate/up GEMM "
                        "HBM bytes per launch; writes profiles/gate_up_gemm_traffic.json")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate CPU time budget of the oracle baseline (0 = skip)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (counter calibration)")
    return p.parse_args()


class Hip:
    """hipEvent helpers through the HIP runtime (events live on the caller's stream)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.L.hipEventRecord(e, stream) == 0

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.hpp", "kernels.hpp"):
        with open(os.path.join(ROOT, "invariant_moe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(per_launch_bytes_alg: float):
    """HBM bytes per launch of the gate/up GEMM from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


def _counter_means(path, counter, name_pred):
    import csv
    vals = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and name_pred(row["Kernel_Name"]):
                vals.append(float(row["Counter_Value"]))
    return vals


def traffic_summary(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the gate/up GEMM, each
    scaled by the bytes a 1 GiB device copy really moves over what the same
    counter reports for it."""
    gated = lambda n: "k_grouped_gemm_bf16<" in n and ", true, " in n
    copy = lambda n: "copyBuffer" in n
    f = _counter_means(fetch_csv, "FETCH_SIZE", gated)
    w = _counter_means(write_csv, "WRITE_SIZE", gated)
    cf = _counter_means(cal_fetch_csv, "FETCH_SIZE", copy)
    cw = _counter_means(cal_write_csv, "WRITE_SIZE", copy)
    if not (f and w and cf and cw):
        raise SystemExit("traffic summary: missing counter rows")
    n = float(1 << 30)
    kf = n / (sum(cf) / len(cf) * 1024.0)
    kw = n / (sum(cw) / len(cw) * 1024.0)
    fetch = sum(f) / len(f) * 1024.0 * kf
    write = sum(w) / len(w) * 1024.0 * kw
    d = {"kernel": "k_grouped_gemm_bf16 gate/up (gated) launch",
         "kernel_source_hash": kernel_source_hash(),
         "dispatches": [len(f), len(w)],
         "fetch_size_kib_avg": round(sum(f) / len(f), 1),
         "write_size_kib_avg": round(sum(w) / len(w), 1),
         "copy_factor_fetch": round(kf, 4), "copy_factor_write": round(kw, 4),
         "fetch_bytes_per_launch": int(fetch), "write_bytes_per_launch": int(write),
         "bytes_per_launch": int(fetch + write)}
    with open(PROFILE_TRAFFIC, "w") as fh:
        json.dump(d, fh, indent=1)
        fh.write("\n")
    print(json.dumps(d))


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def tail_measurement(cfg, hip, sptr, steps: int):
    """The MoE tail at the recipe's shape: the combine fused with the next
    block's residual add + RMSNorm (one kernel), against the combine followed
    by the standalone norm (two kernels, y written and read back).  Synthetic
    expert outputs, shared output, residual and gain; distinct random experts
    per token and a random pair -> row permutation."""
    import torch

    import invariant_moe_amd as moe

    T, D, E, k = cfg.T, cfg.D, cfg.E, cfg.k
    R = T * k
    dt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    es = 4 if cfg.act == "f32" else 2
    g = torch.Generator(device="cuda").manual_seed(1234)
    o = torch.randn((R, D), device="cuda", generator=g).to(dt)
    sh = torch.randn((T, D), device="cuda", generator=g).to(dt) if cfg.I_shared else None
    res = torch.randn((T, D), device="cuda", generator=g).to(dt)
    gamma = (1.0 + 0.1 * torch.randn(D, device="cuda", generator=g)).to(dt)
    idx = torch.rand((T, E), device="cuda", generator=g).argsort(dim=1)[:, :k].to(torch.int32)
    w = torch.rand((T, k), device="cuda", generator=g)
    w = (w / w.sum(1, keepdim=True)).contiguous()
    pair_row = torch.randperm(R, device="cuda", generator=g).to(torch.int32)
    idx = idx.contiguous()
    y = torch.empty((T, D), dtype=dt, device="cuda")
    h = torch.empty_like(res)
    n = torch.empty_like(res)
    eps = 1e-6

    def unfused():
        moe.combine(o, idx, w, pair_row, sh, out=y)
        moe.residual_rmsnorm(y, res, gamma, eps, residual_out=h, normed=n)

    def fused():
        moe.combine_rmsnorm(o, idx, w, pair_row, sh, res, gamma, eps, residual_out=h, normed=n)

    out = {}
    for name, fn in (("unfused", unfused), ("fused", fused)):
        for _ in range(3):
            fn()
        a, b = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(a, sptr)
        for _ in range(steps):
            fn()
        hip.record(b, sptr)
        torch.cuda.synchronize()
        out[name] = hip.elapsed_ms(a, b) / steps
    # algorithmic bytes of the fused kernel: expert rows, shared row, residual
    # in, residual and normed out, gain, slot indices / weights / rows
    fused_bytes = (R * D + (T * D if sh is not None else 0) + 3 * T * D + D) * es + R * 12
    unfused_bytes = fused_bytes + 2 * T * D * es  # y written, then read
    gbs = fused_bytes / (out["fused"] * 1e-3) / 1e9
    return {"fused_us": round(out["fused"] * 1e3, 2), "unfused_us": round(out["unfused"] * 1e3, 2),
            "fused_alg_bytes": int(fused_bytes), "unfused_alg_bytes": int(unfused_bytes),
            "fused_gbs": round(gbs, 1), "fused_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "unfused_gbs": round(unfused_bytes / (out["unfused"] * 1e-3) / 1e9, 1),
            "kernel": "k_residual_rmsnorm (combine fused with residual add + RMSNorm)"}


def w4a8_measurement(dl, x, ids, hip, sptr, steps: int):
    """The routed expert FFN of an MXFP4-weight workload, on this batch's routed
    rows: bf16 activations (MXFP4 decoded to bf16, bf16 MFMA) against MXFP8
    activations on the scaled FP4 x FP8 MFMA (moe_grouped_swiglu_w4a8)."""
    import torch

    import invariant_moe_amd as moe

    cfg = dl.cfg
    T, D, E, k, I = cfg.T, cfg.D, cfg.E, cfg.k, cfg.I
    R = T * k
    idx, _ = moe.router_topk(x, dl.w_router, dl.bias, ids, E, k, cfg.route)
    _, offsets, row_token, _, _ = moe.permute(idx, E)
    w = moe.ExpertWeights(dl.gate, dl.up, dl.down, dl.gate_scale, dl.up_scale, dl.down_scale)
    out = torch.empty((R, D), dtype=x.dtype, device=x.device)

    def w4a16():
        moe.grouped_swiglu(x, row_token, offsets, R, E, w, out=out)

    def w4a8():
        moe.grouped_swiglu_w4a8(x, row_token, offsets, R, E, w, out=out)

    res = {}
    for name, fn in (("w4a16", w4a16), ("w4a8", w4a8)):
        for _ in range(3):
            fn()
        a, b = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(a, sptr)
        for _ in range(steps):
            fn()
        hip.record(b, sptr)
        torch.cuda.synchronize()
        res[name] = hip.elapsed_ms(a, b) / steps
    flops = 6 * R * D * I
    return {"w4a16_ms": round(res["w4a16"], 4), "w4a8_ms": round(res["w4a8"], 4),
            "w4a16_tflops": round(flops / (res["w4a16"] * 1e-3) / 1e12, 1),
            "w4a8_tflops": round(flops / (res["w4a8"] * 1e-3) / 1e12, 1),
            "w4a8_frac_of_fp8_peak": round(flops / (res["w4a8"] * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
            "rows": R, "includes": "activation quantisation, tile tables, both GEMMs",
            "kernel": "k_grouped_gemm_w4a8 (v_mfma_scale_f32_16x16x128_f8f6f4) vs "
                      "k_grouped_gemm_bf16 on decoded MXFP4"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {args.gpus} requested); the layer is "
              "not sharded across GPUs here.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return

    import numpy as np
    import torch

    import invariant_moe_amd as moe
    import synth
    from synth import device as sdev

    cfg = synth.CONFIGS[args.config]
    if args.T is not None:
        cfg = cfg.with_T(args.T)
    if args.w4a8 and cfg.wdtype != "mxfp4":
        print("bench.py: --w4a8 needs a recipe with MXFP4 routed weights (recipe 5)",
              file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    hip = Hip()

    print(f"[bench] uploading recipe {cfg.cid} ({cfg.name}) T={cfg.T}", file=sys.stderr, flush=True)
    dl = sdev.upload_layer(cfg, dev)
    wbytes_routed = dl.gate.numel() * dl.gate.element_size() * 3  # gate + up + down (+pack)
    if dl.gate_scale is not None:
        wbytes_routed += 3 * dl.gate_scale.numel()
    # replicas so the weights do not stay in the 256 MB last-level cache
    nrep = args.replicas or max(1, min(8, int(np.ceil(1.2e9 / max(wbytes_routed, 1)))))
    layers = [sdev.layer_object(dl, args.glu, args.w4a8)]
    for _ in range(nrep - 1):
        c = sdev.DeviceLayer(cfg, dl.w_router, dl.bias, dl.gate.clone(), dl.up.clone(),
                             dl.down.clone(),
                             None if dl.gate_scale is None else dl.gate_scale.clone(),
                             None if dl.up_scale is None else dl.up_scale.clone(),
                             None if dl.down_scale is None else dl.down_scale.clone(),
                             None if dl.sh_gate is None else dl.sh_gate.clone(),
                             None if dl.sh_up is None else dl.sh_up.clone(),
                             None if dl.sh_down is None else dl.sh_down.clone())
        layers.append(sdev.layer_object(c, args.glu, args.w4a8))
    x = sdev.x_device(cfg, dev)
    ids = sdev.token_ids_device(cfg, dev)
    y = torch.empty((cfg.T, cfg.D), dtype=x.dtype, device=dev)

    # routing statistics of this batch (for the algorithmic byte count)
    idx, _ = moe.router_topk(x, dl.w_router, dl.bias, ids, cfg.E, cfg.k, cfg.route)
    counts = torch.bincount(idx.flatten().long(), minlength=cfg.E).cpu().numpy()
    U = int((counts > 0).sum())

    for i in range(args.warmup):
        layers[i % nrep].forward(x, ids, out=y)
    torch.cuda.synchronize()

    K = args.steps
    # Pass 1 (the measurement): K steps with no instrumentation inside; one
    # event pair and the host clock bracket them.
    ev0, ev1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(ev0, sptr)
    for i in range(K):
        layers[i % nrep].forward(x, ids, out=y)
    hip.record(ev1, sptr)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = hip.elapsed_ms(ev0, ev1)
    ms_per_step = max(wall * 1e3, gpu_ms) / K

    # Pass 2: the same steps with events between the stages (each event
    # record costs GPU time, so these sum to more than a step of pass 1).
    evs = [[hip.event() for _ in range(6)] for _ in range(K)]
    for i in range(K):
        moe.set_stage_events(evs[i])
        layers[i % nrep].forward(x, ids, out=y)
    moe.set_stage_events(None)
    torch.cuda.synchronize()
    stage_ms = np.array([[hip.elapsed_ms(evs[i][s], evs[i][s + 1]) for s in range(5)]
                         for i in range(K)])
    stage_avg = stage_ms.mean(0)
    # Pass 3: kernel-only time of the two GEMM launches, from events recorded
    # at the kernels' own start and end (hipExtLaunchKernel).
    K2 = min(K, 50)
    kev = [[hip.event() for _ in range(10)] for _ in range(K2)]
    for i in range(K2):
        moe.set_stage_events(kev[i])
        layers[i % nrep].forward(x, ids, out=y)
    moe.set_stage_events(None)
    torch.cuda.synchronize()
    try:
        kern_ms = np.array([[hip.elapsed_ms(kev[i][6], kev[i][7]),
                             hip.elapsed_ms(kev[i][8], kev[i][9])] for i in range(K2)]).mean(0)
    except AssertionError:  # a library without kernel events: stage times instead
        kern_ms = stage_avg[[2, 3]]
    gu_ms = float(kern_ms[0])

    tail = tail_measurement(cfg, hip, sptr, min(K, 50))
    w4a8 = (w4a8_measurement(dl, x, ids, hip, sptr, min(K, 20))
            if cfg.wdtype == "mxfp4" and cfg.D % 128 == 0 and cfg.I % 128 == 0 else None)

    # algorithmic work of the gate/up SwiGLU GEMM launch (routed + shared groups)
    T, D, E, k, I, Is = cfg.T, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared
    R = T * k
    es = 4 if cfg.act == "f32" else 2
    if cfg.wdtype == "mxfp4":
        w_gu = U * 2 * I * (D // 2 + D // 32)
    else:
        w_gu = U * 2 * I * D * es
    w_gu += 2 * Is * D * es
    gu_bytes = w_gu + T * D * es + (R * I + T * Is) * es
    gu_flops = 4 * R * D * I + 4 * T * D * Is
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
    traffic = measured_traffic(gu_bytes)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": "k_grouped_gemm_bf16 (gate/up + SwiGLU)",
                "alg_bytes_per_launch": int(gu_bytes),
                "avg_launch_ms": round(gu_ms, 5),
                "mfma_tflops": round(gu_flops / (gu_ms * 1e-3) / 1e12, 2),
                "mfma_frac": round(gu_flops / (gu_ms * 1e-3) / 1e12 /
                                   (FP8_PEAK_TFLOPS if args.w4a8 else BF16_PEAK_TFLOPS), 4)}
    if cfg.act == "f32":
        roofline["bound"] = "hbm"

    # whole-layer algorithmic traffic (touched experts once, shared, router, x, y)
    layer_w = w_gu * 3 // 2 if cfg.wdtype != "mxfp4" else U * 3 * I * (D // 2 + D // 32) + 3 * Is * D * es
    layer_bytes = layer_w + (E * D * es if cfg.route != "hash" else 0) + 2 * T * D * es
    layer_flops = 6 * R * D * I + 6 * T * D * Is + (2 * T * D * E if cfg.route != "hash" else 0)

    # CPU oracle on the host cores (bounded sample of the same workload)
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        xs = synth.x_tokens(cfg)
        idsn = synth.token_ids(cfg) if cfg.route == "hash" else None
        T_s = cfg.T
        if cfg.D * cfg.I * cfg.k > 1 << 26:  # large layers: a 16-token slice
            T_s = min(16, cfg.T)
            xs = np.ascontiguousarray(xs[:T_s])
            idsn = None if idsn is None else np.ascontiguousarray(idsn[:T_s])
        lg_idx = None
        experts = {}
        if cfg.route == "hash":
            lg_idx, _ = oracle.route(None, None, idsn, T_s, E, k, "hash")
        else:
            lg = oracle.router_logits(xs, synth.router_weight(cfg))
            lg_idx, _ = oracle.route(lg, synth.router_bias(cfg), None, T_s, E, k, cfg.route)
        for e in np.unique(lg_idx):
            experts[int(e)] = synth.expert_matrices(cfg, int(e))
        wr = synth.router_weight(cfg) if cfg.route != "hash" else None
        bias = synth.router_bias(cfg)
        sh = synth.shared_matrices(cfg)
        runs, t_cpu = 0, 0.0
        while runs == 0 or t_cpu < args.cpu_seconds:
            c0 = time.perf_counter()
            oracle.layer_forward(xs, idsn, wr, bias, experts, sh, T_s, D, E, k, I,
                                 Is, cfg.route, cfg.wdtype, glu=args.glu)
            t_cpu += time.perf_counter() - c0
            runs += 1
        cpu = {"value": round(runs * T_s / t_cpu, 2), "unit": "tokens/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{runs} x oracle layer forward of {T_s} tokens of the same recipe "
                         f"({t_cpu:.1f} s)"}

    tokens_per_s = cfg.T / (ms_per_step * 1e-3)
    out = {
        "metric": "MoE-layer tokens/s; %MFMA peak (prefill), %HBM GB/s (decode)",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.act == "f32" else "bf16",
        "data": "synthetic (seeded Philox inputs of the recipe's shapes and distributions)",
        "config": {"workload": f"MoE layer recipe {cfg.cid} ({cfg.name}): T={T}, D={D}, E={E} "
                               f"routed + {1 if Is else 0} shared, top-{k} {cfg.route}, I={I}, "
                               f"I_shared={Is}, weights {cfg.wdtype}"
                               + ("" if args.glu == "swiglu" else f", {args.glu} activation")
                               + (", MXFP8 activations (FP4 x FP8)" if args.w4a8 else ""),
                   "T": T, "D": D, "E": E, "k": k, "I": I, "I_shared": Is,
                   "routing": cfg.route, "weights": cfg.wdtype, "activation": args.glu,
                   "activation_format": "mxfp8" if args.w4a8 else cfg.act,
                   "parallelism": "single GPU",
                   "weight_replicas": nrep, "experts_touched": U,
                   "max_rows_per_expert": int(counts.max())},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "tail": tail,
        "w4a8": w4a8,
        "layer": {"alg_bytes": int(layer_bytes), "flops": int(layer_flops),
                  "gbs": round(layer_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                  "hbm_frac": round(layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "tflops": round(layer_flops / (ms_per_step * 1e-3) / 1e12, 2),
                  "stage_ms": {n: round(float(v), 5) for n, v in zip(moe.STAGES, stage_avg)},
                  "kernel_ms": {"gate_up_gemm": round(float(kern_ms[0]), 5),
                                "down_gemm": round(float(kern_ms[1]), 5)},
                  "gpu_event_ms_per_step": round(gpu_ms / K, 5)},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
