"""Throughput of the RoPE-aware rotated INT4 attention path on one MI355X.

One step = the whole hot path on one batch already resident in HBM:
rotattn_quantize_qk (3D RoPE + Walsh-Hadamard + per-block INT4 Q/K) ->
rotattn_quantize_v (per-channel INT4 V + column sums) -> rotattn_attention
(fused INT4 flash loop, FP16 fallback tiles and merge when routing is on).

Metric: attention TOPS = 4 B H L^2 D / step time (D the nominal head dim),
on the 720p-style workload (B=1, H=40, L=75600, D=128). The roofline entry
reports the INT4 attention kernel alone against the INT8 matrix-core peak
(5.0 POP/s dense; the INT4 codes are multiplied exactly on the FP6 matrix path,
whose dense rate is twice that). The CPU baseline is the oracle (numpy) on a bounded
sample of the same workload.

With --sparse F the step is the block-sparse path instead (RainFusion2.0
sections 3.1-3.4): rotattn_quantize_qk with block sums -> rotattn_quantize_v ->
rotattn_block_mask (top round(F * NB) key blocks per 128-row query block, plus
the first-frame sink) -> rotattn_sparse_attention; `value` then counts the
executed ops (4 D per kept score element) and the line also carries the
density and the dense-equivalent rate.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 720p] [--sparse F]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402

METRIC = "attention TOPS (4·B·H·L²·D/s) and % of INT8 MFMA peak, 75600-token 40-head"
INT8_PEAK_TOPS = 5000.0     # MI355X dense INT8 matrix-core peak, 5.0 POP/s
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ("int4_quantized_flashattention_amd/csrc/attn_int4.hip", "int4_quantized_flashattention_amd/csrc/common.h")


def measured_traffic(workload: str):
    """HBM bytes per launch of the INT4 attention kernel, from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary of this workload (calibrated against a plain copy), or None when there is none or the kernel
    sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"int4_attn_kernel_{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].strip().split(": ", 1)
            vals[k] = v
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if vals.get("kernel_source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(vals["traffic_bytes_per_launch"])


def cpu_baseline(w: W.Workload, x, seconds: float = 12.0, chunk: int = 512):
    """Oracle (numpy, 1 BLAS thread) on head 0: its Q/K/V prologue, then the INT4 flash loop over all keys
    for consecutive chunks of `chunk` query rows until `seconds` of CPU time have passed (at least one chunk).
    Only the flash-loop rows are credited with ops; the prologue time is included in the denominator."""
    from threadpoolctl import threadpool_limits

    from oracle import core as O
    with threadpool_limits(1):
        t0 = time.perf_counter()
        q, k, v = x["q"][0, 0], x["k"][0, 0], x["v"][0, 0]
        qp = O.qk_prologue(q, w.prefix, w.grid, w.split, w.base, w.rotation)
        kp = O.qk_prologue(k, w.prefix, w.grid, w.split, w.base, w.rotation)
        vc, sv, cs = O.quantize_v(v)
        t_pro = time.perf_counter() - t0
        done = 0
        while done < w.L and (done == 0 or time.perf_counter() - t0 < seconds):
            rows = np.arange(done, min(done + chunk, w.L))
            O.int4_flash_rows(qp["codes"], qp["scale"], kp["codes"], kp["scale"], vc, sv, cs, w.L, w.D, rows)
            done += rows.size
        dt = time.perf_counter() - t0
    ops = 4.0 * done * w.L * w.D
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": 1, "kind": "oracle",
            "sample": f"head 0 of {w.name}: Q/K/V prologue of all {w.L} tokens ({t_pro:.1f} s) + INT4 flash loop "
                      f"for query rows 0..{done - 1} over all {w.L} keys; {dt:.1f} s in total on 1 thread, "
                      f"ops credited for those {done} rows only",
            "seconds": round(dt, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p", choices=list(W.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time bound of the oracle baseline sample (whole 512-row chunks)")
    ap.add_argument("--sparse", type=float, default=None, metavar="F",
                    help="block-sparse path keeping the top round(F * NB) key blocks per 128-row query block")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (scales HBM traffic counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU sharding is design only "
                                   "(per-head split, see DESIGN.md)", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import int4_quantized_flashattention_amd as R

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return

    w = W.WORKLOADS[args.workload]
    if args.sparse is not None:
        return sparse_main(args, w)
    t_gen = time.perf_counter()
    x = W.full_inputs(w, threads=16)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    q = torch.from_numpy(x["q"]).to(dev)
    k = torch.from_numpy(x["k"]).to(dev)
    v = torch.from_numpy(x["v"]).to(dev)
    mask_np = W.head_fallback_mask(w)
    mask = torch.from_numpy(mask_np).to(dev) if mask_np is not None else None
    p = R.problem_from_workload(w)
    need_rope = mask is not None or np.isfinite(w.tau)
    qk = R.binding.alloc_qk(p, dev, need_rope)
    vq = R.binding.alloc_v(p, dev)
    out = torch.empty((w.B, w.H, w.L, w.D), dtype=torch.float16, device=dev)
    ws = {c: (torch.empty(max(1, R.workspace_bytes(p, c)), dtype=torch.uint8, device=dev))
          for c in (R.binding.CALL_QUANTIZE_QK, R.binding.CALL_QUANTIZE_V, R.binding.CALL_ATTENTION)}
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        R.rotattn_quantize_qk(p, q, k, out=qk, ws=ws[0], stream=stream)
        if ev is not None:
            ev[1].record(stream)
        R.rotattn_quantize_v(p, v, out=vq, ws=ws[1], stream=stream)
        if ev is not None:
            ev[2].record(stream)
        R.rotattn_attention(p, qk, vq, v=v if need_rope else None, head_fallback=mask, out=out, ws=ws[2],
                            stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_qk = np.array([e[0].elapsed_time(e[1]) for e in evs])
    t_v = np.array([e[1].elapsed_time(e[2]) for e in evs])
    t_att = np.array([e[2].elapsed_time(e[3]) for e in evs])
    t_step = np.array([e[0].elapsed_time(e[3]) for e in evs])
    ms_per_step = float(t_step.mean())
    ops = w.credited_ops()
    value = ops / (ms_per_step * 1e-3) / 1e12
    att_ms = float(t_att.mean())
    achieved = ops / (att_ms * 1e-3) / 1e12
    s = R.get_sizes(p)
    # compulsory HBM bytes of the prologue: fp16 Q and K in, codes + scales + flags out
    qk_bytes = 2 * w.B * w.H * w.L * w.D * 2 + 2 * s.qk_codes_bytes + 2 * s.qk_scale_bytes + 2 * s.qk_flag_bytes
    rec = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i4", "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} L={w.L} D={w.D} grid={'x'.join(map(str, w.grid))} "
                               f"prefix={w.prefix} rotation={'group64' if w.rotation else 'full'}",
                   "global_batch": w.B, "seq_len": w.L, "heads": w.H, "head_dim": w.D, "parallelism": "none"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": measured_traffic(w.name), "traffic_unit": "HBM bytes per launch",
                     "kernel": "int4_attn_kernel (rotattn_attention)", "avg_ms": round(att_ms, 4)},
        "breakdown_ms": {"quantize_qk": round(float(t_qk.mean()), 4), "quantize_v": round(float(t_v.mean()), 4),
                         "attention": round(att_ms, 4),
                         "prologue_qk_GBps": round(qk_bytes / (t_qk.mean() * 1e-3) / 1e9, 1)},
        "wall_s_timed": round(wall, 3), "input_gen_s": round(t_gen, 1),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(rec))


def sparse_main(args, w):
    """The block-sparse step (see the module docstring); one JSON line like main()'s."""
    import torch

    import int4_quantized_flashattention_amd as R
    if np.isfinite(w.tau) or W.head_fallback_mask(w) is not None:
        print(json.dumps({"error": f"workload {w.name} routes blocks to FP16; the block-sparse path has no FP16 "
                                   "fallback"}))
        sys.exit(2)
    x = W.full_inputs(w, threads=16)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[t]).to(dev) for t in ("q", "k", "v"))
    p = R.problem_from_workload(w)
    s = R.get_sizes(p)
    topn = max(1, int(round(args.sparse * s.NB)))
    qk = R.binding.alloc_qk(p, dev, False, block_sums=True)
    vq = R.binding.alloc_v(p, dev)
    mask = torch.empty((w.B, w.H, s.mask_rows, s.mask_words), dtype=torch.int32, device=dev)
    out = torch.empty((w.B, w.H, w.L, w.D), dtype=torch.float16, device=dev)
    ws = {c: torch.empty(max(1, R.workspace_bytes(p, c)), dtype=torch.uint8, device=dev)
          for c in (R.binding.CALL_QUANTIZE_QK, R.binding.CALL_QUANTIZE_V, R.binding.CALL_SPARSE_ATTENTION)}
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        R.rotattn_quantize_qk(p, q, k, out=qk, ws=ws[R.binding.CALL_QUANTIZE_QK], stream=stream)
        R.rotattn_quantize_v(p, v, out=vq, ws=ws[R.binding.CALL_QUANTIZE_V], stream=stream)
        if ev is not None:
            ev[1].record(stream)
        R.rotattn_block_mask(p, qk, topn, out=mask, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        R.rotattn_sparse_attention(p, qk, vq, mask, out=out, ws=ws[R.binding.CALL_SPARSE_ATTENTION], stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_pro = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    t_mask = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    t_att = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    ms_per_step = float(np.mean([e[0].elapsed_time(e[3]) for e in evs]))
    bits = R.mask_to_bool(mask.cpu().numpy().astype(np.uint32), s.NB)   # [B, H, rows, NB]
    rows = np.minimum(128, w.L - 128 * np.arange(s.mask_rows))
    keys = np.minimum(64, w.L - 64 * np.arange(s.NB))
    kept_scores = float(np.einsum("bhij,i,j->", bits.astype(np.float64), rows.astype(np.float64),
                                  keys.astype(np.float64)))
    density = kept_scores / (w.B * w.H * float(w.L) * w.L)
    ops = 4.0 * kept_scores * w.D
    achieved = ops / (t_att * 1e-3) / 1e12
    rec = {
        "metric": "block-sparse attention TOPS executed (4 D per kept score element) and % of INT8 MFMA peak",
        "value": round(ops / (ms_per_step * 1e-3) / 1e12, 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i4", "data": "synthetic",
        "config": {"workload": f"{w.name} block-sparse: B={w.B} H={w.H} L={w.L} D={w.D} "
                               f"grid={'x'.join(map(str, w.grid))} topn={topn} of NB={s.NB}",
                   "global_batch": w.B, "seq_len": w.L, "heads": w.H, "head_dim": w.D, "parallelism": "none"},
        "density": round(density, 4),
        "dense_equivalent_TOPS": round(w.credited_ops() / (ms_per_step * 1e-3) / 1e12, 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": None,
                     "kernel": "int4_attn_kernel, block-sparse (rotattn_sparse_attention)", "avg_ms": round(t_att, 4)},
        "breakdown_ms": {"quantize_qk_and_v": round(t_pro, 4), "block_mask": round(t_mask, 4),
                         "sparse_attention": round(t_att, 4)},
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
