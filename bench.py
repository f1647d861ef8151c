"""Throughput of the RoPE-aware rotated INT4 attention path on one MI355X.

One step = the whole hot path on one batch already resident in HBM:
rotattn_quantize_qk (3D RoPE + Walsh-Hadamard + per-block INT4 Q/K) ->
rotattn_quantize_v (per-channel INT4 V + column sums) -> rotattn_attention
(fused INT4 flash loop, FP16 fallback tiles and merge when routing is on).

Metric: attention TOPS = 4 B H L^2 D / step time (D the nominal head dim),
on the 720p-style workload (B=1, H=40, L=75600, D=128), and the INT4
attention kernel's credited rate as a share of the INT8 matrix-core peak
(5.0 POP/s dense), which the metric names (`int8_peak_share`). The roofline
entry prices that kernel on the unit that executes it: both of its products
run as FP6 E2M3 `v_mfma_scale_f32_32x32x64_f8f6f4` instructions (the INT4
codes are exact in E2M3), whose dense peak is derived from the device:
CUs x engine clock x 16384 ops per CU and clock (4 SIMDs, one 32x32x64
product of 131072 ops every 32 cycles each); 10.07 POP/s at 256 CUs and
2.4 GHz. `achieved` counts the operations the kernel executes, 2 (D' + D)
per score element (D' = 192 for the per-group rotation). The kernel is in fact
bound by its vector ALU (the float32 softmax of every score), which caps the
products well below that peak; `valu_busy` carries rocprof's VALUBusy of the
kernel from the committed profile of the workload. The CPU baseline is
the oracle (numpy) on a bounded sample of the same workload, over the host's
cores; the same leg reports the fidelity of the GPU output (cosine
similarity to exact float64 attention on sampled rows).

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
INT8_PEAK_TOPS = 5000.0     # MI355X dense INT8 matrix-core peak, 5.0 POP/s (published)
FP6_PEAK_PUBLISHED_TOPS = 10100.0   # MI355X dense FP6/FP4 matrix-core peak (published)
FP6_OPS_PER_CU_CLK = 4 * 32 * 32 * 64 * 2 // 32   # 4 SIMDs x one 32x32x64 FP6 product per 32 cycles
HBM_PEAK_GBS = 8000.0


def device_peak():
    """(CUs, peak engine clock in GHz, FP6 dense peak in TOPS) of device 0 from the HIP runtime."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    val = ctypes.c_int(0)
    attrs = {}
    for name, code in (("clock_khz", 5), ("cus", 63)):   # hipDeviceAttributeClockRate, ...MultiprocessorCount
        if hip.hipDeviceGetAttribute(ctypes.byref(val), code, 0) != 0:
            raise RuntimeError("hipDeviceGetAttribute failed")
        attrs[name] = val.value
    ghz = attrs["clock_khz"] / 1e6
    return attrs["cus"], ghz, attrs["cus"] * ghz * 1e9 * FP6_OPS_PER_CU_CLK / 1e12
KERNEL_SOURCES = ("int4_quantized_flashattention_amd/csrc/attn_int4.hip", "int4_quantized_flashattention_amd/csrc/common.h")


def profiled(workload: str) -> dict:
    """Per-launch figures of the INT4 attention kernel from the committed rocprofv3 summary of this workload
    (`profiles/int4_attn_kernel_<workload>.md`, its "- key: value" lines): HBM traffic from FETCH_SIZE /
    WRITE_SIZE calibrated against a plain copy, and VALUBusy. Empty when there is no summary or the kernel
    sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"int4_attn_kernel_{workload}.md")
    if not os.path.exists(path):
        return {}
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].strip().split(": ", 1)
            vals[k] = v
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if vals.get("kernel_source_sha256") != h.hexdigest():
        return {}
    return vals


def measured_traffic(workload: str):
    """HBM bytes per launch of the INT4 attention kernel (profiled), or None."""
    v = profiled(workload).get("traffic_bytes_per_launch")
    return int(v) if v is not None else None


def measured_valu_busy(workload: str):
    """rocprof's VALUBusy of the INT4 attention kernel (profiled), or None."""
    v = profiled(workload).get("valu_busy")
    return float(v) if v is not None else None


def baseline_heads(w: W.Workload):
    """Heads of the CPU baseline, one per usable host core (the affinity mask, capped by OMP_NUM_THREADS when
    that is set, e.g. to the host cores that go with one GPU), spread evenly over the workload's heads."""
    cores = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit():
        cores = min(cores, int(cap))
    cores = max(1, min(cores, w.H))
    return [int(round(i * (w.H - 1) / max(cores - 1, 1))) for i in range(cores)] if cores > 1 else [0]


def _oracle_worker(task):
    """One head of the CPU baseline: its Q/K/V prologue, then the INT4 flash loop over all keys for consecutive
    chunks of query rows until `seconds` have passed (at least one chunk). Untimed extras: exact attention of the
    worker's `fid_rows` (for the fidelity report) and the share of its Q/K blocks that tau = 0.05 would flag."""
    name, h, seconds, chunk, row0, fid_rows = task
    from threadpoolctl import threadpool_limits

    from oracle import core as O
    w = W.WORKLOADS[name]
    q, k, v = (W.head_tensor(w, 0, h, t) for t in ("q", "k", "v"))
    with threadpool_limits(1):
        t0 = time.perf_counter()
        qp = O.qk_prologue(q, w.prefix, w.grid, w.split, w.base, w.rotation)
        kp = O.qk_prologue(k, w.prefix, w.grid, w.split, w.base, w.rotation)
        vc, sv, cs = O.quantize_v(v)
        t_pro = time.perf_counter() - t0
        done = 0
        while done < w.L and (done == 0 or time.perf_counter() - t0 < seconds):
            r0 = (row0 + done) % w.L
            rows = np.arange(r0, min(r0 + chunk, w.L))
            O.int4_flash_rows(qp["codes"], qp["scale"], kp["codes"], kp["scale"], vc, sv, cs, w.L, w.D, rows)
            done += rows.size
        dt = time.perf_counter() - t0
        exact = None
        if fid_rows is not None:
            exact = O.exact_attention(q, k, v, prefix=w.prefix, grid=w.grid, split=w.split, base=w.base,
                                      rows=fid_rows)
    flagged = float(np.mean(np.concatenate([qp["nsr"], kp["nsr"]]) > 0.05))
    return {"head": h, "rows": done, "seconds": dt, "prologue_s": t_pro, "exact": exact, "tau005_share": flagged}


def cpu_baseline(w: W.Workload, seconds: float = 12.0, chunk: int = 256, fid=None):
    """The oracle (numpy, one BLAS thread per process) over the host's cores: one process per core, each on its
    own head (heads spread evenly over the workload), running that head's prologue and then its flash loop for
    chunks of query rows until `seconds` have passed. Throughput = all credited ops (4 rows L D per flash row)
    over the longest worker's time (prologue included). fid: {head: rows} of GPU output rows whose cosine
    similarity to exact attention is reported (computed outside the timed part)."""
    import multiprocessing as mp
    heads = baseline_heads(w)
    cores = len(heads)
    fid = fid or {}
    tasks = [(w.name, h, seconds, chunk, (i * 997 * 64) % w.L, fid.get(h)) for i, h in enumerate(heads)]
    ctx = mp.get_context("spawn")   # fresh interpreters: the workers never touch the GPU runtime
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        res = pool.map(_oracle_worker, tasks)
    wall = time.perf_counter() - t0
    rows = sum(r["rows"] for r in res)
    dt = max(r["seconds"] for r in res)
    ops = 4.0 * rows * w.L * w.D
    out = {"value": ops / dt / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
           "sample": f"{cores} processes, one per core, each on one head of {w.name} (heads {heads}): the head's "
                     f"Q/K/V prologue of all {w.L} tokens, then the INT4 flash loop for {chunk}-row chunks of "
                     f"queries over all {w.L} keys for about {seconds:.0f} s; {rows} query rows in all, ops "
                     f"credited for those rows only, over the longest worker's {dt:.1f} s",
           "seconds": round(dt, 2), "pool_wall_s": round(wall, 2),
           "tau005_flag_share": round(float(np.mean([r["tau005_share"] for r in res])), 5)}
    return out, {r["head"]: r["exact"] for r in res if r["exact"] is not None}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p", choices=list(W.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time bound of the oracle baseline sample (whole 256-row chunks per worker)")
    ap.add_argument("--sparse", type=float, default=None, metavar="F",
                    help="block-sparse path keeping the top round(F * NB) key blocks per 128-row query block")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (scales HBM traffic counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "rotattn runs on one GPU; multi-GPU sharding is design only "
                                   "(each GPU would take whole heads)", "n_gpus": args.gpus}))
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
    att_call = R.binding.CALL_ATTENTION if mask is None else R.binding.CALL_ATTENTION_HEAD_FALLBACK
    ws = {c: (torch.empty(max(1, R.workspace_bytes(p, c)), dtype=torch.uint8, device=dev))
          for c in (R.binding.CALL_QUANTIZE_QK, R.binding.CALL_QUANTIZE_V, att_call)}
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        R.rotattn_quantize_qk(p, q, k, out=qk, ws=ws[R.binding.CALL_QUANTIZE_QK], stream=stream)
        if ev is not None:
            ev[1].record(stream)
        R.rotattn_quantize_v(p, v, out=vq, ws=ws[R.binding.CALL_QUANTIZE_V], stream=stream)
        if ev is not None:
            ev[2].record(stream)
        R.rotattn_attention(p, qk, vq, v=v if need_rope else None, head_fallback=mask, out=out, ws=ws[att_call],
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
    credited_rate = ops / (att_ms * 1e-3) / 1e12
    # operations the kernel executes: 2 (D' + D) per score element (equal to the credited 4 D when D' = D)
    executed = 2.0 * (w.Dp + w.D) * w.B * w.H * float(w.L) ** 2
    achieved = executed / (att_ms * 1e-3) / 1e12
    cus, ghz, fp6_peak = device_peak()
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
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": round(fp6_peak, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / fp6_peak, 4), "traffic": measured_traffic(w.name),
                     "traffic_unit": "HBM bytes per launch", "kernel": "int4_attn_kernel (rotattn_attention)",
                     "avg_ms": round(att_ms, 4), "mfma_dtype": "fp6 e2m3 (v_mfma_scale_f32_32x32x64_f8f6f4)",
                     "peak_derivation": f"{cus} CUs x {ghz:.3f} GHz x {FP6_OPS_PER_CU_CLK} ops per CU-clock",
                     "peak_published": FP6_PEAK_PUBLISHED_TOPS,
                     "executed_ops_per_score": 2 * (w.Dp + w.D),
                     # the unit that binds the kernel: the per-score float32 softmax keeps the vector ALU
                     # this busy (profiled; null once the kernel sources change), which caps the matrix cores
                     "valu_busy": measured_valu_busy(w.name)},
        "int8_peak_share": round(credited_rate / INT8_PEAK_TOPS, 4),
        "credited_attention_TOPS": round(credited_rate, 3),
        "breakdown_ms": {"quantize_qk": round(float(t_qk.mean()), 4), "quantize_v": round(float(t_v.mean()), 4),
                         "attention": round(att_ms, 4),
                         "prologue_qk_GBps": round(qk_bytes / (t_qk.mean() * 1e-3) / 1e9, 1)},
        "wall_s_timed": round(wall, 3), "input_gen_s": round(t_gen, 1),
    }
    if not args.no_cpu_baseline:
        # fidelity sample: the first 64 rows of the first, middle and last query blocks of every head the CPU
        # baseline runs, read back from the last timed step's output
        NB = s.NB
        fid_rows = np.concatenate([np.arange(qb * 64, min(qb * 64 + 64, w.L)) for qb in (0, NB // 2, NB - 1)])
        heads = baseline_heads(w)
        idx = torch.from_numpy(fid_rows).to(dev)
        gpu_rows = {h: out[0, h].index_select(0, idx).float().cpu().numpy().astype(np.float64) for h in heads}
        base, exact = cpu_baseline(w, args.cpu_seconds, fid={h: fid_rows for h in heads})
        rec["cpu_baseline"] = base
        from oracle import core as O
        hs = sorted(exact)
        rec["fidelity"] = {
            "cosine_vs_exact": round(O.cosine_similarity(np.concatenate([gpu_rows[h] for h in hs]),
                                                         np.concatenate([exact[h] for h in hs])), 5),
            "per_head_min": round(min(O.cosine_similarity(gpu_rows[h], exact[h]) for h in hs), 5),
            "sample": f"GPU output of heads {hs}, rows of query blocks 0, {NB // 2}, {NB - 1} (first 64 rows "
                      f"each), against exact float64 attention (no quantization)",
            "tau005_flag_share": base.pop("tau005_flag_share"),
        }
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
    achieved = 2.0 * (w.Dp + w.D) * kept_scores / (t_att * 1e-3) / 1e12
    cus, ghz, fp6_peak = device_peak()
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
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": round(fp6_peak, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / fp6_peak, 4), "traffic": None,
                     "kernel": "int4_attn_kernel, block-sparse (rotattn_sparse_attention)", "avg_ms": round(t_att, 4),
                     "mfma_dtype": "fp6 e2m3 (v_mfma_scale_f32_32x32x64_f8f6f4)",
                     "peak_derivation": f"{cus} CUs x {ghz:.3f} GHz x {FP6_OPS_PER_CU_CLK} ops per CU-clock"},
        "int8_peak_share": round(ops / (t_att * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
        "breakdown_ms": {"quantize_qk_and_v": round(t_pro, 4), "block_mask": round(t_mask, 4),
                         "sparse_attention": round(t_att, 4)},
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
