"""Benchmark of the fused attention library on one MI355X.

One "step" is one sdpa_forward call over the workload's synthetic inputs, which
are resident in HBM before timing starts (attention kernel, plus the combine
pass when the call splits its keys).  The headline workload is the chunked
prefill of 1024 queries over a 32768-key prefix (B1 Hq16 Hkv8 D256 fp16,
causal, bottom-right aligned).  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--extra | --no-extra] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks: dense fp16/bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
# and HBM3E bandwidth
PEAK_MFMA_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
HEADLINE = "chunked_prefill_32k"
EXTRA = ["causal_h64_16k", "sliding_32k", "global_d512_32k", "causal_d64_16k", "causal_d80_16k",
         "causal_d128_16k", "causal_d192_16k",
         "causal_dk192_dv256_16k", "chunked_prefill_32k_bias", "decode_q4_128k", "decode_q1_128k", "decode_q4kv_128k", "tiny_causal"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_workload(wl, steps, warmup):
    """Mean ms per call, measured with HIP events on the stream the library runs on."""
    import torch

    import flash_attention_head_amd as fa
    from flash_attention_head_amd import workloads as W

    if wl.name in W.Q4KV:
        return time_q4kv(wl, steps, warmup)
    q, k, v = (t.cuda() for t in W.draw(wl))
    bias = W.draw_bias(wl)
    bias = bias.cuda() if bias is not None else None
    out = torch.empty(tuple(q.shape[:3]) + (wl.dv,), dtype=q.dtype, device=q.device)
    # decode / verify steps (qL <= 4) run as they do in a generation loop:
    # over a KV cache, here a full one of kL rows per head
    cache = wl.qL <= 4
    if cache:
        need = fa.sdpa_workspace_bytes_kv_view(wl.B, wl.Hq, wl.Hkv, wl.qL, wl.kL, wl.kL, wl.D)
    else:
        need = fa.sdpa_workspace_bytes_dv(wl.B, wl.Hq, wl.Hkv, wl.qL, wl.kL, wl.D, wl.dv)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        if cache:
            fa.sdpa_kv_cache(q, k, v, wl.kL, scale=wl.scale, causal=wl.causal, window=wl.window,
                             q_offset=wl.q_offset, out=out, workspace=ws, stream=stream)
        else:
            fa.sdpa(q, k, v, scale=wl.scale, causal=wl.causal, window=wl.window,
                    q_offset=wl.q_offset, bias=bias, out=out, workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per = sorted(a.elapsed_time(b) for a, b in ev)
    mean = sum(per) / len(per)
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return {"wall_ms": wall_ms, "event_ms_mean": mean, "event_ms_min": per[0],
            "event_ms_median": per[len(per) // 2], "workspace_bytes": need,
            "entry": "sdpa_forward_kv_view" if cache else ("sdpa_forward_bias" if bias is not None else
                                                           "sdpa_forward_dv" if wl.dv != wl.D else "sdpa_forward")}


def time_q4kv(wl, steps, warmup):
    """Mean ms per sdpa_forward_q4kv call over 4-bit K/V (HIP events on its stream)."""
    import torch

    import flash_attention_head_amd as fa
    from flash_attention_head_amd import workloads as W

    ins = [t.cuda() for t in W.draw_q4kv(wl)]
    out = torch.empty_like(ins[0])
    # a full 4-bit cache of kL rows
    need = fa.sdpa_workspace_bytes_kv_view(wl.B, wl.Hq, wl.Hkv, wl.qL, wl.kL, wl.kL, wl.D)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        fa.sdpa_q4kv(*ins, kv_len=wl.kL, scale=wl.scale, causal=wl.causal, window=wl.window, q_offset=wl.q_offset,
                     out=out, workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per = sorted(a.elapsed_time(b) for a, b in ev)
    del ins, out, ws
    torch.cuda.empty_cache()
    return {"wall_ms": wall_ms, "event_ms_mean": sum(per) / len(per), "event_ms_min": per[0],
            "event_ms_median": per[len(per) // 2], "workspace_bytes": need, "entry": "sdpa_forward_q4kv"}


def summarize(wl, t):
    from flash_attention_head_amd import workloads as W

    fl = W.flops(wl)
    io = (W.q4kv_bytes(wl) if wl.name in W.Q4KV else
          W.io_bytes(wl.B, wl.Hq, wl.Hkv, wl.qL, wl.kL, wl.D, Dv=wl.dv)["total"])
    ms = t["event_ms_mean"]
    r = {"ms": round(ms, 4), "ms_min": round(t["event_ms_min"], 4),
         "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
         "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
         "hbm_gbs": round(io / (ms * 1e-3) / 1e9, 1),
         "hbm_frac": round(io / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "entry": t["entry"]}
    return r


def measured_traffic(wl_name):
    """HBM bytes per call from the committed counter summary, if the kernels are unchanged.

    profiles/hbm_traffic_<workload>.md records FETCH_SIZE + WRITE_SIZE per call (scaled by a
    plain copy's reading) and a hash of the kernel sources they were taken with; a different
    hash means the counters describe older kernels, and traffic is reported as null.
    """
    import hashlib

    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{wl_name}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", " ")):
            k, _, v = line.partition(":")
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("attn_kernels.hip", "sdpa_api.cpp", "sdpa_internal.h"):
        with open(os.path.join(ROOT, "flash_attention_head_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256") != h.hexdigest():
        return None
    try:
        return int(fields["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def read_reference(nbytes=1 << 30, steps=10):
    """Plain streaming kernels over nbytes, the context for the decode lines' HBM rate (the
    same bytes as their K and V): torch's sum over the buffer as bf16 and as fp32 (reads
    only), and a device-to-device copy of it (its read and written bytes both counted)."""
    import torch

    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)

    def rate(fn, moved):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        gbs = moved / (ms * 1e-3) / 1e9
        return {"gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4), "ms": round(ms, 4)}

    out = {"sum_bf16": rate(lambda: x.sum(), nbytes),
           "sum_fp32": rate(lambda: x.view(torch.float32).sum(), nbytes),
           "copy": rate(lambda: y.copy_(x), 2 * nbytes),
           "bytes": nbytes}
    del x, y
    torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, target_s=15.0):
    """The fp64 oracle on a bounded, seeded sample of the workload's rows."""
    import numpy as np

    import oracle
    from flash_attention_head_amd import workloads as W

    q, k, v = W.draw(wl)
    qb, kb, vb = W.bits(q), W.bits(k), W.bits(v)
    threads = min(16, oracle.default_threads())
    rng = np.random.default_rng(wl.seed)
    total = wl.B * wl.Hq * wl.qL
    vis = W.visible_keys(wl.qL, wl.kL, wl.causal, wl.window, wl.q_offset)

    def run(n):
        rows = np.sort(rng.choice(total, size=min(n, total), replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.sdpa_rows_f64(qb, kb, vb, rows, scale=wl.scale, causal=wl.causal,
                             window=wl.window, q_offset=wl.q_offset, dtype=wl.dtype,
                             threads=threads)
        dt = time.perf_counter() - t0
        fl = 4.0 * wl.D * float(vis[rows % wl.qL].sum())
        return rows.size, dt, fl

    n, dt, fl = run(4 * threads)  # calibration
    n2 = int(max(threads, min(total, n * target_s / max(dt, 1e-3))))
    n, dt, fl = run(n2)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} seeded random query rows of {total} ({wl.name}), all their visible "
                      f"keys, {fl / 1e9:.1f} GFLOP in {dt:.1f} s on {threads} host threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--extra", dest="extra", action="store_true", default=True)
    ap.add_argument("--no-extra", dest="extra", action="store_false")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-reference", action="store_true",
                    help="only run a plain 1 GiB device copy three times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (got --gpus {args.gpus}); the "
              "attention path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch

    import flash_attention_head_amd as fa
    from flash_attention_head_amd import workloads as W

    if not os.path.exists(fa.library_path()):
        from flash_attention_head_amd import build

        build.build()
    fa.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_reference:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_reference_bytes": 1 << 30, "dispatches": 3}), flush=True)
        return

    wl = W.WORKLOADS[args.workload]
    log(f"[bench] {wl.name}: warmup {args.warmup}, steps {args.steps}")
    t = time_workload(wl, args.steps, args.warmup)
    head = summarize(wl, t)
    log(f"[bench] {wl.name}: {head}")
    fl = W.flops(wl)

    extra = {}
    if args.extra:
        for name in EXTRA:
            if name == wl.name:
                continue
            w2 = W.WORKLOADS[name]
            log(f"[bench] extra {name}")
            t2 = time_workload(w2, max(5, args.steps // 2), 2)
            extra[name] = summarize(w2, t2)
            log(f"[bench] {name}: {extra[name]}")

    # null arm: the headline workload timed again after everything else, so
    # the line carries its own run-to-run spread
    null_arm = None
    if args.extra:
        log(f"[bench] {wl.name} again (null arm)")
        t_again = time_workload(wl, args.steps, args.warmup)
        null_arm = {"first_ms": round(t["event_ms_mean"], 4), "repeat_ms": round(t_again["event_ms_mean"], 4),
                    "rel_diff": round(t_again["event_ms_mean"] / t["event_ms_mean"] - 1.0, 4)}
        log(f"[bench] null arm: {null_arm}")

    read_ref = None
    if args.extra:
        log("[bench] plain streaming read (context for the decode lines)")
        read_ref = read_reference()
        log(f"[bench] read reference: {read_ref}")

    base = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a row sample)")
        base = cpu_baseline(wl)
        log(f"[bench] cpu baseline: {base}")

    achieved = fl / (t["event_ms_mean"] * 1e-3) / 1e12
    line = {
        "metric": "attention TFLOP/s & % MFMA peak (prefill D=256, L=32K); decode HBM GB/s",
        "value": round(fl / (t["wall_ms"] * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W.DTYPE_NAMES[wl.dtype],
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "qL": wl.qL,
                   "kL": wl.kL, "D": wl.D, "causal": wl.causal, "window": wl.window,
                   "q_offset": wl.q_offset, "flop_per_step": fl},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                     "traffic": measured_traffic(wl.name),
                     "traffic_unit": "bytes per call (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "kernel": "attn_tile_kernel (+ combine_kernel when keys are split), one "
                               "sdpa_forward call, HIP events on its stream"},
        "cpu_baseline": base,
        "extra": extra,
        "hbm_read_reference": read_ref,
        "null_arm": null_arm,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
