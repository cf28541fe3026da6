"""Benchmark of the fused attention library on one MI355X.

One "step" is one call of the library's entry point over the workload's
synthetic inputs, which are resident in HBM before timing starts (the
attention kernel, plus the combine pass when the call splits its keys).  The
headline workload is the chunked prefill of 1024 queries over a 32768-key
prefix (B1 Hq16 Hkv8 D256 fp16, causal, bottom-right aligned).  Prints ONE
JSON line.

Measurement protocol (after the null-arm method of lablup/mlxcel issue #2160,
Acceptance Criteria): every workload ("arm") is drawn and uploaded once; then
after one untimed round over every arm, the arms are timed in turn, round
after round (at least 3 rounds, every other one in the reverse order), each
time with HIP events around each of `steps` calls on the stream the library
runs on.  The headline is timed twice per round (its second arm is the null arm:
the same call, so its spread is run-to-run noise).  Reported per arm: the
median and the minimum over all timed calls, and each round's median.  A few
paired comparisons (4-bit against 16-bit decode, the additive mask against
none, the cache view against plain decode) report their median per-round
ratio and are labelled "unresolved" when it lies inside the null arm's spread.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--rounds R] [--workload NAME]
                  [--extra | --no-extra] [--no-cpu-baseline] [--no-memory]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
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
         "causal_d128_16k", "causal_d192_16k", "causal_dk192_dv256_16k", "chunked_prefill_32k_bias",
         "decode_q4_128k", "decode_q1_128k", "decode_q4_128k_plain", "decode_q4kv_128k", "tiny_causal"]
# paired comparisons: (arm, against)
PAIRS = [("decode_q4kv_128k", "decode_q4_128k"), ("chunked_prefill_32k_bias", "chunked_prefill_32k"),
         ("decode_q4_128k", "decode_q4_128k_plain")]
NULL = "chunked_prefill_32k#null"
# host threads of the oracle timing: the host cores this GPU's share of the box
# holds (16 per GPU), or fewer if fewer are available
CPU_SHARE = 16


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Arm:
    """One workload's inputs on the GPU and the call that runs it."""

    def __init__(self, name):
        import torch

        import flash_attention_head_amd as fa
        from flash_attention_head_amd import workloads as W

        base = name.split("#")[0]
        self.name = name
        # "_plain": the decode workload through sdpa_forward (1024-key chunks)
        # instead of a cache view
        wl_name = base[:-len("_plain")] if base.endswith("_plain") else base
        self.wl = wl = W.WORKLOADS[wl_name]
        self.plain = base.endswith("_plain")
        self.stream = torch.cuda.current_stream()
        if wl.name in W.Q4KV:
            ins = [t.cuda() for t in W.draw_q4kv(wl)]
            self.out = torch.empty_like(ins[0])
            need = fa.sdpa_workspace_bytes_kv_view(wl.B, wl.Hq, wl.Hkv, wl.qL, wl.kL, wl.kL, wl.D)
            self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
            self.entry = "sdpa_forward_q4kv"

            def call():
                fa.sdpa_q4kv(*ins, kv_len=wl.kL, scale=wl.scale, causal=wl.causal, window=wl.window,
                             q_offset=wl.q_offset, out=self.out, workspace=self.ws, stream=self.stream)
        else:
            q, k, v = (t.cuda() for t in W.draw(wl))
            bias = W.draw_bias(wl)
            bias = bias.cuda() if bias is not None else None
            self.out = torch.empty(tuple(q.shape[:3]) + (wl.dv,), dtype=q.dtype, device=q.device)
            # decode / verify steps (qL <= 4) run as in a generation loop: over a
            # KV cache, here a full one of kL rows per head
            cache = wl.qL <= 4 and not self.plain
            if cache:
                need = fa.sdpa_workspace_bytes_kv_view(wl.B, wl.Hq, wl.Hkv, wl.qL, wl.kL, wl.kL, wl.D)
            else:
                need = fa.sdpa_workspace_bytes_dv(wl.B, wl.Hq, wl.Hkv, wl.qL, wl.kL, wl.D, wl.dv)
            self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
            self.entry = ("sdpa_forward_kv_view" if cache else "sdpa_forward_bias" if bias is not None else
                          "sdpa_forward_dv" if wl.dv != wl.D else "sdpa_forward")

            def call():
                if cache:
                    fa.sdpa_kv_cache(q, k, v, wl.kL, scale=wl.scale, causal=wl.causal, window=wl.window,
                                     q_offset=wl.q_offset, out=self.out, workspace=self.ws, stream=self.stream)
                else:
                    fa.sdpa(q, k, v, scale=wl.scale, causal=wl.causal, window=wl.window, q_offset=wl.q_offset,
                            bias=bias, out=self.out, workspace=self.ws, stream=self.stream)
        self.workspace_bytes = need
        self.call = call
        self.rounds = []       # per round: sorted event ms of its calls
        self.wall = []         # per round: wall ms per call

    def release(self):
        """Drop the device buffers (the timings stay)."""
        self.call = None
        self.out = self.ws = None

    def time(self, steps, warmup):
        import torch

        for _ in range(warmup):
            self.call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t0 = time.perf_counter()
        for a, b in ev:
            a.record(self.stream)
            self.call()
            b.record(self.stream)
        torch.cuda.synchronize()
        self.wall.append((time.perf_counter() - t0) * 1e3 / steps)
        self.rounds.append(sorted(a.elapsed_time(b) for a, b in ev))

    def summary(self):
        from flash_attention_head_amd import workloads as W

        wl = self.wl
        every = sorted(x for r in self.rounds for x in r)
        med, mn = statistics.median(every), every[0]
        fl = W.flops(wl)
        io = (W.q4kv_bytes(wl) if wl.name in W.Q4KV else
              W.io_bytes(wl.B, wl.Hq, wl.Hkv, wl.qL, wl.kL, wl.D, Dv=wl.dv)["total"])
        return {"ms_median": round(med, 4), "ms_min": round(mn, 4),
                "round_medians": [round(statistics.median(r), 4) for r in self.rounds],
                "calls": len(every),
                "tflops": round(fl / (med * 1e-3) / 1e12, 2),
                "mfma_frac": round(fl / (med * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
                "hbm_gbs": round(io / (med * 1e-3) / 1e9, 1),
                "hbm_frac": round(io / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "entry": self.entry, "workspace_bytes": self.workspace_bytes}


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
    csrc = os.path.join(ROOT, "flash_attention_head_amd", "csrc")
    for f in sorted(os.listdir(csrc)):  # every kernel and host source
        with open(os.path.join(csrc, f), "rb") as fh:
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


def memory_sweep():
    """Peak device memory of one call against inputs, in the layout of the mlx PR #3660
    Microbenchmarks table: 16 query / 8 KV heads at head dim 256 (fp16, causal) over qL
    {1024, 2048} x kL; and the 64-head causal layer (bf16) over L 2K..16K."""
    import torch

    import flash_attention_head_amd as fa

    MiB = 1 << 20
    rows = []
    shapes = [("16/8 heads D256 f16", 16, 8, qL, kL, torch.float16)
              for qL, kL in [(1024, 8192), (1024, 16384), (1024, 32768), (1024, 65536), (1024, 131072),
                             (2048, 65536), (2048, 131072)]]
    shapes += [("64/64 heads D256 bf16", 64, 64, L, L, torch.bfloat16) for L in (2048, 4096, 8192, 16384)]
    for what, Hq, Hkv, qL, kL, dt in shapes:
        g = torch.Generator(device="cuda")
        g.manual_seed(1)
        q = torch.randn((1, Hq, qL, 256), device="cuda", dtype=dt, generator=g)
        k = torch.randn((1, Hkv, kL, 256), device="cuda", dtype=dt, generator=g)
        v = torch.randn((1, Hkv, kL, 256), device="cuda", dtype=dt, generator=g)
        inputs = sum(t.numel() * t.element_size() for t in (q, k, v))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        out = fa.sdpa(q, k, v, causal=True)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated()
        ws = fa.sdpa_workspace_bytes(1, Hq, Hkv, qL, kL, 256)
        rows.append({"heads": what, "qL": qL, "kL": kL, "inputs_mib": round(inputs / MiB, 1),
                     "peak_mib": round(peak / MiB, 1), "peak_minus_inputs_mib": round((peak - inputs) / MiB, 1),
                     "output_mib": round(out.numel() * out.element_size() / MiB, 1),
                     "workspace_mib": round(ws / MiB, 1)})
        del q, k, v, out
        torch.cuda.empty_cache()
    return rows


def oracle_rate(wl, seconds, threads, draw=None):
    """The fp64 oracle on a bounded seeded sample of a workload's rows (all rows when they
    fit the time): GFLOP/s on the algorithmic FLOP of the rows run, and the time the whole
    call would take at that rate."""
    import numpy as np

    import oracle
    from flash_attention_head_amd import workloads as W

    q, k, v = draw if draw is not None else W.draw(wl)
    qb, kb, vb = W.bits(q), W.bits(k), W.bits(v)
    rng = np.random.default_rng(wl.seed)
    total = wl.B * wl.Hq * wl.qL
    vis = W.visible_keys(wl.qL, wl.kL, wl.causal, wl.window, wl.q_offset)

    def run(n):
        rows = np.sort(rng.choice(total, size=min(n, total), replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.sdpa_rows_f64(qb, kb, vb, rows, scale=wl.scale, causal=wl.causal, window=wl.window,
                             q_offset=wl.q_offset, dtype=wl.dtype, threads=threads)
        dt = time.perf_counter() - t0
        return rows.size, dt, 4.0 * wl.D * float(vis[rows % wl.qL].sum())

    n, dt, fl = run(min(total, 2 * threads))  # calibration
    n2 = int(max(threads, min(total, n * seconds / max(dt, 1e-3))))
    n, dt, fl = run(n2)
    rate = fl / dt
    full = n == total
    return {"rows": n, "of_rows": total, "seconds": round(dt, 2), "gflops": round(rate / 1e9, 2),
            "call_s": round(W.flops(wl) / rate, 2) if not full else round(dt, 2),
            "call_s_kind": "measured (every row)" if full else "extrapolated from the sample by FLOP",
            "threads": threads}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--extra", dest="extra", action="store_true", default=True)
    ap.add_argument("--no-extra", dest="extra", action="store_false")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-memory", action="store_true")
    ap.add_argument("--copy-reference", action="store_true",
                    help="only run a plain 1 GiB device copy three times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (got --gpus {args.gpus}); the "
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

    head = args.workload
    names = [head]
    if args.extra:
        names += [n for n in EXTRA if n != head] + [head + "#null"]
    arms = {}
    for n in names:
        log(f"[bench] prepare {n}")
        arms[n] = Arm(n)
    rounds = max(1, args.rounds)
    # one untimed round over every arm first: the clocks settle under the
    # full mix of calls before any round is timed
    log("[bench] warm-up round")
    for n in names:
        for _ in range(max(1, args.warmup)):
            arms[n].call()
    torch.cuda.synchronize()
    for r in range(rounds):
        # every other round in the reverse order: an arm's place in a round
        # moves its time (fixed-order A/B runs of one kernel read 1-3% apart)
        for n in (names if r % 2 == 0 else names[::-1]):
            steps = args.steps if n.split("#")[0] == head else max(5, args.steps // 2)
            arms[n].time(steps, 1)
        log(f"[bench] round {r + 1}: " + ", ".join(f"{n} {statistics.median(arms[n].rounds[-1]):.4f}"
                                                  for n in names))
    extra = {n: arms[n].summary() for n in names if n != head}
    ha = arms[head]
    hs = ha.summary()

    # null arm and paired comparisons: per round, the ratio of round medians
    def ratios(a, b):
        return [statistics.median(x) / statistics.median(y) - 1.0 for x, y in zip(arms[a].rounds, arms[b].rounds)]

    null_arm = comparisons = None
    if head + "#null" in arms:
        nr = ratios(head + "#null", head)
        spread = max(abs(x) for x in nr)
        null_arm = {"arm": head + "#null", "round_ratios": [round(x, 4) for x in nr], "spread": round(spread, 4)}
        comparisons = []
        for a, b in PAIRS:
            if a in arms and b in arms:
                rr = ratios(a, b)
                m = statistics.median(rr)
                comparisons.append({"arm": a, "against": b, "median_ratio_minus_1": round(m, 4),
                                    "round_ratios": [round(x, 4) for x in rr],
                                    "status": "resolved" if abs(m) > spread else "unresolved"})
        log(f"[bench] null arm {null_arm}; comparisons {comparisons}")

    read_ref = None
    if args.extra:
        log("[bench] plain streaming read (context for the decode lines)")
        read_ref = read_reference()

    mem = None
    if args.extra and not args.no_memory:
        log("[bench] peak-memory sweep (every arm's buffers freed first)")
        import gc

        for n in list(arms):
            if n != head:
                arms[n].release()
                del arms[n]
        ha.release()
        gc.collect()  # an arm's call closes over the arm: a cycle
        torch.cuda.empty_cache()
        mem = memory_sweep()

    base, oracle_rows = None, None
    if not args.no_cpu_baseline:
        import oracle

        threads = min(CPU_SHARE, oracle.default_threads())
        hw = arms[head].wl
        log(f"[bench] cpu baseline: the oracle on a sample of {hw.name} ({threads} threads)")
        r0 = oracle_rate(hw, 15.0, threads)
        base = {"value": round(r0["gflops"] / 1e3, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": f"{r0['rows']} seeded random query rows of {r0['of_rows']} ({hw.name}), all their "
                          f"visible keys, in {r0['seconds']} s on {threads} host threads; the whole call "
                          f"would take {r0['call_s']} s ({r0['call_s_kind']})"}
        if args.extra:
            oracle_rows = {}
            for n, secs in [("tiny_causal", 2.0), ("sliding_32k", 4.0), ("decode_q4_128k", 6.0),
                            ("causal_h64_16k", 4.0), ("global_d512_32k", 4.0)]:
                log(f"[bench] oracle rate on {n}")
                oracle_rows[n] = oracle_rate(W.WORKLOADS[n], secs, threads)

    # the headline line: value from the host wall clock around the timed calls
    # (median over rounds), roofline.achieved from the HIP events of the same calls
    fl = W.flops(ha.wl)
    wall_ms = statistics.median(ha.wall)
    achieved = fl / (hs["ms_median"] * 1e-3) / 1e12
    wl = ha.wl
    line = {
        "metric": "attention TFLOP/s & % MFMA peak (prefill D=256, L=32K); decode HBM GB/s",
        "value": round(fl / (wall_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W.DTYPE_NAMES[wl.dtype],
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "qL": wl.qL,
                   "kL": wl.kL, "D": wl.D, "causal": wl.causal, "window": wl.window,
                   "q_offset": wl.q_offset, "flop_per_step": fl, "rounds": rounds},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                     "traffic": measured_traffic(wl.name),
                     "traffic_unit": "bytes per call (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "kernel": "attn_tile_kernel (+ combine when keys are split), one sdpa_forward call; "
                               "median of HIP-event times on its stream over all rounds"},
        "cpu_baseline": base,
        "headline_arm": hs,
        "extra": extra,
        "null_arm": null_arm,
        "comparisons": comparisons,
        "hbm_read_reference": read_ref,
        "peak_memory": mem,
        "oracle_rates": oracle_rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
