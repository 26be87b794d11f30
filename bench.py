"""Benchmark of the DiT hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--images I] [--no-cpu]

Prints ONE JSON line on stdout (progress goes to stderr):
  value      block-forward TFLOP/s at the 1024-px block (L=512 text + N=4096
             image rows, hidden 3072, 24 heads x 128, SwiGLU ffn 12288, bf16
             weights), algorithmic FLOPs (2*M*N*K per product, 4*H*S^2*d for
             attention, the modulation GEMV) over the measured time of K
             consecutive dit_block_forward calls (inputs resident in HBM);
  images_per_s  the whole path for one image: positions and rotary tables,
             the text-row prologue, the schedule's modulation planned
             (dit_plan_schedule: each modulation weight read once for the
             4 steps) and 4 Euler steps of a 32-block DiT (random-init bf16
             weights), timed over I images; `unplanned` the same without
             the plan (each step computes its own modulation);
  roofline   the dominant kernel's algorithmic TFLOP/s from HIP events around
             its launches, against the bf16 dense MFMA peak;
  per_step_ms   p50 / min / max of single block forwards (HIP events per call);
  hbm_kernels   the HBM-bound kernels' algorithmic bytes per launch over their
             launch time (stage timers), against 8 TB/s;
  calibration   secondary denominators measured on this machine: a chained large
             bf16 GEMM rate (20 chained 8192^3 products, the vendor library)
             and a 1 GiB device copy's bandwidth;
  cpu_baseline  the CPU oracle timed on this host on a bounded sample;
  power      the socket power and graphics clocks amd-smi reports while the
             block runs in a loop for --power-seconds (read-only queries from
             a child process; null if amd-smi is absent).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_INT8_TOPS = 5033.2        # dense INT8 matrix cores, twice the bf16 rate
PEAK_HBM_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--images", type=int, default=2)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-denoise", action="store_true", help="skip the 32-block image timing")
    p.add_argument("--no-int8", action="store_true", help="skip the int8-weight block timing")
    p.add_argument("--no-parallel", action="store_true", help="skip the parallel-block timing")
    p.add_argument("--no-double", action="store_true", help="skip the double-stream block timing")
    p.add_argument("--no-runs", action="store_true", help="skip the timing of the block with modulation runs")
    p.add_argument("--no-sandwich", action="store_true", help="skip the sandwich block timing")
    p.add_argument("--no-cached", action="store_true", help="skip the timing of the step with cached reference rows")
    p.add_argument("--no-w8a8", action="store_true", help="skip the W8A8 block timing")
    p.add_argument("--no-unfused", action="store_true", help="skip the unfused q/k/v prep arm's timing")
    p.add_argument("--no-calibration", action="store_true", help="skip the GEMM and copy calibration")
    p.add_argument("--power-seconds", type=float, default=5.0,
                   help="seconds of block loop under amd-smi power and clock sampling (0: skip)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run one 1 GiB device-to-device copy (a kernel of known traffic, the "
                        "scale reference for FETCH_SIZE / WRITE_SIZE counter runs)")
    p.add_argument("--traffic-json", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "profiles", "traffic.json"),
                   help="measured HBM bytes per launch of the dominant kernel (from counter runs)")
    p.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                   help="no GPU work: turn the counter_collection.csv files of a FETCH_SIZE run and a "
                        "WRITE_SIZE run (both with --copy-calibration), and optionally of a run of the MFMA "
                        "counters, into --traffic-json")
    return p.parse_args()


def stage_flops(S, D, H, F):
    """Algorithmic FLOPs of each block stage at S rows."""
    return {
        "mod": 2 * 6 * D * D,
        "qkv": 2 * S * D * 3 * D,
        "attn": 4 * H * S * S * 128,
        "out": 2 * S * D * D,
        "up": 2 * S * D * 2 * F,
        "down": 2 * S * F * D,
    }


STAGE_SOURCE = {"qkv": "k_gemm.hip", "out": "k_gemm.hip", "up": "k_gemm.hip", "down": "k_gemm.hip",
                "attn": "k_attn.hip", "mod": "k_misc.hip", "par_in": "k_gemm.hip", "par_out": "k_gemm.hip",
                "norm": "k_misc.hip", "qk_prep": "k_misc.hip", "euler": "k_misc.hip", "quant": "k_misc.hip",
                "post": "k_misc.hip"}


def stage_bytes(S, D, H, F):
    """Compulsory HBM bytes per launch of the block's stages at S rows (bf16
    operands, fp32 residual): every operand read once, every result written
    once, no re-reads."""
    return {
        "mod": 6 * D * D * 2,                                   # W_mod
        "norm1": S * D * 4 + S * D * 2,                         # x in, h out
        "norm2": S * D * 4 + S * D * 2,
        "qkv": S * D * 2 + 3 * D * D * 2 + 3 * S * D * 2,       # h, W_qkv, q k v out
        "attn": 3 * S * D * 2 + S * D * 2,                      # q k v in, o out
        "out": S * D * 2 + D * D * 2 + 2 * S * D * 4,           # o, W_out, x read + write
        "up": S * D * 2 + 2 * F * D * 2 + S * F * 2,            # h2, W_up, a out
        "down": S * F * 2 + F * D * 2 + 2 * S * D * 4,          # a, W_down, x read + write
        "qk_prep": 3 * S * D * 2 + 3 * S * D * 2,               # projection in, q k vt out
    }


def sh_blocks_bytes(block_bytes, blocks=32):
    """Compulsory bytes of one denoise step of the 32-block DiT: its blocks'
    (the small in/out products and the final layer are under 0.1 %)."""
    return blocks * block_bytes


def percentiles(ms):
    a = sorted(ms)
    return {"p50": round(a[len(a) // 2], 4), "min": round(a[0], 4), "max": round(a[-1], 4), "reps": len(a)}


def time_each(torch, fn, reps):
    """Per-call ms of fn() from a pair of HIP events around each call on the
    current stream (fn's launches go to that stream)."""
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def calibration(torch):
    """Secondary denominators (never replacing the spec peaks): the rate of 20
    chained 8192^3 bf16 products through torch.matmul (the vendor GEMM
    library), and the bandwidth of a 1 GiB device-to-device copy."""
    n = 8192
    a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    c = torch.empty_like(a)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(20):
        torch.matmul(a, b, out=c)
    e1.record(st)
    torch.cuda.synchronize()
    gemm = 20 * 2 * n ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(10):
        dst.copy_(src)
    e1.record(st)
    torch.cuda.synchronize()
    copy = 10 * 2 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"gemm_bf16_chained_tflops": round(gemm, 1), "gemm_note": "20 chained 8192^3 bf16 torch.matmul",
            "copy_gbs": round(copy, 1), "copy_note": "1 GiB device-to-device copy, read + write bytes"}


def hbm_rows(stages, counts_bytes):
    """{stage: {ms, bytes, gbs, frac}} for the HBM-bound stages present."""
    out = {}
    for k, nbytes in counts_bytes.items():
        if k in stages and stages[k] > 0:
            gbs = nbytes / (stages[k] * 1e-3) / 1e9
            out[k] = {"ms": round(stages[k], 4), "bytes": int(nbytes), "gbs": round(gbs, 1),
                      "frac": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def source_sha(name):
    import hashlib
    p = os.path.join(os.path.dirname(os.path.abspath(__file__)), "diffusion_transformer_amd", "csrc", name)
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(args, stage):
    """HBM bytes per launch of `stage`'s kernel measured by the FETCH_SIZE and
    WRITE_SIZE counter runs (scaled by a plain copy of known size), as
    recorded in profiles/traffic.json; None when absent or when the kernel's
    source has changed since the counters were taken."""
    try:
        with open(args.traffic_json) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(stage)
    if not rec or rec.get("source_sha256") != source_sha(STAGE_SOURCE[stage]):
        return None
    return rec.get("bytes_per_launch")


def summarize_counters(fetch_csv, write_csv, out_json, mfma_csv=None):
    """Per-launch HBM bytes and matrix-core use of the path's kernels from
    rocprofv3 counter runs (one counter set per run).  FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) are each scaled so that the 1 GiB
    calibration copy reads and writes exactly 1 GiB.  The optional third run
    holds SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and
    SQ_INSTS_VALU_MFMA_MOPS_BF16 / _I8.  GRBM_GUI_ACTIVE arrives summed over
    the chip's 8 XCDs: per XCD it is the dispatch's active cycles, and over
    the dispatch's duration it gives the clock the chip ran at.  The matrix
    cores' busy fraction is busy cycles / (active cycles x 1024 SIMDs); the
    counted MFMA work is MOPS x 512 FLOP (or int8 ops).  Kernels are keyed by stage: the block's
    launches come in a fixed order (GEMV, norm, QKV, attention, OUT, norm,
    UP, DOWN), which tells the OUT and DOWN launches of the shared
    gated-residual product apart; the bf16 ping-pong forms are keyed by the
    stage alone, the int8 block-32 (B32) and W8A8 (I8) forms with a suffix."""
    import csv
    import collections
    import re

    def load(path, counters):
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        names = {}
        for r in csv.DictReader(open(path)):
            c = r["Counter_Name"]
            if c not in counters:
                continue
            d = int(r["Dispatch_Id"])
            per[d][c] += float(r["Counter_Value"])
            per[d]["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            names[d] = r["Kernel_Name"]
        return per, names

    def stages_of(names):
        stage_of, pending, after_dq = {}, None, False
        for d in sorted(d for d in names if "dit::" in names[d]):
            n = names[d]
            pp = re.search(r"k_gemm_p3<(\d), (true|false), (true|false), (true|false)>", n)
            rg = re.search(r"k_gemm<\d+, \d+, (?:true|false), (\d)>", n)
            epi = int(pp.group(1)) if pp else int(rg.group(1)) if rg else None
            suffix = ""
            if pp and pp.group(3) == "true":
                suffix = "_w8a8"
            elif pp and pp.group(4) == "true":
                suffix = "_b32"
            st = None
            if pp and pp.group(2) == "true":
                st = "par_out"                   # parallel block: [OUT | DOWN] over [o | a]
            elif epi == 4:
                st = "par_in"                    # parallel block: [QKV | UP]
            elif epi == 3:
                st = "qkv"
            elif epi == 2:
                st = "up"
            elif epi == 1:
                st = "down" if pending == "up" else "out"
            elif "k_attention" in n:
                st = "attn"
            elif "k_gemv" in n:
                st = "mod"
            elif "k_modnorm" in n:
                st = "norm"
            elif "k_qk_prep" in n:
                st = "qk_prep"
            elif "k_euler" in n:
                st = "euler"
            elif "k_quant_rows" in n:
                st = "quant"
            elif "k_post_norm_gate" in n:
                st = "post"
            elif "k_dequant_bf16" in n:
                st = "dequant"
            if st is None:
                continue
            if st == "dequant":        # the bf16 product after it runs on dequantised int8 weights
                after_dq = True
            elif st != "quant":        # a W8A8 block quantizes o and a between its products
                pending = st
            if pp or rg:
                if after_dq and pp:
                    suffix = "_dq"
                after_dq = False
                st = st + (suffix if pp else "_regstaged")
            stage_of[d] = st
        return stage_of

    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per, names = load(path, {counter})
        copy_kib = sum(v[counter] for d, v in per.items() if "copyBuffer" in names[d])
        scale = (1 << 30) / 1024.0 / copy_kib if copy_kib else None
        acc = collections.defaultdict(list)
        for d, st in stages_of(names).items():
            acc[st].append(per[d][counter])
        for st, v in acc.items():
            rec = res.setdefault(st, {})
            rec[counter.lower() + "_kib_mean"] = sum(v) / len(v)
            rec[counter.lower() + "_scale"] = scale
            rec["launches"] = len(v)
    if mfma_csv:
        cs = {"SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_I8"}
        per, names = load(mfma_csv, cs)
        acc = collections.defaultdict(list)
        for d, st in stages_of(names).items():
            acc[st].append(per[d])
        for st, v in acc.items():
            rec = res.setdefault(st, {})
            xcd = 8
            busy = [x["SQ_VALU_MFMA_BUSY_CYCLES"] / (x["GRBM_GUI_ACTIVE"] / xcd * 1024) for x in v if x["GRBM_GUI_ACTIVE"]]
            ghz = [x["GRBM_GUI_ACTIVE"] / xcd / x["ns"] for x in v if x["ns"] > 0]
            rec["mfma_busy_frac"] = round(sum(busy) / len(busy), 4) if busy else None
            rec["clock_ghz"] = round(sum(ghz) / len(ghz), 3) if ghz else None
            rec["mfma_bf16_flop_mean"] = sum(x["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for x in v) / len(v) * 512
            rec["mfma_i8_op_mean"] = sum(x["SQ_INSTS_VALU_MFMA_MOPS_I8"] for x in v) / len(v) * 512
            rec["mfma_launches"] = len(v)
    for st, rec in res.items():
        if rec.get("fetch_size_scale") and rec.get("write_size_scale"):
            rec["bytes_per_launch"] = int(1024 * (rec["fetch_size_kib_mean"] * rec["fetch_size_scale"]
                                                  + rec["write_size_kib_mean"] * rec["write_size_scale"]))
        base = st.split("_")[0] if st.split("_")[0] in STAGE_SOURCE else st
        src = STAGE_SOURCE.get(base) or STAGE_SOURCE.get(st) or ("k_gemm.hip" if "regstaged" in st else "k_misc.hip")
        rec["source_sha256"] = source_sha(src)
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    print(json.dumps(res, indent=1, sort_keys=True))


def sample_power(torch, run, seconds):
    """Runs `run` (a batch of block forwards) back to back for `seconds` while
    a thread queries amd-smi (socket power, graphics clock of each XCD) about
    twice a second from a child process.  Returns the means and extremes of
    the samples taken after the first second, or an error note."""
    import shutil
    import subprocess
    import threading
    exe = shutil.which("amd-smi")
    if exe is None:
        return {"error": "amd-smi not found"}
    samples, errors = [], []
    stop = threading.Event()
    t_start = time.time()

    def poll():
        while not stop.is_set():
            try:
                r = subprocess.run([exe, "metric", "-p", "-c", "--json"], capture_output=True, text=True, timeout=10)
                d = json.loads(r.stdout)["gpu_data"][0]
                clk = [v["clk"]["value"] for k, v in d["clock"].items()
                       if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
                if time.time() - t_start > 1.0 and clk:
                    samples.append((float(d["power"]["socket_power"]["value"]), sum(clk) / len(clk),
                                    min(clk), max(clk)))
            except Exception as e:   # noqa: BLE001 -- a missing field or a failed query
                errors.append(str(e)[:120])
            stop.wait(0.4)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    n, t0 = 0, time.time()
    while time.time() - t0 < seconds:
        n += run()
        torch.cuda.synchronize()
    dt = time.time() - t0
    stop.set()
    th.join(timeout=15)
    if not samples:
        return {"error": "no amd-smi samples" + (f": {errors[0]}" if errors else "")}
    w = [a[0] for a in samples]
    return {"samples": len(samples), "seconds": round(dt, 2), "ms_per_block": round(1e3 * dt / n, 4),
            "socket_w_mean": round(sum(w) / len(w), 1), "socket_w_max": max(w),
            "gfx_mhz_mean": round(sum(a[1] for a in samples) / len(samples), 1),
            "gfx_mhz_min": min(a[2] for a in samples), "gfx_mhz_max": max(a[3] for a in samples),
            "tool": "amd-smi metric -p -c --json"}


def time_blocks(L, torch, ctx, bw, x, seq, sh, steps, warmup, parallel=False):
    fwd = ctx.parallel_block_forward if parallel else ctx.block_forward
    for _ in range(warmup):
        fwd(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        fwd(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_call(torch, fn, steps, warmup):
    """Average ms of fn() over steps calls on the current stream, after warmup calls."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def stage_split(ctx, fn, steps):
    """Per-stage ms per call from the library's stage timers over steps calls."""
    ctx.timing(True)
    for _ in range(steps):
        fn()
    t = ctx.timing_read()
    ctx.timing(False)
    return {k: round(v[0] / steps, 4) for k, v in t.items() if v[1]}


def main():
    args = parse()
    if args.summarize_counters:
        c = args.summarize_counters
        summarize_counters(c[0], c[1], args.traffic_json, c[2] if len(c) > 2 else None)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the path is sized for one "
              "GPU's share and no multi-GPU run is made.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from diffusion_transformer_amd import lib as L
    from diffusion_transformer_amd import synth

    torch.cuda.set_device(0)
    out = {}
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: one 1 GiB device-to-device copy")
        del src, dst

    # ---------------------------------------------------------------- block forward (bf16)
    sh = synth.SHAPES["s4608"]
    S, D, H, F = sh.S, sh.hidden, sh.heads, sh.ffn
    arch = L.make_arch(hidden=D, heads=H, ffn=F)
    ctx = L.Context(arch, max_rows=S)
    log("generating the 1024-px block inputs")
    case = synth.block_case("s4608")
    bw = L.BlockWeights.from_host(case["block"])

    class Seq:
        pass

    seq = Seq()
    seq.pos = torch.empty((S, 3), dtype=torch.int32, device="cuda")
    seq.cos = torch.empty((S, 64), dtype=torch.float32, device="cuda")
    seq.sin = torch.empty_like(seq.cos)
    seq.vec = torch.empty(D, dtype=torch.float32, device="cuda")
    ctx.positions(sh.L, sh.h, sh.w, seq.pos)
    ctx.rope_tables(seq.pos, S, seq.cos, seq.sin)
    ctx.time_vector(L.dev_bf16(case["w_t1"]), L.dev_bf16(case["w_t2"]), float(case["t"]), seq.vec)
    x = L.dev_f32(case["x"])
    fl = stage_flops(S, D, H, F)
    total_flops = sum(fl.values())
    log(f"block forward: {args.warmup} warmup + {args.steps} timed steps")
    ms = time_blocks(L, torch, ctx, bw, x, seq, sh, args.steps, args.warmup)
    tflops = total_flops / (ms * 1e-3) / 1e12
    log(f"block: {ms:.3f} ms  {tflops:.1f} TFLOP/s  ({100 * tflops / PEAK_BF16_TFLOPS:.1f} % of bf16 peak)")

    # per-stage breakdown with HIP events on the library's stream
    ctx.timing(True)
    for _ in range(args.steps):
        ctx.block_forward(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    tm = ctx.timing_read()
    ctx.timing(False)
    stages = {k: v[0] / v[1] for k, v in tm.items() if v[1]}
    log("stages (ms): " + ", ".join(f"{k} {v:.3f}" for k, v in stages.items()))
    per_step = percentiles(time_each(torch, lambda: ctx.block_forward(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N),
                                     max(20, args.steps)))
    log(f"single block forwards: p50 {per_step['p50']:.3f} ms, min {per_step['min']:.3f} ms")
    power = None
    if args.power_seconds > 0:
        log(f"block loop for {args.power_seconds:.0f} s under amd-smi power and clock sampling")

        def batch():
            for _ in range(50):
                ctx.block_forward(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
            return 50
        power = sample_power(torch, batch, args.power_seconds)
        log(f"power: {power}")
    sb_bytes = stage_bytes(S, D, H, F)
    block_bytes = sum(v for k, v in sb_bytes.items() if k != "qk_prep")
    hbm = hbm_rows(stages, {k: sb_bytes[k] for k in ("mod", "norm1", "norm2")})
    dom = max((k for k in stages if k in fl), key=lambda k: stages[k])
    dom_tf = fl[dom] / (stages[dom] * 1e-3) / 1e12
    roofline = {"kernel": f"{dom} product" if dom not in ("attn", "mod") else dom, "bound": "mfma",
                "achieved": round(dom_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic_for(args, dom),
                "flops_per_launch": fl[dom], "avg_ms": round(stages[dom], 4)}
    del bw, x

    # ---------------------------------------------------------------- parallel block (bf16)
    par = None
    if not args.no_parallel:
        log("parallel block (one norm, [QKV | UP] and [OUT | DOWN] products)")
        pb = dict(case["block"])
        pb["w_mod"] = np.ascontiguousarray(pb["w_mod"][:3 * D])
        bwp = L.BlockWeights.from_host(pb)
        xp = L.dev_f32(case["x"])
        par_flops = total_flops - 2 * 3 * D * D
        msp = time_blocks(L, torch, ctx, bwp, xp, seq, sh, args.steps, args.warmup, parallel=True)
        ctx.timing(True)
        for _ in range(args.steps):
            ctx.parallel_block_forward(bwp, xp, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
        tmp = ctx.timing_read()
        ctx.timing(False)
        par_tf = par_flops / (msp * 1e-3) / 1e12
        par = {"ms": round(msp, 4), "tflops": round(par_tf, 2),
               "frac_bf16_peak": round(par_tf / PEAK_BF16_TFLOPS, 4), "flops_per_step": par_flops,
               "stages_ms": {k: round(v[0] / v[1], 4) for k, v in tmp.items() if v[1]}}
        log(f"parallel block: {msp:.3f} ms  {par_tf:.1f} TFLOP/s")
        del bwp, xp

    # ---------------------------------------------------------------- double-stream block (bf16)
    dbl = None
    if not args.no_double:
        log("double-stream block (text and image weights, joint attention)")
        other = synth.block_case("s4608", seed=sh.seed + 100)
        bwt = L.BlockWeights.from_host(other["block"])
        bwi = L.BlockWeights.from_host(case["block"])
        xd = L.dev_f32(case["x"])
        dbl_flops = total_flops + 2 * 6 * D * D          # a second modulation GEMV

        def dfwd():
            ctx.double_block_forward(bwt, bwi, xd, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
        msd = time_call(torch, dfwd, args.steps, args.warmup)
        dbl_tf = dbl_flops / (msd * 1e-3) / 1e12
        dbl = {"ms": round(msd, 4), "tflops": round(dbl_tf, 2),
               "frac_bf16_peak": round(dbl_tf / PEAK_BF16_TFLOPS, 4), "flops_per_step": dbl_flops,
               "stages_ms_per_step": stage_split(ctx, dfwd, args.steps)}
        log(f"double-stream block: {msd:.3f} ms  {dbl_tf:.1f} TFLOP/s")
        del bwt, bwi, xd, other

    # ---------------------------------------------------------------- modulation runs (bf16)
    runs_res = None
    if not args.no_runs:
        log("block with two modulation rows (text rows on one, image rows on the other)")
        bwr = L.BlockWeights.from_host(case["block"])
        xr = L.dev_f32(case["x"])
        vecs = torch.empty((2, D), dtype=torch.float32, device="cuda")
        vecs[0].copy_(seq.vec)
        vecs[1].copy_(torch.from_numpy(synth.normal((D,), seed=sh.seed + 200, std=0.13)).float())
        runs = [(0, sh.L, 1), (sh.L, S, 0)]
        runs_flops = total_flops + 2 * 6 * D * D         # a second modulation GEMV

        def rfwd():
            ctx.block_forward_runs(bwr, xr, vecs, runs, seq.cos, seq.sin, sh.L, sh.N)
        msr = time_call(torch, rfwd, args.steps, args.warmup)
        runs_tf = runs_flops / (msr * 1e-3) / 1e12
        runs_res = {"ms": round(msr, 4), "tflops": round(runs_tf, 2),
                    "frac_bf16_peak": round(runs_tf / PEAK_BF16_TFLOPS, 4), "flops_per_step": runs_flops,
                    "runs": runs, "stages_ms_per_step": stage_split(ctx, rfwd, args.steps)}
        log(f"block with modulation runs: {msr:.3f} ms  {runs_tf:.1f} TFLOP/s")
        del bwr, xr, vecs

    # ---------------------------------------------------------------- cached reference rows (bf16)
    cached = None
    if not args.no_cached:
        first = S - 1024
        log(f"block step with 1024 cached reference rows (rows {first}..{S - 1} read only)")
        bwc = L.BlockWeights.from_host(case["block"])
        xc = L.dev_f32(case["x"])
        slot = torch.empty(2 * H * (S - first) * 128, dtype=torch.bfloat16, device="cuda")
        ctx.block_forward_cached(bwc, xc, seq.vec, seq.cos, seq.sin, sh.L, sh.N, first, slot, True)

        def cfwd():
            ctx.block_forward_cached(bwc, xc, seq.vec, seq.cos, seq.sin, sh.L, sh.N, first, slot, False)
        msc = time_call(torch, cfwd, args.steps, args.warmup)
        # algorithmic work of the step: the products over `first` rows, the
        # attention of `first` queries against all S keys, the GEMV
        c_flops = (2 * first * D * (3 * D + D + 2 * F + F) + 4 * H * first * S * 128 + 2 * 6 * D * D)
        c_tf = c_flops / (msc * 1e-3) / 1e12
        cached = {"ms": round(msc, 4), "tflops": round(c_tf, 2), "first": first, "flops_per_step": c_flops,
                  "stages_ms_per_step": stage_split(ctx, cfwd, args.steps)}
        log(f"cached step: {msc:.3f} ms  {c_tf:.1f} TFLOP/s")
        del bwc, xc, slot

    # ---------------------------------------------------------------- sandwich block (bf16)
    sw = None
    if not args.no_sandwich:
        log("sandwich block (attention and MLP outputs normed before their gates)")
        sb = dict(case["block"])
        sb["post_attn"] = synth.normal((D,), seed=sh.seed + 300, std=0.2, mean=1.0)
        sb["post_mlp"] = synth.normal((D,), seed=sh.seed + 301, std=0.2, mean=1.0)
        bws = L.BlockWeights.from_host(sb)
        xs = L.dev_f32(case["x"])

        def sfwd():
            ctx.block_forward(bws, xs, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
        mss = time_call(torch, sfwd, args.steps, args.warmup)
        sw_tf = total_flops / (mss * 1e-3) / 1e12
        sw = {"ms": round(mss, 4), "tflops": round(sw_tf, 2), "frac_bf16_peak": round(sw_tf / PEAK_BF16_TFLOPS, 4),
              "flops_per_step": total_flops, "stages_ms_per_step": stage_split(ctx, sfwd, args.steps)}
        log(f"sandwich block: {mss:.3f} ms  {sw_tf:.1f} TFLOP/s")
        post = sw["stages_ms_per_step"].get("post")
        if post:    # two launches a block: y read, x read and written, fp32 [S, D] each
            hbm.update(hbm_rows({"post": post / 2}, {"post": 12 * S * D}))
        del bws, xs, sb

    # ---------------------------------------------------------------- unfused q/k/v prep (B arm)
    unfused = None
    if not args.no_unfused:
        log("block with the q/k/v prep as a pass of its own (unfused arm)")
        bwu = L.BlockWeights.from_host(case["block"])
        xu = L.dev_f32(case["x"])
        ctx.set_qk_prep(False)

        def ufwd():
            ctx.block_forward(bwu, xu, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
        msu = time_call(torch, ufwd, args.steps, args.warmup)
        u_st = stage_split(ctx, ufwd, args.steps)
        ctx.set_qk_prep(True)
        u_tf = total_flops / (msu * 1e-3) / 1e12
        unfused = {"ms": round(msu, 4), "tflops": round(u_tf, 2), "frac_bf16_peak": round(u_tf / PEAK_BF16_TFLOPS, 4),
                   "stages_ms_per_step": u_st, "arm": "unfused (QKV product stores bf16, then k_qk_prep)"}
        hbm.update(hbm_rows(u_st, {"qk_prep": sb_bytes["qk_prep"]}))
        log(f"unfused-arm block: {msu:.3f} ms  {u_tf:.1f} TFLOP/s; prep pass {u_st.get('qk_prep', 0):.4f} ms")
        del bwu, xu
    del case
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- int8 block
    int8_tf = int8i = None
    if not args.no_int8:
        log("int8-weight block")
        c8 = synth.block_case("s4608_int8")
        bw8 = L.BlockWeights.from_host(c8["block"])
        x8 = L.dev_f32(c8["x"])
        ms8 = time_blocks(L, torch, ctx, bw8, x8, seq, sh, args.steps, args.warmup)
        int8_tf = total_flops / (ms8 * 1e-3) / 1e12
        int8_st = stage_split(ctx, lambda: ctx.block_forward(bw8, x8, seq.vec, seq.cos, seq.sin, sh.L, sh.N), args.steps)
        log(f"int8 block (dequantisation pass, bf16 products): {ms8:.3f} ms  {int8_tf:.1f} TFLOP/s; stages " +
            ", ".join(f"{k} {v:.3f}" for k, v in int8_st.items()))
        if int8_st.get("dequant"):      # codes + scales read, bf16 written: 2.0625 + 2 bytes a weight
            nw = 3 * D * D + D * D + 2 * F * D + F * D
            hbm.update(hbm_rows({"dequant": int8_st["dequant"] / 4}, {"dequant": nw // 4 * (1 + 1 / 16 + 2)}))
        ctx.set_int8_products(True)
        try:
            ms8i = time_blocks(L, torch, ctx, bw8, x8, seq, sh, args.steps, args.warmup)
            int8i_st = stage_split(ctx, lambda: ctx.block_forward(bw8, x8, seq.vec, seq.cos, seq.sin, sh.L, sh.N),
                                   args.steps)
        finally:
            ctx.set_int8_products(False)
        int8i = {"ms": round(ms8i, 4), "tflops": round(total_flops / (ms8i * 1e-3) / 1e12, 2),
                 "stages_ms_per_step": int8i_st,
                 "arm": "codes converted inside each product (dit_set_int8_products(ctx, 1))"}
        log(f"int8 block (codes converted inside the products): {ms8i:.3f} ms")
        del bw8, x8, c8
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- W8A8 block
    w8 = None
    if not args.no_w8a8:
        log("W8A8 block (INT8 weight rows, INT8 activation rows, int8 matrix cores)")
        cw = synth.block_case("s4608_w8a8")
        bww = L.BlockWeights.from_host(cw["block"])
        xw = L.dev_f32(cw["x"])

        def wfwd():
            ctx.block_forward(bww, xw, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
        msw = time_call(torch, wfwd, args.steps, args.warmup)
        w_tf = total_flops / (msw * 1e-3) / 1e12
        w_st = stage_split(ctx, wfwd, args.steps)
        up_ops = stage_flops(S, D, H, F)["up"]
        up_tops = up_ops / (w_st["up"] * 1e-3) / 1e12
        w8 = {"ms": round(msw, 4), "tflops": round(w_tf, 2), "flops_per_step": total_flops,
              "stages_ms_per_step": w_st,
              "roofline": {"kernel": "W8A8 up product (int8 matrix cores)", "bound": "mfma",
                           "achieved": round(up_tops, 1), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                           "frac": round(up_tops / PEAK_INT8_TOPS, 4), "ops_per_launch": up_ops,
                           "avg_ms": w_st["up"]}}
        log(f"W8A8 block: {msw:.3f} ms  {w_tf:.1f} TFLOP/s (int8 ops)")
        q_st = w_st.get("quant")
        if q_st:    # two launches a block: o (D wide) and a (F wide), bf16 in, INT8 + scale out
            hbm.update(hbm_rows({"quant": q_st / 2}, {"quant": (3 * S * D + 3 * S * F) // 2 + 8 * S}))
        bwr = L.BlockWeights.from_host(cw["block"], rotated=True)

        def rfwd8():
            ctx.block_forward(bwr, xw, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
        msr8 = time_call(torch, rfwd8, args.steps, args.warmup)
        r_tf = total_flops / (msr8 * 1e-3) / 1e12
        w8["convrot"] = {"ms": round(msr8, 4), "tflops": round(r_tf, 2),
                         "stages_ms_per_step": stage_split(ctx, rfwd8, args.steps),
                         "weights": "INT8 rows in the rotated basis; inputs rotated by the regular Hadamard of 256"}
        log(f"W8A8 block with ConvRot: {msr8:.3f} ms  {r_tf:.1f} TFLOP/s (int8 ops)")
        del bww, xw, cw, bwr
        torch.cuda.empty_cache()
    ctx.close()

    calib = None if args.no_calibration else calibration(torch)
    if calib:
        log(f"calibration: chained 8192^3 bf16 GEMM {calib['gemm_bf16_chained_tflops']} TFLOP/s, "
            f"1 GiB copy {calib['copy_gbs']} GB/s")

    # ---------------------------------------------------------------- whole image
    img = img8 = imgi8 = None
    if not args.no_denoise:
        img = bench_images(torch, L, synth, args.images)
        if img.get("euler_ms"):   # x read and written, v read: fp32 [N, 64]
            hbm.update(hbm_rows({"euler": img["euler_ms"]}, {"euler": 3 * 4 * sh.N * 64}))
        if not args.no_w8a8:
            img8 = bench_images(torch, L, synth, args.images, w8a8=True)
        if not args.no_int8:
            imgi8 = bench_images(torch, L, synth, args.images, int8=True)

    # ---------------------------------------------------------------- CPU oracle
    cpu = None if args.no_cpu else cpu_baseline()

    out = {
        "metric": "DiT block fwd TFLOP/s (% bf16 MFMA peak) at N=4096; images/s, 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dit_block_forward, 1024-px block: L=512 text + N=4096 image rows, "
                               "hidden 3072, 24 heads x 128, SwiGLU ffn 12288, bf16 weights",
                   "L": sh.L, "N": sh.N, "hidden": D, "heads": H, "head_dim": 128, "ffn": F,
                   "flops_per_step": total_flops},
        "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "block_bytes": block_bytes,
        "frac_hbm": round(block_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "per_step_ms": per_step,
        "power": power,
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "roofline": roofline,
        "hbm_kernels": hbm,
        "calibration": calib,
        "int8_block_tflops": None if int8_tf is None else round(int8_tf, 2),
        "int8_block": None if int8_tf is None else {"ms": round(ms8, 4), "tflops": round(int8_tf, 2),
                                                    "stages_ms_per_step": int8_st,
                                                    "arm": "dequantisation pass per weight, then bf16 products",
                                                    "in_product": int8i},
        "unfused_qk_prep_block": unfused,
        "parallel_block": par,
        "double_block": dbl,
        "runs_block": runs_res,
        "sandwich_block": sw,
        "cached_step": cached,
        "w8a8_block": w8,
    }
    if img:
        img = dict(img)
        img.pop("euler_ms", None)
        img["image_frac_bf16_peak"] = round(img["image_tflops"] / PEAK_BF16_TFLOPS, 4)
        img_bytes = 4 * sh_blocks_bytes(block_bytes)
        img["image_bytes"] = img_bytes
        img["image_frac_hbm"] = round(img_bytes / (img["ms_per_image"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        out.update(img)
    if img8:
        out["w8a8_image"] = {k: img8[k] for k in ("images_per_s", "ms_per_image", "unplanned", "image_finite", "image_workload")}
    if imgi8:
        out["int8_image"] = {k: imgi8[k] for k in ("images_per_s", "ms_per_image", "unplanned", "image_finite", "image_workload")}
    out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def bench_images(torch, L, synth, images, w8a8=False, int8=False):
    """Whole path per image at the 1024-px DiT: 32 blocks, 4 Euler steps;
    with w8a8, blocks of INT8 weight rows (W8A8 products); with int8, int8
    block-32 weights (dequantised before the bf16 products)."""
    sh = synth.SHAPES["dit32"]
    S, D, H, F, lat = sh.S, sh.hidden, sh.heads, sh.ffn, sh.latent
    arch = L.make_arch(hidden=D, heads=H, ffn=F, latent=lat, text_dim=sh.text_dim)
    ctx = L.Context(arch, max_rows=S)
    kind = "W8A8" if w8a8 else "int8 block-32" if int8 else "bf16"
    log(f"generating 32 blocks of random {kind} weights on the GPU")
    g = torch.Generator(device="cuda")
    g.manual_seed(sh.seed)

    def w(o, i):
        t = torch.randn((o, i), generator=g, device="cuda", dtype=torch.float32).mul_(0.02)
        return t.to(torch.bfloat16)

    def q8(o, i):
        return torch.randint(-127, 128, (o, i), generator=g, device="cuda", dtype=torch.int8)

    def s8(o):
        return torch.full((o,), 0.02 * 3 ** 0.5 / 127, device="cuda", dtype=torch.float32)

    def sb(o, i):   # block-32 scales |N(0,1)| * 0.01 in bf16
        return torch.randn((o, i // 32), generator=g, device="cuda").abs_().mul_(0.01).to(torch.bfloat16)

    blocks = []
    dims = {"w_qkv": (3 * D, D), "w_out": (D, D), "w_up": (2 * F, D), "w_down": (D, F)}
    for _ in range(sh.blocks):
        if w8a8:
            t = {}
            for n, (o, i) in dims.items():
                t["q8_" + n], t["s8_" + n] = q8(o, i), s8(o)
        elif int8:
            t = {}
            for n, (o, i) in dims.items():
                t["q_" + n], t["s_" + n] = q8(o, i), sb(o, i)
        else:
            t = {n: w(o, i) for n, (o, i) in dims.items()}
        t.update({"w_mod": w(6 * D, D), "q_norm": torch.ones(128, device="cuda"),
                  "k_norm": torch.ones(128, device="cuda")})
        blocks.append(L.BlockWeights(t, int8=int8))
    top = {"w_t1": w(D, sh.time_dim), "w_t2": w(D, D), "w_in": w(D, lat), "w_txt": w(D, sh.text_dim),
           "w_fmod": w(2 * D, D), "w_final": w(lat, D)}
    model = L.ModelWeights(top, blocks)
    x0 = torch.randn((sh.N, lat), generator=g, device="cuda")
    ctx_feats = torch.randn((sh.L, sh.text_dim), generator=g, device="cuda")
    pos = torch.empty((S, 3), dtype=torch.int32, device="cuda")
    cs = torch.empty((S, 64), dtype=torch.float32, device="cuda")
    sn = torch.empty_like(cs)
    txt = torch.empty((sh.L, D), dtype=torch.float32, device="cuda")
    sig = np.linspace(1.0, 0.0, 5).astype(np.float32)

    def one_image(x, planned=True):
        ctx.positions(sh.L, sh.h, sh.w, pos)
        ctx.rope_tables(pos, S, cs, sn)
        ctx.prologue(model, ctx_feats, sh.L, txt)
        ctx.plan_schedule(model, sig[:4] if planned else [])
        for i in range(4):
            ctx.denoise_step(model, x, txt, cs, sn, sh.L, sh.N, float(sig[i]), float(sig[i + 1]))

    x = x0.clone()
    st = torch.cuda.current_stream()

    def timed(planned):
        one_image(x, planned)              # warm-up image
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(images):
            x.copy_(x0)
            one_image(x, planned)
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / images
    ms_un = timed(False)
    ms = timed(True)
    finite = bool(torch.isfinite(x).all().item())

    # the per-image prologue on its own (positions, tables, text rows), and
    # the Euler update's launch time from the stage timers
    def prologue():
        ctx.positions(sh.L, sh.h, sh.w, pos)
        ctx.rope_tables(pos, S, cs, sn)
        ctx.prologue(model, ctx_feats, sh.L, txt)
    pro = percentiles(time_each(torch, prologue, 10))
    ctx.timing(True)
    x.copy_(x0)
    one_image(x)
    tm = ctx.timing_read()
    ctx.timing(False)
    euler_ms = tm["euler"][0] / tm["euler"][1] if tm["euler"][1] else None
    blk = sum(stage_flops(S, D, H, F).values())
    img_flops = 4 * (sh.blocks * blk + 2 * sh.N * lat * D + 2 * sh.N * D * lat + 2 * D * 256
                     + 2 * D * D + 2 * 2 * D * D) + 2 * sh.L * sh.text_dim * D
    log(f"image{'' if kind == 'bf16' else ' (' + kind + ')'}: {ms:.1f} ms  {1000 / ms:.3f} img/s  {img_flops / ms / 1e9:.1f} TFLOP/s  "
        f"finite={finite}  (unplanned {ms_un:.1f} ms)")
    ctx.close()
    del model, blocks, top
    torch.cuda.empty_cache()
    return {"images_per_s": round(1000.0 / ms, 4), "ms_per_image": round(ms, 2),
            "prologue_ms": pro, "steps_ms": round(ms - pro["p50"], 2), "euler_ms": euler_ms,
            "image_tflops": round(img_flops / ms / 1e9, 2), "image_flops": img_flops,
            "unplanned": {"images_per_s": round(1000.0 / ms_un, 4), "ms_per_image": round(ms_un, 2)},
            "image_workload": "32-block DiT, 4 Euler steps (sigmas 1, .75, .5, .25, 0), L=512 + N=4096, "
                              f"latent 64, text features 4096-d, batch 1, random-init {kind} "
                              "block weights",
            "image_finite": finite}


def cpu_baseline():
    """The CPU oracle (float64 NumPy) on one whole block forward of the same
    1024-px workload (same seed), reported in the metric's unit."""
    import oracle as O
    from diffusion_transformer_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    case = synth.block_case("s4608")
    sh = case["shape"]
    oa = O.Arch(sh.hidden, sh.heads, 128, sh.ffn)
    pos = O.positions(sh.L, sh.h, sh.w)
    cs, sn = O.rope_tables(pos)
    b = case["block"]
    bw = O.BlockWeights(w_qkv=b["w_qkv"], w_out=b["w_out"], w_up=b["w_up"], w_down=b["w_down"],
                        w_mod=b["w_mod"], q_norm=b["q_norm"], k_norm=b["k_norm"])
    # whole block forwards until at least 10 s of CPU work, at most 8 of them
    t0 = time.perf_counter()
    reps = 0
    while reps < 8 and (reps == 0 or time.perf_counter() - t0 < 10.0):
        vec = O.time_vector(float(case["t"]), case["w_t1"], case["w_t2"])
        O.block_forward(case["x"], bw, vec, cs, sn, oa)
        reps += 1
    dt = time.perf_counter() - t0
    flops = O.block_flops(sh.S, oa) * reps
    log(f"cpu oracle: {dt:.1f} s for {reps} block(s), {flops / 1e9:.1f} GFLOP ({threads} threads)")
    per_block = dt / reps
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2), "blocks": reps,
            "image_seconds_extrapolated": round(4 * 32 * per_block, 1),
            "image_note": "extrapolated: 4 steps x 32 blocks x the measured seconds per block (the in/out products "
                          "and the text rows are under 0.1 % of the work)",
            "sample": f"{reps} whole block forward(s) of the float64 NumPy oracle on the same 1024-px block "
                      "(L=512 + N=4096 rows, hidden 3072, 24x128 heads, ffn 12288), 1652.6 GFLOP each, "
                      "repeated until 10 s of CPU work (at most 8)"}


if __name__ == "__main__":
    main()
