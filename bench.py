#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X: fused attention forward + decode.

One step = one pass of the whole path over one batch of synthetic input:
  * forward, bf16, B=2 H=Hkv=32 D=128 S=8192, no mod, with LSE (the headline);
  * decode, f16, B=1 H=32 D=128, KV length 32768, additive pad mask, with LSE.
Inputs are seeded N(0,1) (mask_mods_amd.inputs) and resident in HBM before timing.

Printed: one JSON line with the forward TFLOP/s as `value`, its roofline (MFMA
bound) and the decode GB/s with its roofline (HBM bound); the two headline calls
again by the pages' report method (10 warmup calls, 12 samples of 100 calls, mean,
std, CV); the other flex cases at S=8192, 4096 and 2048 and at D=64; GQA
cross-attention; decode at KV lengths 1, 17, 1000 and 4096, GQA, paged and a
mixed-length batch of 8; the backward; and the CPU oracle timed on a bounded sample
of the forward workload, on the tiny fp32 workload and on the full decode call, on
this host's cores.

    python bench.py [--steps K] [--warmup W] [--seed N] [--gpus 1] [--no-cpu-baseline]
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

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
MFMA_FP8_PEAK_TFLOPS = 5033.2    # twice the bf16 rate (dense fp8)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
SETTLE_S = 0.5                   # untimed headline steps before any timing (clock settle)
SEED = 0                         # --seed: added to every input seed of the run


def sd(n: int) -> int:
    """The run's seed for input stream n (the same streams as with --seed 0, shifted)."""
    return n + SEED
PAGES_NO_MOD_MI300X_TFLOPS = 470.1  # FlyDSL PR #931 report, no_mod at this workload (MI300X)

FWD = dict(B=2, H=32, S=8192, D=128)
DEC = dict(B=1, H=32, L=32768, D=128)
FWD_KERNEL = "fwd_pipe_kernel"  # the headline (D 128, no mod) runs the software-pipelined forward
DEC_KERNELS = ("decode_split_kernel", "decode_merge_kernel")
FP8_KERNEL = "fwd_fp8_kernel"
KERNEL_SOURCES = ["mask_mods_amd/csrc/fwd_pipe.h", "mask_mods_amd/csrc/fwd_tile.h",
                  "mask_mods_amd/csrc/fwd_mfma.h", "mask_mods_amd/csrc/fwd_fp8.h",
                  "mask_mods_amd/csrc/fwd_common.h", "mask_mods_amd/csrc/common.h",
                  "mask_mods_amd/csrc/decode.hip", "mask_mods_amd/csrc/kernels.h"]
# the pages' report method (FlyDSL PR, Performance Report): warmup 10, then 12 samples of
# 100 iterations each, mean +- std and the coefficient of variation
PAGES_WARMUP, PAGES_SAMPLES, PAGES_ITERS = 10, 12, 100


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def fwd_flops(B, H, Sq, Skv, D, causal=False):
    f = 4.0 * B * H * Sq * Skv * D
    return f / 2 if causal else f


def fwd_bytes(B, H, S, D, elt=2):
    return 4 * B * H * S * D * elt + B * H * S * 4


def fp8_bytes(B, H, S, D):
    """Q, K, V in one byte per element, O in bf16, LSE in fp32: each moved once."""
    return 3 * B * H * S * D + 2 * B * H * S * D + 4 * B * H * S


def dec_bytes(B, H, L, D, elt=2):
    return B * H * L * D * elt * 2 + B * H * L * 2 + 2 * B * H * D * elt + B * H * 4


def window_pairs(S, w):
    """Visited (i, j) pairs of |i-j| <= w AND j <= i over an S x S square."""
    return sum(min(i, w) + 1 for i in range(S))


def load_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it is current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    ent = t.get(kernel)
    if not ent or ent.get("src_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_configs(xd):
    """The oracle on the tiny fp32 workload and on the headline decode call, each in full."""
    import oracle
    from mask_mods_amd import inputs
    out = {}
    x = inputs.attention_inputs(sd(0), 1, 2, 2, 128, 128, 64, "f32")
    args = [inputs.bits_to_f64(x[n], "f32") for n in ("q", "k", "v")]
    t0 = time.perf_counter()
    for _ in range(10):
        oracle.attention(*args, scale=0.125)
    dt = (time.perf_counter() - t0) / 10
    out["tiny_fp32_b1_h2_s128_d64"] = {"seconds": dt, "note": "full workload, mean of 10 calls"}
    Bd, Hd, L, Dd = DEC["B"], DEC["H"], DEC["L"], DEC["D"]
    qd, kd, vd = (inputs.bits_to_f64(xd[n], "f16") for n in ("q", "k", "v"))
    t0 = time.perf_counter()
    oracle.attention(qd, kd, vd, scale=0.08837890625, Skv=L, add_mask=inputs.bits_to_f64(xd["mask"], "f16"))
    dt = time.perf_counter() - t0
    out["decode_f16_b1_h32_d128_l32768"] = {"seconds": dt, "GBs": dec_bytes(Bd, Hd, L, Dd) / dt / 1e9,
                                            "note": "full workload, one call"}
    return out


def cpu_baseline(x, target_s=10.0, xd=None):
    """Time the oracle on random rows of the forward workload (bounded sample)."""
    import oracle
    from mask_mods_amd import inputs
    B, H, S, D = FWD["B"], FWD["H"], FWD["S"], FWD["D"]
    qd, kd, vd = (inputs.bits_to_f64(x[n], "bf16") for n in ("q", "k", "v"))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    g = np.random.default_rng(sd(123))
    threads = oracle.max_threads()
    probe = g.integers(0, B * H * S, size=4096)
    t0 = time.perf_counter()
    oracle.attention(qd, kd, vd, scale=scale, rows=probe)
    dt = max(time.perf_counter() - t0, 1e-6)
    n = int(min(max(4096 * target_s / dt, 4096), 400000))
    rows = g.integers(0, B * H * S, size=n)
    t0 = time.perf_counter()
    oracle.attention(qd, kd, vd, scale=scale, rows=rows)
    dt = time.perf_counter() - t0
    flops = n * 4.0 * S * D
    res = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{n} random query rows of the B2 H32 D128 S8192 bf16 no-mod forward "
                     f"(each row against all {S} keys), fp64, {dt:.1f} s; full workload "
                     f"extrapolates to {B * H * S / (n / dt):.0f} s",
           "seconds": dt}
    if xd is not None:
        res["full_configs"] = cpu_configs(xd)
    return res


COPY_BYTES = 1 << 30  # --only copy: 1 GiB read and 1 GiB written per call


def _read_counters(path):
    import csv
    import collections
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            out[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def _find(root, sub, suffix):
    for dp, _, files in os.walk(os.path.join(root, sub)):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(dp, fn)
    raise FileNotFoundError(f"{sub}/*{suffix} under {root}")


def ingest(root):
    """Turn rocprofv3 outputs under `root` into profiles/traffic.json and profiles/*.md.

    Expects sub-directories fetch_{fwd,decode,copy} and write_{fwd,decode,copy} from
    `rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --kernel-trace -f csv -- python bench.py --only X`
    and `trace` from `rocprofv3 --kernel-trace --stats -f csv -- python bench.py`.
    FETCH_SIZE / WRITE_SIZE are in KiB per dispatch; each is scaled by the factor that
    maps the copy kernel's reading onto the bytes it really moves.
    """
    def per_dispatch(sub, counter, match):
        data = _read_counters(_find(root, sub, "counter_collection.csv"))
        vals = [v for k, cs in data.items() if match(k) for v in cs.get(counter, [])]
        if not vals:
            raise RuntimeError(f"no {counter} samples for {sub}")
        return sum(vals) / len(vals) * 1024.0

    is_copy = lambda k: "copyBuffer" in k or "copy" in k.lower() and "mm::" not in k
    f_copy = per_dispatch("fetch_copy", "FETCH_SIZE", is_copy)
    w_copy = per_dispatch("write_copy", "WRITE_SIZE", is_copy)
    kf, kw = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    res = {"calibration": {"copy_bytes": COPY_BYTES, "fetch_raw_bytes": f_copy, "write_raw_bytes": w_copy,
                           "fetch_factor": round(kf, 4), "write_factor": round(kw, 4)}}
    h = kernel_source_hash()
    for name, sub, match, alg in [
        (FWD_KERNEL, "fwd", lambda k: FWD_KERNEL in k, fwd_bytes(FWD["B"], FWD["H"], FWD["S"], FWD["D"])),
        ("decode", "decode", lambda k: "decode_" in k, dec_bytes(DEC["B"], DEC["H"], DEC["L"], DEC["D"])),
        (FP8_KERNEL, "fp8", lambda k: FP8_KERNEL in k, fp8_bytes(FWD["B"], FWD["H"], FWD["S"], FWD["D"])),
    ]:
        fr = _read_counters(_find(root, "fetch_" + sub, "counter_collection.csv"))
        wr = _read_counters(_find(root, "write_" + sub, "counter_collection.csv"))
        fb = sum(sum(cs["FETCH_SIZE"]) / len(cs["FETCH_SIZE"]) for k, cs in fr.items() if match(k)) * 1024 * kf
        wb = sum(sum(cs["WRITE_SIZE"]) / len(cs["WRITE_SIZE"]) for k, cs in wr.items() if match(k)) * 1024 * kw
        res[name] = {"src_hash": h, "fetch_bytes": round(fb), "write_bytes": round(wb),
                     "bytes_per_launch": round(fb + wb), "algorithmic_bytes": alg,
                     "ratio_to_algorithmic": round((fb + wb) / alg, 3)}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def to_fp8(t, torch):
    """Per-tensor e4m3 quantisation on the device: (t / s) rounded, s = max|t| / 448."""
    s = (t.float().abs().max() / 448.0).item()
    return (t.float() / s).to(torch.float8_e4m3fn), s


def time_calls(torch, stream, fn, n=20, warmup=5):
    """Mean seconds per call of fn over n calls after warmup (HIP events on the stream)."""
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e-3


def pages_stats(torch, stream, fn):
    """The pages' method: PAGES_WARMUP calls, then PAGES_SAMPLES samples of PAGES_ITERS
    calls each; per-call time in microseconds, mean +- std over samples, CV in percent."""
    for _ in range(PAGES_WARMUP):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(PAGES_SAMPLES)]
    for e0, e1 in ev:
        e0.record(stream)
        for _ in range(PAGES_ITERS):
            fn()
        e1.record(stream)
    torch.cuda.synchronize()
    us = np.array([e0.elapsed_time(e1) / PAGES_ITERS * 1e3 for e0, e1 in ev])
    return {"mean_us": round(float(us.mean()), 2), "std_us": round(float(us.std()), 2),
            "cv_pct": round(float(us.std() / us.mean() * 100), 2),
            "method": f"{PAGES_WARMUP} warmup, {PAGES_SAMPLES} samples x {PAGES_ITERS} calls"}


def graph_stats(torch, dev, call, snapshot, last_set, eager):
    """The pages' method on a captured HIP graph of PAGES_ITERS calls (no host launch cost
    in the timed region): PAGES_SAMPLES replays after a warmup replay. Each replay's last
    output is checked against an eager call on the same inputs (bitwise: the kernels are
    deterministic); the replays alternate with that eager work and synchronisations."""
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(PAGES_ITERS):
            call()
    torch.cuda.synchronize()
    st = last_set()  # the inputs of the graph's last call
    stream = torch.cuda.current_stream(dev)
    us, ok = [], True
    for i in range(PAGES_SAMPLES + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        o_g, l_g = snapshot()
        o_e, l_e = eager(st)
        torch.cuda.synchronize()
        ok &= bool(torch.equal(o_g, o_e)) and bool(torch.equal(l_g, l_e))
        if i > 0:
            us.append(e0.elapsed_time(e1) / PAGES_ITERS * 1e3)
    del g
    us = np.array(us)
    return {"mean_us": round(float(us.mean()), 2), "std_us": round(float(us.std()), 2),
            "cv_pct": round(float(us.std() / us.mean() * 100), 2),
            "method": f"HIP graph of {PAGES_ITERS} calls, {PAGES_SAMPLES} replays after one warmup replay",
            "replays_equal_eager": ok}


def profile_one(args, torch, mm, inputs, dev):
    """Run one kernel family only (for rocprofv3 passes); prints a small JSON line."""
    def dev_tensor(bits, dtype):
        tt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tt).to(dev)

    if args.only == "copy":
        n = COPY_BYTES // 2  # fp16 elements: 1 GiB read + 1 GiB written per copy
        src = torch.ones(n, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)
        unit_bytes = 2 * n
    elif args.only == "fp8":
        B, H, S, D = FWD["B"], FWD["H"], FWD["S"], FWD["D"]
        x = inputs.attention_inputs(sd(2), B, H, H, S, S, D, "bf16")
        q, k, v = (dev_tensor(x[n], "bf16") for n in ("q", "k", "v"))
        (q8, sq), (k8, sk), (v8, sv) = (to_fp8(t, torch) for t in (q, k, v))
        out = torch.empty_like(q)
        lse = torch.empty(B, H, S, dtype=torch.float32, device=dev)
        scale = float(np.float32(1.0 / math.sqrt(D)))
        fn = lambda: mm.attn_fwd(q8, k8, v8, scale, descale=(sq, sk, sv), out=out, lse=lse)
        unit_bytes = fp8_bytes(B, H, S, D)
    elif args.only == "bwd":
        B, H, S, D = FWD["B"], FWD["H"], FWD["S"], FWD["D"]
        x = inputs.attention_inputs(sd(2), B, H, H, S, S, D, "bf16")
        q, k, v = (dev_tensor(x[n], "bf16") for n in ("q", "k", "v"))
        scale = float(np.float32(1.0 / math.sqrt(D)))
        out, lse = mm.attn_fwd(q, k, v, scale)
        g = np.random.default_rng(sd(11))
        dout = torch.from_numpy(g.standard_normal((B, H, S, D), dtype=np.float32)).to(dev).bfloat16()
        ws = torch.empty(mm.bwd_workspace_size(B, H, S) // 4 + 4, dtype=torch.float32, device=dev)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        fn = lambda: mm.attn_bwd(q, k, v, out, lse, dout, scale, workspace=ws,
                                 dq=grads[0], dk=grads[1], dv=grads[2])
        unit_bytes = 8 * B * H * S * D * 2 + 2 * B * H * S * 4  # q k v o dO in, dq dk dv out, lse
    elif args.only == "gqa":
        # GQA decode (B1 Hq32 Hkv8 L32768 D128 f16, pad mask), three input sets in rotation
        # (408 MB, past the 256 MB Infinity Cache) as in the benchmark's case
        Hq, Hkv, L, D = DEC["H"], 8, DEC["L"], DEC["D"]
        sets = []
        for r in range(3):
            xg = inputs.decode_inputs(sd(3 + r), 1, Hq, Hkv, [L], D, "f16")
            sets.append(tuple(dev_tensor(xg[n], "f16") for n in ("q", "k", "v", "mask")))
        ws = torch.empty(mm.decode_workspace_size(1, Hq, L, D, Hkv=Hkv) // 4 + 4, dtype=torch.float32, device=dev)
        calls = [0]

        def fn():
            gq, gk, gv, gm = sets[calls[0] % 3]
            calls[0] += 1
            mm.attn_decode(gq, gk, gv, L, 0.08837890625, mask=gm, workspace=ws)
        unit_bytes = Hkv * L * D * 2 * 2 + Hq * L * 2 + 2 * Hq * D * 2 + Hq * 4
    elif args.only in ("window", "causal2048"):
        # the banded forward (WINDOW(256) AND causal at the headline shape) and the short
        # causal forward (S 2048), for their own counter passes
        B, H, D = FWD["B"], FWD["H"], FWD["D"]
        S = FWD["S"] if args.only == "window" else 2048
        x = inputs.attention_inputs(sd(2), B, H, H, S, S, D, "bf16")
        q, k, v = (dev_tensor(x[n], "bf16") for n in ("q", "k", "v"))
        out = torch.empty_like(q)
        lse = torch.empty(B, H, S, dtype=torch.float32, device=dev)
        scale = float(np.float32(1.0 / math.sqrt(D)))
        kw = dict(window=256, mask_flags=mm.MASK_CAUSAL) if args.only == "window" else dict(causal=True)
        fn = lambda: mm.attn_fwd(q, k, v, scale, out=out, lse=lse, **kw)
        unit_bytes = fwd_bytes(B, H, S, D)
    elif args.only == "fwd":
        B, H, S, D = FWD["B"], FWD["H"], FWD["S"], FWD["D"]
        x = inputs.attention_inputs(sd(2), B, H, H, S, S, D, "bf16")
        q, k, v = (dev_tensor(x[n], "bf16") for n in ("q", "k", "v"))
        out = torch.empty_like(q)
        lse = torch.empty(B, H, S, dtype=torch.float32, device=dev)
        scale = float(np.float32(1.0 / math.sqrt(D)))
        fn = lambda: mm.attn_fwd(q, k, v, scale, out=out, lse=lse)
        unit_bytes = fwd_bytes(B, H, S, D)
    else:
        Bd, Hd, L, Dd = DEC["B"], DEC["H"], DEC["L"], DEC["D"]
        x = inputs.decode_inputs(sd(1), Bd, Hd, Hd, [L], Dd, "f16")
        dq, dk, dv, dm = (dev_tensor(x[n], "f16") for n in ("q", "k", "v", "mask"))
        ws = torch.empty(mm.decode_workspace_size(Bd, Hd, L, Dd) // 4 + 4, dtype=torch.float32, device=dev)
        fn = lambda: mm.attn_decode(dq, dk, dv, L, 0.08837890625, mask=dm, workspace=ws)
        unit_bytes = dec_bytes(Bd, Hd, L, Dd)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(args.steps, 1)
    print(json.dumps({"only": args.only, "ms_per_call": round(ms, 4), "steps": args.steps,
                      "algorithmic_bytes_per_call": unit_bytes,
                      "src_hash": kernel_source_hash()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--seed", type=int, default=0, help="offset added to every input seed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cases", action="store_true", help="skip the other flex cases")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--only", choices=["fwd", "fp8", "bwd", "decode", "copy", "window", "causal2048", "gqa"], default=None,
                    help="profiling aid: run just one kernel family (or a plain 1 GiB device copy "
                         "used to calibrate the HBM byte counters) and print its timing")
    ap.add_argument("--ingest", metavar="DIR", default=None,
                    help="host only: turn rocprofv3 PMC outputs under DIR into profiles/traffic.json")
    args = ap.parse_args()
    if args.ingest:
        return ingest(args.ingest)
    global SEED
    SEED = args.seed
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(attention shards by (batch, head) with no exchange between GPUs, so each "
              "GPU would run the same kernels on its own share).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mask_mods_amd as mm
    from mask_mods_amd import inputs

    mm.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only is not None:
        return profile_one(args, torch, mm, inputs, dev)

    def dev_tensor(bits, dtype):
        tt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tt).to(dev)

    # ---- inputs (seeded, synthetic), resident in HBM
    B, H, S, D = FWD["B"], FWD["H"], FWD["S"], FWD["D"]
    xf = inputs.attention_inputs(sd(2), B, H, H, S, S, D, "bf16")
    q, k, v = (dev_tensor(xf[n], "bf16") for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    lse = torch.empty(B, H, S, dtype=torch.float32, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(D)))

    Bd, Hd, L, Dd = DEC["B"], DEC["H"], DEC["L"], DEC["D"]
    xd = inputs.decode_inputs(sd(1), Bd, Hd, Hd, [L], Dd, "f16")
    dq, dk, dv = (dev_tensor(xd[n], "f16") for n in ("q", "k", "v"))
    dmask = dev_tensor(xd["mask"], "f16")
    dout = torch.empty_like(dq)
    dlse = torch.empty(Bd, Hd, dtype=torch.float32, device=dev)
    ws = torch.empty(mm.decode_workspace_size(Bd, Hd, L, Dd) // 4 + 4, dtype=torch.float32, device=dev)
    dscale = 0.08837890625
    torch.cuda.synchronize()

    def fwd():
        mm.attn_fwd(q, k, v, scale, out=out, lse=lse)

    def dec():
        mm.attn_decode(dq, dk, dv, L, dscale, mask=dmask, workspace=ws, out=dout, lse=dlse)

    stream = torch.cuda.current_stream(dev)
    # Untimed: SETTLE_S seconds of headline steps bring the GPU clock to its loaded steady
    # state, which takes longer than a few steps (started cold with 5 warmup steps, the
    # timed steps read about 3% slow and 7x as spread; the report method's first samples
    # likewise)
    settle_steps = 0
    t_settle = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_settle:
        for _ in range(10):
            fwd()
            dec()
        settle_steps += 10
        torch.cuda.synchronize()
    # the pages' report method on the two headline calls: mean +- std over 12 samples of
    # 100 calls after 10 warmup calls, and the coefficient of variation
    fwd_pages = pages_stats(torch, stream, fwd)
    dec_pages = pages_stats(torch, stream, dec)

    for _ in range(args.warmup):
        fwd()
        dec()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        dec()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    fwd_ms = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)])
    dec_ms = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)])
    ms_per_step = (t1 - t0) * 1e3 / K

    flops = fwd_flops(B, H, S, S, D)
    fwd_avg_s = fwd_ms.mean() * 1e-3
    tflops = flops / fwd_avg_s / 1e12
    dbytes = dec_bytes(Bd, Hd, L, Dd)
    dec_avg_s = dec_ms.mean() * 1e-3
    gbs = dbytes / dec_avg_s / 1e9


    # ---- other flex cases at the same shape (context; same kernel family)
    cases = {}
    if not args.no_cases:
        W = 256
        specs = {
            "causal": dict(causal=True),
            "alibi": dict(score_mod=mm.SCORE_ALIBI),
            "sliding_window": dict(window=W, mask_flags=mm.MASK_CAUSAL),
            "causal_via_mask": dict(mask_flags=mm.MASK_CAUSAL),
        }
        # block-sparse: the causal classes from mm_block_mask_create, and an i.i.d. table
        # with half of the blocks empty (a quarter full, a quarter partial, no predicate)
        nqb, nkb = S // mm.BLOCK_Q, S // mm.BLOCK_KV
        bm_causal = mm.block_mask_create(S, S, causal=True)
        bm_rand_np = inputs.random_block_mask(sd(7), (B, H, nqb, nkb), p_empty=0.5, p_full=0.25)
        bm_rand = torch.from_numpy(bm_rand_np).to(dev)
        specs["block_causal"] = dict(causal=True, block_mask=bm_causal)
        specs["block_sparse_50"] = dict(block_mask=bm_rand)
        block_pairs = int((bm_rand_np != 0).sum()) * mm.BLOCK_Q * mm.BLOCK_KV
        # document mask (packed sequences, a mask_mod over captured id tensors): 16
        # documents of random lengths per sequence, causal inside each document
        docs_np = inputs.packed_document_ids(sd(7), B, S, 16)
        specs["document_causal"] = dict(causal=True, q_doc=torch.from_numpy(docs_np).to(dev))
        doc_pairs = H * sum(int(n) * (int(n) + 1) // 2
                            for row in docs_np for n in np.unique(row, return_counts=True)[1])
        # fp8 (e4m3) inputs: the same draws quantised per tensor on the device
        (q8, sq), (k8, sk), (v8, sv) = (to_fp8(t, torch) for t in (q, k, v))
        fp8_kw = dict(q=q8, k=k8, v=v8, descale=(sq, sk, sv))
        specs["fp8_no_mod"] = dict(fp8_kw)
        specs["fp8_causal"] = dict(fp8_kw, causal=True)
        for name, kw in specs.items():
            kw = dict(kw)
            qq, kk, vv = kw.pop("q", q), kw.pop("k", k), kw.pop("v", v)
            # the pages' report method (a 20-call window showed the first case after the
            # headline runs up to 8% slower than the same kernel timed later)
            st = pages_stats(torch, stream, lambda: mm.attn_fwd(qq, kk, vv, scale, out=out, lse=lse, **kw))
            t = st["mean_us"] * 1e-6
            dense = fwd_flops(B, H, S, S, D)
            if name in ("causal", "causal_via_mask", "block_causal", "fp8_causal"):
                alg = dense / 2
            elif name == "block_sparse_50":
                alg = 4.0 * D * block_pairs  # block_pairs: kept pairs summed over (b, h)
            elif name == "sliding_window":
                alg = 4.0 * B * H * D * window_pairs(S, W)
            elif name == "document_causal":
                alg = 4.0 * D * doc_pairs  # kept pairs summed over (b, h)
            else:
                alg = dense
            ent = {"us": round(t * 1e6, 1), "std_us": st["std_us"], "cv_pct": st["cv_pct"],
                   "tflops_dense_equiv": round(dense / t / 1e12, 1),
                   "tflops_algorithmic": round(alg / t / 1e12, 1)}
            if name == "causal":
                ent["tflops_causal_half"] = round(dense / 2 / t / 1e12, 1)
            if name.startswith("fp8"):
                ent["frac_fp8_peak"] = round(alg / t / 1e12 / MFMA_FP8_PEAK_TFLOPS, 4)
            ent["latency_vs_no_mod"] = round(t / fwd_avg_s, 3)
            cases[name] = ent
        # the sliding window ∧ causal at widths from 0 (one key per row: the launch then
        # only streams Q, K, V and O through HBM once) to 4096: the banded cases' floor
        ladder = {}
        for Wl in (0, 64, 256, 1024, 4096):
            kw = dict(window=Wl, mask_flags=mm.MASK_CAUSAL)
            t = time_calls(torch, stream, lambda kw=kw: mm.attn_fwd(q, k, v, scale, out=out, lse=lse, **kw))
            ladder[str(Wl)] = {"us": round(t * 1e6, 1),
                               "tflops_algorithmic": round(4.0 * B * H * D * window_pairs(S, Wl) / t / 1e12, 1),
                               "hbm_tb_s_min_traffic": round(4.0 * B * H * S * D * 2 / t / 1e12, 2)}
        cases["sliding_window_ladder"] = ladder
        cases["method"] = (f"flex cases: {PAGES_WARMUP} warmup, {PAGES_SAMPLES} samples x {PAGES_ITERS} calls "
                           "(mean, std); window ladder: 20 calls after 5 warmup")

    # ---- the dense workload's shorter lengths with every flex case (S 2048 and 4096), and
    # the D 64 variant (S 2048 and 8192): the pages' tables report each case at each length
    scases = {}
    if not args.no_cases:
        W = 256
        short = {"no_mod": dict(), "causal": dict(causal=True), "alibi": dict(score_mod=mm.SCORE_ALIBI),
                 "sliding_window": dict(window=W, mask_flags=mm.MASK_CAUSAL),
                 "causal_via_mask": dict(mask_flags=mm.MASK_CAUSAL)}
        for Ds, lens, names in ((D, (2048, 4096), list(short)), (64, (2048, 8192), ["no_mod", "causal", "alibi"])):
            for Ss in lens:
                xs = inputs.attention_inputs(sd(2), B, H, H, Ss, Ss, Ds, "bf16")
                sq_, sk_, sv_ = (dev_tensor(xs[n], "bf16") for n in ("q", "k", "v"))
                sout = torch.empty_like(sq_)
                slse = torch.empty(B, H, Ss, dtype=torch.float32, device=dev)
                ss_ = float(np.float32(1.0 / math.sqrt(Ds)))
                t_nomod = None
                for cname in names:
                    kw = short[cname]
                    # the pages' report method: a call here is 40-1400 us, so 20 calls would
                    # time a window short enough for clock ramps and the previous case to show
                    st = pages_stats(torch, stream, lambda: mm.attn_fwd(sq_, sk_, sv_, ss_, out=sout, lse=slse, **kw))
                    t = st["mean_us"] * 1e-6
                    dense = fwd_flops(B, H, Ss, Ss, Ds)
                    if cname in ("causal", "causal_via_mask"):
                        alg = dense / 2
                    elif cname == "sliding_window":
                        alg = 4.0 * B * H * Ds * window_pairs(Ss, W)
                    else:
                        alg = dense
                    t_nomod = t if cname == "no_mod" else t_nomod
                    scases[f"d{Ds}_s{Ss}_{cname}"] = {
                        "us": round(t * 1e6, 1), "std_us": st["std_us"], "cv_pct": st["cv_pct"],
                        "tflops_dense_equiv": round(dense / t / 1e12, 1),
                        "tflops_algorithmic": round(alg / t / 1e12, 1),
                        "frac_bf16_peak": round(alg / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                        "latency_vs_no_mod": round(t / t_nomod, 3) if t_nomod else None}
                del sq_, sk_, sv_, sout

    # ---- GQA cross-attention at its own shape: B2 Hq32 Hkv8 D128 Sq1024 Skv8192, bf16 and
    # f16, with the hash mask_mod that drops about 5% of the query rows, then also
    # WINDOW(256) AND causal on raw (top-left) indices. Kept pairs are counted from the
    # kernel's own LSE: a dropped row is the only kind with LSE = -inf here.
    gcases = {}
    if not args.no_cases:
        Bg, Hqg, Hkvg, Sqg, Skvg, Wg = 2, 32, 8, 1024, 8192, 256
        rd = (20240, int(0.05 * 2 ** 32))
        dense_g = fwd_flops(Bg, Hqg, Sqg, Skvg, D)
        for dt in ("bf16", "f16"):
            xg = inputs.attention_inputs(sd(4), Bg, Hqg, Hkvg, Sqg, Skvg, D, dt)
            gq, gk, gv = (dev_tensor(xg[n], dt) for n in ("q", "k", "v"))
            gout = torch.empty_like(gq)
            glse = torch.empty(Bg, Hqg, Sqg, dtype=torch.float32, device=dev)
            for wname, kw in (("rowdrop", {}), ("rowdrop_window", dict(window=Wg, mask_flags=mm.MASK_CAUSAL))):
                for _ in range(5):
                    mm.attn_fwd(gq, gk, gv, scale, rowdrop=rd, out=gout, lse=glse, **kw)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                n = 20
                e0.record(stream)
                for _ in range(n):
                    mm.attn_fwd(gq, gk, gv, scale, rowdrop=rd, out=gout, lse=glse, **kw)
                e1.record(stream)
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1) / n * 1e-3
                live = torch.isfinite(glse).cpu().numpy()  # [B, Hq, Sq]
                per_row = (np.full(Sqg, Skvg) if wname == "rowdrop"
                           else np.minimum(np.arange(Sqg), Wg) + 1)
                kept = int((live * per_row[None, None, :]).sum())
                gcases[f"{dt}_{wname}"] = {
                    "us": round(t * 1e6, 1), "tflops_dense_equiv": round(dense_g / t / 1e12, 1),
                    "tflops_algorithmic": round(4.0 * D * kept / t / 1e12, 1),
                    "rows_dropped": round(1.0 - float(live.mean()), 4)}

    traffic_fwd = load_traffic(FWD_KERNEL)
    traffic_dec = load_traffic("decode")
    res = {
        "metric": "attn fwd TFLOPS bf16 B2 H32 D128 S8192 (+% MFMA peak); decode KV GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "seed": args.seed,
        "settle": {"seconds": SETTLE_S, "steps": settle_steps,
                   "note": "untimed headline steps before the report method and the warmup"},
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tflops / PAGES_NO_MOD_MI300X_TFLOPS, 3),
        "vs_baseline_ref": "pages' FlyDSL no_mod on MI300X (gfx942), 470.1 TFLOP/s: context, other hardware",
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fwd bf16 B2 H32 Hkv32 D128 S8192 no-mod +LSE; "
                               "decode f16 B1 H32 D128 L32768 pad-mask +LSE",
                   "global_batch": B, "seq_len": S, "parallelism": "none (1 GPU)"},
        "fwd_ms": round(float(fwd_ms.mean()), 4),
        "fwd_ms_std": round(float(fwd_ms.std()), 4),
        "fwd_pages_method": {**fwd_pages, "tflops": round(flops / (fwd_pages["mean_us"] * 1e-6) / 1e12, 1)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_fwd, "kernel": FWD_KERNEL,
                     "algorithmic": f"{flops:.4e} flop per launch (4*B*H*S*S*D)"},
        "decode": {
            "value": round(gbs, 1), "unit": "GB/s", "us": round(dec_avg_s * 1e6, 2),
            "pages_method": {**dec_pages, "GBs": round(dbytes / (dec_pages["mean_us"] * 1e-6) / 1e9, 1)},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_dec,
                         "kernel": "+".join(DEC_KERNELS),
                         "algorithmic": f"{dbytes} bytes per call (K+V+mask+q+out+lse)"},
        },
        "cases_s8192": cases,
        "cases_dense_short": ({"workload": "fwd bf16 B2 H32 +LSE: D128 at Sq=Skv 2048 and 4096 with every flex "
                                           "case, D64 at 2048 and 8192; causal half-counted, sliding window "
                                           "over visited pairs",
                               "method": f"{PAGES_WARMUP} warmup, {PAGES_SAMPLES} samples x {PAGES_ITERS} "
                                         "calls per case (mean, std)",
                               **scases} if scases else {}),
        "cases_gqa_cross": {"workload": "fwd B2 Hq32 Hkv8 D128 Sq1024 Skv8192, ~5% of query rows dropped "
                                        "by a hash mask_mod; _window adds |i-j|<=256 AND j<=i (top-left)",
                            **gcases} if gcases else {},
    }
    # decode variants: GQA (Hq 32 / Hkv 8: K/V streamed once per kv head) and a paged
    # cache (B 8, 64-key pages scattered over a pool by a seeded permutation)
    if not args.no_cases:
        dcases = {}
        def time_dec(fn, n=20):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n * 1e-3
        Hkv_g = 8
        # 136 MB per call: three input sets (408 MB) in rotation, so that the 256 MB
        # Infinity Cache cannot serve a call's K/V from the previous one
        gsets = []
        for r in range(3):
            xg = inputs.decode_inputs(sd(3 + r), 1, Hd, Hkv_g, [L], Dd, "f16")
            gsets.append(tuple(dev_tensor(xg[n], "f16") for n in ("q", "k", "v", "mask")))
        gws = torch.empty(mm.decode_workspace_size(1, Hd, L, Dd, Hkv=Hkv_g) // 4 + 4, dtype=torch.float32, device=dev)
        gcall = [0]

        def gqa_call():
            gq, gk, gv, gm = gsets[gcall[0] % len(gsets)]
            gcall[0] += 1
            mm.attn_decode(gq, gk, gv, L, dscale, mask=gm, workspace=gws)
        t = time_dec(gqa_call)
        gbytes = 1 * Hkv_g * L * Dd * 2 * 2 + 1 * Hd * L * 2 + 2 * 1 * Hd * Dd * 2 + 1 * Hd * 4
        dcases["gqa_b1_h32_kv8_l32768"] = {"us": round(t * 1e6, 2), "GBs": round(gbytes / t / 1e9, 1),
                                           "bytes": gbytes, "rotation": "3 input sets, 408 MB"}
        del gsets
        Bp, page = 8, 64
        pages = L // page
        gp = np.random.default_rng(sd(5))
        perm = torch.from_numpy(gp.permutation(Bp * pages).reshape(Bp, pages).astype(np.int32)).to(dev)
        pk = torch.randn(Bp * pages, Hd, page, Dd, device=dev).half()
        pv = torch.randn_like(pk)
        pq = torch.randn(Bp, Hd, 1, Dd, device=dev).half()
        pws = torch.empty(mm.decode_workspace_size(Bp, Hd, L, Dd) // 4 + 4, dtype=torch.float32, device=dev)
        t = time_dec(lambda: mm.attn_decode(pq, pk, pv, L, dscale, workspace=pws, block_table=perm))
        pbytes = Bp * Hd * L * Dd * 2 * 2 + 2 * Bp * Hd * Dd * 2 + Bp * Hd * 4 + Bp * pages * 4
        dcases["paged_b8_h32_l32768_page64"] = {"us": round(t * 1e6, 2), "GBs": round(pbytes / t / 1e9, 1),
                                                "bytes": pbytes}
        ck = torch.randn(Bp, Hd, L, Dd, device=dev).half()
        cv = torch.randn_like(ck)
        del pk, pv
        t = time_dec(lambda: mm.attn_decode(pq, ck, cv, L, dscale, workspace=pws))
        cbytes = Bp * Hd * L * Dd * 2 * 2 + 2 * Bp * Hd * Dd * 2 + Bp * Hd * 4
        dcases["contiguous_b8_h32_l32768"] = {"us": round(t * 1e6, 2), "GBs": round(cbytes / t / 1e9, 1),
                                              "bytes": cbytes}
        del ck, cv

        # latency ladder of the pages' decode table: B1 H32 D128 f16 with the pad mask at
        # KV lengths 1, 17, 1000 and 4096 (32768 is the headline call above). From 1000 on,
        # enough input sets rotate that one pass over them exceeds the 256 MB Infinity
        # Cache, so every call streams its K/V from HBM; below that the call is launch-bound.
        gen = torch.Generator(device=dev)
        gen.manual_seed(sd(17))
        ladder = {}
        for Ll in (1, 17, 1000, 4096):
            per_set = dec_bytes(1, Hd, Ll, Dd)
            nsets = -(-300_000_000 // per_set) if Ll >= 1000 else 1
            sets = []
            for r in range(nsets):
                lk = torch.randn(1, Hd, Ll, Dd, device=dev, generator=gen).half()
                lv = torch.randn(1, Hd, Ll, Dd, device=dev, generator=gen).half()
                lq = torch.randn(1, Hd, 1, Dd, device=dev, generator=gen).half()
                lm = torch.zeros(1, Hd, 1, Ll, device=dev, dtype=torch.float16)
                pad = int(torch.randint(0, Ll, (1,), generator=gen, device=dev))
                if pad:
                    lm[..., Ll - pad:] = float("-inf")
                sets.append((lq, lk, lv, lm))
            lws = torch.empty(mm.decode_workspace_size(1, Hd, Ll, Dd) // 4 + 4, dtype=torch.float32, device=dev)
            lout = torch.empty(1, Hd, 1, Dd, device=dev, dtype=torch.float16)
            llse = torch.empty(1, Hd, device=dev, dtype=torch.float32)
            lcall = [0]

            def ladder_call():
                lq, lk, lv, lm = sets[lcall[0] % nsets]
                lcall[0] += 1
                mm.attn_decode(lq, lk, lv, Ll, dscale, mask=lm, workspace=lws, out=lout, lse=llse)
            st = pages_stats(torch, stream, ladder_call)
            ent = {**st, "GBs": round(per_set / (st["mean_us"] * 1e-6) / 1e9, 1),
                   "bytes": per_set, "rotation": f"{nsets} input sets, {nsets * per_set / 1e6:.0f} MB"}
            ent["graph"] = graph_stats(torch, dev, ladder_call, lambda: (lout.clone(), llse.clone()),
                                       lambda: (sets[(lcall[0] - 1) % nsets]),
                                       lambda st_: mm.attn_decode(*st_[:3], Ll, dscale, mask=st_[3], workspace=lws))
            ladder[f"l{Ll}"] = ent
            del sets
        ladder["l32768"] = {**dec_pages, "GBs": round(dbytes / (dec_pages["mean_us"] * 1e-6) / 1e9, 1),
                            "bytes": dbytes, "rotation": f"1 input set of {dbytes / 1e6:.0f} MB"}
        ladder["l32768"]["graph"] = graph_stats(
            torch, dev, dec, lambda: (dout.clone(), dlse.clone()), lambda: None,
            lambda _: mm.attn_decode(dq, dk, dv, L, dscale, mask=dmask, workspace=ws))
        res["decode_latency"] = {"workload": "decode f16 B1 H32 D128 +pad mask +LSE at KV length L", **ladder}

        # a batch of 8 sequences whose KV lengths are drawn from the ladder's lengths (cache
        # capacity 32768, per-sequence lengths passed to the kernel)
        Bm = 8
        lens_m = np.random.default_rng(sd(29)).choice([1, 17, 1000, 4096, 32768], size=Bm)
        mk = torch.randn(Bm, Hd, L, Dd, device=dev, generator=gen).half()
        mv = torch.randn(Bm, Hd, L, Dd, device=dev, generator=gen).half()
        mq = torch.randn(Bm, Hd, 1, Dd, device=dev, generator=gen).half()
        mlens = torch.from_numpy(lens_m.astype(np.int32)).to(dev)
        mws = torch.empty(mm.decode_workspace_size(Bm, Hd, L, Dd) // 4 + 4, dtype=torch.float32, device=dev)
        kvmax = int(lens_m.max())
        st = pages_stats(torch, stream, lambda: mm.attn_decode(mq, mk, mv, kvmax, dscale, seq_lens=mlens,
                                                               workspace=mws))
        mbytes = int(sum(Hd * int(n) * Dd * 2 * 2 for n in lens_m)) + 2 * Bm * Hd * Dd * 2 + Bm * Hd * 4 + Bm * 4
        dcases["mixed_b8_h32"] = {**st, "GBs": round(mbytes / (st["mean_us"] * 1e-6) / 1e9, 1), "bytes": mbytes,
                                  "lens": [int(n) for n in lens_m], "Scap": L}
        del mk, mv
        res["decode_cases"] = dcases

    # backward (bf16, same shape): dq, dk, dv of sum(dO * O) from the forward's O and LSE
    if not args.no_cases:
        g = np.random.default_rng(sd(11))
        dout = torch.from_numpy(g.standard_normal((B, H, S, D), dtype=np.float32)).to(dev).bfloat16()
        bws = torch.empty(mm.bwd_workspace_size(B, H, S) // 4 + 4, dtype=torch.float32, device=dev)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        bwd = {}
        bcases = [("no_mod", {}), ("causal", dict(causal=True))]
        if "document_causal" in cases:
            bcases.append(("document_causal", dict(causal=True, q_doc=torch.from_numpy(docs_np).to(dev))))
        for name, kw in bcases:
            o_b = torch.empty_like(q)
            l_b = torch.empty(B, H, S, dtype=torch.float32, device=dev)
            mm.attn_fwd(q, k, v, scale, out=o_b, lse=l_b, **kw)
            run = lambda: mm.attn_bwd(q, k, v, o_b, l_b, dout, scale, workspace=bws,
                                      dq=grads[0], dk=grads[1], dv=grads[2], **kw)
            for _ in range(3):
                run()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 10
            e0.record(stream)
            for _ in range(n):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / n * 1e-3
            # five products of the forward's size (S and dP recomputed, dV, dK, dQ):
            # 2.5 x the forward's flops (half for causal)
            if name == "document_causal":
                alg = 2.5 * 4.0 * D * doc_pairs
            else:
                alg = 2.5 * fwd_flops(B, H, S, S, D) * (0.5 if kw else 1.0)
            bwd[name] = {"us": round(t * 1e6, 1), "tflops_algorithmic": round(alg / t / 1e12, 1),
                         "frac_bf16_peak": round(alg / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        res["bwd"] = {"workload": "bf16 B2 H32 D128 S8192, dq/dk/dv from the forward's O and LSE",
                      "algorithmic": "2.5 x 4*B*H*S*S*D flop (five S-sized products; causal half; "
                                     "documents: 2.5 x 4*D per kept pair)",
                      **bwd}
    if "fp8_no_mod" in cases:
        c8 = cases["fp8_no_mod"]
        a8 = fwd_flops(B, H, S, S, D) / (c8["us"] * 1e-6) / 1e12
        res["fp8"] = {
            "value": round(a8, 1), "unit": "TFLOP/s", "us": c8["us"],
            "roofline": {"bound": "mfma", "achieved": round(a8, 1), "peak": MFMA_FP8_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(a8 / MFMA_FP8_PEAK_TFLOPS, 4),
                         "traffic": load_traffic(FP8_KERNEL), "kernel": FP8_KERNEL,
                         "algorithmic": "4*B*H*S*S*D flop per launch; e4m3 Q/K/V, bf16 O"},
        }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(xf, args.cpu_seconds, xd=xd)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
