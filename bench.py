#!/usr/bin/env python3
"""Throughput benchmark of the sliding-window attention hot path on one MI355X.

One step = one band-tiled forward over the Mistral-7B-shaped workload
(B=1, 32 query / 8 KV heads, d=128, N=16384, W=4096, bf16, Q/K scaled by 0.5)
with inputs already resident in HBM.  `value` is the in-band throughput
4 * B * Hq * d * sum_i |S_i| / time, in TFLOP/s, where |S_i| is row i's
allowed-key count (only in-band pairs count; masked work inside edge tiles
counts against the kernel).  The same line carries:
  * roofline   -- the band kernel against the bf16 dense matrix-core peak,
                  with HIP-event timing on the launch stream, and the HBM
                  traffic measured by rocprofv3 counters when the summary in
                  profiles/ was taken on the current kernel source;
  * decode     -- the rolling-window decode step (64 sequences, W=4096 ring,
                  32/8 heads, d=128) in GB/s of algorithmic bytes vs 8 TB/s;
  * chunk      -- chunked prefill over the rolling cache (4 sequences x 4096
                  new tokens, cached lengths 0 / 1500 / 4095 / 61440) in
                  in-band TFLOP/s, and the ring append of the same chunk;
  * variants   -- the same layer under the two-sided band, differential
                  attention and global-token masks (in-band TFLOP/s);
  * other_prefill -- the other two prefill workloads of the metric: the
                  Gemma-3-shaped SWA-1024 forward at N=65536 (in-band TFLOP/s)
                  and the local+strided mask at N=8192, which is small and
                  HBM-bound (in-band TFLOP/s and GB/s of Q+K+V+O);
  * cpu_baseline -- the float64 oracle on the host cores over the whole
                  prefill workload (run before the GPU is touched, since its
                  worker pool forks).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "band8_traffic_mistral16k.txt")
BAND_SOURCES = ["sparse_causal_attention_band_amd/csrc/swa_band_fwd.hip",
                "sparse_causal_attention_band_amd/csrc/swa_internal.h",
                "sparse_causal_attention_band_amd/build.py"]


def allowed_pairs(N: int, W: int, stride: int) -> int:
    """sum_i |S_i|: min(i+1, W) band keys, plus for stride > 0 the multiples
    of stride strictly below the band start i-W+1."""
    total = 0
    for i in range(N):
        total += min(i + 1, W)
        if stride > 0 and i >= W:
            total += (i - W) // stride + 1
    return total


def _code_only(text: str) -> str:
    """C/C++ source without comments, whitespace collapsed: a comment edit
    leaves the compiled kernel, and so its measured traffic, unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split())


def band_source_hash() -> str:
    h = hashlib.sha256()
    for rel in BAND_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        if rel.endswith((".hip", ".h")):
            text = _code_only(text)
        h.update(text.encode("utf-8"))
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if it is missing or was taken on another kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != band_source_hash() or kv.get("workload") != workload:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, q, k, v, rows):
    import numpy as np

    import oracle

    workers = min(16, len(os.sched_getaffinity(0)))
    qs = q.float().numpy()
    ks = k.float().numpy()
    vs = v.float().numpy()
    t0 = time.perf_counter()
    _, used = oracle.attn_fwd_parallel(qs, ks, vs, cfg.window, cfg.stride, 1 / math.sqrt(cfg.d),
                                       np.asarray(rows), workers=workers)
    dt = time.perf_counter() - t0
    pairs = 0
    for i in rows:
        pairs += min(i + 1, cfg.window)
        if cfg.stride > 0 and i >= cfg.window:
            pairs += (i - cfg.window) // cfg.stride + 1
    flops = 4.0 * cfg.B * cfg.Hq * cfg.d * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "sample": f"query rows {rows[0]}..{rows[-1]} of every (batch, head) of {cfg.name} "
                      f"({pairs * cfg.B * cfg.Hq:.3e} allowed pairs, float64 numpy, {dt:.2f} s wall)"}


def decode_cpu_baseline(cfg, q, kr, vr, pos):
    import oracle

    t0 = time.perf_counter()
    oracle.decode(q.float().numpy(), kr.float().numpy(), vr.float().numpy(), pos.numpy(), cfg.window,
                  1 / math.sqrt(cfg.d))
    dt = time.perf_counter() - t0
    return dt


def two_sided_pairs(N: int, left: int, right: int) -> int:
    """sum_i |S_i| of the two-sided band: min(i, left) + min(N-1-i, right) + 1."""
    return sum(min(i, left) + min(N - 1 - i, right) + 1 for i in range(N))


def global_pairs(N: int, W: int, g) -> int:
    """sum_i |S_i| of the causal window plus global positions g: a global row
    reads i + 1 keys, another row its min(i+1, W) band keys plus the global
    positions below its band."""
    gs = sorted(set(g))
    gset = set(gs)
    total = 0
    below = 0  # global positions < i - W + 1 (the band start)
    for i in range(N):
        while below < len(gs) and gs[below] < i - W + 1:
            below += 1
        total += (i + 1) if i in gset else min(i + 1, W) + below
    return total


def variant_legs(swa, inputs, torch, dev, args):
    """The Mistral-shaped layer (B=1, 32/8 heads, d=128, N=16384, bf16) under
    the other masks: two-sided band (left = right = 2048, the [i - W/2,
    i + W/2] window with W = 4096), differential attention (two maps, W =
    4096, lam per head in [0.5, 0.8]) and W = 4096 plus 16 global positions
    (0 and every 1024th).  In-band TFLOP/s counts only allowed pairs."""
    cfg = inputs.MISTRAL
    q, k, v = (x.to(dev) for x in inputs.prefill_inputs(cfg))
    B, Hq, Hkv, N, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d
    steps, warm = max(5, args.steps // 3), 2
    res = {}

    def leg(name, fn, pairs_per_head, maps=1, extra=None):
        per, _ = time_launches(lambda i=0: fn(), steps, warm, torch)
        ms = sum(per) / len(per)
        fl = 4.0 * B * Hq * d * pairs_per_head * maps
        res[name] = {"value": round(fl / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                     "frac_mfma": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "avg_ms": round(ms, 4), "algorithmic_flops": fl}
        if extra:
            res[name].update(extra)

    out = torch.empty_like(q)
    leg("two_sided_l2048_r2048", lambda: swa.attn_fwd_two_sided(q, k, v, 2048, 2048, out=out),
        two_sided_pairs(N, 2048, 2048))
    q2, k2 = q.flip(2).contiguous(), k.flip(2).contiguous()
    lam = torch.linspace(0.5, 0.8, Hq, device=dev)
    leg("diff_w4096", lambda: swa.diff_attn_fwd(q, k, q2, k2, v, lam, 4096, out=out),
        allowed_pairs(N, 4096, 0), maps=2)
    g = [0] + list(range(1024, N, 1024))
    gi = torch.tensor(g, dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, swa.global_workspace_bytes(B, Hq, Hkv, N, d, len(g))), dtype=torch.uint8, device=dev)
    leg("global_w4096_g16", lambda: swa.attn_fwd_global(q, k, v, 4096, gi, out=out, workspace=ws),
        global_pairs(N, 4096, g), extra={"global_positions": len(g)})
    return res


def other_prefill_legs(swa, inputs, torch, dev, args):
    """The Gemma-3-shaped SWA-1024 forward (B=2, 32/16 heads, N=65536) and
    the local+strided forward (W=256 plus every 128th key, 16 heads, d=64,
    N=8192), each timed like the main leg with fewer steps."""
    res = {}
    for cfg, steps in ((inputs.GEMMA, max(5, args.steps // 5)), (inputs.STRIDED, args.steps)):
        q, k, v = (x.to(dev) for x in inputs.prefill_inputs(cfg))
        out = torch.empty_like(q)
        per, _ = time_launches(lambda i=0: swa.attn_fwd(q, k, v, window=cfg.window, stride=cfg.stride, out=out),
                               steps, 10, torch)
        ms = sum(per) / len(per)
        fl = 4.0 * cfg.B * cfg.Hq * cfg.d * allowed_pairs(cfg.N, cfg.window, cfg.stride)
        tf = fl / (ms * 1e-3) / 1e12
        leg = {"value": round(tf, 2), "unit": "TFLOP/s", "frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
               "avg_ms": round(ms, 4), "steps": steps, "algorithmic_flops": fl}
        if cfg.stride:
            # compulsory HBM bytes: Q and O per query head, K and V per KV head
            nb = 2 * (2 * cfg.B * cfg.Hq + 2 * cfg.B * cfg.Hkv) * cfg.N * cfg.d
            leg.update({"algorithmic_bytes": nb, "GB_s": round(nb / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        res[cfg.name] = leg
        del q, k, v, out
        torch.cuda.empty_cache()
    return res


def time_launches(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return per, wall


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the warm-up also brings the GPU clock up after the host-side baseline
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="mistral", choices=["mistral", "gemma", "strided"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-chunk", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the two-sided, differential and global-token legs")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the Gemma-shaped and local+strided prefill legs")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the design notes describe how the band kernel would shard).", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_causal_attention_band_amd as swa
    from sparse_causal_attention_band_amd import inputs

    cfg = {"mistral": inputs.MISTRAL, "gemma": inputs.GEMMA, "strided": inputs.STRIDED}[args.workload]
    q, k, v = inputs.prefill_inputs(cfg)
    pairs = allowed_pairs(cfg.N, cfg.window, cfg.stride)
    flops = 4.0 * cfg.B * cfg.Hq * cfg.d * pairs

    dcfg = inputs.DECODE
    dq, dkr, dvr, dpos = inputs.decode_inputs(dcfg)

    cpu = None
    dec_cpu_s = None
    if not args.no_cpu_baseline:
        rows = list(range(cfg.N))  # the whole workload: every row of every (batch, head)
        cpu = cpu_baseline(cfg, q, k, v, rows)
        if not args.no_decode:
            dec_cpu_s = decode_cpu_baseline(dcfg, dq, dkr, dvr, dpos)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)

    def step(i=0):
        swa.attn_fwd(qd, kd, vd, window=cfg.window, stride=cfg.stride, out=out)

    per, wall = time_launches(step, args.steps, args.warmup, torch)
    ms = sum(per) / len(per)
    value = flops / (ms * 1e-3) / 1e12
    traffic = read_traffic(cfg.name)
    roof = {"bound": "mfma", "achieved": round(value, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
            "kernel": "band8_kernel<d=128, band>" if cfg.Hq // cfg.Hkv % 4 == 0 and cfg.stride == 0
            else "band_fwd_kernel<bf16, d=%d>" % cfg.d, "avg_launch_ms": round(ms, 4),
            "algorithmic_flops_per_launch": flops}

    line = {
        "metric": "SWA prefill in-band TFLOP/s (% bf16 MFMA peak); decode GB/s (% HBM peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "N": cfg.N, "d": cfg.d,
                   "window": cfg.window, "stride": cfg.stride, "allowed_pairs_per_head": pairs},
        "roofline": roof,
        "cpu_baseline": cpu,
    }

    if not args.no_decode:
        del qd, kd, vd, out
        B, Hq, Hkv, d, W = dcfg.B, dcfg.Hq, dcfg.Hkv, dcfg.d, dcfg.window
        dqd, dposd = dq.to(dev), dpos.to(dev)
        # two ring copies, alternated, so consecutive steps do not re-read a
        # cache-resident ring
        rings = [(dkr.to(dev), dvr.to(dev)), (dkr.to(dev), dvr.to(dev))]
        dout = torch.empty_like(dqd)
        need = swa.decode_workspace_bytes(B, Hq, Hkv, d, W)
        ws = torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else None

        def dstep(i=0):
            kr_, vr_ = rings[i % 2]
            swa.decode(dqd, kr_, vr_, dposd, out=dout, workspace=ws)

        dper, dwall = time_launches(dstep, max(args.steps, 20), args.warmup, torch)
        dms = sum(dper) / len(dper)
        n = dpos.clamp(min=0).clamp(max=W).to(torch.int64)
        dbytes = int(n.sum()) * 2 * Hkv * d * 2 + 2 * B * Hq * d * 2 + 4 * B
        gbs = dbytes / (dms * 1e-3) / 1e9
        line["decode"] = {"workload": dcfg.name, "value": round(gbs, 1), "unit": "GB/s",
                          "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "avg_step_ms": round(dms, 4),
                          "algorithmic_bytes_per_step": dbytes,
                          "kernels": "decode_split_kernel<bf16,128,4> (one split: no merge kernel)",
                          "cpu_baseline": None if dec_cpu_s is None else
                          {"value": round(dbytes / dec_cpu_s / 1e9, 3), "unit": "GB/s", "cores": 1,
                           "kind": "oracle", "sample": f"whole {dcfg.name} step, float64 numpy, {dec_cpu_s:.2f} s"}}

    if not args.no_chunk:
        ccfg = inputs.CHUNK
        cq, ck, cv, ckr, cvr, cp0 = (x.to(dev) for x in inputs.chunk_inputs(ccfg))
        cout = torch.empty_like(cq)

        def cstep(i=0):
            swa.chunk_prefill(cq, ck, cv, ckr, cvr, cp0, out=cout)

        def astep(i=0):
            # same slots every step (p0 fixed): the ring contents do not
            # change the work of either kernel
            swa.ring_append(ck, cv, cp0, ckr, cvr)

        cper, _ = time_launches(cstep, args.steps, args.warmup, torch)
        aper, _ = time_launches(astep, args.steps, args.warmup, torch)
        cms, ams = sum(cper) / len(cper), sum(aper) / len(aper)
        cpairs = sum(min(p + r + 1, ccfg.window) for p in ccfg.p0 for r in range(ccfg.T))
        cflops = 4.0 * ccfg.Hq * ccfg.d * cpairs
        abytes = 2 * 2 * len(ccfg.p0) * ccfg.Hkv * min(ccfg.T, ccfg.window) * ccfg.d * 2  # K,V read + write
        line["chunk"] = {"workload": ccfg.name, "p0": list(ccfg.p0), "value": round(cflops / (cms * 1e-3) / 1e12, 2),
                         "unit": "TFLOP/s", "frac_mfma": round(cflops / (cms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "avg_launch_ms": round(cms, 4), "algorithmic_flops_per_launch": cflops,
                         "kernel": "band8_kernel<d=128, chunk>",
                         "ring_append": {"avg_launch_ms": round(ams, 4), "bytes": abytes,
                                         "GB_s": round(abytes / (ams * 1e-3) / 1e9, 1)}}
        del cq, ck, cv, ckr, cvr, cp0, cout

    if not args.no_variants:
        line["variants"] = variant_legs(swa, inputs, torch, dev, args)
    if not args.no_other and args.workload == "mistral":
        line["other_prefill"] = other_prefill_legs(swa, inputs, torch, dev, args)

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
