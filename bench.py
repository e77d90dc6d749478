#!/usr/bin/env python3
"""One-GPU benchmark: fused RoPE + causal attention forward (TFLOP/s against
the bf16 matrix-core peak) and the standalone ragged RoPE op (HBM GB/s).

A step is one fused forward over the workload (default: 1x8x4096x64 bf16,
NeoX RoPE base 10000, causal); inputs are resident in HBM before timing.
W untimed warmup steps, then exactly K timed steps between two device
synchronisations; rank 0 prints ONE JSON line.

  value          whole-job TFLOP/s = algorithmic flops / wall time per step
                 (algorithmic flops: 4*D per query/key pair the mask allows);
                 the K steps run back to back between two synchronisations
  roofline       the fused kernel: flops per launch / mean launch duration,
                 from one HIP event pair on the launch stream around the K
                 launches, against 2500 TFLOP/s
  rope_apply     the ragged RoPE workload (8192 tokens, 32 Q + 8 K heads,
                 rot 64 of 128): algorithmic bytes / mean launch duration
                 (measured the same way), cycling through enough buffer sets
                 to defeat the 256 MB last-level cache, against 8 TB/s
  cpu_baseline   the fp64 CPU oracle on the same workload (whole heads),
                 timed on this host's cores
  comparators    context rows mirroring "RoPE + PoPE Attention Kernels"'
                 benchmark table: the same kernel without rotation ("flash"),
                 and rope_apply on copies of Q/K followed by it ("unfused"),
                 with peak extra device memory
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

METRIC = "fused RoPE+causal attn fwd TFLOP/s (%MFMA peak); rope_apply HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth, published
# "RoPE + PoPE Attention Kernels", median runtime table: rope (rotate, then
# flash) at 1x8x4096x64 on an unnamed CUDA GPU -- context, not a target.
PAGE_ROPE_MS = {"causal_neox_bf16_1x8x4096x64": 31.984, "causal_neox_bf16_1x8x1024x64": 4.431,
                "causal_neox_bf16_1x8x2048x64": 8.717, "causal_neox_bf16_2x8x1024x64": 4.749,
                "causal_neox_bf16_4x8x1024x64": 9.057, "causal_gptj_bf16_1x8x512x64": 1.811}


def parse_args():
    from rotary_position_embedding_rope_amd import workloads as wl
    names = [w.name for w in wl.ATTENTION_WORKLOADS]
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=wl.HEADLINE.name, choices=names)
    ap.add_argument("--rope-steps", type=int, default=100)
    ap.add_argument("--rope-sets", type=int, default=10,
                    help="distinct Q/K buffer sets cycled by the rope_apply timing")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-comparators", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--bwd-steps", type=int, default=30)
    ap.add_argument("--only", choices=["all", "fused", "rope_apply", "decode", "backward", "copy"],
                    default="all",
                    help="restrict the timed kernels (for profiler runs); 'copy' runs only a "
                         "plain 256 MiB device copy, the calibration for HBM byte counters")
    ap.add_argument("--sweep", action="store_true",
                    help="also time every attention workload (printed to stderr)")
    ap.add_argument("--balance", action="store_true",
                    help="pass a workspace: balanced (split query tile) schedule")
    return ap.parse_args()


def kernel_source_digest(name: str) -> str:
    src = ROOT / "rotary_position_embedding_rope_amd" / "csrc" / name
    return hashlib.sha256(src.read_bytes()).hexdigest()[:16]


def recorded_traffic(profile: str, source: str):
    """HBM bytes per launch recorded from rocprofv3 FETCH_SIZE/WRITE_SIZE runs
    in profiles/<profile>, valid only while the kernel source is unchanged."""
    path = ROOT / "profiles" / profile
    if not path.exists():
        return None
    text = path.read_text()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_digest(source):
        return None
    return float(m_b.group(1))


def time_launches(torch, launch, steps, warmup, stream, rotate=None):
    """Warm up, then the timed region: `steps` launches back to back on
    `stream`, between device synchronisations, with one HIP event pair on the
    stream around them.  A second, untimed-for-value pass puts an event pair
    around each launch for the spread of single-launch durations.  Returns
    (wall ms per launch, event ms per launch in the timed region, sorted
    single-launch event ms)."""
    def run(i):
        if rotate:
            rotate(i)
        else:
            launch()

    for i in range(warmup):
        run(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for i in range(steps):
        run(i)
    b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    event_ms = a.elapsed_time(b)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (x, y) in enumerate(evs):
        x.record(stream)
        run(i)
        y.record(stream)
    torch.cuda.synchronize()
    durs = sorted(x.elapsed_time(y) for x, y in evs)
    return wall_ms / steps, event_ms / steps, durs


def bench_fused(torch, api, wl, w, steps, warmup, balance=False):
    dev = torch.device("cuda:0")
    tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    q, k, v = (torch.from_numpy(a).to(tdt).to(dev) for a in wl.attention_inputs(w))
    cos, sin = api.tables_build(w.base, w.rot, w.table_rows, device=dev)
    out = torch.empty_like(q)
    launch = api.prepare_flash_attn_fwd(q, k, v, out, cos, sin, w.q_off, w.k_off, w.rot, w.layout,
                                        w.causal, workspace="auto" if balance else None)
    stream = torch.cuda.current_stream(dev)
    ms_step, kernel_ms, durs = time_launches(torch, launch, steps, warmup, stream)
    return dict(q=q, k=k, v=v, cos=cos, sin=sin, out=out, ms_step=ms_step, kernel_ms=kernel_ms,
                p10=durs[len(durs) // 10], p50=durs[len(durs) // 2], p90=durs[(9 * len(durs)) // 10])


def bench_rope_apply(torch, api, wl, steps, sets, w=None):
    """rope_apply on a ragged batch (wl.RAGGED_ROPE unless given), cycling
    `sets` independent Q/K buffers so the last-level cache cannot hold them."""
    w = w or wl.RAGGED_ROPE
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    dev = torch.device("cuda:0")
    d = wl.rope_apply_inputs(w)
    q0 = torch.from_numpy(d["q"]).to(tdt).to(dev)
    k0 = torch.from_numpy(d["k"]).to(tdt).to(dev)
    pos = torch.from_numpy(d["positions"]).to(dev)
    cos, sin = api.tables_build(w.base, w.rot_dim, w.table_rows, device=dev)
    bufs = [(q0.clone(), k0.clone()) for _ in range(sets)]
    launches = [api.prepare_rope_apply(qb, kb, pos, cos, sin, w.rot_dim, w.layout) for qb, kb in bufs]
    stream = torch.cuda.current_stream(dev)
    ms_step, kernel_ms, durs = time_launches(torch, None, steps, sets, stream,
                                             rotate=lambda i: launches[i % sets]())
    nbytes = w.algorithmic_bytes()
    gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    set_mb = (q0.numel() + k0.numel()) * q0.element_size() / 2 ** 20
    traffic = (recorded_traffic("rope_apply_ragged_8192tok_traffic.md", "rope_apply.hip")
               if w is wl.RAGGED_ROPE else None)
    return {
        "workload": w.name, "value": round(gbs, 1), "unit": "GB/s",
        "ms_per_launch": round(kernel_ms, 5), "wall_ms_per_launch": round(ms_step, 5),
        "single_launch_p10_ms": round(durs[len(durs) // 10], 5),
        "single_launch_p90_ms": round(durs[(9 * len(durs)) // 10], 5),
        "buffer_sets": sets, "cycled_mib": round(set_mb * sets, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": nbytes},
    }


def bench_backward(torch, api, wl, steps, warmup):
    """The backward of the fused forward on the bench workload: one step is
    the two kernels of rope_flash_attn_bwd (Q and K rotated once into the
    workspace with the row sums dO.O, then the merged dK/dV and dQ launch),
    inputs and the forward's output and row statistics resident in HBM."""
    w = wl.HEADLINE
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(a).to(torch.bfloat16).to(dev) for a in wl.attention_inputs(w))
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 1000)
    dout = torch.randn(q.shape, generator=g, device=dev).to(torch.bfloat16)
    cos, sin = api.tables_build(w.base, w.rot, w.table_rows, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    o = api.flash_attn_fwd(q, k, v, cos, sin, w.q_off, w.k_off, w.rot, w.layout, w.causal, lse=lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    launch = api.prepare_flash_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, cos, sin, w.q_off, w.k_off,
                                        w.rot, w.layout, w.causal)
    stream = torch.cuda.current_stream(dev)
    ms_step, kernel_ms, durs = time_launches(torch, launch, steps, warmup, stream)
    flops = w.bwd_flops()
    tf = flops / (kernel_ms * 1e-3) / 1e12
    return {
        "workload": w.name, "value": round(tf, 2), "unit": "TFLOP/s",
        "ms_per_step": round(kernel_ms, 5), "wall_ms_per_step": round(ms_step, 5),
        "single_step_p10_ms": round(durs[len(durs) // 10], 5),
        "single_step_p90_ms": round(durs[(9 * len(durs)) // 10], 5),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(f"flash_bwd_bf16_{w.name}_traffic.md",
                                                 "flash_bwd_bf16.hip"),
                     "algorithmic_flops": flops},
    }


def bench_decode(torch, api, wl, steps, warmup):
    """The decode step of the continuous batch (wl.DECODE): HBM bytes the
    step must move over the time of one step (both kernels of the step)."""
    w = wl.DECODE
    dev = torch.device("cuda:0")
    d = wl.decode_inputs(w, with_cache=False)
    q, k_new, v_new = (torch.from_numpy(d[n]).to(torch.bfloat16).to(dev) for n in ("q", "k_new", "v_new"))
    lens = torch.from_numpy(d["lens"]).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    shape = (w.B, w.H_kv, w.S_max, w.D)
    k_cache = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    v_cache = torch.empty_like(k_cache)
    for b in range(w.B):   # one request at a time keeps the fp32 temporaries small
        k_cache[b] = torch.randn(shape[1:], generator=g, device=dev)
        v_cache[b] = torch.randn(shape[1:], generator=g, device=dev)
    cos, sin = api.tables_build(w.base, w.rot, w.S_max, device=dev)
    out = torch.empty_like(q)
    launch = api.prepare_decode_attn_fwd(q, k_new, v_new, k_cache, v_cache, lens, out, cos, sin,
                                         w.rot, w.layout)
    stream = torch.cuda.current_stream(dev)
    ms_step, kernel_ms, durs = time_launches(torch, launch, steps, warmup, stream)
    nbytes = w.algorithmic_bytes()
    gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    res = {
        "workload": w.name, "value": round(gbs, 1), "unit": "GB/s",
        "ms_per_step": round(kernel_ms, 5), "wall_ms_per_step": round(ms_step, 5),
        "single_step_p10_ms": round(durs[len(durs) // 10], 5),
        "single_step_p90_ms": round(durs[(9 * len(durs)) // 10], 5),
        "cached_tokens": int(d["lens"].astype("int64").sum()),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic(f"decode_bf16_{w.name}_traffic.md", "decode_bf16.hip"),
                     "algorithmic_bytes": nbytes},
    }
    del k_cache, v_cache
    return res


def comparators(torch, api, wl, w, r, steps, warmup):
    """Rotation-free kernel ("flash") and rope_apply-on-copies + flash
    ("unfused"), with peak extra device memory of one forward each."""
    dev = r["q"].device
    stream = torch.cuda.current_stream(dev)
    q, k, v = r["q"], r["k"], r["v"]
    out = torch.empty_like(q)
    flash = api.prepare_flash_attn_fwd(q, k, v, out, rot_dim=0, causal=w.causal,
                                       q_pos_offset=w.q_off, k_pos_offset=w.k_off)
    flash_ms = time_launches(torch, flash, steps, warmup, stream)[1]
    T = w.Sq

    def unfused():
        qt = q.permute(0, 2, 1, 3).reshape(w.B * T, w.H, w.D).contiguous()
        kt = k.permute(0, 2, 1, 3).reshape(w.B * w.Sk, w.H, w.D).contiguous()
        pq = torch.arange(w.q_off, w.q_off + T, dtype=torch.int32, device=dev).repeat(w.B)
        api.rope_apply(qt, None, pq, r["cos"], r["sin"], w.rot, w.layout)
        pk = torch.arange(w.k_off, w.k_off + w.Sk, dtype=torch.int32, device=dev).repeat(w.B)
        api.rope_apply(None, kt, pk, r["cos"], r["sin"], w.rot, w.layout)
        qr = qt.reshape(w.B, T, w.H, w.D).permute(0, 2, 1, 3).contiguous()
        kr = kt.reshape(w.B, w.Sk, w.H, w.D).permute(0, 2, 1, 3).contiguous()
        return api.flash_attn_fwd(qr, kr, v, rot_dim=0, causal=w.causal, q_pos_offset=w.q_off,
                                  k_pos_offset=w.k_off)

    def extra_mem(fn):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        res = fn()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev) - base
        del res
        return round(peak / 2 ** 20, 3)

    unfused_ms = time_launches(torch, unfused, max(steps // 4, 5), 3, stream)[0]
    fused_mem = extra_mem(lambda: api.flash_attn_fwd(q, k, v, r["cos"], r["sin"], w.q_off, w.k_off,
                                                     w.rot, w.layout, w.causal))
    unfused_mem = extra_mem(unfused)
    return {"fused_ms": round(r["kernel_ms"], 5), "flash_no_rope_ms": round(flash_ms, 5),
            "unfused_rope_then_flash_ms": round(unfused_ms, 5),
            "extra_mem_mib": {"fused": fused_mem, "unfused": unfused_mem}}


def copy_calibration(torch, steps, nbytes=256 * 2 ** 20):
    """A plain device-to-device copy of known size: the reference that scales
    the profiler's FETCH_SIZE / WRITE_SIZE readings to bytes."""
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_per_launch": nbytes, "launches": steps}


def cpu_baseline(wl, w, seconds):
    """The oracle on whole heads of the workload, cycled until `seconds` pass."""
    import numpy as np

    import oracle
    orc = oracle.load()
    q, k, v = wl.attention_inputs(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    pairs_per_head = w.visible_pairs() // (w.B * w.H)
    done, t0 = 0, time.perf_counter()
    while True:
        b, h = heads[done % len(heads)]
        sl = (slice(b, b + 1), slice(h, h + 1))
        g = h // (w.H // w.Hkv)   # the key/value head of query head h
        skv = (slice(b, b + 1), slice(g, g + 1))
        orc.attention(np.ascontiguousarray(q[sl]), np.ascontiguousarray(k[skv]),
                      np.ascontiguousarray(v[skv]), q_off=w.q_off, k_off=w.k_off, rot_dim=w.rot,
                      base=w.base, layout=w.layout, causal=w.causal)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    tflops = 4 * w.D * pairs_per_head * done / dt / 1e12
    return {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": orc.threads(), "kind": "oracle",
            "sample": f"{done} whole heads of {w.name} (fp64 C oracle with OpenMP; "
                      f"{dt:.1f} s, rope + dense masked softmax per head)"}


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py runs on exactly one GPU: this library has no multi-GPU path; "
                         "use --gpus 1\n")
        sys.exit(2)

    import torch

    from rotary_position_embedding_rope_amd import api
    from rotary_position_embedding_rope_amd import workloads as wl

    if args.only == "copy":
        print(json.dumps(copy_calibration(torch, args.steps)), flush=True)
        return
    w = {x.name: x for x in wl.ATTENTION_WORKLOADS}[args.workload]
    result = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
              "config": {"workload": w.name, "B": w.B, "H": w.H, "Sq": w.Sq, "Sk": w.Sk, "D": w.D,
                         "layout": w.layout, "rope_base": w.base, "rot_dim": w.rot,
                         "q_pos_offset": w.q_off, "k_pos_offset": w.k_off, "causal": w.causal,
                         "accumulate": "fp32", "device": torch.cuda.get_device_name(0)}}

    if args.only in ("all", "fused"):
        r = bench_fused(torch, api, wl, w, args.steps, args.warmup, balance=args.balance)
        flops = w.flops()
        value = flops / (r["ms_step"] * 1e-3) / 1e12
        achieved = flops / (r["kernel_ms"] * 1e-3) / 1e12
        result["value"] = round(value, 2)
        result["ms_per_step"] = round(r["ms_step"], 5)
        result["kernel_ms"] = {"mean": round(r["kernel_ms"], 5),
                               "single_launch_p10": round(r["p10"], 5),
                               "single_launch_p50": round(r["p50"], 5),
                               "single_launch_p90": round(r["p90"], 5)}
        result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                              "traffic": recorded_traffic(f"flash_fwd_bf16_{w.name}_traffic.md",
                                                          "flash_fwd_bf16.hip"),
                              "algorithmic_flops": flops}
        if w.name in PAGE_ROPE_MS:
            result["vs_baseline"] = round(PAGE_ROPE_MS[w.name] / r["ms_step"], 2)
        if args.only == "all" and not args.no_comparators:
            result["comparators"] = comparators(torch, api, wl, w, r, max(args.steps // 2, 10),
                                                args.warmup)
        for key in ("q", "k", "v", "out"):
            r.pop(key)
        del r
    if args.only in ("all", "fused"):
        # the same workload with fp16 storage (the fp16 matrix cores)
        wf = wl.HEADLINE_F16
        rf = bench_fused(torch, api, wl, wf, args.steps, args.warmup)
        tf = wf.flops() / (rf["kernel_ms"] * 1e-3) / 1e12
        result["fused_f16"] = {"workload": wf.name, "value": round(tf, 2), "unit": "TFLOP/s",
                               "kernel_ms": round(rf["kernel_ms"], 5),
                               "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        del rf
    if args.only in ("all", "rope_apply"):
        result["rope_apply"] = bench_rope_apply(torch, api, wl, args.rope_steps, args.rope_sets)
        # the same batch with fp16 storage (same bytes, same kernel family)
        rf = bench_rope_apply(torch, api, wl, args.rope_steps, args.rope_sets, w=wl.RAGGED_ROPE_F16)
        result["rope_apply"]["f16"] = {k: rf[k] for k in ("workload", "value", "unit", "ms_per_launch")}
        result["rope_apply"]["f16"]["frac"] = rf["roofline"]["frac"]
    if args.only in ("all", "backward"):
        result["backward"] = bench_backward(torch, api, wl, args.bwd_steps, max(args.warmup // 4, 3))
    if args.only in ("all", "decode"):
        result["decode"] = bench_decode(torch, api, wl, args.decode_steps, max(args.warmup // 4, 3))
    if args.sweep:
        for x in wl.ATTENTION_WORKLOADS:
            if x.dtype != "bf16":
                continue
            rx = bench_fused(torch, api, wl, x, args.steps, args.warmup, balance=args.balance)
            tf = x.flops() / (rx["kernel_ms"] * 1e-3) / 1e12
            sys.stderr.write(f"sweep {x.name:55s} kernel {rx['kernel_ms'] * 1e3:9.2f} us  "
                             f"{tf:8.1f} TFLOP/s  {tf / PEAK_BF16_TFLOPS * 100:5.1f}% of peak\n")
            del rx
    torch.cuda.synchronize()
    if not args.no_cpu_baseline and args.only == "all":
        result["cpu_baseline"] = cpu_baseline(wl, w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
