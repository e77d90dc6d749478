#!/usr/bin/env python3
"""One-GPU benchmark: fused RoPE + causal attention forward (TFLOP/s against
the bf16 matrix-core peak) and the standalone ragged RoPE op (HBM GB/s).

A step is one fused forward over the workload (default: 1x8x4096x64 bf16,
NeoX RoPE base 10000, causal); inputs are resident in HBM before timing.
W untimed warmup steps, then exactly K timed steps between two device
synchronisations; rank 0 prints ONE JSON line.

  value          whole-job TFLOP/s = algorithmic flops / wall time per step
                 (algorithmic flops: 4*D per query/key pair the mask allows);
                 the K steps run back to back between two synchronisations,
                 after W warmup steps that follow HEADLINE_PREWARM_S seconds
                 of back-to-back launches (the sustained state: the GPU
                 leaves its idle power state only after ~20-25 ms of work);
                 kernel_ms.cold_mean is the same W/K measurement taken first,
                 right after setting up the inputs
  roofline       the fused kernel: flops per launch / mean launch duration,
                 from one HIP event pair on the launch stream around the K
                 launches, against 2500 TFLOP/s
  max_abs_err    the timed kernel's output against the fp64 oracle, in the
                 same run (every element)
  clock          the per-XCD shader clocks amd-smi reports while the bench
                 workload runs back to back (the 2500 TFLOP/s peak assumes
                 2400 MHz)
  loop_ceiling   the attention inner step alone (scores, exponentials, row
                 sums, P V on LDS-resident tiles, no global traffic, rotation
                 or barriers; librope_calib.so) in every built variant; its
                 best rate per head dim is what a kernel running that step
                 can reach here, and each bf16 forward roofline carries
                 frac_of_loop_ceiling beside frac.  Measured before the
                 forward, so the forward's warmup and timed steps start on a
                 GPU already at its sustained clock
  configs        the other benchmark workloads, each timed the same way
                 (after PREWARM_S seconds of its own launches, which let the
                 shader clock settle) with its own roofline fraction and
                 same-run oracle error:
                 the fp32 parity case, the page-shaped 1x8x512x64 GPT-J case,
                 the 1x8xSx64 NeoX sweep, the ragged rope_apply batch (with
                 ceiling_gbs: librope_calib.so's in-place stream of the same
                 rotated spans, read and written once, and the same bytes
                 contiguous) and the 2048 x 16384 chunked prefill with its query
                 offset (plus its 8-key/value-head variant); the six
                 page-shaped workloads also carry the comparators below
  comparators    context rows mirroring "RoPE + PoPE Attention Kernels"'
                 benchmark table: the same kernel without rotation ("flash"),
                 and rope_apply on copies of Q/K followed by it ("unfused"),
                 with peak extra device memory of one forward each
  cpu_baseline   the fp64 CPU oracle on the same workload (whole heads),
                 timed on this host's cores; single-thread and rope_apply
                 oracle rates beside it
  backward, decode   the backward step and the decode step (context); the
                 decode step carries ceiling_gbs, librope_calib.so's
                 read-only stream over the same number of bytes
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
PEAK_F32_VALU_TFLOPS = 157.3   # MI355X fp32 vector peak, published (the fp32 kernel's units)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth, published
# "RoPE + PoPE Attention Kernels", median runtime table: rope (rotate, then
# flash) on an unnamed CUDA GPU -- context, not a target.
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
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config list")
    ap.add_argument("--no-clock", action="store_true", help="skip the amd-smi shader-clock sample")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--bwd-steps", type=int, default=30)
    ap.add_argument("--only", choices=["all", "fused", "rope_apply", "decode", "backward", "copy", "ceilings"],
                    default="all",
                    help="restrict the timed kernels (for profiler runs): 'fused' times only "
                         "--workload; 'copy' runs only a plain 256 MiB device copy, the "
                         "calibration for HBM byte counters; 'ceilings' only the measurement "
                         "kernels (attention inner step, in-place stream)")
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


def fused_traffic(w):
    """Recorded HBM bytes per launch of the fused forward kernel that runs w
    (head dim 128 in 16-bit storage: flash_fwd_pp.hip, else
    flash_fwd_bf16.hip), or None."""
    if w.dtype == "f32":
        return None
    if w.D == 128:
        return recorded_traffic(f"flash_fwd_pp_{w.name}_traffic.md", "flash_fwd_pp.hip")
    return recorded_traffic(f"flash_fwd_bf16_{w.name}_traffic.md", "flash_fwd_bf16.hip")


# Seconds of a measurement's own launches, back to back, before its W warmup
# steps.  The GPU leaves its idle power state only after ~20-25 ms of
# sustained work and drops back within ~20-100 ms of idle: the head-dim-64
# forward takes 41.0-41.4 us per launch when timed right after an idle
# period and 35.3-35.7 us once the GPU has been busy for 25 ms or more.
# Measurements here are of the sustained state a running job sees; the
# headline also reports its first, cold measurement (kernel_ms.cold_*).
PREWARM_S = 0.1
HEADLINE_PREWARM_S = 0.2


def time_launches(torch, launch, steps, warmup, stream, rotate=None, prewarm_s=0.0):
    """Warm up, then the timed region: `steps` launches back to back on
    `stream`, between device synchronisations, with one HIP event pair on the
    stream around them.  A second, untimed-for-value pass puts an event pair
    around each launch for the spread of single-launch durations.  Returns
    (wall ms per launch, event ms per launch in the timed region, sorted
    single-launch event ms).

    With prewarm_s > 0 the launches first run back to back for that long
    (PREWARM_S): the chunked prefill's first 25 launches after a memory-bound
    phase averaged 0.60 ms, 0.52-0.53 ms once settled, with or without cache
    reuse between launches."""
    def run(i):
        if rotate:
            rotate(i)
        else:
            launch()

    if prewarm_s > 0:
        t_end = time.perf_counter() + prewarm_s
        i = 0
        while time.perf_counter() < t_end:
            for _ in range(8):
                run(i)
                i += 1
            torch.cuda.synchronize()
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


def _tdt(torch, dtype):
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]


CLOCK_OFF = False   # --no-clock


def under_profiler() -> bool:
    """True inside rocprofv3, whose preloaded tool would also load into (and
    initialise the GPU in) any child process bench.py starts."""
    return any(k.startswith("ROCPROF") for k in os.environ) or "rocprofiler" in os.environ.get("LD_PRELOAD", "")


def sample_clock(torch, launch, kernel_ms, busy_s=3.0, delay_s=1.0):
    """The shader clock under this workload: `amd-smi metric --clock` run as
    a child process `delay_s` into `busy_s` seconds of back-to-back launches
    (per-XCD gfx clocks, MHz).  None when amd-smi is missing or fails, with
    --no-clock, and under a profiler (no child process is started there)."""
    import shutil
    import subprocess
    import threading
    if CLOCK_OFF or under_profiler():
        return None
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    got = {}

    def probe():
        time.sleep(delay_s)
        try:
            r = subprocess.run([exe, "metric", "--clock", "--json"], capture_output=True, text=True, timeout=30)
            d = json.loads(r.stdout)
            clocks = (d["gpu_data"] if isinstance(d, dict) else d)[0]["clock"]
            got["gfx_mhz"] = [clocks[k]["clk"]["value"] for k in sorted(clocks) if k.startswith("gfx_")]
        except (OSError, ValueError, KeyError, IndexError, TypeError, subprocess.SubprocessError):
            pass

    t = threading.Thread(target=probe)
    t.start()
    t0 = time.perf_counter()
    n = max(1, int(busy_s * 1e3 / kernel_ms))
    for i in range(n):
        launch()
        if i % 256 == 255 and time.perf_counter() - t0 > busy_s:
            break
    torch.cuda.synchronize()
    t.join()
    if not got.get("gfx_mhz"):
        return None
    return {"gfx_mhz": got["gfx_mhz"], "max_mhz": 2400,
            "sampled": f"amd-smi metric --clock, {delay_s:.1f} s into back-to-back launches of this workload"}


def bench_fused(torch, api, wl, w, steps, warmup, prewarm_s=0.0):
    dev = torch.device("cuda:0")
    arrays = wl.attention_inputs(w)
    q, k, v = (torch.from_numpy(a).to(_tdt(torch, w.dtype)).to(dev) for a in arrays)
    cos, sin = api.tables_build(w.base, w.rot, w.table_rows, device=dev)
    out = torch.empty_like(q)
    launch = api.prepare_flash_attn_fwd(q, k, v, out, cos, sin, w.q_off, w.k_off, w.rot, w.layout,
                                        w.causal)   # the library's default (cached) workspace
    stream = torch.cuda.current_stream(dev)
    ms_step, kernel_ms, durs = time_launches(torch, launch, steps, warmup, stream, prewarm_s=prewarm_s)
    return dict(arrays=arrays, q=q, k=k, v=v, cos=cos, sin=sin, out=out, launch=launch, ms_step=ms_step,
                kernel_ms=kernel_ms, p10=durs[len(durs) // 10], p50=durs[len(durs) // 2],
                p90=durs[(9 * len(durs)) // 10])


def device_label(torch):
    props = torch.cuda.get_device_properties(0)
    name = torch.cuda.get_device_name(0) or "AMD GPU"
    return f"{name} ({getattr(props, 'gcnArchName', '?')}, {props.multi_processor_count} CUs)"


def sample_rows(w, n_random=40, seed=0):
    """(b, h, i) rows for a same-run spot check: tile edges of three heads and
    random rows."""
    import numpy as np
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(w.B):
        for h in sorted({0, w.H - 1, w.H // 2}):
            for i in (0, 1, 31, 32, 63, 64, 127, 128, 255, 256, w.Sq // 2, w.Sq - 2, w.Sq - 1):
                if 0 <= i < w.Sq:
                    rows.add((b, h, i))
    for _ in range(n_random):
        rows.add((int(rng.integers(w.B)), int(rng.integers(w.H)), int(rng.integers(w.Sq))))
    return sorted(rows)


def fused_error(orc, w, r, full_pairs_limit=2 * 10 ** 8):
    """Max |GPU - oracle| over every output element (sampled rows for the
    largest workloads), with what was compared."""
    import numpy as np
    q, k, v = r["arrays"]
    got = r["out"].float().cpu().numpy().astype(np.float64)
    kw = dict(q_off=w.q_off, k_off=w.k_off, rot_dim=w.rot, base=w.base, layout=w.layout,
              causal=w.causal)
    if w.visible_pairs() <= full_pairs_limit:
        want = orc.attention(q, k, v, **kw)
        return float(np.abs(got - want).max()), "every element"
    rows = sample_rows(w)
    want = orc.attention_rows(q, k, v, rows, **kw)
    g = np.stack([got[b, h, i] for b, h, i in rows])
    return float(np.abs(g - want).max()), f"{len(rows)} sampled rows"


def fused_entry(torch, api, wl, orc, w, config, steps, warmup, comparators_too=False, clock=False):
    r = bench_fused(torch, api, wl, w, steps, warmup, prewarm_s=PREWARM_S)
    flops = w.flops()
    tf = flops / (r["kernel_ms"] * 1e-3) / 1e12
    f32 = w.dtype == "f32"
    peak = PEAK_F32_VALU_TFLOPS if f32 else PEAK_BF16_TFLOPS
    err, checked = fused_error(orc, w, r)
    e = {"config": config, "workload": w.name, "shape": w.label(), "dtype": w.dtype,
         "ms": round(r["kernel_ms"], 5), "wall_ms": round(r["ms_step"], 5),
         "single_launch_p10_ms": round(r["p10"], 5), "single_launch_p90_ms": round(r["p90"], 5),
         "value": round(tf, 2), "unit": "TFLOP/s",
         "roofline": {"bound": "alu" if f32 else "mfma", "achieved": round(tf, 2), "peak": peak,
                      "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                      "traffic": fused_traffic(w),
                      "algorithmic_flops": flops},
         "max_abs_err": err, "err_checked": checked, "tolerance": 1e-5 if f32 else 2e-2}
    if comparators_too:
        e["comparators"] = comparators(torch, api, wl, w, r, max(steps // 2, 10), warmup)
    if clock:
        e["clock"] = sample_clock(torch, r["launch"], r["kernel_ms"])
    return e


def bench_rope_apply(torch, api, wl, steps, sets, orc=None, w=None):
    """rope_apply on a ragged batch (wl.RAGGED_ROPE unless given), cycling
    `sets` independent Q/K buffers so the last-level cache cannot hold them;
    with `orc`, a fresh copy is rotated once more and compared with the
    oracle (every element)."""
    import numpy as np
    w = w or wl.RAGGED_ROPE
    tdt = _tdt(torch, w.dtype)
    dev = torch.device("cuda:0")
    d = wl.rope_apply_inputs(w)
    q0 = torch.from_numpy(d["q"]).to(tdt).to(dev)
    k0 = torch.from_numpy(d["k"]).to(tdt).to(dev)
    pos = torch.from_numpy(d["positions"]).to(dev)
    cos, sin = api.tables_build(w.base, w.rot_dim, w.table_rows, device=dev)
    bufs = [(q0.clone(), k0.clone()) for _ in range(sets)]
    launches = [api.prepare_rope_apply(qb, kb, pos, cos, sin, w.rot_dim, w.layout) for qb, kb in bufs]
    stream = torch.cuda.current_stream(dev)
    ms_step, kernel_ms, durs = time_launches(torch, None, steps, sets, stream, prewarm_s=PREWARM_S,
                                             rotate=lambda i: launches[i % sets]())
    nbytes = w.algorithmic_bytes()
    gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    set_mb = (q0.numel() + k0.numel()) * q0.element_size() / 2 ** 20
    traffic = (recorded_traffic("rope_apply_ragged_8192tok_traffic.md", "rope_apply.hip")
               if w is wl.RAGGED_ROPE else None)
    res = {
        "config": 4, "workload": w.name, "value": round(gbs, 1), "unit": "GB/s",
        "ms_per_launch": round(kernel_ms, 5), "wall_ms_per_launch": round(ms_step, 5),
        "single_launch_p10_ms": round(durs[len(durs) // 10], 5),
        "single_launch_p90_ms": round(durs[(9 * len(durs)) // 10], 5),
        "buffer_sets": sets, "cycled_mib": round(set_mb * sets, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": nbytes},
    }
    del bufs, launches
    if orc is not None:
        qf, kf = q0.clone(), k0.clone()
        api.rope_apply(qf, kf, pos, cos, sin, w.rot_dim, w.layout)
        torch.cuda.synchronize()
        err = 0.0
        for x_in, x_out in ((d["q"], qf), (d["k"], kf)):
            p = np.broadcast_to(d["positions"][:, None], x_in.shape[:2])
            want = orc.rope(x_in, p, base=w.base, rot_dim=w.rot_dim, layout=w.layout)
            got = x_out.float().cpu().numpy().astype(np.float64)
            err = max(err, float(np.abs(got - want).max()))
        res["max_abs_err"] = err
        res["err_checked"] = "every element"
    return res


def streaming_ceiling(torch, w, steps, sets, row_vecs=None, span_vecs=None):
    """The in-place stream of librope_calib.so over rope_apply's footprint on
    workload w: each 16-byte vector of the rotated span of every head row
    read and written back once (row_vecs / span_vecs: the head row and its
    rotated span in vectors; equal values stream a contiguous range of the
    same size), cycling `sets` buffers as the rope_apply timing does.  GB/s
    of read + written bytes: what a plain kernel moving the same bytes the
    same way reaches on this GPU."""
    from rotary_position_embedding_rope_amd import calib
    dev = torch.device("cuda:0")
    esz = 2 if w.dtype in ("bf16", "f16") else 4
    row = row_vecs or w.D * esz // 16
    span = span_vecs or w.rot_dim * esz // 16
    n_vec = w.n_tokens * (w.H_q + w.H_kv) * (w.rot_dim * esz // 16)
    words = -(-n_vec // span) * row * 4
    bufs = [torch.zeros(words, dtype=torch.int32, device=dev) for _ in range(sets)]
    stream = torch.cuda.current_stream(dev)
    _, ms, _ = time_launches(torch, None, steps, sets, stream, prewarm_s=PREWARM_S,
                             rotate=lambda i: calib.stream_inplace(bufs[i % sets], n_vec, row, span, stream))
    del bufs
    return round(32 * n_vec / (ms * 1e-3) / 1e9, 1)


def read_ceiling(torch, nbytes, steps):
    """librope_calib.so's read-only stream over `nbytes` (one buffer, larger
    than the 256 MB last-level cache at the decode step's size): GB/s of a
    plain kernel reading that many bytes once, the decode step's ceiling."""
    from rotary_position_embedding_rope_amd import calib
    dev = torch.device("cuda:0")
    n_vec = nbytes // 16
    buf = torch.zeros(4 * n_vec, dtype=torch.int32, device=dev)
    hit = torch.zeros(1, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    _, ms, _ = time_launches(torch, lambda: calib.stream_read(buf, n_vec, 0x7A5C3E1D, hit, stream), steps,
                             max(steps // 5, 2), stream, prewarm_s=PREWARM_S)
    del buf
    return round(16 * n_vec / (ms * 1e-3) / 1e9, 1)


def loop_ceilings(torch, iters=512, launches=5):
    """Every variant of the attention inner-step kernel of librope_calib.so
    (scores, exponentials, row sums, P V on LDS-resident tiles; no global
    traffic, rotation or barriers), one workgroup per CU, timed with a HIP
    event pair around `launches` launches: TFLOP/s, fraction of the bf16
    peak and ns per 32-row x 64-key wave tile per SIMD.  The best rate per
    head dim bounds what any kernel running this step reaches here."""
    import numpy as np
    from rotary_position_embedding_rope_amd import calib
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    wgs = torch.cuda.get_device_properties(dev).multi_processor_count
    rng = np.random.default_rng(7)
    rows, best = [], {}
    for D, wps, pipe in calib.LOOP_VARIANTS:
        n_k, n_v, n_q, n_out, _ = calib.loop_shapes(D, wps, wgs)
        kt, vt, qt = (torch.from_numpy(rng.normal(0, 0.25, n).astype(np.float32)).to(torch.bfloat16).to(dev)
                      for n in (n_k, n_v, n_q))
        out = torch.empty(n_out, dtype=torch.float32, device=dev)

        def launch():
            calib.attn_loop(D, wps, pipe, iters, wgs, kt, vt, qt, out, stream=stream)

        _, ms, _ = time_launches(torch, launch, launches, 1, stream, prewarm_s=PREWARM_S / 2)
        flops = 4.0 * 64 * 32 * D * iters * 4 * wps * wgs
        tf = flops / (ms * 1e-3) / 1e12
        ns_tile = ms * 1e6 / (iters * wps)
        rows.append({"head_dim": D, "waves_per_simd": wps, "pipelined": bool(pipe), "tflops": round(tf, 1),
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "ns_per_wave_tile_per_simd": round(ns_tile, 1)})
        best[D] = max(best.get(D, 0.0), tf)
        del kt, vt, qt, out
    return {"variants": rows, "best_tflops": {str(d): round(t, 1) for d, t in best.items()},
            "iters": iters, "workgroups": wgs}


def bench_backward(torch, api, wl, orc, steps, warmup):
    """The backward of the fused forward on the bench workload: one step is
    the kernels of rope_flash_attn_bwd (Q and K rotated once into the
    workspace with the row sums dO.O, then the merged dK/dV and dQ launch),
    inputs and the forward's output and row statistics resident in HBM."""
    import numpy as np
    w = wl.HEADLINE
    dev = torch.device("cuda:0")
    arrays = wl.attention_inputs(w)
    q, k, v = (torch.from_numpy(a).to(torch.bfloat16).to(dev) for a in arrays)
    dout_np = wl.round_to(np.random.default_rng(w.seed + 1000).standard_normal(arrays[0].shape), "bf16")
    dout = torch.from_numpy(dout_np).to(torch.bfloat16).to(dev)
    cos, sin = api.tables_build(w.base, w.rot, w.table_rows, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    o = api.flash_attn_fwd(q, k, v, cos, sin, w.q_off, w.k_off, w.rot, w.layout, w.causal, lse=lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    launch = api.prepare_flash_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, cos, sin, w.q_off, w.k_off,
                                        w.rot, w.layout, w.causal)
    stream = torch.cuda.current_stream(dev)
    ms_step, kernel_ms, durs = time_launches(torch, launch, steps, warmup, stream, prewarm_s=PREWARM_S)
    flops = w.bwd_flops()
    tf = flops / (kernel_ms * 1e-3) / 1e12
    res = {
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
    if orc is not None:
        refs = orc.attention_bwd(*arrays, dout_np, q_off=w.q_off, k_off=w.k_off, base=w.base,
                                 layout=w.layout)
        rel = {}
        for name, g, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
            got = g.float().cpu().numpy().astype(np.float64)
            rel[name] = round(float(np.abs(got - ref).max() / np.abs(ref).max()), 6)
        res["max_rel_err"] = rel
        res["err_checked"] = "every element (max |err| / max |ref| per tensor; bar 2e-2)"
    return res


def bench_decode(torch, api, wl, orc, steps, warmup):
    """The decode step of the continuous batch (wl.DECODE): HBM bytes the
    step must move over the time of one step (both kernels of the step)."""
    import numpy as np
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
    ms_step, kernel_ms, durs = time_launches(torch, launch, steps, warmup, stream, prewarm_s=PREWARM_S)
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
    if orc is not None:
        # one more step on the resident caches: each launch appends at the same
        # rows, so the cache rows below L are the seeded values; requests
        # 0, 7 and 15 against the oracle (cache rows taken as rotated keys)
        api.decode_attn_fwd(q, k_new, v_new, k_cache, v_cache, lens, cos, sin, w.rot, w.layout, out=out)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        err = 0.0
        for b in (0, 7, 15):
            L = int(d["lens"][b])
            kc = k_cache[b, :, :L + 1].float().cpu().numpy().astype(np.float64)
            vc = v_cache[b, :, :L + 1].float().cpu().numpy().astype(np.float64)
            qr = orc.rope(d["q"][b][:, None, :], [L], base=w.base, layout=w.layout)
            want = orc.attention(qr[None], kc[None], vc[None], q_off=L, k_off=0, rot_dim=0,
                                 causal=True)[0, :, 0, :]
            err = max(err, float(np.abs(got[b] - want).max()))
        res["max_abs_err"] = err
        res["err_checked"] = "every output row of requests 0, 7 and 15"
    del k_cache, v_cache
    res["ceiling_gbs"] = read_ceiling(torch, nbytes, steps)
    res["frac_of_ceiling"] = round(gbs / res["ceiling_gbs"], 4)
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
        kt = k.permute(0, 2, 1, 3).reshape(w.B * w.Sk, w.Hkv, w.D).contiguous()
        pq = torch.arange(w.q_off, w.q_off + T, dtype=torch.int32, device=dev).repeat(w.B)
        api.rope_apply(qt, None, pq, r["cos"], r["sin"], w.rot, w.layout)
        pk = torch.arange(w.k_off, w.k_off + w.Sk, dtype=torch.int32, device=dev).repeat(w.B)
        api.rope_apply(None, kt, pk, r["cos"], r["sin"], w.rot, w.layout)
        qr = qt.reshape(w.B, T, w.H, w.D).permute(0, 2, 1, 3).contiguous()
        kr = kt.reshape(w.B, w.Sk, w.Hkv, w.D).permute(0, 2, 1, 3).contiguous()
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
    """The oracle on whole heads of the workload, cycled until `seconds` pass;
    beside it the oracle's rope on the ragged batch (GB/s) and single-thread
    times of the fp32 and the 1x8x512x64 cases."""
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
    threads = orc.threads()
    res = {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{done} whole heads of {w.name} (fp64 C oracle with OpenMP; "
                     f"{dt:.1f} s, rope + dense masked softmax per head)"}

    def rope_rate():
        rw = wl.RAGGED_ROPE
        d = wl.rope_apply_inputs(rw)
        t = time.perf_counter()
        for x in (d["q"], d["k"]):
            orc.rope(x, np.broadcast_to(d["positions"][:, None], x.shape[:2]), base=rw.base,
                     rot_dim=rw.rot_dim, layout=rw.layout)
        return rw.algorithmic_bytes() / (time.perf_counter() - t) / 1e9

    def attn_ms(x):
        a = wl.attention_inputs(x)
        t = time.perf_counter()
        orc.attention(*a, q_off=x.q_off, k_off=x.k_off, rot_dim=x.rot, base=x.base, layout=x.layout,
                      causal=x.causal)
        return (time.perf_counter() - t) * 1e3

    res["rope_apply"] = {"value": round(rope_rate(), 3), "unit": "GB/s", "cores": threads,
                         "sample": f"the whole {wl.RAGGED_ROPE.name} batch"}
    orc.set_threads(1)
    try:
        res["single_thread"] = {
            "rope_apply_gbs": round(rope_rate(), 3),
            wl.TINY_F32.name + "_ms": round(attn_ms(wl.TINY_F32), 3),
            wl.SMALL_BF16.name + "_ms": round(attn_ms(wl.SMALL_BF16), 3),
        }
    finally:
        orc.set_threads(threads)
    return res


def main():
    args = parse_args()
    global CLOCK_OFF
    CLOCK_OFF = args.no_clock
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
    if args.only == "ceilings":
        out = {"loop_ceiling": loop_ceilings(torch),
               "stream_half_row_gbs": streaming_ceiling(torch, wl.RAGGED_ROPE, args.rope_steps, args.rope_sets),
               "stream_contiguous_gbs": streaming_ceiling(torch, wl.RAGGED_ROPE, args.rope_steps, args.rope_sets,
                                                          row_vecs=8, span_vecs=8),
               "stream_read_gbs": read_ceiling(torch, wl.DECODE.algorithmic_bytes(), args.decode_steps)}
        print(json.dumps(out), flush=True)
        return
    orc = None
    if args.only == "all":
        import oracle
        orc = oracle.load()
    w = {x.name: x for x in wl.ATTENTION_WORKLOADS}[args.workload]
    result = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
              "config": {"workload": w.name, "B": w.B, "H": w.H, "Sq": w.Sq, "Sk": w.Sk, "D": w.D,
                         "layout": w.layout, "rope_base": w.base, "rot_dim": w.rot,
                         "q_pos_offset": w.q_off, "k_pos_offset": w.k_off, "causal": w.causal,
                         "accumulate": "fp32", "device": device_label(torch)}}

    if args.only == "all":
        # the measurement kernels run first: besides giving the ceilings, they
        # bring the GPU to the clock it holds under sustained work before the
        # forward's own W warmup and K timed steps
        result["loop_ceiling"] = loop_ceilings(torch)
    if args.only in ("all", "fused"):
        # first the cold measurement (W warmup and K timed launches right
        # after setting up the inputs), reported beside; then the same W and
        # K after HEADLINE_PREWARM_S of back-to-back launches: the value
        r = bench_fused(torch, api, wl, w, args.steps, args.warmup)
        cold_ms, cold_kernel_ms = r["ms_step"], r["kernel_ms"]
        stream = torch.cuda.current_stream(torch.device("cuda:0"))
        ms_step, kernel_ms, durs = time_launches(torch, r["launch"], args.steps, args.warmup, stream,
                                                 prewarm_s=HEADLINE_PREWARM_S)
        r.update(ms_step=ms_step, kernel_ms=kernel_ms, p10=durs[len(durs) // 10], p50=durs[len(durs) // 2],
                 p90=durs[(9 * len(durs)) // 10])
        flops = w.flops()
        value = flops / (r["ms_step"] * 1e-3) / 1e12
        achieved = flops / (r["kernel_ms"] * 1e-3) / 1e12
        result["value"] = round(value, 2)
        result["ms_per_step"] = round(r["ms_step"], 5)
        result["kernel_ms"] = {"mean": round(r["kernel_ms"], 5),
                               "single_launch_p10": round(r["p10"], 5),
                               "single_launch_p50": round(r["p50"], 5),
                               "single_launch_p90": round(r["p90"], 5),
                               "cold_mean": round(cold_kernel_ms, 5), "cold_wall_per_step": round(cold_ms, 5),
                               "prewarm_s": HEADLINE_PREWARM_S}
        result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                              "traffic": fused_traffic(w),
                              "algorithmic_flops": flops}
        if w.name in PAGE_ROPE_MS:
            result["vs_baseline"] = round(PAGE_ROPE_MS[w.name] / r["ms_step"], 2)
        if args.only == "all":
            result["clock"] = sample_clock(torch, r["launch"], r["kernel_ms"])
            best = result["loop_ceiling"]["best_tflops"].get(str(w.D))
            if best and w.dtype != "f32":
                result["roofline"]["loop_ceiling_tflops"] = best
                result["roofline"]["frac_of_loop_ceiling"] = round(achieved / best, 4)
        if orc is not None:
            result["max_abs_err"], result["err_checked"] = fused_error(orc, w, r)
        del r
    if args.only == "all" and not args.no_configs:
        configs = [fused_entry(torch, api, wl, orc, wl.TINY_F32, 1, args.steps, args.warmup),
                   fused_entry(torch, api, wl, orc, wl.SMALL_BF16, 2, args.steps, args.warmup, True)]
        for x in wl.SWEEP_BF16:
            configs.append(fused_entry(torch, api, wl, orc, x, 3, args.steps, args.warmup, True))
        ra = bench_rope_apply(torch, api, wl, args.rope_steps, args.rope_sets, orc)
        ra["ceiling_gbs"] = streaming_ceiling(torch, wl.RAGGED_ROPE, args.rope_steps, args.rope_sets)
        ra["ceiling_contiguous_gbs"] = streaming_ceiling(torch, wl.RAGGED_ROPE, args.rope_steps, args.rope_sets,
                                                         row_vecs=8, span_vecs=8)
        ra["frac_of_ceiling"] = round(ra["value"] / ra["ceiling_gbs"], 4)
        configs.append(ra)
        configs.append(fused_entry(torch, api, wl, orc, wl.PREFILL_OFFSET, 5, args.steps, args.warmup, clock=True))
        configs.append(fused_entry(torch, api, wl, orc, wl.PREFILL_GQA, "5-gqa", args.steps, args.warmup))
        best = result.get("loop_ceiling", {}).get("best_tflops", {})
        for e in configs:
            if e.get("unit") == "TFLOP/s" and e.get("dtype") != "f32":
                d = {x.name: x for x in wl.ATTENTION_WORKLOADS}.get(e["workload"])
                ceil = best.get(str(d.D)) if d is not None else None
                if ceil:
                    e["roofline"]["loop_ceiling_tflops"] = ceil
                    e["roofline"]["frac_of_loop_ceiling"] = round(e["value"] / ceil, 4)
        result["configs"] = configs
        # the headline workload with fp16 storage (the fp16 matrix cores)
        wf = wl.HEADLINE_F16
        rf = bench_fused(torch, api, wl, wf, args.steps, args.warmup, prewarm_s=PREWARM_S)
        tf = wf.flops() / (rf["kernel_ms"] * 1e-3) / 1e12
        result["fused_f16"] = {"workload": wf.name, "value": round(tf, 2), "unit": "TFLOP/s",
                               "kernel_ms": round(rf["kernel_ms"], 5),
                               "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                               "max_abs_err": fused_error(orc, wf, rf)[0]}
        del rf
    if args.only == "rope_apply" or (args.only == "all" and args.no_configs):
        result["rope_apply"] = bench_rope_apply(torch, api, wl, args.rope_steps, args.rope_sets, orc)
    if args.only == "all":
        # the same batch with fp16 storage (same bytes, same kernel family)
        rf = bench_rope_apply(torch, api, wl, args.rope_steps, args.rope_sets, w=wl.RAGGED_ROPE_F16)
        result["rope_apply_f16"] = {k: rf[k] for k in ("workload", "value", "unit", "ms_per_launch")}
        result["rope_apply_f16"]["frac"] = rf["roofline"]["frac"]
    if args.only in ("all", "backward"):
        result["backward"] = bench_backward(torch, api, wl, orc, args.bwd_steps, max(args.warmup // 4, 3))
    if args.only in ("all", "decode"):
        result["decode"] = bench_decode(torch, api, wl, orc, args.decode_steps, max(args.warmup // 4, 3))
    torch.cuda.synchronize()
    if not args.no_cpu_baseline and args.only == "all":
        result["cpu_baseline"] = cpu_baseline(wl, w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
