"""Decode-step benchmark: steps/s and achieved HBM bandwidth of the streaming decode step.

Default workload: the 28-layer talker-family stack at m=1 (hidden 2048, 16 q / 8 kv heads x 128,
SwiGLU 6144, 2048-slot cache), float32 with bf16-rounded synthetic weights, run over positions
0..K-1 of a fresh stream (K = 2048 covers the whole cache).  Inputs, weights and state are resident
in HBM before the timed region; each step's input row is a slice of a pre-drawn device tensor.

One JSON line on stdout:
  value        steps/s over the K timed steps (one step = the whole layer stack for one position)
  roofline     the dominant kernel (the FFN gate/up GEMV with its fused norm and SwiGLU): its
               algorithmic bytes per launch / its mean launch time, from HIP event pairs that each
               launch of the profiled eager steps stamps around the kernel's own execution
  cpu_baseline the CPU oracle on a bounded sample of the same run (first positions), host cores
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--config", type=int, default=4, help="workload id (4: the m=1 talker)")
    ap.add_argument("--eager", action="store_true", help="launch kernels one by one, no graph")
    ap.add_argument("--profile-steps", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-timed", action="store_true",
                    help="warmup + timed steps only (for running under a profiler)")
    ap.add_argument("--prefill-block", type=int, default=8,
                    help="rows per sdec_prefill call in the prefill measurement (0: skip it)")
    ap.add_argument("--prefill-blocks", type=int, default=32,
                    help="timed prefill calls, positions from 0")
    ap.add_argument("--no-variant", action="store_true",
                    help="skip the FlowLM-variant measurement (workload 6)")
    ap.add_argument("--no-rvq", action="store_true",
                    help="skip the split-RVQ measurement (64 frames, 8 codebooks of 2048 bins)")
    ap.add_argument("--no-seanet", action="store_true",
                    help="skip the streaming SEANet-decoder measurement")
    ap.add_argument("--no-pocket", action="store_true",
                    help="skip the Pocket-style codec frame timing")
    ap.add_argument("--fixed-positions", type=int, default=1,
                    help="also time the step at fixed positions 0, R/2 and R-1 (0: skip)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (codec stacks 1-3, the m=8 talker 5)")
    ap.add_argument("--config-cpu-seconds", type=float, default=3.0,
                    help="budget of each other workload's oracle sample (0: none)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes three times (the "
                         "known-size kernel that calibrates HBM byte counters)")
    return ap.parse_args()


def layer_weight_bytes(cfg):
    d, f, qw, kw = cfg.d_model, cfg.d_ff, cfg.q_width, cfg.kv_width
    mats = (qw + 2 * kw) * d + d * qw + (2 if cfg.ffn == 0 else 1) * f * d + d * f
    vecs = 2 * d * (2 if cfg.norm == 1 else 1) + (2 * cfg.head_dim if cfg.qk_norm else 0) \
        + (2 * d if cfg.layer_scale else 0)
    return 4 * (mats + vecs)


def step_bytes(cfg, pos, ring, window):
    """Algorithmic HBM bytes of one step at `pos` (each weight, live K/V row and position-ring
    word read once, the new K/V rows written once, the m input and output rows)."""
    w = cfg.n_layers * layer_weight_bytes(cfg)
    if cfg.final_norm:
        w += 4 * cfg.d_model * (2 if cfg.norm == 1 else 1)
    live = min(pos + 1, window, ring)
    kv_row = 2 * 4 * cfg.kv_width
    per_stream = cfg.n_layers * (kv_row * live + kv_row + 4 * ring) + 2 * 4 * cfg.d_model
    return w + cfg.m * per_stream


def weight_bytes(cfg):
    w = cfg.n_layers * layer_weight_bytes(cfg)
    if cfg.final_norm:
        w += 4 * cfg.d_model * (2 if cfg.norm == 1 else 1)
    return w


def block_bytes(cfg, pos, t, ring, window):
    """Algorithmic HBM bytes of one prefill block of t rows from `pos`: every weight once for the
    block, plus per row what a single step at that position moves besides the weights."""
    w = weight_bytes(cfg)
    return w + sum(step_bytes(cfg, pos + r, ring, window) - w for r in range(t))


def ffn_up_bytes(cfg):
    d, f = cfg.d_model, cfg.d_ff
    mats = (2 if cfg.ffn == 0 else 1) * f * d
    return 4 * (mats + d * (2 if cfg.norm == 1 else 1) + cfg.m * d + cfg.m * f)


def kernel_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel sources they were
    taken on (kernels.hip, dev.h, kernels.h) are the current ones; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    src = b"".join(open(os.path.join(ROOT, "streaming_ar_transformer_amd", "csrc", n), "rb").read()
                   for n in ("kernels.hip", "dev.h", "kernels.h"))
    digest = hashlib.sha256(src).hexdigest()[:16]
    rec = json.load(open(path)).get(f"{kernel}@{workload}")
    if not rec or rec.get("source_sha256_16") != digest:
        return None
    return rec.get("bytes_per_launch")


def host_info():
    """The host the oracle runs on: CPU model, BLAS library and its thread count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        import numpy  # noqa: F401  (loads the BLAS threadpoolctl reports)
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            i = infos[0]
            blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')})"
            threads = max(j.get("num_threads", 1) for j in infos)
    except Exception:
        pass
    return model, blas, threads


def cpu_baseline(cfg, layers, final, xs, budget_s):
    import numpy as np  # noqa: F401
    import oracle
    model, blas, threads = host_info()
    orc = oracle.OracleDecoder(cfg, layers, final)
    t0 = time.perf_counter()
    n = 0
    while n < xs.shape[0]:
        orc.step(xs[n], n, first=(n == 0))
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "blas": blas,
            "sample": f"positions 0..{n - 1} of a fresh stream of this workload "
                      f"({n} steps, {dt:.1f} s, NumPy float32, BLAS threads={threads})"}


def oracle_rate(cfg, layers, final, xs, pos0, budget_s, setup=None):
    """Oracle steps/s on the first positions of a run from `pos0` (at least one step)."""
    import oracle
    orc = oracle.OracleDecoder(cfg, layers, final)
    if setup is not None:
        setup(orc)
    t0 = time.perf_counter()
    n = 0
    while n < xs.shape[0]:
        orc.step(xs[n], pos0 + n, first=(n == 0 and setup is None))
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"steps_per_s": round(n / dt, 2), "steps": n, "seconds": round(dt, 2)}


def bench_configs(ids, dl4, df4, stream, cpu_s):
    """Steps/s and algorithmic GB/s of the other workloads on the graph path: the codec stacks
    over their whole runs from a fresh stream, the m=8 talker over its 256 positions after the
    4096-position import; each next to the oracle on a bounded sample."""
    import numpy as np
    import torch
    from streaming_ar_transformer_amd import sdec, workloads as wl
    from streaming_ar_transformer_amd.device import to_device, upload_weights
    out = {}
    for cid in ids:
        cfg = wl.CONFIGS[cid]
        layers, final = wl.make_weights(cfg)
        if cid == 5:
            dl, df = dl4, df4  # the same talker: config 4's weights
        else:
            dl, df = upload_weights(layers, final)
        xs_host = wl.make_inputs(cfg, cfg.steps)
        xs = to_device(xs_host)
        dec = sdec.Decoder(cfg, dl, df)
        pos0 = cfg.start_pos
        setup = None
        if pos0:
            pos_ring = np.full(cfg.ring, 0xFFFFFFFF, np.uint32)
            pos_ring[:pos0] = np.arange(pos0, dtype=np.uint32)
            pre = {}
            for s in range(cfg.m):
                pre.update(wl.make_prefill(cfg, streams=[s]))
                K, V = pre[s]
                for li in range(cfg.n_layers):
                    kp, vp, pp = dec.kv_view(s, li)
                    sdec.copy_to_device(kp, K[li])
                    sdec.copy_to_device(vp, V[li])
                sdec.copy_to_device(pp, pos_ring)

            def setup(orc, pre=pre):
                for s in range(cfg.m):
                    orc.import_kv(s, pre[s][0], pre[s][1], np.arange(pos0))
        # one warmup step records the graph; the state it leaves is restored below
        first0 = not pos0
        if pos0:
            dec.set_next_position(pos0)
        warm = torch.empty((cfg.m, cfg.d_model), device="cuda")
        warm.copy_(xs[0])
        dec.step(warm, pos0, first=first0, stream=stream)
        torch.cuda.synchronize()
        if pos0:
            # the warmup pushed position pos0 into every stream's ring: clear that slot again
            for s in range(cfg.m):
                _, _, pp = dec.kv_view(s, 0)
                sdec.copy_to_device(pp, pos_ring)
            dec.set_next_position(pos0)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(cfg.steps):
            dec.step(xs[i], pos0 + i, first=(i == 0 and first0), stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / cfg.steps
        dec.close()
        bts = float(np.mean([step_bytes(cfg, pos0 + i, cfg.ring, cfg.window)
                             for i in range(cfg.steps)]))
        gbs = bts / (ms * 1e-3) / 1e9
        rec = {"steps": cfg.steps, "positions": f"{pos0}..{pos0 + cfg.steps - 1}", "m": cfg.m,
               "steps_per_s": round(1000.0 / ms, 1), "tokens_per_s": round(cfg.m * 1000.0 / ms, 1),
               "ms_per_step": round(ms, 5), "hbm_gbs": round(gbs, 1),
               "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_step": int(bts),
               "mode": "hipgraph"}
        if cpu_s > 0:
            rec["oracle"] = oracle_rate(cfg, layers, final, xs_host, pos0, cpu_s, setup)
        out[cfg.name] = rec
        print(f"{cfg.name}: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s"
              + (f", oracle {rec['oracle']['steps_per_s']} steps/s" if cpu_s > 0 else ""),
              file=sys.stderr, flush=True)
        del xs
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(independent streams shard across GPUs with no exchange: run one process per GPU)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {n * 4} bytes x3", file=sys.stderr)
        return

    from streaming_ar_transformer_amd import sdec, workloads as wl
    from streaming_ar_transformer_amd.device import to_device, upload_weights

    torch.cuda.set_device(0)
    cfg = wl.CONFIGS[args.config]
    ring, window = cfg.ring, cfg.window
    unbounded = cfg.is_unbounded
    t0 = time.perf_counter()
    layers, final = wl.make_weights(cfg)
    dl, df = upload_weights(layers, final)
    n_in = max(args.steps, args.warmup, 1)
    xs_host = wl.make_inputs(cfg, n_in)
    xs = to_device(xs_host)  # [n, m, d] resident in HBM
    dec = sdec.Decoder(cfg, dl, df, eager=args.eager)
    mode = {sdec.PATH_GRAPH: "hipgraph", sdec.PATH_EAGER: "eager"}[dec.path]
    torch.cuda.synchronize()
    print(f"setup {time.perf_counter() - t0:.1f}s: {cfg.name}", file=sys.stderr, flush=True)

    def positions(n):
        # A fresh stream from position 0; an unbounded stack restarts (first=1) when full.
        out = []
        p = 0
        for _ in range(n):
            if unbounded and p >= ring:
                p = 0
            out.append(p)
            p += 1
        return out

    # warmup
    wpos = positions(args.warmup)
    for i, p in enumerate(wpos):
        dec.step(xs[i], p, first=(p == 0))
    torch.cuda.synchronize()
    # reload the inputs the warmup overwrote, start a fresh stream
    xs.copy_(torch.from_numpy(xs_host))
    dec.reset()
    torch.cuda.synchronize()

    tpos = positions(args.steps)
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i, p in enumerate(tpos):
        dec.step(xs[i], p, first=(p == 0), stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ms_per_step = ms / args.steps
    steps_per_s = 1000.0 / ms_per_step
    bytes_avg = float(np.mean([step_bytes(cfg, p, ring, window) for p in tpos]))
    hbm_gbs = bytes_avg / (ms_per_step * 1e-3) / 1e9
    print(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step, {hbm_gbs:.0f} GB/s "
          f"({100 * hbm_gbs / PEAK_HBM_GBS:.1f}% of peak)", file=sys.stderr, flush=True)
    if args.only_timed:
        dec.close()
        return

    # the step at fixed positions: a seeded N(0, 1) K/V import of positions 0..p-1, then repeated
    # steps at p (each re-stamps slot p with p, so every repetition attends the same p + 1 slots)
    fixed = None
    if args.fixed_positions and cfg.m == 1:
        fixed = {}
        xs.copy_(torch.from_numpy(xs_host))
        fpos = [p for p in (0, ring // 2, ring - 1) if p < ring]
        pre = wl.make_prefill(cfg, n_pos=max(fpos), streams=[0])[0] if max(fpos) else None
        for p in fpos:
            dec.reset()
            pos_ring = np.full(ring, 0xFFFFFFFF, np.uint32)
            if p:
                pos_ring[:p] = np.arange(p, dtype=np.uint32)
                for li in range(cfg.n_layers):
                    kp, vp, pp = dec.kv_view(0, li)
                    sdec.copy_to_device(kp, pre[0][li, :p])
                    sdec.copy_to_device(vp, pre[1][li, :p])
                sdec.copy_to_device(pp, pos_ring)
            else:
                _, _, pp = dec.kv_view(0, 0)
                sdec.copy_to_device(pp, pos_ring)
            reps = min(64, xs.shape[0] - 4)
            for i in range(reps + 4):  # each step takes (and overwrites) its own input row
                if i == 4:
                    torch.cuda.synchronize()
                    start.record(stream)
                dec.set_next_position(p)
                dec.step(xs[i], p, stream=stream)
            end.record(stream)
            torch.cuda.synchronize()
            fms = start.elapsed_time(end) / reps
            fb = step_bytes(cfg, p, ring, window)
            fixed[str(p)] = {"us_per_step": round(fms * 1e3, 1),
                             "hbm_gbs": round(fb / (fms * 1e-3) / 1e9, 1)}
        print("fixed positions: " + ", ".join(f"p={k}: {v['us_per_step']} us" for k, v in fixed.items()),
              file=sys.stderr, flush=True)

    # per-kernel launch times from profiled eager steps (each launch stamps a HIP event pair around
    # its own execution)
    xs.copy_(torch.from_numpy(xs_host))
    dec.reset()
    prof = None
    for i, p in enumerate(positions(args.profile_steps)):
        prof = dec.step_profile(xs[i], p, first=(p == 0), stream=stream, into=prof)
    kernels = {k: {"mean_us": round(1e3 * v[0] / v[1], 2), "launches": v[1]}
               for k, v in prof.items() if v[1]}
    up_us = 1e3 * prof["ffn_up"][0] / prof["ffn_up"][1]
    up_bytes = ffn_up_bytes(cfg)
    for k, b in (("qkv", 4 * ((cfg.q_width + 2 * cfg.kv_width) * cfg.d_model)),
                 ("o_proj", 4 * cfg.d_model * cfg.q_width), ("ffn_up", up_bytes),
                 ("ffn_down", 4 * cfg.d_model * cfg.d_ff)):
        if k in kernels:
            kernels[k]["weight_gbs"] = round(b / (kernels[k]["mean_us"] * 1e-6) / 1e9, 1)
    achieved = up_bytes / (up_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": kernel_traffic("ffn_up", cfg.name),
                "kernel": "k_gemv ffn gate/up + RMSNorm + SwiGLU",
                "bytes_per_launch": up_bytes, "mean_launch_us": round(up_us, 2)}
    dec.close()

    # prefill: blocks of `prefill_block` positions of one stream per sdec_prefill call
    prefill = None
    tb = args.prefill_block
    if tb > 1 and cfg.m == 1:
        nb = args.prefill_blocks
        if unbounded:
            nb = min(nb, ring // tb)
        pdec = sdec.Decoder(cfg, dl, df, max_prefill=tb)
        xb = torch.empty((nb, tb, cfg.d_model), device="cuda")
        src = torch.from_numpy(np.ascontiguousarray(xs_host[:tb, 0])).cuda()
        for i in range(nb):
            xb[i].copy_(src)
        for i in range(2):  # warmup blocks
            pdec.prefill(xb[i], i * tb, first=(i == 0), stream=stream)
        for i in range(nb):
            xb[i].copy_(src)
        pdec.reset(stream=stream)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(nb):
            pdec.prefill(xb[i], i * tb, first=(i == 0), stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        pms = start.elapsed_time(end) / nb
        pbytes = float(np.mean([block_bytes(cfg, i * tb, tb, ring, window) for i in range(nb)]))
        pgbs = pbytes / (pms * 1e-3) / 1e9
        prefill = {"block": tb, "positions": f"0..{nb * tb - 1}", "ms_per_block": round(pms, 4),
                   "tokens_per_s": round(tb * 1000.0 / pms, 1), "hbm_gbs": round(pgbs, 1),
                   "hbm_frac": round(pgbs / PEAK_HBM_GBS, 4), "bytes_per_block": int(pbytes),
                   "mode": "eager"}
        print(f"prefill {nb} blocks of {tb}: {pms * 1e3:.1f} us/block, "
              f"{tb * 1000.0 / pms:.0f} tokens/s, {pgbs:.0f} GB/s", file=sys.stderr, flush=True)
        pdec.close()

    # the FlowLM backbone variant of the same step (workload 6), graph path, a fresh stream
    variant = None
    if not args.no_variant and args.config == 4:
        vcfg = wl.CONFIGS[6]
        vl, vf = wl.make_weights(vcfg)
        vdl, vdf = upload_weights(vl, vf)
        vhost = wl.make_inputs(vcfg, vcfg.ring)
        vx = to_device(vhost)
        vdec = sdec.Decoder(vcfg, vdl, vdf)
        for i in range(32):
            vdec.step(vx[i], i, first=(i == 0), stream=stream)
        vx.copy_(torch.from_numpy(vhost))
        vdec.reset(stream=stream)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(vcfg.ring):
            vdec.step(vx[i], i, first=(i == 0), stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        vms = start.elapsed_time(end) / vcfg.ring
        vbytes = float(np.mean([step_bytes(vcfg, i, vcfg.ring, vcfg.window)
                                for i in range(vcfg.ring)]))
        vgbs = vbytes / (vms * 1e-3) / 1e9
        variant = {"workload": vcfg.name, "positions": f"0..{vcfg.ring - 1}",
                   "steps_per_s": round(1000.0 / vms, 1), "ms_per_step": round(vms, 5),
                   "hbm_gbs": round(vgbs, 1), "hbm_frac": round(vgbs / PEAK_HBM_GBS, 4),
                   "bytes_per_step": int(vbytes), "mode": "hipgraph"}
        print(f"{vcfg.name}: {vms * 1e3:.1f} us/step, {vgbs:.0f} GB/s", file=sys.stderr, flush=True)
        vdec.close()

    # split RVQ: encode and decode of a batch of latent frames
    rvq = None
    if not args.no_rvq and args.config == 4:
        rc = wl.RVQ_CONFIGS[1]
        R = wl.make_rvq(rc)
        dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in R.items()
               if k != "latents"}
        lat = torch.from_numpy(R["latents"]).cuda()
        q = sdec.RVQ(rc.dim, rc.vq, rc.bins, rc.nq, rc.frames, dev)
        codes = torch.empty((rc.frames, rc.nq), dtype=torch.int32, device="cuda")
        out = torch.empty((rc.frames, rc.dim), device="cuda")
        reps = 20
        for _ in range(3):
            q.encode(lat, codes, stream=stream)
            q.decode(codes, out, stream=stream)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(reps):
            q.encode(lat, codes, stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        enc_ms = start.elapsed_time(end) / reps
        start.record(stream)
        for _ in range(reps):
            q.decode(codes, out, stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        dec_ms = start.elapsed_time(end) / reps
        cb_bytes = 4 * rc.nq * rc.bins * rc.vq
        rvq = {"workload": rc.name, "frames": rc.frames,
               "encode_ms": round(enc_ms, 4), "encode_frames_per_s": round(rc.frames * 1e3 / enc_ms, 1),
               "decode_ms": round(dec_ms, 4), "decode_frames_per_s": round(rc.frames * 1e3 / dec_ms, 1),
               "codebook_bytes": cb_bytes,
               "encode_codebook_gbs": round(cb_bytes / (enc_ms * 1e-3) / 1e9, 1)}
        print(f"{rc.name}: encode {enc_ms * 1e3:.1f} us, decode {dec_ms * 1e3:.1f} us per "
              f"{rc.frames} frames", file=sys.stderr, flush=True)
        q.close()

    # streaming SEANet-style codec decoder: 16 latent columns -> 1920 samples per frame
    seanet = None
    if not args.no_seanet and args.config == 4:
        from streaming_ar_transformer_amd.seanet import SEANetDecoder
        scfg = wl.SEANET_CONFIGS[1]
        sw, sx = wl.make_seanet(scfg)
        sdev = {k: torch.from_numpy(v).cuda() for k, v in sw.items()}
        xf = torch.from_numpy(sx[0]).cuda()
        sdec_ = SEANetDecoder(scfg, sdev)
        n = 32
        for i in range(4):
            sdec_.step(xf, first=(i == 0), stream=stream)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(n):
            sdec_.step(xf, stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        sms = start.elapsed_time(end) / n
        seanet = {"workload": scfg.name, "frames": n, "ms_per_frame": round(sms, 4),
                  "frames_per_s": round(1000.0 / sms, 1), "samples_per_frame": 1920,
                  "realtime_factor_24khz": round(80.0 / sms, 1), "mode": "eager"}
        print(f"{scfg.name}: {sms * 1e3:.1f} us/frame", file=sys.stderr, flush=True)
        sdec_.close()

    # Pocket-style codec frame: latent -> 1x1 conv -> channel-wise convtr -> transpose -> the
    # 2-layer transformer over 16 positions (one prefill block of 16) -> transpose -> SEANet
    pocket = None
    if not args.no_pocket and args.config == 4:
        from streaming_ar_transformer_amd.pocket import PocketCodecFrame
        pc = wl.POCKET_CONFIGS[1]
        pconv, ptr, psw = wl.make_pocket_frame(pc)
        dconv = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in pconv.items()}
        dtr, _ = upload_weights(ptr, {})
        dsw = {k: torch.from_numpy(v).cuda() for k, v in psw.items()}
        fr = PocketCodecFrame(pc, dconv, dtr, dsw)
        n = 64  # 1024 positions: the 266-slot ring wraps three times
        for i in range(4):
            fr.decode_frame(dconv["latents"][i % pc.frames], first=(i == 0), stream=stream)
        fr.decode_frame(dconv["latents"][0], first=True, stream=stream)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(1, n + 1):
            fr.decode_frame(dconv["latents"][i % pc.frames], stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        fms = start.elapsed_time(end) / n
        pocket = {"workload": pc.name, "frames": n, "positions": f"{pc.up_stride}..{(n + 1) * pc.up_stride - 1}",
                  "ms_per_frame": round(fms, 4), "frames_per_s": round(1000.0 / fms, 1),
                  "samples_per_frame": pc.samples_per_frame,
                  "realtime_factor_24khz": round(1000.0 * pc.samples_per_frame / 24000.0 / fms, 1),
                  "mode": "eager"}
        if not args.no_cpu_baseline:
            import oracle
            nf = 4
            t0 = time.perf_counter()
            oracle.decode_frames(pconv["latents"][:nf], pconv, pc.transformer, ptr,
                                 wl.seanet_layers(pc.seanet), psw, pc.up_stride)
            pocket["cpu_oracle_ms_per_frame"] = round(1e3 * (time.perf_counter() - t0) / nf, 2)
        print(f"{pc.name}: {fms * 1e3:.1f} us/frame", file=sys.stderr, flush=True)
        fr.close()

    configs = None
    if not args.no_configs and args.config == 4:
        configs = bench_configs((1, 2, 3, 5), dl, df, stream,
                                0.0 if args.no_cpu_baseline else args.config_cpu_seconds)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, layers, final, xs_host, args.cpu_seconds)

    line = {
        "metric": "decode steps/s + achieved HBM GB/s (% of peak), 28L talker step at m=1",
        "value": round(steps_per_s, 2), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.n_layers, "hidden": cfg.d_model,
                   "q_heads": cfg.n_q_heads, "kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "ffn": cfg.d_ff, "m": cfg.m, "ring": ring,
                   "window": window, "positions": f"{tpos[0]}..{tpos[-1]}",
                   "mode": mode},
        "hbm_gbs": round(hbm_gbs, 1), "hbm_frac": round(hbm_gbs / PEAK_HBM_GBS, 4),
        "bytes_per_step": int(bytes_avg),
        "roofline": roofline, "fixed_positions": fixed, "eager_kernels": kernels,
        "prefill": prefill, "variant": variant,
        "rvq": rvq, "seanet": seanet, "pocket_frame": pocket, "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
