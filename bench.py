"""Frame-step benchmark: Moshi-7B-shaped RQ-Transformer, bfloat16 weights, B=1, on one MI355X.

One step = one 80 ms frame through the whole hot path (ring, embedding sum, 32 temporal layers,
text head + argmax, 8 depformer codebook steps, ring update), issued as one persistent kernel
launch per frame (--exec graph: one hipGraph replay; --exec stream: kernel by kernel).  Other
workloads (--config): int8 weights, a long-context prefill, 64 conversations stepped together.  After W warm-up frames the session is reset and K frames are timed from offset 0 (the
workload: 250 greedy frames, seed-1 random-init weights, uniform user tokens).

Prints one JSON line with frames/s, the roofline of the dominant kernel (measured with HIP
events on the session stream) and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "frames/s (80 ms) at B=1, Moshi-7B shape bf16; % of HBM roofline"


# HBM bytes per dispatch of the dominant kernels, from two rocprofv3 --pmc runs (FETCH_SIZE,
# WRITE_SIZE) scaled by a 256 MiB device-to-device copy in the same runs (profiles/ holds the
# summaries and commands).  Valid only for the kernel sources they were taken on (the files the
# B=1 frame kernels and the attentions are compiled from, and the launch code): the bench reports
# traffic null when their hash differs.
TRAFFIC = {
    "sources_sha256": "e96a3a61a7fec6268960c6789760727408e7f95a931faed3ea9acd7394af001f",
    "per_dispatch": {  # config/KV storage/kernel
        "moshi7b_bf16_b1/f32/frame_persistent": 14875330104,  # profiles/frame_moshi7b_bf16_b1_hbm_traffic.md
        "moshi7b_bf16_b1/f32/gate_in": 185045486,
        "moshi7b_bf16_b64/bf16/attn": 517918216,  # profiles/frame_moshi7b_bf16_b64_hbm_traffic.md
    },
}


TRAFFIC_SOURCES = ("device_common.h", "kernels.h", "batch.h", "frame_persistent.h", "persistent_variants.h",
                   "persistent_hd128_bf16_kvf32.hip", "moshi_api.hip")


def sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "rq_transformer_frame_amd", "csrc")
    for name in TRAFFIC_SOURCES:
        h.update(name.encode())
        with open(os.path.join(src, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(config: str, kv: str, kernel: str):
    if TRAFFIC["sources_sha256"] != sources_sha256():
        return None
    return TRAFFIC["per_dispatch"].get(f"{config}/{kv}/{kernel}")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


KV_ALG = 2  # bytes per cached element that the method moves: a bfloat16 KV cache, whatever the
            # storage the session keeps (float32 by default, for parity)


def stage_bytes(cfg, band: str, n_kv: float, rows: int = 1, kve: int = KV_ALG) -> dict:
    """Algorithmic HBM bytes of one launch of each stage: the weights it must stream once, the
    KV it must read (n_kv positions per conversation, kve bytes per element: bfloat16 for the
    algorithmic count), and its activation vectors (read once, written once), for `rows`
    conversations."""
    D, F, Dd, Fd, Q = cfg.d_model, cfg.ffn_hidden, cfg.dep_d_model, cfg.dep_ffn_hidden, cfg.dep_q
    Vt, Va, L = cfg.text_card, cfg.audio_card, cfg.n_layers
    # bytes per weight (Q4_0 packs two per byte) and per weight row of the band's float32 scales:
    # one per row (int8), one per 32-column block (Q4_0, q8_0)
    we = {"f32": 4, "bf16": 2, "i8": 1, "q4": 0.5, "q8": 1}[band]
    sc_row = 4 if band == "i8" else 0
    sc_blk = 4 / 32 if band in ("q4", "q8") else 0

    def lin(n, k):
        return int(n * k * we + n * sc_row + n * k * sc_blk)

    f = 4 * rows  # float32 activations, one row per conversation
    return {
        "embed": (2 * Q + 1) * D * (2 if band != "f32" else 4) * rows + 2 * D * f,
        "qkv": lin(3 * D, D) + 2 * D * f + D * f + 2 * D * kve * rows,
        "attn": 2 * n_kv * D * kve * rows + 2 * D * f,
        "out_proj": lin(D, D) + D * f + 2 * D * f,
        "gate_in": lin(2 * F, D) + 2 * D * f + F * f,
        "gate_out": lin(D, F) + F * f + 2 * D * f,
        "text_head": lin(Vt, D) + 2 * D * f + Vt * f + D * f,
        "dep_in": lin(Q * Dd, D) + D * f + Q * Dd * f,
        "dep_qkv": lin(3 * Dd, Dd) + 2 * Dd * f + 3 * Dd * f,
        "dep_out": lin(Dd, Dd) + 4 * Dd * f,
        "dep_gate_in": lin(2 * Fd, Dd) + 2 * Dd * f + Fd * f,
        "dep_gate_out": lin(Dd, Fd) + Fd * f + 2 * Dd * f,
        "dep_head": lin(Va, Dd) + Dd * f + Va * f,
        "frame_end": 0,
    }


def frame_bytes(weight_bytes: int, cfg, kve: int, positions) -> float:
    """Weights (streamed once per frame for all conversations) + the KV every conversation reads
    (kve bytes per element: KV_ALG for the algorithmic count), per frame, averaged over the frames:
    positions is [B][frames] (or [frames] at B = 1)."""
    pos = np.atleast_2d(np.asarray(positions))
    n = np.minimum(pos + 1, cfg.context)
    return weight_bytes + float(np.mean(n.sum(axis=0))) * cfg.n_layers * 2 * cfg.d_model * kve


def host_record() -> dict:
    """The GPU host's CPU: logical CPUs, model name and RAM (from /proc)."""
    rec = {"nproc": os.cpu_count(), "cpu_model": None, "ram_gb": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    rec["cpu_model"] = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    rec["ram_gb"] = round(int(line.split()[1]) / 2 ** 20, 1)
                    break
    except OSError:  # pragma: no cover
        pass
    return rec


def tiny_oracle_fps() -> dict:
    """The oracle on the tiny float32 configuration (all 16 frames), with the BLAS thread pool at
    its default size and limited to one thread."""
    import threadpoolctl

    import synth
    from oracle import OracleLM
    cfg = synth.TINY
    lm = OracleLM(cfg, synth.gen_weights(cfg))
    users = synth.user_tokens(cfg, cfg.frames)
    out = {}
    for label, limit in (("all_cores", None), ("one_core", 1)):
        with threadpoolctl.threadpool_limits(limits=limit):
            threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
            st = lm.new_state()
            t0 = time.perf_counter()
            for f in range(cfg.frames):
                lm.step(st, users[f])
            out[label] = {"frames_per_s": round(cfg.frames / (time.perf_counter() - t0), 2), "threads": int(threads)}
    return out


def cpu_baseline(cfg, weights, users, budget_s: float, max_frames: int):
    """The oracle as it stands, on the host cores, over the first frames of the same workload."""
    from oracle import OracleLM
    try:
        import threadpoolctl
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    t = time.time()
    lm = OracleLM(cfg, weights)
    log(f"oracle weights widened to float32 in {time.time() - t:.1f}s")
    st = lm.new_state()
    done, t0 = 0, time.perf_counter()
    while done < max_frames and (done < 2 or time.perf_counter() - t0 < budget_s):
        lm.step(st, users[done])
        done += 1
    dt = time.perf_counter() - t0
    del lm
    return {"value": done / dt, "unit": "frames/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {done} frames (offset 0..{done - 1}) of the same 7B bf16 B=1 workload, "
                      f"float32 numpy oracle with the bf16 weights widened, {dt:.1f}s",
            "host": host_record(), "tiny_f32_16_frames": tiny_oracle_fps()}


MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def prefill_flops(cfg, T: int, p0: int = 0):
    """Algorithmic flops of a teacher-forced prefill of T positions from offset p0, as (projections,
    attention): every temporal projection once per position (2 flops per weight), and per layer and
    position the scores and the weighted sum over its min(pos + 1, context) cached positions
    (2 x 2 x d_model flops each)."""
    D, F, L = cfg.d_model, cfg.ffn_hidden, cfg.n_layers
    params = L * (3 * D * D + D * D + 2 * F * D + D * F)
    pos = np.arange(p0, p0 + T)
    ctx = np.minimum(pos + 1, cfg.context).sum()
    return 2.0 * params * T, 4.0 * D * L * float(ctx)


def prefill_main(args, cfg):
    """Prompt throughput: K teacher-forced prefills of cfg.prefill frames from offset 0 (each after a
    reset), timed on the host around the synchronous moshi_prefill_forced calls."""
    import rq_transformer_frame_amd as rq
    import synth
    T = cfg.prefill
    K = args.steps if args.steps is not None else cfg.frames
    W = max(1, args.warmup if args.warmup is not None else 1)
    t = time.time()
    weights = synth.gen_weights(cfg)
    log(f"generated {cfg.name} weights (seed {cfg.seed}) in {time.time() - t:.1f}s")
    text, agent, user = synth.prefill_tokens(cfg, T)
    sess = rq.Session(cfg, exec="graph", kv=args.kv)
    sess.load_weights(weights)
    del weights
    for _ in range(W):
        sess.reset()
        sess.prefill_forced(0, text, agent, user)
    times = []
    for _ in range(K):
        sess.reset()
        t0 = time.perf_counter()
        sess.prefill_forced(0, text, agent, user)
        times.append(time.perf_counter() - t0)
    sess.close()
    dt = float(np.sum(times))
    per = dt / K
    proj, attn = prefill_flops(cfg, T)
    fl = proj + attn
    tflops = fl / per / 1e12
    log(f"{K} prefills of {T} frames: {per * 1e3:.1f} ms each, {T / per:.0f} prompt frames/s, {tflops:.1f} TFLOP/s")
    return {
        "metric": f"prompt frames/s (teacher-forced prefill of {T} frames), Moshi-7B shape bf16",
        "value": round(T / per, 1), "unit": "prompt frames/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(1000 * per, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: teacher-forced prefill of {T} frames of uniform tokens from offset 0 "
                               f"(seed {cfg.seed}), temporal layers only, row batches on the matrix cores",
                   "batch": 1, "band": cfg.band, "kv": args.kv, "accumulate": "f32",
                   "activations": "bf16 hi + lo parts (two products per step)"},
        "roofline": {"bound": "mfma", "kernel": "whole prefill (matrix-core projections, attention, epilogues)",
                     "achieved": round(tflops, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": fl, "avg_us": round(per * 1e6, 1),
                     # the projections run two bf16 products per step (activation hi and lo parts)
                     "mfma_issued_tflops": round(2 * proj / per / 1e12, 1)},
        "cpu_baseline": None,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed frames (default: the workload's frame count)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 10; prefill 1)")
    ap.add_argument("--config", default="moshi7b_bf16_b1")
    ap.add_argument("--exec", default="persistent", choices=["graph", "persistent", "stream"])
    ap.add_argument("--profile-frames", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--kv", default=None, choices=["f32", "bf16"],
                    help="KV cache storage (default: bf16 for batched conversations, else f32)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="first copy this many MiB device to device (a kernel of known traffic, for "
                         "scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the B=1 frame step does not shard; batched conversations would be data-parallel, one "
              "process per GPU)", file=sys.stderr)
        sys.exit(2)
    if args.profile_frames < 1:
        ap.error("--profile-frames must be at least 1 (the per-stage profile gives the roofline)")

    import rq_transformer_frame_amd as rq
    import synth

    if args.copy_mb:
        import torch
        a = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {args.copy_mb} MiB device to device")
        del a, b

    cfg = synth.CONFIGS[args.config]
    if args.kv is None:
        args.kv = "bf16" if cfg.batch > 1 else "f32"
    if cfg.name.endswith("_prefill"):
        print(json.dumps(prefill_main(args, cfg)), flush=True)
        return
    band = cfg.band
    B = cfg.batch
    t = time.time()
    weights = synth.gen_weights(cfg)
    log(f"generated {cfg.name} weights (seed {cfg.seed}) in {time.time() - t:.1f}s")
    K, W = (args.steps if args.steps is not None else cfg.frames), (args.warmup if args.warmup is not None else 10)
    nprof = args.profile_frames
    nframes = nprof + W + K

    kv = args.kv
    kve = 4 if kv == "f32" else 2  # bytes per cached element as stored
    if B > 1 and args.exec == "persistent":  # the persistent frame kernel serves one conversation
        args.exec = "graph"
    sess = rq.Session(cfg, exec=args.exec, kv=kv)
    t = time.time()
    sess.load_weights(weights)
    log(f"loaded weights in {time.time() - t:.1f}s")
    lin_bytes, all_bytes = sess.weight_bytes()

    # untimed setup: teacher-forced prefixes (long-context prefill, or per-conversation start
    # offsets of the batched workload)
    starts = np.zeros(B, np.int64)
    if cfg.prefill:
        starts[:] = cfg.prefill
    elif cfg.max_start_offset:
        starts[:] = synth.start_offsets(cfg)
    prefill_s = None

    def prefill():
        for b in range(B):
            if starts[b]:
                text, agent, user = synth.prefill_tokens(cfg, int(starts[b]), conv=b)
                sess.prefill_forced(b, text, agent, user)

    if starts.any():
        t = time.time()
        prefill()
        prefill_s = time.time() - t
        log(f"prefilled {int(starts.sum())} positions over {B} conversation(s) in {prefill_s:.2f}s")
    # users[f] is [B][Q] (B = 1: [1][Q])
    users = np.stack([synth.user_tokens(cfg, nframes, conv=b, start_frame=int(starts[b])) for b in range(B)], axis=1)

    # per-stage HIP-event profile on the session stream (kernels launched one by one)
    prof = sess.profile_frames(users[:nprof])
    from_zero = not starts.any()
    if from_zero:
        sess.reset()
        pos0 = starts
    else:
        pos0 = starts + nprof
    sb = stage_bytes(cfg, band, n_kv=float(np.mean(np.minimum(pos0 + 1, cfg.context))), rows=B)
    stages = {}
    for name, (n, us) in prof.items():
        if n:
            stages[name] = {"launches": n, "avg_us": us / n, "total_us_per_frame": us / nprof,
                            "bytes_per_launch": sb[name],
                            "gbs": sb[name] / (us / n) / 1e3 if us > 0 else None}
    dom = max((k for k in stages if k != "frame_end"), key=lambda k: stages[k]["total_us_per_frame"])
    prof_frame_us = sum(v["total_us_per_frame"] for v in stages.values())
    log(f"profiled {nprof} frames; dominant stage {dom}: "
        f"{stages[dom]['avg_us']:.1f} us/launch, {stages[dom]['gbs']:.0f} GB/s")

    f0 = 0 if from_zero else nprof
    for f in range(W):
        sess.step(users[f0 + f])
    # back to the start of the workload (offset 0, or the end of the prefilled prefixes, prefilled
    # again untimed), so the timed frames sit at the workload's own positions
    sess.reset()
    if not from_zero:
        prefill()
    ft = 0
    tpos = starts[:, None] + np.arange(K)[None, :]  # positions of the timed frames
    sess.gpu_time(1)  # HIP events around each frame's device work, on the session stream
    t0 = time.perf_counter()
    for f in range(K):
        sess.step(users[ft + f])
    dt = time.perf_counter() - t0
    gpu_us, gpu_n = sess.gpu_time(0)
    fps = K / dt
    fb = frame_bytes(lin_bytes, cfg, KV_ALG, tpos)
    kv_surplus = frame_bytes(lin_bytes, cfg, kve, tpos) - fb  # extra KV bytes of a float32 cache
    log(f"{K} frames in {dt:.3f}s: {fps:.1f} frames/s ({B * fps:.1f} conversation-frames/s), "
        f"{fb / (dt / K) / 1e9:.0f} GB/s frame-level; GPU {gpu_us / gpu_n:.1f} us/frame")
    sess.close()
    ceiling = rq.debug_read_bw(1 << 30, 20)
    log(f"streaming-read ceiling: {ceiling:.0f} GB/s")

    if args.exec == "persistent":
        # the whole frame is one kernel: its algorithmic bytes are the frame's
        avg = gpu_us / gpu_n
        roofline = {"bound": "hbm", "kernel": "k_frame_persistent (one launch per frame)",
                    "achieved": round(fb / avg / 1e3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(fb / avg / 1e3 / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(cfg.name, kv, "frame_persistent"),
                    "bytes_per_launch": fb, "avg_us": round(avg, 2),
                    "frac_of_ceiling": round(fb / avg / 1e3 / ceiling, 4)}
    else:
        d = stages[dom]
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(d["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(d["gbs"] / HBM_PEAK_GBS, 4), "traffic": measured_traffic(cfg.name, kv, dom),
                    "bytes_per_launch": d["bytes_per_launch"], "avg_us": round(d["avg_us"], 2),
                    "frac_of_ceiling": round(d["gbs"] / ceiling, 4)}

    cpu = None
    if not args.no_cpu_baseline and from_zero and B == 1:
        cpu = cpu_baseline(cfg, weights, users[:, 0], args.cpu_seconds, max_frames=len(users))
        log(f"cpu baseline: {cpu['value']:.3f} frames/s on {cpu['cores']} threads")

    metric, unit, value, what = METRIC, "frames/s", fps, "greedy frames from offset 0"
    if band == "i8":
        metric = "frames/s (80 ms) at B=1, Moshi-7B shape int8 per-row weights; % of HBM roofline"
    if band in ("q4", "q8"):
        metric = (f"frames/s (80 ms) at B=1, Moshi-7B shape {'Q4_0' if band == 'q4' else 'q8_0'} block-scaled "
                  "weights; % of HBM roofline")
    if cfg.prefill:
        metric = f"frames/s (80 ms) at B=1 after a {cfg.prefill}-frame prefill, Moshi-7B shape bf16; % of HBM roofline"
        what = f"greedy frames at positions {int(tpos.min())}..{int(tpos.max())} after a teacher-forced prefill"
    if B > 1:
        metric = f"conversation-frames/s at B={B}, Moshi-7B shape bf16; % of HBM roofline"
        unit, value = "conversation-frames/s", B * fps
        what = (f"greedy frames of {B} conversations stepped together, each after a teacher-forced prefix "
                f"of U{{0..{cfg.max_start_offset - 1}}} frames")
    out = {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(1000 * dt / K, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if band == "bf16" else band, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: Moshi-7B-shaped RQ-Transformer frame step, {K} {what}, "
                               f"seed-{cfg.seed} N(0,0.02) weights, uniform user tokens",
                   "batch": B, "band": band, "kv": kv, "accumulate": "f32", "exec": args.exec,
                   "weight_bytes_per_frame": lin_bytes,
                   "prefill_positions": int(starts.sum()), "prefill_s": None if prefill_s is None else round(prefill_s, 3)},
        "tokens_per_s": round(9 * B * fps, 1),
        "frame_roofline": {"bytes_per_frame": fb, "achieved_gbs": round(fb / (dt / K) / 1e9, 1),
                           "frac": round(fb / (dt / K) / 1e9 / HBM_PEAK_GBS, 4),
                           "read_ceiling_gbs": round(ceiling, 1),
                           "frac_of_ceiling": round(fb / (dt / K) / 1e9 / ceiling, 4),
                           "kv_storage_surplus_bytes": kv_surplus,
                           "gpu_us_per_frame": round(gpu_us / gpu_n, 2)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages": {k: {kk: (round(vv, 2) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for k, v in stages.items()},
        "profiled_frame_us": round(prof_frame_us, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
