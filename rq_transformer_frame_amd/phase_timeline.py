"""Where a B=1 frame of the persistent executor goes, phase kind by phase kind.

    python -m rq_transformer_frame_amd.phase_timeline [--config moshi7b_bf16_b1] [--frames 130]
        [--first 20] [--every 10]

Runs greedy frames from offset 0 with the kernel's phase record switched on and reads the record
of every `every`-th frame from `first` on.  A phase's time is the gap between its completion and
the previous phase's, as block 0 sees them: for a flag phase, when every block's flag is up; for a
depformer exchange phase, when block 0 holds every input of the next phase.  The first phase is
counted from block 0's arrival at it (the embedding sum before it is left out).  Prints a markdown
table of microseconds per frame by phase kind, averaged over the sampled frames.
"""
from __future__ import annotations

import argparse
import collections
import time

import numpy as np

TEMPORAL = ("qkv", "attention", "out_proj", "gate_in", "gate_out")
DEPFORMER = ("dep_qkv", "dep_attention+out_proj", "dep_gate_in", "dep_gate_out")


def phase_kind(p: int, n_layers: int, dep_layers: int) -> str:
    """Kind of phase p of the persistent frame kernel: 5 per temporal layer, the text head (with
    depformer_in), then per codebook step 4 per depformer layer and the codebook head."""
    if p < 5 * n_layers:
        return TEMPORAL[p % 5]
    if p == 5 * n_layers:
        return "text_head+dep_in"
    k = (p - 5 * n_layers - 1) % (4 * dep_layers + 1)
    return "dep_head" if k == 4 * dep_layers else DEPFORMER[k % 4]


def main():
    import rq_transformer_frame_amd as rq
    import synth

    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="moshi7b_bf16_b1")
    ap.add_argument("--frames", type=int, default=130)
    ap.add_argument("--first", type=int, default=20)
    ap.add_argument("--every", type=int, default=10)
    args = ap.parse_args()
    cfg = synth.CONFIGS[args.config]
    t = time.time()
    weights = synth.gen_weights(cfg)
    print(f"[phase_timeline] generated {cfg.name} weights in {time.time() - t:.1f}s", flush=True)
    users = synth.user_tokens(cfg, args.frames)
    acc = collections.defaultdict(float)
    count = collections.Counter()
    sampled = []
    with rq.Session(cfg, exec="persistent") as s:
        s.load_weights(weights)
        del weights
        s.phase_times(1)
        for f in range(args.frames):
            s.step(users[f])
            if f >= args.first and (f - args.first) % args.every == 0:
                nph = 5 * cfg.n_layers + 1 + cfg.dep_q * (4 * cfg.dep_layers + 1)  # the kernel's phases
                done = s.phase_times(-1)[:nph, 1]
                dur = np.diff(np.concatenate([[0.0], done]))
                for p, d in enumerate(dur):
                    k = phase_kind(p, cfg.n_layers, cfg.dep_layers)
                    acc[k] += d
                    if len(sampled) == 0:
                        count[k] += 1
                sampled.append(f)
    n = len(sampled)
    total = sum(acc.values()) / n
    print(f"{cfg.name}, persistent executor: frames at positions {sampled[0]}..{sampled[-1]} "
          f"(every {args.every}), {total:.1f} us per frame from block 0's first arrival\n")
    print("| phase kind | phases per frame | us per frame | us per phase | share |")
    print("|---|---|---|---|---|")
    for k, v in sorted(acc.items(), key=lambda x: -x[1]):
        print(f"| {k} | {count[k]} | {v / n:.1f} | {v / n / count[k]:.2f} | {100 * v / n / total:.1f}% |")


if __name__ == "__main__":
    main()
