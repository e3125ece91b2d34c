#!/usr/bin/env python3
"""Benchmark of the KDA gated delta-rule step library on one MI355X.

Headline (one JSON line on stdout): T = 1 decode at B = 512, H = 12,
K = V = 128, bf16 pool of 1024 slots with 5% inactive rows, microseconds per
call. A step is one kda_decode call over one batch. Calls rotate over four
disjoint (pool, slot set, input) combinations so that one call's state
(~190 MiB) is not left in the 256 MiB Infinity Cache for the next call that
reads it; the timed region is K back-to-back calls bracketed by device
synchronisation. Kernel durations come from HIP events recorded on the
launch stream around every timed call.

The same line carries the roofline of the decode kernel (algorithmic bytes /
event-timed duration against 8 TB/s), a CPU baseline (the CPU oracle timed on
this host), and further measured points (decode batch sweep, verify, prefill)
under "points".
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--points", choices=["all", "none"], default="all",
                    help="also measure the decode sweep / verify / prefill points")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    return ap.parse_args()


# ---------------------------------------------------------------------------
# timing

def time_calls(calls, steps, warmup, torch):
    """Run `warmup` then `steps` calls (rotating through `calls`). Returns
    (wall_seconds, per-call event durations in ms)."""
    n = len(calls)
    for i in range(warmup):
        calls[i % n]()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        calls[i % n]()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])


# ---------------------------------------------------------------------------
# decode

def make_pools(torch, synth, H=12, N=1024):
    """Two bf16 pools of N slots (seeded N(0, 0.05) state)."""
    pools = []
    for p in range(2):
        rng = np.random.Generator(np.random.PCG64(synth.seed_for(1, 0, p)))
        bits = synth.pool_bits(rng, N, H)
        pools.append(torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16))
        del bits
    return pools


class DecodeSetup:
    """Four rotating (pool, index set, inputs) combinations for batch B: two
    pools x two disjoint index sets, each with its own seeded inputs."""

    def __init__(self, B, torch, kda, synth, pools, H=12, N=1024):
        self.B, self.H = B, H
        self.kda, self.torch = kda, torch
        W = H * 128
        self.W = W
        rng = np.random.Generator(np.random.PCG64(synth.seed_for(1, B, 99)))
        perm = rng.permutation(N)
        sets = []
        for s in range(2):
            chosen = perm[s * B:(s + 1) * B] if 2 * B <= N else perm[:B]
            idx = chosen.astype(np.int64)
            n_bad = int(round(0.05 * B))
            for i, pos in enumerate(sorted(rng.choice(B, size=n_bad, replace=False))):
                idx[pos] = -1 if i % 2 == 0 else N + int(rng.integers(0, 1000))
            sets.append(idx.astype(np.int32))
        self.n_active = int(((sets[0] >= 0) & (sets[0] < N)).sum())
        self.combos = []
        for j in range(4):
            c = synth.decode_case(B=B, N=1, H=H, seed=synth.seed_for(1, B) + j)
            qkv = self._bf16(c["qkv"])
            self.combos.append(dict(
                q=qkv[:, :W], k=qkv[:, W:2 * W], v=qkv[:, 2 * W:], g=self._bf16(c["gate"]),
                b=self._bf16(c["beta"]), a_log=torch.from_numpy(c["a_log"]).cuda(),
                dtb=torch.from_numpy(c["dt_bias"]).cuda(), pool=pools[j % 2],
                idx=torch.from_numpy(sets[(j // 2) % 2]).cuda(),
                out=torch.empty((B, W), dtype=torch.bfloat16, device="cuda")))

    def _bf16(self, a):
        t = self.torch
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(t.bfloat16)

    def calls(self):
        kda = self.kda

        def mk(c):
            return lambda: kda.kda_decode(c["q"], c["k"], c["v"], c["g"], c["b"], c["a_log"],
                                          c["dtb"], c["pool"], c["idx"], c["out"])
        return [mk(c) for c in self.combos]


def cpu_baseline_decode(B, budget_s, synth):
    """Time the CPU oracle on the same decode workload (one full B-row call
    per run; runs repeat until the budget is used, at least once)."""
    import oracle
    case = synth.decode_case(B=B, N=1024, H=12)
    H, W = 12, 12 * 128
    f32 = synth.f32_from_bits
    # gather the active rows' slots into a compact pool (inactive rows -> -1)
    idx = case["idx"].astype(np.int64)
    active = (idx >= 0) & (idx < case["N"])
    slots = idx[active]
    cidx = np.full(B, -1, np.int32)
    cidx[active] = np.arange(slots.size, dtype=np.int32)
    q, k, v = (np.ascontiguousarray(f32(case["qkv"][:, i * W:(i + 1) * W]).reshape(B, H, 128))
               for i in range(3))
    gate = np.ascontiguousarray(f32(case["gate"]).reshape(B, H, 128))
    beta = np.ascontiguousarray(f32(case["beta"]))
    base_pool = np.ascontiguousarray(f32(case["pool"][slots]))
    times = []
    t_start = time.perf_counter()
    while True:
        pool = base_pool.copy()
        t0 = time.perf_counter()
        oracle.decode(q, k, v, gate, beta, case["a_log"], case["dt_bias"], -5.0, 1.0, pool, cidx)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 20:
            break
    return dict(value=round(float(np.median(times)) * 1e6, 1), unit="us_per_call",
                cores=oracle.threads(), kind="oracle",
                sample=f"full T=1 decode call, B={B}, H=12, N=1024 pool (5% inactive), "
                       f"fp32 oracle, median of {len(times)} runs, "
                       f"{platform.processor() or platform.machine()}")


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the KDA step shards by rows and heads with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import gated_delta_rule_step_amd as kda
    from gated_delta_rule_step_amd import synth, workmodel as wm

    kda.lib()
    torch.cuda.init()
    dev_name = torch.cuda.get_device_name(0)
    log(f"bench: device {dev_name}")

    B = 512
    pools = make_pools(torch, synth)
    setup = DecodeSetup(B, torch, kda, synth, pools)
    log(f"bench: decode B={B} set up ({setup.n_active} active rows)")
    wall, ev = time_calls(setup.calls(), args.steps, args.warmup, torch)
    us_wall = wall / args.steps * 1e6
    us_ev = float(ev.mean()) * 1e3
    nbytes = wm.decode_bytes(setup.n_active, B - setup.n_active)
    gbs = nbytes / (us_ev * 1e-6) / 1e9
    log(f"bench: decode B={B}: {us_wall:.2f} us/step wall, {us_ev:.2f} us kernel avg, "
        f"{gbs:.0f} GB/s")

    points = []
    if args.points == "all":
        for Bp in (1, 8, 32, 128):
            sp = DecodeSetup(Bp, torch, kda, synth, pools)
            st = max(args.steps, 200)
            w, e = time_calls(sp.calls(), st, args.warmup, torch)
            nb = wm.decode_bytes(sp.n_active, Bp - sp.n_active)
            points.append(dict(kind="decode", B=Bp, us_per_call=round(float(e.mean()) * 1e3, 2),
                               us_median=round(float(np.median(e)) * 1e3, 2),
                               GBps=round(nb / (float(e.mean()) * 1e-3) / 1e9, 1)))
            log(f"bench: decode B={Bp}: {points[-1]}")
            del sp
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        cpu = cpu_baseline_decode(B, args.cpu_budget_s, synth)
        log(f"bench: cpu baseline {cpu}")

    line = {
        "metric": "KDA decode/verify us per call + HBM GB/s (% peak), H=12 K=V=128, B=1..512",
        "value": round(us_wall, 3),
        "unit": "us_per_call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_wall / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 storage, fp32 math",
        "data": "synthetic (seeded N(0,1) q/k/v/gate/beta, N(0,0.05) state)",
        "config": {"workload": "kda_decode T=1, B=512, H=12, K=V=128, bf16 pool N=1024, "
                               "5% inactive rows, packed q/k/v views",
                   "B": B, "H": 12, "T": 1, "pool_slots": 1024, "device": dev_name},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": wm.HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / wm.HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": "decode_kernel<8,true>",
                     "kernel_us_avg": round(us_ev, 3), "algorithmic_bytes": nbytes},
        "cpu_baseline": cpu,
        "points": points,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
