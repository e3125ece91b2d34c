#!/usr/bin/env python3
"""Benchmark of the KDA gated delta-rule step library on one MI355X.

Headline (one JSON line on stdout): T = 1 decode at B = 512, H = 12,
K = V = 128, bf16 pool of 1024 slots with 5% inactive rows, microseconds per
call. A step is one kda_decode call over one batch. Calls rotate over four
(pool, slot set, inputs) combinations -- two 1024-slot pools times two
disjoint slot sets -- so the state a call reads (~190 MiB) was last touched
three calls earlier, past the 256 MiB Infinity Cache. The K timed calls are
replayed from HIP graphs (K launches exactly), bracketed by device
synchronisation; HIP events on the launch stream around the timed region
give the average kernel duration. Before timing, the headline workload is
replayed for one second: a fresh process runs its first tens of
milliseconds of sustained load ~10-15% slower.

The line also carries the roofline of the decode kernel (algorithmic bytes
per call / average duration, against 8 TB/s), the CPU oracle timed on this
host, and further measured points under "points": the decode batch sweep and
the verify workloads (T = 8 / 4, bare checkpoint, fold rates, deep window)
and the varlen prefill workloads (4 documents and the 14-document mix of
16384 tokens, H = 64 and 12).

--mode profile runs a short fixed sequence (decode B = 512, the verify
workloads at B = 512 whose traffic is counted, and a known-size device copy for
counter calibration) for rocprofv3; --mode profile-prefill runs 4 prefill
calls on each document set at H = 64 and at H = 12, then the same copies.
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

H = 12
N_SLOTS = 1024


# HBM bytes per call of a workload from two rocprofv3 --pmc passes (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch, summed over the call's kernels) over
# `bench.py --mode profile` / `--mode profile-prefill`, scaled by what the same
# counters read for a device copy of known size in the same run (FETCH x 2.0,
# WRITE x 1.0); the summaries are in profiles/. A figure holds only for the
# kernel sources the counters were taken on: the digests turn it into null
# once those sources change.
_DEC_SRC = ("gated_delta_rule_step_amd/csrc/kda_decode.hip",
            "gated_delta_rule_step_amd/csrc/kda_common.h", "gated_delta_rule_step_amd/build.py")
_DEC_SHA = ("84c78a8d6498618efb1a4d7b64592ce8060e9db6d865bb021275a99a6dec8ae7",
            "2fe55975814488bcd43f46e6ffd9805dc1139ce860b017fe31783558c0e3b22e",
            "90c1cd82031d88b6ff81e4330b9f109c95bf3e9b0f031a3208f41099dfb3fb5f")
_VER_SRC = ("gated_delta_rule_step_amd/csrc/kda_verify.hip",) + _DEC_SRC[1:]
_VER_SHA = ("3e6ca5522e82c662fc18e380962fbbb2c1895663a619f60314014b129b10ac5b",) + _DEC_SHA[1:]
_PF_SRC = ("gated_delta_rule_step_amd/csrc/kda_prefill.hip",
           "gated_delta_rule_step_amd/csrc/kda_prefill_split.hip",
           "gated_delta_rule_step_amd/csrc/kda_launch.h") + _DEC_SRC[1:]
_PF_SHA = ("c15ff32ad2c76e94ffed06bc44b615ffca296dab0f3fe35f4712ccc00384cdc6",
           "5e7aa29c6b822a0400ee3401e6840a3c44a1d957ed360c4688ee6b02b8b09b9f",
           "f0d19f52b61dfbe88a4f7021b78ca69e8965e900fcdf2a3b68436948e8179958") + _DEC_SHA[1:]


def _ct(src, sha, fetch_kib, write_kib):
    return dict(sources=src, sha256=sha, fetch_kib=fetch_kib, write_kib=write_kib,
                fetch_scale=2.0, write_scale=1.0)


COUNTED_TRAFFIC = {
    "decode B=512": _ct(_DEC_SRC, _DEC_SHA, 96508.344, 188160.961),
    "verify T=8 B=512 bare": _ct(_VER_SRC, _VER_SHA, 123843.391, 61440.0),
    "verify T=8 B=512 fm=9 100% fold": _ct(_VER_SRC, _VER_SHA, 138465.023, 258048.188),
    "verify T=4 B=512 fm=13 100% fold": _ct(_VER_SRC, _VER_SHA, 143754.445, 227328.0),
    "verify T=8 B=512 W32 fm=25 hist~U{0..24}": _ct(_VER_SRC, _VER_SHA, 160222.203, 124416.0),
    # the fused kernel (H = 64), or the preparation + chain kernels summed (H = 12)
    "prefill 4 docs (3840, 3776, 3200, 3072) H=64": _ct(_PF_SRC, _PF_SHA, 455747.391, 230400.0),
    "prefill 4 docs (3840, 3776, 3200, 3072) H=12": _ct(_PF_SRC, _PF_SHA, 235868.531, 357119.508),
    "prefill 14-doc mix, 16384 tokens H=64": _ct(_PF_SRC, _PF_SHA, 547233.688, 290816.0),
    "prefill 14-doc mix, 16384 tokens H=12": _ct(_PF_SRC, _PF_SHA, 282825.203, 423161.594),
}


def counted_traffic(workload):
    import hashlib
    ent = COUNTED_TRAFFIC.get(workload)
    if ent is None:
        return None
    for rel, digest in zip(ent["sources"], ent["sha256"]):
        with open(os.path.join(ROOT, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    return int(round((ent["fetch_kib"] * ent["fetch_scale"]
                      + ent["write_kib"] * ent["write_scale"]) * 1024))


# verify points (B = 512) whose counted traffic the profile sequence measures
VERIFY_TRAFFIC = {
    "T=8 bare (0% fold)": "verify T=8 B=512 bare",
    "T=8 fm=9 100% fold": "verify T=8 B=512 fm=9 100% fold",
    "T=4 fm=13 100% fold": "verify T=4 B=512 fm=13 100% fold",
    "T=8 W32 fm=25 hist~U{0..24}": "verify T=8 B=512 W32 fm=25 hist~U{0..24}",
}
# the verify configurations of the points (label -> VerifySetup arguments)
VERIFY_CFGS = [
    dict(label="T=8 bare (0% fold)", T=8, hist_max=0),
    dict(label="T=4 bare (0% fold)", T=4, hist_max=0),
    dict(label="T=8 fm=9 50% fold", T=8, fold_p=0.5),
    dict(label="T=8 fm=9 100% fold", T=8, fold_p=1.0),
    dict(label="T=4 fm=13 100% fold", T=4, fold_p=1.0),
    dict(label="T=8 W32 fm=25 hist~U{0..24}", T=8, w_ring=32, flush_min=25, hist_max=24),
    dict(label="T=8 bare, pre-computed gate and beta", T=8, hist_max=0, gate_mode=3),
    dict(label="T=8 fm=9 50% fold, per-head gate", T=8, fold_p=0.5, gate_mode=4),
    dict(label="T=8 bare, fp16 checkpoints", T=8, hist_max=0, state="fp16"),
    dict(label="T=8 fm=9 100% fold, fp16 checkpoints", T=8, fold_p=1.0, state="fp16"),
    dict(label="T=8 bare, fp8 checkpoints", T=8, hist_max=0, state="fp8"),
    dict(label="T=8 fm=9 100% fold, fp8 checkpoints", T=8, fold_p=1.0, state="fp8"),
]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--points", choices=["all", "none"], default="all",
                    help="also measure the decode sweep and the verify points")
    ap.add_argument("--mode", choices=["bench", "profile", "profile-prefill"], default="bench")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    return ap.parse_args()


# ---------------------------------------------------------------------------
# timing

def time_graphs(calls, steps, warmup, torch, min_warm_s=0.0):
    """Replay exactly `steps` launches (rotating through `calls`) from HIP
    graphs after `warmup` eager launches (and, with min_warm_s, after repeated
    graph replays until that much time has passed: the first tens of
    milliseconds of sustained load run ~10-15% slower on a fresh process).
    Returns (wall seconds, event ms)."""
    n = len(calls)
    for i in range(max(warmup, n)):
        calls[i % n]()
    torch.cuda.synchronize()
    per = n * max(1, 32 // n)
    reps, rem = divmod(steps, per)

    def capture(count):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(count):
                    calls[i % n]()
        torch.cuda.current_stream().wait_stream(s)
        return g

    g_main = capture(per) if reps else None
    g_rem = capture(rem) if rem else None
    t_warm = time.perf_counter()
    while True:
        if g_main is not None:
            g_main.replay()
        if g_rem is not None:
            g_rem.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t_warm >= min_warm_s:
            break
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps):
        g_main.replay()
    if g_rem is not None:
        g_rem.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1)


def launch_percentiles(calls, n, torch):
    """Per-launch kernel time: n eager launches (rotating through `calls`),
    each bracketed by HIP events recorded on the launch stream. Returns the
    10th, 50th and 90th percentiles in us."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[i][0].record()
        calls[i % len(calls)]()
        ev[i][1].record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    p10, p50, p90 = np.percentile(t, [10, 50, 90])
    return dict(p10=round(float(p10), 3), p50=round(float(p50), 3), p90=round(float(p90), 3),
                launches=n, method="eager launches, one HIP event pair each on the launch stream")


# ---------------------------------------------------------------------------
# workloads

def bf16_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def fp16_pools(torch, pools):
    """The same two pools with fp16 state elements (state_dtype 1)."""
    return [p.to(torch.float16) for p in pools]


def fp8_pools(torch, pools):
    """The same two pools with fp8 e4m3 state elements (state_dtype 2)."""
    return [p.to(torch.float8_e4m3fn) for p in pools]


def make_pools(torch, synth):
    """Two bf16 pools of 1024 slots (seeded N(0, 0.05) state)."""
    pools = []
    for p in range(2):
        rng = np.random.Generator(np.random.PCG64(synth.seed_for(1, 0, p)))
        pools.append(bf16_dev(torch, synth.pool_bits(rng, N_SLOTS, H)))
    return pools


def index_sets(synth, B, tag, inactive_frac=0.05):
    """Two disjoint slot sets of B rows (when 2B <= 1024), each with
    round(inactive_frac * B) rows set to -1 or >= 1024."""
    rng = np.random.Generator(np.random.PCG64(synth.seed_for(1, B, tag)))
    perm = rng.permutation(N_SLOTS)
    sets = []
    for s in range(2):
        idx = (perm[s * B:(s + 1) * B] if 2 * B <= N_SLOTS else perm[:B]).astype(np.int64)
        n_bad = int(round(inactive_frac * B))
        for i, pos in enumerate(sorted(rng.choice(B, size=n_bad, replace=False))):
            idx[pos] = -1 if i % 2 == 0 else N_SLOTS + int(rng.integers(0, 1000))
        sets.append(idx.astype(np.int32))
    return sets


def cold_sets(synth, B, tag, inactive_frac=0.05):
    """All 1024 slots split into 1024 // B disjoint sets of B rows, each with
    round(inactive_frac * B) rows set to -1 or >= 1024."""
    rng = np.random.Generator(np.random.PCG64(synth.seed_for(1, B, tag + 1000)))
    perm = rng.permutation(N_SLOTS)
    sets = []
    for s in range(N_SLOTS // B):
        idx = perm[s * B:(s + 1) * B].astype(np.int64)
        n_bad = int(round(inactive_frac * B))
        for i, pos in enumerate(sorted(rng.choice(B, size=n_bad, replace=False))):
            idx[pos] = -1 if i % 2 == 0 else N_SLOTS + int(rng.integers(0, 1000))
        sets.append(idx.astype(np.int32))
    return sets


class DecodeSetup:
    """Decode workload. Default: four (pool, slot set, inputs) combinations
    (two pools x two disjoint slot sets). cold=True: every slot of both pools
    once per pass, 2 * 1024 // B combinations with inputs of their own, so a
    combination's state was last touched ~800 MB of traffic earlier (past the
    256 MB Infinity Cache): the small batches are timed cold."""

    def __init__(self, B, torch, kda, synth, pools, gate_mode=0, cold=False):
        self.B, self.gate_mode = B, gate_mode
        W = H * 128
        self.combos = []
        if cold:
            sets = cold_sets(synth, B, 99)
            n = 2 * len(sets)
            c = synth.decode_case(B=B * n, N=1, H=H, seed=synth.seed_for(1, B, 7))
            qkv, gate, beta = (bf16_dev(torch, c[x]) for x in ("qkv", "gate", "beta"))
            a_log, dtb = torch.from_numpy(c["a_log"]).cuda(), torch.from_numpy(c["dt_bias"]).cuda()
            for j in range(n):
                r = slice(j * B, (j + 1) * B)
                self.combos.append(dict(
                    q=qkv[r, :W], k=qkv[r, W:2 * W], v=qkv[r, 2 * W:], g=gate[r], b=beta[r],
                    a_log=a_log, dtb=dtb, pool=pools[j % 2],
                    idx=torch.from_numpy(sets[j // 2]).cuda(),
                    out=torch.empty((B, W), dtype=torch.bfloat16, device="cuda")))
            self.n_active = int(np.mean([((x >= 0) & (x < N_SLOTS)).sum() for x in sets]))
            self.kda = kda
            return
        sets = index_sets(synth, B, 99)
        self.n_active = int(((sets[0] >= 0) & (sets[0] < N_SLOTS)).sum())
        for j in range(4):
            c = synth.decode_case(B=B, N=1, H=H, seed=synth.seed_for(1, B) + j)
            if gate_mode & 4:
                c = synth.per_head_gate(c, bool(gate_mode & 1), synth.seed_for(1, B, 120) + j)
            elif gate_mode:
                c = synth.precomputed_gate(c, gate_mode, synth.seed_for(1, B, 100) + j)
            qkv = bf16_dev(torch, c["qkv"])
            self.combos.append(dict(
                q=qkv[:, :W], k=qkv[:, W:2 * W], v=qkv[:, 2 * W:], g=bf16_dev(torch, c["gate"]),
                b=bf16_dev(torch, c["beta"]), a_log=torch.from_numpy(c["a_log"]).cuda(),
                dtb=torch.from_numpy(c["dt_bias"]).cuda(), pool=pools[j % 2],
                idx=torch.from_numpy(sets[(j // 2) % 2]).cuda(),
                out=torch.empty((B, W), dtype=torch.bfloat16, device="cuda")))
        self.kda = kda

    def calls(self):
        kda = self.kda

        gm = self.gate_mode
        pre = bool(gm & 1)

        def mk(c):
            return lambda: kda.kda_decode(c["q"], c["k"], c["v"], c["g"], c["b"],
                                          None if pre else c["a_log"], None if pre else c["dtb"],
                                          c["pool"], c["idx"], c["out"], gate_mode=gm)
        return [mk(c) for c in self.combos]


class VerifySetup:
    """Verify workload: T draft tokens per row, pools shared with decode,
    one synthetic ring set per pool; per-row hist_len / cache_base drawn as in
    the tests (fold probability p, or hist ~ U{0..hist_max})."""

    def __init__(self, B, T, torch, kda, synth, pools, rings, w_ring=16, flush_min=None,
                 fold_p=0.0, hist_max=None, gate_mode=0, cold=False):
        self.B, self.T, self.w_ring, self.gate_mode = B, T, w_ring, gate_mode
        W = H * 128
        self.combos = []
        if cold:  # as DecodeSetup(cold=True); the rows share one hist / fold pattern
            assert gate_mode == 0
            sets = cold_sets(synth, B, 77, inactive_frac=0.0)
            n = 2 * len(sets)
            c = synth.verify_case(B=B * n, T=T, N=1, H=H, w_ring=w_ring, flush_min=flush_min,
                                  fold_p=fold_p, hist_max=hist_max,
                                  seed=synth.seed_for(3, B, T) + 7)
            self.flush_min = c["flush_min"]
            self.hist = c["hist_len"][:B].copy()
            self.fold = (self.hist + T >= c["flush_min"])
            qkv, gate, beta = (bf16_dev(torch, c[x]) for x in ("qkv", "gate", "beta"))
            a_log, dtb = torch.from_numpy(c["a_log"]).cuda(), torch.from_numpy(c["dt_bias"]).cuda()
            hist = torch.from_numpy(self.hist).cuda()
            for j in range(n):
                r = slice(j * B, (j + 1) * B)
                kc, uc, gc = rings[j % 2]
                self.combos.append(dict(
                    q=qkv[r, :, :W], k=qkv[r, :, W:2 * W], v=qkv[r, :, 2 * W:], g=gate[r],
                    b=beta[r], a_log=a_log, dtb=dtb, pool=pools[j % 2],
                    idx=torch.from_numpy(sets[j // 2]).cuda(), kc=kc, uc=uc, gc=gc, hist=hist,
                    base=torch.from_numpy(c["cache_base"][r].copy()).cuda(),
                    out=torch.empty((B, T, W), dtype=torch.bfloat16, device="cuda")))
            self.kda = kda
            return
        sets = index_sets(synth, B, 77, inactive_frac=0.0)
        for j in range(4):
            c = synth.verify_case(B=B, T=T, N=1, H=H, w_ring=w_ring, flush_min=flush_min,
                                  fold_p=fold_p, hist_max=hist_max,
                                  seed=synth.seed_for(3, B, T) + j)
            if gate_mode & 4:
                c = synth.per_head_gate(c, bool(gate_mode & 1), synth.seed_for(3, B, 120 + T) + j)
            elif gate_mode:
                c = synth.precomputed_gate(c, gate_mode, synth.seed_for(3, B, 100 + T) + j)
            self.flush_min = c["flush_min"]
            if j == 0:
                self.hist = c["hist_len"].copy()
                self.fold = (c["hist_len"] + T >= c["flush_min"])
            qkv = bf16_dev(torch, c["qkv"])
            kc, uc, gc = rings[j % 2]
            self.combos.append(dict(
                q=qkv[..., :W], k=qkv[..., W:2 * W], v=qkv[..., 2 * W:],
                g=bf16_dev(torch, c["gate"]), b=bf16_dev(torch, c["beta"]),
                a_log=torch.from_numpy(c["a_log"]).cuda(),
                dtb=torch.from_numpy(c["dt_bias"]).cuda(), pool=pools[j % 2],
                idx=torch.from_numpy(sets[(j // 2) % 2]).cuda(), kc=kc, uc=uc, gc=gc,
                hist=torch.from_numpy(self.hist).cuda(),
                base=torch.from_numpy(c["cache_base"]).cuda(),
                out=torch.empty((B, T, W), dtype=torch.bfloat16, device="cuda")))
        self.kda = kda

    def calls(self):
        kda, fm, w, gm = self.kda, self.flush_min, self.w_ring, self.gate_mode
        pre = bool(gm & 1)

        def mk(c):
            return lambda: kda.kda_verify_ucache_flush(
                c["q"], c["k"], c["v"], c["g"], c["b"], None if pre else c["a_log"],
                None if pre else c["dtb"], c["pool"],
                c["idx"], c["kc"], c["uc"], c["gc"], c["hist"], c["base"], c["out"],
                flush_min=fm, w_ring=w, gate_mode=gm)
        return [mk(c) for c in self.combos]


def make_rings(torch, synth):
    rings = []
    for p in range(2):
        kc, uc, gc = synth.synthetic_rings((N_SLOTS, H, 32, 128), synth.seed_for(3, 0, p))
        rings.append((bf16_dev(torch, kc), bf16_dev(torch, uc), torch.from_numpy(gc).cuda()))
    return rings


class PrefillSetup:
    """Prefill workload: packed documents of the given lengths, H heads,
    inputs drawn on the device from a seeded generator with the same
    distributions as the test cases (q, k, v, gate, beta logits N(0, 1),
    A_log U(-1, 1), dt_bias N(0, 0.1), initial states N(0, 0.05) in a pool of
    2 slots per document)."""

    def __init__(self, lens, H, torch, kda, synth, gate_mode=0, ckpt_interval=0, state="bf16",
                 ring_tail=0):
        self.lens, self.H, self.gate_mode = tuple(lens), H, gate_mode
        n_docs, T, W = len(lens), int(sum(lens)), H * 128
        gen = torch.Generator(device="cuda")
        gen.manual_seed(synth.seed_for(4, H, n_docs))

        def randn(*shape, std=1.0):
            x = torch.randn(*shape, generator=gen, device="cuda", dtype=torch.float32)
            return (x * std).to(torch.bfloat16)
        self.q, self.k, self.v, self.g = (randn(T, W) for _ in range(4))
        self.beta = randn(T, H)
        if gate_mode & 1:  # the log-decay itself, U(-6, 0.5) (clamped into [-5, 0])
            u = torch.rand(T, W, generator=gen, device="cuda")
            self.g = (u * 6.5 - 6.0).to(torch.bfloat16)
        if gate_mode & 2:  # beta itself, U(0, 1)
            self.beta = torch.rand(T, H, generator=gen, device="cuda").to(torch.bfloat16)
        self.a_log = torch.rand(H, generator=gen, device="cuda") * 2.0 - 1.0
        self.dtb = torch.randn(H * 128, generator=gen, device="cuda") * 0.1
        if gate_mode & 4:  # one gate value (and dt_bias) per token and head
            self.g = randn(T, H)
            self.dtb = torch.randn(H, generator=gen, device="cuda") * 0.1
        N = 2 * n_docs
        self.pool = randn(N, H, 128, 128, std=0.05)
        if state != "bf16":
            self.pool = self.pool.to({"fp16": torch.float16, "fp8": torch.float8_e4m3fn}[state])
        self.idx = torch.randperm(N, generator=gen, device="cuda")[:n_docs].to(torch.int32)
        cu = np.zeros(n_docs + 1, np.int32)
        cu[1:] = np.cumsum(lens)
        self.cu_h = torch.from_numpy(cu)
        self.cu_d = self.cu_h.cuda()
        self.out = torch.empty((T, W), dtype=torch.bfloat16, device="cuda")
        self.ws = torch.empty(kda.kda_prefill_workspace_size(n_docs, T, H), dtype=torch.uint8,
                              device="cuda")
        # intermediate checkpoints every ckpt_interval tokens (0: none)
        self.ck = self.ck_starts = None
        self.ck_interval, self.ck_rows = max(ckpt_interval, 16), 0
        if ckpt_interval:
            counts = np.asarray(lens) // ckpt_interval
            self.ck_rows = int(counts.sum())
            starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
            self.ck_starts = torch.from_numpy(starts).cuda()
            self.ck = torch.empty((self.ck_rows, H, 128, 128), dtype=self.pool.dtype,
                                  device="cuda")
        # hand-off of each document's last tokens to a 32-row verify ring
        self.ring_tail, self.ring, self.base = ring_tail, None, None
        if ring_tail:
            self.ring = (torch.zeros((N, H, 32, 128), dtype=torch.bfloat16, device="cuda"),
                         torch.zeros((N, H, 32, 128), dtype=torch.bfloat16, device="cuda"),
                         torch.zeros((N, H, 32, 128), dtype=torch.float32, device="cuda"))
            self.base = torch.randint(0, 32, (n_docs,), generator=gen, device="cuda",
                                      dtype=torch.int32)
        self.kda = kda

    def calls(self):
        s = self

        pre = bool(s.gate_mode & 1)

        def call():
            s.kda.kda_prefill_varlen(s.cu_h, s.cu_d, s.q, s.k, s.v, s.g, s.beta,
                                     None if pre else s.a_log, None if pre else s.dtb,
                                     s.pool, s.idx, s.out, workspace=s.ws,
                                     gate_mode=s.gate_mode, checkpoints=s.ck,
                                     checkpoint_cu_starts=s.ck_starts,
                                     checkpoint_interval=s.ck_interval, ring=s.ring,
                                     cache_base=s.base, ring_tail=s.ring_tail)
        return [call]


def cpu_baseline_decode(B, budget_s, synth):
    """The CPU oracle on the same decode workload: one full B-row call per
    run; runs repeat until the budget is used (at least one)."""
    import oracle
    case = synth.decode_case(B=B, N=N_SLOTS, H=H)
    W = H * 128
    f32 = synth.f32_from_bits
    # gather the active rows' slots into a compact pool (inactive rows -> -1)
    idx = case["idx"].astype(np.int64)
    active = (idx >= 0) & (idx < N_SLOTS)
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
                sample=f"full T=1 decode call, B={B}, H=12, 1024-slot pool (5% inactive), "
                       f"fp32 oracle with OpenMP over (row, head), median of {len(times)} runs, "
                       f"host {platform.machine()} with {os.cpu_count()} logical CPUs")


def cpu_single_row(synth):
    """The oracle on the single-row workload (B = 1, H = 12, a 4-slot pool,
    state index 2): one T = 1 call, and a 16-step rollout (16 calls in
    sequence on the same slot, each with a token of its own); seconds, median
    of 5 runs each."""
    import oracle
    f32 = synth.f32_from_bits
    case = synth.decode_case(B=16, N=4, H=H, seed=synth.seed_for(0, 1))
    W = H * 128
    q, k, v = (np.ascontiguousarray(f32(case["qkv"][:, i * W:(i + 1) * W]).reshape(16, H, 128))
               for i in range(3))
    gate = np.ascontiguousarray(f32(case["gate"]).reshape(16, H, 128))
    beta = np.ascontiguousarray(f32(case["beta"]))
    base_pool = np.ascontiguousarray(f32(case["pool"]))
    idx = np.array([2], np.int32)

    def steps(n):
        pool = base_pool.copy()
        t0 = time.perf_counter()
        for t in range(n):
            oracle.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], gate[t:t + 1], beta[t:t + 1],
                          case["a_log"], case["dt_bias"], -5.0, 1.0, pool, idx)
        return time.perf_counter() - t0
    one = float(np.median([steps(1) for _ in range(5)]))
    roll = float(np.median([steps(16) for _ in range(5)]))
    return dict(single_call_s=round(one, 6), rollout_16_steps_s=round(roll, 6),
                sample="B=1, H=12, 4-slot pool, state index 2; one T=1 call and a 16-step "
                       "rollout, fp32 oracle, median of 5 runs each")


# ---------------------------------------------------------------------------

def run_profile(torch, kda, synth, pools):
    """Fixed short sequence for rocprofv3, in this dispatch order: 8 decode
    calls (B = 512), then 8 verify calls (B = 512) of each workload in
    VERIFY_TRAFFIC (in its order), then 4 device copies of 402,653,184 B."""
    dec = DecodeSetup(512, torch, kda, synth, pools)
    for c in dec.calls() * 2:
        c()
    torch.cuda.synchronize()
    rings = make_rings(torch, synth)
    for cfg in VERIFY_CFGS:
        if cfg["label"] not in VERIFY_TRAFFIC:
            continue
        kw = {k: v for k, v in cfg.items() if k not in ("label", "T")}
        ver = VerifySetup(512, cfg["T"], torch, kda, synth, pools, rings, **kw)
        for c in ver.calls() * 2:
            c()
        torch.cuda.synchronize()
        del ver
    src, dst = pools
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("profile: 8 x decode B=512; 8 x verify B=512 of each of " + ", ".join(VERIFY_TRAFFIC)
        + "; 4 x copy 402653184 B")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the KDA step shards by rows and heads with no exchange).", file=sys.stderr)
        sys.exit(2)
    import torch

    import gated_delta_rule_step_amd as kda
    from gated_delta_rule_step_amd import synth, workmodel as wm

    kda.lib()
    torch.cuda.init()
    dev_name = torch.cuda.get_device_name(0)
    log(f"bench: device {dev_name}")
    pools = make_pools(torch, synth)

    if args.mode == "profile":
        run_profile(torch, kda, synth, pools)
        return
    if args.mode == "profile-prefill":
        for lens in (synth.DOCS_4, synth.DOCS_14):
            for Hp in (64, 12):
                ps = PrefillSetup(lens, Hp, torch, kda, synth)
                for c in ps.calls() * 4:
                    c()
                torch.cuda.synchronize()
                del ps
        src, dst = pools
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("profile: 4 x prefill at H=64 then H=12, on the 4-document set, then the 14-doc "
            "mix; 4 x copy 402653184 B")
        return

    B = 512
    setup = DecodeSetup(B, torch, kda, synth, pools)
    log(f"bench: decode B={B} set up ({setup.n_active} active rows)")
    wall, ev_ms = time_graphs(setup.calls(), args.steps, args.warmup, torch, min_warm_s=1.0)
    us_wall = wall / args.steps * 1e6
    us_ev = ev_ms * 1e3 / args.steps
    nbytes = wm.decode_bytes(setup.n_active, B - setup.n_active)
    gbs = nbytes / (us_ev * 1e-6) / 1e9
    log(f"bench: decode B={B}: {us_wall:.2f} us/step wall, {us_ev:.2f} us/call (events), "
        f"{gbs:.0f} GB/s")
    dist = launch_percentiles(setup.calls(), 200, torch)
    log(f"bench: decode B={B} per-launch percentiles {dist}")

    points = []
    if args.points == "all":
        for Bp in (1, 8, 32, 128):
            sp = DecodeSetup(Bp, torch, kda, synth, pools, cold=True)
            n = len(sp.combos)
            st = max(256, n)
            _, e = time_graphs(sp.calls(), st, args.warmup, torch, min_warm_s=0.3)
            us = e * 1e3 / st
            nb = wm.decode_bytes(sp.n_active, Bp - sp.n_active)
            points.append(dict(kind="decode", B=Bp, T=1, us_per_call=round(us, 3),
                               GBps=round(nb / (us * 1e-6) / 1e9, 1),
                               hbm_frac=round(nb / (us * 1e-6) / 1e9 / wm.HBM_PEAK_GBS, 4),
                               cold=f"{n} combinations rotated, ~{(n - 1) * nb / 1e6:.0f} MB "
                                    "touched between reuses"))
            log(f"bench: {points[-1]}")
        points.append(dict(kind="decode", B=B, T=1, us_per_call=round(us_ev, 3),
                           GBps=round(gbs, 1), hbm_frac=round(gbs / wm.HBM_PEAK_GBS, 4)))
        # the other gate conventions and the fp16 and fp8 states at the headline size
        f16, f8 = fp16_pools(torch, pools), fp8_pools(torch, pools)
        for gm, variant, pp, sbytes in ((3, dict(gate="pre-computed g and beta"), pools, 2),
                                        (4, dict(gate="per-head gate (GDN-style)"), pools, 2),
                                        (0, dict(state="fp16"), f16, 2),
                                        (0, dict(state="fp8 e4m3"), f8, 1)):
            sp = DecodeSetup(B, torch, kda, synth, pp, gate_mode=gm)
            _, e = time_graphs(sp.calls(), args.steps, args.warmup, torch, min_warm_s=0.3)
            us = e * 1e3 / args.steps
            nb = wm.decode_bytes(sp.n_active, B - sp.n_active, state_bytes=sbytes)
            points.append(dict(kind="decode", B=B, T=1, **variant,
                               us_per_call=round(us, 3), GBps=round(nb / (us * 1e-6) / 1e9, 1),
                               hbm_frac=round(nb / (us * 1e-6) / 1e9 / wm.HBM_PEAK_GBS, 4)))
            log(f"bench: {points[-1]}")
        del f16, f8
        rings = make_rings(torch, synth)
        vcfgs = VERIFY_CFGS
        low = {"fp16": fp16_pools(torch, pools), "fp8": fp8_pools(torch, pools)}
        for Bv in (1, 32, 512):
            for cfg in vcfgs:
                if Bv != 512 and cfg["label"] not in ("T=8 bare (0% fold)", "T=8 fm=9 100% fold"):
                    continue
                kw = {k: v for k, v in cfg.items() if k not in ("label", "T", "state")}
                vs = VerifySetup(Bv, cfg["T"], torch, kda, synth, low.get(cfg.get("state"), pools),
                                 rings, cold=Bv < 512, **kw)
                st = max(args.steps, 256 if Bv < 512 else 100, len(vs.combos))
                _, e = time_graphs(vs.calls(), st, args.warmup, torch, min_warm_s=0.3)
                us = e * 1e3 / st
                nb = wm.verify_bytes(cfg["T"], vs.hist, vs.fold,
                                     state_bytes=1 if cfg.get("state") == "fp8" else 2)
                fl = wm.verify_flops(cfg["T"], vs.hist)
                extra = {}
                if Bv < 512:
                    extra["cold"] = (f"{len(vs.combos)} combinations rotated, "
                                     f"~{(len(vs.combos) - 1) * nb / 1e6:.0f} MB touched between "
                                     "reuses")
                if Bv == 512 and cfg["label"] in VERIFY_TRAFFIC:
                    extra["traffic_bytes"] = counted_traffic(VERIFY_TRAFFIC[cfg["label"]])
                points.append(dict(kind="verify", B=Bv, label=cfg["label"],
                                   fold_frac=round(float(np.mean(vs.fold)), 3),
                                   mean_hist=round(float(np.mean(vs.hist)), 2),
                                   us_per_call=round(us, 3),
                                   GBps=round(nb / (us * 1e-6) / 1e9, 1),
                                   hbm_frac=round(nb / (us * 1e-6) / 1e9 / wm.HBM_PEAK_GBS, 4),
                                   TFLOPs=round(fl / (us * 1e-6) / 1e12, 2), **extra))
                log(f"bench: {points[-1]}")
                del vs
        del rings, low
        torch.cuda.empty_cache()
        d4 = ("4 docs (3840, 3776, 3200, 3072)", synth.DOCS_4)
        pcfgs = [(name, lens, Hp, 0, 0, "bf16", 0)
                 for name, lens in (d4, ("14-doc mix, 16384 tokens", synth.DOCS_14))
                 for Hp in (64, 12)]
        pcfgs += [(*d4, 12, 3, 0, "bf16", 0), (*d4, 12, 4, 0, "bf16", 0),
                  (*d4, 12, 0, 64, "bf16", 0), (*d4, 12, 0, 0, "fp16", 0),
                  (*d4, 12, 0, 0, "fp8", 0), (*d4, 12, 0, 0, "bf16", 8)]
        for name, lens, Hp, gm, cki, sdt, rt in pcfgs:
            ps = PrefillSetup(lens, Hp, torch, kda, synth, gate_mode=gm, ckpt_interval=cki,
                              state=sdt, ring_tail=rt)
            st = max(10, min(args.steps, 50))
            _, e = time_graphs(ps.calls(), st, 2, torch, min_warm_s=0.3)
            us = e * 1e3 / st
            # each checkpoint row writes H states
            sbytes = 1 if sdt == "fp8" else 2
            nb = (wm.prefill_bytes(lens, Hp, state_bytes=sbytes) +
                  ps.ck_rows * Hp * 128 * 128 * sbytes)
            fl = wm.prefill_flops(lens, Hp)
            extra = {"gate": {3: "pre-computed g and beta", 4: "per-head gate (GDN-style)"}[gm]} \
                if gm else {}
            if cki:
                extra["checkpoints"] = f"every {cki} tokens ({ps.ck_rows} rows)"
            if sdt != "bf16":
                extra["state"] = sdt
            if rt:
                extra["handoff"] = f"last {rt} tokens of each document to the verify ring"
            if not (gm or cki or rt) and sdt == "bf16":
                extra["kernels"] = ("fused 64-token chunk kernel"
                                    if len(lens) * Hp >= kda.FUSED_MIN_CHAINS
                                    else "preparation + chain (16-token chunks, workspace)")
                extra["traffic_bytes"] = counted_traffic(f"prefill {name} H={Hp}")
            points.append(dict(kind="prefill", H=Hp, docs=name, tokens=int(sum(lens)),
                               **extra, us_per_call=round(us, 1),
                               Mtok_per_s=round(sum(lens) / (us * 1e-6) / 1e6, 2),
                               GBps=round(nb / (us * 1e-6) / 1e9, 1),
                               hbm_frac=round(nb / (us * 1e-6) / 1e9 / wm.HBM_PEAK_GBS, 4),
                               TFLOPs=round(fl / (us * 1e-6) / 1e12, 2),
                               mfma_frac=round(fl / (us * 1e-6) / 1e12
                                               / wm.BF16_MFMA_PEAK_TFLOPS, 4)))
            log(f"bench: {points[-1]}")
            del ps
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        cpu = cpu_baseline_decode(B, args.cpu_budget_s, synth)
        cpu["single_row_workload"] = cpu_single_row(synth)
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
        "config": {"workload": "kda_decode T=1, B=512, H=12, K=V=128, bf16 pool of 1024 slots, "
                               "5% inactive rows, q/k/v strided views of packed rows",
                   "B": B, "H": H, "T": 1, "pool_slots": N_SLOTS, "device": dev_name},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": wm.HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / wm.HBM_PEAK_GBS, 4),
                     "traffic": counted_traffic("decode B=512"),
                     "kernel": "kda::decode_kernel<4, true, 0, 0>",
                     "kernel_us_avg": round(us_ev, 3), "kernel_us_percentiles": dist,
                     "algorithmic_bytes": nbytes},
        "cpu_baseline": cpu,
        "points": points,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
