"""Seeded synthetic inputs for the KDA step: shapes and value distributions only.

This module holds no arithmetic of the method. It draws random numbers
(numpy PCG64), quantises them to bf16 with torch's own fp32 -> bfloat16 cast,
and lays them out the way the C-ABI consumes them. Both the GPU tests and the
CPU oracle consume the same arrays.

Distributions (all workloads): q, k, v, raw gate and beta logits ~ N(0, 1) in
bf16; A_log ~ U(-1, 1) fp32 per head; dt_bias ~ N(0, 0.1) fp32 per key
channel; pool state ~ N(0, 0.05) in bf16. Seeds follow
seed = 20261202 + 1000 * workload + 10 * B + T; pools of more than 64 slots
come from one seeded pool per (N, H), cached within a process.

Layouts (all C-contiguous; bf16 tensors are uint16 arrays of bf16 bits):
  decode  qkv [B, 3*H*128] = [q | k | v] per row, gate [B, H*128], beta [B, H]
  verify  qkv [B, T, 3*H*128], gate [B, T, H*128], beta [B, T, H]
  prefill q, k [Ttot, H, 128], v [Ttot, H, 128], gate [Ttot, H*128], beta [Ttot, H]
  pool [N, H, 128 (V), 128 (K)]; rings k/g [N, H, R, 128], u [N, H, R, 128].
"""
from __future__ import annotations

import functools

import numpy as np
import torch

HEAD_DIM = 128
BASE_SEED = 20261202

# Fourteen-document mix summing to 16384 tokens with ragged chunk tails (the
# pages quote a 14-document prefill workload without its lengths).
DOCS_14 = (4096, 3000, 2048, 1500, 1200, 1024, 1000, 700, 600, 500, 300, 217, 128, 71)
# Four documents of the context-parallel forward-state walk workload.
DOCS_4 = (3840, 3776, 3200, 3072)


def seed_for(workload: int, B: int = 0, T: int = 0) -> int:
    return BASE_SEED + 1000 * workload + 10 * B + T


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bits (uint16) using torch's fp32 -> bfloat16 cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def f32_from_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) -> the exact float32 values they encode."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng, shape, std=1.0):
    return bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def gate_params(rng, H: int):
    a_log = rng.uniform(-1.0, 1.0, size=H).astype(np.float32)
    dt_bias = (rng.standard_normal(size=H * HEAD_DIM, dtype=np.float32) * np.float32(0.1))
    return a_log, dt_bias.astype(np.float32)


def pool_bits(rng, N: int, H: int, std: float = 0.05, chunk_slots: int = 64) -> np.ndarray:
    out = np.empty((N, H, HEAD_DIM, HEAD_DIM), dtype=np.uint16)
    for s in range(0, N, chunk_slots):
        e = min(N, s + chunk_slots)
        out[s:e] = _normal_bf16(rng, (e - s, H, HEAD_DIM, HEAD_DIM), std)
    return out


@functools.lru_cache(maxsize=2)
def _pool_cached(N: int, H: int, seed: int) -> np.ndarray:
    p = pool_bits(np.random.Generator(np.random.PCG64(seed)), N, H)
    p.setflags(write=False)
    return p


def shared_pool(N: int, H: int) -> np.ndarray:
    """A seeded N(0, 0.05) bf16 pool of N slots (a fresh writable copy of a
    per-process cached array; the pool's seed depends on N and H only)."""
    return _pool_cached(N, H, BASE_SEED + 7 * N + H).copy()


def filler_bits(shape, salt: int = 0) -> np.ndarray:
    """Cheap deterministic bf16 bit patterns for memory that must stay
    untouched (any values, including NaN and inf encodings)."""
    n = int(np.prod(shape))
    x = (np.arange(n, dtype=np.uint64) * np.uint64(2654435761) + np.uint64(salt)) >> np.uint64(13)
    return (x & np.uint64(0xFFFF)).astype(np.uint16).reshape(shape)


def state_indices(rng, B: int, N: int, inactive_frac: float = 0.05) -> np.ndarray:
    """First B entries of a seeded permutation of 0..N-1 (B <= N); then
    round(inactive_frac * B) seeded positions set alternately to -1 and N + r."""
    if B <= N:
        idx = rng.permutation(N)[:B].astype(np.int64)
    else:  # more rows than slots: only the first N rows can be distinct
        idx = np.concatenate([rng.permutation(N), np.full(B - N, -1)]).astype(np.int64)
    n_bad = int(round(inactive_frac * B))
    if n_bad:
        pos = rng.choice(B, size=n_bad, replace=False)
        for i, p in enumerate(sorted(pos)):
            idx[p] = -1 if i % 2 == 0 else N + int(rng.integers(0, 1000))
    return idx.astype(np.int32)


def precomputed_gate(case: dict, gate_mode: int, seed: int, g_low: float = -6.0) -> dict:
    """A copy of a decode, verify or prefill case whose gate and / or beta
    inputs follow the pre-computed convention (gate_mode bit 1: the log-decay
    itself, drawn U(g_low, 0.5), by default U(-6, 0.5) so that some values lie
    outside [-5, 0]; bit 2: beta itself, drawn U(0, 1)), as bf16 bits;
    case["gate_mode"] records it."""
    rng = np.random.Generator(np.random.PCG64(seed))
    c = dict(case)
    c["gate_mode"] = int(gate_mode)
    if gate_mode & 1:
        c["gate"] = bf16_bits(rng.uniform(g_low, 0.5, case["gate"].shape).astype(np.float32))
    if gate_mode & 2:
        c["beta"] = bf16_bits(rng.uniform(0.0, 1.0, case["beta"].shape).astype(np.float32))
    return c


def per_head_gate(case: dict, precomputed: bool, seed: int) -> dict:
    """A copy of a decode, verify or prefill case with one gate value per token
    and head (gate_mode bit 4): raw logits N(0, 1) with dt_bias N(0, 0.1) per
    head, or pre-computed log-decays U(-6, 0.5) (gate_mode bit 1 as well)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    c = dict(case)
    H = case["H"]
    shape = case["gate"].shape[:-1] + (H,)
    if precomputed:
        c["gate"] = bf16_bits(rng.uniform(-6.0, 0.5, shape).astype(np.float32))
    else:
        c["gate"] = _normal_bf16(rng, shape)
        c["dt_bias"] = (rng.standard_normal(H) * 0.1).astype(np.float32)
    c["gate_mode"] = case.get("gate_mode", 0) | 4 | (1 if precomputed else 0)
    return c


def fp16_state(case: dict) -> dict:
    """A copy of a decode, verify or prefill case whose pool holds fp16 state
    (state_dtype 1): the same state values, stored as binary16 bits."""
    c = dict(case)
    c["pool"] = f32_from_bits(case["pool"]).astype(np.float16).view(np.uint16)
    c["state_dtype"] = 1
    return c


def fp8_state(case: dict) -> dict:
    """A copy of a decode, verify or prefill case whose pool holds fp8 e4m3
    state (state_dtype 2): the state values cast with torch's float8_e4m3fn
    conversion (the N(0, 0.05) values lie far inside its +-448 range), stored
    as bytes."""
    c = dict(case)
    x = torch.from_numpy(np.ascontiguousarray(f32_from_bits(case["pool"])))
    c["pool"] = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    c["state_dtype"] = 2
    return c


def decode_case(B: int, N: int = 1024, H: int = 12, seed: int | None = None,
                inactive_frac: float = 0.05, idx: np.ndarray | None = None) -> dict:
    rng = np.random.Generator(np.random.PCG64(seed_for(1, B) if seed is None else seed))
    W = H * HEAD_DIM
    case = dict(B=B, H=H, N=N, lower_bound=-5.0, scale=1.0)
    case["qkv"] = _normal_bf16(rng, (B, 3 * W))
    case["gate"] = _normal_bf16(rng, (B, W))
    case["beta"] = _normal_bf16(rng, (B, H))
    case["a_log"], case["dt_bias"] = gate_params(rng, H)
    case["pool"] = pool_bits(rng, N, H) if N <= 64 else shared_pool(N, H)
    case["idx"] = state_indices(rng, B, N, inactive_frac) if idx is None else np.asarray(idx, np.int32)
    return case


def verify_case(B: int, T: int, N: int = 1024, H: int = 12, R: int = 32, w_ring: int = 16,
                flush_min: int | None = None, fold_p: float = 0.0, seed: int | None = None,
                workload: int = 2, inactive_frac: float = 0.0,
                hist_max: int | None = None) -> dict:
    """Draft-token inputs plus per-row hist_len / cache_base. Rows fold with
    probability fold_p, or, when hist_max is given, hist ~ U{0..hist_max}. The ring contents
    are left empty (zeros); callers fill history rows (the tests run the oracle
    over seeded history tokens, the benchmark uses synthetic_rings)."""
    if flush_min is None:
        flush_min = {8: 9, 4: 13}.get(T, w_ring - T + 1)
    rng = np.random.Generator(np.random.PCG64(seed_for(workload, B, T) if seed is None else seed))
    W = H * HEAD_DIM
    case = dict(B=B, T=T, H=H, N=N, R=R, w_ring=w_ring, flush_min=flush_min,
                lower_bound=-5.0, scale=1.0)
    case["qkv"] = _normal_bf16(rng, (B, T, 3 * W))
    case["gate"] = _normal_bf16(rng, (B, T, W))
    case["beta"] = _normal_bf16(rng, (B, T, H))
    case["a_log"], case["dt_bias"] = gate_params(rng, H)
    case["pool"] = pool_bits(rng, N, H) if N <= 64 else shared_pool(N, H)
    case["idx"] = state_indices(rng, B, N, inactive_frac)
    # Fold rows draw hist in [max(0, fm - T), min(fm - 1, w_ring - T)]; the rest
    # draw hist in [0, fm - T - 1] (empty when fm <= T: then every row folds).
    fold_hi = min(flush_min - 1, w_ring - T)
    fold_lo = max(0, flush_min - T)
    fold = rng.random(B) < fold_p
    hist = np.zeros(B, np.int64)
    for b in range(B):
        if hist_max is not None:  # uniform history length, fold decided by hist
            hist[b] = rng.integers(0, hist_max + 1)
        elif fold[b] or flush_min - T - 1 < 0:
            hist[b] = rng.integers(fold_lo, fold_hi + 1) if fold_hi >= fold_lo else 0
        else:
            hist[b] = rng.integers(0, flush_min - T)
    case["hist_len"] = hist.astype(np.int32)
    case["cache_base"] = rng.integers(0, R, size=B).astype(np.int32)
    case["k_cache"] = np.zeros((N, H, R, HEAD_DIM), np.uint16)
    case["u_cache"] = np.zeros((N, H, R, HEAD_DIM), np.uint16)
    case["g_cache"] = np.zeros((N, H, R, HEAD_DIM), np.float32)
    case["hist_rng_seed"] = int(rng.integers(0, 2**31 - 1))
    return case


def synthetic_rings(shape, seed: int):
    """Ring arrays (k_cache, u_cache bf16 bits; g_cache fp32) of `shape`
    [N, H, R, 128] with plausible magnitudes: keys ~ U(-0.15, 0.15),
    corrections ~ U(-0.5, 0.5), cumulative log-decay decreasing along the ring
    by U(0, 2) per row. For timing only: no state was stepped to make them."""
    rng = np.random.Generator(np.random.PCG64(seed))
    N = shape[0]
    kc = np.empty(shape, np.uint16)
    uc = np.empty(shape, np.uint16)
    gc = np.empty(shape, np.float32)
    for s in range(0, N, 64):
        e = min(N, s + 64)
        sub = (e - s,) + tuple(shape[1:])
        kc[s:e] = bf16_bits(rng.random(sub, dtype=np.float32) * np.float32(0.3) - np.float32(0.15))
        uc[s:e] = bf16_bits(rng.random(sub, dtype=np.float32) - np.float32(0.5))
        gc[s:e] = -np.cumsum(rng.random(sub, dtype=np.float32) * np.float32(2.0), axis=2,
                             dtype=np.float32)
    return kc, uc, gc


def history_tokens(case: dict, n_tok: int) -> dict:
    """Seeded raw inputs for n_tok history tokens per row (same distributions
    as draft tokens): qkv [B, n_tok, 3*H*128], gate [B, n_tok, H*128], beta [B, n_tok, H]."""
    rng = np.random.Generator(np.random.PCG64(case["hist_rng_seed"]))
    B, H = case["B"], case["H"]
    W = H * HEAD_DIM
    return dict(qkv=_normal_bf16(rng, (B, n_tok, 3 * W)), gate=_normal_bf16(rng, (B, n_tok, W)),
                beta=_normal_bf16(rng, (B, n_tok, H)))


def prefill_case(doc_lens, H: int = 64, seed: int | None = None, n_slots: int | None = None,
                 use_initial_state: bool = True, inactive_docs=()) -> dict:
    doc_lens = tuple(int(x) for x in doc_lens)
    n_docs = len(doc_lens)
    Ttot = int(sum(doc_lens))
    rng = np.random.Generator(np.random.PCG64(seed_for(4, H, n_docs) if seed is None else seed))
    N = 2 * max(n_docs, 1) if n_slots is None else n_slots
    case = dict(n_docs=n_docs, H=H, N=N, Ttot=Ttot, lower_bound=-5.0, scale=1.0,
                use_initial_state=use_initial_state)
    cu = np.zeros(n_docs + 1, np.int32)
    cu[1:] = np.cumsum(doc_lens)
    case["cu_seqlens"] = cu
    case["q"] = _normal_bf16(rng, (Ttot, H, HEAD_DIM))
    case["k"] = _normal_bf16(rng, (Ttot, H, HEAD_DIM))
    case["v"] = _normal_bf16(rng, (Ttot, H, HEAD_DIM))
    case["gate"] = _normal_bf16(rng, (Ttot, H * HEAD_DIM))
    case["beta"] = _normal_bf16(rng, (Ttot, H))
    case["a_log"], case["dt_bias"] = gate_params(rng, H)
    case["pool"] = pool_bits(rng, N, H)
    idx = rng.permutation(N)[:n_docs].astype(np.int32) if N >= n_docs else \
        np.arange(n_docs, dtype=np.int32)
    for d in inactive_docs:
        idx[d] = -1
    case["idx"] = idx
    return case
