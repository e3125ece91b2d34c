"""Shared helpers for the GPU parity tests: device transfer of bf16 bit arrays,
the parity criteria, and oracle runs over the touched pool slots only."""
from __future__ import annotations

import numpy as np

from gated_delta_rule_step_amd import synth

f32 = synth.f32_from_bits
HD = 128

# Parity criteria for floating-point results:
#  * outputs: |got - ref| <= 1e-2 + 1.6e-2 |ref| element-wise;
#  * stored bf16 state / ring rows: |got - ref| <= 2 bf16 ulps of
#    max(|ref|, 2^-12) (the floor covers elements that cancel to ~0);
#  * cumulative log-decay (fp32): |got - ref| <= 1e-5 + 1e-5 |ref|.
OUT_ATOL, OUT_RTOL = 1e-2, 1.6e-2
# Next to the element-wise test, a normwise one: ||got - ref||_2 <= NORM * ||ref||_2
# over the outputs compared. At the configs' inputs the outputs are small (median
# |o| ~ 0.025), where the element-wise bound is dominated by OUT_ATOL; the normwise
# bound is the one that sees a systematic error of a few per mille. Decode and
# verify keep fp32 (or split-bf16) state products: 2e-3, about one bf16 rounding of
# every element; prefill's output path takes single-term bf16 products: 5e-3.
OUT_NORM = 2e-3
OUT_NORM_PREFILL = 5e-3
STATE_ULPS, STATE_FLOOR = 2, 2.0 ** -12


def dev_bf16(a, device="cuda"):
    import torch
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)


def dev(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bits(t) -> np.ndarray:
    """A tensor's bit patterns: uint16 for 2-byte elements, uint8 for fp8."""
    import torch
    if t.element_size() == 1:
        return t.detach().contiguous().view(torch.uint8).cpu().numpy()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_ulp(x):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), STATE_FLOOR))) - 7)


# fp16 state (state_dtype 1): 2 fp16 ulps of max(|ref|, 2^-9). The floor gives
# the same absolute allowance near zero as the bf16 criterion (2 * 2^-12 *
# 2^-7 = 2^-18): that allowance covers the arithmetic's error, which does not
# depend on the storage format; above 2^-9 the check is 8 times tighter than
# the bf16 one.
STATE_FLOOR_F16 = 2.0 ** -9


def f16_ulp(x):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), STATE_FLOOR_F16))) - 10)


# fp8 e4m3 state (state_dtype 2): 1 fp8 ulp of max(|ref|, 2^-6), the smallest
# normal (below it the spacing is the subnormal 2^-9). The oracle rounds to
# fp8 at the same storage points, and the fp32 arithmetic differs between the
# two sides by far less than one fp8 step, so a stored element differs by at
# most the one step a value near a rounding boundary can fall either way.
STATE_FLOOR_F8 = 2.0 ** -6
STATE_ULPS_F8 = 1


def f8_ulp(x):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), STATE_FLOOR_F8))) - 3)


# Pools of any state element type (case["state_dtype"]: 0 bf16, 1 fp16, 2 fp8).
def pool_vals(case, pool_bits):
    """The values a pool's bit patterns hold, as float32."""
    sd = case.get("state_dtype", 0)
    if sd == 1:
        return np.ascontiguousarray(pool_bits).view(np.float16).astype(np.float32)
    if sd == 2:
        import torch
        b = torch.from_numpy(np.ascontiguousarray(pool_bits, dtype=np.uint8))
        return b.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    return f32(pool_bits)


def pool_dev(case, pool_bits, device="cuda"):
    import torch
    sd = case.get("state_dtype", 0)
    if sd == 1:
        a = np.ascontiguousarray(pool_bits)
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.float16)
    if sd == 2:
        a = np.ascontiguousarray(pool_bits, dtype=np.uint8)
        return torch.from_numpy(a).to(device).view(torch.float8_e4m3fn)
    return dev_bf16(pool_bits, device)


def check_pool(case, got_bits, ref, what="state"):
    """check_state in the pool's element type: 2 ulps of that type above its floor."""
    sd = case.get("state_dtype", 0)
    if not sd:
        return check_state(got_bits, ref, what)
    got = pool_vals(case, got_bits).astype(np.float64).reshape(ref.shape)
    ref = ref.astype(np.float64)
    tol = STATE_ULPS * f16_ulp(ref) if sd == 1 else STATE_ULPS_F8 * f8_ulp(ref)
    bad = ~(np.abs(got - ref) <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, np.abs(got - ref) / tol, -np.inf)),
                             ref.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements beyond "
                             f"{STATE_ULPS if sd == 1 else STATE_ULPS_F8} {'fp16' if sd == 1 else 'fp8'} ulps; worst at "
                             f"{i}: got {got[i]!r} "
                             f"ref {ref[i]!r}")


def normwise_error(got, ref) -> float:
    """||got - ref||_2 / ||ref||_2 (0 when both are zero)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(got - ref))
    return num / den if den > 0 else (0.0 if num == 0 else np.inf)


def check_out(got_bits, ref, what="output", norm=OUT_NORM):
    got = f32(got_bits).astype(np.float64).reshape(ref.shape)
    ref = ref.astype(np.float64)
    excess = np.abs(got - ref) - (OUT_ATOL + OUT_RTOL * np.abs(ref))
    bad = ~(excess <= 0)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, excess, -np.inf)), ref.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; "
                             f"worst at {i}: got {got[i]!r} ref {ref[i]!r}")
    e = normwise_error(got, ref)
    if not e <= norm:
        raise AssertionError(f"{what}: normwise error {e:.3e} above {norm:.1e}")


def check_state(got_bits, ref, what="state"):
    got = f32(got_bits).astype(np.float64).reshape(ref.shape)
    ref = ref.astype(np.float64)
    tol = STATE_ULPS * bf16_ulp(ref)
    bad = ~(np.abs(got - ref) <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, np.abs(got - ref) / tol, -np.inf)),
                             ref.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements beyond "
                             f"{STATE_ULPS} bf16 ulps; worst at {i}: got {got[i]!r} "
                             f"ref {ref[i]!r}")


def check_gcache(got, ref, what="g_cache"):
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    bad = ~(np.abs(got - ref) <= 1e-5 + 1e-5 * np.abs(ref))
    if bad.any():
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance")


def compact_slots(idx, N):
    """Map the active rows' slots onto a compact pool: returns (slots, cidx)
    where slots lists the distinct active slots and cidx indexes them (-1 for
    inactive rows)."""
    idx = np.asarray(idx, np.int64)
    active = (idx >= 0) & (idx < N)
    slots = idx[active]
    cidx = np.full(idx.shape, -1, np.int32)
    cidx[active] = np.arange(slots.size, dtype=np.int32)
    return slots, cidx


def split_qkv(qkv_bits, H):
    """Packed [..., 3*H*128] rows -> float32 q, k, v of shape [..., H, 128]."""
    W = H * HD
    q = f32(qkv_bits[..., :W]).reshape(*qkv_bits.shape[:-1], H, HD)
    k = f32(qkv_bits[..., W:2 * W]).reshape(*qkv_bits.shape[:-1], H, HD)
    v = f32(qkv_bits[..., 2 * W:]).reshape(*qkv_bits.shape[:-1], H, HD)
    return np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v)


def oracle_decode(orc, case, pool_bits=None):
    """Run the fp32 oracle on a decode case over its touched slots.
    Returns (out [B,H,128] f32, slots, new_state[len(slots),H,128,128] f32)."""
    H, N = case["H"], case["N"]
    pool_bits = case["pool"] if pool_bits is None else pool_bits
    slots, cidx = compact_slots(case["idx"], N)
    cpool = np.ascontiguousarray(pool_vals(case, pool_bits[slots]))
    q, k, v = split_qkv(case["qkv"], H)
    gm = case.get("gate_mode", 0)
    a_log, dt_bias = (None, None) if gm & 1 else (case["a_log"], case["dt_bias"])
    gshape = (-1, H) if gm & 4 else (-1, H, HD)  # per-head gate: one value per head
    out = orc.decode(q, k, v, np.ascontiguousarray(f32(case["gate"]).reshape(gshape)),
                     np.ascontiguousarray(f32(case["beta"])), a_log, dt_bias,
                     case["lower_bound"], case["scale"], cpool, cidx, bf16_storage=True,
                     real=np.float32, gate_mode=gm, state_dtype=case.get("state_dtype", 0))
    return out, slots, cpool


def report_accuracy(name: str, **figures) -> None:
    """Append accuracy figures (e.g. normwise errors against an fp64 oracle run)
    as one JSON line to the file named by KDA_ACCURACY_LOG, if set, and print them."""
    import json
    import os
    line = json.dumps(dict(test=name, **{k: float(v) for k, v in figures.items()}))
    print(line)
    path = os.environ.get("KDA_ACCURACY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")
