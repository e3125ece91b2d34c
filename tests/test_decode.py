"""GPU parity of kda_decode (T = 1) against the CPU oracle, through the C ABI.

Operation: "feat(kda): add packed-input CuTe decode kernel" -- packed bf16 QKV
rows, raw gate and beta logits, bf16 pool updated in place, out-of-range
state indices give zero output and leave the pool untouched.
"""
import numpy as np
import pytest

from gated_delta_rule_step_amd import synth
from tests.helpers import (HD, bits, check_out, check_pool, check_state, dev, dev_bf16, f32,
                           oracle_decode, pool_dev, split_qkv)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

INT32_MIN, INT32_MAX = -(2 ** 31), 2 ** 31 - 1


def _kda():
    import gated_delta_rule_step_amd as kda
    return kda


def run_decode(case, pool=None, out=None, scale=None, lower_bound=None, stream=None):
    """Launch kda_decode on a case; q/k/v are views of one packed row."""
    H = case["H"]
    W = H * HD
    qkv = dev_bf16(case["qkv"])
    pool = pool_dev(case, case["pool"]) if pool is None else pool
    B = case["B"]
    if out is None:
        out = torch.full((B, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    gm = case.get("gate_mode", 0)
    a_log, dt_bias = (None, None) if gm & 1 else (dev(case["a_log"]), dev(case["dt_bias"]))
    _kda().kda_decode(qkv[:, :W], qkv[:, W:2 * W], qkv[:, 2 * W:], dev_bf16(case["gate"]),
                      dev_bf16(case["beta"]), a_log, dt_bias, pool,
                      dev(case["idx"]), out,
                      lower_bound=case["lower_bound"] if lower_bound is None else lower_bound,
                      scale=case["scale"] if scale is None else scale, gate_mode=gm,
                      stream=stream)
    return pool, out


def check_case(orc, case, pool_dev, out_dev):
    ref_out, slots, ref_state = oracle_decode(orc, case)
    torch.cuda.synchronize()
    got_pool = bits(pool_dev)
    check_out(bits(out_dev), ref_out, "decode output")
    check_pool(case, got_pool[slots], ref_state, "decode state")
    untouched = np.ones(case["N"], bool)
    untouched[slots] = False
    assert np.array_equal(got_pool[untouched], case["pool"][untouched]), \
        "slots of inactive rows or unused slots changed"
    active = np.isin(np.arange(case["B"]), np.nonzero(
        (case["idx"] >= 0) & (case["idx"] < case["N"]))[0])
    ob = bits(out_dev).reshape(case["B"], -1)
    assert np.all(ob[~active] == 0), "inactive rows must output +0.0"


@pytest.mark.parametrize("gate_mode,B", [(1, 512), (2, 512), (3, 512), (3, 32)])
def test_precomputed_gate_conventions(orc, gate_mode, B):
    """[decode] "T=1 fast path inside recurrent_kda": the pre-computed form
    (log-space g, decay = exp(g); pre-sigmoided beta), alone or together, at
    B = 512 (and 32) with 5 % inactive rows; A_log and dt_bias are not passed
    when the gate is pre-computed."""
    case = synth.precomputed_gate(synth.decode_case(B=B, H=12), gate_mode,
                                  synth.seed_for(1, B, 100 + gate_mode))
    pool, out = run_decode(case)
    check_case(orc, case, pool, out)


@pytest.mark.parametrize("gate_mode,B", [(1, 64), (3, 512), (5, 64)])
def test_no_decay_floor(orc, gate_mode, B):
    """lower_bound = -INFINITY with pre-computed log-decays drawn U(-20, 0.5):
    no floor, decays down to exp(-20) (per channel, and per head with bit 4)."""
    case = synth.decode_case(B=B, H=12)
    if gate_mode & 4:
        case = synth.per_head_gate(case, True, synth.seed_for(1, B, 170))
        rng = np.random.Generator(np.random.PCG64(synth.seed_for(1, B, 171)))
        case["gate"] = synth.bf16_bits(rng.uniform(-20.0, 0.5, case["gate"].shape)
                                       .astype(np.float32))
    else:
        case = synth.precomputed_gate(case, gate_mode, synth.seed_for(1, B, 172), g_low=-20.0)
    case["lower_bound"] = -np.inf
    pool, out = run_decode(case)
    check_case(orc, case, pool, out)


@pytest.mark.parametrize("B", [1, 32, 512])
def test_fp16_state(orc, B):
    """An fp16 state pool (state_dtype 1), B = 1, 32 and 512 (the three tile
    sizes) with inactive rows:
    the state is read and written as binary16, outputs stay bf16."""
    case = synth.fp16_state(synth.decode_case(B=B, H=12))
    pool, out = run_decode(case)
    check_case(orc, case, pool, out)


@pytest.mark.parametrize("B", [1, 32, 512])
def test_fp8_state(orc, B):
    """An fp8 e4m3 state pool (state_dtype 2), B = 1, 32 and 512 (the three
    tile sizes) with inactive rows: the state is read and written as one byte per element (round to
    nearest even, saturating), outputs stay bf16."""
    case = synth.fp8_state(synth.decode_case(B=B, H=12))
    pool, out = run_decode(case)
    check_case(orc, case, pool, out)


@pytest.mark.parametrize("pre,B", [(False, 512), (True, 512), (False, 32)])
def test_per_head_gate(orc, pre, B):
    """The per-head (scalar, GDN-style) gate, raw and pre-computed, at B = 512
    (and 32): gate [B, H] and dt_bias [H]."""
    case = synth.per_head_gate(synth.decode_case(B=B, H=12), pre,
                               synth.seed_for(1, B, 120 + int(pre)))
    pool, out = run_decode(case)
    check_case(orc, case, pool, out)


def test_single_row_slot2_of_4(orc):
    """One row, a 4-slot pool, index 2: slots 0, 1, 3 stay bitwise untouched."""
    case = synth.decode_case(B=1, N=4, H=12, seed=synth.seed_for(0, 1), idx=[2])
    pool, out = run_decode(case)
    check_case(orc, case, pool, out)


def test_rollout_16_steps_teacher_forced(orc):
    """16 consecutive decode calls on slot 2; each step is checked against the
    oracle stepping from the GPU's previous state. The free-running drift of
    the bf16 state against an fp64 oracle run is reported."""
    case = synth.decode_case(B=1, N=4, H=12, seed=synth.seed_for(0, 1), idx=[2])
    pool = dev_bf16(case["pool"])
    ref64 = f32(case["pool"][[2]]).astype(np.float64)
    rng = np.random.Generator(np.random.PCG64(synth.seed_for(0, 1, 16)))
    for step in range(16):
        tok = synth.decode_case(B=1, N=4, H=12, seed=int(rng.integers(2 ** 31)), idx=[2])
        tok["pool"] = bits(pool)
        prev = tok["pool"].copy()
        _, out = run_decode(tok, pool=pool)
        torch.cuda.synchronize()
        ref_out, slots, ref_state = oracle_decode(orc, tok, pool_bits=prev)
        check_out(bits(out), ref_out, f"rollout step {step} output")
        check_state(bits(pool)[slots], ref_state, f"rollout step {step} state")
        q, k, v = split_qkv(tok["qkv"], 12)
        orc.decode(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                   f32(tok["gate"]).reshape(1, 12, HD).astype(np.float64),
                   f32(tok["beta"]).astype(np.float64), tok["a_log"].astype(np.float64),
                   tok["dt_bias"].astype(np.float64), -5.0, 1.0, ref64,
                   np.zeros(1, np.int32), bf16_storage=False, real=np.float64)
    got = f32(bits(pool)[2]).astype(np.float64)
    err = got - ref64[0]
    rms = np.sqrt(np.mean(ref64[0] ** 2))
    normwise = np.linalg.norm(err) / np.linalg.norm(ref64[0])
    print(f"16-step free-running drift vs fp64: normwise {normwise:.3e}, "
          f"max |err| / rms(state) {np.abs(err).max() / rms:.3e}")
    # bf16 storage rounds the state once per step (relative 2^-9): after 16
    # steps the normwise drift stays at the level of a few roundings
    assert normwise < 2e-2


@pytest.mark.parametrize("B", [1, 8, 32, 128, 512])
def test_batch_sweep_packed_rows(orc, B):
    """Pool of 1024 slots, a seeded permutation subset with 5% of rows
    inactive (-1 or >= N); q/k/v are views of one packed row."""
    case = synth.decode_case(B=B, N=1024, H=12)
    pool, out = run_decode(case)
    check_case(orc, case, pool, out)


@pytest.mark.parametrize("B,H", [(64, 2), (255, 2), (513, 2), (70, 5)])
def test_two_heads_large_pool(orc, B, H):
    """Two (or five) heads: four (ten) workgroups per row, all on one XCD from
    64 rows on; a 3000-slot pool, 5 % inactive rows and INT32_MIN / INT32_MAX
    indices."""
    case = synth.decode_case(B=B, N=3000, H=H, seed=synth.seed_for(1, B, 130 + H))
    case["idx"][[3, 10]] = [INT32_MIN, INT32_MAX]
    pool, out = run_decode(case)
    check_case(orc, case, pool, out)


def test_extreme_indices_and_all_inactive(orc):
    case = synth.decode_case(B=6, N=8, H=12, seed=11, idx=[INT32_MIN, 3, INT32_MAX, 8, -1, 0])
    pool, out = run_decode(case)
    check_case(orc, case, pool, out)
    dead = synth.decode_case(B=5, N=8, H=12, seed=12, idx=[-1, 8, INT32_MIN, INT32_MAX, 9])
    pool, out = run_decode(dead)
    torch.cuda.synchronize()
    assert np.array_equal(bits(pool), dead["pool"])
    assert np.all(bits(out) == 0)


def test_empty_pool_gives_zero_output(orc):
    case = synth.decode_case(B=3, N=1, H=12, seed=13, idx=[0, 1, -1])
    case["pool"] = case["pool"][:0]
    case["N"] = 0
    empty = torch.empty((0, 12, HD, HD), dtype=torch.bfloat16, device="cuda")
    _, out = run_decode(case, pool=empty)
    torch.cuda.synchronize()
    assert np.all(bits(out) == 0)


def test_read_out_scale_and_other_head_counts(orc):
    case = synth.decode_case(B=7, N=16, H=5, seed=14, inactive_frac=0.0)
    case["scale"] = 128 ** -0.5
    pool, out = run_decode(case)
    check_case(orc, case, pool, out)


@pytest.mark.parametrize("B,N", [(4, 6), (9, 6), (350, 360)])
def test_misaligned_views_odd_strides_and_padded_pool(orc, B, N):
    """Unaligned bases and odd strides take the scalar path (at each of its
    tile sizes); the pool has padded slots (slot stride > H*128*128, odd)."""
    H = 12
    case = synth.decode_case(B=B, N=N, H=H, seed=15 + B, inactive_frac=0.2)
    W = H * HD
    rs = 3 * W + 3  # odd row stride
    buf = torch.zeros(B * rs + 8, dtype=torch.bfloat16, device="cuda")
    rows = buf[1:1 + B * rs].view(B, rs)  # base offset by one element
    rows[:, :3 * W] = dev_bf16(case["qkv"])
    gbuf = torch.zeros(B * (W + 5) + 1, dtype=torch.bfloat16, device="cuda")
    gate = gbuf[1:1 + B * (W + 5)].view(B, W + 5)[:, :W]
    gate.copy_(dev_bf16(case["gate"]))
    ss = H * HD * HD + 7
    pbuf = torch.full((N * ss + 1,), 3.0, dtype=torch.bfloat16, device="cuda")
    pool = pbuf[1:1 + N * ss].view(N, ss)
    pool[:, :H * HD * HD] = dev_bf16(case["pool"].reshape(N, -1))
    obuf = torch.full((B * (W + 3) + 1,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = obuf[1:1 + B * (W + 3)].view(B, W + 3)[:, :W]
    dtb_buf = torch.zeros(H * HD + 1, dtype=torch.float32, device="cuda")
    dtb_buf[1:] = dev(case["dt_bias"])
    _kda().kda_decode(rows[:, :W], rows[:, W:2 * W], rows[:, 2 * W:3 * W], gate,
                      dev_bf16(case["beta"]), dev(case["a_log"]), dtb_buf[1:], pool,
                      dev(case["idx"]), out)
    torch.cuda.synchronize()
    ref_out, slots, ref_state = oracle_decode(orc, case)
    check_out(bits(out), ref_out, "misaligned decode output")
    pb = bits(pool)
    check_state(pb[slots, :H * HD * HD].reshape(-1, H, HD, HD), ref_state,
                "misaligned decode state")
    # padding and guard elements are untouched
    assert np.all(f32(pb[:, H * HD * HD:]) == 3.0)
    assert np.all(np.isnan(f32(bits(obuf)[1:].reshape(B, W + 3)[:, W:])))
    assert np.isnan(f32(bits(obuf)[:1])).all()


def test_guard_bands_untouched_and_deterministic(orc):
    case = synth.decode_case(B=32, N=64, H=12, seed=16)
    W = 12 * HD
    obuf = torch.full((34, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    pbuf = torch.full((66, 12, HD, HD), float("nan"), dtype=torch.bfloat16, device="cuda")
    pbuf[1:65] = dev_bf16(case["pool"])
    pool, out = run_decode(case, pool=pbuf[1:65], out=obuf[1:33])
    check_case(orc, case, pool, out)
    assert np.all(np.isnan(f32(bits(obuf[0])))) and np.all(np.isnan(f32(bits(obuf[33]))))
    assert np.all(np.isnan(f32(bits(pbuf[0])))) and np.all(np.isnan(f32(bits(pbuf[65]))))
    # a second run from the same inputs is bitwise identical
    pool2, out2 = run_decode(case)
    torch.cuda.synchronize()
    assert np.array_equal(bits(pool2), bits(pool)) and np.array_equal(bits(out2), bits(out))


def test_graph_replay_with_changed_inputs(orc):
    """Capture one decode in a HIP graph, then replay it with new inputs and
    indices copied into the captured buffers; every replay matches eager."""
    B, H, N = 16, 12, 40
    base = synth.decode_case(B=B, N=N, H=H, seed=17)
    W = H * HD
    qkv = dev_bf16(base["qkv"])
    gate, beta = dev_bf16(base["gate"]), dev_bf16(base["beta"])
    a_log, dtb, idx = dev(base["a_log"]), dev(base["dt_bias"]), dev(base["idx"])
    pool = dev_bf16(base["pool"])
    out = torch.zeros((B, W), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the side stream before capture
        _kda().kda_decode(qkv[:, :W], qkv[:, W:2 * W], qkv[:, 2 * W:], gate, beta, a_log, dtb,
                          pool, idx, out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _kda().kda_decode(qkv[:, :W], qkv[:, W:2 * W], qkv[:, 2 * W:], gate, beta, a_log, dtb,
                          pool, idx, out)
    for r in range(3):
        case = synth.decode_case(B=B, N=N, H=H, seed=100 + r)
        qkv.copy_(dev_bf16(case["qkv"]))
        gate.copy_(dev_bf16(case["gate"]))
        beta.copy_(dev_bf16(case["beta"]))
        a_log.copy_(dev(case["a_log"]))
        dtb.copy_(dev(case["dt_bias"]))
        idx.copy_(dev(case["idx"]))
        pool.copy_(dev_bf16(case["pool"]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_case(orc, case, pool, out)
