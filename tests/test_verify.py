"""GPU parity of kda_verify_ucache_flush against the CPU oracle, through the C ABI.

Operation: "feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3 (KDA)"
-- T draft tokens per row verified against a checkpoint plus a (k_hat, u, G)
ring; the ring is folded into the checkpoint once hist + T >= flush_min.
History rows are produced by the oracle stepping seeded history tokens from
the checkpoint; ring rows that hold no live history are poisoned with NaN and
must never be read or written.
"""
import numpy as np
import pytest

from gated_delta_rule_step_amd import synth
from tests.helpers import (HD, bits, check_gcache, check_out, check_pool, check_state,
                           compact_slots, dev, dev_bf16, f32, normwise_error, pool_dev, pool_vals,
                           report_accuracy, split_qkv)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16_NAN = np.uint16(0x7FC0)


def _kda():
    import gated_delta_rule_step_amd as kda
    return kda


def _tok_arrays(qkv, gate, beta, H):
    q, k, v = split_qkv(qkv, H)
    if gate.shape[-1] == H:  # per-head gate: one value per token and head
        g = np.ascontiguousarray(f32(gate))
    else:
        g = np.ascontiguousarray(f32(gate).reshape(*gate.shape[:-1], H, HD))
    return q, k, v, g, np.ascontiguousarray(f32(beta))


def build_case(orc, B, T, w_ring=16, flush_min=None, fold_p=0.0, hist_max=None, N=1024, H=12,
               workload=3, inactive_frac=0.0, seed=None, state_dtype=0):
    """A verify case whose live ring history comes from the oracle (state_dtype
    1: fp16 checkpoints, 2: fp8 e4m3 checkpoints)."""
    case = synth.verify_case(B=B, T=T, N=N, H=H, w_ring=w_ring, flush_min=flush_min,
                             fold_p=fold_p, hist_max=hist_max, workload=workload,
                             inactive_frac=inactive_frac, seed=seed)
    if state_dtype == 1:
        case = synth.fp16_state(case)
    elif state_dtype == 2:
        case = synth.fp8_state(case)
    R = case["R"]
    slots, cidx = compact_slots(case["idx"], N)
    case["slots"], case["cidx"] = slots, cidx
    # Oracle view: compact pool / rings over the active rows' slots.
    cpool = np.ascontiguousarray(pool_vals(case, case["pool"][slots]))
    n = len(slots)
    kc = np.zeros((n, H, R, HD), np.float32)
    uc = np.zeros((n, H, R, HD), np.float32)
    gc = np.zeros((n, H, R, HD), np.float32)
    hmax = int(case["hist_len"].max()) if B else 0
    if hmax > 0:
        ht = synth.history_tokens(case, hmax)
        q, k, v, g, be = _tok_arrays(ht["qkv"], ht["gate"], ht["beta"], H)
        zero = np.zeros(B, np.int32)
        orc.verify(q, k, v, g, be, case["a_log"], case["dt_bias"], -5.0, 1.0, cpool, cidx, kc,
                   uc, gc, zero, case["cache_base"], 10 ** 6, 10 ** 6, bf16_storage=True,
                   real=np.float32)
    # Poison every row that is not live history, for every active row.
    for b in range(B):
        if cidx[b] < 0:
            continue
        hl, base = int(case["hist_len"][b]), int(case["cache_base"][b])
        for j in range(max(hl, 0), R):
            r = (base + j) % R
            kc[cidx[b], :, r] = np.nan
            uc[cidx[b], :, r] = np.nan
            gc[cidx[b], :, r] = np.nan
    case["okc"], case["ouc"], case["ogc"], case["opool"] = kc, uc, gc, cpool
    # GPU view: full pool; rings of touched slots from the oracle arrays, all
    # other ring rows random (must stay untouched).
    gkc = synth.filler_bits((N, H, R, HD), 1)
    guc = synth.filler_bits((N, H, R, HD), 2)
    ggc = (synth.filler_bits((N, H, R, HD), 3).astype(np.uint32) << 16).view(np.float32)
    gkc[slots] = orc.bf16_round_bits(kc)
    guc[slots] = orc.bf16_round_bits(uc)
    ggc[slots] = gc
    case["k_cache"], case["u_cache"], case["g_cache"] = gkc, guc, ggc
    return case


def run_gpu(case, flush_min=None, qkv=None, gate=None, beta=None, T=None, hist=None, base=None,
            dev_state=None):
    """Launch verify; returns the device tensors (pool, k_cache, u_cache, g_cache, out)."""
    H, B = case["H"], case["B"]
    T = case["T"] if T is None else T
    W = H * HD
    qkv = dev_bf16(case["qkv"] if qkv is None else qkv)
    if dev_state is None:
        dev_state = dict(pool=pool_dev(case, case["pool"]), kc=dev_bf16(case["k_cache"]),
                         uc=dev_bf16(case["u_cache"]), gc=dev(case["g_cache"]))
    out = torch.full((B, T, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    _kda().kda_verify_ucache_flush(
        qkv[..., :W], qkv[..., W:2 * W], qkv[..., 2 * W:],
        dev_bf16(case["gate"] if gate is None else gate),
        dev_bf16(case["beta"] if beta is None else beta),
        None if case.get("gate_mode", 0) & 1 else dev(case["a_log"]),
        None if case.get("gate_mode", 0) & 1 else dev(case["dt_bias"]),
        dev_state["pool"], dev(case["idx"]), dev_state["kc"],
        dev_state["uc"], dev_state["gc"],
        dev(case["hist_len"] if hist is None else hist),
        dev(case["cache_base"] if base is None else base), out,
        flush_min=case["flush_min"] if flush_min is None else flush_min, w_ring=case["w_ring"],
        lower_bound=case["lower_bound"], scale=case["scale"], gate_mode=case.get("gate_mode", 0))
    dev_state["out"] = out
    return dev_state


def run_oracle(orc, case, flush_min=None, qkv=None, gate=None, beta=None, hist=None, base=None):
    H = case["H"]
    q, k, v, g, be = _tok_arrays(case["qkv"] if qkv is None else qkv,
                                 case["gate"] if gate is None else gate,
                                 case["beta"] if beta is None else beta, H)
    gm = case.get("gate_mode", 0)
    a_log, dt_bias = (None, None) if gm & 1 else (case["a_log"], case["dt_bias"])
    return orc.verify(q, k, v, g, be, a_log, dt_bias, case["lower_bound"],
                      case["scale"], case["opool"], case["cidx"], case["okc"], case["ouc"],
                      case["ogc"], case["hist_len"] if hist is None else hist,
                      case["cache_base"] if base is None else base,
                      case["flush_min"] if flush_min is None else flush_min, case["w_ring"],
                      bf16_storage=True, real=np.float32, gate_mode=gm,
                      state_dtype=case.get("state_dtype", 0))


def check_all(case, st, ref_out, pool0, kc0, uc0, gc0, T=None, hist=None, base=None,
              flush_min=None):
    """Compare GPU results with the oracle's and check everything else is untouched."""
    torch.cuda.synchronize()
    B, H, R = case["B"], case["H"], case["R"]
    T = case["T"] if T is None else T
    # int64 copies: hist + T must not wrap for hist_len near INT32_MAX
    hist = np.asarray(case["hist_len"] if hist is None else hist, np.int64)
    base = np.asarray(case["cache_base"] if base is None else base, np.int64)
    fm = case["flush_min"] if flush_min is None else flush_min
    slots, cidx = case["slots"], case["cidx"]
    check_out(bits(st["out"]), ref_out.reshape(B, T, H * HD), "verify output")
    pool, kc, uc, gc = bits(st["pool"]), bits(st["kc"]), bits(st["uc"]), \
        st["gc"].cpu().numpy()
    written = np.zeros((case["N"], H, R), bool)  # ring rows the call may write
    for b in range(B):
        c = cidx[b]
        if c < 0 or hist[b] < 0 or hist[b] + T > case["w_ring"] or not 0 <= base[b] < R:
            assert np.all(bits(st["out"])[b] == 0), "inactive row must output zeros"
            continue
        s = slots[c]
        rows = [(base[b] + hist[b] + t) % R for t in range(T)]
        written[s, :, rows] = True
        check_state(kc[s][:, rows], case["okc"][c][:, rows], f"k_cache row {b}")
        check_state(uc[s][:, rows], case["ouc"][c][:, rows], f"u_cache row {b}")
        check_gcache(gc[s][:, rows], case["ogc"][c][:, rows], f"g_cache row {b}")
        if hist[b] + T >= fm:
            check_pool(case, pool[s], case["opool"][c], f"folded checkpoint row {b}")
        else:
            assert np.array_equal(pool[s], pool0[s]), f"checkpoint of row {b} must not change"
    untouched = ~written
    assert np.array_equal(kc[untouched], kc0[untouched]), "k_cache rows outside the draft rows changed"
    assert np.array_equal(uc[untouched], uc0[untouched]), "u_cache rows outside the draft rows changed"
    assert np.array_equal(gc[untouched].view(np.uint32), gc0[untouched].view(np.uint32)), \
        "g_cache rows outside the draft rows changed"
    folded = set()
    for b in range(B):
        c = cidx[b]
        if c >= 0 and hist[b] >= 0 and hist[b] + T <= case["w_ring"] and 0 <= base[b] < R \
                and hist[b] + T >= fm:
            folded.add(int(slots[c]))
    others = np.array([s for s in range(case["N"]) if s not in folded], dtype=np.int64)
    assert np.array_equal(pool[others], pool0[others]), "checkpoints that do not fold changed"


def verify_roundtrip(orc, case, **kw):
    snap = (case["pool"].copy(), case["k_cache"].copy(), case["u_cache"].copy(),
            case["g_cache"].copy())
    st = run_gpu(case, **kw)
    ref = run_oracle(orc, case, **kw)
    check_all(case, st, ref, *snap, **{k: v for k, v in kw.items() if k == "flush_min"})
    return st


@pytest.mark.parametrize("T", [8, 4])
@pytest.mark.parametrize("B", [1, 32, 512])
def test_bare_checkpoint_no_history(orc, T, B):
    """Draft tokens from a bare checkpoint (hist = 0, W16, flush_min 9 / 13):
    outputs, ring appends, untouched checkpoint."""
    case = build_case(orc, B, T, workload=2, hist_max=0)
    assert np.all(case["hist_len"] == 0)
    verify_roundtrip(orc, case)


@pytest.mark.parametrize("T,fm", [(8, 9), (4, 13)])
@pytest.mark.parametrize("p", [0.0, 0.5, 1.0])
@pytest.mark.parametrize("B", [1, 32, 512])
def test_ring_history_and_fold(orc, T, fm, p, B):
    case = build_case(orc, B, T, w_ring=16, flush_min=fm, fold_p=p)
    verify_roundtrip(orc, case)


@pytest.mark.parametrize("T,fm,p,gate_mode", [(8, 9, 0.5, 3), (4, 13, 1.0, 1), (8, 9, 0.0, 2)])
def test_precomputed_gate_conventions(orc, T, fm, p, gate_mode):
    """The pre-computed gate and / or beta convention on the draft tokens, with
    ring history and folding rows, B = 512 (the history itself was written
    under the raw convention, as a caller switching conventions would see)."""
    case = build_case(orc, 512, T, w_ring=16, flush_min=fm, fold_p=p)
    case = synth.precomputed_gate(case, gate_mode, synth.seed_for(3, 512, 100 + gate_mode))
    verify_roundtrip(orc, case)


@pytest.mark.parametrize("T,fm,p,hist_max,w,B", [(8, 9, 0.5, None, 16, 512),
                                                (8, 9, 0.0, 0, 16, 512),
                                                (8, 25, 0.0, 24, 32, 512),
                                                (8, 9, 1.0, None, 16, 32)])
def test_fp16_checkpoints(orc, T, fm, p, hist_max, w, B):
    """fp16 checkpoints (state_dtype 1) at B = 512 (and 32, where folds use
    non-temporal stores): the checkpoint product on fp16 MFMA operands, folds
    stored as binary16, rings still bf16."""
    case = build_case(orc, B, T, w_ring=w, flush_min=fm, fold_p=p, hist_max=hist_max,
                      state_dtype=1)
    verify_roundtrip(orc, case)


@pytest.mark.parametrize("T,fm,p,hist_max,w,B", [(8, 9, 0.5, None, 16, 512),
                                                (8, 9, 0.0, 0, 16, 512),
                                                (8, 25, 0.0, 24, 32, 512),
                                                (8, 9, 1.0, None, 16, 32)])
def test_fp8_checkpoints(orc, T, fm, p, hist_max, w, B):
    """fp8 e4m3 checkpoints (state_dtype 2) at B = 512 (and 32, where folds use
    non-temporal stores): the checkpoint widened to bf16 B operands (exactly),
    folds stored as fp8, rings still bf16."""
    case = build_case(orc, B, T, w_ring=w, flush_min=fm, fold_p=p, hist_max=hist_max,
                      state_dtype=2)
    verify_roundtrip(orc, case)


@pytest.mark.parametrize("pre", [False, True])
def test_per_head_gate(orc, pre):
    """The per-head (scalar) gate on the draft tokens, raw and pre-computed, with
    ring history and folding rows, B = 512; the history was written under the
    per-channel gate (the ring keeps only cumulative G rows)."""
    case = build_case(orc, 512, 8, w_ring=16, flush_min=9, fold_p=0.5)
    case = synth.per_head_gate(case, pre, synth.seed_for(3, 512, 120 + int(pre)))
    verify_roundtrip(orc, case)


@pytest.mark.parametrize("B", [1, 32, 512])
def test_deep_window_w32(orc, B):
    """w_ring = 32, T = 8, flush_min = 25, hist ~ U{0..24} (fold iff hist >= 17)."""
    case = build_case(orc, B, 8, w_ring=32, flush_min=25, hist_max=24)
    verify_roundtrip(orc, case)


@pytest.mark.parametrize("T,fm,state_dtype", [(1, 32, 0), (2, 31, 0), (1, 32, 2)])
def test_deep_window_full_capacity(orc, T, fm, state_dtype):
    """w_ring = 32 at full capacity: every row folds with hist = 31 (T = 1) or
    29-30 (T = 2), so the deep-ring fold's history product uses its whole
    K = 32 step; bf16 and fp8 checkpoints."""
    case = build_case(orc, 32, T, w_ring=32, flush_min=fm, fold_p=1.0,
                      state_dtype=state_dtype)
    assert case["hist_len"].min() >= fm - T
    verify_roundtrip(orc, case)


@pytest.mark.parametrize("gate_mode", [3, 4])
def test_deep_window_gate_kinds(orc, gate_mode):
    """w_ring = 32 (the deep-ring instance, hist ~ U{0..24}) with the
    pre-computed gate and beta (3) and with one gate per head (4)."""
    case = build_case(orc, 32, 8, w_ring=32, flush_min=25, hist_max=24)
    if gate_mode == 4:
        case = synth.per_head_gate(case, False, synth.seed_for(3, 32, 140))
    else:
        case = synth.precomputed_gate(case, gate_mode, synth.seed_for(3, 32, 141))
    verify_roundtrip(orc, case)


@pytest.mark.parametrize("T,fm,w,gate_mode,lb,misaligned", [
    (8, 9, 16, 0, -12.0, False),        # raw gate, T |lb| = 96 >= 80
    (8, 9, 16, 1, -np.inf, False),      # pre-computed log-decay down to -20, no floor
    (4, 13, 16, 3, -np.inf, False),     # and pre-sigmoided beta
    (8, 25, 32, 1, -np.inf, False),     # 32-row window (hist ~ U{0..24})
    (8, 9, 16, 0, -12.0, True),         # the scalar (unaligned) path
    (4, 13, 16, 1, -np.inf, True)])
def test_unfactored_exponentials(orc, T, fm, w, gate_mode, lb, misaligned):
    """lower_bound <= -80 / T selects the instance that forms each weight
    exp(Gam_r - Gam_j) directly instead of as exp(Gam_r) * exp(-Gam_j) (whose
    factors could overflow): ring history and folding rows, B = 64, vector
    and scalar paths; pre-computed log-decays drawn U(-20, 0.5), so that the
    cumulative decay of a draft reaches well past exp(-80)."""
    B = 64
    if w == 32:
        case = build_case(orc, B, T, w_ring=32, flush_min=fm, hist_max=24, N=96)
    else:
        case = build_case(orc, B, T, w_ring=w, flush_min=fm, fold_p=0.5, N=96)
    if gate_mode:
        case = synth.precomputed_gate(case, gate_mode, synth.seed_for(3, B, 160 + T),
                                      g_low=-20.0)
    case["lower_bound"] = float(lb)
    if not misaligned:
        verify_roundtrip(orc, case)
        return
    snap = (case["pool"].copy(), case["k_cache"].copy(), case["u_cache"].copy(),
            case["g_cache"].copy())
    H = case["H"]
    W = H * HD
    rs = T * (3 * W + 1)
    buf = torch.zeros(B * rs + 2, dtype=torch.bfloat16, device="cuda")
    rows = buf[1:1 + B * rs].view(B, T, 3 * W + 1)
    rows[..., :3 * W] = dev_bf16(case["qkv"])
    obuf = torch.full((B * T * (W + 1) + 1,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = obuf[1:].view(B, T, W + 1)[..., :W]
    st = dict(pool=dev_bf16(case["pool"]), kc=dev_bf16(case["k_cache"]),
              uc=dev_bf16(case["u_cache"]), gc=dev(case["g_cache"]), out=out)
    pre = gate_mode & 1
    _kda().kda_verify_ucache_flush(
        rows[..., :W], rows[..., W:2 * W], rows[..., 2 * W:3 * W], dev_bf16(case["gate"]),
        dev_bf16(case["beta"]), None if pre else dev(case["a_log"]),
        None if pre else dev(case["dt_bias"]), st["pool"], dev(case["idx"]), st["kc"],
        st["uc"], st["gc"], dev(case["hist_len"]), dev(case["cache_base"]), out,
        flush_min=fm, w_ring=w, lower_bound=float(lb), gate_mode=gate_mode)
    ref = run_oracle(orc, case)
    check_all(case, st, ref, *snap)


@pytest.mark.parametrize("T,fm,w,hist_max,p", [(8, 9, 16, None, 0.5), (4, 13, 16, None, 1.0),
                                               (8, 25, 32, 24, 0.0)])
def test_accuracy_against_fp64(orc, T, fm, w, hist_max, p):
    """Outputs and folded checkpoints against an fp64 oracle run on the same
    inputs (the same bf16 checkpoint and ring rows) with no storage rounding:
    what the bf16 MFMA products (split operands) and the bf16 stores cost.
    Reported, and bounded normwise (outputs 3e-3, folded checkpoints 3e-3)."""
    B = 128
    case = build_case(orc, B, T, w_ring=w, flush_min=fm, fold_p=p, hist_max=hist_max, N=256)
    st = run_gpu(case)
    H = case["H"]
    q, k, v, g, be = _tok_arrays(case["qkv"], case["gate"], case["beta"], H)
    d = np.float64
    pool64 = case["opool"].astype(d)
    kc64, uc64, gc64 = (case[n].astype(d) for n in ("okc", "ouc", "ogc"))
    ref = orc.verify(q.astype(d), k.astype(d), v.astype(d), g.astype(d), be.astype(d),
                     case["a_log"].astype(d), case["dt_bias"].astype(d), case["lower_bound"],
                     case["scale"], pool64, case["cidx"], kc64, uc64, gc64, case["hist_len"],
                     case["cache_base"], fm, w, bf16_storage=False, real=d)
    torch.cuda.synchronize()
    got = f32(bits(st["out"])).reshape(ref.shape).astype(d)
    e_out = normwise_error(got, ref)
    folds = [b for b in range(B) if case["cidx"][b] >= 0 and case["hist_len"][b] + T >= fm]
    pool = f32(bits(st["pool"]))
    if folds:
        gs = np.stack([pool[case["slots"][case["cidx"][b]]] for b in folds])
        rs = np.stack([pool64[case["cidx"][b]] for b in folds])
        e_ck = normwise_error(gs, rs)
    else:
        e_ck = 0.0
    report_accuracy(f"verify T={T} w={w} fm={fm}", out_normwise=e_out, fold_normwise=e_ck,
                    folds=len(folds))
    assert e_out <= 3e-3 and e_ck <= 3e-3, (e_out, e_ck)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 7])
def test_other_draft_lengths(orc, T):
    case = build_case(orc, 24, T, w_ring=16, flush_min=16 - T + 1, fold_p=0.5, N=64)
    verify_roundtrip(orc, case)


@pytest.mark.parametrize("T,fm", [(8, 9), (4, 13)])
def test_committed_state_after_acceptance(orc, T, fm):
    """Verify from a bare checkpoint, accept a ~ U{0..T} tokens (bookkeeping
    hist = a), then a forced fold (flush_min = 1, one dummy token) commits the
    state after the accepted tokens. Each call is compared with the oracle
    started from the GPU's state before that call."""
    B = 32
    case = build_case(orc, B, T, workload=2, flush_min=fm, hist_max=0)
    st = verify_roundtrip(orc, case)
    rng = np.random.Generator(np.random.PCG64(synth.seed_for(2, B, T) + 1))
    acc = rng.integers(0, T + 1, size=B).astype(np.int32)
    hist = case["hist_len"] + acc
    dummy = synth.verify_case(B=B, T=1, N=1, H=case["H"], seed=5)
    snap = (bits(st["pool"]), bits(st["kc"]), bits(st["uc"]), st["gc"].cpu().numpy())
    # teacher forcing: the oracle's forced fold starts from the GPU's state
    slots = case["slots"]
    case["opool"] = np.ascontiguousarray(f32(snap[0][slots]))
    case["okc"] = np.ascontiguousarray(f32(snap[1][slots]))
    case["ouc"] = np.ascontiguousarray(f32(snap[2][slots]))
    case["ogc"] = np.ascontiguousarray(snap[3][slots])
    case["T"] = 1
    st2 = run_gpu(case, flush_min=1, qkv=dummy["qkv"], gate=dummy["gate"], beta=dummy["beta"],
                  T=1, hist=hist, dev_state=st)
    ref = run_oracle(orc, case, flush_min=1, qkv=dummy["qkv"], gate=dummy["gate"],
                     beta=dummy["beta"], hist=hist)
    check_all(case, st2, ref, *snap, T=1, hist=hist, flush_min=1)


def test_inactive_rows_and_bad_ring_metadata(orc):
    B, T = 10, 4
    case = build_case(orc, B, T, w_ring=16, flush_min=13, fold_p=0.5, N=16, inactive_frac=0.0)
    case["idx"][0] = -1
    case["idx"][1] = 16
    case["idx"][2] = np.iinfo(np.int32).min
    case["hist_len"][3] = -1          # negative history
    case["hist_len"][4] = 13          # hist + T > w_ring
    case["cache_base"][5] = 32        # base outside the ring
    case["cache_base"][6] = -1
    imax = np.iinfo(np.int32).max     # hist + T would wrap to a negative int32
    case["hist_len"][7] = imax
    case["hist_len"][8] = imax - 3
    slots, cidx = compact_slots(case["idx"], case["N"])
    case["slots"], case["cidx"] = slots, cidx
    case["opool"] = np.ascontiguousarray(f32(case["pool"][slots]))
    n = len(slots)
    for key in ("okc", "ouc", "ogc"):
        case[key] = np.full((n, 12, 32, HD), np.nan, np.float32)
    for b in range(B):
        if cidx[b] >= 0:
            case["okc"][cidx[b]] = f32(case["k_cache"][slots[cidx[b]]])
            case["ouc"][cidx[b]] = f32(case["u_cache"][slots[cidx[b]]])
            case["ogc"][cidx[b]] = case["g_cache"][slots[cidx[b]]]
    verify_roundtrip(orc, case)


def test_empty_pool(orc):
    case = synth.verify_case(B=3, T=8, N=1, H=12, seed=3)
    W = 12 * HD
    qkv = dev_bf16(case["qkv"])
    empty = torch.empty((0, 12, HD, HD), dtype=torch.bfloat16, device="cuda")
    ring = torch.empty((0, 12, 32, HD), dtype=torch.bfloat16, device="cuda")
    gring = torch.empty((0, 12, 32, HD), dtype=torch.float32, device="cuda")
    out = torch.full((3, 8, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    _kda().kda_verify_ucache_flush(
        qkv[..., :W], qkv[..., W:2 * W], qkv[..., 2 * W:], dev_bf16(case["gate"]),
        dev_bf16(case["beta"]), dev(case["a_log"]), dev(case["dt_bias"]), empty,
        dev(np.array([0, 1, -1], np.int32)), ring, ring, gring, dev(case["hist_len"]),
        dev(case["cache_base"]), out, flush_min=9)
    torch.cuda.synchronize()
    assert np.all(bits(out) == 0)


def test_misaligned_scalar_path(orc):
    """Unaligned q/k/v/out views take the scalar path and give the same result."""
    B, T, H = 6, 4, 12
    case = build_case(orc, B, T, w_ring=16, flush_min=13, fold_p=0.5, N=16)
    snap = (case["pool"].copy(), case["k_cache"].copy(), case["u_cache"].copy(),
            case["g_cache"].copy())
    W = H * HD
    rs = T * (3 * W + 1)
    buf = torch.zeros(B * rs + 2, dtype=torch.bfloat16, device="cuda")
    rows = buf[1:1 + B * rs].view(B, T, 3 * W + 1)
    rows[..., :3 * W] = dev_bf16(case["qkv"])
    obuf = torch.full((B * T * (W + 1) + 1,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = obuf[1:].view(B, T, W + 1)[..., :W]
    st = dict(pool=dev_bf16(case["pool"]), kc=dev_bf16(case["k_cache"]),
              uc=dev_bf16(case["u_cache"]), gc=dev(case["g_cache"]), out=out)
    _kda().kda_verify_ucache_flush(
        rows[..., :W], rows[..., W:2 * W], rows[..., 2 * W:3 * W], dev_bf16(case["gate"]),
        dev_bf16(case["beta"]), dev(case["a_log"]), dev(case["dt_bias"]), st["pool"],
        dev(case["idx"]), st["kc"], st["uc"], st["gc"], dev(case["hist_len"]),
        dev(case["cache_base"]), out, flush_min=13, w_ring=16)
    ref = run_oracle(orc, case)
    check_all(case, st, ref, *snap)
    assert np.all(np.isnan(f32(bits(obuf[1:].view(B, T, W + 1)[..., W:]))))


def test_deterministic_and_graph_replay(orc):
    """Two eager runs are bitwise identical; a captured graph replayed three
    times (inputs restored between replays) reproduces the eager result."""
    case = build_case(orc, 16, 8, w_ring=16, flush_min=9, fold_p=0.5, N=40)
    st1 = run_gpu(case)
    st2 = run_gpu(case)
    torch.cuda.synchronize()
    for key in ("out", "pool", "kc", "uc"):
        assert np.array_equal(bits(st1[key]), bits(st2[key])), key
    assert np.array_equal(st1["gc"].cpu().numpy().view(np.uint32),
                          st2["gc"].cpu().numpy().view(np.uint32))
    st = dict(pool=dev_bf16(case["pool"]), kc=dev_bf16(case["k_cache"]),
              uc=dev_bf16(case["u_cache"]), gc=dev(case["g_cache"]))
    W = 12 * HD
    qkv = dev_bf16(case["qkv"])
    gate, beta = dev_bf16(case["gate"]), dev_bf16(case["beta"])
    a_log, dtb, idx = dev(case["a_log"]), dev(case["dt_bias"]), dev(case["idx"])
    hist, base = dev(case["hist_len"]), dev(case["cache_base"])
    out = torch.zeros((16, 8, W), dtype=torch.bfloat16, device="cuda")

    def call():
        _kda().kda_verify_ucache_flush(qkv[..., :W], qkv[..., W:2 * W], qkv[..., 2 * W:], gate,
                                       beta, a_log, dtb, st["pool"], idx, st["kc"], st["uc"],
                                       st["gc"], hist, base, out, flush_min=9, w_ring=16)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        st["pool"].copy_(dev_bf16(case["pool"]))
        st["kc"].copy_(dev_bf16(case["k_cache"]))
        st["uc"].copy_(dev_bf16(case["u_cache"]))
        st["gc"].copy_(dev(case["g_cache"]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, ref in (("out", st1["out"]), ("pool", st1["pool"]), ("kc", st1["kc"]),
                         ("uc", st1["uc"])):
            got = out if key == "out" else st[key]
            assert np.array_equal(bits(got), bits(ref)), key
