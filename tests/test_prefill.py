"""GPU parity of kda_prefill_varlen against the CPU oracle's token-by-token
recurrence, through the C ABI.

Operation: "feat(kda): add CuTe DSL recurrent prefill backend" -- packed
documents delimited by cu_seqlens, optional initial states from a bf16 pool
addressed by state indices, per-token outputs and final states; the chunked
result must equal the token-by-token recurrence.
"""
import numpy as np
import pytest

from gated_delta_rule_step_amd import synth
from tests.helpers import (HD, OUT_NORM_PREFILL, bits, check_gcache, check_out, check_pool,
                           check_state, dev, dev_bf16, f32, normwise_error, pool_dev, pool_vals,
                           report_accuracy)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _kda():
    import gated_delta_rule_step_amd as kda
    return kda


def run_prefill(case, pool=None, packed=False, use_initial_state=None, lower_bound=None,
                checkpoints=None, ckpt_starts=None, ckpt_interval=16, ring=None, cache_base=None,
                ring_tail=0, misaligned=False):
    """Launch kda_prefill_varlen on a case. packed: q/k/v are strided views of
    one [Ttot, 3*H*128] buffer and out is a view with a padded row. misaligned:
    q/k/v/out start one element into rows of W + 1 elements (2-byte aligned
    bases, odd strides: the scalar path)."""
    gm = case.get("gate_mode", 0)
    H, Ttot = case["H"], case["Ttot"]
    W = H * HD
    if misaligned:
        def view(a):
            buf = torch.full((Ttot, W + 1), float("nan"), dtype=torch.bfloat16, device="cuda")
            if a is not None:
                buf[:, 1:] = dev_bf16(a.reshape(Ttot, W))
            return buf[:, 1:]
        q, k, v = (view(case[n]) for n in ("q", "k", "v"))
        out = view(None)
    elif packed:
        qkv = np.concatenate([case["q"].reshape(Ttot, W), case["k"].reshape(Ttot, W),
                              case["v"].reshape(Ttot, W)], axis=1)
        qkv_d = dev_bf16(qkv)
        q, k, v = qkv_d[:, :W], qkv_d[:, W:2 * W], qkv_d[:, 2 * W:]
        out_buf = torch.full((Ttot, W + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
        out = out_buf[:, :W]
    else:
        q, k, v = (dev_bf16(case[n].reshape(Ttot, W)) for n in ("q", "k", "v"))
        out = torch.full((Ttot, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    pool = pool_dev(case, case["pool"]) if pool is None else pool
    cu_h = torch.from_numpy(case["cu_seqlens"].copy())
    uis = case["use_initial_state"] if use_initial_state is None else use_initial_state
    _kda().kda_prefill_varlen(cu_h, dev(case["cu_seqlens"]), q, k, v, dev_bf16(case["gate"]),
                              dev_bf16(case["beta"]), None if gm & 1 else dev(case["a_log"]),
                              None if gm & 1 else dev(case["dt_bias"]),
                              pool, dev(case["idx"]), out, use_initial_state=uis,
                              lower_bound=case["lower_bound"] if lower_bound is None
                              else lower_bound, scale=case["scale"], gate_mode=gm,
                              checkpoints=checkpoints,
                              checkpoint_cu_starts=None if ckpt_starts is None
                              else dev(ckpt_starts), checkpoint_interval=ckpt_interval,
                              ring=ring, cache_base=None if cache_base is None
                              else dev(cache_base), ring_tail=ring_tail)
    return pool, out


def oracle_prefill(orc, case, heads=None, use_initial_state=None, lower_bound=None,
                   ckpt=None, ckpt_starts=None, ckpt_interval=16, ring=None, cache_base=None,
                   ring_tail=0):
    """fp32 token-by-token oracle over the heads listed (all by default).
    Returns (out [Ttot, nh, 128], pool [N, nh, 128, 128] float32 after the run)."""
    H, Ttot = case["H"], case["Ttot"]
    hs = np.arange(H) if heads is None else np.asarray(heads)
    q = f32(case["q"])[:, hs]
    k = f32(case["k"])[:, hs]
    v = f32(case["v"])[:, hs]
    gm = case.get("gate_mode", 0)
    if gm & 4:  # per-head gate: one value per token and head
        g = f32(case["gate"]).reshape(Ttot, H)[:, hs]
    else:
        g = f32(case["gate"]).reshape(Ttot, H, HD)[:, hs]
    b = f32(case["beta"])[:, hs]
    pool = pool_vals(case, case["pool"])[:, hs]
    uis = case["use_initial_state"] if use_initial_state is None else use_initial_state
    lb = case["lower_bound"] if lower_bound is None else lower_bound
    c = np.ascontiguousarray
    pool = c(pool)
    pre = bool(gm & 1)
    out = orc.prefill(case["cu_seqlens"], c(q), c(k), c(v), c(g), c(b),
                      None if pre else c(case["a_log"][hs]),
                      None if pre else c(case["dt_bias"].reshape(H, -1)[hs]), lb,
                      case["scale"], pool, case["idx"], use_initial_state=uis,
                      bf16_storage=True, real=np.float32, gate_mode=gm, checkpoints=ckpt,
                      checkpoint_starts=ckpt_starts, checkpoint_interval=ckpt_interval,
                      state_dtype=case.get("state_dtype", 0), ring=ring, cache_base=cache_base,
                      ring_tail=ring_tail)
    return out, pool


def check_prefill(orc, case, pool_dev, out_dev, heads=None, use_initial_state=None,
                  lower_bound=None):
    H, Ttot, N = case["H"], case["Ttot"], case["N"]
    hs = np.arange(H) if heads is None else np.asarray(heads)
    ref_out, ref_pool = oracle_prefill(orc, case, heads, use_initial_state, lower_bound)
    torch.cuda.synchronize()
    got_out = bits(out_dev).reshape(Ttot, H, HD)[:, hs]
    got_pool = bits(pool_dev)
    idx = case["idx"].astype(np.int64)
    active = (idx >= 0) & (idx < N)
    cu = case["cu_seqlens"]
    for d in range(case["n_docs"]):
        t0, t1 = cu[d], cu[d + 1]
        if active[d]:
            if t1 > t0:
                check_out(got_out[t0:t1], ref_out[t0:t1], f"prefill output doc {d}",
                          norm=OUT_NORM_PREFILL)
            check_pool(case, got_pool[idx[d]][hs], ref_pool[idx[d]], f"prefill state doc {d}")
        else:
            assert np.all(got_out[t0:t1] == 0), f"inactive doc {d} must output +0.0"
    touched = np.zeros(N, bool)
    touched[idx[active]] = True
    assert np.array_equal(got_pool[~touched], case["pool"][~touched]), \
        "slots of inactive documents or unused slots changed"


# ---------------------------------------------------------------------------
# small cases: every chunk boundary, ragged tails, zero-length documents

SMALL_DOCS = (1, 15, 16, 17, 0, 33, 50, 2, 64, 31)

# The library runs the fused 64-token kernel when a call has at least 256
# (document, head) chains and the two-stage form (16-token preparation kernel,
# then the chain) below that; the small cases run on both, the "fused" variant
# with enough heads.
PATHS = ["split", "fused"]
FUSED_MIN_CHAINS = 256


def heads_for(path, n_docs, H_split):
    if path == "split":
        assert n_docs * H_split < FUSED_MIN_CHAINS
        return H_split
    return max(H_split, -(-FUSED_MIN_CHAINS // max(n_docs, 1)))


@pytest.mark.parametrize("path,H0", [("split", 1), ("split", 3), ("fused", 3)])
def test_small_docs_ragged(orc, path, H0):
    H = heads_for(path, len(SMALL_DOCS), H0)
    case = synth.prefill_case(SMALL_DOCS, H=H, seed=synth.seed_for(4, H, 1))
    pool, out = run_prefill(case)
    check_prefill(orc, case, pool, out)


@pytest.mark.parametrize("path", PATHS)
def test_single_token_doc(orc, path):
    """One token: the prefill equals one decode step."""
    H = heads_for(path, 1, 1)
    case = synth.prefill_case((1,), H=H, seed=synth.seed_for(4, 1, 2))
    pool, out = run_prefill(case)
    check_prefill(orc, case, pool, out)


@pytest.mark.parametrize("path", PATHS)
def test_no_initial_state(orc, path):
    """use_initial_state = 0: chains start from zeros; a zero-length document
    leaves a zero state in its slot."""
    case = synth.prefill_case((20, 0, 37, 16), H=heads_for(path, 4, 2), seed=synth.seed_for(4, 2, 3),
                              use_initial_state=False)
    pool, out = run_prefill(case)
    check_prefill(orc, case, pool, out)
    z = case["idx"][1]
    assert np.all(bits(pool)[z] == 0), "zero-length document without initial state: zeros"


@pytest.mark.parametrize("path", PATHS)
def test_zero_length_keeps_state(orc, path):
    """use_initial_state = 1: a zero-length document leaves its slot bitwise."""
    case = synth.prefill_case((0, 5, 0), H=heads_for(path, 3, 2), seed=synth.seed_for(4, 2, 4))
    pool, out = run_prefill(case)
    check_prefill(orc, case, pool, out)
    for d in (0, 2):
        s = case["idx"][d]
        assert np.array_equal(bits(pool)[s], case["pool"][s])


@pytest.mark.parametrize("path", PATHS)
def test_inactive_docs(orc, path):
    """Documents whose slot is -1 or >= N: zero outputs, pool untouched."""
    case = synth.prefill_case((18, 40, 7, 23), H=heads_for(path, 4, 2), seed=synth.seed_for(4, 2, 5),
                              inactive_docs=(1,))
    case["idx"][3] = case["N"] + 5
    pool, out = run_prefill(case)
    check_prefill(orc, case, pool, out)


@pytest.mark.parametrize("path", PATHS)
def test_packed_views_and_padded_out(orc, path):
    """q / k / v as strided views of one packed row, out with a padded row."""
    case = synth.prefill_case((29, 16, 3, 130), H=heads_for(path, 4, 2), seed=synth.seed_for(4, 2, 6))
    pool, out = run_prefill(case, packed=True)
    check_prefill(orc, case, pool, out)


@pytest.mark.parametrize("path", PATHS)
def test_misaligned_views(orc, path):
    """Unaligned q / k / v / out bases and odd token strides: the scalar-load
    form of each kernel, over ragged documents with checkpoints."""
    case = synth.prefill_case(SMALL_DOCS, H=heads_for(path, 10, 2), seed=synth.seed_for(4, 2, 60))
    counts = np.diff(case["cu_seqlens"]) // 16
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
    _ckpt_roundtrip(orc, case, 16, starts, int(counts.sum()), misaligned=True)


def test_many_docs_natural_order(orc):
    """More documents than the launch orders by length (300; the fused kernel)."""
    rng = np.random.Generator(np.random.PCG64(synth.seed_for(4, 1, 7)))
    lens = tuple(int(x) for x in rng.integers(0, 24, size=300))
    case = synth.prefill_case(lens, H=1, seed=synth.seed_for(4, 1, 8))
    pool, out = run_prefill(case)
    check_prefill(orc, case, pool, out)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("gate_mode", [1, 2, 3])
def test_precomputed_gate_conventions(orc, gate_mode, path):
    """The pre-computed gate and / or beta convention over ragged documents."""
    case = synth.prefill_case(SMALL_DOCS, H=heads_for(path, 10, 3), seed=synth.seed_for(4, 3, 12))
    case = synth.precomputed_gate(case, gate_mode, synth.seed_for(4, 3, 100 + gate_mode))
    pool, out = run_prefill(case)
    check_prefill(orc, case, pool, out)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("pre", [False, True])
def test_per_head_gate(orc, pre, path):
    """The per-head (scalar) gate, raw and pre-computed, over ragged documents."""
    case = synth.prefill_case(SMALL_DOCS, H=heads_for(path, 10, 3), seed=synth.seed_for(4, 3, 13))
    case = synth.per_head_gate(case, pre, synth.seed_for(4, 3, 120 + int(pre)))
    pool, out = run_prefill(case)
    check_prefill(orc, case, pool, out)


def test_precomputed_gate_full_h12(orc):
    """Both pre-computed conventions on the 4-document set at H = 12."""
    case = synth.precomputed_gate(synth.prefill_case(synth.DOCS_4, H=12), 3,
                                  synth.seed_for(4, 12, 103))
    pool, out = run_prefill(case)
    check_prefill(orc, case, pool, out)


def _ckpt_roundtrip(orc, case, interval, starts, rows, heads=None, misaligned=False):
    """Prefill with intermediate checkpoints; compare written rows with the
    oracle's, check that every other row is untouched and that outputs and
    final states match as without checkpoints."""
    H = case["H"]
    hs = np.arange(H) if heads is None else np.asarray(heads)
    fill = synth.filler_bits((rows, H, HD, HD), 7)
    if case.get("state_dtype", 0) == 2:  # one-byte elements
        fill = (fill & 0xFF).astype(np.uint8)
    ck = pool_dev(case, fill)
    pool, out = run_prefill(case, checkpoints=ck, ckpt_starts=starts, ckpt_interval=interval,
                            misaligned=misaligned)
    check_prefill(orc, case, pool, out, heads=heads)
    ref_ck = np.zeros((rows, len(hs), HD, HD), np.float32)
    oracle_prefill(orc, case, heads=heads, ckpt=ref_ck, ckpt_starts=starts,
                   ckpt_interval=interval)
    got = bits(ck)
    lens = np.diff(case["cu_seqlens"])
    active = (case["idx"] >= 0) & (case["idx"] < case["N"])
    written = np.zeros(rows, bool)
    for d, n in enumerate(lens):
        if not active[d]:
            continue
        for i in range(1, n // interval + 1):
            r = int(starts[d]) + i - 1
            if 0 <= r < rows:
                written[r] = True
                check_pool(case, got[r][hs], ref_ck[r], f"checkpoint row {r} (doc {d}, i {i})")
    assert np.array_equal(got[~written], fill[~written]), "rows that are not checkpoints changed"
    return written


@pytest.mark.parametrize("path", PATHS)
def test_checkpoints_small_docs(orc, path):
    """Checkpoints every 16 tokens over ragged documents: one inactive
    document, a gap row, and a last row outside the buffer (skipped)."""
    case = synth.prefill_case(SMALL_DOCS, H=heads_for(path, 10, 3), seed=synth.seed_for(4, 3, 20))
    case["idx"][5] = -1  # the 33-token document: inactive, no checkpoints
    lens = np.diff(case["cu_seqlens"])
    counts = lens // 16
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
    starts[6:] += 1          # a gap row before the 50-token document
    rows = int(starts[-1] + counts[-1]) - 1   # the last checkpoint falls outside
    written = _ckpt_roundtrip(orc, case, 16, starts, rows)
    assert written.sum() == counts[np.arange(len(lens)) != 5].sum() - 1


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("interval", [48, 64, 80])
def test_checkpoints_longer_interval(orc, interval, path):
    case = synth.prefill_case((100, 47, 96, 130), H=heads_for(path, 4, 2), seed=synth.seed_for(4, 2, 21),
                              use_initial_state=False)
    counts = np.diff(case["cu_seqlens"]) // interval
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
    _ckpt_roundtrip(orc, case, interval, starts, int(counts.sum()))


def test_checkpoints_every_chunk_long_docs(orc):
    """Two-stage form: a checkpoint after every 16 tokens over documents of 20
    to 40 chunks, so the chain's record loads, output stores and checkpoint
    stores interleave over many chunks and every position of its unrolled
    chunk loop."""
    case = synth.prefill_case((640, 333, 481), H=heads_for("split", 3, 2),
                              seed=synth.seed_for(4, 2, 23))
    counts = np.diff(case["cu_seqlens"]) // 16
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
    _ckpt_roundtrip(orc, case, 16, starts, int(counts.sum()))


@pytest.mark.parametrize("docs", ["small", "small-fused", "docs4"])
def test_fp16_state(orc, docs):
    """fp16 initial and final states (state_dtype 1): ragged documents with
    checkpoints every 16 tokens (both paths), and the 4-document set at H = 12."""
    if docs.startswith("small"):
        H = heads_for("fused" if docs == "small-fused" else "split", 10, 3)
        case = synth.fp16_state(synth.prefill_case(SMALL_DOCS, H=H, seed=synth.seed_for(4, 3, 22)))
        counts = np.diff(case["cu_seqlens"]) // 16
        starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
        _ckpt_roundtrip(orc, case, 16, starts, int(counts.sum()))
    else:
        case = synth.fp16_state(synth.prefill_case(synth.DOCS_4, H=12))
        pool, out = run_prefill(case)
        check_prefill(orc, case, pool, out)


@pytest.mark.parametrize("docs", ["small", "small-fused", "docs4"])
def test_fp8_state(orc, docs):
    """fp8 e4m3 initial and final states (state_dtype 2): ragged documents
    with checkpoints every 16 tokens, a zero-length document started from
    zeros (both paths), and the 4-document set at H = 12."""
    if docs.startswith("small"):
        path = "fused" if docs == "small-fused" else "split"
        case = synth.fp8_state(synth.prefill_case(SMALL_DOCS, H=heads_for(path, 10, 3),
                                                  seed=synth.seed_for(4, 3, 23)))
        counts = np.diff(case["cu_seqlens"]) // 16
        starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
        _ckpt_roundtrip(orc, case, 16, starts, int(counts.sum()))
        case = synth.fp8_state(synth.prefill_case((20, 0, 37), H=heads_for(path, 3, 2),
                                                  seed=synth.seed_for(4, 2, 24),
                                                  use_initial_state=False))
        pool, out = run_prefill(case)
        check_prefill(orc, case, pool, out)
        assert np.all(bits(pool)[case["idx"][1]] == 0)
    else:
        case = synth.fp8_state(synth.prefill_case(synth.DOCS_4, H=12))
        pool, out = run_prefill(case)
        check_prefill(orc, case, pool, out)


def test_checkpoints_full_h12(orc):
    """The 4-document set at H = 12 with a checkpoint every 256 tokens (53 rows)."""
    case = synth.prefill_case(synth.DOCS_4, H=12)
    counts = np.diff(case["cu_seqlens"]) // 256
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
    _ckpt_roundtrip(orc, case, 256, starts, int(counts.sum()))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("lb", [-5.5, -1.0, 0.0])
def test_lower_bound_range(orc, lb, path):
    """The accepted range of lower_bound, including its end (|lb| = 5.5)."""
    case = synth.prefill_case((40, 9, 70), H=heads_for(path, 3, 2), seed=synth.seed_for(4, 2, 9))
    case["a_log"] = np.full_like(case["a_log"], 1.0)  # strong decay: the clamp is active
    pool, out = run_prefill(case, lower_bound=lb)
    check_prefill(orc, case, pool, out, lower_bound=lb)


def test_lower_bound_rejected():
    case = synth.prefill_case((4,), H=1, seed=synth.seed_for(4, 1, 10))
    with pytest.raises(_kda().KdaError):
        run_prefill(case, lower_bound=-6.0)


@pytest.mark.parametrize("path", PATHS)
def test_large_values(orc, path):
    """v and the initial states scaled by 2^16 (exact in bf16): the
    corrections u reach ~1e5, beyond the fp16 range the fused kernel's
    state-update operands take unscaled, so its waves take their power-of-two
    scaling path. The recurrence is linear in (initial state, v) and power-of-
    two scaling commutes with rounding, so the results divided by 2^16 (exact)
    must meet the usual criteria against the oracle of the unscaled case."""
    case = synth.prefill_case((70, 9, 64, 33), H=heads_for(path, 4, 2),
                              seed=synth.seed_for(4, 2, 70))
    big = dict(case)
    sc = np.float32(65536.0)
    for name in ("v", "pool"):
        x = f32(case[name]) * sc
        big[name] = synth.bf16_bits(x)
        assert np.array_equal(f32(big[name]), x)
    pool, out = run_prefill(big)
    torch.cuda.synchronize()
    down = [dev_bf16(synth.bf16_bits(f32(bits(t)) / sc)) for t in (pool, out)]
    check_prefill(orc, case, down[0], down[1])


@pytest.mark.parametrize("path", PATHS)
def test_deterministic(orc, path):
    case = synth.prefill_case((70, 33), H=heads_for(path, 2, 2), seed=synth.seed_for(4, 2, 11))
    _, out1 = run_prefill(case)
    pool2, out2 = run_prefill(case)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out1), bits(out2))


@pytest.mark.parametrize("path", PATHS)
def test_graph_replay_after_replanning_lengths(orc, path):
    """A graph captured with one set of document lengths, replayed after the
    device cu_seqlens was rewritten with other lengths of the same count and
    total (the host copy, which plans the launch order, is stale): each replay
    equals an eager call with the new lengths bit for bit, and that call
    matches the oracle. Replays alternate with eager work and synchronisation."""
    kda = _kda()
    L1, L2 = (40, 0, 97, 19), (100, 33, 0, 23)
    H = heads_for(path, 4, 2)
    case = synth.prefill_case(L2, H=H, seed=synth.seed_for(4, H, 50))
    Ttot, W = case["Ttot"], H * HD
    assert sum(L1) == Ttot
    q, k, v = (dev_bf16(case[n].reshape(Ttot, W)) for n in ("q", "k", "v"))
    g, b = dev_bf16(case["gate"]), dev_bf16(case["beta"])
    a_log, dtb, idx = dev(case["a_log"]), dev(case["dt_bias"]), dev(case["idx"])
    pool0 = pool_dev(case, case["pool"])
    cu1 = np.concatenate([[0], np.cumsum(L1)]).astype(np.int32)
    cu2 = case["cu_seqlens"]
    ws = torch.empty(max(kda.kda_prefill_workspace_size(4, Ttot, H), 1), dtype=torch.uint8,
                     device="cuda")

    def call(cu_h, cu_d, pool, out):
        kda.kda_prefill_varlen(cu_h, cu_d, q, k, v, g, b, a_log, dtb, pool, idx, out,
                               workspace=ws, lower_bound=case["lower_bound"],
                               scale=case["scale"])

    # eager reference with the new lengths
    pool_e = pool0.clone()
    out_e = torch.full((Ttot, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    call(torch.from_numpy(cu2.copy()), dev(cu2), pool_e, out_e)
    torch.cuda.synchronize()
    check_prefill(orc, case, pool_e, out_e)
    # capture with the old lengths (host and device copies)
    cu_d = dev(cu1)
    pool_g = pool0.clone()
    out_g = torch.full((Ttot, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    call(torch.from_numpy(cu1.copy()), cu_d, pool_g, out_g)  # warm-up outside the graph
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call(torch.from_numpy(cu1.copy()), cu_d, pool_g, out_g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    cu_d.copy_(dev(cu2))
    for rep in range(3):
        pool_g.copy_(pool0)
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_g), bits(out_e)), f"replay {rep}: outputs differ"
        assert np.array_equal(bits(pool_g), bits(pool_e)), f"replay {rep}: states differ"


# ---------------------------------------------------------------------------
# full sizes: 4 documents (3840, 3776, 3200, 3072) and the 14-document mix
# (16384 tokens each), H = 12 (all heads) and H = 64 (sampled heads)

@pytest.mark.parametrize("docs", ["docs4", "docs14"])
def test_full_h12(orc, docs):
    lens = synth.DOCS_4 if docs == "docs4" else synth.DOCS_14
    case = synth.prefill_case(lens, H=12)
    pool, out = run_prefill(case)
    check_prefill(orc, case, pool, out)


@pytest.mark.parametrize("docs", ["docs4", "docs14"])
def test_full_h64_sampled_heads(orc, docs):
    lens = synth.DOCS_4 if docs == "docs4" else synth.DOCS_14
    case = synth.prefill_case(lens, H=64)
    pool, out = run_prefill(case)
    check_prefill(orc, case, pool, out, heads=[0, 9, 21, 33, 47, 63])


@pytest.mark.parametrize("docs,H,heads", [("docs4", 12, None), ("docs14", 64, [0, 17, 40, 63])])
def test_accuracy_against_fp64(orc, docs, H, heads):
    """Outputs and final states against an fp64 oracle run on the same inputs
    with no storage rounding: what the chunked bf16 MFMA products and the bf16
    stores cost over whole documents. Reported, and bounded normwise (outputs
    5e-3, final states 3e-3)."""
    lens = synth.DOCS_4 if docs == "docs4" else synth.DOCS_14
    case = synth.prefill_case(lens, H=H)
    pool_d, out_d = run_prefill(case)
    hs = np.arange(H) if heads is None else np.asarray(heads)
    d = np.float64
    Ttot = case["Ttot"]
    c = np.ascontiguousarray
    pool64 = c(pool_vals(case, case["pool"])[:, hs].astype(d))
    ref = orc.prefill(case["cu_seqlens"], c(f32(case["q"])[:, hs].astype(d)),
                      c(f32(case["k"])[:, hs].astype(d)), c(f32(case["v"])[:, hs].astype(d)),
                      c(f32(case["gate"]).reshape(Ttot, H, HD)[:, hs].astype(d)),
                      c(f32(case["beta"])[:, hs].astype(d)), c(case["a_log"][hs].astype(d)),
                      c(case["dt_bias"].reshape(H, -1)[hs].astype(d)), case["lower_bound"],
                      case["scale"], pool64, case["idx"], use_initial_state=True,
                      bf16_storage=False, real=d)
    torch.cuda.synchronize()
    got_out = f32(bits(out_d)).reshape(Ttot, H, HD)[:, hs].astype(d)
    e_out = normwise_error(got_out, ref)
    slots = case["idx"].astype(np.int64)
    got_st = f32(bits(pool_d))[slots][:, hs].astype(d)
    e_st = normwise_error(got_st, pool64[slots])
    report_accuracy(f"prefill {docs} H={H}", out_normwise=e_out, state_normwise=e_st)
    assert e_out <= 5e-3 and e_st <= 3e-3, (e_out, e_st)


# ---------------------------------------------------------------------------
# hand-off to the verify ring: a document's last min(ring_tail, tokens after
# its last 16-token boundary) tokens become ring history rows (k_hat, u, G)
# and its slot receives the state before them

RING_R = 32


def _ring_fill(N, H, R=RING_R):
    kc = synth.filler_bits((N, H, R, HD), 11)
    uc = synth.filler_bits((N, H, R, HD), 12)
    gc = (synth.filler_bits((N, H, R, HD), 13).astype(np.uint32) << 16).view(np.float32)
    return kc, uc, gc


def _handoff_check(orc, case, ring_tail, base, ckpt_interval=None):
    """Prefill with hand-off on the GPU and in the oracle; compare outputs,
    slot states, every handed-off ring row and (optionally) checkpoints, and
    check that nothing else was written."""
    H, N, Ttot = case["H"], case["N"], case["Ttot"]
    kc0, uc0, gc0 = _ring_fill(N, H)
    ring_d = (dev_bf16(kc0), dev_bf16(uc0), dev(gc0))
    lens = np.diff(case["cu_seqlens"])
    ck = starts = fill = ref_ck = None
    rows = 0
    if ckpt_interval:
        counts = lens // ckpt_interval
        starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
        rows = int(counts.sum())
        fill = synth.filler_bits((rows, H, HD, HD), 14)
        ck = pool_dev(case, fill)
        ref_ck = np.zeros((rows, H, HD, HD), np.float32)
    pool, out = run_prefill(case, ring=ring_d, cache_base=base, ring_tail=ring_tail,
                            checkpoints=ck, ckpt_starts=starts,
                            ckpt_interval=ckpt_interval or 16)
    ring_o = tuple(np.full((N, H, RING_R, HD), np.nan, np.float32) for _ in range(3))
    ref_out, ref_pool = oracle_prefill(orc, case, ckpt=ref_ck, ckpt_starts=starts,
                                       ckpt_interval=ckpt_interval or 16, ring=ring_o,
                                       cache_base=base, ring_tail=ring_tail)
    torch.cuda.synchronize()
    got_out = bits(out).reshape(Ttot, H, HD)
    got_pool = bits(pool)
    gk, gu = bits(ring_d[0]), bits(ring_d[1])
    gg = ring_d[2].cpu().numpy()
    idx = case["idx"].astype(np.int64)
    active = (idx >= 0) & (idx < N) & (base >= 0) & (base < RING_R)
    cu = case["cu_seqlens"]
    written = np.zeros((N, RING_R), bool)
    n_rows = 0
    for d in range(case["n_docs"]):
        t0, t1 = cu[d], cu[d + 1]
        if not active[d]:
            assert np.all(got_out[t0:t1] == 0), f"inactive doc {d} must output +0.0"
            continue
        if t1 > t0:
            check_out(got_out[t0:t1], ref_out[t0:t1], f"hand-off output doc {d}",
                      norm=OUT_NORM_PREFILL)
        s_ = idx[d]
        check_pool(case, got_pool[s_], ref_pool[s_], f"hand-off state doc {d}")
        r = orc.handoff_tail(int(t1 - t0), ring_tail)
        for j in range(r):
            row = (int(base[d]) + j) % RING_R
            written[s_, row] = True
            check_state(gk[s_, :, row], ring_o[0][s_, :, row], f"k_hat row {j} doc {d}")
            check_state(gu[s_, :, row], ring_o[1][s_, :, row], f"u row {j} doc {d}")
            check_gcache(gg[s_, :, row], ring_o[2][s_, :, row], f"G row {j} doc {d}")
        n_rows += r
    def others(a):  # [N, H, R, 128] -> [N, R, H, 128], indexed by (slot, ring row)
        return a.transpose(0, 2, 1, 3)[~written]
    assert np.array_equal(others(gk), others(kc0)), "k_cache rows outside the hand-off changed"
    assert np.array_equal(others(gu), others(uc0)), "u_cache rows outside the hand-off changed"
    assert np.array_equal(others(gg.view(np.uint32)), others(gc0.view(np.uint32))), \
        "g_cache rows outside the hand-off changed"
    touched = np.zeros(N, bool)
    touched[idx[active]] = True
    assert np.array_equal(got_pool[~touched], case["pool"][~touched])
    if ckpt_interval:
        got_ck = bits(ck)
        ck_written = np.zeros(rows, bool)
        for d, n in enumerate(lens):
            if not active[d]:
                continue
            kept = n - orc.handoff_tail(int(n), ring_tail)
            for i in range(1, kept // ckpt_interval + 1):
                row = int(starts[d]) + i - 1
                ck_written[row] = True
                check_pool(case, got_ck[row], ref_ck[row], f"checkpoint {row} doc {d}")
        assert np.array_equal(got_ck[~ck_written], fill[~ck_written])
        return n_rows, int((~ck_written).sum())
    return n_rows, 0


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("ring_tail", [16, 5, 1])
def test_handoff_small_docs(orc, ring_tail, path):
    """Ragged documents (every chunk-boundary case, a zero-length document),
    ring rows wrapping past the ring's end, one document with a ring base
    out of range (inactive)."""
    case = synth.prefill_case(SMALL_DOCS, H=heads_for(path, 10, 3),
                              seed=synth.seed_for(4, 3, 30 + ring_tail))
    base = np.array([0, 31, 20, 17, 5, 30, -1, 9, 28, 3], np.int32)
    n_rows, _ = _handoff_check(orc, case, ring_tail, base)
    expect = sum(min(ring_tail, n - 16 * ((n - 1) // 16)) for i, n in enumerate(SMALL_DOCS)
                 if n > 0 and i != 6)
    assert n_rows == expect


@pytest.mark.parametrize("path", PATHS)
def test_handoff_with_checkpoints_fp16_and_no_initial_state(orc, path):
    """Hand-off with checkpoints every 16 tokens (a checkpoint at a
    document's end is not written when tokens were handed off), fp16
    states, chains from zeros, a ring base of R (inactive)."""
    case = synth.fp16_state(synth.prefill_case(SMALL_DOCS, H=heads_for(path, 10, 2),
                                               seed=synth.seed_for(4, 2, 40),
                                               use_initial_state=False))
    base = np.array([4, 8, 12, 16, 20, 24, 28, RING_R, 1, 2], np.int32)
    _, skipped = _handoff_check(orc, case, 16, base, ckpt_interval=16)
    # skipped rows: the 64-token document's last (its tail is 16 tokens), the
    # 16-token document's only one, and the inactive 2-token document has none
    assert skipped == 2


def test_handoff_full_h12(orc):
    """The 4-document set at H = 12 with an 8-token hand-off."""
    case = synth.prefill_case(synth.DOCS_4, H=12)
    base = np.array([0, 8, 16, 24], np.int32)
    n_rows, _ = _handoff_check(orc, case, 8, base)
    assert n_rows == 8 * 4


@pytest.mark.parametrize("path", PATHS)
def test_handoff_then_verify(orc, path):
    """Prefill hands off to the ring, then a verify call of 8 draft tokens
    (flush_min 9, 16-row window) resumes from it with hist_len = the tail:
    GPU prefill + GPU verify against oracle prefill + oracle verify."""
    kda = _kda()
    lens = (40, 37, 3, 16, 0, 32, 7)
    H, T, fm = heads_for(path, 7, 3), 8, 9
    case = synth.prefill_case(lens, H=H, seed=synth.seed_for(4, H, 50))
    N = case["N"]
    base = np.array([5, 31, 0, 12, 7, 20, 27], np.int32)
    hist = kda.prefill_handoff_hist(torch.from_numpy(case["cu_seqlens"].copy()), 8).numpy()
    assert hist.tolist() == [8, 5, 3, 8, 0, 8, 7]
    kc0, uc0, gc0 = _ring_fill(N, H)
    ring_d = (dev_bf16(kc0), dev_bf16(uc0), dev(gc0))
    pool, _ = run_prefill(case, ring=ring_d, cache_base=base, ring_tail=8)
    torch.cuda.synchronize()
    # what the GPU prefill left, for the teacher-forced check of the fold
    pre_pool = f32(bits(pool))
    pre_k, pre_u = f32(bits(ring_d[0])), f32(bits(ring_d[1]))
    pre_g = ring_d[2].cpu().numpy()
    ring_o = tuple(np.full((N, H, RING_R, HD), np.nan, np.float32) for _ in range(3))
    _, ref_pool = oracle_prefill(orc, case, ring=ring_o, cache_base=base, ring_tail=8)
    # draft tokens, one row per document
    rng = np.random.Generator(np.random.PCG64(synth.seed_for(4, H, 51)))
    B, W = len(lens), H * HD
    qkv = synth.bf16_bits(rng.standard_normal((B, T, 3 * W)).astype(np.float32))
    gate = synth.bf16_bits(rng.standard_normal((B, T, W)).astype(np.float32))
    beta = synth.bf16_bits(rng.standard_normal((B, T, H)).astype(np.float32))
    qkv_d = dev_bf16(qkv)
    out = torch.full((B, T, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    kda.kda_verify_ucache_flush(qkv_d[..., :W], qkv_d[..., W:2 * W], qkv_d[..., 2 * W:],
                                dev_bf16(gate), dev_bf16(beta), dev(case["a_log"]),
                                dev(case["dt_bias"]), pool, dev(case["idx"]), *ring_d,
                                dev(hist), dev(base), out, flush_min=fm, w_ring=16,
                                lower_bound=case["lower_bound"], scale=case["scale"])
    q = np.ascontiguousarray(f32(qkv[..., :W]).reshape(B, T, H, HD))
    k = np.ascontiguousarray(f32(qkv[..., W:2 * W]).reshape(B, T, H, HD))
    v = np.ascontiguousarray(f32(qkv[..., 2 * W:]).reshape(B, T, H, HD))
    g = np.ascontiguousarray(f32(gate).reshape(B, T, H, HD))
    ref_out = orc.verify(q, k, v, g, np.ascontiguousarray(f32(beta)), case["a_log"],
                         case["dt_bias"], case["lower_bound"], case["scale"], ref_pool,
                         case["idx"], *ring_o, hist, base, fm, 16, bf16_storage=True,
                         real=np.float32)
    torch.cuda.synchronize()
    check_out(bits(out).reshape(B, T, H, HD), ref_out, "verify after hand-off")
    got_pool = bits(pool)
    folded = 0
    for d in range(B):
        s_ = case["idx"][d]
        if hist[d] + T < fm:
            continue
        folded += 1
        # the fold commits the replay of what the prefill handed off
        for h in range(H):
            S = orc.replay(np.ascontiguousarray(pre_pool[s_, h]), pre_k[s_, h], pre_u[s_, h],
                           pre_g[s_, h], int(base[d]), int(hist[d]), real=np.float32)
            check_state(got_pool[s_, h], S, f"folded checkpoint doc {d} head {h}")
    assert folded == B - 1  # every document but the empty one
