"""Pins for the CPU oracle: each check compares the oracle with something other
than itself (exact rationals, a different formula, a library routine, a closed
form, or an invariant of the method), so that a dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them.

Pages cited by title:
  [verify]  "feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3 (KDA)"
  [decode]  "feat(kda): add packed-input CuTe decode kernel"
  [prefill] "feat(kda): add CuTe DSL recurrent prefill backend"
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

from gated_delta_rule_step_amd import synth

F64 = np.float64
F32 = np.float32
INT32_MIN = -(2 ** 31)
INT32_MAX = 2 ** 31 - 1


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(rng, n, m=None):
    x = rng.standard_normal((n,) if m is None else (m, n))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# bf16 round-to-nearest-even ([decode] "Kernel design": bf16 storage with RNE)

def _torch_bf16_bits(x_f32):
    t = torch.from_numpy(x_f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_on_random_patterns(orc):
    rng = _rng(1)
    bits = rng.integers(0, 2 ** 32, size=10_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    ours = orc.bf16_round_bits(x)
    ref = _torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN (payload may differ between implementations).
    back = synth.f32_from_bits(ours[nan])
    assert np.all(np.isnan(back))


def test_bf16_rne_tie_classes(orc):
    rng = _rng(2)
    upper = rng.integers(0, 2 ** 16, size=200_000, dtype=np.uint64).astype(np.uint32)
    pats = []
    for low in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
        pats.append((upper << 16) | low)
    # explicit boundary classes: largest finite, overflow to inf, subnormals, zeros
    pats.append(np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0xFF7FFFFF, 0x00008000,
                          0x00018000, 0x80008000, 0x00000000, 0x80000000, 0x7F800000,
                          0xFF800000], dtype=np.uint32))
    bits = np.concatenate(pats).astype(np.uint32)
    x = bits.view(np.float32)
    nan = np.isnan(x)
    assert np.array_equal(orc.bf16_round_bits(x)[~nan], _torch_bf16_bits(x)[~nan])


# ---------------------------------------------------------------------------
# Core step: brute force with exact rationals, through a different formula.
# S_new (K x V) = (I - beta k k^T) diag(alpha) S + beta k v^T, o = scale S_new^T q,
# the generalized-Householder form of the delta rule with per-channel decay.

def _frac_step(S_kv, q, k, v, alpha, beta, scale):
    K = len(k)
    V = len(v)
    DS = [[alpha[i] * S_kv[i][j] for j in range(V)] for i in range(K)]
    Hm = [[(1 if i == j else 0) - beta * k[i] * k[j] for j in range(K)] for i in range(K)]
    Snew = [[sum(Hm[i][m] * DS[m][j] for m in range(K)) + beta * k[i] * v[j] for j in range(V)]
            for i in range(K)]
    o = [scale * sum(Snew[i][j] * q[i] for i in range(K)) for j in range(V)]
    return Snew, o


@pytest.mark.parametrize("K,V,T", [(1, 1, 3), (2, 3, 4), (4, 4, 5), (3, 2, 2)])
def test_step_matches_exact_rational_householder_form(orc, K, V, T):
    rng = _rng(10 + K * 7 + V)
    S = rng.standard_normal((V, K))  # oracle orientation: [V][K]
    S_kv = [[Fraction(S[j, i]) for j in range(V)] for i in range(K)]
    S_or = S.copy()
    for _ in range(T):
        q = rng.standard_normal(K)
        k = rng.standard_normal(K)
        k /= np.linalg.norm(k)
        v = rng.standard_normal(V)
        g = -rng.uniform(0, 3, K)
        beta = float(rng.uniform(0, 1))
        scale = float(rng.uniform(0.5, 1.5))
        alpha = [Fraction(math.exp(x)) for x in g]
        S_kv, o_ex = _frac_step(S_kv, [Fraction(x) for x in q], [Fraction(x) for x in k],
                                [Fraction(x) for x in v], alpha, Fraction(beta), Fraction(scale))
        o, _ = orc.step(S_or, q, k, v, g, beta, scale, real=F64)
        ex_S = np.array([[float(S_kv[i][j]) for i in range(K)] for j in range(V)])
        ex_o = np.array([float(x) for x in o_ex])
        np.testing.assert_allclose(S_or, ex_S, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(o, ex_o, rtol=1e-12, atol=1e-12)


def test_step_fp32_close_to_fp64(orc):
    rng = _rng(11)
    K = V = 128
    S = rng.standard_normal((V, K)) * 0.05
    q, k = _unit(rng, K), _unit(rng, K)
    v = rng.standard_normal(V)
    g = -rng.uniform(0, 5, K)
    S64 = S.copy()
    S32 = S.astype(F32)
    o64, u64 = orc.step(S64, q, k, v, g, 0.7, 1.0, real=F64)
    o32, u32 = orc.step(S32, q.astype(F32), k.astype(F32), v.astype(F32), g.astype(F32),
                        0.7, 1.0, real=F32)
    np.testing.assert_allclose(o32, o64, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(u32, u64, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(S32, S64, rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------------------
# Invariants of the step (benchmark spec of the method).

def _decode_inputs(rng, B, H, N, real):
    K = V = 128
    d = dict(q=rng.standard_normal((B, H, K)), k=rng.standard_normal((B, H, K)),
             v=rng.standard_normal((B, H, V)), graw=rng.standard_normal((B, H, K)),
             beta_logit=rng.standard_normal((B, H)), a_log=rng.uniform(-1, 1, H),
             dt_bias=rng.standard_normal(H * K) * 0.1,
             pool=rng.standard_normal((N, H, V, K)) * 0.05)
    d = {n: np.ascontiguousarray(a.astype(real)) for n, a in d.items()}
    # bf16-representable values, as the GPU path receives them
    for n in ("q", "k", "v", "graw", "beta_logit", "pool"):
        d[n] = synth.f32_from_bits(synth.bf16_bits(d[n])).astype(real)
    return d


def test_beta0_gate0_leaves_state_bitwise_unchanged(orc):
    rng = _rng(20)
    B, H, N = 3, 2, 4
    d = _decode_inputs(rng, B, H, N, F32)
    d["a_log"][:] = -np.inf           # exp(A_log) = 0  -> g = 0, alpha = 1
    d["beta_logit"][:] = -np.inf      # sigmoid(-inf) = 0 -> beta = 0
    d["pool"][d["pool"] == 0] = 0.25  # avoid -0.0 + 0.0 sign flips
    pool0 = d["pool"].copy()
    idx = np.array([2, 0, 3], np.int32)
    out = orc.decode(d["q"], d["k"], d["v"], d["graw"], d["beta_logit"], d["a_log"],
                     d["dt_bias"], -5.0, 1.0, d["pool"], idx, bf16_storage=True, real=F32)
    assert np.array_equal(d["pool"].view(np.uint32), pool0.view(np.uint32))
    # and the read-out is then the plain matrix-vector product with the old state
    for b in range(B):
        for h in range(H):
            qn = d["q"][b, h].astype(F64)
            qh = qn / np.linalg.norm(qn)
            ref = pool0[idx[b], h].astype(F64) @ qh
            np.testing.assert_allclose(out[b, h], ref, rtol=1e-2, atol=1e-2)


def test_beta1_gives_exact_retrieval(orc):
    """beta = 1 writes v exactly under k_hat: S_new k_hat = v for a unit key."""
    rng = _rng(21)
    K = V = 128
    for real, tol in ((F64, 1e-12), (F32, 1e-5)):
        S = (rng.standard_normal((V, K)) * 0.05).astype(real)
        k = _unit(rng, K).astype(real)
        v = rng.standard_normal(V).astype(real)
        orc.step(S, _unit(rng, K).astype(real), k, v, (-rng.uniform(0, 5, K)).astype(real),
                 1.0, 1.0, real=real)
        np.testing.assert_allclose(S.astype(F64) @ k.astype(F64), v, rtol=tol, atol=tol)
    # through the raw path: beta logit +inf -> beta = 1; the key is normalised
    # in-kernel with a 1e-6 epsilon, so retrieval holds to ~1e-6 / |k|^2
    B, H, N = 2, 3, 2
    d = _decode_inputs(rng, B, H, N, F64)
    d["beta_logit"][:] = np.inf
    idx = np.array([1, 0], np.int32)
    orc.decode(d["q"], d["k"], d["v"], d["graw"], d["beta_logit"], d["a_log"],
               d["dt_bias"], -5.0, 1.0, d["pool"], idx, bf16_storage=False, real=F64)
    for b in range(B):
        for h in range(H):
            kk = d["k"][b, h]
            got = d["pool"][idx[b], h] @ (kk / np.linalg.norm(kk))
            np.testing.assert_allclose(got, d["v"][b, h], rtol=1e-7, atol=1e-7)


def test_orthonormal_keys_recall_every_value(orc):
    """Textbook associative memory: no decay, beta = 1, orthonormal keys:
    after writing n (key, value) pairs into an empty state, S k_i = v_i."""
    rng = _rng(22)
    K = V = 128
    n = 40
    keys, _ = np.linalg.qr(rng.standard_normal((K, n)))
    keys = keys.T.copy()
    vals = rng.standard_normal((n, V))
    S = np.zeros((V, K))
    for i in range(n):
        orc.step(S, keys[i].copy(), keys[i].copy(), vals[i].copy(), np.zeros(K), 1.0, 1.0,
                 real=F64)
    for i in range(n):
        np.testing.assert_allclose(S @ keys[i], vals[i], rtol=1e-11, atol=1e-11)


def test_beta0_closed_form_pure_decay(orc):
    rng = _rng(23)
    K = V = 128
    S0 = rng.standard_normal((V, K))
    S = S0.copy()
    G = np.zeros(K)
    for _ in range(6):
        q = _unit(rng, K)
        k = _unit(rng, K)
        g = -rng.uniform(0, 5, K)
        G += g
        o, u = orc.step(S, q, k, rng.standard_normal(V), g, 0.0, 0.5, real=F64)
        ref_S = S0 * np.exp(G)[None, :]
        np.testing.assert_allclose(S, ref_S, rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(o, 0.5 * ref_S @ q, rtol=1e-11, atol=1e-14)
        assert np.all(u == 0)


# ---------------------------------------------------------------------------
# Prologue: library routines and the gate's range.

def test_prologue_against_library_routines(orc):
    rng = _rng(30)
    K = 128
    for _ in range(20):
        q, k = rng.standard_normal(K) * 3, rng.standard_normal(K)
        graw = rng.standard_normal(K) * 4
        bl = float(rng.standard_normal() * 6)
        qh, kh, g, beta = orc.prologue(q, k, graw, bl, 0.0, np.zeros(K), -1e30, real=F64)
        np.testing.assert_allclose(qh, q / np.linalg.norm(q), rtol=1e-7)
        np.testing.assert_allclose(kh, k / np.linalg.norm(k), rtol=1e-7)
        # A_log = 0, dt_bias = 0, no clamp: g = -softplus(graw) = -log(1 + e^graw)
        np.testing.assert_allclose(g, -np.logaddexp(0.0, graw), rtol=1e-12, atol=1e-15)
        assert beta == pytest.approx(float(scipy.special.expit(bl)), rel=1e-14)


def test_gate_range_and_monotonicity(orc):
    rng = _rng(31)
    K = 128
    lb = -5.0
    prev = None
    for a_log in np.linspace(-3, 3, 13):
        graw = np.linspace(-30, 30, K)
        _, _, g, _ = orc.prologue(rng.standard_normal(K), rng.standard_normal(K), graw, 0.0,
                                  float(a_log), rng.standard_normal(K) * 0.1 * 0, lb, real=F64)
        assert np.all(g <= 0) and np.all(g >= lb)
        # decay strengthens (g decreases) as the raw gate logit grows
        assert np.all(np.diff(g) <= 0)
        # and as A_log grows, at fixed logits (until the clamp)
        if prev is not None:
            assert np.all(g <= prev + 1e-15)
        prev = g
    # the clamp is reached for large logits and not for very negative ones
    assert g[-1] == lb and g[0] > lb


def test_prologue_fp32_matches_fp64(orc):
    rng = _rng(32)
    K = 128
    q, k, graw = (rng.standard_normal(K).astype(F32) for _ in range(3))
    dtb = (rng.standard_normal(K) * 0.1).astype(F32)
    r32 = orc.prologue(q, k, graw, 0.3, 0.2, dtb, -5.0, real=F32)
    r64 = orc.prologue(q.astype(F64), k.astype(F64), graw.astype(F64), 0.3, 0.2,
                       dtb.astype(F64), -5.0, real=F64)
    for a, b in zip(r32[:3], r64[:3]):
        np.testing.assert_allclose(a, b, rtol=2e-6, atol=1e-6)
    assert r32[3] == pytest.approx(r64[3], rel=1e-6)


# ---------------------------------------------------------------------------
# Decode index handling ([decode] opening description; empty-pool review point)

def test_decode_inactive_rows_zero_and_pool_untouched(orc):
    rng = _rng(40)
    B, H, N = 6, 2, 4
    d = _decode_inputs(rng, B, H, N, F32)
    idx = np.array([-1, 3, N, INT32_MIN, INT32_MAX, 0], np.int32)
    pool0 = d["pool"].copy()
    out = orc.decode(d["q"], d["k"], d["v"], d["graw"], d["beta_logit"], d["a_log"],
                     d["dt_bias"], -5.0, 1.0, d["pool"], idx, real=F32)
    for b in (0, 2, 3, 4):
        assert np.all(out[b] == 0) and not np.any(np.signbit(out[b]))
    for s in (1, 2):
        assert np.array_equal(d["pool"][s].view(np.uint32), pool0[s].view(np.uint32))
    for s in (0, 3):
        assert not np.array_equal(d["pool"][s], pool0[s])


def test_decode_empty_pool_all_inactive(orc):
    rng = _rng(41)
    d = _decode_inputs(rng, 3, 2, 1, F32)
    empty = np.zeros((0, 2, 128, 128), F32)
    out = orc.decode(d["q"], d["k"], d["v"], d["graw"], d["beta_logit"], d["a_log"],
                     d["dt_bias"], -5.0, 1.0, empty, np.array([0, 1, -1], np.int32), real=F32)
    assert np.all(out == 0)


def test_decode_bf16_storage_points(orc):
    """With storage rounding on, the written state and outputs are bf16 values
    equal to the bf16 rounding of the unrounded fp32 results."""
    rng = _rng(42)
    d = _decode_inputs(rng, 2, 2, 2, F32)
    idx = np.array([1, 0], np.int32)
    p_r, p_u = d["pool"].copy(), d["pool"].copy()
    args = [d[n] for n in ("q", "k", "v", "graw", "beta_logit", "a_log", "dt_bias")]
    o_r = orc.decode(*args, -5.0, 1.0, p_r, idx, bf16_storage=True, real=F32)
    o_u = orc.decode(*args, -5.0, 1.0, p_u, idx, bf16_storage=False, real=F32)
    assert np.array_equal(synth.f32_from_bits(synth.bf16_bits(o_u)), o_r)
    assert np.array_equal(synth.f32_from_bits(synth.bf16_bits(p_u)), p_r)


# ---------------------------------------------------------------------------
# Ring replay, verify and fold ([verify] "What it does", "API", "Caching")

def _tok(rng, T, H, K=128, V=128):
    return dict(q=rng.standard_normal((1, T, H, K)), k=rng.standard_normal((1, T, H, K)),
                v=rng.standard_normal((1, T, H, V)), graw=rng.standard_normal((1, T, H, K)),
                beta_logit=rng.standard_normal((1, T, H)))


def _seq_reference(orc, S0, toks, h, a_log, dt_bias, lb, scale):
    """Sequential stepping of one head from S0 over all tokens in toks (fp64)."""
    S = S0.copy()
    outs = []
    T = toks["q"].shape[1]
    for t in range(T):
        qh, kh, g, beta = orc.prologue(toks["q"][0, t, h], toks["k"][0, t, h],
                                       toks["graw"][0, t, h], toks["beta_logit"][0, t, h],
                                       a_log[h], dt_bias[h * 128:(h + 1) * 128], lb, real=F64)
        o, _ = orc.step(S, qh, kh, toks["v"][0, t, h].copy(), g, beta, scale, real=F64)
        outs.append(o)
    return S, np.array(outs)


def _slice(toks, a, b):
    return {n: np.ascontiguousarray(x[:, a:b]) for n, x in toks.items()}


def _verify(orc, toks, pool, kc, uc, gc, hist, base, fm, w, a_log, dt_bias, lb=-5.0, scale=1.0,
            real=F64, bf16=False, idx=0):
    return orc.verify(toks["q"], toks["k"], toks["v"], toks["graw"], toks["beta_logit"], a_log,
                      dt_bias, lb, scale, pool, np.array([idx], np.int32), kc, uc, gc,
                      np.array([hist], np.int32), np.array([base], np.int32), fm, w,
                      bf16_storage=bf16, real=real)


def _empty_ring(H, R=32):
    return (np.zeros((1, H, R, 128)), np.zeros((1, H, R, 128)), np.zeros((1, H, R, 128)))


@pytest.mark.parametrize("base,n_hist", [(0, 5), (29, 8), (13, 16)])
def test_replay_equals_sequential_stepping(orc, base, n_hist):
    rng = _rng(50 + base)
    H = 2
    a_log, dtb = rng.uniform(-1, 1, H), rng.standard_normal(H * 128) * 0.1
    S0 = rng.standard_normal((1, H, 128, 128)) * 0.05
    toks = _tok(rng, n_hist, H)
    kc, uc, gc = _empty_ring(H)
    pool = S0.copy()
    # append n_hist tokens to the ring from a bare checkpoint, without folding
    _verify(orc, toks, pool, kc, uc, gc, 0, base, 10 ** 6, 10 ** 6, a_log, dtb)
    assert np.array_equal(pool, S0)  # no fold: the checkpoint is untouched
    for h in range(H):
        S_seq, _ = _seq_reference(orc, S0[0, h], toks, h, a_log, dtb, -5.0, 1.0)
        S_rep = orc.replay(S0[0, h].copy(), kc[0, h].copy(), uc[0, h].copy(), gc[0, h].copy(),
                           base, n_hist, real=F64)
        np.testing.assert_allclose(S_rep, S_seq, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("T,fm,w,hist", [(8, 9, 16, 5), (4, 13, 16, 9), (8, 25, 32, 20),
                                         (8, 9, 16, 0), (4, 13, 16, 3)])
def test_verify_outputs_and_fold_equal_sequential(orc, T, fm, w, hist):
    rng = _rng(60 + T + hist)
    H, base = 2, 27
    a_log, dtb = rng.uniform(-1, 1, H), rng.standard_normal(H * 128) * 0.1
    S0 = rng.standard_normal((1, H, 128, 128)) * 0.05
    toks = _tok(rng, hist + T, H)
    kc, uc, gc = _empty_ring(H)
    pool = S0.copy()
    if hist:
        _verify(orc, _slice(toks, 0, hist), pool, kc, uc, gc, 0, base, 10 ** 6, 10 ** 6,
                a_log, dtb)
    # poison every ring row that is not live history: must never be read
    for j in range(hist, 32):
        r = (base + j) % 32
        kc[0, :, r] = np.nan
        uc[0, :, r] = np.nan
        gc[0, :, r] = np.nan
    out = _verify(orc, _slice(toks, hist, hist + T), pool, kc, uc, gc, hist, base, fm, w,
                  a_log, dtb)
    fold = hist + T >= fm
    for h in range(H):
        S_hist, _ = _seq_reference(orc, S0[0, h], _slice(toks, 0, hist), h, a_log, dtb, -5.0, 1.0)
        _, outs = _seq_reference(orc, S_hist, _slice(toks, hist, hist + T), h, a_log, dtb,
                                 -5.0, 1.0)
        np.testing.assert_allclose(out[0, :, h], outs, rtol=1e-10, atol=1e-12)
        if fold:
            np.testing.assert_allclose(pool[0, h], S_hist, rtol=1e-10, atol=1e-12)
        else:
            assert np.array_equal(pool[0, h], S0[0, h])
        # ring rows for the draft tokens: k_hat and the cumulative log-decay,
        # restarted at 0 on a fold and continued from G_{hist-1} otherwise
        G = np.zeros(128)
        if not fold and hist:
            G = G + gc[0, h, (base + hist - 1) % 32]
        for t in range(T):
            r = (base + hist + t) % 32
            kk = toks["k"][0, hist + t, h]
            np.testing.assert_allclose(kc[0, h, r], kk / np.linalg.norm(kk), rtol=1e-7)
            _, _, g, _ = orc.prologue(toks["q"][0, hist + t, h], kk, toks["graw"][0, hist + t, h],
                                      toks["beta_logit"][0, hist + t, h], a_log[h],
                                      dtb[h * 128:(h + 1) * 128], -5.0, real=F64)
            G = G + g
            np.testing.assert_allclose(gc[0, h, r], G, rtol=1e-13, atol=1e-13)


def test_fold_split_point_associativity(orc):
    """The committed state does not depend on where folds happen: two call
    sequences over the same 16 accepted tokens, folding at different points,
    commit the sequential state (observed with a forced fold, flush_min = 1)."""
    rng = _rng(70)
    H = 1
    a_log, dtb = rng.uniform(-1, 1, H), rng.standard_normal(H * 128) * 0.1
    S0 = rng.standard_normal((1, H, 128, 128)) * 0.05
    toks = _tok(rng, 17, H)
    S_ref, _ = _seq_reference(orc, S0[0, 0], _slice(toks, 0, 16), 0, a_log, dtb, -5.0, 1.0)

    def run(plan):
        pool = S0.copy()
        kc, uc, gc = _empty_ring(H)
        hist, base, pos = 0, 5, 0
        for T, fm in plan:
            _verify(orc, _slice(toks, pos, pos + T), pool, kc, uc, gc, hist, base, fm, 32,
                    a_log, dtb)
            if hist + T >= fm:
                base, hist = (base + hist) % 32, T
            else:
                hist += T
            pos += T
        _verify(orc, _slice(toks, 16, 17), pool, kc, uc, gc, hist, base, 1, 32, a_log, dtb)
        return pool[0, 0]

    a = run([(8, 100), (8, 100)])           # no fold until the final forced one
    b = run([(4, 100), (4, 5), (8, 100)])   # fold after 4 tokens
    c = run([(8, 1), (4, 1), (4, 100)])     # fold on every call but the last
    for got in (a, b, c):
        np.testing.assert_allclose(got, S_ref, rtol=1e-10, atol=1e-12)


def test_deep_window_cumulative_decay_range(orc):
    """W32, T=8, gates at the lower bound: G reaches -5 * 32 = -160 and the
    replay stays finite (all replay weights exp(G_L - G_j) <= 1)."""
    H = 1
    a_log, dtb = np.zeros(H), np.zeros(128)
    rng = _rng(80)
    S0 = rng.standard_normal((1, H, 128, 128)) * 0.05
    toks = _tok(rng, 32, H)
    toks["graw"][:] = 60.0  # softplus(60) = 60 -> clamped at -5
    kc, uc, gc = _empty_ring(H)
    pool = S0.copy()
    _verify(orc, _slice(toks, 0, 24), pool, kc, uc, gc, 0, 3, 10 ** 6, 10 ** 6, a_log, dtb)
    out = _verify(orc, _slice(toks, 24, 32), pool, kc, uc, gc, 24, 3, 25, 32, a_log, dtb,
                  real=F64)
    # 24 history tokens clamped at -5 each: G_23 = -120 exactly (sums of -5
    # are exact in fp64), the lowest value the ring holds after the fold
    assert gc.min() == -120.0
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(pool))
    S_seq, outs = _seq_reference(orc, S0[0, 0], _slice(toks, 0, 24), 0, a_log, dtb, -5.0, 1.0)
    np.testing.assert_allclose(pool[0, 0], S_seq, rtol=1e-10, atol=1e-300)
    # fp32 G of 24 clamped tokens is exactly -120 (sums of -5 are exact)
    kc2, uc2, gc2 = (x.astype(F32) for x in _empty_ring(H))
    pool2 = S0.astype(F32)
    t32 = {n: x.astype(F32) for n, x in _slice(toks, 0, 24).items()}
    _verify(orc, t32, pool2, kc2, uc2, gc2, 0, 3, 10 ** 6, 10 ** 6, a_log.astype(F32),
            dtb.astype(F32), real=F32)
    assert gc2[0, 0, (3 + 23) % 32].min() == -120.0


def test_verify_inactive_rows(orc):
    rng = _rng(90)
    H, T, R = 2, 4, 32
    a_log, dtb = rng.uniform(-1, 1, H), rng.standard_normal(H * 128) * 0.1
    toks = _tok(rng, T, H)
    toks = {n: np.repeat(x, 5, axis=0) for n, x in toks.items()}
    N = 3
    pool = rng.standard_normal((N, H, 128, 128))
    kc, uc, gc = (rng.standard_normal((N, H, R, 128)) for _ in range(3))
    snap = [x.copy() for x in (pool, kc, uc, gc)]
    # bad slot, negative hist, hist + T > w_ring, cache_base out of range, all-bad,
    # and hist_len within T of INT32_MAX (hist + T would wrap to a negative int32)
    toks = {n: np.concatenate([x, x[:2]], axis=0) for n, x in toks.items()}
    imax = np.iinfo(np.int32).max
    idx = np.array([-1, 0, 1, 2, N, 0, 1], np.int32)
    hist = np.array([0, -1, 13, 0, 0, imax, imax - 3], np.int32)
    base = np.array([0, 0, 0, R, 0, 0, 0], np.int32)
    out = orc.verify(toks["q"], toks["k"], toks["v"], toks["graw"], toks["beta_logit"], a_log,
                     dtb, -5.0, 1.0, pool, idx, kc, uc, gc, hist, base, 13, 16,
                     bf16_storage=False, real=F64)
    assert np.all(out == 0)
    for a, b in zip((pool, kc, uc, gc), snap):
        assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# Prefill ([prefill]: cu_seqlens contract, zero-length documents)

def _prefill_inputs(rng, lens, H, real=F64, N=None):
    Tt = int(sum(lens))
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    N = 2 * len(lens) if N is None else N
    d = dict(q=rng.standard_normal((Tt, H, 128)), k=rng.standard_normal((Tt, H, 128)),
             v=rng.standard_normal((Tt, H, 128)), graw=rng.standard_normal((Tt, H, 128)),
             beta_logit=rng.standard_normal((Tt, H)), a_log=rng.uniform(-1, 1, H),
             dt_bias=rng.standard_normal(H * 128) * 0.1,
             pool=rng.standard_normal((N, H, 128, 128)) * 0.05)
    d = {n: np.ascontiguousarray(a.astype(real)) for n, a in d.items()}
    d["cu"] = cu
    d["idx"] = rng.permutation(N)[:len(lens)].astype(np.int32)
    return d


def _pf_args(d):
    return (d["cu"], d["q"], d["k"], d["v"], d["graw"], d["beta_logit"], d["a_log"],
            d["dt_bias"], -5.0, 1.0)


@pytest.mark.parametrize("chunk", [1, 16, 64])
def test_chunked_form_equals_token_by_token(orc, chunk):
    rng = _rng(100 + chunk)
    d = _prefill_inputs(rng, (0, 17, 64, 100, 130), H=2)
    p1, p2 = d["pool"].copy(), d["pool"].copy()
    o1 = orc.prefill(*_pf_args(d), p1, d["idx"], bf16_storage=False, real=F64)
    o2 = orc.prefill_chunked(*_pf_args(d), p2, d["idx"], chunk, real=F64)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(p2, p1, rtol=1e-10, atol=1e-11)


def test_chunked_form_zero_initial_state(orc):
    rng = _rng(105)
    d = _prefill_inputs(rng, (70, 0, 33), H=1)
    p1, p2 = d["pool"].copy(), d["pool"].copy()
    o1 = orc.prefill(*_pf_args(d), p1, d["idx"], use_initial_state=False, bf16_storage=False,
                     real=F64)
    o2 = orc.prefill_chunked(*_pf_args(d), p2, d["idx"], 64, use_initial_state=False, real=F64)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(p2, p1, rtol=1e-10, atol=1e-11)
    # zero-length document without an initial state: final state is zeros
    assert np.all(p1[d["idx"][1]] == 0)


def test_prefill_equals_repeated_decode(orc):
    """Prefill over one document equals T = 1 decode steps on the same slot."""
    rng = _rng(106)
    d = _prefill_inputs(rng, (9,), H=2, real=F32)
    for n in ("q", "k", "v", "graw", "beta_logit", "pool"):
        d[n] = synth.f32_from_bits(synth.bf16_bits(d[n]))
    pool_p, pool_d = d["pool"].copy(), d["pool"].copy()
    out_p = orc.prefill(*_pf_args(d), pool_p, d["idx"], real=F32)
    for t in range(9):
        sl = slice(t, t + 1)
        o = orc.decode(d["q"][sl].copy(), d["k"][sl].copy(), d["v"][sl].copy(),
                       d["graw"][sl].copy(), d["beta_logit"][sl].copy(), d["a_log"],
                       d["dt_bias"], -5.0, 1.0, pool_d, d["idx"][:1].copy(), bf16_storage=False,
                       real=F32)
        np.testing.assert_allclose(out_p[t], synth.f32_from_bits(synth.bf16_bits(o[0])),
                                   rtol=0, atol=0)
    assert np.array_equal(pool_p, synth.f32_from_bits(synth.bf16_bits(pool_d)))


def test_prefill_document_isolation_and_inactive(orc):
    rng = _rng(107)
    d = _prefill_inputs(rng, (20, 15, 0, 11), H=2, real=F32)
    d["idx"][3] = -1  # inactive document
    p1 = d["pool"].copy()
    o1 = orc.prefill(*_pf_args(d), p1, d["idx"], real=F32)
    # perturb document 1's inputs: documents 0 and 3 are bitwise unchanged
    d2 = {n: (x.copy() if isinstance(x, np.ndarray) else x) for n, x in d.items()}
    d2["v"][20:35] += 1.0
    d2["graw"][20:35] -= 0.5
    p2 = d2["pool"].copy()
    o2 = orc.prefill(*_pf_args(d2), p2, d2["idx"], real=F32)
    assert np.array_equal(o1[:20], o2[:20])
    assert np.array_equal(p1[d["idx"][0]], p2[d["idx"][0]])
    assert not np.array_equal(o1[20:35], o2[20:35])
    assert np.all(o1[35:] == 0)
    # the zero-length document with an initial state leaves its slot as it was
    assert np.array_equal(p1[d["idx"][2]], d["pool"][d["idx"][2]])
    # slots not referenced by an active document are untouched
    used = set(int(x) for x in d["idx"][:3])
    for s in range(d["pool"].shape[0]):
        if s not in used:
            assert np.array_equal(p1[s].view(np.uint32), d["pool"][s].view(np.uint32))


# ---------------------------------------------------------------------------
# Pre-computed gate convention ([decode] "T=1 fast path inside recurrent_kda":
# the raw form computes decay and sigmoid in-kernel; the API-default form takes
# log-space g and pre-sigmoided beta, decay = exp(g)).

PRE = 1 | 2  # pre-computed gate and pre-sigmoided beta


def _gate_np(graw, a_log, dt_bias, lb):
    """The raw gate written out with numpy's own routines (fp64): softplus as
    log(1 + e^x) through logaddexp, then the clamp."""
    H = a_log.shape[0]
    x = graw.reshape(graw.shape[:-2] + (H, 128)) + dt_bias.reshape(H, 128)
    g = -np.exp(a_log)[:, None] * np.logaddexp(0.0, x)
    return np.maximum(lb, g)


def test_precomputed_mode_equals_raw_mode_fed_the_gate(orc):
    """Decode, verify and prefill in the pre-computed mode, given g and beta
    computed independently from the raw inputs, reproduce the raw mode."""
    rng = _rng(200)
    lb = -5.0
    B, H, N = 3, 2, 4
    d = _decode_inputs(rng, B, H, N, F64)
    g = _gate_np(d["graw"], d["a_log"], d["dt_bias"], lb)
    beta = scipy.special.expit(d["beta_logit"])
    idx = np.array([3, 0, 1], np.int32)
    p_raw, p_pre = d["pool"].copy(), d["pool"].copy()
    o_raw = orc.decode(d["q"], d["k"], d["v"], d["graw"], d["beta_logit"], d["a_log"],
                       d["dt_bias"], lb, 1.0, p_raw, idx, bf16_storage=False, real=F64)
    o_pre = orc.decode(d["q"], d["k"], d["v"], np.ascontiguousarray(g), beta, None, None, lb,
                       1.0, p_pre, idx, bf16_storage=False, real=F64, gate_mode=PRE)
    np.testing.assert_allclose(o_pre, o_raw, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(p_pre, p_raw, rtol=1e-12, atol=1e-14)

    toks = _tok(rng, 4, H)
    toks = {n: a.astype(F64) for n, a in toks.items()}
    a_log, dt_bias = rng.uniform(-1, 1, H), rng.standard_normal(H * 128) * 0.1
    R = 32
    res = []
    for mode in (0, PRE):
        pool = d["pool"][:2].copy()
        kc, uc, gc = (np.zeros((2, H, R, 128)) for _ in range(3))
        hist = np.zeros(1, np.int32)
        base = np.array([5], np.int32)
        if mode:
            gr = np.ascontiguousarray(_gate_np(toks["graw"], a_log, dt_bias, lb))
            bl = scipy.special.expit(toks["beta_logit"])
            al = db = None
        else:
            gr, bl, al, db = toks["graw"], toks["beta_logit"], a_log, dt_bias
        out = orc.verify(toks["q"], toks["k"], toks["v"], gr, bl, al, db, lb, 1.0, pool,
                         np.array([1], np.int32), kc, uc, gc, hist, base, 5, 16,
                         bf16_storage=False, real=F64, gate_mode=mode)
        res.append((out, pool, kc, uc, gc))
    for a, b in zip(res[0], res[1]):
        np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-14)

    p = _prefill_inputs(rng, (21, 0, 9), H=2)
    gp = np.ascontiguousarray(_gate_np(p["graw"], p["a_log"], p["dt_bias"], lb))
    bp = scipy.special.expit(p["beta_logit"])
    q1, q2 = p["pool"].copy(), p["pool"].copy()
    o1 = orc.prefill(*_pf_args(p), q1, p["idx"], bf16_storage=False, real=F64)
    o2 = orc.prefill(p["cu"], p["q"], p["k"], p["v"], gp, bp, None, None, lb, 1.0, q2, p["idx"],
                     bf16_storage=False, real=F64, gate_mode=PRE)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(q2, q1, rtol=1e-12, atol=1e-14)
    # and its chunked form agrees with it
    q3 = p["pool"].copy()
    o3 = orc.prefill_chunked(p["cu"], p["q"], p["k"], p["v"], gp, bp, None, None, lb, 1.0, q3,
                             p["idx"], 16, real=F64, gate_mode=PRE)
    np.testing.assert_allclose(o3, o1, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(q3, q1, rtol=1e-10, atol=1e-11)


def test_precomputed_prologue_uses_g_and_beta_as_given(orc):
    """The pre-computed prologue passes g through inside [lb, 0], clamps it
    outside, and passes beta through; each bit acts alone."""
    rng = _rng(201)
    K = 128
    lb = -3.0
    q, k = rng.standard_normal(K), rng.standard_normal(K)
    g_in = np.concatenate([rng.uniform(lb, 0, K - 4), [lb - 1.0, -1e30, 0.5, 0.0]])
    _, _, g, beta = orc.prologue(q, k, g_in, 0.37, 0.0, np.zeros(K), lb, real=F64, gate_mode=3)
    np.testing.assert_array_equal(g[:K - 4], g_in[:K - 4])
    np.testing.assert_array_equal(g[K - 4:], [lb, lb, 0.0, 0.0])
    assert beta == 0.37
    # gate bit only: beta still goes through the sigmoid
    _, _, g1, beta1 = orc.prologue(q, k, g_in, 0.37, 0.0, np.zeros(K), lb, real=F64, gate_mode=1)
    np.testing.assert_array_equal(g1, g)
    assert beta1 == pytest.approx(float(scipy.special.expit(0.37)), rel=1e-15)
    # beta bit only: the gate is still the raw formula (A_log = 0, dt_bias = 0)
    graw = rng.standard_normal(K)
    _, _, g2, beta2 = orc.prologue(q, k, graw, 0.37, 0.0, np.zeros(K), -1e30, real=F64,
                                   gate_mode=2)
    np.testing.assert_allclose(g2, -np.logaddexp(0.0, graw), rtol=1e-12, atol=1e-15)
    assert beta2 == 0.37


def test_precomputed_beta1_exact_retrieval_and_beta0_pure_decay(orc):
    """With beta = 1 given exactly, decode writes v under k_hat (S_new k_hat = v);
    with beta = 0 and g given, the state is exp(g)-decayed and nothing else."""
    rng = _rng(202)
    B, H, N = 2, 2, 3
    d = _decode_inputs(rng, B, H, N, F64)
    g = -rng.uniform(0, 5, (B, H, 128))
    idx = np.array([2, 0], np.int32)
    pool = d["pool"].copy()
    orc.decode(d["q"], d["k"], d["v"], g, np.ones((B, H)), None, None, -5.0, 1.0, pool, idx,
               bf16_storage=False, real=F64, gate_mode=PRE)
    for b in range(B):
        for h in range(H):
            kk = d["k"][b, h]
            got = pool[idx[b], h] @ (kk / np.sqrt(kk @ kk + 1e-6))
            # |k_hat|^2 = 1 - 1e-6 / |k|^2 (the norm's epsilon): retrieval to ~1e-8
            np.testing.assert_allclose(got, d["v"][b, h], rtol=1e-7, atol=1e-7)
    pool = d["pool"].copy()
    out = orc.decode(d["q"], d["k"], d["v"], g, np.zeros((B, H)), None, None, -5.0, 0.5, pool,
                     idx, bf16_storage=False, real=F64, gate_mode=PRE)
    for b in range(B):
        for h in range(H):
            ref = d["pool"][idx[b], h] * np.exp(g[b, h])[None, :]
            np.testing.assert_allclose(pool[idx[b], h], ref, rtol=1e-14, atol=1e-300)
            qq = d["q"][b, h]
            np.testing.assert_allclose(out[b, h], 0.5 * ref @ (qq / np.sqrt(qq @ qq + 1e-6)),
                                       rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Prefill intermediate checkpoints ([prefill]: output, final state,
# checkpoints; checkpoint_cu_starts). Reading: the state after every
# `interval` tokens of a document.

def test_prefill_checkpoints_equal_truncated_prefills(orc):
    """Checkpoint i of document d equals the final state of the same prefill
    run on d's first i * interval tokens; the final state is unchanged by
    asking for checkpoints; rows outside the buffer and inactive documents
    write nothing."""
    rng = _rng(210)
    lens = (40, 0, 64, 15, 33)
    interval = 16
    d = _prefill_inputs(rng, lens, H=2)
    d["idx"][3] = -1  # inactive: no checkpoints
    counts = [n // interval for n in lens]          # 2, 0, 4, 0, 2
    starts = np.array([0, 2, 2, 6, 7], np.int64)    # row 6 is a gap; doc 4 takes 7 and 8
    rows = 8                                        # doc 4's row 8 lies outside: skipped
    ck = np.full((rows, 2, 128, 128), -7.0)
    p1 = d["pool"].copy()
    o1 = orc.prefill(*_pf_args(d), p1, d["idx"], bf16_storage=False, real=F64,
                     checkpoints=ck, checkpoint_starts=starts, checkpoint_interval=interval)
    p0 = d["pool"].copy()
    o0 = orc.prefill(*_pf_args(d), p0, d["idx"], bf16_storage=False, real=F64)
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(p1, p0)
    written = np.zeros(rows, bool)
    for doc, n in enumerate(lens):
        if d["idx"][doc] < 0:
            continue
        for i in range(1, counts[doc] + 1):
            row = starts[doc] + i - 1
            if row >= rows:
                continue
            # the same document truncated to its first i * interval tokens
            t0 = int(d["cu"][doc])
            sl = slice(t0, t0 + i * interval)
            sub = dict(cu=np.array([0, i * interval], np.int32),
                       **{n_: np.ascontiguousarray(d[n_][sl])
                          for n_ in ("q", "k", "v", "graw", "beta_logit")})
            pool = d["pool"].copy()
            orc.prefill(sub["cu"], sub["q"], sub["k"], sub["v"], sub["graw"],
                        sub["beta_logit"], d["a_log"], d["dt_bias"], -5.0, 1.0, pool,
                        d["idx"][doc:doc + 1].copy(), bf16_storage=False, real=F64)
            np.testing.assert_array_equal(ck[row], pool[d["idx"][doc]])
            written[row] = True
    assert written.tolist() == [True] * 6 + [False, True]
    assert np.all(ck[~written] == -7.0)


# ---------------------------------------------------------------------------
# Per-head (scalar) gate: GDN's decay, which [verify] "What it does" contrasts
# with KDA's per-key-channel gate. Reading: the same gate formula on per-head
# inputs, applied to every key channel.

PER_HEAD = 4


@pytest.mark.parametrize("pre", [0, 1])
def test_per_head_gate_equals_broadcast_channel_gate(orc, pre):
    """Decode, verify and prefill with one gate value per head reproduce,
    bit for bit, the per-channel mode given that value (and dt_bias)
    repeated over the 128 key channels; raw and pre-computed forms."""
    rng = _rng(220 + pre)
    lb = -5.0
    B, H, N = 3, 2, 4
    d = _decode_inputs(rng, B, H, N, F64)
    gh = rng.standard_normal((B, H)) if not pre else rng.uniform(-6, 0.5, (B, H))
    dth = rng.standard_normal(H) * 0.1
    g_bc = np.ascontiguousarray(np.repeat(gh[:, :, None], 128, axis=2))
    dt_bc = np.ascontiguousarray(np.repeat(dth, 128))
    al, dhd, dbc = (None, None, None) if pre else (d["a_log"], dth, dt_bc)
    idx = np.array([3, 0, 1], np.int32)
    p1, p2 = d["pool"].copy(), d["pool"].copy()
    o1 = orc.decode(d["q"], d["k"], d["v"], np.ascontiguousarray(gh), d["beta_logit"], al, dhd,
                    lb, 1.0, p1, idx, bf16_storage=False, real=F64, gate_mode=PER_HEAD | pre)
    o2 = orc.decode(d["q"], d["k"], d["v"], g_bc, d["beta_logit"], al, dbc, lb, 1.0, p2, idx,
                    bf16_storage=False, real=F64, gate_mode=pre)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(p1, p2)
    # the per-head decay really is one value across the key channels
    assert not np.array_equal(p1, d["pool"])

    toks = {n: a.astype(F64) for n, a in _tok(rng, 4, H).items()}
    gt = rng.standard_normal((1, 4, H)) if not pre else rng.uniform(-6, 0.5, (1, 4, H))
    gt_bc = np.ascontiguousarray(np.repeat(gt[..., None], 128, axis=3))
    res = []
    for gm, gr, db in ((PER_HEAD | pre, np.ascontiguousarray(gt), dhd), (pre, gt_bc, dbc)):
        pool = d["pool"][:2].copy()
        kc, uc, gc = (np.zeros((2, H, 32, 128)) for _ in range(3))
        out = orc.verify(toks["q"], toks["k"], toks["v"], gr, toks["beta_logit"], al, db, lb,
                         1.0, pool, np.array([1], np.int32), kc, uc, gc,
                         np.zeros(1, np.int32), np.array([30], np.int32), 5, 16,
                         bf16_storage=False, real=F64, gate_mode=gm)
        res.append((out, pool, kc, uc, gc))
    for a, b in zip(*res):
        np.testing.assert_array_equal(a, b)

    p = _prefill_inputs(rng, (21, 0, 9), H=2)
    T = p["q"].shape[0]
    gp = rng.standard_normal((T, 2)) if not pre else rng.uniform(-6, 0.5, (T, 2))
    gp_bc = np.ascontiguousarray(np.repeat(gp[..., None], 128, axis=2))
    outs = []
    for gm, gr, db in ((PER_HEAD | pre, np.ascontiguousarray(gp), dhd), (pre, gp_bc, dbc)):
        pool = p["pool"].copy()
        o = orc.prefill(p["cu"], p["q"], p["k"], p["v"], gr, p["beta_logit"],
                        None if pre else p["a_log"], db, lb, 1.0, pool, p["idx"],
                        bf16_storage=False, real=F64, gate_mode=gm)
        oc = orc.prefill_chunked(p["cu"], p["q"], p["k"], p["v"], gr, p["beta_logit"],
                                 None if pre else p["a_log"], db, lb, 1.0, p["pool"].copy(),
                                 p["idx"], 16, real=F64, gate_mode=gm)
        outs.append((o, pool, oc))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
    np.testing.assert_allclose(outs[0][2], outs[0][0], rtol=1e-10, atol=1e-11)


# ---------------------------------------------------------------------------
# fp16 state option ([verify] "Caching": the GDN kernel offers an fp16
# checkpoint-state mode). The rounding is written from the binary16 format;
# torch's float32 -> float16 cast is the independent reference.

def test_f16_rne_matches_torch(orc):
    rng = _rng(230)
    bits = rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    # every class near the binary16 range: ties, subnormals, overflow edge
    special = []
    for e in range(-26, 17):
        base = np.float32(2.0 ** e)
        for k in range(0, 1 << 11, 37):
            m = np.float32(1 + k / 2048.0)
            special.append(base * m)
            special.append(base * (m + np.float32(2.0 ** -11)))  # exact binary16 ties
    special += [65504.0, 65519.996, 65520.0, 65536.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.5,
                6.0e-8, 5.96e-8, 0.0, -0.0, np.inf, -np.inf]
    sp = np.array(special, np.float32)
    x = np.concatenate([x, sp, -sp])
    ours = orc.f16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # and back: fp16 bits -> fp32 is exact (torch's widening)
    allb = np.arange(65536, dtype=np.uint16)
    allb = allb[(allb & 0x7c00) != 0x7c00]  # finite encodings
    back = orc.f16_bits_to_f32(allb)
    np.testing.assert_array_equal(back, torch.from_numpy(allb.view(np.int16)).view(
        torch.float16).to(torch.float32).numpy())


def _f16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float16).to(
        torch.float32).numpy()


# fp8 e4m3 state option (the decode page names byte reduction as the lever that
# remains; the format is OCP e4m3fn, saturating at +-448). torch's float8_e4m3fn
# cast of the clamped value is the independent reference.

def _f8(x):
    x = np.clip(np.ascontiguousarray(x, np.float32), -448.0, 448.0)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float32).numpy()


def test_f8_rne_matches_torch(orc):
    rng = _rng(232)
    bits = rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    allv = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(
        torch.float32).numpy()
    fin = np.unique(allv[np.isfinite(allv)])
    mids = ((fin[1:].astype(np.float64) + fin[:-1]) / 2).astype(np.float32)  # exact ties
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    sp = np.concatenate([fin, mids, up, dn, rng.standard_normal(100_000).astype(np.float32) * 0.05,
                         np.array([447, 449, 464, 465, 480, 1e4, np.inf, 2.0 ** -10,
                                   2.0 ** -11, 1.5 * 2.0 ** -10, 1e-30, 0.0], np.float32)])
    x = np.concatenate([x, sp, -sp])
    ours = orc.f8_round_bits(x)
    ref = torch.from_numpy(np.clip(x, -448.0, 448.0)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)
    # and back: every finite encoding widens exactly
    allb = np.arange(256, dtype=np.uint8)
    finite = np.isfinite(allv)
    np.testing.assert_array_equal(orc.f8_bits_to_f32(allb)[finite], allv[finite])
    assert np.all(np.isnan(orc.f8_bits_to_f32(allb)[~finite]))


@pytest.mark.parametrize("state_dtype", [1, 2])
def test_low_byte_state_rounds_only_the_state_storage_points(orc, state_dtype):
    """Decode, verify (fold) and prefill with fp16 (1) or fp8 (2) state equal
    the same run without state rounding followed by torch's cast of the stored
    states; outputs keep their bf16 rounding."""
    cast = {1: _f16, 2: _f8}[state_dtype]
    rng = _rng(231)
    B, H, N = 3, 2, 4
    d = _decode_inputs(rng, B, H, N, F32)
    d["pool"] = cast(d["pool"])
    idx = np.array([3, 0, 1], np.int32)
    pa, pb = d["pool"].copy(), d["pool"].copy()
    args = (d["q"], d["k"], d["v"], d["graw"], d["beta_logit"], d["a_log"], d["dt_bias"], -5.0,
            1.0)
    oa = orc.decode(*args, pa, idx, bf16_storage=True, real=F32, state_dtype=state_dtype)
    ob = orc.decode(*args, pb, idx, bf16_storage=False, real=F32)
    np.testing.assert_array_equal(pa[idx], cast(pb[idx]))
    np.testing.assert_array_equal(oa, synth.f32_from_bits(synth.bf16_bits(ob)))
    assert not np.array_equal(pa[idx], synth.f32_from_bits(synth.bf16_bits(pb[idx])))

    toks = {n: synth.f32_from_bits(synth.bf16_bits(a)) for n, a in _tok(rng, 4, H).items()}
    R = 32
    res = []
    for st, bf in ((state_dtype, True), (0, False)):
        pool = d["pool"][:2].copy()
        kc = np.zeros((2, H, R, 128), np.float32)
        uc = np.zeros_like(kc)
        gc = np.zeros_like(kc)
        # three history rows written by an earlier call, then a folding call
        h0 = {n: a[:, :3].copy() for n, a in toks.items()}
        orc.verify(h0["q"], h0["k"], h0["v"], h0["graw"], h0["beta_logit"], d["a_log"],
                   d["dt_bias"], -5.0, 1.0, pool, np.array([1], np.int32), kc, uc, gc,
                   np.zeros(1, np.int32), np.array([30], np.int32), 10, 16,
                   bf16_storage=True, real=F32, state_dtype=st)
        h1 = {n: a[:, 3:].copy() for n, a in toks.items()}
        out = orc.verify(h1["q"], h1["k"], h1["v"], h1["graw"], h1["beta_logit"], d["a_log"],
                         d["dt_bias"], -5.0, 1.0, pool, np.array([1], np.int32), kc, uc, gc,
                         np.array([3], np.int32), np.array([30], np.int32), 4, 16,
                         bf16_storage=bf, real=F32, state_dtype=st)
        res.append((out, pool))
    np.testing.assert_array_equal(res[0][1][1], cast(res[1][1][1]))  # the folded checkpoint

    p = _prefill_inputs(rng, (21, 0, 40), H=2, real=F32)
    for n in ("q", "k", "v", "graw", "beta_logit"):
        p[n] = synth.f32_from_bits(synth.bf16_bits(p[n]))
    p["pool"] = cast(p["pool"])
    ck_a = np.zeros((3, 2, 128, 128), np.float32)
    ck_b = np.zeros_like(ck_a)
    starts = np.array([0, 1, 1], np.int64)
    qa, qb = p["pool"].copy(), p["pool"].copy()
    orc.prefill(*_pf_args(p), qa, p["idx"], real=F32, state_dtype=state_dtype, checkpoints=ck_a,
                checkpoint_starts=starts, checkpoint_interval=16)
    orc.prefill(*_pf_args(p), qb, p["idx"], bf16_storage=False, real=F32, checkpoints=ck_b,
                checkpoint_starts=starts, checkpoint_interval=16)
    np.testing.assert_array_equal(qa[p["idx"]], cast(qb[p["idx"]]))
    np.testing.assert_array_equal(ck_a, cast(ck_b))


# ---------------------------------------------------------------------------
# Prefill hand-off to speculative decoding (reading): a document's last
# min(ring_tail, tokens after its last 16-token boundary) tokens become ring
# history entries ([verify] "Caching": k_hat, u and the cumulative log-decay G)
# and the pool receives the state before them.

def _ring_nan(N, H, R=32):
    return tuple(np.full((N, H, R, 128), np.nan) for _ in range(3))


@pytest.mark.parametrize("ring_tail,expect", [(16, [0, 5, 16, 1, 8, 4]),
                                              (7, [0, 5, 7, 1, 7, 4]),
                                              (3, [0, 3, 3, 1, 3, 3])])
def test_handoff_ring_replays_to_the_full_prefill_state(orc, ring_tail, expect):
    """The checkpoint plus the handed-off ring rows replay to the final state
    of the same prefill without hand-off; outputs are bitwise unchanged; each
    (slot, head) ring holds exactly the expected number of rows, at
    cache_base onwards (wrapping), and nothing else is written."""
    rng = _rng(240 + ring_tail)
    lens = (0, 5, 16, 17, 40, 100)
    H = 2
    d = _prefill_inputs(rng, lens, H=H)
    N = d["pool"].shape[0]
    base = np.array([3, 30, 25, 0, 31, 17], np.int32)
    p0 = d["pool"].copy()
    o0 = orc.prefill(*_pf_args(d), p0, d["idx"], bf16_storage=False, real=F64)
    p1 = d["pool"].copy()
    ring = _ring_nan(N, H)
    o1 = orc.prefill(*_pf_args(d), p1, d["idx"], bf16_storage=False, real=F64, ring=ring,
                     cache_base=base, ring_tail=ring_tail)
    np.testing.assert_array_equal(o1, o0)
    kc, uc, gc = ring
    for doc, n in enumerate(lens):
        s = d["idx"][doc]
        r = expect[doc]
        assert orc.handoff_tail(n, ring_tail) == r
        for h in range(H):
            rows = [(int(base[doc]) + j) % 32 for j in range(r)]
            filled = ~np.isnan(kc[s, h, :, 0])
            assert sorted(np.nonzero(filled)[0].tolist()) == sorted(rows)
            assert np.array_equal(filled, ~np.isnan(uc[s, h, :, 0]))
            assert np.array_equal(filled, ~np.isnan(gc[s, h, :, 0]))
            S = orc.replay(p1[s, h], np.nan_to_num(kc[s, h]), np.nan_to_num(uc[s, h]),
                           np.nan_to_num(gc[s, h]), int(base[doc]), r, real=F64)
            np.testing.assert_allclose(S, p0[s, h], rtol=1e-10, atol=1e-12)
            if r:  # G is a cumulative log-decay: non-increasing over the entries
                G = gc[s, h, rows]
                assert np.all(np.diff(G, axis=0) <= 0) and np.all(G <= 0)
    untouched = np.setdiff1d(np.arange(N), d["idx"])
    assert np.all(np.isnan(kc[untouched]))
    np.testing.assert_array_equal(p1[untouched], d["pool"][untouched])


@pytest.mark.parametrize("T,fm,ring_tail", [(8, 9, 8), (4, 13, 8)])
def test_handoff_then_verify_equals_the_longer_prefill(orc, T, fm, ring_tail):
    """Prefill with hand-off, then a verify call on T draft tokens from the
    handed-off ring (hist = the tail, W16), gives the outputs the prefill of
    the documents with the draft tokens appended gives at those positions;
    a folding call commits the no-hand-off final state, and a non-folding
    call leaves a ring that replays to the longer prefill's final state."""
    rng = _rng(250 + T)
    lens = (40, 37, 3, 16, 0, 32)
    H = 2
    n_docs = len(lens)
    d = _prefill_inputs(rng, lens, H=H)
    dr = _prefill_inputs(rng, (T,) * n_docs, H=H)  # draft tokens, doc by doc
    base = np.array([5, 31, 0, 12, 7, 20], np.int32)
    hist = np.array([orc.handoff_tail(n, ring_tail) for n in lens], np.int32)
    pool = d["pool"].copy()
    ring = tuple(np.zeros((pool.shape[0], H, 32, 128)) for _ in range(3))
    orc.prefill(*_pf_args(d), pool, d["idx"], bf16_storage=False, real=F64, ring=ring,
                cache_base=base, ring_tail=ring_tail)
    drafts = {n: np.ascontiguousarray(dr[n].reshape((n_docs, T) + dr[n].shape[1:]))
              for n in ("q", "k", "v", "graw", "beta_logit")}
    out_v = orc.verify(drafts["q"], drafts["k"], drafts["v"], drafts["graw"],
                       drafts["beta_logit"], d["a_log"], d["dt_bias"], -5.0, 1.0, pool,
                       d["idx"], *ring, hist, base, fm, 16, bf16_storage=False, real=F64)
    # the longer prefill: each document followed by its draft tokens
    cu = np.zeros(n_docs + 1, np.int32)
    cu[1:] = np.cumsum(np.array(lens) + T)
    cat = {}
    for n in ("q", "k", "v", "graw", "beta_logit"):
        parts = []
        for doc in range(n_docs):
            parts.append(d[n][d["cu"][doc]:d["cu"][doc + 1]])
            parts.append(drafts[n][doc])
        cat[n] = np.ascontiguousarray(np.concatenate(parts))
    long_pool = d["pool"].copy()
    o_long = orc.prefill(cu, cat["q"], cat["k"], cat["v"], cat["graw"], cat["beta_logit"],
                         d["a_log"], d["dt_bias"], -5.0, 1.0, long_pool, d["idx"],
                         bf16_storage=False, real=F64)
    short_pool = d["pool"].copy()
    orc.prefill(*_pf_args(d), short_pool, d["idx"], bf16_storage=False, real=F64)
    for doc in range(n_docs):
        s = d["idx"][doc]
        np.testing.assert_allclose(out_v[doc], o_long[cu[doc] + lens[doc]:cu[doc + 1]],
                                   rtol=1e-9, atol=1e-11)
        fold = hist[doc] + T >= fm
        for h in range(H):
            if fold:
                np.testing.assert_allclose(pool[s, h], short_pool[s, h], rtol=1e-10, atol=1e-12)
            else:
                S = orc.replay(pool[s, h], ring[0][s, h], ring[1][s, h], ring[2][s, h],
                               int(base[doc]), int(hist[doc]) + T, real=F64)
                np.testing.assert_allclose(S, long_pool[s, h], rtol=1e-9, atol=1e-11)
    # both branches are exercised: every document folds at (8, 9) but the
    # empty one, none at (4, 13)
    assert np.sum(hist + T >= fm) == (n_docs - 1 if fm == 9 else 0)


def test_handoff_checkpoints_stop_before_the_tail_and_bad_base_is_inactive(orc):
    """Checkpoints cover only the tokens before the tail (a checkpoint at the
    document's end is not written when tokens were handed off); a document
    whose cache_base lies outside [0, R) writes zero outputs and nothing
    else."""
    rng = _rng(260)
    lens = (64, 20, 33)
    H = 2
    d = _prefill_inputs(rng, lens, H=H)
    N = d["pool"].shape[0]
    starts = np.array([0, 4, 5], np.int64)
    ck0 = np.full((8, H, 128, 128), -3.0)
    ck1 = ck0.copy()
    p0, p1 = d["pool"].copy(), d["pool"].copy()
    base = np.array([0, 9, -1], np.int32)  # doc 2: bad base
    o0 = orc.prefill(*_pf_args(d), p0, d["idx"], bf16_storage=False, real=F64, checkpoints=ck0,
                     checkpoint_starts=starts, checkpoint_interval=16)
    ring = _ring_nan(N, H)
    o1 = orc.prefill(*_pf_args(d), p1, d["idx"], bf16_storage=False, real=F64, checkpoints=ck1,
                     checkpoint_starts=starts, checkpoint_interval=16, ring=ring,
                     cache_base=base, ring_tail=16)
    # doc 0 (64 tokens, tail 16): rows 0..2 as before, row 3 (token 64) not written
    np.testing.assert_array_equal(ck1[0:3], ck0[0:3])
    assert np.all(ck0[3] != -3.0) and np.all(ck1[3] == -3.0)
    # doc 1 (20 tokens, tail 4): row 4 (token 16) as before
    np.testing.assert_array_equal(ck1[4], ck0[4])
    # doc 2: inactive
    t0, t1 = d["cu"][2], d["cu"][3]
    assert np.all(o1[t0:t1] == 0) and np.any(o0[t0:t1] != 0)
    assert np.all(ck1[5:] == -3.0)
    s2 = d["idx"][2]
    np.testing.assert_array_equal(p1[s2], d["pool"][s2])
    assert np.all(np.isnan(ring[0][s2]))
    np.testing.assert_array_equal(o1[:t0], o0[:t0])
