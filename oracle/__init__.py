"""CPU oracle for the KDA gated delta-rule step (decode, verify+fold, prefill).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and by
the benchmark's CPU-baseline leg, never by the GPU library or its binding.

The arithmetic lives in ``kda_oracle.cpp`` (plain C++17 loops, built with g++,
no HIP). This module builds it, loads it with ctypes and passes dense numpy
arrays. Every array argument is a C-contiguous numpy array of the working
precision (float32 = parity target, float64 = invariants and drift); bf16
tensors are passed as their exact float values. Functions update the arrays
they document as outputs in place.

Readings that are "parity unpinned" (the oracle encodes them; no page fixes
them): the gate formula, the L2-norm epsilon, the ring addressing through
cache_base, the state orientation [V][K] and A_log being per head.

gate_mode (every entry): 0 takes raw gate and beta logits; bit GATE_PRECOMPUTED
takes the log-decay g itself (clamped into [lower_bound, 0]; a_log and dt_bias
may be None); bit BETA_PRESIGMOID takes beta itself; bit GATE_PER_HEAD takes one
gate value per token and head (graw [..., H], dt_bias [H]), applied to every key
channel.

state_dtype (decode, verify, prefill): 0 stores the state (pool write-back, fold
checkpoint, prefill final and intermediate states) in bf16, 1 in fp16 (round to
nearest even, written from the binary16 definition), 2 in fp8 e4m3 (the OCP
e4m3fn format, round to nearest even, saturating at +-448); outputs and ring
rows stay bf16. Pool inputs are passed as their exact values either way.

Prefill hand-off (ring_tail > 0, a reading): a document's last tokens, at most
those after its last 16-token boundary and at most ring_tail, go to the verify
ring as history entries (k_hat, u, cumulative G from the stored state), and the
pool slot receives the state before them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source (host
# code only), loaded instead of _LIB when KDA_ORACLE_LIB names it; the process
# must then preload gcc's libasan (see tests/test_sanitizers.py).
SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
_lib = None

_I32P = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile kda_oracle.cpp into liboracle.so with g++ (OpenMP, IEEE math);
    sanitize=True builds liboracle_san.so with -fsanitize=address,undefined
    (aborting on the first report) instead."""
    out = SAN_LIB if sanitize else _LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp"
        extra = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer", "-g"] if sanitize else []
        cmd = ["g++", "-std=c++17", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", *extra, _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = os.environ.get("KDA_ORACLE_LIB")
        if path:  # an alternative build of the same source (the sanitizer leg)
            _lib = ctypes.CDLL(path)
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _suffix(real) -> str:
    real = np.dtype(real)
    if real == np.float32:
        return "f32"
    if real == np.float64:
        return "f64"
    raise TypeError(f"oracle precision must be float32 or float64, got {real}")


def _rp(a, real):
    ctype = ctypes.c_float if np.dtype(real) == np.float32 else ctypes.c_double
    if a is None:  # an input the chosen gate mode does not read
        return ctypes.POINTER(ctype)()
    assert a.dtype == np.dtype(real) and a.flags["C_CONTIGUOUS"], (a.dtype, real)
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _ip(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_I32P)


def _rs(x, real):
    return (ctypes.c_float if np.dtype(real) == np.float32 else ctypes.c_double)(float(x))


def threads() -> int:
    return int(lib().orc_max_threads())


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def f16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 bits, round-to-nearest-even (uint16 array of x's shape)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f16_round(ctypes.c_int64(x.size), x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                        out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)))
    return out


def f8_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> fp8 e4m3 bits, round-to-nearest-even, saturating at +-448 (uint8)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_f8_round(ctypes.c_int64(x.size), x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    return out


def f8_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """fp8 e4m3 bits -> fp32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint8)
    out = np.empty(b.shape, dtype=np.float32)
    lib().orc_f8_to_float(ctypes.c_int64(b.size), b.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                          out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return out


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """fp16 bits -> fp32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    lib().orc_f16_to_float(ctypes.c_int64(b.size), b.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                           out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return out


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round-to-nearest-even (uint16 array of x's shape)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_round(ctypes.c_int64(x.size), x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                         out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)))
    return out


GATE_PRECOMPUTED = 1  # gate_mode bit: graw holds the log-decay g itself
BETA_PRESIGMOID = 2   # gate_mode bit: beta_logit holds beta itself
GATE_PER_HEAD = 4     # gate_mode bit: one gate value (and dt_bias) per head


def prologue(q, k, graw, beta_logit, a_log_h, dt_bias_h, lower_bound, real=np.float64,
             gate_mode=0):
    """One head's per-token prologue -> (q_hat, k_hat, g, beta)."""
    K = q.shape[0]
    qh, kh, g = (np.zeros(K, real) for _ in range(3))
    beta = np.zeros(1, real)
    f = getattr(lib(), "orc_prologue_" + _suffix(real))
    f(ctypes.c_int(K), _rp(q, real), _rp(k, real), _rp(graw, real), _rs(beta_logit, real),
      _rs(a_log_h or 0.0, real), _rp(dt_bias_h, real), _rs(lower_bound, real),
      ctypes.c_int(gate_mode), _rp(qh, real), _rp(kh, real), _rp(g, real), _rp(beta, real))
    return qh, kh, g, float(beta[0])


def step(S, qh, kh, v, g, beta, scale, real=np.float64):
    """One step on S ([V][K], updated in place) -> (o, u)."""
    V, K = S.shape
    o = np.zeros(V, real)
    u = np.zeros(V, real)
    f = getattr(lib(), "orc_step_" + _suffix(real))
    f(ctypes.c_int(K), ctypes.c_int(V), _rp(S, real), _rp(qh, real), _rp(kh, real), _rp(v, real),
      _rp(g, real), _rs(beta, real), _rs(scale, real), _rp(o, real), _rp(u, real))
    return o, u


def replay(ckpt, kc, uc, gc, base, hist, real=np.float64):
    """Ring replay for one (slot, head): ckpt [V][K], kc/gc [R][K], uc [R][V] -> S_cur."""
    V, K = ckpt.shape
    R = kc.shape[0]
    S = np.zeros((V, K), real)
    f = getattr(lib(), "orc_replay_" + _suffix(real))
    f(ctypes.c_int(K), ctypes.c_int(V), _rp(ckpt, real), _rp(kc, real), _rp(uc, real),
      _rp(gc, real), ctypes.c_int(R), ctypes.c_int(base), ctypes.c_int(hist), _rp(S, real))
    return S


def decode(q, k, v, graw, beta_logit, a_log, dt_bias, lower_bound, scale, pool, idx,
           bf16_storage=True, real=np.float32, gate_mode=0, state_dtype=0):
    """T=1 decode. q/k/graw [B,H,K], v [B,H,V], beta_logit [B,H], pool [N,H,V,K]
    (updated in place), idx int32 [B]. Returns out [B,H,V]."""
    B, H, K = q.shape
    V = v.shape[2]
    N = pool.shape[0]
    out = np.zeros((B, H, V), real)
    f = getattr(lib(), "orc_decode_" + _suffix(real))
    f(B, H, K, V, _rp(q, real), _rp(k, real), _rp(v, real), _rp(graw, real),
      _rp(beta_logit, real), _rp(a_log, real), _rp(dt_bias, real), _rs(lower_bound, real),
      _rs(scale, real), _rp(pool, real), ctypes.c_int64(N), _ip(idx), _rp(out, real),
      ctypes.c_int(1 if bf16_storage else 0), ctypes.c_int(gate_mode),
      ctypes.c_int(int(state_dtype)))
    return out


def verify(q, k, v, graw, beta_logit, a_log, dt_bias, lower_bound, scale, pool, idx,
           k_cache, u_cache, g_cache, hist_len, cache_base, flush_min, w_ring,
           bf16_storage=True, real=np.float32, gate_mode=0, state_dtype=0):
    """Verify+fold. q/k/graw [B,T,H,K], v [B,T,H,V], beta_logit [B,T,H]; pool [N,H,V,K],
    k_cache/g_cache [N,H,R,K], u_cache [N,H,R,V] all updated in place. Returns out [B,T,H,V]."""
    B, T, H, K = q.shape
    V = v.shape[3]
    N = pool.shape[0]
    R = k_cache.shape[2]
    out = np.zeros((B, T, H, V), real)
    f = getattr(lib(), "orc_verify_" + _suffix(real))
    f(B, T, H, K, V, _rp(q, real), _rp(k, real), _rp(v, real), _rp(graw, real),
      _rp(beta_logit, real), _rp(a_log, real), _rp(dt_bias, real), _rs(lower_bound, real),
      _rs(scale, real), _rp(pool, real), ctypes.c_int64(N), _ip(idx), _rp(k_cache, real),
      _rp(u_cache, real), _rp(g_cache, real), ctypes.c_int(R), _ip(hist_len), _ip(cache_base),
      ctypes.c_int(flush_min), ctypes.c_int(w_ring), _rp(out, real),
      ctypes.c_int(1 if bf16_storage else 0), ctypes.c_int(gate_mode),
      ctypes.c_int(int(state_dtype)))
    return out


def _prefill_args(cu, q, k, v, graw, beta_logit, a_log, dt_bias, lower_bound, scale, pool, idx,
                  use_initial_state, out, real):
    n_docs = cu.shape[0] - 1
    Ttot, H, K = q.shape
    V = v.shape[2]
    N = pool.shape[0]
    return (n_docs, H, K, V, _ip(cu), _rp(q, real), _rp(k, real), _rp(v, real), _rp(graw, real),
            _rp(beta_logit, real), _rp(a_log, real), _rp(dt_bias, real), _rs(lower_bound, real),
            _rs(scale, real), _rp(pool, real), ctypes.c_int64(N), _ip(idx),
            ctypes.c_int(1 if use_initial_state else 0), _rp(out, real))


def prefill(cu, q, k, v, graw, beta_logit, a_log, dt_bias, lower_bound, scale, pool, idx,
            use_initial_state=True, bf16_storage=True, real=np.float32, gate_mode=0,
            checkpoints=None, checkpoint_starts=None, checkpoint_interval=16, state_dtype=0,
            ring=None, cache_base=None, ring_tail=0):
    """Token-by-token varlen prefill. q/k/graw [Ttot,H,K], v [Ttot,H,V], beta_logit [Ttot,H],
    cu int32 [n_docs+1], idx int32 [n_docs], pool [N,H,V,K] updated in place. -> out [Ttot,H,V].
    checkpoints [rows,H,V,K] (updated in place) with checkpoint_starts int64 [n_docs]: the
    state after every checkpoint_interval tokens of each active document.
    ring = (k_cache [N,H,R,K], u_cache [N,H,R,V], g_cache [N,H,R,K]), updated in place, with
    cache_base int32 [n_docs] and ring_tail > 0: each active document hands its last
    min(ring_tail, tokens after its last 16-token boundary) tokens to the ring as history
    entries, and the pool receives the state before them (see handoff_tail)."""
    out = np.zeros((q.shape[0], q.shape[1], v.shape[2]), real)
    f = getattr(lib(), "orc_prefill_tbt_" + _suffix(real))
    if checkpoints is None:
        ck, rows, starts = _rp(None, real), 0, ctypes.POINTER(ctypes.c_int64)()
    else:
        assert checkpoint_starts.dtype == np.int64 and checkpoint_starts.flags["C_CONTIGUOUS"]
        ck, rows = _rp(checkpoints, real), checkpoints.shape[0]
        starts = checkpoint_starts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    f(*_prefill_args(cu, q, k, v, graw, beta_logit, a_log, dt_bias, lower_bound, scale, pool,
                     idx, use_initial_state, out, real), ctypes.c_int(1 if bf16_storage else 0),
      ctypes.c_int(gate_mode), ck, ctypes.c_int64(rows), starts,
      ctypes.c_int(int(checkpoint_interval)), ctypes.c_int(int(state_dtype)),
      *_ring_args(ring, cache_base, ring_tail, real))
    return out


def _ring_args(ring, cache_base, ring_tail, real):
    if not ring_tail:
        return (_rp(None, real), _rp(None, real), _rp(None, real), ctypes.c_int(0), _I32P(),
                ctypes.c_int(0))
    kc, uc, gc = ring
    return (_rp(kc, real), _rp(uc, real), _rp(gc, real), ctypes.c_int(kc.shape[2]),
            _ip(cache_base), ctypes.c_int(int(ring_tail)))


def handoff_tail(length, ring_tail):
    """Tokens a document of `length` tokens hands to the ring: at most those after
    its last 16-token boundary, and at most ring_tail."""
    if length <= 0 or ring_tail <= 0:
        return 0
    return min(ring_tail, length - 16 * ((length - 1) // 16))


def prefill_chunked(cu, q, k, v, graw, beta_logit, a_log, dt_bias, lower_bound, scale, pool, idx,
                    chunk, use_initial_state=True, real=np.float64, gate_mode=0):
    """Chunkwise (WY/UT) model of the same prefill, no storage rounding. -> out [Ttot,H,V]."""
    out = np.zeros((q.shape[0], q.shape[1], v.shape[2]), real)
    f = getattr(lib(), "orc_prefill_chunked_" + _suffix(real))
    f(*_prefill_args(cu, q, k, v, graw, beta_logit, a_log, dt_bias, lower_bound, scale, pool,
                     idx, use_initial_state, out, real), ctypes.c_int(int(chunk)),
      ctypes.c_int(gate_mode))
    return out


if __name__ == "__main__":  # pragma: no cover
    print(build(force=True), file=sys.stderr)
