"""C-ABI library checks that run without a GPU: the library loads, exports
every entry point include/kda.h declares, and rejects invalid host arguments
before launching anything (these calls return before any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULLP, SHAPE, STRIDE, UNSUP, SEQ, WS, LAUNCH, SCRATCH = range(9)


@pytest.fixture(scope="module")
def lib():
    import gated_delta_rule_step_amd as kda
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_step_amd import build
        build.build()
    return kda.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "kda_status_string", "kda_decode", "kda_verify_ucache_flush",
        "kda_prefill_workspace_size", "kda_prefill_varlen", "kda_prefill_varlen_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    import gated_delta_rule_step_amd as kda
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    import gated_delta_rule_step_amd as kda
    seen = set()
    for s in range(9):
        txt = kda.kda_status_string(s)
        assert txt and txt != "unknown status"
        seen.add(txt)
    assert len(seen) == 9
    assert kda.kda_status_string(99) == "unknown status"


def _decode(lib, **kw):
    a = dict(B=2, H=12, K=128, V=128, q=1 << 20, qs=4608, k=1 << 20, ks=4608, v=1 << 20,
             vs=4608, g=1 << 20, gs=1536, b=1 << 20, bs=12, alog=1 << 20, dtb=1 << 20,
             lb=-5.0, scale=1.0, gm=0, sd=0, pool=1 << 20, N=4, ss=12 * 128 * 128, idx=1 << 20,
             out=1 << 20, os=1536)
    a.update(kw)
    P = ctypes.c_void_p
    return lib.kda_decode(a["B"], a["H"], a["K"], a["V"], P(a["q"]), a["qs"], P(a["k"]),
                          a["ks"], P(a["v"]), a["vs"], P(a["g"]), a["gs"], P(a["b"]), a["bs"],
                          P(a["alog"]), P(a["dtb"]), a["lb"], a["scale"], a["gm"], a["sd"],
                          P(a["pool"]),
                          a["N"], a["ss"], P(a["idx"]), P(a["out"]), a["os"], P(0))


def test_decode_host_validation(lib):
    assert _decode(lib, K=64) == UNSUP
    assert _decode(lib, V=256) == UNSUP
    assert _decode(lib, B=-1) == SHAPE
    assert _decode(lib, H=0) == SHAPE
    assert _decode(lib, N=-3) == SHAPE
    assert _decode(lib, q=0) == NULLP
    assert _decode(lib, out=0) == NULLP
    assert _decode(lib, idx=0) == NULLP
    assert _decode(lib, pool=0) == NULLP            # pool needed when N > 0
    assert _decode(lib, os=100) == STRIDE           # output rows overlap
    assert _decode(lib, ss=1000) == STRIDE          # slots overlap
    assert _decode(lib, qs=-8) == STRIDE
    # B = 0 is a no-op that needs no pointer at all and launches nothing
    assert _decode(lib, B=0, q=0, k=0, v=0, g=0, b=0, alog=0, dtb=0, pool=0, idx=0,
                   out=0) == OK


def test_gate_mode_validation(lib):
    """gate_mode: raw gate logits need A_log and dt_bias; the pre-computed
    gate reads neither (NULL accepted) and needs lower_bound <= 0; unknown
    bits are rejected. The same rules hold on all three entry points."""
    assert _decode(lib, alog=0) == NULLP
    assert _decode(lib, dtb=0) == NULLP
    assert _decode(lib, gm=2, alog=0) == NULLP        # pre-sigmoided beta alone: raw gate
    assert _decode(lib, gm=8) == UNSUP
    assert _decode(lib, gm=-1) == UNSUP
    assert _decode(lib, gm=1, lb=0.5) == UNSUP
    assert _decode(lib, gm=1, lb=float("nan")) == UNSUP
    # B = 0: nothing is launched, so the NULL checks pass (unknown bits do not)
    assert _decode(lib, B=0, gm=1, alog=0, dtb=0, lb=float("-inf")) == OK
    assert _decode(lib, B=0, gm=8) == UNSUP
    assert _decode(lib, gm=4 | 1, lb=0.5) == UNSUP   # per-head pre-computed: same rule
    assert _verify(lib, gm=1, lb=0.25) == UNSUP
    assert _verify(lib, gm=16) == UNSUP
    assert _verify(lib, B=0, gm=3) == OK


def test_state_dtype_validation(lib):
    """state_dtype: bf16 (0), fp16 (1) or fp8 (2), and the last two only on
    the vectorised layout (16-byte aligned bases, strides in multiples of 8)."""
    assert _decode(lib, sd=3) == UNSUP
    assert _decode(lib, sd=2, q=(1 << 20) + 2) == UNSUP
    assert _decode(lib, sd=2, ss=12 * 128 * 128 + 4) == UNSUP
    assert _decode(lib, sd=-1) == UNSUP
    assert _decode(lib, sd=1, q=(1 << 20) + 2) == UNSUP   # unaligned q: no vectorised path
    assert _decode(lib, sd=1, qs=4610) == UNSUP
    assert _decode(lib, B=0, sd=1) == OK
    assert _verify(lib, sd=5) == UNSUP
    assert _verify(lib, sd=1, rs=8 * 4608 + 2) == UNSUP


def _verify(lib, **kw):
    a = dict(B=2, T=8, H=12, K=128, V=128, ptr=1 << 20, rs=8 * 4608, ts=4608, brs=96, bts=12,
             grs=8 * 1536, gts=1536, lb=-5.0, scale=1.0, N=4, ss=12 * 128 * 128, R=32,
             fm=9, w=16, restart=1, ors=8 * 1536, ots=1536, kc=1 << 20, hist=1 << 20, gm=0,
             sd=0)
    a.update(kw)
    P = ctypes.c_void_p
    p = P(a["ptr"])
    return lib.kda_verify_ucache_flush(
        a["B"], a["T"], a["H"], a["K"], a["V"], p, a["rs"], a["ts"], p, a["rs"], a["ts"],
        p, a["rs"], a["ts"], p, a["grs"], a["gts"], p, a["brs"], a["bts"], p, p, a["lb"],
        a["scale"], a["gm"], a["sd"], p, a["N"], a["ss"], p, P(a["kc"]), p, p, a["R"],
        P(a["hist"]), p,
        a["fm"],
        a["w"], a["restart"], p, a["ors"], a["ots"], P(0))


def test_verify_host_validation(lib):
    assert _verify(lib, T=0) == UNSUP
    assert _verify(lib, T=9) == UNSUP
    assert _verify(lib, w=24) == UNSUP
    assert _verify(lib, R=0) == SHAPE
    assert _verify(lib, R=15) == UNSUP                # fewer ring rows than the window
    assert _verify(lib, restart=0) == UNSUP
    assert _verify(lib, fm=0) == UNSUP
    assert _verify(lib, fm=10) == UNSUP               # 10 - 1 + 8 > 16: ring capacity
    assert _verify(lib, T=4, fm=14) == UNSUP
    assert _verify(lib, w=32, fm=16) == UNSUP         # W32 needs flush_min > 16
    assert _verify(lib, kc=0) == NULLP
    assert _verify(lib, hist=0) == NULLP
    assert _verify(lib, ots=100) == STRIDE            # output tokens overlap
    assert _verify(lib, ors=1536, ots=1536) == STRIDE  # rows and tokens collide
    assert _verify(lib, B=0) == OK


def test_prefill_workspace_and_validation(lib):
    P = ctypes.c_void_p
    # calls with at least 256 (document, head) chains run the fused kernel and
    # need no workspace; with fewer, the two-stage form keeps one 29,696-byte
    # chunk record per (chunk slot, head), and chunk slots number fewer than
    # n_docs + floor(total_tokens / 16)
    rec = 29696
    assert lib.kda_prefill_workspace_size(4, 13888, 64, 128, 128) == 0
    assert lib.kda_prefill_workspace_size(14, 16384, 64, 128, 128) == 0
    assert lib.kda_prefill_workspace_size(3, 13888, 64, 128, 128) == (3 + 868) * 64 * rec
    assert lib.kda_prefill_workspace_size(14, 16384, 12, 128, 128) == (14 + 1024) * 12 * rec
    assert lib.kda_prefill_workspace_size(3, 0, 12, 128, 128) == 0
    assert lib.kda_prefill_workspace_size(4, 13888, 64, 64, 128) == 0

    def call(cu, total, **kw):
        p = P(1 << 20)
        a = dict(n=len(cu) - 1, H=2, K=128, ws=1 << 40, ots=256, lb=-5.0, ws_ptr=p, gm=0, sd=0,
                 ck=P(0), ck_rows=0, ck_starts=P(0), ck_int=16, kc=P(0), uc=P(0), gc=P(0),
                 R=0, base=P(0), tail=0)
        a.update(kw)
        arr = (ctypes.c_int32 * len(cu))(*cu)
        return lib.kda_prefill_varlen(a["n"], total, a["H"], a["K"], 128, arr, p, p, 256, p,
                                      256, p, 256, p, 256, p, 2, p, p, a["lb"], 1.0, a["gm"],
                                      a["sd"], p, 4,
                                      2 * 128 * 128, p, 1, p, a["ots"], a["ck"], a["ck_rows"],
                                      a["ck_starts"], a["ck_int"], a["kc"], a["uc"], a["gc"],
                                      a["R"], a["base"], a["tail"], a["ws_ptr"], a["ws"], P(0))

    assert call([1, 5], 5) == SEQ       # must start at 0
    assert call([0, 5, 3], 3) == SEQ    # must not decrease
    assert call([0, 5, 7], 9) == SEQ    # must end at total_tokens
    assert call([0, 5], 5, K=64) == UNSUP
    assert call([0, 5], 5, ots=8) == STRIDE
    assert call([0, 1], 1, ots=0) == STRIDE   # one token: out rows still H*128 apart
    # 16-token chunks need |lower_bound| <= 5.5 (each decay factor within e^44)
    assert call([0, 5], 5, lb=-5.6) == UNSUP
    assert call([0, 5], 5, lb=float("nan")) == UNSUP
    assert call([0], 0) == OK           # no documents: nothing to do
    assert call([0, 5], 5, gm=8) == UNSUP
    assert call([0, 5], 5, sd=3) == UNSUP
    # intermediate checkpoints: on chunk boundaries, a row count, a starts array
    q = P(1 << 20)
    assert call([0, 5], 5, ck=q, ck_rows=3, ck_starts=q, ck_int=24) == UNSUP
    assert call([0, 5], 5, ck=q, ck_rows=3, ck_starts=q, ck_int=0) == UNSUP
    assert call([0, 5], 5, ck=q, ck_rows=-1, ck_starts=q) == SHAPE
    assert call([0, 5], 5, ck=q, ck_rows=3) == NULLP
    assert call([0], 0, ck=q, ck_rows=3, ck_starts=q, ck_int=32) == OK
    assert call([0, 5], 5, gm=1, lb=0.5) == UNSUP  # also outside the prefill's |lb| <= 5.5
    # hand-off to the verify ring: at most one chunk's tokens, distinct rows,
    # every ring pointer
    assert call([0, 5], 5, tail=17, kc=q, uc=q, gc=q, R=32, base=q) == UNSUP
    assert call([0, 5], 5, tail=-1) == UNSUP
    assert call([0, 5], 5, tail=4, kc=q, uc=q, gc=q, R=3, base=q) == SHAPE
    for miss in ("kc", "uc", "gc", "base"):
        kw = dict(tail=4, kc=q, uc=q, gc=q, R=32, base=q)
        kw[miss] = P(0)
        assert call([0, 5], 5, **kw) == NULLP, miss
    assert call([0], 0, tail=4, R=32) == OK  # no documents: nothing read
    assert call([0, 5], 5, ws=2 * rec - 1) == WS   # one slot, two heads
    assert call([0, 5], 5, ws=2 * rec, ws_ptr=P(0)) == NULLP
    assert call([0, 5], 5, ws=2 * rec, ws_ptr=P((1 << 20) + 128)) == UNSUP  # 256-byte aligned


def test_prefill_noalloc_validation(lib):
    """The allocation-free prefill refuses, before any device call, a call whose
    workspace would exceed its fixed scratch (and bad shapes)."""
    import gated_delta_rule_step_amd as kda
    P = ctypes.c_void_p
    assert kda.NOALLOC_SCRATCH_BYTES == 64 << 20

    def call(n, total, H=1, K=128):
        cu = (ctypes.c_int32 * 2)(0, total)
        p = P(1 << 20)
        return lib.kda_prefill_varlen_noalloc(n, total, H, K, 128, cu, p, p, 128, p, 128, p, 128,
                                              p, 128, p, 1, p, p, -5.0, 1.0, 0, 0, p, 1,
                                              128 * 128, p, 1, p, 128, P(0), 0, P(0), 16, P(0),
                                              P(0), P(0), 0, P(0), 0, P(0))

    # one chain of 36,800 tokens: (1 + 2300) records of 29,696 bytes > 64 MiB
    assert kda.kda_prefill_workspace_size(1, 36800, 1) > kda.NOALLOC_SCRATCH_BYTES
    assert call(1, 36800) == SCRATCH
    assert call(-1, 0) == SHAPE
    assert call(1, 16, H=0) == SHAPE
    assert call(1, 16, K=64) == UNSUP
