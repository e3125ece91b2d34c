"""kda_prefill_varlen_noalloc, the prefill entry point that allocates nothing,
against kda_prefill_varlen on the same inputs: two calls in a row on the
two-stage path (fewer than 256 chains, so the library's scratch carries the
per-chunk records), the second with fewer documents and tokens so that it runs
over what the first left there; a call on the fused path (no scratch); and a
call whose workspace would exceed the scratch, refused before any launch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_delta_rule_step_amd as kda
from gated_delta_rule_step_amd import synth
from tests.helpers import HD, bits, dev, dev_bf16, pool_dev

pytestmark = pytest.mark.gpu


def _call(fn, case, ckpt_interval=None):
    """One prefill call through `fn` on fresh copies of the case's device
    buffers; returns (out, pool, checkpoints) as bit arrays."""
    H, Ttot = case["H"], case["Ttot"]
    W = H * HD
    q, k, v = (dev_bf16(case[n].reshape(Ttot, W)) for n in ("q", "k", "v"))
    out = torch.full((Ttot, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    pool = pool_dev(case, case["pool"])
    ck = starts = None
    if ckpt_interval:
        counts = np.diff(case["cu_seqlens"]) // ckpt_interval
        starts = dev(np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64))
        ck = torch.full((max(int(counts.sum()), 1), H, HD, HD), float("nan"),
                        dtype=torch.bfloat16, device="cuda")
    fn(torch.from_numpy(case["cu_seqlens"].copy()), dev(case["cu_seqlens"]), q, k, v,
       dev_bf16(case["gate"]), dev_bf16(case["beta"]), dev(case["a_log"]),
       dev(case["dt_bias"]), pool, dev(case["idx"]), out,
       use_initial_state=case["use_initial_state"], lower_bound=case["lower_bound"],
       scale=case["scale"], checkpoints=ck, checkpoint_cu_starts=starts,
       checkpoint_interval=ckpt_interval or 16)
    torch.cuda.synchronize()
    return bits(out), bits(pool), None if ck is None else bits(ck)


def _same(a, b, what):
    for x, y, part in zip(a, b, ("output", "pool", "checkpoints")):
        if x is None and y is None:
            continue
        assert np.array_equal(x, y), f"{what}: {part} differs from kda_prefill_varlen"


def test_noalloc_matches_workspace_entry_point():
    # first call: 5 documents x 6 heads = 30 chains (two-stage path), checkpoints
    big = synth.prefill_case((100, 37, 64, 0, 230), H=6, seed=synth.seed_for(9, 6, 1))
    need = kda.kda_prefill_workspace_size(big["n_docs"], big["Ttot"], big["H"])
    assert 0 < need <= kda.NOALLOC_SCRATCH_BYTES
    print(f"noalloc call 1: docs {big['n_docs']} H {big['H']} tokens {big['Ttot']} "
          f"scratch {need} B", flush=True)
    _same(_call(kda.kda_prefill_varlen_noalloc, big, 16),
          _call(kda.kda_prefill_varlen, big, 16), "call 1")
    # second call, smaller: 2 documents x 3 heads
    small = synth.prefill_case((20, 33), H=3, seed=synth.seed_for(9, 3, 2))
    need2 = kda.kda_prefill_workspace_size(small["n_docs"], small["Ttot"], small["H"])
    assert 0 < need2 < need
    print(f"noalloc call 2: docs {small['n_docs']} H {small['H']} tokens {small['Ttot']} "
          f"scratch {need2} B", flush=True)
    _same(_call(kda.kda_prefill_varlen_noalloc, small),
          _call(kda.kda_prefill_varlen, small), "call 2")


def test_noalloc_fused_path():
    # 4 documents x 64 heads = 256 chains: the fused kernel, no scratch
    case = synth.prefill_case((70, 5, 128, 33), H=64, seed=synth.seed_for(9, 64, 3))
    assert kda.kda_prefill_workspace_size(case["n_docs"], case["Ttot"], case["H"]) == 0
    print("noalloc fused call: docs 4 H 64", flush=True)
    _same(_call(kda.kda_prefill_varlen_noalloc, case), _call(kda.kda_prefill_varlen, case),
          "fused call")


def test_noalloc_scratch_limit():
    # one chain of 36,800 tokens needs (1 + 2300) * 29,696 B > 64 MiB of workspace
    T = 36800
    assert kda.kda_prefill_workspace_size(1, T, 1) > kda.NOALLOC_SCRATCH_BYTES
    z = torch.zeros((T, HD), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(z)
    pool = torch.zeros((1, 1, HD, HD), dtype=torch.bfloat16, device="cuda")
    f = torch.zeros(HD, dtype=torch.float32, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.kda_prefill_varlen_noalloc(
            torch.tensor([0, T], dtype=torch.int32), dev(np.array([0, T], np.int32)), z, z, z,
            z, torch.zeros((T, 1), dtype=torch.bfloat16, device="cuda"),
            torch.zeros(1, dtype=torch.float32, device="cuda"), f, pool,
            dev(np.array([0], np.int32)), out)
    assert e.value.status == 8
    assert torch.count_nonzero(out).item() == 0
