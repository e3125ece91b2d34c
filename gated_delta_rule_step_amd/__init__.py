"""Python binding of the KDA step library (libkda.so, HIP for gfx950).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks dtype/device/contiguity of the innermost dimension,
and passes raw pointers, element strides and the current HIP stream to the C
ABI declared in include/kda.h. All arithmetic runs in the library's kernels;
there is no fallback. If libkda.so is missing the first call raises.

bf16 tensors are torch.bfloat16; A_log and dt_bias are float32; indices and
ring metadata are int32.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")
HEAD_DIM = 128

_lib = None

_c = ctypes
_P = _c.c_void_p
_I32 = _c.c_int32
_I64 = _c.c_int64
_F = _c.c_float

_SIGS = {
    "kda_status_string": (_c.c_char_p, [_c.c_int]),
    "kda_decode": (_c.c_int, [_I32, _I32, _I32, _I32,
                              _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                              _P, _P, _F, _F, _I32, _I32, _P, _I64, _I64, _P, _P, _I64, _P]),
    "kda_verify_ucache_flush": (_c.c_int, [_I32, _I32, _I32, _I32, _I32,
                                           _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64,
                                           _P, _I64, _I64, _P, _I64, _I64,
                                           _P, _P, _F, _F, _I32, _I32, _P, _I64, _I64, _P,
                                           _P, _P, _P, _I32, _P, _P, _I32, _I32, _I32,
                                           _P, _I64, _I64, _P]),
    "kda_prefill_workspace_size": (_c.c_size_t, [_I32, _I64, _I32, _I32, _I32]),
    "kda_prefill_varlen": (_c.c_int, [_I32, _I64, _I32, _I32, _I32, _P, _P,
                                      _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                                      _P, _P, _F, _F, _I32, _I32, _P, _I64, _I64, _P, _I32,
                                      _P, _I64, _P, _I64, _P, _I32, _P, _P, _P, _I32, _P,
                                      _I32, _P, _c.c_size_t, _P]),
    "kda_prefill_varlen_noalloc": (_c.c_int, [_I32, _I64, _I32, _I32, _I32, _P, _P,
                                              _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                                              _P, _P, _F, _F, _I32, _I32, _P, _I64, _I64, _P,
                                              _I32, _P, _I64, _P, _I64, _P, _I32, _P, _P, _P,
                                              _I32, _P, _I32, _P]),
}

# Scratch held by the library per device for kda_prefill_varlen_noalloc
# (KDA_NOALLOC_SCRATCH_BYTES in include/kda.h).
NOALLOC_SCRATCH_BYTES = 64 << 20
# Prefill calls with at least this many (document, head) chains run the fused
# 64-token chunk kernel (no workspace); fewer run the two-stage form.
FUSED_MIN_CHAINS = 256


# gate_mode bits (include/kda.h): g_raw holds the log-decay g itself (A_log and
# dt_bias may then be None); beta_raw holds beta itself.
GATE_PRECOMPUTED = 1
BETA_PRESIGMOID = 2


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {kda_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libkda.so (built in-tree by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def kda_status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise KdaError(fn, status)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return _P(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return _P(t.data_ptr()) if t is not None else _P(0)


def _bf16(name, t, last_contig=True):
    import torch
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if last_contig and t.stride(-1) != 1:
        raise ValueError(f"{name}: the innermost dimension must be contiguous")


def _f32(name, t, optional=False):
    import torch
    if optional and t is None:
        return
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 GPU tensor")


def _i32(name, t):
    import torch
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor")


def _state_dtype(state_pool) -> int:
    """KDA_STATE_BF16 (0), KDA_STATE_FP16 (1) or KDA_STATE_FP8 (2, torch's
    float8_e4m3fn), from the pool tensor's dtype."""
    import torch
    if state_pool.dtype == torch.float16:
        return 1
    if state_pool.dtype == torch.float8_e4m3fn:
        return 2
    _bf16("state_pool", state_pool)
    return 0


def _pool_geometry(state_pool, H):
    """Pool: bf16, fp16 or fp8 e4m3 tensor whose dim 0 indexes slots; each slot's first
    H*128*128 elements are contiguous. Returns (num_slots, slot_stride)."""
    if not state_pool.is_cuda or state_pool.stride(-1) != 1:
        raise ValueError("state_pool must be a GPU tensor with a contiguous last dimension")
    n = state_pool.shape[0]
    inner = state_pool[0] if n > 0 else None
    if n > 0 and not inner.is_contiguous():
        raise ValueError("state_pool: each slot must be contiguous")
    if n > 0 and inner.numel() < H * HEAD_DIM * HEAD_DIM:
        raise ValueError("state_pool: slot smaller than H*128*128")
    return n, (state_pool.stride(0) if n > 0 else H * HEAD_DIM * HEAD_DIM)


def _ring_rows(k_cache, u_cache, g_cache, N, H) -> int:
    """The three ring tensors must each be [N, H, R, 128] with one R; returns R."""
    shapes = [tuple(t.shape) for t in (k_cache, u_cache, g_cache)]
    R = shapes[0][2] if len(shapes[0]) == 4 else -1
    for name, sh in zip(("k_cache", "u_cache", "g_cache"), shapes):
        if sh != (N, H, R, HEAD_DIM):
            raise ValueError(f"{name} must be [N={N}, H={H}, R, 128] with the same R as "
                             f"k_cache, got {list(sh)}")
    return R


def kda_decode(q, k, v, g_raw, beta_raw, A_log, dt_bias, state_pool, state_indices, out,
               lower_bound: float = -5.0, scale: float = 1.0, gate_mode: int = 0,
               stream=None) -> None:
    """T=1 decode. q, k, v, g_raw, out: bf16 [B, H*128] (row-strided views
    allowed); beta_raw bf16 [B, H]; A_log fp32 [H]; dt_bias fp32 [H*128];
    state_pool bf16 or fp16 [N, ...] (slot-major; its dtype selects the state
    element type); state_indices int32 [B]."""
    B, W = q.shape
    H = W // HEAD_DIM
    for n, t in (("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw),
                 ("out", out)):
        _bf16(n, t)
    pre = bool(gate_mode & GATE_PRECOMPUTED)
    _f32("A_log", A_log, optional=pre)
    _f32("dt_bias", dt_bias, optional=pre)
    _i32("state_indices", state_indices)
    N, slot_stride = _pool_geometry(state_pool, H)
    st = lib().kda_decode(B, H, HEAD_DIM, HEAD_DIM,
                          _ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0),
                          _ptr(g_raw), g_raw.stride(0), _ptr(beta_raw), beta_raw.stride(0),
                          _ptr(A_log), _ptr(dt_bias), float(lower_bound), float(scale),
                          int(gate_mode), _state_dtype(state_pool),
                          _ptr(state_pool) if N else _P(0), N, slot_stride,
                          _ptr(state_indices), _ptr(out), out.stride(0), _stream(stream))
    _check("kda_decode", st)


def kda_verify_ucache_flush(q, k, v, g_raw, beta_raw, A_log, dt_bias, state_pool,
                            state_indices, k_cache, u_cache, g_cache, hist_len, cache_base,
                            out, flush_min: int, w_ring: int = 16,
                            restart_hist_on_flush: bool = True, lower_bound: float = -5.0,
                            scale: float = 1.0, gate_mode: int = 0, stream=None) -> None:
    """Verify+fold. q, k, v, g_raw, out: bf16 [B, T, H*128]; beta_raw bf16
    [B, T, H]; k_cache/u_cache bf16 [N, H, R, 128]; g_cache fp32 [N, H, R, 128];
    hist_len, cache_base int32 [B]."""
    B, T, W = q.shape
    H = W // HEAD_DIM
    for n, t in (("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw),
                 ("out", out), ("k_cache", k_cache), ("u_cache", u_cache)):
        _bf16(n, t)
    pre = bool(gate_mode & GATE_PRECOMPUTED)
    _f32("A_log", A_log, optional=pre)
    _f32("dt_bias", dt_bias, optional=pre)
    _f32("g_cache", g_cache)
    for n, t in (("state_indices", state_indices), ("hist_len", hist_len),
                 ("cache_base", cache_base)):
        _i32(n, t)
    if not (k_cache.is_contiguous() and u_cache.is_contiguous()):
        raise ValueError("ring caches must be contiguous")
    N, slot_stride = _pool_geometry(state_pool, H)
    R = _ring_rows(k_cache, u_cache, g_cache, N, H)
    st = lib().kda_verify_ucache_flush(
        B, T, H, HEAD_DIM, HEAD_DIM,
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1),
        _ptr(v), v.stride(0), v.stride(1), _ptr(g_raw), g_raw.stride(0), g_raw.stride(1),
        _ptr(beta_raw), beta_raw.stride(0), beta_raw.stride(1),
        _ptr(A_log), _ptr(dt_bias), float(lower_bound), float(scale), int(gate_mode),
        _state_dtype(state_pool), _ptr(state_pool) if N else _P(0), N, slot_stride,
        _ptr(state_indices), _ptr(k_cache), _ptr(u_cache), _ptr(g_cache), R, _ptr(hist_len), _ptr(cache_base),
        int(flush_min), int(w_ring), 1 if restart_hist_on_flush else 0,
        _ptr(out), out.stride(0), out.stride(1), _stream(stream))
    _check("kda_verify_ucache_flush", st)


def kda_prefill_workspace_size(n_docs: int, total_tokens: int, H: int) -> int:
    return int(lib().kda_prefill_workspace_size(n_docs, total_tokens, H, HEAD_DIM, HEAD_DIM))


def kda_prefill_varlen(cu_seqlens_host, cu_seqlens, q, k, v, g_raw, beta_raw, A_log, dt_bias,
                       state_pool, state_indices, out, workspace=None,
                       use_initial_state: bool = True, lower_bound: float = -5.0,
                       scale: float = 1.0, gate_mode: int = 0, checkpoints=None,
                       checkpoint_cu_starts=None, checkpoint_interval: int = 16,
                       ring=None, cache_base=None, ring_tail: int = 0,
                       stream=None) -> None:
    """Varlen prefill. cu_seqlens_host: CPU int32 [n_docs+1]; cu_seqlens: the
    same on the GPU; q, k, v, g_raw, out: bf16 [Ttot, H*128] (token-strided);
    beta_raw bf16 [Ttot, H]; state_indices int32 [n_docs]; workspace: uint8
    GPU tensor of >= kda_prefill_workspace_size(...) bytes, or None to have
    one allocated here for this call. checkpoints: bf16 [rows, H, 128, 128]
    (contiguous) receiving the state after every checkpoint_interval tokens of
    each document at rows checkpoint_cu_starts[d] + i (int64 GPU tensor
    [n_docs]), or None. ring = (k_cache bf16, u_cache bf16, g_cache fp32, each
    [N, H, R, 128]) with cache_base int32 [n_docs] and ring_tail in 1..16: each
    document hands its last prefill_handoff_hist(...)[d] tokens to the ring at
    rows cache_base[d] onwards, and its slot receives the state before them."""
    import torch
    args = _prefill_args(cu_seqlens_host, cu_seqlens, q, k, v, g_raw, beta_raw, A_log, dt_bias,
                         state_pool, state_indices, out, use_initial_state, lower_bound, scale,
                         gate_mode, checkpoints, checkpoint_cu_starts, checkpoint_interval, ring,
                         cache_base, ring_tail)
    if workspace is None:
        need = kda_prefill_workspace_size(args[0], args[1], args[2])
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kda_prefill_varlen(*args, _ptr(workspace), ws_bytes, _stream(stream))
    _check("kda_prefill_varlen", st)


def kda_prefill_varlen_noalloc(cu_seqlens_host, cu_seqlens, q, k, v, g_raw, beta_raw, A_log,
                               dt_bias, state_pool, state_indices, out,
                               use_initial_state: bool = True, lower_bound: float = -5.0,
                               scale: float = 1.0, gate_mode: int = 0, checkpoints=None,
                               checkpoint_cu_starts=None, checkpoint_interval: int = 16,
                               ring=None, cache_base=None, ring_tail: int = 0,
                               stream=None) -> None:
    """kda_prefill_varlen without a workspace: allocates nothing (here or in the
    library). Where a workspace is needed the library's per-device scratch of
    NOALLOC_SCRATCH_BYTES serves; a call needing more raises KdaError
    (KDA_ERR_SCRATCH_LIMIT). Calls on one device share that scratch, so calls
    on different streams must be ordered."""
    args = _prefill_args(cu_seqlens_host, cu_seqlens, q, k, v, g_raw, beta_raw, A_log, dt_bias,
                         state_pool, state_indices, out, use_initial_state, lower_bound, scale,
                         gate_mode, checkpoints, checkpoint_cu_starts, checkpoint_interval, ring,
                         cache_base, ring_tail)
    st = lib().kda_prefill_varlen_noalloc(*args, _stream(stream))
    _check("kda_prefill_varlen_noalloc", st)


def _prefill_args(cu_seqlens_host, cu_seqlens, q, k, v, g_raw, beta_raw, A_log, dt_bias,
                  state_pool, state_indices, out, use_initial_state, lower_bound, scale,
                  gate_mode, checkpoints, checkpoint_cu_starts, checkpoint_interval, ring,
                  cache_base, ring_tail):
    """Checks and the C arguments shared by both prefill entry points, up to
    (not including) the workspace and the stream."""
    import torch
    if cu_seqlens_host.dtype != torch.int32 or cu_seqlens_host.is_cuda or \
            not cu_seqlens_host.is_contiguous():
        raise ValueError("cu_seqlens_host must be a contiguous int32 CPU tensor")
    _i32("cu_seqlens", cu_seqlens)
    _i32("state_indices", state_indices)
    n_docs = cu_seqlens_host.shape[0] - 1
    Ttot, W = q.shape
    H = W // HEAD_DIM
    for n, t in (("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw),
                 ("out", out)):
        _bf16(n, t)
    pre = bool(gate_mode & GATE_PRECOMPUTED)
    _f32("A_log", A_log, optional=pre)
    _f32("dt_bias", dt_bias, optional=pre)
    N, slot_stride = _pool_geometry(state_pool, H)
    ck_rows = 0
    if checkpoints is not None:
        if checkpoints.dtype != state_pool.dtype or not checkpoints.is_cuda:
            raise ValueError("checkpoints must be a GPU tensor of the state pool's dtype")
        if not checkpoints.is_contiguous() or \
                checkpoints.numel() != checkpoints.shape[0] * H * HEAD_DIM * HEAD_DIM:
            raise ValueError("checkpoints must be a contiguous bf16 [rows, H, 128, 128] tensor")
        if checkpoint_cu_starts is None or checkpoint_cu_starts.dtype != torch.int64 or \
                not checkpoint_cu_starts.is_cuda or not checkpoint_cu_starts.is_contiguous():
            raise ValueError("checkpoint_cu_starts must be a contiguous int64 GPU tensor")
        ck_rows = checkpoints.shape[0]
    kc = uc = gc = None
    R = 0
    if ring_tail:
        kc, uc, gc = ring
        _bf16("k_cache", kc)
        _bf16("u_cache", uc)
        _f32("g_cache", gc)
        _i32("cache_base", cache_base)
        if not (kc.is_contiguous() and uc.is_contiguous() and gc.is_contiguous()):
            raise ValueError("ring caches must be contiguous")
        R = _ring_rows(kc, uc, gc, N, H)
    cu_h = _P(cu_seqlens_host.data_ptr())
    return (
        n_docs, Ttot, H, HEAD_DIM, HEAD_DIM, cu_h, _ptr(cu_seqlens),
        _ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0),
        _ptr(g_raw), g_raw.stride(0), _ptr(beta_raw), beta_raw.stride(0),
        _ptr(A_log), _ptr(dt_bias), float(lower_bound), float(scale), int(gate_mode),
        _state_dtype(state_pool), _ptr(state_pool) if N else _P(0), N, slot_stride,
        _ptr(state_indices), 1 if use_initial_state else 0, _ptr(out), out.stride(0),
        _ptr(checkpoints), ck_rows, _ptr(checkpoint_cu_starts), int(checkpoint_interval),
        _ptr(kc), _ptr(uc), _ptr(gc), R, _ptr(cache_base), int(ring_tail))


def prefill_handoff_hist(cu_seqlens_host, ring_tail: int):
    """Ring history entries each document hands off (the hist_len of its next
    verify call): min(ring_tail, tokens after its last 16-token boundary), 0 for
    an empty document. CPU int32 tensor [n_docs]."""
    import torch
    lens = (cu_seqlens_host[1:] - cu_seqlens_host[:-1]).to(torch.int64)
    last = lens - 16 * torch.div(lens - 1, 16, rounding_mode="floor")
    return torch.where(lens > 0, torch.clamp(last, max=int(ring_tail)),
                       torch.zeros_like(lens)).to(torch.int32)
