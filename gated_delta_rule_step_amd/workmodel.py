"""Algorithmic (compulsory) bytes and flops of one call of each entry point.

Byte model, per head of 128 x 128 bf16 state and per token:
  state   SB   = 128 * 128 * 2           = 32,768 B per head
  inputs  TOK_IN  = q, k, v, gate (4 * 128 * 2) + beta (2) = 1,026 B per head
  output  TOK_OUT = 128 * 2              = 256 B per head
  ring    RING_ROW = k_hat (256) + u (256) + G (128 * 4) = 1,024 B per head
Per row (12 heads) that is 393,216 B of state, 12,312 B of token input and
3,072 B of output; "feat(kda): add packed-input CuTe decode kernel", section
"DRAM utilization", prints the same model (786 KB round trip per row, ~402 MB
of state at B = 512, ~15 KB of activations per row), and its 207.7 MB of
DRAM reads at B = 512 equal B * (state + inputs + index).

state_bytes (every model below) is the state element size: 2 for bf16 and
fp16, 1 for fp8 e4m3, which halves SB.
"""
from __future__ import annotations

D = 128
SB = D * D * 2
TOK_IN = 4 * D * 2 + 2
TOK_OUT = D * 2
RING_ROW = D * 2 + D * 2 + D * 4
IDX = 4
FLOP_STEP = 3 * 2 * D * D + D * D  # decay, S'k, rank-1 update, S q per token-head

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense


def _sb(state_bytes: int) -> int:
    return D * D * state_bytes


def decode_bytes(n_active: int, n_inactive: int, H: int = 12, state_bytes: int = 2) -> int:
    """T = 1 decode: an active row reads and writes its state, reads one
    token of inputs and its index, writes one output row; an inactive row
    reads its index and writes a zero output row."""
    active = 2 * _sb(state_bytes) * H + TOK_IN * H + TOK_OUT * H + IDX
    inactive = TOK_OUT * H + IDX
    return n_active * active + n_inactive * inactive


def decode_read_bytes(n_rows: int, H: int = 12) -> int:
    return n_rows * (SB * H + TOK_IN * H + IDX)


def decode_flops(n_active: int, H: int = 12) -> int:
    return n_active * H * FLOP_STEP


def verify_bytes(T: int, hist, fold, n_inactive: int = 0, H: int = 12,
                 state_bytes: int = 2) -> int:
    """Verify+fold: an active row reads its checkpoint, its hist live ring rows
    and T tokens of inputs, writes T outputs and T ring rows, and writes the
    checkpoint back when it folds; plus three int32 of metadata per row."""
    total = 0
    for h_len, f in zip(hist, fold):
        sb = _sb(state_bytes)
        total += sb * H + int(h_len) * RING_ROW * H + T * (TOK_IN + TOK_OUT + RING_ROW) * H
        total += sb * H if f else 0
        total += 3 * IDX
    total += n_inactive * (T * TOK_OUT * H + 3 * IDX)
    return total


def verify_flops(T: int, hist, H: int = 12) -> int:
    return sum(H * (T * FLOP_STEP + int(h) * 2 * D * D) for h in hist)


def prefill_bytes(doc_lens, H: int, n_active_docs: int | None = None,
                  state_bytes: int = 2) -> int:
    """Prefill: per token-head q, k, v, gate, beta in and o out; per
    (document, head) one initial state read and one final state write."""
    n = len(doc_lens) if n_active_docs is None else n_active_docs
    tokens = sum(doc_lens)
    return (tokens * H * (TOK_IN + TOK_OUT) + n * H * 2 * _sb(state_bytes) +
            (len(doc_lens) + 1) * IDX)


def chunk_flops(c: int, K: int = D, V: int = D) -> int:
    """Flops of the chunkwise (WY/UT) form for one chunk of c tokens and one
    head: gated Gram and QK products, the triangular solve, W and U0, the
    state products W S and (e^G q) S, P U, and the state update."""
    return int(2 * K * c * c + (2 * c ** 3) // 3 + 2 * K * c * (c + 1) + 6 * c * K * V
               + V * c * (c + 1) + K * V)


def prefill_flops(doc_lens, H: int, chunk: int = 64) -> int:
    total = 0
    for n in doc_lens:
        full, tail = divmod(int(n), chunk)
        total += full * chunk_flops(chunk) + (chunk_flops(tail) if tail else 0)
    return total * H
