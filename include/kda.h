/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA gated delta-rule step library.
 *
 * The method (Kimi Delta Attention): per head h, a state S that maps 128 key
 * channels to 128 value channels is updated for every token by
 *   S' = diag(exp(g)) S                (per-key-channel decay)
 *   u  = beta * (v - S' k_hat)         (delta-rule correction, L2-normalised key)
 *   S  = S' + k_hat u^T                (rank-1 write)
 *   o  = scale * S q_hat               (read-out)
 * as described on "feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3
 * (KDA)" (sections "What it does" and "Caching") and "feat(kda): add
 * packed-input CuTe decode kernel" (opening description, "Kernel design").
 * The per-token prologue computed inside every entry point:
 *   q_hat = q / sqrt(|q|^2 + 1e-6), k_hat = k / sqrt(|k|^2 + 1e-6)   (fp32)
 *   g_c   = max(lower_bound, -exp(A_log[h]) * softplus(graw_c + dt_bias[h*128 + c]))
 *   beta  = sigmoid(beta_logit)
 * The pages name these inputs (raw gate, fp32 A_log and dt_bias,
 * lower_bound = -5, beta as a logit, in-kernel QK L2 norm) but print no
 * formula; the gate formula and the epsilon are this library's reading.
 *
 * Gate convention (argument gate_mode of every entry point; "feat(kda): add
 * packed-input CuTe decode kernel", section "T=1 fast path inside
 * recurrent_kda": the raw form above, and the API-default pre-computed form
 * with log-space g and pre-sigmoided beta, decay = exp(g)):
 *  - 0: g_raw holds gate logits and beta_raw beta logits (the formulas above);
 *  - KDA_GATE_PRECOMPUTED: g_raw holds the log-decay g_c itself, used as
 *    min(0, max(lower_bound, g_c)) -- the range the raw gate lands in (a
 *    reading); A_log and dt_bias are not read and may be NULL; lower_bound
 *    must be <= 0 (-INFINITY: no floor), else KDA_ERR_UNSUPPORTED;
 *  - KDA_BETA_PRESIGMOID: beta_raw holds beta itself, used as given;
 *  - KDA_GATE_PER_HEAD: the scalar (per-head) decay of GDN, which "feat(kda):
 *    ReplaySSM verify+flush decode kernel for Kimi K3 (KDA)" ("What it does")
 *    contrasts with KDA's per-key-channel gate: g_raw holds ONE value per
 *    token and head, at the offset a beta value has (h, not h*128), and
 *    dt_bias holds H values; the gate formula above (or the pre-computed
 *    value) is applied to that value and the result decays every key channel
 *    of the head (a reading).
 * The bits combine; any other bit gives KDA_ERR_UNSUPPORTED.
 *
 * State element type (argument state_dtype of every entry point): the pages'
 * GDN verify kernel offers "an optional fp16 checkpoint-state mode"
 * ("feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3 (KDA)",
 * "Caching"). KDA_STATE_BF16 (0) keeps the pool, the verify checkpoints and the
 * prefill states in bf16; KDA_STATE_FP16 (1) keeps them in fp16 (IEEE binary16,
 * rounded to nearest even), the same 2 bytes with 3 more fraction bits and a
 * range of +-65504. KDA_STATE_FP8 (2) keeps them in one byte, the OCP FP8
 * E4M3 format ("e4m3fn": bias 7, 3 fraction bits, largest finite value 448, no
 * infinities), rounded to nearest even with magnitudes beyond 448 saturated to
 * 448: the byte reduction the decode page ("feat(kda): add packed-input CuTe
 * decode kernel") names as the lever left at its measured HBM fraction; it
 * halves the state traffic at the cost of a 2^-4 relative step. Token inputs,
 * outputs and the verify rings stay bf16 and g_cache fp32. fp16 and fp8 states
 * need the vectorised layout (16-byte aligned bases, strides in multiples of
 * 8), else KDA_ERR_UNSUPPORTED; any other value also gives
 * KDA_ERR_UNSUPPORTED.
 *
 * Conventions common to every entry point
 *  - Every pointer is a DEVICE pointer, except those whose name ends in _host.
 *  - bf16 tensors are passed as `const void*` / `void*` holding raw bf16 bits.
 *  - Strides and offsets are in ELEMENTS of the tensor's own type.
 *  - Head h of a q, k, v, gate or out row sits at element offset h*128 of the
 *    row; head h of a beta row at offset h.
 *  - State pool: bf16 slots of slot_stride elements (slot_stride >= H*128*128,
 *    padding allowed). Inside a slot, head h starts at h*16384 and holds the
 *    128 x 128 state with element (v, c) -- value channel v, key channel c --
 *    at v*128 + c (key channels contiguous). The pages fix only the shape
 *    [N, H, 128, 128]; this orientation makes S k_hat a contiguous dot product.
 *  - The caller owns every buffer. The library never allocates or frees
 *    memory, never synchronises, and keeps no state between calls; each call
 *    only enqueues kernels on `stream` (asynchronous, capture-safe).
 *  - Pool, rings and checkpoints are updated in place. `out` must not alias
 *    any input, pool or ring. Active state indices must be pairwise distinct
 *    (duplicates are undefined behaviour).
 *  - Any 2-byte-aligned bf16 pointer and any stride is accepted; a vectorised
 *    path runs when bases are 16-byte aligned and strides are multiples of 8.
 *
 * Errors
 *  - Host-visible problems (null pointers, shapes, strides, unsupported
 *    configurations) return an error BEFORE anything is launched; no buffer
 *    is touched.
 *  - Device-visible bad values never fault and never reach memory they do not
 *    own: a row whose state index lies outside [0, num_slots) (or whose ring
 *    metadata is out of range, see kda_verify_ucache_flush) is INACTIVE: its
 *    outputs are written as +0.0 and its pool, ring and checkpoint are left
 *    bitwise untouched. num_slots = 0 makes every row inactive.
 *  - KDA_ERR_LAUNCH: the HIP runtime rejected a launch.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KDA_GATE_PRECOMPUTED = 1,  /* gate_mode bit: g_raw is the log-decay itself */
  KDA_BETA_PRESIGMOID = 2,   /* gate_mode bit: beta_raw is beta itself */
  KDA_GATE_PER_HEAD = 4      /* gate_mode bit: one gate value (and dt_bias) per head */
};

enum {
  KDA_STATE_BF16 = 0,  /* state_dtype: pool / checkpoint elements are bf16 */
  KDA_STATE_FP16 = 1,  /* state_dtype: pool / checkpoint elements are fp16 */
  KDA_STATE_FP8 = 2    /* state_dtype: pool / checkpoint elements are fp8 e4m3 */
};

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL_POINTER = 1,
  KDA_ERR_BAD_SHAPE = 2,
  KDA_ERR_BAD_STRIDE = 3,
  KDA_ERR_UNSUPPORTED = 4,
  KDA_ERR_BAD_SEQLENS = 5,
  KDA_ERR_WORKSPACE_TOO_SMALL = 6,
  KDA_ERR_LAUNCH = 7,
  KDA_ERR_SCRATCH_LIMIT = 8  /* kda_prefill_varlen_noalloc: the call needs more
                                than KDA_NOALLOC_SCRATCH_BYTES of workspace */
} kda_status;

/* Static, NUL-terminated description of a status code ("unknown status" for
 * values outside the enum). Never fails. */
const char* kda_status_string(kda_status s);

/*
 * kda_decode -- one token (T = 1) per batch row against an in-place pool.
 *
 * Passage: "feat(kda): add packed-input CuTe decode kernel", opening
 * description (packed bf16 QKV rows [B, 3*12*128], raw gate and beta logits,
 * fp32 math, bf16 pool [N, 12, 128, 128] updated in place, rows whose state
 * index is negative or past the end give zero output and leave the pool
 * untouched) and section "T=1 fast path inside recurrent_kda" (q/k/v/g/beta
 * as independent strided views, padded pools, in-kernel pool indexing).
 *
 *  B                  rows (>= 0; B = 0 is a no-op)
 *  H                  heads (>= 1)
 *  K, V               must both be 128
 *  q, k, v            bf16 [B, H*128] views with row strides q_row_stride,
 *                     k_row_stride, v_row_stride (may be three views into one
 *                     packed [B, 3*H*128] row)
 *  g_raw              bf16 [B, H*128] raw gate logits (or the log-decay, see
 *                     gate_mode; [B, H] with KDA_GATE_PER_HEAD), row stride
 *                     g_row_stride
 *  beta_raw           bf16 [B, H] beta logits (or beta), row stride beta_row_stride
 *  A_log              fp32 [H] (not read with KDA_GATE_PRECOMPUTED)
 *  dt_bias            fp32 [H*128], or [H] with KDA_GATE_PER_HEAD (not read
 *                     with KDA_GATE_PRECOMPUTED)
 *  lower_bound        clamp of the log-decay (the pages use -5.0)
 *  scale              read-out scale
 *  gate_mode          0, or any of KDA_GATE_PRECOMPUTED, KDA_BETA_PRESIGMOID,
 *                     KDA_GATE_PER_HEAD
 *  state_dtype        KDA_STATE_BF16, KDA_STATE_FP16 or KDA_STATE_FP8 (the
 *                     pool's elements)
 *  state_pool         pool of state_dtype elements, num_slots slots of
 *                     slot_stride elements
 *                     (may be NULL only when num_slots == 0)
 *  state_indices      int32 [B]: the pool slot of each row
 *  out                bf16 [B, H*128], row stride out_row_stride
 *  stream             HIP stream the kernel is enqueued on
 *
 * Row strides must be >= H*128 (>= H for beta), slot_stride >= H*128*128.
 */
kda_status kda_decode(int32_t B, int32_t H, int32_t K, int32_t V,
                      const void* q, int64_t q_row_stride,
                      const void* k, int64_t k_row_stride,
                      const void* v, int64_t v_row_stride,
                      const void* g_raw, int64_t g_row_stride,
                      const void* beta_raw, int64_t beta_row_stride,
                      const float* A_log, const float* dt_bias,
                      float lower_bound, float scale, int32_t gate_mode,
                      int32_t state_dtype,
                      void* state_pool, int64_t num_slots, int64_t slot_stride,
                      const int32_t* state_indices,
                      void* out, int64_t out_row_stride,
                      hipStream_t stream);

/*
 * kda_verify_ucache_flush -- speculative-decode verification of T draft
 * tokens per row with a (k_hat, u, G) ring cache folded into the checkpoint.
 *
 * Passage: "feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3
 * (KDA)", sections "What it does" (append k, u and the per-channel decay to a
 * ring instead of writing the state per token; fold the ring into the
 * checkpoint once flush_min is reached), "API" (T inferred from the draft
 * length; T = 8 with flush_min 9, T = 4 with flush_min 13; restart_hist_on_flush)
 * and "Caching" (k_cache/u_cache bf16 [pool, H, 32, 128], g_cache fp32
 * cumulative log-decay; replay weights w_j = exp(G_P - G_j)).
 *
 * Ring contract (the pages give names and fragments; this is the reading the
 * library implements). Per row b with slot s = state_indices[b],
 * hist = hist_len[b], base = cache_base[b], R = ring_rows:
 *  - history entry j < hist lives in ring row (base + j) mod R of slot s and
 *    holds k_hat_j (bf16), u_j (bf16) and G_j (fp32, cumulative log-decay of
 *    history tokens 0..j);
 *  - S_cur = diag(exp(G_L)) S_ckpt + sum_j diag(exp(G_L - G_j)) k_hat_j u_j^T,
 *    G_L = G_{hist-1} (S_cur = S_ckpt when hist = 0), in fp32;
 *  - fold = (hist + T >= flush_min);
 *  - draft token t = 0..T-1 steps from S_cur in order: out[b, t] is its
 *    read-out; ring row (base + hist + t) mod R receives k_hat_t, u_t and
 *    G = G_base + g_0 + ... + g_t (fp32, accumulated in token order), with
 *    G_base = 0 when folding and G_{hist-1} (0 if hist = 0) otherwise;
 *  - when folding, the checkpoint slot receives bf16(S_cur);
 *  - the library never writes hist_len or cache_base. With a accepted tokens
 *    the caller's next call uses fold ? (base + hist mod R, a) : (base, hist + a).
 * A row is inactive (zero outputs, no pool or ring writes) when its slot is
 * outside [0, num_slots), hist < 0, hist + T > w_ring, or base is outside
 * [0, R).
 *
 *  B, T               rows (>= 0) and draft tokens per row (1..8)
 *  H, K, V            heads (>= 1); K = V = 128
 *  q, k, v, g_raw     bf16, element (b, t, h*128 + c) at
 *                     b*row_stride + t*tok_stride + h*128 + c
 *  beta_raw           bf16, element (b, t, h) at b*row_stride + t*tok_stride + h
 *  A_log, dt_bias, lower_bound, scale, gate_mode, state_dtype, state_pool,
 *  num_slots, slot_stride, state_indices  as for kda_decode (the pool holds the
 *                     checkpoints)
 *  k_cache, u_cache   bf16 [num_slots, H, ring_rows, 128]
 *  g_cache            fp32 [num_slots, H, ring_rows, 128]
 *  ring_rows          R, physical ring rows per (slot, head) (>= w_ring)
 *  hist_len, cache_base  int32 [B]
 *  flush_min          fold threshold (>= 1)
 *  w_ring             logical window, 16 or 32; 32 requires flush_min > 16;
 *                     flush_min - 1 + T <= w_ring (capacity)
 *  restart_hist_on_flush  must be 1
 *  out                bf16, element (b, t, h*128 + v) at
 *                     b*out_row_stride + t*out_tok_stride + h*128 + v
 * KDA_ERR_UNSUPPORTED for T outside 1..8, w_ring not 16/32, ring_rows <
 * w_ring, restart_hist_on_flush != 1, flush_min < 1, the capacity rule, or
 * w_ring == 32 with flush_min <= 16.
 */
kda_status kda_verify_ucache_flush(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                   const void* q, int64_t q_row_stride, int64_t q_tok_stride,
                                   const void* k, int64_t k_row_stride, int64_t k_tok_stride,
                                   const void* v, int64_t v_row_stride, int64_t v_tok_stride,
                                   const void* g_raw, int64_t g_row_stride, int64_t g_tok_stride,
                                   const void* beta_raw, int64_t beta_row_stride,
                                   int64_t beta_tok_stride,
                                   const float* A_log, const float* dt_bias,
                                   float lower_bound, float scale, int32_t gate_mode,
                                   int32_t state_dtype,
                                   void* state_pool, int64_t num_slots, int64_t slot_stride,
                                   const int32_t* state_indices,
                                   void* k_cache, void* u_cache, float* g_cache,
                                   int32_t ring_rows,
                                   const int32_t* hist_len, const int32_t* cache_base,
                                   int32_t flush_min, int32_t w_ring,
                                   int32_t restart_hist_on_flush,
                                   void* out, int64_t out_row_stride, int64_t out_tok_stride,
                                   hipStream_t stream);

/*
 * kda_prefill_workspace_size -- bytes of device workspace kda_prefill_varlen
 * needs for these sizes (0 when nothing is needed, or when K or V is not 128).
 * Pure host arithmetic. 0 when n_docs * H >= 256: those calls run the fused
 * kernel, which keeps every chunk's operands on chip. Below that, one
 * 29,696-byte chunk record per (chunk slot, head), with
 * (n_docs + floor(total_tokens / 16)) chunk slots, since a document's
 * 16-token chunks are numbered from its index plus floor(first token / 16).
 */
size_t kda_prefill_workspace_size(int32_t n_docs, int64_t total_tokens, int32_t H, int32_t K,
                                  int32_t V);

/*
 * kda_prefill_varlen -- chunked prefill over packed documents.
 *
 * Passage: "feat(kda): add CuTe DSL recurrent prefill backend" (packed
 * variable-length documents delimited by cu_seqlens, which must start at 0 and
 * be non-decreasing, zero-length documents allowed; optional initial and final
 * states in a pool addressed by state indices; chunked recurrence in two
 * stages, an intra-chunk preparation and a sequential chain over chunks).
 * The result is the token-by-token recurrence of every (document, head) chain.
 * Two forms, chosen from n_docs * H alone: with at least 256 (document, head)
 * chains, one fused kernel (a workgroup per chain prepares each 64-token
 * chunk and advances the state through it, no workspace); with fewer, a
 * preparation kernel over every 16-token chunk of every chain writes records
 * to the workspace and a chain kernel consumes them. Both give the same
 * recurrence within rounding.
 *
 *  n_docs             documents (>= 0)
 *  total_tokens       tokens over all documents (>= 0)
 *  H, K, V            heads (>= 1); K = V = 128
 *  cu_seqlens_host    int32 [n_docs + 1], HOST copy: validated and used to plan
 *  cu_seqlens         int32 [n_docs + 1], device copy with the same contents
 *  q, k, v, g_raw     bf16, element (t, h*128 + c) at t*tok_stride + h*128 + c
 *  beta_raw           bf16, element (t, h) at t*beta_tok_stride + h
 *  A_log, dt_bias, lower_bound, scale, gate_mode, state_dtype  as for kda_decode
 *                     (checkpoints, below, use the state element type too)
 *  state_pool, num_slots, slot_stride  as for kda_decode
 *  state_indices      int32 [n_docs]: slot of each document (initial and final
 *                     state); a document whose slot is outside [0, num_slots)
 *                     gets zero outputs and no state write
 *  use_initial_state  1: start each chain from its slot; 0: from zeros
 *  out                bf16, element (t, h*128 + v) at t*out_tok_stride + h*128 + v
 *  checkpoints        NULL (no intermediate checkpoints), or rows (of the state
 *                     element type, see state_dtype) of H
 *                     states laid out like a pool slot (row r, head h at
 *                     (r*H + h)*16384, element (v, c) at v*128 + c). The page
 *                     returns "output, final state, checkpoints" with an int64
 *                     checkpoint_cu_starts; the positions are this library's
 *                     reading: an active document d stores its state after its
 *                     first i*checkpoint_interval tokens, i = 1 ..
 *                     floor(len_d / checkpoint_interval), into row
 *                     checkpoint_cu_starts[d] + i - 1; rows outside
 *                     [0, checkpoint_rows) are skipped; inactive documents store
 *                     none. Rounded like the final state.
 *  checkpoint_rows    rows of `checkpoints` (>= 0)
 *  checkpoint_cu_starts  int64 [n_docs] device array (read only when
 *                     checkpoints is not NULL)
 *  checkpoint_interval  tokens between checkpoints: a positive multiple of 16
 *                     (the chunk), else KDA_ERR_UNSUPPORTED
 *  k_cache, u_cache, g_cache, ring_rows, cache_base, ring_tail
 *                     hand-off to speculative decoding (this library's reading
 *                     of a prefill that leaves each sequence in the form
 *                     kda_verify_ucache_flush resumes from: a checkpoint plus
 *                     ring history, "feat(kda): ReplaySSM verify+flush decode
 *                     kernel for Kimi K3 (KDA)", "Caching"). ring_tail = 0: off,
 *                     the ring arguments are not read (may be NULL). 1..16: an
 *                     active document d of len_d > 0 tokens hands its last
 *                     r_d = min(ring_tail, len_d - 16*floor((len_d - 1)/16))
 *                     tokens (never more than those after its last 16-token
 *                     boundary) to the ring of its slot s = state_indices[d]:
 *                     its slot receives the state after its first len_d - r_d
 *                     tokens instead of the final state, and tail token j
 *                     (0 <= j < r_d) writes ring row (cache_base[d] + j) mod
 *                     ring_rows with k_hat_j and u_j (bf16) and G_j (fp32, the
 *                     log-decay summed over tail tokens 0..j), exactly the rows
 *                     a verify call would have appended. The next verify call
 *                     for d takes hist_len = r_d and the same cache_base.
 *                     Outputs are unchanged; checkpoints cover only the first
 *                     len_d - r_d tokens. k_cache and u_cache are bf16 and
 *                     g_cache fp32, each [num_slots, H, ring_rows, 128];
 *                     cache_base is int32 [n_docs]; a document whose
 *                     cache_base lies outside [0, ring_rows) is inactive (zero
 *                     outputs, nothing written). ring_tail outside 0..16 gives
 *                     KDA_ERR_UNSUPPORTED, ring_rows < ring_tail
 *                     KDA_ERR_BAD_SHAPE, a NULL ring pointer with ring_tail > 0
 *                     KDA_ERR_NULL_POINTER.
 *  workspace          device buffer of >= kda_prefill_workspace_size(...) bytes,
 *                     256-byte aligned (may be NULL when that size is 0); the
 *                     per-chunk operands pass through it from the preparation
 *                     kernel to the chain kernel, and its contents are
 *                     meaningless after the call
 * A zero-length document writes no output; its final state equals its
 * initial state (left untouched with use_initial_state = 1, written as zeros
 * with use_initial_state = 0).
 * KDA_ERR_BAD_SEQLENS when cu_seqlens_host[0] != 0, it decreases, or its last
 * entry differs from total_tokens; KDA_ERR_WORKSPACE_TOO_SMALL when
 * workspace_bytes is short; KDA_ERR_NULL_POINTER when a workspace is needed
 * and NULL; KDA_ERR_UNSUPPORTED when the workspace is not 256-byte aligned,
 * when out_tok_stride exceeds 2^25 elements (16 output rows must span less
 * than 2^31 bytes) or when |lower_bound| > 5.5 (both forms factor each decay
 * weight exp(G_r - G_j) within a 16-token block into two exps of at most
 * 8 |lower_bound| each, which must stay well inside the fp32 range). The call
 * launches the fused kernel, or a preparation kernel and then a chain kernel,
 * on the stream; the longest documents are started first (for up to 256
 * documents; natural order beyond).
 * Outputs are written in bf16 (round to nearest even); the final states are
 * rounded to bf16 once, at the end of each chain.
 */
kda_status kda_prefill_varlen(int32_t n_docs, int64_t total_tokens, int32_t H, int32_t K,
                              int32_t V,
                              const int32_t* cu_seqlens_host, const int32_t* cu_seqlens,
                              const void* q, int64_t q_tok_stride,
                              const void* k, int64_t k_tok_stride,
                              const void* v, int64_t v_tok_stride,
                              const void* g_raw, int64_t g_tok_stride,
                              const void* beta_raw, int64_t beta_tok_stride,
                              const float* A_log, const float* dt_bias,
                              float lower_bound, float scale, int32_t gate_mode,
                              int32_t state_dtype,
                              void* state_pool, int64_t num_slots, int64_t slot_stride,
                              const int32_t* state_indices, int32_t use_initial_state,
                              void* out, int64_t out_tok_stride,
                              void* checkpoints, int64_t checkpoint_rows,
                              const int64_t* checkpoint_cu_starts, int32_t checkpoint_interval,
                              void* k_cache, void* u_cache, float* g_cache, int32_t ring_rows,
                              const int32_t* cache_base, int32_t ring_tail,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * kda_prefill_varlen_noalloc -- kda_prefill_varlen without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Every argument means what it means for kda_prefill_varlen. Where that call
 * needs a workspace (kda_prefill_workspace_size(...) > 0: fewer than 256
 * (document, head) chains), this one uses a scratch array of
 * KDA_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * (created when its code object is loaded there, kept until the process
 * ends); calls with 256 chains or more need none and have no size limit here.
 * Nothing is allocated and nothing in the scratch needs clearing (every
 * record the chain reads is written by the same call's preparation kernel).
 * The first call on a device looks up that device's scratch address (with the
 * device current) and keeps it.
 * All calls on one device share its scratch: two calls whose kernels may
 * overlap (different streams without ordering between them) race and give
 * wrong results; order them on one stream or with events.
 * KDA_ERR_SCRATCH_LIMIT when kda_prefill_workspace_size(...) exceeds
 * KDA_NOALLOC_SCRATCH_BYTES (nothing is read or launched); KDA_ERR_LAUNCH when
 * the scratch address cannot be obtained; otherwise the statuses of
 * kda_prefill_varlen.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

kda_status kda_prefill_varlen_noalloc(int32_t n_docs, int64_t total_tokens, int32_t H,
                                      int32_t K, int32_t V,
                                      const int32_t* cu_seqlens_host, const int32_t* cu_seqlens,
                                      const void* q, int64_t q_tok_stride,
                                      const void* k, int64_t k_tok_stride,
                                      const void* v, int64_t v_tok_stride,
                                      const void* g_raw, int64_t g_tok_stride,
                                      const void* beta_raw, int64_t beta_tok_stride,
                                      const float* A_log, const float* dt_bias,
                                      float lower_bound, float scale, int32_t gate_mode,
                                      int32_t state_dtype,
                                      void* state_pool, int64_t num_slots, int64_t slot_stride,
                                      const int32_t* state_indices, int32_t use_initial_state,
                                      void* out, int64_t out_tok_stride,
                                      void* checkpoints, int64_t checkpoint_rows,
                                      const int64_t* checkpoint_cu_starts,
                                      int32_t checkpoint_interval,
                                      void* k_cache, void* u_cache, float* g_cache,
                                      int32_t ring_rows, const int32_t* cache_base,
                                      int32_t ring_tail, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
