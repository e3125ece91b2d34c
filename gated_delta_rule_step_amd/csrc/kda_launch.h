// Kernel parameter blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// gate_mode bits (kda.h): the gate input holds the log-decay itself; the beta
// input holds beta itself.
constexpr int32_t kGatePrecomputed = 1;
constexpr int32_t kBetaPresigmoid = 2;
constexpr int32_t kGatePerHead = 4;  // one gate value (and dt_bias) per head
// The kernels are compiled per gate kind: gate_mode & (kGatePrecomputed | kGatePerHead).
constexpr int32_t kGateKindMask = kGatePrecomputed | kGatePerHead;

// All strides in elements. bf16 tensors are uint16_t bit patterns.
struct DecodeParams {
  int32_t B, H;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  int64_t q_row_stride, k_row_stride, v_row_stride, g_row_stride, beta_row_stride;
  const float* A_log;
  const float* dt_bias;
  float lower_bound, scale;
  int32_t gate_mode;
  int32_t state_fmt;  // pool element format: kStateBf16, kStateFp16, kStateFp8
  void* state_pool;
  int64_t num_slots, slot_stride;
  const int32_t* state_indices;
  uint16_t* out;
  int64_t out_row_stride;
};

struct VerifyParams {
  int32_t B, T, H;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  int64_t q_row_stride, q_tok_stride, k_row_stride, k_tok_stride, v_row_stride, v_tok_stride;
  int64_t g_row_stride, g_tok_stride, beta_row_stride, beta_tok_stride;
  const float* A_log;
  const float* dt_bias;
  float lower_bound, scale;
  int32_t gate_mode;
  int32_t state_fmt;  // checkpoint element format (kStateBf16 ...); rings stay bf16
  void* state_pool;
  int64_t num_slots, slot_stride;
  const int32_t* state_indices;
  uint16_t* k_cache;
  uint16_t* u_cache;
  float* g_cache;
  int32_t ring_rows;
  const int32_t* hist_len;
  const int32_t* cache_base;
  int32_t flush_min, w_ring;
  uint16_t* out;
  int64_t out_row_stride, out_tok_stride;
};

struct PrefillParams {
  int32_t n_docs, H;
  int64_t total_tokens;
  const int32_t* cu_seqlens;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  int64_t q_tok_stride, k_tok_stride, v_tok_stride, g_tok_stride, beta_tok_stride;
  const float* A_log;
  const float* dt_bias;
  float lower_bound, scale;
  int32_t gate_mode;
  int32_t state_fmt;  // pool and checkpoint element format (kStateBf16 ...)
  void* state_pool;
  int64_t num_slots, slot_stride;
  const int32_t* state_indices;
  int32_t use_initial_state;
  uint16_t* out;
  int64_t out_tok_stride;
  void* ckpt;                  // NULL: no intermediate checkpoints
  int64_t ckpt_rows;
  const int64_t* ckpt_starts;  // [n_docs]
  int32_t ckpt_interval;       // tokens, a multiple of 16
  // hand-off to the verify ring: each active document's last
  // min(ring_tail, tokens of its last chunk) tokens become ring history rows
  // ([num_slots][H][ring_rows][128]) and the pool gets the state before them
  uint16_t* k_cache;
  uint16_t* u_cache;
  float* g_cache;
  int32_t ring_rows;
  const int32_t* cache_base;   // [n_docs]
  int32_t ring_tail;           // 0: no hand-off
  void* workspace;
};

hipError_t launch_decode(const DecodeParams& p, bool vec, hipStream_t stream);
hipError_t launch_verify(const VerifyParams& p, bool vec, hipStream_t stream);

// Prefill needs the host copy of cu_seqlens to plan its launches. Calls with
// at least kFusedMinChains (document, head) chains -- one per CU of the chip,
// a fixed count so that the workspace size does not depend on the device --
// run the fused 64-token kernel (no workspace); calls with fewer run the
// two-stage form (a preparation kernel over all 16-token chunks, then the
// chain), which needs a workspace.
constexpr int64_t kFusedMinChains = 256;
size_t prefill_workspace_bytes(int32_t n_docs, int64_t total_tokens, int32_t H);
hipError_t launch_prefill(const PrefillParams& p, const int32_t* cu_host, bool vec,
                          hipStream_t stream);
size_t prefill_split_workspace_bytes(int32_t n_docs, int64_t total_tokens, int32_t H);
hipError_t launch_prefill_split(const PrefillParams& p, const int32_t* cu_host, bool vec,
                                hipStream_t stream);

}  // namespace kda
