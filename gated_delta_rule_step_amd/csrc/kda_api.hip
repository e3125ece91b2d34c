// C ABI of the KDA step library: host-side validation, variant choice and
// kernel launch. Nothing here allocates or synchronises; the only state kept
// is the per-device address of the allocation-free prefill's scratch array.

#include <stdint.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_launch.h"
#include "kda_common.h"

// state_dtype values are the kernels' state format indices
static_assert(KDA_STATE_BF16 == kda::kStateBf16 && KDA_STATE_FP16 == kda::kStateFp16 &&
                  KDA_STATE_FP8 == kda::kStateFp8,
              "state format numbering");

namespace {

constexpr int64_t D = 128;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool mult8(int64_t s) { return (s & 7) == 0; }

// An output tensor indexed by (row, token) must not write one element twice:
// either row-major over tokens or token-major over rows.
bool out_layout_ok(int64_t rows, int64_t toks, int64_t row_stride, int64_t tok_stride,
                   int64_t width) {
  if (row_stride < 0 || tok_stride < 0) return false;
  const bool r_ok = rows <= 1 || row_stride >= width;
  const bool t_ok = toks <= 1 || tok_stride >= width;
  if (rows <= 1 || toks <= 1) return r_ok && t_ok;
  const bool row_major = tok_stride >= width && row_stride >= toks * tok_stride;
  const bool tok_major = row_stride >= width && tok_stride >= rows * row_stride;
  return row_major || tok_major;
}

kda_status launch_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH; }

// The gate input joins the vectorised-path test only when it is read as
// 128-channel rows (a per-head gate is one value per token and head).
bool gate_vec_ok(int32_t gate_mode, const void* g, int64_t s0, int64_t s1) {
  return (gate_mode & KDA_GATE_PER_HEAD) || (aligned16(g) && mult8(s0) && mult8(s1));
}

// gate_mode: only the two documented bits; the pre-computed gate clamps into
// [lower_bound, 0], so lower_bound must be <= 0 (not NaN) there. A_log and
// dt_bias are read only for raw gate logits.
kda_status check_gate(int32_t gate_mode, float lower_bound, const float* A_log,
                      const float* dt_bias) {
  if (gate_mode & ~(KDA_GATE_PRECOMPUTED | KDA_BETA_PRESIGMOID | KDA_GATE_PER_HEAD))
    return KDA_ERR_UNSUPPORTED;
  if (gate_mode & KDA_GATE_PRECOMPUTED) {
    if (!(lower_bound <= 0.0f)) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
  }
  return (A_log && dt_bias) ? KDA_OK : KDA_ERR_NULL_POINTER;
}

}  // namespace

extern "C" const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case KDA_ERR_BAD_SHAPE: return "invalid shape argument";
    case KDA_ERR_BAD_STRIDE: return "invalid stride argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
    case KDA_ERR_BAD_SEQLENS: return "cu_seqlens must start at 0, never decrease and end at total_tokens";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than kda_prefill_workspace_size()";
    case KDA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case KDA_ERR_SCRATCH_LIMIT:
      return "the call needs more workspace than the library's fixed scratch "
             "(KDA_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

extern "C" kda_status kda_decode(int32_t B, int32_t H, int32_t K, int32_t V, const void* q,
                                 int64_t q_row_stride, const void* k, int64_t k_row_stride,
                                 const void* v, int64_t v_row_stride, const void* g_raw,
                                 int64_t g_row_stride, const void* beta_raw,
                                 int64_t beta_row_stride, const float* A_log,
                                 const float* dt_bias, float lower_bound, float scale,
                                 int32_t gate_mode, int32_t state_dtype, void* state_pool,
                                 int64_t num_slots,
                                 int64_t slot_stride, const int32_t* state_indices, void* out,
                                 int64_t out_row_stride, hipStream_t stream) {
  if (B < 0 || H < 1 || num_slots < 0) return KDA_ERR_BAD_SHAPE;
  if (K != D || V != D) return KDA_ERR_UNSUPPORTED;
  if (state_dtype < KDA_STATE_BF16 || state_dtype > KDA_STATE_FP8) return KDA_ERR_UNSUPPORTED;
  if (const kda_status gs = check_gate(gate_mode, lower_bound, A_log, dt_bias)) {
    if (gs == KDA_ERR_UNSUPPORTED || B > 0) return gs;
  }
  if (B == 0) return KDA_OK;
  if (!q || !k || !v || !g_raw || !beta_raw || !state_indices || !out)
    return KDA_ERR_NULL_POINTER;
  if (num_slots > 0 && !state_pool) return KDA_ERR_NULL_POINTER;
  const int64_t W = int64_t(H) * D;
  if (q_row_stride < 0 || k_row_stride < 0 || v_row_stride < 0 || g_row_stride < 0 ||
      beta_row_stride < 0 || out_row_stride < 0 || slot_stride < 0)
    return KDA_ERR_BAD_STRIDE;
  if (B > 1 && out_row_stride < W) return KDA_ERR_BAD_STRIDE;
  if (num_slots > 1 && slot_stride < W * D) return KDA_ERR_BAD_STRIDE;

  kda::DecodeParams p;
  p.B = B;
  p.H = H;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = static_cast<const uint16_t*>(g_raw);
  p.beta = static_cast<const uint16_t*>(beta_raw);
  p.q_row_stride = q_row_stride;
  p.k_row_stride = k_row_stride;
  p.v_row_stride = v_row_stride;
  p.g_row_stride = g_row_stride;
  p.beta_row_stride = beta_row_stride;
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.lower_bound = lower_bound;
  p.scale = scale;
  p.gate_mode = gate_mode;
  p.state_fmt = state_dtype;  // kda_state_dtype values are the kernels' format indices
  p.state_pool = state_pool;
  p.num_slots = num_slots;
  p.slot_stride = slot_stride;
  p.state_indices = state_indices;
  p.out = static_cast<uint16_t*>(out);
  p.out_row_stride = out_row_stride;
  const bool vec = aligned16(q) && aligned16(k) &&
                   gate_vec_ok(gate_mode, g_raw, g_row_stride, 0) && aligned16(dt_bias) &&
                   (num_slots == 0 || aligned16(state_pool)) && mult8(q_row_stride) &&
                   mult8(k_row_stride) && mult8(slot_stride);
  // fp16 and fp8 states: the vectorised path only (16-byte aligned bases, strides in
  // multiples of 8)
  if (p.state_fmt != KDA_STATE_BF16 && !vec) return KDA_ERR_UNSUPPORTED;
  return launch_status(kda::launch_decode(p, vec, stream));
}

extern "C" kda_status kda_verify_ucache_flush(
    int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, const void* q, int64_t q_row_stride,
    int64_t q_tok_stride, const void* k, int64_t k_row_stride, int64_t k_tok_stride,
    const void* v, int64_t v_row_stride, int64_t v_tok_stride, const void* g_raw,
    int64_t g_row_stride, int64_t g_tok_stride, const void* beta_raw, int64_t beta_row_stride,
    int64_t beta_tok_stride, const float* A_log, const float* dt_bias, float lower_bound,
    float scale, int32_t gate_mode, int32_t state_dtype, void* state_pool, int64_t num_slots,
    int64_t slot_stride, const int32_t* state_indices, void* k_cache, void* u_cache, float* g_cache,
    int32_t ring_rows, const int32_t* hist_len, const int32_t* cache_base, int32_t flush_min,
    int32_t w_ring, int32_t restart_hist_on_flush, void* out, int64_t out_row_stride,
    int64_t out_tok_stride, hipStream_t stream) {
  if (B < 0 || H < 1 || num_slots < 0 || ring_rows < 1) return KDA_ERR_BAD_SHAPE;
  if (K != D || V != D || T < 1 || T > 8) return KDA_ERR_UNSUPPORTED;
  if (w_ring != 16 && w_ring != 32) return KDA_ERR_UNSUPPORTED;
  if (ring_rows < w_ring || restart_hist_on_flush != 1 || flush_min < 1) return KDA_ERR_UNSUPPORTED;
  if (flush_min - 1 + T > w_ring) return KDA_ERR_UNSUPPORTED;  // ring capacity
  if (w_ring == 32 && flush_min <= 16) return KDA_ERR_UNSUPPORTED;
  if (state_dtype < KDA_STATE_BF16 || state_dtype > KDA_STATE_FP8) return KDA_ERR_UNSUPPORTED;
  if (const kda_status gs = check_gate(gate_mode, lower_bound, A_log, dt_bias)) {
    if (gs == KDA_ERR_UNSUPPORTED || B > 0) return gs;
  }
  if (B == 0) return KDA_OK;
  if (!q || !k || !v || !g_raw || !beta_raw || !state_indices || !out || !hist_len ||
      !cache_base)
    return KDA_ERR_NULL_POINTER;
  if (num_slots > 0 && (!state_pool || !k_cache || !u_cache || !g_cache))
    return KDA_ERR_NULL_POINTER;
  const int64_t W = int64_t(H) * D;
  const int64_t in_strides[] = {q_row_stride, q_tok_stride, k_row_stride, k_tok_stride,
                                v_row_stride, v_tok_stride, g_row_stride, g_tok_stride,
                                beta_row_stride, beta_tok_stride, slot_stride};
  for (int64_t s : in_strides)
    if (s < 0) return KDA_ERR_BAD_STRIDE;
  if (!out_layout_ok(B, T, out_row_stride, out_tok_stride, W)) return KDA_ERR_BAD_STRIDE;
  if (num_slots > 1 && slot_stride < W * D) return KDA_ERR_BAD_STRIDE;

  kda::VerifyParams p;
  p.B = B;
  p.T = T;
  p.H = H;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = static_cast<const uint16_t*>(g_raw);
  p.beta = static_cast<const uint16_t*>(beta_raw);
  p.q_row_stride = q_row_stride;
  p.q_tok_stride = q_tok_stride;
  p.k_row_stride = k_row_stride;
  p.k_tok_stride = k_tok_stride;
  p.v_row_stride = v_row_stride;
  p.v_tok_stride = v_tok_stride;
  p.g_row_stride = g_row_stride;
  p.g_tok_stride = g_tok_stride;
  p.beta_row_stride = beta_row_stride;
  p.beta_tok_stride = beta_tok_stride;
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.lower_bound = lower_bound;
  p.scale = scale;
  p.gate_mode = gate_mode;
  p.state_fmt = state_dtype;  // kda_state_dtype values are the kernels' format indices
  p.state_pool = state_pool;
  p.num_slots = num_slots;
  p.slot_stride = slot_stride;
  p.state_indices = state_indices;
  p.k_cache = static_cast<uint16_t*>(k_cache);
  p.u_cache = static_cast<uint16_t*>(u_cache);
  p.g_cache = g_cache;
  p.ring_rows = ring_rows;
  p.hist_len = hist_len;
  p.cache_base = cache_base;
  p.flush_min = flush_min;
  p.w_ring = w_ring;
  p.out = static_cast<uint16_t*>(out);
  p.out_row_stride = out_row_stride;
  p.out_tok_stride = out_tok_stride;
  const bool vec = aligned16(q) && aligned16(k) && aligned16(v) &&
                   gate_vec_ok(gate_mode, g_raw, g_row_stride, g_tok_stride) &&
                   aligned16(dt_bias) && aligned16(out) &&
                   (num_slots == 0 || (aligned16(state_pool) && aligned16(k_cache) &&
                                       aligned16(u_cache) && aligned16(g_cache))) &&
                   mult8(q_row_stride) && mult8(q_tok_stride) && mult8(k_row_stride) &&
                   mult8(k_tok_stride) && mult8(v_row_stride) && mult8(v_tok_stride) &&
                   mult8(out_row_stride) && mult8(out_tok_stride) && mult8(slot_stride);
  // fp16 and fp8 states: the vectorised path only (16-byte aligned bases, strides in
  // multiples of 8)
  if (p.state_fmt != KDA_STATE_BF16 && !vec) return KDA_ERR_UNSUPPORTED;
  return launch_status(kda::launch_verify(p, vec, stream));
}

extern "C" size_t kda_prefill_workspace_size(int32_t n_docs, int64_t total_tokens, int32_t H,
                                             int32_t K, int32_t V) {
  if (n_docs < 0 || total_tokens < 0 || H < 1 || K != D || V != D) return 0;
  return kda::prefill_workspace_bytes(n_docs, total_tokens, H);
}

namespace {

kda_status prefill_impl(
    int32_t n_docs, int64_t total_tokens, int32_t H, int32_t K, int32_t V,
    const int32_t* cu_seqlens_host, const int32_t* cu_seqlens, const void* q,
    int64_t q_tok_stride, const void* k, int64_t k_tok_stride, const void* v,
    int64_t v_tok_stride, const void* g_raw, int64_t g_tok_stride, const void* beta_raw,
    int64_t beta_tok_stride, const float* A_log, const float* dt_bias, float lower_bound,
    float scale, int32_t gate_mode, int32_t state_dtype, void* state_pool, int64_t num_slots,
    int64_t slot_stride, const int32_t* state_indices, int32_t use_initial_state, void* out, int64_t out_tok_stride,
    void* checkpoints, int64_t checkpoint_rows, const int64_t* checkpoint_cu_starts,
    int32_t checkpoint_interval, void* k_cache, void* u_cache, float* g_cache, int32_t ring_rows,
    const int32_t* cache_base, int32_t ring_tail, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  if (n_docs < 0 || total_tokens < 0 || H < 1 || num_slots < 0) return KDA_ERR_BAD_SHAPE;
  if (K != D || V != D) return KDA_ERR_UNSUPPORTED;
  // 16-token chunks factor each decay weight into two exps of at most 8 |lb|.
  if (!(lower_bound >= -5.5f && lower_bound <= 5.5f)) return KDA_ERR_UNSUPPORTED;
  if (!cu_seqlens_host) return KDA_ERR_NULL_POINTER;
  if (cu_seqlens_host[0] != 0) return KDA_ERR_BAD_SEQLENS;
  for (int32_t d = 0; d < n_docs; ++d)
    if (cu_seqlens_host[d + 1] < cu_seqlens_host[d]) return KDA_ERR_BAD_SEQLENS;
  if (int64_t(cu_seqlens_host[n_docs]) != total_tokens) return KDA_ERR_BAD_SEQLENS;
  if (state_dtype < KDA_STATE_BF16 || state_dtype > KDA_STATE_FP8) return KDA_ERR_UNSUPPORTED;
  if (const kda_status gs = check_gate(gate_mode, lower_bound, A_log, dt_bias)) {
    if (gs == KDA_ERR_UNSUPPORTED || n_docs > 0) return gs;
  }
  if (checkpoints) {
    if (checkpoint_rows < 0) return KDA_ERR_BAD_SHAPE;
    // checkpoints sit on 16-token chunk boundaries
    if (checkpoint_interval < 16 || checkpoint_interval % 16 != 0) return KDA_ERR_UNSUPPORTED;
  }
  // the hand-off tail lies inside a document's last 16-token chunk
  if (ring_tail < 0 || ring_tail > 16) return KDA_ERR_UNSUPPORTED;
  if (ring_tail > 0 && ring_rows < ring_tail) return KDA_ERR_BAD_SHAPE;
  if (n_docs == 0) return KDA_OK;
  if (ring_tail > 0 && (!k_cache || !u_cache || !g_cache || !cache_base))
    return KDA_ERR_NULL_POINTER;
  if (!cu_seqlens || !state_indices) return KDA_ERR_NULL_POINTER;
  if (checkpoints && !checkpoint_cu_starts) return KDA_ERR_NULL_POINTER;
  if (total_tokens > 0 && (!q || !k || !v || !g_raw || !beta_raw || !out))
    return KDA_ERR_NULL_POINTER;
  if (num_slots > 0 && !state_pool) return KDA_ERR_NULL_POINTER;
  const int64_t W = int64_t(H) * D;
  if (q_tok_stride < 0 || k_tok_stride < 0 || v_tok_stride < 0 || g_tok_stride < 0 ||
      beta_tok_stride < 0 || out_tok_stride < 0 || slot_stride < 0)
    return KDA_ERR_BAD_STRIDE;
  // also for a single token: a chunk's padding rows must fall outside the
  // output rows it stores
  if (total_tokens >= 1 && out_tok_stride < W) return KDA_ERR_BAD_STRIDE;
  // a 16-token chunk of outputs is stored through one 32-bit buffer range
  if (out_tok_stride > (int64_t(1) << 25)) return KDA_ERR_UNSUPPORTED;
  if (num_slots > 1 && slot_stride < W * D) return KDA_ERR_BAD_STRIDE;
  const size_t need = kda::prefill_workspace_bytes(n_docs, total_tokens, H);
  if (workspace_bytes < need) return KDA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return workspace ? KDA_ERR_UNSUPPORTED : KDA_ERR_NULL_POINTER;

  kda::PrefillParams p;
  p.n_docs = n_docs;
  p.H = H;
  p.total_tokens = total_tokens;
  p.cu_seqlens = cu_seqlens;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = static_cast<const uint16_t*>(g_raw);
  p.beta = static_cast<const uint16_t*>(beta_raw);
  p.q_tok_stride = q_tok_stride;
  p.k_tok_stride = k_tok_stride;
  p.v_tok_stride = v_tok_stride;
  p.g_tok_stride = g_tok_stride;
  p.beta_tok_stride = beta_tok_stride;
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.lower_bound = lower_bound;
  p.scale = scale;
  p.gate_mode = gate_mode;
  p.state_fmt = state_dtype;  // kda_state_dtype values are the kernels' format indices
  p.state_pool = state_pool;
  p.num_slots = num_slots;
  p.slot_stride = slot_stride;
  p.state_indices = state_indices;
  p.use_initial_state = use_initial_state ? 1 : 0;
  p.out = static_cast<uint16_t*>(out);
  p.out_tok_stride = out_tok_stride;
  p.ckpt = checkpoints;
  p.ckpt_rows = checkpoints ? checkpoint_rows : 0;
  p.ckpt_starts = checkpoint_cu_starts;
  p.ckpt_interval = checkpoints ? checkpoint_interval : 16;
  p.k_cache = static_cast<uint16_t*>(k_cache);
  p.u_cache = static_cast<uint16_t*>(u_cache);
  p.g_cache = g_cache;
  p.ring_rows = ring_tail > 0 ? ring_rows : 0;
  p.cache_base = cache_base;
  p.ring_tail = ring_tail;
  p.workspace = workspace;
  const bool vec = aligned16(q) && aligned16(k) && aligned16(v) &&
                   gate_vec_ok(gate_mode, g_raw, g_tok_stride, 0) && aligned16(dt_bias) &&
                   aligned16(out) && (num_slots == 0 || aligned16(state_pool)) &&
                   aligned16(checkpoints) && mult8(q_tok_stride) && mult8(k_tok_stride) &&
                   mult8(v_tok_stride) && mult8(out_tok_stride) && mult8(slot_stride);
  // fp16 and fp8 states: the vectorised path only (16-byte aligned bases, strides in
  // multiples of 8)
  if (p.state_fmt != KDA_STATE_BF16 && !vec) return KDA_ERR_UNSUPPORTED;
  return launch_status(kda::launch_prefill(p, cu_seqlens_host, vec, stream));
}

// Scratch of kda_prefill_varlen_noalloc: one copy per device, created when the
// library's code object is loaded there and held until the process ends. Host
// code never uses the symbol itself as an address (on the host it names a
// stand-in): each device's address comes from hipGetSymbolAddress, taken once
// with that device current and kept in scratch_addr.
constexpr size_t kScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices];

// The current device's scratch address (looked up on its first call).
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    scratch_addr[dev] = ptr;
  }
  *out = scratch_addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" kda_status kda_prefill_varlen(
    int32_t n_docs, int64_t total_tokens, int32_t H, int32_t K, int32_t V,
    const int32_t* cu_seqlens_host, const int32_t* cu_seqlens, const void* q,
    int64_t q_tok_stride, const void* k, int64_t k_tok_stride, const void* v,
    int64_t v_tok_stride, const void* g_raw, int64_t g_tok_stride, const void* beta_raw,
    int64_t beta_tok_stride, const float* A_log, const float* dt_bias, float lower_bound,
    float scale, int32_t gate_mode, int32_t state_dtype, void* state_pool, int64_t num_slots,
    int64_t slot_stride, const int32_t* state_indices, int32_t use_initial_state, void* out,
    int64_t out_tok_stride, void* checkpoints, int64_t checkpoint_rows,
    const int64_t* checkpoint_cu_starts, int32_t checkpoint_interval, void* k_cache,
    void* u_cache, float* g_cache, int32_t ring_rows, const int32_t* cache_base,
    int32_t ring_tail, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return prefill_impl(n_docs, total_tokens, H, K, V, cu_seqlens_host, cu_seqlens, q,
                      q_tok_stride, k, k_tok_stride, v, v_tok_stride, g_raw, g_tok_stride,
                      beta_raw, beta_tok_stride, A_log, dt_bias, lower_bound, scale, gate_mode,
                      state_dtype, state_pool, num_slots, slot_stride, state_indices,
                      use_initial_state, out, out_tok_stride, checkpoints, checkpoint_rows,
                      checkpoint_cu_starts, checkpoint_interval, k_cache, u_cache, g_cache,
                      ring_rows, cache_base, ring_tail, workspace, workspace_bytes, stream);
}

extern "C" kda_status kda_prefill_varlen_noalloc(
    int32_t n_docs, int64_t total_tokens, int32_t H, int32_t K, int32_t V,
    const int32_t* cu_seqlens_host, const int32_t* cu_seqlens, const void* q,
    int64_t q_tok_stride, const void* k, int64_t k_tok_stride, const void* v,
    int64_t v_tok_stride, const void* g_raw, int64_t g_tok_stride, const void* beta_raw,
    int64_t beta_tok_stride, const float* A_log, const float* dt_bias, float lower_bound,
    float scale, int32_t gate_mode, int32_t state_dtype, void* state_pool, int64_t num_slots,
    int64_t slot_stride, const int32_t* state_indices, int32_t use_initial_state, void* out,
    int64_t out_tok_stride, void* checkpoints, int64_t checkpoint_rows,
    const int64_t* checkpoint_cu_starts, int32_t checkpoint_interval, void* k_cache,
    void* u_cache, float* g_cache, int32_t ring_rows, const int32_t* cache_base,
    int32_t ring_tail, hipStream_t stream) {
  if (n_docs < 0 || total_tokens < 0 || H < 1) return KDA_ERR_BAD_SHAPE;
  if (K != D || V != D) return KDA_ERR_UNSUPPORTED;
  const size_t need = kda::prefill_workspace_bytes(n_docs, total_tokens, H);
  if (need > kScratchBytes) return KDA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return KDA_ERR_LAUNCH;
  return prefill_impl(n_docs, total_tokens, H, K, V, cu_seqlens_host, cu_seqlens, q,
                      q_tok_stride, k, k_tok_stride, v, v_tok_stride, g_raw, g_tok_stride,
                      beta_raw, beta_tok_stride, A_log, dt_bias, lower_bound, scale, gate_mode,
                      state_dtype, state_pool, num_slots, slot_stride, state_indices,
                      use_initial_state, out, out_tok_stride, checkpoints, checkpoint_rows,
                      checkpoint_cu_starts, checkpoint_interval, k_cache, u_cache, g_cache,
                      ring_rows, cache_base, ring_tail, ws, kScratchBytes, stream);
}
