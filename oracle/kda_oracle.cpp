// CPU oracle for the KDA gated delta-rule step.
//
// TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
// benchmark's CPU-baseline leg load this library. The GPU library never links
// it, and it includes no header and no helper of the GPU library.
//
// Plain, slow, obviously-correct loops. Every routine is a function template
// on the arithmetic type Real (float is the parity target, double serves the
// invariant and drift checks). All arrays are dense and hold values of type
// Real; a bf16 tensor is passed as Real values that happen to be
// bf16-representable. When `bf16_storage` is non-zero, values are rounded to
// bf16 (round-to-nearest-even) exactly where the GPU path stores bf16: every
// output o, a decode state write-back, ring k-hat and u rows, a fold
// checkpoint, and a prefill final state. Nothing else is rounded.
//
// State layout (a reading; the pages fix only the shape [N, H, 128, 128]): one
// head's state S is a V x K matrix stored row-major, element (v, k) at
// v*K + k. With S in that orientation the pages' correction term
// u = beta * (v - S k_hat) is an ordinary matrix-vector product
// ("feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3 (KDA)",
// section "Caching").
//
// Parallelism: OpenMP over independent (row, head) or (document, head) units
// only; every unit runs the plain sequential loops below.
//
// Pins: each function is checked by the CPU test suite against brute force,
// closed forms and invariants. The gate formula, the L2-norm epsilon and the
// ring addressing are readings of the pages and are "parity unpinned" beyond
// the invariants listed with each function.

#include <algorithm>
#include <cmath>
#include <limits>
#include <cstdint>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// ---------------------------------------------------------------------------
// bf16 round-to-nearest-even from binary32. The pages store every bf16 value
// with round-to-nearest-even ("feat(kda): add packed-input CuTe decode
// kernel", section "Kernel design", bf16 register economy). Written from the
// IEEE-754 definition: keep the top 16 bits, rounding on the 16 dropped bits
// with ties going to the even result; NaN stays NaN (quieted).
uint16_t bf16_rne_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) {  // NaN: keep sign and payload top, force quiet
    return static_cast<uint16_t>((u >> 16) | 0x0040u);
  }
  const uint32_t upper = u >> 16;
  const uint32_t lower = u & 0xffffu;
  uint32_t r = upper;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) r += 1;  // carries into exponent as needed
  return static_cast<uint16_t>(r);
}

float bf16_bits_to_float(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Round a Real to the nearest bf16 value. For Real = double the value is first
// rounded to binary32 (nearest-even), then to bf16; this double rounding only
// matters for the drift diagnostic, never for the fp32 parity target.
template <class Real>
Real to_bf16(Real x) {
  return static_cast<Real>(bf16_bits_to_float(bf16_rne_bits(static_cast<float>(x))));
}

template <class Real>
Real store(Real x, int bf16_storage) {
  return bf16_storage ? to_bf16(x) : x;
}

// ---------------------------------------------------------------------------
// binary16 (fp16) round-to-nearest-even from binary32, for the fp16 state
// option (the pages' GDN kernel offers "an optional fp16 checkpoint-state
// mode"; "feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3 (KDA)",
// "Caching"). Written from the IEEE-754 binary16 format: 1 sign, 5 exponent
// (bias 15) and 10 fraction bits; values from 65520 up overflow to infinity;
// below 2^-14 the result is a subnormal m * 2^-24; ties go to the even result.
uint16_t f16_rne_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return static_cast<uint16_t>(sign | 0x7e00u | ((a >> 13) & 0x3ffu));
  if (a >= 0x477ff000u) return static_cast<uint16_t>(sign | 0x7c00u);  // 65520 and up: inf
  uint32_t r;
  if (a >= 0x38800000u) {  // normal binary16
    const uint32_t e = (a >> 23) - 127 + 15;
    const uint32_t m = a & 0x7fffffu;
    r = (e << 10) | (m >> 13);
    const uint32_t rem = m & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) r += 1;  // may carry into the exponent
  } else {
    const uint32_t e = a >> 23;
    if (e == 0) return static_cast<uint16_t>(sign);  // binary32 subnormal: far below 2^-25
    const uint32_t m = (a & 0x7fffffu) | 0x800000u;  // value = m * 2^(e - 150)
    const uint32_t shift = 126 - e;                  // value * 2^24 = m >> shift
    if (shift > 24) return static_cast<uint16_t>(sign);  // below 2^-25: rounds to zero
    r = m >> shift;
    const uint32_t rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (r & 1u))) r += 1;  // 1024 is the smallest normal
  }
  return static_cast<uint16_t>(sign | r);
}

float f16_bits_to_float(uint16_t b) {
  const uint32_t sign = static_cast<uint32_t>(b & 0x8000u) << 16;
  const uint32_t e = (b >> 10) & 0x1fu, m = b & 0x3ffu;
  float f;
  if (e == 0) {
    f = std::ldexp(static_cast<float>(m), -24);
  } else if (e == 31) {
    const uint32_t u = 0x7f800000u | (m << 13);
    std::memcpy(&f, &u, 4);
  } else {
    const uint32_t u = ((e - 15 + 127) << 23) | (m << 13);
    std::memcpy(&f, &u, 4);
  }
  uint32_t v;
  std::memcpy(&v, &f, 4);
  v |= sign;
  std::memcpy(&f, &v, 4);
  return f;
}

// ---------------------------------------------------------------------------
// FP8 E4M3 (the OCP 8-bit format "e4m3fn": 1 sign, 4 exponent bits with bias
// 7, 3 fraction bits; no infinities, S.1111.111 is NaN, so the largest finite
// value is 448 = 1.75 * 2^8; below 2^-6 the value is a subnormal m * 2^-9)
// for the fp8 state option, the byte reduction the decode page names as the
// remaining lever ("feat(kda): add packed-input CuTe decode kernel"). Written
// from that definition: round to nearest, ties to even; magnitudes beyond 448
// saturate to 448 (a reading: a stored state must stay finite).
uint8_t f8_rne_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  const uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return static_cast<uint8_t>(sign | 0x7fu);  // NaN
  if (a > 0x43e00000u) a = 0x43e00000u;                              // saturate at 448
  uint32_t r;
  if (a >= 0x3c800000u) {  // normal: |x| >= 2^-6
    const uint32_t e = (a >> 23) - 127 + 7;
    const uint32_t m = a & 0x7fffffu;
    r = (e << 3) | (m >> 20);
    const uint32_t rem = m & 0xfffffu, half = 0x80000u;
    if (rem > half || (rem == half && (r & 1u))) r += 1;  // may carry into the exponent
  } else {
    const uint32_t e = a >> 23;
    if (e == 0) return static_cast<uint8_t>(sign);  // binary32 subnormal: rounds to zero
    const uint32_t m = (a & 0x7fffffu) | 0x800000u;  // value = m * 2^(e - 150)
    const uint32_t shift = 141 - e;                  // value * 2^9 = m >> shift
    if (shift > 24) return static_cast<uint8_t>(sign);  // below 2^-10: rounds to zero
    r = m >> shift;
    const uint32_t rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (r & 1u))) r += 1;  // 8 is the smallest normal
  }
  return static_cast<uint8_t>(sign | r);
}

float f8_bits_to_float(uint8_t b) {
  const uint32_t e = (b >> 3) & 0xfu, m = b & 0x7u;
  float f;
  if (e == 15 && m == 7) {
    f = std::numeric_limits<float>::quiet_NaN();
  } else if (e == 0) {
    f = std::ldexp(static_cast<float>(m), -9);
  } else {
    f = std::ldexp(static_cast<float>(8 + m), static_cast<int>(e) - 10);
  }
  return (b & 0x80u) ? -f : f;
}

// State storage points (pool write-back, fold checkpoint, prefill final and
// intermediate states): bf16 (state_dtype 0), fp16 (1) or fp8 e4m3 (2).
template <class Real>
Real store_state(Real x, int bf16_storage, int state_dtype) {
  if (!bf16_storage) return x;
  if (state_dtype == 1)
    return static_cast<Real>(f16_bits_to_float(f16_rne_bits(static_cast<float>(x))));
  if (state_dtype == 2)
    return static_cast<Real>(f8_bits_to_float(f8_rne_bits(static_cast<float>(x))));
  return to_bf16(x);
}

// ---------------------------------------------------------------------------
// Per-token prologue for one head.
//
// * L2 normalisation of q and k over the K key channels, in the working
//   precision ("feat(kda): add packed-input CuTe decode kernel", section "T=1
//   fast path inside recurrent_kda": in-kernel QK L2 norm). Reading: the
//   epsilon 1e-6 sits inside the square root.
// * Gate: the raw per-channel gate logit, the per-channel dt_bias and the
//   per-head A_log give the log-decay
//       g_c = max(lower_bound, -exp(A_log) * softplus(graw_c + dt_bias_c)),
//   which always lies in [lower_bound, 0]. The pages name the inputs (A_log,
//   dt_bias, lower_bound = -5, decay computed in fp32) but print no formula
//   (same page and section; "feat(kda): ReplaySSM verify+flush decode kernel
//   for Kimi K3 (KDA)", section "API"). Reading: the Mamba-style softplus gate
//   clamped at lower_bound. softplus(x) = log1p(exp(x)), or x when x > 20.
// * beta = sigmoid(beta logit) (beta_is_logit in the fast-path section).
// * gate_mode (same page, same section: the raw form, where the kernel computes
//   the decay and the sigmoid, and the API-default pre-computed form, log-space
//   g and pre-sigmoided beta, with decay = exp(g)):
//     bit 0 (pre-computed gate): graw holds the log-decay itself; it is used
//       clamped into [lower_bound, 0], the range the raw gate lands in
//       (reading); a_log and dt_bias are not read and may be null;
//     bit 1 (pre-sigmoided beta): beta_logit holds beta itself;
//     bit 2 (per-head gate, the scalar decay of GDN, which that page contrasts
//       with KDA's per-key-channel gate): graw holds one value per head and
//       dt_bias one per head; the resulting log-decay applies to every key
//       channel (reading: the same gate formula on the per-head inputs).
constexpr int kGatePrecomputed = 1;
constexpr int kBetaPresigmoid = 2;
constexpr int kGatePerHead = 4;

template <class Real>
void prologue(int K, const Real* q, const Real* k, const Real* graw, Real beta_logit,
              Real a_log, const Real* dt_bias, Real lower_bound, int gate_mode,
              Real* qh, Real* kh, Real* g, Real* beta) {
  Real sq = 0, sk = 0;
  for (int c = 0; c < K; ++c) {
    sq += q[c] * q[c];
    sk += k[c] * k[c];
  }
  const Real nq = std::sqrt(sq + static_cast<Real>(1e-6));
  const Real nk = std::sqrt(sk + static_cast<Real>(1e-6));
  for (int c = 0; c < K; ++c) {
    qh[c] = q[c] / nq;
    kh[c] = k[c] / nk;
  }
  const bool per_head = gate_mode & kGatePerHead;
  if (gate_mode & kGatePrecomputed) {
    for (int c = 0; c < K; ++c) {
      const Real gc = per_head ? graw[0] : graw[c];
      g[c] = std::min(static_cast<Real>(0), std::max(lower_bound, gc));
    }
  } else {
    const Real ea = std::exp(a_log);
    for (int c = 0; c < K; ++c) {
      const Real x = per_head ? graw[0] + dt_bias[0] : graw[c] + dt_bias[c];
      const Real sp = x > static_cast<Real>(20) ? x : std::log1p(std::exp(x));
      g[c] = std::max(lower_bound, -ea * sp);
    }
  }
  *beta = (gate_mode & kBetaPresigmoid)
              ? beta_logit
              : static_cast<Real>(1) / (static_cast<Real>(1) + std::exp(-beta_logit));
}

// The per-head gate parameters, or nothing in the pre-computed gate mode.
template <class Real>
Real alog_of(const Real* a_log, int h, int gate_mode) {
  return (gate_mode & kGatePrecomputed) ? static_cast<Real>(0) : a_log[h];
}
template <class Real>
const Real* dtb_of(const Real* dt_bias, int h, int K, int gate_mode) {
  if (gate_mode & kGatePrecomputed) return nullptr;
  return dt_bias + static_cast<int64_t>(h) * ((gate_mode & kGatePerHead) ? 1 : K);
}
// Gate values per token and head: K per-channel values, or one per head.
inline int gate_width(int K, int gate_mode) { return (gate_mode & kGatePerHead) ? 1 : K; }

// ---------------------------------------------------------------------------
// One gated delta-rule step for one head, the plain definition, in the order
// the method states it (north-star statement of the step; "feat(kda):
// ReplaySSM verify+flush decode kernel for Kimi K3 (KDA)", section "Caching",
// for u):
//   S' = diag(exp(g)) S        (decay per key channel)
//   u  = beta * (v - S' k_hat) (correction; S' k_hat is S'^T k_hat in K x V terms)
//   S  = S' + k_hat u^T        (rank-1 update)
//   o  = scale * S q_hat       (read-out from the updated state)
// S is V x K row-major (see the header). u may be null.
template <class Real>
void step(int K, int V, Real* S, const Real* qh, const Real* kh, const Real* vv,
          const Real* g, Real beta, Real scale, Real* o, Real* u_out) {
  std::vector<Real> alpha(K), u(V);
  for (int c = 0; c < K; ++c) alpha[c] = std::exp(g[c]);
  for (int r = 0; r < V; ++r)
    for (int c = 0; c < K; ++c) S[r * K + c] *= alpha[c];
  for (int r = 0; r < V; ++r) {
    Real d = 0;
    for (int c = 0; c < K; ++c) d += S[r * K + c] * kh[c];
    u[r] = beta * (vv[r] - d);
  }
  for (int r = 0; r < V; ++r)
    for (int c = 0; c < K; ++c) S[r * K + c] += kh[c] * u[r];
  for (int r = 0; r < V; ++r) {
    Real d = 0;
    for (int c = 0; c < K; ++c) d += S[r * K + c] * qh[c];
    o[r] = scale * d;
  }
  if (u_out)
    for (int r = 0; r < V; ++r) u_out[r] = u[r];
}

inline bool slot_active(int32_t idx, int64_t num_slots) {
  return idx >= 0 && static_cast<int64_t>(idx) < num_slots;
}

int64_t i64(int x) { return static_cast<int64_t>(x); }

// ---------------------------------------------------------------------------
// T = 1 serving decode against an in-place state pool ("feat(kda): add
// packed-input CuTe decode kernel", opening description): a row whose state
// index lies outside [0, N) writes zero output and leaves the pool untouched;
// an empty pool makes every row inactive.
//
// q, k, graw: [B][H][K]; v: [B][H][V]; beta_logit: [B][H]; a_log: [H];
// dt_bias: [H*K]; pool: [N][H][V][K]; idx: [B]; out: [B][H][V].
template <class Real>
void decode(int B, int H, int K, int V, const Real* q, const Real* k, const Real* v,
            const Real* graw, const Real* beta_logit, const Real* a_log, const Real* dt_bias,
            Real lower_bound, Real scale, Real* pool, int64_t N, const int32_t* idx,
            Real* out, int bf16_storage, int gate_mode, int state_dtype) {
  const int64_t KV = i64(K) * V;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      Real* o = out + (i64(b) * H + h) * V;
      if (!slot_active(idx[b], N)) {
        for (int r = 0; r < V; ++r) o[r] = 0;
        continue;
      }
      const int64_t tk = (i64(b) * H + h) * K;
      const int64_t tg = (i64(b) * H + h) * gate_width(K, gate_mode);
      std::vector<Real> qh(K), kh(K), g(K), S(KV);
      Real beta;
      prologue<Real>(K, q + tk, k + tk, graw + tg, beta_logit[i64(b) * H + h],
                     alog_of(a_log, h, gate_mode), dtb_of(dt_bias, h, K, gate_mode),
                     lower_bound, gate_mode, qh.data(), kh.data(), g.data(), &beta);
      Real* slot = pool + (i64(idx[b]) * H + h) * KV;
      std::copy(slot, slot + KV, S.begin());
      step<Real>(K, V, S.data(), qh.data(), kh.data(), v + (i64(b) * H + h) * V, g.data(),
                 beta, scale, o, nullptr);
      for (int64_t e = 0; e < KV; ++e) slot[e] = store_state(S[e], bf16_storage, state_dtype);
      for (int r = 0; r < V; ++r) o[r] = store(o[r], bf16_storage);
    }
  }
}

// ---------------------------------------------------------------------------
// Ring replay ("feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3
// (KDA)", sections "What it does" and "Caching"): a checkpoint S_ckpt plus
// `hist` history entries (k_hat_j, u_j, G_j), where G_j is the cumulative
// log-decay of tokens 0..j since the checkpoint, stands for the state
//   S_cur = diag(exp(G_L)) S_ckpt + sum_j diag(exp(G_L - G_j)) k_hat_j u_j^T,
// G_L = G_{hist-1}; in the V x K orientation element (v, c) is
//   exp(G_L[c]) S_ckpt[v][c] + sum_j exp(G_L[c] - G_j[c]) k_hat_j[c] u_j[v].
// The replay weight exp(G_L - G_j) is the pages' w_j = exp(G_P - G_j).
// History entry j lives in ring row (base + j) mod R (reading).
template <class Real>
void replay(int K, int V, const Real* ckpt, const Real* kc, const Real* uc, const Real* gc,
            int R, int base, int hist, Real* S) {
  const int64_t KV = i64(K) * V;
  if (hist == 0) {
    std::copy(ckpt, ckpt + KV, S);
    return;
  }
  const Real* GL = gc + i64((base + hist - 1) % R) * K;
  for (int r = 0; r < V; ++r)
    for (int c = 0; c < K; ++c) S[r * K + c] = std::exp(GL[c]) * ckpt[r * K + c];
  for (int j = 0; j < hist; ++j) {
    const int64_t row = (base + j) % R;
    const Real* kj = kc + row * K;
    const Real* uj = uc + row * V;
    const Real* Gj = gc + row * K;
    for (int r = 0; r < V; ++r)
      for (int c = 0; c < K; ++c) S[r * K + c] += std::exp(GL[c] - Gj[c]) * kj[c] * uj[r];
  }
}

// ---------------------------------------------------------------------------
// Speculative-decode verify with the (k_hat, u, G) ring and the fold into the
// checkpoint ("feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3
// (KDA)", sections "What it does", "API", "Caching"). The pages give names and
// fragments; the contract below is the plainest consistent reading:
//  * a row is active iff 0 <= idx < N, 0 <= hist, hist + T <= w_ring and
//    0 <= base < R; an inactive row writes zero outputs and nothing else;
//  * fold = (hist + T >= flush_min);
//  * S_cur = replay(checkpoint, history rows 0..hist-1);
//  * draft token t steps from S_cur in order: o_t is the read-out after
//    token t; ring row (base + hist + t) mod R receives k_hat_t, u_t and the
//    cumulative log-decay, which starts at 0 when folding
//    (restart_hist_on_flush) and at G_{hist-1} otherwise (0 when hist = 0),
//    and adds g_t channel-wise in token order;
//  * when folding, the checkpoint receives S_cur (the state before the draft
//    tokens).
// q, k, graw: [B][T][H][K]; v: [B][T][H][V]; beta_logit: [B][T][H];
// pool: [N][H][V][K]; kc, gc: [N][H][R][K]; uc: [N][H][R][V];
// hist, base: [B]; out: [B][T][H][V].
template <class Real>
void verify(int B, int T, int H, int K, int V, const Real* q, const Real* k, const Real* v,
            const Real* graw, const Real* beta_logit, const Real* a_log, const Real* dt_bias,
            Real lower_bound, Real scale, Real* pool, int64_t N, const int32_t* idx, Real* kc,
            Real* uc, Real* gc, int R, const int32_t* hist_len, const int32_t* cache_base,
            int flush_min, int w_ring, Real* out, int bf16_storage, int gate_mode,
            int state_dtype) {
  const int64_t KV = i64(K) * V;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const int hist = hist_len[b], base = cache_base[b];
      // hist <= w_ring - T: the sum hist + T would overflow for hist near INT32_MAX
      const bool active = slot_active(idx[b], N) && hist >= 0 && hist <= w_ring - T &&
                          base >= 0 && base < R;
      if (!active) {
        for (int t = 0; t < T; ++t)
          for (int r = 0; r < V; ++r) out[((i64(b) * T + t) * H + h) * V + r] = 0;
        continue;
      }
      const int64_t sh = i64(idx[b]) * H + h;
      Real* ckpt = pool + sh * KV;
      Real* kcs = kc + sh * R * K;
      Real* ucs = uc + sh * R * V;
      Real* gcs = gc + sh * R * K;
      std::vector<Real> S(KV), Scur(KV);
      replay<Real>(K, V, ckpt, kcs, ucs, gcs, R, base, hist, Scur.data());
      S = Scur;
      const bool fold = hist + T >= flush_min;
      std::vector<Real> G(K, static_cast<Real>(0));
      if (!fold && hist > 0) {
        const Real* GL = gcs + i64((base + hist - 1) % R) * K;
        for (int c = 0; c < K; ++c) G[c] = GL[c];
      }
      std::vector<Real> qh(K), kh(K), g(K), u(V);
      for (int t = 0; t < T; ++t) {
        const int64_t tk = ((i64(b) * T + t) * H + h) * K;
        const int64_t tv = ((i64(b) * T + t) * H + h) * V;
        const int64_t tg = ((i64(b) * T + t) * H + h) * gate_width(K, gate_mode);
        Real beta;
        prologue<Real>(K, q + tk, k + tk, graw + tg, beta_logit[(i64(b) * T + t) * H + h],
                       alog_of(a_log, h, gate_mode), dtb_of(dt_bias, h, K, gate_mode),
                       lower_bound, gate_mode, qh.data(), kh.data(), g.data(), &beta);
        Real* o = out + tv;
        step<Real>(K, V, S.data(), qh.data(), kh.data(), v + tv, g.data(), beta, scale, o,
                   u.data());
        for (int r = 0; r < V; ++r) o[r] = store(o[r], bf16_storage);
        const int64_t row = (base + hist + t) % R;
        for (int c = 0; c < K; ++c) {
          G[c] += g[c];
          kcs[row * K + c] = store(kh[c], bf16_storage);
          gcs[row * K + c] = G[c];
        }
        for (int r = 0; r < V; ++r) ucs[row * V + r] = store(u[r], bf16_storage);
      }
      if (fold)
        for (int64_t e = 0; e < KV; ++e) ckpt[e] = store_state(Scur[e], bf16_storage, state_dtype);
    }
  }
}

// ---------------------------------------------------------------------------
// Varlen prefill, token by token ("feat(kda): add CuTe DSL recurrent prefill
// backend": packed documents delimited by cu_seqlens, which starts at 0 and
// never decreases; zero-length documents allowed; optional initial state and
// final state). Each (document, head) chain starts from its pool slot
// (use_initial_state != 0) or from zeros, steps through the document's tokens
// in order, writes every output, and writes the final state into the slot. A
// document whose slot index is outside [0, N) writes zero outputs and leaves
// the pool untouched. A zero-length document with an initial state writes
// nothing.
// Intermediate checkpoints (same page: the prefill returns "output, final
// state, checkpoints", with checkpoint_cu_starts, int64; the positions are a
// reading): when ckpt is not null, an active document also stores its state
// after its first i * interval tokens, i = 1 .. floor(len / interval), into
// checkpoint row ckpt_starts[d] + i - 1 (rows outside [0, ckpt_rows) are
// skipped), rounded like the final state.
// Hand-off to speculative decoding (a reading: the prefill leaves each
// document in the form the verify step resumes from, a checkpoint plus ring
// history, as in "feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3
// (KDA)", "Caching"): with ring_tail > 0 an active document of length len hands
// its last r = min(ring_tail, len - 16 * floor((len - 1) / 16)) tokens (at most
// the tokens after its last 16-token boundary, the prefill's chunk) to the
// ring: the slot receives the state after the first len - r tokens, and tail
// token j = 0 .. r-1 writes history entry j into ring row (cache_base[d] + j)
// mod R of the slot: k_hat, u (the token's correction) and G, the cumulative
// log-decay of tail tokens 0..j. Outputs are unchanged; checkpoints only cover
// the first len - r tokens. A document whose cache_base lies outside [0, R) is
// inactive when ring_tail > 0.
// q, k, graw: [Ttot][H][K]; v: [Ttot][H][V]; beta_logit: [Ttot][H];
// cu: [n_docs + 1]; idx: [n_docs]; pool: [N][H][V][K]; out: [Ttot][H][V];
// ckpt: [ckpt_rows][H][V][K]; ckpt_starts: [n_docs]; kc, gc: [N][H][R][K];
// uc: [N][H][R][V]; cache_base: [n_docs].
template <class Real>
void prefill_tbt(int n_docs, int H, int K, int V, const int32_t* cu, const Real* q,
                 const Real* k, const Real* v, const Real* graw, const Real* beta_logit,
                 const Real* a_log, const Real* dt_bias, Real lower_bound, Real scale,
                 Real* pool, int64_t N, const int32_t* idx, int use_initial_state, Real* out,
                 int bf16_storage, int gate_mode, Real* ckpt, int64_t ckpt_rows,
                 const int64_t* ckpt_starts, int interval, int state_dtype, Real* kc, Real* uc,
                 Real* gc, int R, const int32_t* cache_base, int ring_tail) {
  const int64_t KV = i64(K) * V;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int d = 0; d < n_docs; ++d) {
    for (int h = 0; h < H; ++h) {
      const int t0 = cu[d], t1 = cu[d + 1];
      const int len = t1 - t0;
      const bool ring_ok = ring_tail == 0 || (cache_base[d] >= 0 && cache_base[d] < R);
      if (!slot_active(idx[d], N) || !ring_ok) {
        for (int t = t0; t < t1; ++t)
          for (int r = 0; r < V; ++r) out[(i64(t) * H + h) * V + r] = 0;
        continue;
      }
      Real* slot = pool + (i64(idx[d]) * H + h) * KV;
      if (t1 == t0 && use_initial_state) continue;
      const int last = len > 0 ? len - 16 * ((len - 1) / 16) : 0;
      const int tail = std::min(ring_tail, last);
      const int kept = len - tail;  // tokens whose state the slot receives
      std::vector<Real> S(KV, static_cast<Real>(0));
      if (use_initial_state) std::copy(slot, slot + KV, S.begin());
      if (kept == 0)
        for (int64_t e = 0; e < KV; ++e) slot[e] = store_state(S[e], bf16_storage, state_dtype);
      std::vector<Real> qh(K), kh(K), g(K), u(V), G(K, static_cast<Real>(0));
      for (int t = t0; t < t1; ++t) {
        const int64_t tk = (i64(t) * H + h) * K;
        const int64_t tg = (i64(t) * H + h) * gate_width(K, gate_mode);
        Real beta;
        prologue<Real>(K, q + tk, k + tk, graw + tg, beta_logit[i64(t) * H + h],
                       alog_of(a_log, h, gate_mode), dtb_of(dt_bias, h, K, gate_mode),
                       lower_bound, gate_mode, qh.data(), kh.data(), g.data(), &beta);
        Real* o = out + (i64(t) * H + h) * V;
        step<Real>(K, V, S.data(), qh.data(), kh.data(), v + (i64(t) * H + h) * V, g.data(),
                   beta, scale, o, u.data());
        for (int r = 0; r < V; ++r) o[r] = store(o[r], bf16_storage);
        const int done = t - t0 + 1;  // tokens of the document consumed
        if (ckpt && done % interval == 0 && done <= kept) {
          const int64_t row = ckpt_starts[d] + done / interval - 1;
          if (row >= 0 && row < ckpt_rows) {
            Real* c = ckpt + (row * H + h) * KV;
            for (int64_t e = 0; e < KV; ++e) c[e] = store_state(S[e], bf16_storage, state_dtype);
          }
        }
        if (done == kept)
          for (int64_t e = 0; e < KV; ++e) slot[e] = store_state(S[e], bf16_storage, state_dtype);
        if (done > kept) {  // a tail token: ring history entry done - kept - 1
          const int64_t sh = i64(idx[d]) * H + h;
          const int64_t row = (cache_base[d] + (done - kept - 1)) % R;
          Real* kr = kc + (sh * R + row) * K;
          Real* gr = gc + (sh * R + row) * K;
          Real* ur = uc + (sh * R + row) * V;
          for (int c = 0; c < K; ++c) {
            G[c] += g[c];
            kr[c] = store(kh[c], bf16_storage);
            gr[c] = G[c];
          }
          for (int r = 0; r < V; ++r) ur[r] = store(u[r], bf16_storage);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The chunkwise (WY / UT-transform) form of the same recurrence, a model used
// only to check, on the CPU, the chunk algebra that a chunked GPU prefill
// relies on. The pages name the chunking ("feat(kda): add CuTe DSL recurrent
// prefill backend", BT = 16 chunks) but print no formulas; the form below is
// the WY representation of a product of generalized Householder transforms
// (Yang et al., "Parallelizing Linear Transformers with the Delta Rule over
// Sequence Length", 2024) with the decay carried per key channel.
// For a chunk of c positions r = 1..c entering with state S0 (K x V terms),
// with Gam_r = g_1 + ... + g_r per channel:
//   A[r][j] = sum_ch k_r k_j exp(Gam_r - Gam_j)     (j < r)
//   P[r][j] = sum_ch q_r k_j exp(Gam_r - Gam_j)     (j <= r)
//   Tm      = (I + diag(beta) A)^-1                 (unit lower triangular)
//   Wm      = Tm diag(beta) (exp(Gam) * K)          U0 = Tm diag(beta) V
//   U       = U0 - Wm S0                            (rows are the u_r)
//   O       = scale * ((exp(Gam) * Q) S0 + P U)
//   S_c     = diag(exp(Gam_c)) S0 + (exp(Gam_c - Gam) * K)^T U
// Evaluated in Real with plain exponentials (used at Real = double, whose
// range holds exp(+-320)). Tm is applied by forward substitution.
template <class Real>
void prefill_chunked(int n_docs, int H, int K, int V, const int32_t* cu, const Real* q,
                     const Real* k, const Real* v, const Real* graw, const Real* beta_logit,
                     const Real* a_log, const Real* dt_bias, Real lower_bound, Real scale,
                     Real* pool, int64_t N, const int32_t* idx, int use_initial_state,
                     Real* out, int chunk, int gate_mode) {
  const int64_t KV = i64(K) * V;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int d = 0; d < n_docs; ++d) {
    for (int h = 0; h < H; ++h) {
      const int t0 = cu[d], t1 = cu[d + 1];
      if (!slot_active(idx[d], N)) {
        for (int t = t0; t < t1; ++t)
          for (int r = 0; r < V; ++r) out[(i64(t) * H + h) * V + r] = 0;
        continue;
      }
      Real* slot = pool + (i64(idx[d]) * H + h) * KV;
      if (t1 == t0 && use_initial_state) continue;
      // S0 in K x V orientation for readability of the algebra: s0[c][r].
      std::vector<Real> s0(KV, static_cast<Real>(0));
      if (use_initial_state)
        for (int r = 0; r < V; ++r)
          for (int c = 0; c < K; ++c) s0[i64(c) * V + r] = slot[i64(r) * K + c];
      for (int c0 = t0; c0 < t1; c0 += chunk) {
        const int n = std::min(chunk, t1 - c0);
        std::vector<Real> Q(i64(n) * K), Kh(i64(n) * K), Gm(i64(n) * K), Vv(i64(n) * V),
            be(n);
        std::vector<Real> g(K);
        for (int r = 0; r < n; ++r) {
          const int t = c0 + r;
          const int64_t tk = (i64(t) * H + h) * K;
          const int64_t tg = (i64(t) * H + h) * gate_width(K, gate_mode);
          prologue<Real>(K, q + tk, k + tk, graw + tg, beta_logit[i64(t) * H + h],
                         alog_of(a_log, h, gate_mode), dtb_of(dt_bias, h, K, gate_mode),
                         lower_bound, gate_mode, &Q[i64(r) * K], &Kh[i64(r) * K], g.data(),
                         &be[r]);
          for (int c = 0; c < K; ++c)
            Gm[i64(r) * K + c] = (r ? Gm[i64(r - 1) * K + c] : static_cast<Real>(0)) + g[c];
          for (int x = 0; x < V; ++x) Vv[i64(r) * V + x] = v[(i64(t) * H + h) * V + x];
        }
        std::vector<Real> A(i64(n) * n, 0), P(i64(n) * n, 0);
        for (int r = 0; r < n; ++r)
          for (int j = 0; j <= r; ++j) {
            Real a = 0, p = 0;
            for (int c = 0; c < K; ++c) {
              const Real w = std::exp(Gm[i64(r) * K + c] - Gm[i64(j) * K + c]);
              a += Kh[i64(r) * K + c] * Kh[i64(j) * K + c] * w;
              p += Q[i64(r) * K + c] * Kh[i64(j) * K + c] * w;
            }
            if (j < r) A[i64(r) * n + j] = a;
            P[i64(r) * n + j] = p;
          }
        // Wm and U0 by forward substitution: (I + diag(beta) A) X = diag(beta) Y.
        std::vector<Real> Wm(i64(n) * K), U(i64(n) * V);
        for (int r = 0; r < n; ++r) {
          for (int c = 0; c < K; ++c) {
            Real x = be[r] * std::exp(Gm[i64(r) * K + c]) * Kh[i64(r) * K + c];
            for (int j = 0; j < r; ++j) x -= be[r] * A[i64(r) * n + j] * Wm[i64(j) * K + c];
            Wm[i64(r) * K + c] = x;
          }
          for (int x = 0; x < V; ++x) {
            Real y = be[r] * Vv[i64(r) * V + x];
            for (int j = 0; j < r; ++j) y -= be[r] * A[i64(r) * n + j] * U[i64(j) * V + x];
            U[i64(r) * V + x] = y;
          }
        }
        // U = U0 - Wm S0
        for (int r = 0; r < n; ++r)
          for (int x = 0; x < V; ++x) {
            Real acc = 0;
            for (int c = 0; c < K; ++c) acc += Wm[i64(r) * K + c] * s0[i64(c) * V + x];
            U[i64(r) * V + x] -= acc;
          }
        // O = scale * ((exp(Gam) * Q) S0 + P U)
        for (int r = 0; r < n; ++r)
          for (int x = 0; x < V; ++x) {
            Real acc = 0;
            for (int c = 0; c < K; ++c)
              acc += std::exp(Gm[i64(r) * K + c]) * Q[i64(r) * K + c] * s0[i64(c) * V + x];
            for (int j = 0; j <= r; ++j) acc += P[i64(r) * n + j] * U[i64(j) * V + x];
            out[(i64(c0 + r) * H + h) * V + x] = scale * acc;
          }
        // S_c = diag(exp(Gam_c)) S0 + (exp(Gam_c - Gam) * K)^T U
        const Real* Gc = &Gm[i64(n - 1) * K];
        for (int c = 0; c < K; ++c)
          for (int x = 0; x < V; ++x) {
            Real acc = std::exp(Gc[c]) * s0[i64(c) * V + x];
            for (int r = 0; r < n; ++r)
              acc += std::exp(Gc[c] - Gm[i64(r) * K + c]) * Kh[i64(r) * K + c] *
                     U[i64(r) * V + x];
            s0[i64(c) * V + x] = acc;
          }
      }
      for (int r = 0; r < V; ++r)
        for (int c = 0; c < K; ++c) slot[i64(r) * K + c] = s0[i64(c) * V + r];
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// C entry points, one per precision. `Real` arrays as documented above.
#define ORC_INSTANTIATE(SUF, Real)                                                            \
  extern "C" void orc_prologue_##SUF(int K, const Real* q, const Real* k, const Real* graw,   \
                                     Real beta_logit, Real a_log, const Real* dt_bias,        \
                                     Real lower_bound, int gate_mode, Real* qh, Real* kh,     \
                                     Real* g, Real* beta) {                                   \
    prologue<Real>(K, q, k, graw, beta_logit, a_log, dt_bias, lower_bound, gate_mode, qh, kh, \
                   g, beta);                                                                  \
  }                                                                                           \
  extern "C" void orc_step_##SUF(int K, int V, Real* S, const Real* qh, const Real* kh,       \
                                 const Real* v, const Real* g, Real beta, Real scale,         \
                                 Real* o, Real* u) {                                          \
    step<Real>(K, V, S, qh, kh, v, g, beta, scale, o, u);                                     \
  }                                                                                           \
  extern "C" void orc_replay_##SUF(int K, int V, const Real* ckpt, const Real* kc,            \
                                   const Real* uc, const Real* gc, int R, int base, int hist, \
                                   Real* S) {                                                 \
    replay<Real>(K, V, ckpt, kc, uc, gc, R, base, hist, S);                                   \
  }                                                                                           \
  extern "C" void orc_decode_##SUF(int B, int H, int K, int V, const Real* q, const Real* k,  \
                                   const Real* v, const Real* graw, const Real* beta_logit,   \
                                   const Real* a_log, const Real* dt_bias, Real lower_bound,  \
                                   Real scale, Real* pool, int64_t N, const int32_t* idx,     \
                                   Real* out, int bf16_storage, int gate_mode,                \
                                   int state_dtype) {                                          \
    decode<Real>(B, H, K, V, q, k, v, graw, beta_logit, a_log, dt_bias, lower_bound, scale,   \
                 pool, N, idx, out, bf16_storage, gate_mode, state_dtype);                     \
  }                                                                                           \
  extern "C" void orc_verify_##SUF(                                                           \
      int B, int T, int H, int K, int V, const Real* q, const Real* k, const Real* v,         \
      const Real* graw, const Real* beta_logit, const Real* a_log, const Real* dt_bias,       \
      Real lower_bound, Real scale, Real* pool, int64_t N, const int32_t* idx, Real* kc,      \
      Real* uc, Real* gc, int R, const int32_t* hist_len, const int32_t* cache_base,          \
      int flush_min, int w_ring, Real* out, int bf16_storage, int gate_mode,                  \
      int state_dtype) {                                                                       \
    verify<Real>(B, T, H, K, V, q, k, v, graw, beta_logit, a_log, dt_bias, lower_bound,       \
                 scale, pool, N, idx, kc, uc, gc, R, hist_len, cache_base, flush_min, w_ring, \
                 out, bf16_storage, gate_mode, state_dtype);                                   \
  }                                                                                           \
  extern "C" void orc_prefill_tbt_##SUF(                                                      \
      int n_docs, int H, int K, int V, const int32_t* cu, const Real* q, const Real* k,       \
      const Real* v, const Real* graw, const Real* beta_logit, const Real* a_log,             \
      const Real* dt_bias, Real lower_bound, Real scale, Real* pool, int64_t N,               \
      const int32_t* idx, int use_initial_state, Real* out, int bf16_storage,                 \
      int gate_mode, Real* ckpt, int64_t ckpt_rows, const int64_t* ckpt_starts,               \
      int interval, int state_dtype, Real* kc, Real* uc, Real* gc, int R,                      \
      const int32_t* cache_base, int ring_tail) {                                             \
    prefill_tbt<Real>(n_docs, H, K, V, cu, q, k, v, graw, beta_logit, a_log, dt_bias,         \
                      lower_bound, scale, pool, N, idx, use_initial_state, out, bf16_storage, \
                      gate_mode, ckpt, ckpt_rows, ckpt_starts, interval, state_dtype, kc, uc,  \
                      gc, R, cache_base, ring_tail);                                          \
  }                                                                                           \
  extern "C" void orc_prefill_chunked_##SUF(                                                  \
      int n_docs, int H, int K, int V, const int32_t* cu, const Real* q, const Real* k,       \
      const Real* v, const Real* graw, const Real* beta_logit, const Real* a_log,             \
      const Real* dt_bias, Real lower_bound, Real scale, Real* pool, int64_t N,               \
      const int32_t* idx, int use_initial_state, Real* out, int chunk, int gate_mode) {       \
    prefill_chunked<Real>(n_docs, H, K, V, cu, q, k, v, graw, beta_logit, a_log, dt_bias,     \
                          lower_bound, scale, pool, N, idx, use_initial_state, out, chunk,    \
                          gate_mode);                                                         \
  }

ORC_INSTANTIATE(f32, float)
ORC_INSTANTIATE(f64, double)

extern "C" void orc_bf16_round(int64_t n, const float* in, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne_bits(in[i]);
}

extern "C" void orc_f16_round(int64_t n, const float* in, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_rne_bits(in[i]);
}

extern "C" void orc_f16_to_float(int64_t n, const uint16_t* in, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_bits_to_float(in[i]);
}

extern "C" void orc_f8_round(int64_t n, const float* in, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f8_rne_bits(in[i]);
}

extern "C" void orc_f8_to_float(int64_t n, const uint8_t* in, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f8_bits_to_float(in[i]);
}

extern "C" int orc_max_threads() {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

extern "C" void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
