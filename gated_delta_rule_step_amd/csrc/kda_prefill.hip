// Chunked varlen prefill of the KDA recurrence (gfx950): one fused kernel,
// one 512-thread workgroup per (document, head), 64-token chunks.
//
// Operation: "feat(kda): add CuTe DSL recurrent prefill backend" -- packed
// documents delimited by cu_seqlens; each (document, head) chain runs the
// gated delta-rule recurrence over its tokens from an optional initial state
// and leaves its final state in the pool; the work splits into an intra-chunk
// preparation and a sequential chain over chunks, the two stages of that
// page's prefill. The result equals the token-by-token recurrence.
//
// Chunkwise form (WY representation of the delta rule, Yang et al.,
// "Parallelizing Linear Transformers with the Delta Rule over Sequence
// Length", 2024, with the decay carried per key channel). For a chunk of
// c <= 64 tokens r entering with state S (S[k][v] here: key channel k, value
// channel v), Gam_r = g_0 + ... + g_r per key channel:
//   A[r,j] = sum_k k_r k_j exp(Gam_r - Gam_j)            (j < r)
//   P[r,j] = sum_k q_r k_j exp(Gam_r - Gam_j)            (j <= r)
//   T      = (I + diag(beta) A)^-1,  T' = T diag(beta)
//   W      = T' (exp(Gam) k),  U0 = T' V
//   U      = U0 - W S             (rows are the per-token corrections u_r)
//   O      = scale ((exp(Gam) q) S + P U)
//   S      = diag(exp(Gam_e)) S + (exp(Gam_e - Gam) k)^T U
// with Gam_e the prefix at the last token that enters the state (the chunk's
// last token, or the last one before a hand-off tail). The lines up to U0 do
// not depend on the state ("preparation"); the last three are the chain.
//
// Precision. The products the state depends on (A, W S) run on bf16 MFMA
// with their fp32 operands split into bf16 hi + lo parts and three terms
// (hi hi + hi lo + lo hi). T' is never formed: the diagonal 16 x 16 blocks
// of T are the finite product (I + N)(I + N^2)(I + N^4)(I + N^8) of their
// strictly lower part N = -diag(beta) A, on fp32 MFMA; W and U0 then follow
// by blocked forward substitution over the four 16-token blocks on bf16
// MFMA, three terms, with beta and the unit diagonals applied exactly in
// fp32. The state update and P U take fp16 hi + lo (three and two terms),
// P is stored in fp16 (|P| <= 1); O = (exp(Gam) q) S takes the state in two
// terms against the bf16 exp(Gam) q. O is stored in bf16.
//
// Decay factoring. A chunk is four 16-token blocks b (block-local prefix
// lam_r, block total tau_b, block start o_b = Gam at the token before it).
// Diagonal blocks of A and P factor exp(Gam_r - Gam_j) around the block's
// midpoint (both factors within exp(+-8 |lower_bound|), |lower_bound| <= 5.5);
// off-diagonal blocks around a block boundary between the two tokens, so both
// factors are at most 1 and a factor underflows only where the weight is
// negligible: pairs (1,0), (2,1) at o_1, o_2; (3,2) at o_3; (2,0), (3,0),
// (3,1) at o_2.
//
// Layouts. Token-owner phases: wave w holds block b = (w/2) xor (w/4) (blocks
// 0 and 3, and 1 and 2, share a SIMD) and key channels 64 (w%2) + 32 s +
// 8 (lane/16) + i, i < 8, of token 16 b + lane%16; chain
// phases: wave w owns value channels 16 w .. 16 w + 15 of the fp32 state,
// held as eight 16 x 16 accumulator tiles (key channels 16 m + 4 (lane/16) + i).

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 f16x8 __attribute__((__vector_size__(8 * sizeof(__fp16))));

constexpr int CH = 64;       // tokens per chunk (at most)
constexpr int NTHR = 512;    // threads per workgroup
constexpr int kMaxOrderedDocs = 256;

// ---- LDS layout (bytes). Arrays of one phase group alias those of another
// only when a barrier separates the last read from the first write.
constexpr int VRS = D + 8;     // bf16 row of v (token-major)
constexpr int KGS = D + 8;     // bf16 row of the right operands of A / P
constexpr int TRS = CH + 4;    // 16-bit row of channel-major arrays (x^T, k~^T) and of P
constexpr int AMS = CH + 4;    // fp32 row of A (scaled by beta)

constexpr int L_NRM = 0;                                // f32 [2][64][2] norm partials
constexpr int L_TAU = L_NRM + 2 * CH * 2 * 4;           // f32 [4][128] block totals
constexpr int L_CUT = L_TAU + 4 * D * 4;                // f32 [128] prefix at the cut
constexpr int L_BETA = L_CUT + D * 4;                   // f32 [64]
constexpr int L_EG = L_BETA + CH * 4;                   // f32 [128] exp(Gam_e)
constexpr int L_SEM = L_EG + D * 4;                     // f32 [4][128] exp(tau_b / 2)
constexpr int L_SEO = L_SEM + 4 * D * 4;                // f32 [4][128] exp(o_b)
constexpr int L_SPH = L_SEO + 4 * D * 4;                // f32 [4][128] exp(Gam_e - o_b - tau_b)
constexpr int L_SO = L_SPH + 4 * D * 4;                 // f32 [4][128] o_b
constexpr int L_ST1 = L_SO + 4 * D * 4;                 // f32 [128] exp(tau_1)
constexpr int L_ST2 = L_ST1 + D * 4;                    // f32 [128] exp(tau_2)
constexpr int L_SGE = L_ST2 + D * 4;                    // f32 [128] Gam_e
constexpr int L_NF = L_SGE + D * 4;                     // bf16 [4 b][2 hl][64 lane][4] T_bb - I
constexpr int L_LF = L_NF + 4 * 2 * 64 * 8;             // bf16 [6][2 hl][64 lane][4] L_ba, a < b
constexpr int L_DTB = L_LF + 6 * 2 * 64 * 8;            // f32 [128] dt_bias of the head
constexpr int L_VR = L_DTB + D * 4;                     // bf16 [64][VRS] v
constexpr int L_QOP = L_VR + CH * VRS * 2;              // bf16 [4 b][4 kt][64 lane][8]
constexpr int L_PM = L_QOP + 4 * 4 * 64 * 16;           // fp16 [64][TRS] P
constexpr int WTS = D + 8;     // bf16 row of W (token-major)
constexpr int L_WTH = L_PM + CH * TRS * 2;              // bf16 [64][WTS] W, hi part
constexpr int L_X1 = L_WTH + CH * WTS * 2;              // region X1 (below)
constexpr int X1_BYTES = 2 * D * TRS * 2;               //   KGR | AM + WTL | KT
constexpr int L_X2 = L_X1 + X1_BYTES;                   // region X2: PART | XT | OST
constexpr int X2_BYTES = 2 * D * TRS * 2;
constexpr int kLdsBytes = L_X2 + X2_BYTES;
// region X1 tenants
constexpr int KGR_BYTES = 4 * 2 * 16 * KGS * 2;         // bf16 [4 slots][2 hl][16][KGS]
constexpr int AM_BYTES = CH * AMS * 4;                  // f32 [64][AMS]
constexpr int KT_BYTES = 2 * D * TRS * 2;               // fp16 [2 hl][128][TRS]
constexpr int WTL_BYTES = CH * WTS * 2;                 // bf16 [64][WTS] W, lo part, after AM
// region X2 tenants
constexpr int PART_BYTES = 10 * 2 * 256 * 4;            // f32 [10 pairs][A, P][64 lanes][4]
constexpr int XT_BYTES = 2 * D * TRS * 2;               // bf16 [2 hl][128][TRS]
constexpr int OSS = D + 8;                              // bf16 row of the staged outputs
constexpr int OST_BYTES = CH * OSS * 2;                 // bf16 [64][OSS]
static_assert(KGR_BYTES <= X1_BYTES && KT_BYTES <= X1_BYTES && AM_BYTES + WTL_BYTES <= X1_BYTES,
              "region X1");
static_assert(PART_BYTES <= X2_BYTES && XT_BYTES <= X2_BYTES && OST_BYTES <= X2_BYTES,
              "region X2");
static_assert(kLdsBytes <= 160 * 1024, "LDS of one CU");
static_assert(L_VR % 16 == 0 && L_QOP % 16 == 0 && L_PM % 16 == 0 && L_WTH % 16 == 0 &&
                  L_X1 % 16 == 0 && L_X2 % 16 == 0 && L_NF % 16 == 0 && L_LF % 16 == 0 &&
                  L_DTB % 16 == 0 &&
                  AM_BYTES % 16 == 0,
              "16-byte aligned arrays");

struct DocOrder {
  int32_t n;  // 0: natural order
  int32_t doc[kMaxOrderedDocs];
};

// Pair numbering of the 16 x 16 blocks of A and P computed per chunk.
// (0,0) (1,1) (1,0) (2,2) (2,0) (2,1) (3,3) (3,2) (3,0) (3,1)
__device__ __forceinline__ int pair_id(int b, int a) {
  constexpr int base[4] = {0, 1, 3, 6};
  if (a == b) return base[b];
  if (b == 1) return 2;
  if (b == 2) return a == 0 ? 4 : 5;
  return a == 2 ? 7 : (a == 0 ? 8 : 9);
}

// Keeps the scheduler from moving instructions across this point (it would
// otherwise hoist every LDS fragment load of an unrolled loop to its top).
__device__ __forceinline__ void fence_sched() { __builtin_amdgcn_sched_barrier(0); }

// Workgroup barrier for LDS traffic only: this wave's LDS accesses complete
// (lgkmcnt 0), then s_barrier. Unlike __syncthreads() it does not wait for
// outstanding global loads, so the next chunk's inputs stay in flight across
// the chain's barriers. No global memory is shared between the waves.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The value unchanged, but opaque to the compiler: lane-dependent addresses
// derived from it are recomputed in each phase of each chunk instead of being
// hoisted out of the chunk loop (hundreds of them would not fit in registers).
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Per-phase copies of the lane's indices (see fresh()).
#define KDA_PHASE_IDS                                   \
  const int ln_ = fresh(lane);                          \
  const int n16 = ln_ & 15, g4 = ln_ >> 4;              \
  const int tr = 16 * tb + n16, cb = 64 * hc + 8 * g4;  \
  const int v = 16 * wave + n16;                        \
  (void)n16; (void)g4; (void)tr; (void)cb; (void)v

__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_h(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));  // bf16 operands of the K = 16 MFMA
__device__ __forceinline__ f32x4 mma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 8 fp32 -> bf16x8 (round to nearest even), and the hi + lo split.
__device__ __forceinline__ u32x4 pack8(const float* x) {
  return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
               pack_bf16x2(x[6], x[7])};
}
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    lo[e] = pack_bf16x2(x[2 * e] - bf_lo(hi[e]), x[2 * e + 1] - bf_hi(hi[e]));
  }
}
__device__ __forceinline__ void split4(const f32x4 x, u32x2& hi, u32x2& lo) {
  hi[0] = pack_bf16x2(x[0], x[1]);
  hi[1] = pack_bf16x2(x[2], x[3]);
  lo[0] = pack_bf16x2(x[0] - bf_lo(hi[0]), x[1] - bf_hi(hi[0]));
  lo[1] = pack_bf16x2(x[2] - bf_lo(hi[1]), x[3] - bf_hi(hi[1]));
}

// The same split in fp16 (11-bit halves: the residual is ~2^-22 of |x|, against
// ~2^-16 for bf16), for operands whose magnitude the fp16 range holds: the
// state update's k~ and the read-out's P (both at most 1 in magnitude) and U
// (scaled by a power of two where a wave's tile would not fit).
__device__ __forceinline__ void split8h(const float* x, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = pack_f16x2(x[2 * e], x[2 * e + 1]);
    lo[e] = pack_f16x2(x[2 * e] - f16_lo(hi[e]), x[2 * e + 1] - f16_hi(hi[e]));
  }
}
__device__ __forceinline__ uint16_t to_f16(float x) {
  return static_cast<uint16_t>(pack_f16x2(x, 0.0f) & 0xffffu);
}

__device__ __forceinline__ void split4s(const f32x4 x, s16x4& hi, s16x4& lo) {
  u32x2 h, l;
  split4(x, h, l);
  hi = __builtin_bit_cast(s16x4, h);
  lo = __builtin_bit_cast(s16x4, l);
}

template <int N>
__device__ __forceinline__ float dpp_shr(float x) {  // row_shr:N, zero shifted in
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x110 + N, 0xF, 0xF, true));
}

template <bool VEC>
__device__ __forceinline__ u32x2 gload4(const uint16_t* p) {
  if constexpr (VEC) {
    return *reinterpret_cast<const u32x2*>(p);
  } else {
    return u32x2{uint32_t(p[0]) | (uint32_t(p[1]) << 16), uint32_t(p[2]) | (uint32_t(p[3]) << 16)};
  }
}
template <bool VEC>
__device__ __forceinline__ void gstore4(uint16_t* p, u32x2 w) {
  if constexpr (VEC) {
    *reinterpret_cast<u32x2*>(p) = w;
  } else {
    p[0] = uint16_t(w[0] & 0xffffu);
    p[1] = uint16_t(w[0] >> 16);
    p[2] = uint16_t(w[1] & 0xffffu);
    p[3] = uint16_t(w[1] >> 16);
  }
}

// Four consecutive state elements (the 4 key channels of one accumulator
// entry) in the state format SF.
template <int SF, bool VEC>
__device__ __forceinline__ f32x4 st4_load(const void* base, int64_t e) {
  if constexpr (SF == kStateFp8) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(base) + e);
    const f32x2 a = f8x2_lo(w), b = f8x2_hi(w);
    return f32x4{a[0], a[1], b[0], b[1]};
  } else {
    const u32x2 w = gload4<VEC>(static_cast<const uint16_t*>(base) + e);
    return f32x4{st_lo<SF>(w[0]), st_hi<SF>(w[0]), st_lo<SF>(w[1]), st_hi<SF>(w[1])};
  }
}
template <int SF, bool VEC>
__device__ __forceinline__ void st4_store(void* base, int64_t e, f32x4 a) {
  if constexpr (SF == kStateFp8) {
    *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(base) + e) = pack_f8x4(a[0], a[1], a[2], a[3]);
  } else {
    gstore4<VEC>(static_cast<uint16_t*>(base) + e,
                 u32x2{st_pack<SF>(a[0], a[1]), st_pack<SF>(a[2], a[3])});
  }
}

// Raw token inputs of one lane (token-owner layout): two runs of eight
// channels (cb + 32 s .. + 7) of q, k, g, v, and the beta bits.
struct Raw {
  u32x4 q[2], k[2], g[2], v[2];
  uint32_t b;
};

// Token row tb + tr: tb is uniform (a chunk's first token), tr the lane's row;
// two runs of 8 channels (16-byte loads on the vectorised path). The inputs
// come in four groups (q; k; g; v and beta). Inside the chunk loop each group
// is issued at its own point of the previous chunk's chain: the workgroup's
// 64 KB of loads per chunk issued at once stall every wave at issue behind
// the vector memory path.
enum RawPart { kRawQ, kRawK, kRawG, kRawVB };

template <int PART, bool VEC, bool GHEAD>
__device__ __forceinline__ void load_raw_part(const PrefillParams& p, int64_t tb, int tr, int h,
                                              int cb, bool valid, Raw& r) {
  constexpr u32x4 z = {0u, 0u, 0u, 0u};
  if constexpr (PART == kRawQ || PART == kRawK) {
    u32x4(&dst)[2] = PART == kRawQ ? r.q : r.k;
    if (valid) {  // lanes past the document's end issue no load
      const uint16_t* base = PART == kRawQ ? p.q : p.k;
      const int64_t ts = PART == kRawQ ? p.q_tok_stride : p.k_tok_stride;
      const uint16_t* x = base + tb * ts + (int64_t(tr) * ts + h * D + cb);
#pragma unroll
      for (int s = 0; s < 2; ++s) dst[s] = load8_bits<VEC>(x + 32 * s);
    } else {
      dst[0] = dst[1] = z;
    }
  } else if constexpr (PART == kRawG) {
    if (valid) {
      const int64_t t = tb + tr;
      if constexpr (GHEAD) {
        const uint32_t gh = p.g[t * p.g_tok_stride + h];
        const uint32_t g2 = gh | (gh << 16);  // the value in both halves: all 16 channels
        r.g[0] = r.g[1] = u32x4{g2, g2, g2, g2};
      } else {
        const uint16_t* g = p.g + t * p.g_tok_stride + h * D + cb;
#pragma unroll
        for (int s = 0; s < 2; ++s) r.g[s] = load8_bits<VEC>(g + 32 * s);
      }
    } else {
      r.g[0] = r.g[1] = z;
    }
  } else {
    if (valid) {
      const int64_t t = tb + tr;
      const uint16_t* v = p.v + tb * p.v_tok_stride + (int64_t(tr) * p.v_tok_stride + h * D + cb);
#pragma unroll
      for (int s = 0; s < 2; ++s) r.v[s] = load8_bits<VEC>(v + 32 * s);
      r.b = p.beta[t * p.beta_tok_stride + h];
    } else {
      r.v[0] = r.v[1] = z;
      r.b = 0u;
    }
  }
}

template <bool VEC, bool GHEAD>
__device__ __forceinline__ void load_raw(const PrefillParams& p, int64_t tb, int tr, int h,
                                         int cb, bool valid, Raw& r) {
  load_raw_part<kRawQ, VEC, GHEAD>(p, tb, tr, h, cb, valid, r);
  load_raw_part<kRawK, VEC, GHEAD>(p, tb, tr, h, cb, valid, r);
  load_raw_part<kRawG, VEC, GHEAD>(p, tb, tr, h, cb, valid, r);
  load_raw_part<kRawVB, VEC, GHEAD>(p, tb, tr, h, cb, valid, r);
}

__device__ __forceinline__ void unpack16(const u32x4 (&w)[2], float (&x)[16]) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * s + 2 * i] = bf_lo(w[s][i]);
      x[8 * s + 2 * i + 1] = bf_hi(w[s][i]);
    }
  }
}

// 16 per-channel fp32 values of this lane's channels from an LDS array of 128.
__device__ __forceinline__ void lds_ch16(const float* a, int cb, float (&x)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(a + cb + 32 * (j >> 1) + 4 * (j & 1));
    x[4 * j] = w[0];
    x[4 * j + 1] = w[1];
    x[4 * j + 2] = w[2];
    x[4 * j + 3] = w[3];
  }
}
__device__ __forceinline__ void lds_st16(float* a, int cb, const float (&x)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<f32x4*>(a + cb + 32 * (j >> 1) + 4 * (j & 1)) =
        f32x4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
}

}  // namespace

// SF: state element format of the pool and the checkpoints; GK: gate kind
// (kGatePrecomputed / kGatePerHead bits).
template <bool VEC, int GK, int SF>
__global__ __launch_bounds__(NTHR, 1) void prefill_kernel(PrefillParams p, DocOrder ord) {
  constexpr bool GRAW = !(GK & kGatePrecomputed);
  constexpr bool GHEAD = (GK & kGatePerHead) != 0;
  static_assert(VEC || SF == kStateBf16, "fp16 and fp8 states use the vectorised layout");
  extern __shared__ __align__(16) uint8_t lds[];
  float* NRM = reinterpret_cast<float*>(lds + L_NRM);
  float* TAU = reinterpret_cast<float*>(lds + L_TAU);
  float* CUT = reinterpret_cast<float*>(lds + L_CUT);
  float* BETA = reinterpret_cast<float*>(lds + L_BETA);
  float* EG = reinterpret_cast<float*>(lds + L_EG);
  float* SEM = reinterpret_cast<float*>(lds + L_SEM);
  float* SEO = reinterpret_cast<float*>(lds + L_SEO);
  float* SPH = reinterpret_cast<float*>(lds + L_SPH);
  float* SO = reinterpret_cast<float*>(lds + L_SO);
  float* ST1 = reinterpret_cast<float*>(lds + L_ST1);
  float* ST2 = reinterpret_cast<float*>(lds + L_ST2);
  float* SGE = reinterpret_cast<float*>(lds + L_SGE);
  s16x4* NF = reinterpret_cast<s16x4*>(lds + L_NF);  // A fragments of the K = 16 MFMA
  s16x4* LF = reinterpret_cast<s16x4*>(lds + L_LF);
  float* DTB = reinterpret_cast<float*>(lds + L_DTB);
  uint16_t* VR = reinterpret_cast<uint16_t*>(lds + L_VR);
  uint8_t* QOP = lds + L_QOP;
  uint16_t* PM = reinterpret_cast<uint16_t*>(lds + L_PM);
  uint16_t* WTH = reinterpret_cast<uint16_t*>(lds + L_WTH);
  uint16_t* KGR = reinterpret_cast<uint16_t*>(lds + L_X1);
  float* AM = reinterpret_cast<float*>(lds + L_X1);
  uint16_t* WTL = reinterpret_cast<uint16_t*>(lds + L_X1 + AM_BYTES);  // W lo, beside AM
  uint16_t* KT = reinterpret_cast<uint16_t*>(lds + L_X1);
  float* PART = reinterpret_cast<float*>(lds + L_X2);
  uint16_t* XT = reinterpret_cast<uint16_t*>(lds + L_X2);
  uint16_t* OST = reinterpret_cast<uint16_t*>(lds + L_X2);  // chunk outputs (after P5)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int g4 = lane >> 4;
  const int n16 = lane & 15;
  const int h = int(blockIdx.x % p.H);
  const int rank = int(blockIdx.x / p.H);
  const int doc = ord.n > 0 ? ord.doc[rank] : rank;
  const int64_t t0 = p.cu_seqlens[doc];
  const int64_t len = int64_t(p.cu_seqlens[doc + 1]) - t0;
  const int32_t slot = p.state_indices[doc];
  const int32_t rbase = p.ring_tail > 0 ? p.cache_base[doc] : 0;
  const bool active = slot >= 0 && int64_t(slot) < p.num_slots && rbase >= 0 &&
                      (p.ring_tail == 0 || rbase < p.ring_rows);
  if (!active) {  // zero outputs, no state access
    for (int64_t e = tid; e < len * D; e += NTHR)
      p.out[(t0 + e / D) * p.out_tok_stride + h * D + (e % D)] = 0;
    return;
  }
  const int64_t se = int64_t(slot) * p.slot_stride + int64_t(h) * HEAD_ELEMS;  // element offset
  if (len == 0) {  // final state = initial state: untouched, or zeros without one
    if (!p.use_initial_state) {
      uint16_t* z = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(p.state_pool) +
                                                se * kStateBytes<SF>);
      for (int e = tid; e < HEAD_ELEMS * kStateBytes<SF> / 2; e += NTHR) z[e] = 0;
    }
    return;
  }

  // hand-off: the last `tail` tokens go to the ring; the state passed on
  // (checkpoints, final) covers the first `kept` tokens
  const int c_last16 = int(len - 16 * ((len - 1) / 16));
  const int tail = p.ring_tail > 0 ? min(p.ring_tail, c_last16) : 0;
  const int64_t kept = len - tail;
  const int64_t ckpt_row0 = p.ckpt ? p.ckpt_starts[doc] : 0;
  const int ivl = p.ckpt ? p.ckpt_interval : 0;
  const int64_t ring0 = (int64_t(slot) * p.H + h) * int64_t(p.ring_rows);

  // token-owner identity
  // waves w and w + 4 share a SIMD: blocks 0 and 3 (the lightest and the
  // heaviest operand and pair work) pair up, and blocks 1 and 2
  const int tb = (wave >> 1) ^ (wave >> 2), hc = wave & 1;
  const int tr = 16 * tb + n16;        // token of this lane within the chunk
  const int cb = 64 * hc + 8 * g4;     // first channel of the lane's two runs of 8
  // chain identity: value channel of this lane
  const int v = 16 * wave + n16;

  // P above its block diagonal: the blocks the read-out's products read that
  // are always zero ((0,1) and (2,3)); nothing else writes them.
  for (int e = tid; e < 2 * 256; e += NTHR) {
    const int blk = e >> 8, r = (e >> 4) & 15, cc = e & 15;
    PM[(32 * blk + r) * TRS + 32 * blk + 16 + cc] = 0;
  }

  // ---- initial state in the accumulator layout
  f32x4 acc[8];
  if (p.use_initial_state) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
      acc[m] = st4_load<SF, VEC>(p.state_pool, se + int64_t(v) * D + 16 * m + 4 * g4);
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int len32 = int(len);  // cu_seqlens is int32: a document holds < 2^31 tokens
  auto chunk_len = [&](int pos) {
    int c = min(CH, len32 - pos);
    if (ivl) c = min(c, ivl - pos % ivl);
    return c;
  };
  Raw raw;
  {
    const int c0 = chunk_len(0);
    load_raw<VEC, GHEAD>(p, t0, tr, h, cb, tr < c0, raw);
  }
  const float neg_ea = GRAW ? -fexp(p.A_log[h]) : 0.f;
  if constexpr (GRAW) {  // the head's dt_bias, read by every chunk's prologue
    if (tid < D) DTB[tid] = GHEAD ? p.dt_bias[h] : p.dt_bias[h * D + tid];
  }
  __syncthreads();
  const bool presig = (p.gate_mode & kBetaPresigmoid) != 0;

  for (int pos = 0; pos < len32;) {
    const int c = chunk_len(pos);
    const bool last = pos + c == len32;
    const int pe = last ? c - tail : c;  // tokens of this chunk that enter the state
    const bool cut = pe < c;
    const bool valid = tr < c;

    // ================= P1: token prologue (token-owner layout)
    float qf[16], kf[16], lam[16];
    {
      KDA_PHASE_IDS;
      float gr[16], dtb[16];
      if constexpr (GRAW) lds_ch16(DTB, cb, dtb);
      unpack16(raw.q, qf);
      unpack16(raw.k, kf);
      unpack16(raw.g, gr);
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sq = fmaf(qf[e], qf[e], sq);
        sk = fmaf(kf[e], kf[e], sk);
      }
      sq += __shfl_xor(sq, 16);
      sq += __shfl_xor(sq, 32);
      sk += __shfl_xor(sk, 16);
      sk += __shfl_xor(sk, 32);
      if (g4 == 0) {
        NRM[(hc * CH + tr) * 2] = sq;
        NRM[(hc * CH + tr) * 2 + 1] = sk;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float ge;
        if constexpr (GRAW) ge = fgate(gr[e] + dtb[e], neg_ea, p.lower_bound);
        else ge = gate_given(gr[e], p.lower_bound);
        ge = valid ? ge : 0.f;
        // inclusive prefix over the 16 tokens of the block (one DPP row)
        ge += dpp_shr<1>(ge);
        ge += dpp_shr<2>(ge);
        ge += dpp_shr<4>(ge);
        ge += dpp_shr<8>(ge);
        lam[e] = ge;
      }
      if (n16 == 15) lds_st16(TAU + tb * D, cb, lam);
      if (cut && pe > 0 && tr == pe - 1) lds_st16(CUT, cb, lam);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        *reinterpret_cast<u32x4*>(VR + tr * VRS + cb + 32 * s) = raw.v[s];
      if (hc == 0 && g4 == 0) {
        const float braw = bf1(uint16_t(raw.b));
        const float bt = valid ? (presig ? braw : fsigmoid(braw)) : 0.f;
        BETA[tr] = bt;
      }
    }
    lds_barrier();  // b1

    // ================= P1.5: per (block, channel) scalars
    {
      const int tid_ = fresh(tid);
      const int bb = tid_ >> 7, cc = tid_ & 127;
      const float t0_ = TAU[cc], t1_ = TAU[D + cc], t2_ = TAU[2 * D + cc], t3_ = TAU[3 * D + cc];
      const float tau[4] = {t0_, t1_, t2_, t3_};
      float o = 0.f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
        if (a < bb) o += tau[a];
      const float tbb = tau[bb];
      const float glast = ((t0_ + t1_) + t2_) + t3_;
      float gend = glast;
      if (cut) {
        if (pe == 0) {
          gend = 0.f;
        } else {
          const int bc = (pe - 1) >> 4;
          float oc = 0.f;
#pragma unroll
          for (int a = 0; a < 4; ++a)
            if (a < bc) oc += tau[a];
          gend = oc + CUT[cc];
        }
      }
      SEM[bb * D + cc] = fexp(0.5f * tbb);
      SEO[bb * D + cc] = fexp(o);
      SPH[bb * D + cc] = fexp(gend - o - tbb);
      SO[bb * D + cc] = o;
      if (bb == 0) {
        EG[cc] = fexp(gend);
        ST1[cc] = fexp(t1_);
        ST2[cc] = fexp(t2_);
        SGE[cc] = gend;
      }
    }
    lds_barrier();  // b1.5

    // ================= P2: operands (token-owner layout), one slice of 8 channels
    // at a time; diagonal blocks of A and P from the wave's own registers
    u32x4 kFh[2], kFl[2], qFh[2], qFl[2];     // left operands of the off-diagonal pairs
    u32x4 kF2h[2], kF2l[2], qF2h[2], qF2l[2];  // block 3 towards blocks 0 and 1 (reference o_2)
    u32x4 xh[2], xl[2];               // exp(Gam) k_hat, for W
    u32x4 kth[2], ktl[2];             // exp(Gam_e - Gam) k_hat (fp16), for the state update
    f32x4 accA[4], accP[4];           // this wave's partial sums of its pairs
    {
      KDA_PHASE_IDS;
      const float rq = __builtin_amdgcn_rsqf(NRM[tr * 2] + NRM[(CH + tr) * 2] + 1e-6f);
      const float rk = __builtin_amdgcn_rsqf(NRM[tr * 2 + 1] + NRM[(CH + tr) * 2 + 1] + 1e-6f);
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) accA[i] = accP[i] = z;
      f32x4 a0 = z, a1 = z, a2 = z, pp = z;  // diagonal block (tb, tb)
      const bool ring_row = cut && tr >= pe && tr < c;
      // ring row (rbase + tr - pe) mod R: rbase < R and tr - pe < tail <= R
      int rr = rbase + tr - pe;
      rr = rr >= p.ring_rows ? rr - p.ring_rows : rr;
      const int64_t rrow = ring0 + rr;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // per-channel scalars of this slice: runs (s, 0) and (s, 1)
        float tau[8], em[8], eo[8], ph[8];
        auto ch8 = [&](const float* a, float (&x)[8]) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(a + cb + 32 * s + 4 * h2);
            x[4 * h2] = w[0]; x[4 * h2 + 1] = w[1]; x[4 * h2 + 2] = w[2]; x[4 * h2 + 3] = w[3];
          }
        };
        ch8(TAU + tb * D, tau);
        ch8(SEM + tb * D, em);
        ch8(SEO + tb * D, eo);
        ch8(SPH + tb * D, ph);
        float kL[8], kR[8], qL[8], kF[8], qF[8], kG[8], y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int E8 = 8 * s + e;
          const float qh = qf[E8] * rq, kh = kf[E8] * rk;
          // exp(lam - tau/2) and its reciprocal: the midpoint factors (within e^+-44)
          const float E = fexp(lam[E8] - 0.5f * tau[e]);
          const float Ei = __builtin_amdgcn_rcpf(E);
          const float F = E * em[e];   // exp(lam)        <= 1
          const float G = Ei * em[e];  // exp(tau - lam)  <= 1
          kL[e] = kh * E;
          kR[e] = kh * Ei;
          qL[e] = qh * E;
          kF[e] = kh * F;
          qF[e] = qh * F;
          kG[e] = kh * G;
        }
        {  // diagonal block: three hi / lo terms for A and for P
          u32x4 lh, ll, rh, rl, qh8, ql8;
          split8(kL, lh, ll);
          split8(kR, rh, rl);
          split8(qL, qh8, ql8);
          a0 = mma(lh, rh, a0);
          a1 = mma(lh, rl, a1);
          a2 = mma(ll, rh, a2);
          pp = mma(qh8, rh, pp);
          pp = mma(qh8, rl, pp);
          pp = mma(ql8, rh, pp);
        }
        split8(kF, kFh[s], kFl[s]);
        split8(qF, qFh[s], qFl[s]);
        // Q~ = exp(Gam) q_hat -> the chain's fragment (block tb, kt = 2 hc + s)
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = qF[e] * eo[e];
        {  // channels 8 g4 .. +7 of the slice go to the fragments of chain lanes
           // g = 2 (g4 % 2) and g + 1 (key channels 4 g + i in the first half of a
           // fragment, 16 + 4 g + i in the second; half g4 / 2)
          const u32x4 w = pack8(y);
          uint8_t* base = QOP + (tb * 4 + 2 * hc + s) * 64 * 16 + (g4 >> 1) * 8;
          const int gq = 2 * (g4 & 1);
          *reinterpret_cast<u32x2*>(base + (n16 + 16 * gq) * 16) = u32x2{w[0], w[1]};
          *reinterpret_cast<u32x2*>(base + (n16 + 16 * (gq + 1)) * 16) = u32x2{w[2], w[3]};
        }
        // x = exp(Gam) k_hat
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = kF[e] * eo[e];
        split8(y, xh[s], xl[s]);
        // k~ = exp(Gam_e - Gam) k_hat (zero for tokens that do not enter the state)
        if (!cut) {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = kG[e] * ph[e];
        } else {
          float so[8], sge[8];
          ch8(SO + tb * D, so);
          ch8(SGE, sge);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int E8 = 8 * s + e;
            y[e] = tr < pe ? kf[E8] * rk * fexp(sge[e] - so[e] - lam[E8]) : 0.f;
          }
          if (ring_row) {  // hand-off: ring rows of the tail tokens (k_hat, G)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int E8 = 8 * s + e;
              const int ch = cb + 32 * s + e;
              p.k_cache[rrow * D + ch] = to_bf16(kf[E8] * rk);
              p.g_cache[rrow * D + ch] = so[e] + lam[E8] - sge[e];
            }
          }
        }
        split8h(y, kth[s], ktl[s]);
        if (tb == 3) {  // left operands towards blocks 0 and 1: reference o_2 (x exp(tau_2))
          float t2[8], b2[8];
          ch8(ST2, t2);  // one value per channel
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            y[e] = kF[e] * t2[e];
            b2[e] = qF[e] * t2[e];
          }
          split8(y, kF2h[s], kF2l[s]);
          split8(b2, qF2h[s], qF2l[s]);
        }
        // right operands of the off-diagonal pairs -> LDS, slots 0..2: exp(tau_b - lam) k_hat
        auto put_right = [&](int sl, const float* x) {
          u32x4 hi, lo;
          split8(x, hi, lo);
          *reinterpret_cast<u32x4*>(KGR + ((sl * 2 + 0) * 16 + n16) * KGS + cb + 32 * s) = hi;
          *reinterpret_cast<u32x4*>(KGR + ((sl * 2 + 1) * 16 + n16) * KGS + cb + 32 * s) = lo;
        };
        if (tb <= 2) put_right(tb, kG);
        if (tb == 0) {  // slot 3: block 0 towards reference o_2 (x exp(tau_1))
          float t1[8];
          ch8(ST1, t1);
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = kG[e] * t1[e];
          put_right(3, y);
        }
      }
      accA[0] = a0 + (a1 + a2);
      accP[0] = pp;
    }
    lds_barrier();  // b2

    // ================= P3: off-diagonal blocks of A and P (partials over this half)
    {
      KDA_PHASE_IDS;
      auto offdiag = [&](int slot_r, const u32x4 (&lh)[2], const u32x4 (&ll)[2],
                         const u32x4 (&qh)[2], const u32x4 (&ql)[2], f32x4& A, f32x4& P) {
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, pp = a0;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u32x4 rh = *reinterpret_cast<const u32x4*>(
              KGR + ((slot_r * 2 + 0) * 16 + n16) * KGS + cb + 32 * s);
          const u32x4 rl = *reinterpret_cast<const u32x4*>(
              KGR + ((slot_r * 2 + 1) * 16 + n16) * KGS + cb + 32 * s);
          a0 = mma(lh[s], rh, a0);
          a1 = mma(lh[s], rl, a1);
          a2 = mma(ll[s], rh, a2);
          pp = mma(qh[s], rh, pp);
          pp = mma(qh[s], rl, pp);
          pp = mma(ql[s], rh, pp);
        }
        A = a0 + (a1 + a2);
        P = pp;
      };
      if (tb == 1) {
        offdiag(0, kFh, kFl, qFh, qFl, accA[1], accP[1]);            // (1,0)
      } else if (tb == 2) {
        offdiag(3, kFh, kFl, qFh, qFl, accA[1], accP[1]);            // (2,0)
        offdiag(1, kFh, kFl, qFh, qFl, accA[2], accP[2]);            // (2,1)
      } else if (tb == 3) {
        offdiag(2, kFh, kFl, qFh, qFl, accA[1], accP[1]);            // (3,2)
        offdiag(3, kF2h, kF2l, qF2h, qF2l, accA[2], accP[2]);        // (3,0)
        offdiag(1, kF2h, kF2l, qF2h, qF2l, accA[3], accP[3]);        // (3,1)
      }
      {  // the half that combines A below publishes P, and the other way round
        const int np = tb + 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < np) {
            const int a = i == 0 ? tb : (tb == 1 ? 0 : (tb == 2 ? i - 1 : (i == 1 ? 2 : i - 2)));
            const int pid = pair_id(tb, a);
            *reinterpret_cast<f32x4*>(PART + ((pid * 2 + (hc ^ 1)) * 64 + ln_) * 4) =
                hc ? accA[i] : accP[i];
          }
        }
      }
    }
    lds_barrier();  // b3

    // ================= P3b: A (scaled by beta) and P, whole sums, masked; the
    // channel half hc = 0 completes A, hc = 1 completes P
    {
      KDA_PHASE_IDS;
      const int np = tb + 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < np) {
          const int a = i == 0 ? tb : (tb == 1 ? 0 : (tb == 2 ? i - 1 : (i == 1 ? 2 : i - 2)));
          const int pid = pair_id(tb, a);
          const f32x4 part = *reinterpret_cast<const f32x4*>(PART + ((pid * 2 + hc) * 64 + ln_) * 4);
          if (hc == 0) {
            const f32x4 A = accA[i] + part;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int rl = 4 * g4 + q;  // row within the block; column n16
              const int r = 16 * tb + rl, j = 16 * a + n16;
              AM[r * AMS + j] = (a < tb || n16 < rl) ? A[q] * BETA[r] : 0.f;
            }
          } else {
            const f32x4 P = accP[i] + part;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int rl = 4 * g4 + q;
              const int r = 16 * tb + rl, j = 16 * a + n16;
              PM[r * TRS + j] = to_f16((a < tb || n16 <= rl) ? P[q] : 0.f);
            }
          }
        }
      }
    }
    lds_barrier();  // b4

    // ================= P4a: x^T -> LDS (every wave); diagonal blocks of T (waves 0-3)
    {
      KDA_PHASE_IDS;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int e = 8 * s + 2 * w + hf;
            const int ch = cb + 32 * (e >> 3) + (e & 7);
            XT[ch * TRS + tr] = uint16_t(hf ? xh[s][w] >> 16 : xh[s][w] & 0xffffu);
            XT[D * TRS + ch * TRS + tr] = uint16_t(hf ? xl[s][w] >> 16 : xl[s][w] & 0xffffu);
          }
        }
      }
      if (wave < 4) {
        // T_bb = (I + L_bb)^-1 = (I + N)(I + N^2)(I + N^4)(I + N^8), N = -L_bb
        // (strictly lower, so N^16 = 0), on fp32 MFMA; wave b takes block b.
        // A matrix is held in the accumulator layout (Z: rows 4 g4 + i, column
        // n16), and where it enters as a left factor also transposed (Zt): a
        // 16 x 16 x 4 step ks contracts the index 4 g4 + ks, which both forms
        // hold in element ks.
        const int b = wave;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 Nz, Nt, Id;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          Nz[q] = -AM[(16 * b + 4 * g4 + q) * AMS + 16 * b + n16];
          Id[q] = (4 * g4 + q == n16) ? 1.f : 0.f;
        }
        Nt = -*reinterpret_cast<const f32x4*>(AM + (16 * b + n16) * AMS + 16 * b + 4 * g4);
        auto prod = [&](f32x4 Xt, f32x4 Y) {  // (X Y) in the Z layout
          f32x4 r = z;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) r = mma_f32(Xt[ks], Y[ks], r);
          return r;
        };
        auto prodT = [&](f32x4 Xt, f32x4 Y) {  // (X Y)^T in the Z layout
          f32x4 r = z;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) r = mma_f32(Y[ks], Xt[ks], r);
          return r;
        };
        const f32x4 N2z = prod(Nt, Nz), N2t = prodT(Nt, Nz);
        const f32x4 N4z = prod(N2t, N2z), N4t = prodT(N2t, N2z);
        const f32x4 N8z = prod(N4t, N4z);
        const f32x4 N3t = prodT(Nt, N2z);
        const f32x4 X1t = ((Id + Nt) + N2t) + N3t;
        const f32x4 X2t = X1t + prodT(X1t, N4z);
        // T_bb^T in the Z layout is T_bb in the A-operand layout of the K = 16
        // MFMA (lane: row n16, k = 4 g4 + i); the substitution below takes T_bb - I
        const f32x4 Nb = (X2t + prodT(X2t, N8z)) - Id;
        split4s(Nb, NF[(2 * b) * 64 + ln_], NF[(2 * b + 1) * 64 + ln_]);
      } else if (wave < 7) {
        // the blocks L_ba (a < b) in the same layout, two per wave:
        // 0 (1,0), 1 (2,0), 2 (2,1), 3 (3,0), 4 (3,1), 5 (3,2)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int li = 2 * (wave - 4) + k;
          const int b = li == 0 ? 1 : (li < 3 ? 2 : 3);
          const int a = li - (b == 1 ? 0 : (b == 2 ? 1 : 3));
          const f32x4 x = *reinterpret_cast<const f32x4*>(AM + (16 * b + n16) * AMS + 16 * a + 4 * g4);
          split4s(x, LF[(2 * li) * 64 + ln_], LF[(2 * li + 1) * 64 + ln_]);
        }
      }
    }
    lds_barrier();  // b5

    // ================= P5: W = T' X and U0 = T' V, T' = (I + L)^-1 diag(beta), by
    // blocked forward substitution: Y_b = T_bb (beta_b R_b - sum_{a<b} L_ba Y_a).
    // Wave w takes the channel tile 16 w.. of X (W, to LDS token-major) and the
    // value tile 16 w.. of V (U0, kept for C1); the blocks are 16 x 16 x 16 bf16
    // MFMAs with hi + lo operands (three terms). beta enters in fp32 and the unit
    // diagonal of T_bb exactly: only the products L_ba Y_a and (T_bb - I) Z_b
    // are split.
    f32x4 u0[4];
    {
      KDA_PHASE_IDS;
      // A operands (lane: row n16, k = 4 g4 + e): L_10, L_20, L_21, L_30, L_31, L_32
      // and N_b = T_bb - I
      s16x4 lh[6], ll[6], nh[4], nl[4];
#pragma unroll
      for (int li = 0; li < 6; ++li) {
        lh[li] = LF[(2 * li) * 64 + ln_];
        ll[li] = LF[(2 * li + 1) * 64 + ln_];
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        nh[b] = NF[(2 * b) * 64 + ln_];
        nl[b] = NF[(2 * b + 1) * 64 + ln_];
      }
      // R rows 16 b + 4 g4 + i, column n16 of the tile, all read up front (the
      // blocks below form one dependent chain): X as hi + lo of x^T (channel
      // 16 wave + n16), V (value channel v)
      u32x2 xh2[4], xl2[4];
      uint16_t vr[4][4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        xh2[b] = *reinterpret_cast<const u32x2*>(XT + (16 * wave + n16) * TRS + 16 * b + 4 * g4);
        xl2[b] = *reinterpret_cast<const u32x2*>(XT + D * TRS + (16 * wave + n16) * TRS + 16 * b + 4 * g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[b][i] = VR[(16 * b + 4 * g4 + i) * VRS + v];
      }
      // the solved blocks Y_a of both tiles, split (B operands of the later blocks)
      s16x4 yh[2][4], yl[2][4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f32x4 bet = *reinterpret_cast<const f32x4*>(BETA + 16 * b + 4 * g4);
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
          f32x4 r;
          if (tile == 0) {
            const u32x2 h2 = xh2[b], l2 = xl2[b];
            r = f32x4{bf_lo(h2[0]) + bf_lo(l2[0]), bf_hi(h2[0]) + bf_hi(l2[0]),
                      bf_lo(h2[1]) + bf_lo(l2[1]), bf_hi(h2[1]) + bf_hi(l2[1])};
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = bf1(vr[b][i]);
          }
          // Blocks 0 and 1 go into one K = 32 product (operands concatenated). The
          // 16 x 16 x 32 and 16 x 16 x 16 products keep separate accumulators,
          // summed on the VALU: a chain in which one shape's result is the
          // other's accumulator input gave wrong results.
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
          f32x4 sum = zero, s16 = zero;
          const int l0 = b == 1 ? 0 : (b == 2 ? 1 : 3);  // first L block of row b
          if (b >= 2) {
            auto cat = [](s16x4 x, s16x4 y) {
              const u32x2 a = __builtin_bit_cast(u32x2, x), c = __builtin_bit_cast(u32x2, y);
              return u32x4{a[0], a[1], c[0], c[1]};
            };
            const u32x4 lh2 = cat(lh[l0], lh[l0 + 1]), ll2 = cat(ll[l0], ll[l0 + 1]);
            const u32x4 yh2 = cat(yh[tile][0], yh[tile][1]), yl2 = cat(yl[tile][0], yl[tile][1]);
            sum = mma(lh2, yh2, sum);
            sum = mma(lh2, yl2, sum);
            sum = mma(ll2, yh2, sum);
          }
#pragma unroll
          for (int a = 0; a < b; ++a) {
            if (b >= 2 && a < 2) continue;
            s16 = mma16(lh[l0 + a], yh[tile][a], s16);
            s16 = mma16(lh[l0 + a], yl[tile][a], s16);
            s16 = mma16(ll[l0 + a], yh[tile][a], s16);
          }
          sum += s16;
          const f32x4 z = r * bet - sum;
          s16x4 zh, zl;
          split4s(z, zh, zl);
          f32x4 t = {0.f, 0.f, 0.f, 0.f};
          t = mma16(nh[b], zh, t);
          t = mma16(nh[b], zl, t);
          t = mma16(nl[b], zh, t);
          const f32x4 y = z + t;
          split4s(y, yh[tile][b], yl[tile][b]);
          if (tile == 1) {
            u0[b] = y;
          } else {
            // W rows 16 b + 4 g4 + i, key channel c = 16 wave + n16, stored at
            // 32 (c >> 5) + 8 ((c & 15) >> 2) + 4 ((c >> 4) & 1) + (c & 3): C1's
            // eight channels of one operand (the state fragment's order) are
            // then one contiguous 16-byte piece
            const u32x2 hb = __builtin_bit_cast(u32x2, yh[0][b]);
            const u32x2 lb = __builtin_bit_cast(u32x2, yl[0][b]);
            const int pc = 32 * (wave >> 1) + 8 * (n16 >> 2) + 4 * (wave & 1) + (n16 & 3);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int o = (16 * b + 4 * g4 + i) * WTS + pc;
              WTH[o] = uint16_t(i & 1 ? hb[i >> 1] >> 16 : hb[i >> 1] & 0xffffu);
              WTL[o] = uint16_t(i & 1 ? lb[i >> 1] >> 16 : lb[i >> 1] & 0xffffu);
            }
          }
        }
      }
    }
    lds_barrier();  // b7

    // ================= C1: U = U0 - W S, O = Q~ S (chain; wave: value tile)
    const int npos = pos + c;
    const int cn_next = npos < len32 ? chunk_len(npos) : 0;  // the next chunk's length (0: none)
    f32x4 oo[4];
    u32x4 uh[2], ul[2];  // this wave's U tile in fp16 hi + lo, times u_sc
    bool u_big = false;  // wave-uniform: u_sc = 2^-s, u_isc = 2^s, else both 1
    float u_sc = 1.f, u_isc = 1.f;
    {
      KDA_PHASE_IDS;
      u32x4 sh[4], sl[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const float sv[8] = {acc[2 * kt][0],     acc[2 * kt][1],     acc[2 * kt][2],
                             acc[2 * kt][3],     acc[2 * kt + 1][0], acc[2 * kt + 1][1],
                             acc[2 * kt + 1][2], acc[2 * kt + 1][3]};
        split8(sv, sh[kt], sl[kt]);
      }
      f32x4 uu[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        fence_sched();
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 y0 = z, y1 = z, y2 = z, yq = z;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          // W row 16 b + n16, key channels 32 kt + 4 g4 .. +3 and 32 kt + 16 + 4 g4 .. +3
          // (the order of the state's B fragment), stored contiguously
          const int wo = (16 * b + n16) * WTS + 32 * kt + 8 * g4;
          const u32x4 wh = *reinterpret_cast<const u32x4*>(WTH + wo);
          const u32x4 wl = *reinterpret_cast<const u32x4*>(WTL + wo);
          const u32x4 qq = *reinterpret_cast<const u32x4*>(QOP + ((b * 4 + kt) * 64 + ln_) * 16);
          y0 = mma(wh, sh[kt], y0);
          y1 = mma(wh, sl[kt], y1);
          y2 = mma(wl, sh[kt], y2);
          yq = mma(qq, sh[kt], yq);
          yq = mma(qq, sl[kt], yq);  // the state's low part: only q~'s rounding remains
        }
        uu[b] = u0[b] - (y0 + (y1 + y2));
        oo[b] = yq;
      }
      // U goes to the fp16 products below. A tile with an element of 2^14 or
      // more (inputs far outside the usual range) is scaled by 2^-s first, so
      // that hi + lo stay finite; the products are scaled back by 2^s.
      float um = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) um = fmaxf(um, fabsf(uu[b][q]));
      u_big = __builtin_amdgcn_ballot_w64(um >= 16384.f) != 0;
      if (cut) {  // hand-off: ring rows of the tail tokens receive u (bf16)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          fence_sched();
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 16 * b + 4 * g4 + q;
            if (r >= pe && r < c) {
              int rr = rbase + r - pe;
              rr = rr >= p.ring_rows ? rr - p.ring_rows : rr;
              p.u_cache[(ring0 + rr) * D + v] = to_bf16(uu[b][q]);
            }
          }
        }
      }
      // The scaling lives in branches of its own (around the products, not in
      // them), so that the usual case runs none of it.
      if (__builtin_expect(u_big, 0)) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) um = fmaxf(um, __shfl_xor(um, o));
        const int ex = int((__float_as_uint(um) >> 23) & 0xffu) - 127;  // >= 14
        const int sh = __builtin_amdgcn_readfirstlane(min(ex - 13, 126));
        u_sc = __uint_as_float(uint32_t(127 - sh) << 23);
        u_isc = __uint_as_float(uint32_t(127 + sh) << 23);
#pragma unroll
        for (int b = 0; b < 4; ++b) uu[b] *= u_sc;
      }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const float x8[8] = {uu[2 * pp][0],     uu[2 * pp][1],     uu[2 * pp][2],
                             uu[2 * pp][3],     uu[2 * pp + 1][0], uu[2 * pp + 1][1],
                             uu[2 * pp + 1][2], uu[2 * pp + 1][3]};
        split8h(x8, uh[pp], ul[pp]);
      }
    }
    lds_barrier();  // b8: W fragments read; k~^T may overwrite them

    {  // next chunk's raw inputs, in flight during C2 and C3 (always assigned, zeros
       // past the document's end, so that they are dead from P1 to here): q
      KDA_PHASE_IDS;
      load_raw_part<kRawQ, VEC, GHEAD>(p, t0 + npos, tr, h, cb, tr < cn_next, raw);
    }

    // ================= k~^T -> LDS (token-owner registers); C2: O += P U, output
    {
      KDA_PHASE_IDS;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int e = 8 * s + 2 * w + hf;
            const int ch = cb + 32 * (e >> 3) + (e & 7);
            KT[ch * TRS + tr] = uint16_t(hf ? kth[s][w] >> 16 : kth[s][w] & 0xffffu);
            KT[D * TRS + ch * TRS + tr] = uint16_t(hf ? ktl[s][w] >> 16 : ktl[s][w] & 0xffffu);
          }
        }
      }
      load_raw_part<kRawK, VEC, GHEAD>(p, t0 + npos, tr, h, cb, tr < cn_next, raw);
      if (__builtin_expect(u_big, 0)) {
#pragma unroll
        for (int b = 0; b < 4; ++b) oo[b] *= u_sc;
      }
      const float osc = p.scale * u_isc;  // undoes the scaling of U (1 as a rule)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          if (pp == 1 && b < 2) continue;
          const uint16_t* prow = PM + (16 * b + n16) * TRS + 32 * pp;
          const u32x2 a0 = *reinterpret_cast<const u32x2*>(prow + 4 * g4);
          const u32x2 a1 = *reinterpret_cast<const u32x2*>(prow + 16 + 4 * g4);
          const u32x4 pa = {a0[0], a0[1], a1[0], a1[1]};
          oo[b] = mma_h(pa, uh[pp], oo[b]);
          oo[b] = mma_h(pa, ul[pp], oo[b]);
        }
        // outputs staged in LDS (the x^T region, free until the next chunk's
        // A / P partials), stored below as whole 16-byte pieces of token rows
#pragma unroll
        for (int q = 0; q < 4; ++q)
          OST[(16 * b + 4 * g4 + q) * OSS + v] = to_bf16(osc * oo[b][q]);
      }
      load_raw_part<kRawG, VEC, GHEAD>(p, t0 + npos, tr, h, cb, tr < cn_next, raw);
    }
    lds_barrier();  // b9

    {  // this chunk's output rows: 64 rows x 16 pieces of 8 channels, two per thread
      const int t_ = fresh(tid);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int id = t_ + NTHR * k2;
        const int r = id >> 4, c8 = 8 * (id & 15);
        if (r < c) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(OST + r * OSS + c8);
          store8_raw<VEC>(p.out + (t0 + pos + r) * p.out_tok_stride + h * D + c8, w);
        }
      }
    }

    // ================= C3: S = diag(exp(Gam_e)) S + k~^T U
    if (__builtin_expect(u_big, 0)) {
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] *= u_sc;
    }
    {
      KDA_PHASE_IDS;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        fence_sched();
        const f32x4 eg = *reinterpret_cast<const f32x4*>(EG + 16 * m + 4 * g4);
        f32x4 a = acc[m] * eg;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const uint16_t* kr_h = KT + (16 * m + n16) * TRS + 32 * pp;
          const uint16_t* kr_l = KT + D * TRS + (16 * m + n16) * TRS + 32 * pp;
          const u32x2 h0 = *reinterpret_cast<const u32x2*>(kr_h + 4 * g4);
          const u32x2 h1 = *reinterpret_cast<const u32x2*>(kr_h + 16 + 4 * g4);
          const u32x2 l0 = *reinterpret_cast<const u32x2*>(kr_l + 4 * g4);
          const u32x2 l1 = *reinterpret_cast<const u32x2*>(kr_l + 16 + 4 * g4);
          const u32x4 kh8 = {h0[0], h0[1], h1[0], h1[1]};
          const u32x4 kl8 = {l0[0], l0[1], l1[0], l1[1]};
          a = mma_h(kh8, uh[pp], a);
          a = mma_h(kh8, ul[pp], a);
          a = mma_h(kl8, uh[pp], a);
        }
        acc[m] = a;
        if (m == 0) load_raw_part<kRawVB, VEC, GHEAD>(p, t0 + npos, tr, h, cb, tr < cn_next, raw);
      }
    }
    if (__builtin_expect(u_big, 0)) {
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] *= u_isc;
    }
    // intermediate checkpoint after this chunk
    if (ivl && npos % ivl == 0 && npos <= kept) {
      KDA_PHASE_IDS;
      const int64_t row = ckpt_row0 + npos / ivl - 1;  // (32-bit division)
      if (row >= 0 && row < p.ckpt_rows) {
        const int64_t ce = (row * p.H + h) * int64_t(HEAD_ELEMS);
#pragma unroll
        for (int m = 0; m < 8; ++m)
          st4_store<SF, VEC>(p.ckpt, ce + int64_t(v) * D + 16 * m + 4 * g4, acc[m]);
      }
    }
    pos = npos;
  }

  // ---- final state (the state after the first `kept` tokens)
#pragma unroll
  for (int m = 0; m < 8; ++m)
    st4_store<SF, VEC>(p.state_pool, se + int64_t(v) * D + 16 * m + 4 * g4, acc[m]);
}

size_t prefill_workspace_bytes(int32_t n_docs, int64_t total_tokens, int32_t H) {
  if (int64_t(n_docs) * H < kFusedMinChains)
    return prefill_split_workspace_bytes(n_docs, total_tokens, H);
  return 0;  // the fused kernel keeps every chunk's operands in LDS
}

hipError_t launch_prefill(const PrefillParams& p, const int32_t* cu_host, bool vec,
                          hipStream_t stream) {
  const int64_t blocks = int64_t(p.n_docs) * p.H;
  if (blocks == 0) return hipSuccess;
  if (blocks < kFusedMinChains) return launch_prefill_split(p, cu_host, vec, stream);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  // Longest documents first: their chains bound the makespan.
  DocOrder ord;
  ord.n = 0;
  if (p.n_docs <= kMaxOrderedDocs) {
    ord.n = p.n_docs;
    for (int d = 0; d < p.n_docs; ++d) ord.doc[d] = d;
    for (int i = 1; i < p.n_docs; ++i) {  // stable insertion sort, descending length
      const int d = ord.doc[i];
      const int32_t ld = cu_host[d + 1] - cu_host[d];
      int j = i - 1;
      while (j >= 0 && cu_host[ord.doc[j] + 1] - cu_host[ord.doc[j]] < ld) {
        ord.doc[j + 1] = ord.doc[j];
        --j;
      }
      ord.doc[j + 1] = d;
    }
  }
  // fp16 and fp8 states run on the vectorised path only (the host requires it)
  if (p.state_fmt != kStateBf16 && !vec) return hipErrorInvalidValue;
  const int gk = p.gate_mode & kGateKindMask;
  const void* fn = nullptr;
#define KDA_PF(V, G, S) reinterpret_cast<const void*>(&prefill_kernel<V, G, S>)
#define KDA_PF_G(V, S)                                                   \
  (gk == 0 ? KDA_PF(V, 0, S) : gk == 1 ? KDA_PF(V, 1, S) : gk == 4 ? KDA_PF(V, 4, S) \
                                                                   : KDA_PF(V, 5, S))
  if (p.state_fmt == kStateFp16) fn = KDA_PF_G(true, kStateFp16);
  else if (p.state_fmt == kStateFp8) fn = KDA_PF_G(true, kStateFp8);
  else if (vec) fn = KDA_PF_G(true, kStateBf16);
  else fn = KDA_PF_G(false, kStateBf16);
#define KDA_PF_ALL                                                                      \
  KDA_PF(true, 0, kStateBf16), KDA_PF(true, 1, kStateBf16), KDA_PF(true, 4, kStateBf16),     \
      KDA_PF(true, 5, kStateBf16), KDA_PF(true, 0, kStateFp16), KDA_PF(true, 1, kStateFp16), \
      KDA_PF(true, 4, kStateFp16), KDA_PF(true, 5, kStateFp16), KDA_PF(true, 0, kStateFp8),  \
      KDA_PF(true, 1, kStateFp8), KDA_PF(true, 4, kStateFp8), KDA_PF(true, 5, kStateFp8),    \
      KDA_PF(false, 0, kStateBf16), KDA_PF(false, 1, kStateBf16),                           \
      KDA_PF(false, 4, kStateBf16), KDA_PF(false, 5, kStateBf16)
  // the dynamic LDS limit of every instance is raised once per process
  static const hipError_t attr = [] {
    const void* fns[] = {KDA_PF_ALL};
    for (const void* f : fns) {
      const hipError_t e =
          hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (attr != hipSuccess) return attr;
#undef KDA_PF_ALL
#undef KDA_PF_G
#undef KDA_PF
  void* args[] = {const_cast<PrefillParams*>(&p), &ord};
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(blocks)), dim3(NTHR), args,
                         static_cast<size_t>(kLdsBytes), stream);
}

}  // namespace kda
