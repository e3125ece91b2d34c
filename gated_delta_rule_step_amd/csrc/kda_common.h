// Device helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

constexpr int D = 128;             // head dimension (K = V = 128)
constexpr int HEAD_ELEMS = D * D;  // one head's state, elements

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Buffer resources (raw, gfx9 family descriptor word 3) and the cache-policy
// bits of a buffer store that mark it non-temporal.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kStoreNontemporal = 2;

// ---------------------------------------------------------------------------
// bf16 <-> fp32. Widening is exact (bits move to the top half). Narrowing uses
// the gfx950 hardware conversion v_cvt_pk_bf16_f32 (round to nearest even),
// the rounding the state, ring and outputs are stored with.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf1(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 x = {lo, hi};
  bf16x2 r = __builtin_convertvector(x, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t to_bf16(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.0f) & 0xffffu);
}

// fp16 (binary16) state elements: widening is exact (v_cvt_f32_f16);
// narrowing is v_cvt_pk_f16_f32, round to nearest even.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
}

// fp8 e4m3 state elements (the OCP e4m3fn format: bias 7, largest finite
// 448, no infinities). Widening is exact (v_cvt_pk_f32_fp8); narrowing is
// v_cvt_pk_fp8_f32, round to nearest even, after a clamp to +-448 with
// v_med3_f32, so that an out-of-range value saturates instead of becoming NaN.
__device__ __forceinline__ f32x2 f8x2_lo(uint32_t w) {  // bytes 0, 1
  return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
}
__device__ __forceinline__ f32x2 f8x2_hi(uint32_t w) {  // bytes 2, 3
  return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
}
__device__ __forceinline__ float f8_sat(float x) { return __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f); }
__device__ __forceinline__ uint32_t pack_f8x4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(f8_sat(a), f8_sat(b), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(f8_sat(c), f8_sat(d), r, true);
  return static_cast<uint32_t>(r);
}
// Two fp32 values that are exactly bf16 (e.g. widened fp8) as a bf16 pair:
// the top halves of both words, one v_perm_b32.
__device__ __forceinline__ uint32_t pack_bf16x2_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// ---------------------------------------------------------------------------
// State element formats: bf16, fp16 or fp8 e4m3 (the state_dtype argument).
constexpr int kStateBf16 = 0;
constexpr int kStateFp16 = 1;
constexpr int kStateFp8 = 2;
template <int SF>
constexpr int kStateBytes = SF == kStateFp8 ? 1 : 2;

// A state word of two elements, bf16 or fp16.
template <int SF>
__device__ __forceinline__ float st_lo(uint32_t w) {
  static_assert(SF != kStateFp8, "two-element words hold 16-bit formats");
  return SF == kStateFp16 ? f16_lo(w) : bf_lo(w);
}
template <int SF>
__device__ __forceinline__ float st_hi(uint32_t w) {
  static_assert(SF != kStateFp8, "two-element words hold 16-bit formats");
  return SF == kStateFp16 ? f16_hi(w) : bf_hi(w);
}
template <int SF>
__device__ __forceinline__ uint32_t st_pack(float lo, float hi) {
  static_assert(SF != kStateFp8, "two-element words hold 16-bit formats");
  return SF == kStateFp16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}

// Eight consecutive state elements: 16 bytes (bf16, fp16) or 8 bytes (fp8).
template <int SF>
using St8 = typename std::conditional<SF == kStateFp8, u32x2, u32x4>::type;

template <int SF>
__device__ __forceinline__ void st8_unpack(St8<SF> w, float (&x)[8]) {
  if constexpr (SF == kStateFp8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f32x2 a = f8x2_lo(w[i]), b = f8x2_hi(w[i]);
      x[4 * i] = a[0];
      x[4 * i + 1] = a[1];
      x[4 * i + 2] = b[0];
      x[4 * i + 3] = b[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = st_lo<SF>(w[i]);
      x[2 * i + 1] = st_hi<SF>(w[i]);
    }
  }
}

template <int SF>
__device__ __forceinline__ St8<SF> st8_pack(const float (&x)[8]) {
  St8<SF> w;
  if constexpr (SF == kStateFp8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) w[i] = pack_f8x4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = st_pack<SF>(x[2 * i], x[2 * i + 1]);
  }
  return w;
}

// Non-temporal loads and stores of 8 state elements at element offset `e`
// (aligned to 8 elements: the vectorised layout).
template <int SF>
__device__ __forceinline__ St8<SF> st8_load_nt(const void* base, int64_t e) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const St8<SF>*>(static_cast<const uint8_t*>(base) + e * kStateBytes<SF>));
}
template <int SF>
__device__ __forceinline__ void st8_store_nt(void* base, int64_t e, St8<SF> w) {
  __builtin_nontemporal_store(
      w, reinterpret_cast<St8<SF>*>(static_cast<uint8_t*>(base) + e * kStateBytes<SF>));
}
template <int SF>
__device__ __forceinline__ void st8_store(void* base, int64_t e, St8<SF> w) {
  *reinterpret_cast<St8<SF>*>(static_cast<uint8_t*>(base) + e * kStateBytes<SF>) = w;
}

// 8 consecutive bf16 -> 8 floats; VEC: one 128-bit load (16-byte aligned).
template <bool VEC>
__device__ __forceinline__ void load8_bf16(const uint16_t* p, float (&x)[8]) {
  if constexpr (VEC) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf_lo(w[i]);
      x[2 * i + 1] = bf_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = bf1(p[i]);
  }
}

// 8 consecutive bf16 as raw bits (plain loads: token inputs, shared by the
// waves of a head through L2), and their widening to fp32.
template <bool VEC>
__device__ __forceinline__ u32x4 load8_bits(const uint16_t* p) {
  if constexpr (VEC) {
    return *reinterpret_cast<const u32x4*>(p);
  } else {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = uint32_t(p[2 * i]) | (uint32_t(p[2 * i + 1]) << 16);
    return w;
  }
}
__device__ __forceinline__ void unpack8_bf16(u32x4 w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf_lo(w[i]);
    x[2 * i + 1] = bf_hi(w[i]);
  }
}

template <bool VEC>
__device__ __forceinline__ u32x4 load8_raw(const uint16_t* p) {
  if constexpr (VEC) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  } else {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = uint32_t(p[2 * i]) | (uint32_t(p[2 * i + 1]) << 16);
    return w;
  }
}

template <bool VEC>
__device__ __forceinline__ void store8_raw(uint16_t* p, u32x4 w) {
  if constexpr (VEC) {
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[2 * i] = static_cast<uint16_t>(w[i] & 0xffffu);
      p[2 * i + 1] = static_cast<uint16_t>(w[i] >> 16);
    }
  }
}

template <bool VEC>
__device__ __forceinline__ void load8_f32(const float* p, float (&x)[8]) {
  if constexpr (VEC) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = p[i];
  }
}

// ---------------------------------------------------------------------------
// Cross-lane sums inside one 16-lane DPP row. xor-1 and xor-2 quad
// permutations make each quad uniform, then the half-row and row mirrors fold
// quads and halves; every lane of the row ends with the row total.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

// ---------------------------------------------------------------------------
// Per-token scalar pieces of the prologue (fp32).
// Log-decay of one key channel: max(lb, -exp(A_log) * softplus(x)),
// x = raw gate + dt_bias; softplus(x) = log1p(exp(x)), or x above 20.
__device__ __forceinline__ float gate_logdecay(float x, float neg_exp_alog, float lb) {
  const float sp = x > 20.0f ? x : log1pf(expf(x));
  return fmaxf(lb, neg_exp_alog * sp);
}
__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + expf(-x)); }

// The same pieces on the hardware transcendentals (v_exp_f32 / v_log_f32,
// base 2, ~1 ulp), for the kernels whose prologue sits on the critical path.
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }
__device__ __forceinline__ float fgate(float x, float neg_exp_alog, float lb) {
  const float sp = x > 20.0f ? x : LN2 * __builtin_amdgcn_logf(1.0f + fexp(x));
  return fmaxf(lb, neg_exp_alog * sp);
}
__device__ __forceinline__ float fsigmoid(float x) { return 1.0f / (1.0f + fexp(-x)); }

// Pre-computed gate: the given log-decay, clamped into [lb, 0] (the range the
// raw gate lands in).
__device__ __forceinline__ float gate_given(float g, float lb) {
  return fminf(0.0f, fmaxf(lb, g));
}

}  // namespace kda
