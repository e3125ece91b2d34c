// Device helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int D = 128;             // head dimension (K = V = 128)
constexpr int HEAD_ELEMS = D * D;  // one head's state, elements

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// A state word of two elements, bf16 or (SF16) fp16.
template <bool SF16>
__device__ __forceinline__ float st_lo(uint32_t w) { return SF16 ? f16_lo(w) : bf_lo(w); }
template <bool SF16>
__device__ __forceinline__ float st_hi(uint32_t w) { return SF16 ? f16_hi(w) : bf_hi(w); }
template <bool SF16>
__device__ __forceinline__ uint32_t st_pack(float lo, float hi) {
  return SF16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
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
