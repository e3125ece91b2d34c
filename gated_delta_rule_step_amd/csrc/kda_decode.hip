// T = 1 KDA decode against an in-place state pool (gfx950): bf16, fp16 or fp8
// e4m3 elements.
//
// Operation: "feat(kda): add packed-input CuTe decode kernel" (opening
// description and "T=1 fast path inside recurrent_kda"): per (row, head),
// decay the state per key channel, form u = beta (v - S' k_hat), write
// S = S' + k_hat u^T back in place and read out o = scale S q_hat. Rows whose
// slot index is outside [0, N) write zero output and touch nothing else.
//
// The kernel is HBM-bound (32 KiB read + 32 KiB written per head for ~115
// kflop), so the design is about streaming the state:
//  * one wave owns a tile of ROWS = 4 * LOADS value rows of one (row, head);
//    the tile, row, head and slot are wave-uniform, so addressing runs on
//    the scalar unit;
//  * lane l covers key channels 8*(l%16) .. +7 of value rows
//    vbase + 4*i + l/16 (i < LOADS): every state access is a 128-bit load or
//    store (64-bit with fp8 elements) and one load instruction covers four
//    full rows;
//  * the token inputs are loaded together with the slot index, the LOADS
//    state loads follow as soon as the index is known, and the prologue
//    (on the hardware exp/log) runs while the state is in flight; each
//    updated 4-row group is stored as soon as it is computed (holding all
//    stores back to the end measured ~15% slower);
//  * the two dot products S'k_hat and S'q_hat of a row are reduced over the
//    16 lanes of a DPP row (no LDS, no barrier); each state element takes one
//    multiply for the decay, two FMAs for the reductions and one FMA for the
//    update, and the read-out uses o = scale (S' q_hat + u (k_hat . q_hat));
//  * fp32 math, bf16 storage: unpack by shift/mask, repack with the hardware
//    round-to-nearest-even conversion; state traffic uses non-temporal hints.

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

// GK, the gate kind: kGatePrecomputed clear = raw gate logits (log-decay from
// A_log, dt_bias, lower_bound), set = the log-decay itself; kGatePerHead set =
// one gate value (and dt_bias) per head for all key channels.
// SF: the pool's element format (kStateBf16, kStateFp16, kStateFp8); the
// 16-bit formats move 8 elements per 128-bit access, fp8 per 64-bit access.
// A register budget that keeps at least five waves per SIMD (at most 96
// VGPRs; the allocation rounds to 8). The 8- and 16-row tiles need far
// fewer; the fp8 64-row tile holds twice the state words and keeps four.
template <int LOADS, int SF>
constexpr int kDecodeWaves = (SF == kStateFp8 && LOADS == 16) ? 4 : 5;

template <int LOADS, bool VEC, int GK, int SF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kDecodeWaves<LOADS, SF>)))
void decode_kernel(DecodeParams p, int group) {
  constexpr bool GRAW = !(GK & kGatePrecomputed);
  constexpr bool GHEAD = (GK & kGatePerHead) != 0;
  constexpr int ROWS = 4 * LOADS;
  constexpr int VBLOCKS = D / ROWS;
  const int lane = threadIdx.x & 63;
  // The tile, and with it the row, head and slot, is uniform over the wave:
  // said so with readfirstlane, the address arithmetic runs on the scalar
  // unit and the slot index is a scalar load.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Workgroups go to the eight XCDs round-robin by block index. The grid is a
  // multiple of 8 * group blocks, and block i runs logical block
  // (8*(k/group) + i%8)*group + k%group with k = i/8, so that every run of
  // `group` consecutive logical blocks shares one XCD: at least the two
  // workgroups of one head (16-row tiles), which then fetch the head's token
  // inputs into one L2, and with large batches all workgroups of one row, so
  // that an XCD works on an eighth of the slots at a time.
  const unsigned pb = blockIdx.x;
  const unsigned xk = pb >> 3, xg = xk / unsigned(group), xr = xk - xg * unsigned(group);
  const unsigned lb = (xg * 8u + (pb & 7u)) * unsigned(group) + xr;
  const int64_t tile = int64_t(lb) * (blockDim.x >> 6) + wave;
  const int vb = int(tile % VBLOCKS);
  const int64_t bh = tile / VBLOCKS;
  if (bh >= int64_t(p.B) * p.H) return;
  const int h = int(bh % p.H);
  const int64_t b = bh / p.H;
  const int kb = lane & 15;  // key channels 8*kb .. 8*kb+7
  const int rg = lane >> 4;  // row group: rows vbase + 4*i + rg
  const int vbase = vb * ROWS;

  uint16_t* outp = p.out + b * p.out_row_stride + int64_t(h) * D + vbase;
  const int32_t slot = p.state_indices[b];

  // The token inputs do not depend on the slot: their loads are issued before
  // the slot index is waited on, and before the state loads, so that the
  // prologue below runs while the state is still in flight (the memory
  // counter completes loads in issue order).
  const u32x4 qw = load8_bits<VEC>(p.q + b * p.q_row_stride + h * D + kb * 8);
  const u32x4 kw = load8_bits<VEC>(p.k + b * p.k_row_stride + h * D + kb * 8);
  u32x4 gw = {0u, 0u, 0u, 0u};
  uint16_t gh = 0;
  if constexpr (GHEAD) gh = p.g[b * p.g_row_stride + h];
  else gw = load8_bits<VEC>(p.g + b * p.g_row_stride + h * D + kb * 8);
  float dtb[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float alog = 0.f;
  if constexpr (GRAW) {
    if constexpr (GHEAD) {
      const float dh = p.dt_bias[h];
#pragma unroll
      for (int c = 0; c < 8; ++c) dtb[c] = dh;
    } else {
      load8_f32<VEC>(p.dt_bias + h * D + kb * 8, dtb);
    }
    alog = p.A_log[h];
  }
  const uint16_t bw = p.beta[b * p.beta_row_stride + h];
  uint16_t vw[LOADS];
  const uint16_t* vp = p.v + b * p.v_row_stride + h * D + vbase + rg;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) vw[i] = vp[4 * i];

  // Pin the token words in registers here: otherwise the compiler sinks their
  // loads below the branch, behind the wait for the slot index.
  asm volatile("" ::"v"(qw), "v"(kw), "v"(gw));

  if (!(slot >= 0 && int64_t(slot) < p.num_slots)) {
    if (lane < ROWS) outp[lane] = 0;
    return;
  }

  // State loads.
  static_assert(VEC || SF == kStateBf16, "fp16 and fp8 states use the vectorised layout");
  const int64_t se = int64_t(slot) * p.slot_stride + int64_t(h) * HEAD_ELEMS +
                     int64_t(vbase + rg) * D + kb * 8;  // element offset
  uint16_t* sp = static_cast<uint16_t*>(p.state_pool) + se;  // 16-bit formats
  St8<SF> s[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    if constexpr (SF == kStateFp8) s[i] = st8_load_nt<SF>(p.state_pool, se + i * 4 * D);
    else s[i] = load8_raw<VEC>(sp + i * 4 * D);
  }

  // Per-token prologue for this lane's 8 key channels, on the hardware
  // exponential and logarithm (about 1 ulp in fp32).
  float q[8], k[8], gr[8];
  unpack8_bf16(qw, q);
  unpack8_bf16(kw, k);
  if constexpr (GHEAD) {
#pragma unroll
    for (int c = 0; c < 8; ++c) gr[c] = bf1(gh);
  } else {
    unpack8_bf16(gw, gr);
  }
  const float neg_ea = GRAW ? -fexp(alog) : 0.f;
  const float braw = bf1(bw);
  const float beta = (p.gate_mode & kBetaPresigmoid) ? braw : fsigmoid(braw);
  float vrow[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) vrow[i] = bf1(vw[i]);

  float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    sq = fmaf(q[c], q[c], sq);
    sk = fmaf(k[c], k[c], sk);
    sqk = fmaf(q[c], k[c], sqk);
  }
  sq = row16_sum(sq);
  sk = row16_sum(sk);
  sqk = row16_sum(sqk);
  const float rq = 1.0f / sqrtf(sq + 1e-6f);
  const float rk = 1.0f / sqrtf(sk + 1e-6f);
  const float kq = sqk * rq * rk;  // k_hat . q_hat
  float al[8], kh[8], qh[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    al[c] = fexp(GRAW ? fgate(gr[c] + dtb[c], neg_ea, p.lower_bound)
                      : gate_given(gr[c], p.lower_bound));
    kh[c] = k[c] * rk;
    qh[c] = q[c] * rq;
  }

  float osel = 0.f;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    float x[8];
    st8_unpack<SF>(s[i], x);
    // the decayed row S' = alpha * S, then both dot products from it
    float dk = 0.f, dq = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      x[c] *= al[c];
      dk = fmaf(x[c], kh[c], dk);
      dq = fmaf(x[c], qh[c], dq);
    }
    dk = row16_sum(dk);
    dq = row16_sum(dq);
    const float u = beta * (vrow[i] - dk);
    const float o = p.scale * fmaf(u, kq, dq);
    if (kb == i) osel = o;
    float a[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) a[c] = fmaf(kh[c], u, x[c]);
    const St8<SF> w = st8_pack<SF>(a);
    if constexpr (SF == kStateFp8) st8_store_nt<SF>(p.state_pool, se + i * 4 * D, w);
    else store8_raw<VEC>(sp + i * 4 * D, w);
  }
  if (kb < LOADS) outp[4 * kb + rg] = to_bf16(osel);
}

// Launch shape: 256-thread workgroups of four independent waves. A wave
// lives for one tile, so the bytes in flight per CU grow with the waves a
// SIMD holds: 16-row tiles (4 loads per lane, ~67 VGPRs, seven waves per
// SIMD) streamed the B = 512 pool ~4% faster than 32-row tiles at five
// waves, and as fast at B = 128. Up to 64 heads take 8-row tiles (2 loads)
// so that a few heads still spread over many CUs. fp8 states move 8 bytes
// per load; from 4096 heads they take 64-row tiles (16 loads of 8 bytes,
// the same 32 registers of state per wave as the 32-row bf16 tile), which
// measured faster than 16- or 32-row fp8 tiles.
hipError_t launch_decode(const DecodeParams& p, bool vec, hipStream_t stream) {
  const int64_t heads = int64_t(p.B) * p.H;
  const bool fp8 = p.state_fmt == kStateFp8;
  const int size = heads <= 64 ? 0 : (fp8 && heads >= 4096 ? 2 : 1);
  const int loads = size == 0 ? 2 : (size == 1 ? 4 : 16);
  const int64_t tiles = heads * (D / (4 * loads));
  // XCD groups (see the kernel): one row's workgroups from 64 rows on with
  // 16-bit states (B = 512: 70.7 against 72.1 us for head pairs; neutral at
  // B = 128, 3 % slower for fp8 at B = 128), else head pairs. Padding blocks
  // exit at once.
  const int64_t row_blocks = int64_t(p.H) * (D / (4 * loads)) / 4;
  const int group =
      (!fp8 && p.B >= 64 && row_blocks > 2 && row_blocks <= 4096) ? int(row_blocks) : 2;
  const int64_t blocks = ((tiles + 3) / 4 + 8 * group - 1) / (8 * group) * (8 * group);
  if (tiles == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const int gk = p.gate_mode & kGateKindMask;
#define KDA_DECODE_LAUNCH(L, V, F)                                                              \
  do {                                                                                          \
    switch (gk) {                                                                               \
      case 0: hipLaunchKernelGGL((decode_kernel<L, V, 0, F>), grid, block, 0, stream, p, group); break; \
      case 1: hipLaunchKernelGGL((decode_kernel<L, V, 1, F>), grid, block, 0, stream, p, group); break; \
      case 4: hipLaunchKernelGGL((decode_kernel<L, V, 4, F>), grid, block, 0, stream, p, group); break; \
      default: hipLaunchKernelGGL((decode_kernel<L, V, 5, F>), grid, block, 0, stream, p, group);      \
    }                                                                                           \
  } while (0)
#define KDA_DECODE_SIZES(V, F)                 \
  do {                                         \
    if (size == 0) KDA_DECODE_LAUNCH(2, V, F); \
    else KDA_DECODE_LAUNCH(4, V, F);           \
  } while (0)
  // fp16 and fp8 states run on the vectorised path only (the host requires it)
  if (p.state_fmt != kStateBf16 && !vec) return hipErrorInvalidValue;
  if (p.state_fmt == kStateFp16) {
    KDA_DECODE_SIZES(true, kStateFp16);
  } else if (fp8) {
    if (size == 2) KDA_DECODE_LAUNCH(16, true, kStateFp8);
    else KDA_DECODE_SIZES(true, kStateFp8);
  } else if (vec) {
    KDA_DECODE_SIZES(true, kStateBf16);
  } else {
    KDA_DECODE_SIZES(false, kStateBf16);
  }
#undef KDA_DECODE_SIZES
#undef KDA_DECODE_LAUNCH
  return hipGetLastError();
}

}  // namespace kda
