// Speculative-decode verify with the (k_hat, u, G) ring and the fold into the
// checkpoint (gfx950).
//
// Operation: "feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3
// (KDA)", sections "What it does", "API" and "Caching". One workgroup (four
// waves) owns one (row, head). With S_cur the state the ring stands for,
//   S_cur = diag(exp(G_L)) S_ckpt + sum_{j<hist} diag(exp(G_L - G_j)) k_j u_j^T,
// the T draft tokens are processed as one chunk of the chunkwise (WY) form of
// the recurrence instead of T sequential state updates:
//   Gam_t  = g_0 + ... + g_t                        (per key channel)
//   A[r,j] = sum_c k_r k_j exp(Gam_r - Gam_j)        (j < r)
//   P[r,j] = sum_c q_r k_j exp(Gam_r - Gam_j)        (j <= r)
//   W      = (I + diag(beta) A)^-1 diag(beta) (exp(Gam) * K)
//   U0     = (I + diag(beta) A)^-1 diag(beta) V
//   u_t    = U0_t - (W S_cur)_t                      (the per-token corrections)
//   o_t    = scale * ((exp(Gam_t) * q_t) S_cur + sum_{j<=t} P[t,j] u_j)
// ("S k" is the state applied to a key vector, as in u = beta (v - S k).)
// S_cur only enters through X S_cur with X = [W; exp(Gam) * Q], so the replay
// is never materialised for the outputs:
//   X S_cur = (X * exp(G_L)) S_ckpt + C U_hist,  C[m,j] = X_m . (exp(G_L - G_j) * k_j).
// (X * exp(G_L)) S_ckpt is the only product with the full 128 x 128 state. The
// checkpoint is exact in bf16, so it feeds v_mfma_f32_16x16x32_bf16 directly
// as the B operand (128-bit loads straight into B fragments); the fp32 left
// operand is split into bf16 hi + lo parts (two MFMAs into one fp32
// accumulator, ~2^-17 relative error). Everything else is small and runs on
// the VALU in fp32. A folding row also materialises S_cur element-wise (fp32)
// and stores it in bf16 over the checkpoint.
//
// Prologue cost matters as much as the state stream here, so:
//  * transcendentals use the hardware v_exp_f32 / v_log_f32;
//  * when T * |lower_bound| < 80 every exp(Gam_r - Gam_j) factors into
//    exp(Gam_r) * exp(-Gam_j) (both finite in fp32), so the Gram products are
//    plain FMAs over precomputed rows (FACT); otherwise each weight is one
//    exp of a difference;
//  * a 16-lane group reads 4 + 4 channels per lane (two 256-byte runs per
//    row), which keeps LDS accesses free of bank conflicts;
//  * ring rows wrap by one conditional subtraction (base < R and
//    hist + T <= R).

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 f16x8 __attribute__((__vector_size__(8 * sizeof(__fp16))));  // MFMA f16 operand

constexpr int TMAX = 8;
// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8) for vmcnt(8), the other counters unconstrained: all but
// the newest 8 vector-memory operations (the checkpoint loads) have completed.
constexpr int kVmcntBehindCheckpoint = 8 | (7 << 4) | (15 << 8);
// Token rows (and the MFMA result rows that reuse them) are padded to XS
// floats: rows 4 apart, or 16 rows read by one fragment load, then fall on
// different banks.
constexpr int XS = D + 4;

// LDS layout (floats unless noted); hm = history capacity (w_ring - T).
struct Smem {
  float* qa;      // [TMAX][XS] q_hat, then exp(Gam) * q_hat           (X rows T..2T-1)
  float* ka;      // [TMAX][XS] k_hat, then exp(Gam) * k_hat, then W    (X rows 0..T-1)
  float* kb;      // [TMAX][XS] g, then Gam, then exp(-Gam) * k_hat (FACT)
  float* vv;      // [TMAX][XS] v, then U0
  float* y;       // [2*TMAX][XS] MFMA result rows (over qa and ka)
  float* am;      // [TMAX][TMAX]
  float* pm;      // [TMAX][TMAX]
  float* beta;    // [TMAX]
  float* egl;     // [D] exp(G_L)
  float* cm;      // [2*TMAX][hm]
  // History rows j < hm, 1 KiB each (kHistF floats): G_j, then
  // exp(G_L - G_j) * k_j (fp32, in place) | k_j (bf16 bits, as read from the
  // ring) | u_j (bf16 bits). One 16-byte direct-to-LDS load per lane moves a
  // whole row.
  float* dh;      // row j at dh + j * kHistF
  uint16_t* kr;   // row j at kr + j * kHistU
  uint16_t* uh;   // row j at uh + j * kHistU
};
constexpr int kHistF = 256;  // floats per history row (1 KiB)
constexpr int kHistU = 512;  // 16-bit words per history row

__host__ __device__ inline size_t smem_bytes(int hm) {
  const size_t f = size_t(4) * TMAX * XS + 2 * TMAX * TMAX + TMAX + D + size_t(2 * TMAX) * hm +
                   size_t(hm) * kHistF;
  return f * 4;
}

__device__ inline Smem carve(float* base, int hm) {
  Smem s;
  float* p = base;
  s.qa = p; p += TMAX * XS;
  s.ka = p; p += TMAX * XS;
  s.y = s.qa;
  s.kb = p; p += TMAX * XS;
  s.vv = p; p += TMAX * XS;
  s.am = p; p += TMAX * TMAX;
  s.pm = p; p += TMAX * TMAX;
  s.beta = p; p += TMAX;
  s.egl = p; p += D;
  s.cm = p; p += 2 * TMAX * hm;
  // 16-byte aligned: 4 * TMAX * XS + 2 * TMAX * TMAX + TMAX + D and 2 * TMAX
  // floats are multiples of 4
  s.dh = p;
  s.kr = reinterpret_cast<uint16_t*>(p + D);
  s.uh = reinterpret_cast<uint16_t*>(p + D) + D;
  return s;
}

template <bool VEC>
__device__ __forceinline__ u32x2 load4_raw(const uint16_t* p) {
  if constexpr (VEC) {
    return *reinterpret_cast<const u32x2*>(p);
  } else {
    return u32x2{uint32_t(p[0]) | (uint32_t(p[1]) << 16), uint32_t(p[2]) | (uint32_t(p[3]) << 16)};
  }
}

template <bool VEC>
__device__ __forceinline__ f32x4 load4_f32(const float* p) {
  if constexpr (VEC) return *reinterpret_cast<const f32x4*>(p);
  else return f32x4{p[0], p[1], p[2], p[3]};
}

// The 8 channels of lane kb (0..15) inside a 16-lane group: 4kb..4kb+3 and
// 64+4kb..64+4kb+3.
__device__ __forceinline__ int chan(int kb, int half) { return half * 64 + 4 * kb; }

__device__ __forceinline__ void lds_read8(const float* row, int kb, float* x) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(row + chan(kb, 0));
  const f32x4 b = *reinterpret_cast<const f32x4*>(row + chan(kb, 1));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

}  // namespace

// Raw token inputs of one item: thread tid covers token tid / 32 (T <= 8),
// channels 4 (tid % 32) .. +3.
struct TokRegs {
  u32x2 q, k, g, v;
  f32x4 dtb;
  uint32_t braw;
};

template <bool VEC, int GK>
__device__ __forceinline__ void load_tokens(const VerifyParams& p, int64_t item, int tid,
                                            TokRegs& r) {
  constexpr bool GRAW = !(GK & kGatePrecomputed);
  constexpr bool GHEAD = (GK & kGatePerHead) != 0;
  const int h = int(item % p.H);
  const int64_t b = item / p.H;
  const int t = tid >> 5, c = 4 * (tid & 31);
  if (t < p.T) {
    r.q = load4_raw<VEC>(p.q + b * p.q_row_stride + t * p.q_tok_stride + h * D + c);
    r.k = load4_raw<VEC>(p.k + b * p.k_row_stride + t * p.k_tok_stride + h * D + c);
    if constexpr (GHEAD) {  // one gate value per head, in all four channel slots
      const uint32_t gh = p.g[b * p.g_row_stride + t * p.g_tok_stride + h];
      r.g = u32x2{gh | (gh << 16), gh | (gh << 16)};
    } else {
      r.g = load4_raw<VEC>(p.g + b * p.g_row_stride + t * p.g_tok_stride + h * D + c);
    }
    r.v = load4_raw<VEC>(p.v + b * p.v_row_stride + t * p.v_tok_stride + h * D + c);
    if constexpr (!GRAW) {
      r.dtb = f32x4{0.f, 0.f, 0.f, 0.f};
    } else if constexpr (GHEAD) {
      const float dh = p.dt_bias[h];
      r.dtb = f32x4{dh, dh, dh, dh};
    } else {
      r.dtb = load4_f32<VEC>(p.dt_bias + h * D + c);
    }
    r.braw = p.beta[b * p.beta_row_stride + t * p.beta_tok_stride + h];
  }
}

// Grid: one 256-thread workgroup per item (row, head), item = row * H + head.
// GK, the gate kind: kGatePrecomputed clear = raw gate logits, set = the
// log-decay itself; kGatePerHead set = one gate value per head. SF: the
// checkpoint format. fp16 checkpoints make the product below run on
// v_mfma_f32_16x16x32_f16 with fp16 hi / lo A fragments; fp8 checkpoints are
// widened to bf16 (exactly) as B fragments of the bf16 product. The rings
// stay bf16.
template <bool VEC, bool FACT, int GK, int SF, bool DEEP>
__global__ __launch_bounds__(256) void verify_kernel(VerifyParams p, int hm) {
  constexpr bool GRAW = !(GK & kGatePrecomputed);
  constexpr int MF = SF == kStateFp16 ? kStateFp16 : kStateBf16;  // MFMA operand format
  static_assert(VEC || SF == kStateBf16, "fp16 and fp8 checkpoints use the vectorised layout");
  extern __shared__ __align__(16) float smem_raw[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int T = p.T;
  const int R = p.ring_rows;
  const int64_t item = blockIdx.x;
  const int h = int(item % p.H);
  const int64_t b = item / p.H;
  const int fv = lane & 15, fk = (lane >> 4) * 8;
  const int kb = lane & 15;

  const int32_t slot = p.state_indices[b];
  const int hist = p.hist_len[b];
  const int base = p.cache_base[b];
  // hist <= w_ring - T rather than hist + T <= w_ring: a hist_len near
  // INT32_MAX must not wrap into an active row
  const bool active = slot >= 0 && int64_t(slot) < p.num_slots && hist >= 0 &&
                      hist <= p.w_ring - T && base >= 0 && base < R;
  uint16_t* outb = p.out + b * p.out_row_stride + int64_t(h) * D;
  if (!active) {
    for (int e = tid; e < T * D; e += 256) outb[int64_t(e >> 7) * p.out_tok_stride + (e & 127)] = 0;
    return;
  }
  Smem s = carve(smem_raw, hm);
  const float neg_ea = GRAW ? -fexp(p.A_log[h]) : 0.f;
  // Token words first; every global load phases 2-5 need is issued before
  // the checkpoint loads (the memory counter is in order: waiting on a load
  // issued after them would also wait for the 32 KiB checkpoint read).
  TokRegs tk;
  load_tokens<VEC, GK>(p, item, tid, tk);
  const bool fold = hist + T >= p.flush_min;
  const int64_t sh = int64_t(slot) * p.H + h;
  // the checkpoint: element offset ce; ckpt addresses the 16-bit formats
  const int64_t ce = int64_t(slot) * p.slot_stride + int64_t(h) * HEAD_ELEMS;
  uint16_t* ckpt = static_cast<uint16_t*>(p.state_pool) + int64_t(slot) * p.slot_stride +
                   int64_t(h) * HEAD_ELEMS;
  uint16_t* kc = p.k_cache + sh * R * D;
  uint16_t* uc = p.u_cache + sh * R * D;
  float* gc = p.g_cache + sh * R * D;
  // ring row of history / draft position j (0 <= j < hist + T <= R, base < R)
  auto ring_row = [&](int j) { const int r = base + j; return r >= R ? r - R : r; };

  St8<SF> sf[2][4];
  // ---- 2. per-token prologue (token t on lanes 32 t .. 32 t + 31, four
  // channels per lane), run while the checkpoint B fragments stream in (wave
  // w owns value columns 32w .. 32w+31 in two 16-column blocks; fragment
  // (blk, st) holds v = 32w + 16*blk + lane%16, key channels
  // 32*st + 8*(lane/16) .. +7).
  // History rows j < hist go straight from the ring into LDS (no register
  // destinations), one row per instruction: lanes 0-31 move G_j (512 B),
  // lanes 32-47 k_j and lanes 48-63 u_j (256 B each), 16 bytes per lane, into
  // the row's 1 KiB LDS block; wave w takes rows j = w mod 4. Like every
  // other load of the item they are issued before the checkpoint loads and
  // covered by the explicit vmcnt(8) at the start of the prologue math (and
  // the barrier after it, for the rows of the other waves).
  if constexpr (VEC) {
    const float* src_g = gc + 4 * lane;
    const uint16_t* src_k = (lane < 48 ? kc : uc) + 8 * (lane & 15);
    for (int j = wave; j < hist; j += 4) {
      const int64_t row = ring_row(j);
      const void* src = lane < 32 ? static_cast<const void*>(src_g + row * D)
                                  : static_cast<const void*>(src_k + row * D);
      __builtin_amdgcn_global_load_lds(src, s.dh + j * kHistF, 16, 0, 0);
    }
  }
  // G_{hist-1} of key channel tid % 128 (phase 3).
  float gl = 0.f;
  if (hist > 0) gl = gc[int64_t(ring_row(hist - 1)) * D + (tid & 127)];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int st = 0; st < 4; ++st)
      if constexpr (SF == kStateFp8)
        sf[blk][st] = st8_load_nt<SF>(p.state_pool,
                                      ce + int64_t(32 * wave + 16 * blk + fv) * D + 32 * st + fk);
      else
        sf[blk][st] = load8_raw<VEC>(ckpt + int64_t(32 * wave + 16 * blk + fv) * D + 32 * st + fk);
  __builtin_amdgcn_sched_barrier(0);
  {
    const int t = tid >> 5, c0 = 4 * (tid & 31);
    // Every load but the 8 checkpoint loads is complete from here on. The
    // token words are used only through an OR with an opaque zero defined
    // here, so no use of them is hoisted above the checkpoint loads (where
    // waiting for them would delay that read).
    __builtin_amdgcn_s_waitcnt(kVmcntBehindCheckpoint);
    uint32_t zero = 0;
    __asm__ volatile("" : "+v"(zero));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      tk.q[i] |= zero;
      tk.k[i] |= zero;
      tk.g[i] |= zero;
      tk.v[i] |= zero;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) tk.dtb[i] = __uint_as_float(__float_as_uint(tk.dtb[i]) | zero);
    tk.braw |= zero;
    if (t < T) {
      float q[4], k[4], gr[4], vv[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        q[2 * i] = bf_lo(tk.q[i]);
        q[2 * i + 1] = bf_hi(tk.q[i]);
        k[2 * i] = bf_lo(tk.k[i]);
        k[2 * i + 1] = bf_hi(tk.k[i]);
        gr[2 * i] = bf_lo(tk.g[i]);
        gr[2 * i + 1] = bf_hi(tk.g[i]);
        vv[2 * i] = bf_lo(tk.v[i]);
        vv[2 * i + 1] = bf_hi(tk.v[i]);
      }
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sq = fmaf(q[c], q[c], sq);
        sk = fmaf(k[c], k[c], sk);
      }
      sq = row16_sum(sq);
      sk = row16_sum(sk);
      sq += __shfl_xor(sq, 16);
      sk += __shfl_xor(sk, 16);
      const float rq = 1.0f / sqrtf(sq + 1e-6f);
      const float rk = 1.0f / sqrtf(sk + 1e-6f);
      f32x4 qn, kn, gn, vn;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        qn[c] = q[c] * rq;
        kn[c] = k[c] * rk;
        gn[c] = GRAW ? fgate(gr[c] + tk.dtb[c], neg_ea, p.lower_bound)
                     : gate_given(gr[c], p.lower_bound);
        vn[c] = vv[c];
      }
      *reinterpret_cast<f32x4*>(s.qa + t * XS + c0) = qn;
      *reinterpret_cast<f32x4*>(s.ka + t * XS + c0) = kn;
      *reinterpret_cast<f32x4*>(s.kb + t * XS + c0) = gn;
      *reinterpret_cast<f32x4*>(s.vv + t * XS + c0) = vn;
      if ((tid & 31) == 0) {
        const float braw = bf1(uint16_t(tk.braw));
        s.beta[t] = (p.gate_mode & kBetaPresigmoid) ? braw : fsigmoid(braw);
      }
    }
  }
  __syncthreads();

  // ---- 3. two threads own key channel c (tokens split by parity): the
  // ring's k_hat rows, Gam_t (from 0) and the ring's
  // G_t = G_base + g_0 + ... + g_t in token order (G_base = 0 when folding,
  // else G_{hist-1}); exp(G_L); with FACT the rows exp(Gam) * q, exp(Gam) * k
  // and exp(-Gam) * k. Threads 128..255 also stage the live history rows:
  // D_j = exp(G_L - G_j) * k_j (fp32) and u_j (bf16). History rows
  // (j < hist) and draft rows (hist .. hist+T-1) never coincide. (These
  // history loads come after the checkpoint read, so a row with history
  // waits for it here.)
  {
    const int c = tid & 127;
    const int half = tid >> 7;  // tokens t with t % 2 == half
    // Both threads of a channel read its whole gate column before either
    // rewrites the rows (barrier below).
    float gcol[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) gcol[t] = t < T ? s.kb[t * XS + c] : 0.f;
    if (half == 1 && hist > 0) {
      if constexpr (VEC) {
        // the history rows are in LDS (waited for in phase 2, barrier above)
        for (int j = 0; j < hist; ++j)
          s.dh[j * kHistF + c] = fexp(gl - s.dh[j * kHistF + c]) * bf1(s.kr[j * kHistU + c]);
      } else {
        for (int j = 0; j < hist; ++j) {
          const int64_t row = ring_row(j);
          s.dh[j * kHistF + c] = fexp(gl - gc[row * D + c]) * bf1(kc[row * D + c]);
          s.uh[j * kHistU + c] = uc[row * D + c];
        }
      }
    }
    __syncthreads();
    if (half == 0) s.egl[c] = fexp(gl);
    float gam = 0.f, gacc = fold ? 0.f : gl;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        gam += gcol[t];
        gacc += gcol[t];
        if ((t & 1) == half) {
          const int64_t row = ring_row(hist + t);
          const float kh = s.ka[t * XS + c];
          __builtin_nontemporal_store(gacc, gc + row * D + c);
          // (stored here rather than in phase 2: a store there makes the
          // compiler wait on the checkpoint loads before the next barrier)
          __builtin_nontemporal_store(to_bf16(kh), kc + row * D + c);
          if constexpr (FACT) {
            const float ea = fexp(gam), eb = fexp(-gam);
            s.qa[t * XS + c] *= ea;
            s.ka[t * XS + c] = kh * ea;
            s.kb[t * XS + c] = kh * eb;
          } else {
            s.kb[t * XS + c] = gam;
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- 3b. fold: S_cur = exp(G_L) * S_ckpt + sum_j u_j D_j over this wave's
  // fragments, stored in the state format over the checkpoint. It needs only the
  // checkpoint fragments, exp(G_L), D_j and u_j, all ready here, so its stores
  // drain while phases 4-7 run. (The checkpoint fragments stay in registers
  // for phase 6.) With no history S_cur is the checkpoint itself and nothing
  // is rewritten.
  if (fold && hist > 0) {
    // the head's checkpoint as a buffer range (non-temporal stores)
    const __amdgpu_buffer_rsrc_t fold_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint8_t*>(p.state_pool) + ce * kStateBytes<SF>, 0, HEAD_ELEMS * kStateBytes<SF>,
        kBufferWord3);
    // DEEP (rings holding 16 or more history rows): with hist >= 8 the sum
    // over the history rows, sum_j u_j D_j, runs on MFMA as one K = 32 step
    // (rows j >= hist zero on both sides): A = D^T with its 16 rows permuted
    // so that row m is key channel 32 st + 8 (m / 4) + 4 half + m % 4, split
    // into three bf16 terms (24 significant bits), B = the ring's u rows
    // (bf16, exact). The result lands in each lane's own checkpoint row and
    // key channels 32 st + fk + 4 half + i, the layout of the fragments.
    f32x4 hs[2][4][2];
    const bool mfma_hist = DEEP && hist >= 8;
    if constexpr (DEEP) {
      if (mfma_hist) {
        bf16x8 ub[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const int v = 32 * wave + 16 * blk + fv;
          u32x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = fk + 2 * i;
            const uint32_t u0 = j < hist ? s.uh[j * kHistU + v] : 0u;
            const uint32_t u1 = j + 1 < hist ? s.uh[(j + 1) * kHistU + v] : 0u;
            w[i] = u0 | (u1 << 16);
          }
          ub[blk] = __builtin_bit_cast(bf16x8, w);
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int kk = 32 * st + 8 * (fv >> 2) + 4 * half + (fv & 3);
            float a[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int j = fk + e;
              a[e] = j < hist ? s.dh[j * kHistF + kk] : 0.f;
            }
            u32x4 t1, t2, t3;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              t1[i] = pack_bf16x2(a[2 * i], a[2 * i + 1]);
              const float r0 = a[2 * i] - bf_lo(t1[i]), r1 = a[2 * i + 1] - bf_hi(t1[i]);
              t2[i] = pack_bf16x2(r0, r1);
              t3[i] = pack_bf16x2(r0 - bf_lo(t2[i]), r1 - bf_hi(t2[i]));
            }
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, t1);
            const bf16x8 a2 = __builtin_bit_cast(bf16x8, t2);
            const bf16x8 a3 = __builtin_bit_cast(bf16x8, t3);
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
              f32x4 acc = {0.f, 0.f, 0.f, 0.f};
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, ub[blk], acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, ub[blk], acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3, ub[blk], acc, 0, 0, 0);
              hs[blk][st][half] = acc;
            }
          }
        }
      }
    }
    // S_cur for fragment (blk, st) of this lane, packed in the state format
    auto fold_piece = [&](int blk, int st, int v) {
      const int k0 = 32 * st + fk;
      float x[8];
      if constexpr (SF == kStateFp8) {
        st8_unpack<SF>(sf[blk][st], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= s.egl[k0 + e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = st_lo<SF>(sf[blk][st][e]) * s.egl[k0 + 2 * e];
          x[2 * e + 1] = st_hi<SF>(sf[blk][st][e]) * s.egl[k0 + 2 * e + 1];
        }
      }
      if (mfma_hist) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += hs[blk][st][e >> 2][e & 3];
      } else {
        for (int j = 0; j < hist; ++j) {
          const float uj = bf1(s.uh[j * kHistU + v]);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = fmaf(uj, s.dh[j * kHistF + k0 + e], x[e]);
        }
      }
      return st8_pack<SF>(x);
    };
    // Stores: whole 128-byte lines, non-temporally (B = 512, 100 % fold,
    // bf16: 127.6 us with half lines through L2, 123.6 us with whole lines
    // through L2, 117.7 us whole lines non-temporal; at B = 32 non-temporal
    // stores also avoid writing back dirty L2 lines at the end of the
    // kernel). They are buffer stores: a generic store with a non-temporal
    // hint was merged by the compiler with a plain one across a branch,
    // losing the hint.
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int v = 32 * wave + 16 * blk + fv;
      const bool low = fv < 8;
      if constexpr (SF == kStateFp8) {
        // Whole 128-byte lines from 8-byte fp8 pieces, in two exchanges.
        // (1) Lane groups g and g ^ 1 (lanes l and l ^ 16, ds_swizzle) trade
        // one piece per fragment pair pp, so that each lane holds 16
        // contiguous bytes of its row: g even the st = 2pp piece of channel
        // blocks g and g + 1, g odd the st = 2pp + 1 piece of blocks g - 1
        // and g; the four lanes of a row then cover bytes 64pp .. 64pp + 63
        // (lane offset og). (2) Lanes fv and fv ^ 8 swap their pp = 1 halves
        // (DPP row_ror:8), and each store writes whole lines of 8 rows, as
        // for the 16-bit formats.
        const bool godd = (lane >> 4) & 1;
        u32x4 d[2];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const St8<SF> a = fold_piece(blk, 2 * pp, v);
          const St8<SF> b = fold_piece(blk, 2 * pp + 1, v);
          const St8<SF> send = godd ? a : b;
          u32x2 recv;
#pragma unroll
          for (int i = 0; i < 2; ++i)  // bit mode: lane l reads lane l ^ 16
            recv[i] = static_cast<uint32_t>(
                __builtin_amdgcn_ds_swizzle(static_cast<int>(send[i]), 0x401F));
          d[pp] = godd ? u32x4{recv[0], recv[1], b[0], b[1]} : u32x4{a[0], a[1], recv[0], recv[1]};
        }
        const int og = 16 * (lane >> 5) + 32 * ((lane >> 4) & 1);  // byte offset in 64pp..64pp+63
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          r[i] = static_cast<uint32_t>(
              __builtin_amdgcn_update_dpp(0, static_cast<int>(d[1][i]), 0x128, 0xF, 0xF, false));
        const int bA = (low ? v : v - 8) * D + (low ? 0 : 64) + og;  // byte offsets in the head
        const int bB = (low ? v + 8 : v) * D + (low ? 64 : 0) + og;
        __builtin_amdgcn_raw_buffer_store_b128(low ? d[0] : r, fold_rsrc, bA, 0, kStoreNontemporal);
        __builtin_amdgcn_raw_buffer_store_b128(low ? r : d[0], fold_rsrc, bB, 0, kStoreNontemporal);
      } else {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const St8<SF> w0 = fold_piece(blk, 2 * pp, v);
          const St8<SF> w1 = fold_piece(blk, 2 * pp + 1, v);
          if constexpr (VEC) {
            // Whole 128-byte lines: a fragment holds 64 bytes of each of 16
            // rows, so lanes fv and fv ^ 8 swap their st = 2pp + 1 pieces
            // (DPP row_ror:8) and each store then writes channels 64pp ..
            // 64pp + 63 of 8 rows: rows 0-7 of the block (lanes fv < 8 their
            // own st = 2pp piece, lanes fv >= 8 the received st = 2pp + 1
            // piece of row v - 8), then rows 8-15 the other way round.
            u32x4 r;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              r[i] = static_cast<uint32_t>(
                  __builtin_amdgcn_update_dpp(0, static_cast<int>(w1[i]), 0x128, 0xF, 0xF, false));
            const int eA = (low ? v : v - 8) * D + 64 * pp + (low ? 0 : 32) + fk;
            const int eB = (low ? v + 8 : v) * D + 64 * pp + (low ? 32 : 0) + fk;
            const u32x4 dA = low ? w0 : r;
            const u32x4 dB = low ? r : w0;
            __builtin_amdgcn_raw_buffer_store_b128(dA, fold_rsrc, 2 * eA, 0, kStoreNontemporal);
            __builtin_amdgcn_raw_buffer_store_b128(dB, fold_rsrc, 2 * eB, 0, kStoreNontemporal);
          } else {
            // the scalar path: one store per fragment
            const int e0 = v * D + 64 * pp + fk;  // element offset in the head
            store8_raw<VEC>(ckpt + e0, w0);
            store8_raw<VEC>(ckpt + e0 + 32, w1);
          }
        }
      }
    }
  }

  // ---- 4. A and P: one (r, j) pair per 16-lane group, 8 channels per lane.
  {
    const int grp = tid >> 4;
    const int npairs = T * (T + 1) / 2;
    for (int pi = grp; pi < npairs; pi += 16) {
      // r = floor((sqrt(8 pi + 1) - 1) / 2); the true value is at least 0.1
      // below r + 1 for pi < 36, so a 0.01 margin absorbs sqrt rounding.
      const int r = int((sqrtf(8.0f * pi + 1.0f) - 1.0f) * 0.5f + 0.01f);
      const int j = pi - r * (r + 1) / 2;
      float a = 0.f, pp = 0.f;
      if constexpr (FACT) {
        float x[8], y[8], z[8];
        lds_read8(s.ka + r * XS, kb, x);
        lds_read8(s.qa + r * XS, kb, y);
        lds_read8(s.kb + j * XS, kb, z);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          a = fmaf(x[c], z[c], a);
          pp = fmaf(y[c], z[c], pp);
        }
      } else {
        float gr_[8], gj[8], kr[8], kj[8], qr[8];
        lds_read8(s.kb + r * XS, kb, gr_);
        lds_read8(s.kb + j * XS, kb, gj);
        lds_read8(s.ka + r * XS, kb, kr);
        lds_read8(s.ka + j * XS, kb, kj);
        lds_read8(s.qa + r * XS, kb, qr);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float w = kj[c] * fexp(gr_[c] - gj[c]);
          a = fmaf(kr[c], w, a);
          pp = fmaf(qr[c], w, pp);
        }
      }
      a = row16_sum(a);
      pp = row16_sum(pp);
      if (kb == 0) {
        s.am[r * TMAX + j] = j < r ? a : 0.f;
        s.pm[r * TMAX + j] = pp;
      }
    }
  }
  __syncthreads();

  // ---- 5. forward substitution. Threads 0..127 own key channel c of W
  // (written over row r of ka; X rows T.. are the exp(Gam) * q rows in qa);
  // threads 128..255 own value channel c of U0 (in place in vv).
  {
    const int c = tid & 127;
    if (tid < 128) {
      float w[TMAX];
#pragma unroll
      for (int r = 0; r < TMAX; ++r) {
        if (r < T) {
          float x;
          if constexpr (FACT) {
            x = s.ka[r * XS + c];
          } else {
            const float ea = fexp(s.kb[r * XS + c]);
            x = ea * s.ka[r * XS + c];
            s.qa[r * XS + c] *= ea;
          }
#pragma unroll
          for (int j = 0; j < r; ++j) x = fmaf(-s.am[r * TMAX + j], w[j], x);
          w[r] = s.beta[r] * x;
          s.ka[r * XS + c] = w[r];
        }
      }
    } else {
      float u0[TMAX];
#pragma unroll
      for (int r = 0; r < TMAX; ++r) {
        if (r < T) {
          float x = s.vv[r * XS + c];
#pragma unroll
          for (int j = 0; j < r; ++j) x = fmaf(-s.am[r * TMAX + j], u0[j], x);
          u0[r] = s.beta[r] * x;
          s.vv[r * XS + c] = u0[r];
        }
      }
    }
  }
  __syncthreads();

  // ---- 5b. C[m, j] = X_m . D_j (history correction), rows m < 2T, entries j < hist.
  // Deep rings, from 8 entries on: one MFMA product per 16 entries (wave w
  // takes entries 16 w ..): A = the X rows (lane row m = lane % 16, zero from
  // 2T on), B = the D_j rows (zero from hist on), four 32-channel steps, both
  // split into bf16 hi and lo, three terms. Otherwise one 16-lane group per
  // row m and a dot product per entry (in the 16-row-window instance the
  // product's registers would cost occupancy on every call).
  if (DEEP && hist >= 8) {
    if (16 * wave < hist) {
      const int m = fv, j = 16 * wave + fv;
      const float* xrow = m < T ? s.ka + m * XS : s.qa + (m - T) * XS;
      const float* drow = s.dh + j * kHistF;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      f32x4 c0 = z, c1 = z, c2 = z;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int k0 = 32 * st + fk;
        f32x4 x0 = z, x1 = z, d0 = z, d1 = z;
        if (m < 2 * T) {
          x0 = *reinterpret_cast<const f32x4*>(xrow + k0);
          x1 = *reinterpret_cast<const f32x4*>(xrow + k0 + 4);
        }
        if (j < hist) {
          d0 = *reinterpret_cast<const f32x4*>(drow + k0);
          d1 = *reinterpret_cast<const f32x4*>(drow + k0 + 4);
        }
        u32x4 xh, xl, dhi, dlo;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          xh[i] = pack_bf16x2(x0[2 * i], x0[2 * i + 1]);
          xh[2 + i] = pack_bf16x2(x1[2 * i], x1[2 * i + 1]);
          xl[i] = pack_bf16x2(x0[2 * i] - bf_lo(xh[i]), x0[2 * i + 1] - bf_hi(xh[i]));
          xl[2 + i] = pack_bf16x2(x1[2 * i] - bf_lo(xh[2 + i]), x1[2 * i + 1] - bf_hi(xh[2 + i]));
          dhi[i] = pack_bf16x2(d0[2 * i], d0[2 * i + 1]);
          dhi[2 + i] = pack_bf16x2(d1[2 * i], d1[2 * i + 1]);
          dlo[i] = pack_bf16x2(d0[2 * i] - bf_lo(dhi[i]), d0[2 * i + 1] - bf_hi(dhi[i]));
          dlo[2 + i] = pack_bf16x2(d1[2 * i] - bf_lo(dhi[2 + i]), d1[2 * i + 1] - bf_hi(dhi[2 + i]));
        }
        const bf16x8 axh = __builtin_bit_cast(bf16x8, xh), axl = __builtin_bit_cast(bf16x8, xl);
        const bf16x8 bdh = __builtin_bit_cast(bf16x8, dhi), bdl = __builtin_bit_cast(bf16x8, dlo);
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(axh, bdh, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(axh, bdl, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(axl, bdh, c2, 0, 0, 0);
      }
      const f32x4 c = c0 + (c1 + c2);  // rows 4 (lane / 16) + i, entry 16 wave + lane % 16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mr = 4 * (lane >> 4) + i;
        if (mr < 2 * T && j < hist) s.cm[mr * hm + j] = c[i];
      }
    }
  } else if (hist > 0) {
    const int grp = tid >> 4;
    if (grp < 2 * T) {
      const float* xrow = grp < T ? s.ka + grp * XS : s.qa + (grp - T) * XS;
      float x[8];
      lds_read8(xrow, kb, x);
      for (int j = 0; j < hist; ++j) {
        float d[8];
        lds_read8(s.dh + j * kHistF, kb, d);
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) a = fmaf(x[c], d[c], a);
        a = row16_sum(a);
        if (kb == 0) s.cm[grp * hm + j] = a;
      }
    }
  }
  __syncthreads();

  // ---- 6. Y = (X * exp(G_L)) S_ckpt on MFMA. Lane (g, m) builds its A
  // fragment from X row m (W rows in ka, exp(Gam) q rows in qa, zero rows
  // from 2T on): 8 fp32 channels scaled by exp(G_L) and split into bf16 hi
  // and lo parts, shared by both 16-column blocks; four 32-channel steps.
  {
    const float* xrow = fv < T ? s.ka + fv * XS : s.qa + (fv - T) * XS;
    const bool xzero = fv >= 2 * T;
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int k0 = 32 * st + fk;
      f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
      if (!xzero) {
        x0 = *reinterpret_cast<const f32x4*>(xrow + k0);
        x1 = *reinterpret_cast<const f32x4*>(xrow + k0 + 4);
      }
      const f32x4 e0 = *reinterpret_cast<const f32x4*>(s.egl + k0);
      const f32x4 e1 = *reinterpret_cast<const f32x4*>(s.egl + k0 + 4);
      u32x4 hi, lo;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float a = x0[2 * i] * e0[2 * i], b = x0[2 * i + 1] * e0[2 * i + 1];
        const float c = x1[2 * i] * e1[2 * i], d = x1[2 * i + 1] * e1[2 * i + 1];
        // hi / lo split in the format of the checkpoint operand
        hi[i] = st_pack<MF>(a, b);
        hi[2 + i] = st_pack<MF>(c, d);
        lo[i] = st_pack<MF>(a - st_lo<MF>(hi[i]), b - st_hi<MF>(hi[i]));
        lo[2 + i] = st_pack<MF>(c - st_lo<MF>(hi[2 + i]), d - st_hi<MF>(hi[2 + i]));
      }
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        if constexpr (MF == kStateFp16) {
          const f16x8 ahi = __builtin_bit_cast(f16x8, hi);
          const f16x8 alo = __builtin_bit_cast(f16x8, lo);
          const f16x8 bfr = __builtin_bit_cast(f16x8, sf[blk][st]);
          acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bfr, acc[blk], 0, 0, 0);
          acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bfr, acc[blk], 0, 0, 0);
        } else {
          const bf16x8 ahi = __builtin_bit_cast(bf16x8, hi);
          const bf16x8 alo = __builtin_bit_cast(bf16x8, lo);
          u32x4 bw;
          if constexpr (SF == kStateFp8) {  // fp8 -> bf16 is exact
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const f32x2 x01 = f8x2_lo(sf[blk][st][i]), x23 = f8x2_hi(sf[blk][st][i]);
              bw[2 * i] = pack_bf16x2_exact(x01[0], x01[1]);
              bw[2 * i + 1] = pack_bf16x2_exact(x23[0], x23[1]);
            }
          } else {
            bw = sf[blk][st];
          }
          const bf16x8 bfr = __builtin_bit_cast(bf16x8, bw);
          acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bfr, acc[blk], 0, 0, 0);
          acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bfr, acc[blk], 0, 0, 0);
        }
      }
    }
    // History correction C U_hist (C = X D^T from phase 5b, 2T x hist; U_hist
    // the ring's bf16 u rows, exact as B operands): one more K = 32
    // contraction over history entries j = 8 (lane / 16) + e, with C split into
    // bf16 hi and lo; entries j >= hist are zero on both sides.
    if (hist > 0) {
      float cr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = fk + e;
        cr[e] = (!xzero && j < hist) ? s.cm[fv * hm + j] : 0.f;
      }
      u32x4 hi, lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = pack_bf16x2(cr[2 * i], cr[2 * i + 1]);
        lo[i] = pack_bf16x2(cr[2 * i] - bf_lo(hi[i]), cr[2 * i + 1] - bf_hi(hi[i]));
      }
      const bf16x8 chi = __builtin_bit_cast(bf16x8, hi);
      const bf16x8 clo = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int v = 32 * wave + 16 * blk + fv;
        u32x4 ub;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = fk + 2 * i;
          const uint32_t u0 = j < hist ? s.uh[j * kHistU + v] : 0u;
          const uint32_t u1 = j + 1 < hist ? s.uh[(j + 1) * kHistU + v] : 0u;
          ub[i] = u0 | (u1 << 16);
        }
        const bf16x8 bu = __builtin_bit_cast(bf16x8, ub);
        acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(chi, bu, acc[blk], 0, 0, 0);
        acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(clo, bu, acc[blk], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave has read its X rows: Y may overwrite them
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int v = 32 * wave + 16 * blk + fv;
#pragma unroll
      for (int i = 0; i < 4; ++i) s.y[((lane >> 4) * 4 + i) * XS + v] = acc[blk][i];
    }
  }
  __syncthreads();

  // ---- 7. two threads own value channel v (tokens split by parity): u_t,
  // o_t, ring u rows, outputs. Each computes every u_j it needs (u_t only
  // depends on Y and U0).
  {
    const int v = tid & 127;
    const int half = tid >> 7;
    float u[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        u[t] = s.vv[t * XS + v] - s.y[t * XS + v];
        if ((t & 1) == half) {
          float yq = s.y[(T + t) * XS + v];
#pragma unroll
          for (int j = 0; j <= t; ++j) yq = fmaf(s.pm[t * TMAX + j], u[j], yq);
          __builtin_nontemporal_store(to_bf16(p.scale * yq), outb + int64_t(t) * p.out_tok_stride + v);
          __builtin_nontemporal_store(to_bf16(u[t]), uc + int64_t(ring_row(hist + t)) * D + v);
        }
      }
    }
  }
}

hipError_t launch_verify(const VerifyParams& p, bool vec, hipStream_t stream) {
  const int64_t blocks = int64_t(p.B) * p.H;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int hm = p.w_ring - p.T;  // history capacity: hist + T <= w_ring
  const size_t lds = smem_bytes(hm);
  // exp(Gam_r) * exp(-Gam_j) stays finite when |Gam| <= T * |lower_bound| < 80.
  const bool fact = p.lower_bound > -80.0f / float(p.T) && p.lower_bound <= 0.0f;
  dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const int gk = p.gate_mode & kGateKindMask;
#define KDA_VERIFY_LAUNCH(V, F, S, DP)                                                             \
  do {                                                                                             \
    switch (gk) {                                                                                  \
      case 0:                                                                                      \
        hipLaunchKernelGGL((verify_kernel<V, F, 0, S, DP>), grid, block, lds, stream, p, hm); \
        break;                                                                                     \
      case 1:                                                                                      \
        hipLaunchKernelGGL((verify_kernel<V, F, 1, S, DP>), grid, block, lds, stream, p, hm); \
        break;                                                                                     \
      case 4:                                                                                      \
        hipLaunchKernelGGL((verify_kernel<V, F, 4, S, DP>), grid, block, lds, stream, p, hm); \
        break;                                                                                     \
      default:                                                                                     \
        hipLaunchKernelGGL((verify_kernel<V, F, 5, S, DP>), grid, block, lds, stream, p, hm); \
    }                                                                                              \
  } while (0)
  // Deep rings (16 or more history rows, the 32-row window): the fold's
  // history sum on MFMA (see the kernel). These workgroups already hold
  // three per CU for their LDS, so the extra registers cost no occupancy;
  // built for the vectorised path with factored exponentials only.
  const bool deep = hm >= 16 && vec && fact;
  // fp16 and fp8 checkpoints run on the vectorised path only (the host requires it)
  if (p.state_fmt != kStateBf16 && !vec) return hipErrorInvalidValue;
  if (p.state_fmt == kStateFp16) {
    if (deep) KDA_VERIFY_LAUNCH(true, true, kStateFp16, true);
    else if (fact) KDA_VERIFY_LAUNCH(true, true, kStateFp16, false);
    else KDA_VERIFY_LAUNCH(true, false, kStateFp16, false);
  } else if (p.state_fmt == kStateFp8) {
    if (deep) KDA_VERIFY_LAUNCH(true, true, kStateFp8, true);
    else if (fact) KDA_VERIFY_LAUNCH(true, true, kStateFp8, false);
    else KDA_VERIFY_LAUNCH(true, false, kStateFp8, false);
  } else if (vec) {
    if (deep) KDA_VERIFY_LAUNCH(true, true, kStateBf16, true);
    else if (fact) KDA_VERIFY_LAUNCH(true, true, kStateBf16, false);
    else KDA_VERIFY_LAUNCH(true, false, kStateBf16, false);
  } else {
    if (fact) KDA_VERIFY_LAUNCH(false, true, kStateBf16, false);
    else KDA_VERIFY_LAUNCH(false, false, kStateBf16, false);
  }
#undef KDA_VERIFY_LAUNCH
  return hipGetLastError();
}

}  // namespace kda
