// Speculative-decode verify with the (k_hat, u, G) ring and the fold into the
// checkpoint (gfx950).
//
// Operation: "feat(kda): ReplaySSM verify+flush decode kernel for Kimi K3
// (KDA)", sections "What it does", "API" and "Caching". One workgroup (four
// waves) owns one (row, head). With S_cur the state the ring stands for,
//   S_cur = diag(exp(G_L)) S_ckpt + sum_{j<hist} diag(exp(G_L - G_j)) k_j u_j^T,
// the T draft tokens are processed as one chunk of the chunkwise (WY)
// form of the recurrence instead of T sequential state updates:
//   Gam_t  = g_0 + ... + g_t                        (per key channel)
//   A[r,j] = sum_c k_r k_j exp(Gam_r - Gam_j)        (j < r)
//   P[r,j] = sum_c q_r k_j exp(Gam_r - Gam_j)        (j <= r)
//   W      = (I + diag(beta) A)^-1 diag(beta) (exp(Gam) * K)
//   U0     = (I + diag(beta) A)^-1 diag(beta) V
//   u_t    = U0_t - (W S_cur)_t                      (the per-token corrections)
//   o_t    = scale * ((exp(Gam_t) * q_t) S_cur + sum_{j<=t} P[t,j] u_j)
// (S k means the state applied to a key vector, as in u = beta (v - S k)).
// Because S_cur only enters through X S_cur with X = [W; exp(Gam) * Q], the
// replay never needs to be materialised for the outputs:
//   X S_cur = (X * exp(G_L)) S_ckpt + C U_hist,  C[m,j] = X_m . (exp(G_L - G_j) * k_j).
// (X * exp(G_L)) S_ckpt is the only product with the full 128 x 128 state. The
// checkpoint is exact in bf16, so it feeds v_mfma_f32_16x16x32_bf16 directly
// as the B operand (128-bit loads straight into B fragments); the fp32 left
// operand is split into bf16 hi + lo parts (two MFMAs into one fp32
// accumulator, ~2^-17 relative error). Everything else is small and runs on
// the VALU in fp32. A folding row also materialises S_cur element-wise (fp32)
// and stores it in bf16 over the checkpoint.

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int TMAX = 8;
constexpr int XLD = D + 8;  // padded bf16 row of the MFMA left operand (bank spread)

// Dynamic LDS carve-up (floats unless noted). hm = history capacity of the
// launch (w_ring - T).
struct Smem {
  float* qh;    // [TMAX][D] q_hat; aliased by y after the left operand is built
  float* kh;    // [TMAX][D] k_hat
  float* y;     // [2*TMAX][D] MFMA result rows (aliases qh, kh)
  float* gam;   // [TMAX][D] g_t, then Gam_t in place
  float* vv;    // [TMAX][D] v_t, then U0_t in place
  float* xf;    // [2*TMAX][D] X rows in fp32 (for C)
  uint16_t* xop;  // [2][2*TMAX][XLD] bf16 hi / lo of X * exp(G_L)
  float* am;    // [TMAX][TMAX]
  float* pm;    // [TMAX][TMAX]
  float* beta;  // [TMAX]
  float* egl;   // [D] exp(G_L)
  float* cm;    // [2*TMAX][hm]
  float* dh;    // [hm][D] exp(G_L - G_j) * k_j
  uint16_t* uh;  // [hm][D] u_j (bf16 bits)
};

__host__ __device__ inline size_t smem_bytes(int hm) {
  size_t f = 0;
  f += 2 * TMAX * D;          // qh, kh (y)
  f += TMAX * D;              // gam
  f += TMAX * D;              // vv
  f += 2 * TMAX * D;          // xf
  f += 2 * TMAX * TMAX + TMAX + D;
  f += size_t(2 * TMAX) * hm;  // cm
  f += size_t(hm) * D;         // dh
  size_t bytes = f * 4;
  bytes += size_t(2) * 2 * TMAX * XLD * 2;  // xop
  bytes += size_t(hm) * D * 2;               // uh
  return (bytes + 15) & ~size_t(15);
}

__device__ inline Smem carve(float* base, int hm) {
  Smem s;
  float* p = base;
  s.qh = p; p += TMAX * D;
  s.kh = p; p += TMAX * D;
  s.y = s.qh;
  s.gam = p; p += TMAX * D;
  s.vv = p; p += TMAX * D;
  s.xf = p; p += 2 * TMAX * D;
  s.am = p; p += TMAX * TMAX;
  s.pm = p; p += TMAX * TMAX;
  s.beta = p; p += TMAX;
  s.egl = p; p += D;
  s.cm = p; p += 2 * TMAX * hm;
  s.dh = p; p += size_t(hm) * D;
  s.xop = reinterpret_cast<uint16_t*>(p);
  s.uh = s.xop + 2 * 2 * TMAX * XLD;
  return s;
}

template <bool VEC>
__device__ __forceinline__ void load_bfrag(const uint16_t* p, u32x4& w) {
  w = load8_raw<VEC>(p);
}

}  // namespace

// Grid: one 256-thread workgroup per (row, head), row-major over heads.
template <bool VEC>
__global__ __launch_bounds__(256) void verify_kernel(VerifyParams p, int hm) {
  extern __shared__ __align__(16) float smem_raw[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = int(blockIdx.x % p.H);
  const int64_t b = blockIdx.x / p.H;
  const int T = p.T;
  const int R = p.ring_rows;

  const int32_t slot = p.state_indices[b];
  const int hist = p.hist_len[b];
  const int base = p.cache_base[b];
  const bool active = slot >= 0 && int64_t(slot) < p.num_slots && hist >= 0 &&
                      hist + T <= p.w_ring && base >= 0 && base < R;
  uint16_t* outb = p.out + b * p.out_row_stride + int64_t(h) * D;
  if (!active) {
    for (int e = tid; e < T * D; e += 256) outb[int64_t(e / D) * p.out_tok_stride + (e % D)] = 0;
    return;
  }
  const bool fold = hist + T >= p.flush_min;
  Smem s = carve(smem_raw, hm);
  const int64_t sh = int64_t(slot) * p.H + h;
  uint16_t* ckpt = p.state_pool + int64_t(slot) * p.slot_stride + int64_t(h) * HEAD_ELEMS;
  uint16_t* kc = p.k_cache + sh * R * D;
  uint16_t* uc = p.u_cache + sh * R * D;
  float* gc = p.g_cache + sh * R * D;

  // ---- 1. checkpoint B fragments: wave w owns value columns 32w .. 32w+31
  // (two 16-column blocks); fragment (blk, s): v = 32w + 16*blk + lane%16,
  // key channels 32*s + 8*(lane/16) .. +7.
  const int fv = lane & 15, fk = (lane >> 4) * 8;
  u32x4 sf[2][4];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int st = 0; st < 4; ++st)
      load_bfrag<VEC>(ckpt + int64_t(32 * wave + 16 * blk + fv) * D + 32 * st + fk, sf[blk][st]);

  // ---- 2. per-token prologue: token t on wave t/4, lanes 16*(t%4) .. +15,
  // key channels 8*(lane%16) .. +7.
  {
    const int t = wave * 4 + (lane >> 4);
    const int c0 = (lane & 15) * 8;
    if (t < T) {
      float q[8], k[8], gr[8], vv[8], dtb[8];
      load8_bf16<VEC>(p.q + b * p.q_row_stride + t * p.q_tok_stride + h * D + c0, q);
      load8_bf16<VEC>(p.k + b * p.k_row_stride + t * p.k_tok_stride + h * D + c0, k);
      load8_bf16<VEC>(p.g + b * p.g_row_stride + t * p.g_tok_stride + h * D + c0, gr);
      load8_bf16<VEC>(p.v + b * p.v_row_stride + t * p.v_tok_stride + h * D + c0, vv);
      load8_f32<VEC>(p.dt_bias + h * D + c0, dtb);
      const float neg_ea = -expf(p.A_log[h]);
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        sq = fmaf(q[c], q[c], sq);
        sk = fmaf(k[c], k[c], sk);
      }
      sq = row16_sum(sq);
      sk = row16_sum(sk);
      const float rq = 1.0f / sqrtf(sq + 1e-6f);
      const float rk = 1.0f / sqrtf(sk + 1e-6f);
      u32x4 kb16;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        s.qh[t * D + c0 + c] = q[c] * rq;
        s.kh[t * D + c0 + c] = k[c] * rk;
        s.gam[t * D + c0 + c] = gate_logdecay(gr[c] + dtb[c], neg_ea, p.lower_bound);
        s.vv[t * D + c0 + c] = vv[c];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) kb16[j] = pack_bf16x2(k[2 * j] * rk, k[2 * j + 1] * rk);
      const int row = (base + hist + t) % R;
      store8_raw<VEC>(kc + int64_t(row) * D + c0, kb16);
      if ((lane & 15) == 0)
        s.beta[t] = sigmoidf(bf1(p.beta[b * p.beta_row_stride + t * p.beta_tok_stride + h]));
    }
  }
  __syncthreads();

  // ---- 3. cumulative decays and ring history. Threads 0..127 own key
  // channel c: Gam_t = g_0 + ... + g_t (from 0, in place over g_t) and the
  // ring's G_t = G_base + g_0 + ... + g_t (token order; G_base = 0 when
  // folding, else G_{hist-1}), plus exp(G_L). Threads 128..255 stage the live
  // history rows: D_j = exp(G_L - G_j) * k_j (fp32) and u_j (bf16). History
  // rows j < hist and the draft rows hist .. hist+T-1 never coincide because
  // hist + T <= w_ring <= R.
  {
    const int c = tid & 127;
    const float gl = hist > 0 ? gc[int64_t((base + hist - 1) % R) * D + c] : 0.f;
    if (tid < 128) {
      s.egl[c] = expf(gl);
      float gam = 0.f, gacc = fold ? 0.f : gl;
      for (int t = 0; t < T; ++t) {
        const float g = s.gam[t * D + c];
        gam += g;
        gacc += g;
        s.gam[t * D + c] = gam;
        gc[int64_t((base + hist + t) % R) * D + c] = gacc;
      }
    } else {
      for (int j = 0; j < hist; ++j) {
        const int64_t row = (base + j) % R;
        s.dh[j * D + c] = expf(gl - gc[row * D + c]) * bf1(kc[row * D + c]);
        s.uh[j * D + c] = uc[row * D + c];
      }
    }
  }
  __syncthreads();

  // ---- 4. A and P: one (r, j) pair per 16-lane group, 8 channels per lane.
  {
    const int grp = tid >> 4;
    const int c0 = (tid & 15) * 8;
    const int npairs = T * (T + 1) / 2;
    for (int pi = grp; pi < npairs; pi += 16) {
      int r = 0;
      while ((r + 1) * (r + 2) / 2 <= pi) ++r;
      const int j = pi - r * (r + 1) / 2;
      float a = 0.f, pp = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float e = expf(s.gam[r * D + c0 + c] - s.gam[j * D + c0 + c]);
        const float kj = s.kh[j * D + c0 + c] * e;
        a = fmaf(s.kh[r * D + c0 + c], kj, a);
        pp = fmaf(s.qh[r * D + c0 + c], kj, pp);
      }
      a = row16_sum(a);
      pp = row16_sum(pp);
      if ((tid & 15) == 0) {
        s.am[r * TMAX + j] = j < r ? a : 0.f;
        s.pm[r * TMAX + j] = pp;
      }
    }
  }
  __syncthreads();

  // ---- 5. forward substitution. Threads 0..127 own key channel c of W and
  // build X = [W; exp(Gam) * Q] (fp32 copy for C, bf16 hi/lo of X * exp(G_L)
  // for the MFMA); threads 128..255 own value channel c of U0 (in place).
  {
    const int c = tid & 127;
    if (tid < 128) {
      float w[TMAX];
      const float eg = s.egl[c];
      for (int r = 0; r < T; ++r) {
        float x = expf(s.gam[r * D + c]) * s.kh[r * D + c];
        for (int j = 0; j < r; ++j) x = fmaf(-s.am[r * TMAX + j], w[j], x);
        w[r] = s.beta[r] * x;
      }
      for (int m = 0; m < 2 * TMAX; ++m) {
        float x = 0.f;
        if (m < T) x = w[m];
        else if (m < 2 * T) x = expf(s.gam[(m - T) * D + c]) * s.qh[(m - T) * D + c];
        s.xf[m * D + c] = x;
        const float xs = x * eg;
        const uint16_t hi = to_bf16(xs);
        const uint16_t lo = to_bf16(xs - bf1(hi));
        s.xop[m * XLD + c] = hi;
        s.xop[2 * TMAX * XLD + m * XLD + c] = lo;
      }
    } else {
      float u0[TMAX];
      for (int r = 0; r < T; ++r) {
        float x = s.vv[r * D + c];
        for (int j = 0; j < r; ++j) x = fmaf(-s.am[r * TMAX + j], u0[j], x);
        u0[r] = s.beta[r] * x;
        s.vv[r * D + c] = u0[r];
      }
    }
  }
  __syncthreads();

  // ---- 5b. C[m, j] = X_m . D_j (history correction), one pair per group.
  if (hist > 0) {
    const int grp = tid >> 4;
    const int c0 = (tid & 15) * 8;
    const int npairs = 2 * T * hist;
    for (int pi = grp; pi < npairs; pi += 16) {
      const int m = pi / hist, j = pi % hist;
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) a = fmaf(s.xf[m * D + c0 + c], s.dh[j * D + c0 + c], a);
      a = row16_sum(a);
      if ((tid & 15) == 0) s.cm[m * hm + j] = a;
    }
  }

  // ---- 6. Y = (X * exp(G_L)) S_ckpt on MFMA: per 16-column block, four
  // 32-channel steps, hi and lo parts into one accumulator. y aliases qh/kh,
  // whose last reads were in phase 5 (before the barrier above).
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8 bfr = __builtin_bit_cast(bf16x8, sf[blk][st]);
      const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(s.xop + fv * XLD + 32 * st + fk);
      const bf16x8 alo =
          *reinterpret_cast<const bf16x8*>(s.xop + 2 * TMAX * XLD + fv * XLD + 32 * st + fk);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bfr, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bfr, acc, 0, 0, 0);
    }
    const int v = 32 * wave + 16 * blk + fv;
#pragma unroll
    for (int i = 0; i < 4; ++i) s.y[((lane >> 4) * 4 + i) * D + v] = acc[i];
  }
  __syncthreads();

  // ---- 7. threads 0..127 own value channel v: u_t, o_t, ring u rows, outputs.
  if (tid < 128) {
    const int v = tid;
    float u[TMAX];
    for (int t = 0; t < T; ++t) {
      float yw = s.y[t * D + v];
      float yq = s.y[(T + t) * D + v];
      for (int j = 0; j < hist; ++j) {
        const float uj = bf1(s.uh[j * D + v]);
        yw = fmaf(s.cm[t * hm + j], uj, yw);
        yq = fmaf(s.cm[(T + t) * hm + j], uj, yq);
      }
      u[t] = s.vv[t * D + v] - yw;
      for (int j = 0; j <= t; ++j) yq = fmaf(s.pm[t * TMAX + j], u[j], yq);
      outb[int64_t(t) * p.out_tok_stride + v] = to_bf16(p.scale * yq);
      uc[int64_t((base + hist + t) % R) * D + v] = to_bf16(u[t]);
    }
  }

  // ---- 8. fold: S_cur = exp(G_L) * S_ckpt + sum_j u_j D_j over this wave's
  // fragments, stored in bf16 over the checkpoint. With no history S_cur is
  // the checkpoint itself and nothing is rewritten.
  if (fold && hist > 0) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int v = 32 * wave + 16 * blk + fv;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int k0 = 32 * st + fk;
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf_lo(sf[blk][st][e]) * s.egl[k0 + 2 * e];
          x[2 * e + 1] = bf_hi(sf[blk][st][e]) * s.egl[k0 + 2 * e + 1];
        }
        for (int j = 0; j < hist; ++j) {
          const float uj = bf1(s.uh[j * D + v]);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = fmaf(uj, s.dh[j * D + k0 + e], x[e]);
        }
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
        store8_raw<VEC>(ckpt + int64_t(v) * D + k0, w);
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
  dim3 grid(static_cast<unsigned>(blocks)), block(256);
  if (vec) hipLaunchKernelGGL((verify_kernel<true>), grid, block, lds, stream, p, hm);
  else hipLaunchKernelGGL((verify_kernel<false>), grid, block, lds, stream, p, hm);
  return hipGetLastError();
}

}  // namespace kda
