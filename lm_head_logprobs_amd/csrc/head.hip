// Per-token kernels of the fused head: log-sum-exp merge, label/support logit
// gathers, weights and loss (combine), the dense softmax-gradient operand
// (form_g), dh finalisation and the deterministic loss/metric reduction.
//
// Method: prime-rl pull request 4233, PR description (RLLoss formula, the
// estimator sum_v u_v f(v) of E_q[f], weights per loss type, KL over the same
// support).  The gradient treats every importance weight as a constant:
//   dL/dz_t = (kappa_t p_t - s_t w_t e_a + sum_e (s_t c_e - beta u_e) e_{v_e}) / D
//   kappa_t = s_t (w_t - sum_e c_e) + beta sum_e u_e,   c_e = u_e w_e.
// On the dense backward the whole of dL/dz is one bf16 operand G: the
// kappa_t p_t part is formed in place over the forward's e^(z - m), then the
// label and entry coefficients are added into the same elements (fold_sparse,
// from the vocabulary-sorted entry list).  On the sparse backward (kappa = 0)
// only the per-entry coefficients exist, applied in fp32 by gathers of W rows
// (dh) and a bucketed scatter of h rows (dW).
#include "kernels.h"

namespace rl {
namespace {

constexpr int NT = 256;

// Fixed-order block reduction over 256 threads (4 waves): butterfly inside
// each wave, then the 4 wave results summed in wave order.
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return ((sh[0] + sh[1]) + sh[2]) + sh[3];
}
__device__ __forceinline__ float block_max(float v, float* sh) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

template <typename T>
__device__ __forceinline__ float dot_row_part(const T* __restrict__ x, const T* __restrict__ y,
                                              int64_t H, int start, int stride) {
  constexpr int VEC = Elem<T>::VEC;
  float acc = 0.0f;
  for (int64_t c = (int64_t)start * VEC; c < H; c += (int64_t)stride * VEC) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(x + c);
    const u32x4 b = *reinterpret_cast<const u32x4*>(y + c);
    float fa[VEC], fb[VEC];
    Elem<T>::unpack(a, fa);
    Elem<T>::unpack(b, fb);
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc = fmaf(fa[i], fb[i], acc);
  }
  return acc;
}

// dst[c][r] = src[r][c] for r < R, zero for R <= r < Rpad (c < C).  64 x 64
// tiles through LDS; 16-byte loads of source rows and 16-byte stores of
// destination rows.  C and ld_src are multiples of the vector width.
template <typename T>
__global__ void __launch_bounds__(NT) transpose_kernel(const T* __restrict__ src, int64_t ld_src,
                                                       int64_t R, int64_t C, T* __restrict__ dst,
                                                       int64_t Rpad) {
  constexpr int VEC = Elem<T>::VEC, CPR = 64 / VEC;  // chunks per 64-element row
  __shared__ T tile[64][64 + VEC];                    // [c][r]
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  for (int q = threadIdx.x; q < 64 * CPR; q += NT) {
    const int rl = q / CPR, cl = (q % CPR) * VEC;
    const int64_t r = r0 + rl, c = c0 + cl;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R && c < C) v = *reinterpret_cast<const u32x4*>(src + r * ld_src + c);
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int k = 0; k < VEC; ++k) tile[cl + k][rl] = e[k];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 64 * CPR; q += NT) {
    const int cl = q / CPR, rl = (q % CPR) * VEC;
    const int64_t c = c0 + cl, r = r0 + rl;
    if (c >= C || r >= Rpad) continue;
    u32x4 v;
    T* e = reinterpret_cast<T*>(&v);
#pragma unroll
    for (int k = 0; k < VEC; ++k) e[k] = tile[cl][rl + k];
    *reinterpret_cast<u32x4*>(dst + c * Rpad + r) = v;
  }
}

// Label and support logits (before 1/tau) of every gradient entry (labels,
// then the CSR entries), computed in the vocabulary-sorted order of
// csc_build.  Entries of one id are adjacent there, so the id's W row comes
// from HBM once and then from cache; the token rows h_t that each entry
// gathers are a few tens of MB and stay in the Infinity Cache.  (Gathering W
// rows per token instead reads 2H bytes of W per entry, most of them from
// HBM.)  One wave per 64 sorted entries, 16 at a time: each lane keeps 16
// partial dot products and a transposing lane-swap butterfly reduces them in
// a fixed order.  An id outside [0, V) gives NaN.
template <typename T>
__global__ void __launch_bounds__(NT) entry_logits_kernel(
    const T* __restrict__ h, const T* __restrict__ W, int64_t H, int64_t V,
    const int32_t* __restrict__ skeys, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ row_of, int64_t N, int64_t E, float* __restrict__ z) {
  constexpr int VEC = Elem<T>::VEC, G = 16;
  const int lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6)) * 64;
  const int r = lane >> 4;
  const int off = ((r & 1) << 1) | (r >> 1);  // row r of the butterfly holds entry 4 j + off
#pragma unroll 1
  for (int g = 0; g < 64 / G; ++g) {
    const int64_t i0 = base + G * g;
    if (i0 >= E) break;
    const T* wr[G];
    const T* hr[G];
    bool ok[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int64_t i = i0 + k;
      const bool in = i < E;
      const int32_t key = in ? skeys[i] : -1;
      const int32_t e = in ? perm[i] : 0;
      // (a support entry before the first CSR row, possible only with bad
      // offsets, has row -1)
      const int64_t t = e < N ? e : row_of[e - N];
      const bool t_ok = t >= 0 && t < N;
      ok[k] = key >= 0 && key < V && t_ok;
      wr[k] = W + (ok[k] ? (int64_t)key : 0) * H;  // valid rows; the product is discarded
      hr[k] = h + (in && t_ok ? t : 0) * H;
    }
    float f[G];
#pragma unroll
    for (int k = 0; k < G; ++k) f[k] = 0.0f;
    for (int64_t c = (int64_t)lane * VEC; c < H; c += 64 * VEC) {
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(wr[k] + c);
        const u32x4 b = *reinterpret_cast<const u32x4*>(hr[k] + c);
        float fa[VEC], fb[VEC];
        Elem<T>::unpack(a, fa);
        Elem<T>::unpack(b, fb);
#pragma unroll
        for (int q = 0; q < VEC; ++q) f[k] = fmaf(fa[q], fb[q], f[k]);
      }
    }
    // permlane32_swap pairs, then permlane16_swap pairs, then a row scan:
    // lane 15 of row r holds the total of entry 4 j + off.
    float gsum[G / 2];
#pragma unroll
    for (int k = 0; k < G / 2; ++k) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(f[2 * k]),
                                                       __float_as_uint(f[2 * k + 1]), false, false);
      gsum[k] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
#pragma unroll
    for (int j = 0; j < G / 4; ++j) {
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(gsum[2 * j]),
                                                       __float_as_uint(gsum[2 * j + 1]), false,
                                                       false);
      float v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      v = dpp_add<0x111, 0xf>(v);  // row_shr:1
      v = dpp_add<0x112, 0xf>(v);  // row_shr:2
      v = dpp_add<0x114, 0xf>(v);  // row_shr:4
      v = dpp_add<0x118, 0xf>(v);  // row_shr:8
      const int k = 4 * j + off;
      // ok[k] with a lane-dependent k: select it without dynamic register indexing
      bool okk = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) okk = (off == q) ? ok[4 * j + q] : okk;
      if ((lane & 15) == 15 && i0 + k < E) z[perm[i0 + k]] = okk ? v : NAN;
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(NT) combine_kernel(CombineArgs a) {
  __shared__ float sh[8];
  __shared__ float wsum[4][6];
  const int tid = threadIdx.x;
  const int64_t tl = blockIdx.x;
  const int64_t t = a.t0 + tl;
  const T* h = static_cast<const T*>(a.h) + t * a.H;
  const T* W = static_cast<const T*>(a.W);

  // Merge the per-tile online-softmax partials: LSE and entropy.
  const float* pm = a.part_m + tl * a.J;
  const float* ps = a.part_s + tl * a.J;
  const float* pt = a.part_t + tl * a.J;
  float mx = -INFINITY;
  for (int64_t j = tid; j < a.J; j += NT) mx = fmaxf(mx, pm[j]);
  const float M = block_max(mx, sh);
  float S = 0.0f, Tq = 0.0f;
  for (int64_t j = tid; j < a.J; j += NT) {
    const float dm = pm[j] - M;
    const float e = __expf(dm);
    S += ps[j] * e;
    Tq += e * (pt[j] + dm * ps[j]);
  }
  S = block_sum(S, sh);
  Tq = block_sum(Tq, sh);
  const float logS = logf(S);
  const float lse = M + logS;
  const float ent = logS - Tq / S;

  // Label logit and log-probability.  An id outside [0, V) reads nothing and
  // yields NaN (such inputs are reported by the validation call).
  const int32_t lab = a.labels[t];
  const bool lab_ok = lab >= 0 && lab < a.V;
  float za;
  if (a.zent != nullptr) {
    za = a.inv_t * a.zent[t];
  } else {
    za = a.inv_t * block_sum(lab_ok ? dot_row_part<T>(h, W + (int64_t)lab * a.H, a.H, tid, NT)
                                    : 0.0f, sh);
  }
  if (!lab_ok) za = NAN;
  const float lp = za - lse;
  const float lq = a.infer_lp[t];
  bool keep;
  const float w = rl_weight(lp, lq, a.wp, &keep);
  const float s = a.adv_tau * a.adv[t];
  // beta_t: the KL coefficient, scaled by 1/sqrt(1 + age) under inv_sqrt staleness
  const int32_t age = a.age != nullptr ? max(a.age[t], 0) : 0;
  const float beta =
      a.staleness == RL_STALENESS_INV_SQRT ? a.beta * rsqrtf(1.0f + (float)age) : a.beta;

  // Support entries: one wave per entry, entries strided over the 4 waves;
  // each wave keeps its own running sums, combined in wave order.
  const int wave = tid >> 6, lane = tid & 63;
  float sc = 0.0f, cent = 0.0f, su = 0.0f, kl = 0.0f, sm = 0.0f;
  int64_t e0 = 0, e1 = 0;
  if (a.off != nullptr) {
    // Device offsets are clamped into [0, nnz] so a corrupted copy cannot
    // send a read out of bounds.
    e0 = min(max(a.off[t], (int64_t)0), a.nnz);
    e1 = min(max(a.off[t + 1], e0), a.nnz);
  }
  if (a.off != nullptr && a.zent != nullptr) {
    // entry logits precomputed (entry_logits_kernel): one entry per lane
    for (int64_t eb = e0 + tid - lane; eb < e1; eb += NT) {
      const int64_t e = eb + lane;
      if (e < e1) {
        const float lpe = a.inv_t * a.zent[a.N + e] - lse;
        const float ue = a.u[e];
        const float lqe = a.logq != nullptr ? a.logq[e] : logf(ue);
        bool ke;
        const float we = rl_weight(lpe, lqe, a.wp, &ke);
        const float ce = ue * we;
        sc += ce;
        cent += ce * lpe;
        su += ue;
        kl += ue * (lqe - lpe);
        sm += ue * __expf(lpe - lqe);
        a.coef[a.N + e] = (s * ce - beta * ue) * a.inv_t * a.inv_D;
        if (a.o_support_lp != nullptr) a.o_support_lp[e] = lpe;
      }
    }
    sc = wave_sum(sc);
    cent = wave_sum(cent);
    su = wave_sum(su);
    kl = wave_sum(kl);
    sm = wave_sum(sm);
  } else if (a.off != nullptr) {
    // Wave w takes entries w, w + 4, ... in order; four of them per step so
    // that their row loads are in flight together (the order of every sum is
    // unchanged).
    for (int64_t eb = e0 + wave; eb < e1; eb += 16) {
      float zq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t ej = eb + 4 * j;
        const int32_t v = ej < e1 ? a.ids[ej] : -1;
        const bool v_ok = v >= 0 && v < a.V;
        const int64_t vs = v_ok ? v : 0;  // a valid row; its product is discarded
        zq[j] = dot_row_part<T>(h, W + vs * a.H, a.H, lane, 64);
        zq[j] = v_ok ? zq[j] : NAN;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) zq[j] = wave_sum(zq[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
      const int64_t e = eb + 4 * j;
      if (e >= e1) break;
      const float ze = a.inv_t * zq[j];
      const float lpe = ze - lse;
      const float ue = a.u[e];
      const float lqe = a.logq != nullptr ? a.logq[e] : logf(ue);
      bool ke;
      const float we = rl_weight(lpe, lqe, a.wp, &ke);
      const float ce = ue * we;
      sc += ce;
      cent += ce * lpe;
      su += ue;
      kl += ue * (lqe - lpe);
      sm += ue * __expf(lpe - lqe);
      if (lane == 0) {
        a.coef[a.N + e] = (s * ce - beta * ue) * a.inv_t * a.inv_D;
        if (a.o_support_lp != nullptr) a.o_support_lp[e] = lpe;
      }
      }
    }
  }
  __syncthreads();
  if (lane == 0) {
    wsum[wave][0] = sc;
    wsum[wave][1] = cent;
    wsum[wave][2] = su;
    wsum[wave][3] = kl;
    wsum[wave][4] = sm;
  }
  __syncthreads();
  if (tid == 0) {
    float acc[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) acc[k] = ((wsum[0][k] + wsum[1][k]) + wsum[2][k]) + wsum[3][k];
    sc = acc[0];
    cent = acc[1];
    su = acc[2];
    kl = acc[3];
    sm = acc[4];
    const float klt = a.beta != 0.0f ? kl : 0.0f;
    const float loss = -s * (w * lp - cent) + beta * klt - a.gamma * ent;
    const float kappa = s * (w - sc) + beta * su;
    a.lse[t] = lse;
    // the dense coefficient with the entropy bonus folded in:
    // p (kappa + gamma (log p + H)) = p (kappa + gamma (H - lse) + gamma z)
    a.kappa_s[t] = (kappa + a.gamma * (ent - lse)) * a.inv_t * a.inv_D;
    a.coef[t] = -s * w * a.inv_t * a.inv_D;
    float* st = a.stats + t * STAT_N;
    st[STAT_LOSS] = loss;
    st[STAT_MASKED] = keep ? 0.0f : 1.0f;
    st[STAT_SMASS] = sm;
    st[STAT_HAS_SUPPORT] = (e1 > e0) ? 1.0f : 0.0f;
    st[STAT_TVFAIL] = fabsf(expf(lp) - expf(lq)) > a.wp.eps ? 1.0f : 0.0f;
    st[STAT_KL] = klt;
    st[STAT_ABS_KAPPA] = fabsf(kappa);
    st[STAT_ENTROPY] = ent;
    st[STAT_BETA] = beta;
    st[STAT_KL_AGE0] = age == 0 ? klt : 0.0f;
    st[STAT_AGE0] = age == 0 ? 1.0f : 0.0f;
    if (a.o_logprobs) a.o_logprobs[t] = lp;
    if (a.o_entropy) a.o_entropy[t] = ent;
    if (a.o_weight) a.o_weight[t] = w;
    if (a.o_keep) a.o_keep[t] = keep ? 1 : 0;
    if (a.o_token_loss) a.o_token_loss[t] = loss;
  }
}

// G (in place over P) and Gt from P = e^(z - m_tile) (token-major [Tc, ldp]):
// g[t, v] = exp(m - lse[t]) * P[t, v] * (kap[t] + gs (m + log P[t, v])) with
// m = m[t, v / vtile] (gs = 0 without the entropy bonus).  Tiles of 64
// tokens x 128 vocabulary entries (one online-softmax tile column per WG).
// Padding is written as zeros: G columns V..ldp and Gt columns Tc..Tck, which
// the dh and dW contractions read as part of their K ranges.
template <typename T>
__global__ void __launch_bounds__(NT) form_g_kernel(T* __restrict__ P, int64_t ldp,
                                                    T* __restrict__ Gt, int64_t ldgt,
                                                    const float* __restrict__ part_m, int64_t J,
                                                    int vtile, const float* __restrict__ lse,
                                                    const float* __restrict__ kap, float gs,
                                                    int64_t V, int64_t Tc, int write_g) {
  constexpr int VEC = Elem<T>::VEC, CPR = 128 / VEC;  // chunks per 128-wide P row
  __shared__ float scale[64], scale_b[64], mtile[64];
  __shared__ T tile[128][64 + VEC];  // [v][t]
  const int64_t t0 = (int64_t)blockIdx.x * 64, v0 = (int64_t)blockIdx.y * 128;
  if (threadIdx.x < 64) {
    const int64_t t = t0 + threadIdx.x;
    const float m = t < Tc ? part_m[t * J + v0 / vtile] : 0.0f;
    const float e = t < Tc ? __expf(m - lse[t]) : 0.0f;
    scale[threadIdx.x] = t < Tc ? kap[t] * e : 0.0f;
    scale_b[threadIdx.x] = gs * e;
    mtile[threadIdx.x] = m;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 64 * CPR; q += NT) {
    const int tl = q / CPR, vl = (q % CPR) * VEC;
    const int64_t t = t0 + tl, v = v0 + vl;
    float g[VEC];
    if (t < Tc) {
      T* row = P + t * ldp + v;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(row);
      float x[VEC];
      Elem<T>::unpack(raw, x);
      const float sc = scale[tl];
      if (gs != 0.0f) {
        // entropy bonus: x (sc + sb (m + log x)), 0 where x underflowed
        const float sb = scale_b[tl], m = mtile[tl];
#pragma unroll
        for (int k = 0; k < VEC; ++k)
          g[k] = (v + k < V && x[k] > 0.0f) ? x[k] * (sc + sb * (m + __logf(x[k]))) : 0.0f;
      } else {
#pragma unroll
        for (int k = 0; k < VEC; ++k) g[k] = (v + k < V) ? sc * x[k] : 0.0f;
      }
      const u32x4 packed = Elem<T>::pack(g);
      if (write_g) *reinterpret_cast<u32x4*>(row) = packed;
      Elem<T>::unpack(packed, g);  // the rounded values go to Gt as well
    } else {
#pragma unroll
      for (int k = 0; k < VEC; ++k) g[k] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < VEC; ++k) tile[vl + k][tl] = Elem<T>::from_f32(g[k]);
  }
  if (Gt == nullptr) return;
  __syncthreads();
  constexpr int CPT = 64 / VEC;  // chunks per 64-token Gt row segment
  for (int q = threadIdx.x; q < 128 * CPT; q += NT) {
    const int vl = q / CPT, tl = (q % CPT) * VEC;
    const int64_t v = v0 + vl;
    if (v >= V) continue;
    u32x4 out;
    T* e = reinterpret_cast<T*>(&out);
#pragma unroll
    for (int k = 0; k < VEC; ++k) e[k] = tile[vl][tl + k];
    *reinterpret_cast<u32x4*>(Gt + v * ldgt + t0 + tl) = out;
  }
}

// src [S rows, C cols] row-major -> tiled [C rows, S cols] (see kernels.h).
// One workgroup writes one 16 KB block (256 tiled rows x 32 tiled columns):
// it reads the 32 x 256 source patch with 16-byte loads into LDS, then writes
// the block contiguously in its swizzled order.  Out-of-range entries are 0.
// With dst2 the same patch also goes, untransposed, into 32 rows of the eight
// blocks of dst2's layout that it spans (2 KB contiguous per block).
__global__ void __launch_bounds__(NT) to_tiled_t_kernel(const bf16_t* __restrict__ src,
                                                        int64_t ld_src, int64_t S, int64_t C,
                                                        bf16_t* __restrict__ dst, int64_t KB,
                                                        bf16_t* __restrict__ dst2, int64_t KB2) {
  constexpr int PITCH = TILE_ROWS + 8;
  __shared__ __attribute__((aligned(16))) bf16_t tile[TILE_K][PITCH];  // [k][row]
  const int64_t rb = blockIdx.x, kb = blockIdx.y;
  const int64_t c0 = rb * TILE_ROWS, s0 = kb * TILE_K;
  for (int q = threadIdx.x; q < TILE_K * (TILE_ROWS / 8); q += NT) {
    const int sl = q / (TILE_ROWS / 8), cl = (q % (TILE_ROWS / 8)) * 8;
    const int64_t sr = s0 + sl, c = c0 + cl;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (sr < S && c < C) v = *reinterpret_cast<const u32x4*>(src + sr * ld_src + c);
    *reinterpret_cast<u32x4*>(&tile[sl][cl]) = v;
  }
  __syncthreads();
  if (dst != nullptr && kb < KB) {
    bf16_t* blk = dst + (rb * KB + kb) * (TILE_ROWS * TILE_K);
    for (int p = threadIdx.x; p < TILE_ROWS * 4; p += NT) {
      const int r = p >> 2, ch = (p & 3) ^ tile_swz(r);
      u32x4 out;
      bf16_t* e = reinterpret_cast<bf16_t*>(&out);
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] = tile[8 * ch + k][r];
      *reinterpret_cast<u32x4*>(blk + p * 8) = out;
    }
  }
  if (dst2 != nullptr) {
    // rows s0 % 256 + sl of panel s0 / 256; block c0 / 32 + b holds columns
    // c0 + 32 b ..; thread q: chunk q % 4 of row (q / 4) % 32 of block q / 128
    const int64_t pr = s0 / TILE_ROWS;
    const int r0 = (int)(s0 % TILE_ROWS);
    for (int q = threadIdx.x; q < TILE_K * 4 * (TILE_ROWS / TILE_K); q += NT) {
      const int c = q & 3, sl = (q >> 2) & (TILE_K - 1), b = q >> 7;
      const int64_t kb2 = c0 / TILE_K + b;
      if (kb2 >= KB2) continue;
      const int r = r0 + sl;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&tile[sl][TILE_K * b + 8 * c]);
      *reinterpret_cast<u32x4*>(dst2 + ((pr * KB2 + kb2) * TILE_ROWS + r) * TILE_K +
                                ((c ^ tile_swz(r)) << 3)) = v;
    }
  }
}

// Dense-gradient pass over the tiled layout (bf16).  The forward GEMM left
// e^(z - m_j) in G's tiled blocks (256 tokens x 32 vocabulary entries, each
// inside one vocabulary tile j).  Every element is scaled in place by
// kappa_t e^(m_tj - LSE_t) (with the entropy bonus, by
// e^(m_tj - LSE_t) (kappa_t + gs (m_tj + log x)), kappa_t holding the rest of
// that term), zero past Tc and V.  Both backward GEMMs read this one copy
// (dW through transposing LDS reads).  A workgroup takes NBLK consecutive
// blocks of one token panel and issues all their loads first (NBLK = 2, at
// the 16k shape: 4 was 8% faster than one block per workgroup and 2 another
// 1.7%; an in-place streaming probe ran 5.87 TB/s with two blocks per
// workgroup against 5.54 with four).
template <int NBLK>
__global__ void __launch_bounds__(NT) form_g_blocks_kernel(
    bf16_t* __restrict__ G, int64_t KB_g, const float* __restrict__ part_m, int64_t J, int vtile,
    const float* __restrict__ lse, const float* __restrict__ kap, float gs, int64_t V,
    int64_t Tc) {
  const int64_t tp = blockIdx.x, kb0 = (int64_t)blockIdx.y * NBLK;
  bf16_t* blk0 = G + (tp * KB_g + kb0) * (TILE_ROWS * TILE_K);
  // streaming: each element is read and written once here
  u32x4 raw[NBLK][4];
#pragma unroll
  for (int b = 0; b < NBLK; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      raw[b][q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          blk0 + b * (TILE_ROWS * TILE_K) + (threadIdx.x + NT * q) * 8));
  // The per-token values of all four rows, loaded before the first store:
  // loaded after it, each would wait for that store too (one in-order
  // counter for loads and stores).
  float lq[4], kq[4], mq[4][NBLK];
  int jt[NBLK];  // vocabulary tile of each block (uniform)
#pragma unroll
  for (int b = 0; b < NBLK; ++b)
    jt[b] = __builtin_amdgcn_readfirstlane((int)(((int)kb0 + b) * TILE_K / vtile));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // rows past Tc read row Tc - 1 (Tc > 0) and drop the values: no branches
    const int r = (threadIdx.x + NT * q) >> 2;
    const int64_t t = tp * TILE_ROWS + r;
    const bool tok = t < Tc;
    const int64_t tr = tok ? t : Tc - 1;
    const float l = lse[tr], k = kap[tr];
    lq[q] = tok ? l : 0.0f;
    kq[q] = tok ? k : 0.0f;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const float m = part_m[tr * J + jt[b]];
      mq[q][b] = tok ? m : 0.0f;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int p = threadIdx.x + NT * q;  // 16-byte chunk of a block
    const int r = p >> 2, lc = (p & 3) ^ tile_swz(r);
    const int64_t t = tp * TILE_ROWS + r;
    const bool tok = t < Tc;
    const float l = lq[q], kt = kq[q];
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int64_t kb = kb0 + b, v = kb * TILE_K + lc * 8;
      const float m = mq[q][b];
      const float e = tok ? __expf(m - l) : 0.0f;
      const float sc = kt * e;
      float x[8];
      Elem<bf16_t>::unpack(raw[b][q], x);
      if (gs != 0.0f) {
        // entropy bonus: x (sc + sb (m + log x)), 0 where x underflowed
        const float sb = gs * e;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          x[k] = (v + k < V && x[k] > 0.0f) ? x[k] * (sc + sb * (m + __logf(x[k]))) : 0.0f;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = (v + k < V) ? sc * x[k] : 0.0f;
      }
      __builtin_nontemporal_store(Elem<bf16_t>::pack(x),
                                  reinterpret_cast<u32x4*>(blk0 + b * (TILE_ROWS * TILE_K) + p * 8));
    }
  }
}

// ---- label and support coefficients folded into the dense operand --------------
// Element offsets of (token tl of the chunk, vocabulary id v) in G and of
// (v, tl) in Gt: the tiled block layouts (16-byte chunks XOR-swizzled by row)
// or, untiled, row-major [Tc, ldg] and [V, ldgt].
struct GIndex {
  int tiled;
  int64_t ldg, ldgt;  // tiled: blocks per G row panel (KB_g) and per Gt row panel (KB_gt)
  __device__ __forceinline__ int64_t g(int64_t tl, int64_t v) const {
    return tiled ? tiled_offset(tl, v, ldg) : tl * ldg + v;
  }
  __device__ __forceinline__ int64_t gt(int64_t v, int64_t tl) const {
    return tiled ? tiled_offset(v, tl, ldgt) : v * ldgt + tl;
  }
};

// Adds c to the operand element (tl, v) in G (when it holds G) and in Gt (when
// present); both hold the same rounded value.  G holds the scaled operand only
// when it was written; otherwise the previous value is read from Gt.
template <typename T>
__device__ __forceinline__ void fold_add(T* G, int write_g, T* Gt, const GIndex& ix, int64_t tl,
                                         int64_t v, float c) {
  const int64_t ig = ix.g(tl, v), igt = ix.gt(v, tl);
  const float old = Gt != nullptr ? Elem<T>::to_f32(Gt[igt]) : Elem<T>::to_f32(G[ig]);
  const T nv = Elem<T>::from_f32(old + c);
  if (write_g) G[ig] = nv;
  if (Gt != nullptr) Gt[igt] = nv;
}

// One thread per token of the chunk: its label coefficient (one entry per
// token, so no two threads touch one element).
template <typename T>
__global__ void __launch_bounds__(NT) fold_labels_kernel(T* G, int write_g, T* Gt, GIndex ix,
                                                         const int32_t* __restrict__ labels,
                                                         const float* __restrict__ coef,
                                                         int64_t t0, int64_t Tc, int64_t V) {
  const int64_t tl = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (tl >= Tc) return;
  const int32_t v = labels[t0 + tl];
  if (v < 0 || v >= V) return;
  fold_add(G, write_g, Gt, ix, tl, (int64_t)v, coef[t0 + tl]);
}

// One thread per position of the vocabulary-sorted entry list.  A token's
// repeated ids are adjacent there (stable sort, entries in token order), so
// the first position of each (id, token) run sums the run's coefficients in
// entry order and updates the element once; the others do nothing.  Label
// entries (index < N) are folded separately, before.
template <typename T>
__global__ void __launch_bounds__(NT) fold_support_kernel(
    T* G, int write_g, T* Gt, GIndex ix, const int32_t* __restrict__ skeys,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ row_of,
    const float* __restrict__ coef, int64_t E, int64_t N, int64_t t0, int64_t Tc, int64_t V) {
  const int64_t p = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (p >= E) return;
  const int32_t i = perm[p];
  const int32_t v = skeys[p];
  if (i < N || v < 0 || v >= V) return;
  const int64_t t = row_of[i - N];
  if (t < t0 || t >= t0 + Tc) return;
  if (p > 0) {
    const int32_t ip = perm[p - 1];
    if (ip >= N && skeys[p - 1] == v && row_of[ip - N] == t) return;  // not the run's first
  }
  float c = coef[i];
  for (int64_t q = p + 1; q < E; ++q) {
    const int32_t iq = perm[q];
    if (iq < N || skeys[q] != v || row_of[iq - N] != t) break;
    c += coef[iq];
  }
  fold_add(G, write_g, Gt, ix, t - t0, (int64_t)v, c);
}

template <typename T, typename GT>
__global__ void __launch_bounds__(NT) finalize_dh_kernel(
    const float* __restrict__ part, int splits, int64_t split_stride, const T* __restrict__ W,
    const int32_t* __restrict__ labels, const int64_t* __restrict__ off,
    const int32_t* __restrict__ ids, const float* __restrict__ coef, int64_t t0, int64_t N,
    int64_t nnz, int64_t V, int64_t H, int with_sparse, GT* __restrict__ dh) {
  constexpr int VEC = 8;  // columns per thread per step
  const int64_t tl = blockIdx.x;
  const int64_t t = t0 + tl;
  // without with_sparse the label and support terms are already in the partials
  const int64_t e0 = (with_sparse && off) ? min(max(off[t], (int64_t)0), nnz) : 0;
  const int64_t e1 = (with_sparse && off) ? min(max(off[t + 1], e0), nnz) : 0;
  const int32_t lab = labels[t];
  const bool lab_ok = with_sparse && lab >= 0 && lab < V;
  const float cl = coef[t];
  for (int64_t c = (int64_t)threadIdx.x * VEC; c < H; c += (int64_t)NT * VEC) {
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
    for (int sp = 0; sp < splits; ++sp) {
      const float* p = part + sp * split_stride + tl * H + c;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += p[i];
    }
    if (lab_ok) {
      const T* wr = W + (int64_t)lab * H + c;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = fmaf(cl, Elem<T>::to_f32(wr[i]), acc[i]);
    }
    // entries in groups of 8 with their row loads issued together; an id
    // outside [0, V) reads row 0 with coefficient 0
    for (int64_t eb = e0; eb < e1; eb += 8) {
      float ce[8];
      const T* wr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t e = eb + j;
        const int32_t v = e < e1 ? ids[e] : -1;
        const bool ok = v >= 0 && v < V;
        ce[j] = ok ? coef[N + e] : 0.0f;
        wr[j] = W + (ok ? (int64_t)v : 0) * H + c;
      }
      constexpr int EV = Elem<T>::VEC, NV = VEC / EV;  // 16-byte loads per row piece
      u32x4 raw[8][NV];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int q = 0; q < NV; ++q) raw[j][q] = *reinterpret_cast<const u32x4*>(wr[j] + q * EV);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float x[VEC];
#pragma unroll
        for (int q = 0; q < NV; ++q) Elem<T>::unpack(raw[j][q], x + q * EV);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] = fmaf(ce[j], x[i], acc[i]);
      }
    }
    GT* o = dh + t * H + c;
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = Elem<GT>::from_f32(acc[i]);
  }
}

__global__ void __launch_bounds__(1024) reduce_final_kernel(const float* __restrict__ stats,
                                                            int64_t N, float inv_D, float* loss,
                                                            float* metrics) {
  __shared__ double sh[STAT_N][16];
  double acc[STAT_N];
#pragma unroll
  for (int k = 0; k < STAT_N; ++k) acc[k] = 0.0;
  for (int64_t t = threadIdx.x; t < N; t += 1024) {
    const float* st = stats + t * STAT_N;
#pragma unroll
    for (int k = 0; k < STAT_N; ++k) {
      if (k == STAT_ABS_KAPPA)
        acc[k] = fmax(acc[k], (double)st[k]);
      else
        acc[k] += (double)st[k];
    }
  }
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < STAT_N; ++k) {
    double v = acc[k];
    if (k == STAT_ABS_KAPPA) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
    } else {
      v = wave_sum_d(v);
    }
    if (lane == 0) sh[k][w] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double r[STAT_N];
#pragma unroll
    for (int k = 0; k < STAT_N; ++k) {
      double v = sh[k][0];
      for (int i = 1; i < 16; ++i) v = (k == STAT_ABS_KAPPA) ? fmax(v, sh[k][i]) : v + sh[k][i];
      r[k] = v;
    }
    const double n = (double)N;
    *loss = (float)(r[STAT_LOSS] * (double)inv_D);
    if (metrics) {
      metrics[RL_METRIC_MASKED_FRACTION] = (float)(r[STAT_MASKED] / n);
      metrics[RL_METRIC_SUPPORT_MASS] =
          r[STAT_HAS_SUPPORT] > 0 ? (float)(r[STAT_SMASS] / r[STAT_HAS_SUPPORT]) : 0.0f;
      metrics[RL_METRIC_MASK_TV] = (float)(r[STAT_TVFAIL] / n);
      metrics[RL_METRIC_KL] = (float)(r[STAT_KL] / n);
      metrics[RL_METRIC_KL_BETA] = (float)(r[STAT_BETA] / n);
      metrics[RL_METRIC_MAX_ABS_KAPPA] = (float)r[STAT_ABS_KAPPA];
      metrics[RL_METRIC_ENTROPY_MEAN] = (float)(r[STAT_ENTROPY] / n);
      metrics[RL_METRIC_KL_AGE0] =
          r[STAT_AGE0] > 0 ? (float)(r[STAT_KL_AGE0] / r[STAT_AGE0]) : 0.0f;
    }
  }
}

// One wave per row; its lanes write the row's entries (coalesced).
__global__ void csr_rows_kernel(const int64_t* __restrict__ off, int64_t N, int64_t nnz,
                                int32_t* __restrict__ row_of) {
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= N) return;
  if (t == 0)  // entries before the first row keep a marker no bucket reads
    for (int64_t e = lane; e < min(max(off[0], (int64_t)0), nnz); e += 64) row_of[e] = -1;
  const int64_t e0 = min(max(off[t], (int64_t)0), nnz);
  const int64_t e1 = min(max(off[t + 1], e0), nnz);
  for (int64_t e = e0 + lane; e < e1; e += 64) row_of[e] = (int32_t)t;
}

}  // namespace

hipError_t transpose_pad(int dtype, const void* src, int64_t ld_src, int64_t R, int64_t C,
                         void* dst, int64_t Rpad, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(Rpad, 64), (unsigned)ceil_div(C, 64));
  if (dtype == RL_DTYPE_BF16)
    hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, dim3(NT), 0, s,
                       static_cast<const bf16_t*>(src), ld_src, R, C, static_cast<bf16_t*>(dst),
                       Rpad);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(NT), 0, s,
                       static_cast<const float*>(src), ld_src, R, C, static_cast<float*>(dst),
                       Rpad);
  return hipGetLastError();
}

hipError_t entry_logits(int dtype, const void* h, const void* W, int64_t H, int64_t V,
                        const int32_t* skeys, const int32_t* perm, const int32_t* row_of,
                        int64_t N, int64_t E, float* z, hipStream_t s) {
  if (E <= 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(E, (int64_t)(NT / 64) * 64));
  if (dtype == RL_DTYPE_BF16)
    hipLaunchKernelGGL(entry_logits_kernel<bf16_t>, grid, dim3(NT), 0, s,
                       static_cast<const bf16_t*>(h), static_cast<const bf16_t*>(W), H, V, skeys,
                       perm, row_of, N, E, z);
  else
    hipLaunchKernelGGL(entry_logits_kernel<float>, grid, dim3(NT), 0, s,
                       static_cast<const float*>(h), static_cast<const float*>(W), H, V, skeys,
                       perm, row_of, N, E, z);
  return hipGetLastError();
}

hipError_t combine(int dtype, const CombineArgs& a, hipStream_t s) {
  if (a.Tc <= 0) return hipSuccess;
  if (dtype == RL_DTYPE_BF16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3((unsigned)a.Tc), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)a.Tc), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t form_g(int dtype, void* P, int64_t ldp, void* Gt, int64_t ldgt, const float* part_m,
                  int64_t J, int vtile, const float* lse_c, const float* kappa_c, float gs,
                  int64_t V, int64_t Tc, int64_t Tck, int write_g, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(Tck, 64), (unsigned)ceil_div(ldp, 128));
  if (dtype == RL_DTYPE_BF16)
    hipLaunchKernelGGL(form_g_kernel<bf16_t>, grid, dim3(NT), 0, s, static_cast<bf16_t*>(P), ldp,
                       static_cast<bf16_t*>(Gt), ldgt, part_m, J, vtile, lse_c, kappa_c, gs, V,
                       Tc, write_g);
  else
    hipLaunchKernelGGL(form_g_kernel<float>, grid, dim3(NT), 0, s, static_cast<float*>(P), ldp,
                       static_cast<float*>(Gt), ldgt, part_m, J, vtile, lse_c, kappa_c, gs, V,
                       Tc, write_g);
  return hipGetLastError();
}

hipError_t to_tiled_t(const bf16_t* src, int64_t ld_src, int64_t S, int64_t C, bf16_t* dst,
                      int64_t KB, int64_t kb_write, hipStream_t s, bf16_t* dst2, int64_t KB2) {
  if (dst2 != nullptr && KB2 < ceil_div(C, TILE_K)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)ceil_div(C, TILE_ROWS), (unsigned)kb_write);
  hipLaunchKernelGGL(to_tiled_t_kernel, grid, dim3(NT), 0, s, src, ld_src, S, C, dst, KB, dst2,
                     KB2);
  return hipGetLastError();
}

hipError_t form_g_blocks(bf16_t* G, int64_t KB_g, const float* part_m, int64_t J, int vtile,
                         const float* lse_c, const float* kappa_c, float gs, int64_t V,
                         int64_t Tc, hipStream_t s) {
  if (Tc <= 0) return hipSuccess;
  const unsigned panels = (unsigned)ceil_div(Tc, TILE_ROWS);
  if (KB_g % 2 == 0)
    hipLaunchKernelGGL(form_g_blocks_kernel<2>, dim3(panels, (unsigned)(KB_g / 2)), dim3(NT), 0,
                       s, G, KB_g, part_m, J, vtile, lse_c, kappa_c, gs, V, Tc);
  else
    hipLaunchKernelGGL(form_g_blocks_kernel<1>, dim3(panels, (unsigned)KB_g), dim3(NT), 0, s, G,
                       KB_g, part_m, J, vtile, lse_c, kappa_c, gs, V, Tc);
  return hipGetLastError();
}

hipError_t finalize_dh(int dtype, int grad_dtype, const float* part, int splits,
                       int64_t split_stride, const void* W, const int32_t* labels,
                       const int64_t* off, const int32_t* ids, const float* coef, int64_t t0,
                       int64_t Tc, int64_t N, int64_t nnz, int64_t V, int64_t H,
                       int with_sparse, void* dh, hipStream_t s) {
  if (Tc <= 0) return hipSuccess;
  const dim3 grid((unsigned)Tc);
#define RL_FIN(T, GT)                                                                           \
  hipLaunchKernelGGL((finalize_dh_kernel<T, GT>), grid, dim3(NT), 0, s, part, splits,          \
                     split_stride, static_cast<const T*>(W), labels, off, ids, coef, t0, N, nnz, \
                     V, H, with_sparse, static_cast<GT*>(dh))
  if (dtype == RL_DTYPE_BF16) {
    if (grad_dtype == RL_DTYPE_BF16) RL_FIN(bf16_t, bf16_t); else RL_FIN(bf16_t, float);
  } else {
    if (grad_dtype == RL_DTYPE_BF16) RL_FIN(float, bf16_t); else RL_FIN(float, float);
  }
#undef RL_FIN
  return hipGetLastError();
}

hipError_t fold_sparse(int dtype, void* G, int write_g, void* Gt, int tiled, int64_t ldg,
                       int64_t ldgt, const int32_t* labels, const int32_t* skeys,
                       const int32_t* perm, const int32_t* row_of, const float* coef, int64_t N,
                       int64_t nnz, int64_t t0, int64_t Tc, int64_t V, hipStream_t s) {
  if (Tc <= 0) return hipSuccess;
  const GIndex ix{tiled, ldg, ldgt};
  const int64_t E = N + nnz;
#define RL_FOLD(T)                                                                               \
  do {                                                                                           \
    hipLaunchKernelGGL(fold_labels_kernel<T>, dim3((unsigned)ceil_div(Tc, NT)), dim3(NT), 0, s,  \
                       static_cast<T*>(G), write_g, static_cast<T*>(Gt), ix, labels, coef, t0,  \
                       Tc, V);                                                                   \
    if (nnz > 0)                                                                                 \
      hipLaunchKernelGGL(fold_support_kernel<T>, dim3((unsigned)ceil_div(E, NT)), dim3(NT), 0,   \
                         s, static_cast<T*>(G), write_g, static_cast<T*>(Gt), ix, skeys, perm,  \
                         row_of, coef, E, N, t0, Tc, V);                                         \
  } while (0)
  if (dtype == RL_DTYPE_BF16) RL_FOLD(bf16_t); else RL_FOLD(float);
#undef RL_FOLD
  return hipGetLastError();
}

// beta is not needed here: each token's KL coefficient (beta, or its
// staleness-scaled value) is applied in combine, before the per-token stats.
hipError_t reduce_final(const float* stats, int64_t N, float inv_D, float /*beta*/, float* loss,
                        float* metrics, hipStream_t s) {
  hipLaunchKernelGGL(reduce_final_kernel, dim3(1), dim3(1024), 0, s, stats, N, inv_D, loss,
                     metrics);
  return hipGetLastError();
}

hipError_t csr_rows(const int64_t* off, int64_t N, int64_t nnz, int32_t* row_of, hipStream_t s) {
  hipLaunchKernelGGL(csr_rows_kernel, dim3((unsigned)ceil_div(N, 4)), dim3(256), 0, s, off, N,
                     nnz, row_of);
  return hipGetLastError();
}

}  // namespace rl
