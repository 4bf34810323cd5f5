// Loss-only mismatch replay: one HBM pass over (lp, lq, A) fp32 triples.
//
// Per token (P = e^lp, Q = e^lq, r = e^(lp - lq)):
//  * IPO for each eps (IPO documentation page, "Masking by Probability, Not
//    Ratio"; weight from prime-rl PR 4233, "What changes"): masked iff
//    |P - Q| > eps, w = kept * min(r, max_ratio), l = -A w lp;
//  * IcePop band (same sources): low r < lo, high r > hi, w = kept * r;
//  * REINFORCE: l = -A lp;
//  * PPO with the rollout log-prob as old policy (Rollout Correction Methods
//    page, "Bypassing PPO importance sampling") and dual clip (Tencent
//    article on KL/clip/entropy, section 2): J = min(rA, clip(r) A), for
//    A < 0 J = max(J, c A), l = -J;
//  * decoupled PPO with token-level truncated IS ("Decoupled, 3-policy PPO
//    Importance Sampling", "Importance Sampling / Token Level"), with the
//    proximal policy equal to the trainer policy: w = min(r, U), l = -w A.
// Each 256-thread block handles 1024 consecutive tokens (one 16-byte load per
// stream per thread), writes a uint16 mask word and the primary IPO weight per
// token, and one row of fp64 partial sums.  A single-block pass then sums
// the block rows in block order, so the totals are deterministic.
#include "kernels.h"

namespace rl {
namespace {

constexpr int NT = 256;
constexpr int PER = 4;
constexpr int NS = RL_ELEM_SUM_COUNT;

struct ElemP {
  int n_eps, primary;
  float eps[RL_ELEM_MAX_EPS];
  float M, lo, hi, cl, ch, c, U;
};

__device__ __forceinline__ void token(float lp, float lq, float A, const ElemP& p, double* acc,
                                      uint32_t* word, float* wprim) {
  const float P = expf(lp), Q = expf(lq), r = expf(lp - lq);
  const float dPQ = fabsf(P - Q);
  uint32_t wd = 0;
  float wp = 0.0f;
#pragma unroll
  for (int i = 0; i < RL_ELEM_MAX_EPS; ++i) {
    if (i < p.n_eps) {
      const bool masked = dPQ > p.eps[i];
      const float w = masked ? 0.0f : fminf(r, p.M);
      wd |= (uint32_t)masked << (RL_ELEM_BIT_IPO0 + i);
      acc[3 * i + 0] += masked ? 0.0 : 1.0;
      acc[3 * i + 1] += (double)(-A * w * lp);
      acc[3 * i + 2] += (double)w;
      if (i == p.primary) wp = w;
    }
  }
  {
    const bool low = r < p.lo, high = r > p.hi, kept = !(low || high);
    const float w = kept ? r : 0.0f;
    wd |= ((uint32_t)low << RL_ELEM_BIT_ICEPOP_LOW) | ((uint32_t)high << RL_ELEM_BIT_ICEPOP_HIGH);
    acc[RL_ELEM_ICEPOP_KEPT] += kept ? 1.0 : 0.0;
    acc[RL_ELEM_ICEPOP_LOW] += low ? 1.0 : 0.0;
    acc[RL_ELEM_ICEPOP_HIGH] += high ? 1.0 : 0.0;
    acc[RL_ELEM_ICEPOP_LOSS] += (double)(-A * w * lp);
    acc[RL_ELEM_ICEPOP_WEIGHT] += (double)w;
  }
  acc[RL_ELEM_REINFORCE_LOSS] += (double)(-A * lp);
  {
    const float J1 = r * A;
    const float J2 = fminf(fmaxf(r, 1.0f - p.cl), 1.0f + p.ch) * A;
    const float Jmin = fminf(J1, J2);
    const float cA = p.c * A;
    const bool neg = A < 0.0f;
    const bool dual = neg && (cA > Jmin);
    const float J = neg ? fmaxf(Jmin, cA) : Jmin;
    const bool clip = J2 < J1;
    wd |= ((uint32_t)clip << RL_ELEM_BIT_PPO_CLIP) | ((uint32_t)dual << RL_ELEM_BIT_DUAL_CLIP);
    acc[RL_ELEM_PPO_LOSS] += (double)(-J);
    acc[RL_ELEM_PPO_CLIP] += clip ? 1.0 : 0.0;
    acc[RL_ELEM_PPO_CLIP_LOWER] += dual ? 1.0 : 0.0;
    acc[RL_ELEM_PPO_KL] += (double)(lq - lp);
  }
  {
    const bool trunc = r > p.U;
    const float w = fminf(r, p.U);
    wd |= (uint32_t)trunc << RL_ELEM_BIT_TIS_TRUNC;
    acc[RL_ELEM_TIS_LOSS] += (double)(-w * A);
    acc[RL_ELEM_TIS_TRUNC] += trunc ? 1.0 : 0.0;
    acc[RL_ELEM_TIS_WEIGHT] += (double)w;
  }
  *word = wd;
  *wprim = wp;
}

// Fixed-order block reduction of NS doubles: wave butterflies, then wave order.
__device__ __forceinline__ void block_reduce_store(double* acc, double* out) {
  __shared__ double sh[4][NS];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const double v = wave_sum_d(acc[k]);
    if (lane == 0) sh[w][k] = v;
  }
  __syncthreads();
  if (threadIdx.x < NS) {
    const int k = threadIdx.x;
    out[k] = ((sh[0][k] + sh[1][k]) + sh[2][k]) + sh[3][k];
  }
}

__global__ void __launch_bounds__(NT) elem_main_kernel(const float* __restrict__ lp,
                                                       const float* __restrict__ lq,
                                                       const float* __restrict__ adv, int64_t N,
                                                       ElemP p, uint16_t* __restrict__ word,
                                                       float* __restrict__ wprim,
                                                       double* __restrict__ partials) {
  double acc[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) acc[k] = 0.0;
  const int64_t i0 = ((int64_t)blockIdx.x * NT + threadIdx.x) * PER;
  if (i0 + PER <= N) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(lp + i0);
    const f32x4 b = *reinterpret_cast<const f32x4*>(lq + i0);
    const f32x4 c = *reinterpret_cast<const f32x4*>(adv + i0);
    uint32_t wd[PER];
    float wv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) token(a[k], b[k], c[k], p, acc, &wd[k], &wv[k]);
    if (word) {
      uint2 pk;
      pk.x = wd[0] | (wd[1] << 16);
      pk.y = wd[2] | (wd[3] << 16);
      *reinterpret_cast<uint2*>(word + i0) = pk;
    }
    if (wprim) {
      f32x4 o = {wv[0], wv[1], wv[2], wv[3]};
      *reinterpret_cast<f32x4*>(wprim + i0) = o;
    }
  } else {
    for (int64_t i = i0; i < N; ++i) {
      uint32_t wd;
      float wv;
      token(lp[i], lq[i], adv[i], p, acc, &wd, &wv);
      if (word) word[i] = (uint16_t)wd;
      if (wprim) wprim[i] = wv;
    }
  }
  block_reduce_store(acc, partials + (int64_t)blockIdx.x * NS);
}

__global__ void __launch_bounds__(NT) elem_final_kernel(const double* __restrict__ partials,
                                                        int64_t nb, double* __restrict__ sums) {
  double acc[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) acc[k] = 0.0;
  for (int64_t b = threadIdx.x; b < nb; b += NT) {
    const double* row = partials + b * NS;
#pragma unroll
    for (int k = 0; k < NS; ++k) acc[k] += row[k];
  }
  block_reduce_store(acc, sums);
}

}  // namespace

int64_t elem_num_blocks(int64_t N) { return std::max<int64_t>(ceil_div(N, (int64_t)NT * PER), 1); }

hipError_t elementwise(const float* lp, const float* lq, const float* adv, int64_t N,
                       const rl_elem_cfg& c, uint16_t* word, float* w_primary, double* partials,
                       double* sums, hipStream_t s) {
  ElemP p;
  p.n_eps = c.n_eps;
  p.primary = c.primary_eps_index;
  for (int i = 0; i < RL_ELEM_MAX_EPS; ++i) p.eps[i] = c.eps[i];
  p.M = c.max_ratio;
  p.lo = c.icepop_lo;
  p.hi = c.icepop_hi;
  p.cl = c.clip_low;
  p.ch = c.clip_high;
  p.c = c.clip_c;
  p.U = c.tis_upper;
  const int64_t nb = elem_num_blocks(N);
  hipLaunchKernelGGL(elem_main_kernel, dim3((unsigned)nb), dim3(NT), 0, s, lp, lq, adv, N, p,
                     word, w_primary, partials);
  hipLaunchKernelGGL(elem_final_kernel, dim3(1), dim3(NT), 0, s, partials, nb, sums);
  return hipGetLastError();
}

}  // namespace rl
