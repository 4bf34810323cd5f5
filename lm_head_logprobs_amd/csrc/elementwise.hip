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
// Each 256-thread block handles 2048 consecutive tokens (two 16-byte loads per
// stream per thread, non-temporal), writes a uint16 mask word and the primary
// IPO weight per token, and one row of fp64 partial sums (fp32 per thread over
// 8 tokens, fp64 from the wave reduction on).  A single-block pass then sums
// the block rows in a fixed order, so the totals are deterministic.
#include "kernels.h"

namespace rl {
namespace {

constexpr int NT = 256;
constexpr int PER = 8;  // tokens per thread (multiple of 4)
constexpr int NS = RL_ELEM_SUM_COUNT;

struct ElemP {
  int n_eps, primary;
  float eps[RL_ELEM_MAX_EPS];
  float M, lo, hi, cl, ch, c, U;
};

__device__ __forceinline__ void token(float lp, float lq, float A, const ElemP& p, float* acc,
                                      uint32_t* word, float* wprim) {
  const float P = __expf(lp), Q = __expf(lq), r = __expf(lp - lq);
  const float dPQ = fabsf(P - Q);
  uint32_t wd = 0;
  float wp = 0.0f;
#pragma unroll
  for (int i = 0; i < RL_ELEM_MAX_EPS; ++i) {
    if (i < p.n_eps) {
      const bool masked = dPQ > p.eps[i];
      const float w = masked ? 0.0f : fminf(r, p.M);
      wd |= (uint32_t)masked << (RL_ELEM_BIT_IPO0 + i);
      acc[3 * i + 0] += masked ? 0.0f : 1.0f;
      acc[3 * i + 1] += -A * w * lp;
      acc[3 * i + 2] += w;
      if (i == p.primary) wp = w;
    }
  }
  {
    const bool low = r < p.lo, high = r > p.hi, kept = !(low || high);
    const float w = kept ? r : 0.0f;
    wd |= ((uint32_t)low << RL_ELEM_BIT_ICEPOP_LOW) | ((uint32_t)high << RL_ELEM_BIT_ICEPOP_HIGH);
    acc[RL_ELEM_ICEPOP_KEPT] += kept ? 1.0f : 0.0f;
    acc[RL_ELEM_ICEPOP_LOW] += low ? 1.0f : 0.0f;
    acc[RL_ELEM_ICEPOP_HIGH] += high ? 1.0f : 0.0f;
    acc[RL_ELEM_ICEPOP_LOSS] += -A * w * lp;
    acc[RL_ELEM_ICEPOP_WEIGHT] += w;
  }
  acc[RL_ELEM_REINFORCE_LOSS] += -A * lp;
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
    acc[RL_ELEM_PPO_LOSS] += -J;
    acc[RL_ELEM_PPO_CLIP] += clip ? 1.0f : 0.0f;
    acc[RL_ELEM_PPO_CLIP_LOWER] += dual ? 1.0f : 0.0f;
    acc[RL_ELEM_PPO_KL] += lq - lp;
  }
  {
    const bool trunc = r > p.U;
    const float w = fminf(r, p.U);
    wd |= (uint32_t)trunc << RL_ELEM_BIT_TIS_TRUNC;
    acc[RL_ELEM_TIS_LOSS] += -w * A;
    acc[RL_ELEM_TIS_TRUNC] += trunc ? 1.0f : 0.0f;
    acc[RL_ELEM_TIS_WEIGHT] += w;
  }
  *word = wd;
  *wprim = wp;
}

// Fixed-order block reduction of NS sums through LDS: every thread stores its
// fp32 partials; lane k of each wave then adds the 64 values of sum k of its
// wave in fp64 and lane order; finally the 4 wave results are added in wave
// order.  Deterministic and free of cross-lane shuffles.
__device__ __forceinline__ void block_reduce_store(const float* acc, double* out) {
  __shared__ float vals[NS][NT + 1];
  __shared__ double wsum[4][NS];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < NS; ++k) vals[k][threadIdx.x] = acc[k];
  __syncthreads();
  if (lane < NS) {
    double sacc = 0.0;
    const float* row = &vals[lane][w * 64];
#pragma unroll 8
    for (int i = 0; i < 64; ++i) sacc += (double)row[i];
    wsum[w][lane] = sacc;
  }
  __syncthreads();
  if (threadIdx.x < NS) {
    const int k = threadIdx.x;
    out[k] = ((wsum[0][k] + wsum[1][k]) + wsum[2][k]) + wsum[3][k];
  }
}

__global__ void __launch_bounds__(NT) elem_main_kernel(const float* __restrict__ lp,
                                                       const float* __restrict__ lq,
                                                       const float* __restrict__ adv, int64_t N,
                                                       ElemP p, uint16_t* __restrict__ word,
                                                       float* __restrict__ wprim,
                                                       double* __restrict__ partials) {
  float acc[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) acc[k] = 0.0f;
  // PER consecutive tokens per thread, as PER/4 16-byte vectors per stream;
  // the vectors of one thread are NT*4 tokens apart so a wave's loads are
  // contiguous.
  const int64_t base = (int64_t)blockIdx.x * NT * PER + (int64_t)threadIdx.x * 4;
  if (base + (int64_t)NT * 4 * (PER / 4 - 1) + 4 <= N) {
    f32x4 a[PER / 4], b[PER / 4], c[PER / 4];
#pragma unroll
    for (int v = 0; v < PER / 4; ++v) {
      const int64_t i0 = base + (int64_t)v * NT * 4;
      a[v] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(lp + i0));
      b[v] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(lq + i0));
      c[v] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(adv + i0));
    }
#pragma unroll
    for (int v = 0; v < PER / 4; ++v) {
      const int64_t i0 = base + (int64_t)v * NT * 4;
      uint32_t wd[4];
      float wv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) token(a[v][k], b[v][k], c[v][k], p, acc, &wd[k], &wv[k]);
      if (word) {
        uint2 pk;
        pk.x = wd[0] | (wd[1] << 16);
        pk.y = wd[2] | (wd[3] << 16);
        __builtin_nontemporal_store(pk.x, reinterpret_cast<uint32_t*>(word + i0));
        __builtin_nontemporal_store(pk.y, reinterpret_cast<uint32_t*>(word + i0) + 1);
      }
      if (wprim) {
        f32x4 o = {wv[0], wv[1], wv[2], wv[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(wprim + i0));
      }
    }
  } else {
    for (int v = 0; v < PER / 4; ++v)
      for (int k = 0; k < 4; ++k) {
        const int64_t i = base + (int64_t)v * NT * 4 + k;
        if (i >= N) continue;
        uint32_t wd;
        float wv;
        token(lp[i], lq[i], adv[i], p, acc, &wd, &wv);
        if (word) word[i] = (uint16_t)wd;
        if (wprim) wprim[i] = wv;
      }
  }
  block_reduce_store(acc, partials + (int64_t)blockIdx.x * NS);
}

// Sum of the per-block rows: thread t adds rows t, t + NT, ... in that
// order (all NS sums, fp64), then a fixed-order tree over the threads in LDS.
__global__ void __launch_bounds__(NT) elem_final_kernel(const double* __restrict__ partials,
                                                        int64_t nb, double* __restrict__ sums) {
  __shared__ double part[NS][NT];
  double acc[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) acc[k] = 0.0;
  for (int64_t b = threadIdx.x; b < nb; b += NT) {
    const double* row = partials + b * NS;
#pragma unroll
    for (int k = 0; k < NS; ++k) acc[k] += row[k];
  }
#pragma unroll
  for (int k = 0; k < NS; ++k) part[k][threadIdx.x] = acc[k];
  __syncthreads();
  for (int stride = NT / 2; stride > 0; stride >>= 1) {
    for (int q = threadIdx.x; q < NS * stride; q += NT) {
      const int k = q / stride, i = q % stride;
      part[k][i] += part[k][i + stride];
    }
    __syncthreads();
  }
  if (threadIdx.x < NS) sums[threadIdx.x] = part[threadIdx.x][0];
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
  return hipGetLastError();
}

hipError_t elementwise_final(const double* partials, int64_t N, double* sums, hipStream_t s) {
  hipLaunchKernelGGL(elem_final_kernel, dim3(1), dim3(NT), 0, s, partials, elem_num_blocks(N),
                     sums);
  return hipGetLastError();
}

}  // namespace rl
