// Sequence-aware rollout correction over a replay of (lp, lq, A) fp32 token
// triples cut into sequences (Rollout Correction Methods page: "Config keys",
// "Importance Sampling", "Rejection Sampling", "Veto Mechanism", and the
// metrics of "Mismatch Monitoring Metrics" and "IS/RS Correction Metrics").
// With no separate proximal policy the token log ratio is d = lp - lq.
//
// Four stages, every reduction in a fixed order:
//  1. chunks of 256 tokens (one wave each): fp64 chunk totals of d and min d,
//     fp32 chunk totals of rho = e^d, lp and lq; token-level metric sums;
//     the chunk's words of the sequence-start bitmap cleared;
//  2. one wave per sequence: the sequence totals from the chunk totals of the
//     chunks it covers whole plus its boundary pieces read directly; the
//     sequence-level IS weight, rejection and veto decisions (in fp64); the
//     per-sequence metric terms; the sequence's start bit and the first
//     sequence of every chunk that begins inside it;
//  3. chunks again: each token finds its sequence from the chunk's first
//     sequence and a popcount of the start bits before it, then its bounded
//     weight, flags, and the sums for batch normalisation and the loss;
//  4. one block: the raw totals in a fixed order, then the metrics.
// Token log ratios are formed in fp64 (exact for fp32 inputs), so token-level
// decisions are the exact comparisons of the definition.
#include "kernels.h"

namespace rl {
namespace {

constexpr int NT = 256;
constexpr int kMaxBlocks = 1024;
constexpr int kChunk = 256;

// Raw totals: rows of per-block partials, total-major.
enum { R1_D = 0, R1_RHO, R1_K3, R1_CHI2, R1_ABSD, R1_CAT, R1_COUNT };  // stage 1
enum {
  R2_LPPL_T = 0, R2_PPL_T, R2_LPPL_R, R2_PPL_R, R2_DIFF, R2_ABSDIFF, R2_RATIO, R2_CHI2S, R2_VETO,
  R2_WBEFORE, R2_COUNT  // stage 2
};
enum {
  R3_TIS_LOW = 0, R3_TIS_HIGH, R3_RS_LOW, R3_RS_HIGH, R3_KEPT, R3_W_AFTER, R3_W_KEPT, R3_WA_KEPT,
  R3_MIN, R3_MAX, R3_COUNT  // stage 3; the last two are a min and a max
};
constexpr int R_TOTAL = R1_COUNT + R2_COUNT + R3_COUNT;

struct ChunkTot {
  double d, rho, lp, lq, min_d;
};

struct MisP {
  int tis_level, tis_mode, use_rs, rs_level, veto_on;
  double lL, lU;    // log TIS bounds
  double rlL, rlU;  // log RS bounds
  double lC;        // log veto threshold
};

__device__ __forceinline__ double wave_min_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmin(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_min_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// The xor butterflies above leave the same bits in every lane (each step adds
// a + b in one lane and b + a in its partner); reading lane 0 makes that
// visible to the compiler, so branches on the value are scalar.
__device__ __forceinline__ double uniform_d(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// The 4-token vector of lane `lane` in chunk c: whole (16-byte loads) or at
// the end of the input (element loads; tokens past N read as 0).
struct Tok4 {
  float lp[4], lq[4];
  bool in[4];
};
__device__ __forceinline__ Tok4 load_tok4(const float* __restrict__ lp,
                                          const float* __restrict__ lq, int64_t N, int c,
                                          int lane) {
  Tok4 t;
  const int64_t t0 = (int64_t)c * kChunk + 4 * lane;
  if (t0 + 4 <= N) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(lp + t0));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(lq + t0));
#pragma unroll
    for (int j = 0; j < 4; ++j) t.lp[j] = a[j], t.lq[j] = b[j], t.in[j] = true;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t.in[j] = t0 + j < N;
      t.lp[j] = t.in[j] ? lp[t0 + j] : 0.0f;
      t.lq[j] = t.in[j] ? lq[t0 + j] : 0.0f;
    }
  }
  return t;
}

// ---- stage 1: chunk totals and token metric sums ----------------------------
__global__ void __launch_bounds__(NT)
mis_chunk_kernel(const float* __restrict__ lp, const float* __restrict__ lq, int64_t N, int nch,
                 MisP p, ChunkTot* __restrict__ ct, uint32_t* __restrict__ bitmap,
                 double* __restrict__ part1) {
  __shared__ double fs[4][4];
  __shared__ double wt[4][8];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int stride = 4 * (int)gridDim.x;
  float f[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // k3 terms, rho^2 - 1, |d|, catastrophic count
  double wd = 0.0, wrho = 0.0;              // wave sums of the chunk totals
  for (int c = wv * (int)gridDim.x + (int)blockIdx.x; c < nch; c += stride) {
    const Tok4 t = load_tok4(lp, lq, N, c, lane);
    double sd = 0.0, mind = __builtin_inf();
    float v3[3] = {0.0f, 0.0f, 0.0f};  // rho, lp, lq
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double d = (double)t.lp[j] - (double)t.lq[j];
      const float x = (float)d;
      const float rho = __expf(x);
      // q = e^x - 1 - x and e^x - 1 without cancellation near x = 0: below
      // |x| = 0.5 the Taylor series to x^8 (truncation < 5e-8 relative)
      const float ser =
          x * x *
          (0.5f + x * (1.0f / 6 + x * (1.0f / 24 + x * (1.0f / 120 +
                                                       x * (1.0f / 720 + x * (1.0f / 5040 +
                                                                              x * (1.0f / 40320)))))));
      const bool small = fabsf(x) < 0.5f;
      const float q = small ? ser : (rho - 1.0f) - x;
      const float em1 = small ? x + ser : rho - 1.0f;
      if (t.in[j]) {
        sd += d;
        mind = fmin(mind, d);
        v3[0] += rho;
        v3[1] += t.lp[j];
        v3[2] += t.lq[j];
        f[0] += q;                               // e^d - d - 1
        f[1] = fmaf(em1, em1 + 2.0f, f[1]);      // rho^2 - 1
        f[2] += fabsf(x);
        f[3] += (p.veto_on && d < p.lC) ? 1.0f : 0.0f;
      }
    }
    const double tsd = uniform_d(wave_sum_d(sd));
    const double tmin = uniform_d(wave_min_d(mind));
    wave_totals<3>(v3, fs[wv], lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const double trho = fs[wv][0];
    if (lane == 0) {
      ChunkTot r;
      r.d = tsd, r.rho = trho, r.lp = fs[wv][1], r.lq = fs[wv][2], r.min_d = tmin;
      ct[c] = r;
    }
    if (lane < 8) bitmap[(int64_t)c * 8 + lane] = 0u;
    wd += tsd;
    wrho += trho;
    __builtin_amdgcn_wave_barrier();
  }
  wave_totals<4>(f, wt[wv], lane);
  if (lane == 0) wt[wv][4] = wd, wt[wv][5] = wrho;
  __syncthreads();
  if (threadIdx.x < R1_COUNT) {
    const int k = threadIdx.x;
    const int src = k == R1_D ? 4 : k == R1_RHO ? 5 : k - 2;  // k3, chi2, |d|, cat at 0..3
    part1[(int64_t)k * gridDim.x + blockIdx.x] =
        ((wt[0][src] + wt[1][src]) + wt[2][src]) + wt[3][src];
  }
}

// ---- stage 2: one wave per sequence ------------------------------------------
__global__ void __launch_bounds__(NT)
mis_seq_kernel(const float* __restrict__ lp, const float* __restrict__ lq, int64_t N,
               const int64_t* __restrict__ off, int S, MisP p, const ChunkTot* __restrict__ ct,
               float* __restrict__ seq_w, uint32_t* __restrict__ seq_flags,
               int* __restrict__ firstseq, uint32_t* __restrict__ bitmap,
               double* __restrict__ part2) {
  __shared__ double wt[4][R2_COUNT];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int stride = 4 * (int)gridDim.x;
  double acc[R2_COUNT];  // wave-uniform
#pragma unroll
  for (int k = 0; k < R2_COUNT; ++k) acc[k] = 0.0;
  for (int s = wv * (int)gridDim.x + (int)blockIdx.x; s < S; s += stride) {
    // clamped to [0, N] so that offsets that disagree with the host copy
    // cannot send a read out of bounds (the host checked its own copy)
    const int64_t b = std::min<int64_t>(std::max<int64_t>(off[s], 0), N - 1);
    const int64_t e = std::min<int64_t>(std::max<int64_t>(off[s + 1], b + 1), N);
    const int c0 = (int)(b / kChunk), c1 = (int)((e - 1) / kChunk);
    double sd = 0.0, srho = 0.0, slp = 0.0, slq = 0.0, mind = __builtin_inf();
    // chunks covered whole: their totals, lane i taking c0 + i, c0 + i + 64, ...
    for (int c = c0 + lane; c <= c1; c += 64) {
      const int64_t cb = (int64_t)c * kChunk, ce = std::min<int64_t>(cb + kChunk, N);
      if (cb >= b && ce <= e) {
        const ChunkTot r = ct[c];
        sd += r.d, srho += r.rho, slp += r.lp, slq += r.lq, mind = fmin(mind, r.min_d);
      }
    }
    // the chunks at either end that the sequence covers only in part
#pragma unroll
    for (int side = 0; side < 2; ++side) {
      const int c = side == 0 ? c0 : c1;
      if (side == 1 && c1 == c0) break;
      const int64_t cb = (int64_t)c * kChunk, ce = std::min<int64_t>(cb + kChunk, N);
      if (cb >= b && ce <= e) continue;
      const Tok4 t = load_tok4(lp, lq, N, c, lane);
      const int64_t t0 = cb + 4 * lane;
      float r = 0.0f, a = 0.0f, q = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = t.in[j] && t0 + j >= b && t0 + j < e;
        const double d = (double)t.lp[j] - (double)t.lq[j];
        if (in) {
          sd += d;
          mind = fmin(mind, d);
          r += __expf((float)d);
          a += t.lp[j];
          q += t.lq[j];
        }
      }
      srho += r, slp += a, slq += q;
    }
    sd = uniform_d(wave_sum_d(sd));
    srho = uniform_d(wave_sum_d(srho));
    slp = uniform_d(wave_sum_d(slp));
    slq = uniform_d(wave_sum_d(slq));
    mind = uniform_d(wave_min_d(mind));
    const double n = (double)(e - b);
    // importance weight of the sequence-level modes
    uint32_t fl = 0;
    float w_b = 0.0f;
    double wbefore = 0.0;
    if (p.tis_level != RL_LEVEL_TOKEN) {
      const double lw = p.tis_level == RL_LEVEL_SEQUENCE ? sd : sd / n;
      const bool low = p.tis_mode != RL_TIS_TRUNCATE && lw < p.lL;
      const bool high = lw > p.lU;
      double x;
      if (p.tis_mode == RL_TIS_TRUNCATE) x = exp(fmin(lw, p.lU));
      else if (p.tis_mode == RL_TIS_CLIP) x = exp(fmin(fmax(lw, p.lL), p.lU));
      else x = (low || high) ? 0.0 : exp(lw);
      w_b = (float)x;
      fl |= (low ? RL_MIS_F_TIS_LOW : 0u) | (high ? RL_MIS_F_TIS_HIGH : 0u);
      wbefore = n * exp(lw);
    }
    if (p.use_rs && p.rs_level != RL_LEVEL_TOKEN) {
      const double ls = p.rs_level == RL_LEVEL_SEQUENCE ? log(srho / n) : sd / n;
      fl |= (ls < p.rlL ? RL_MIS_F_RS_LOW : 0u) | (ls > p.rlU ? RL_MIS_F_RS_HIGH : 0u);
    }
    const bool vetoed = p.veto_on && mind < p.lC;
    fl |= vetoed ? RL_MIS_F_VETO : 0u;
    if (lane == 0) {
      seq_w[s] = w_b;
      seq_flags[s] = fl;
      atomicOr(&bitmap[b >> 5], 1u << (b & 31));
    }
    // the first sequence of every chunk whose first token lies in [b, e)
    for (int c = (int)((b + kChunk - 1) / kChunk) + lane; (int64_t)c * kChunk < e; c += 64)
      firstseq[c] = s;
    const double lt = -slp / n, lr = -slq / n;
    acc[R2_LPPL_T] += lt;
    acc[R2_PPL_T] += exp(lt);
    acc[R2_LPPL_R] += lr;
    acc[R2_PPL_R] += exp(lr);
    acc[R2_DIFF] += lt - lr;
    acc[R2_ABSDIFF] += fabs(lt - lr);
    acc[R2_RATIO] += exp(lt - lr);
    acc[R2_CHI2S] += expm1(2.0 * sd);
    acc[R2_VETO] += vetoed ? 1.0 : 0.0;
    acc[R2_WBEFORE] += wbefore;
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < R2_COUNT; ++k) wt[wv][k] = acc[k];
  }
  __syncthreads();
  if (threadIdx.x < R2_COUNT) {
    const int k = threadIdx.x;
    part2[(int64_t)k * gridDim.x + blockIdx.x] = ((wt[0][k] + wt[1][k]) + wt[2][k]) + wt[3][k];
  }
}

// ---- stage 3: per token ------------------------------------------------------
__global__ void __launch_bounds__(NT)
mis_token_kernel(const float* __restrict__ lp, const float* __restrict__ lq,
                 const float* __restrict__ adv, int64_t N, int nch, int S, MisP p,
                 const float* __restrict__ seq_w, const uint32_t* __restrict__ seq_flags,
                 const int* __restrict__ firstseq, const uint32_t* __restrict__ bitmap,
                 float* __restrict__ weight, uint8_t* __restrict__ flags,
                 double* __restrict__ part3) {
  __shared__ double wt[4][8];
  __shared__ float wmm[4][2];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int stride = 4 * (int)gridDim.x;
  // counts (exact in fp32 per thread) and weight sums
  float f[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  float wmin = __builtin_inff(), wmax = -__builtin_inff();
  // A chunk's vector inputs: the lane's four tokens and their advantages.
  struct In {
    Tok4 t;
    float A[4];
  };
  auto load_in = [&](int c) {
    In x;
    x.t = load_tok4(lp, lq, N, c, lane);
    const int64_t t0 = (int64_t)c * kChunk + 4 * lane;
    if (t0 + 4 <= N) {
      const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(adv + t0));
#pragma unroll
      for (int j = 0; j < 4; ++j) x.A[j] = a[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) x.A[j] = x.t.in[j] ? adv[t0 + j] : 0.0f;
    }
    return x;
  };
  // Each wave loads its next chunk's inputs before it works on the current
  // one, and the four tokens' sequence values are gathered together ahead of
  // that prefetch (loads and stores share one in-order counter: a gather
  // issued token by token, after the previous chunk's stores, waited for
  // each of them in turn).
  const int cfirst = wv * (int)gridDim.x + (int)blockIdx.x;
  In cur;
  if (cfirst < nch) cur = load_in(cfirst);
  for (int c = cfirst; c < nch; c += stride) {
    const int64_t t0 = (int64_t)c * kChunk + 4 * lane;
    // sequence of each token: the chunk's first sequence plus the starts in
    // (chunk start, token]
    const int s0 = std::min(std::max(firstseq[c], 0), S - 1);
    // the chunk's eight start-bit words are wave-uniform (scalar loads); the
    // lane's own word is selected from them rather than loaded per lane
    const uint32_t* bw = bitmap + (int64_t)c * 8;
    const int k = lane >> 3;  // word of the lane's 4 tokens
    int before = 0;
    uint32_t mk = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t m = __builtin_amdgcn_readfirstlane(bw[i]);
      m = i == 0 ? (m & ~1u) : m;
      before += i < k ? __builtin_popcount(m) : 0;
      mk = i == k ? m : mk;
    }
    const int bit0 = (4 * lane) & 31;
    // starts at or before the lane's first token within its word
    int cnt = before + __builtin_popcount(mk & (bit0 == 31 ? ~0u : ((2u << bit0) - 1u)));
    uint32_t sf[4];
    float swv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j > 0) cnt += (mk >> (bit0 + j)) & 1u;
      const int sj = std::min(s0 + cnt, S - 1);  // in range even for inconsistent offsets
      sf[j] = seq_flags[sj];
      swv[j] = p.tis_level != RL_LEVEL_TOKEN ? seq_w[sj] : 0.0f;
    }
    In nxt;  // read only when the loop goes on
    if (c + stride < nch) nxt = load_in(c + stride);
    const Tok4& t = cur.t;
    const float* A = cur.A;
    float wout[4];
    uint32_t fw = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double d = (double)t.lp[j] - (double)t.lq[j];
      uint32_t fl = 0;
      float w_b = 0.0f;
      if (t.in[j]) {
        const uint32_t sfj = sf[j];
        if (p.tis_level == RL_LEVEL_TOKEN) {
          const bool low = p.tis_mode != RL_TIS_TRUNCATE && d < p.lL;
          const bool high = d > p.lU;
          if (p.tis_mode == RL_TIS_TRUNCATE) w_b = __expf((float)fmin(d, p.lU));
          else if (p.tis_mode == RL_TIS_CLIP) w_b = __expf((float)fmin(fmax(d, p.lL), p.lU));
          else w_b = (low || high) ? 0.0f : __expf((float)d);
          fl |= (low ? RL_MIS_F_TIS_LOW : 0u) | (high ? RL_MIS_F_TIS_HIGH : 0u);
        } else {
          w_b = swv[j];
          fl |= sfj & (RL_MIS_F_TIS_LOW | RL_MIS_F_TIS_HIGH);
        }
        if (p.use_rs) {
          if (p.rs_level == RL_LEVEL_TOKEN)
            fl |= (d < p.rlL ? RL_MIS_F_RS_LOW : 0u) | (d > p.rlU ? RL_MIS_F_RS_HIGH : 0u);
          else
            fl |= sfj & (RL_MIS_F_RS_LOW | RL_MIS_F_RS_HIGH);
        }
        fl |= sfj & RL_MIS_F_VETO;
        fl |= (p.veto_on && d < p.lC) ? RL_MIS_F_CATASTROPHIC : 0u;
        const bool rej = (fl & (RL_MIS_F_RS_LOW | RL_MIS_F_RS_HIGH | RL_MIS_F_VETO)) != 0u;
        fl |= rej ? RL_MIS_F_REJECTED : 0u;
        const float w = rej ? 0.0f : w_b;
        f[R3_TIS_LOW] += (fl & RL_MIS_F_TIS_LOW) ? 1.0f : 0.0f;
        f[R3_TIS_HIGH] += (fl & RL_MIS_F_TIS_HIGH) ? 1.0f : 0.0f;
        f[R3_RS_LOW] += (fl & RL_MIS_F_RS_LOW) ? 1.0f : 0.0f;
        f[R3_RS_HIGH] += (fl & RL_MIS_F_RS_HIGH) ? 1.0f : 0.0f;
        f[R3_KEPT] += rej ? 0.0f : 1.0f;
        f[R3_W_AFTER] += w_b;
        f[R3_W_KEPT] += w;
        f[R3_WA_KEPT] = fmaf(w, A[j], f[R3_WA_KEPT]);
        if (!rej) wmin = fminf(wmin, w), wmax = fmaxf(wmax, w);
        wout[j] = w;
      } else {
        wout[j] = 0.0f;
      }
      fw |= fl << (8 * j);
    }
    if (t0 + 4 <= N) {
      if (weight) {
        const f32x4 o = {wout[0], wout[1], wout[2], wout[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(weight + t0));
      }
      if (flags) __builtin_nontemporal_store(fw, reinterpret_cast<uint32_t*>(flags + t0));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (t0 + j < N) {
          if (weight) weight[t0 + j] = wout[j];
          if (flags) flags[t0 + j] = (uint8_t)(fw >> (8 * j));
        }
    }
    cur = nxt;
  }
  wave_totals<8>(f, wt[wv], lane);
  wmin = wave_min_f(wmin);
  wmax = wave_max_f(wmax);
  if (lane == 0) wmm[wv][0] = wmin, wmm[wv][1] = wmax;
  __syncthreads();
  if (threadIdx.x < R3_COUNT) {
    const int k = threadIdx.x;
    double v;
    if (k == R3_MIN)
      v = fminf(fminf(wmm[0][0], wmm[1][0]), fminf(wmm[2][0], wmm[3][0]));
    else if (k == R3_MAX)
      v = fmaxf(fmaxf(wmm[0][1], wmm[1][1]), fmaxf(wmm[2][1], wmm[3][1]));
    else
      v = ((wt[0][k] + wt[1][k]) + wt[2][k]) + wt[3][k];
    part3[(int64_t)k * gridDim.x + blockIdx.x] = v;
  }
}

// ---- stage 4: raw totals and the metrics, one block ------------------------------
// Wave w reduces raw rows w, w + 16, ...: lane l adds entries l, l + 64, ...
// of the row in order, then a fixed xor tree (min and max for R3_MIN and
// R3_MAX).  Thread 0 then forms the metrics.
constexpr int FT = 1024;  // threads of the final block

__global__ void __launch_bounds__(FT)
mis_final_kernel(const double* __restrict__ part1, int64_t nb1, const double* __restrict__ part2,
                 int64_t nb2, const double* __restrict__ part3, int64_t nb3, int64_t N, int64_t S,
                 int tis_level, int batch_norm, double* __restrict__ m) {
  __shared__ double raw[R_TOTAL];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int r = wv; r < R_TOTAL; r += FT / 64) {
    const double* row;
    int64_t nb;
    int op = 0;  // 0 sum, 1 min, 2 max
    if (r < R1_COUNT) {
      row = part1 + (int64_t)r * nb1, nb = nb1;
    } else if (r < R1_COUNT + R2_COUNT) {
      row = part2 + (int64_t)(r - R1_COUNT) * nb2, nb = nb2;
    } else {
      const int k = r - R1_COUNT - R2_COUNT;
      row = part3 + (int64_t)k * nb3, nb = nb3;
      op = k == R3_MIN ? 1 : k == R3_MAX ? 2 : 0;
    }
    const double id = op == 1 ? __builtin_inf() : op == 2 ? -__builtin_inf() : 0.0;
    double v = id;
    // rows hold at most kMaxBlocks = 1024 entries: 16 per lane, all loads of a
    // round issued before the first add
    for (int64_t base = lane; base < nb; base += 64 * 16) {
      double x[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t b = base + 64 * j;
        x[j] = b < nb ? row[b] : id;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) v = op == 1 ? fmin(v, x[j]) : op == 2 ? fmax(v, x[j]) : v + x[j];
    }
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) {
      const double o = __shfl_xor(v, d, 64);
      v = op == 1 ? fmin(v, o) : op == 2 ? fmax(v, o) : v + o;
    }
    if (lane == 0) raw[r] = v;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  const double* r1 = raw;
  const double* r2 = raw + R1_COUNT;
  const double* r3 = raw + R1_COUNT + R2_COUNT;
  const double n = (double)N, s = (double)S;
  const double kept = r3[R3_KEPT], wk = r3[R3_W_KEPT];
  const double factor = (batch_norm && wk > 0.0) ? kept / wk : 1.0;
  m[RL_MIS_TRAINING_LOG_PPL] = r2[R2_LPPL_T] / s;
  m[RL_MIS_TRAINING_PPL] = r2[R2_PPL_T] / s;
  m[RL_MIS_ROLLOUT_LOG_PPL] = r2[R2_LPPL_R] / s;
  m[RL_MIS_ROLLOUT_PPL] = r2[R2_PPL_R] / s;
  m[RL_MIS_KL] = -r1[R1_D] / n;
  m[RL_MIS_K3_KL] = r1[R1_K3] / n;
  m[RL_MIS_LOG_PPL_DIFF] = r2[R2_DIFF] / s;
  m[RL_MIS_LOG_PPL_ABS_DIFF] = r2[R2_ABSDIFF] / s;
  m[RL_MIS_PPL_RATIO] = r2[R2_RATIO] / s;
  m[RL_MIS_CHI2_TOKEN] = r1[R1_CHI2] / n;
  m[RL_MIS_CHI2_SEQ] = r2[R2_CHI2S] / s;
  m[RL_MIS_LOGPROB_ABS_DIFF] = r1[R1_ABSD] / n;
  m[RL_MIS_TIS_WEIGHT_BEFORE_BOUND] =
      (tis_level == RL_LEVEL_TOKEN ? r1[R1_RHO] : r2[R2_WBEFORE]) / n;
  m[RL_MIS_TIS_WEIGHT_AFTER_BOUND] = r3[R3_W_AFTER] / n;
  m[RL_MIS_TIS_FRACTION_LOW] = r3[R3_TIS_LOW] / n;
  m[RL_MIS_TIS_FRACTION_HIGH] = r3[R3_TIS_HIGH] / n;
  m[RL_MIS_RS_FRACTION_LOW] = r3[R3_RS_LOW] / n;
  m[RL_MIS_RS_FRACTION_HIGH] = r3[R3_RS_HIGH] / n;
  m[RL_MIS_CATASTROPHIC_TOKEN_FRACTION] = r1[R1_CAT] / n;
  m[RL_MIS_CATASTROPHIC_SEQ_FRACTION] = r2[R2_VETO] / s;
  m[RL_MIS_IS_RATIO_MEAN_AFTER_TIS_RS] = wk / n;
  m[RL_MIS_BATCH_NORM_FACTOR] = factor;
  m[RL_MIS_IS_RATIO_MEAN_FINAL] = kept > 0.0 ? factor * wk / kept : 0.0;
  m[RL_MIS_IS_RATIO_MIN_FINAL] = kept > 0.0 ? factor * r3[R3_MIN] : 0.0;
  m[RL_MIS_IS_RATIO_MAX_FINAL] = kept > 0.0 ? factor * r3[R3_MAX] : 0.0;
  const double loss_sum = -factor * r3[R3_WA_KEPT];
  m[RL_MIS_LOSS] = kept > 0.0 ? loss_sum / kept : 0.0;
  m[RL_MIS_LOSS_SUM] = loss_sum;
  m[RL_MIS_KEPT_TOKENS] = kept;
  m[RL_MIS_REJECTED_TOKENS] = n - kept;
}

int64_t chunk_blocks(int64_t nch) { return std::min<int64_t>(ceil_div(nch, 4), kMaxBlocks); }
int64_t seq_blocks(int64_t S) { return std::min<int64_t>(ceil_div(S, 4), kMaxBlocks); }

}  // namespace

MisLayout mis_layout(int64_t N, int64_t S) {
  MisLayout L;
  const int64_t nch = ceil_div(N, kChunk);
  L.nch = nch;
  L.nb1 = chunk_blocks(nch);
  L.nb2 = seq_blocks(S);
  L.nb3 = L.nb1;
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o += round_up(bytes, 256);
    return at;
  };
  L.ct = take(nch * (int64_t)sizeof(ChunkTot));
  L.firstseq = take(nch * 4);
  L.bitmap = take(nch * 32);
  L.seq_w = take(S * 4);
  L.seq_flags = take(S * 4);
  L.part1 = take(R1_COUNT * L.nb1 * 8);
  L.part2 = take(R2_COUNT * L.nb2 * 8);
  L.part3 = take(R3_COUNT * L.nb3 * 8);
  L.bytes = o;
  return L;
}

hipError_t mis_stage(int stage, const float* lp, const float* lq, const float* adv, int64_t N,
                     const int64_t* off_dev, int64_t S, const rl_mis_cfg& c, float* weight,
                     uint8_t* flags, double* metrics, void* ws, hipStream_t s) {
  const MisLayout L = mis_layout(N, S);
  char* base = static_cast<char*>(ws);
  ChunkTot* ct = reinterpret_cast<ChunkTot*>(base + L.ct);
  int* firstseq = reinterpret_cast<int*>(base + L.firstseq);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + L.bitmap);
  float* seq_w = reinterpret_cast<float*>(base + L.seq_w);
  uint32_t* seq_flags = reinterpret_cast<uint32_t*>(base + L.seq_flags);
  double* part1 = reinterpret_cast<double*>(base + L.part1);
  double* part2 = reinterpret_cast<double*>(base + L.part2);
  double* part3 = reinterpret_cast<double*>(base + L.part3);
  MisP p;
  p.tis_level = c.tis_level, p.tis_mode = c.tis_mode, p.use_rs = c.use_rs;
  p.rs_level = c.rs_level, p.veto_on = c.veto > 0.0f;
  p.lL = std::log((double)c.tis_lower), p.lU = std::log((double)c.tis_upper);
  const float rl = std::isnan(c.rs_lower) ? c.tis_lower : c.rs_lower;
  const float ru = std::isnan(c.rs_upper) ? c.tis_upper : c.rs_upper;
  p.rlL = std::log((double)rl), p.rlU = std::log((double)ru);
  p.lC = p.veto_on ? std::log((double)c.veto) : -__builtin_inf();
  const int nch = (int)L.nch;
  switch (stage) {
    case 0:
      hipLaunchKernelGGL(mis_chunk_kernel, dim3((unsigned)L.nb1), dim3(NT), 0, s, lp, lq, N, nch,
                         p, ct, bitmap, part1);
      break;
    case 1:
      hipLaunchKernelGGL(mis_seq_kernel, dim3((unsigned)L.nb2), dim3(NT), 0, s, lp, lq, N,
                         off_dev, (int)S, p, ct, seq_w, seq_flags, firstseq, bitmap, part2);
      break;
    case 2:
      hipLaunchKernelGGL(mis_token_kernel, dim3((unsigned)L.nb3), dim3(NT), 0, s, lp, lq, adv, N,
                         nch, (int)S, p, seq_w, seq_flags, firstseq, bitmap, weight, flags, part3);
      break;
    default:
      hipLaunchKernelGGL(mis_final_kernel, dim3(1), dim3(FT), 0, s, part1, L.nb1, part2, L.nb2,
                         part3, L.nb3, N, S, c.tis_level, c.batch_normalize, metrics);
      break;
  }
  return hipGetLastError();
}

}  // namespace rl
