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
//
// The pass reads 12 bytes and writes 6 per token, so it is HBM-bound only if
// the arithmetic stays below about 70 VALU operations per token (wave64 fp32
// VALU issues one instruction per 4 cycles per SIMD).  To get there:
//  * |P - Q| = |Q (r - 1)| needs two exponentials, not three;
//  * the eps count is a template parameter (no per-eps branches);
//  * every mask bit's count is the popcount of the compare's own lane mask,
//    accumulated per wave on the scalar unit, which runs beside the VALU;
//  * the loss and weight sums are plain fp32 FMAs per thread.
// The grid holds at most kMaxBlocks blocks, all resident at once.  Each block
// writes its raw totals (float sums, counts, tokens) in fp64, stored
// total-major, and a second launch with one block per output sum combines
// the raw totals that output needs over the blocks in a fixed order, so the
// results are deterministic.
#include <mutex>

#include "kernels.h"

namespace rl {
namespace {

constexpr int NT = 256;
constexpr int kMaxBlocks = 1024;  // 4 resident 256-thread blocks per CU, 256 CUs
constexpr int NS = RL_ELEM_SUM_COUNT;

struct ElemP {
  float eps[RL_ELEM_MAX_EPS];
  float eps_primary;
  float M, lo, hi;
  float clo, chi;  // 1 - clip_low, 1 + clip_high
  float c, U;
  float ninf, pinf;  // -inf, +inf, held in VGPRs (see fmin_)
};

template <int NE>
struct Sums {
  static constexpr int NF = 2 * NE + 7;  // fp32 per-thread sums
  static constexpr int NC = NE + 5;      // wave-uniform mask-bit counts
  // float slots
  static constexpr int IPO = 0;          // 2i: sum w*(-A lp), 2i+1: sum w
  static constexpr int ICE = 2 * NE;     // loss, weight
  static constexpr int REINF = 2 * NE + 2;
  static constexpr int PPO_J = 2 * NE + 3;   // sum J   (loss = -sum)
  static constexpr int PPO_D = 2 * NE + 4;   // sum lp - lq (kl = -sum)
  static constexpr int TIS_WA = 2 * NE + 5;  // sum w A (loss = -sum)
  static constexpr int TIS_W = 2 * NE + 6;
  // count slots
  static constexpr int C_IPO = 0;        // masked count per eps
  static constexpr int C_LOW = NE, C_HIGH = NE + 1, C_CLIP = NE + 2, C_DUAL = NE + 3,
                       C_TRUNC = NE + 4;
};

// min / max as one v_med3_f32 against an infinity the compiler cannot see
// (with a literal infinity it turns the median into v_min / v_max, which in
// IEEE mode need their operands quieted first: two extra operations).  The
// inputs are finite.
__device__ __forceinline__ float fmin_(float a, float b, const ElemP& p) {
  return __builtin_amdgcn_fmed3f(a, b, p.ninf);
}
__device__ __forceinline__ float fmax_(float a, float b, const ElemP& p) {
  return __builtin_amdgcn_fmed3f(a, b, p.pinf);
}

__device__ __forceinline__ uint32_t lane_count(bool b) {
  return (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(b));
}

// One token.  Returns its mask word; adds into the per-thread float sums f
// and the per-wave counts c.  Every lane of the wave must call it (the counts
// are popcounts of whole-wave lane masks).  With GUARD, lanes whose `ok` is
// false (past the end of the input) contribute nothing.
template <int NE, bool GUARD>
__device__ __forceinline__ uint32_t token(float lp, float lq, float A, bool ok, const ElemP& p,
                                          float* f, uint32_t* c, float* wprim) {
  using S = Sums<NE>;
  if (GUARD && !ok) lp = lq = A = 0.0f;  // zero loss terms; weights are zeroed below
  const float d = lp - lq;
  const float r = __expf(d);
  const float Q = __expf(lq);
  const float dPQ = fabsf(fmaf(Q, r, -Q));  // |P - Q| with P = Q r
  const float Alp = -A * lp;
  const float rm = (GUARD && !ok) ? 0.0f : fmin_(r, p.M, p);
  uint32_t wd = 0;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const bool masked = dPQ > p.eps[i];  // false for the zeroed lanes (eps >= 0)
    const float w = masked ? 0.0f : rm;
    f[S::IPO + 2 * i] = fmaf(w, Alp, f[S::IPO + 2 * i]);
    f[S::IPO + 2 * i + 1] += w;
    wd |= masked ? (1u << (RL_ELEM_BIT_IPO0 + i)) : 0u;
    c[S::C_IPO + i] += lane_count(masked);
  }
  *wprim = dPQ > p.eps_primary ? 0.0f : rm;
  {
    bool low = r < p.lo, high = r > p.hi;
    if (GUARD) low = low && ok, high = high && ok;
    const float w = (low || high || (GUARD && !ok)) ? 0.0f : r;
    f[S::ICE] = fmaf(w, Alp, f[S::ICE]);
    f[S::ICE + 1] += w;
    wd |= (low ? (1u << RL_ELEM_BIT_ICEPOP_LOW) : 0u) |
          (high ? (1u << RL_ELEM_BIT_ICEPOP_HIGH) : 0u);
    c[S::C_LOW] += lane_count(low);
    c[S::C_HIGH] += lane_count(high);
  }
  f[S::REINF] += Alp;
  {
    // with A = 0 every term below is 0 and neither bit is set
    const float J1 = r * A;
    const float J2 = __builtin_amdgcn_fmed3f(r, p.clo, p.chi) * A;
    const float Jmin = fmin_(J1, J2, p);
    const float cA = p.c * A;
    const bool neg = A < 0.0f;
    const bool dual = neg && (cA > Jmin);
    const float J = neg ? fmax_(Jmin, cA, p) : Jmin;
    const bool clip = J2 < J1;
    f[S::PPO_J] += J;
    f[S::PPO_D] += d;
    wd |= (clip ? (1u << RL_ELEM_BIT_PPO_CLIP) : 0u) |
          (dual ? (1u << RL_ELEM_BIT_DUAL_CLIP) : 0u);
    c[S::C_CLIP] += lane_count(clip);
    c[S::C_DUAL] += lane_count(dual);
  }
  {
    bool trunc = r > p.U;
    if (GUARD) trunc = trunc && ok;
    const float w = (GUARD && !ok) ? 0.0f : fmin_(r, p.U, p);
    f[S::TIS_WA] = fmaf(w, A, f[S::TIS_WA]);
    f[S::TIS_W] += w;
    wd |= trunc ? (1u << RL_ELEM_BIT_TIS_TRUNC) : 0u;
    c[S::C_TRUNC] += lane_count(trunc);
  }
  // Pin the word and the weight in VGPRs here: otherwise the compiler sinks
  // their selects down to the stores and keeps every lane mask of the four
  // tokens alive in SGPRs until then.
  float wp = *wprim;
  __asm__ volatile("" : "+v"(wd), "+v"(wp));
  *wprim = wp;
  return wd;
}

struct Chunk {
  f32x4 lp, lq, A;
};

// The lane's 4-token vector of a whole 64-vector chunk.
__device__ __forceinline__ Chunk load_full(const f32x4* __restrict__ lp,
                                           const f32x4* __restrict__ lq,
                                           const f32x4* __restrict__ adv, int ch) {
  const int64_t v = (int64_t)ch * 64;
  return {__builtin_nontemporal_load(lp + v), __builtin_nontemporal_load(lq + v),
          __builtin_nontemporal_load(adv + v)};
}

// WORD / WPRIM: whether the mask words / primary weights are stored (as
// template parameters, so the token loop has no branches around the stores).
//
// Work split: the input is cut into chunks of 64 4-token vectors (one 16-byte
// vector per lane per stream).  Global wave slot s = wave * gridDim.x + block
// takes chunks s, s + S, s + 2S, ... (S = 4 gridDim.x, all slots resident),
// so the chunks left over after whole rounds go to wave 0 of distinct blocks,
// which sit on distinct CUs.  Each wave loads its next chunk before it works
// on the current one.
template <int NE, bool WORD, bool WPRIM>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 8)))
elem_main_kernel(const float* __restrict__ lp, const float* __restrict__ lq,
                 const float* __restrict__ adv, int64_t N, ElemP pk, uint16_t* __restrict__ word,
                 float* __restrict__ wprim, double* __restrict__ partials) {
  using S = Sums<NE>;
  float f[S::NF];
  uint32_t c[S::NC];
#pragma unroll
  for (int k = 0; k < S::NF; ++k) f[k] = 0.0f;
#pragma unroll
  for (int k = 0; k < S::NC; ++k) c[k] = 0;
  // The thresholds live in VGPRs (the asm hides that they are uniform): the
  // SGPRs are needed for the lane masks and the wave counts.
  ElemP p;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    p.eps[i] = pk.eps[i];
    __asm__ volatile("" : "+v"(p.eps[i]));
  }
  p.eps_primary = pk.eps_primary, p.M = pk.M, p.lo = pk.lo, p.hi = pk.hi;
  p.clo = pk.clo, p.chi = pk.chi, p.c = pk.c, p.U = pk.U;
  __asm__ volatile("" : "+v"(p.eps_primary), "+v"(p.M), "+v"(p.lo), "+v"(p.hi));
  __asm__ volatile("" : "+v"(p.clo), "+v"(p.chi), "+v"(p.c), "+v"(p.U));
  p.ninf = -__builtin_inff(), p.pinf = __builtin_inff();
  __asm__ volatile("" : "+v"(p.ninf), "+v"(p.pinf));
  // Chunk indices are 32-bit (the host limits N to 2^38 tokens).
  const int nfull = (int)(N / 256);  // chunks of 256 tokens entirely in range
  // The wave index is made provably uniform so that every branch below is a
  // scalar branch and the counts stay whole-wave values.
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int stride = 4 * (int)gridDim.x;
  const int slot = wv * (int)gridDim.x + (int)blockIdx.x;
  const f32x4* lp4 = reinterpret_cast<const f32x4*>(lp) + lane;
  const f32x4* lq4 = reinterpret_cast<const f32x4*>(lq) + lane;
  const f32x4* adv4 = reinterpret_cast<const f32x4*>(adv) + lane;
  int nown = 0;  // whole chunks this wave covers
  Chunk cur;
  if (slot < nfull) cur = load_full(lp4, lq4, adv4, slot);
  for (int ch = slot; ch < nfull; ch += stride) {
    Chunk nxt;
    if (ch + stride < nfull) nxt = load_full(lp4, lq4, adv4, ch + stride);
    ++nown;
    uint32_t wd[4];
    float wv4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wd[j] = token<NE, false>(cur.lp[j], cur.lq[j], cur.A[j], true, p, f, c, &wv4[j]);
      // one token's lane masks live at a time (they are SGPR pairs)
      __builtin_amdgcn_sched_barrier(0);
    }
    const int64_t v = (int64_t)ch * 64 + lane;
    if constexpr (WORD) {
      const u32x2 pk = {wd[0] | (wd[1] << 16), wd[2] | (wd[3] << 16)};
      __builtin_nontemporal_store(pk, reinterpret_cast<u32x2*>(word) + v);
    }
    if constexpr (WPRIM) {
      f32x4 o = {wv4[0], wv4[1], wv4[2], wv4[3]};
      __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(wprim) + v);
    }
    cur = nxt;
  }
  int64_t ntok = (int64_t)nown * 256;  // tokens this wave covers (uniform)
  // The chunk that holds the end of the input (N % 256 tokens), read token by
  // token, belongs to the slot that the round-robin gives it.
  if (N % 256 != 0 && nfull % stride == slot) {
    ntok += N % 256;
    const int64_t i0 = ((int64_t)nfull * 64 + lane) * 4;
    float x[4], y[4], z[4], wv4[4];
    uint32_t wd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = i0 + j < N;
      x[j] = in ? lp[i0 + j] : 0.0f;
      y[j] = in ? lq[i0 + j] : 0.0f;
      z[j] = in ? adv[i0 + j] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wd[j] = token<NE, true>(x[j], y[j], z[j], i0 + j < N, p, f, c, &wv4[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int j = 0; j < 4; ++j) {
      if (i0 + j < N) {
        if constexpr (WORD) word[i0 + j] = (uint16_t)wd[j];
        if constexpr (WPRIM) wprim[i0 + j] = wv4[j];
      }
    }
  }

  // Block reduction in a fixed order, into the block's row of raw totals:
  // the NF float sums, then the NC counts, then the token count.  Float sums:
  // a fixed fp32 butterfly over the wave's lanes, then the 4 wave totals
  // added in wave order in fp64.  Counts: wave totals (already scalar), added exactly.
  constexpr int NR = S::NF + S::NC + 1;
  static_assert(NR == 3 * NE + 13 && NR <= NS, "raw totals must fit the workspace rows");
  __shared__ double wtot[4][NR];
  const int w = wv;
  wave_totals<S::NF>(f, wtot[w], lane);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < S::NC; ++k) wtot[w][S::NF + k] = (double)c[k];
    wtot[w][NR - 1] = (double)ntok;
  }
  __syncthreads();
  if (threadIdx.x < NR) {
    const int k = threadIdx.x;
    partials[(int64_t)k * gridDim.x + blockIdx.x] =
        ((wtot[0][k] + wtot[1][k]) + wtot[2][k]) + wtot[3][k];
  }
}

// Which raw totals make up output sum k: v = t * tokens + ca * raw[a] + cb *
// raw[b], the coefficients 0 or +-1 (a, b index the raw rows; an output
// with no term reads the token row with coefficient 0).
struct OutMap {
  int a, b;
  double ct, ca, cb;
};

__device__ OutMap out_map(int k, int NE) {
  const int NF = 2 * NE + 7, NC = NE + 5, TOK = NF + NC;
  const int ICE = 2 * NE, REINF = 2 * NE + 2, PPO_J = 2 * NE + 3, PPO_D = 2 * NE + 4,
            TIS_WA = 2 * NE + 5, TIS_W = 2 * NE + 6;
  const int C_LOW = NF + NE, C_HIGH = NF + NE + 1, C_CLIP = NF + NE + 2, C_DUAL = NF + NE + 3,
            C_TRUNC = NF + NE + 4;
  if (k < 3 * RL_ELEM_MAX_EPS) {
    const int i = k / 3, m = k % 3;
    if (i >= NE) return {TOK, 0, 0.0, 0.0, 0.0};
    if (m == 0) return {NF + i, 0, 1.0, -1.0, 0.0};  // tokens - masked
    return {2 * i + (m - 1), 0, 0.0, 1.0, 0.0};
  }
  switch (k) {
    case RL_ELEM_ICEPOP_KEPT: return {C_LOW, C_HIGH, 1.0, -1.0, -1.0};
    case RL_ELEM_ICEPOP_LOW: return {C_LOW, 0, 0.0, 1.0, 0.0};
    case RL_ELEM_ICEPOP_HIGH: return {C_HIGH, 0, 0.0, 1.0, 0.0};
    case RL_ELEM_ICEPOP_LOSS: return {ICE, 0, 0.0, 1.0, 0.0};
    case RL_ELEM_ICEPOP_WEIGHT: return {ICE + 1, 0, 0.0, 1.0, 0.0};
    case RL_ELEM_REINFORCE_LOSS: return {REINF, 0, 0.0, 1.0, 0.0};
    case RL_ELEM_PPO_LOSS: return {PPO_J, 0, 0.0, -1.0, 0.0};
    case RL_ELEM_PPO_CLIP: return {C_CLIP, 0, 0.0, 1.0, 0.0};
    case RL_ELEM_PPO_CLIP_LOWER: return {C_DUAL, 0, 0.0, 1.0, 0.0};
    case RL_ELEM_PPO_KL: return {PPO_D, 0, 0.0, -1.0, 0.0};
    case RL_ELEM_TIS_LOSS: return {TIS_WA, 0, 0.0, -1.0, 0.0};
    case RL_ELEM_TIS_TRUNC: return {C_TRUNC, 0, 0.0, 1.0, 0.0};
    case RL_ELEM_TIS_WEIGHT: return {TIS_W, 0, 0.0, 1.0, 0.0};
    default: return {TOK, 0, 0.0, 0.0, 0.0};
  }
}

// One block per output sum.  Thread t adds, for each raw row the output
// uses, that row's values of blocks t, t + NT, ... in that order (all loads
// of a round issued together); wave 0 then adds the four waves' values per
// lane and a fixed xor-shuffle tree over its lanes.  Rows with a zero coefficient are not read, so a non-finite float sum
// never reaches a count.  An output combines at most one float sum (with
// coefficient +-1) with exact integer counts, so summing each row on its own
// gives the same value as summing the per-block combinations.
__global__ void __launch_bounds__(NT) elem_final_kernel(const double* __restrict__ partials,
                                                        int64_t nb, int NE,
                                                        double* __restrict__ sums) {
  __shared__ double part[NT];
  const OutMap m = out_map((int)blockIdx.x, NE);
  const int TOK = 3 * NE + 12;
  const double* row[3] = {partials + (int64_t)m.a * nb, partials + (int64_t)TOK * nb,
                          partials + (int64_t)m.b * nb};
  const double co[3] = {m.ca, m.ct, m.cb};
  double acc = 0.0;
  for (int64_t base = threadIdx.x; base < nb; base += 4 * NT) {
    double x[3][4];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t b = base + (int64_t)j * NT;
        x[r][j] = (co[r] != 0.0 && b < nb) ? row[r][b] : 0.0;
      }
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += co[r] * x[r][j];
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    double v = ((part[l] + part[l + 64]) + part[l + 128]) + part[l + 192];
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d);
    if (l == 0) sums[blockIdx.x] = v;
  }
}

template <int NE>
void launch_main(int64_t nb, const float* lp, const float* lq, const float* adv, int64_t N,
                 const ElemP& p, uint16_t* word, float* wprim, double* partials, hipStream_t s) {
  const dim3 g((unsigned)nb), b(NT);
  if (word && wprim)
    hipLaunchKernelGGL((elem_main_kernel<NE, true, true>), g, b, 0, s, lp, lq, adv, N, p, word,
                       wprim, partials);
  else if (word)
    hipLaunchKernelGGL((elem_main_kernel<NE, true, false>), g, b, 0, s, lp, lq, adv, N, p, word,
                       wprim, partials);
  else if (wprim)
    hipLaunchKernelGGL((elem_main_kernel<NE, false, true>), g, b, 0, s, lp, lq, adv, N, p, word,
                       wprim, partials);
  else
    hipLaunchKernelGGL((elem_main_kernel<NE, false, false>), g, b, 0, s, lp, lq, adv, N, p, word,
                       wprim, partials);
}

// Scratch of rl_loss_elementwise_noalloc: the per-block raw totals of the
// largest grid, in the library's own device memory (one copy per GPU, held
// until the process ends).  Every block writes its whole row before the final
// pass reads it, so nothing in it has to start at zero.  Host code reaches it
// only through the address hipGetSymbolAddress returns for the current
// device.
static __device__ __align__(256) double scratch[(int64_t)NS * kMaxBlocks];

}  // namespace

int64_t elem_noalloc_scratch_bytes() { return (int64_t)sizeof(scratch); }

hipError_t elem_noalloc_scratch(double** out) {
  static std::mutex mu;
  static double* ptrs[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (ptrs[dev] == nullptr) {  // set-up, once per device
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = static_cast<double*>(p);
  }
  *out = ptrs[dev];
  return hipSuccess;
}

int64_t elem_num_blocks(int64_t N) {
  const int64_t nch = (std::max<int64_t>(N, 1) + 255) / 256;  // 64-vector chunks
  return std::min<int64_t>(ceil_div(nch, (int64_t)4), kMaxBlocks);
}

hipError_t elementwise(const float* lp, const float* lq, const float* adv, int64_t N,
                       const rl_elem_cfg& c, uint16_t* word, float* w_primary, double* partials,
                       double* /*sums*/, hipStream_t s) {
  ElemP p;
  for (int i = 0; i < RL_ELEM_MAX_EPS; ++i) p.eps[i] = i < c.n_eps ? c.eps[i] : 0.0f;
  p.eps_primary = c.eps[c.primary_eps_index];
  p.M = c.max_ratio;
  p.lo = c.icepop_lo;
  p.hi = c.icepop_hi;
  p.clo = 1.0f - c.clip_low;
  p.chi = 1.0f + c.clip_high;
  p.c = c.clip_c;
  p.U = c.tis_upper;
  const int64_t nb = elem_num_blocks(N);
  switch (c.n_eps) {
    case 1: launch_main<1>(nb, lp, lq, adv, N, p, word, w_primary, partials, s); break;
    case 2: launch_main<2>(nb, lp, lq, adv, N, p, word, w_primary, partials, s); break;
    case 3: launch_main<3>(nb, lp, lq, adv, N, p, word, w_primary, partials, s); break;
    case 4: launch_main<4>(nb, lp, lq, adv, N, p, word, w_primary, partials, s); break;
    case 5: launch_main<5>(nb, lp, lq, adv, N, p, word, w_primary, partials, s); break;
    case 6: launch_main<6>(nb, lp, lq, adv, N, p, word, w_primary, partials, s); break;
    case 7: launch_main<7>(nb, lp, lq, adv, N, p, word, w_primary, partials, s); break;
    case 8: launch_main<8>(nb, lp, lq, adv, N, p, word, w_primary, partials, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t elementwise_final(const double* partials, int64_t N, int n_eps, double* sums,
                            hipStream_t s) {
  hipLaunchKernelGGL(elem_final_kernel, dim3(NS), dim3(NT), 0, s, partials, elem_num_blocks(N), n_eps,
                     sums);
  return hipGetLastError();
}

}  // namespace rl
