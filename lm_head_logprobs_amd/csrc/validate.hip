// Sampler-evidence validation of the per-token CSR support (prime-rl PR 4233,
// "What changes": the checks run on the GPU on the CSR entries once per step
// before the optimizer; the TokenSupport bullet fixes the layout).  Each
// thread ORs the flags it finds into one int32 word (integer atomics only).
#include "kernels.h"

namespace rl {
namespace {

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

__device__ __forceinline__ bool finite_nonpos(float x) { return isfinite(x) && x <= 0.0f; }

// One wave per token: lane 0 checks the token's own inputs; the lanes stride
// over the token's CSR row for the replay checks (row mass in fp64, summed
// per lane then across the wave in a fixed order; label present).
__global__ void validate_tokens_kernel(int64_t N, int64_t V, int64_t nnz,
                                       const int32_t* __restrict__ labels,
                                       const float* __restrict__ infer_lp,
                                       const float* __restrict__ adv,
                                       const int64_t* __restrict__ off,
                                       const int32_t* __restrict__ ids,
                                       const float* __restrict__ u, int replayed,
                                       int32_t* __restrict__ flags) {
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= N) return;
  int32_t f = 0;
  const int32_t lab = labels[t];
  if (lane == 0) {
    if (lab < 0 || lab >= V) f |= RL_BAD_LABEL;
    if (!finite_nonpos(infer_lp[t])) f |= RL_BAD_INFER_LOGPROB;
    if (!isfinite(adv[t])) f |= RL_BAD_ADV;
  }
  if (off != nullptr) {
    const int64_t e0 = off[t], e1 = off[t + 1];
    bool row_ok = e0 >= 0 && e1 >= e0 && e1 <= nnz;
    if (t == 0 && e0 != 0) row_ok = false;
    if (t == N - 1 && e1 != nnz) row_ok = false;
    if (!row_ok) {
      if (lane == 0) f |= RL_BAD_OFFSETS;
    } else if (replayed) {
      double mass = 0.0;
      bool has_label = false;
      for (int64_t e = e0 + lane; e < e1; e += 64) {
        mass += (double)u[e];
        has_label |= (ids[e] == lab);
      }
      mass = wave_sum_d(mass);
      has_label = __any(has_label);
      if (lane == 0) {
        if (!(fabs(mass - 1.0) <= 1e-3)) f |= RL_BAD_REPLAY_MASS;
        if (!has_label) f |= RL_BAD_REPLAY_LABEL;
      }
    }
  }
  if (f) atomicOr(flags, f);
}

__global__ void validate_entries_kernel(int64_t nnz, int64_t V, const int32_t* __restrict__ ids,
                                        const float* __restrict__ u,
                                        const float* __restrict__ logq,
                                        int32_t* __restrict__ flags) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= nnz) return;
  int32_t f = 0;
  const int32_t v = ids[e];
  if (v < 0 || v >= V) f |= RL_BAD_ID;
  const float ue = u[e];
  if (!(isfinite(ue) && ue >= 0.0f)) f |= RL_BAD_U;
  if (logq != nullptr && !finite_nonpos(logq[e])) f |= RL_BAD_LOGQ;
  if (f) atomicOr(flags, f);
}

}  // namespace

hipError_t validate(int64_t N, int64_t V, int64_t nnz, const int32_t* labels,
                    const float* infer_lp, const float* adv, const int64_t* off,
                    const int32_t* ids, const float* u, const float* logq, int replayed,
                    int32_t* flags, hipStream_t s) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, s, flags);
  hipLaunchKernelGGL(validate_tokens_kernel, dim3((unsigned)ceil_div(N, 4)), dim3(256), 0, s, N,
                     V, nnz, labels, infer_lp, adv, off, ids, u, replayed, flags);
  if (off != nullptr && nnz > 0)
    hipLaunchKernelGGL(validate_entries_kernel, dim3((unsigned)ceil_div(nnz, 256)), dim3(256), 0,
                       s, nnz, V, ids, u, logq, flags);
  return hipGetLastError();
}

}  // namespace rl
