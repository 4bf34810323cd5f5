// Machine calibration: what the matrix pipe and HBM deliver on this device,
// measured with kernels that do nothing else.  Not part of the loss path; the
// benchmark reports these figures beside the published peaks.
//
// MFMA: every wave runs CAL_CHAINS independent v_mfma_f32_16x16x32_bf16
// chains from registers only (no memory traffic inside the loop), two waves
// per SIMD as in the GEMMs.  The operands are either all zero or uniform
// random bf16 values, with each MFMA of the unrolled body taking a different
// (A, B) fragment pair, so that operand toggling is close to a real GEMM's.
// Block b's first thread records the shader-clock counter and the fixed-rate
// wall clock before the loop and after the block's last wave has finished
// it; the ratio of the two deltas is the clock the loop ran at.
//
// Copy: a grid-stride copy of 16-byte vectors, four in flight per thread;
// with dst == src it writes every vector back where it was read (an in-place
// read-modify-write stream).
#include <hip/hip_runtime.h>

#include "common.h"

namespace rl {
namespace {

constexpr int CAL_NT = 256;
constexpr int CAL_CHAINS = 16;
constexpr int CAL_FRAGS = 4;  // A and B fragments each: 16 distinct pairs
constexpr int64_t CAL_FLOP_PER_MFMA = 2 * 16 * 16 * 32;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  // integer hash (xor-shift-multiply finaliser); any fixed bijection will do
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ void __launch_bounds__(CAL_NT) calib_mfma_kernel(int random, int64_t iters,
                                                            float* __restrict__ sink,
                                                            int64_t* __restrict__ stamps) {
  bf16x8 a[CAL_FRAGS], b[CAL_FRAGS];
  const uint32_t gid = blockIdx.x * CAL_NT + threadIdx.x;
#pragma unroll
  for (int f = 0; f < CAL_FRAGS; ++f)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t ua = mix32(gid * 64u + f * 16u + k);
      const uint32_t ub = mix32(gid * 64u + f * 16u + 8u + k);
      // uniform on [-2, 2) with 16 random bits, rounded to bf16
      a[f][k] = (__bf16)(random ? ((float)(ua & 0xffffu) - 32768.0f) * (1.0f / 16384.0f) : 0.0f);
      b[f][k] = (__bf16)(random ? ((float)(ub & 0xffffu) - 32768.0f) * (1.0f / 16384.0f) : 0.0f);
    }
  f32x4 acc[CAL_CHAINS];
#pragma unroll
  for (int c = 0; c < CAL_CHAINS; ++c) {
    // distinct starting values: identical ones let the compiler share
    // registers between chains and then copy them around inside the loop
    const float z = (float)(c * CAL_NT + (int)threadIdx.x) * 0x1p-20f;
    acc[c] = f32x4{z, z, z, z};
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    stamps[4 * blockIdx.x + 0] = clock64();
    stamps[4 * blockIdx.x + 2] = wall_clock64();
  }
  // The MFMAs are written as inline asm with the accumulator tied to the
  // result ("+a"): left to itself the compiler gives half the chains the
  // untied form and copies their accumulators around inside the loop.  The
  // compiler does not track hazards through inline asm, so the operands are
  // fenced: written to their registers, then 24 wait states, before the loop
  // (VALU write to MFMA source), and 24 wait states before the accumulators
  // are read after it
  // (MFMA result to VALU read: at most 19 for these 8-pass MFMAs).  Inside
  // the loop a chain's next MFMA comes 16 MFMAs after its previous one.
#pragma unroll
  for (int f = 0; f < CAL_FRAGS; ++f) __asm__ volatile("" : "+v"(a[f]), "+v"(b[f]));
#pragma unroll
  for (int c = 0; c < CAL_CHAINS; ++c) __asm__ volatile("" : "+a"(acc[c]));
  __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CAL_CHAINS; ++c)
      __asm__ volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                       : "+a"(acc[c])
                       : "v"(a[c % CAL_FRAGS]), "v"(b[c / CAL_FRAGS]));
  }
  __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
  for (int c = 0; c < CAL_CHAINS; ++c) __asm__ volatile("" : "+a"(acc[c]));
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < CAL_CHAINS; ++c) s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
  sink[gid] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    stamps[4 * blockIdx.x + 1] = clock64();
    stamps[4 * blockIdx.x + 3] = wall_clock64();
  }
}

__global__ void __launch_bounds__(CAL_NT) calib_copy_kernel(const u32x4* src, u32x4* dst,
                                                            int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * CAL_NT * 4;
  for (int64_t base = (int64_t)blockIdx.x * CAL_NT * 4 + threadIdx.x; base < n; base += stride) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = base + (int64_t)j * CAL_NT;
      if (i < n) v[j] = src[i];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = base + (int64_t)j * CAL_NT;
      if (i < n) dst[i] = v[j];
    }
  }
}

}  // namespace
}  // namespace rl

extern "C" {

rl_status rl_calib_mfma_bf16(int32_t random_operands, int32_t n_blocks, int64_t iters,
                             float* sink_dev, int64_t* stamps_dev, double* flop,
                             int32_t* wall_clock_khz, void* stream) {
  // n_blocks * iters is bounded so that one launch stays within seconds (about
  // 9 s at the full matrix rate of 512 blocks).
  if (sink_dev == nullptr || stamps_dev == nullptr || flop == nullptr ||
      wall_clock_khz == nullptr || n_blocks < 1 || n_blocks > (1 << 20) || iters < 1 ||
      iters > ((int64_t)1 << 32) || (int64_t)n_blocks * iters > ((int64_t)1 << 34))
    return RL_E_ARG;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return RL_E_HIP;
  *wall_clock_khz = khz;
  *flop = (double)n_blocks * (rl::CAL_NT / RL_WAVE) * (double)iters * rl::CAL_CHAINS *
          (double)rl::CAL_FLOP_PER_MFMA;
  hipLaunchKernelGGL(rl::calib_mfma_kernel, dim3((unsigned)n_blocks), dim3(rl::CAL_NT), 0,
                     static_cast<hipStream_t>(stream), random_operands != 0 ? 1 : 0, iters,
                     sink_dev, stamps_dev);
  return hipGetLastError() == hipSuccess ? RL_OK : RL_E_HIP;
}

rl_status rl_calib_copy(const void* src, void* dst, int64_t bytes, int32_t n_blocks,
                        void* stream) {
  if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16 != 0 || n_blocks < 1 ||
      n_blocks > (1 << 20) || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return RL_E_ARG;
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (s != d && s < d + bytes && d < s + bytes) return RL_E_ARG;  // partial overlap
  hipLaunchKernelGGL(rl::calib_copy_kernel, dim3((unsigned)n_blocks), dim3(rl::CAL_NT), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? RL_OK : RL_E_HIP;
}

}  // extern "C"
