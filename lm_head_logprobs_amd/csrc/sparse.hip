// Sparse part of the LM-head backward.
//
// The label and support terms of dL/dz touch one vocabulary row each
// (prime-rl PR 4233, "What changes": when every token's logit gradient lies on
// its label and support the head uses a deterministic CSR matmul instead of
// the dense softmax backward).  For dh they are gathered per token
// (finalize_dh).  For dW each vocabulary row v needs the sum over the entries
// that hit v of coef * h[token]; the entries are bucketed by v with a stable
// LSD radix sort (8-bit digits), so every bucket lists its entries in entry
// order and each dW row is summed in that fixed order.  Integer atomics are
// used only for counting; no floating-point value depends on thread timing.
#include "kernels.h"

namespace rl {
namespace {

constexpr int RS_NT = 256;
constexpr int RS_ITEMS = 4;  // per thread
constexpr int RS_BLOCK = RS_NT * RS_ITEMS;

// Keys are vocabulary ids; an id outside [0, V) goes to the extra bucket V,
// which no dW row reads (such inputs are reported by the validation call).
__global__ void csc_init_kernel(const int32_t* __restrict__ labels,
                                const int32_t* __restrict__ ids, int64_t N, int64_t E, int64_t V,
                                int32_t* __restrict__ keys, int32_t* __restrict__ idx) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= E) return;
  const int32_t k = i < N ? labels[i] : ids[i - N];
  keys[i] = (k < 0 || k >= V) ? (int32_t)V : k;
  idx[i] = (int32_t)i;
}

// Positions handled by (block, wave, sub-chunk c, lane), in entry order.
__device__ __forceinline__ int64_t rs_pos(int64_t blk, int wave, int c, int lane) {
  return blk * RS_BLOCK + wave * (RS_BLOCK / 4) + c * 64 + lane;
}

__global__ void __launch_bounds__(RS_NT) rs_hist_kernel(const int32_t* __restrict__ keys,
                                                        int64_t E, int shift,
                                                        int32_t* __restrict__ hist, int64_t nb) {
  __shared__ int32_t cnt[256];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < RS_ITEMS; ++c) {
    const int64_t p = rs_pos(blockIdx.x, wave, c, lane);
    if (p < E) atomicAdd(&cnt[(keys[p] >> shift) & 255], 1);
  }
  __syncthreads();
  hist[(int64_t)threadIdx.x * nb + blockIdx.x] = cnt[threadIdx.x];
}

// Exclusive scan of n ints in place, in three launches: tiles of SC_TILE ints
// (SC_ITEMS contiguous per thread) are summed in parallel, the tile sums are
// scanned by one workgroup, then every tile is scanned again from its offset.
constexpr int SC_NT = 256, SC_ITEMS = 16, SC_TILE = SC_NT * SC_ITEMS;

// Inclusive prefix of v over the workgroup's threads (in thread order); the
// total goes to *total.
__device__ __forceinline__ int32_t block_inclusive_scan(int32_t v, int32_t* sh, int32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t x = __shfl_up(v, o, 64);
    if (lane >= o) v += x;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  int32_t before = 0, all = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
    before += i < w ? sh[i] : 0;
    all += sh[i];
  }
  __syncthreads();
  *total = all;
  return v + before;
}

__global__ void __launch_bounds__(SC_NT) scan_tile_sums_kernel(const int32_t* __restrict__ a,
                                                               int64_t n,
                                                               int32_t* __restrict__ tsum) {
  __shared__ int32_t sh[SC_NT / 64];
  const int64_t b = (int64_t)blockIdx.x * SC_TILE + (int64_t)threadIdx.x * SC_ITEMS;
  int32_t v = 0;
#pragma unroll
  for (int j = 0; j < SC_ITEMS; ++j) v += b + j < n ? a[b + j] : 0;
  int32_t total;
  block_inclusive_scan(v, sh, &total);
  if (threadIdx.x == 0) tsum[blockIdx.x] = total;
}

// One workgroup: exclusive scan of the nt tile sums, 1024 at a time.
__global__ void __launch_bounds__(1024) scan_tsum_kernel(int32_t* __restrict__ tsum, int64_t nt) {
  __shared__ int32_t sh[16];
  int32_t carry = 0;
  for (int64_t base = 0; base < nt; base += 1024) {
    const int64_t i = base + threadIdx.x;
    const int32_t v = i < nt ? tsum[i] : 0;
    int32_t total;
    const int32_t inc = block_inclusive_scan(v, sh, &total);
    if (i < nt) tsum[i] = carry + inc - v;
    carry += total;
  }
}

__global__ void __launch_bounds__(SC_NT) scan_apply_kernel(int32_t* __restrict__ a, int64_t n,
                                                           const int32_t* __restrict__ tsum) {
  __shared__ int32_t sh[SC_NT / 64];
  const int64_t b = (int64_t)blockIdx.x * SC_TILE + (int64_t)threadIdx.x * SC_ITEMS;
  int32_t x[SC_ITEMS];
  int32_t v = 0;
#pragma unroll
  for (int j = 0; j < SC_ITEMS; ++j) {
    x[j] = b + j < n ? a[b + j] : 0;
    v += x[j];
  }
  int32_t total;
  int32_t run = block_inclusive_scan(v, sh, &total) - v + tsum[blockIdx.x];
#pragma unroll
  for (int j = 0; j < SC_ITEMS; ++j) {
    if (b + j < n) a[b + j] = run;
    run += x[j];
  }
}

int64_t scan_tiles(int64_t n) { return std::max<int64_t>(ceil_div(n, SC_TILE), 1); }

hipError_t exclusive_scan(int32_t* a, int64_t n, int32_t* tsum, hipStream_t s) {
  const int64_t nt = scan_tiles(n);
  hipLaunchKernelGGL(scan_tile_sums_kernel, dim3((unsigned)nt), dim3(SC_NT), 0, s, a, n, tsum);
  hipLaunchKernelGGL(scan_tsum_kernel, dim3(1), dim3(1024), 0, s, tsum, nt);
  hipLaunchKernelGGL(scan_apply_kernel, dim3((unsigned)nt), dim3(SC_NT), 0, s, a, n, tsum);
  return hipGetLastError();
}

__global__ void __launch_bounds__(RS_NT) rs_scatter_kernel(
    const int32_t* __restrict__ keys_in, const int32_t* __restrict__ idx_in, int64_t E,
    int shift, const int32_t* __restrict__ offs, int64_t nb, int32_t* __restrict__ keys_out,
    int32_t* __restrict__ idx_out) {
  __shared__ int32_t wcnt[4][256];
  __shared__ int32_t wbase[4][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int d = threadIdx.x; d < 4 * 256; d += RS_NT) (&wcnt[0][0])[d] = 0;
  __syncthreads();
  int32_t key[RS_ITEMS], dig[RS_ITEMS], ix[RS_ITEMS];
  bool ok[RS_ITEMS];
#pragma unroll
  for (int c = 0; c < RS_ITEMS; ++c) {
    const int64_t p = rs_pos(blockIdx.x, wave, c, lane);
    ok[c] = p < E;
    key[c] = ok[c] ? keys_in[p] : 0;
    ix[c] = ok[c] ? idx_in[p] : 0;
    dig[c] = (key[c] >> shift) & 255;
    if (ok[c]) atomicAdd(&wcnt[wave][dig[c]], 1);
  }
  __syncthreads();
  {
    const int d = threadIdx.x;
    int32_t run = offs[(int64_t)d * nb + blockIdx.x];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wbase[w][d] = run;
      run += wcnt[w][d];
    }
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int c = 0; c < RS_ITEMS; ++c) {
    uint64_t peers = __ballot(ok[c]);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (dig[c] >> b) & 1;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const int rank = __popcll(peers & lt_mask);
    volatile int32_t* wb = &wbase[wave][0];
    if (ok[c]) {
      const int32_t dst = wb[dig[c]] + rank;
      keys_out[dst] = key[c];
      idx_out[dst] = ix[c];
    }
    __builtin_amdgcn_wave_barrier();
    if (ok[c] && (__ffsll((long long)peers) - 1) == lane) wb[dig[c]] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

// start[v] = first sorted position with key >= v, for v in [0, V + 1]
// (keys lie in [0, V]; bucket V holds out-of-range ids).
__global__ void csc_bounds_kernel(const int32_t* __restrict__ keys, int64_t E, int64_t V,
                                  int32_t* __restrict__ start) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p > E) return;
  const int64_t kp = (p == 0) ? -1 : keys[p - 1];
  const int64_t kc = (p == E) ? V + 1 : keys[p];
  for (int64_t v = kp + 1; v <= kc; ++v) start[v] = (int32_t)p;
}

template <typename T>
__global__ void __launch_bounds__(256) sparse_dw_kernel(
    const T* __restrict__ h, int64_t H, int64_t N, int64_t V, const int32_t* __restrict__ start,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ row_of,
    const float* __restrict__ coef, float* __restrict__ dW, int overwrite) {
  constexpr int VEC = 8;
  for (int64_t v = blockIdx.x; v < V; v += gridDim.x) {
    const int32_t s = start[v], e = start[v + 1];
    if (s == e && !overwrite) continue;
    for (int64_t c = (int64_t)threadIdx.x * VEC; c < H; c += 256 * VEC) {
      float acc[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
      // the bucket's entries in order, in groups of 8 whose loads are issued
      // together; an entry outside every row (corrupted offsets) reads row 0
      // with coefficient 0
      constexpr int EV = Elem<T>::VEC, NV = VEC / EV;  // 16-byte loads per row piece
      for (int32_t pb = s; pb < e; pb += 8) {
        float cf[8];
        const T* hr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int32_t p = pb + j;
          const int32_t i = p < e ? perm[p] : 0;
          const int64_t tok = p < e ? (i < N ? (int64_t)i : (int64_t)row_of[i - N]) : -1;
          const bool ok = tok >= 0 && tok < N;
          cf[j] = ok ? coef[i] : 0.0f;
          hr[j] = h + (ok ? tok : 0) * H + c;
        }
        u32x4 raw[8][NV];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int q = 0; q < NV; ++q)
            raw[j][q] = *reinterpret_cast<const u32x4*>(hr[j] + q * EV);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float x[VEC];
#pragma unroll
          for (int q = 0; q < NV; ++q) Elem<T>::unpack(raw[j][q], x + q * EV);
#pragma unroll
          for (int k = 0; k < VEC; ++k) acc[k] = fmaf(cf[j], x[k], acc[k]);
        }
      }
      float* o = dW + v * H + c;
#pragma unroll
      for (int k = 0; k < VEC; ++k) o[k] = overwrite ? acc[k] : o[k] + acc[k];
    }
  }
}

}  // namespace

// The digit histogram (256 per sort block) followed by the scan's tile sums.
int64_t csc_hist_len(int64_t E) {
  const int64_t n = 256 * std::max<int64_t>(ceil_div(E, RS_BLOCK), 1);
  return n + scan_tiles(n);
}

hipError_t csc_build(const int32_t* labels, const int32_t* ids, int64_t N, int64_t nnz,
                     int64_t V, const CscWork& w, const int32_t** perm_out,
                     const int32_t** keys_out, hipStream_t s) {
  const int64_t E = N + nnz;
  const int64_t nb = std::max<int64_t>(ceil_div(E, RS_BLOCK), 1);
  int bits = 1;
  while (bits < 31 && ((int64_t)1 << bits) < V + 1) ++bits;
  const int passes = (bits + 7) / 8;
  hipLaunchKernelGGL(csc_init_kernel, dim3((unsigned)ceil_div(E, 256)), dim3(256), 0, s, labels,
                     ids, N, E, V, w.keys_a, w.idx_a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int32_t *ki = w.keys_a, *ii = w.idx_a, *ko = w.keys_b, *io = w.idx_b;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = 8 * pass;
    hipLaunchKernelGGL(rs_hist_kernel, dim3((unsigned)nb), dim3(RS_NT), 0, s, ki, E, shift,
                       w.hist, nb);
    err = exclusive_scan(w.hist, 256 * nb, w.hist + 256 * nb, s);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(rs_scatter_kernel, dim3((unsigned)nb), dim3(RS_NT), 0, s, ki, ii, E, shift,
                       w.hist, nb, ko, io);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    int32_t* tk = ki;
    ki = ko;
    ko = tk;
    int32_t* ti = ii;
    ii = io;
    io = ti;
  }
  hipLaunchKernelGGL(csc_bounds_kernel, dim3((unsigned)ceil_div(E + 1, 256)), dim3(256), 0, s,
                     ki, E, V, w.start);
  *perm_out = ii;
  if (keys_out != nullptr) *keys_out = ki;
  return hipGetLastError();
}

hipError_t sparse_dw(int dtype, const void* h, int64_t H, int64_t N, int64_t V,
                     const int32_t* start, const int32_t* perm, const int32_t* row_of,
                     const float* coef, float* dW, int overwrite, hipStream_t s) {
  const unsigned grid = (unsigned)std::min<int64_t>(V, 8192);
  if (dtype == RL_DTYPE_BF16)
    hipLaunchKernelGGL(sparse_dw_kernel<bf16_t>, dim3(grid), dim3(256), 0, s,
                       static_cast<const bf16_t*>(h), H, N, V, start, perm, row_of, coef, dW,
                       overwrite);
  else
    hipLaunchKernelGGL(sparse_dw_kernel<float>, dim3(grid), dim3(256), 0, s,
                       static_cast<const float*>(h), H, N, V, start, perm, row_of, coef, dW,
                       overwrite);
  return hipGetLastError();
}

}  // namespace rl
