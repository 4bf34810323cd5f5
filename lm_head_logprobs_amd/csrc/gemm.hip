// Matrix-core GEMM C = A B^T for the LM head (gfx950 MFMA).
//
// Both operands are K-contiguous ("NT"): A [M,K] and B [N,K] row-major.  The
// three contractions of the head all take this form once the backward
// operands are laid out K-contiguous:
//   forward   S^T[V,Tc]  = W[V,H]     . h_c[Tc,H]^T        (K = H)
//   dh        dh[Tc,H]   = G[Tc,V]    . (W^T)[H,V]^T       (K = V, split-K)
//   dW        dW[V,H]    = G^T[V,Tc]  . (h_c^T)[H,Tc]^T    (K = Tc)
// bf16 inputs use v_mfma_f32_32x32x16_bf16, fp32 inputs v_mfma_f32_32x32x2_f32;
// both accumulate in fp32 and share the 32x32 accumulator layout
//   lane l, register r  ->  row 8*(r/4) + 4*(l/32) + r%4,  column l%32.
//
// Tiling: a 256-thread workgroup (4 waves as 2x2) owns a BM x BN tile; each
// wave owns (BM/2) x (BN/2) as 32x32 MFMA blocks.  K advances BK at a time
// through two LDS buffers: the next tile's global loads are issued before the
// MFMAs on the current one, then written to the other buffer.  Rows of LDS are
// padded by 16 bytes.  Workgroups are remapped so that consecutive tiles land
// on one XCD (dispatch is round-robin over the 8 XCDs) and grouped 8 tiles
// along M so neighbours share B panels in that XCD's L2.
#include "kernels.h"

namespace rl {
namespace {

template <typename T> struct MM;
template <> struct MM<bf16_t> {
  static constexpr int KSTEP = 16;
  typedef bf16x8 frag_t;
  __device__ __forceinline__ static f32x16 mma(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Rows r0..r0+31, K slice k0..k0+15: lane l takes 8 consecutive K values of
  // row r0 + l%32 starting at k0 + 8*(l/32).  Both operands use the same K map.
  __device__ __forceinline__ static frag_t load(const bf16_t* s, int ld, int r0, int k0,
                                                int lane) {
    return *reinterpret_cast<const frag_t*>(s + (r0 + (lane & 31)) * ld + k0 + 8 * (lane >> 5));
  }
};
template <> struct MM<float> {
  static constexpr int KSTEP = 2;
  typedef float frag_t;
  __device__ __forceinline__ static f32x16 mma(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag_t load(const float* s, int ld, int r0, int k0,
                                                int lane) {
    return s[(r0 + (lane & 31)) * ld + k0 + (lane >> 5)];
  }
};

template <typename T> struct Tile;
template <> struct Tile<bf16_t> { static constexpr int BM = 128, BN = 128, BK = 64; };
template <> struct Tile<float> { static constexpr int BM = 128, BN = 128, BK = 32; };

constexpr int NT = 256;
constexpr int GROUP_M = 8;

struct TileCoord {
  int64_t m0, n0;
  int split;
  bool valid;
};

__device__ __forceinline__ TileCoord map_tile(int tiles_m, int tiles_n, int splits, int BM,
                                              int BN) {
  TileCoord tc;
  const int nwg = gridDim.x;  // a multiple of 8
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int per_split = tiles_m * tiles_n;
  tc.valid = logical < per_split * splits;
  if (!tc.valid) return tc;
  tc.split = logical / per_split;
  const int rem = logical - tc.split * per_split;
  const int group = rem / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsize = min(GROUP_M, tiles_m - first_m);
  const int within = rem - group * GROUP_M * tiles_n;
  const int tm = first_m + within % gsize;
  const int tn = within / gsize;
  tc.m0 = (int64_t)tm * BM;
  tc.n0 = (int64_t)tn * BN;
  return tc;
}

// Epilogue context handed to the epilogue functors.
struct EpiCtx {
  int64_t m0, n0;
  int wm_off, wn_off;  // wave tile origin inside the block tile
  int wave_m;          // 0/1
  int lane;
  int split;
  float* red;  // LDS scratch, at least 2 * BN * 2 floats
};

template <typename T, class Epi>
__global__ void __launch_bounds__(NT) gemm_nt_kernel(const T* __restrict__ A, int64_t lda,
                                                     const T* __restrict__ B, int64_t ldb,
                                                     int64_t M, int64_t N, int64_t K,
                                                     int64_t k_split, int tiles_m, int tiles_n,
                                                     int splits, Epi epi) {
  constexpr int BM = Tile<T>::BM, BN = Tile<T>::BN, BK = Tile<T>::BK;
  constexpr int VEC = Elem<T>::VEC;
  constexpr int LD = BK + VEC;  // padded row, in elements
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int KV = BK / VEC;  // vectors per tile row
  constexpr int A_IT = BM * KV / NT, B_IT = BN * KV / NT;
  static_assert(A_IT * NT == BM * KV && B_IT * NT == BN * KV, "tile/threads mismatch");

  __shared__ __attribute__((aligned(16))) T As[2][BM * LD];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * LD];

  const TileCoord tc = map_tile(tiles_m, tiles_n, splits, BM, BN);
  if (!tc.valid) return;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t kb = (int64_t)tc.split * k_split;
  const int64_t ke = min(K, kb + k_split);
  const int nk = (int)ceil_div(max<int64_t>(ke - kb, 0), BK);

  u32x4 ra[A_IT], rb[B_IT];
  auto gload = [&](int kt) {
    const int64_t k0 = kb + (int64_t)kt * BK;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      const int q = tid + NT * i;
      const int row = q / KV, kv = (q % KV) * VEC;
      const int64_t gr = tc.m0 + row, gk = k0 + kv;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gr < M && gk < ke) v = *reinterpret_cast<const u32x4*>(A + gr * lda + gk);
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      const int q = tid + NT * i;
      const int row = q / KV, kv = (q % KV) * VEC;
      const int64_t gr = tc.n0 + row, gk = k0 + kv;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gr < N && gk < ke) v = *reinterpret_cast<const u32x4*>(B + gr * ldb + gk);
      rb[i] = v;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      const int q = tid + NT * i;
      const int row = q / KV, kv = (q % KV) * VEC;
      *reinterpret_cast<u32x4*>(&As[buf][row * LD + kv]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      const int q = tid + NT * i;
      const int row = q / KV, kv = (q % KV) * VEC;
      *reinterpret_cast<u32x4*>(&Bs[buf][row * LD + kv]) = rb[i];
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (nk > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += MM<T>::KSTEP) {
      typename MM<T>::frag_t a[MB], b[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i) a[i] = MM<T>::load(As[buf], LD, wm * WM + 32 * i, kk, lane);
#pragma unroll
      for (int j = 0; j < NB; ++j) b[j] = MM<T>::load(Bs[buf], LD, wn * WN + 32 * j, kk, lane);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = MM<T>::mma(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  EpiCtx ctx;
  ctx.m0 = tc.m0;
  ctx.n0 = tc.n0;
  ctx.wm_off = wm * WM;
  ctx.wn_off = wn * WN;
  ctx.wave_m = wm;
  ctx.lane = lane;
  ctx.split = tc.split;
  ctx.red = reinterpret_cast<float*>(&As[0][0]);
  epi.template apply<MB, NB, BN>(acc, ctx);
}

// Row/column of accumulator element (i, j, r) for this lane.
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Forward epilogue: rows are vocabulary entries, columns tokens.  Per column
// and block tile: m = max z, s = sum e^(z-m), t = sum e^(z-m) (z-m) over the
// tile's valid rows; optionally stores e^(z-m) to Pt[v, t].
template <typename T> struct FwdEpi {
  float inv_t;
  int64_t V, Tc, J;
  float *pm, *ps, *pt;
  T* Pt;
  int64_t ldp;

  template <int MB, int NB, int BN>
  __device__ __forceinline__ void apply(f32x16 (&acc)[MB][NB], const EpiCtx& c) const {
    const int64_t jt = c.m0 / FWD_VTILE;
    const int lc = c.lane & 31;
    float* red = c.red;  // [2][BN] maxima then [2][BN] s and [2][BN] t
    float mcol[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = c.m0 + c.wm_off + acc_row(i, r, c.lane);
          if (row < V) mx = fmaxf(mx, acc[i][j][r] * inv_t);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      mcol[j] = mx;
    }
    __syncthreads();  // the LDS main-loop buffers are free from here
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (c.lane < 32) red[c.wave_m * BN + c.wn_off + 32 * j + lc] = mcol[j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = c.wn_off + 32 * j + lc;
      mcol[j] = fmaxf(red[col], red[BN + col]);
    }
    float scol[NB], tcol[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t col = c.n0 + c.wn_off + 32 * j + lc;
      float s = 0.0f, t = 0.0f;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = c.m0 + c.wm_off + acc_row(i, r, c.lane);
          if (row < V) {
            const float d = acc[i][j][r] * inv_t - mcol[j];
            const float e = __expf(d);
            s += e;
            t += e * d;
            if (Pt != nullptr && col < Tc) Pt[row * ldp + col] = Elem<T>::from_f32(e);
          }
        }
      s += __shfl_xor(s, 32, 64);
      t += __shfl_xor(t, 32, 64);
      scol[j] = s;
      tcol[j] = t;
    }
    float* rs = red + 2 * BN;
    float* rt = red + 4 * BN;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (c.lane < 32) {
        rs[c.wave_m * BN + c.wn_off + 32 * j + lc] = scol[j];
        rt[c.wave_m * BN + c.wn_off + 32 * j + lc] = tcol[j];
      }
    __syncthreads();
    if (c.wave_m == 0 && c.lane < 32) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int colb = c.wn_off + 32 * j + lc;
        const int64_t col = c.n0 + colb;
        if (col < Tc) {
          pm[col * J + jt] = mcol[j];
          ps[col * J + jt] = rs[colb] + rs[BN + colb];
          pt[col * J + jt] = rt[colb] + rt[BN + colb];
        }
      }
    }
  }
};

// C[split][row][col] = acc  (fp32).
struct StoreEpi {
  float* C;
  int64_t ldc, split_stride, M, N;
  template <int MB, int NB, int BN>
  __device__ __forceinline__ void apply(f32x16 (&acc)[MB][NB], const EpiCtx& c) const {
    float* Cs = C + (int64_t)c.split * split_stride;
    const int lc = c.lane & 31;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int64_t col = c.n0 + c.wn_off + 32 * j + lc;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = c.m0 + c.wm_off + acc_row(i, r, c.lane);
          if (row < M) Cs[row * ldc + col] = acc[i][j][r];
        }
      }
  }
};

// dW[row][col] (=|+=) acc.
struct DwEpi {
  float* C;
  int64_t ldc, M, N;
  int accumulate;
  template <int MB, int NB, int BN>
  __device__ __forceinline__ void apply(f32x16 (&acc)[MB][NB], const EpiCtx& c) const {
    const int lc = c.lane & 31;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int64_t col = c.n0 + c.wn_off + 32 * j + lc;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = c.m0 + c.wm_off + acc_row(i, r, c.lane);
          if (row < M) {
            float* p = C + row * ldc + col;
            *p = accumulate ? (*p + acc[i][j][r]) : acc[i][j][r];
          }
        }
      }
  }
};

template <typename T, class Epi>
hipError_t launch(const T* A, int64_t lda, const T* B, int64_t ldb, int64_t M, int64_t N,
                  int64_t K, int splits, int64_t k_split, const Epi& epi, hipStream_t s) {
  constexpr int BM = Tile<T>::BM, BN = Tile<T>::BN;
  const int64_t tm = ceil_div(M, BM), tn = ceil_div(N, BN);
  const int64_t total = tm * tn * splits;
  if (total <= 0) return hipSuccess;
  if (total > (int64_t)1 << 30) return hipErrorInvalidValue;
  const int64_t grid = round_up(total, 8);
  hipLaunchKernelGGL((gemm_nt_kernel<T, Epi>), dim3((unsigned)grid), dim3(NT), 0, s, A, lda, B,
                     ldb, M, N, K, k_split, (int)tm, (int)tn, splits, epi);
  return hipGetLastError();
}

}  // namespace

int gemm_k_tile(int dtype) { return dtype == RL_DTYPE_BF16 ? Tile<bf16_t>::BK : Tile<float>::BK; }

hipError_t gemm_fwd(int dtype, const void* W, const void* hc, int64_t V, int64_t Tc, int64_t H,
                    const FwdEpiArgs& a, hipStream_t s) {
  static_assert(Tile<bf16_t>::BM == FWD_VTILE && Tile<float>::BM == FWD_VTILE, "vocab tile");
  if (dtype == RL_DTYPE_BF16) {
    FwdEpi<bf16_t> e{a.inv_t, a.V, a.Tc, a.J, a.part_m, a.part_s, a.part_t,
                     static_cast<bf16_t*>(a.Pt), a.ldp};
    return launch<bf16_t>(static_cast<const bf16_t*>(W), H, static_cast<const bf16_t*>(hc), H, V,
                          Tc, H, 1, round_up(H, Tile<bf16_t>::BK), e, s);
  }
  FwdEpi<float> e{a.inv_t, a.V, a.Tc, a.J, a.part_m, a.part_s, a.part_t,
                  static_cast<float*>(a.Pt), a.ldp};
  return launch<float>(static_cast<const float*>(W), H, static_cast<const float*>(hc), H, V, Tc,
                       H, 1, round_up(H, Tile<float>::BK), e, s);
}

hipError_t gemm_store(int dtype, const void* A, int64_t lda, const void* B, int64_t ldb,
                      int64_t M, int64_t N, int64_t K, int splits, int64_t k_split, float* C,
                      int64_t ldc, int64_t split_stride, hipStream_t s) {
  StoreEpi e{C, ldc, split_stride, M, N};
  if (dtype == RL_DTYPE_BF16)
    return launch<bf16_t>(static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(B), ldb,
                          M, N, K, splits, k_split, e, s);
  return launch<float>(static_cast<const float*>(A), lda, static_cast<const float*>(B), ldb, M, N,
                       K, splits, k_split, e, s);
}

hipError_t gemm_dw(int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M,
                   int64_t N, int64_t K, float* C, int64_t ldc, int accumulate, hipStream_t s) {
  DwEpi e{C, ldc, M, N, accumulate};
  const int bk = gemm_k_tile(dtype);
  if (dtype == RL_DTYPE_BF16)
    return launch<bf16_t>(static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(B), ldb,
                          M, N, K, 1, round_up(K, bk), e, s);
  return launch<float>(static_cast<const float*>(A), lda, static_cast<const float*>(B), ldb, M, N,
                       K, 1, round_up(K, bk), e, s);
}

}  // namespace rl
