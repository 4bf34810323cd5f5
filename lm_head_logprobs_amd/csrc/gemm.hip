// Matrix-core GEMM C = A B^T for the LM head (gfx950 MFMA).
//
// Both operands are K-contiguous ("NT"): A [M,K] and B [N,K] row-major.  The
// three contractions of the head all take this form once the backward
// operands are laid out K-contiguous:
//   forward   S^T[V,Tc]  = W[V,H]      . h_c[Tc,H]^T       (K = H)
//   dh        dh[Tc,H]   = G[Tc,V]     . (W^T)[H,V]^T      (K = V, split-K)
//   dW        dW[V,H]    = G^T[V,Tc]   . (h_c^T)[H,Tc]^T   (K = Tc; G^T read from
//                                                            G's layout, see ATR)
// Accumulation is fp32.  The epilogues are written against an accumulator
// layout (Acc16 / Acc32 below) that maps lane and register to row and column.
//
// bf16 kernel (the hot path).  A 512-thread workgroup (8 waves as 2x4, two
// per SIMD) owns a 256 x 256 output tile; each wave owns 128 x 64 as 8 x 4
// blocks of v_mfma_f32_16x16x32_bf16 with its 128 accumulators in AGPRs
// (VGPRs in the persistent forward, whose epilogue reads each one twice).
// With two waves per SIMD one wave's MFMAs keep the matrix pipe busy while
// the other issues its loads or waits at the barrier.  With random
// operands this shape sustains a higher MFMA rate than 32x32x16 (measured
// about 84% against 72% of the dense peak in a loop without memory traffic).
// K advances 32 at a time through a ring of LDS buffers (32 KB each: A then
// B), four stages (128 KB) in the forward and dh, five (160 KB) in the
// persistent dW, whose G stages come from HBM.
// Operand tiles are copied global -> LDS by buffer_load_dwordx4 ... lds: each
// wave instruction fills 1 KB of LDS (16 bytes per lane, consecutive), no
// VGPR staging.  Loads run one stage less than the ring ahead; a stage is
// waited for with an explicit vmcnt and one barrier, placed among the stage's
// MFMAs so that MFMAs are in flight across it.  Out-of-range rows or K columns are given a
// buffer offset past the descriptor's range, which the hardware reads as zero.
// In LDS a tile row is 64 bytes (32 bf16 = four 16-byte chunks); chunk c of
// row r is stored at position c ^ tile_swz(r) (kernels.h), which keeps the
// fragment reads free of bank conflicts.  The backward operands, and the
// bf16 forward's tiled copies of W and h_c, arrive in a tiled layout whose
// 16 KB blocks are exactly this LDS image, so each stage load is one
// contiguous copy (row-major operands with 300 KB row strides touch 256
// pages per stage).
// Workgroups are remapped so consecutive tiles land on one XCD (dispatch is
// round-robin over the 8 XCDs).  The forward GEMM groups 4 tiles along M
// (with its tiled operands 4 and 6 timed 0.03-0.06 ms faster per 16k step
// than 8; 2, 3 and 16 slower);
// the backward GEMMs walk blocks of 4 x 8 tiles with N fastest, so the 32
// tiles an XCD runs at once cover at most 8 N-tiles and each slice of the
// large operand (G) is fetched into that XCD's L2 once for all of them.
//
// fp32 kernel (small problems).  Same tile mapping and epilogues, register
// staged loads, v_mfma_f32_32x32x2_f32 (layout Acc32).
#include <atomic>
#include <type_traits>

#include "kernels.h"

namespace rl {
namespace {

constexpr int NT = 256;
constexpr int GROUP_M = 4;
constexpr int OOB = (int)0x80000000;  // a buffer offset past any descriptor's range

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

// Blocks of 4 x 8 tiles (M x N), N fastest inside a block, blocks walked
// along N and then M; same XCD remap as map_tile.
__device__ __forceinline__ TileCoord map_tile_blocks(int tiles_m, int tiles_n, int splits,
                                                     int BM, int BN) {
  constexpr int BMT = 4, BNT = 8;
  TileCoord tc;
  const int nwg = gridDim.x;  // a multiple of 8
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int per_split = tiles_m * tiles_n;
  tc.valid = logical < per_split * splits;
  if (!tc.valid) return tc;
  tc.split = logical / per_split;
  const int rem = logical - tc.split * per_split;
  const int band = rem / (BMT * tiles_n);  // BMT rows of tiles
  const int first_m = band * BMT;
  const int hm = min(BMT, tiles_m - first_m);
  const int within = rem - band * BMT * tiles_n;
  const int blk = within / (hm * BNT);
  const int first_n = blk * BNT;
  const int wn = min(BNT, tiles_n - first_n);
  const int inb = within - blk * hm * BNT;
  tc.m0 = (int64_t)(first_m + inb / wn) * BM;
  tc.n0 = (int64_t)(first_n + inb % wn) * BN;
  return tc;
}

// Epilogue context handed to the epilogue functors.
struct EpiCtx {
  int64_t m0, n0;
  int wm_off, wn_off;  // wave tile origin inside the block tile
  int wave_m;          // 0/1
  int lane;
  int split;
  char* smem;          // the workgroup's LDS (free once the main loop is done)
  int smem_bytes;
};

// Accumulator layouts.  Register r of block (i, j) in lane l holds the wave
// tile's element (row(i, r, l), col(j, l)); the lanes holding one column are
// combined with col_max / col_sum (a fixed butterfly, so the result does not
// depend on timing), after which col_owner lanes hold the column's value.
// Registers 4q .. 4q+3 always hold four consecutive rows.
struct Acc32 {  // v_mfma_f32_32x32x* : 32 x 32 blocks, 16 registers per lane
  using V = f32x16;
  static constexpr int R = 16;
  static __device__ __forceinline__ int row(int i, int r, int lane) {
    return 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  }
  static __device__ __forceinline__ int col(int j, int lane) { return 32 * j + (lane & 31); }
  static __device__ __forceinline__ float col_max(float x) {
    return fmaxf(x, __shfl_xor(x, 32, 64));
  }
  static __device__ __forceinline__ float col_sum(float x) { return x + __shfl_xor(x, 32, 64); }
  static __device__ __forceinline__ bool col_owner(int lane) { return lane < 32; }
};
struct Acc16 {  // v_mfma_f32_16x16x32_bf16 : 16 x 16 blocks, 4 registers per lane
  using V = f32x4;
  static constexpr int R = 4;
  static __device__ __forceinline__ int row(int i, int r, int lane) {
    return 16 * i + 4 * (lane >> 4) + r;
  }
  static __device__ __forceinline__ int col(int j, int lane) { return 16 * j + (lane & 15); }
  static __device__ __forceinline__ float col_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    return fmaxf(x, __shfl_xor(x, 32, 64));
  }
  static __device__ __forceinline__ float col_sum(float x) {
    x += __shfl_xor(x, 16, 64);
    return x + __shfl_xor(x, 32, 64);
  }
  static __device__ __forceinline__ bool col_owner(int lane) { return lane < 16; }
};
// The same layout with the accumulators in VGPRs (the MFMAs' VGPR form): an
// epilogue that reads every accumulator more than once then needs no AGPR
// copies (v_accvgpr_read) for it.  Acc16 keeps them in AGPRs.
struct Acc16V : Acc16 {};

// ------------------------------------------------------------- epilogues ---

// Forward epilogue: rows are vocabulary entries, columns tokens.  Per column
// (token) and block tile of BM vocabulary rows: m = max z, s = sum e^(z-m),
// t = sum e^(z-m)(z-m) over the valid rows, with z = inv_t * acc.  When P is
// given, e^(z-m) is stored per element: bf16 into the tiled block layout of G
// (tiled_offset with ldp blocks per 256-token panel; every position of the
// tile is written, the dense-gradient pass zeroes those past V and Tc), fp32
// token-major P[t, v] (leading dimension ldp).  The exponent is formed as one
// fma on the raw accumulator, (acc * inv_t - m) * log2(e), fed to exp2; t is
// accumulated in that scaled unit and multiplied by ln 2 once.
// FULL: every tile of the launch lies inside V (the edge row of tiles, if
// any, gets a launch of its own); STORE: P is written.  Both are fixed per
// kernel so that no branch around the epilogue's variants keeps the
// accumulators alive in scratch.  m_base is the launch's first vocabulary row.
template <typename T, bool FULL_, bool STORE_> struct FwdEpi {
  static constexpr bool TILED_P = sizeof(T) == 2;
  float inv_t;
  int64_t V, Tc, J;
  float *pm, *ps, *pt;
  T* P;
  int64_t ldp;
  int64_t m_base;

  // No data-dependent branches while the accumulators are live: validity is
  // a select, the P store is a template parameter, and every lane writes the
  // reduced column values (all lanes of a column hold the same value after
  // the butterfly), so the main loop keeps each accumulator in place.
  template <class L, bool FULL, bool STORE, int MB, int NB, int BM, int BN>
  __device__ __forceinline__ void columns(typename L::V (&acc)[MB][NB], const EpiCtx& c,
                                          int vrows, float* red) const {
    constexpr float LOG2E = 1.4426950408889634f;
    static_assert(!TILED_P || (BN == TILE_ROWS && BM % TILE_K == 0), "tile = token panel");
    // Column maxima of the raw accumulators (inv_t > 0 keeps the order).
    float mraw[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < L::R; ++r) {
          const bool ok = FULL || L::row(i, r, c.lane) < vrows;
          mx = fmaxf(mx, ok ? acc[i][j][r] : -INFINITY);
        }
      mx = L::col_max(mx);
      red[c.wave_m * BN + c.wn_off + L::col(j, c.lane)] = mx;
    }
    // The exponent pass reads the accumulators again from AGPRs: without this
    // the compiler keeps the max pass's VGPR copies alive across the barrier,
    // spills other values, and the spill reloads wait for every outstanding
    // memory operation (the next tile's operand loads, this tile's stores).
    if constexpr (std::is_same<L, Acc16>::value) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) __asm__ volatile("" : "+a"(acc[i][j]));
    } else if constexpr (std::is_same<L, Acc16V>::value) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) __asm__ volatile("" : "+v"(acc[i][j]));
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = c.wn_off + L::col(j, c.lane);
      mraw[j] = fmaxf(red[col], red[BN + col]);
    }
    const float k2 = inv_t * LOG2E;
    float* rs = red + 2 * BN;
    float* rt = red + 4 * BN;
    // Tiled P stores (layout Acc16).  A lane holds 4 consecutive vocabulary
    // rows (16 i + 4 g, g = lane / 16) of token column 16 j + lane % 16.
    // Blocks i and i + 1 (i even) span one 32-row group, i.e. one 64-byte
    // row of G's tiled block for each token; a 16-lane row swap
    // (permlane16_swap on the packed values of the two blocks) leaves lane
    // row g holding one whole 16-byte chunk of that row, chunk
    // ((g & 1) << 1) | (g >> 1), so one 16-byte store per lane writes the
    // 16 tokens' rows as 1 KB of contiguous memory.  Sixteen columns to the
    // right is +512 elements, the next 32-row group +8192; the rest depends
    // only on the lane (wn_off and 16 j are multiples of 16, so the chunk
    // swizzle of a row depends on lane % 16 alone).
    T* pl = nullptr;
    if constexpr (TILED_P && STORE) {
      static_assert(std::is_base_of<Acc16, L>::value, "tiled P store assumes the 16x16 layout");
      static_assert(MB % 2 == 0, "row blocks pair up into 32-row groups");
      const int g = c.lane >> 4, l = c.lane & 15;
      const int chunk = ((g & 1) << 1) | (g >> 1);
      pl = P +
           ((c.n0 / TILE_ROWS) * ldp + (m_base + c.m0 + c.wm_off) / TILE_K) *
               (TILE_ROWS * TILE_K) +
           (c.wn_off + l) * TILE_K + ((chunk ^ tile_swz(l)) << 3);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int colb = c.wn_off + L::col(j, c.lane);
      const float off = -mraw[j] * k2;
      float s = 0.0f, t = 0.0f;
      uint32_t keep __attribute__((ext_vector_type(2))) = {0u, 0u};  // packed block i - 1
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int rq = 0; rq < L::R / 4; ++rq) {
          float e4[4];
#pragma unroll
          for (int r3 = 0; r3 < 4; ++r3) {
            const int r = rq * 4 + r3;
            const bool ok = FULL || L::row(i, r, c.lane) < vrows;
            const float d2 = fmaf(acc[i][j][r], k2, off);  // (z - m) log2(e)
            const float e = ok ? __builtin_amdgcn_exp2f(d2) : 0.0f;
            s += e;
            t = fmaf(e, d2, t);
            e4[r3] = e;
          }
          if constexpr (STORE) {
            const int vloc = c.wm_off + L::row(i, rq * 4, c.lane);  // multiple of 4
            if constexpr (TILED_P) {
              typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
              typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
              bf16x4 pk;
#pragma unroll
              for (int r3 = 0; r3 < 4; ++r3) pk[r3] = (__bf16)e4[r3];
              const u32x2 w = __builtin_bit_cast(u32x2, pk);
              if ((i & 1) == 0) {
                keep = w;
              } else {
                const auto lo2 = __builtin_amdgcn_permlane16_swap(keep[0], w[0], false, false);
                const auto hi2 = __builtin_amdgcn_permlane16_swap(keep[1], w[1], false, false);
                const u32x4 v = {lo2[0], hi2[0], lo2[1], hi2[1]};
                // streaming store: P is read back only after the whole GEMM
                __builtin_nontemporal_store(
                    v, reinterpret_cast<u32x4*>(pl + (i >> 1) * (TILE_ROWS * TILE_K) +
                                                16 * j * TILE_K));
              }
            } else {
              const int64_t col = c.n0 + colb;
              if (col < Tc) {
#pragma unroll
                for (int r3 = 0; r3 < 4; ++r3) {
                  const int64_t v = m_base + c.m0 + vloc + r3;
                  if (v < V) P[col * ldp + v] = Elem<T>::from_f32(e4[r3]);
                }
              }
            }
          }
        }
      s = L::col_sum(s);
      t = L::col_sum(t);
      rs[c.wave_m * BN + colb] = s;
      rt[c.wave_m * BN + colb] = t * 0.6931471805599453f;  // back to units of z
    }
    (void)mraw;
  }

  template <class L, int MB, int NB, int BM, int BN>
  __device__ __forceinline__ void apply(typename L::V (&acc)[MB][NB], const EpiCtx& c) const {
    const int64_t jt = (m_base + c.m0) / BM;
    __syncthreads();  // the previous users of the scratch area are done
    float* red = reinterpret_cast<float*>(c.smem);  // [2][BN] x 3
    const int64_t vr = V - m_base - c.m0 - c.wm_off;
    const int vrows = (int)(vr < 0 ? 0 : (vr > 2 * BM ? 2 * BM : vr));
    columns<L, FULL_, STORE_, MB, NB, BM, BN>(acc, c, vrows, red);
    __syncthreads();
    if (c.wave_m == 0 && L::col_owner(c.lane)) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int colb = c.wn_off + L::col(j, c.lane);
        const int64_t col = c.n0 + colb;
        if (col < Tc) {
          pm[col * J + jt] = fmaxf(red[colb], red[BN + colb]) * inv_t;
          ps[col * J + jt] = red[2 * BN + colb] + red[3 * BN + colb];
          pt[col * J + jt] = red[4 * BN + colb] + red[5 * BN + colb];
        }
      }
    }
  }
};

// Branch-free fp32 store of the wave tile (=, or += when ACC) through a
// buffer descriptor spanning the workgroup tile: elements outside [M, N]
// get an offset past the descriptor's range, whose stores the hardware drops
// and whose loads read 0.  Keeping the epilogue free of branches lets the
// compiler keep every accumulator in one register block through the main
// loop.  Offsets are 32-bit: the launchers require ldc < 2^21.
template <class L, bool ACC, int MB, int NB, int BM, int BN>
__device__ __forceinline__ void store_tile(typename L::V (&acc)[MB][NB], const EpiCtx& c,
                                           float* C, int64_t ldc, int64_t M, int64_t N) {
  const int64_t rows = min<int64_t>(M - c.m0, BM), cols = min<int64_t>(N - c.n0, BN);
  // The tile origin is uniform; readfirstlane makes that visible to the
  // compiler so the descriptor lives in SGPRs (no per-store waterfall).
  const uint64_t a = reinterpret_cast<uint64_t>(C + c.m0 * ldc + c.n0);
  const uint64_t au = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const int bytes = __builtin_amdgcn_readfirstlane((int)(((rows - 1) * ldc + cols) * 4));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(au), (short)0, bytes, 0x00020000);
  const int ld = (int)ldc;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int cl = c.wn_off + L::col(j, c.lane);
#pragma unroll
      for (int r = 0; r < L::R; ++r) {
        const int rl = c.wm_off + L::row(i, r, c.lane);
        const int off = (rl < rows && cl < cols) ? (rl * ld + cl) * 4 : OOB;
        float v = acc[i][j][r];
        if constexpr (ACC)
          v += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, off, 0, 0);
      }
    }
}

// C[split][row][col] = acc  (fp32).
struct StoreEpi {
  float* C;
  int64_t ldc, split_stride, M, N;
  template <class L, int MB, int NB, int BM, int BN>
  __device__ __forceinline__ void apply(typename L::V (&acc)[MB][NB], const EpiCtx& c) const {
    store_tile<L, false, MB, NB, BM, BN>(acc, c, C + (int64_t)c.split * split_stride, ldc, M, N);
  }
};

// dW[row][col] = acc, or += acc when ACC.
template <bool ACC>
struct DwEpi {
  float* C;
  int64_t ldc, M, N;
  template <class L, int MB, int NB, int BM, int BN>
  __device__ __forceinline__ void apply(typename L::V (&acc)[MB][NB], const EpiCtx& c) const {
    store_tile<L, ACC, MB, NB, BM, BN>(acc, c, C, ldc, M, N);
  }
};

// One DPP quad permutation (lanes 4q .. 4q+3 exchange values).
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// 4 x 4 transpose inside each quad of lanes: lane 4q + b holds x[r] = M[r][b]
// and receives y[k] = M[b][k].  Two exchange rounds (distance 2, then 1).
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x, int b) {
  const bool hi = (b & 2) != 0, odd = (b & 1) != 0;
  const float r0 = quad_perm<0x4E>(hi ? x[0] : x[2]);  // lanes b ^ 2
  const float r1 = quad_perm<0x4E>(hi ? x[1] : x[3]);
  const float z0 = hi ? r0 : x[0], z1 = hi ? r1 : x[1];
  const float z2 = hi ? x[2] : r0, z3 = hi ? x[3] : r1;
  const float u0 = quad_perm<0xB1>(odd ? z0 : z1);  // lanes b ^ 1
  const float u1 = quad_perm<0xB1>(odd ? z2 : z3);
  f32x4 y;
  y[0] = odd ? u0 : z0;
  y[1] = odd ? z1 : u0;
  y[2] = odd ? u1 : z2;
  y[3] = odd ? z3 : u1;
  return y;
}

// dW (=|+=) acc with 16-byte accesses (layout Acc16): a quad transpose gives
// lane 16 g + 4 a + b row 16 i + 4 g + b, columns 16 j + 4 a .. + 3 of every
// block, so each lane writes (and, when accumulating, reads) 32 float4
// instead of 128 floats.  Elements outside [M, N] get an offset past the
// descriptor's range (N is a multiple of 4 here).  The accumulate pass reads
// in two halves of 16 loads, so that at most 64 VGPRs hold loaded values.
// Returns nothing; every lane issues exactly 32 stores (the persistent kernel
// counts them in its stage waits).
template <bool ACC>
struct DwEpiT {
  float* C;
  int64_t ldc, M, N;
  static constexpr int STORES = 32;
  template <class L, int MB, int NB, int BM, int BN>
  __device__ __forceinline__ void apply(typename L::V (&acc)[MB][NB], const EpiCtx& c) const {
    static_assert(std::is_same<L, Acc16>::value && MB * NB == 32, "32 blocks of 16 x 16");
    const int64_t rows = min<int64_t>(M - c.m0, BM), cols = min<int64_t>(N - c.n0, BN);
    const uint64_t a = reinterpret_cast<uint64_t>(C + c.m0 * ldc + c.n0);
    const uint64_t au = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const int bytes = __builtin_amdgcn_readfirstlane((int)(((rows - 1) * ldc + cols) * 4));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(au), (short)0, bytes, 0x00020000);
    const int ld = (int)ldc;
    const int g = c.lane >> 4, q = (c.lane >> 2) & 3, b = c.lane & 3;
    auto offset = [&](int i, int j) {
      const int rl = c.wm_off + 16 * i + 4 * g + b, cl = c.wn_off + 16 * j + 4 * q;
      return (rl < rows && cl < cols) ? (rl * ld + cl) * 4 : OOB;
    };
    // Blocks in two batches of 16 (block q = (i, j) with i = q / NB, j = q % NB).
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 old[16];
      if constexpr (ACC) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int q = 16 * half + e;
          old[e] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, offset(q / NB, q % NB), 0, 0));
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int q = 16 * half + e;
        f32x4 y = quad_transpose(acc[q / NB][q % NB], b);
        if constexpr (ACC) {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] += __uint_as_float(old[e][r]);
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), rs,
                                               offset(q / NB, q % NB), 0, 0);
      }
    }
  }
};

// ------------------------------------------------------------ bf16 kernel ---

// K advances 32 at a time through a ring of BF_ST = 4 stages of 32 KB (the
// forward and dh: a ring of five, filling the 160 KB of LDS, was slightly
// slower for both; the persistent dW has its own, DW_ST).
constexpr int BF_BM = 256, BF_BN = 256, BF_BK = 32, BF_ST = 4;
constexpr int BF_STAGE_A = BF_BM * BF_BK * 2;  // bytes
constexpr int BF_STAGE = (BF_BM + BF_BN) * BF_BK * 2;
constexpr int BF_LDS = BF_ST * BF_STAGE;  // the ring; the epilogues reuse it (128 KB)
static_assert(BF_LDS >= 6 * BF_BN * 4, "forward epilogue reductions");
static_assert(BF_STAGE_A == TILE_BLOCK_BYTES, "a stage of one operand is one tiled block");

// Buffer descriptor (gfx9): base, stride 0, num_records = bytes, default config.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int32_t)(a & 0xffffffffu);
  r[1] = (int32_t)(a >> 32);
  r[2] = (int32_t)bytes;
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from `rsrc` + voffset + soffset into LDS at lds_addr +
// 16 * lane (lds_addr and soffset wave-uniform).  Issued as inline asm so the
// compiler adds no vmcnt waits of its own; the main loop waits explicitly.
// Offsets past the descriptor's range read zeros.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t lds_addr, int voffset,
                                           int soffset = 0) {
#pragma unroll
  for (int i = 0; i < 4; ++i) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  soffset = __builtin_amdgcn_readfirstlane(soffset);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr), "v"(voffset), "s"(rsrc), "s"(soffset) : "memory");
}
// Four loads into consecutive 1 KB of LDS under one M0, from four per-lane
// source offsets: load i adds the immediate offset i KB to both its source
// and its destination, so v_i must hold the piece's source offset less i KB.
__device__ __forceinline__ void load_lds16_4v(i32x4 rsrc, uint32_t lds_addr, int v0, int v1,
                                              int v2, int v3, int soffset) {
#pragma unroll
  for (int i = 0; i < 4; ++i) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  soffset = __builtin_amdgcn_readfirstlane(soffset);
  asm volatile(
      "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
      "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds"
      :: "s"(lds_addr), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(rsrc), "s"(soffset)
      : "memory");
}
// Four such loads of consecutive 1 KB pieces (source and destination both
// step by 1 KB) under one M0: the instruction's immediate offset moves the
// LDS destination as well as the source (checked on the GPU).
__device__ __forceinline__ void load_lds16_x4(i32x4 rsrc, uint32_t lds_addr, int voffset,
                                              int soffset = 0) {
#pragma unroll
  for (int i = 0; i < 4; ++i) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  soffset = __builtin_amdgcn_readfirstlane(soffset);
  asm volatile(
      "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen offset:3072 lds"
      :: "s"(lds_addr), "v"(voffset), "s"(rsrc), "s"(soffset) : "memory");
}

// ATR pieces: wave instruction q copies half q & 1 (16 rows) of piece q >> 1;
// the byte offset of a copying wave's piece i from its first (q even).
__host__ __device__ constexpr int atr_piece_step(int i) {
  return (i >> 1) * TILE_BLOCK_BYTES + (i & 1) * 1024;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until the oldest stage not yet waited for has landed, given how many
// younger stages (LPS loads per thread each) were issued after it, and
// whether NST stores (an epilogue's) were issued after it as well.
template <int LPS, int NST = 0>
__device__ __forceinline__ void wait_stage(int younger, bool stores = false) {
  static_assert(3 * LPS + NST < 64, "vmcnt");
  if (NST > 0 && stores) {
    if (younger >= 3)
      wait_vmcnt<3 * LPS + NST>();
    else if (younger == 2)
      wait_vmcnt<2 * LPS + NST>();
    else if (younger == 1)
      wait_vmcnt<LPS + NST>();
    else
      wait_vmcnt<NST>();
  } else if (younger >= 3) {
    wait_vmcnt<3 * LPS>();
  } else if (younger == 2) {
    wait_vmcnt<2 * LPS>();
  } else if (younger == 1) {
    wait_vmcnt<LPS>();
  } else {
    wait_vmcnt<0>();
  }
}
static_assert(BF_ST - 2 <= 3, "wait_stage covers up to three younger stages");

// Of a stage's 32 MFMAs per wave, BF_PRE issue before the stage barrier and
// the rest after it, interleaved with the next stage's fragment reads (one
// read per MFMA while both last).
constexpr int BF_PRE = 16;
template <int NR, int NM>
__device__ __forceinline__ void reads_between_mfmas() {
  constexpr int P = NR < NM ? NR : NM;
#pragma unroll
  for (int q = 0; q < P; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
  }
  if constexpr (NR > P) __builtin_amdgcn_sched_group_barrier(0x100, NR - P, 0);
  if constexpr (NM > P) __builtin_amdgcn_sched_group_barrier(0x008, NM - P, 0);
}

// TILED = false: A [M, lda] and B [N, ldb] row-major, any K (multiple of 8).
// TILED = true: A and B in the tiled block layout (tiled_offset in
// kernels.h) with lda / ldb = blocks per 256-row panel; K is a multiple of 32
// or the blocks are zero past K.
//
constexpr int BF_NT = 512;  // 8 waves
// A stage is 32 wave instructions of 1 KB (16 per operand).  Only the first
// BF_DMAW waves issue them, BF_PER per operand each; the other waves only
// read fragments and issue MFMAs, so on every SIMD one wave keeps the matrix
// pipe fed while the other waits on the copy path.
constexpr int BF_DMAW = 4;
constexpr int BF_PER = 16 / BF_DMAW;  // 1 KB pieces per operand per copying wave
constexpr int BF_LPS = 2 * BF_PER;    // direct-to-LDS loads per copying wave per stage
static_assert(BF_DMAW * BF_PER == 16 && BF_PER % 2 == 0, "copy split");
// The persistent dW kernel's split (its waits also count 32 epilogue stores).
// dW's wave layout: row blocks per wave (4: 4 x 2 waves of 64 x 128, which
// halves the transposing reads of G per wave against 8, 2 x 4 waves of
// 128 x 64).
constexpr int DW_MB = 4;
constexpr int BT_DMAW = 4;
constexpr int BT_PER = 16 / BT_DMAW;
constexpr int BT_LPS = 2 * BT_PER;
static_assert(BT_DMAW * BT_PER == 16 && BT_PER % 2 == 0, "copy split");

// Software pipeline per stage kt (one K-step of 32): the MFMAs of row blocks
// 0..3 issue from fragments read during the previous stage, then the wave
// waits for stage kt+1 and passes the barrier while those MFMAs execute,
// refills the buffer of stage kt (whose fragments every wave read before the
// barrier), reads stage kt+1's fragments and issues the MFMAs of row blocks
// 4..7.  The refill therefore cannot race with fragment reads.
//
// ATR (with TILED): A is given transposed, as the tiled layout of A^T [K, M]
// with lda = blocks per 256-row panel of A^T (the dense gradient G [tokens,
// vocabulary] for dW = G^T h).  Stage kt of A then is rows (k0 % 256) .. +31
// of the eight blocks m0/32 .. +7 of panel k0 / 256: eight 2 KB pieces, one
// per 32-column group, copied verbatim.  Its fragments are read with
// ds_read_b64_tr_b16: for row block i (16 columns of A^T, half of a piece)
// lane j of 16-lane group g reads the 8 bytes at row 8 g + j / 4 (then
// 8 g + 4 + j / 4), columns 4 (j % 4) .. +3, and receives column j % 16 of
// rows 8 g .. 8 g + 3 (then + 4 .. 7): exactly the MFMA A fragment (row j,
// k = 8 g .. 8 g + 7).  The split start must be a multiple of 256.
template <bool TILED, class Epi, bool ATR = false>
__global__ void __launch_bounds__(BF_NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_bf16_kernel(const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ B,
                 int64_t ldb, int64_t M, int64_t N, int64_t K, int64_t k_split, int tiles_m,
                 int tiles_n, int splits, Epi epi) {
  static_assert(TILED || !ATR, "transposed A comes in the tiled layout");
  __shared__ __attribute__((aligned(1024))) char lds[BF_LDS];
  const TileCoord tc = TILED ? map_tile_blocks(tiles_m, tiles_n, splits, BF_BM, BF_BN)
                              : map_tile(tiles_m, tiles_n, splits, BF_BM, BF_BN);
  if (!tc.valid) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int wm = wave >> 2, wn = wave & 3;                      // 128 x 64 sub-tile
  const int64_t kb = (int64_t)tc.split * k_split;
  const int64_t ke = min(K, kb + k_split);
  const int nk = (int)ceil_div(max<int64_t>(ke - kb, 0), BF_BK);
  i32x4 rsa, rsb;
  // Copy slots of a copying wave: its piece i of each operand sits at the
  // lane's base offset plus a uniform step (sa_step / sb_step).
  int offa, offb, kc = 0;
  int sa_step = 1024, sb_step = 1024;
  // ATR: the A blocks of this tile's columns that exist (the rest read zero).
  const int64_t a_blk0 = tc.m0 / TILE_K;
  const uint32_t a_bytes =
      ATR ? (uint32_t)(min<int64_t>(BF_BM / TILE_K, lda - a_blk0) * TILE_BLOCK_BYTES) : 0u;
  if constexpr (TILED) {
    // Panel of this tile: blocks [m0/256 * lda + kb/32, ...), 16 KB each.
    const int64_t ba = (tc.m0 / BF_BM) * lda + kb / BF_BK;
    const int64_t bb = (tc.n0 / BF_BN) * ldb + kb / BF_BK;
    rsa = make_rsrc(A + ba * (TILE_BLOCK_BYTES / 2), (uint32_t)(nk * TILE_BLOCK_BYTES));
    rsb = make_rsrc(B + bb * (TILE_BLOCK_BYTES / 2), (uint32_t)(nk * TILE_BLOCK_BYTES));
    offa = offb = (wave * BF_PER * 64 + lane) * 16;
    if constexpr (ATR) {
      const int q = wave * BF_PER;  // even
      offa = (q >> 1) * TILE_BLOCK_BYTES + (lane >> 2) * 64 + (lane & 3) * 16;
    }
  } else {
    const int64_t rows_a = min<int64_t>(M - tc.m0, BF_BM), rows_b = min<int64_t>(N - tc.n0, BF_BN);
    rsa = make_rsrc(A + tc.m0 * lda, (uint32_t)(rows_a * lda * 2));
    rsb = make_rsrc(B + tc.n0 * ldb, (uint32_t)(rows_b * ldb * 2));
    // Slot p = (wave * BF_PER + i) * 64 + lane: tile row p/4, stored chunk p%4
    // holds logical chunk (p%4) ^ tile_swz(row).  Piece i is 16 rows further
    // down, which keeps tile_swz(row); rows past the tile's extent lie past
    // the descriptor's range and read zero.
    const int p = wave * BF_PER * 64 + lane;
    const int row = p >> 2, ch = (p & 3) ^ tile_swz(row);
    kc = 8 * ch;
    offa = (int)((row * lda + kb + 8 * ch) * 2);
    offb = (int)((row * ldb + kb + 8 * ch) * 2);
    sa_step = (int)(16 * lda * 2);
    sb_step = (int)(16 * ldb * 2);
  }
  const bool copier = wave < BF_DMAW;
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  auto issue = [&](int kt) {
    if (!copier) return;
    const uint32_t sa = lds_base + (uint32_t)((kt % BF_ST) * BF_STAGE);
    const uint32_t sb = sa + BF_STAGE_A;
    int oa, ob;
    i32x4 ra = rsa;
    if constexpr (ATR) {
      // rows 32 ks .. of panel ks / 8 (ks = the stage's 32-row group of A^T)
      const int64_t ks = kb / BF_BK + kt;
      ra = make_rsrc(A + ((ks >> 3) * lda + a_blk0) * (TILE_BLOCK_BYTES / 2), a_bytes);
      oa = offa + (int)(ks & 7) * (TILE_ROWS / 8 * TILE_K * 2);
      ob = offb + kt * TILE_BLOCK_BYTES;
    } else if constexpr (TILED) {
      oa = offa + kt * TILE_BLOCK_BYTES;
      ob = offb + kt * TILE_BLOCK_BYTES;
    } else {
      const int k0 = kt * BF_BK;
      const bool kok = kb + k0 + kc < ke;
      oa = kok ? offa + 2 * k0 : OOB;
      ob = kok ? offb + 2 * k0 : OOB;
    }
    if constexpr (TILED && BF_PER == 4) {
      // tiled operands: a copying wave's four pieces are consecutive 1 KB
      // runs of one block (A only without ATR)
      const uint32_t dst = (uint32_t)(wave * BF_PER * 1024);
      if constexpr (ATR) {
#pragma unroll
        for (int i = 0; i < BF_PER; ++i)
          load_lds16(ra, sa + dst + i * 1024, oa, atr_piece_step(i));
      } else {
        load_lds16_x4(ra, sa + dst, oa);
      }
      load_lds16_x4(rsb, sb + dst, ob);
    } else {
#pragma unroll
      for (int i = 0; i < BF_PER; ++i) {
        const uint32_t dst = (uint32_t)((wave * BF_PER + i) * 1024);
        load_lds16(ra, sa + dst, oa, ATR ? atr_piece_step(i) : i * sa_step);
        load_lds16(rsb, sb + dst, ob, i * sb_step);
      }
    }
  };
  // Fragment byte offsets inside a stage: in 16-row block i the lane reads
  // row 16 i + lane % 16, 16-byte chunk lane / 16 (k = 8 (lane / 16) .. +7).
  // Sixteen rows down keep tile_swz(row), so block i sits at +1 KB * i.
  int fa0, fb0;
  {
    const int ch = lane >> 4;
    int row = wm * 128 + (lane & 15);
    fa0 = row * 64 + 16 * (ch ^ tile_swz(row));
    row = wn * 64 + (lane & 15);
    fb0 = BF_STAGE_A + row * 64 + 16 * (ch ^ tile_swz(row));
  }
  // ATR: transposed-read offsets ftr[half][second] inside a piece; row
  // block i of the wave is piece 4 wm + i / 2, half i & 1.
  int ftr[2][2] = {{0, 0}, {0, 0}};
  if constexpr (ATR) {
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int r = 8 * g + 4 * sec + (j >> 2);
        const int c = 2 * h + ((j & 3) >> 1);
        ftr[h][sec] = r * 64 + ((c ^ tile_swz(r)) << 4) + 8 * (j & 1);
      }
  }
  auto read_a = [&](const char* sn, int i) -> bf16x8 {
    if constexpr (ATR) {
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef v4s __attribute__((address_space(3))) * lds_v4s;
      const char* pc = sn + (4 * wm + (i >> 1)) * (BF_STAGE_A / 8);
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(pc + ftr[i & 1][0]));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(pc + ftr[i & 1][1]));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return *reinterpret_cast<const bf16x8*>(sn + fa0 + 1024 * i);
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < BF_ST - 1; ++s)
      if (s < nk) issue(s);
    if (copier) wait_stage<BF_LPS>(min(nk - 1, BF_ST - 2));
    __syncthreads();
    if (BF_ST - 1 < nk) issue(BF_ST - 1);
    // Two fragment sets used in turn (no register moves carry fragments from
    // one stage to the next).  kstep: stage kt's MFMAs from x, with stage
    // kt+1 awaited, the buffer of stage kt refilled and stage kt+1's
    // fragments read into y.
    bf16x8 ca[8], cb[4], da[8], db[4];
    auto read_stage = [&](const char* sn, bf16x8 (&ya)[8], bf16x8 (&yb)[4]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ya[i] = read_a(sn, i);
#pragma unroll
      for (int j = 0; j < 4; ++j) yb[j] = *reinterpret_cast<const bf16x8*>(sn + fb0 + 1024 * j);
    };
    // STEADY (compile time): kt + BF_ST < nk, so BF_ST - 2 stages are
    // younger than stage kt + 1 and stage kt + BF_ST is refilled.
    auto kstep = [&](auto steady, int kt, bf16x8 (&xa)[8], bf16x8 (&xb)[4], bf16x8 (&ya)[8],
                     bf16x8 (&yb)[4]) {
      constexpr bool STEADY = decltype(steady)::value;
#pragma unroll
      for (int q = 0; q < BF_PRE; ++q)
        acc[q / 4][q % 4] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[q / 4], xb[q % 4], acc[q / 4][q % 4], 0, 0, 0);
      // Stage kt+1 has landed once at most the stages issued after it
      // (kt+2, kt+3) are outstanding.
      if constexpr (STEADY) {
        if (copier) wait_vmcnt<(BF_ST - 2) * BF_LPS>();
      } else {
        if (copier) wait_stage<BF_LPS>(min(nk - 2 - kt, BF_ST - 2));
      }
      __syncthreads();
      if (STEADY || kt + BF_ST < nk) issue(kt + BF_ST);  // into the buffer of stage kt
      read_stage(lds + ((unsigned)(kt + 1) % BF_ST) * BF_STAGE, ya, yb);
#pragma unroll
      for (int q = BF_PRE; q < 32; ++q)
        acc[q / 4][q % 4] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[q / 4], xb[q % 4], acc[q / 4][q % 4], 0, 0, 0);
      // One fragment read of the next stage per MFMA after the barrier (dh,
      // the long-K contraction: 7.21 -> 6.79 ms on the 16k step against all
      // reads first); the next step's MFMAs, which need those fragments,
      // stay out of this part.  The transposed-A variant (20 reads; dW of
      // short chunks) keeps all reads first.
      if constexpr (ATR) {
        __builtin_amdgcn_sched_group_barrier(0x100, 20, 0);           // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 32 - BF_PRE, 0);  // MFMAs
      } else {
        reads_between_mfmas<12, 32 - BF_PRE>();
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // With an even stage count one step runs before the pairs, so the last
    // stage always ends up in ca/cb and no branch follows the loop.
    const std::false_type gen;
    const std::true_type std_;
    int kt = 0;
    if (nk % 2 == 0) {
      read_stage(lds, da, db);
      kstep(gen, 0, da, db, ca, cb);
      kt = 1;
    } else {
      read_stage(lds, ca, cb);
    }
    for (; kt + 1 + BF_ST < nk; kt += 2) {
      kstep(std_, kt, ca, cb, da, db);
      kstep(std_, kt + 1, da, db, ca, cb);
    }
    for (; kt + 2 < nk; kt += 2) {
      kstep(gen, kt, ca, cb, da, db);
      kstep(gen, kt + 1, da, db, ca, cb);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[i], cb[j], acc[i][j], 0, 0, 0);
  }
  // Hand the accumulators to the epilogue as AGPR blocks: this keeps the
  // register allocator from rotating them through the main loop.
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) __asm__ volatile("" : "+a"(acc[i][j]));
  EpiCtx ctx;
  ctx.m0 = tc.m0;
  ctx.n0 = tc.n0;
  ctx.wm_off = wm * 128;
  ctx.wn_off = wn * 64;
  ctx.wave_m = wm;
  ctx.lane = lane;
  ctx.split = tc.split;
  ctx.smem = lds;
  ctx.smem_bytes = BF_LDS;
  epi.template apply<Acc16, 8, 4, BF_BM, BF_BN>(acc, ctx);
}

// Persistent variant for a short K loop (the forward, K = H), on tiled
// operands: one workgroup per CU walks its tiles in order and the
// stage ring runs on across tile boundaries, so the first stages of the next
// tile are in flight while the epilogue of the current one runs (the
// epilogue's LDS is the ring slot of the tile's last stage).  Tiles of XCD x are the logical tiles
// [x * ceil(T / 8), ...) of map_tile's order, taken round-robin by its
// workgroups, so the tiles an XCD runs at once are consecutive as before.
// Requires K to be a multiple of BF_BK with at least BF_ST stages.  The
// epilogue's stores count in vmcnt like the loads, in issue order; a wait
// that ignores them (counts only younger stages) also waits for the stores
// issued after the awaited stage, which is correct and measured to cost
// nothing here.  EVEN_NK: the stage count K / BF_BK is even (fixed per
// launch; it decides which fragment set holds the last stage).  Both
// operands come in the tiled block layout (lda / ldb = blocks per 256-row
// panel, zero past K), so a copying wave's pieces are consecutive 1 KB runs
// (8.00 -> 7.55 ms per 16k step against row-major operands with 4 KB row
// strides, whose pieces came from 16-row-apart runs).
template <class Epi, bool EVEN_NK>
__global__ void __launch_bounds__(BF_NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_bf16_persist(const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ B,
                  int64_t ldb, [[maybe_unused]] int64_t M, [[maybe_unused]] int64_t N, int64_t K,
                  int tiles_m, int tiles_n, Epi epi) {
  __shared__ __attribute__((aligned(1024))) char lds[BF_LDS];
  static_assert(BF_STAGE >= 6 * BF_BN * 4, "the epilogue's reductions fit one stage");
  const int total = tiles_m * tiles_n;
  const int per_xcd = gridDim.x >> 3;  // the grid is a multiple of 8
  const int chunk = (int)ceil_div(total, 8);
  const int lo = (blockIdx.x & 7) * chunk, hi = min(total, lo + chunk);
  int t = lo + (blockIdx.x >> 3);
  if (t >= hi) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int wm = wave >> 2, wn = wave & 3;
  const int nk = (int)ceil_div(K, BF_BK);
  // Per-lane offsets, tile independent: the operand copy slots (rows past a
  // tile's extent fall outside its descriptor and read zero; K is a multiple
  // of BF_BK here) and the fragment reads.  They are formed from an opaque
  // copy of the lane index before the first tile and again after every
  // epilogue, so they are not live (and not spilled) across the epilogue.
  static_assert(BF_PER == 4, "four pieces per operand and copying wave");
  struct LaneOffs {
    int oc, fa, fb;
  };
  const bool copier = wave < BF_DMAW;
  auto lane_offs = [&]() {
    int l;
    __asm__ volatile("v_and_b32 %0, 63, %1" : "=v"(l) : "v"(tid));
    LaneOffs o;
    // the wave's pieces: 1 KB runs wave * BF_PER .. of each operand's block
    o.oc = (wave * BF_PER * 64 + l) * 16;
    const int ch = l >> 4;
    int row = wm * 128 + (l & 15);
    o.fa = row * 64 + 16 * (ch ^ tile_swz(row));
    row = wn * 64 + (l & 15);
    o.fb = BF_STAGE_A + row * 64 + 16 * (ch ^ tile_swz(row));
    return o;
  };
  LaneOffs lof = lane_offs();
  auto coords = [&](int lt, int64_t& m0, int64_t& n0) {
    const int group = lt / (GROUP_M * tiles_n);
    const int first_m = group * GROUP_M;
    const int gsize = min(GROUP_M, tiles_m - first_m);
    const int within = lt - group * GROUP_M * tiles_n;
    m0 = (int64_t)(first_m + within % gsize) * BF_BM;
    n0 = (int64_t)(within / gsize) * BF_BN;
  };
  // Descriptors are uniform; readfirstlane keeps them in SGPRs across the
  // tile loop.
  // The panel's blocks; rows past the matrix are zero in the layout.
  auto panel = [&](const bf16_t* X, int64_t r0, int64_t ld) {
    i32x4 r = make_rsrc(X + (r0 / BF_BM) * ld * (TILE_BLOCK_BYTES / 2),
                        (uint32_t)(nk * TILE_BLOCK_BYTES));
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
    return r;
  };
  int64_t m0, n0;
  coords(t, m0, n0);
  i32x4 rsa = panel(A, m0, lda), rsb = panel(B, n0, ldb), nrsa = rsa, nrsb = rsb;
  int tnext = t + per_xcd;
  bool has_next = tnext < hi;
  int64_t nm0 = 0, nn0 = 0;
  if (has_next) {
    coords(tnext, nm0, nn0);
    nrsa = panel(A, nm0, lda);
    nrsb = panel(B, nn0, ldb);
  }
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  // The byte offset of stage kt passes through an opaque SGPR copy, so the
  // per-lane offsets are formed at each issue instead of being kept as
  // induction variables (registers are short in the K loop).
  auto issue = [&](i32x4 ra, i32x4 rb, int kt, int slot) {
    if (!copier) return;
    const uint32_t sa = lds_base + (uint32_t)(slot * BF_STAGE);
    const uint32_t sb = sa + BF_STAGE_A;
    int kblk;
    __asm__ volatile("s_lshl_b32 %0, %1, 14"
                     : "=s"(kblk)
                     : "s"(__builtin_amdgcn_readfirstlane(kt)));  // kt * TILE_BLOCK_BYTES
    const uint32_t dst = (uint32_t)(wave * BF_PER * 1024);
    load_lds16_x4(ra, sa + dst, lof.oc, kblk);
    load_lds16_x4(rb, sb + dst, lof.oc, kblk);
  };
  bf16x8 ca[8], cb[4], da[8], db[4];  // two fragment sets, used in turn
  // In the order the MFMAs consume them: row block 0, the column blocks, the
  // other row blocks (the forward 0.04 ms faster per 16k step; dh and dW keep
  // row blocks first, 0.01 and 0.05 ms faster that way).
  auto read_frags = [&](int slot, bf16x8 (&fa)[8], bf16x8 (&fb)[4]) {
    const char* sn = lds + slot * BF_STAGE;
    fa[0] = *reinterpret_cast<const bf16x8*>(sn + lof.fa);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(sn + lof.fb + 1024 * j);
#pragma unroll
    for (int i = 1; i < 8; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(sn + lof.fa + 1024 * i);
  };
  // First tile: stages 0 .. BF_ST-2, then stage 0 awaited, stage BF_ST-1
  // issued.
  int gb = 0;  // ring position of the current tile's stage 0
#pragma unroll
  for (int s = 0; s < BF_ST - 1; ++s) issue(rsa, rsb, s, s);
  if (copier) wait_stage<BF_LPS>(BF_ST - 2);
  __syncthreads();
  issue(rsa, rsb, BF_ST - 1, BF_ST - 1);
  if constexpr (EVEN_NK) read_frags(0, da, db);
  else read_frags(0, ca, cb);
  for (;;) {
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
    // Stage kt's MFMAs from fragments xa/xb, with stage kt+1 awaited, the
    // buffer of stage kt refilled and stage kt+1's fragments read into ya/yb.
    // STEADY (compile time) marks the steps with kt + BF_ST < nk: BF_ST - 2
    // stages are younger than stage kt + 1 and the refill is this tile's
    // stage kt + BF_ST, so the wait and the refill need no run-time choice.
    auto kstep = [&](auto steady, int kt, bf16x8 (&xa)[8], bf16x8 (&xb)[4], bf16x8 (&ya)[8],
                     bf16x8 (&yb)[4]) {
      constexpr bool STEADY = decltype(steady)::value;
#pragma unroll
      for (int q = 0; q < BF_PRE; ++q)
        acc[q / 4][q % 4] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[q / 4], xb[q % 4], acc[q / 4][q % 4], 0, 0, 0);
      // Stage kt+1 has landed once at most the stages issued after it are
      // outstanding (BF_ST - 2, except at the end of the last tile).
      if constexpr (STEADY) {
        if (copier) wait_vmcnt<(BF_ST - 2) * BF_LPS>();
      } else {
        if (copier) wait_stage<BF_LPS>(has_next ? BF_ST - 2 : min(nk - 2 - kt, BF_ST - 2));
      }
      __syncthreads();
      // Refill the buffer of stage kt with stage kt + BF_ST of this tile or,
      // past its end, with the first stages of the next tile.
      const int slot = (unsigned)(gb + kt) % BF_ST;
      if constexpr (STEADY) {
        issue(rsa, rsb, kt + BF_ST, slot);
      } else {
        if (kt + BF_ST < nk) issue(rsa, rsb, kt + BF_ST, slot);
        else if (has_next) issue(nrsa, nrsb, kt + BF_ST - nk, slot);
      }
      read_frags((unsigned)(gb + kt + 1) % BF_ST, ya, yb);
#pragma unroll
      for (int q = BF_PRE; q < 32; ++q)
        acc[q / 4][q % 4] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[q / 4], xb[q % 4], acc[q / 4][q % 4], 0, 0, 0);
      // One fragment read of the next stage per MFMA after the barrier: 8.65
      // -> 8.34 ms on the 16k step against all reads first.
      reads_between_mfmas<12, 32 - BF_PRE>();
    };
    auto last = [&](bf16x8 (&xa)[8], bf16x8 (&xb)[4]) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], xb[j], acc[i][j], 0, 0, 0);
    };
    // Stages 0 .. nk-2 in pairs, the two fragment sets swapping roles, so
    // no register moves carry fragments from one stage to the next; the last
    // stage is peeled off (no fragment register is undefined on the way out).
    // With an even stage count, stage 0's fragments are in da/db and one step
    // runs before the pairs, so the last stage always ends up in ca/cb: the
    // parity is a template parameter, and no branch with live accumulators
    // surrounds the loop.
    // The pairs run in two loops: the steady ones, then the last steps
    // (whose refill switches to the next tile, and at the end of the last
    // tile fewer stages follow).
    const std::false_type gen;
    const std::true_type std_;
    int kt = 0;
    if constexpr (EVEN_NK) {
      kstep(gen, 0, da, db, ca, cb);
      kt = 1;
    }
    for (; kt + 1 + BF_ST < nk; kt += 2) {
      kstep(std_, kt, ca, cb, da, db);
      kstep(std_, kt + 1, da, db, ca, cb);
    }
    for (; kt + 2 < nk; kt += 2) {
      kstep(gen, kt, ca, cb, da, db);
      kstep(gen, kt + 1, da, db, ca, cb);
    }
    last(ca, cb);  // kt = nk - 1
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) __asm__ volatile("" : "+v"(acc[i][j]));
    // The lane index enters the epilogue through an opaque copy, so that
    // nothing the epilogue derives from it is hoisted out of the tile loop
    // (where it would hold registers through the K loop).
    int elane;
    __asm__ volatile("v_and_b32 %0, 63, %1" : "=v"(elane) : "v"(tid));
    EpiCtx ctx;
    ctx.m0 = m0;
    ctx.n0 = n0;
    ctx.wm_off = wm * 128;
    ctx.wn_off = wn * 64;
    ctx.wave_m = wm;
    ctx.lane = elane;
    ctx.split = 0;
    // The epilogue's LDS is the ring slot of this tile's last stage: the next
    // tile's first BF_ST - 1 stages fill the other slots, and the epilogue's
    // opening barrier follows every wave's last fragment read from this one.
    ctx.smem = lds + ((gb + nk - 1) % BF_ST) * BF_STAGE;
    ctx.smem_bytes = BF_STAGE;
    epi.template apply<Acc16V, 8, 4, BF_BM, BF_BN>(acc, ctx);
    if (!has_next) break;
    // Advance: stages 0 .. BF_ST-2 of the next tile are in flight (issued in
    // the last iterations above); await stage 0, then, past a barrier that
    // ends the epilogue's use of its slot, issue stage BF_ST-1 there.
    gb += nk;
    m0 = nm0;
    n0 = nn0;
    rsa = nrsa;
    rsb = nrsb;
    tnext += per_xcd;
    has_next = tnext < hi;
    if (has_next) {
      coords(tnext, nm0, nn0);
      nrsa = panel(A, nm0, lda);
      nrsb = panel(B, nn0, ldb);
    }
    lof = lane_offs();
    if (copier) wait_stage<BF_LPS>(BF_ST - 2);
    __syncthreads();
    issue(rsa, rsb, BF_ST - 1, (gb + BF_ST - 1) % BF_ST);
    if constexpr (EVEN_NK) read_frags(gb % BF_ST, da, db);
    else read_frags(gb % BF_ST, ca, cb);
  }
}

// The persistent dW runs a ring of five stages (the whole 160 KB of LDS; its
// epilogue uses none): one stage more lookahead for G, whose stages come from
// HBM (16k step against four stages: dW 8.01 -> 7.86 ms on one box, 7.88 ->
// 7.81 ms on another).
constexpr int DW_ST = 5;
static_assert(DW_ST - 2 <= 3, "wait_stage covers up to three younger stages");

// Persistent variant for tiled operands with a long K loop (the dW
// contraction, K = the chunk's tokens): one workgroup per CU walks its tiles
// in the blocked order of map_tile_blocks (XCD x takes the logical tiles
// [x * ceil(T / 8), ...) round-robin), and the stage ring runs on across tile
// boundaries as in gemm_bf16_persist.  What this buys is the epilogue: its
// Epi::STORES stores per lane are issued after the first DW_ST - 1 stages of
// the next tile and drain while those stages' MFMAs run.  The stage waits of
// the next tile's first DW_ST - 2 K-steps count the stores as younger
// operations (so they do not wait for them); the next one waits for them.
// With ATR, A is given
// as A^T in the tiled layout (G for dW) and read transposed, as in
// gemm_bf16_kernel.  A stage of A^T is 32 rows of one 256-row panel; with
// AFLAT (every byte of A^T a stage can reach lies within 4 GB of the tile's
// first block column) one descriptor per tile serves all panels and a stage's
// panel and row offset is a 32-bit scalar offset, else the descriptor is
// rebuilt at each stage (64-bit address arithmetic: about 12 scalar
// instructions per K-step).  Requires K / BF_BK >= DW_ST stages and one split.
template <class Epi, bool ATR, int MB, bool EVEN_NK, bool AFLAT>
__global__ void __launch_bounds__(BF_NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_bf16_persist_t(const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ B,
                    int64_t ldb, [[maybe_unused]] int64_t M, [[maybe_unused]] int64_t N,
                    int64_t K, int tiles_m, int tiles_n, Epi epi) {
  constexpr int NST = Epi::STORES;
  static_assert((DW_ST - 2) * BT_LPS + NST < 64, "stage waits must fit vmcnt");
  __shared__ __attribute__((aligned(1024))) char lds[DW_ST * BF_STAGE];
  const int total = tiles_m * tiles_n;
  const int per_xcd = gridDim.x >> 3;  // the grid is a multiple of 8
  const int chunk = (int)ceil_div(total, 8);
  const int lo = (blockIdx.x & 7) * chunk, hi = min(total, lo + chunk);
  int t = lo + (blockIdx.x >> 3);
  if (t >= hi) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  // Wave tiles of 16 MB x 16 NB (MB row blocks, NB column blocks of 16): 8 x 4
  // blocks as 2 x 4 waves, or 4 x 8 blocks as 4 x 2 waves.
  constexpr int NB = 32 / MB, WN = 16 / NB;
  static_assert(MB == 8 || MB == 4, "wave layouts 2 x 4 and 4 x 2");
  const int wm = wave / WN, wn = wave % WN;
  const int nk = (int)ceil_div(K, BF_BK);
  // Blocks of 4 x 8 tiles (M x N), N fastest inside a block.
  auto coords = [&](int lt, int64_t& m0, int64_t& n0) {
    constexpr int BMT = 4, BNT = 8;
    const int band = lt / (BMT * tiles_n);
    const int first_m = band * BMT;
    const int hm = min(BMT, tiles_m - first_m);
    const int within = lt - band * BMT * tiles_n;
    const int blk = within / (hm * BNT);
    const int first_n = blk * BNT;
    const int wn_ = min(BNT, tiles_n - first_n);
    const int inb = within - blk * hm * BNT;
    m0 = (int64_t)(first_m + inb / wn_) * BF_BM;
    n0 = (int64_t)(first_n + inb % wn_) * BF_BN;
  };
  // Per tile: B's panel descriptor; A's first block column (ATR: its
  // descriptor spans every panel of A^T with AFLAT, else it is rebased at
  // every 256-row panel) or panel descriptor.
  struct Tile {
    int64_t m0, n0;
    i32x4 ra, rb;
    uint32_t a_bytes;
  };
  // ATR: bytes of one 256-row panel of A^T, and the blocks of a tile's
  // column range (8, fewer only at the right edge of A^T)
  const uint32_t lda_bytes = (uint32_t)(lda * TILE_BLOCK_BYTES);
  auto tile = [&](int lt) {
    Tile T;
    coords(lt, T.m0, T.n0);
    i32x4 rb = make_rsrc(B + (T.n0 / BF_BN) * ldb * (TILE_BLOCK_BYTES / 2),
                         (uint32_t)(nk * TILE_BLOCK_BYTES));
    const int64_t cols = min<int64_t>(BF_BM / TILE_K, lda - T.m0 / TILE_K);
    i32x4 ra = ATR && AFLAT
                   ? make_rsrc(A + (T.m0 / TILE_K) * (TILE_BLOCK_BYTES / 2),
                               (uint32_t)((ceil_div(nk, 8) - 1) * lda_bytes +
                                          cols * TILE_BLOCK_BYTES))
                   : make_rsrc(A + (T.m0 / BF_BM) * lda * (TILE_BLOCK_BYTES / 2),
                               (uint32_t)(nk * TILE_BLOCK_BYTES));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      T.rb[i] = __builtin_amdgcn_readfirstlane(rb[i]);
      T.ra[i] = __builtin_amdgcn_readfirstlane(ra[i]);
    }
    T.a_bytes = ATR ? (uint32_t)(cols * TILE_BLOCK_BYTES) : 0u;
    return T;
  };
  // Per-lane copy-slot and fragment offsets (tile independent), formed from
  // an opaque copy of the lane index before the first tile and after every
  // epilogue.
  struct LaneOffs {
    int oa, oa2, ob, fa, fb;  // oa2: the source of pieces 2, 3 less their 2 and 3 KB steps
    int ftr[2][2];
  };
  const bool copier = wave < BT_DMAW;
  auto lane_offs = [&]() {
    int l;
    __asm__ volatile("v_and_b32 %0, 63, %1" : "=v"(l) : "v"(tid));
    LaneOffs o;
    {
      const int q = wave * BT_PER;  // the copying wave's first piece (even)
      o.ob = (q * 64 + l) * 16;
      o.oa = ATR ? (q >> 1) * TILE_BLOCK_BYTES + (l >> 2) * 64 + (l & 3) * 16 : o.ob;
      o.oa2 = o.oa + (ATR ? atr_piece_step(2) - 2048 : 0);
    }
    const int ch = l >> 4;
    int row = wm * 16 * MB + (l & 15);
    o.fa = row * 64 + 16 * (ch ^ tile_swz(row));
    row = wn * 16 * NB + (l & 15);
    o.fb = BF_STAGE_A + row * 64 + 16 * (ch ^ tile_swz(row));
    const int g = l >> 4, j = l & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int r = 8 * g + 4 * sec + (j >> 2);
        const int c = 2 * h + ((j & 3) >> 1);
        o.ftr[h][sec] = r * 64 + ((c ^ tile_swz(r)) << 4) + 8 * (j & 1);
      }
    return o;
  };
  LaneOffs lof = lane_offs();
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  auto issue = [&](const Tile& T, int kt, int slot) {
    if (!copier) return;
    const uint32_t sa = lds_base + (uint32_t)(slot * BF_STAGE);
    const uint32_t sb = sa + BF_STAGE_A;
    i32x4 ra = T.ra;
    int abase = kt * TILE_BLOCK_BYTES;
    if constexpr (ATR && AFLAT) {
      // rows 32 (kt % 8) .. of the 256-row panel kt / 8 of A^T
      abase = (int)((uint32_t)(kt >> 3) * lda_bytes + (uint32_t)(kt & 7) * (TILE_ROWS / 8 * TILE_K * 2));
    } else if constexpr (ATR) {
      ra = make_rsrc(A + ((int64_t)(kt >> 3) * lda + T.m0 / TILE_K) * (TILE_BLOCK_BYTES / 2),
                     T.a_bytes);
      abase = (kt & 7) * (TILE_ROWS / 8 * TILE_K * 2);
    }
    // Four 1 KB pieces per operand and copying wave, each operand's under one
    // M0 write: A's pieces i sit at atr_piece_step(i) (two 2 KB runs 16 KB
    // apart with ATR), which the per-lane offsets oa (pieces 0, 1) and oa2
    // (pieces 2, 3) absorb less the loads' own 1 KB steps.
    static_assert(BT_PER == 4 && (!ATR || (atr_piece_step(1) == 1024 &&
                                           atr_piece_step(3) - atr_piece_step(2) == 1024)),
                  "piece layout");
    const uint32_t dst = (uint32_t)(wave * BT_PER * 1024);
    load_lds16_4v(ra, sa + dst, lof.oa, lof.oa, lof.oa2, lof.oa2, abase);
    load_lds16_x4(T.rb, sb + dst, lof.ob, kt * TILE_BLOCK_BYTES);
  };
  auto read_frags = [&](int slot, bf16x8 (&fa)[MB], bf16x8 (&fb)[NB]) {
    const char* sn = lds + slot * BF_STAGE;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if constexpr (ATR) {
        typedef short v4s __attribute__((ext_vector_type(4)));
        typedef v4s __attribute__((address_space(3))) * lds_v4s;
        // row block i of the wave is piece (wm MB + i) / 2 (32 rows each), half i & 1
        const char* pc = sn + ((MB / 2) * wm + (i >> 1)) * (BF_STAGE_A / 8);
        const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(pc + lof.ftr[i & 1][0]));
        const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(pc + lof.ftr[i & 1][1]));
        fa[i] = __builtin_bit_cast(bf16x8,
                                   __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        fa[i] = *reinterpret_cast<const bf16x8*>(sn + lof.fa + 1024 * i);
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(sn + lof.fb + 1024 * j);
  };
  Tile cur = tile(t);
  int tnext = t + per_xcd;
  bool has_next = tnext < hi;
  Tile nxt = cur;
  if (has_next) nxt = tile(tnext);
  bf16x8 ca[MB], cb[NB], da[MB], db[NB];  // two fragment sets, used in turn
  int gb = 0;  // ring position of the current tile's stage 0
#pragma unroll
  for (int s = 0; s < DW_ST - 1; ++s) issue(cur, s, s);
  if (copier) wait_stage<BT_LPS>(DW_ST - 2);
  __syncthreads();
  issue(cur, DW_ST - 1, DW_ST - 1);
  if constexpr (EVEN_NK) read_frags(0, da, db);
  else read_frags(0, ca, cb);
  bool stores_out = false;  // the previous tile's epilogue stores may be in flight
  // Ring slot of the current stage, (gb + kt) % DW_ST, carried from step to
  // step (a modulo by 5 per use cost about 15 scalar instructions per K-step).
  int sl = 0;
  for (;;) {
    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
    // Stage kt's MFMAs from x, with stage kt+1 awaited, the buffer of stage
    // kt refilled and stage kt+1's fragments read into y.
    // STEADY (a compile-time flag) marks the steps with kt >= DW_ST - 2 and
    // kt + DW_ST < nk: no previous stores are younger than stage kt + 1,
    // DW_ST - 2 stages are, and the refill is this tile's stage kt + DW_ST,
    // so the wait and the refill need no run-time choice (which otherwise
    // costs a cascade of scalar branches per step).
    auto kstep = [&](auto steady, int kt, bf16x8 (&xa)[MB], bf16x8 (&xb)[NB],
                     bf16x8 (&ya)[MB], bf16x8 (&yb)[NB]) {
      constexpr bool STEADY = decltype(steady)::value;
      // first half of the stage's MFMAs: blocks 0 .. 15 (block q = (q / NB, q % NB))
#pragma unroll
      for (int q = 0; q < BF_PRE; ++q)
        acc[q / NB][q % NB] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            xa[q / NB], xb[q % NB], acc[q / NB][q % NB], 0, 0, 0);
      // Await stage kt + 1.  Younger than it: up to DW_ST - 2 stages (fewer
      // at the end of the last tile), plus the previous epilogue's stores
      // when stage kt + 1 was issued before them (stages 0 .. DW_ST-2).
      if constexpr (STEADY) {
        if (copier) wait_vmcnt<(DW_ST - 2) * BT_LPS>();
      } else {
        if (copier)
          wait_stage<BT_LPS, NST>(has_next ? DW_ST - 2 : min(nk - 2 - kt, DW_ST - 2),
                                  stores_out && kt + 1 <= DW_ST - 2);
      }
      __syncthreads();
      const int slot = sl;  // stage kt's, refilled with stage kt + DW_ST
      int sn = sl + 1;      // stage kt + 1's
      sn = sn == DW_ST ? 0 : sn;
      if constexpr (STEADY) {
        issue(cur, kt + DW_ST, slot);
      } else {
        if (kt + DW_ST < nk) issue(cur, kt + DW_ST, slot);
        else if (has_next) issue(nxt, kt + DW_ST - nk, slot);
      }
      read_frags(sn, ya, yb);
      sl = sn;
#pragma unroll
      for (int q = BF_PRE; q < 32; ++q)
        acc[q / NB][q % NB] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            xa[q / NB], xb[q % NB], acc[q / NB][q % NB], 0, 0, 0);
      // One fragment read of the next stage per MFMA after the barrier (16
      // reads with MB = 4: 8 transposing, 8 plain): 8.61 -> 8.20 ms on the
      // 16k step against all reads first, and all reads first timed the
      // same as the compiler's order.  The next step's MFMAs, which need
      // those fragments (and, where the two halves of a transposing read did
      // not land in adjacent registers, the moves that join them), stay
      // below this part.
      reads_between_mfmas<(ATR ? 2 * MB : MB) + NB, 32 - BF_PRE>();
      __builtin_amdgcn_sched_barrier(0);
    };
    // With an even stage count one step runs before the pairs, so the last
    // stage always ends up in ca/cb (the parity is fixed per launch).  With
    // an even count (the default chunk) the pairs run in three loops: the
    // first steps (previous stores may be younger), the steady middle, the
    // last steps (the refill switches to the next tile, and at the end of the
    // last tile fewer stages follow).  An odd count takes the general steps
    // throughout (the split made the compiler spill in that variant).
    const std::false_type gen;
    const std::true_type std_;
    int kt = 0;
    if constexpr (EVEN_NK) {
      kstep(gen, 0, da, db, ca, cb);
      kt = 1;
      for (; kt < DW_ST - 2 && kt + 2 < nk; kt += 2) {
        kstep(gen, kt, ca, cb, da, db);
        kstep(gen, kt + 1, da, db, ca, cb);
      }
      for (; kt + 1 + DW_ST < nk; kt += 2) {
        kstep(std_, kt, ca, cb, da, db);
        kstep(std_, kt + 1, da, db, ca, cb);
      }
    }
    for (; kt + 2 < nk; kt += 2) {
      kstep(gen, kt, ca, cb, da, db);
      kstep(gen, kt + 1, da, db, ca, cb);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[i], cb[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) __asm__ volatile("" : "+a"(acc[i][j]));
    int elane;
    __asm__ volatile("v_and_b32 %0, 63, %1" : "=v"(elane) : "v"(tid));
    EpiCtx ctx;
    ctx.m0 = cur.m0;
    ctx.n0 = cur.n0;
    ctx.wm_off = wm * 16 * MB;
    ctx.wn_off = wn * 16 * NB;
    ctx.wave_m = wm;
    ctx.lane = elane;
    ctx.split = 0;
    ctx.smem = nullptr;  // the ring is in use by the next tile's stages
    ctx.smem_bytes = 0;
    epi.template apply<Acc16, MB, NB, BF_BM, BF_BN>(acc, ctx);
    if (!has_next) break;
    // Advance: stages 0 .. DW_ST-2 of the next tile were issued before the
    // epilogue's stores; await stage 0 (younger: the other stages and the
    // stores), then issue stage DW_ST-1.
    gb += nk;
    sl = gb % DW_ST;
    cur = nxt;
    tnext += per_xcd;
    has_next = tnext < hi;
    if (has_next) nxt = tile(tnext);
    lof = lane_offs();
    if (copier) wait_stage<BT_LPS, NST>(DW_ST - 2, true);
    __syncthreads();
    issue(cur, DW_ST - 1, (gb + DW_ST - 1) % DW_ST);
    if constexpr (EVEN_NK) read_frags(gb % DW_ST, da, db);
    else read_frags(gb % DW_ST, ca, cb);
    stores_out = true;
  }
}

// ------------------------------------------------------------ fp32 kernel ---

constexpr int F_BM = 128, F_BN = 128, F_BK = 16;

template <class Epi>
__global__ void __launch_bounds__(NT) gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                      const float* __restrict__ B, int64_t ldb,
                                                      int64_t M, int64_t N, int64_t K,
                                                      int64_t k_split, int tiles_m, int tiles_n,
                                                      int splits, Epi epi) {
  constexpr int VEC = 4, LD = F_BK + VEC;
  constexpr int MB = 2, NB = 2, KV = F_BK / VEC;
  constexpr int A_IT = F_BM * KV / NT, B_IT = F_BN * KV / NT;
  __shared__ __attribute__((aligned(16))) float As[2][F_BM * LD];
  __shared__ __attribute__((aligned(16))) float Bs[2][F_BN * LD];
  __shared__ __attribute__((aligned(16))) char scratch[6 * F_BN * 4];
  const TileCoord tc = map_tile(tiles_m, tiles_n, splits, F_BM, F_BN);
  if (!tc.valid) return;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t kb = (int64_t)tc.split * k_split;
  const int64_t ke = min(K, kb + k_split);
  const int nk = (int)ceil_div(max<int64_t>(ke - kb, 0), F_BK);
  u32x4 ra[A_IT], rb[B_IT];
  auto gload = [&](int kt) {
    const int64_t k0 = kb + (int64_t)kt * F_BK;
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
      *reinterpret_cast<u32x4*>(&As[buf][(q / KV) * LD + (q % KV) * VEC]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      const int q = tid + NT * i;
      *reinterpret_cast<u32x4*>(&Bs[buf][(q / KV) * LD + (q % KV) * VEC]) = rb[i];
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
    for (int kk = 0; kk < F_BK; kk += 2) {
      float a[MB], b[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        a[i] = As[buf][(wm * 64 + 32 * i + (lane & 31)) * LD + kk + (lane >> 5)];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        b[j] = Bs[buf][(wn * 64 + 32 * j + (lane & 31)) * LD + kk + (lane >> 5)];
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }
  EpiCtx ctx;
  ctx.m0 = tc.m0;
  ctx.n0 = tc.n0;
  ctx.wm_off = wm * 64;
  ctx.wn_off = wn * 64;
  ctx.wave_m = wm;
  ctx.lane = lane;
  ctx.split = tc.split;
  ctx.smem = scratch;
  ctx.smem_bytes = sizeof(scratch);
  epi.template apply<Acc32, MB, NB, F_BM, F_BN>(acc, ctx);
}

template <bool TILED, class Epi, bool ATR = false>
hipError_t launch_bf16(const bf16_t* A, int64_t lda, const bf16_t* B, int64_t ldb, int64_t M,
                       int64_t N, int64_t K, int splits, int64_t k_split, const Epi& epi,
                       hipStream_t s) {
  const int64_t tm = ceil_div(M, BF_BM), tn = ceil_div(N, BF_BN);
  const int64_t total = tm * tn * splits;
  if (total <= 0) return hipSuccess;
  if (total > (int64_t)1 << 30) return hipErrorInvalidValue;
  // Buffer offsets are 32-bit: a tile's operand panel must stay below 2 GiB.
  const int64_t panel = TILED ? ceil_div(k_split, BF_BK) * TILE_BLOCK_BYTES
                              : (int64_t)BF_BM * std::max(lda, ldb) * 2;
  if (panel >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (ATR && (splits > 1 || ceil_div(M, TILE_K) > lda)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<TILED, Epi, ATR>), dim3((unsigned)round_up(total, 8)),
                     dim3(BF_NT), 0, s, A, lda, B, ldb, M, N, K, k_split, (int)tm, (int)tn, splits,
                     epi);
  return hipGetLastError();
}

// Compute units of the current device (cached per device; calls from
// several threads may query concurrently and store the same value).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Row-major operands (K = lda = ldb columns), one split: the
// one-tile-per-workgroup kernel.  The bf16 forward comes here only when H
// has fewer K blocks than the persistent kernel's ring (it reads tiled
// copies otherwise).
template <class Epi>
hipError_t launch_bf16_rows(const bf16_t* A, int64_t lda, const bf16_t* B, int64_t ldb,
                            int64_t M, int64_t N, int64_t K, const Epi& epi, hipStream_t s) {
  return launch_bf16<false>(A, lda, B, ldb, M, N, K, 1, round_up(K, BF_BK), epi, s);
}

// Both operands in the tiled block layout (kb = blocks per 256-row panel,
// at least ceil(K / BF_BK)): the persistent kernel, which needs at least
// BF_ST stages and the device's CU count; returns hipErrorNotSupported
// otherwise (the caller then takes the row-major operands).
template <class Epi>
hipError_t launch_bf16_tiled_persist(const bf16_t* A, const bf16_t* B, int64_t kb, int64_t M,
                                     int64_t N, int64_t K, const Epi& epi, hipStream_t s) {
  const int64_t tm = ceil_div(M, BF_BM), tn = ceil_div(N, BF_BN);
  const int64_t total = tm * tn;
  const int64_t nk = ceil_div(K, BF_BK);
  const int cus = cu_count() / 8 * 8;
  if (total <= 0) return hipSuccess;
  if (nk < BF_ST || kb < nk || cus <= 0 || total > (int64_t)1 << 30) return hipErrorNotSupported;
  if (nk * TILE_BLOCK_BYTES >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int64_t grid = std::min<int64_t>(round_up(total, 8), cus);
  if (nk % 2 == 0)
    hipLaunchKernelGGL((gemm_bf16_persist<Epi, true>), dim3((unsigned)grid), dim3(BF_NT), 0, s,
                       A, kb, B, kb, M, N, K, (int)tm, (int)tn, epi);
  else
    hipLaunchKernelGGL((gemm_bf16_persist<Epi, false>), dim3((unsigned)grid), dim3(BF_NT), 0, s,
                       A, kb, B, kb, M, N, K, (int)tm, (int)tn, epi);
  return hipGetLastError();
}

template <class Epi>
hipError_t launch_f32(const float* A, int64_t lda, const float* B, int64_t ldb, int64_t M,
                      int64_t N, int64_t K, int splits, int64_t k_split, const Epi& epi,
                      hipStream_t s) {
  const int64_t tm = ceil_div(M, F_BM), tn = ceil_div(N, F_BN);
  const int64_t total = tm * tn * splits;
  if (total <= 0) return hipSuccess;
  if (total > (int64_t)1 << 30) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_f32_kernel<Epi>), dim3((unsigned)round_up(total, 8)), dim3(NT), 0, s,
                     A, lda, B, ldb, M, N, K, k_split, (int)tm, (int)tn, splits, epi);
  return hipGetLastError();
}

}  // namespace

int gemm_k_tile(int dtype) { return dtype == RL_DTYPE_BF16 ? BF_BK : F_BK; }
int fwd_vtile(int dtype) { return dtype == RL_DTYPE_BF16 ? BF_BM : F_BM; }

bool gemm_fwd_tiled_ok(int64_t H) { return ceil_div(H, BF_BK) >= BF_ST; }

hipError_t gemm_fwd(int dtype, const void* W, const void* hc, int64_t V, int64_t Tc, int64_t H,
                    const FwdEpiArgs& a, hipStream_t s, const void* Wf, const void* hf,
                    int64_t kbf) {
  // Full tiles, then the edge row of tiles (if V is not a multiple of the
  // tile height) in a launch of its own.  With tiled copies of W and h_c
  // (Wf, hf: kbf blocks per panel) the persistent kernel reads those.
  auto run = [&](auto tag_t, auto store) -> hipError_t {
    using T = decltype(tag_t);
    constexpr bool STORE = decltype(store)::value;
    const int BM = sizeof(T) == 2 ? BF_BM : F_BM;
    const int64_t Vfull = V / BM * BM;
    const T* Wt = static_cast<const T*>(W);
    auto launch = [&](auto epi, int64_t m0, int64_t M) -> hipError_t {
      if constexpr (sizeof(T) == 2) {
        if (Wf != nullptr && hf != nullptr) {
          const hipError_t e = launch_bf16_tiled_persist(
              static_cast<const bf16_t*>(Wf) + (m0 / BF_BM) * kbf * (TILE_BLOCK_BYTES / 2),
              static_cast<const bf16_t*>(hf), kbf, M, Tc, H, epi, s);
          if (e != hipErrorNotSupported) return e;
        }
        return launch_bf16_rows(Wt + m0 * H, H, static_cast<const bf16_t*>(hc), H, M, Tc, H,
                                epi, s);
      } else {
        return launch_f32(Wt + m0 * H, H, static_cast<const float*>(hc), H, M, Tc, H, 1,
                          round_up(H, F_BK), epi, s);
      }
    };
    if (Vfull > 0) {
      FwdEpi<T, true, STORE> e{a.inv_t, a.V, a.Tc, a.J, a.part_m, a.part_s, a.part_t,
                               static_cast<T*>(a.P), a.ldp, 0};
      const hipError_t err = launch(e, 0, Vfull);
      if (err != hipSuccess) return err;
    }
    if (V > Vfull) {
      FwdEpi<T, false, STORE> e{a.inv_t, a.V, a.Tc, a.J, a.part_m, a.part_s, a.part_t,
                                static_cast<T*>(a.P), a.ldp, Vfull};
      return launch(e, Vfull, V - Vfull);
    }
    return hipSuccess;
  };
  if (dtype == RL_DTYPE_BF16)
    return a.P ? run(bf16_t{}, std::true_type{}) : run(bf16_t{}, std::false_type{});
  return a.P ? run(float{}, std::true_type{}) : run(float{}, std::false_type{});
}

hipError_t gemm_store(int dtype, const void* A, int64_t lda, const void* B, int64_t ldb,
                      int64_t M, int64_t N, int64_t K, int splits, int64_t k_split, float* C,
                      int64_t ldc, int64_t split_stride, hipStream_t s) {
  if (ldc >= ((int64_t)1 << 21)) return hipErrorInvalidValue;
  StoreEpi e{C, ldc, split_stride, M, N};
  if (dtype == RL_DTYPE_BF16)  // tiled operands
    return launch_bf16<true>(static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(B),
                             ldb, M, N, K, splits, k_split, e, s);
  return launch_f32(static_cast<const float*>(A), lda, static_cast<const float*>(B), ldb, M, N, K,
                    splits, k_split, e, s);
}

hipError_t gemm_dw(int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M,
                   int64_t N, int64_t K, float* C, int64_t ldc, int accumulate, hipStream_t s) {
  if (ldc >= ((int64_t)1 << 21)) return hipErrorInvalidValue;
  const int bk = gemm_k_tile(dtype);
  // bf16: the persistent kernel (epilogue stores overlapped with the next
  // tile) when the K loop has at least DW_ST stages and the CU count is known.
  if (dtype == RL_DTYPE_BF16 && ceil_div(K, BF_BK) >= DW_ST && N % 4 == 0) {
    const int64_t tm = ceil_div(M, BF_BM), tn = ceil_div(N, BF_BN);
    const int64_t total = tm * tn;
    const int cus = cu_count() / 8 * 8;
    if (total <= 0) return hipSuccess;
    if (cus > 0 && total <= ((int64_t)1 << 30)) {
      if (ceil_div(M, TILE_K) > lda) return hipErrorInvalidValue;
      if (ceil_div(K, BF_BK) * TILE_BLOCK_BYTES >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
      const int64_t grid = std::min<int64_t>(round_up(total, 8), cus);
      // one descriptor per tile when the stages' reach into G (the last
      // panel's 8 block columns included) stays below 4 GB
      const int64_t nk = ceil_div(K, BF_BK);
      const bool flat = (ceil_div(nk, 8) - 1) * lda * TILE_BLOCK_BYTES +
                            (BF_BM / TILE_K) * TILE_BLOCK_BYTES <= (int64_t)UINT32_MAX;
      auto go = [&](auto e) {
        auto launch = [&](auto even, auto aflat) {
          hipLaunchKernelGGL((gemm_bf16_persist_t<decltype(e), true, DW_MB, decltype(even)::value,
                                                  decltype(aflat)::value>),
                             dim3((unsigned)grid), dim3(BF_NT), 0, s,
                             static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(B),
                             ldb, M, N, K, (int)tm, (int)tn, e);
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        if (nk % 2 == 0)
          flat ? launch(T_{}, T_{}) : launch(T_{}, F_{});
        else
          flat ? launch(F_{}, T_{}) : launch(F_{}, F_{});
        return hipGetLastError();
      };
      return accumulate ? go(DwEpiT<true>{C, ldc, M, N}) : go(DwEpiT<false>{C, ldc, M, N});
    }
  }
  auto run = [&](auto e) {
    if (dtype == RL_DTYPE_BF16)  // tiled operands, A given as G (transposed reads)
      return launch_bf16<true, decltype(e), true>(static_cast<const bf16_t*>(A), lda,
                                                  static_cast<const bf16_t*>(B), ldb, M, N, K, 1,
                                                  round_up(K, bk), e, s);
    return launch_f32(static_cast<const float*>(A), lda, static_cast<const float*>(B), ldb, M, N,
                      K, 1, round_up(K, bk), e, s);
  };
  return accumulate ? run(DwEpi<true>{C, ldc, M, N}) : run(DwEpi<false>{C, ldc, M, N});
}

}  // namespace rl
