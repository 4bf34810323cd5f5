// Launchers of the device kernels (internal to librlloss).
#pragma once

#include "common.h"

namespace rl {

// Forward GEMM tile extent along the vocabulary for a dtype: the
// online-softmax partials are kept per (token, block of that many rows).
int fwd_vtile(int dtype);

struct FwdEpiArgs {
  float inv_t;
  int64_t V, Tc, J;      // vocabulary, tokens in the chunk, vocab tiles
  float* part_m;         // [Tc, J] tile max of z
  float* part_s;         // [Tc, J] sum exp(z - m)
  float* part_t;         // [Tc, J] sum exp(z - m) (z - m)
  void* P;               // exp(z - m) per element, or null: bf16 into G's tiled layout
                         // (ldp = blocks per 256-token panel), fp32 token-major [Tc, ldp]
  int64_t ldp;
};

// S^T = W h_c^T with the online-softmax epilogue.  W [V,H], h_c [Tc,H].
// Wf, hf (bf16, optional): the same operands in the tiled block layout,
// kbf >= ceil(H / 32) blocks per 256-row panel (Wf's panels covering V, hf's
// Tc), which the persistent kernel reads instead when it applies.
hipError_t gemm_fwd(int dtype, const void* W, const void* hc, int64_t V, int64_t Tc, int64_t H,
                    const FwdEpiArgs& a, hipStream_t s, const void* Wf = nullptr,
                    const void* hf = nullptr, int64_t kbf = 0);
// Whether the bf16 forward can read tiled operands at this H (it needs at
// least as many K stages as its LDS ring holds).
bool gemm_fwd_tiled_ok(int64_t H);

// C[split] = A[:, ks] B[:, ks]^T (fp32 out), split-K over K in `splits` slices
// of k_split elements (a multiple of the K tile).  A [M,K] lda, B [N,K] ldb.
hipError_t gemm_store(int dtype, const void* A, int64_t lda, const void* B, int64_t ldb,
                      int64_t M, int64_t N, int64_t K, int splits, int64_t k_split, float* C,
                      int64_t ldc, int64_t split_stride, hipStream_t s);

// dW (=|+=) A B^T in fp32.  bf16: A is given as A^T = G [K rows, M cols] in
// the tiled layout (lda = its blocks per 256-row panel) and read transposed;
// B^T tiled.  fp32: A and B row-major.
hipError_t gemm_dw(int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M,
                   int64_t N, int64_t K, float* C, int64_t ldc, int accumulate, hipStream_t s);

int gemm_k_tile(int dtype);

// Tiled block layout of a bf16 operand [R rows, K columns] (the backward
// GEMM operands): 256 x 32 blocks of 16 KB, block (rb, kb) at index
// rb * KB + kb (KB = blocks per 256-row panel); inside a block row r holds
// four 16-byte chunks, logical chunk c stored at position c ^ tile_swz(r).
// Rows >= R and columns >= K of a block are zero.  The same swizzle is the
// LDS image of a GEMM stage.  It keeps both fragment reads of the GEMMs free
// of LDS bank conflicts (measured with SQ_LDS_BANK_CONFLICT): ds_read_b128 of
// one chunk of 16 consecutive rows, and ds_read_b64_tr_b16 of two chunks of
// rows {8g + i, 8g + 4 + i} (g, i < 4), which needs rows r and r + 8 to use
// disjoint chunk pairs.
constexpr int TILE_ROWS = 256, TILE_K = 32, TILE_BLOCK_BYTES = TILE_ROWS * TILE_K * 2;
__host__ __device__ inline int tile_swz(int64_t r) {
  return (int)(((r >> 1) & 3) ^ (((r >> 3) & 1) * 3));
}
__host__ __device__ inline int64_t tiled_offset(int64_t r, int64_t k, int64_t KB) {
  return ((r / TILE_ROWS) * KB + k / TILE_K) * (TILE_ROWS * TILE_K) + (r % TILE_ROWS) * TILE_K +
         ((((k % TILE_K) >> 3) ^ tile_swz(r % TILE_ROWS)) << 3) + (k & 7);
}

// src [S rows, C cols] row-major (ld_src) -> tiled [C rows, S cols] with KB
// blocks per panel (dst; the blocks kb < min(kb_write, KB) of every panel are
// written, zeros past S and C) and, when dst2 is given, the untransposed
// tiled copy [S rows, C cols] with KB2 >= ceil(C / 32) blocks per panel (its
// rows below 32 kb_write, zeros past S and C).  Either output may be null.
hipError_t to_tiled_t(const bf16_t* src, int64_t ld_src, int64_t S, int64_t C, bf16_t* dst,
                      int64_t KB, int64_t kb_write, hipStream_t s, bf16_t* dst2 = nullptr,
                      int64_t KB2 = 0);

// bf16 dense gradient in the tiled layout: G holds e^(z - m) as left by the
// forward GEMM (KB_g blocks per 256-token panel, panels covering Tc); every
// element becomes kappa_t e^(m_tj - LSE_t) e^(z - m_tj) (with the entropy
// bonus as in form_g below), zero past Tc and V, in place.
hipError_t form_g_blocks(bf16_t* G, int64_t KB_g, const float* part_m, int64_t J, int vtile,
                         const float* lse_c, const float* kappa_c, float gs, int64_t V,
                         int64_t Tc, hipStream_t s);

// dst[c][r] = src[r][c] for r < R, 0 for R <= r < Rpad; c < C.
hipError_t transpose_pad(int dtype, const void* src, int64_t ld_src, int64_t R, int64_t C,
                         void* dst, int64_t Rpad, hipStream_t s);

struct CombineArgs {
  // inputs
  const void* h;  // [N,H] full batch
  const void* W;  // [V,H]
  const int32_t* labels;
  const float* infer_lp;
  const float* adv;
  const int64_t* off;  // device offsets [N+1] or null
  const int32_t* ids;
  const float* u;
  const float* logq;  // may be null
  const float *part_m, *part_s, *part_t;  // [Tc, J]
  int64_t t0, Tc, N, H, V, J, nnz;
  WeightParams wp;
  float adv_tau, beta, inv_t, inv_D;
  const float* zent;   // [N + nnz] label then support logits (before 1/tau), or null:
                       // then combine forms them as dot products itself
  const int32_t* age;  // [N] policy age or null (all 0)
  int staleness;       // rl_kl_staleness: beta_t = beta / sqrt(1 + age_t) when inv_sqrt
  float gamma;         // entropy bonus coefficient
  // outputs (global token index)
  float* lse;         // [N]
  float* kappa_s;     // [N] (kappa_t + gamma (H_t - lse_t)) * inv_t / D
  float* stats;       // [N, 8] per-token reduction inputs
  float* coef;        // [N + nnz] gradient coefficient of label / entry (times inv_t / D)
  float* o_logprobs;  // nullable
  float* o_entropy;
  float* o_weight;
  uint8_t* o_keep;
  float* o_token_loss;
  float* o_support_lp;  // [nnz] nullable
};
constexpr int STAT_LOSS = 0, STAT_MASKED = 1, STAT_SMASS = 2, STAT_HAS_SUPPORT = 3,
              STAT_TVFAIL = 4, STAT_KL = 5, STAT_ABS_KAPPA = 6, STAT_ENTROPY = 7, STAT_BETA = 8,
              STAT_KL_AGE0 = 9, STAT_AGE0 = 10, STAT_N = 11;
hipError_t combine(int dtype, const CombineArgs& a, hipStream_t s);

// z[e] = h[token(e)] . W[id(e)] for the N + nnz gradient entries (labels
// first, then support entries; token(e) = e for labels, row_of[e - N] after),
// computed in the vocabulary-sorted order (skeys / perm of csc_build).  h is
// the whole batch [N, H].  NaN for an id outside [0, V).
hipError_t entry_logits(int dtype, const void* h, const void* W, int64_t H, int64_t V,
                        const int32_t* skeys, const int32_t* perm, const int32_t* row_of,
                        int64_t N, int64_t E, float* z, hipStream_t s);

// G (in place over P, if write_g) and Gt from P = exp(z - m_tile):
// g[t, v] = exp(m - lse[t]) * P[t, v] * (kappa_s[t] + gs * (m + log P[t, v])),
// m = m[t, v / vtile], gs = gamma inv_t / D (the entropy-bonus term; 0 = off).
// ldp must be a multiple of 128; Gt columns up to Tck (multiple of 64).
hipError_t form_g(int dtype, void* P, int64_t ldp, void* Gt, int64_t ldgt, const float* part_m,
                  int64_t J, int vtile, const float* lse_c, const float* kappa_c, float gs,
                  int64_t V, int64_t Tc, int64_t Tck, int write_g, hipStream_t s);

// dh[t] = sum_s part[s][t] + sum over label/entries of coef * W[v] ; grad dtype.
hipError_t finalize_dh(int dtype, int grad_dtype, const float* part, int splits,
                       int64_t split_stride, const void* W, const int32_t* labels,
                       const int64_t* off, const int32_t* ids, const float* coef, int64_t t0,
                       int64_t Tc, int64_t N, int64_t nnz, int64_t V, int64_t H,
                       int with_sparse, void* dh, hipStream_t s);

// The label and support coefficients of the chunk's tokens added into the
// dense operand (G, when write_g, and Gt, when non-null; tiled layouts with
// ldg = KB_g, ldgt = KB_gt, else row-major strides): labels one per token,
// then support entries from the vocabulary-sorted list (skeys / perm of
// csc_build), a token's repeated ids summed in entry order.
hipError_t fold_sparse(int dtype, void* G, int write_g, void* Gt, int tiled, int64_t ldg,
                       int64_t ldgt, const int32_t* labels, const int32_t* skeys,
                       const int32_t* perm, const int32_t* row_of, const float* coef, int64_t N,
                       int64_t nnz, int64_t t0, int64_t Tc, int64_t V, hipStream_t s);

hipError_t reduce_final(const float* stats, int64_t N, float inv_D, float beta, float* loss,
                        float* metrics, hipStream_t s);

// CSR entry -> row index.
hipError_t csr_rows(const int64_t* off, int64_t N, int64_t nnz, int32_t* row_of, hipStream_t s);

// Vocab-major bucketing of the N + nnz gradient entries (labels first, then
// support entries), stable in entry order.  Writes start[V+2] (bucket V holds
// out-of-range ids) and the sorted entry permutation.
struct CscWork {
  int32_t *keys_a, *keys_b, *idx_a, *idx_b, *hist, *start;
  int64_t hist_len;
};
int64_t csc_hist_len(int64_t E);
hipError_t csc_build(const int32_t* labels, const int32_t* ids, int64_t N, int64_t nnz,
                     int64_t V, const CscWork& w, const int32_t** perm_out,
                     const int32_t** keys_out, hipStream_t s);

// dW[v] (=|+=) sum over entries in bucket v of coef * h[tok].
hipError_t sparse_dw(int dtype, const void* h, int64_t H, int64_t N, int64_t V,
                     const int32_t* start, const int32_t* perm, const int32_t* row_of,
                     const float* coef, float* dW, int overwrite, hipStream_t s);

// Loss-only replay.
int64_t elem_num_blocks(int64_t N);
hipError_t elementwise(const float* lp, const float* lq, const float* adv, int64_t N,
                       const rl_elem_cfg& c, uint16_t* word, float* w_primary, double* partials,
                       double* sums, hipStream_t s);
// partials: the main pass's per-block raw totals; n_eps selects their layout.
hipError_t elementwise_final(const double* partials, int64_t N, int n_eps, double* sums,
                             hipStream_t s);
// The library-owned partials of the allocation-free entry point on the
// current device (its address looked up at the first call there), and their
// size, enough for the largest grid.
hipError_t elem_noalloc_scratch(double** partials);
int64_t elem_noalloc_scratch_bytes();

// Sequence-aware rollout correction over a replay (four launches in order:
// stage 0 chunk totals, 1 sequences, 2 tokens, 3 raw totals and metrics).
// Workspace offsets in bytes from the workspace base; N tokens, S sequences.
struct MisLayout {
  int64_t nch, nb1, nb2, nb3;
  int64_t ct, firstseq, bitmap, seq_w, seq_flags, part1, part2, part3, bytes;
};
MisLayout mis_layout(int64_t N, int64_t S);
hipError_t mis_stage(int stage, const float* lp, const float* lq, const float* adv, int64_t N,
                     const int64_t* off_dev, int64_t S, const rl_mis_cfg& c, float* weight,
                     uint8_t* flags, double* metrics, void* ws, hipStream_t s);

// Validation.
hipError_t validate(int64_t N, int64_t V, int64_t nnz, const int32_t* labels,
                    const float* infer_lp, const float* adv, const int64_t* off,
                    const int32_t* ids, const float* u, const float* logq, int replayed,
                    int32_t* flags, hipStream_t s);

}  // namespace rl
