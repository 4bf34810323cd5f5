/*
 * rlloss.h -- C ABI of the fused LM-head + RL policy loss library (gfx950).
 *
 * The method (prime-rl pull request 4233, PR description):
 *   z_t     = W h_t / tau                        (LM head, vocabulary V)
 *   log p_t = log_softmax(z_t)                   (full vocabulary)
 *   loss_t  = -adv_tau * A_t * ( w(a_t) * log p_t(a_t)
 *                                - sum_e sg[u_e * w_e] * log p_t(v_e) )
 *             + beta_t * KL(q || p) - entropy_coeff * H_t
 *   L       = sum_t loss_t / D
 * with w the importance weight of the loss type ("What changes": ipo
 * 1(|p-q| <= eps) * min(p/q, max_importance_ratio); icepop
 * 1(low <= p/q <= high) * p/q; reinforce 1), e = (v_e, u_e) the entries of a
 * ragged per-token support in CSR form (int32 ids, host int64 offsets:
 * "TokenSupport" bullet), and KL(q || p) = sum_e u_e (log q(v_e) - log p(v_e))
 * over the same support (KL bullet; exact estimator on a replayed support
 * with u = q, k1 on sampler draws with u = 1/K).  Importance weights are
 * held constant in the gradient.  beta_t = kl_coeff, divided by
 * sqrt(1 + age_t) under the inv_sqrt KL staleness with a per-token policy
 * age (KL bullet).  H_t is the entropy of the training softmax; the entropy
 * bonus follows the Tencent article on KL/clip/entropy, section 3 (policy
 * loss minus entropy_coeff times the entropy).
 *
 * Conventions for every entry point:
 *  - Array arguments are device pointers unless the name ends in _host.
 *  - The caller owns every buffer.  The library allocates no device memory:
 *    temporary storage comes from the caller's workspace.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    All device work is enqueued asynchronously on it; the call returns
 *    without synchronising (except rl_validate_support_sync).
 *  - Argument, configuration and CSR-structure errors are detected on the
 *    host and returned before anything is enqueued.  Malformed data that only
 *    the device can see (ids out of range, non-finite values) is reported by
 *    rl_validate_support, not by the compute calls.
 *  - Row-major layouts throughout; bf16 values are stored as raw 16-bit
 *    words (IEEE bfloat16).
 *  - Results are deterministic: the same inputs and configuration on the same
 *    device give bitwise identical outputs (no floating-point atomics).
 */
#ifndef RLLOSS_H
#define RLLOSS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* rl_status travels as a 32-bit int across the ABI; in C++ it is given that
 * underlying type, so any int a caller passes (e.g. to rl_status_string) is a
 * valid value of the type. */
#ifdef __cplusplus
#define RL_STATUS_BASE : int32_t
#else
#define RL_STATUS_BASE
#endif
typedef enum rl_status RL_STATUS_BASE {
  RL_OK = 0,
  RL_E_ARG = 1,           /* null pointer, bad size or dtype, size overflow */
  RL_E_CFG = 2,           /* inconsistent or out-of-range configuration     */
  RL_E_CSR = 3,           /* host offsets are not a valid CSR               */
  RL_E_WORKSPACE = 4,     /* workspace missing or smaller than required     */
  RL_E_HIP = 5,           /* a HIP runtime call or kernel launch failed     */
  RL_E_INVALID_INPUT = 6  /* rl_validate_support_sync found bad data        */
} rl_status;

typedef enum rl_dtype { RL_DTYPE_FP32 = 0, RL_DTYPE_BF16 = 1 } rl_dtype;

typedef enum rl_loss_type {
  RL_LOSS_IPO = 0,       /* w = 1(|p-q| <= ipo_eps) * min(p/q, max_ratio) */
  RL_LOSS_ICEPOP = 1,    /* w = 1(icepop_lo <= p/q <= icepop_hi) * p/q    */
  RL_LOSS_REINFORCE = 2  /* w = 1                                         */
} rl_loss_type;

typedef enum rl_kl_estimator {
  RL_KL_NONE = 0,
  RL_KL_EXACT = 1,  /* replayed support, u = q: the KL is exact           */
  RL_KL_K1 = 2      /* sampler draws, u = 1/K: the k1 estimate            */
} rl_kl_estimator;

typedef enum rl_kl_staleness {
  RL_STALENESS_NONE = 0,     /* beta_t = kl_coeff                               */
  RL_STALENESS_INV_SQRT = 1  /* beta_t = kl_coeff / sqrt(1 + policy_age[t])     */
} rl_kl_staleness;

typedef enum rl_backward {
  RL_BWD_AUTO = 0,    /* SPARSE for reinforce without KL or entropy bonus on a
                         support, else DENSE                                      */
  RL_BWD_DENSE = 1,   /* full softmax backward through the LM head                */
  RL_BWD_SPARSE = 2,  /* gradient only on label + support entries (requires
                         reinforce, no KL, no entropy bonus, a support)            */
  RL_BWD_NONE = 3     /* forward only: no dh, no dW                                */
} rl_backward;

/* Indices into rl_loss_out.metrics (prime-rl PR 4233, "Metrics" bullet). */
enum {
  RL_METRIC_MASKED_FRACTION = 0, /* fraction of tokens whose label weight indicator is 0   */
  RL_METRIC_SUPPORT_MASS = 1,    /* mean over tokens with a support of sum_e u_e p/q      */
  RL_METRIC_MASK_TV = 2,         /* fraction of tokens with |p - q| > ipo_eps (label)     */
  RL_METRIC_KL = 3,              /* mean KL_t (0 without KL)                              */
  RL_METRIC_KL_BETA = 4,         /* mean beta_t (0 without KL)                            */
  RL_METRIC_MAX_ABS_KAPPA = 5,   /* max_t |kappa_t|, the net softmax coefficient          */
  RL_METRIC_ENTROPY_MEAN = 6,    /* mean entropy of the training softmax                  */
  RL_METRIC_KL_AGE0 = 7,         /* mean KL_t over tokens of policy age 0 (0 if none)     */
  RL_METRIC_COUNT = 8
};

typedef struct rl_loss_cfg {
  int64_t N;            /* tokens, >= 1                                         */
  int64_t H;            /* hidden size, >= 8 and a multiple of 8                */
  int64_t V;            /* vocabulary, 1 .. 2^31-1                              */
  int64_t nnz;          /* support entries (0 without a support)                */
  int64_t token_chunk;  /* tokens per pass through the head; 0 = default 8192   */
  int32_t dtype;        /* rl_dtype of h and W                                  */
  int32_t grad_dtype;   /* rl_dtype of dh (dW is always fp32)                   */
  int32_t loss_type;    /* rl_loss_type                                         */
  int32_t kl_estimator; /* rl_kl_estimator                                      */
  int32_t backward;     /* rl_backward                                          */
  int32_t replayed;     /* 1: the support is a replayed truncated set, u = q    */
  int32_t accumulate_dW;/* 1: dW += gradient, 0: dW = gradient                  */
  int32_t kl_staleness; /* rl_kl_staleness                                      */
  float ipo_eps;        /* IPO threshold on |p - q|, >= 0                       */
  float max_ratio;      /* IPO cap on p/q, > 0                                  */
  float icepop_lo;      /* IcePop band, 0 <= lo <= hi                           */
  float icepop_hi;
  float adv_tau;        /* advantage scale                                      */
  float kl_coeff;       /* beta, >= 0                                           */
  float inv_temperature;/* 1/tau, > 0                                           */
  float loss_norm;      /* D, > 0 (the caller passes e.g. the token count)      */
  float entropy_coeff;  /* entropy bonus gamma, finite (0 = off)                */
  int32_t reserved1;    /* must be 0                                            */
} rl_loss_cfg;

typedef struct rl_loss_out {
  float* loss;              /* [1]            required                          */
  float* token_loss;        /* [N]            nullable                          */
  float* logprobs;          /* [N]            nullable, log p_t(a_t)            */
  float* entropy;           /* [N]            nullable                          */
  float* weight;            /* [N]            nullable, w(a_t)                  */
  uint8_t* keep;            /* [N]            nullable, 1 = weight indicator on */
  float* support_logprobs;  /* [nnz]          nullable, log p_t(v_e)            */
  void* dh;                 /* [N,H]          nullable, grad_dtype              */
  float* dW;                /* [V,H] fp32     nullable                          */
  float* metrics;           /* [RL_METRIC_COUNT] nullable                       */
} rl_loss_out;

/*
 * rl_loss_workspace_size -- bytes of device workspace rl_loss_fwd_bwd needs
 * for `cfg` (with `has_support` = 1 when a CSR support will be passed and
 * `want_dh`/`want_dW` = 1 when those outputs will be non-null).
 * Errors: RL_E_ARG (null, bad sizes, overflow), RL_E_CFG.
 */
rl_status rl_loss_workspace_size(const rl_loss_cfg* cfg, int32_t has_support,
                                 int32_t want_dh, int32_t want_dW, size_t* bytes);

/*
 * rl_loss_fwd_bwd -- the fused LM head + RLLoss forward and backward.
 *
 *  h                 [N,H] dtype     hidden states
 *  W                 [V,H] dtype     head weights (nn.Linear [out,in] layout)
 *  labels            [N] int32       sampled token ids, in [0, V)
 *  infer_logprobs    [N] fp32        sampler log q(label), finite, <= 0
 *  adv               [N] fp32        advantages A_t
 *  policy_age        [N] int32       nullable: per-token policy age (engine
 *                                    weight-version lag) for the inv_sqrt KL
 *                                    staleness; NULL = every token has age 0;
 *                                    negative ages are read as 0
 *  csr_offsets_host  [N+1] int64     host; NULL = no support (then nnz = 0)
 *  csr_offsets_dev   [N+1] int64     device copy of the same offsets
 *  csr_ids           [nnz] int32     support ids in [0, V); repeats allowed
 *  csr_u             [nnz] fp32      estimator weights u_e >= 0
 *  csr_logq          [nnz] fp32      sampler log q(v_e); NULL = log(u_e)
 *  workspace         device, >= rl_loss_workspace_size() bytes, any contents
 *
 * Backward: dh = (dL/dz) W / tau, dW = (dL/dz)^T h / tau with
 *   dL/dz_t = (kappa_t p_t + gamma p_t (log p_t + H_t) - s_t w_t e_a
 *              + sum_e (s_t u_e w_e - beta_t u_e) e_{v_e}) / D,
 *   kappa_t = s_t (w_t - sum_e u_e w_e) + beta_t sum_e u_e,  s_t = adv_tau A_t,
 *   gamma = entropy_coeff.
 * The sparse backward drops the kappa_t p_t term (exact when kappa_t = 0,
 * e.g. reinforce without KL with sum_e u_e = 1 per row; the
 * RL_METRIC_MAX_ABS_KAPPA metric reports the dropped coefficient).
 * Errors: RL_E_ARG, RL_E_CFG, RL_E_CSR, RL_E_WORKSPACE, RL_E_HIP.
 */
rl_status rl_loss_fwd_bwd(const void* h, const void* W, const int32_t* labels,
                          const float* infer_logprobs, const float* adv,
                          const int32_t* policy_age, const int64_t* csr_offsets_host,
                          const int64_t* csr_offsets_dev,
                          const int32_t* csr_ids, const float* csr_u, const float* csr_logq,
                          const rl_loss_cfg* cfg, const rl_loss_out* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Loss-only mismatch replay over (log p_train, log q_infer, A) triples.
 * Sources: IPO documentation page ("Masking by Probability, Not Ratio");
 * Rollout Correction Methods page ("Bypassing PPO importance sampling",
 * "Decoupled, 3-policy PPO Importance Sampling", "Importance Sampling",
 * token level); the Tencent article on KL/clip/entropy, section 2 (dual clip,
 * defaults 0.2 / 0.2 / 3.0); prime-rl PR 4233 (weights, loss form).
 * Per token: P = e^lp, Q = e^lq, r = e^(lp-lq);
 *   IPO[i]:   masked iff |P-Q| > eps[i];  w = kept * min(r, max_ratio);  l = -A w lp
 *   IcePop:   low iff r < lo, high iff r > hi; w = kept * r;               l = -A w lp
 *   REINFORCE: l = -A lp
 *   PPO-bypass with dual clip: J = min(rA, clip(r, 1-clip_low, 1+clip_high) A),
 *             for A < 0 J = max(J, clip_c A); l = -J.  clip bit: clipped term
 *             smaller; dual bit: A < 0 and clip_c A > min(...)
 *   Decoupled token TIS, truncate, pi_old := pi_train: rho = r,
 *             w = min(rho, tis_upper); l = -w A.  trunc bit: rho > tis_upper
 * ------------------------------------------------------------------------ */
#define RL_ELEM_MAX_EPS 8

typedef struct rl_elem_cfg {
  int32_t n_eps;              /* 1 .. RL_ELEM_MAX_EPS                         */
  int32_t primary_eps_index;  /* which eps gives out->w_primary               */
  float eps[RL_ELEM_MAX_EPS]; /* IPO thresholds, >= 0                         */
  float max_ratio;            /* > 0                                          */
  float icepop_lo, icepop_hi; /* 0 <= lo <= hi                                */
  float clip_low, clip_high;  /* PPO clip, in [0, 1) and >= 0                 */
  float clip_c;               /* dual-clip constant, > 1                      */
  float tis_upper;            /* TIS truncation bound, > 0                    */
} rl_elem_cfg;

/* Mask-word bits (uint16 per token). */
#define RL_ELEM_BIT_IPO0 0          /* bits 0..7: IPO eps[i] masked */
#define RL_ELEM_BIT_ICEPOP_LOW 8
#define RL_ELEM_BIT_ICEPOP_HIGH 9
#define RL_ELEM_BIT_PPO_CLIP 10
#define RL_ELEM_BIT_DUAL_CLIP 11
#define RL_ELEM_BIT_TIS_TRUNC 12

/* Indices into rl_elem_out.sums (fp64; counts are exact integers). */
enum {
  RL_ELEM_IPO_KEPT = 0,        /* + 3*i for eps[i]: kept count        */
  RL_ELEM_IPO_LOSS = 1,        /* + 3*i: sum of l                     */
  RL_ELEM_IPO_WEIGHT = 2,      /* + 3*i: sum of w                     */
  RL_ELEM_ICEPOP_KEPT = 24,
  RL_ELEM_ICEPOP_LOW = 25,
  RL_ELEM_ICEPOP_HIGH = 26,
  RL_ELEM_ICEPOP_LOSS = 27,
  RL_ELEM_ICEPOP_WEIGHT = 28,
  RL_ELEM_REINFORCE_LOSS = 29,
  RL_ELEM_PPO_LOSS = 30,
  RL_ELEM_PPO_CLIP = 31,
  RL_ELEM_PPO_CLIP_LOWER = 32,
  RL_ELEM_PPO_KL = 33,         /* sum of lq - lp                      */
  RL_ELEM_TIS_LOSS = 34,
  RL_ELEM_TIS_TRUNC = 35,
  RL_ELEM_TIS_WEIGHT = 36,
  RL_ELEM_SUM_COUNT = 37
};

typedef struct rl_elem_out {
  uint16_t* mask_word;  /* [N] nullable */
  float* w_primary;     /* [N] nullable: IPO weight at eps[primary_eps_index] */
  double* sums;         /* [RL_ELEM_SUM_COUNT] required */
} rl_elem_out;

/* Largest N rl_loss_elementwise accepts. */
#define RL_ELEM_MAX_N (((int64_t)1) << 38)

/* Workspace bytes for rl_loss_elementwise with N tokens (at most
 * RL_ELEM_SUM_COUNT * 1024 doubles, 296 KiB). */
rl_status rl_elementwise_workspace_size(int64_t N, size_t* bytes);

/*
 * rl_loss_elementwise -- one pass over lp, lq, A [N] fp32 (device), 1 <= N <=
 * RL_ELEM_MAX_N.  lp, lq, adv, mask_word and w_primary 16-byte aligned.  The
 * sums are deterministic: the same inputs give the same bits on every call.
 * Errors: RL_E_ARG, RL_E_CFG, RL_E_WORKSPACE, RL_E_HIP.
 */
rl_status rl_loss_elementwise(const float* lp, const float* lq, const float* adv, int64_t N,
                              const rl_elem_cfg* cfg, const rl_elem_out* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * rl_loss_elementwise_noalloc -- rl_loss_elementwise for callers that cannot
 * allocate device memory or own a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same passes, limits,
 * outputs and results (bit for bit) as rl_loss_elementwise; it allocates
 * nothing and needs no workspace.  Its scratch (the per-block partial sums)
 * is a fixed array of RL_ELEM_NOALLOC_SCRATCH_BYTES in the library's own
 * device memory, one per GPU, kept until the process ends; the first call on
 * a device looks up its address.  Every call overwrites what it reads, so no
 * state carries over between calls, but all calls on one GPU share that
 * array: calls that may overlap in time on one GPU (unordered streams) race
 * and must not be made.  N beyond RL_ELEM_MAX_N is RL_E_ARG (the scratch
 * does not grow with N beyond 1024 blocks).
 * Errors: RL_E_ARG, RL_E_CFG, RL_E_HIP.
 */
#define RL_ELEM_NOALLOC_SCRATCH_BYTES (RL_ELEM_SUM_COUNT * 1024 * 8)
rl_status rl_loss_elementwise_noalloc(const float* lp, const float* lq, const float* adv,
                                      int64_t N, const rl_elem_cfg* cfg, const rl_elem_out* out,
                                      void* stream);

/* ---------------------------------------------------------------------------
 * Sequence-aware rollout correction over a replay (Rollout Correction Methods
 * page: "Config keys", "Importance Sampling", "Rejection Sampling", "Veto
 * Mechanism"; metrics from "Mismatch Monitoring Metrics" and "IS/RS
 * Correction Metrics").  The replay has no separate proximal policy
 * (pi_old := pi_train), so per token d = lp - lq, the token ratio is
 * rho = e^d and the decoupled PPO inner ratio is 1.  With sequences s given
 * by offsets and n_s tokens each:
 *   IS weight:  token  log w = d_t;  sequence  log w = sum_s d;
 *               geometric  log w = (1/n_s) sum_s d
 *   TIS mode:   truncate  w' = min(w, U);  clip  w' = min(max(w, L), U);
 *               mask  w' = w if L <= w <= U else 0 (the token stays in the
 *               loss average)
 *   RS:         statistic  token rho_t;  sequence (1/n_s) sum_s rho;
 *               geometric  e^{(1/n_s) sum_s d}; outside [rs_lower, rs_upper]
 *               the token (or the whole sequence) is rejected: weight 0, out
 *               of the loss average
 *   veto:       veto > 0: a sequence holding a token with rho < veto is
 *               rejected whole (with or without RS)
 *   batch norm: factor = kept / sum over kept tokens of w' (1 when off or
 *               when that sum is 0)
 *   loss:       l_t = -factor w'_t A_t over kept tokens; loss = sum / kept
 * Bounds are inclusive; decisions compare log weights with log bounds.
 * ------------------------------------------------------------------------ */
typedef enum rl_is_level {
  RL_LEVEL_TOKEN = 0,
  RL_LEVEL_SEQUENCE = 1,
  RL_LEVEL_GEOMETRIC = 2
} rl_is_level;

typedef enum rl_tis_mode { RL_TIS_TRUNCATE = 0, RL_TIS_CLIP = 1, RL_TIS_MASK = 2 } rl_tis_mode;

typedef struct rl_mis_cfg {
  int32_t tis_level;       /* rl_is_level                                      */
  int32_t tis_mode;        /* rl_tis_mode                                      */
  float tis_lower;         /* L > 0 (truncate ignores it)                      */
  float tis_upper;         /* U >= L                                           */
  int32_t use_rs;          /* 0 or 1                                           */
  int32_t rs_level;        /* rl_is_level                                      */
  float rs_lower;          /* > 0; NaN: tis_lower                              */
  float rs_upper;          /* >= rs_lower; NaN: tis_upper                      */
  float veto;              /* 0: off; > 0: the veto threshold C                */
  int32_t batch_normalize; /* 0 or 1                                           */
} rl_mis_cfg;

/* Per-token flag bits (uint8 per token). */
#define RL_MIS_F_TIS_LOW 0x01     /* w below L (clip, mask)                        */
#define RL_MIS_F_TIS_HIGH 0x02    /* w above U (truncate, clip, mask)              */
#define RL_MIS_F_RS_LOW 0x04      /* rejection statistic below rs_lower            */
#define RL_MIS_F_RS_HIGH 0x08     /* rejection statistic above rs_upper            */
#define RL_MIS_F_VETO 0x10        /* the token's sequence is vetoed                */
#define RL_MIS_F_CATASTROPHIC 0x20 /* the token's own rho is below the veto        */
#define RL_MIS_F_REJECTED 0x40    /* out of the loss (RS or veto)                  */

/* Indices into rl_mis_out.metrics (fp64).  Token means over the N tokens
 * unless stated; "per sequence" values are the mean over sequences of the
 * per-sequence quantity, with log ppl_s = -(1/n_s) sum_s log pi. */
enum {
  RL_MIS_TRAINING_LOG_PPL = 0,   /* per sequence: log ppl of lp                    */
  RL_MIS_TRAINING_PPL,           /* per sequence: e^(log ppl of lp)                */
  RL_MIS_ROLLOUT_LOG_PPL,        /* per sequence                                   */
  RL_MIS_ROLLOUT_PPL,            /* per sequence                                   */
  RL_MIS_KL,                     /* mean of lq - lp                                */
  RL_MIS_K3_KL,                  /* mean of e^d - d - 1                            */
  RL_MIS_LOG_PPL_DIFF,           /* per sequence: training - rollout log ppl       */
  RL_MIS_LOG_PPL_ABS_DIFF,       /* per sequence: |training - rollout log ppl|     */
  RL_MIS_PPL_RATIO,              /* per sequence: e^(training - rollout log ppl)   */
  RL_MIS_CHI2_TOKEN,             /* mean of rho^2, minus 1                         */
  RL_MIS_CHI2_SEQ,               /* mean over sequences of e^(2 sum_s d), minus 1  */
  RL_MIS_LOGPROB_ABS_DIFF,       /* mean of |d|                                    */
  RL_MIS_TIS_WEIGHT_BEFORE_BOUND, /* mean of w                                     */
  RL_MIS_TIS_WEIGHT_AFTER_BOUND, /* mean of w'                                     */
  RL_MIS_TIS_FRACTION_LOW,       /* fraction with w < L (clip, mask)               */
  RL_MIS_TIS_FRACTION_HIGH,      /* fraction with w > U (truncate, clip, mask)     */
  RL_MIS_RS_FRACTION_LOW,        /* fraction rejected below rs_lower               */
  RL_MIS_RS_FRACTION_HIGH,       /* fraction rejected above rs_upper               */
  RL_MIS_CATASTROPHIC_TOKEN_FRACTION,
  RL_MIS_CATASTROPHIC_SEQ_FRACTION, /* over sequences                              */
  RL_MIS_IS_RATIO_MEAN_AFTER_TIS_RS, /* mean of the weight output (rejected: 0)    */
  RL_MIS_BATCH_NORM_FACTOR,
  RL_MIS_IS_RATIO_MEAN_FINAL,    /* over kept tokens, factor included              */
  RL_MIS_IS_RATIO_MIN_FINAL,     /* over kept tokens (0 if none)                   */
  RL_MIS_IS_RATIO_MAX_FINAL,     /* over kept tokens (0 if none)                   */
  RL_MIS_LOSS,                   /* loss_sum / kept (0 if none)                    */
  RL_MIS_LOSS_SUM,
  RL_MIS_KEPT_TOKENS,
  RL_MIS_REJECTED_TOKENS,
  RL_MIS_METRIC_COUNT = 29
};

typedef struct rl_mis_out {
  float* weight;    /* [N] nullable: w' of kept tokens, 0 for rejected ones,
                       before batch normalisation (the final weight is
                       metrics[RL_MIS_BATCH_NORM_FACTOR] * weight)           */
  uint8_t* flags;   /* [N] nullable: RL_MIS_F_* bits                         */
  double* metrics;  /* [RL_MIS_METRIC_COUNT] required                        */
} rl_mis_out;

/* Largest N rl_mis_replay accepts. */
#define RL_MIS_MAX_N ((((int64_t)1) << 31) - 256)

/* Workspace bytes for rl_mis_replay with N tokens in S sequences. */
rl_status rl_mis_workspace_size(int64_t N, int64_t S, size_t* bytes);

/*
 * rl_mis_replay -- the correction pass over lp, lq, adv [N] fp32 (device,
 * 16-byte aligned; weight 16-byte and flags 4-byte aligned when given),
 * 1 <= N <= RL_MIS_MAX_N, cut into S >= 1 sequences by int64 offsets
 * [S + 1] given both on the host (checked: offsets[0] = 0, strictly
 * increasing, offsets[S] = N) and on the device (the same values; not
 * re-checked).  Deterministic.  Errors: RL_E_ARG, RL_E_CFG (unknown level
 * or mode, bounds not 0 < L <= U, veto < 0 or not finite), RL_E_CSR (bad
 * offsets), RL_E_WORKSPACE, RL_E_HIP.
 */
rl_status rl_mis_replay(const float* lp, const float* lq, const float* adv, int64_t N,
                        const int64_t* seq_offsets_host, const int64_t* seq_offsets_dev,
                        int64_t S, const rl_mis_cfg* cfg, const rl_mis_out* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Sampler-evidence validation of a CSR support (prime-rl PR 4233, "What
 * changes": checked on the GPU on the CSR entries once per step, before the
 * optimizer).  Flag bits written to *flags_dev (bitwise OR over all items):
 * ------------------------------------------------------------------------ */
#define RL_BAD_LABEL 0x001          /* a label outside [0, V)                    */
#define RL_BAD_ID 0x002             /* a support id outside [0, V)               */
#define RL_BAD_U 0x004              /* a u_e < 0 or not finite                   */
#define RL_BAD_LOGQ 0x008           /* a csr_logq value not finite or > 0        */
#define RL_BAD_INFER_LOGPROB 0x010  /* an infer_logprobs value not finite or > 0 */
#define RL_BAD_REPLAY_MASS 0x020    /* replayed: |sum_e u_e - 1| > 1e-3 in a row */
#define RL_BAD_REPLAY_LABEL 0x040   /* replayed: a row without its own label     */
#define RL_BAD_ADV 0x080            /* an advantage not finite                   */
#define RL_BAD_OFFSETS 0x100        /* device offsets not a CSR of nnz entries   */

/*
 * rl_validate_support -- enqueue the checks; writes one int32 to flags_dev.
 * Any of the csr_* pointers may be NULL when csr_offsets_host is NULL.
 * Errors: RL_E_ARG, RL_E_CSR (host offsets), RL_E_HIP.
 */
rl_status rl_validate_support(int64_t N, int64_t V, int64_t nnz, const int32_t* labels,
                              const float* infer_logprobs, const float* adv,
                              const int64_t* csr_offsets_host, const int64_t* csr_offsets_dev,
                              const int32_t* csr_ids, const float* csr_u, const float* csr_logq,
                              int32_t replayed, int32_t* flags_dev, void* stream);

/*
 * rl_validate_support_sync -- rl_validate_support, then synchronise `stream`
 * and copy the flag word to *flags_host.  Returns RL_E_INVALID_INPUT when
 * any flag is set.  This is the one call that waits for the device.
 */
rl_status rl_validate_support_sync(int64_t N, int64_t V, int64_t nnz, const int32_t* labels,
                                   const float* infer_logprobs, const float* adv,
                                   const int64_t* csr_offsets_host,
                                   const int64_t* csr_offsets_dev, const int32_t* csr_ids,
                                   const float* csr_u, const float* csr_logq, int32_t replayed,
                                   int32_t* flags_dev, int32_t* flags_host, void* stream);

/* ---------------------------------------------------------------------------
 * Opt-in kernel timing.  Between rl_profile_begin and rl_profile_end every
 * kernel the library enqueues is bracketed by two hipEvents on the caller's
 * stream; rl_profile_end waits for those events and reports, per kernel name,
 * the number of launches and the summed event-to-event time.  Off by default;
 * when off no event is recorded.  Process-wide; calls are serialised.
 * ------------------------------------------------------------------------ */
typedef struct rl_profile_entry {
  char name[32];      /* kernel (launch site) name, NUL-terminated */
  int64_t launches;
  double total_ms;
} rl_profile_entry;

rl_status rl_profile_begin(void);
/* Writes at most max_entries entries; *n_entries receives the number of
 * kernel names seen.  Errors: RL_E_ARG (null), RL_E_HIP. */
rl_status rl_profile_end(rl_profile_entry* out, int32_t max_entries, int32_t* n_entries);

/* ---------------------------------------------------------------------------
 * Machine calibration (measurement helpers, not part of the loss path): what
 * the bf16 matrix pipe and HBM deliver on the current device with kernels
 * that do nothing else, to set beside the published peaks.
 * ------------------------------------------------------------------------ */

/*
 * rl_calib_mfma_bf16 -- enqueue n_blocks 256-thread blocks (use 2 per compute
 * unit for two waves per SIMD, as the GEMMs run), each wave issuing
 * iters x 16 v_mfma_f32_16x16x32_bf16 from registers only.  random_operands:
 * 0 = all-zero operands, otherwise uniform random bf16 in [-2, 2).
 *   sink_dev    device float [n_blocks * 256], written (keeps the results live)
 *   stamps_dev  device int64 [n_blocks * 4]; block b writes, before and after
 *               its loop: [4b] shader-clock counter, [4b+1] the same at the
 *               end, [4b+2] / [4b+3] the fixed-rate wall clock at start / end.
 *               Shader clock in Hz = (d[4b+1]-d[4b]) / (d[4b+3]-d[4b+2]) *
 *               *wall_clock_khz * 1000.
 *   flop        host: receives the FLOP count of the launch
 *   wall_clock_khz host: receives the wall-clock counter rate
 * 1 <= n_blocks <= 2^20, 1 <= iters <= 2^32 and n_blocks * iters <= 2^34 (a
 * launch of seconds at most).  Errors: RL_E_ARG, RL_E_HIP.
 */
rl_status rl_calib_mfma_bf16(int32_t random_operands, int32_t n_blocks, int64_t iters,
                             float* sink_dev, int64_t* stamps_dev, double* flop,
                             int32_t* wall_clock_khz, void* stream);

/*
 * rl_calib_copy -- enqueue a grid-stride copy of `bytes` (a multiple of 16,
 * both pointers 16-byte aligned, device memory) from src to dst with
 * n_blocks 256-thread blocks.  dst == src reads and writes back every 16-byte
 * vector in place; any other overlap is RL_E_ARG.  Errors: RL_E_ARG, RL_E_HIP.
 */
rl_status rl_calib_copy(const void* src, void* dst, int64_t bytes, int32_t n_blocks,
                        void* stream);

/* Static description of a status code; never NULL. */
const char* rl_status_string(rl_status s);

/* Library version string, e.g. "rlloss 0.1.0 gfx950". */
const char* rl_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RLLOSS_H */
