// C ABI of librlloss: argument checks, planning, workspace layout, launches.
//
// Fused head + RLLoss (prime-rl PR 4233).  Tokens are processed in chunks of
// Tc rows sliced from the batch with host offsets, so no device value is read
// back.  Per chunk:
//   1. forward GEMM  S^T = W h_c^T  (MFMA) with an online-softmax epilogue:
//      per (token, 256-row vocabulary tile) the max m, sum e^(z-m) and
//      sum e^(z-m)(z-m); and, for a dense backward, P = e^(z-m) [Tc, V]
//   2. combine: per token LSE and entropy from the partials, label and
//      support logits by fp32 dot products, weights, KL, loss, kappa and the
//      per-entry gradient coefficients
//   3. dense backward only: form G (= (kappa p + gamma p (log p + H)) / D)
//      from P in both layouts, add the label and support coefficients into
//      it (from the vocabulary-sorted entry list, built once before the
//      chunks), dh partials = G (W^T)^T split over V, dW (+)= G^T (h_c^T)^T
//   4. dh = the partials (dense) or the label/support rows of W scaled by
//      their coefficients (sparse backward)
// After the chunks: for the sparse backward, dW from the vocabulary buckets;
// then the fixed-order loss and metric reduction.
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernels.h"

namespace {

using namespace rl;

// ---- opt-in event timing of every launch site --------------------------------
enum ProfKind {
  K_GEMM_FWD, K_COMBINE, K_FORM_G, K_GEMM_DH, K_TRANSPOSE_H, K_GEMM_DW, K_FINALIZE_DH,
  K_TRANSPOSE_W, K_CSR_ROWS, K_CSC_BUILD, K_SPARSE_DW, K_REDUCE, K_ELEMENTWISE, K_VALIDATE,
  K_ELEM_FINAL, K_FOLD, K_MIS_CHUNK, K_MIS_SEQ, K_MIS_TOKEN, K_MIS_FINAL, K_ENTRY_LOGITS,
  K_COUNT
};
const char* const kProfNames[K_COUNT] = {
    "gemm_fwd",   "combine",   "form_g",   "gemm_dh",   "transpose_h",
    "gemm_dw",    "finalize_dh", "transpose_w", "csr_rows", "csc_build",
    "sparse_dw",  "reduce",    "elementwise", "validate", "elementwise_final", "fold_sparse",
    "mis_chunk",  "mis_seq",   "mis_token", "mis_final", "entry_logits"};

struct ProfRec {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t timed(int kind, hipStream_t s, F&& f) {
  if (!g_prof_on) return f();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipEvent_t a = prof_event(), b = prof_event();
  if (a == nullptr || b == nullptr) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = f();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  g_prof_recs.push_back({kind, a, b});
  return e;
}

constexpr size_t WS_ALIGN = 256;
// Tokens per pass through the head when the caller leaves token_chunk at 0.
// The dense backward keeps e^(z - m) of one chunk, Tc x V bf16 (2.5 GB at
// V = 152064), never the whole batch; each further chunk costs one
// accumulating pass over dW (about 0.55 ms at H = 2048).
constexpr int64_t DEFAULT_CHUNK = 8192;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  return !__builtin_mul_overflow(a, b, out);
}

struct Layout {
  size_t off = 0;
  bool ok = true;
  size_t take(int64_t n, int64_t elem) {
    int64_t bytes;
    if (!mul_ok(n, elem, &bytes) || bytes > ((int64_t)1 << 56)) {
      ok = false;
      return 0;
    }
    const size_t o = off;
    off = (off + (size_t)bytes + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN;
    return o;
  }
};

struct Plan {
  int64_t N, H, V, nnz, E, Tc, Tcpad, Vpad, J;
  int dtype, gdtype;
  int64_t esz;
  int mode;  // resolved rl_backward
  bool has_support, want_dh, want_dW, dense, kl_active, need_csc;
  float beta;
  int splits;
  int64_t k_split;
  size_t o_pm, o_ps, o_pt, o_lse, o_kap, o_stats, o_coef;
  size_t o_P, o_G, o_Gt, o_Wt, o_ht, o_dhp;
  int vtile;
  bool tiled;             // bf16 dense backward: operands in the tiled block layout
  bool tfwd;              // bf16 forward from tiled copies of W and h_c (o_Wf, o_hf)
  int64_t Tc256, KB_v, KB_t, KB_h;
  size_t o_Wf, o_hf;
  size_t o_ka, o_kb, o_ia, o_ib, o_hist, o_start, o_rows, o_zent;
  bool entry_pass;  // label/support logits by the vocabulary-ordered pass
  size_t total;
};

bool finite(float x) { return std::isfinite(x); }

rl_status check_cfg(const rl_loss_cfg* c, bool has_support) {
  if (c->N < 1 || c->H < 8 || (c->H % 8) != 0 || c->V < 1 || c->nnz < 0) return RL_E_ARG;
  if (c->V > (int64_t)INT32_MAX - 2 || c->N > (int64_t)INT32_MAX) return RL_E_ARG;
  if (c->N + c->nnz > (int64_t)INT32_MAX) return RL_E_ARG;
  if (!has_support && c->nnz != 0) return RL_E_ARG;
  if (c->token_chunk < 0 || c->reserved1 != 0) return RL_E_ARG;
  if ((c->dtype != RL_DTYPE_FP32 && c->dtype != RL_DTYPE_BF16) ||
      (c->grad_dtype != RL_DTYPE_FP32 && c->grad_dtype != RL_DTYPE_BF16))
    return RL_E_ARG;
  if (c->loss_type < RL_LOSS_IPO || c->loss_type > RL_LOSS_REINFORCE) return RL_E_CFG;
  if (!(c->ipo_eps >= 0.0f) || !(c->max_ratio > 0.0f)) return RL_E_CFG;
  if (!(c->icepop_lo >= 0.0f) || !(c->icepop_lo <= c->icepop_hi)) return RL_E_CFG;
  if (!finite(c->adv_tau)) return RL_E_CFG;
  if (!(c->inv_temperature > 0.0f) || !finite(c->inv_temperature)) return RL_E_CFG;
  if (!(c->loss_norm > 0.0f) || !finite(c->loss_norm)) return RL_E_CFG;
  if (c->kl_estimator < RL_KL_NONE || c->kl_estimator > RL_KL_K1) return RL_E_CFG;
  if (!(c->kl_coeff >= 0.0f) || !finite(c->kl_coeff)) return RL_E_CFG;
  if (c->kl_staleness != RL_STALENESS_NONE && c->kl_staleness != RL_STALENESS_INV_SQRT)
    return RL_E_CFG;
  if (!finite(c->entropy_coeff)) return RL_E_CFG;
  const bool kl_active = c->kl_estimator != RL_KL_NONE && c->kl_coeff > 0.0f;
  if (kl_active && !has_support) return RL_E_CFG;
  if (c->kl_estimator == RL_KL_EXACT && !c->replayed) return RL_E_CFG;
  if (c->replayed != 0 && c->replayed != 1) return RL_E_CFG;
  if (c->replayed && !has_support) return RL_E_CFG;
  if (c->accumulate_dW != 0 && c->accumulate_dW != 1) return RL_E_CFG;
  if (c->backward < RL_BWD_AUTO || c->backward > RL_BWD_NONE) return RL_E_CFG;
  // the entropy bonus puts a dense term on every logit
  const bool sparse_ok = c->loss_type == RL_LOSS_REINFORCE && !kl_active && has_support &&
                         c->entropy_coeff == 0.0f;
  if (c->backward == RL_BWD_SPARSE && !sparse_ok) return RL_E_CFG;
  return RL_OK;
}

rl_status make_plan(const rl_loss_cfg* c, bool has_support, bool want_dh, bool want_dW,
                    Plan* p) {
  const rl_status st = check_cfg(c, has_support);
  if (st != RL_OK) return st;
  p->N = c->N;
  p->H = c->H;
  p->V = c->V;
  p->nnz = c->nnz;
  p->E = c->N + c->nnz;
  p->has_support = has_support;
  p->dtype = c->dtype;
  p->gdtype = c->grad_dtype;
  p->esz = c->dtype == RL_DTYPE_BF16 ? 2 : 4;
  p->kl_active = c->kl_estimator != RL_KL_NONE && c->kl_coeff > 0.0f;
  p->beta = p->kl_active ? c->kl_coeff : 0.0f;
  int mode = c->backward;
  if (mode == RL_BWD_AUTO)
    mode = (c->loss_type == RL_LOSS_REINFORCE && !p->kl_active && has_support &&
            c->entropy_coeff == 0.0f)
               ? RL_BWD_SPARSE
               : RL_BWD_DENSE;
  p->mode = mode;
  p->want_dh = want_dh && mode != RL_BWD_NONE;
  p->want_dW = want_dW && mode != RL_BWD_NONE;
  p->dense = mode == RL_BWD_DENSE && (p->want_dh || p->want_dW);
  p->Tc = c->token_chunk > 0 ? std::min(c->token_chunk, c->N) : std::min(DEFAULT_CHUNK, c->N);
  p->Tcpad = round_up(p->Tc, 64);
  p->Vpad = round_up(p->V, 256);
  p->vtile = fwd_vtile(p->dtype);
  p->J = ceil_div(p->V, p->vtile);
  const int bk = gemm_k_tile(p->dtype);
  {
    const int64_t tiles = ceil_div(p->Tc, 128) * ceil_div(p->H, 128);
    int64_t sp = std::max<int64_t>(1, std::min<int64_t>(16, ceil_div(1024, tiles)));
    p->k_split = round_up(ceil_div(p->Vpad, sp), bk);
    p->splits = (int)ceil_div(p->Vpad, p->k_split);
  }
  Layout L;
  const int64_t TJ = p->Tc * p->J;
  p->o_pm = L.take(TJ, 4);
  p->o_ps = L.take(TJ, 4);
  p->o_pt = L.take(TJ, 4);
  p->o_lse = L.take(p->N, 4);
  p->o_kap = L.take(p->N, 4);
  p->o_stats = L.take(p->N, 4 * STAT_N);
  p->o_coef = L.take(p->E, 4);
  p->o_P = p->o_G = p->o_Gt = p->o_Wt = p->o_ht = p->o_dhp = 0;
  p->tiled = p->dense && p->dtype == RL_DTYPE_BF16;
  p->Tc256 = round_up(p->Tc, TILE_ROWS);
  p->KB_v = p->Vpad / TILE_K;
  p->KB_t = p->Tc256 / TILE_K;
  // The persistent forward reads tiled copies of W and h_c (consecutive 1 KB
  // pieces per stage; 5% faster than the row-major operands at the 16k
  // shape): made once per call for W, per chunk for h_c.
  p->KB_h = ceil_div(p->H, TILE_K);
  p->tfwd = p->dtype == RL_DTYPE_BF16 && gemm_fwd_tiled_ok(p->H);
  p->o_Wf = p->o_hf = 0;
  if (p->tfwd) {
    int64_t wf, hf;
    if (!mul_ok(p->Vpad, p->KB_h * TILE_K, &wf) || !mul_ok(p->Tc256, p->KB_h * TILE_K, &hf))
      return RL_E_ARG;
    p->o_Wf = L.take(wf, 2);
    p->o_hf = L.take(hf, 2);
  }
  if (p->dense) {
    int64_t vt, tv, hv, sth;
    const int64_t H256 = round_up(p->H, TILE_ROWS);
    if (!mul_ok(p->Vpad, p->Tc256, &vt) || !mul_ok(p->Tc256, p->Vpad, &tv) ||
        !mul_ok(H256, p->Vpad, &hv) || !mul_ok((int64_t)p->splits * p->Tc, p->H, &sth))
      return RL_E_ARG;
    if (p->tiled) {
      // e^(z - m), then G, in the tiled layout; dW reads it transposed
      p->o_G = L.take(tv, 2);
      if (p->want_dh) {
        p->o_Wt = L.take(hv, 2);
        p->o_dhp = L.take(sth, 4);
      }
      if (p->want_dW) p->o_ht = L.take(H256 * p->Tc256, 2);
    } else {
      p->o_P = L.take(tv, p->esz);  // e^(z - m) token-major [Tc, Vpad], then G in place
      if (p->want_dW) {
        p->o_Gt = L.take(p->V * p->Tcpad, p->esz);
        p->o_ht = L.take(p->H * p->Tcpad, p->esz);
      }
      if (p->want_dh) {
        p->o_Wt = L.take(p->H * p->Vpad, p->esz);
        p->o_dhp = L.take(sth, 4);
      }
    }
  }
  p->o_ka = p->o_kb = p->o_ia = p->o_ib = p->o_hist = p->o_start = p->o_rows = p->o_zent = 0;
  // The vocabulary-sorted entry list: the dense backward folds the support
  // coefficients into G from it; the sparse backward sums the dW rows from it.
  p->need_csc = (p->dense && has_support) || (!p->dense && p->want_dW);
  if (p->need_csc) {
    p->o_ka = L.take(p->E, 4);
    p->o_kb = L.take(p->E, 4);
    p->o_ia = L.take(p->E, 4);
    p->o_ib = L.take(p->E, 4);
    p->o_hist = L.take(csc_hist_len(p->E), 4);
    p->o_start = L.take(p->V + 2, 4);
  }
  if (p->need_csc && has_support) p->o_rows = L.take(p->nnz, 4);
  // Entry logits in vocabulary order gather one h row per entry; that pays
  // when h stays in the 256 MB Infinity Cache (measured: 1.2M top-p entries
  // over 16k tokens, 1.74 -> 0.80 ms).  With a larger h, gathering W rows per
  // token inside combine is cheaper (64k tokens, 590k entries: 1.10 against
  // 1.37 ms).
  p->entry_pass = p->need_csc && has_support &&
                  (double)p->N * (double)p->H * (double)p->esz <= 128.0 * 1024 * 1024;
  if (p->entry_pass) p->o_zent = L.take(p->E, 4);
  if (!L.ok) return RL_E_ARG;
  p->total = L.off;
  return RL_OK;
}

rl_status check_host_csr(const int64_t* off, int64_t N, int64_t nnz) {
  if (off[0] != 0) return RL_E_CSR;
  for (int64_t t = 0; t < N; ++t)
    if (off[t + 1] < off[t]) return RL_E_CSR;
  if (off[N] != nnz) return RL_E_CSR;
  return RL_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define RL_TRY(expr)                              \
  do {                                            \
    if ((expr) != hipSuccess) return RL_E_HIP;    \
  } while (0)

}  // namespace

extern "C" {

const char* rl_status_string(rl_status s) {
  switch (s) {
    case RL_OK: return "ok";
    case RL_E_ARG: return "invalid argument (null pointer, size, dtype, alignment or overflow)";
    case RL_E_CFG: return "invalid or inconsistent loss configuration";
    case RL_E_CSR: return "host CSR offsets are not a valid support (off[0]=0, monotone, off[N]=nnz)";
    case RL_E_WORKSPACE: return "workspace missing, misaligned or smaller than required";
    case RL_E_HIP: return "HIP runtime error or kernel launch failure";
    case RL_E_INVALID_INPUT: return "validation found malformed support or label data";
  }
  return "unknown status";
}

const char* rl_version(void) { return "rlloss 0.1.0 gfx950"; }

rl_status rl_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof_recs) {
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  g_prof_on = true;
  return RL_OK;
}

rl_status rl_profile_end(rl_profile_entry* out, int32_t max_entries, int32_t* n_entries) {
  if (n_entries == nullptr || (out == nullptr && max_entries > 0)) return RL_E_ARG;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = false;
  int64_t cnt[K_COUNT] = {};
  double ms[K_COUNT] = {};
  rl_status st = RL_OK;
  for (auto& r : g_prof_recs) {
    float t = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
      st = RL_E_HIP;
    cnt[r.kind] += 1;
    ms[r.kind] += t;
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  int32_t n = 0;
  for (int k = 0; k < K_COUNT; ++k) {
    if (cnt[k] == 0) continue;
    if (n < max_entries) {
      std::memset(out[n].name, 0, sizeof(out[n].name));
      std::strncpy(out[n].name, kProfNames[k], sizeof(out[n].name) - 1);
      out[n].launches = cnt[k];
      out[n].total_ms = ms[k];
    }
    ++n;
  }
  *n_entries = n;
  return st;
}

rl_status rl_loss_workspace_size(const rl_loss_cfg* cfg, int32_t has_support, int32_t want_dh,
                                 int32_t want_dW, size_t* bytes) {
  if (cfg == nullptr || bytes == nullptr) return RL_E_ARG;
  Plan p{};
  const rl_status st = make_plan(cfg, has_support != 0, want_dh != 0, want_dW != 0, &p);
  if (st != RL_OK) return st;
  *bytes = p.total;
  return RL_OK;
}

rl_status rl_loss_fwd_bwd(const void* h, const void* W, const int32_t* labels,
                          const float* infer_logprobs, const float* adv,
                          const int32_t* policy_age, const int64_t* csr_offsets_host, const int64_t* csr_offsets_dev,
                          const int32_t* csr_ids, const float* csr_u, const float* csr_logq,
                          const rl_loss_cfg* cfg, const rl_loss_out* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (cfg == nullptr || out == nullptr || out->loss == nullptr) return RL_E_ARG;
  if (h == nullptr || W == nullptr || labels == nullptr || infer_logprobs == nullptr ||
      adv == nullptr)
    return RL_E_ARG;
  const bool has_support = csr_offsets_host != nullptr;
  if (has_support && (csr_offsets_dev == nullptr || csr_ids == nullptr || csr_u == nullptr))
    return RL_E_ARG;
  if (!has_support && (csr_offsets_dev != nullptr || csr_ids != nullptr || csr_u != nullptr ||
                       csr_logq != nullptr))
    return RL_E_ARG;
  if (!aligned(h, 16) || !aligned(W, 16) || (out->dh && !aligned(out->dh, 16)) ||
      (out->dW && !aligned(out->dW, 16)))
    return RL_E_ARG;
  Plan p{};
  rl_status st = make_plan(cfg, has_support, out->dh != nullptr, out->dW != nullptr, &p);
  if (st != RL_OK) return st;
  if (has_support) {
    st = check_host_csr(csr_offsets_host, p.N, p.nnz);
    if (st != RL_OK) return st;
  }
  if (p.total > 0 && (workspace == nullptr || workspace_bytes < p.total ||
                      !aligned(workspace, WS_ALIGN)))
    return RL_E_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  auto F = [&](size_t o) { return reinterpret_cast<float*>(ws + o); };
  auto I = [&](size_t o) { return reinterpret_cast<int32_t*>(ws + o); };
  float *pm = F(p.o_pm), *ps = F(p.o_ps), *pt = F(p.o_pt);
  float *lse = F(p.o_lse), *kap = F(p.o_kap), *stats = F(p.o_stats), *coef = F(p.o_coef);
  void* G = p.tiled ? ws + p.o_G : nullptr;
  void* P = p.tiled ? G : p.dense ? ws + p.o_P : nullptr;
  void* Gt = (p.dense && !p.tiled && p.want_dW) ? ws + p.o_Gt : nullptr;
  void* Wt = (p.dense && p.want_dh) ? ws + p.o_Wt : nullptr;
  void* ht = (p.dense && p.want_dW) ? ws + p.o_ht : nullptr;
  float* dhp = (p.dense && p.want_dh) ? F(p.o_dhp) : nullptr;
  const char* hb = static_cast<const char*>(h);

  const WeightParams wp{cfg->loss_type, cfg->ipo_eps, cfg->max_ratio, cfg->icepop_lo,
                        cfg->icepop_hi};
  const float inv_D = 1.0f / cfg->loss_norm;
  const float gs = cfg->entropy_coeff * cfg->inv_temperature * inv_D;  // entropy term of G

  // entries sorted by vocabulary id (and each support entry's token)
  const int32_t* perm = nullptr;
  const int32_t* skeys = nullptr;
  int32_t* rows = (p.need_csc && has_support) ? I(p.o_rows) : nullptr;
  CscWork cw{};
  if (p.need_csc) {
    cw = CscWork{I(p.o_ka), I(p.o_kb), I(p.o_ia), I(p.o_ib), I(p.o_hist), I(p.o_start),
                 csc_hist_len(p.E)};
    if (has_support)
      RL_TRY(timed(K_CSR_ROWS, s, [&] { return csr_rows(csr_offsets_dev, p.N, p.nnz, rows, s); }));
    RL_TRY(timed(K_CSC_BUILD, s, [&] {
      return csc_build(labels, csr_ids, p.N, p.nnz, p.V, cw, &perm, &skeys, s);
    }));
  }
  // label and support logits in vocabulary order (combine then gathers no W rows)
  float* zent = p.entry_pass ? F(p.o_zent) : nullptr;
  if (zent != nullptr)
    RL_TRY(timed(K_ENTRY_LOGITS, s, [&] {
      return entry_logits(p.dtype, h, W, p.H, p.V, skeys, perm, rows, p.N, p.E, zent, s);
    }));

  // W^T for dh (tiled or padded) and the forward's tiled copy of W, from one
  // read of W where both are needed.
  bf16_t* Wf = p.tfwd ? reinterpret_cast<bf16_t*>(ws + p.o_Wf) : nullptr;
  bf16_t* hf = p.tfwd ? reinterpret_cast<bf16_t*>(ws + p.o_hf) : nullptr;
  const bool want_wt = p.dense && p.want_dh;
  if (want_wt || p.tfwd)
    RL_TRY(timed(K_TRANSPOSE_W, s, [&] {
      // bf16 dense is always tiled, so an untiled W^T is only ever fp32
      return p.tiled || p.tfwd
                 ? to_tiled_t(static_cast<const bf16_t*>(W), p.H, p.V, p.H,
                              want_wt ? static_cast<bf16_t*>(Wt) : nullptr, p.KB_v, p.KB_v, s,
                              Wf, p.KB_h)
                 : transpose_pad(p.dtype, W, p.H, p.V, p.H, Wt, p.Vpad, s);
    }));

  for (int64_t c0 = 0; c0 < p.N; c0 += p.Tc) {
    const int64_t tc = std::min(p.Tc, p.N - c0);
    const int64_t tck = round_up(tc, 64);
    const void* hc = hb + c0 * p.H * p.esz;
    FwdEpiArgs fa{cfg->inv_temperature, p.V, tc, p.J, pm, ps, pt, P, p.tiled ? p.KB_v : p.Vpad};
    // h_c tiled for the forward and, on the tiled dense path, h_c^T for dW
    // (its panels to the 256-token boundary, zeros past tc)
    const bool ht_now = p.tfwd && p.tiled && p.want_dW;
    if (p.tfwd)
      RL_TRY(timed(K_TRANSPOSE_H, s, [&] {
        return to_tiled_t(static_cast<const bf16_t*>(hc), p.H, tc, p.H,
                          ht_now ? static_cast<bf16_t*>(ht) : nullptr, p.KB_t,
                          round_up(tc, TILE_ROWS) / TILE_K, s, hf, p.KB_h);
      }));
    RL_TRY(timed(K_GEMM_FWD, s, [&] {
      return gemm_fwd(p.dtype, W, hc, p.V, tc, p.H, fa, s, Wf, hf, p.KB_h);
    }));
    CombineArgs ca{};
    ca.h = h;
    ca.W = W;
    ca.labels = labels;
    ca.infer_lp = infer_logprobs;
    ca.adv = adv;
    ca.off = has_support ? csr_offsets_dev : nullptr;
    ca.ids = csr_ids;
    ca.u = csr_u;
    ca.logq = csr_logq;
    ca.zent = zent;
    ca.part_m = pm;
    ca.part_s = ps;
    ca.part_t = pt;
    ca.t0 = c0;
    ca.Tc = tc;
    ca.N = p.N;
    ca.H = p.H;
    ca.V = p.V;
    ca.J = p.J;
    ca.nnz = p.nnz;
    ca.wp = wp;
    ca.adv_tau = cfg->adv_tau;
    ca.beta = p.beta;
    ca.age = policy_age;
    ca.staleness = cfg->kl_staleness;
    ca.gamma = cfg->entropy_coeff;
    ca.inv_t = cfg->inv_temperature;
    ca.inv_D = inv_D;
    ca.lse = lse;
    ca.kappa_s = kap;
    ca.stats = stats;
    ca.coef = coef;
    ca.o_logprobs = out->logprobs;
    ca.o_entropy = out->entropy;
    ca.o_weight = out->weight;
    ca.o_keep = out->keep;
    ca.o_token_loss = out->token_loss;
    ca.o_support_lp = has_support ? out->support_logprobs : nullptr;
    RL_TRY(timed(K_COMBINE, s, [&] { return combine(p.dtype, ca, s); }));
    if (p.tiled) {
      // G in place only: dh reads it as is, dW with transposed LDS reads.
      RL_TRY(timed(K_FORM_G, s, [&] {
        return form_g_blocks(static_cast<bf16_t*>(G), p.KB_v, pm, p.J, p.vtile, lse + c0,
                             kap + c0, gs, p.V, tc, s);
      }));
      RL_TRY(timed(K_FOLD, s, [&] {
        return fold_sparse(p.dtype, G, 1, nullptr, 1, p.KB_v, p.KB_t, labels, skeys, perm, rows,
                           coef, p.N, p.nnz, c0, tc, p.V, s);
      }));
      if (p.want_dh)
        RL_TRY(timed(K_GEMM_DH, s, [&] {
          return gemm_store(p.dtype, G, p.KB_v, Wt, p.KB_v, tc, p.H, p.Vpad, p.splits, p.k_split,
                            dhp, p.H, p.Tc * p.H, s);
        }));
      if (p.want_dW) {
        if (!ht_now)
          RL_TRY(timed(K_TRANSPOSE_H, s, [&] {
            return to_tiled_t(static_cast<const bf16_t*>(hc), p.H, tc, p.H,
                              static_cast<bf16_t*>(ht), p.KB_t, ceil_div(tc, TILE_K), s);
          }));
        const int acc = (c0 > 0 || cfg->accumulate_dW) ? 1 : 0;
        RL_TRY(timed(K_GEMM_DW, s, [&] {
          return gemm_dw(p.dtype, G, p.KB_v, ht, p.KB_t, p.V, p.H, tc, out->dW, p.H, acc, s);
        }));
      }
    } else if (p.dense) {
      RL_TRY(timed(K_FORM_G, s, [&] {
        return form_g(p.dtype, P, p.Vpad, Gt, p.Tcpad, pm, p.J, p.vtile, lse + c0, kap + c0, gs,
                      p.V, tc, tck, p.want_dh ? 1 : 0, s);
      }));
      RL_TRY(timed(K_FOLD, s, [&] {
        return fold_sparse(p.dtype, P, p.want_dh ? 1 : 0, Gt, 0, p.Vpad, p.Tcpad, labels, skeys,
                           perm, rows, coef, p.N, p.nnz, c0, tc, p.V, s);
      }));
      if (p.want_dh)
        RL_TRY(timed(K_GEMM_DH, s, [&] {
          return gemm_store(p.dtype, P, p.Vpad, Wt, p.Vpad, tc, p.H, p.Vpad, p.splits, p.k_split,
                            dhp, p.H, p.Tc * p.H, s);
        }));
      if (p.want_dW) {
        RL_TRY(timed(K_TRANSPOSE_H, s,
                     [&] { return transpose_pad(p.dtype, hc, p.H, tc, p.H, ht, tck, s); }));
        const int acc = (c0 > 0 || cfg->accumulate_dW) ? 1 : 0;
        RL_TRY(timed(K_GEMM_DW, s, [&] {
          return gemm_dw(p.dtype, Gt, p.Tcpad, ht, tck, p.V, p.H, tck, out->dW, p.H, acc, s);
        }));
      }
    }
    if (p.want_dh)
      RL_TRY(timed(K_FINALIZE_DH, s, [&] {
        return finalize_dh(p.dtype, p.gdtype, dhp, p.dense ? p.splits : 0, p.Tc * p.H, W, labels,
                           has_support ? csr_offsets_dev : nullptr, csr_ids, coef, c0, tc, p.N,
                           p.nnz, p.V, p.H, p.dense ? 0 : 1, out->dh, s);
      }));
  }
  if (!p.dense && p.want_dW) {
    // sparse backward: dW is the label and support terms alone
    const int overwrite = cfg->accumulate_dW ? 0 : 1;
    RL_TRY(timed(K_SPARSE_DW, s, [&] {
      return sparse_dw(p.dtype, h, p.H, p.N, p.V, cw.start, perm, rows, coef, out->dW, overwrite,
                       s);
    }));
  }
  RL_TRY(timed(K_REDUCE, s, [&] {
    return reduce_final(stats, p.N, inv_D, p.beta, out->loss, out->metrics, s);
  }));
  return RL_OK;
}

rl_status rl_elementwise_workspace_size(int64_t N, size_t* bytes) {
  if (bytes == nullptr || N < 1 || N > RL_ELEM_MAX_N) return RL_E_ARG;
  int64_t b;
  if (!mul_ok(elem_num_blocks(N), (int64_t)RL_ELEM_SUM_COUNT * 8, &b)) return RL_E_ARG;
  *bytes = (size_t)b;
  return RL_OK;
}

namespace {
rl_status check_elementwise(const float* lp, const float* lq, const float* adv, int64_t N,
                            const rl_elem_cfg* cfg, const rl_elem_out* out) {
  if (lp == nullptr || lq == nullptr || adv == nullptr || cfg == nullptr || out == nullptr ||
      out->sums == nullptr || N < 1 || N > RL_ELEM_MAX_N)
    return RL_E_ARG;
  if (!aligned(lp, 16) || !aligned(lq, 16) || !aligned(adv, 16) ||
      (out->mask_word && !aligned(out->mask_word, 16)) ||
      (out->w_primary && !aligned(out->w_primary, 16)))
    return RL_E_ARG;
  if (cfg->n_eps < 1 || cfg->n_eps > RL_ELEM_MAX_EPS || cfg->primary_eps_index < 0 ||
      cfg->primary_eps_index >= cfg->n_eps)
    return RL_E_CFG;
  for (int i = 0; i < cfg->n_eps; ++i)
    if (!(cfg->eps[i] >= 0.0f)) return RL_E_CFG;
  if (!(cfg->max_ratio > 0.0f) || !(cfg->icepop_lo >= 0.0f) ||
      !(cfg->icepop_lo <= cfg->icepop_hi) || !(cfg->clip_low >= 0.0f && cfg->clip_low < 1.0f) ||
      !(cfg->clip_high >= 0.0f) || !(cfg->clip_c > 1.0f) || !(cfg->tis_upper > 0.0f))
    return RL_E_CFG;
  return RL_OK;
}
}  // namespace

rl_status rl_loss_elementwise(const float* lp, const float* lq, const float* adv, int64_t N,
                              const rl_elem_cfg* cfg, const rl_elem_out* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const rl_status st = check_elementwise(lp, lq, adv, N, cfg, out);
  if (st != RL_OK) return st;
  size_t need;
  rl_elementwise_workspace_size(N, &need);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
    return RL_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RL_TRY(timed(K_ELEMENTWISE, s, [&] {
    return rl::elementwise(lp, lq, adv, N, *cfg, out->mask_word, out->w_primary,
                           static_cast<double*>(workspace), out->sums, s);
  }));
  RL_TRY(timed(K_ELEM_FINAL, s, [&] {
    return rl::elementwise_final(static_cast<const double*>(workspace), N, cfg->n_eps,
                                 out->sums, s);
  }));
  return RL_OK;
}

rl_status rl_loss_elementwise_noalloc(const float* lp, const float* lq, const float* adv,
                                      int64_t N, const rl_elem_cfg* cfg, const rl_elem_out* out,
                                      void* stream) {
  const rl_status st = check_elementwise(lp, lq, adv, N, cfg, out);
  if (st != RL_OK) return st;
  size_t need;
  rl_elementwise_workspace_size(N, &need);
  if (need > (size_t)elem_noalloc_scratch_bytes()) return RL_E_ARG;  // not reached: N is bounded
  hipStream_t s = static_cast<hipStream_t>(stream);
  double* part = nullptr;
  RL_TRY(elem_noalloc_scratch(&part));
  // no event timing here: this entry point creates nothing
  RL_TRY(rl::elementwise(lp, lq, adv, N, *cfg, out->mask_word, out->w_primary, part, out->sums,
                         s));
  RL_TRY(rl::elementwise_final(part, N, cfg->n_eps, out->sums, s));
  return RL_OK;
}

rl_status rl_mis_workspace_size(int64_t N, int64_t S, size_t* bytes) {
  if (bytes == nullptr || N < 1 || N > RL_MIS_MAX_N || S < 1 || S > N) return RL_E_ARG;
  *bytes = (size_t)rl::mis_layout(N, S).bytes;
  return RL_OK;
}

namespace {
bool level_ok(int32_t v) { return v >= RL_LEVEL_TOKEN && v <= RL_LEVEL_GEOMETRIC; }
bool bound_ok(float lo, float hi) {
  return std::isfinite(lo) && std::isfinite(hi) && lo > 0.0f && hi >= lo;
}
}  // namespace

rl_status rl_mis_replay(const float* lp, const float* lq, const float* adv, int64_t N,
                        const int64_t* seq_offsets_host, const int64_t* seq_offsets_dev,
                        int64_t S, const rl_mis_cfg* cfg, const rl_mis_out* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (lp == nullptr || lq == nullptr || adv == nullptr || seq_offsets_host == nullptr ||
      seq_offsets_dev == nullptr || cfg == nullptr || out == nullptr || out->metrics == nullptr ||
      N < 1 || N > RL_MIS_MAX_N || S < 1 || S > N)
    return RL_E_ARG;
  if (!aligned(lp, 16) || !aligned(lq, 16) || !aligned(adv, 16) ||
      !aligned(seq_offsets_dev, 8) || (out->weight && !aligned(out->weight, 16)) ||
      (out->flags && !aligned(out->flags, 4)))
    return RL_E_ARG;
  const rl_mis_cfg& c = *cfg;
  if (!level_ok(c.tis_level) || !level_ok(c.rs_level) || c.tis_mode < RL_TIS_TRUNCATE ||
      c.tis_mode > RL_TIS_MASK || (c.use_rs != 0 && c.use_rs != 1) ||
      (c.batch_normalize != 0 && c.batch_normalize != 1))
    return RL_E_CFG;
  if (!bound_ok(c.tis_lower, c.tis_upper) || !std::isfinite(c.veto) || c.veto < 0.0f)
    return RL_E_CFG;
  const float rlo = std::isnan(c.rs_lower) ? c.tis_lower : c.rs_lower;
  const float rhi = std::isnan(c.rs_upper) ? c.tis_upper : c.rs_upper;
  if (!bound_ok(rlo, rhi)) return RL_E_CFG;
  if (seq_offsets_host[0] != 0 || seq_offsets_host[S] != N) return RL_E_CSR;
  for (int64_t i = 0; i < S; ++i)
    if (seq_offsets_host[i + 1] <= seq_offsets_host[i]) return RL_E_CSR;
  const rl::MisLayout L = rl::mis_layout(N, S);
  if (workspace == nullptr || workspace_bytes < (size_t)L.bytes || !aligned(workspace, 16))
    return RL_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int kinds[4] = {K_MIS_CHUNK, K_MIS_SEQ, K_MIS_TOKEN, K_MIS_FINAL};
  for (int st = 0; st < 4; ++st) {
    RL_TRY(timed(kinds[st], s, [&] {
      return rl::mis_stage(st, lp, lq, adv, N, seq_offsets_dev, S, c, out->weight, out->flags,
                           out->metrics, workspace, s);
    }));
  }
  return RL_OK;
}

rl_status rl_validate_support(int64_t N, int64_t V, int64_t nnz, const int32_t* labels,
                              const float* infer_logprobs, const float* adv,
                              const int64_t* csr_offsets_host, const int64_t* csr_offsets_dev,
                              const int32_t* csr_ids, const float* csr_u, const float* csr_logq,
                              int32_t replayed, int32_t* flags_dev, void* stream) {
  if (N < 1 || V < 1 || nnz < 0 || labels == nullptr || infer_logprobs == nullptr ||
      adv == nullptr || flags_dev == nullptr)
    return RL_E_ARG;
  const bool has_support = csr_offsets_host != nullptr;
  if (has_support) {
    if (csr_offsets_dev == nullptr || csr_ids == nullptr || csr_u == nullptr) return RL_E_ARG;
    const rl_status st = check_host_csr(csr_offsets_host, N, nnz);
    if (st != RL_OK) return st;
  } else if (nnz != 0) {
    return RL_E_ARG;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  RL_TRY(timed(K_VALIDATE, s, [&] {
    return rl::validate(N, V, nnz, labels, infer_logprobs, adv,
                        has_support ? csr_offsets_dev : nullptr, csr_ids, csr_u, csr_logq,
                        replayed ? 1 : 0, flags_dev, s);
  }));
  return RL_OK;
}

rl_status rl_validate_support_sync(int64_t N, int64_t V, int64_t nnz, const int32_t* labels,
                                   const float* infer_logprobs, const float* adv,
                                   const int64_t* csr_offsets_host,
                                   const int64_t* csr_offsets_dev, const int32_t* csr_ids,
                                   const float* csr_u, const float* csr_logq, int32_t replayed,
                                   int32_t* flags_dev, int32_t* flags_host, void* stream) {
  if (flags_host == nullptr) return RL_E_ARG;
  rl_status st = rl_validate_support(N, V, nnz, labels, infer_logprobs, adv, csr_offsets_host,
                                     csr_offsets_dev, csr_ids, csr_u, csr_logq, replayed,
                                     flags_dev, stream);
  if (st != RL_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RL_TRY(hipMemcpyAsync(flags_host, flags_dev, sizeof(int32_t), hipMemcpyDeviceToHost, s));
  RL_TRY(hipStreamSynchronize(s));
  return *flags_host ? RL_E_INVALID_INPUT : RL_OK;
}

}  // extern "C"
