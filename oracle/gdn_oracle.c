/*
 * Plain CPU oracle for the speculative-decoding-aware Gated DeltaNet (GDN)
 * attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP library: it is a separate, slow,
 * obviously-correct restatement of what the step computes, used to check
 * the GPU path.  All floating-point arithmetic is done in double precision;
 * the only roundings are the ones the storage formats impose:
 *   - the SSM state is an fp32 quantity, so after every token the updated
 *     state is rounded to fp32 (this is also what is written to the pool);
 *   - core_attn_out is bf16, rounded to nearest-even from the double result;
 *   - the conv-state ring holds bf16 inputs, moved bit-for-bit.
 * The conv output is NOT re-quantised before the recurrence (kept in double
 * here, fp32 on the GPU).
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "[GDN] Spec-decoding-aware attention kernel" (vllm-xpu-kernels
 *        pull request 336): sections "Problem", "Changes", "Test Plan".
 *   [P2] "[XE2] Support MTP of QWEN model" (vllm-xpu-kernels pull request
 *        368): the pull-request overview, the review comments on the
 *        interface, the conv-checkpoint review thread and the squashed
 *        commit message (ragged spec rows, conservation check).
 *   [P3] "[Bugfix] Align Qwen GDN gates with speculative tokens" (vLLM pull
 *        request 51812): "Purpose" (gates gathered with the same indices as
 *        mixed_qkv).
 *   The recurrence and the gates.  [P1] "Changes" names the ops (the
 *        gated_delta_rule kernel, fed by "fused_sigmoid_gating") but prints
 *        no formula.  The oracle computes them as the gated delta rule
 *        S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t,
 *        with decay a_t = exp(-exp(A_log) softplus(a+dt_bias)) and write
 *        strength b_t = sigmoid(b): the definition this step is built to
 *        (background: Yang, Kautz, Hatamizadeh, "Gated Delta Networks:
 *        Improving Mamba2 with Delta Rule", ICLR 2025).
 *
 * Readings where the pages are silent (each one is listed in the design
 * notes with its reason):
 *   - state orientation S in R^{dv x dk}, pool layout [slot][Hv][dv][dk];
 *   - q and k are L2-normalised over dk (eps inside the square root), then q
 *     is multiplied by `scale`;
 *   - conv taps: w[c][W-1] multiplies the newest input (cross-correlation
 *     with W-1 samples of history), optional bias, optional SiLU;
 *   - softplus(x) = x for x > 20, else log1p(exp(x));
 *   - GQA: v-head h reads k-head floor(h / (Hv/Hk));
 *   - non-spec rows read the conv window at the ring tail and roll by T_i;
 *   - with per-token checkpoint slots (conv_layout 1) a spec row's conv slots
 *     are its SSM slots, each holding one window (state_len == W-1), and
 *     spec_cache_indices is not used;
 *   - a slot value <= 0 (NULL_BLOCK_ID / pad slot) means "no prior state":
 *     zeros are read and nothing is written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct oracle_dims {
  int32_t num_k_heads;  /* Hk */
  int32_t num_v_heads;  /* Hv */
  int32_t head_k_dim;   /* dk */
  int32_t head_v_dim;   /* dv */
  int32_t conv_width;   /* W  */
  int32_t state_len;    /* L  : ring columns per conv slot */
  int32_t num_slots;    /* slots in both pools */
  int32_t activation;   /* 0 identity, 1 SiLU */
  int32_t use_qk_l2norm;
  int32_t conv_layout;  /* 0 rolled history, 1 per-token checkpoint slots */
  double l2norm_eps;
  double scale;
} oracle_dims;

enum {
  ORACLE_OK = 0,
  ORACLE_ERR_DIMS = -1,
  ORACLE_ERR_META = -2,
  ORACLE_ERR_ALLOC = -3
};

/* ---- storage-format conversions ---------------------------------------- */

/* bf16 -> double is exact: a bf16 value is the top half of an IEEE single. */
static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* double -> bf16, round to nearest, ties to even, computed on the value
 * itself: bf16 keeps 8 significant bits, so the spacing in the binade
 * [2^(e-1), 2^e) is 2^(e-8), and 2^-133 below the smallest normal 2^-126. */
static uint16_t bf16_round(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double ax = fabs(x);
  if (ax == 0.0) return sign;
  if (isinf(ax)) return sign | 0x7F80;
  int e;
  (void)frexp(ax, &e);
  int q = e - 8;
  if (q < -133) q = -133;
  double r = nearbyint(ldexp(ax, -q)); /* default mode: ties to even */
  double v = ldexp(r, q);
  if (v >= ldexp(1.0, 128)) return sign | 0x7F80;
  float f = (float)v; /* exact: v is a bf16 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return sign | (uint16_t)(u >> 16);
}

/* ---- gates -------------------------------------------------------------- */

static double softplus(double x) { return x > 20.0 ? x : log1p(exp(x)); }

/* Decay and write strength of one (token, v-head) (the gates defined in the header); the gate rows are
 * read at the same global row as mixed_qkv [P3 "Purpose"]. */
static void gates_one(uint16_t a_raw, uint16_t b_raw, double A_log,
                      double dt_bias, double* alpha, double* beta) {
  double x = bf16_value(a_raw) + dt_bias;
  *alpha = exp(-exp(A_log) * softplus(x));
  *beta = 1.0 / (1.0 + exp(-bf16_value(b_raw)));
}

/* Exported for the closed-form checks: n gate pairs, head of item t is
 * t % num_v_heads. */
int oracle_gates(int32_t n, int32_t num_v_heads, const uint16_t* a,
                 const uint16_t* b, const float* A_log, const float* dt_bias,
                 double* alpha, double* beta) {
  if (n < 0 || num_v_heads <= 0) return ORACLE_ERR_DIMS;
  for (int32_t t = 0; t < n; ++t) {
    int32_t h = t % num_v_heads;
    gates_one(a[t], b[t], (double)A_log[h], (double)dt_bias[h], &alpha[t],
              &beta[t]);
  }
  return ORACLE_OK;
}

/* ---- shared pieces of one row ------------------------------------------ */

static int dims_ok(const oracle_dims* d) {
  if (!d) return 0;
  if (d->num_k_heads <= 0 || d->num_v_heads <= 0) return 0;
  if (d->num_v_heads % d->num_k_heads) return 0;
  if (d->head_k_dim <= 0 || d->head_v_dim <= 0) return 0;
  if (d->conv_width < 1 || d->state_len < d->conv_width - 1) return 0;
  if (d->num_slots <= 0) return 0;
  if (d->conv_layout != 0 && d->conv_layout != 1) return 0;
  return 1;
}

static int64_t conv_channels(const oracle_dims* d) {
  return 2LL * d->num_k_heads * d->head_k_dim +
         (int64_t)d->num_v_heads * d->head_v_dim;
}

/*
 * Causal depthwise conv of one row, channel by channel, plus the ring roll.
 *   H[l]   : pre-state ring column l of slot `slot` (zeros if !read_hist)
 *   window : H[off .. off+W-2] followed by the row's inputs x_0..x_{T-1}
 *   y_j[c] = act(bias_c + sum_m w[c][m] * window[j+m])
 *   new ring column l = H[shift+l] for l < L-T, else x_{l-(L-T)}
 * Spec rows use off = n_acc-1 and shift = n_acc [P1 "Changes": load shift
 * n_acc-1 at cache_indices column 0, two-pass stage-then-roll with the
 * current input at column state_len-K_call+t]; non-spec rows use the ring
 * tail off = L-W+1 and shift = T.  All reads of H precede the writes.
 * y is written as double into y[j*C + c].
 */
static void conv_row(const oracle_dims* d, const uint16_t* mixed_qkv,
                     const int32_t* rows, int32_t T, const uint16_t* w,
                     const uint16_t* bias, uint16_t* conv_state, int32_t slot,
                     int read_hist, int32_t off, int32_t shift, double* y) {
  const int64_t C = conv_channels(d);
  const int32_t L = d->state_len, W = d->conv_width;
  uint16_t* H = (uint16_t*)calloc((size_t)L, sizeof(uint16_t));
  uint16_t* xs = (uint16_t*)calloc((size_t)(W - 1 + T), sizeof(uint16_t));
  for (int64_t c = 0; c < C; ++c) {
    for (int32_t l = 0; l < L; ++l)
      H[l] = (read_hist && slot > 0)
                 ? conv_state[((int64_t)slot * L + l) * C + c]
                 : (uint16_t)0;
    for (int32_t m = 0; m < W - 1; ++m) xs[m] = H[off + m];
    for (int32_t j = 0; j < T; ++j)
      xs[W - 1 + j] = mixed_qkv[(int64_t)rows[j] * C + c];
    double bc = bias ? bf16_value(bias[c]) : 0.0;
    for (int32_t j = 0; j < T; ++j) {
      double acc = bc;
      for (int32_t m = 0; m < W; ++m)
        acc += bf16_value(w[c * W + m]) * bf16_value(xs[j + m]);
      if (d->activation == 1) acc = acc / (1.0 + exp(-acc));
      y[(int64_t)j * C + c] = acc;
    }
    if (slot > 0) {
      for (int32_t l = 0; l < L; ++l) {
        uint16_t v = (l < L - T) ? H[shift + l]
                                 : mixed_qkv[(int64_t)rows[l - (L - T)] * C + c];
        conv_state[((int64_t)slot * L + l) * C + c] = v;
      }
    }
  }
  free(H);
  free(xs);
}

/*
 * Conv of one spec row with per-token checkpoint slots ("[XE2] Support MTP
 * of QWEN model", review of the spec conv kernel: the conv state is saved
 * after every spec token into that token's cache slot, as the SSM states
 * are).  A slot holds one window: its columns 0..W-2 are the last W-1 conv
 * inputs, oldest first (state_len == W-1).  The window before the row's
 * first token is read from slot load_slot (zeros if <= 0); after token j
 * the last W-1 samples of (window ++ inputs 0..j) go to save_slots[j] when
 * that is > 0, in token order.  Every read of a channel precedes its writes.
 */
static void conv_row_per_token(const oracle_dims* d, const uint16_t* mixed_qkv,
                               const int32_t* rows, int32_t T, const uint16_t* w,
                               const uint16_t* bias, uint16_t* conv_state,
                               int32_t load_slot, const int32_t* save_slots, double* y) {
  const int64_t C = conv_channels(d);
  const int32_t L = d->state_len, W = d->conv_width;
  uint16_t* xs = (uint16_t*)calloc((size_t)(W - 1 + T), sizeof(uint16_t));
  for (int64_t c = 0; c < C; ++c) {
    for (int32_t m = 0; m < W - 1; ++m)
      xs[m] = load_slot > 0 ? conv_state[((int64_t)load_slot * L + m) * C + c] : (uint16_t)0;
    for (int32_t j = 0; j < T; ++j)
      xs[W - 1 + j] = mixed_qkv[(int64_t)rows[j] * C + c];
    double bc = bias ? bf16_value(bias[c]) : 0.0;
    for (int32_t j = 0; j < T; ++j) {
      double acc = bc;
      for (int32_t m = 0; m < W; ++m)
        acc += bf16_value(w[c * W + m]) * bf16_value(xs[j + m]);
      if (d->activation == 1) acc = acc / (1.0 + exp(-acc));
      y[(int64_t)j * C + c] = acc;
    }
    for (int32_t j = 0; j < T; ++j) {
      if (save_slots[j] <= 0) continue;
      for (int32_t m = 0; m < W - 1; ++m)
        conv_state[((int64_t)save_slots[j] * L + m) * C + c] = xs[j + 1 + m];
    }
  }
  free(xs);
}

/*
 * Gated delta rule over the T tokens of one row, for every v-head (the recurrence defined in the header):
 *   S <- alpha S ;  p = S k ;  u = beta (v - p) ;  S <- S + u k^T
 *   (this equals alpha S (I - beta k k^T) + beta v k^T), the state is then
 *   rounded to fp32, and o = scale * S q is written as bf16 at row rows[j].
 * The initial state comes from slot `load_slot` (zeros if <= 0).  After token
 * j the state is written to store_slot(j) when that is > 0: for spec rows
 * store_slot(j) = spec_state_indices[b][j] [P1 "Changes": per-token store
 * slot, raw value <= 0 is NULL_BLOCK_ID]; for non-spec rows only the final
 * state is stored.  The load happens before any store.
 */
static void delta_rule_row(const oracle_dims* d, const double* y,
                           const int32_t* rows, int32_t T, const uint16_t* a,
                           const uint16_t* b, const float* A_log,
                           const float* dt_bias, float* ssm_state,
                           int32_t load_slot, const int32_t* store_slots,
                           uint16_t* core_attn_out) {
  const int32_t Hk = d->num_k_heads, Hv = d->num_v_heads;
  const int32_t dk = d->head_k_dim, dv = d->head_v_dim;
  const int32_t G = Hv / Hk;
  const int64_t C = conv_channels(d);
  const int64_t tile = (int64_t)dv * dk;
  double* S = (double*)malloc(sizeof(double) * (size_t)tile);
  double* q = (double*)malloc(sizeof(double) * (size_t)dk);
  double* k = (double*)malloc(sizeof(double) * (size_t)dk);
  for (int32_t h = 0; h < Hv; ++h) {
    const int32_t ih = h / G;
    if (load_slot > 0) {
      const float* src = ssm_state + ((int64_t)load_slot * Hv + h) * tile;
      for (int64_t e = 0; e < tile; ++e) S[e] = (double)src[e];
    } else {
      for (int64_t e = 0; e < tile; ++e) S[e] = 0.0;
    }
    for (int32_t j = 0; j < T; ++j) {
      const double* yj = y + (int64_t)j * C;
      const double* qsrc = yj + (int64_t)ih * dk;
      const double* ksrc = yj + (int64_t)Hk * dk + (int64_t)ih * dk;
      const double* vsrc = yj + 2LL * Hk * dk + (int64_t)h * dv;
      double qq = 0.0, kk = 0.0;
      for (int32_t c = 0; c < dk; ++c) {
        qq += qsrc[c] * qsrc[c];
        kk += ksrc[c] * ksrc[c];
      }
      double qn = 1.0, kn = 1.0;
      if (d->use_qk_l2norm) {
        qn = 1.0 / sqrt(qq + d->l2norm_eps);
        kn = 1.0 / sqrt(kk + d->l2norm_eps);
      }
      for (int32_t c = 0; c < dk; ++c) {
        q[c] = qsrc[c] * qn;
        k[c] = ksrc[c] * kn;
      }
      double alpha, beta;
      gates_one(a[(int64_t)rows[j] * Hv + h], b[(int64_t)rows[j] * Hv + h],
                (double)A_log[h], (double)dt_bias[h], &alpha, &beta);
      uint16_t* o = core_attn_out + ((int64_t)rows[j] * Hv + h) * dv;
      for (int32_t r = 0; r < dv; ++r) {
        double* Sr = S + (int64_t)r * dk;
        double p = 0.0;
        for (int32_t c = 0; c < dk; ++c) {
          Sr[c] *= alpha;
          p += Sr[c] * k[c];
        }
        double u = beta * (vsrc[r] - p);
        double acc = 0.0;
        for (int32_t c = 0; c < dk; ++c) {
          Sr[c] = (double)(float)(Sr[c] + u * k[c]);
          acc += Sr[c] * q[c];
        }
        o[r] = bf16_round(d->scale * acc);
      }
      int32_t st = store_slots[j];
      if (st > 0) {
        float* dst = ssm_state + ((int64_t)st * Hv + h) * tile;
        for (int64_t e = 0; e < tile; ++e) dst[e] = (float)S[e];
      }
    }
  }
  free(S);
  free(q);
  free(k);
}

/* ---- spec-verify step --------------------------------------------------- */

/*
 * One spec-verify call over num_spec_decodes rows [P1 "Changes", P2 overview
 * and commit message, P3 "Purpose"]:
 *   row b holds tokens [spec_query_start_loc[b], spec_query_start_loc[b+1])
 *   of the spec stream (ragged rows allowed, no rectangular assumption);
 *   token j of the stream lives at global row spec_token_indx[j] (identity
 *   when NULL) of mixed_qkv, a, b and core_attn_out;
 *   conv slot = spec_cache_indices[b] (or spec_state_indices[b][0]);
 *   n = num_accepted_tokens[b]; window offset n-1, roll shift n;
 *   SSM load slot spec_state_indices[b][n-1], store slot [b][j].
 * conv_out (nullable) receives the conv output of each token at its global
 * row, [num_actual_tokens, C] doubles.
 * Preconditions checked here: 1 <= T_b <= K, 1 <= n <= T_b,
 * n-1 + W-1 <= L, slots < num_slots, rows in [0, num_actual_tokens).
 */
int oracle_spec_step(const oracle_dims* d, const uint16_t* mixed_qkv,
                     const uint16_t* a, const uint16_t* b,
                     const uint16_t* conv_weight, const uint16_t* conv_bias,
                     const float* A_log, const float* dt_bias,
                     uint16_t* conv_state, float* ssm_state,
                     int32_t num_actual_tokens, int32_t num_spec_decodes,
                     int32_t K, const int32_t* spec_query_start_loc,
                     const int32_t* spec_cache_indices,
                     const int32_t* spec_state_indices,
                     const int32_t* num_accepted_tokens,
                     const int32_t* spec_token_indx, uint16_t* core_attn_out,
                     double* conv_out) {
  if (!dims_ok(d) || K <= 0 || num_spec_decodes < 0) return ORACLE_ERR_DIMS;
  const int64_t C = conv_channels(d);
  const int32_t L = d->state_len, W = d->conv_width;
  double* y = (double*)malloc(sizeof(double) * (size_t)(C * K));
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
  int32_t* stores = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
  if (!y || !rows || !stores) {
    free(y); free(rows); free(stores);
    return ORACLE_ERR_ALLOC;
  }
  int status = ORACLE_OK;
  for (int32_t bi = 0; bi < num_spec_decodes && status == ORACLE_OK; ++bi) {
    const int32_t j0 = spec_query_start_loc[bi];
    const int32_t T = spec_query_start_loc[bi + 1] - j0;
    const int32_t n = num_accepted_tokens[bi];
    const int32_t* ssi = spec_state_indices + (int64_t)bi * K;
    const int32_t cs = spec_cache_indices ? spec_cache_indices[bi] : ssi[0];
    const int per_token = d->conv_layout == 1;
    if (per_token && (spec_cache_indices || L != W - 1)) {
      status = ORACLE_ERR_DIMS;
      break;
    }
    if (T < 1 || T > K || n < 1 || n > T || (!per_token && n - 1 + W - 1 > L) ||
        cs >= d->num_slots) {
      status = ORACLE_ERR_META;
      break;
    }
    for (int32_t j = 0; j < T; ++j) {
      rows[j] = spec_token_indx ? spec_token_indx[j0 + j] : j0 + j;
      stores[j] = ssi[j];
      if (rows[j] < 0 || rows[j] >= num_actual_tokens ||
          ssi[j] >= d->num_slots)
        status = ORACLE_ERR_META;
    }
    if (status != ORACLE_OK) break;
    if (per_token)
      conv_row_per_token(d, mixed_qkv, rows, T, conv_weight, conv_bias, conv_state,
                         ssi[n - 1], stores, y);
    else
      conv_row(d, mixed_qkv, rows, T, conv_weight, conv_bias, conv_state, cs,
               /*read_hist=*/1, /*off=*/n - 1, /*shift=*/n, y);
    if (conv_out)
      for (int32_t j = 0; j < T; ++j)
        memcpy(conv_out + (int64_t)rows[j] * C, y + (int64_t)j * C,
               sizeof(double) * (size_t)C);
    delta_rule_row(d, y, rows, T, a, b, A_log, dt_bias, ssm_state, ssi[n - 1],
                   stores, core_attn_out);
  }
  free(y);
  free(rows);
  free(stores);
  return status;
}

/* ---- non-spec step (decodes and prefills) ------------------------------ */

/*
 * Non-spec rows [P2 overview: the non-spec token stream; P1 "Changes": the
 * non-spec path is unchanged]: row i holds tokens
 * [query_start_loc[i], query_start_loc[i+1]) of the non-spec stream, at
 * global rows token_indx[j] (identity when NULL).  Slot c = cache_indices[i]
 * serves both pools; init = has_initial_state[i] (1 when NULL) and c > 0.
 * The conv window is the ring tail, the ring rolls by T_i, and only the final
 * state is stored to slot c (when c > 0).  Every row runs the sequential
 * recurrence, whatever its length.
 */
int oracle_nonspec_step(const oracle_dims* d, const uint16_t* mixed_qkv,
                        const uint16_t* a, const uint16_t* b,
                        const uint16_t* conv_weight, const uint16_t* conv_bias,
                        const float* A_log, const float* dt_bias,
                        uint16_t* conv_state, float* ssm_state,
                        int32_t num_actual_tokens, int32_t num_rows,
                        const int32_t* query_start_loc,
                        const int32_t* cache_indices,
                        const uint8_t* has_initial_state,
                        const int32_t* token_indx, uint16_t* core_attn_out,
                        double* conv_out) {
  if (!dims_ok(d) || num_rows < 0) return ORACLE_ERR_DIMS;
  const int64_t C = conv_channels(d);
  const int32_t L = d->state_len, W = d->conv_width;
  int status = ORACLE_OK;
  for (int32_t i = 0; i < num_rows && status == ORACLE_OK; ++i) {
    const int32_t j0 = query_start_loc[i];
    const int32_t T = query_start_loc[i + 1] - j0;
    const int32_t c = cache_indices[i];
    if (T < 0 || c >= d->num_slots) {
      status = ORACLE_ERR_META;
      break;
    }
    if (T == 0) continue;
    const int init = (has_initial_state ? has_initial_state[i] != 0 : 1) && c > 0;
    double* y = (double*)malloc(sizeof(double) * (size_t)(C * T));
    int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
    int32_t* stores = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
    if (!y || !rows || !stores) {
      free(y); free(rows); free(stores);
      return ORACLE_ERR_ALLOC;
    }
    for (int32_t j = 0; j < T; ++j) {
      rows[j] = token_indx ? token_indx[j0 + j] : j0 + j;
      stores[j] = (j == T - 1) ? c : 0;
      if (rows[j] < 0 || rows[j] >= num_actual_tokens) status = ORACLE_ERR_META;
    }
    if (status == ORACLE_OK) {
      conv_row(d, mixed_qkv, rows, T, conv_weight, conv_bias, conv_state, c,
               init, /*off=*/L - W + 1, /*shift=*/T, y);
      if (conv_out)
        for (int32_t j = 0; j < T; ++j)
          memcpy(conv_out + (int64_t)rows[j] * C, y + (int64_t)j * C,
                 sizeof(double) * (size_t)C);
      delta_rule_row(d, y, rows, T, a, b, A_log, dt_bias, ssm_state,
                     init ? c : 0, stores, core_attn_out);
    }
    free(y);
    free(rows);
    free(stores);
  }
  return status;
}

/* Exposed so tests can pin the rounding against numpy's float32 path. */
uint16_t oracle_bf16_round(double x) { return bf16_round(x); }
