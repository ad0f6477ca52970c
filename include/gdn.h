/*
 * gdn.h - C ABI of the MI355X (gfx950) Gated DeltaNet attention step with
 * speculative-decoding support.
 *
 * The step has two stages per token, the two ops the pages name: the
 * spec-aware causal_conv1d and the gated_delta_rule kernel fed by
 * fused_sigmoid_gating ([P1] "Changes"; [P2] overview):
 *   1. a depthwise causal conv1d of width W over the packed projections
 *      mixed_qkv = [q (Hk*dk) | k (Hk*dk) | v (Hv*dv)], reading W-1 samples of
 *      history from a per-sequence conv-state ring and rolling that ring;
 *   2. the gated delta rule on an fp32 state S in R^{dv x dk} per v-head:
 *        alpha = exp(-exp(A_log) * softplus(a + dt_bias)),  beta = sigmoid(b)
 *        S <- alpha S ;  u = beta (v - S k) ;  S <- S + u k^T ;  o = scale S q
 *      i.e. S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *      o_t = S_t q_t, with q and k L2-normalised over dk (optional) and
 *      v-head h reading k-head h / (Hv/Hk).  The pages name these ops but
 *      print neither formula; this is the recurrence and gating the library
 *      defines them as (the standard gated delta rule; background: Yang,
 *      Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025).
 *
 * Speculative-decoding semantics follow three web pages:
 *   [P1] "[GDN] Spec-decoding-aware attention kernel" (vllm-xpu-kernels
 *        pull request 336), sections "Problem" and "Changes";
 *   [P2] "[XE2] Support MTP of QWEN model" (vllm-xpu-kernels pull request
 *        368): the overview (spec/non-spec token streams, token_indx
 *        remapping), the automated review of the interface (optional tensors
 *        checked before use) and the squashed commit message (ragged spec
 *        rows; the conservation check is kept, the rectangular one dropped);
 *   [P3] "[Bugfix] Align Qwen GDN gates with speculative tokens" (vLLM pull
 *        request 51812), "Purpose": gates are read through the same indices
 *        as mixed_qkv.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous.
 *    bf16 values are passed as their 16-bit patterns (gdn_bf16).  Integers
 *    are int32; has_initial_state is one byte per row.
 *  - The caller owns every buffer, including the workspace.  The library
 *    keeps no pointer after returning and allocates no device memory.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    with no host synchronisation; faults inside kernels surface at the
 *    caller's next synchronisation.
 *  - Every call validates its host-side arguments BEFORE enqueuing anything:
 *    on error it returns a negative status, touches no buffer, and
 *    gdn_last_error() describes the problem.  Metadata VALUES that live in
 *    device memory (slots, n_acc, token rows) are not read by the host; the
 *    kernels clamp them so that out-of-range values never cause an
 *    out-of-range access (results are then unspecified).  gdn_check_metadata_host
 *    checks them on host copies.
 *  - Pools: conv_state [num_slots, state_len, C] bf16 (channel-contiguous
 *    ring, column 0 oldest; may be NULL when state_len is 0, a width-1 conv
 *    that keeps no history); ssm_state [num_slots, Hv, dv, dk] fp32.  A slot
 *    value <= 0 is NULL_BLOCK_ID / pad slot: nothing is read (zeros are used)
 *    and nothing is written [P1 "Changes"; P2 review thread].  Rows of one
 *    call must use disjoint slots.
 *  - core_attn_out [num_actual_tokens, Hv, dv] bf16: only rows named by a
 *    token_indx (or the identity mapping) are written.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t gdn_bf16;
typedef void* gdn_stream_t; /* hipStream_t */

/* Status codes. */
enum {
  GDN_OK = 0,
  GDN_ERR_NULL = -1,             /* a required pointer is NULL */
  GDN_ERR_DIMS = -2,             /* inconsistent sizes or counts */
  GDN_ERR_SPEC_PAIR = -3,        /* only one of spec_state_indices /
                                    num_accepted_tokens given [P1 "Changes"] */
  GDN_ERR_MISSING_OPTIONAL = -4, /* an optional tensor needed by the batch is
                                    absent [P2 interface review] */
  GDN_ERR_CONSERVATION = -5,     /* non-spec + spec tokens != num_actual_tokens
                                    [P2 commit message] */
  GDN_ERR_WORKSPACE = -6,        /* workspace NULL or too small */
  GDN_ERR_HIP = -7,              /* a HIP launch failed */
  GDN_ERR_UNSUPPORTED = -8,      /* shape outside what the kernels support,
                                    launch sizes included: at most 2^22
                                    workgroups per row launch (rows x
                                    k-heads, or rows x v-heads with
                                    conv_turns), 65535 64-token prefill
                                    units, 2^24 conv channels */
  GDN_ERR_METADATA = -9          /* gdn_check_metadata_host found a violation */
};

/* Channel order of mixed_qkv's rows [P1 "Test Plan", the reorder_input
 * equivalence test].  Grouped: all q heads, then all k heads, then all v
 * heads (C = 2*Hk*dk + Hv*dv), the input of the pages' reorder_input=True.
 * Per k-head: for each k-head i in turn its q (dk), its k (dk) and the v of
 * its G = Hv/Hk v-heads (G*dv), the projections as produced, read directly
 * (reorder_input=False).  Only the reads of mixed_qkv depend on it: conv
 * weights, conv bias, the conv ring and conv_out stay in grouped order. */
enum { GDN_QKV_GROUPED = 0, GDN_QKV_PER_K_HEAD = 1 };

/* Conv-state contract of spec rows ("[XE2] Support MTP of QWEN model", the
 * conv-checkpoint review thread: both can be right).  Rolled history: one
 * slot per row (spec_cache_indices[b], else spec_state_indices[b][0]) holds
 * a ring of state_len columns read at n_acc-1 and rolled.  Per-token slots:
 * each slot holds one window (state_len == conv_width-1); the window is read
 * from spec_state_indices[b][n_acc-1] and, after token t, the window ending
 * at t is written to spec_state_indices[b][t] (NULL slots skipped), as the
 * SSM states are; spec_cache_indices must then be NULL.  Non-spec rows are
 * the same under both. */
enum { GDN_CONV_ROLLED_HISTORY = 0, GDN_CONV_PER_TOKEN_SLOTS = 1 };

/* Layer shape.  Supported by the kernels: head_k_dim == head_v_dim in
 * {16, 32, 64, 128}; 1 <= conv_width <= 4; conv_width-1 <= state_len <= 16;
 * num_v_heads a multiple of num_k_heads with (Hv/Hk)*head_v_dim <= 1024. */
typedef struct gdn_dims {
  int32_t num_k_heads;   /* Hk */
  int32_t num_v_heads;   /* Hv */
  int32_t head_k_dim;    /* dk */
  int32_t head_v_dim;    /* dv */
  int32_t conv_width;    /* W */
  int32_t state_len;     /* L: ring columns per conv slot (the pool's dim 1) */
  int32_t num_slots;     /* slots in each pool (dim 0) */
  int32_t activation;    /* conv activation: 0 identity, 1 SiLU */
  int32_t use_qk_l2norm; /* 1: q, k <- x / sqrt(sum x^2 + l2norm_eps) */
  float l2norm_eps;
  float scale;           /* multiplies q after normalisation (o = scale S q) */
  int32_t qkv_layout;    /* GDN_QKV_GROUPED (0) or GDN_QKV_PER_K_HEAD (1) */
  int32_t conv_layout;   /* GDN_CONV_ROLLED_HISTORY (0) or GDN_CONV_PER_TOKEN_SLOTS (1) */
} gdn_dims;

/* Largest tokens per row in a spec call (K) and per decode row. */
#define GDN_MAX_ROW_TOKENS 16

/*
 * Graph-padded calls [P1 "Related issues": the size(0) == num_actual_tokens
 * precondition under graph capture; P2: graph-padded spec metadata].  A call
 * enqueues kernels only (no allocation, memset or host synchronisation; the
 * first call per device and kernel raises its LDS limit), so it can be
 * captured into a HIP graph.  The scalars are then frozen, so a captured
 * call is made at padded sizes: num_actual_tokens, row and token counts as
 * the graph's buffers hold them.  Rows that are padding carry NULL (<= 0)
 * slots in every index array (spec_state_indices, spec_cache_indices,
 * non-spec cache indices) and their tokens map to rows of the buffers that
 * no real token uses: they read and write no pool, and only their own
 * output rows are written.  Real rows give the same bits as an unpadded call.
 */

/*
 * gdn_spec_attention - one spec-verify step over `num_spec_decodes` rows.
 *
 * Row b owns tokens [spec_query_start_loc[b], spec_query_start_loc[b+1]) of
 * the spec token stream, 1 <= T_b <= max_spec_len (ragged rows allowed; no
 * rectangular assumption [P2 commit message]).  Stream token j lives at
 * global row spec_token_indx[j] (identity when NULL) of mixed_qkv, a, b and
 * core_attn_out [P2 overview; P3 "Purpose"].
 *
 * Conv [P1 "Changes"]: slot cs = spec_cache_indices[b] (NULL -> column 0 of
 * spec_state_indices, the column-0 contract).  With n = num_accepted_tokens[b]
 * the window is ring columns n-1 .. n+W-3 followed by the row's inputs; the
 * ring becomes columns n .. n+L-T_b-1 of the pre-state followed by the T_b
 * inputs (stage, then roll; sole writer per slot and channel).
 * SSM [P1 "Changes"]: initial state from slot spec_state_indices[b][n-1];
 * the state after token t is stored to spec_state_indices[b][t].
 * Preconditions (unchecked on device): 1 <= n <= T_b, n+W-2 <= L.
 *
 *   mixed_qkv      [num_actual_tokens, C]  C = 2*Hk*dk + Hv*dv
 *   a, b           [num_actual_tokens, Hv]
 *   conv_weight    [C, W]; conv_bias [C] or NULL
 *   A_log, dt_bias [Hv] fp32
 *   spec_state_indices [num_spec_decodes, max_spec_len] (row stride max_spec_len)
 *   num_accepted_tokens [num_spec_decodes]
 *   num_spec_tokens = spec_query_start_loc[num_spec_decodes] (host copy)
 *
 * conv_turns: NULL, or a device array of gdn_conv_turns_count(dims) uint32
 * counters, four per (conv slot, k-head), that the caller zeroes once and
 * keeps (any pools with the same dims may share one array; calls on one
 * array are ordered by the caller).  With it the step runs one workgroup
 * per (row, v-head) rather than per (row, k-head) (dk = dv = 128,
 * Hv > Hk): the G = Hv/Hk workgroups of a k-head each read
 * the shared q/k conv channels, and the last of them to have read its
 * window (told by a wrapping count, 0 .. G-1, per 64 channels) rolls them.
 * The first counter (slot 0, which names no ring) also counts, in large
 * launches (rows of two or more tokens, four or more (row, v-head) units
 * per CU), the units handed out at run time to the CUs that finish first.
 * Every call leaves every counter at 0,
 * metadata that violates the preconditions included.  The results are the
 * same bits either way.
 *
 * num_spec_decodes == 0 is a no-op that returns GDN_OK.
 */
int gdn_spec_attention(const gdn_dims* dims, const gdn_bf16* mixed_qkv,
                       const gdn_bf16* a, const gdn_bf16* b,
                       const gdn_bf16* conv_weight, const gdn_bf16* conv_bias,
                       const float* A_log, const float* dt_bias,
                       gdn_bf16* conv_state, float* ssm_state,
                       int32_t num_actual_tokens, int32_t num_spec_decodes,
                       int32_t num_spec_tokens, int32_t max_spec_len,
                       const int32_t* spec_query_start_loc,
                       const int32_t* spec_cache_indices,
                       const int32_t* spec_state_indices,
                       const int32_t* num_accepted_tokens,
                       const int32_t* spec_token_indx,
                       gdn_bf16* core_attn_out, uint32_t* conv_turns,
                       gdn_stream_t stream);

/* Number of uint32 turn counters gdn_spec_attention / gdn_attention take
 * in conv_turns: 4 * num_slots * num_k_heads (0 for invalid dims). */
size_t gdn_conv_turns_count(const gdn_dims* dims);

/*
 * gdn_attention - a whole layer step over a batch that may mix non-spec rows
 * (decodes, then prefills) and spec rows [P2 overview: the two token
 * streams; P1 "Changes": the spec tensors are optional and absent means the
 * non-spec behaviour].
 *
 * Non-spec rows: num_decodes one-token rows first, then num_prefills rows;
 * row i owns non-spec stream tokens [query_start_loc[i], query_start_loc[i+1])
 * at global rows non_spec_token_indx[j] (identity when NULL).  Slot
 * c = non_spec_state_indices[i] serves both pools; the history is read when
 * has_initial_state[i] != 0 (all rows when NULL) and c > 0.  The conv window
 * is the ring tail, the ring rolls by T_i, and only the final state is stored
 * (when c > 0).  Prefill rows run the chunked form of the recurrence; a
 * prefill row may hold no tokens (it then touches no pool).
 *
 * Spec rows: exactly as gdn_spec_attention.  spec_state_indices and
 * num_accepted_tokens must be given together or not at all (GDN_ERR_SPEC_PAIR).
 * conv_turns (NULL or as for gdn_spec_attention) serves the spec rows and
 * the decodes; a row launch that carries both (decodes and spec rows in one
 * call) runs per k-head either way, the counters untouched.
 *
 * Checks: num_non_spec_tokens + num_spec_tokens == num_actual_tokens
 * (GDN_ERR_CONSERVATION); when both streams are non-empty both token_indx
 * tensors are required.  Prefill rows need a workspace of
 * gdn_workspace_bytes(dims, num_non_spec_tokens, num_prefills) bytes.
 * Launch order: with spec rows, the prefill kernels and then one row kernel
 * for the spec rows and the decodes together; without, the decodes' row
 * kernel and then the prefill kernels.  Rows use disjoint slots, so the
 * order is not observable.
 */
int gdn_attention(const gdn_dims* dims, const gdn_bf16* mixed_qkv,
                  const gdn_bf16* a, const gdn_bf16* b,
                  const gdn_bf16* conv_weight, const gdn_bf16* conv_bias,
                  const float* A_log, const float* dt_bias,
                  gdn_bf16* conv_state, float* ssm_state,
                  int32_t num_actual_tokens,
                  int32_t num_decodes, int32_t num_prefills,
                  int32_t num_non_spec_tokens,
                  const int32_t* query_start_loc,
                  const int32_t* non_spec_state_indices,
                  const uint8_t* has_initial_state,
                  const int32_t* non_spec_token_indx,
                  int32_t num_spec_decodes, int32_t num_spec_tokens,
                  int32_t max_spec_len,
                  const int32_t* spec_query_start_loc,
                  const int32_t* spec_cache_indices,
                  const int32_t* spec_state_indices,
                  const int32_t* num_accepted_tokens,
                  const int32_t* spec_token_indx,
                  gdn_bf16* core_attn_out, uint32_t* conv_turns, void* workspace,
                  size_t workspace_bytes, gdn_stream_t stream);

/*
 * gdn_attention_static - gdn_attention for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace (the
 * caller's conv_turns array, or NULL, is used as it is).  Prefill
 * rows take their scratch from a library-owned static device array of
 * GDN_STATIC_SCRATCH_BYTES per GPU (held by each GPU the library runs on
 * until the process ends); a batch whose prefill rows need more
 * (gdn_workspace_bytes) is rejected with GDN_ERR_WORKSPACE before anything
 * is enqueued.  Nothing is allocated and nothing needs clearing.  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller.
 */
#define GDN_STATIC_SCRATCH_BYTES (64ull << 20)
int gdn_attention_static(const gdn_dims* dims, const gdn_bf16* mixed_qkv,
                         const gdn_bf16* a, const gdn_bf16* b,
                         const gdn_bf16* conv_weight, const gdn_bf16* conv_bias,
                         const float* A_log, const float* dt_bias,
                         gdn_bf16* conv_state, float* ssm_state,
                         int32_t num_actual_tokens,
                         int32_t num_decodes, int32_t num_prefills,
                         int32_t num_non_spec_tokens,
                         const int32_t* query_start_loc,
                         const int32_t* non_spec_state_indices,
                         const uint8_t* has_initial_state,
                         const int32_t* non_spec_token_indx,
                         int32_t num_spec_decodes, int32_t num_spec_tokens,
                         int32_t max_spec_len,
                         const int32_t* spec_query_start_loc,
                         const int32_t* spec_cache_indices,
                         const int32_t* spec_state_indices,
                         const int32_t* num_accepted_tokens,
                         const int32_t* spec_token_indx,
                         gdn_bf16* core_attn_out, uint32_t* conv_turns,
                         gdn_stream_t stream);

/* Bytes of workspace gdn_attention needs for a batch whose non-spec stream
 * has at most max_non_spec_tokens tokens, of which max_prefill_rows rows are
 * prefills.  0 when no prefill row is present. */
size_t gdn_workspace_bytes(const gdn_dims* dims, int32_t max_non_spec_tokens,
                           int32_t max_prefill_rows);

/*
 * Row batch for the stage entry points.  kind = GDN_ROWS_SPEC uses the spec
 * fields (state_indices is [num_rows, max_row_tokens], num_accepted_tokens,
 * cache_indices optional); kind = GDN_ROWS_NON_SPEC uses cache_indices and
 * has_initial_state (optional), one state store per row.  Stage entry
 * points take rows of at most GDN_MAX_ROW_TOKENS tokens.
 */
enum { GDN_ROWS_NON_SPEC = 0, GDN_ROWS_SPEC = 1 };
typedef struct gdn_rows {
  int32_t kind;
  int32_t num_rows;
  int32_t num_tokens;       /* = query_start_loc[num_rows] */
  int32_t max_row_tokens;   /* spec: row stride of state_indices */
  const int32_t* query_start_loc;
  const int32_t* cache_indices;
  const int32_t* state_indices;
  const int32_t* num_accepted_tokens;
  const uint8_t* has_initial_state;
  const int32_t* token_indx;
} gdn_rows;

/* Stage entry points: the conv and the delta rule as separate ops, the split
 * requested in the issue [P1] "Related issues" cites (exposing
 * causal_conv1d and gated_delta_rule as standalone ops, #189; the pull
 * request itself keeps the single op, here gdn_attention).
 * gdn_conv_only runs the conv with the rows' window rule, rolls the rings and
 * writes the fp32 conv output of each token to conv_out[global row][C].
 * gdn_delta_rule_only reads conv_out at the same rows and runs gates, norms
 * and the recurrence with the rows' slot rule.  Calling the two in order
 * gives bit-for-bit the result of the fused entry points. */
int gdn_conv_only(const gdn_dims* dims, const gdn_bf16* mixed_qkv,
                  const gdn_bf16* conv_weight, const gdn_bf16* conv_bias,
                  gdn_bf16* conv_state, int32_t num_actual_tokens,
                  const gdn_rows* rows, float* conv_out, gdn_stream_t stream);
int gdn_delta_rule_only(const gdn_dims* dims, const float* conv_out,
                        const gdn_bf16* a, const gdn_bf16* b,
                        const float* A_log, const float* dt_bias,
                        float* ssm_state, int32_t num_actual_tokens,
                        const gdn_rows* rows, gdn_bf16* core_attn_out,
                        gdn_stream_t stream);

/* A host array for gdn_check_metadata_host: `len` int32 values readable at
 * `data` (NULL with len 0 when the tensor is absent). */
typedef struct gdn_host_i32 {
  const int32_t* data;
  int64_t len;
} gdn_host_i32;

/*
 * gdn_check_metadata_host - validate metadata VALUES on host copies of the
 * tensors, with the meaning they have in gdn_attention (spec rows: as in
 * gdn_spec_attention).  Any group may be absent by passing 0 rows.
 *
 * Every array comes with its length, and each length is checked against
 * what the counts require BEFORE any element is read: query_start_loc
 * >= rows+1, non_spec_state_indices >= rows, non_spec_token_indx >=
 * num_non_spec_tokens, spec_query_start_loc >= num_spec_decodes+1,
 * spec_state_indices >= num_spec_decodes*max_spec_len, num_accepted_tokens
 * and spec_cache_indices >= num_spec_decodes, spec_token_indx >=
 * num_spec_tokens.  A short array is a GDN_ERR_DIMS; the function never
 * reads past `len`.
 *
 * Value checks: query_start_loc starts at 0, is non-decreasing (a prefill
 * row may be empty) and ends at num_non_spec_tokens; decode rows hold one
 * token; spec_query_start_loc starts at 0 and ends at num_spec_tokens; spec
 * rows hold 1..max_spec_len tokens; 1 <= n_acc <= T_b and (rolled history)
 * n_acc + W - 2 <= state_len; slots < num_slots; token rows in
 * [0, num_actual_tokens) and distinct across both streams (the identity
 * mapping when a token_indx is absent); slots of different rows disjoint;
 * num_non_spec_tokens + num_spec_tokens <= num_actual_tokens, with equality
 * when there are non-spec rows (the conservation rule of gdn_attention
 * ["[XE2] Support MTP of QWEN model", commit message]).  Returns GDN_OK,
 * GDN_ERR_DIMS (a count or length) or GDN_ERR_METADATA (a value), with
 * gdn_last_error() naming the first violation.  Host memory only; no HIP call.
 */
int gdn_check_metadata_host(const gdn_dims* dims, int32_t num_actual_tokens,
                            int32_t num_decodes, int32_t num_prefills,
                            int32_t num_non_spec_tokens,
                            gdn_host_i32 query_start_loc,
                            gdn_host_i32 non_spec_state_indices,
                            gdn_host_i32 non_spec_token_indx,
                            int32_t num_spec_decodes, int32_t num_spec_tokens,
                            int32_t max_spec_len,
                            gdn_host_i32 spec_query_start_loc,
                            gdn_host_i32 spec_cache_indices,
                            gdn_host_i32 spec_state_indices,
                            gdn_host_i32 num_accepted_tokens,
                            gdn_host_i32 spec_token_indx);

/* Human-readable status; never NULL. */
const char* gdn_status_string(int status);
/* Message of the last failing call on this thread ("" if none). */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
