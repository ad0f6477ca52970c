// C ABI of the GDN step: argument validation, dispatch to the HIP kernels,
// status strings.  Validation is host-only and runs before any HIP call, so
// a rejected call enqueues nothing and touches no buffer.
//
// The interface rules come from the pages:
//  - the two spec tensors travel together ("[GDN] Spec-decoding-aware
//    attention kernel", "Changes": mismatched pairs are rejected);
//  - every optional tensor the batch needs is checked for presence before
//    use ("[XE2] Support MTP of QWEN model", automated review of the
//    interface);
//  - non-spec tokens + spec tokens == num_actual_tokens, with no rectangular
//    spec_token == num_spec_decodes * K check (same page, commit message).
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <set>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace

namespace gdn {
hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes) {
  // (kernel, device) pairs whose limit is already at least `bytes`
  struct Entry { const void* k; int dev; size_t bytes; };
  static std::mutex mu;
  static std::vector<Entry> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& x : done)
    if (x.k == kernel && x.dev == dev && x.bytes >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done.push_back({kernel, dev, bytes});
  return e;
}
hipError_t device_cu_count(int* cus) {
  static std::mutex mu;
  static std::vector<int> count;  // by device, 0 until queried
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= (int)count.size()) count.resize(dev + 1, 0);
  if (count[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    count[dev] = n > 0 ? n : 1;
  }
  *cus = count[dev];
  return hipSuccess;
}
}  // namespace gdn

namespace {

// Launch limits: a row launch is one workgroup of up to 1024 threads per
// (row, k-head) and a dispatch holds fewer than 2^32 work-items; the chunk
// kernels put the 64-token units of the prefill rows on grid dimension y,
// which holds at most 65535.
constexpr int kMaxConvDim = 1 << 24;
constexpr long long kMaxRowWorkgroups = 1LL << 22;
constexpr long long kMaxPrefillUnits = 65535;

int check_dims(const gdn_dims* d) {
  if (!d) return fail(GDN_ERR_NULL, "dims is NULL");
  if (d->num_k_heads <= 0 || d->num_v_heads <= 0)
    return fail(GDN_ERR_DIMS, "head counts must be positive (Hk=%d, Hv=%d)",
                d->num_k_heads, d->num_v_heads);
  if (d->num_v_heads % d->num_k_heads)
    return fail(GDN_ERR_DIMS, "num_v_heads (%d) must be a multiple of num_k_heads (%d)",
                d->num_v_heads, d->num_k_heads);
  if (d->head_k_dim != d->head_v_dim)
    return fail(GDN_ERR_UNSUPPORTED, "head_k_dim (%d) != head_v_dim (%d) is not supported",
                d->head_k_dim, d->head_v_dim);
  switch (d->head_k_dim) {
    case 16: case 32: case 64: case 128: break;
    default:
      return fail(GDN_ERR_UNSUPPORTED, "head dim %d not in {16,32,64,128}", d->head_k_dim);
  }
  if (d->conv_width < 1 || d->conv_width > gdn::kMaxWidth)
    return fail(GDN_ERR_UNSUPPORTED, "conv_width %d not in [1,4]", d->conv_width);
  if (d->state_len < d->conv_width - 1 || d->state_len > gdn::kMaxStateLen)
    return fail(GDN_ERR_DIMS, "state_len %d not in [conv_width-1, 16]", d->state_len);
  if (d->num_slots <= 0) return fail(GDN_ERR_DIMS, "num_slots must be positive");
  if (d->activation != 0 && d->activation != 1)
    return fail(GDN_ERR_DIMS, "activation must be 0 (identity) or 1 (SiLU)");
  if (d->use_qk_l2norm != 0 && d->use_qk_l2norm != 1)
    return fail(GDN_ERR_DIMS, "use_qk_l2norm must be 0 or 1");
  if (!(d->l2norm_eps >= 0.f)) return fail(GDN_ERR_DIMS, "l2norm_eps must be >= 0");
  if (d->qkv_layout != GDN_QKV_GROUPED && d->qkv_layout != GDN_QKV_PER_K_HEAD)
    return fail(GDN_ERR_DIMS, "qkv_layout must be GDN_QKV_GROUPED (0) or GDN_QKV_PER_K_HEAD (1)");
  if (d->conv_layout != GDN_CONV_ROLLED_HISTORY && d->conv_layout != GDN_CONV_PER_TOKEN_SLOTS)
    return fail(GDN_ERR_DIMS, "conv_layout must be GDN_CONV_ROLLED_HISTORY (0) or "
                              "GDN_CONV_PER_TOKEN_SLOTS (1)");
  if (d->conv_layout == GDN_CONV_PER_TOKEN_SLOTS && d->state_len != d->conv_width - 1)
    return fail(GDN_ERR_DIMS, "per-token conv slots hold one window: state_len must be "
                              "conv_width-1 (%d), got %d", d->conv_width - 1, d->state_len);
  const int G = d->num_v_heads / d->num_k_heads;
  if (G * d->head_v_dim > 1024)
    return fail(GDN_ERR_UNSUPPORTED, "(Hv/Hk)*head_v_dim = %d exceeds 1024", G * d->head_v_dim);
  // channel indices are 32-bit inside the kernels
  const long long C = (long long)d->num_k_heads * (2 * d->head_k_dim + G * d->head_v_dim);
  if (C > kMaxConvDim)
    return fail(GDN_ERR_UNSUPPORTED, "conv dim %lld exceeds %d channels", C, kMaxConvDim);
  return GDN_OK;
}

int conv_dim(const gdn_dims* d) {
  return 2 * d->num_k_heads * d->head_k_dim + d->num_v_heads * d->head_v_dim;
}

void fill_common(gdn::RowArgs& a, const gdn_dims* d, int num_actual_tokens) {
  a = gdn::RowArgs{};
  a.Hk = d->num_k_heads;
  a.Hv = d->num_v_heads;
  a.G = d->num_v_heads / d->num_k_heads;
  a.C = conv_dim(d);
  a.L = d->state_len;
  a.W = d->conv_width;
  a.num_slots = d->num_slots;
  a.act = d->activation;
  a.l2norm = d->use_qk_l2norm;
  a.qkv_layout = d->qkv_layout;
  a.conv_per_token = d->conv_layout == GDN_CONV_PER_TOKEN_SLOTS;
  a.eps = d->l2norm_eps;
  a.scale = d->scale;
  a.num_actual_tokens = num_actual_tokens;
}

int rows_launch_ok(const gdn::RowArgs& a, const gdn_dims* d) {
  // with turn counters the rows may run one workgroup per (row, v-head)
  const long long wgs = ((long long)a.num_rows + (a.more.num_rows > 0 ? a.more.num_rows : 0)) *
                        (a.turns ? a.Hv : a.Hk);
  if (wgs > kMaxRowWorkgroups)
    return fail(GDN_ERR_UNSUPPORTED, "row launch of %lld workgroups (rows x %s) exceeds %lld", wgs,
                a.turns ? "v-heads" : "k-heads", kMaxRowWorkgroups);
  size_t need = gdn::rows_lds_bytes(a, d->head_k_dim, d->head_v_dim);
  if (need > 160 * 1024)
    return fail(GDN_ERR_UNSUPPORTED, "row kernel needs %zu bytes of LDS (max 163840)", need);
  return GDN_OK;
}

int launch(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return GDN_OK;
}

// Shared by gdn_spec_attention and gdn_attention.
struct SpecBatch {
  int num_spec_decodes, num_spec_tokens, max_spec_len;
  const int32_t *sqsl, *cache, *ssi, *nacc, *tix;
};

int check_spec(const SpecBatch& s, int num_actual_tokens) {
  if ((s.ssi == nullptr) != (s.nacc == nullptr))
    return fail(GDN_ERR_SPEC_PAIR,
                "spec_state_indices and num_accepted_tokens must be given together");
  if (s.num_spec_decodes < 0 || s.num_spec_tokens < 0)
    return fail(GDN_ERR_DIMS, "negative spec counts");
  if (s.num_spec_decodes == 0) {
    if (s.num_spec_tokens != 0)
      return fail(GDN_ERR_DIMS, "num_spec_tokens=%d with no spec rows", s.num_spec_tokens);
    return GDN_OK;
  }
  if (!s.ssi) return fail(GDN_ERR_MISSING_OPTIONAL, "spec rows need spec_state_indices");
  if (!s.sqsl) return fail(GDN_ERR_MISSING_OPTIONAL, "spec rows need spec_query_start_loc");
  if (s.max_spec_len < 1 || s.max_spec_len > gdn::kMaxRowTokens)
    return fail(GDN_ERR_UNSUPPORTED, "max_spec_len %d not in [1,%d]", s.max_spec_len,
                gdn::kMaxRowTokens);
  if (s.num_spec_tokens > num_actual_tokens)
    return fail(GDN_ERR_DIMS, "num_spec_tokens %d > num_actual_tokens %d",
                s.num_spec_tokens, num_actual_tokens);
  if ((long long)s.num_spec_tokens > (long long)s.num_spec_decodes * s.max_spec_len)
    return fail(GDN_ERR_DIMS, "num_spec_tokens %d exceeds num_spec_decodes*max_spec_len",
                s.num_spec_tokens);
  return GDN_OK;
}

// conv_state may be NULL when state_len is 0 (a width-1 conv keeps no
// history: the pool has no bytes and is never touched).
int check_layer_ptrs(const gdn_dims* d, const void* qkv, const void* a, const void* b,
                     const void* w, const void* A_log, const void* dt_bias,
                     const void* conv_state, const void* ssm_state, const void* out) {
  if (!qkv) return fail(GDN_ERR_NULL, "mixed_qkv is NULL");
  if (!a || !b) return fail(GDN_ERR_NULL, "gate tensors a/b are NULL");
  if (!w) return fail(GDN_ERR_NULL, "conv_weight is NULL");
  if (!A_log || !dt_bias) return fail(GDN_ERR_NULL, "A_log/dt_bias is NULL");
  if ((!conv_state && d->state_len > 0) || !ssm_state)
    return fail(GDN_ERR_NULL, "state pool is NULL");
  if (!out) return fail(GDN_ERR_NULL, "core_attn_out is NULL");
  return GDN_OK;
}

struct Layer {
  const gdn_dims* d;
  const gdn_bf16 *qkv, *a, *b, *w, *bias;
  const float *A_log, *dt_bias;
  gdn_bf16* conv_state;
  float* ssm_state;
  gdn_bf16* out;
  int num_actual_tokens;
  uint32_t* turns;
};

void fill_layer(gdn::RowArgs& r, const Layer& L) {
  fill_common(r, L.d, L.num_actual_tokens);
  r.qkv = L.qkv;
  r.a = L.a;
  r.b = L.b;
  r.conv_w = L.w;
  r.conv_b = L.bias;
  r.A_log = L.A_log;
  r.dt_bias = L.dt_bias;
  r.conv_pool = L.conv_state;
  r.ssm_pool = L.ssm_state;
  r.out = L.out;
  r.turns = reinterpret_cast<unsigned int*>(L.turns);
}

// Row-kernel arguments of the spec rows.  With `dec` (decode rows) the two
// share one launch: the decodes are its first row set and the spec rows
// follow them in the grid (rows of one call use disjoint slots; measured on
// the mixed batch, decodes first finish 3% sooner than spec rows first).
gdn::RowArgs spec_rows(const Layer& L, const SpecBatch& s, const gdn::RowArgs* dec = nullptr) {
  gdn::RowArgs r{};
  fill_layer(r, L);
  r.kind = gdn::kSpec;
  r.num_rows = s.num_spec_decodes;
  r.num_tokens = s.num_spec_tokens;
  r.row_stride = s.max_spec_len;
  r.max_row_tokens = s.max_spec_len;
  r.qsl = s.sqsl;
  r.cache_idx = s.cache;
  r.ssi = s.ssi;
  r.nacc = s.nacc;
  r.tix = s.tix;
  r.stage = gdn::kFused;
  if (dec) {
    gdn::RowArgs m = *dec;
    m.more.kind = r.kind;
    m.more.num_rows = r.num_rows;
    m.more.num_tokens = r.num_tokens;
    m.more.row_stride = r.row_stride;
    m.more.max_row_tokens = r.max_row_tokens;
    m.more.qsl = r.qsl;
    m.more.cache_idx = r.cache_idx;
    m.more.ssi = r.ssi;
    m.more.nacc = r.nacc;
    m.more.his = r.his;
    m.more.tix = r.tix;
    r = m;
  }
  return r;
}

int run_spec(const Layer& L, const SpecBatch& s, hipStream_t stream) {
  if (s.num_spec_decodes == 0) return GDN_OK;
  const gdn::RowArgs r = spec_rows(L, s);
  if (int e = rows_launch_ok(r, L.d)) return e;
  return launch(gdn::launch_rows(r, L.d->head_k_dim, L.d->head_v_dim, stream),
                "spec row kernel");
}

}  // namespace

extern "C" {

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "required pointer is NULL";
    case GDN_ERR_DIMS: return "inconsistent sizes or counts";
    case GDN_ERR_SPEC_PAIR: return "spec_state_indices and num_accepted_tokens must be given together";
    case GDN_ERR_MISSING_OPTIONAL: return "an optional tensor required by this batch is missing";
    case GDN_ERR_CONSERVATION: return "non-spec tokens + spec tokens != num_actual_tokens";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP launch failed";
    case GDN_ERR_UNSUPPORTED: return "shape not supported by the kernels";
    case GDN_ERR_METADATA: return "metadata violates a precondition";
    default: return "unknown status";
  }
}

const char* gdn_last_error(void) { return g_err; }

size_t gdn_workspace_bytes(const gdn_dims* dims, int32_t max_non_spec_tokens,
                           int32_t max_prefill_rows) {
  if (check_dims(dims) != GDN_OK) return 0;
  if (max_prefill_rows <= 0 || max_non_spec_tokens <= 0) return 0;
  return gdn::prefill_workspace_bytes(dims->num_k_heads, dims->num_v_heads,
                                      dims->head_k_dim, dims->head_v_dim,
                                      max_non_spec_tokens, max_prefill_rows);
}

size_t gdn_conv_turns_count(const gdn_dims* dims) {
  if (check_dims(dims) != GDN_OK) return 0;
  // four per (conv slot, k-head): one per wave of the 2*dk q/k channels at dk = 128
  return (size_t)dims->num_slots * (size_t)dims->num_k_heads * 4;
}

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
                       gdn_bf16* core_attn_out, uint32_t* conv_turns, gdn_stream_t stream) {
  if (int e = check_dims(dims)) return e;
  if (num_actual_tokens < 0) return fail(GDN_ERR_DIMS, "num_actual_tokens < 0");
  SpecBatch s{num_spec_decodes, num_spec_tokens, max_spec_len, spec_query_start_loc,
              spec_cache_indices, spec_state_indices, num_accepted_tokens, spec_token_indx};
  if (int e = check_spec(s, num_actual_tokens)) return e;
  if (num_spec_decodes == 0) return GDN_OK;
  if (dims->conv_layout == GDN_CONV_PER_TOKEN_SLOTS && spec_cache_indices)
    return fail(GDN_ERR_DIMS, "spec_cache_indices is not used with per-token conv slots");
  if (int e = check_layer_ptrs(dims, mixed_qkv, a, b, conv_weight, A_log, dt_bias, conv_state,
                               ssm_state, core_attn_out))
    return e;
  Layer L{dims, mixed_qkv, a, b, conv_weight, conv_bias, A_log, dt_bias,
          conv_state, ssm_state, core_attn_out, num_actual_tokens, conv_turns};
  return run_spec(L, s, static_cast<hipStream_t>(stream));
}

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
                  size_t workspace_bytes, gdn_stream_t stream) {
  if (int e = check_dims(dims)) return e;
  if (num_actual_tokens < 0 || num_decodes < 0 || num_prefills < 0 || num_non_spec_tokens < 0)
    return fail(GDN_ERR_DIMS, "negative counts");
  SpecBatch s{num_spec_decodes, num_spec_tokens, max_spec_len, spec_query_start_loc,
              spec_cache_indices, spec_state_indices, num_accepted_tokens, spec_token_indx};
  if (int e = check_spec(s, num_actual_tokens)) return e;
  if (dims->conv_layout == GDN_CONV_PER_TOKEN_SLOTS && num_spec_decodes > 0 &&
      spec_cache_indices)
    return fail(GDN_ERR_DIMS, "spec_cache_indices is not used with per-token conv slots");
  const int ns_rows = num_decodes + num_prefills;
  if (ns_rows == 0 && num_non_spec_tokens != 0)
    return fail(GDN_ERR_DIMS, "num_non_spec_tokens=%d with no non-spec rows", num_non_spec_tokens);
  if (ns_rows > 0) {
    if (!query_start_loc)
      return fail(GDN_ERR_MISSING_OPTIONAL, "non-spec rows need query_start_loc");
    if (!non_spec_state_indices)
      return fail(GDN_ERR_MISSING_OPTIONAL, "non-spec rows need non_spec_state_indices");
    if (num_non_spec_tokens < num_decodes)
      return fail(GDN_ERR_DIMS, "num_non_spec_tokens %d < decodes %d (a decode has a token)",
                  num_non_spec_tokens, num_decodes);
  }
  if ((long long)num_non_spec_tokens + num_spec_tokens != num_actual_tokens)
    return fail(GDN_ERR_CONSERVATION, "non-spec tokens %d + spec tokens %d != %d",
                num_non_spec_tokens, num_spec_tokens, num_actual_tokens);
  if (num_non_spec_tokens > 0 && num_spec_tokens > 0 && (!non_spec_token_indx || !spec_token_indx))
    return fail(GDN_ERR_MISSING_OPTIONAL,
                "a batch with both streams needs spec_token_indx and non_spec_token_indx");
  if (num_actual_tokens == 0) return GDN_OK;
  if (int e = check_layer_ptrs(dims, mixed_qkv, a, b, conv_weight, A_log, dt_bias, conv_state,
                               ssm_state, core_attn_out))
    return e;
  if (num_prefills > 0) {
    size_t need = gdn_workspace_bytes(dims, num_non_spec_tokens, num_prefills);
    if (!workspace || workspace_bytes < need)
      return fail(GDN_ERR_WORKSPACE, "prefill rows need %zu bytes of workspace (got %zu)",
                  need, workspace ? workspace_bytes : (size_t)0);
    const long long units = ((long long)num_non_spec_tokens + 63) / 64 + num_prefills;
    if (units > kMaxPrefillUnits)
      return fail(GDN_ERR_UNSUPPORTED, "prefill rows span up to %lld 64-token units (max %lld)",
                  units, kMaxPrefillUnits);
  }
  Layer L{dims, mixed_qkv, a, b, conv_weight, conv_bias, A_log, dt_bias,
          conv_state, ssm_state, core_attn_out, num_actual_tokens, conv_turns};
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Decode rows share the spec rows' launch when there are both (one grid,
  // decodes first).
  gdn::RowArgs dec{};
  if (num_decodes > 0) {
    fill_layer(dec, L);
    dec.kind = gdn::kNonSpec;
    dec.num_rows = num_decodes;
    dec.num_tokens = num_non_spec_tokens;
    dec.row_stride = 0;
    dec.max_row_tokens = 1;
    dec.qsl = query_start_loc;
    dec.cache_idx = non_spec_state_indices;
    dec.ssi = nullptr;
    dec.nacc = nullptr;
    dec.his = has_initial_state;
    dec.tix = non_spec_token_indx;
    dec.stage = gdn::kFused;
  }
  const bool merged = num_decodes > 0 && s.num_spec_decodes > 0;
  // every row launch is checked before anything is enqueued
  gdn::RowArgs rows_after{};
  if (s.num_spec_decodes > 0) {
    rows_after = spec_rows(L, s, merged ? &dec : nullptr);
    if (int e = rows_launch_ok(rows_after, dims)) return e;
  }
  const bool decodes_alone = num_decodes > 0 && !merged;
  if (decodes_alone) {
    if (int e = rows_launch_ok(dec, dims)) return e;
  }
  if (num_prefills > 0 && dims->head_k_dim >= 64) {
    if (int e = launch(gdn::prepare_chunked(dims->head_k_dim, dims->head_v_dim),
                       "chunked prefill set-up"))
      return e;
  }
  if (decodes_alone) {
    if (int e = launch(gdn::launch_rows(dec, dims->head_k_dim, dims->head_v_dim, st),
                       "decode row kernel"))
      return e;
  }
  if (num_prefills > 0) {
    gdn::PrefillArgs p;
    std::memset(&p, 0, sizeof p);
    p.Hk = dims->num_k_heads;
    p.Hv = dims->num_v_heads;
    p.G = p.Hv / p.Hk;
    p.C = conv_dim(dims);
    p.L = dims->state_len;
    p.W = dims->conv_width;
    p.num_slots = dims->num_slots;
    p.act = dims->activation;
    p.l2norm = dims->use_qk_l2norm;
    p.dk = dims->head_k_dim;
    p.dv = dims->head_v_dim;
    p.qkv_layout = dims->qkv_layout;
    p.eps = dims->l2norm_eps;
    p.scale = dims->scale;
    p.num_actual_tokens = num_actual_tokens;
    p.qkv = mixed_qkv;
    p.a = a;
    p.b = b;
    p.conv_w = conv_weight;
    p.conv_b = conv_bias;
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.conv_pool = conv_state;
    p.ssm_pool = ssm_state;
    p.out = core_attn_out;
    p.num_rows = num_prefills;
    p.stream_tokens = num_non_spec_tokens;
    p.qsl = query_start_loc + num_decodes;
    p.cache_idx = non_spec_state_indices + num_decodes;
    p.his = has_initial_state ? has_initial_state + num_decodes : nullptr;
    p.tix = non_spec_token_indx;
    p.workspace = workspace;
    if (int e = launch(gdn::launch_prefill(p, dims->head_k_dim, dims->head_v_dim, st),
                       "prefill kernels"))
      return e;
  }
  if (s.num_spec_decodes == 0) return GDN_OK;
  return launch(gdn::launch_rows(rows_after, dims->head_k_dim, dims->head_v_dim, st),
                merged ? "decode and spec row kernel" : "spec row kernel");
}

static int stage_rows(const gdn_dims* dims, const gdn_rows* rows, int num_actual_tokens,
                      gdn::RowArgs& r) {
  if (int e = check_dims(dims)) return e;
  if (!rows) return fail(GDN_ERR_NULL, "rows is NULL");
  if (rows->num_rows < 0 || rows->num_tokens < 0 || num_actual_tokens < 0)
    return fail(GDN_ERR_DIMS, "negative counts");
  if (rows->kind != GDN_ROWS_SPEC && rows->kind != GDN_ROWS_NON_SPEC)
    return fail(GDN_ERR_DIMS, "rows->kind must be GDN_ROWS_SPEC or GDN_ROWS_NON_SPEC");
  if (rows->num_rows > 0) {
    if (!rows->query_start_loc) return fail(GDN_ERR_MISSING_OPTIONAL, "rows need query_start_loc");
    if (rows->max_row_tokens < 1 || rows->max_row_tokens > gdn::kMaxRowTokens)
      return fail(GDN_ERR_UNSUPPORTED, "max_row_tokens %d not in [1,%d]", rows->max_row_tokens,
                  gdn::kMaxRowTokens);
    if (rows->kind == GDN_ROWS_SPEC) {
      if ((rows->state_indices == nullptr) != (rows->num_accepted_tokens == nullptr))
        return fail(GDN_ERR_SPEC_PAIR,
                    "state_indices and num_accepted_tokens must be given together");
      if (!rows->state_indices)
        return fail(GDN_ERR_MISSING_OPTIONAL, "spec rows need state_indices");
      if (dims->conv_layout == GDN_CONV_PER_TOKEN_SLOTS && rows->cache_indices)
        return fail(GDN_ERR_DIMS, "cache_indices is not used by spec rows with per-token conv "
                                  "slots");
    } else if (!rows->cache_indices) {
      return fail(GDN_ERR_MISSING_OPTIONAL, "non-spec rows need cache_indices");
    }
    if (rows->num_tokens > num_actual_tokens && !rows->token_indx)
      return fail(GDN_ERR_DIMS, "rows hold more tokens than num_actual_tokens");
  }
  fill_common(r, dims, num_actual_tokens);
  r.kind = rows->kind == GDN_ROWS_SPEC ? gdn::kSpec : gdn::kNonSpec;
  r.num_rows = rows->num_rows;
  r.num_tokens = rows->num_tokens;
  r.row_stride = rows->max_row_tokens;
  r.max_row_tokens = rows->max_row_tokens;
  r.qsl = rows->query_start_loc;
  r.cache_idx = rows->cache_indices;
  r.ssi = rows->state_indices;
  r.nacc = rows->num_accepted_tokens;
  r.his = rows->has_initial_state;
  r.tix = rows->token_indx;
  return rows_launch_ok(r, dims);
}

int gdn_conv_only(const gdn_dims* dims, const gdn_bf16* mixed_qkv,
                  const gdn_bf16* conv_weight, const gdn_bf16* conv_bias,
                  gdn_bf16* conv_state, int32_t num_actual_tokens,
                  const gdn_rows* rows, float* conv_out, gdn_stream_t stream) {
  gdn::RowArgs r{};
  if (int e = stage_rows(dims, rows, num_actual_tokens, r)) return e;
  if (r.num_rows == 0) return GDN_OK;
  if (!mixed_qkv || !conv_weight || (!conv_state && dims->state_len > 0) || !conv_out)
    return fail(GDN_ERR_NULL, "mixed_qkv, conv_weight, conv_state and conv_out are required");
  r.qkv = mixed_qkv;
  r.conv_w = conv_weight;
  r.conv_b = conv_bias;
  r.conv_pool = conv_state;
  r.y = conv_out;
  r.stage = gdn::kConvOnly;
  return launch(gdn::launch_rows(r, dims->head_k_dim, dims->head_v_dim,
                                 static_cast<hipStream_t>(stream)),
                "conv stage kernel");
}

int gdn_delta_rule_only(const gdn_dims* dims, const float* conv_out,
                        const gdn_bf16* a, const gdn_bf16* b,
                        const float* A_log, const float* dt_bias,
                        float* ssm_state, int32_t num_actual_tokens,
                        const gdn_rows* rows, gdn_bf16* core_attn_out,
                        gdn_stream_t stream) {
  gdn::RowArgs r{};
  if (int e = stage_rows(dims, rows, num_actual_tokens, r)) return e;
  if (r.num_rows == 0) return GDN_OK;
  if (!conv_out || !a || !b || !A_log || !dt_bias || !ssm_state || !core_attn_out)
    return fail(GDN_ERR_NULL,
                "conv_out, a, b, A_log, dt_bias, ssm_state and core_attn_out are required");
  r.y = const_cast<float*>(conv_out);
  r.a = a;
  r.b = b;
  r.A_log = A_log;
  r.dt_bias = dt_bias;
  r.ssm_pool = ssm_state;
  r.out = core_attn_out;
  r.stage = gdn::kDeltaOnly;
  return launch(gdn::launch_rows(r, dims->head_k_dim, dims->head_v_dim,
                                 static_cast<hipStream_t>(stream)),
                "delta-rule stage kernel");
}

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
                            gdn_host_i32 spec_token_indx) {
  if (int e = check_dims(dims)) return e;
  if (num_actual_tokens < 0 || num_decodes < 0 || num_prefills < 0 || num_non_spec_tokens < 0 ||
      num_spec_decodes < 0 || num_spec_tokens < 0)
    return fail(GDN_ERR_DIMS, "negative counts");
  const int ns_rows = num_decodes + num_prefills;
  if (ns_rows == 0 && num_non_spec_tokens != 0)
    return fail(GDN_ERR_DIMS, "num_non_spec_tokens=%d with no non-spec rows", num_non_spec_tokens);
  if (num_spec_decodes == 0 && num_spec_tokens != 0)
    return fail(GDN_ERR_DIMS, "num_spec_tokens=%d with no spec rows", num_spec_tokens);
  const long long streams = (long long)num_non_spec_tokens + num_spec_tokens;
  if (streams > num_actual_tokens)
    return fail(GDN_ERR_CONSERVATION, "non-spec tokens %d + spec tokens %d > num_actual_tokens %d",
                num_non_spec_tokens, num_spec_tokens, num_actual_tokens);
  if (ns_rows > 0 && streams != num_actual_tokens)
    return fail(GDN_ERR_CONSERVATION, "non-spec tokens %d + spec tokens %d != %d",
                num_non_spec_tokens, num_spec_tokens, num_actual_tokens);
  // Lengths first: nothing below reads past what the caller said it holds.
  auto need = [](const gdn_host_i32& a, long long n, bool required, const char* what) -> int {
    if (!a.data) {
      if (required && n > 0) return fail(GDN_ERR_NULL, "%s is required", what);
      return GDN_OK;
    }
    if (a.len < n)
      return fail(GDN_ERR_DIMS, "%s holds %lld values; the counts need %lld", what,
                  (long long)a.len, n);
    return GDN_OK;
  };
  if (ns_rows > 0) {
    if (int e = need(query_start_loc, ns_rows + 1LL, true, "query_start_loc")) return e;
    if (int e = need(non_spec_state_indices, ns_rows, true, "non_spec_state_indices")) return e;
    if (int e = need(non_spec_token_indx, num_non_spec_tokens, false, "non_spec_token_indx"))
      return e;
  }
  if (num_spec_decodes > 0) {
    if (max_spec_len < 1 || max_spec_len > gdn::kMaxRowTokens)
      return fail(GDN_ERR_UNSUPPORTED, "max_spec_len %d not in [1,%d]", max_spec_len,
                  gdn::kMaxRowTokens);
    if (int e = need(spec_query_start_loc, num_spec_decodes + 1LL, true, "spec_query_start_loc"))
      return e;
    if (int e = need(spec_state_indices, (long long)num_spec_decodes * max_spec_len, true,
                     "spec_state_indices"))
      return e;
    if (int e = need(num_accepted_tokens, num_spec_decodes, true, "num_accepted_tokens"))
      return e;
    if (int e = need(spec_cache_indices, num_spec_decodes, false, "spec_cache_indices")) return e;
    if (int e = need(spec_token_indx, num_spec_tokens, false, "spec_token_indx")) return e;
  }
  const int L = dims->state_len, W = dims->conv_width, S = dims->num_slots;
  std::vector<int> row_owner(num_actual_tokens, -1);
  std::vector<int> slot_owner(S, -1);
  int owner = 0;
  auto claim_slot = [&](int slot, int who, const char* what) -> int {
    if (slot >= S) return fail(GDN_ERR_METADATA, "%s slot %d >= num_slots %d", what, slot, S);
    if (slot <= 0) return GDN_OK;
    if (slot_owner[slot] != -1 && slot_owner[slot] != who)
      return fail(GDN_ERR_METADATA, "slot %d used by two rows", slot);
    slot_owner[slot] = who;
    return GDN_OK;
  };
  auto claim_row = [&](int r, int who) -> int {
    if (r < 0 || r >= num_actual_tokens)
      return fail(GDN_ERR_METADATA, "token row %d outside [0,%d)", r, num_actual_tokens);
    if (row_owner[r] != -1) return fail(GDN_ERR_METADATA, "token row %d mapped twice", r);
    row_owner[r] = who;
    return GDN_OK;
  };
  if (ns_rows > 0) {
    const int32_t* qsl = query_start_loc.data;
    if (qsl[0] != 0) return fail(GDN_ERR_METADATA, "query_start_loc[0] != 0");
    for (int i = 0; i < ns_rows; ++i)
      if (qsl[i + 1] < qsl[i])
        return fail(GDN_ERR_METADATA, "query_start_loc decreases at row %d", i);
    if (qsl[ns_rows] != num_non_spec_tokens)
      return fail(GDN_ERR_METADATA, "query_start_loc[%d] = %d, but num_non_spec_tokens = %d",
                  ns_rows, qsl[ns_rows], num_non_spec_tokens);
    // qsl is non-decreasing from 0 to num_non_spec_tokens: every token index
    // below lies inside non_spec_token_indx
    for (int i = 0; i < ns_rows; ++i, ++owner) {
      const int T = qsl[i + 1] - qsl[i];
      if (i < num_decodes && T != 1)
        return fail(GDN_ERR_METADATA, "decode row %d has %d tokens", i, T);
      if (int e = claim_slot(non_spec_state_indices.data[i], owner, "non-spec")) return e;
      for (int j = qsl[i]; j < qsl[i + 1]; ++j)
        if (int e = claim_row(non_spec_token_indx.data ? non_spec_token_indx.data[j] : j, owner))
          return e;
    }
  }
  if (num_spec_decodes > 0) {
    const int32_t* sqsl = spec_query_start_loc.data;
    if (sqsl[0] != 0) return fail(GDN_ERR_METADATA, "spec_query_start_loc[0] != 0");
    for (int bi = 0; bi < num_spec_decodes; ++bi) {
      const int T = sqsl[bi + 1] - sqsl[bi];
      if (T < 1 || T > max_spec_len)
        return fail(GDN_ERR_METADATA, "spec row %d has %d tokens (max %d)", bi, T, max_spec_len);
    }
    if (sqsl[num_spec_decodes] != num_spec_tokens)
      return fail(GDN_ERR_METADATA, "spec_query_start_loc[%d] = %d, but num_spec_tokens = %d",
                  num_spec_decodes, sqsl[num_spec_decodes], num_spec_tokens);
    const bool per_token = dims->conv_layout == GDN_CONV_PER_TOKEN_SLOTS;
    for (int bi = 0; bi < num_spec_decodes; ++bi, ++owner) {
      const int T = sqsl[bi + 1] - sqsl[bi];
      const int n = num_accepted_tokens.data[bi];
      if (n < 1 || n > T)
        return fail(GDN_ERR_METADATA, "spec row %d: num_accepted_tokens %d not in [1,%d]", bi,
                    n, T);
      if (!per_token && n + W - 2 > L)
        return fail(GDN_ERR_METADATA, "spec row %d: window n_acc-1=%d needs state_len >= %d",
                    bi, n - 1, n + W - 2);
      const int32_t* ssi = spec_state_indices.data + (size_t)bi * max_spec_len;
      if (!per_token) {
        const int cs = spec_cache_indices.data ? spec_cache_indices.data[bi] : ssi[0];
        if (int e = claim_slot(cs, owner, "conv")) return e;
      }
      for (int t = 0; t < T; ++t)
        if (int e = claim_slot(ssi[t], owner, "spec state")) return e;
      for (int j = sqsl[bi]; j < sqsl[bi + 1]; ++j)
        if (int e = claim_row(spec_token_indx.data ? spec_token_indx.data[j] : j, owner))
          return e;
    }
  }
  return GDN_OK;
}

// ---- allocation-free variant of gdn_attention ------------------------------
// For callers that cannot allocate device memory: the prefill rows' scratch
// comes from this file-scope array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, so its device address is taken
// once per device with hipGetSymbolAddress and only that address is used.
static __device__ __align__(256) unsigned char scratch[GDN_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (taken on the first call
// on each device).
int static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GDN_ERR_UNSUPPORTED, "device %d beyond the %d the static scratch tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

}  // namespace

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
                         gdn_stream_t stream) {
  if (int e = check_dims(dims)) return e;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  // prefill rows always get the scratch (gdn_attention asks for a workspace
  // whenever there are prefill rows, empty ones included)
  if (num_prefills > 0) {
    const size_t need = gdn_workspace_bytes(dims, num_non_spec_tokens, num_prefills);
    if (need > (size_t)GDN_STATIC_SCRATCH_BYTES)
      return fail(GDN_ERR_WORKSPACE,
                  "prefill rows need %zu bytes of scratch; the static scratch holds %zu "
                  "(use gdn_attention with a workspace)",
                  need, (size_t)GDN_STATIC_SCRATCH_BYTES);
    if (int e = static_scratch(&ws)) return e;
    ws_bytes = GDN_STATIC_SCRATCH_BYTES;
  }
  return gdn_attention(dims, mixed_qkv, a, b, conv_weight, conv_bias, A_log, dt_bias, conv_state,
                       ssm_state, num_actual_tokens, num_decodes, num_prefills,
                       num_non_spec_tokens, query_start_loc, non_spec_state_indices,
                       has_initial_state, non_spec_token_indx, num_spec_decodes,
                       num_spec_tokens, max_spec_len, spec_query_start_loc, spec_cache_indices,
                       spec_state_indices, num_accepted_tokens, spec_token_indx, core_attn_out,
                       conv_turns, ws, ws_bytes, stream);
}

}  // extern "C"
