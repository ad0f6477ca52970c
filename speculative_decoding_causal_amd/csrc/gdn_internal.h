// Internal interface between the C-ABI layer (gdn_api.cpp) and the HIP
// kernels.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kThreads = 256;        // threads per workgroup (4 wave64)
constexpr int kMaxRowTokens = 16;    // tokens per row in the fused kernel
constexpr int kMaxStateLen = 16;
constexpr int kMaxWidth = 4;

enum RowKind : int { kNonSpec = 0, kSpec = 1 };
enum Stage : int { kFused = 0, kConvOnly = 1, kDeltaOnly = 2 };

// Raise a kernel's dynamic LDS limit once per device (kernel launches may be
// captured into a graph; the attribute is set outside any stream work).
hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes);

// Compute units of the current device (queried once per device).
hipError_t device_cu_count(int* cus);

// Everything one launch of the row kernel needs, passed by value.
struct RowArgs {
  // shape
  int Hk, Hv, G, C, L, W, num_slots, act, l2norm;
  int qkv_layout;  // 0 grouped [q | k | v], 1 per k-head [q_i k_i v_i..]
  int conv_per_token;  // spec rows: conv window saved per token (state_len == W-1)
  float eps, scale;
  int num_actual_tokens;
  // layer tensors
  const uint16_t* qkv;
  const uint16_t* a;
  const uint16_t* b;
  const uint16_t* conv_w;
  const uint16_t* conv_b;
  const float* A_log;
  const float* dt_bias;
  uint16_t* conv_pool;
  float* ssm_pool;
  uint16_t* out;
  float* y;  // conv output, [num_actual_tokens, C] (stage entry points)
  // rows
  int kind;
  int num_rows;
  int num_tokens;      // tokens of the stream the rows index
  int row_stride;      // spec: row stride of ssi
  int max_row_tokens;  // tokens processed per row at most (LDS sizing)
  const int* qsl;
  const int* cache_idx;
  const int* ssi;
  const int* nacc;
  const uint8_t* his;
  const int* tix;
  int stage;
  // Per (conv slot, k-head, q/k wave) turn counters (num_slots * Hk * 4, 0 between
  // calls), or null: with them the fused step of one row set (dk = dv = 128,
  // G > 1) runs one workgroup per (row, v-head), and the last of a k-head's
  // G workgroups to read the shared q/k ring channels rolls them.
  unsigned int* turns;
  // Dynamic tail of a (row, v-head) launch (tail_units 0: none).  The grid
  // covers units [0, tail_first) one per workgroup; its last tail_takers
  // workgroups then claim units tail_first + c, c = 0 .. tail_units-1, from
  // a wrapping count in turns[0] (the cell of the NULL conv slot, which the
  // turn protocol never uses) until a claim comes back past the tail.
  int tail_units = 0, tail_takers = 0, tail_first = 0;
  // A second set of rows in the same launch (none when num_rows is 0): its
  // rows follow the first set's in the grid, with their own kind and metadata.
  struct RowSet {
    int kind = 0, num_rows = 0, num_tokens = 0, row_stride = 0, max_row_tokens = 0;
    const int* qsl = nullptr;
    const int* cache_idx = nullptr;
    const int* ssi = nullptr;
    const int* nacc = nullptr;
    const uint8_t* his = nullptr;
    const int* tix = nullptr;
  } more;
};

// Tokens per row the LDS layout of a launch is sized for (both sets).
__host__ __device__ inline int launch_row_tokens(const RowArgs& a) {
  return a.more.num_rows > 0 && a.more.max_row_tokens > a.max_row_tokens ? a.more.max_row_tokens
                                                                          : a.max_row_tokens;
}

// Rows of at most kMaxRowTokens tokens (spec rows and decodes), one
// workgroup per (row, k-head), or per (row, v-head) with turn counters:
// conv + ring roll, gates, norms, recurrence.
hipError_t launch_rows(const RowArgs& a, int dk, int dv, hipStream_t s);
size_t rows_lds_bytes(const RowArgs& a, int dk, int dv);

// Long non-spec rows (prefills): conv over the whole row into a workspace,
// then the delta rule over the row.
struct PrefillArgs {
  int Hk, Hv, G, C, L, W, num_slots, act, l2norm;
  int dk, dv, qkv_layout;
  float eps, scale;
  int num_actual_tokens;
  const uint16_t* qkv;
  const uint16_t* a;
  const uint16_t* b;
  const uint16_t* conv_w;
  const uint16_t* conv_b;
  const float* A_log;
  const float* dt_bias;
  uint16_t* conv_pool;
  float* ssm_pool;
  uint16_t* out;
  int num_rows;        // prefill rows
  int stream_tokens;   // tokens of the non-spec stream (workspace capacity)
  int units;           // capacity of unit_map: stream_tokens/64 rounded up + rows
  const int* unit_map; // [units][2]: (row, 64-token unit of the row), row -1 past the end
  const int* qsl;      // [num_rows+1], non-spec stream indices
  const int* cache_idx;
  const uint8_t* his;
  const int* tix;
  void* workspace;
};
size_t prefill_workspace_bytes(int Hk, int Hv, int dk, int dv,
                               int stream_tokens, int rows);
hipError_t launch_prefill(const PrefillArgs& a, int dk, int dv, hipStream_t s);

// Per-token chunk quantities of the chunked prefill, indexed by non-spec
// stream token and v-head: W [n, Hv, dk], U~ [n, Hv, dv], P [n, Hv, 64],
// G [n, Hv] (cumulative log-decay inside the token's chunk).
struct ChunkWs {
  float* W;
  float* U;
  float* P;
  float* G;
};
hipError_t launch_chunked(const PrefillArgs& a, int dk, int dv, const float* y, const float* glog,
                          const float* gbeta, const ChunkWs& ws, hipStream_t s);
// Raises the chunk kernels' LDS limit (once per device); callers run it
// before enqueuing anything, so a failure leaves every buffer untouched.
hipError_t prepare_chunked(int dk, int dv);

}  // namespace gdn
