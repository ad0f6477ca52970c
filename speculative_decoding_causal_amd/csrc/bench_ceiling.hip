// Measured ceiling for the spec-verify step's state traffic: the load and
// per-token stores of every (row, k-head) state block, with no arithmetic.
// Declared in include/gdn_bench.h; built into libgdn_bench.so, which the
// benchmark loads beside libgdn.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn_bench.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
constexpr int kThreads = 512;
constexpr int kPer = 8;                            // float4 per thread
constexpr int kBlockFloats = kThreads * kPer * 4;  // 64 KiB: one v-head

__device__ __forceinline__ int clamp_i(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// The dynamic tail's claim count (one per GPU, 0 at load and after every
// launch: calls are ordered by the caller).
__device__ unsigned int g_tail_count;

// Unit u = (row, v-head): its block is read once and written to every
// token's slot.  Workgroup i runs on XCD i % 8: the v-heads of a row share
// i % 8.
__device__ __forceinline__ void fan_unit(float* pool, int num_slots, int Hv, int num_rows, int K,
                                         const int* qsl, const int* ssi, const int* nacc,
                                         size_t slot_floats, int u) {
  const int q8 = u >> 3;
  const int ih = q8 % Hv;
  const int row = (q8 / Hv) * 8 + (u & 7);
  if (row >= num_rows) return;
  const int tid = threadIdx.x;
  const int j0 = qsl[row];
  const int T = clamp_i(qsl[row + 1] - j0, 0, K);
  if (T <= 0) return;
  const int* s = ssi + (size_t)row * K;
  const int ls = s[clamp_i(nacc[row], 1, T) - 1];
  const bool load = ls > 0 && ls < num_slots;
  const size_t off = (size_t)ih * kBlockFloats;
  const v4f* src = reinterpret_cast<const v4f*>(pool + (size_t)(load ? ls : 0) * slot_floats + off);
  v4f S[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) S[e] = __builtin_nontemporal_load(src + e * kThreads + tid);
#pragma unroll
  for (int e = 0; e < kPer; ++e) S[e] = load ? S[e] : v4f{0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < T; ++t) {
    const int st = s[t];
    if (st <= 0 || st >= num_slots) continue;
    v4f* dst = reinterpret_cast<v4f*>(pool + (size_t)st * slot_floats + off);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      v4f v = S[e];
      if (e == 0 && tid == 0) v.x += (float)t;
      __builtin_nontemporal_store(v, dst + e * kThreads + tid);
    }
  }
}

// Workgroup i takes unit i; with a tail, the grid's last `takers`
// workgroups (the last to start on each CU) then claim the units from
// tail_first on one at a time, each claim issued a unit ahead of its use,
// as the row kernel's (row, v-head) launches do: every taker claims until
// its first claim past the tail, so tail + takers claims are made per
// launch and the count wraps back to 0.
__global__ void __launch_bounds__(kThreads)
state_fanout(float* pool, int num_slots, int Hv, int num_rows, int K, const int* qsl,
             const int* ssi, const int* nacc, size_t slot_floats, int tail, int takers,
             int tail_first) {
  const bool taker = tail > 0 && static_cast<int>(blockIdx.x) >= static_cast<int>(gridDim.x) - takers;
  if (!taker) {
    fan_unit(pool, num_slots, Hv, num_rows, K, qsl, ssi, nacc, slot_floats, blockIdx.x);
    return;
  }
  __shared__ unsigned int claim_sh[2];
  const unsigned int wrap = static_cast<unsigned int>(tail + takers - 1);
  unsigned int claim = 0;
  if (threadIdx.x == 0) claim = atomicInc(&g_tail_count, wrap);
  int u = blockIdx.x;
  for (int it = 0;; ++it) {
    fan_unit(pool, num_slots, Hv, num_rows, K, qsl, ssi, nacc, slot_floats,
             __builtin_amdgcn_readfirstlane(u));
    // the claim in hand, double-buffered across iterations
    if (threadIdx.x == 0) claim_sh[it & 1] = claim;
    __syncthreads();
    const unsigned int c = __builtin_amdgcn_readfirstlane(claim_sh[it & 1]);
    if (c >= static_cast<unsigned int>(tail)) return;
    u = tail_first + static_cast<int>(c);
    if (threadIdx.x == 0) claim = atomicInc(&g_tail_count, wrap);
  }
}

}  // namespace

extern "C" int gdn_bench_state_fanout(float* ssm_state, int32_t num_slots, int32_t num_k_heads,
                                      int32_t num_v_heads, int32_t head_k_dim,
                                      int32_t head_v_dim, int32_t num_rows,
                                      int32_t max_spec_len, const int32_t* qsl,
                                      const int32_t* ssi, const int32_t* nacc, void* stream) {
  if (!ssm_state || !qsl || !ssi || !nacc || num_k_heads <= 0 || num_v_heads % num_k_heads ||
      num_rows < 0 || max_spec_len < 1 || num_slots <= 0)
    return -1;
  const long long block = (long long)head_v_dim * head_k_dim;
  if (block != kBlockFloats) return -1;
  if (num_rows == 0) return 0;
  const size_t slot_floats = (size_t)num_v_heads * head_v_dim * head_k_dim;
  const unsigned units = (unsigned)((num_rows + 7) / 8 * 8) * (unsigned)num_v_heads;
  // one workgroup per CU (LDS above half of the CU's 160 KiB): the fastest
  // occupancy for this pattern in measurements on MI355X
  constexpr int kLds = 80 * 1024 + 16;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(state_fanout),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != hipSuccess)
    return -7;
  // the dynamic tail: 1/8 of the units, at most two per CU, on grids of at
  // least two units per CU
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -7;
  const unsigned takers = (unsigned)cus & ~7u;
  unsigned tail = units / 8;
  tail = (tail < 2u * takers ? tail : 2u * takers) & ~7u;
  if (takers == 0 || units < 2u * takers || units - tail < takers) tail = 0;
  hipLaunchKernelGGL(state_fanout, dim3(units - tail), dim3(kThreads), kLds,
                     static_cast<hipStream_t>(stream), ssm_state, num_slots, num_v_heads,
                     num_rows, max_spec_len, qsl, ssi, nacc, slot_floats, (int)tail, (int)takers,
                     (int)(units - tail));
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
