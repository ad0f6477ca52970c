// Device helpers shared by the HIP kernels: bf16 conversion, lane
// reductions, gates.  gfx950 (CDNA4, wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// DPP lane moves within a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over groups of LPR consecutive lanes (LPR in 1,2,4,8,16); every lane
// of a group ends with the same bits (each step adds a commutative pair).
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPR >= 2) v += dpp_mov<0xB1>(v);   // quad_perm 1,0,3,2
  if constexpr (LPR >= 4) v += dpp_mov<0x4E>(v);   // quad_perm 2,3,0,1
  if constexpr (LPR >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror
  if constexpr (LPR >= 16) v += dpp_mov<0x140>(v); // row_mirror
  return v;
}

// Butterfly sum over the 64 lanes of a wave; all lanes get the same bits.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Decay alpha = exp(-exp(A_log) * softplus(a + dt_bias)) and write strength
// beta = sigmoid(b) of one (token, v-head).
__device__ __forceinline__ void gate_pair(float a, float b, float A_log,
                                          float dt_bias, float* alpha,
                                          float* beta) {
  float x = a + dt_bias;
  float sp = x > 20.f ? x : log1pf(expf(x));
  *alpha = expf(-expf(A_log) * sp);
  *beta = 1.f / (1.f + expf(-b));
}

// Log of the decay: log alpha = -exp(A_log) * softplus(a + dt_bias).
__device__ __forceinline__ float gate_log(float a, float A_log, float dt_bias) {
  const float x = a + dt_bias;
  const float sp = x > 20.f ? x : log1pf(expf(x));
  return -expf(A_log) * sp;
}

// SiLU x * sigma(x) with the hardware exp2 and reciprocal (about 1 ulp each):
// x -> -inf gives exp2 = inf, rcp = 0, -0; x -> +inf gives x; NaN stays NaN.
__device__ __forceinline__ float silu(float x) {
  const float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.f + e);
}

// Workgroup barrier that orders LDS only: outstanding global loads (prefetches
// into registers) stay in flight across it, unlike __syncthreads(), whose
// workgroup-scope fence also waits for every global access.  Use it only where
// no thread reads, across the barrier, global memory another thread wrote.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Column of mixed_qkv holding grouped channel c ([q heads | k heads | v
// heads]) when the rows are laid out per k-head (q_i, k_i, then the v of
// the k-head's G v-heads, block after block).
__device__ __forceinline__ int per_k_head_column(int c, int Hk, int G, int dk, int dv) {
  const int B = 2 * dk + G * dv;
  if (c < Hk * dk) return (c / dk) * B + c % dk;
  c -= Hk * dk;
  if (c < Hk * dk) return (c / dk) * B + dk + c % dk;
  c -= Hk * dk;
  return (c / (G * dv)) * B + 2 * dk + c % (G * dv);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// A float pair split into bf16 pairs, x = hi + lo + O(2^-17 |x|) with
// hi = bf16(x) and lo = bf16(x - hi); two values per word, the first in the
// low half.  The operands of the chunked prefill's bf16 products.
struct Split2 {
  unsigned hi, lo;
};
__device__ __forceinline__ Split2 split2(float x0, float x1) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  const v2bf h = {(__bf16)x0, (__bf16)x1};
  const unsigned hb = __builtin_bit_cast(unsigned, h);
  const v2bf l = {(__bf16)(x0 - __uint_as_float(hb << 16)),
                  (__bf16)(x1 - __uint_as_float(hb & 0xffff0000u))};
  return {hb, __builtin_bit_cast(unsigned, l)};
}

}  // namespace gdn
