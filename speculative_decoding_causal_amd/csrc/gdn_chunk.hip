// Chunked (WY / UT) form of the gated delta rule for prefill rows, on MFMA.
//
// The recurrence S_t = a_t S_{t-1} + u_t k_t^T, u_t = b_t (v_t - a_t S_{t-1} k_t)
// (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", chunkwise form) is
// evaluated 64 tokens at a time.  With G_t the cumulative log-decay inside a
// chunk (G_t = sum_{s<=t} log a_s) and only decay differences t >= s ever
// exponentiated:
//   A  = strictly-lower( b_t e^{G_t - G_s} k_t.k_s )          (C x C)
//   T  = (I + A)^{-1}                                         (forward substitution)
//   W  = T diag(b e^{G}) K,   U~ = T diag(b) V                 (C x dk, C x dv)
//   P  = lower-incl( e^{G_t - G_s} q_t.k_s )                  (C x C)
// and then, chunk after chunk, from the chunk's initial state S0:
//   U  = U~ - W S0^T                                          (C x dv)
//   O  = diag(e^{G}) Q S0^T + P U                             (C x dv)
//   S  = e^{G_C} S0 + U^T diag(e^{G_C - G_t}) K                (dv x dk)
// which equals running the token recurrence exactly (up to rounding).
//
// chunk_prep_kernel: one workgroup per (row, chunk, v-head) computes W, U~, P
// and G for its chunk (all chunks in parallel).
// chunk_state_kernel: one workgroup per (row, v-head, 16 state rows) carries
// its rows of S through the row's chunks in MFMA accumulators and writes the
// outputs through token_indx.  Dense products use v_mfma_f32_16x16x4f32
// (A[i][k] at lane i+16k, B[k][j] at lane j+16k, D[i][j] at lane j+16*(i/4),
// element i%4).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
constexpr int kC = 64;  // tokens per chunk

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int slot_ok(int s, int n) { return (s > 0 && s < n) ? s : 0; }

struct PRow {
  int j0, T, slot;
  bool init;
};

__device__ __forceinline__ PRow prow(const PrefillArgs& p, int row) {
  PRow r;
  r.j0 = clampi(p.qsl[row], 0, p.stream_tokens);
  const int j1 = clampi(p.qsl[row + 1], r.j0, p.stream_tokens);
  r.T = j1 - r.j0;
  r.slot = slot_ok(p.cache_idx[row], p.num_slots);
  r.init = (p.his ? p.his[row] != 0 : true) && r.slot > 0;
  return r;
}

// Rows of ROWS x COLS floats gathered in one batch of float4 loads (rows
// >= nrow read as zeros), then written to LDS with row pitch PITCH.
template <int ROWS, int COLS>
struct Tile4 {
  static constexpr int kPer = ROWS * COLS / 4 / 256;  // float4 per thread
  v4f v[kPer];
  template <class RowPtr>
  __device__ __forceinline__ void load(RowPtr row_ptr, int nrow) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = (i * 256 + (int)threadIdx.x) * 4;
      const int r = e / COLS, c = e - r * COLS;
      v[i] = r < nrow ? *reinterpret_cast<const v4f*>(row_ptr(r) + c) : v4f{0.f, 0.f, 0.f, 0.f};
    }
  }
  template <int PITCH>
  __device__ __forceinline__ void store(float* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = (i * 256 + (int)threadIdx.x) * 4;
      const int r = e / COLS, c = e - r * COLS;
      *reinterpret_cast<v4f*>(lds + r * PITCH + c) = v[i];
    }
  }
};

// Shared-memory carve-up of chunk_prep_kernel (floats; rows padded by four
// so that MFMA operand reads down a column spread over the banks and rows
// stay 16-byte aligned).
template <int DK>
struct PrepLds {
  static constexpr int ks = 0;                         // [kC][DK+4] keys
  static constexpr int qs = ks + kC * (DK + 4);        // [kC][DK+4] queries, then values
  static constexpr int as = qs + kC * (DK + 4);        // [kC][kC+1] A, then T
  static constexpr int gs = as + kC * (kC + 1);        // [kC] cumulative log-decay
  static constexpr int bs = gs + kC;                   // [kC] beta
  static constexpr int bg = bs + kC;                   // [kC] beta e^G
  static constexpr int total = bg + kC;
};

template <int DK, int DV>
__global__ void __launch_bounds__(256)
chunk_prep_kernel(PrefillArgs p, const float* __restrict__ y, const float* __restrict__ glog,
                  const float* __restrict__ gbeta, ChunkWs ws) {
  static_assert(DK == DV, "dk == dv");
  extern __shared__ __align__(16) float sm[];
  using Lay = PrepLds<DK>;
  float* Ks = sm + Lay::ks;
  float* Qs = sm + Lay::qs;
  float* As = sm + Lay::as;
  float* Gs = sm + Lay::gs;
  float* Bs = sm + Lay::bs;
  float* BG = sm + Lay::bg;
  constexpr int KP = DK + 4, AP = kC + 1;

  const int c = blockIdx.x, h = blockIdx.y;
  const PRow pr = prow(p, blockIdx.z);
  const int t0 = c * kC;
  if (t0 >= pr.T) return;
  const int nt = min(kC, pr.T - t0);
  const int jb = pr.j0 + t0;
  const int ih = h / p.G, Hk = p.Hk, Hv = p.Hv, C = p.C;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  Tile4<kC, DV> vpark;

  // 1. keys, queries and values of the chunk (normalised q/k in the
  //    workspace), gathered in one batch; gates
  {
    Tile4<kC, DK> tk, tq, tv;
    const float* yb = y + (size_t)jb * C;
    tk.load([&](int r) { return yb + (size_t)r * C + Hk * DK + ih * DK; }, nt);
    tq.load([&](int r) { return yb + (size_t)r * C + ih * DK; }, nt);
    tv.load([&](int r) { return yb + (size_t)r * C + 2 * Hk * DK + h * DV; }, nt);
    tk.template store<KP>(Ks);
    tq.template store<KP>(Qs);
    // values wait in registers until Q K^T is done
    vpark = tv;
  }
  if (tid < kC) {
    Gs[tid] = tid < nt ? glog[(size_t)(jb + tid) * Hv + h] : 0.f;
    Bs[tid] = tid < nt ? gbeta[(size_t)(jb + tid) * Hv + h] : 0.f;
  }
  __syncthreads();
  // 2. cumulative log-decay (inclusive scan over the 64 tokens)
  if (wv == 0) {
    float g = Gs[lane];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float up = __shfl_up(g, o, 64);
      if (lane >= o) g += up;
    }
    Gs[lane] = g;
    BG[lane] = Bs[lane] * expf(g);
  }
  __syncthreads();
  // 3. K K^T and Q K^T, 16x16 tiles; wave w owns token-row tile w
  {
    const int i = lane & 15, kk = lane >> 4;
    for (int tj = 0; tj < 4; ++tj) {
      v4f akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int k0 = 0; k0 < DK; k0 += 4) {
        const float ka = Ks[(16 * wv + i) * KP + k0 + kk];
        const float qa = Qs[(16 * wv + i) * KP + k0 + kk];
        const float kb = Ks[(16 * tj + i) * KP + k0 + kk];
        akk = mfma4(ka, kb, akk);
        aqk = mfma4(qa, kb, aqk);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wv + 4 * kk + r, s = 16 * tj + i;
        const float dec = expf(Gs[t] - Gs[s < t ? s : t]);
        As[t * AP + s] = s < t ? Bs[t] * dec * akk[r] : 0.f;
        if (t < nt)
          ws.P[((size_t)(jb + t) * Hv + h) * kC + s] = s <= t ? dec * aqk[r] : 0.f;
      }
    }
  }
  __syncthreads();
  // 4. T = (I + A)^{-1}: lane j of wave 0 solves column j by forward substitution
  if (wv == 0) {
    float X[kC];
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      float x = (t == lane) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < t; ++s) x = fmaf(-As[t * AP + s], X[s], x);
      X[t] = x;
    }
#pragma unroll
    for (int t = 0; t < kC; ++t) As[t * AP + lane] = X[t];
  }
  // values replace the queries (Q K^T is done)
  vpark.template store<KP>(Qs);
  __syncthreads();
  // 5. W = T diag(b e^G) K and U~ = T diag(b) V; wave w owns token tile w
  {
    const int i = lane & 15, kk = lane >> 4;
    for (int n = 0; n < DK / 16; ++n) {
      v4f aw = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int s0 = 0; s0 < kC; s0 += 4) {
        const int s = s0 + kk;
        const float ta = As[(16 * wv + i) * AP + s];
        aw = mfma4(ta, BG[s] * Ks[s * KP + 16 * n + i], aw);
        au = mfma4(ta, Bs[s] * Qs[s * KP + 16 * n + i], au);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wv + 4 * kk + r;
        if (t < nt) {
          const size_t o = ((size_t)(jb + t) * Hv + h) * DK + 16 * n + i;
          ws.W[o] = aw[r];
          ws.U[o] = au[r];
        }
      }
    }
  }
  if (tid < nt) ws.G[(size_t)(jb + tid) * Hv + h] = Gs[tid];
}

// Shared memory of chunk_state_kernel.
template <int DK>
struct StateLds {
  static constexpr int wl = 0;                    // [kC][DK+4] W of the chunk
  static constexpr int ql = wl + kC * (DK + 4);   // [kC][DK+4] queries
  static constexpr int kl = ql + kC * (DK + 4);   // [kC][DK+4] keys
  static constexpr int pl = kl + kC * (DK + 4);   // [kC][kC+4] P
  static constexpr int ss = pl + kC * (kC + 4);   // [16][DK+1] state block
  static constexpr int us = ss + 16 * (DK + 1);   // [kC][17] U block
  static constexpr int gc = us + kC * 17;         // [kC] G
  static constexpr int total = gc + kC;
};

template <int DK, int DV>
__global__ void __launch_bounds__(256)
chunk_state_kernel(PrefillArgs p, const float* __restrict__ y, ChunkWs ws) {
  static_assert(DK == DV && DK % 64 == 0, "dk == dv, multiple of 64");
  extern __shared__ __align__(16) float sm[];
  using Lay = StateLds<DK>;
  float* Wl = sm + Lay::wl;
  float* Ql = sm + Lay::ql;
  float* Kl = sm + Lay::kl;
  float* Pl = sm + Lay::pl;
  float* Ss = sm + Lay::ss;
  float* Us = sm + Lay::us;
  float* Gc = sm + Lay::gc;
  constexpr int KP = DK + 4, AP = kC + 4, SP = DK + 1, UP = 17;
  constexpr int TPW = (DK / 16) / 4;  // state tiles per wave

  const int Hv = p.Hv, Hk = p.Hk, C = p.C;
  const int row = blockIdx.x / Hv, h = blockIdx.x - row * Hv;
  const int blk = blockIdx.y;  // state rows 16*blk .. 16*blk+15
  const PRow pr = prow(p, row);
  if (pr.T <= 0) return;
  const int ih = h / p.G;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;

  // state rows in C layout: tile m = wv*TPW + q holds S[4*lk + r][16m + li]
  v4f St[TPW];
  const size_t tile_base = ((size_t)pr.slot * Hv + h) * DV * DK + (size_t)(16 * blk) * DK;
#pragma unroll
  for (int q = 0; q < TPW; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      St[q][r] = pr.init ? p.ssm_pool[tile_base + (size_t)(4 * lk + r) * DK + 16 * (wv * TPW + q) + li]
                         : 0.f;

  const int nch = (pr.T + kC - 1) / kC;
  // Operands of chunk c+1 are gathered while chunk c is computed.
  Tile4<kC, DK> tw, tq, tk;
  Tile4<kC, kC> tp;
  auto gather = [&](int c) {
    const int jb = pr.j0 + c * kC;
    const int nt = min(kC, pr.T - c * kC);
    const float* yb = y + (size_t)jb * C;
    tw.load([&](int r) { return ws.W + ((size_t)(jb + r) * Hv + h) * DK; }, nt);
    tq.load([&](int r) { return yb + (size_t)r * C + ih * DK; }, nt);
    tk.load([&](int r) { return yb + (size_t)r * C + Hk * DK + ih * DK; }, nt);
    tp.load([&](int r) { return ws.P + ((size_t)(jb + r) * Hv + h) * kC; }, nt);
  };
  gather(0);
  for (int c = 0; c < nch; ++c) {
    const int jb = pr.j0 + c * kC;
    const int nt = min(kC, pr.T - c * kC);
    tw.template store<KP>(Wl);
    tq.template store<KP>(Ql);
    tk.template store<KP>(Kl);
    tp.template store<AP>(Pl);
    if (tid < kC) Gc[tid] = ws.G[(size_t)(jb + (tid < nt ? tid : nt - 1)) * Hv + h];
#pragma unroll
    for (int q = 0; q < TPW; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) Ss[(4 * lk + r) * SP + 16 * (wv * TPW + q) + li] = St[q][r];
    __syncthreads();
    if (c + 1 < nch) gather(c + 1);
    __syncthreads();

    // (a) U = U~ - W S0^T for token tile wv
    {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int k0 = 0; k0 < DK; k0 += 4)
        acc = mfma4(Wl[(16 * wv + li) * KP + k0 + lk], Ss[li * SP + k0 + lk], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wv + 4 * lk + r;
        const float ut =
            t < nt ? ws.U[((size_t)(jb + t) * Hv + h) * DV + 16 * blk + li] : 0.f;
        Us[t * UP + li] = t < nt ? ut - acc[r] : 0.f;
      }
    }
    __syncthreads();

    // (b) outputs of token tile wv: e^{G_t} (Q S0^T)[t] + (P U)[t]
    {
      v4f aq = {0.f, 0.f, 0.f, 0.f}, ap = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int k0 = 0; k0 < DK; k0 += 4)
        aq = mfma4(Ql[(16 * wv + li) * KP + k0 + lk], Ss[li * SP + k0 + lk], aq);
#pragma unroll 4
      for (int s0 = 0; s0 < kC; s0 += 4)
        ap = mfma4(Pl[(16 * wv + li) * AP + s0 + lk], Us[(s0 + lk) * UP + li], ap);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wv + 4 * lk + r;
        if (t < nt) {
          const int j = jb + t;
          int gr = p.tix ? p.tix[j] : j;
          if (gr >= 0 && gr < p.num_actual_tokens)
            p.out[((size_t)gr * Hv + h) * DV + 16 * blk + li] =
                f2bf(fmaf(expf(Gc[t]), aq[r], ap[r]));
        }
      }
    }

    // (c) S = e^{G_C} S0 + U^T diag(e^{G_C - G_t}) K for this wave's tiles
    {
      const float gC = Gc[kC - 1];
      const float eC = expf(gC);
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int m = wv * TPW + q;
        v4f acc = St[q] * eC;
#pragma unroll 4
        for (int s0 = 0; s0 < kC; s0 += 4) {
          const int s = s0 + lk;
          acc = mfma4(Us[s * UP + li], expf(gC - Gc[s]) * Kl[s * KP + 16 * m + li], acc);
        }
        St[q] = acc;
      }
    }
    __syncthreads();
  }
  if (pr.slot > 0) {
#pragma unroll
    for (int q = 0; q < TPW; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p.ssm_pool[tile_base + (size_t)(4 * lk + r) * DK + 16 * (wv * TPW + q) + li] = St[q][r];
  }
}

}  // namespace

size_t chunk_lds_prep(int dk) {
  switch (dk) {
    case 64: return sizeof(float) * PrepLds<64>::total;
    case 128: return sizeof(float) * PrepLds<128>::total;
    default: return 0;
  }
}

size_t chunk_lds_state(int dk) {
  switch (dk) {
    case 64: return sizeof(float) * StateLds<64>::total;
    case 128: return sizeof(float) * StateLds<128>::total;
    default: return 0;
  }
}

template <int DK, int DV>
static hipError_t launch_chunked_typed(const PrefillArgs& a, const float* y, const float* glog,
                                       const float* gbeta, const ChunkWs& ws, hipStream_t s) {
  const size_t l1 = sizeof(float) * PrepLds<DK>::total;
  const size_t l2 = sizeof(float) * StateLds<DK>::total;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_prep_kernel<DK, DV>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)l1);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_state_kernel<DK, DV>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)l2);
  if (e != hipSuccess) return e;
  const int nch = (a.max_row_len + kC - 1) / kC;
  if (nch <= 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_prep_kernel<DK, DV>), dim3(nch, a.Hv, a.num_rows), dim3(256), l1, s,
                     a, y, glog, gbeta, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Head index fastest, so the 16-row blocks of one head share an XCD's L2.
  hipLaunchKernelGGL((chunk_state_kernel<DK, DV>), dim3(a.Hv * a.num_rows, DV / 16), dim3(256), l2,
                     s, a, y, ws);
  return hipGetLastError();
}

hipError_t launch_chunked(const PrefillArgs& a, int dk, int dv, const float* y, const float* glog,
                          const float* gbeta, const ChunkWs& ws, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 64: return launch_chunked_typed<64, 64>(a, y, glog, gbeta, ws, s);
    case 128: return launch_chunked_typed<128, 128>(a, y, glog, gbeta, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
