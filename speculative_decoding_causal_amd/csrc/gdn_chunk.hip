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

// N consecutive floats of LDS (16-byte aligned) into registers.
template <int N>
__device__ __forceinline__ void lds_run(float (&dst)[N], const float* src) {
  static_assert(N % 4 == 0, "runs of float4");
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const v4f v = *reinterpret_cast<const v4f*>(src + 4 * i);
    dst[4 * i] = v.x;
    dst[4 * i + 1] = v.y;
    dst[4 * i + 2] = v.z;
    dst[4 * i + 3] = v.w;
  }
}

// Operand feeding: the sum over k is split so that lane group kk = lane/16
// owns the contiguous range k = kk*(K/4) + m of every MFMA step m; both
// operands use the same split, so each lane reads its operands for all K/4
// steps as one contiguous run.

// Shared-memory carve-up of chunk_prep_kernel (floats).  Row pitches are
// padded by four: rows stay 16-byte aligned and column reads spread over
// the banks.
template <int DK>
struct PrepLds {
  static constexpr int KP = DK + 4, CP = kC + 4;
  static constexpr int ks = 0;                          // [kC][KP]  keys
  static constexpr int qv = ks + kC * KP;               // [kC][KP]  queries, then values
  static constexpr int ts = qv + kC * KP;               // [kC][CP]  A, then T
  static constexpr int gs = ts + kC * CP;               // [kC] cumulative log-decay
  static constexpr int bs = gs + kC;                    // [kC] beta
  static constexpr int bg = bs + kC;                    // [kC] beta e^G
  static constexpr int total = bg + kC;
};

template <int DK, int DV>
__global__ void __launch_bounds__(256)
chunk_prep_kernel(PrefillArgs p, const float* __restrict__ y, const float* __restrict__ glog,
                  const float* __restrict__ gbeta, ChunkWs ws) {
  static_assert(DK == DV, "dk == dv");
  extern __shared__ __align__(16) float sm[];
  using Lay = PrepLds<DK>;
  constexpr int KP = Lay::KP, CP = Lay::CP;
  constexpr int KQ = DK / 4;   // k-run per lane group, Gram products
  constexpr int SQ = kC / 4;   // k-run per lane group, products over tokens
  float* Ks = sm + Lay::ks;
  float* QV = sm + Lay::qv;
  float* Ts = sm + Lay::ts;
  float* Gs = sm + Lay::gs;
  float* Bs = sm + Lay::bs;
  float* BG = sm + Lay::bg;

  const int c = blockIdx.x, h = blockIdx.y;
  const PRow pr = prow(p, blockIdx.z);
  const int t0 = c * kC;
  if (t0 >= pr.T) return;
  const int nt = min(kC, pr.T - t0);
  const int jb = pr.j0 + t0;
  const int ih = h / p.G, Hk = p.Hk, Hv = p.Hv, C = p.C;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;

  // 1. keys, queries and values of the chunk gathered in one batch
  Tile4<kC, DV> tv;
  {
    Tile4<kC, DK> tk, tq;
    const float* yb = y + (size_t)jb * C;
    tk.load([&](int r) { return yb + (size_t)r * C + Hk * DK + ih * DK; }, nt);
    tq.load([&](int r) { return yb + (size_t)r * C + ih * DK; }, nt);
    tv.load([&](int r) { return yb + (size_t)r * C + 2 * Hk * DK + h * DV; }, nt);
    tk.template store<KP>(Ks);
    tq.template store<KP>(QV);
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
  // 3. K K^T and Q K^T: wave w owns token-row tile w
  {
    float ak[KQ], aq[KQ];
    lds_run<KQ>(ak, Ks + (16 * wv + li) * KP + lk * KQ);
    lds_run<KQ>(aq, QV + (16 * wv + li) * KP + lk * KQ);
    for (int tj = 0; tj < 4; ++tj) {
      float bk[KQ];
      lds_run<KQ>(bk, Ks + (16 * tj + li) * KP + lk * KQ);
      v4f akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KQ; ++m) {
        akk = mfma4(ak[m], bk[m], akk);
        aqk = mfma4(aq[m], bk[m], aqk);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wv + 4 * lk + r, s = 16 * tj + li;
        const float dec = expf(Gs[t] - Gs[s < t ? s : t]);
        Ts[t * CP + s] = s < t ? Bs[t] * dec * akk[r] : 0.f;
        if (t < nt)
          ws.P[((size_t)(jb + t) * Hv + h) * kC + s] = s <= t ? dec * aqk[r] : 0.f;
      }
    }
  }
  __syncthreads();
  // 4. T = (I + A)^{-1}: lane j of wave 0 solves column j by forward
  //    substitution (four partial sums per row); the values replace the
  //    queries.
  if (wv == 0) {
    float X[kC];
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      float x0 = (t == lane) ? 1.f : 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
#pragma unroll
      for (int s = 0; s < t; ++s) {
        const float a = Ts[t * CP + s];
        if ((s & 3) == 0) x0 = fmaf(-a, X[s], x0);
        else if ((s & 3) == 1) x1 = fmaf(-a, X[s], x1);
        else if ((s & 3) == 2) x2 = fmaf(-a, X[s], x2);
        else x3 = fmaf(-a, X[s], x3);
      }
      X[t] = (x0 + x1) + (x2 + x3);
    }
#pragma unroll
    for (int t = 0; t < kC; ++t) Ts[t * CP + lane] = X[t];
  }
  tv.template store<KP>(QV);
  __syncthreads();
  // 5. W = T diag(b e^G) K and U~ = T diag(b) V: wave w owns token tile w.
  //    The sum over tokens s takes the interleaved split s = 4m + lane/16, so
  //    the key/value operand is a row-major read spread over the banks.
  {
    float at[SQ], bgr[SQ], br[SQ];
#pragma unroll
    for (int m = 0; m < SQ; ++m) {
      at[m] = Ts[(16 * wv + li) * CP + 4 * m + lk];
      bgr[m] = BG[4 * m + lk];
      br[m] = Bs[4 * m + lk];
    }
    for (int n = 0; n < DK / 16; ++n) {
      v4f aw = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < SQ; ++m) {
        const int srow = (4 * m + lk) * KP + 16 * n + li;
        aw = mfma4(at[m], bgr[m] * Ks[srow], aw);
        au = mfma4(at[m], br[m] * QV[srow], au);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wv + 4 * lk + r;
        if (t < nt) {
          const size_t o = ((size_t)(jb + t) * Hv + h) * DK + 16 * n + li;
          ws.W[o] = aw[r];
          ws.U[o] = au[r];
        }
      }
    }
  }
  if (tid < nt) ws.G[(size_t)(jb + tid) * Hv + h] = Gs[tid];
}

// Shared memory of chunk_state_kernel (floats).
template <int DK>
struct StateLds {
  static constexpr int KP = DK + 4, CP = kC + 4;
  static constexpr int wl = 0;                    // [kC][KP] W of the chunk
  static constexpr int ql = wl + kC * KP;         // [kC][KP] queries
  static constexpr int kl = ql + kC * KP;         // [kC][KP] keys
  static constexpr int pl = kl + kC * KP;         // [kC][CP] P
  static constexpr int ul = pl + kC * CP;         // [kC][16] U~ block
  static constexpr int ss = ul + kC * 16;         // [16][KP] state block
  static constexpr int ut = ss + 16 * KP;         // [16][CP] U^T block
  static constexpr int uts = ut + 16 * CP;        // [16][CP] U^T diag(e^{G_C - G})
  static constexpr int gc = uts + 16 * CP;        // [kC] G
  static constexpr int total = gc + kC;
};

template <int DK, int DV>
__global__ void __launch_bounds__(256)
chunk_state_kernel(PrefillArgs p, const float* __restrict__ y, ChunkWs ws) {
  static_assert(DK == DV && DK % 64 == 0, "dk == dv, multiple of 64");
  extern __shared__ __align__(16) float sm[];
  using Lay = StateLds<DK>;
  constexpr int KP = Lay::KP, CP = Lay::CP;
  constexpr int KQ = DK / 4, SQ = kC / 4;
  constexpr int TPW = (DK / 16) / 4;  // state tiles per wave
  float* Wl = sm + Lay::wl;
  float* Ql = sm + Lay::ql;
  float* Kl = sm + Lay::kl;
  float* Pl = sm + Lay::pl;
  float* Ul = sm + Lay::ul;
  float* Ss = sm + Lay::ss;
  float* UT = sm + Lay::ut;
  float* UTs = sm + Lay::uts;
  float* Gc = sm + Lay::gc;

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
  Tile4<kC, 16> tu;
  auto gather = [&](int c) {
    const int jb = pr.j0 + c * kC;
    const int nt = min(kC, pr.T - c * kC);
    const float* yb = y + (size_t)jb * C;
    tw.load([&](int r) { return ws.W + ((size_t)(jb + r) * Hv + h) * DK; }, nt);
    tq.load([&](int r) { return yb + (size_t)r * C + ih * DK; }, nt);
    tk.load([&](int r) { return yb + (size_t)r * C + Hk * DK + ih * DK; }, nt);
    tp.load([&](int r) { return ws.P + ((size_t)(jb + r) * Hv + h) * kC; }, nt);
    tu.load([&](int r) { return ws.U + ((size_t)(jb + r) * Hv + h) * DV + 16 * blk; }, nt);
  };
  gather(0);
  for (int c = 0; c < nch; ++c) {
    const int jb = pr.j0 + c * kC;
    const int nt = min(kC, pr.T - c * kC);
    tw.template store<KP>(Wl);
    tq.template store<KP>(Ql);
    tk.template store<KP>(Kl);
    tp.template store<CP>(Pl);
    tu.template store<16>(Ul);
    if (tid < kC) Gc[tid] = ws.G[(size_t)(jb + (tid < nt ? tid : nt - 1)) * Hv + h];
#pragma unroll
    for (int q = 0; q < TPW; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) Ss[(4 * lk + r) * KP + 16 * (wv * TPW + q) + li] = St[q][r];
    __syncthreads();
    if (c + 1 < nch) gather(c + 1);

    const float gC = Gc[kC - 1];
    // B operand of S0^T products: S[j][k] for this lane's k-run
    float sb[KQ];
    lds_run<KQ>(sb, Ss + li * KP + lk * KQ);
    // (a) U = U~ - W S0^T for token tile wv; U^T kept plain and decay-scaled
    {
      float aw[KQ];
      lds_run<KQ>(aw, Wl + (16 * wv + li) * KP + lk * KQ);
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KQ; ++m) acc = mfma4(aw[m], sb[m], acc);
      v4f u, us;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wv + 4 * lk + r;
        u[r] = t < nt ? Ul[t * 16 + li] - acc[r] : 0.f;
        us[r] = u[r] * expf(gC - Gc[t]);
      }
      *reinterpret_cast<v4f*>(UT + li * CP + 16 * wv + 4 * lk) = u;
      *reinterpret_cast<v4f*>(UTs + li * CP + 16 * wv + 4 * lk) = us;
    }
    __syncthreads();

    // (b) outputs of token tile wv: e^{G_t} (Q S0^T)[t] + (P U)[t]
    {
      float aqr[KQ], apr[SQ], ubr[SQ];
      lds_run<KQ>(aqr, Ql + (16 * wv + li) * KP + lk * KQ);
      lds_run<SQ>(apr, Pl + (16 * wv + li) * CP + lk * SQ);
      lds_run<SQ>(ubr, UT + li * CP + lk * SQ);
      v4f aq = {0.f, 0.f, 0.f, 0.f}, ap = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KQ; ++m) aq = mfma4(aqr[m], sb[m], aq);
#pragma unroll
      for (int m = 0; m < SQ; ++m) ap = mfma4(apr[m], ubr[m], ap);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wv + 4 * lk + r;
        if (t < nt) {
          const int j = jb + t;
          const int gr = p.tix ? p.tix[j] : j;
          if (gr >= 0 && gr < p.num_actual_tokens)
            p.out[((size_t)gr * Hv + h) * DV + 16 * blk + li] =
                f2bf(fmaf(expf(Gc[t]), aq[r], ap[r]));
        }
      }
    }

    // (c) S = e^{G_C} S0 + U^T diag(e^{G_C - G_t}) K for this wave's tiles
    //     (interleaved split s = 4m + lane/16: row-major key reads)
    {
      float ua[SQ];
#pragma unroll
      for (int m = 0; m < SQ; ++m) ua[m] = UTs[li * CP + 4 * m + lk];
      const float eC = expf(gC);
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int mt = wv * TPW + q;
        v4f acc = St[q] * eC;
#pragma unroll
        for (int m = 0; m < SQ; ++m) acc = mfma4(ua[m], Kl[(4 * m + lk) * KP + 16 * mt + li], acc);
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
