// Chunked (WY / UT) form of the gated delta rule for prefill rows, on MFMA.
//
// The recurrence S_t = a_t S_{t-1} + u_t k_t^T, u_t = b_t (v_t - a_t S_{t-1} k_t)
// (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", chunkwise form) is
// evaluated 64 tokens at a time.  With G_t the cumulative log-decay inside a
// chunk (G_t = sum_{s<=t} log a_s) and only decay differences t >= s ever
// exponentiated:
//   A  = strictly-lower( b_t e^{G_t - G_s} k_t.k_s )          (C x C)
//   T  = (I + A)^{-1}                                         (unit lower)
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
// chunk_state_kernel: one workgroup per (row, v-head, 32 state rows) carries
// its rows of S through the row's chunks in MFMA accumulators and writes the
// outputs through token_indx.  Dense products use v_mfma_f32_16x16x4f32
// (A[i][k] at lane i+16k, B[k][j] at lane j+16k, D[i][j] at lane j+16*(i/4),
// element i%4).
//
// Sums over the 64 tokens of a chunk take 16 MFMA steps m = 4M + e, lane group
// kk = lane/16 adding token s = 16M + 4kk + e: token block M (16 tokens) is one
// group of four steps, so blocks a triangular factor zeroes are skipped, and a
// lane's A operand for a block is one float4.
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

// LDS tiles hold P floats per row (P a multiple of 64, no padding); the
// float4 groups of row r are XOR-permuted by r mod 16.  Float4 reads of 16
// consecutive rows, scalar writes of an MFMA result (rows 4kk+i, 16
// consecutive columns) and scalar reads of rows 4kk+e over 16 consecutive
// columns then all hit distinct banks.
template <int P>
__device__ __forceinline__ int sw(int r, int c) {
  return r * P + (c ^ ((r & 15) << 2));
}

template <int P>
__device__ __forceinline__ v4f ld4(const float* t, int r, int c) {
  return *reinterpret_cast<const v4f*>(t + sw<P>(r, c));
}

// N consecutive floats of row r from column c0 (a multiple of 4).
template <int P, int N>
__device__ __forceinline__ void lds_run(float (&dst)[N], const float* t, int r, int c0) {
  static_assert(N % 4 == 0, "runs of float4");
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const v4f v = ld4<P>(t, r, c0 + 4 * i);
    dst[4 * i] = v.x;
    dst[4 * i + 1] = v.y;
    dst[4 * i + 2] = v.z;
    dst[4 * i + 3] = v.w;
  }
}

// Workgroups go to the XCDs round-robin by linear index.  With Hv a multiple
// of 8 and the head index fastest in the grid, index x lands on XCD x mod 8;
// head (x mod 8) * Hv/8 + x / 8 then gives each XCD a contiguous run of
// heads, so v-heads that share a k-head share that XCD's L2.
__device__ __forceinline__ int head_of(int x, int Hv) {
  return (Hv & 7) ? x : (x & 7) * (Hv >> 3) + (x >> 3);
}

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

// Rows of ROWS x COLS floats gathered in one batch of float4 loads, then
// written to LDS.  Thread x loads row x*4/COLS + i*NT*4/COLS of the tile:
// one uniform base per i and one 32-bit lane offset.  Rows >= nrow are
// loaded too and dropped (zeros kept): every array read this way holds a
// chunk of padding rows past its last token, so the loads stay inside it,
// and no load sits behind a branch.
template <int ROWS, int COLS, int NT = 256>
struct Tile4 {
  static_assert((ROWS * COLS / 4) % NT == 0 && (NT * 4) % COLS == 0, "tile shape");
  static constexpr int kPer = ROWS * COLS / 4 / NT;  // float4 per thread
  static constexpr int kRowStep = NT * 4 / COLS;     // rows between them
  v4f v[kPer];
  // base: row 0, column 0 of the tile (uniform); pitch: floats per row
  __device__ __forceinline__ void load(const float* base, int pitch, int nrow) {
    const int r0 = (int)threadIdx.x * 4 / COLS, c0 = (int)threadIdx.x * 4 % COLS;
    const unsigned off = (unsigned)(r0 * pitch + c0);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const float* bi = base + (size_t)(i * kRowStep) * pitch;
      const v4f x = *reinterpret_cast<const v4f*>(bi + off);
      v[i] = r0 + i * kRowStep < nrow ? x : v4f{0.f, 0.f, 0.f, 0.f};
    }
  }
  // swizzled tile of row length COLS
  __device__ __forceinline__ void store_sw(float* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = (i * NT + (int)threadIdx.x) * 4;
      const int r = e / COLS, c = e - r * COLS;
      *reinterpret_cast<v4f*>(lds + sw<COLS>(r, c)) = v[i];
    }
  }
  // row-major tile with row pitch PITCH (a multiple of 4)
  template <int PITCH>
  __device__ __forceinline__ void store_pitched(float* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = (i * NT + (int)threadIdx.x) * 4;
      const int r = e / COLS, c = e - r * COLS;
      *reinterpret_cast<v4f*>(lds + r * PITCH + c) = v[i];
    }
  }
};

// Shared-memory carve-up of chunk_prep_kernel (floats).
template <int DK>
struct PrepLds {
  static constexpr int MP = 20;                 // pitch of the 16x16 scratch
  static constexpr int ks = 0;                  // [kC][DK] keys
  static constexpr int qv = ks + kC * DK;       // [kC][DK] queries, then values
  static constexpr int as = qv + kC * DK;       // [kC][kC] A
  static constexpr int tt = as + kC * kC;       // [kC][kC] T
  static constexpr int mw = tt + kC * kC;       // [4][16][MP] per-wave scratch
  static constexpr int gs = mw + 4 * 16 * MP;   // [kC] cumulative log-decay
  static constexpr int bs = gs + kC;            // [kC] beta
  static constexpr int bg = bs + kC;            // [kC] beta e^G
  static constexpr int total = bg + kC;
};

template <int DK, int DV>
__global__ void __launch_bounds__(256)
chunk_prep_kernel(PrefillArgs p, const float* __restrict__ y, const float* __restrict__ glog,
                  const float* __restrict__ gbeta, ChunkWs ws) {
  static_assert(DK == DV && DK % 64 == 0, "dk == dv, multiple of 64");
  extern __shared__ __align__(16) float sm[];
  using Lay = PrepLds<DK>;
  constexpr int MP = Lay::MP;
  constexpr int KQ = DK / 4;   // k-run per lane group, Gram products
  float* Ks = sm + Lay::ks;
  float* QV = sm + Lay::qv;
  float* As = sm + Lay::as;
  float* Tt = sm + Lay::tt;
  float* Gs = sm + Lay::gs;
  float* Bs = sm + Lay::bs;
  float* BG = sm + Lay::bg;

  const int row = p.unit_map[2 * blockIdx.y];
  if (row < 0) return;
  const int c = p.unit_map[2 * blockIdx.y + 1], h = head_of(blockIdx.x, p.Hv);
  const PRow pr = prow(p, row);
  const int t0 = c * kC;
  if (t0 >= pr.T) return;
  const int nt = min(kC, pr.T - t0);
  const int jb = pr.j0 + t0;
  const int ih = h / p.G, Hk = p.Hk, Hv = p.Hv, C = p.C;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  float* Mw = sm + Lay::mw + wv * 16 * MP;

  // 1. keys, queries and values of the chunk gathered in one batch
  Tile4<kC, DV> tv;
  {
    Tile4<kC, DK> tk, tq;
    const float* yb = y + (size_t)jb * C;
    tk.load(yb + Hk * DK + ih * DK, C, nt);
    tq.load(yb + ih * DK, C, nt);
    tv.load(yb + 2 * Hk * DK + h * DV, C, nt);
    tk.store_sw(Ks);
    tq.store_sw(QV);
  }
  if (tid < kC) {
    Gs[tid] = tid < nt ? glog[(size_t)(jb + tid) * Hv + h] : 0.f;
    Bs[tid] = tid < nt ? gbeta[(size_t)(jb + tid) * Hv + h] : 0.f;
  }
  // P is zero right of its diagonal blocks
  {
    float* Pg = ws.P + ((size_t)jb * Hv + h) * kC;
#pragma unroll
    for (int i = 0; i < kC * kC / 4 / 256; ++i) {
      const int e = i * 256 + tid, t = e >> 4, g = e & 15;
      if ((g >> 2) > (t >> 4) && t < nt)
        *reinterpret_cast<v4f*>(Pg + (size_t)t * Hv * kC + 4 * g) = v4f{0.f, 0.f, 0.f, 0.f};
    }
  }
  lds_barrier();
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
  lds_barrier();
  // 3. K K^T and Q K^T on the ten 16x16 tiles (ti >= tj) that A and P use:
  //    twenty tile products, five per wave (waves 0 and 2 K K^T, 1 and 3
  //    Q K^T; waves 0 and 1 the even tiles in row order, 2 and 3 the odd).
  {
    const bool qk = (wv & 1) != 0;
    const float* Asrc = qk ? QV : Ks;
#pragma unroll
    for (int it = 0; it < 5; ++it) {
      const int x = 2 * it + (wv >> 1);
      const int ti = x < 1 ? 0 : (x < 3 ? 1 : (x < 6 ? 2 : 3));
      const int tj = x - ti * (ti + 1) / 2;
      float ar[KQ], br[KQ];
      lds_run<DK>(ar, Asrc, 16 * ti + li, lk * KQ);
      lds_run<DK>(br, Ks, 16 * tj + li, lk * KQ);
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KQ; ++m) acc = mfma4(ar[m], br[m], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ti + 4 * lk + r, s = 16 * tj + li;
        const float dec = expf(Gs[t] - Gs[s < t ? s : t]);
        if (!qk)
          As[sw<kC>(t, s)] = s < t ? Bs[t] * dec * acc[r] : 0.f;
        else if (t < nt)
          ws.P[((size_t)(jb + t) * Hv + h) * kC + s] = s <= t ? dec * acc[r] : 0.f;
      }
    }
  }
  lds_barrier();
  // 4. T = (I + A)^{-1} in 16x16 blocks.  Wave w inverts diagonal block w by
  //    forward substitution (lane j of each 16 solves column j) and clears
  //    T's blocks right of it; the values replace the queries meanwhile.
  {
    const int b0 = 16 * wv;
    float X[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float x0 = (t == li) ? 1.f : 0.f, x1 = 0.f;
#pragma unroll
      for (int g = 0; g < (t + 3) / 4; ++g) {
        const v4f a = ld4<kC>(As, b0 + t, b0 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = 4 * g + e;
          if (s < t) {
            if (e & 1) x1 = fmaf(-a[e], X[s], x1);
            else x0 = fmaf(-a[e], X[s], x0);
          }
        }
      }
      X[t] = x0 + x1;
    }
    if (lk == 0) {
#pragma unroll
      for (int t = 0; t < 16; ++t) Tt[sw<kC>(b0 + t, b0 + li)] = X[t];
    }
    for (int cb = wv + 1; cb < 4; ++cb)
      *reinterpret_cast<v4f*>(Tt + sw<kC>(b0 + li, 16 * cb + 4 * lk)) = v4f{0.f, 0.f, 0.f, 0.f};
  }
  tv.store_sw(QV);
  lds_barrier();
  //    Blocks below the diagonal, one diagonal level at a time:
  //    T_ij = -T_ii M with M = sum_{k=j}^{i-1} A_ik T_kj (wave w: j = w).
  for (int lv = 1; lv < 4; ++lv) {
    const bool act = wv < 4 - lv;
    const int i = wv + lv, j = wv;
    if (act) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      for (int k = j; k < i; ++k) {
        const v4f a = ld4<kC>(As, 16 * i + li, 16 * k + 4 * lk);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = mfma4(a[e], Tt[sw<kC>(16 * k + 4 * lk + e, 16 * j + li)], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) Mw[(4 * lk + r) * MP + li] = acc[r];
    }
    lds_barrier();
    if (act) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      const v4f d = ld4<kC>(Tt, 16 * i + li, 16 * i + 4 * lk);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma4(d[e], Mw[(4 * lk + e) * MP + li], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) Tt[sw<kC>(16 * i + 4 * lk + r, 16 * j + li)] = -acc[r];
    }
    lds_barrier();
  }
  // 5. W = T diag(b e^G) K and U~ = T diag(b) V.  Wave w computes column
  //    tiles NW*w .. NW*w+NW-1 for every token tile; token block M feeds
  //    token tiles ti >= M only (T is block lower triangular).
  {
    constexpr int NW = DK / 64;
    v4f aw[4][NW], au[4][NW];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        aw[ti][q] = v4f{0.f, 0.f, 0.f, 0.f};
        au[ti][q] = v4f{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int M = 0; M < 4; ++M) {
      const v4f g4 = *reinterpret_cast<const v4f*>(BG + 16 * M + 4 * lk);
      const v4f b4 = *reinterpret_cast<const v4f*>(Bs + 16 * M + 4 * lk);
      float kb[4][NW], vb[4][NW];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int q = 0; q < NW; ++q) {
          const int sidx = sw<DK>(16 * M + 4 * lk + e, 16 * (NW * wv + q) + li);
          kb[e][q] = g4[e] * Ks[sidx];
          vb[e][q] = b4[e] * QV[sidx];
        }
#pragma unroll
      for (int ti = M; ti < 4; ++ti) {
        const v4f a = ld4<kC>(Tt, 16 * ti + li, 16 * M + 4 * lk);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int q = 0; q < NW; ++q) {
            aw[ti][q] = mfma4(a[e], kb[e][q], aw[ti][q]);
            au[ti][q] = mfma4(a[e], vb[e][q], au[ti][q]);
          }
      }
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ti + 4 * lk + r;
        if (t < nt) {
#pragma unroll
          for (int q = 0; q < NW; ++q) {
            const size_t o = ((size_t)(jb + t) * Hv + h) * DK + 16 * (NW * wv + q) + li;
            ws.W[o] = aw[ti][q][r];
            ws.U[o] = au[ti][q][r];
          }
        }
      }
  }
  if (tid < nt) ws.G[(size_t)(jb + tid) * Hv + h] = Gs[tid];
}

// Shared memory of chunk_state_kernel (floats); RB state rows per workgroup.
template <int DK, int RB>
struct StateLds {
  static constexpr int UP = RB + 4;               // pitch of the U~ block
  static constexpr int wl = 0;                    // [kC][DK] W of the chunk
  static constexpr int ql = wl + kC * DK;         // [kC][DK] queries
  static constexpr int kl = ql + kC * DK;         // [kC][DK] keys
  static constexpr int pl = kl + kC * DK;         // [kC][kC] P
  static constexpr int ul = pl + kC * kC;         // [kC][UP] U~ block (plain)
  static constexpr int ss = ul + kC * UP;         // [RB][DK] state block
  static constexpr int ut = ss + RB * DK;         // [RB][kC] U^T block
  static constexpr int gc = ut + RB * kC;         // [kC] G
  static constexpr int fs = gc + kC;              // [kC] e^{G_C - G_t}
  static constexpr int total = fs + kC;
};

constexpr int kStateThreads = 512;  // 8 waves, two per SIMD
constexpr int kStateRows = 32;      // state rows per workgroup

// Wave w works on token tile tt = w % 4 and state-row tile jt = w / 4 for
// U and the outputs, and on state tiles (jt, TPW*tt + q) for the update.
template <int DK, int DV>
__global__ void __launch_bounds__(kStateThreads)
chunk_state_kernel(PrefillArgs p, const float* __restrict__ y, ChunkWs ws) {
  static_assert(DK == DV && DK % 64 == 0, "dk == dv, multiple of 64");
  constexpr int NT = kStateThreads, RB = kStateRows;
  extern __shared__ __align__(16) float sm[];
  using Lay = StateLds<DK, RB>;
  constexpr int UP = Lay::UP;
  constexpr int KQ = DK / 4;
  constexpr int TPW = DK / 64;  // state column tiles per wave
  float* Wl = sm + Lay::wl;
  float* Ql = sm + Lay::ql;
  float* Kl = sm + Lay::kl;
  float* Pl = sm + Lay::pl;
  float* Ul = sm + Lay::ul;
  float* Ss = sm + Lay::ss;
  float* UT = sm + Lay::ut;
  float* Gc = sm + Lay::gc;
  float* Fs = sm + Lay::fs;

  const int Hv = p.Hv, Hk = p.Hk, C = p.C;
  const int row = blockIdx.x / Hv, h = head_of(blockIdx.x - row * Hv, Hv);
  const int blk = blockIdx.y;  // state rows RB*blk .. RB*blk+RB-1
  const PRow pr = prow(p, row);
  if (pr.T <= 0) return;
  const int ih = h / p.G;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int tt = wv & 3, jt = wv >> 2;

  // state tiles in C layout: St[q] holds S[16 jt + 4 lk + r][16 (TPW tt + q) + li]
  v4f St[TPW];
  const size_t tile_base = ((size_t)pr.slot * Hv + h) * DV * DK + (size_t)(RB * blk + 16 * jt) * DK;
#pragma unroll
  for (int q = 0; q < TPW; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      St[q][r] = pr.init ? p.ssm_pool[tile_base + (size_t)(4 * lk + r) * DK + 16 * (TPW * tt + q) + li]
                         : 0.f;

  const int nch = (pr.T + kC - 1) / kC;
  // Operands of chunk c+1 are gathered while chunk c is computed.
  Tile4<kC, DK, NT> tw, tq, tk;
  Tile4<kC, kC, NT> tp;
  Tile4<kC, RB, NT> tu;
  float tg;     // G of token lane % 64
  int tx[4];    // global rows of this lane's output tokens (-1: none)
  auto gather = [&](int c) {
    const int jb = pr.j0 + c * kC;
    const int nt = min(kC, pr.T - c * kC);
    const float* yb = y + (size_t)jb * C;
    tw.load(ws.W + ((size_t)jb * Hv + h) * DK, Hv * DK, nt);
    tq.load(yb + ih * DK, C, nt);
    tk.load(yb + Hk * DK + ih * DK, C, nt);
    tp.load(ws.P + ((size_t)jb * Hv + h) * kC, Hv * kC, nt);
    tu.load(ws.U + ((size_t)jb * Hv + h) * DV + RB * blk, Hv * DV, nt);
    tg = ws.G[(size_t)(jb + min(lane, nt - 1)) * Hv + h];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tt + 4 * lk + r;
      const int j = jb + min(t, nt - 1);
      const int gr = p.tix ? p.tix[j] : j;
      tx[r] = (t < nt && gr >= 0 && gr < p.num_actual_tokens) ? gr : -1;
    }
  };
  gather(0);
  for (int c = 0; c < nch; ++c) {
    const int nt = min(kC, pr.T - c * kC);
    tw.store_sw(Wl);
    tq.store_sw(Ql);
    tk.store_sw(Kl);
    tp.store_sw(Pl);
    tu.template store_pitched<UP>(Ul);
    if (tid < kC) Gc[tid] = tg;
    int orow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) orow[r] = tx[r];
#pragma unroll
    for (int q = 0; q < TPW; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Ss[sw<DK>(16 * jt + 4 * lk + r, 16 * (TPW * tt + q) + li)] = St[q][r];
    lds_barrier();

    const float gC = Gc[kC - 1];
    if (tid < kC) Fs[tid] = expf(gC - Gc[tid]);
    // B operand of S0^T products: S[j][k], j in row tile jt, this lane's k-run
    float sb[KQ];
    lds_run<DK>(sb, Ss, 16 * jt + li, lk * KQ);
    // (a) U = U~ - W S0^T on (token tile tt, row tile jt), kept as U^T
    {
      float aw[KQ];
      lds_run<DK>(aw, Wl, 16 * tt + li, lk * KQ);
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KQ; ++m) acc = mfma4(aw[m], sb[m], acc);
      v4f u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * lk + r;
        u[r] = t < nt ? Ul[t * UP + 16 * jt + li] - acc[r] : 0.f;
      }
      *reinterpret_cast<v4f*>(UT + sw<kC>(16 * jt + li, 16 * tt + 4 * lk)) = u;
    }
    lds_barrier();
    // the next chunk's operands load during (b) and (c); their registers are
    // free while (a) holds its operand runs
    if (c + 1 < nch) gather(c + 1);

    // (b) outputs on (tt, jt): e^{G_t} (Q S0^T)[t] + (P U)[t]; P is zero
    //     right of the diagonal block
    {
      float aqr[KQ];
      lds_run<DK>(aqr, Ql, 16 * tt + li, lk * KQ);
      v4f aq = {0.f, 0.f, 0.f, 0.f}, ap = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KQ; ++m) aq = mfma4(aqr[m], sb[m], aq);
#pragma unroll
      for (int M = 0; M < 4; ++M) {
        if (M <= tt) {
          const v4f a = ld4<kC>(Pl, 16 * tt + li, 16 * M + 4 * lk);
          const v4f b = ld4<kC>(UT, 16 * jt + li, 16 * M + 4 * lk);
#pragma unroll
          for (int e = 0; e < 4; ++e) ap = mfma4(a[e], b[e], ap);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * lk + r;
        if (orow[r] >= 0)
          p.out[((size_t)orow[r] * Hv + h) * DV + RB * blk + 16 * jt + li] =
              f2bf(fmaf(expf(Gc[t]), aq[r], ap[r]));
      }
    }

    // (c) S = e^{G_C} S0 + U^T diag(e^{G_C - G_t}) K on this wave's tiles
    {
      float ua[16];
#pragma unroll
      for (int M = 0; M < 4; ++M) {
        const v4f a = ld4<kC>(UT, 16 * jt + li, 16 * M + 4 * lk);
        const v4f f = *reinterpret_cast<const v4f*>(Fs + 16 * M + 4 * lk);
#pragma unroll
        for (int e = 0; e < 4; ++e) ua[4 * M + e] = a[e] * f[e];
      }
      const float eC = expf(gC);
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int mt = TPW * tt + q;
        v4f acc = St[q] * eC;
#pragma unroll
        for (int M = 0; M < 4; ++M)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc = mfma4(ua[4 * M + e], Kl[sw<DK>(16 * M + 4 * lk + e, 16 * mt + li)], acc);
        St[q] = acc;
      }
    }
    lds_barrier();
  }
  if (pr.slot > 0) {
#pragma unroll
    for (int q = 0; q < TPW; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p.ssm_pool[tile_base + (size_t)(4 * lk + r) * DK + 16 * (TPW * tt + q) + li] = St[q][r];
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
    case 64: return sizeof(float) * StateLds<64, kStateRows>::total;
    case 128: return sizeof(float) * StateLds<128, kStateRows>::total;
    default: return 0;
  }
}

template <int DK, int DV>
static hipError_t launch_chunked_typed(const PrefillArgs& a, const float* y, const float* glog,
                                       const float* gbeta, const ChunkWs& ws, hipStream_t s) {
  const size_t l1 = sizeof(float) * PrepLds<DK>::total;
  const size_t l2 = sizeof(float) * StateLds<DK, kStateRows>::total;
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(chunk_prep_kernel<DK, DV>), l1);
  if (e != hipSuccess) return e;
  e = ensure_dynamic_lds(reinterpret_cast<const void*>(chunk_state_kernel<DK, DV>), l2);
  if (e != hipSuccess) return e;
  if (a.units <= 0) return hipSuccess;
  // one workgroup per (v-head, 64-token unit of a row), head index fastest
  hipLaunchKernelGGL((chunk_prep_kernel<DK, DV>), dim3(a.Hv, a.units), dim3(256), l1, s,
                     a, y, glog, gbeta, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Head index fastest, so the 16-row blocks of one head share an XCD's L2
  // (grid.x is a multiple of 8 whenever Hv is).
  hipLaunchKernelGGL((chunk_state_kernel<DK, DV>), dim3(a.Hv * a.num_rows, DV / kStateRows),
                     dim3(kStateThreads), l2, s, a, y, ws);
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
