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
// outputs through token_indx.
//
// The blocks of T below its diagonal are solved on v_mfma_f32_16x16x4f32
// (A[i][k] at lane i+16k, B[k][j] at lane j+16k, D[i][j] at lane
// j+16*(i/4), element i%4).  Every other product (K K^T, Q K^T, W, U~ in
// chunk_prep; all of chunk_state) runs on v_mfma_f32_16x16x32_bf16 (lane l
// holds A[l%16][8(l/16)+e] and B[8(l/16)+e][l%16], e = 0..7; D as above)
// with each fp32 operand split into two bf16 values, x = hi + lo +
// O(2^-17 |x|) with hi = bf16(x) and lo = bf16(x - hi); a product is
// hi*hi + hi*lo + lo*hi in fp32 accumulation, about 2^-16 relative error
// per term where one fp32 product has 2^-24, at a sixteenth of the fp32
// MFMA's cycles per term.  Tiles in memory are stored split: a row of n
// floats holds n bf16 hi values, then n bf16 lo values (q and k from the
// conv kernel, W and P from chunk_prep).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
constexpr int kC = 64;  // tokens per chunk
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int slot_ok(int s, int n) { return (s > 0 && s < n) ? s : 0; }

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split1(float x, uint16_t& hi, uint16_t& lo) {
  const __bf16 h = (__bf16)x;
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, (__bf16)(x - (float)h));
}

// An MFMA operand of eight split values.
struct Frag {
  u32x4 hi, lo;
};
__device__ __forceinline__ Frag split8(v4f a, v4f b) {
  const Split2 s0 = split2(a.x, a.y), s1 = split2(a.z, a.w);
  const Split2 s2 = split2(b.x, b.y), s3 = split2(b.z, b.w);
  return {u32x4{s0.hi, s1.hi, s2.hi, s3.hi}, u32x4{s0.lo, s1.lo, s2.lo, s3.lo}};
}
__device__ __forceinline__ v4f mfma_bf(u32x4 a, u32x4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                  __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}
// c + a b with a, b split: the three terms above 2^-16, small ones first
__device__ __forceinline__ v4f mfma3(const Frag& a, const Frag& b, v4f c) {
  c = mfma_bf(a.lo, b.hi, c);
  c = mfma_bf(a.hi, b.lo, c);
  return mfma_bf(a.hi, b.hi, c);
}

// Split tiles in LDS: row r holds COLS bf16 hi values then COLS lo values
// (4 COLS bytes, as many as COLS floats); its 16-byte chunk ch sits at chunk
// ch ^ sig(r), sig a permutation of the row's low four bits.  Row operands
// (A, or B read as rows of B^T: 16 consecutive rows, one chunk) then hit
// every bank once, and so do column operands (B[s][k] read with
// ds_read_b64_tr_b16: 16 lanes take rows s..s+3 at one 32-byte block, the
// next 16 lanes rows s+8..s+11), since sig(r) >> 1 differs on all eight.
__device__ __forceinline__ int sig(int r) {
  return ((r & 3) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1);
}
template <int COLS>
__device__ __forceinline__ int sp_off(int r, int x) {  // x: bf16 index in the row, x % 4 == 0
  return r * 4 * COLS + (((x >> 3) ^ sig(r)) << 4) + ((x & 7) << 1);
}
// A operand A[t][k] (or B[k][t] = T[t][k]) for t = r0 + l%16, k = 32 ks + 8 (l/16) + e
template <int COLS>
__device__ __forceinline__ Frag frag_rows(const char* t, int r, int ks, int lk) {
  Frag f;
  f.hi = *reinterpret_cast<const u32x4*>(t + sp_off<COLS>(r, 32 * ks + 8 * lk));
  f.lo = *reinterpret_cast<const u32x4*>(t + sp_off<COLS>(r, COLS + 32 * ks + 8 * lk));
  return f;
}
// B operand B[s][k] = T[s][k] for s = 32 ks + 8 (l/16) + e, k = 16 mt + l%16:
// lane m of each 16 points at row 8 (l/16) + m/4 (then 4 rows on), columns
// 4 (m%4) .. +3 of the tile; the transposed read hands lane l element l%4 of
// the pieces of lanes 4e + l/4, which is T[.. + e][16 mt + l%16].
__device__ __forceinline__ u32x2 tr_read(const char* t, int off) {
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + off));
  return __builtin_bit_cast(u32x2, v);
}
template <int COLS>
__device__ __forceinline__ Frag frag_cols(const char* t, int ks, int mt, int li, int lk) {
  const int r = 32 * ks + 8 * lk + (li >> 2), x = 16 * mt + 4 * (li & 3);
  const u32x2 h0 = tr_read(t, sp_off<COLS>(r, x)), h1 = tr_read(t, sp_off<COLS>(r + 4, x));
  const u32x2 l0 = tr_read(t, sp_off<COLS>(r, COLS + x));
  const u32x2 l1 = tr_read(t, sp_off<COLS>(r + 4, COLS + x));
  return {u32x4{h0.x, h0.y, h1.x, h1.y}, u32x4{l0.x, l0.y, l1.x, l1.y}};
}
// The S0 tile is read only as rows (16 rows at one chunk) and written by
// lane pairs, one word per lane, four rows 4 apart per instruction; its
// chunk c of row r sits at c ^ (r mod 16), lo chunks also flipping bit 1,
// so the four rows' hi and lo chunk pairs fall on eight different bank
// groups.
template <int COLS>
__device__ __forceinline__ int s0_off(int r, int x) {
  const int flip = x >= COLS ? 2 : 0;
  return r * 4 * COLS + (((x >> 3) ^ (r & 15) ^ flip) << 4) + ((x & 7) << 1);
}
template <int COLS>
__device__ __forceinline__ Frag frag_rows_s0(const char* t, int r, int ks, int lk) {
  Frag f;
  f.hi = *reinterpret_cast<const u32x4*>(t + s0_off<COLS>(r, 32 * ks + 8 * lk));
  f.lo = *reinterpret_cast<const u32x4*>(t + s0_off<COLS>(r, COLS + 32 * ks + 8 * lk));
  return f;
}
// The scaled T tiles of chunk_prep are read only as rows and written four
// consecutive rows per instruction, 8 bytes per lane: chunk c of row r sits
// at c ^ rev4(r mod 16), so rows r and r+1 (bit 0 -> chunk bit 3) land on
// different halves of the banks.
__device__ __forceinline__ int rev4(int r) {
  return ((r & 1) << 3) | ((r & 2) << 1) | ((r & 4) >> 1) | ((r & 8) >> 3);
}
template <int COLS>
__device__ __forceinline__ int t_off(int r, int x) {
  return r * 4 * COLS + (((x >> 3) ^ rev4(r)) << 4) + ((x & 7) << 1);
}
template <int COLS>
__device__ __forceinline__ Frag frag_rows_t(const char* t, int r, int ks, int lk) {
  Frag f;
  f.hi = *reinterpret_cast<const u32x4*>(t + t_off<COLS>(r, 32 * ks + 8 * lk));
  f.lo = *reinterpret_cast<const u32x4*>(t + t_off<COLS>(r, COLS + 32 * ks + 8 * lk));
  return f;
}
// Four consecutive values (columns c..c+3 of row r) into a split tile.
template <int COLS>
__device__ __forceinline__ void store_split4(char* t, int r, int c, v4f v) {
  const Split2 a = split2(v.x, v.y), b = split2(v.z, v.w);
  *reinterpret_cast<u32x2*>(t + sp_off<COLS>(r, c)) = u32x2{a.hi, b.hi};
  *reinterpret_cast<u32x2*>(t + sp_off<COLS>(r, COLS + c)) = u32x2{a.lo, b.lo};
}

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
// loaded too and written as zeros: every array read this way holds a chunk
// of padding rows past its last token, so the loads stay inside it.  No
// load sits behind a branch and no value is tested before it is stored
// (vector loads complete in order, so either would wait for every load
// issued before it).
template <int ROWS, int COLS, int NT = 256>
struct Tile4 {
  static_assert((ROWS * COLS / 4) % NT == 0 && (NT * 4) % COLS == 0, "tile shape");
  static constexpr int kPer = ROWS * COLS / 4 / NT;  // float4 per thread
  static constexpr int kRowStep = NT * 4 / COLS;     // rows between them
  v4f v[kPer];
  // base: row 0, column 0 of the tile (uniform); pitch: floats per row
  __device__ __forceinline__ void load(const float* base, int pitch) {
    const int r0 = (int)threadIdx.x * 4 / COLS, c0 = (int)threadIdx.x * 4 % COLS;
    const unsigned off = (unsigned)(r0 * pitch + c0);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const float* bi = base + (size_t)(i * kRowStep) * pitch;
      v[i] = *reinterpret_cast<const v4f*>(bi + off);
    }
  }
  __device__ __forceinline__ v4f row_or_zero(int i, int r, int nrow) const {
    return r < nrow ? v[i] : v4f{0.f, 0.f, 0.f, 0.f};
  }
  // tile already split (a row of COLS floats' bytes holds COLS hi then COLS
  // lo bf16 values), copied as it is into a split tile of row length COLS
  __device__ __forceinline__ void store_raw_split(char* lds, int nrow) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = (i * NT + (int)threadIdx.x) * 4;
      const int r = e / COLS, c = e - r * COLS;
      *reinterpret_cast<v4f*>(lds + sp_off<COLS>(r, 2 * c)) = row_or_zero(i, r, nrow);
    }
  }
  // the same with every row kept (rows past the tokens only reach results
  // that are dropped)
  __device__ __forceinline__ void store_raw_split(char* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = (i * NT + (int)threadIdx.x) * 4;
      const int r = e / COLS, c = e - r * COLS;
      *reinterpret_cast<v4f*>(lds + sp_off<COLS>(r, 2 * c)) = v[i];
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

// A's ten lower 16x16 blocks (the rest is zero), block (bi, bj) at
// bi (bi + 1) / 2 + bj; inside a block, row r at slot (r & 12) | ((r + r/4) & 3)
// and float4 group g at g ^ (r/4 mod 4).  Scalar writes of an MFMA result
// (rows 4kk + i, 16 columns) and float4 reads of 16 rows then hit every bank
// once.  Offsets in floats; s % 4 == 0 for float4 reads.
__device__ __forceinline__ int as_off(int t, int s) {
  const int bi = t >> 4, bj = s >> 4, r = t & 15, c = s & 15;
  const int slot = (r & 12) | ((r + (r >> 2)) & 3);
  return (bi * (bi + 1) / 2 + bj) * 256 + slot * 16 + ((((c >> 2) ^ (r >> 2)) & 3) << 2) + (c & 3);
}

// Shared memory of chunk_prep_kernel (bytes), sized for two workgroups per
// CU.  The second region holds Q for the Gram products, then T and the
// per-wave scratch, then T diag(b e^G) and T diag(b); V never enters LDS
// (each wave loads its own operands of U~ = T diag(b) V).
template <int DK>
struct PrepLds {
  static constexpr int MP = 20;                     // pitch of the 16x16 scratch
  static constexpr int ks = 0;                      // [kC] split rows of K
  static constexpr int r2 = ks + kC * DK * 4;       // second region:
  static constexpr int qs = r2;                     //   [kC] split rows of Q
  static constexpr int tt = r2;                     //   [kC][kC] fp32 T
  static constexpr int mw = tt + kC * kC * 4;       //   [4][16][MP] fp32 scratch
  static constexpr int tg = r2;                     //   [kC] split rows of T diag(b e^G)
  static constexpr int tb = tg + kC * kC * 4;       //   [kC] split rows of T diag(b)
  static constexpr int r2_bytes = 2 * kC * kC * 4 > kC * DK * 4 ? 2 * kC * kC * 4 : kC * DK * 4;
  static_assert(mw + 4 * 16 * MP * 4 <= r2 + r2_bytes, "scratch fits");
  static constexpr int as = r2 + r2_bytes;          // A, ten 16x16 fp32 blocks
  static constexpr int gs = as + 10 * 256 * 4;      // [kC] cumulative log-decay
  static constexpr int bs = gs + kC * 4;            // [kC] beta
  static constexpr int bg = bs + kC * 4;            // [kC] beta e^G
  static constexpr int total = bg + kC * 4;
  static_assert(total <= 80 * 1024, "two workgroups per CU");
};

template <int DK, int DV>
__global__ void __launch_bounds__(256)
chunk_prep_kernel(PrefillArgs p, const float* __restrict__ y, const float* __restrict__ glog,
                  const float* __restrict__ gbeta, ChunkWs ws) {
  static_assert(DK == DV && DK % 64 == 0, "dk == dv, multiple of 64");
  extern __shared__ __align__(16) char smb[];
  using Lay = PrepLds<DK>;
  constexpr int MP = Lay::MP;
  char* Ks = smb + Lay::ks;
  char* Qs = smb + Lay::qs;
  char* TG = smb + Lay::tg;
  char* TB = smb + Lay::tb;
  float* As = reinterpret_cast<float*>(smb + Lay::as);
  float* Tt = reinterpret_cast<float*>(smb + Lay::tt);
  float* Gs = reinterpret_cast<float*>(smb + Lay::gs);
  float* Bs = reinterpret_cast<float*>(smb + Lay::bs);
  float* BG = reinterpret_cast<float*>(smb + Lay::bg);

  const int row = p.unit_map[2 * blockIdx.y];
  if (row < 0) return;
  const int c = p.unit_map[2 * blockIdx.y + 1], h = head_of(blockIdx.x, p.Hv);
  const PRow pr = prow(p, row);
  const int t0 = c * kC;
  if (t0 >= pr.T) return;
  const int nt = min(kC, pr.T - t0);
  const int jb = pr.j0 + t0;
  const int ih = h / p.G, Hk = p.Hk, Hv = p.Hv, C = p.C;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
  const int li = lane & 15, lk = lane >> 4;
  float* Mw = reinterpret_cast<float*>(smb + Lay::mw) + wv * 16 * MP;

  // 1. keys and queries of the chunk gathered in one batch, and this wave's
  //    operands of U~ = T diag(b) V: V[s][16 (NW w + q) + l%16] for the
  //    lane's tokens s = 32 ks + 8 (l/16) + e (rows past the chunk's tokens
  //    are padding, read and dropped where used)
  constexpr int NW = DK / 64;
  float vr[2][NW][8];
  float g_in = 0.f, b_in = 0.f;  // log-decay and beta of token tid (tid < kC)
  if (tid < kC) {
    const size_t gi = (size_t)(jb + min(tid, nt - 1)) * Hv + h;
    g_in = glog[gi];
    b_in = gbeta[gi];
  }
  {
    Tile4<kC, DK> tk, tq;
    const float* yb = y + (size_t)jb * C;
    tk.load(yb + Hk * DK + ih * DK, C);
    tq.load(yb + ih * DK, C);
    const float* vb = yb + 2 * Hk * DK + h * DV + 16 * NW * wv + li;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int q = 0; q < NW; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) vr[ks][q][e] = vb[(size_t)(32 * ks + 8 * lk + e) * C + 16 * q];
    __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first use
    tk.store_raw_split(Ks, nt);  // K's padding rows would reach W through 0 * x
    tq.store_raw_split(Qs);
  }
  if (tid < kC) {
    Gs[tid] = tid < nt ? g_in : 0.f;
    Bs[tid] = tid < nt ? b_in : 0.f;
  }
  // P is zero right of its diagonal blocks: 16-byte piece g of a split row
  // holds columns 8 (g mod 8) .. +7 (hi for g < 8, lo after)
  {
    float* Pg = ws.P + ((size_t)jb * Hv + h) * kC;
#pragma unroll
    for (int i = 0; i < kC * kC / 4 / 256; ++i) {
      const int e = i * 256 + tid, t = e >> 4, g = e & 15;
      if (((g & 7) >> 1) > (t >> 4) && t < nt)
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
  //    Q K^T; waves 0 and 1 the even tiles in row order, 2 and 3 the odd),
  //    on split operands (B[k][s] = K[s][k] read as rows of K).
  {
    const bool qk = (wv & 1) != 0;
    const char* Asrc = qk ? Qs : Ks;
#pragma unroll
    for (int it = 0; it < 5; ++it) {
      const int x = 2 * it + (wv >> 1);
      const int ti = x < 1 ? 0 : (x < 3 ? 1 : (x < 6 ? 2 : 3));
      const int tj = x - ti * (ti + 1) / 2;
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < DK / 32; ++k)
        acc = mfma3(frag_rows<DK>(Asrc, 16 * ti + li, k, lk), frag_rows<DK>(Ks, 16 * tj + li, k, lk),
                    acc);
      // G and beta of the tile's rows and column read together (no read
      // waits behind a test); decay e^{G_t - G_s} for s < t, 1 otherwise
      const int s = 16 * tj + li, t0 = 16 * ti + 4 * lk;
      const float gs = Gs[s];
      float gt[4], bt[4], v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gt[r] = Gs[t0 + r];
        bt[r] = Bs[t0 + r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + r;
        const float dec = __builtin_amdgcn_exp2f((s < t ? gt[r] - gs : 0.f) * kLog2e);
        v[r] = qk ? (s <= t ? dec * acc[r] : 0.f) : (s < t ? bt[r] * dec * acc[r] : 0.f);
      }
      if (!qk) {
#pragma unroll
        for (int r = 0; r < 4; ++r) As[as_off(t0 + r, s)] = v[r];
      } else {
        // P split, written as words of two columns: lanes 2m and 2m+1 swap
        // two values, then the even lane writes rows 0 and 1 of its four,
        // the odd lane rows 2 and 3
        const bool odd = (li & 1) != 0;
        const float x0 = dpp_mov<0xB1>(odd ? v[0] : v[2]);
        const float x1 = dpp_mov<0xB1>(odd ? v[1] : v[3]);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float xk = k ? x1 : x0;
          const Split2 w = split2(odd ? xk : v[k], odd ? v[k + 2] : xk);
          const int t = t0 + k + (odd ? 2 : 0);
          if (t < nt) {
            unsigned* prow = reinterpret_cast<unsigned*>(ws.P + ((size_t)(jb + t) * Hv + h) * kC);
            prow[(s & ~1) >> 1] = w.hi;
            prow[(kC + (s & ~1)) >> 1] = w.lo;
          }
        }
      }
    }
  }
  lds_barrier();
  // 4. T = (I + A)^{-1} in 16x16 blocks.  Wave w inverts diagonal block w by
  //    forward substitution (lane j of each 16 solves column j) and clears
  //    T's blocks right of it; T replaces the queries.
  {
    const int b0 = 16 * wv;
    float X[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float x0 = (t == li) ? 1.f : 0.f, x1 = 0.f;
#pragma unroll
      for (int g = 0; g < (t + 3) / 4; ++g) {
        const v4f a = *reinterpret_cast<const v4f*>(As + as_off(b0 + t, b0 + 4 * g));
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
  lds_barrier();
  //    Blocks below the diagonal, one diagonal level at a time:
  //    T_ij = -T_ii M with M = sum_{k=j}^{i-1} A_ik T_kj (wave w: j = w).
  for (int lv = 1; lv < 4; ++lv) {
    const bool act = wv < 4 - lv;
    const int i = wv + lv, j = wv;
    if (act) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      for (int k = j; k < i; ++k) {
        const v4f a = *reinterpret_cast<const v4f*>(As + as_off(16 * i + li, 16 * k + 4 * lk));
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
  // 5. W = T diag(b e^G) K and U~ = T diag(b) V on split operands: the
  //    scaled T as rows, K and V as columns.  Wave w computes column tiles
  //    NW*w .. NW*w+NW-1 for every token tile; tokens 32..63 feed token
  //    tiles 2 and 3 only (T is lower triangular).
  //    The scaled T overwrites T: every thread reads its part first.
  {
    constexpr int kPer = kC * kC / 4 / 256;
    v4f tr4[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = (i * 256 + tid) * 4, r = e / kC, cc = e - r * kC;
      tr4[i] = ld4<kC>(Tt, r, cc);
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = (i * 256 + tid) * 4, r = e / kC, cc = e - r * kC;
      const v4f g4 = tr4[i] * *reinterpret_cast<const v4f*>(BG + cc);
      const v4f b4 = tr4[i] * *reinterpret_cast<const v4f*>(Bs + cc);
      const Split2 g0 = split2(g4.x, g4.y), g1 = split2(g4.z, g4.w);
      const Split2 b0 = split2(b4.x, b4.y), b1 = split2(b4.z, b4.w);
      *reinterpret_cast<u32x2*>(TG + t_off<kC>(r, cc)) = u32x2{g0.hi, g1.hi};
      *reinterpret_cast<u32x2*>(TG + t_off<kC>(r, kC + cc)) = u32x2{g0.lo, g1.lo};
      *reinterpret_cast<u32x2*>(TB + t_off<kC>(r, cc)) = u32x2{b0.hi, b1.hi};
      *reinterpret_cast<u32x2*>(TB + t_off<kC>(r, kC + cc)) = u32x2{b0.lo, b1.lo};
    }
  }
  lds_barrier();
  {
    v4f aw[4][NW], au[4][NW];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        aw[ti][q] = v4f{0.f, 0.f, 0.f, 0.f};
        au[ti][q] = v4f{0.f, 0.f, 0.f, 0.f};
      }
    Frag kb[2][NW], vb[2][NW];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        kb[ks][q] = frag_cols<DK>(Ks, ks, NW * wv + q, li, lk);
        v4f v0, v1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v0[e] = 32 * ks + 8 * lk + e < nt ? vr[ks][q][e] : 0.f;
          v1[e] = 32 * ks + 8 * lk + 4 + e < nt ? vr[ks][q][4 + e] : 0.f;
        }
        vb[ks][q] = split8(v0, v1);
      }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks == 1 && ti < 2) continue;
        const Frag ag = frag_rows_t<kC>(TG, 16 * ti + li, ks, lk);
        const Frag ab = frag_rows_t<kC>(TB, 16 * ti + li, ks, lk);
#pragma unroll
        for (int q = 0; q < NW; ++q) {
          aw[ti][q] = mfma3(ag, kb[ks][q], aw[ti][q]);
          au[ti][q] = mfma3(ab, vb[ks][q], au[ti][q]);
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
            const size_t o = ((size_t)(jb + t) * Hv + h) * DK;
            const int col = 16 * (NW * wv + q) + li;
            uint16_t hi, lo;
            split1(aw[ti][q][r], hi, lo);
            uint16_t* wrow = reinterpret_cast<uint16_t*>(ws.W + o);
            wrow[col] = hi;
            wrow[DK + col] = lo;
            ws.U[o + col] = au[ti][q][r];
          }
        }
      }
  }
  if (tid < nt) ws.G[(size_t)(jb + tid) * Hv + h] = Gs[tid];
}

// Shared memory of chunk_state_kernel (bytes); RB state rows per workgroup.
template <int DK, int RB>
struct StateLds {
  static constexpr int UP = RB + 4;                   // pitch of the U~ block (floats)
  static constexpr int wl = 0;                        // [kC] split rows of W (row operand)
  static constexpr int ql = wl + kC * DK * 4;         // [kC] split rows of Q (row operand)
  static constexpr int kl = ql + kC * DK * 4;         // [kC] split rows of K (column operand)
  static constexpr int pl = kl + kC * DK * 4;         // [kC] split rows of P (row operand)
  static constexpr int ul = pl + kC * kC * 4;         // [kC][UP] fp32 U~ block (plain)
  static constexpr int ss = ul + kC * UP * 4;         // [RB] split rows of S0
  static constexpr int ut = ss + RB * DK * 4;         // [RB] split rows of U^T
  static constexpr int uf = ut + RB * kC * 4;         // [RB] split rows of U^T diag(F)
  static constexpr int gc = uf + RB * kC * 4;         // [kC] G
  static constexpr int total = gc + kC * 4;
};

constexpr int kStateThreads = 512;  // 8 waves, two per SIMD
constexpr int kStateRows = 32;      // state rows per workgroup

// Wave w works on token tile tt = w % 4 and state-row tile jt = w / 4 for
// U and the outputs, and on state tiles (jt, TPW*tt + q) for the update.
// Every product contracts over 32-wide steps: k (W S0^T, Q S0^T) or tokens
// (P U, U^T diag(F) K).
template <int DK, int DV>
__global__ void __launch_bounds__(kStateThreads)
chunk_state_kernel(PrefillArgs p, const float* __restrict__ y, ChunkWs ws) {
  static_assert(DK == DV && DK % 64 == 0, "dk == dv, multiple of 64");
  constexpr int NT = kStateThreads, RB = kStateRows;
  extern __shared__ __align__(16) char smb[];
  using Lay = StateLds<DK, RB>;
  constexpr int UP = Lay::UP;
  constexpr int KS = DK / 32;   // k-steps
  constexpr int TPW = DK / 64;  // state column tiles per wave
  char* Wl = smb + Lay::wl;
  char* Ql = smb + Lay::ql;
  char* Kl = smb + Lay::kl;
  char* Pl = smb + Lay::pl;
  float* Ul = reinterpret_cast<float*>(smb + Lay::ul);
  char* Ss = smb + Lay::ss;
  char* UTs = smb + Lay::ut;
  char* UFs = smb + Lay::uf;
  float* Gc = reinterpret_cast<float*>(smb + Lay::gc);

  const int Hv = p.Hv, Hk = p.Hk, C = p.C;
  const int row = blockIdx.x / Hv, h = head_of(blockIdx.x - row * Hv, Hv);
  const int blk = blockIdx.y;  // state rows RB*blk .. RB*blk+RB-1
  const PRow pr = prow(p, row);
  if (pr.T <= 0) return;
  const int ih = h / p.G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
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
  // Operands of chunk c+1 are gathered while chunk c is computed; W, P, Q
  // and K arrive split.
  Tile4<kC, DK, NT> tw, tq, tk;
  Tile4<kC, kC, NT> tp;
  Tile4<kC, RB, NT> tu;
  float tg;     // G of token lane % 64
  int tx[4];    // token_indx of this lane's output tokens (taken and tested where used)
  // Without token_indx the loads below read G's words instead (any readable
  // address: the value is dropped), so that no load sits behind a branch
  // and the waits for earlier loads stay exact.
  const int* tix = p.tix ? p.tix : reinterpret_cast<const int*>(ws.G);
  // The gather comes in four parts, spread over the phases of the previous
  // chunk (W during (a), Q and K during (b), the rest during (c)): the
  // workgroup's 120 KiB pass through the CU's vector memory path at a fixed
  // rate, and a wave whose loads back up there stalls in issue, so loads
  // issued all at once would hold every wave for that long.
  auto gather_w = [&](int c) {
    const int jb = pr.j0 + c * kC;
    tw.load(ws.W + ((size_t)jb * Hv + h) * DK, Hv * DK);
  };
  auto gather_q = [&](int c) { tq.load(y + (size_t)(pr.j0 + c * kC) * C + ih * DK, C); };
  auto gather_k = [&](int c) { tk.load(y + (size_t)(pr.j0 + c * kC) * C + Hk * DK + ih * DK, C); };
  auto gather_rest = [&](int c) {
    const int jb = pr.j0 + c * kC;
    const int nt = min(kC, pr.T - c * kC);
    tp.load(ws.P + ((size_t)jb * Hv + h) * kC, Hv * kC);
    tu.load(ws.U + ((size_t)jb * Hv + h) * DV + RB * blk, Hv * DV);
    tg = ws.G[(size_t)(jb + min(lane, nt - 1)) * Hv + h];
#pragma unroll
    for (int r = 0; r < 4; ++r) tx[r] = tix[jb + min(16 * tt + 4 * lk + r, nt - 1)];
  };
  gather_w(0);
  gather_q(0);
  gather_k(0);
  gather_rest(0);
  for (int c = 0; c < nch; ++c) {
    const int nt = min(kC, pr.T - c * kC);
    const int cn = c + 1 < nch ? c + 1 : c;  // the last chunk gathers itself again
    // Rows past the chunk's tokens reach only dropped results (U and the
    // outputs are tested per token), except through K: 0 * x there would
    // carry a NaN of padding rows into the state.
    tw.store_raw_split(Wl);
    tq.store_raw_split(Ql);
    if (nt < kC)  // only a row's last chunk has rows past its tokens
      tk.store_raw_split(Kl, nt);
    else
      tk.store_raw_split(Kl);
    tp.store_raw_split(Pl);
    tu.template store_pitched<UP>(Ul);
    if (tid < kC) Gc[tid] = tg * kLog2e;  // G in log2 units
    int orow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tt + 4 * lk + r;
      const int gr = p.tix ? tx[r] : pr.j0 + c * kC + min(t, nt - 1);
      orow[r] = (t < nt && gr >= 0 && gr < p.num_actual_tokens) ? gr : -1;
    }
    // S0 split: lanes 2m and 2m+1 hold columns c and c+1 of rows 4 lk + r.
    // They swap two values, then the even lane splits the column pairs of
    // rows 0 and 1 of the four, the odd lane those of rows 2 and 3, and each
    // writes the pairs' hi and lo words.
    {
      const bool odd = (li & 1) != 0;
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const v4f s = St[q];
        const float x0 = dpp_mov<0xB1>(odd ? s[0] : s[2]);  // quad_perm 1,0,3,2
        const float x1 = dpp_mov<0xB1>(odd ? s[1] : s[3]);
        const int col = 16 * (TPW * tt + q) + (li & ~1);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float xk = k ? x1 : x0;
          const Split2 w = split2(odd ? xk : s[k], odd ? s[k + 2] : xk);
          const int row = 16 * jt + 4 * lk + k + (odd ? 2 : 0);
          *reinterpret_cast<unsigned*>(Ss + s0_off<DK>(row, col)) = w.hi;
          *reinterpret_cast<unsigned*>(Ss + s0_off<DK>(row, DK + col)) = w.lo;
        }
      }
    }
    lds_barrier();

    const float gC = Gc[kC - 1];
    // B operand of the S0^T products: S0[j][k], j = 16 jt + li, k in the
    // lane's 8-runs of each k-step
    Frag sb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sb[ks] = frag_rows_s0<DK>(Ss, 16 * jt + li, ks, lk);
    // (a) U = U~ - W S0^T on (token tile tt, row tile jt), kept split as
    //     U^T (B operand of P U) and U^T diag(F), F_t = e^{G_C - G_t} (A
    //     operand of the update)
    {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks == KS / 2) {
          __builtin_amdgcn_sched_barrier(0);
          gather_w(cn);
          __builtin_amdgcn_sched_barrier(0);
        }
        acc = mfma3(frag_rows<DK>(Wl, 16 * tt + li, ks, lk), sb[ks], acc);
      }
      const int t0 = 16 * tt + 4 * lk;
      // every row of the U~ block is readable (padding rows included), so
      // the reads are issued together and the tokens tested afterwards
      float ul[4], gt[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ul[r] = Ul[(t0 + r) * UP + 16 * jt + li];
        gt[r] = Gc[t0 + r];
      }
      v4f u, f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u[r] = t0 + r < nt ? ul[r] - acc[r] : 0.f;
        f[r] = __builtin_amdgcn_exp2f(gC - gt[r]);
      }
      store_split4<kC>(UTs, 16 * jt + li, t0, u);
      store_split4<kC>(UFs, 16 * jt + li, t0, u * f);
    }
    lds_barrier();

    // (b) outputs on (tt, jt): e^{G_t} (Q S0^T)[t] + (P U)[t]; P is zero
    //     right of the diagonal block, so tokens 32..63 matter from tt = 2 on
    {
      float eg[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) eg[r] = __builtin_amdgcn_exp2f(Gc[16 * tt + 4 * lk + r]);
      v4f aq = {0.f, 0.f, 0.f, 0.f}, ap = {0.f, 0.f, 0.f, 0.f};
      __builtin_amdgcn_sched_barrier(0);
      gather_q(cn);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks == KS / 2) {
          __builtin_amdgcn_sched_barrier(0);
          gather_k(cn);
          __builtin_amdgcn_sched_barrier(0);
        }
        aq = mfma3(frag_rows<DK>(Ql, 16 * tt + li, ks, lk), sb[ks], aq);
      }
      ap = mfma3(frag_rows<kC>(Pl, 16 * tt + li, 0, lk), frag_rows<kC>(UTs, 16 * jt + li, 0, lk), ap);
      if (tt >= 2)
        ap = mfma3(frag_rows<kC>(Pl, 16 * tt + li, 1, lk), frag_rows<kC>(UTs, 16 * jt + li, 1, lk), ap);
      // bf16 round to nearest even (the hardware conversion)
      uint16_t* ob = p.out + ((size_t)h * DV + RB * blk + 16 * jt + li);
      const unsigned ostride = (unsigned)(Hv * DV);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint16_t v = __builtin_bit_cast(uint16_t, (__bf16)fmaf(eg[r], aq[r], ap[r]));
        if (orow[r] >= 0) ob[(size_t)(unsigned)orow[r] * ostride] = v;
      }
    }

    // (c) S = e^{G_C} S0 + U^T diag(e^{G_C - G_t}) K on this wave's tiles
    __builtin_amdgcn_sched_barrier(0);
    gather_rest(cn);
    __builtin_amdgcn_sched_barrier(0);
    {
      const Frag ua[2] = {frag_rows<kC>(UFs, 16 * jt + li, 0, lk), frag_rows<kC>(UFs, 16 * jt + li, 1, lk)};
      const float eC = __builtin_amdgcn_exp2f(gC);
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int mt = TPW * tt + q;
        v4f acc = St[q] * eC;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc = mfma3(ua[ks], frag_cols<DK>(Kl, ks, mt, li, lk), acc);
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

template <int DK, int DV>
static hipError_t launch_chunked_typed(const PrefillArgs& a, const float* y, const float* glog,
                                       const float* gbeta, const ChunkWs& ws, hipStream_t s) {
  const size_t l1 = PrepLds<DK>::total;
  const size_t l2 = StateLds<DK, kStateRows>::total;
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

hipError_t prepare_chunked(int dk, int dv) {
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 64:
    case 128: {
      const size_t l1 = dk == 64 ? PrepLds<64>::total : PrepLds<128>::total;
      const size_t l2 = dk == 64 ? StateLds<64, kStateRows>::total : StateLds<128, kStateRows>::total;
      const void* prep = dk == 64 ? reinterpret_cast<const void*>(chunk_prep_kernel<64, 64>)
                                  : reinterpret_cast<const void*>(chunk_prep_kernel<128, 128>);
      const void* state = dk == 64 ? reinterpret_cast<const void*>(chunk_state_kernel<64, 64>)
                                   : reinterpret_cast<const void*>(chunk_state_kernel<128, 128>);
      hipError_t e = ensure_dynamic_lds(prep, l1);
      return e != hipSuccess ? e : ensure_dynamic_lds(state, l2);
    }
    default: return hipErrorInvalidValue;
  }
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
