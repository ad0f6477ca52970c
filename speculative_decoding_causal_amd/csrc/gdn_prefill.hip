// Non-spec prefill rows (rows of any length).
//
// Launches on the caller's stream:
//   0. prefill_map: one workgroup lists the 64-token units of the rows, row
//      after row, so the kernels below launch one workgroup per unit that
//      exists rather than per (row, longest possible row) pair.
//   1. conv_prefill: one thread per (4 channels, 16 tokens of a row)
//      slides the width-W window along the row and writes the fp32 conv
//      output to the workspace at the token's non-spec stream index, q and
//      k L2-normalised (q scaled) by a reduction over the lanes of a head
//      and, for the chunked form, split into bf16 hi and lo values;
//      the workgroups of a unit also evaluate the gates of every v-head at
//      the token's global row (log-decay and beta).  The thread of the
//      row's first tokens is the only one that reads the ring history and
//      it alone rolls the ring by T afterwards, so reads of the pre-state
//      precede the writes.
//   2. for head dims below 64, kq_prefill: k.q per (token, k-head).
//   3. the chunked WY/UT recurrence on MFMA (gdn_chunk.hip) for head dims 64
//      and 128; for smaller heads, delta_prefill: one workgroup per (row,
//      v-head, block of state rows) carries its rows in VGPRs through the
//      row, the per-token operands staged in LDS 32 tokens at a time.  The
//      final state is stored to the row's slot.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kSeg = 64;    // tokens per unit of the unit map
constexpr int kChunk = 32;  // tokens staged per LDS refill in the recurrence

typedef float v4f __attribute__((ext_vector_type(4)));

struct WsLayout {
  size_t y, kq, ga, gb, W, U, P, G, map, total;
  int units;
};

// Units of 64 tokens the rows can hold: each row adds at most one partial unit.
int unit_capacity(int stream_tokens, int rows) {
  return (stream_tokens + kSeg - 1) / kSeg + rows;
}

WsLayout ws_layout(int Hk, int Hv, int dk, int dv, int stream_tokens, int rows) {
  const size_t C = 2ull * Hk * dk + (size_t)Hv * dv;
  const size_t n = stream_tokens > 0 ? (size_t)stream_tokens : 0;
  // Arrays the chunk kernels read a 64-token tile at a time carry 64
  // padding rows, so a row's last tile can be loaded whole.
  const size_t np = n + 64;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WsLayout w;
  size_t o = 0;
  w.y = o;  o += al(np * C * 4);
  w.kq = o; o += al(n * Hk * 4);
  w.ga = o; o += al(n * Hv * 4);
  w.gb = o; o += al(n * Hv * 4);
  w.W = o;  o += al(np * Hv * dk * 4);
  w.U = o;  o += al(np * Hv * dv * 4);
  w.P = o;  o += al(np * Hv * 64 * 4);
  w.G = o;  o += al(np * Hv * 4);
  w.units = unit_capacity(stream_tokens > 0 ? stream_tokens : 0, rows > 0 ? rows : 0);
  w.map = o; o += al((size_t)w.units * 2 * 4);
  w.total = o;
  return w;
}

__device__ __forceinline__ int slot_or_null(int s, int num_slots) {
  return (s > 0 && s < num_slots) ? s : 0;
}

struct PrefillRow {
  int j0, T, slot;
  bool init;
};

__device__ __forceinline__ PrefillRow prefill_row(const PrefillArgs& p, int row) {
  PrefillRow r;
  r.j0 = clampi(p.qsl[row], 0, p.stream_tokens);
  int j1 = clampi(p.qsl[row + 1], r.j0, p.stream_tokens);
  r.T = j1 - r.j0;
  r.slot = slot_or_null(p.cache_idx[row], p.num_slots);
  r.init = (p.his ? p.his[row] != 0 : true) && r.slot > 0;
  return r;
}

__device__ __forceinline__ int global_row(const PrefillArgs& p, int j) {
  int r = p.tix ? p.tix[j] : j;
  return (r >= 0 && r < p.num_actual_tokens) ? r : -1;
}

// The 64-token units of the rows in row order: map[2i] = row, map[2i+1] =
// unit within the row; entries from the last unit up to cap hold row -1.
// One workgroup: rows are taken 1024 at a time, their unit counts scanned,
// then wave w writes the units of rows w, w+16, ... one lane per unit.
constexpr int kMapThreads = 1024;
__global__ void __launch_bounds__(kMapThreads)
prefill_map_kernel(PrefillArgs p, int* __restrict__ map, int cap) {
  __shared__ int start[kMapThreads + 1];
  __shared__ int wsum[kMapThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;
  for (int r0 = 0; r0 < p.num_rows; r0 += kMapThreads) {
    const int r = r0 + tid;
    int n = 0;
    if (r < p.num_rows) n = (prefill_row(p, r).T + kSeg - 1) / kSeg;
    int x = n;  // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int up = __shfl_up(x, o, 64);
      if (lane >= o) x += up;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    if (wv == 0) {
      int w = lane < kMapThreads / 64 ? wsum[lane] : 0;
#pragma unroll
      for (int o = 1; o < kMapThreads / 64; o <<= 1) {
        const int up = __shfl_up(w, o, 64);
        if (lane >= o) w += up;
      }
      if (lane < kMapThreads / 64) wsum[lane] = w;
    }
    __syncthreads();
    const int excl = carry + (wv > 0 ? wsum[wv - 1] : 0) + x - n;
    start[tid] = excl;
    if (tid == kMapThreads - 1) start[kMapThreads] = excl + n;
    __syncthreads();
    const int nr = min(kMapThreads, p.num_rows - r0);
    for (int i = wv; i < nr; i += kMapThreads / 64) {
      const int s0 = start[i], cnt = start[i + 1] - s0;
      for (int u = lane; u < cnt && s0 + u < cap; u += 64) {
        map[2 * (s0 + u)] = r0 + i;
        map[2 * (s0 + u) + 1] = u;
      }
    }
    // Rows whose query_start_loc ranges overlap (values nothing has
    // checked) can list more units than the map holds; those past `cap` are
    // dropped, so the count saturates there instead of overflowing.
    carry = min(start[kMapThreads], cap);
    __syncthreads();
  }
  for (int i = carry + tid; i < cap; i += kMapThreads) {
    map[2 * i] = -1;
    map[2 * i + 1] = 0;
  }
}

// Four consecutive channels per thread: one 8-byte load per token and one
// 16-byte store per output (channel blocks are multiples of 16 in both
// layouts of mixed_qkv, so the four are contiguous in either).
constexpr int kCh = 4;
constexpr int kTokThread = 16;  // tokens per thread: a quarter of a 64-token unit

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(unsigned int u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(unsigned int u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ void unpack4(u32x2 v, bool live, float (&x)[kCh]) {
  x[0] = live ? bf_lo(v.x) : 0.f;
  x[1] = live ? bf_hi(v.x) : 0.f;
  x[2] = live ? bf_lo(v.y) : 0.f;
  x[3] = live ? bf_hi(v.y) : 0.f;
}

// grid (units, C / (kCh * kThreads), 4): thread (x, y, z) convolves channels
// 4 * (y * kThreads + tid) .. +3 over tokens [16 z, 16 z + 16) of its unit.
// q and k leave L2-normalised (q also scaled): the DK/4 lanes holding one
// head's channels reduce the sum of squares per token (heads start at lane
// multiples of DK/4, and q/k/v boundaries fall on head boundaries).  The
// workgroups of a unit also evaluate the gates of its tokens, log-decay ga
// and write strength gb per (token, v-head), the pairs spread over the
// channel blocks.
// Every load goes to an address that exists and unwanted values are dropped
// afterwards (a load behind a branch is waited for where the branch joins):
// slot 0's ring stands in without history, the taps for an empty ring or an
// empty mixed_qkv (they hold C*W >= C values), row 0 for a token outside the
// batch, the segment's last token for positions past it.
// WT > 0 fixes the conv width and ACT >= 0 the activation at compile time
// (the tap and window tests then fold away); WT = 0, ACT = -1 read them from
// the arguments.
template <int DK, int WT, int ACT>
__global__ void __launch_bounds__(kThreads)
conv_prefill_kernel(PrefillArgs p, float* __restrict__ y, float* __restrict__ ga,
                    float* __restrict__ gb) {
  constexpr int LPH = DK / kCh;  // lanes per head
  static_assert(LPH >= 4 && LPH <= 32, "head dim");
  const int C = p.C, L = p.L, W = WT > 0 ? WT : p.W;
  const bool act = ACT >= 0 ? ACT != 0 : p.act != 0;
  const int c = (blockIdx.y * kThreads + threadIdx.x) * kCh;
  // the thread's four channels lie in one block: q (normalised, scaled), k
  // (normalised) or v (as is)
  const bool is_qk = c < 2 * p.Hk * DK;
  const float qscale = c < p.Hk * DK ? p.scale : 1.f;
  // Threads past the last channel stay for the lane-by-lane row gather
  // below (its values are read from lanes 0 .. 34 of every wave) and leave
  // after it; until then they only form addresses, loading nothing.
  const bool chan_live = c < C;
  const int row = p.unit_map[2 * blockIdx.x], seg = p.unit_map[2 * blockIdx.x + 1];
  if (row < 0) return;
  const PrefillRow pr = prefill_row(p, row);
  const int base = seg * kSeg + blockIdx.z * kTokThread;
  if (base >= pr.T) return;
  const int end = min(pr.T, base + kTokThread);
  const int cin = p.qkv_layout ? per_k_head_column(c, p.Hk, p.G, p.dk, p.dv) : c;
  const uint16_t* ring = L > 0 ? p.conv_pool + (size_t)(pr.init ? pr.slot : 0) * L * C + c
                               : p.conv_w + c;
  const uint16_t* xs = p.num_actual_tokens > 0 ? p.qkv : p.conv_w;
  auto in_ptr = [&](int r) -> const u32x2* {
    return reinterpret_cast<const u32x2*>(xs + (size_t)(r >= 0 ? r : 0) * (xs == p.qkv ? C : 0) +
                                          (xs == p.qkv ? cin : c));
  };
  auto ring_col = [&](int col) -> const u32x2* {
    const int cc = L > 0 ? (col < 0 ? 0 : (col > L - 1 ? L - 1 : col)) : 0;
    return reinterpret_cast<const u32x2*>(ring + (size_t)cc * C);
  };

  // Global rows of the positions this thread reads, one per lane in one
  // coalesced load, then made uniform lane by lane: lanes 0..15 the
  // segment's tokens, 16..18 the window before them, 19..34 the inputs the
  // rolled ring takes (row positions T-L .. T-1); every position is clamped
  // into the row.  Then every vector load of the segment in one round:
  // inputs, window, taps, bias, and (for the rolling thread) the roll's
  // sources.
  const bool roller = seg == 0 && blockIdx.z == 0 && pr.slot > 0 && L > 0;
  int rr[kTokThread], hr[kMaxWidth - 1], ir[kMaxStateLen];
  {
    const int lane = threadIdx.x & 63;
    int t;
    if (lane < kTokThread) t = base + lane;
    else if (lane < kTokThread + kMaxWidth - 1) t = base - (W - 1) + (lane - kTokThread);
    else t = pr.T - L + (lane - kTokThread - (kMaxWidth - 1));
    t = t < 0 ? 0 : (t > end - 1 && lane < kTokThread ? end - 1 : (t > pr.T - 1 ? pr.T - 1 : t));
    const int rl = global_row(p, pr.j0 + t);
#pragma unroll
    for (int i = 0; i < kTokThread; ++i) rr[i] = __builtin_amdgcn_readlane(rl, i);
#pragma unroll
    for (int m = 0; m < kMaxWidth - 1; ++m) hr[m] = __builtin_amdgcn_readlane(rl, kTokThread + m);
#pragma unroll
    for (int l = 0; l < kMaxStateLen; ++l)
      ir[l] = __builtin_amdgcn_readlane(rl, kTokThread + kMaxWidth - 1 + l);
  }
  if (!chan_live) return;
  u32x2 xv[kTokThread], hv[kMaxWidth - 1], iv[kMaxWidth - 1];
  uint16_t wr[kMaxWidth][kCh];
#pragma unroll
  for (int i = 0; i < kTokThread; ++i) xv[i] = *in_ptr(rr[i]);
#pragma unroll
  for (int m = 0; m < kMaxWidth - 1; ++m) {
    hv[m] = *ring_col(L + base - (W - 1) + m);
    iv[m] = *in_ptr(hr[m]);
  }
#pragma unroll
  for (int m = 0; m < kMaxWidth; ++m)
#pragma unroll
    for (int e = 0; e < kCh; ++e) wr[m][e] = p.conv_w[(size_t)(c + e) * W + (m < W ? m : W - 1)];
  const u32x2 br = *reinterpret_cast<const u32x2*>((p.conv_b ? p.conv_b : p.conv_w) + c);
  // Gate pairs (token of the segment, v-head): spread over the channel
  // blocks, kGP per thread; their stream rows, A_log and dt_bias join this
  // round, a and b follow once the rows are known.
  constexpr int kGP = 4;
  const int Hv = p.Hv;
  const int live_thr = (C / kCh - (int)blockIdx.y * kThreads) < kThreads
                           ? (C / kCh - (int)blockIdx.y * kThreads) : kThreads;
  const int npairs = kTokThread * Hv;
  const int per_blk = (npairs + gridDim.y - 1) / gridDim.y;
  int gidx[kGP], graw[kGP];
  float gl[kGP], gd[kGP];
#pragma unroll
  for (int k = 0; k < kGP; ++k) {
    const int q = (int)threadIdx.x + k * live_thr;
    const int idx = (int)blockIdx.y * per_blk + q;
    gidx[k] = (q < per_blk && idx < npairs) ? idx : -1;
    const int ic = gidx[k] >= 0 ? gidx[k] : 0;
    const int i = ic / Hv, h = ic - i * Hv;
    const int t = base + i < end ? base + i : end - 1;
    graw[k] = p.tix ? 0 : pr.j0 + t;
    gl[k] = p.A_log[h];
    gd[k] = p.dt_bias[h];
  }
  if (p.tix) {
#pragma unroll
    for (int k = 0; k < kGP; ++k) {
      const int ic = gidx[k] >= 0 ? gidx[k] : 0;
      const int i = ic / Hv;
      const int t = base + i < end ? base + i : end - 1;
      graw[k] = p.tix[pr.j0 + t];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  uint16_t graw_a[kGP], graw_b[kGP];
  {
    const bool rows_ok = p.num_actual_tokens > 0;
    const uint16_t* sa = rows_ok ? p.a : reinterpret_cast<const uint16_t*>(p.A_log);
    const uint16_t* sb = rows_ok ? p.b : sa;
#pragma unroll
    for (int k = 0; k < kGP; ++k) {
      const int ic = gidx[k] >= 0 ? gidx[k] : 0;
      const int h = ic - (ic / Hv) * Hv;
      graw[k] = (graw[k] >= 0 && graw[k] < p.num_actual_tokens) ? graw[k] : -1;
      const size_t gi = rows_ok ? (size_t)(graw[k] >= 0 ? graw[k] : 0) * Hv + h : (size_t)h;
      graw_a[k] = sa[gi];
      graw_b[k] = sb[gi];
    }
  }

  // taps and bias
  float w[kMaxWidth][kCh], wl[kCh], bias[kCh];
#pragma unroll
  for (int m = 0; m < kMaxWidth; ++m)
#pragma unroll
    for (int e = 0; e < kCh; ++e) w[m][e] = m < W ? bf2f(wr[m][e]) : 0.f;
#pragma unroll
  for (int e = 0; e < kCh; ++e) {
    wl[e] = 0.f;
#pragma unroll
    for (int m = 0; m < kMaxWidth; ++m)
      if (m == W - 1) wl[e] = w[m][e];
  }
  unpack4(br, p.conv_b != nullptr, bias);
  // Window before the first token: positions base-(W-1) .. base-1, which are
  // ring columns L + t (zeros without history) for t < 0, inputs otherwise.
  float win[kMaxWidth - 1][kCh];
#pragma unroll
  for (int m = 0; m < kMaxWidth - 1; ++m) {
    const int t = base - (W - 1) + m;
    const bool hist = t < 0;
    const bool live = m < W - 1 && (hist ? (pr.init && L + t >= 0) : hr[m] >= 0);
    unpack4(hist ? hv[m] : iv[m], live, win[m]);
  }
  // the window slides over the inputs
#pragma unroll
  for (int i = 0; i < kTokThread; ++i) {
    const int t = base + i;
    if (t >= end) break;
    float xt[kCh];
    unpack4(xv[i], rr[i] >= 0, xt);
    float o[kCh];
#pragma unroll
    for (int e = 0; e < kCh; ++e) {
      float acc = bias[e];
#pragma unroll
      for (int m = 0; m < kMaxWidth - 1; ++m)
        if (m < W - 1) acc = fmaf(w[m][e], win[m][e], acc);
      acc = fmaf(wl[e], xt[e], acc);
      o[e] = act ? silu(acc) : acc;
    }
    {
      float ss = o[0] * o[0];
      ss = fmaf(o[1], o[1], ss);
      ss = fmaf(o[2], o[2], ss);
      ss = fmaf(o[3], o[3], ss);
      ss = group_sum<(LPH < 16 ? LPH : 16)>(ss);
      if constexpr (LPH == 32) {
        // every lane of a 16-lane row now holds the row's sum; a head is two
        // rows: add the other row's sum (swizzle: lane xor 16 within each 32)
        ss += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, ss),
                                                                   0x401F));
      }
      // hardware reciprocal square root (within 1 ulp); q also takes the
      // scale, with or without the norm
      const float f = is_qk ? (p.l2norm ? __builtin_amdgcn_rsqf(ss + p.eps) : 1.f) * qscale : 1.f;
#pragma unroll
      for (int e = 0; e < kCh; ++e) o[e] *= f;
    }
    float* yrow = y + (size_t)(pr.j0 + t) * C;
    if (DK >= 64 && c < 2 * p.Hk * DK) {
      // q and k of the chunked form leave split: a head's DK floats hold
      // its DK hi then its DK lo bf16 values
      const Split2 s0 = split2(o[0], o[1]), s1 = split2(o[2], o[3]);
      unsigned* hb = reinterpret_cast<unsigned*>(yrow + (c / DK) * DK) + (c % DK) / 2;
      *reinterpret_cast<u32x2*>(hb) = u32x2{s0.hi, s1.hi};
      *reinterpret_cast<u32x2*>(hb + DK / 2) = u32x2{s0.lo, s1.lo};
    } else {
      *reinterpret_cast<float4*>(yrow + c) = make_float4(o[0], o[1], o[2], o[3]);
    }
    // slide the window: drop the oldest sample, append x_t
#pragma unroll
    for (int m = 0; m < kMaxWidth - 2; ++m)
#pragma unroll
      for (int e = 0; e < kCh; ++e)
        if (m < W - 2) win[m][e] = win[m + 1][e];
#pragma unroll
    for (int m = 0; m < kMaxWidth - 1; ++m)
#pragma unroll
      for (int e = 0; e < kCh; ++e)
        if (m == W - 2) win[m][e] = xt[e];
  }
  // Gates of this thread's pairs: log-decay ga and write strength gb.
#pragma unroll
  for (int k = 0; k < kGP; ++k) {
    if (gidx[k] < 0) continue;
    const int i = gidx[k] / Hv, h = gidx[k] - i * Hv;
    if (base + i >= end) continue;
    const float av = graw[k] >= 0 ? bf2f(graw_a[k]) : 0.f;
    const float bv = graw[k] >= 0 ? bf2f(graw_b[k]) : 0.f;
    ga[(size_t)(pr.j0 + base + i) * Hv + h] = gate_log(av, gl[k], gd[k]);
    gb[(size_t)(pr.j0 + base + i) * Hv + h] = 1.f / (1.f + expf(-bv));
  }
  // Pairs beyond kGP per thread (many v-heads on few channel blocks).
  for (int q = (int)threadIdx.x + kGP * live_thr; q < per_blk; q += live_thr) {
    const int idx = (int)blockIdx.y * per_blk + q;
    if (idx >= npairs) break;
    const int i = idx / Hv, h = idx - i * Hv;
    if (base + i >= end) continue;
    const int r = global_row(p, pr.j0 + base + i);
    const float av = r >= 0 ? bf2f(p.a[(size_t)r * Hv + h]) : 0.f;
    const float bv = r >= 0 ? bf2f(p.b[(size_t)r * Hv + h]) : 0.f;
    ga[(size_t)(pr.j0 + base + i) * Hv + h] = gate_log(av, p.A_log[h], p.dt_bias[h]);
    gb[(size_t)(pr.j0 + base + i) * Hv + h] = 1.f / (1.f + expf(-bv));
  }
  // Roll: new column l <- (history ++ inputs)[T + l].  All sources are
  // loaded (in column order; their rows are known since the start) before
  // the first ring store: vector loads complete in order, so the store of
  // column l, which waits for its own source, also follows the read of
  // column l.  Only this thread writes these channels, and only the thread
  // of the row's first tokens reads history.
  if (roller) {
    uint16_t* wring = p.conv_pool + (size_t)pr.slot * L * C + c;
    u32x2 rhv[kMaxStateLen], riv[kMaxStateLen], nv[kMaxStateLen];
#pragma unroll
    for (int l = 0; l < kMaxStateLen; ++l) {
      rhv[l] = *ring_col(pr.T + l);        // position pr.T + l of (history ++ inputs)
      riv[l] = *in_ptr(ir[l]);
    }
#pragma unroll
    for (int l = 0; l < kMaxStateLen; ++l) {
      const bool hist = pr.T + l < L;
      const bool live = hist ? pr.init : ir[l] >= 0;
      nv[l] = live ? (hist ? rhv[l] : riv[l]) : u32x2{0u, 0u};
    }
#pragma unroll
    for (int l = 0; l < kMaxStateLen; ++l)
      if (l < L) *reinterpret_cast<u32x2*>(wring + (size_t)l * C) = nv[l];
  }
}

// k.q per (token, k-head) from the normalised conv output, for the token
// recurrence (head dims below 64).
template <int DK>
__global__ void __launch_bounds__(kThreads)
kq_prefill_kernel(PrefillArgs p, const float* __restrict__ y, float* __restrict__ kq) {
  const int j = blockIdx.x;
  const int lo = clampi(p.qsl[0], 0, p.stream_tokens);
  const int hi = clampi(p.qsl[p.num_rows], lo, p.stream_tokens);
  if (j < lo || j >= hi) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int Hk = p.Hk, C = p.C;
  const float* yj = y + (size_t)j * C;
  for (int i = wv; i < Hk; i += kThreads / 64) {
    float dot = 0.f;
    for (int c = lane; c < DK; c += 64) dot = fmaf(yj[Hk * DK + i * DK + c], yj[i * DK + c], dot);
    dot = wave_sum(dot);
    if (lane == 0) kq[(size_t)j * Hk + i] = dot;
  }
}

template <int DK, int DV>
__global__ void __launch_bounds__(kThreads)
delta_prefill_kernel(PrefillArgs p, const float* __restrict__ y,
                     const float* __restrict__ kqv, const float* __restrict__ gav,
                     const float* __restrict__ gbv) {
  constexpr int LPR = DK / 16;
  constexpr int RPW = 64 / LPR;
  constexpr int RB = (kThreads / 64) * RPW;  // state rows per workgroup
  __shared__ __align__(16) float ks[kChunk][DK];
  __shared__ __align__(16) float qs[kChunk][DK];
  __shared__ float vsh[kChunk][RB];
  __shared__ float obs[kChunk][RB];
  __shared__ float al[kChunk], be[kChunk], kqs[kChunk];
  __shared__ int rows[kChunk];

  const int h = blockIdx.y;
  const int rb0 = blockIdx.x * RB;
  if (rb0 >= DV) return;
  const PrefillRow pr = prefill_row(p, blockIdx.z);
  if (pr.T <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int jl = lane % LPR, gl = lane / LPR;
  const int Hk = p.Hk, Hv = p.Hv, C = p.C;
  const int ih = h / p.G;
  const int rho = rb0 + wv * RPW + gl;  // this lane group's state row
  const bool live = rho < DV;
  const size_t tile = ((size_t)pr.slot * Hv + h) * DV * DK + (size_t)(live ? rho : 0) * DK;

  v4f S[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
    S[n] = (pr.init && live)
               ? *reinterpret_cast<const v4f*>(p.ssm_pool + tile + (n * LPR + jl) * 4)
               : v4f{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < pr.T; c0 += kChunk) {
    const int n_t = min(kChunk, pr.T - c0);
    __syncthreads();
    for (int idx = tid; idx < n_t * DK; idx += kThreads) {
      int t = idx / DK, c = idx - t * DK;
      const float* yj = y + (size_t)(pr.j0 + c0 + t) * C;
      ks[t][c] = yj[Hk * DK + ih * DK + c];
      qs[t][c] = yj[ih * DK + c];
    }
    for (int idx = tid; idx < n_t * RB; idx += kThreads) {
      int t = idx / RB, rr = idx - t * RB;
      vsh[t][rr] = (rb0 + rr < DV)
                       ? y[(size_t)(pr.j0 + c0 + t) * C + 2 * Hk * DK + h * DV + rb0 + rr]
                       : 0.f;
    }
    if (tid < n_t) {
      const size_t j = (size_t)(pr.j0 + c0 + tid);
      al[tid] = gav[j * Hv + h];
      be[tid] = gbv[j * Hv + h];
      kqs[tid] = kqv[j * Hk + ih];
      rows[tid] = global_row(p, (int)j);
    }
    __syncthreads();
    for (int t = 0; t < n_t; ++t) {
      v4f kv[4], qv[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        kv[n] = *reinterpret_cast<const v4f*>(&ks[t][(n * LPR + jl) * 4]);
        qv[n] = *reinterpret_cast<const v4f*>(&qs[t][(n * LPR + jl) * 4]);
      }
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        a0 = fmaf(S[n].x, kv[n].x, a0); a1 = fmaf(S[n].x, qv[n].x, a1);
        a0 = fmaf(S[n].y, kv[n].y, a0); a1 = fmaf(S[n].y, qv[n].y, a1);
        a0 = fmaf(S[n].z, kv[n].z, a0); a1 = fmaf(S[n].z, qv[n].z, a1);
        a0 = fmaf(S[n].w, kv[n].w, a0); a1 = fmaf(S[n].w, qv[n].w, a1);
      }
      const float pk = group_sum<LPR>(a0), pq = group_sum<LPR>(a1);
      const float alpha = expf(al[t]), beta = be[t];
      const float vr = live ? vsh[t][rho - rb0] : 0.f;
      const float u = beta * (vr - alpha * pk);
      const float o = fmaf(alpha, pq, u * kqs[t]);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        S[n].x = fmaf(u, kv[n].x, alpha * S[n].x);
        S[n].y = fmaf(u, kv[n].y, alpha * S[n].y);
        S[n].z = fmaf(u, kv[n].z, alpha * S[n].z);
        S[n].w = fmaf(u, kv[n].w, alpha * S[n].w);
      }
      if (jl == 0 && live) obs[t][rho - rb0] = o;
    }
    __syncthreads();
    for (int idx = tid; idx < n_t * RB; idx += kThreads) {
      int t = idx / RB, rr = idx - t * RB;
      int r = rows[t];
      if (r >= 0 && rb0 + rr < DV)
        p.out[((size_t)r * Hv + h) * DV + rb0 + rr] = f2bf(obs[t][rr]);
    }
  }
  if (pr.slot > 0 && live) {
#pragma unroll
    for (int n = 0; n < 4; ++n)
      *reinterpret_cast<v4f*>(p.ssm_pool + tile + (n * LPR + jl) * 4) = S[n];
  }
}

template <int DK, int DV>
hipError_t launch_prefill_typed(const PrefillArgs& args, hipStream_t s) {
  const WsLayout w = ws_layout(args.Hk, args.Hv, DK, DV, args.stream_tokens, args.num_rows);
  char* ws = static_cast<char*>(args.workspace);
  float* y = reinterpret_cast<float*>(ws + w.y);
  float* kq = reinterpret_cast<float*>(ws + w.kq);
  float* ga = reinterpret_cast<float*>(ws + w.ga);
  float* gb = reinterpret_cast<float*>(ws + w.gb);
  int* map = reinterpret_cast<int*>(ws + w.map);
  PrefillArgs a = args;
  a.units = w.units;
  a.unit_map = map;
  hipLaunchKernelGGL(prefill_map_kernel, dim3(1), dim3(kMapThreads), 0, s, a, map, w.units);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g1(a.units, (a.C / kCh + kThreads - 1) / kThreads, kSeg / kTokThread);
  // the usual layer (width 4, SiLU) takes the specialised kernel
  auto conv = a.W == 4 && a.act ? conv_prefill_kernel<DK, 4, 1> : conv_prefill_kernel<DK, 0, -1>;
  hipLaunchKernelGGL(conv, g1, dim3(kThreads), 0, s, a, y, ga, gb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (DK < 64) {
    hipLaunchKernelGGL(kq_prefill_kernel<DK>, dim3(a.stream_tokens), dim3(kThreads), 0, s, a, y,
                       kq);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (DK >= 64) {
    ChunkWs cw{reinterpret_cast<float*>(ws + w.W), reinterpret_cast<float*>(ws + w.U),
               reinterpret_cast<float*>(ws + w.P), reinterpret_cast<float*>(ws + w.G)};
    return launch_chunked(a, DK, DV, y, ga, gb, cw, s);
  } else {
    constexpr int RB = (kThreads / 64) * (64 / (DK / 16));
    dim3 g3((DV + RB - 1) / RB, a.Hv, a.num_rows);
    hipLaunchKernelGGL((delta_prefill_kernel<DK, DV>), g3, dim3(kThreads), 0, s, a, y, kq, ga, gb);
    return hipGetLastError();
  }
}

}  // namespace

size_t prefill_workspace_bytes(int Hk, int Hv, int dk, int dv, int stream_tokens,
                               int rows) {
  if (rows <= 0) return 0;
  return ws_layout(Hk, Hv, dk, dv, stream_tokens, rows).total;
}

hipError_t launch_prefill(const PrefillArgs& a, int dk, int dv, hipStream_t s) {
  if (a.num_rows <= 0 || a.stream_tokens <= 0) return hipSuccess;
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 16: return launch_prefill_typed<16, 16>(a, s);
    case 32: return launch_prefill_typed<32, 32>(a, s);
    case 64: return launch_prefill_typed<64, 64>(a, s);
    case 128: return launch_prefill_typed<128, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
