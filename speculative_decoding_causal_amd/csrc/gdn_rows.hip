// Fused GDN step for short rows (spec-verify rows and one-token decodes).
//
// One workgroup per (row, k-head).  The workgroup owns every conv channel
// that k-head i reads - its q block, its k block and the v blocks of its
// G = Hv/Hk v-heads - so it is the only reader and the only writer of those
// channels of the row's conv slot: the "stage, then roll" contract of
// "[GDN] Spec-decoding-aware attention kernel" ("Changes") holds inside one
// workgroup, with the pre-state staged in LDS before the ring is rewritten.
//
// With turn counters (RowArgs::turns) the fused step of a launch with one
// row set runs one workgroup per (row, v-head) instead (dk = dv = 128,
// G > 1): half the state per workgroup at G = 2, twice the workgroups.  The
// G workgroups of a k-head each read and convolve the shared q and k
// channels; each rolls its own v channels, and the q/k channels are rolled
// by the last of the G to have consumed its window.  Each of the 2*dk/64
// waves that hold q/k channels, once its loads of them have returned, steps
// its counter of (conv slot, k-head, wave) with a wrapping increment (0, 1,
// .., G-1, 0); the wave that finds G-1 is the last reader of those 64
// channels and rewrites them at its end.  Every row steps a counter 0 or G
// times, so the counters are back at 0 after every call (graph replays
// included), and no workgroup ever waits for another.
//
// When such a launch runs one workgroup per CU, its last units form a
// dynamic tail: the last workgroup of each CU claims them one at a time
// from a wrapping count in the counter cell of the NULL conv slot (slot 0,
// which the turns never use), so the CUs of a faster XCD take more of them.
// (On MI355X one XCD's workgroups can take up to 10% longer than another's
// for the same work, and the same XCDs are the slower ones from run to run.)
//
// Phases:
//   1. conv: stage the ring columns and the row's inputs (gathered through
//      token_indx) in LDS and convolve (spec rows: window at n_acc-1;
//      non-spec rows: ring tail);
//   2. gates (read at the same global rows, per the gate-gather fix of
//      "[Bugfix] Align Qwen GDN gates with speculative tokens");
//   3. the recurrence, streaming the G*dv state rows of the k-head's v-heads
//      through VGPRs: each state row of dk floats is spread over dk/16 lanes
//      (16 floats, four float4 each), so row dot products need dk/16-lane DPP
//      sums and every global access moves full 128-byte lines (at dk = 128
//      the waves' rows interleave, so one instruction of the workgroup
//      covers 64 consecutive rows).  The q/k L2 norms and k.q come from the
//      same lanes' sums over their 16 channels, so no phase of their own
//      stands between the conv and the first state store.  The state of
//      each token is stored to its slot (spec) or only the final one
//      (non-spec).  The initial-state load precedes every store of the row.
//   4. outputs remapped through token_indx, as bf16; then the ring roll
//      (spec rows: shift n_acc; non-spec rows: shift T), from the pre-state
//      still staged in LDS, after the state stores it would otherwise delay.
//
// The per-token arithmetic is identical for spec and non-spec rows, so a
// spec row whose history is fully accepted reproduces sequential decodes
// bit for bit.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

struct RowPlan {
  int T;           // tokens processed
  int j0;          // first stream index
  int conv_slot;   // ring slot read/written (<= 0: none)
  bool read_hist;  // read the ring (else zeros)
  int off;         // ring column of the first window sample
  int shift;       // roll: new column l <- old column shift + l
  int load_slot;   // initial state slot (<= 0: zero state)
  const int* save; // per-token conv slots (spec rows, per-token layout), else null
};

// Read-only inputs that no kernel of the step writes (metadata, A_log,
// dt_bias), read through the constant address space: a uniform address then
// takes a scalar load even after the unit's own stores (a workgroup that
// goes on to a claimed unit reads its metadata after storing states).
template <class T>
__device__ __forceinline__ T ldc(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

__device__ __forceinline__ int slot_or_null(int s, int num_slots) {
  return (s > 0 && s < num_slots) ? s : 0;
}

__device__ RowPlan plan_row(const RowArgs& p, int row) {
  RowPlan r;
  int j0 = clampi(ldc(p.qsl + row), 0, p.num_tokens);
  int j1 = clampi(ldc(p.qsl + row + 1), j0, p.num_tokens);
  r.j0 = j0;
  r.T = min(j1 - j0, p.max_row_tokens);
  const int L = p.L, W = p.W;
  r.save = nullptr;
  if (p.kind == kSpec && p.conv_per_token) {
    // one window per slot (L == W-1): read at the slot of token n_acc-1,
    // saved after every token to that token's slot
    const int* ssi = p.ssi + (size_t)row * p.row_stride;
    const int T = r.T > 0 ? r.T : 1;
    r.load_slot = slot_or_null(ldc(ssi + clampi(ldc(p.nacc + row), 1, T) - 1), p.num_slots);
    r.conv_slot = r.load_slot;
    r.read_hist = true;
    r.off = 0;
    r.shift = 0;
    r.save = ssi;
  } else if (p.kind == kSpec) {
    const int* ssi = p.ssi + (size_t)row * p.row_stride;
    int T = r.T > 0 ? r.T : 1;
    // n_acc outside [1, min(T, L-W+2)] is a precondition violation; clamp so
    // every access stays inside the slot.
    const int nacc = ldc(p.nacc + row);
    const int n = clampi(nacc, 1, min(T, L - W + 2));
    r.conv_slot = slot_or_null(p.cache_idx ? ldc(p.cache_idx + row) : ldc(ssi), p.num_slots);
    r.read_hist = true;
    r.off = n - 1;
    r.shift = n;
    r.load_slot = slot_or_null(ldc(ssi + clampi(nacc, 1, T) - 1), p.num_slots);
  } else {
    int c = slot_or_null(ldc(p.cache_idx + row), p.num_slots);
    bool init = (p.his ? ldc(p.his + row) != 0 : true) && c > 0;
    r.conv_slot = c;
    r.read_hist = init;
    r.off = L - W + 1;
    r.shift = r.T;
    r.load_slot = init ? c : 0;
  }
  return r;
}

// LDS carve-up shared by the launcher (size) and the kernel (offsets).
struct Lds {
  int rows, stores;  // int[kMaxRowTokens] each
  int zb;            // uint16 [(L + Tm) * NCH]
  int qs, ks;        // float [Tm * DK]
  int vs, ob;        // float [Tm * NR]
  int ga, gb;        // float [Tm * G]
  int total;
};

__host__ __device__ inline int align16(int x) { return (x + 15) & ~15; }

__host__ __device__ inline Lds lds_layout(int DK, int DV, int G, int L, int Tm) {
  Lds l;
  const int NCH = 2 * DK + G * DV, NR = G * DV;
  int o = 0;
  l.rows = o;   o += align16(kMaxRowTokens * 4);
  l.stores = o; o += align16(kMaxRowTokens * 4);
  l.qs = o;     o += align16(Tm * DK * 4);
  l.ks = o;     o += align16(Tm * DK * 4);
  l.vs = o;     o += align16(Tm * NR * 4);
  l.ob = o;     o += align16(Tm * NR * 4);
  l.ga = o;     o += align16(Tm * G * 4);
  l.gb = o;     o += align16(Tm * G * 4);
  l.zb = o;     o += align16((L + Tm) * NCH * 2);
  l.total = o;
  return l;
}

typedef float v4f __attribute__((ext_vector_type(4)));

// For dk = 128: state rows per lane (R), threads per workgroup (T), the
// waves per SIMD the registers are fitted to (WPE; 2 leaves the 128 KiB
// (row, k-head) unit room for its registers), rows taken through all tokens
// at a time (RB), whether snapshots use non-temporal stores, the row order
// (ORDER: 1 interleaves the waves, so each instruction of the workgroup
// covers 64 consecutive state rows) and a floor on the dynamic LDS (LDS_MIN:
// above half of the CU's 160 KiB, so one workgroup runs per CU); all chosen
// by measurement on MI355X: with more than three (row, k-head) units per CU,
// one interleaved workgroup per CU moves the state about 2% faster than two
// banded ones.
#ifndef GDN_ROWS_R128
#define GDN_ROWS_R128 4
#endif
#ifndef GDN_ROWS_T128
#define GDN_ROWS_T128 512
#endif
#ifndef GDN_ROWS_WPE128
#define GDN_ROWS_WPE128 2
#endif
#ifndef GDN_ROWS_RB128
#define GDN_ROWS_RB128 4
#endif
#ifndef GDN_NT_STORE
#define GDN_NT_STORE 1
#endif
#ifndef GDN_ROWS_ORDER128
#define GDN_ROWS_ORDER128 1
#endif
#ifndef GDN_ROWS_LDS_MIN128
#define GDN_ROWS_LDS_MIN128 (80 * 1024 + 16)
#endif
// (row, v-head) units: state rows per lane (one pass over dv rows), waves
// per SIMD, when the one-per-CU floor (and with it the dynamic tail)
// applies (rows of at least VH_FLOOR_TOKENS tokens on at least
// VH_FLOOR_UNITS units per CU; one-token rows and smaller grids run faster
// with several workgroups per CU), and
// whether launches that carry decodes and spec rows together take them
// (VH_MIXED: the one-token decodes repeat the q/k conv per v-head for a
// single state update, and such a launch measured faster per k-head).
#ifndef GDN_ROWS_RV128
#define GDN_ROWS_RV128 2
#endif
#ifndef GDN_ROWS_WPE_VH128
#define GDN_ROWS_WPE_VH128 4
#endif
#ifndef GDN_ROWS_VH_FLOOR_TOKENS
#define GDN_ROWS_VH_FLOOR_TOKENS 2
#endif
#ifndef GDN_ROWS_VH_FLOOR_UNITS
#define GDN_ROWS_VH_FLOOR_UNITS 4
#endif
#ifndef GDN_ROWS_VH_MIXED
#define GDN_ROWS_VH_MIXED 0
#endif
// Dynamic tail of (row, v-head) launches that run one workgroup per CU:
// 1/TAIL_DIV of the units (0: off), at most TAIL_ROUNDS units per CU, taken
// by the last workgroup of each CU.  Measured on MI355X (one process,
// alternating): K=3, 64 rows 96.9 us (97.9 without); K=4, 96 rows 175.9
// (179.0); K=4, 256 rows 459.5 with two units per CU (470.3).
#ifndef GDN_ROWS_TAIL_DIV
#define GDN_ROWS_TAIL_DIV 8
#endif
#ifndef GDN_ROWS_TAIL_ROUNDS
#define GDN_ROWS_TAIL_ROUNDS 2
#endif

// State snapshots go through a buffer resource per (token slot, unit): the
// slot's block is a scalar base and each lane's row a 32-bit offset, so no
// 64-bit lane addresses stay live across the tokens.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void store_row4(__amdgpu_buffer_rsrc_t rs, unsigned off, v4f v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rs, off, 0, GDN_NT_STORE ? 2 : 0);
}

// Load the R state rows of one lane group: rows rho0 + s*RPW, 16 columns
// each (four float4 at columns (n*LPR + jl)*4).  No load sits behind a
// branch (a branch join would wait for it): `base` is readable even for a
// NULL slot (slot 0 stands in) and rows past NR re-read row NR-1;
// zero_rows drops those values where the rows are first used, so the loads
// stay in flight until then.
template <int DK, int R, int LPR, int SS>
__device__ __forceinline__ void load_rows(v4f (&S)[R][4], const float* base, int rho0, int jl,
                                          int NR) {
#pragma unroll
  for (int s = 0; s < R; ++s) {
    const int rho = rho0 + s * SS;
    const unsigned off = static_cast<unsigned>((rho < NR ? rho : NR - 1) * DK + jl * 4) * 4u;  // bytes
    const float* row = reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + off);
#pragma unroll
    for (int n = 0; n < 4; ++n)
      S[s][n] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(row + n * LPR * 4));
  }
}

template <int R, int SS>
__device__ __forceinline__ void zero_rows(v4f (&S)[R][4], bool valid, int rho0, int NR) {
#pragma unroll
  for (int s = 0; s < R; ++s) {
    const bool keep = valid && rho0 + s * SS < NR;
#pragma unroll
    for (int n = 0; n < 4; ++n) S[s][n] = keep ? S[s][n] : v4f{0.f, 0.f, 0.f, 0.f};
  }
}

// Inputs of one conv channel, gathered into registers in one batch: ring
// columns (LM >= L), the row's inputs (KT >= T), taps and bias.
template <int LM, int KT>
struct ChanIn {
  uint16_t h[LM];         // raw ring columns (dropped without history / past L)
  uint16_t x[KT];         // raw inputs (dropped for tokens outside the batch)
  uint16_t w[kMaxWidth];  // raw bf16 taps (dropped past W)
  uint16_t bias;          // raw bf16 bias (dropped without one)
  bool hist;
};

template <int KT>
__device__ __forceinline__ int pick(const int (&v)[KT], int j) {
  int r = -1;
#pragma unroll
  for (int jj = 0; jj < KT; ++jj)
    if (jj == j) r = v[jj];
  return r;
}

// Channel of position pc of a unit: the q and k blocks of k-head ih, then
// the v blocks of the unit's v-heads from hv0 on.
__device__ __forceinline__ int channel_of(int pc, int ih, int hv0, int Hk, int DK, int DV) {
  if (pc < DK) return ih * DK + pc;
  if (pc < 2 * DK) return Hk * DK + ih * DK + (pc - DK);
  return 2 * Hk * DK + hv0 * DV + (pc - 2 * DK);
}

// Column of mixed_qkv for channel position pc (grouped channel c): with the
// per-k-head layout k-head ih's channels are one block [q, k, v of its G
// v-heads].
__device__ __forceinline__ int input_column(const RowArgs& p, int pc, int c, int ih, int hv0,
                                            int DK, int DV) {
  const int bp = pc < 2 * DK ? pc : 2 * DK + (hv0 - ih * p.G) * DV + (pc - 2 * DK);
  return p.qkv_layout ? ih * (2 * DK + p.G * DV) + bp : c;
}

template <int LM, int KT>
__device__ __forceinline__ void load_chan(ChanIn<LM, KT>& in, const RowArgs& p,
                                          const RowPlan& rp, int c, int cin,
                                          const int (&rj)[KT]) {
  // Every load goes to an address that exists and unwanted values are
  // dropped afterwards: a load behind a branch is waited for where the
  // branch joins, one memory round trip each.  Stand-ins: slot 0's ring for
  // a row without history, the taps for an empty ring, a missing bias or an
  // empty mixed_qkv (the taps hold C*W >= C values), row 0 for a token
  // outside the batch, the last tap for taps past W.
  const bool hist = rp.read_hist && rp.conv_slot > 0;
  const uint16_t* ring = p.L > 0
      ? p.conv_pool + (size_t)(hist ? rp.conv_slot : 0) * p.L * p.C + c
      : p.conv_w + c;
  const int lmax = p.L > 0 ? p.L - 1 : 0;
  const uint16_t* xs = p.num_actual_tokens > 0 ? p.qkv : p.conv_w;
  const uint16_t* bs = p.conv_b ? p.conv_b : p.conv_w;
#pragma unroll
  for (int l = 0; l < LM; ++l) in.h[l] = ring[(size_t)(l < lmax ? l : lmax) * p.C];
#pragma unroll
  for (int j = 0; j < KT; ++j) in.x[j] = xs[(size_t)(rj[j] >= 0 ? rj[j] : 0) * p.C + cin];
#pragma unroll
  for (int m = 0; m < kMaxWidth; ++m)
    in.w[m] = p.conv_w[(size_t)c * p.W + (m < p.W ? m : p.W - 1)];
  in.bias = bs[c];
  in.hist = hist;
}

// Taps and bias as floats, zero past W and without a bias.
template <int LM, int KT>
__device__ __forceinline__ void taps_of(const ChanIn<LM, KT>& in, const RowArgs& p,
                                        float (&w)[kMaxWidth], float& bias) {
#pragma unroll
  for (int m = 0; m < kMaxWidth; ++m) w[m] = m < p.W ? bf2f(in.w[m]) : 0.f;
  bias = p.conv_b ? bf2f(in.bias) : 0.f;
}

// Stage one channel's pre-state and inputs in this thread's LDS column
// zb[.][pc] (runtime window offsets are cheap there).
template <int LM, int KT>
__device__ __forceinline__ void stage_chan(const ChanIn<LM, KT>& in, int L, int T, int pc,
                                           int NCH, uint16_t* zb, const int (&rj)[KT]) {
#pragma unroll
  for (int l = 0; l < LM; ++l)
    if (l < L) zb[l * NCH + pc] = in.hist ? in.h[l] : (uint16_t)0;
#pragma unroll
  for (int j = 0; j < KT; ++j)
    if (j < T) zb[(L + j) * NCH + pc] = rj[j] >= 0 ? in.x[j] : (uint16_t)0;
}

// Roll one staged channel's ring (or write its per-token windows); every
// ring write follows every read of the pre-state (all of it is in LDS).
__device__ __forceinline__ void roll_chan(const RowArgs& p, const RowPlan& rp, int c, int pc,
                                          int NCH, int T, const uint16_t* zb) {
  const int L = p.L;
  if (rp.save) {
    // per-token slots: the window after token t is staged rows t+1 .. t+W-1
    // (L == W-1 history rows, then the inputs), in token order
    for (int t = 0; t < T; ++t) {
      const int s = slot_or_null(rp.save[t], p.num_slots);
      if (s <= 0) continue;
      uint16_t* wslot = p.conv_pool + (size_t)s * L * p.C + c;
      for (int l = 0; l < L; ++l) wslot[(size_t)l * p.C] = zb[(t + 1 + l) * NCH + pc];
    }
  } else if (rp.conv_slot > 0) {
    uint16_t* wring = p.conv_pool + (size_t)rp.conv_slot * L * p.C + c;
    for (int l = 0; l < L; ++l) {
      const int src = l < L - T ? rp.shift + l : T + l;
      wring[(size_t)l * p.C] = zb[src * NCH + pc];
    }
  }
}

// Convolve one staged channel and, with `roll`, roll its ring.
template <int KT>
__device__ __forceinline__ void conv_chan(const float (&w)[kMaxWidth], float bias,
                                          const RowArgs& p, const RowPlan& rp, int c, int pc,
                                          int NCH, int T, const uint16_t* zb, float* dst,
                                          int dstride, const int (&rj)[KT], bool roll) {
  const int L = p.L, W = p.W;
  auto emit = [&](int j, float acc) {
    if (p.act) acc = silu(acc);
    if (p.stage == kConvOnly) {
      const int r = pick<KT>(rj, j);
      if (r >= 0) p.y[(size_t)r * p.C + c] = acc;
    } else {
      dst[j * dstride] = acc;
    }
  };
  // Window sample i = j + m of token j is staged row off + i among the
  // pre-state columns, or input row i - (W-1) after them.
  if constexpr (KT <= 8) {
    // short rows: every token's samples read in one batch (a read per loop
    // step would wait for each in turn); samples the taps never reach
    // repeat the last staged row
    constexpr int NS = KT + kMaxWidth - 1;
    float z[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      int zi = i < W - 1 ? rp.off + i : L + i - (W - 1);
      zi = zi < L + T ? zi : L + T - 1;
      z[i] = bf2f(zb[zi * NCH + pc]);
    }
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      if (j < T) {
        float acc = bias;
#pragma unroll
        for (int m = 0; m < kMaxWidth; ++m) acc = m < W ? fmaf(w[m], z[j + m], acc) : acc;
        emit(j, acc);
      }
    }
  } else {
    for (int j = 0; j < T; ++j) {
      float acc = bias;
#pragma unroll
      for (int m = 0; m < kMaxWidth; ++m) {
        if (m < W) {
          const int idx = j + m;
          const int zi = idx < W - 1 ? rp.off + idx : L + idx - (W - 1);
          acc = fmaf(w[m], bf2f(zb[zi * NCH + pc]), acc);
        }
      }
      emit(j, acc);
    }
  }
  if (roll) roll_chan(p, rp, c, pc, NCH, T, zb);
}

// NT threads per workgroup, R state rows per lane; WPE waves per SIMD is the
// occupancy the register budget is fitted to.  LM / KT bound state_len and
// the tokens per row for the register gathers of the conv phase.
// One unit of the launch: virtual workgroup index vb, mapped to (row, head)
// as below.  A claim of the dynamic tail, when `post`, is written to *tail_sh
// by thread 0 before the phase-2 barrier (its result is back by then, the
// state loads being younger).  Returns whether it got that far.
template <int DK, int DV, int R, int NT, int WPE, int LM, int KT, int RB, bool FUSED, int ORDER,
          bool VH>
__device__ __forceinline__ bool rows_unit(const RowArgs& pa, const int vb, const bool post,
                                          const unsigned int claim, unsigned int* tail_sh) {
  static_assert(R % RB == 0, "row batch");
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int LPR = DK / 16;    // lanes per state row
  constexpr int RPW = 64 / LPR;   // state rows per wave per sub-pass
  static_assert(DK % 64 == 0 || DK == 16 || DK == 32, "dk");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int Hk = pa.Hk, G = pa.G, C = pa.C, L = pa.L;
  // The unit: k-head ih and its GU v-heads from hv0 on (all G of them, or
  // one with turn counters).
  const int GU = VH ? 1 : G;
  const int NU = VH ? Hk * G : Hk;  // units per row
  // Workgroup i runs on XCD i % 8: the units of a row share i % 8, so
  // each XCD's L2 fetches a row's metadata and gate rows once.  The grid is
  // padded to whole groups of 8 rows.
  const int q8 = vb >> 3;
  const int hu = q8 % NU;
  const int ih = VH ? hu / G : hu;
  const int hv0 = VH ? hu : hu * G;
  int row = (q8 / NU) * 8 + (vb & 7);
  if (row >= pa.num_rows + (pa.more.num_rows > 0 ? pa.more.num_rows : 0)) return false;
  const int NCH = 2 * DK + GU * DV;
  const int NR = GU * DV;
  const int Tm = launch_row_tokens(pa);
  // rows of the second set take its kind and metadata (uniform selects)
  RowArgs p = pa;
  if (row >= pa.num_rows) {
    row -= pa.num_rows;
    p.kind = pa.more.kind;
    p.num_rows = pa.more.num_rows;
    p.num_tokens = pa.more.num_tokens;
    p.row_stride = pa.more.row_stride;
    p.max_row_tokens = pa.more.max_row_tokens;
    p.qsl = pa.more.qsl;
    p.cache_idx = pa.more.cache_idx;
    p.ssi = pa.more.ssi;
    p.nacc = pa.more.nacc;
    p.his = pa.more.his;
    p.tix = pa.more.tix;
  }

  const RowPlan rp = plan_row(p, row);
  const int T = rp.T;
  if (T <= 0) return false;

  const Lds lay = lds_layout(DK, DV, GU, L, Tm);
  int* rows_s = reinterpret_cast<int*>(smem + lay.rows);
  int* st_s = reinterpret_cast<int*>(smem + lay.stores);
  float* qs = reinterpret_cast<float*>(smem + lay.qs);
  float* ks = reinterpret_cast<float*>(smem + lay.ks);
  float* vs = reinterpret_cast<float*>(smem + lay.vs);
  float* ob = reinterpret_cast<float*>(smem + lay.ob);
  float* ga = reinterpret_cast<float*>(smem + lay.ga);
  float* gb = reinterpret_cast<float*>(smem + lay.gb);
  uint16_t* zb = reinterpret_cast<uint16_t*>(smem + lay.zb);

  // Global rows of the row's tokens (uniform scalar loads) and, in LDS for
  // the later phases, rows and state-store slots.
  int rj[KT];
#pragma unroll
  for (int j = 0; j < KT; ++j) {
    int r = -1;
    if (j < T) {
      r = p.tix ? ldc(p.tix + rp.j0 + j) : rp.j0 + j;
      if (r < 0 || r >= p.num_actual_tokens) r = -1;
    }
    rj[j] = r;
  }
  if (tid < T) {
    rows_s[tid] = rj[0];
#pragma unroll
    for (int j = 1; j < KT; ++j)
      if (tid == j) rows_s[tid] = rj[j];
    int st;
    if (p.kind == kSpec)
      st = slot_or_null(p.ssi[(size_t)row * p.row_stride + tid], p.num_slots);
    else
      st = (tid == T - 1) ? rp.conv_slot : 0;
    st_s[tid] = st;
  }

  // The conv and gate inputs are gathered in one batch of loads (vector loads
  // complete in order, so nothing slow may be issued ahead of them).
  // The fused step knows its stage at compile time (no branch around its
  // loads); the stage entry points read it from the arguments.
  const int stage = FUSED ? kFused : p.stage;
  const bool conv_stage = stage != kDeltaOnly;
  const bool have_chan = conv_stage && tid < NCH;
  const int c0 = channel_of(tid, ih, hv0, Hk, DK, DV);
  float w0[kMaxWidth], bias0 = 0.f;
  float a_log0, dt_bias0;
  // State rows of this lane (first pass), their slot and head block.
  const int jl = lane % LPR, gl = lane / LPR;
  const size_t slot_stride = (size_t)p.Hv * DV * DK;
  const size_t head_off = (size_t)hv0 * DV * DK;
  const bool load_valid = rp.load_slot > 0;
  const float* load_base = p.ssm_pool + (size_t)(load_valid ? rp.load_slot : 0) * slot_stride +
                           head_off;
  constexpr int kRowsPerWavePass = RPW * R;
  constexpr int kRowsPerPass = (NT / 64) * kRowsPerWavePass;
  // Rows of a lane: ORDER 0 gives each wave a band of RPW*R consecutive
  // rows (sub-row stride RPW); ORDER 1 interleaves the waves, so that the
  // workgroup's instruction s covers NT/64*RPW consecutive rows (sub-row
  // stride NT/64*RPW).
  constexpr int SS = ORDER ? (NT / 64) * RPW : RPW;
  const int wave_row0 = ORDER ? wv * RPW : wv * kRowsPerWavePass;
  constexpr bool kEarlyRows = LM + KT <= 10;
  v4f S[R][4];
  // waves holding the q/k channels (one channel per thread, 64 per wave)
  constexpr int kQKW = 2 * DK / 64;
  static_assert(!VH || 2 * DK <= NT, "one q/k channel per thread");
  unsigned int turn_old = 0;
  {
    // Gate inputs join the same batch (no branch around the loads): rows
    // outside the batch read row 0; with no token rows, or in the conv-only
    // stage (no gates), the loads go to A_log or the taps and are dropped.
    const bool have_gate0 = stage != kConvOnly && tid < T * GU;
    const bool gate_rows = stage != kConvOnly && p.num_actual_tokens > 0;
    const uint16_t* gsrc_a = gate_rows ? p.a
        : (stage != kConvOnly ? reinterpret_cast<const uint16_t*>(p.A_log) : p.conv_w);
    const uint16_t* gsrc_b = gate_rows ? p.b : gsrc_a;
    const int gr = have_gate0 ? pick<KT>(rj, tid / GU) : -1;
    const int gh = hv0 + tid % GU;
    const size_t gi = gate_rows ? (size_t)(gr >= 0 ? gr : 0) * p.Hv + gh : (size_t)gh;
    const uint16_t raw_a = gsrc_a[gi], raw_b = gsrc_b[gi];
    // the head's A_log and dt_bias too (the taps stand in for the conv-only
    // stage, which has no gates), so phase 2 issues no load behind the state
    const float* gsrc_l = stage != kConvOnly ? p.A_log : reinterpret_cast<const float*>(p.conv_w);
    const float* gsrc_d = stage != kConvOnly ? p.dt_bias : gsrc_l;
    a_log0 = ldc(gsrc_l + gh);
    dt_bias0 = ldc(gsrc_d + gh);
    // Every thread loads a channel (threads past the last one repeat it) so
    // that no load waits behind a per-thread branch.
    ChanIn<LM, KT> in0;
    if (conv_stage) {
      const int pcl = tid < NCH ? tid : NCH - 1;
      const int cl = tid < NCH ? c0 : channel_of(pcl, ih, hv0, Hk, DK, DV);
      load_chan<LM, KT>(in0, p, rp, cl, input_column(p, pcl, cl, ih, hv0, DK, DV), rj);
    }
    // The first pass of state rows follows the conv and gate inputs in the
    // same stream of loads: it lands while the conv runs (vector loads
    // complete in order, so the conv waits only for its own inputs).
    // (Only with the smallest register gathers: the others leave no room.)
    if constexpr (kEarlyRows) {
      if (stage != kConvOnly)
        load_rows<DK, R, LPR, SS>(S, load_base, wave_row0 + gl, jl, NR);
      // keep the state loads ahead of the staging, which waits for the conv inputs
      __builtin_amdgcn_sched_barrier(0);
    }
    if (have_chan) stage_chan<LM, KT>(in0, L, T, tid, NCH, zb, rj);
    if (have_gate0) {
      // raw gate inputs; turned into alpha/beta below
      ga[tid] = gr >= 0 ? bf2f(raw_a) : 0.f;
      gb[tid] = gr >= 0 ? bf2f(raw_b) : 0.f;
    }
    if (have_chan) taps_of<LM, KT>(in0, p, w0, bias0);
    // The turn of a q/k wave, once every conv load of the wave has
    // returned: the counter's address carries an opaque zero computed from
    // all of them (a wave's loads return together, lane by lane), so the
    // step cannot be issued earlier.  Its result is first read after the
    // gates, with the state loads ahead of it.  (A wrapping increment: an add of a
    // uniform value would be rewritten into a wave-wide one that waits for
    // its result at once.)
    if constexpr (VH) {
      if (wv < kQKW && rp.conv_slot > 0) {
        int dep = in0.bias;
#pragma unroll
        for (int l = 0; l < LM; ++l) dep ^= in0.h[l];
#pragma unroll
        for (int j = 0; j < KT; ++j) dep ^= in0.x[j];
#pragma unroll
        for (int m = 0; m < kMaxWidth; ++m) dep ^= in0.w[m];
        int zero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(zero) : "v"(dep));
        const size_t cell = ((size_t)rp.conv_slot * Hk + ih) * kQKW + wv;
        if (lane == 0) turn_old = atomicInc(p.turns + cell + zero, (unsigned int)(G - 1));
      }
    }
  }
  // ---- phase 1: conv (or load of a precomputed conv output) -------------
  for (int pc = tid; pc < NCH; pc += NT) {
    const int c = pc == tid ? c0 : channel_of(pc, ih, hv0, Hk, DK, DV);
    // the fused step rolls its rings at its end, off the path to the first
    // state store; the conv-only stage ends here
    const bool roll = stage == kConvOnly;
    float* dst;
    int dstride;
    if (pc < DK) { dst = qs + pc; dstride = DK; }
    else if (pc < 2 * DK) { dst = ks + (pc - DK); dstride = DK; }
    else { dst = vs + (pc - 2 * DK); dstride = NR; }
    if (!conv_stage) {
      for (int j = 0; j < T; ++j) {
        const int r = pick<KT>(rj, j);
        dst[j * dstride] = r >= 0 ? p.y[(size_t)r * C + c] : 0.f;
      }
      continue;
    }
    if (pc == tid) {
      conv_chan<KT>(w0, bias0, p, rp, c, pc, NCH, T, zb, dst, dstride, rj, roll);
    } else {
      ChanIn<LM, KT> in;
      load_chan<LM, KT>(in, p, rp, c, input_column(p, pc, c, ih, hv0, DK, DV), rj);
      stage_chan<LM, KT>(in, L, T, pc, NCH, zb, rj);
      float w[kMaxWidth], bias;
      taps_of<LM, KT>(in, p, w, bias);
      conv_chan<KT>(w, bias, p, rp, c, pc, NCH, T, zb, dst, dstride, rj, roll);
    }
  }
  if (stage == kConvOnly) return false;
  if constexpr (!kEarlyRows)
    load_rows<DK, R, LPR, SS>(S, load_base, wave_row0 + gl, jl, NR);



  // ---- phase 2: gates -------------------------------------------------------
  if (tid < T * GU) gate_pair(ga[tid], gb[tid], a_log0, dt_bias0, &ga[tid], &gb[tid]);
  for (int idx = tid + NT; idx < T * GU; idx += NT) {
    const int j = idx / GU, g = idx - j * GU, h = hv0 + g;
    const int r = pick<KT>(rj, j);
    const float av = r >= 0 ? bf2f(p.a[(size_t)r * p.Hv + h]) : 0.f;
    const float bv = r >= 0 ? bf2f(p.b[(size_t)r * p.Hv + h]) : 0.f;
    gate_pair(av, bv, p.A_log[h], p.dt_bias[h], &ga[idx], &gb[idx]);
  }
  // The phases hand data over through LDS only: every global address a
  // thread writes (its ring channels, its state rows, an output) is read, if
  // at all, by that same thread, so the barrier orders LDS alone and waits
  // neither for the state loads nor for stores still in flight.
  if constexpr (VH) {
    if (post && tid == 0) *tail_sh = claim;
  }
  lds_barrier();
  // the last of the k-head's G waves to take its turn rolls the shared
  // channels; without a ring slot nothing is read, and the wave of one
  // fixed workgroup writes (per-token windows)
  bool roll_qk = false;
  if constexpr (VH) {
    if (wv < kQKW)
      roll_qk = rp.conv_slot > 0
                    ? __builtin_amdgcn_readfirstlane(turn_old) == (unsigned int)(G - 1)
                    : hv0 % G == G - 1;
  }
  // ---- phase 3: recurrence over the state rows -----------------------------
  // Rows are taken RB at a time through all the row's tokens, so the first
  // snapshots are stored as soon as those rows' loads have arrived.
  for (int r0 = wave_row0; r0 < NR; r0 += kRowsPerPass) {
    const bool full = r0 + (R - 1) * SS + RPW <= NR;
    const int rho0 = r0 + gl;
    if (r0 != wave_row0) load_rows<DK, R, LPR, SS>(S, load_base, rho0, jl, NR);
    zero_rows<R, SS>(S, load_valid, rho0, NR);
#pragma unroll
    for (int sb = 0; sb < R; sb += RB) {
      for (int j = 0; j < T; ++j) {
        // S k and S q against the raw conv outputs, and |q|^2, |k|^2 and
        // k.q: each lane holds 16 channels, the LPR lanes of a row all DK,
        // so every row group gets the token's norms from its own sums.
        float pk[RB], pq[RB];
#pragma unroll
        for (int q = 0; q < RB; ++q) { pk[q] = 0.f; pq[q] = 0.f; }
        float sq = 0.f, sk = 0.f, dkq = 0.f;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const v4f kv = *reinterpret_cast<const v4f*>(ks + j * DK + (n * LPR + jl) * 4);
          const v4f qv = *reinterpret_cast<const v4f*>(qs + j * DK + (n * LPR + jl) * 4);
          sq = fmaf(qv.x, qv.x, sq); sk = fmaf(kv.x, kv.x, sk); dkq = fmaf(kv.x, qv.x, dkq);
          sq = fmaf(qv.y, qv.y, sq); sk = fmaf(kv.y, kv.y, sk); dkq = fmaf(kv.y, qv.y, dkq);
          sq = fmaf(qv.z, qv.z, sq); sk = fmaf(kv.z, kv.z, sk); dkq = fmaf(kv.z, qv.z, dkq);
          sq = fmaf(qv.w, qv.w, sq); sk = fmaf(kv.w, kv.w, sk); dkq = fmaf(kv.w, qv.w, dkq);
#pragma unroll
          for (int q = 0; q < RB; ++q) {
            const v4f x = S[sb + q][n];
            pk[q] = fmaf(x.x, kv.x, pk[q]); pq[q] = fmaf(x.x, qv.x, pq[q]);
            pk[q] = fmaf(x.y, kv.y, pk[q]); pq[q] = fmaf(x.y, qv.y, pq[q]);
            pk[q] = fmaf(x.z, kv.z, pk[q]); pq[q] = fmaf(x.z, qv.z, pq[q]);
            pk[q] = fmaf(x.w, kv.w, pk[q]); pq[q] = fmaf(x.w, qv.w, pq[q]);
          }
        }
        sq = group_sum<LPR>(sq);
        sk = group_sum<LPR>(sk);
        dkq = group_sum<LPR>(dkq);
        // k^ = k ik, q^ = q iq scale: l2 norms with eps inside the root, by the
        // hardware reciprocal square root (within 1 ulp)
        const float ik = p.l2norm ? __builtin_amdgcn_rsqf(sk + p.eps) : 1.f;
        const float iqs = (p.l2norm ? __builtin_amdgcn_rsqf(sq + p.eps) : 1.f) * p.scale;
#pragma unroll
        for (int q = 0; q < RB; ++q) {
          pk[q] = group_sum<LPR>(pk[q]) * ik;
          pq[q] = group_sum<LPR>(pq[q]) * iqs;
        }
        const float kqj = dkq * ik * iqs;
        float al[RB], u[RB];
        if constexpr (ORDER == 0 && DV % kRowsPerWavePass == 0) {
          // The wave's rows lie in one v-head: its gates are wave-uniform.
          const int g = r0 / DV;
          const float alw = __builtin_bit_cast(
              float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ga[j * GU + g])));
          const float bew = __builtin_bit_cast(
              float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, gb[j * GU + g])));
#pragma unroll
          for (int q = 0; q < RB; ++q) {
            const int rho = rho0 + (sb + q) * SS;
            const float vr = vs[j * NR + (rho < NR ? rho : NR - 1)];
            al[q] = alw;
            // S_new = al S + u k^T with u = be (v - al S k); o = S_new q.
            u[q] = bew * (vr - alw * pk[q]);
            const float o = fmaf(alw, pq[q], u[q] * kqj);
            if (jl == 0 && rho < NR) ob[j * NR + rho] = o;
          }
        } else if constexpr (ORDER == 1 && DV % SS == 0) {
          // Interleaved rows: a lane's row offset within its sub-pass
          // (wave_row0 + gl) stays below SS, so sub-row sb + q of every lane
          // lies in the same v-head and its gates are wave-uniform.
#pragma unroll
          for (int q = 0; q < RB; ++q) {
            const int rho = rho0 + (sb + q) * SS;
            const int gq = (r0 - wave_row0 + (sb + q) * SS) / DV;
            const int g = gq < GU ? gq : GU - 1;
            al[q] = __builtin_bit_cast(
                float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ga[j * GU + g])));
            const float be = __builtin_bit_cast(
                float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, gb[j * GU + g])));
            const float vr = vs[j * NR + (rho < NR ? rho : NR - 1)];
            u[q] = be * (vr - al[q] * pk[q]);
            const float o = fmaf(al[q], pq[q], u[q] * kqj);
            if (jl == 0 && rho < NR) ob[j * NR + rho] = o;
          }
        } else {
#pragma unroll
          for (int q = 0; q < RB; ++q) {
            const int rho = rho0 + (sb + q) * SS;
            const int rr = rho < NR ? rho : NR - 1;
            const int g = rr / DV;
            al[q] = ga[j * GU + g];
            const float be = gb[j * GU + g];
            const float vr = vs[j * NR + rr];
            u[q] = be * (vr - al[q] * pk[q]);
            const float o = fmaf(al[q], pq[q], u[q] * kqj);
            if (jl == 0 && rho < NR) ob[j * NR + rho] = o;
          }
        }
        // u k^ = (u ik) k
#pragma unroll
        for (int q = 0; q < RB; ++q) u[q] *= ik;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const v4f kv = *reinterpret_cast<const v4f*>(ks + j * DK + (n * LPR + jl) * 4);
#pragma unroll
          for (int q = 0; q < RB; ++q) {
            v4f& x = S[sb + q][n];
            x.x = fmaf(u[q], kv.x, al[q] * x.x);
            x.y = fmaf(u[q], kv.y, al[q] * x.y);
            x.z = fmaf(u[q], kv.z, al[q] * x.z);
            x.w = fmaf(u[q], kv.w, al[q] * x.w);
          }
        }
        // the token's store slot is the workgroup's: a scalar base address,
        // 32-bit lane offsets
        const int st = __builtin_amdgcn_readfirstlane(st_s[j]);
        if (st > 0) {
          const __amdgpu_buffer_rsrc_t rs =
              block_rsrc(p.ssm_pool + (size_t)st * slot_stride + head_off, NR * DK * 4);
#pragma unroll
          for (int q = 0; q < RB; ++q) {
            const int rho = rho0 + (sb + q) * SS;
            if (full || rho < NR) {
              const unsigned off = static_cast<unsigned>(rho * DK + jl * 4) * 4u;  // bytes
#pragma unroll
              for (int n = 0; n < 4; ++n) store_row4(rs, off + n * LPR * 16, S[sb + q][n]);
            }
          }
        }
      }
    }
  }
  lds_barrier();

  // ---- phase 4: outputs, then the ring rolls -------------------------------
  uint16_t* out = p.out;
  for (int idx = tid; idx < T * NR; idx += NT) {
    int j = idx / NR, rr = idx - j * NR;
    int r = rows_s[j];
    if (r >= 0) out[((size_t)r * p.Hv + hv0) * DV + rr] = f2bf(ob[idx]);
  }
  // Each thread rolls the channels it staged (their pre-state and inputs
  // are still in its LDS column); with v-head units the shared q/k channels
  // only in the wave that was their last reader.
  if (conv_stage) {
    for (int pc = tid; pc < NCH; pc += NT) {
      if (VH && pc < 2 * DK && !roll_qk) continue;
      roll_chan(p, rp, channel_of(pc, ih, hv0, Hk, DK, DV), pc, NCH, T, zb);
    }
  }
  return true;
}

// Workgroup i takes unit i.  With a dynamic tail, the last tail_takers
// workgroups (the last to start on each CU) go on to claim the tail's units
// one at a time, each claim issued a whole unit ahead of its use, so a CU
// that finishes early takes more of the tail than one on a slower XCD.  The
// count wraps at tail_units + tail_takers - 1: every taker claims until its
// first claim past the tail, so exactly that many claims are made per launch
// and the count is back at 0 after every launch.
template <int DK, int DV, int R, int NT, int WPE, int LM, int KT, int RB, bool FUSED, int ORDER,
          bool VH>
__global__ void __launch_bounds__(NT, WPE)
gdn_rows_kernel(RowArgs pa) {
  if constexpr (VH) {
    // the claim in hand, double-buffered: a wave still reading one
    // iteration's entry never meets the next iteration's write
    __shared__ unsigned int tail_sh[2];
    const bool taker = pa.tail_units > 0 &&
                       static_cast<int>(blockIdx.x) >= static_cast<int>(gridDim.x) - pa.tail_takers;
    if (!taker) {
      // every workgroup but the takers: one unit, no loop around it
      rows_unit<DK, DV, R, NT, WPE, LM, KT, RB, FUSED, ORDER, VH>(pa, blockIdx.x, false, 0u, nullptr);
      return;
    }
    const unsigned int wrap = static_cast<unsigned int>(pa.tail_units + pa.tail_takers - 1);
    unsigned int claim = 0;
    if (threadIdx.x == 0) claim = atomicInc(pa.turns, wrap);
#if defined(__HIP_DEVICE_COMPILE__)
    // the kernel's one explicit argument opens its argument segment
    typedef const __attribute__((address_space(4))) RowArgs* KArgs;
    KArgs kp = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
#endif
    int vb = blockIdx.x;
    for (int it = 0;; ++it) {
      // each unit reads the arguments afresh (scalar loads of the kernel
      // argument block): nothing is hoisted across units and kept live
      // through the loop (the host pass generates no code for this body)
#if defined(__HIP_DEVICE_COMPILE__)
      asm volatile("" : "+s"(kp));
      const RowArgs a = *kp;
#else
      const RowArgs& a = pa;
#endif
      // the unit is the workgroup's (an SGPR), whatever the compiler makes
      // of the loop around it
      vb = __builtin_amdgcn_readfirstlane(vb);
      const int ib = __builtin_amdgcn_readfirstlane(it) & 1;
      const bool posted = rows_unit<DK, DV, R, NT, WPE, LM, KT, RB, FUSED, ORDER, VH>(
          a, vb, true, claim, &tail_sh[ib]);
      if (!posted && threadIdx.x == 0) tail_sh[ib] = claim;
      // the claim is visible, and the unit's LDS free for the next one
      lds_barrier();
      const unsigned int c = __builtin_amdgcn_readfirstlane(tail_sh[ib]);
      if (c >= static_cast<unsigned int>(pa.tail_units)) return;
      vb = pa.tail_first + static_cast<int>(c);
      if (threadIdx.x == 0) claim = atomicInc(pa.turns, wrap);
    }
  } else {
    rows_unit<DK, DV, R, NT, WPE, LM, KT, RB, FUSED, ORDER, VH>(pa, blockIdx.x, false, 0u, nullptr);
  }
}

template <int DK, int DV, int R, int NT, int WPE, int LM, int KT>
hipError_t launch_typed(const RowArgs& a, hipStream_t s) {
  constexpr int RB = DK == 128 ? GDN_ROWS_RB128 : R;
  constexpr int ORDER = DK == 128 ? GDN_ROWS_ORDER128 : 0;
  const int rows = a.num_rows + (a.more.num_rows > 0 ? a.more.num_rows : 0);
  const unsigned rows8 = static_cast<unsigned>((rows + 7) / 8 * 8);  // whole groups of 8
  int cus = 0;
  if (DK == 128) {
    hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
  }
  // (row, v-head) units whenever the caller passes turn counters (one row
  // set per launch): one workgroup per CU, with the dynamic tail, for rows
  // of two tokens or more on grids of at least four units per CU, several
  // per CU otherwise.  Measured on MI355X (one process, alternating,
  // Qwen3-Next heads; several per CU, no tail, in brackets): K=3, 48 rows
  // 75.9 us (78.8); K=2, 64 rows 74.9 (77.1); K=2, 128 rows 141.3 (144.9);
  // K=3, 32 rows 53.9 (53.8); one token, 256 rows 202.4 (177.1).
  if constexpr (DK == 128 && DV == 128) {
    const unsigned vunits = rows8 * static_cast<unsigned>(a.Hv);
    if (a.turns && a.G > 1 && a.stage == kFused && (GDN_ROWS_VH_MIXED || a.more.num_rows == 0)) {
      constexpr int RV = GDN_ROWS_RV128;
      const Lds lay = lds_layout(DK, DV, 1, a.L, launch_row_tokens(a));
      const bool floor = launch_row_tokens(a) >= GDN_ROWS_VH_FLOOR_TOKENS &&
                         vunits >= GDN_ROWS_VH_FLOOR_UNITS * static_cast<unsigned>(cus);
      const int lds = floor && lay.total < GDN_ROWS_LDS_MIN128 ? GDN_ROWS_LDS_MIN128 : lay.total;
      auto kern = gdn_rows_kernel<DK, DV, RV, NT, GDN_ROWS_WPE_VH128, LM, KT, RV, true, ORDER, true>;
      if (lds > 64 * 1024) {
        hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), lds);
        if (e != hipSuccess) return e;
      }
      // dynamic tail: the last workgroup of each CU (the grid's last
      // `takers`) goes on to claim the last `tail` units at run time
      RowArgs b = a;
      const unsigned takers = static_cast<unsigned>(cus) & ~7u;
      unsigned tail = GDN_ROWS_TAIL_DIV > 0 ? vunits / (GDN_ROWS_TAIL_DIV > 0 ? GDN_ROWS_TAIL_DIV : 1) : 0u;
      tail = (tail < GDN_ROWS_TAIL_ROUNDS * takers ? tail : GDN_ROWS_TAIL_ROUNDS * takers) & ~7u;
      if (floor && tail > 0 && takers > 0 && vunits - tail >= takers) {
        b.tail_units = static_cast<int>(tail);
        b.tail_takers = static_cast<int>(takers);
        b.tail_first = static_cast<int>(vunits - tail);
      }
      hipLaunchKernelGGL(kern, dim3(vunits - static_cast<unsigned>(b.tail_units)), dim3(NT), lds, s, b);
      return hipGetLastError();
    }
  }
  const Lds lay = lds_layout(DK, DV, a.G, a.L, launch_row_tokens(a));
  // units: (row, k-head)
  const unsigned units = rows8 * static_cast<unsigned>(a.Hk);
  const bool one_per_cu = DK == 128 && units > 3u * static_cast<unsigned>(cus);
  const int lds = one_per_cu && lay.total < GDN_ROWS_LDS_MIN128 ? GDN_ROWS_LDS_MIN128 : lay.total;
  auto kern = a.stage == kFused ? gdn_rows_kernel<DK, DV, R, NT, WPE, LM, KT, RB, true, ORDER, false>
                                : gdn_rows_kernel<DK, DV, R, NT, WPE, LM, KT, RB, false, ORDER, false>;
  if (lds > 64 * 1024) {
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(units);
  hipLaunchKernelGGL(kern, grid, dim3(NT), lds, s, a);
  return hipGetLastError();
}

// Short rows on a short ring take the small register gathers.
template <int DK, int DV, int R, int NT, int WPE>
hipError_t launch_sized(const RowArgs& a, hipStream_t s) {
  const int tm = launch_row_tokens(a);
  if (a.L <= 6 && tm <= 4) return launch_typed<DK, DV, R, NT, WPE, 6, 4>(a, s);
  if (a.L <= 8 && tm <= 4) return launch_typed<DK, DV, R, NT, WPE, 8, 4>(a, s);
  return launch_typed<DK, DV, R, NT, WPE, kMaxStateLen, kMaxRowTokens>(a, s);
}

}  // namespace

size_t rows_lds_bytes(const RowArgs& a, int dk, int dv) {
  return static_cast<size_t>(lds_layout(dk, dv, a.G, a.L, launch_row_tokens(a)).total);
}

hipError_t launch_rows(const RowArgs& a, int dk, int dv, hipStream_t s) {
  if (a.num_rows <= 0 && a.more.num_rows <= 0) return hipSuccess;
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 16: return launch_sized<16, 16, 1, 256, 4>(a, s);
    case 32: return launch_sized<32, 32, 1, 256, 4>(a, s);
    case 64: return launch_sized<64, 64, 2, 256, 4>(a, s);
    case 128:
      return launch_sized<128, 128, GDN_ROWS_R128, GDN_ROWS_T128, GDN_ROWS_WPE128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
