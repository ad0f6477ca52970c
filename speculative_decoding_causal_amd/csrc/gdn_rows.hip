// Fused GDN step for short rows (spec-verify rows and one-token decodes).
//
// One workgroup per (row, k-head).  The workgroup owns every conv channel
// that k-head i reads - its q block, its k block and the v blocks of its
// G = Hv/Hk v-heads - so it is the only reader and the only writer of those
// channels of the row's conv slot: the "stage, then roll" contract of
// "[GDN] Spec-decoding-aware attention kernel" ("Changes") holds inside one
// workgroup, with the pre-state staged in LDS before the ring is rewritten.
//
// Phases:
//   1. conv: stage the ring columns and the row's inputs (gathered through
//      token_indx) in LDS, convolve, roll the ring (spec rows: window at
//      n_acc-1, shift n_acc; non-spec rows: ring tail, shift T);
//   2. gates (read at the same global rows, per the gate-gather fix of
//      "[Bugfix] Align Qwen GDN gates with speculative tokens"), q/k L2 norms
//      with wave reductions;
//   3. the recurrence, streaming the G*dv state rows of the k-head's v-heads
//      through VGPRs: each state row of dk floats is spread over dk/16 lanes
//      (16 floats, four float4 each), so row dot products need dk/16-lane DPP
//      sums and every global access moves full 128-byte lines.  The state of
//      each token is stored to its slot (spec) or only the final one
//      (non-spec).  The initial-state load precedes every store of the row.
//   4. outputs remapped through token_indx, as bf16.
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
};

__device__ __forceinline__ int slot_or_null(int s, int num_slots) {
  return (s > 0 && s < num_slots) ? s : 0;
}

__device__ RowPlan plan_row(const RowArgs& p, int row) {
  RowPlan r;
  int j0 = clampi(p.qsl[row], 0, p.num_tokens);
  int j1 = clampi(p.qsl[row + 1], j0, p.num_tokens);
  r.j0 = j0;
  r.T = min(j1 - j0, p.max_row_tokens);
  const int L = p.L, W = p.W;
  if (p.kind == kSpec) {
    const int* ssi = p.ssi + (size_t)row * p.row_stride;
    int T = r.T > 0 ? r.T : 1;
    // n_acc outside [1, min(T, L-W+2)] is a precondition violation; clamp so
    // every access stays inside the slot.
    const int nacc = p.nacc[row];
    const int n = clampi(nacc, 1, min(T, L - W + 2));
    r.conv_slot = slot_or_null(p.cache_idx ? p.cache_idx[row] : ssi[0], p.num_slots);
    r.read_hist = true;
    r.off = n - 1;
    r.shift = n;
    r.load_slot = slot_or_null(ssi[clampi(nacc, 1, T) - 1], p.num_slots);
  } else {
    int c = slot_or_null(p.cache_idx[row], p.num_slots);
    bool init = (p.his ? p.his[row] != 0 : true) && c > 0;
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
  int kq;            // float [Tm]
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
  l.kq = o;     o += align16(Tm * 4);
  l.zb = o;     o += align16((L + Tm) * NCH * 2);
  l.total = o;
  return l;
}

typedef float v4f __attribute__((ext_vector_type(4)));

template <int DK, int DV, int R>
__global__ void __launch_bounds__(kThreads)
gdn_rows_kernel(RowArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int LPR = DK / 16;    // lanes per state row
  constexpr int RPW = 64 / LPR;   // state rows per wave per sub-pass
  static_assert(DK % 64 == 0 || DK == 16 || DK == 32, "dk");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int Hk = p.Hk, G = p.G, C = p.C, L = p.L, W = p.W;
  const int row = blockIdx.x / Hk;
  const int ih = blockIdx.x - row * Hk;
  const int NCH = 2 * DK + G * DV;
  const int NR = G * DV;
  const int Tm = p.max_row_tokens;

  const RowPlan rp = plan_row(p, row);
  const int T = rp.T;
  if (T <= 0) return;

  const Lds lay = lds_layout(DK, DV, G, L, Tm);
  int* rows_s = reinterpret_cast<int*>(smem + lay.rows);
  int* st_s = reinterpret_cast<int*>(smem + lay.stores);
  float* qs = reinterpret_cast<float*>(smem + lay.qs);
  float* ks = reinterpret_cast<float*>(smem + lay.ks);
  float* vs = reinterpret_cast<float*>(smem + lay.vs);
  float* ob = reinterpret_cast<float*>(smem + lay.ob);
  float* ga = reinterpret_cast<float*>(smem + lay.ga);
  float* gb = reinterpret_cast<float*>(smem + lay.gb);
  float* kq = reinterpret_cast<float*>(smem + lay.kq);
  uint16_t* zb = reinterpret_cast<uint16_t*>(smem + lay.zb);

  if (tid < T) {
    int r = p.tix ? p.tix[rp.j0 + tid] : rp.j0 + tid;
    rows_s[tid] = (r >= 0 && r < p.num_actual_tokens) ? r : -1;
    int st;
    if (p.kind == kSpec)
      st = slot_or_null(p.ssi[(size_t)row * p.row_stride + tid], p.num_slots);
    else
      st = (tid == T - 1) ? rp.conv_slot : 0;
    st_s[tid] = st;
  }
  __syncthreads();

  // ---- phase 1: conv (or load of a precomputed conv output) -------------
  const int stage = p.stage;
  for (int pc = tid; pc < NCH; pc += kThreads) {
    int c;
    if (pc < DK) c = ih * DK + pc;
    else if (pc < 2 * DK) c = Hk * DK + ih * DK + (pc - DK);
    else c = 2 * Hk * DK + ih * NR + (pc - 2 * DK);
    float* dst;
    int dstride;
    if (pc < DK) { dst = qs + pc; dstride = DK; }
    else if (pc < 2 * DK) { dst = ks + (pc - DK); dstride = DK; }
    else { dst = vs + (pc - 2 * DK); dstride = NR; }

    if (stage == kDeltaOnly) {
      for (int j = 0; j < T; ++j) {
        int r = rows_s[j];
        dst[j * dstride] = r >= 0 ? p.y[(size_t)r * C + c] : 0.f;
      }
      continue;
    }
    const bool hist = rp.read_hist && rp.conv_slot > 0;
    const uint16_t* ring = p.conv_pool + (size_t)rp.conv_slot * L * C + c;
    for (int l = 0; l < L; ++l) zb[l * NCH + pc] = hist ? ring[(size_t)l * C] : 0;
    for (int j = 0; j < T; ++j) {
      int r = rows_s[j];
      zb[(L + j) * NCH + pc] = r >= 0 ? p.qkv[(size_t)r * C + c] : 0;
    }
    float w[kMaxWidth];
#pragma unroll
    for (int m = 0; m < kMaxWidth; ++m) w[m] = m < W ? bf2f(p.conv_w[(size_t)c * W + m]) : 0.f;
    const float bias = p.conv_b ? bf2f(p.conv_b[c]) : 0.f;
    for (int j = 0; j < T; ++j) {
      float acc = bias;
#pragma unroll
      for (int m = 0; m < kMaxWidth; ++m) {
        if (m < W) {
          int idx = j + m;
          int zi = idx < W - 1 ? rp.off + idx : L + idx - (W - 1);
          acc = fmaf(w[m], bf2f(zb[zi * NCH + pc]), acc);
        }
      }
      if (p.act) acc = silu(acc);
      if (stage == kConvOnly) {
        int r = rows_s[j];
        if (r >= 0) p.y[(size_t)r * C + c] = acc;
      } else {
        dst[j * dstride] = acc;
      }
    }
    if (rp.conv_slot > 0) {
      uint16_t* wring = p.conv_pool + (size_t)rp.conv_slot * L * C + c;
      for (int l = 0; l < L; ++l) {
        int src = l < L - T ? rp.shift + l : T + l;
        wring[(size_t)l * C] = zb[src * NCH + pc];
      }
    }
  }
  if (stage == kConvOnly) return;

  // ---- phase 2: gates and q/k norms ---------------------------------------
  for (int idx = tid; idx < T * G; idx += kThreads) {
    int j = idx / G, g = idx - j * G, h = ih * G + g;
    int r = rows_s[j];
    float av = r >= 0 ? bf2f(p.a[(size_t)r * p.Hv + h]) : 0.f;
    float bv = r >= 0 ? bf2f(p.b[(size_t)r * p.Hv + h]) : 0.f;
    gate_pair(av, bv, p.A_log[h], p.dt_bias[h], &ga[idx], &gb[idx]);
  }
  __syncthreads();
  for (int j = wv; j < T; j += kThreads / 64) {
    float sq = 0.f, sk = 0.f;
    for (int c = lane; c < DK; c += 64) {
      float q = qs[j * DK + c], k = ks[j * DK + c];
      sq = fmaf(q, q, sq);
      sk = fmaf(k, k, sk);
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    float iq = p.l2norm ? 1.f / sqrtf(sq + p.eps) : 1.f;
    float ik = p.l2norm ? 1.f / sqrtf(sk + p.eps) : 1.f;
    float dot = 0.f;
    for (int c = lane; c < DK; c += 64) {
      float q = qs[j * DK + c] * iq * p.scale;
      float k = ks[j * DK + c] * ik;
      qs[j * DK + c] = q;
      ks[j * DK + c] = k;
      dot = fmaf(k, q, dot);
    }
    dot = wave_sum(dot);
    if (lane == 0) kq[j] = dot;
  }
  __syncthreads();

  // ---- phase 3: recurrence over the state rows -----------------------------
  const int jl = lane % LPR, gl = lane / LPR;
  const size_t slot_stride = (size_t)p.Hv * DV * DK;
  const size_t head_off = (size_t)ih * NR * DK;
  for (int r0 = wv * RPW * R; r0 < NR; r0 += (kThreads / 64) * RPW * R) {
    v4f S[R][4];
    int rho[R];
#pragma unroll
    for (int s = 0; s < R; ++s) rho[s] = r0 + s * RPW + gl;
    if (rp.load_slot > 0) {
      const float* base = p.ssm_pool + (size_t)rp.load_slot * slot_stride + head_off;
#pragma unroll
      for (int s = 0; s < R; ++s)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          S[s][n] = rho[s] < NR
                        ? *reinterpret_cast<const v4f*>(base + (size_t)rho[s] * DK + (n * LPR + jl) * 4)
                        : v4f{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int s = 0; s < R; ++s)
#pragma unroll
        for (int n = 0; n < 4; ++n) S[s][n] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    for (int j = 0; j < T; ++j) {
      v4f kv[4], qv[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        kv[n] = *reinterpret_cast<const v4f*>(ks + j * DK + (n * LPR + jl) * 4);
        qv[n] = *reinterpret_cast<const v4f*>(qs + j * DK + (n * LPR + jl) * 4);
      }
      float pk[R], pq[R];
#pragma unroll
      for (int s = 0; s < R; ++s) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          a0 = fmaf(S[s][n].x, kv[n].x, a0); a1 = fmaf(S[s][n].x, qv[n].x, a1);
          a0 = fmaf(S[s][n].y, kv[n].y, a0); a1 = fmaf(S[s][n].y, qv[n].y, a1);
          a0 = fmaf(S[s][n].z, kv[n].z, a0); a1 = fmaf(S[s][n].z, qv[n].z, a1);
          a0 = fmaf(S[s][n].w, kv[n].w, a0); a1 = fmaf(S[s][n].w, qv[n].w, a1);
        }
        pk[s] = group_sum<LPR>(a0);
        pq[s] = group_sum<LPR>(a1);
      }
      const float kqj = kq[j];
#pragma unroll
      for (int s = 0; s < R; ++s) {
        const int rr = rho[s] < NR ? rho[s] : NR - 1;
        const int g = rr / DV;
        const float al = ga[j * G + g], be = gb[j * G + g];
        const float vr = vs[j * NR + rr];
        // S_new = al S + u k^T with u = be (v - al S k); o = S_new q.
        const float u = be * (vr - al * pk[s]);
        const float o = fmaf(al, pq[s], u * kqj);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          S[s][n].x = fmaf(u, kv[n].x, al * S[s][n].x);
          S[s][n].y = fmaf(u, kv[n].y, al * S[s][n].y);
          S[s][n].z = fmaf(u, kv[n].z, al * S[s][n].z);
          S[s][n].w = fmaf(u, kv[n].w, al * S[s][n].w);
        }
        if (jl == 0 && rho[s] < NR) ob[j * NR + rho[s]] = o;
      }
      const int st = st_s[j];
      if (st > 0) {
        float* base = p.ssm_pool + (size_t)st * slot_stride + head_off;
#pragma unroll
        for (int s = 0; s < R; ++s)
          if (rho[s] < NR)
#pragma unroll
            for (int n = 0; n < 4; ++n)
              __builtin_nontemporal_store(
                  S[s][n], reinterpret_cast<v4f*>(base + (size_t)rho[s] * DK + (n * LPR + jl) * 4));
      }
    }
  }
  __syncthreads();

  // ---- phase 4: outputs ----------------------------------------------------
  uint16_t* out = p.out;
  for (int idx = tid; idx < T * NR; idx += kThreads) {
    int j = idx / NR, rr = idx - j * NR;
    int r = rows_s[j];
    if (r >= 0) out[((size_t)r * p.Hv + ih * G) * DV + rr] = f2bf(ob[idx]);
  }
}

template <int DK, int DV, int R>
hipError_t launch_typed(const RowArgs& a, hipStream_t s) {
  const Lds lay = lds_layout(DK, DV, a.G, a.L, a.max_row_tokens);
  auto kern = gdn_rows_kernel<DK, DV, R>;
  if (lay.total > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       lay.total);
    if (e != hipSuccess) return e;
  }
  dim3 grid(static_cast<unsigned>(a.num_rows) * static_cast<unsigned>(a.Hk));
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lay.total, s, a);
  return hipGetLastError();
}

}  // namespace

size_t rows_lds_bytes(const RowArgs& a, int dk, int dv) {
  return static_cast<size_t>(lds_layout(dk, dv, a.G, a.L, a.max_row_tokens).total);
}

hipError_t launch_rows(const RowArgs& a, int dk, int dv, hipStream_t s) {
  if (a.num_rows <= 0) return hipSuccess;
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 16: return launch_typed<16, 16, 1>(a, s);
    case 32: return launch_typed<32, 32, 1>(a, s);
    case 64: return launch_typed<64, 64, 2>(a, s);
    case 128: return launch_typed<128, 128, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
