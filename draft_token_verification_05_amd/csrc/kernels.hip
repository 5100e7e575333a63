// gfx950 kernels of the speculative-decoding verify step.
//
// Three launches per call:
//   k_prep      one workgroup: exclusive scans of gamma (packed offsets), the
//               row -> request maps, counter reset, layout validation.
//   k_rowstats  one workgroup per (task, vocabulary chunk).  A task is a
//               (target row, draft row) pair (stochastic / NKL) or a single
//               target row (greedy / tree / NKL bonus row).  Each workgroup
//               streams its chunk with 16-byte loads and reduces it to
//               (max, sum exp, argmax, KL cross term); the last workgroup of a
//               task merges the chunk partials, and the last task of a request
//               runs the per-request decision (first-reject scan, tree
//               resolve) and writes the outputs.
//   k_draw      stochastic mode only: one workgroup per (request, chunk) of
//               the terminal row; float64 chunk sums of the residual
//               max(0, p - q) (or of p for a bonus token); the last workgroup
//               of a request selects the chunk and draws the token by a
//               block-wide prefix sum.
//
// Formulas follow these passages:
//   softmax(logits / T), p(x), q(x)     -- "Chain of Draft" page, section 3.2
//                                          (compute_nkl); "投机采样" page,
//                                          verification loop of the engine.
//   alpha = min(1, p/q), accept u<=alpha,
//   redraw from max(0, p-q)/norm        -- "投机采样" page, section 核心算法数学原理.
//   greedy accept d_i == argmax P_i     -- Gemma-4 MTP page, section 2.3.
//   NKL = KL(q||p) / ln V, accept < delta -- "Chain of Draft" page, section 3.2.
//   tree drafts, longest accepted path   -- "Parallel Drafting" page, section 2.2;
//                                          Gemma-4 MTP page, section 6.2.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cstdint>

#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr double kLog2eD = 1.44269504088896340736;
constexpr float kLn2 = 0.693147180559945309417f;

// ----------------------------------------------------------------------------
// element access
// ----------------------------------------------------------------------------

template <int DT>
struct Elem;
template <>
struct Elem<SV_DTYPE_BF16> {
  static constexpr int P = 8;
  static constexpr uint32_t kPadPair = 0xFF7FFF7Fu;  // two bf16 -3.39e38 (pad for positions >= V)
  static constexpr float kPad = -3.38953139e38f;      // the pad's value (bf16 0xFF7F)
};
template <>
struct Elem<SV_DTYPE_F32> {
  static constexpr int P = 4;
  static constexpr uint32_t kPadPair = 0xFF7FFFFFu;  // -FLT_MAX
  static constexpr float kPad = -FLT_MAX;
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Raw 16 bytes holding elements [e0, e0 + P) of `row`; positions >= V hold the
// pad pattern.  VEC: rows are 16-byte aligned, so full vectors use one load.
template <int DT, bool VEC>
__device__ __forceinline__ uint4 fetch(const void* base, int64_t row, int64_t V, int64_t e0) {
  constexpr int P = Elem<DT>::P;
  if (VEC && e0 + P <= V) {
    const char* ptr = static_cast<const char*>(base) + (row * V + e0) * (DT == SV_DTYPE_BF16 ? 2 : 4);
    return *reinterpret_cast<const uint4*>(ptr);
  }
  uint32_t w[4] = {Elem<DT>::kPadPair, Elem<DT>::kPadPair, Elem<DT>::kPadPair, Elem<DT>::kPadPair};
  if (DT == SV_DTYPE_BF16) {
    const uint16_t* r = static_cast<const uint16_t*>(base) + row * V;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e0 + e < V) {
        const uint32_t h = r[e0 + e];
        const int sh = (e & 1) * 16;
        w[e >> 1] = (w[e >> 1] & ~(0xFFFFu << sh)) | (h << sh);
      }
    }
  } else {
    const uint32_t* r = static_cast<const uint32_t*>(base) + row * V;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e0 + e < V) w[e] = r[e0 + e];
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int DT>
__device__ __forceinline__ void unpack(const uint4& q, float* v) {
  if (DT == SV_DTYPE_BF16) {
    v[0] = bf_lo(q.x); v[1] = bf_hi(q.x); v[2] = bf_lo(q.y); v[3] = bf_hi(q.y);
    v[4] = bf_lo(q.z); v[5] = bf_hi(q.z); v[6] = bf_lo(q.w); v[7] = bf_hi(q.w);
  } else {
    v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
    v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
  }
}

template <int DT>
__device__ __forceinline__ float load_scalar(const void* base, int64_t row, int64_t V, int64_t y) {
  if (DT == SV_DTYPE_BF16) return __uint_as_float((uint32_t)(static_cast<const uint16_t*>(base)[row * V + y]) << 16);
  return static_cast<const float*>(base)[row * V + y];
}

// ----------------------------------------------------------------------------
// wave64 reductions (DPP within rows of 16 lanes, then the four row results).
// Every lane of the wave must be active.  Deterministic: the combination
// order is fixed by lane position.
// ----------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v, int old) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float lanef(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v, v));   // quad_perm(1,0,3,2)
  v = fmaxf(v, dpp<0x4E>(v, v));   // quad_perm(2,3,0,1)
  v = fmaxf(v, dpp<0x124>(v, v));  // row_ror:4
  v = fmaxf(v, dpp<0x128>(v, v));  // row_ror:8
  return fmaxf(fmaxf(lanef(v, 0), lanef(v, 16)), fmaxf(lanef(v, 32), lanef(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp<0xB1>(v, 0.f);
  v = v + dpp<0x4E>(v, 0.f);
  v = v + dpp<0x124>(v, 0.f);
  v = v + dpp<0x128>(v, 0.f);
  return (lanef(v, 0) + lanef(v, 16)) + (lanef(v, 32) + lanef(v, 48));
}
__device__ __forceinline__ int wave_min_int(int v) {
  v = min(v, dppi<0xB1>(v, v));
  v = min(v, dppi<0x4E>(v, v));
  v = min(v, dppi<0x124>(v, v));
  v = min(v, dppi<0x128>(v, v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_max_int(int v) {
  v = max(v, dppi<0xB1>(v, v));
  v = max(v, dppi<0x4E>(v, v));
  v = max(v, dppi<0x124>(v, v));
  v = max(v, dppi<0x128>(v, v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// butterfly sum: every lane ends with the same bits (a + b == b + a in IEEE)
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// workgroup-wide reductions through LDS (all threads must call)
__device__ __forceinline__ int block_min_int(int v, int* sh) {
  v = wave_min_int(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  int r = sh[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = min(r, sh[k]);
  return r;
}
__device__ __forceinline__ int block_max_int(int v, int* sh) {
  v = wave_max_int(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  int r = sh[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = max(r, sh[k]);
  return r;
}
__device__ __forceinline__ float block_max(float v, float* sh) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = fmaxf(r, sh[k]);
  return r;
}
__device__ __forceinline__ double block_sum_d(double v, double* sh) {
  v = wave_sum_d(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  double r = sh[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r += sh[k];
  return r;
}

// exclusive prefix sum over the workgroup's threads in float64; returns the
// exclusive prefix of this thread, `total` receives the sum.
__device__ __forceinline__ double block_exclusive_scan_d(double v, double* sh, double& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  __syncthreads();
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  double before = 0.0;
  for (int k = 0; k < w; ++k) before += sh[k];
  double tot = 0.0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) tot += sh[k];
  total = tot;
  return before + incl - v;
}

__device__ __forceinline__ bool unit_ok(float u) { return u >= 0.0f && u < 1.0f; }
__device__ __forceinline__ bool temp_ok(float t) { return t > 0.0f && t <= FLT_MAX; }

// exp((x - m) / T) = exp2(dx * L), L = log2(e)/T split as Lhi + Llo (float32);
// the rounding error of dx*Lhi is recovered exactly by an fma, so the
// exponent carries no systematic rounding (no effective temperature shift).
__device__ __forceinline__ float exp_hp(float dx, float Lhi, float Llo) {
  const float p1 = dx * Lhi;
  const float err = fmaf(dx, Lhi, -p1);
  const float corr = fmaf(dx, Llo, err);
  const float E = __builtin_amdgcn_exp2f(p1);
  const float e = fmaf(E * kLn2, corr, E);
  return p1 >= -160.0f ? e : 0.0f;
}

// ----------------------------------------------------------------------------
// k_prep
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(kPrepThreads) void k_prep(Params p) {
  __shared__ long long sh_w[kPrepThreads / 64];
  __shared__ int sh_bad;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  long long carry = 0;  // 64-bit: a bogus gamma cannot wrap the sum around
  for (int base = 0; base < p.B; base += kPrepThreads) {
    const int b = base + tid;
    long long g = 0;
    if (b < p.B) {
      g = p.gamma[b];
      if (g < 0) {
        sh_bad = 1;  // benign race: every writer stores 1
        g = 0;
      }
    }
    long long incl = g;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) sh_w[w] = incl;
    __syncthreads();
    long long before = 0, tile = 0;
    for (int k = 0; k < kPrepThreads / 64; ++k) {
      if (k < w) before += sh_w[k];
      tile += sh_w[k];
    }
    if (b < p.B) {
      const long long excl = carry + before + incl - g;
      // values are only used when the whole layout checks out (sum == R_d < 2^31)
      p.d_off[b] = (int)excl;
      p.t_off[b] = (int)(excl + b);
    }
    carry += tile;
    __syncthreads();
  }
  if (tid == 0) {
    p.d_off[p.B] = (int)carry;
    p.t_off[p.B] = (int)(carry + p.B);
  }
  const bool bad = sh_bad != 0 || carry != (long long)p.R_d;
  if (tid == 0) p.hdr[0] = bad ? 1 : 0;
  if (bad) {
    for (int b = tid; b < p.B; b += kPrepThreads) p.out_num[b] = -1;
    return;
  }
  for (int i = tid; i < p.n_task; i += kPrepThreads) p.cnt_task[i] = 0u;
  for (int b = tid; b < p.B; b += kPrepThreads) {
    p.cnt_req[b] = 0u;
    p.cnt_draw[b] = 0u;
  }
  __syncthreads();  // offsets written by other threads of this workgroup
  for (int b = tid; b < p.B; b += kPrepThreads) {
    const int g = p.gamma[b], d0 = p.d_off[b], t0 = p.t_off[b];
    for (int k = 0; k < g; ++k) p.pair2req[d0 + k] = b;
    for (int k = 0; k <= g; ++k) p.row2req[t0 + k] = b;
  }
}

// ----------------------------------------------------------------------------
// per-request decisions (run by the workgroup that completes a request's last
// task; every thread of the workgroup calls them)
// ----------------------------------------------------------------------------

struct DecideShared {
  int i[kWaves];
  int bad;
};

__device__ void finish_invalid(const Params& p, int b, int t0, int g) {
  for (int k = threadIdx.x; k <= g; k += kThreads) p.out_tokens[t0 + k] = -1;
  if (threadIdx.x == 0) {
    p.out_num[b] = -1;
    if (p.out_resid) p.out_resid[b] = __builtin_nanf("");
    if (p.out_tree_node) p.out_tree_node[b] = -1;
  }
}

// NKL = KL(q || p) / ln V.  The KL comes from the task's merged statistics:
// KL = (W/s_d - (m_d - m_t)) / T - log(s_d / s_t), W = sum e^{(d-m_d)/T} (d - t),
// or from the second pass when that form loses too much to cancellation.
// With a single token both distributions are the same point mass: NKL = 0.
__device__ __forceinline__ float nkl_of(const TaskStat& s, int V) { return V > 1 ? s.kl / logf((float)V) : 0.0f; }

__device__ void decide_stochastic(const Params& p, int b, DecideShared& sh) {
  const int g = p.gamma[b], t0 = p.t_off[b], d0 = p.d_off[b];
  const float T = p.temp[b];
  bool bad = !(g <= p.max_gamma) || !temp_ok(T) || !unit_ok(p.ur[b]);
  int first = INT_MAX;
  for (int i = threadIdx.x; i < g; i += kThreads) {
    const int x = p.tokens[d0 + i];
    const float u = p.ua[d0 + i];
    if (x < 0 || x >= p.V || !unit_ok(u)) {
      bad = true;
      continue;
    }
    const TaskStat s = p.stat[d0 + i];
    const float tx = p.gat[2 * (d0 + i)], dx = p.gat[2 * (d0 + i) + 1];
    // log p(x) - log q(x) = ((t_x - m_t) - (d_x - m_d)) / T + log(s_d / s_t)
    const float lr = ((tx - s.m_t) - (dx - s.m_d)) / T + (float)log(s.s_d / s.s_t);
    const float alpha = fminf(1.0f, expf(lr));
    if (!(u <= alpha)) first = min(first, i);
    if (p.out_p_x) p.out_p_x[d0 + i] = (float)((double)expf((tx - s.m_t) / T) / s.s_t);
    if (p.out_q_x) p.out_q_x[d0 + i] = (float)((double)expf((dx - s.m_d) / T) / s.s_d);
    if (p.out_nkl) p.out_nkl[d0 + i] = nkl_of(s, p.V);
  }
  if (threadIdx.x == 0) sh.bad = 0;
  __syncthreads();
  if (bad) sh.bad = 1;
  const int j0 = block_min_int(first, sh.i);  // contains barriers
  const int j = j0 == INT_MAX ? g : j0;
  if (sh.bad) {
    finish_invalid(p, b, t0, g);
    if (threadIdx.x == 0) p.term[b].kind = kTermNone;
    return;
  }
  for (int k = threadIdx.x; k <= g; k += kThreads)
    if (k != j) p.out_tokens[t0 + k] = k < j ? p.tokens[d0 + k] : -1;
  if (threadIdx.x == 0) {
    p.out_num[b] = j;
    Term tm;
    tm.j = j;
    tm.trow = t0 + j;
    tm.pad = 0;
    if (j < g) {
      const TaskStat s = p.stat[d0 + j];
      tm.kind = kTermResidual;
      tm.drow = d0 + j;
      tm.m_t = s.m_t;
      tm.m_d = s.m_d;
      tm.k0 = (float)(s.s_t / s.s_d);
    } else {
      tm.kind = kTermBonus;
      tm.drow = -1;
      tm.m_t = tm.m_d = tm.k0 = 0.0f;
    }
    p.term[b] = tm;
  }
}

// greedy (mode 1) and NKL (mode 2)
template <int MODE>
__device__ void decide_argmax_chain(const Params& p, int b, DecideShared& sh) {
  const int g = p.gamma[b], t0 = p.t_off[b], d0 = p.d_off[b];
  bool bad = !(g <= p.max_gamma);
  float T = 1.0f;
  if (MODE == SV_MODE_NKL) {
    T = p.temp[b];
    bad = bad || !temp_ok(T);
  }
  int first = INT_MAX;
  for (int i = threadIdx.x; i < g; i += kThreads) {
    const int x = p.tokens[d0 + i];
    if (x < 0 || x >= p.V) {
      bad = true;
      continue;
    }
    bool acc;
    if (MODE == SV_MODE_GREEDY) {
      acc = (x == p.stat[t0 + i].idx);
    } else {
      const TaskStat s = p.stat[d0 + i];
      const float nkl = nkl_of(s, p.V);
      p.out_nkl[d0 + i] = nkl;
      if (p.out_p_x || p.out_q_x) {
        const float tx = p.gat[2 * (d0 + i)], dx = p.gat[2 * (d0 + i) + 1];
        if (p.out_p_x) p.out_p_x[d0 + i] = (float)((double)expf((tx - s.m_t) / T) / s.s_t);
        if (p.out_q_x) p.out_q_x[d0 + i] = (float)((double)expf((dx - s.m_d) / T) / s.s_d);
      }
      acc = nkl < p.delta;
    }
    if (!acc) first = min(first, i);
  }
  if (threadIdx.x == 0) sh.bad = 0;
  __syncthreads();
  if (bad) sh.bad = 1;
  const int j0 = block_min_int(first, sh.i);
  const int j = j0 == INT_MAX ? g : j0;
  if (sh.bad) {
    finish_invalid(p, b, t0, g);
    return;
  }
  int term_tok;
  if (MODE == SV_MODE_GREEDY)
    term_tok = p.stat[t0 + j].idx;
  else
    term_tok = j < g ? p.stat[d0 + j].idx : p.stat[p.R_d + b].idx;
  for (int k = threadIdx.x; k <= g; k += kThreads)
    p.out_tokens[t0 + k] = k < j ? p.tokens[d0 + k] : (k == j ? term_tok : -1);
  if (threadIdx.x == 0) p.out_num[b] = j;
}

// Tree resolve.  node_info[n] packs (depth << 1) | accepted; parents precede
// children, so one ordered pass settles every node.
__device__ void decide_tree(const Params& p, int b, DecideShared& sh, int16_t* node_info, int16_t* par) {
  const int g = p.gamma[b], t0 = p.t_off[b], d0 = p.d_off[b];
  const int N = g + 1;
  bool bad = !(g <= p.max_gamma);
  if (threadIdx.x == 0) sh.bad = 0;
  __syncthreads();
  if (!bad) {
    for (int n = 1 + threadIdx.x; n < N; n += kThreads) {
      const int pa = p.parents[d0 + n - 1];
      const int x = p.tokens[d0 + n - 1];
      if (pa < 0 || pa >= n || x < 0 || x >= p.V) {
        bad = true;
        continue;
      }
      par[n] = (int16_t)pa;
      node_info[n] = (int16_t)((x == p.stat[t0 + pa].idx) ? 1 : 0);  // edge match, before ancestry
    }
  }
  if (bad) sh.bad = 1;
  __syncthreads();
  if (sh.bad) {
    finish_invalid(p, b, t0, g);
    return;
  }
  if (threadIdx.x == 0) {
    node_info[0] = 1;  // root: depth 0, accepted
    for (int n = 1; n < N; ++n) {
      const int pi = node_info[par[n]];
      node_info[n] = (int16_t)((((pi >> 1) + 1) << 1) | (pi & node_info[n] & 1));
    }
  }
  __syncthreads();
  // deepest accepted node, lowest id on ties
  int key = -1;
  for (int n = threadIdx.x; n < N; n += kThreads) {
    const int ni = node_info[n];
    if (ni & 1) key = max(key, ((ni >> 1) << 13) | (8191 - n));
  }
  const int best_key = block_max_int(key, sh.i);
  const int best = 8191 - (best_key & 8191);
  const int depth = best_key >> 13;
  for (int k = depth + 1 + threadIdx.x; k <= g; k += kThreads) p.out_tokens[t0 + k] = -1;
  if (threadIdx.x == 0) {
    for (int v = best; v != 0; v = par[v]) p.out_tokens[t0 + (node_info[v] >> 1) - 1] = p.tokens[d0 + v - 1];
    p.out_tokens[t0 + depth] = p.stat[t0 + best].idx;
    p.out_num[b] = depth;
    if (p.out_tree_node) p.out_tree_node[b] = best;
  }
}

// ----------------------------------------------------------------------------
// k_rowstats
// ----------------------------------------------------------------------------

struct RowShared {
  float m[2][kWaves];
  float s[2][kWaves];
  float w[kWaves];
  int i[kWaves];
  double d[2 + kWaves];
  int last_chunk;  // this workgroup completed the task
  int last_task;   // ... and the request
  int refine;
  DecideShared dec;
};

// g(w) = e^w - 1 - w >= 0, accurate for small |w| (Taylor series to w^9)
__device__ __forceinline__ float g_small(float w) {
  float t = fmaf(w, 1.0f / 362880.0f, 1.0f / 40320.0f);
  t = fmaf(w, t, 1.0f / 5040.0f);
  t = fmaf(w, t, 1.0f / 720.0f);
  t = fmaf(w, t, 1.0f / 120.0f);
  t = fmaf(w, t, 1.0f / 24.0f);
  t = fmaf(w, t, 1.0f / 6.0f);
  t = fmaf(w, t, 0.5f);
  return w * w * t;
}

// KL(q || p) of one row pair in a second pass, written as the sum of the
// non-negative terms q_y * g(w_y), w_y = log(p_y / q_y).  Because
// sum q e^w = sum p = 1, this equals sum q log(q/p) exactly, has no
// cancellation, and an error eps in the log normaliser ratio only adds
// g(eps) = O(eps^2).  Run by all threads of one workgroup.
template <int DT, bool VEC>
__device__ double kl_second_pass(const Params& p, int trow, int drow, float m_t, float m_d, double s_t, double s_d,
                                 float T, float Lhi, double* shd) {
  constexpr int P = Elem<DT>::P;
  constexpr int U = 4;
  const int64_t V = p.V;
  const float invT = (float)(1.0 / (double)T);
  const float lr = (float)log(s_d / s_t);
  const float inv_sd = (float)(1.0 / s_d), inv_st = (float)(1.0 / s_t);
  double acc = 0.0;
  for (int64_t base = 0; base < V; base += (int64_t)kThreads * P * U) {
    uint4 qt[U], qd[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t e0 = base + ((int64_t)k * kThreads + threadIdx.x) * P;
      qt[k] = fetch<DT, VEC>(p.target, trow, V, e0);
      qd[k] = fetch<DT, VEC>(p.draft, drow, V, e0);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      float vt[P], vd[P];
      unpack<DT>(qt[k], vt);
      unpack<DT>(qd[k], vd);
      float part = 0.f;  // P non-negative terms in float32, then float64
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const float dt = vt[e] - m_t, dd = vd[e] - m_d;
        const float q = __builtin_amdgcn_exp2f(dd * Lhi) * inv_sd;
        const float w = fmaf(dt - dd, invT, lr);
        float term;
        if (fabsf(w) < 0.5f) {
          term = q * g_small(w);
        } else {
          // q g(w) = p - q - q w; also right where q underflows but p does not
          const float pp = __builtin_amdgcn_exp2f(dt * Lhi) * inv_st;
          term = (pp - q) - q * w;
        }
        part += term;  // positions past the end of the row give p = q = 0
      }
      acc += (double)part;
    }
  }
  return block_sum_d(acc, shd);
}

template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void k_rowstats(Params p) {
  constexpr int P = Elem<DT>::P;
  constexpr int NE = kUA * P;  // elements per thread per row
  __shared__ RowShared sh;
  // tree resolve scratch exists in the tree-mode kernel only
  __shared__ int16_t tree_info[MODE == SV_MODE_TREE_GREEDY ? SV_MAX_GAMMA + 1 : 1];
  __shared__ int16_t tree_par[MODE == SV_MODE_TREE_GREEDY ? SV_MAX_GAMMA + 1 : 1];

  if (p.hdr[0] != 0) return;  // layout error (found by k_prep)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int item = blockIdx.x;
  const int task = item / p.nch_a;
  const int chunk = item - task * p.nch_a;
  const int64_t V = p.V;

  // task -> (request, target row, draft row)
  int b, trow, drow;
  bool pair;
  if (MODE == SV_MODE_STOCHASTIC || (MODE == SV_MODE_NKL && task < p.R_d)) {
    b = p.pair2req[task];
    trow = task + b;
    drow = task;
    pair = true;
  } else if (MODE == SV_MODE_NKL) {
    b = task - p.R_d;
    trow = p.d_off[b + 1] + b;  // t_off[b] + gamma_b: the bonus row
    drow = -1;
    pair = false;
  } else {
    b = p.row2req[task];
    trow = task;
    drow = -1;
    pair = false;
  }
  const bool want_idx = MODE != SV_MODE_STOCHASTIC;
  const bool want_soft = pair;
  const bool want_w = pair && p.want_w;

  // issue the loads
  const int64_t e_chunk = (int64_t)chunk * (kThreads * NE);
  uint4 qt[kUA], qd[kUA];
#pragma unroll
  for (int k = 0; k < kUA; ++k) qt[k] = fetch<DT, VEC>(p.target, trow, V, e_chunk + ((int64_t)k * kThreads + tid) * P);
  if (pair) {
#pragma unroll
    for (int k = 0; k < kUA; ++k) qd[k] = fetch<DT, VEC>(p.draft, drow, V, e_chunk + ((int64_t)k * kThreads + tid) * P);
  }
  // exp((x - m)/T) = exp2((x - m) * L), L = log2(e)/T = Lhi + Llo
  float T = 1.0f, Lhi = 0.0f, Llo = 0.0f;
  if (want_soft) {
    T = p.temp[b];
    const double Ld = kLog2eD / (double)T;
    Lhi = (float)Ld;
    Llo = (float)(Ld - (double)Lhi);
  }
  // gather of the logits at the drafted token (one workgroup per pair holds it)
  float gx_t = 0.f, gx_d = 0.f;
  bool gathered = false;
  if (pair && tid == 0) {
    const int x = p.tokens[drow];
    if (x >= e_chunk && x < e_chunk + (int64_t)kThreads * NE && x < V && x >= 0) {
      gx_t = load_scalar<DT>(p.target, trow, V, x);
      gx_d = load_scalar<DT>(p.draft, drow, V, x);
      gathered = true;
    }
  }

  // ---- target row: max, argmax, sum exp (exponent from the exact difference x - m)
  float vt[NE];
#pragma unroll
  for (int k = 0; k < kUA; ++k) unpack<DT>(qt[k], vt + k * P);
  float mt = vt[0];
#pragma unroll
  for (int e = 1; e < NE; ++e) mt = fmaxf(mt, vt[e]);
  int it = INT_MAX;
  if (want_idx) {
#pragma unroll
    for (int k = kUA - 1; k >= 0; --k)
#pragma unroll
      for (int e = P - 1; e >= 0; --e)
        if (vt[k * P + e] == mt) it = (int)(e_chunk + ((int64_t)k * kThreads + tid) * P + e);
  }
  float st = 0.f, md = 0.f, sd = 0.f, wd = 0.f;
  if (want_soft) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int e = 0; e < NE; e += 4) {
      a0 += __builtin_amdgcn_exp2f((vt[e] - mt) * Lhi);
      a1 += __builtin_amdgcn_exp2f((vt[e + 1] - mt) * Lhi);
      a2 += __builtin_amdgcn_exp2f((vt[e + 2] - mt) * Lhi);
      a3 += __builtin_amdgcn_exp2f((vt[e + 3] - mt) * Lhi);
    }
    st = (a0 + a1) + (a2 + a3);
    if (mt == Elem<DT>::kPad) st = 0.f;  // lane beyond the end of the row: no terms
    // ---- draft row (same accumulation pattern, so identical rows give identical sums)
    float vd[NE];
#pragma unroll
    for (int k = 0; k < kUA; ++k) unpack<DT>(qd[k], vd + k * P);
    md = vd[0];
#pragma unroll
    for (int e = 1; e < NE; ++e) md = fmaxf(md, vd[e]);
    float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f;
    if (want_w) {
      float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f;
#pragma unroll
      for (int e = 0; e < NE; e += 4) {
        const float e0 = __builtin_amdgcn_exp2f((vd[e] - md) * Lhi);
        const float e1 = __builtin_amdgcn_exp2f((vd[e + 1] - md) * Lhi);
        const float e2 = __builtin_amdgcn_exp2f((vd[e + 2] - md) * Lhi);
        const float e3 = __builtin_amdgcn_exp2f((vd[e + 3] - md) * Lhi);
        b0 += e0;
        b1 += e1;
        b2 += e2;
        b3 += e3;
        w0 = fmaf(e0, vd[e] - vt[e], w0);
        w1 = fmaf(e1, vd[e + 1] - vt[e + 1], w1);
        w2 = fmaf(e2, vd[e + 2] - vt[e + 2], w2);
        w3 = fmaf(e3, vd[e + 3] - vt[e + 3], w3);
      }
      wd = (w0 + w1) + (w2 + w3);
    } else {
#pragma unroll
      for (int e = 0; e < NE; e += 4) {
        b0 += __builtin_amdgcn_exp2f((vd[e] - md) * Lhi);
        b1 += __builtin_amdgcn_exp2f((vd[e + 1] - md) * Lhi);
        b2 += __builtin_amdgcn_exp2f((vd[e + 2] - md) * Lhi);
        b3 += __builtin_amdgcn_exp2f((vd[e + 3] - md) * Lhi);
      }
    }
    sd = (b0 + b1) + (b2 + b3);
    if (md == Elem<DT>::kPad) sd = wd = 0.f;
  }

  // ---- wave reduction of the lane partials (rescale factors from exact differences)
  const float Mt = wave_max(mt);
  if (want_idx) it = wave_min_int(mt == Mt ? it : INT_MAX);
  if (want_soft) {
    st = wave_sum(st * exp_hp(mt - Mt, Lhi, Llo));
    const float Md = wave_max(md);
    const float f = exp_hp(md - Md, Lhi, Llo);
    sd = wave_sum(sd * f);
    if (want_w) wd = wave_sum(wd * f);
    md = Md;
  }
  if (lane == 0) {
    sh.m[0][wv] = Mt;
    sh.s[0][wv] = st;
    sh.m[1][wv] = md;
    sh.s[1][wv] = sd;
    sh.w[wv] = wd;
    sh.i[wv] = it;
  }
  __syncthreads();
  // ---- workgroup partial (float64 from here on)
  if (tid == 0) {
    PartA pa;
    float M = sh.m[0][0], Md2 = sh.m[1][0];
    for (int k = 1; k < kWaves; ++k) {
      M = fmaxf(M, sh.m[0][k]);
      Md2 = fmaxf(Md2, sh.m[1][k]);
    }
    int I = INT_MAX;
    double S = 0.0, Sd = 0.0, W = 0.0;
    for (int k = 0; k < kWaves; ++k) {
      if (sh.m[0][k] == M) I = min(I, sh.i[k]);
      if (want_soft) {
        S += (double)sh.s[0][k] * (double)exp_hp(sh.m[0][k] - M, Lhi, Llo);
        const double f = (double)exp_hp(sh.m[1][k] - Md2, Lhi, Llo);
        Sd += (double)sh.s[1][k] * f;
        W += (double)sh.w[k] * f;
      }
    }
    pa.m_t = M;
    pa.s_t = S;
    pa.m_d = Md2;
    pa.s_d = Sd;
    pa.w = W;
    pa.idx = I;
    pa.pad = 0;
    p.part_a[item] = pa;
    if (gathered) {
      p.gat[2 * drow] = gx_t;
      p.gat[2 * drow + 1] = gx_d;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned old = atomicAdd(&p.cnt_task[task], 1u);
    sh.last_chunk = (old == (unsigned)(p.nch_a - 1));
  }
  __syncthreads();
  if (!sh.last_chunk) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // ---- last workgroup of the task: merge the chunk partials (wave 0, fixed order)
  if (wv == 0) {
    float m1 = -FLT_MAX, m2 = -FLT_MAX;
    double s1 = 0.0, s2 = 0.0, w2 = 0.0;
    int i1 = INT_MAX;
    for (int ch = lane; ch < p.nch_a; ch += 64) {
      const PartA q = p.part_a[(int64_t)task * p.nch_a + ch];
      if (q.m_t > m1) {
        if (want_soft) s1 = s1 * (double)exp_hp(m1 - q.m_t, Lhi, Llo) + q.s_t;
        m1 = q.m_t;
        i1 = q.idx;
      } else {
        if (want_soft) s1 += q.s_t * (double)exp_hp(q.m_t - m1, Lhi, Llo);
        if (q.m_t == m1) i1 = min(i1, q.idx);
      }
      if (want_soft) {
        if (q.m_d > m2) {
          const double f = (double)exp_hp(m2 - q.m_d, Lhi, Llo);
          s2 = s2 * f + q.s_d;
          w2 = w2 * f + q.w;
          m2 = q.m_d;
        } else {
          const double f = (double)exp_hp(q.m_d - m2, Lhi, Llo);
          s2 += q.s_d * f;
          w2 += q.w * f;
        }
      }
    }
    const float M1 = wave_max(m1);
    const int I1 = wave_min_int(m1 == M1 ? i1 : INT_MAX);
    double S1 = 0.0, S2 = 0.0, W2 = 0.0;
    float M2 = 0.f;
    if (want_soft) {
      S1 = wave_sum_d(s1 * (double)exp_hp(m1 - M1, Lhi, Llo));
      M2 = wave_max(m2);
      const double f = (double)exp_hp(m2 - M2, Lhi, Llo);
      S2 = wave_sum_d(s2 * f);
      W2 = wave_sum_d(w2 * f);
    }
    if (lane == 0) {
      TaskStat ts;
      ts.m_t = M1;
      ts.s_t = S1;
      ts.m_d = M2;
      ts.s_d = S2;
      ts.w = W2;
      ts.idx = I1;
      ts.kl = 0.0f;
      int refine = 0;
      if (want_w) {
        // one-pass KL and a bound on its rounding error (a few 1e-7 of the
        // magnitude of the terms that cancel)
        const double a = W2 / S2 / (double)T, bm = ((double)M2 - (double)M1) / (double)T, lg = log(S2 / S1);
        const double kl = a - bm - lg;
        const double err = 4e-7 * (fabs(a) + fabs(bm) + fabs(lg) + 1.0);
        refine = err > 1e-5 * kl;
        if (MODE == SV_MODE_NKL && p.V > 1) {
          const double lnV = log((double)p.V);
          refine |= fabs(kl / lnV - (double)p.delta) < 2.0 * err / lnV;
        }
        ts.kl = (float)kl;
      }
      p.stat[task] = ts;
      sh.refine = refine;
      sh.d[0] = S1;
      sh.d[1] = S2;
      sh.m[0][0] = M1;
      sh.m[1][0] = M2;
    }
  }
  __syncthreads();
  if (sh.refine) {
    const double kl = kl_second_pass<DT, VEC>(p, trow, drow, sh.m[0][0], sh.m[1][0], sh.d[0], sh.d[1], T, Lhi, sh.d + 2);
    if (tid == 0) p.stat[task].kl = (float)kl;
  }
  if (tid == 0) {
    p.cnt_task[task] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int g = p.gamma[b];
    const unsigned need = (unsigned)(MODE == SV_MODE_STOCHASTIC ? g : g + 1);
    const unsigned old = atomicAdd(&p.cnt_req[b], 1u);
    sh.last_task = (old == need - 1);
  }
  __syncthreads();
  if (!sh.last_task) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // ---- last task of the request: decide
  if (MODE == SV_MODE_STOCHASTIC)
    decide_stochastic(p, b, sh.dec);
  else if (MODE == SV_MODE_TREE_GREEDY)
    decide_tree(p, b, sh.dec, tree_info, tree_par);
  else
    decide_argmax_chain<MODE>(p, b, sh.dec);
  if (tid == 0) p.cnt_req[b] = 0u;
}

// ----------------------------------------------------------------------------
// k_draw (stochastic mode)
// ----------------------------------------------------------------------------

struct DrawShared {
  double d[kWaves];
  float f[kWaves];
  int i[kWaves];
  int last;
  double ta[kThreads], tb[kThreads];  // one tile of chunk partials
  float tm[kThreads];
  double a_tot, b_tot, S, base;
  float mrow;
  int cstar, lastpos_chunk;
};

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_draw(Params p) {
  constexpr int P = Elem<DT>::P;
  constexpr int NE = kUC * P;
  constexpr int64_t CH = (int64_t)kThreads * NE;
  __shared__ DrawShared sh;
  if (p.hdr[0] != 0) return;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.nch_c;
  const int chunk = blockIdx.x - b * p.nch_c;
  const int64_t V = p.V;
  const int g = p.gamma[b];
  const int t0 = p.t_off[b];
  const float T = p.temp[b];
  const float ur = p.ur[b];

  int kind, j, trow, drow;
  float Mt = 0.f, Md = 0.f, k0 = 0.f;
  if (g == 0) {
    // nothing drafted: the step is a plain draw from target row 0
    if (!temp_ok(T) || !unit_ok(ur)) {
      if (chunk == 0 && tid == 0) {
        p.out_num[b] = -1;
        p.out_tokens[t0] = -1;
        if (p.out_resid) p.out_resid[b] = __builtin_nanf("");
      }
      return;
    }
    kind = kTermBonus;
    j = 0;
    trow = t0;
    drow = -1;
  } else {
    const Term tm = p.term[b];
    kind = tm.kind;
    if (kind == kTermNone) return;
    j = tm.j;
    trow = tm.trow;
    drow = tm.drow;
    Mt = tm.m_t;
    Md = tm.m_d;
    k0 = tm.k0;
  }
  const double Ld = kLog2eD / (double)T;
  const float Lhi = (float)Ld;
  const float Llo = (float)(Ld - (double)Lhi);
  const int64_t e_chunk = (int64_t)chunk * CH;

  // ---- chunk partial sums
  uint4 qt[kUC], qd[kUC];
#pragma unroll
  for (int k = 0; k < kUC; ++k) qt[k] = fetch<DT, VEC>(p.target, trow, V, e_chunk + ((int64_t)k * kThreads + tid) * P);
  if (kind == kTermResidual) {
#pragma unroll
    for (int k = 0; k < kUC; ++k) qd[k] = fetch<DT, VEC>(p.draft, drow, V, e_chunk + ((int64_t)k * kThreads + tid) * P);
  }
  float vt[NE];
#pragma unroll
  for (int k = 0; k < kUC; ++k) unpack<DT>(qt[k], vt + k * P);
  double A = 0.0, Bs = 0.0, Ap = 0.0, Bp = 0.0;
  float mc = 0.f;
  if (kind == kTermResidual) {
    float vd[NE];
#pragma unroll
    for (int k = 0; k < kUC; ++k) unpack<DT>(qd[k], vd + k * P);
#pragma unroll
    for (int k = 0; k < kUC; ++k) {
      float sa = 0.f, sb = 0.f, sap = 0.f, sbp = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const float a = exp_hp(vt[k * P + e] - Mt, Lhi, Llo);
        const float bb = exp_hp(vd[k * P + e] - Md, Lhi, Llo);
        sa += a;
        sb += bb;
        const bool in = a > k0 * bb;
        sap += in ? a : 0.f;
        sbp += in ? bb : 0.f;
      }
      A += (double)sa;
      Bs += (double)sb;
      Ap += (double)sap;
      Bp += (double)sbp;
    }
  } else {
    float m = vt[0];
#pragma unroll
    for (int e = 1; e < NE; ++e) m = fmaxf(m, vt[e]);
    mc = block_max(m, sh.f);
#pragma unroll
    for (int k = 0; k < kUC; ++k) {
      float sa = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) sa += exp_hp(vt[k * P + e] - mc, Lhi, Llo);
      A += (double)sa;
    }
  }
  A = block_sum_d(A, sh.d);
  if (kind == kTermResidual) {
    Bs = block_sum_d(Bs, sh.d);
    Ap = block_sum_d(Ap, sh.d);
    Bp = block_sum_d(Bp, sh.d);
  }
  if (tid == 0) {
    PartC pc;
    pc.a = A;
    pc.b = Bs;
    pc.ap = Ap;
    pc.bp = Bp;
    pc.m = mc;
    pc.pad[0] = pc.pad[1] = pc.pad[2] = 0;
    p.part_c[(int64_t)b * p.nch_c + chunk] = pc;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned old = atomicAdd(&p.cnt_draw[b], 1u);
    sh.last = (old == (unsigned)(p.nch_c - 1));
  }
  __syncthreads();
  if (!sh.last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // ---- last workgroup of the request: choose the chunk.  Chunk partials are
  // staged through LDS a tile at a time and combined by thread 0 in chunk
  // order, so the result does not depend on which workgroup finished last.
  const PartC* pcs = p.part_c + (int64_t)b * p.nch_c;
  const int nch = p.nch_c;
  // stage 1: totals of a and b, and the row maximum (bonus)
  {
    double at = 0.0, bt = 0.0;
    float M = -FLT_MAX;
    for (int base = 0; base < nch; base += kThreads) {
      const int ch = base + tid;
      if (ch < nch) {
        const PartC q = pcs[ch];
        sh.ta[tid] = q.a;
        sh.tb[tid] = q.b;
        sh.tm[tid] = q.m;
      }
      __syncthreads();
      if (tid == 0) {
        const int n = min(kThreads, nch - base);
        for (int k = 0; k < n; ++k) {
          at += sh.ta[k];
          bt += sh.tb[k];
          M = fmaxf(M, sh.tm[k]);
        }
      }
      __syncthreads();
    }
    if (tid == 0) {
      sh.a_tot = at;
      sh.b_tot = bt;
      sh.mrow = M;
    }
    __syncthreads();
  }
  const double K = kind == kTermResidual ? sh.a_tot / sh.b_tot : 0.0;
  const float Mrow = sh.mrow;
  // chunk weight: residual  sum_{a > k0 b}(a - K b) = A+ - K B+ ; bonus  A_c exp((m_c - M)/T)
  auto weight = [&](const PartC& q, int fb) -> double {
    if (kind == kTermResidual) return fb ? q.a : q.ap - K * q.bp;
    return q.a * exp2(((double)q.m - (double)Mrow) * Ld);
  };
  int fallback = 0;
  // stage 2: total mass S
  double S;
  {
    double tot = 0.0;
    for (int base = 0; base < nch; base += kThreads) {
      const int ch = base + tid;
      if (ch < nch) sh.ta[tid] = weight(pcs[ch], 0);
      __syncthreads();
      if (tid == 0) {
        const int n = min(kThreads, nch - base);
        for (int k = 0; k < n; ++k) tot += sh.ta[k];
      }
      __syncthreads();
    }
    if (tid == 0) sh.S = tot;
    __syncthreads();
    S = sh.S;
    if (kind == kTermResidual && !(S > 0.0)) {
      // max(0, p - q) vanished numerically: draw from p_j instead
      fallback = 1;
      S = sh.a_tot;
    }
  }
  const double target = (double)ur * S;
  // stage 3: first chunk whose cumulative weight exceeds the target
  if (tid == 0) {
    sh.cstar = -1;
    sh.lastpos_chunk = -1;
    sh.base = 0.0;
  }
  __syncthreads();
  {
    double cum = 0.0;
    for (int base = 0; base < nch; base += kThreads) {
      const int ch = base + tid;
      if (ch < nch) sh.ta[tid] = weight(pcs[ch], fallback);
      __syncthreads();
      if (tid == 0 && sh.cstar < 0) {
        const int n = min(kThreads, nch - base);
        for (int k = 0; k < n; ++k) {
          if (sh.ta[k] > 0.0) sh.lastpos_chunk = base + k;
          const double nxt = cum + sh.ta[k];
          if (nxt > target) {
            sh.cstar = base + k;
            sh.base = cum;
            break;
          }
          cum = nxt;
        }
      }
      __syncthreads();
      if (sh.cstar >= 0) break;  // uniform: read after the barrier
    }
  }
  int cstar = sh.cstar;
  bool take_last = false;
  if (cstar < 0) {  // rounding left the target at/after the end: last token with mass
    cstar = sh.lastpos_chunk >= 0 ? sh.lastpos_chunk : nch - 1;
    take_last = true;
  }
  const double cbase = sh.base;

  // ---- re-read chunk c*: thread t owns NE consecutive tokens
  const int64_t y0 = (int64_t)cstar * CH + (int64_t)tid * NE;
  double r[NE];
  double tsum = 0.0;
  const double chunk_factor =
      (kind == kTermBonus) ? exp2(((double)pcs[cstar].m - (double)Mrow) * Ld) : 1.0;
  const float ref = (kind == kTermBonus) ? pcs[cstar].m : Mt;
#pragma unroll
  for (int k = 0; k < kUC; ++k) {
    const uint4 q = fetch<DT, VEC>(p.target, trow, V, y0 + k * P);
    float v[P];
    unpack<DT>(q, v);
    float vdd[P];
    if (kind == kTermResidual && !fallback) {
      const uint4 qq = fetch<DT, VEC>(p.draft, drow, V, y0 + k * P);
      unpack<DT>(qq, vdd);
    }
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const float a = exp_hp(v[e] - ref, Lhi, Llo);
      double rv;
      if (kind == kTermResidual && !fallback) {
        const float bb = exp_hp(vdd[e] - Md, Lhi, Llo);
        rv = (a > k0 * bb) ? (double)a - K * (double)bb : 0.0;
      } else {
        rv = (double)a * chunk_factor;
      }
      if (y0 + k * P + e >= V) rv = 0.0;
      r[k * P + e] = rv;
      tsum += rv;
    }
  }
  double tot;
  const double excl = block_exclusive_scan_d(tsum, sh.d, tot);
  (void)tot;
  int cand = INT_MAX;
  int lastpos = -1;
  {
    double cum = cbase + excl;
    const bool mine = !take_last && cum <= target && cum + tsum > target;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      if (r[e] > 0.0) lastpos = (int)(y0 + e);
      if (mine && cand == INT_MAX) {
        cum += r[e];
        if (cum > target) cand = (int)(y0 + e);
      }
    }
  }
  const int ystar0 = block_min_int(cand, sh.i);
  const int ylast = block_max_int(lastpos, sh.i);
  if (tid == 0) {
    int y = ystar0 != INT_MAX ? ystar0 : ylast;
    if (y < 0 || y >= p.V) y = (int)min<int64_t>(V - 1, (int64_t)cstar * CH);
    p.out_tokens[t0 + j] = y;
    if (g == 0) p.out_num[b] = 0;
    if (p.out_resid) p.out_resid[b] = (kind == kTermResidual && !fallback) ? (float)(S / sh.a_tot) : 1.0f;
    p.cnt_draw[b] = 0u;
  }
}

}  // namespace

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------

int launch_prep(const Params& p, void* stream) {
  hipLaunchKernelGGL(k_prep, dim3(1), dim3(kPrepThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

template <int DT, bool VEC>
static void rowstats_dispatch(const Params& p, hipStream_t s, dim3 grid) {
  switch (p.mode) {
    case SV_MODE_STOCHASTIC: hipLaunchKernelGGL((k_rowstats<DT, VEC, SV_MODE_STOCHASTIC>), grid, dim3(kThreads), 0, s, p); break;
    case SV_MODE_GREEDY: hipLaunchKernelGGL((k_rowstats<DT, VEC, SV_MODE_GREEDY>), grid, dim3(kThreads), 0, s, p); break;
    case SV_MODE_NKL: hipLaunchKernelGGL((k_rowstats<DT, VEC, SV_MODE_NKL>), grid, dim3(kThreads), 0, s, p); break;
    default: hipLaunchKernelGGL((k_rowstats<DT, VEC, SV_MODE_TREE_GREEDY>), grid, dim3(kThreads), 0, s, p); break;
  }
}

int launch_rowstats(const Params& p, bool vec, void* stream) {
  const int64_t n = (int64_t)p.n_task * p.nch_a;
  if (n <= 0) return 0;
  const dim3 grid((unsigned)n);
  hipStream_t s = (hipStream_t)stream;
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) rowstats_dispatch<SV_DTYPE_BF16, true>(p, s, grid);
    else rowstats_dispatch<SV_DTYPE_BF16, false>(p, s, grid);
  } else {
    if (vec) rowstats_dispatch<SV_DTYPE_F32, true>(p, s, grid);
    else rowstats_dispatch<SV_DTYPE_F32, false>(p, s, grid);
  }
  return (int)hipGetLastError();
}

int launch_draw(const Params& p, bool vec, void* stream) {
  const int64_t n = (int64_t)p.B * p.nch_c;
  if (n <= 0) return 0;
  const dim3 grid((unsigned)n);
  hipStream_t s = (hipStream_t)stream;
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) hipLaunchKernelGGL((k_draw<SV_DTYPE_BF16, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((k_draw<SV_DTYPE_BF16, false>), grid, dim3(kThreads), 0, s, p);
  } else {
    if (vec) hipLaunchKernelGGL((k_draw<SV_DTYPE_F32, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((k_draw<SV_DTYPE_F32, false>), grid, dim3(kThreads), 0, s, p);
  }
  return (int)hipGetLastError();
}

}  // namespace sv
